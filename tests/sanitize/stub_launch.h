// stub_launch.h -- what the stub launchers of the sanitizer build record.
#pragma once
#include "launch.h"

struct StubLog {
    int launches = 0;
    int symbol_lookups = 0;
    int fwd_d = 0;
    gqa::FwdArgs fwd{};
    gqa::DecodeArgs dec{};
    gqa::CombineArgs comb{};
};
extern StubLog g_stub;
