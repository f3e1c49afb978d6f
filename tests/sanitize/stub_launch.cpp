// stub_launch.cpp -- host stand-ins for the kernel launchers of libgqa_attn.so
// (launch.h) and the HIP calls api.hip makes, for the sanitizer build of the
// C ABI layer.  Each launcher records its argument block; nothing runs.
#include "stub_launch.h"

StubLog g_stub;

hipError_t hipGetLastError(void) { return hipSuccess; }
hipError_t hipGetDevice(int *device)
{
    *device = 0;
    return hipSuccess;
}
hipError_t hipGetSymbolAddress(void **devPtr, const void *symbol)
{
    *devPtr = const_cast<void *>(symbol);
    ++g_stub.symbol_lookups;
    return hipSuccess;
}

namespace gqa {
int launch_fwd_bf16(const FwdArgs &a, int D, hipStream_t)
{
    g_stub.fwd = a;
    g_stub.fwd_d = D;
    ++g_stub.launches;
    return 0;
}
int launch_fwd_bf16_shard(const FwdArgs &a, int D, hipStream_t s) { return launch_fwd_bf16(a, D, s); }
int fwd_bf16_waves_per_block() { return 8; }
int fwd_bf16_rows_per_wave() { return 32; }
int launch_decode_bf16(const DecodeArgs &a, int, int, hipStream_t)
{
    g_stub.dec = a;
    ++g_stub.launches;
    return 0;
}
int launch_decode_fp8(const DecodeArgs &a, int Dk, int Dv, hipStream_t s) { return launch_decode_bf16(a, Dk, Dv, s); }
int launch_mla_decode(const DecodeArgs &a, hipStream_t s) { return launch_decode_bf16(a, 576, 512, s); }
int launch_mla_decode_topk(const DecodeArgs &a, hipStream_t s) { return launch_decode_bf16(a, 576, 512, s); }
int mla_topk_max_chunk() { return 4096; }
int mla_heads_per_block() { return 128; }
int decode_bf16_key_tile() { return 32; }
int decode_bf16_flat_workgroups(int) { return 2048; }
int decode_bf16_flat_first_round(int) { return 1024; }
int decode_fp8_flat_workgroups(int) { return 2048; }
int decode_bf16_heads_per_block(int Dk, int) { return Dk == 576 ? 128 : 32; }
int launch_fwd_f32(const F32FwdArgs &, int, hipStream_t)
{
    ++g_stub.launches;
    return 0;
}
int launch_decode_f32(const DecodeArgs &a, int D, hipStream_t s) { return launch_decode_bf16(a, D, D, s); }
int launch_combine(const CombineArgs &a, hipStream_t)
{
    g_stub.comb = a;
    ++g_stub.launches;
    return 0;
}
int launch_merge(const MergeArgs &, hipStream_t)
{
    ++g_stub.launches;
    return 0;
}
} // namespace gqa
