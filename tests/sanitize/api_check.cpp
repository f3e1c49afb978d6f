// api_check.cpp -- drives every exported entry point of the C ABI layer
// (causal_grouped_query_amd/csrc/api.hip, built host-only against stub
// launchers) under AddressSanitizer and UndefinedBehaviorSanitizer.  Invalid
// calls must return their documented code without a launch; valid calls must
// launch with the argument blocks the geometry implies.  The pointers are
// aligned stand-in addresses that nothing may dereference: a host read of
// one would fault under the sanitizers.  Exit status 0 iff every check holds.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "gqa_attn.h"
#include "stub_launch.h"

static int failures = 0;
#define CHECK(cond, what)                                                  \
    do {                                                                   \
        if (!(cond)) {                                                     \
            fprintf(stderr, "FAIL %s:%d: %s\n", __FILE__, __LINE__, what); \
            ++failures;                                                    \
        }                                                                  \
    } while (0)

static void *const P = (void *)(uintptr_t)0x100000;  // aligned, never dereferenced
static int *const IP = (int *)(uintptr_t)0x200000;

// a call that must fail with `code` and launch nothing
#define REJECT(call, code)                                      \
    do {                                                        \
        const int before = g_stub.launches;                     \
        const int rc_ = (call);                                 \
        CHECK(rc_ == (code), #call);                            \
        CHECK(g_stub.launches == before, "launch on rejection"); \
    } while (0)

int main()
{
    CHECK(strcmp(gqa_attn_strerror(GQA_OK), "success") == 0, "strerror");
    CHECK(strcmp(gqa_attn_strerror(12345), "unknown error code") == 0, "strerror unknown");

    // ---- forward ----
    int before = g_stub.launches;
    CHECK(gqa_attn_fwd(P, P, P, P, 4, 32, 8, 4096, 4096, 128, 128, 0.088f, 1, GQA_BF16, nullptr) == GQA_OK, "fwd ok");
    CHECK(g_stub.launches == before + 1, "fwd launches once");
    CHECK(g_stub.fwd.Gt == 4 && g_stub.fwd.Pt == 64 && g_stub.fwd.n_qt == 64 && g_stub.fwd.n_units == 32, "fwd grid");
    CHECK(fabsf(g_stub.fwd.c - 0.088f * 1.4426950f) < 1e-6f, "fwd folded scale");
    REJECT(gqa_attn_fwd(nullptr, P, P, P, 1, 4, 2, 8, 8, 128, 128, 0.1f, 1, GQA_BF16, nullptr), GQA_ERR_INVALID_ARG);
    REJECT(gqa_attn_fwd(P, P, P, P, 1, 6, 4, 8, 8, 128, 128, 0.1f, 1, GQA_BF16, nullptr), GQA_ERR_INVALID_ARG);
    REJECT(gqa_attn_fwd(P, P, P, P, 1, 4, 2, 9, 8, 128, 128, 0.1f, 1, GQA_BF16, nullptr), GQA_ERR_INVALID_ARG);
    REJECT(gqa_attn_fwd(P, P, P, P, 1, 4, 2, 8, 8, 128, 128, NAN, 1, GQA_BF16, nullptr), GQA_ERR_INVALID_ARG);
    REJECT(gqa_attn_fwd(P, P, P, P, 1, 4, 2, 8, 8, 96, 96, 0.1f, 1, GQA_BF16, nullptr), GQA_ERR_UNSUPPORTED);
    REJECT(gqa_attn_fwd(P, P, P, P, 1, 4, 2, 8, 8, 128, 128, 0.1f, 1, (gqa_dtype)7, nullptr), GQA_ERR_INVALID_ARG);
    REJECT(gqa_attn_fwd(P, P, P, P, 0x7fffffff, 64, 1, 0x7fffffff, 0x7fffffff, 128, 128, 0.1f, 1, GQA_BF16,
                        nullptr), GQA_ERR_UNSUPPORTED);  // the grid would overflow

    // ---- packed variable-length forward ----
    before = g_stub.launches;
    CHECK(gqa_attn_fwd_varlen(P, P, P, P, IP, IP, nullptr, nullptr, 8, 32, 8, 16384, 16384, 128, 128, 128, 32 * 128,
                              128, 8 * 128, 128, 8 * 128, 128, 32 * 128, 0.088f, 1, 4096, GQA_BF16, nullptr) == GQA_OK,
          "varlen ok");
    CHECK(g_stub.launches == before + 1 && g_stub.fwd.varlen == 1, "varlen launch");
    CHECK(g_stub.fwd.total_q == 16384 && g_stub.fwd.total_k == 16384 && g_stub.fwd.window == 4096, "varlen bounds");
    REJECT(gqa_attn_fwd_varlen(P, P, P, P, IP, IP, nullptr, nullptr, 8, 32, 8, 16, -1, 128, 128, 128, 32 * 128, 128,
                               8 * 128, 128, 8 * 128, 128, 32 * 128, 0.1f, 1, 0, GQA_BF16, nullptr),
           GQA_ERR_INVALID_ARG);
    REJECT(gqa_attn_fwd_varlen(P, P, P, P, IP, IP, nullptr, nullptr, 8, 32, 8, 16, 16, 128, 128, 128, 32 * 128, 128,
                               8 * 128, 128, 8 * 128, 128, 32 * 128, 0.1f, 0, 4, GQA_BF16, nullptr),
           GQA_ERR_INVALID_ARG);  // a window needs causal attention
    before = g_stub.launches;
    CHECK(gqa_attn_fwd_varlen(P, P, P, P, IP, IP, nullptr, nullptr, 2, 8, 2, 0, 0, 128, 128, 128, 8 * 128, 128,
                              2 * 128, 128, 2 * 128, 128, 8 * 128, 0.1f, 1, 0, GQA_BF16, nullptr) == GQA_OK &&
              g_stub.launches == before,
          "no query token: nothing launched");

    // ---- key shard and merge ----
    float *FP = (float *)P;
    CHECK(gqa_attn_fwd_shard(P, P, P, FP, FP, 8, 64, 1, 512, 2048, 128, 128, 15872, 0, 0.088f, 1, GQA_BF16,
                             nullptr) == GQA_OK,
          "shard ok");
    CHECK(g_stub.fwd.q_minus_k == 15872, "shard offset");
    REJECT(gqa_attn_fwd_shard(P, P, P, FP, FP, 8, 64, 1, 512, 2048, 128, 128, -1, 0, 0.1f, 1, GQA_BF16, nullptr),
           GQA_ERR_INVALID_ARG);
    REJECT(gqa_attn_fwd_shard(P, P, P, FP, FP, 8, 64, 1, 512, 2048, 128, 128, 1LL << 31, 0, 0.1f, 1, GQA_BF16,
                              nullptr), GQA_ERR_UNSUPPORTED);
    CHECK(gqa_attn_merge(FP, FP, P, 8, 262144, 128, GQA_BF16, nullptr) == GQA_OK, "merge ok");
    REJECT(gqa_attn_merge(FP, FP, P, 0, 262144, 128, GQA_BF16, nullptr), GQA_ERR_INVALID_ARG);
    REJECT(gqa_attn_merge(FP, FP, P, 8, 262144, 130, GQA_BF16, nullptr), GQA_ERR_UNSUPPORTED);

    // ---- split-KV decode ----
    const int B = 64, Hq = 32, Hkv = 8, T = 8192, D = 128;
    const long long sb = (long long)Hkv * T * D, sh = (long long)T * D, st = D;
    const int S = gqa_attn_decode_splits(B, Hq, Hkv, T, D, D, GQA_BF16);
    CHECK(S >= 3 && S <= 1024, "default splits");
    const size_t ws = gqa_attn_decode_workspace_size(B, Hq, D, S);
    CHECK(ws >= (size_t)B * Hq * S * (D + 1) * 4 && ws % 256 == 0, "workspace size");
    char *W = (char *)(uintptr_t)0x4000000;
    before = g_stub.launches;
    CHECK(gqa_attn_decode(P, P, P, P, IP, B, Hq, Hkv, T, D, D, sb, sh, st, sb, sh, st, 0.088f, 0, W, ws, GQA_BF16,
                          nullptr) == GQA_OK,
          "decode ok");
    CHECK(g_stub.launches == before + 2, "decode: partial kernel + combine");
    CHECK(g_stub.dec.S == S && g_stub.dec.n_wg == 2048 && g_stub.dec.n_first == 1024, "decode flat schedule");
    CHECK((char *)g_stub.dec.queue == W + ws - 256, "decode piece counter at the workspace end");
    CHECK((char *)g_stub.dec.part_o == W && (char *)g_stub.dec.part_lse == W + (size_t)B * Hq * S * D * 4,
          "decode workspace layout");
    CHECK(g_stub.comb.part_o == g_stub.dec.part_o && g_stub.comb.S == S && g_stub.comb.out_bf16 == 1, "combine args");
    REJECT(gqa_attn_decode(P, P, P, P, IP, B, Hq, Hkv, T, D, D, sb, sh, st, sb, sh, st, 0.088f, 0, W, ws - 1,
                           GQA_BF16, nullptr), GQA_ERR_WORKSPACE);
    REJECT(gqa_attn_decode(P, P, P, P, IP, B, Hq, Hkv, T, D, D, sb, sh, st, sb, sh, st, 0.088f, 1025, W, ws,
                           GQA_BF16, nullptr), GQA_ERR_INVALID_ARG);
    REJECT(gqa_attn_decode(P, P, P, P, IP, B, Hq, Hkv, T, D, D, sb, sh, 100, sb, sh, st, 0.088f, 0, W, ws, GQA_BF16,
                           nullptr), GQA_ERR_INVALID_ARG);  // row stride below the row width
    void *const V2 = (void *)(uintptr_t)0x300000;
    REJECT(gqa_attn_decode(P, P, V2, P, IP, 16, 128, 1, 4096, 576, 512, 4096LL * 576, 4096LL * 576, 576,
                           4096LL * 576, 4096LL * 576, 576, 0.07f, 0, W, 1 << 30, GQA_BF16, nullptr),
           GQA_ERR_UNSUPPORTED);  // MLA with a value that is not the key's latent prefix
    CHECK(gqa_attn_decode(P, P, P, P, IP, 16, 128, 1, 4096, 576, 512, 4096LL * 576, 4096LL * 576, 576,
                          4096LL * 576, 4096LL * 576, 576, 0.07f, 0, W, 1 << 30, GQA_BF16, nullptr) == GQA_OK,
          "absorbed MLA decode");
    CHECK(gqa_attn_decode_window(P, P, P, P, IP, B, Hq, Hkv, T, D, D, sb, sh, st, sb, sh, st, 0.088f, 4096, 0, W, ws,
                                 GQA_BF16, nullptr) == GQA_OK && g_stub.dec.window == 4096,
          "decode window");

    // ---- FP8 cache ----
    const float *SP = (const float *)P;
    CHECK(gqa_attn_decode_fp8(P, P, P, SP, SP, P, IP, B, Hq, Hkv, T, D, D, sb, sh, st, sb, sh, st, Hkv * T, T, 1,
                              Hkv * T, T, 1, 0.088f, 0, 0, W, ws, nullptr) == GQA_OK && g_stub.dec.fp8 == 1,
          "fp8 ok");
    CHECK(g_stub.dec.S == gqa_attn_decode_fp8_splits(B, Hq, Hkv, T, D, D) && g_stub.dec.S <= S &&
              g_stub.dec.queue == nullptr,
          "fp8 default splits, no piece queue");
    REJECT(gqa_attn_decode_fp8_splits(B, Hq, Hkv, T, 576, 512), GQA_ERR_UNSUPPORTED);
    REJECT(gqa_attn_decode_fp8(P, P, P, SP, SP, P, IP, B, Hq, Hkv, T, D, D, sb, sh, st, sb, sh, st, Hkv * T, T, 1,
                               Hkv * T, T, 1, 0.088f, 0, 2, W, ws, nullptr), GQA_ERR_INVALID_ARG);

    // ---- top-k sparse decode ----
    const int St = gqa_attn_decode_topk_splits(16, 128, 2048, 576, 512, GQA_BF16);
    const size_t wst = gqa_attn_decode_workspace_size(16, 128, 512, St);
    CHECK(gqa_attn_decode_topk(P, P, P, IP, IP, 16, 128, 32768, 2048, 576, 512, 32768LL * 576, 576, 0.07f, 0, W, wst,
                               GQA_BF16, nullptr) == GQA_OK,
          "topk ok");
    CHECK(g_stub.dec.topk == 2048 && g_stub.dec.chunk % 32 == 0 && g_stub.dec.chunk <= 4096, "topk slices");
    REJECT(gqa_attn_decode_topk(P, P, P, IP, IP, 16, 128, 32768, 2048, 576, 512, 32768LL * 576, 576, 0.07f, 0, W,
                                wst, GQA_F32, nullptr), GQA_ERR_UNSUPPORTED);

    // ---- allocation-free decode ----
    before = g_stub.launches;
    CHECK(gqa_attn_decode_noalloc(P, P, P, P, IP, B, Hq, Hkv, T, D, D, sb, sh, st, sb, sh, st, 0.088f, 0, GQA_BF16,
                                  nullptr) == GQA_OK,
          "noalloc ok");
    CHECK(g_stub.launches == before + 2 && g_stub.symbol_lookups == 1, "noalloc launches, one lookup");
    const size_t lse_off = ((size_t)B * Hq * S * D * 4 + 255) & ~(size_t)255;
    CHECK((char *)g_stub.dec.part_lse == (char *)g_stub.dec.part_o + lse_off, "noalloc compact layout");
    CHECK(gqa_attn_decode_noalloc(P, P, P, P, IP, 2, 8, 2, 100, D, D, 2LL * 100 * D, 100LL * D, D, 2LL * 100 * D,
                                  100LL * D, D, 0.1f, 0, GQA_BF16, nullptr) == GQA_OK &&
              g_stub.symbol_lookups == 1,
          "noalloc second call reuses the device address");
    REJECT(gqa_attn_decode_noalloc(P, P, P, P, IP, 1024, 128, 1, 64, 576, 512, 64LL * 576, 64LL * 576, 576,
                                   64LL * 576, 64LL * 576, 576, 0.07f, 16, GQA_BF16, nullptr), GQA_ERR_WORKSPACE);
    REJECT(gqa_attn_decode_noalloc(nullptr, P, P, P, IP, B, Hq, Hkv, T, D, D, sb, sh, st, sb, sh, st, 0.088f, 0,
                                   GQA_BF16, nullptr), GQA_ERR_INVALID_ARG);
    CHECK(gqa_attn_decode_noalloc_scratch_bytes(B, Hq, D, S, GQA_BF16) ==
              ((lse_off + (size_t)B * Hq * S * 4 + 255) & ~(size_t)255) + 256,
          "noalloc scratch size");

    if (failures) fprintf(stderr, "%d check(s) failed\n", failures);
    else printf("api checks passed\n");
    return failures ? 1 : 0;
}
