// combine.hip -- exact log-sum-exp merge of split-KV decode partials.
//
// Each split s of a row holds a normalised partial output o_s over its key
// chunk and lse_s = log2 of that chunk's softmax normaliser (in the scaled,
// base-2 units the partial kernels use).  Softmax over the union of chunks
// is recovered exactly (up to rounding) as
//     L = log2 sum_s 2^{lse_s},   o = sum_s 2^{lse_s - L} o_s,
// the same merge online softmax applies tile by tile ("A Visual Guide to
// Attention", section on sources and execution).  Empty chunks carry
// lse = -inf and weigh nothing (their partial outputs are loaded but
// selected away, whatever they hold); a row with no keys at all yields
// zeros.  Partial outputs are fp32 and the merge accumulates in fp32.
#include "launch.h"

namespace gqa {

namespace {

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kCT = 128;  // threads per row at most; each owns 4 output dims
constexpr int kCB = 16;   // partial outputs loaded together before any is used

// Latency, not bandwidth, bounds this pass (a few MB in total), so every
// load is issued before its value is needed: the row's lse values (lane s
// holds split s) and the first kCB partial outputs in one round trip, one
// more per further batch of kCB partial outputs
// (unconditional loads of in-bounds slots; slots past the split count and
// empty slots get weight 0 and are selected away, whatever they hold).
template <bool OUT_BF16>
__global__ __launch_bounds__(kCT) void combine_kernel(CombineArgs p)
{
    using PT = float;
    using PT4 = f32x4;
    // row b * Hq + head, last row first: the flat decode cuts the streams at
    // the end of its tile order into the most pieces, so the rows that need
    // more than one batch of partial loads start first
    const size_t row = (size_t)gridDim.x - 1 - blockIdx.x;
    const float *lse = p.part_lse + row * p.S;
    const PT *po = (const PT *)p.part_o + row * (size_t)p.S * p.Dv;
    const int ns = p.S;
    const int lane = threadIdx.x & 63;
    const int dim = threadIdx.x * 4;
    const int d0 = min(dim, p.Dv - 4);  // lanes past Dv mirror the last dims and store nothing

    auto load_batch = [&](PT4 (&v)[kCB], int s0, int sb, int n) {
#pragma unroll
        for (int i = 0; i < kCB; ++i) v[i] = *(const PT4 *)(po + (size_t)(s0 + min(sb + i, n - 1)) * p.Dv + d0);
    };
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    float wsum = 0.f;
    auto add_batch = [&](const PT4 (&v)[kCB], int sb, int n, float wl) {
#pragma unroll
        for (int i = 0; i < kCB; ++i) {
            const float wi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), min(sb + i, 63)));
            const float w = sb + i < n ? wi : 0.f;
            const bool use = w != 0.f;
            wsum += w;
            acc[0] = use ? fmaf(w, (float)v[i][0], acc[0]) : acc[0];
            acc[1] = use ? fmaf(w, (float)v[i][1], acc[1]) : acc[1];
            acc[2] = use ? fmaf(w, (float)v[i][2], acc[2]) : acc[2];
            acc[3] = use ? fmaf(w, (float)v[i][3], acc[3]) : acc[3];
        }
    };

    float ll = lane < ns ? lse[lane] : -INFINITY;
    PT4 v[kCB];
    load_batch(v, 0, 0, min(64, ns));  // in flight together with the lse load
    float L = ll;
    // slots past the last non-empty one weigh nothing: no batch is loaded
    // for them (a split count above what a row uses costs no round trip)
    int used = 0;
    for (int s0 = 0; s0 < ns; s0 += 64) {
        const float x = s0 == 0 ? ll : (s0 + lane < ns ? lse[s0 + lane] : -INFINITY);
        L = fmaxf(L, x);
        const unsigned long long nz = __ballot(!(x == -INFINITY));
        if (nz) used = s0 + 64 - __builtin_clzll(nz);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) L = fmaxf(L, __shfl_xor(L, o));
    if (L != -INFINITY) {
        for (int s0 = 0; s0 < used; s0 += 64) {
            if (s0 > 0) ll = s0 + lane < ns ? lse[s0 + lane] : -INFINITY;
            const float wl = __builtin_amdgcn_exp2f(ll - L);  // 0 for lse = -inf
            const int n = min(64, used - s0);
            for (int sb = 0; sb < n; sb += kCB) {
                if (s0 > 0 || sb > 0) load_batch(v, s0, sb, n);
                add_batch(v, sb, n, wl);
            }
        }
    }
    if (dim >= p.Dv) return;
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    if (OUT_BF16) {
        uint16_t *out = (uint16_t *)p.out + row * p.Dv + d0;
        bf16x4 r = {(__bf16)(acc[0] * inv), (__bf16)(acc[1] * inv), (__bf16)(acc[2] * inv),
                    (__bf16)(acc[3] * inv)};
        *(bf16x4 *)out = r;
    } else {
        float *out = (float *)p.out + row * p.Dv + d0;
        *(float4 *)out = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
    }
}

// Merge of gathered partial results (sequence-parallel shards): many rows,
// few parts.  One thread per (row, 4 output dims); the threads of a row each
// read the row's S lse values (the same addresses) and form the weights
// themselves, then stream the S partial outputs.
constexpr int kMT = 256;  // threads per merge workgroup

template <bool OUT_BF16>
__global__ __launch_bounds__(kMT) void merge_kernel(MergeArgs p)
{
    constexpr int kB = 8;  // parts whose loads are in flight together
    const int per_row = p.Dv / 4;
    const long long t = (long long)blockIdx.x * kMT + threadIdx.x;
    if (t >= p.rows * per_row) return;
    const long long row = t / per_row;
    const int d0 = (int)(t - row * per_row) * 4;
    const float *lr = p.lse + row * p.l_rs;
    const float *orow = p.o + row * p.o_rs + d0;
    // Batches of kB parts with the part index clamped to the last one, so
    // every load is unconditional and in bounds (a repeated part does not
    // change the max, and gets weight 0 below); each batch is one round trip.
    float L = -INFINITY;
    for (int s0 = 0; s0 < p.S; s0 += kB) {
        float l[kB];
#pragma unroll
        for (int i = 0; i < kB; ++i) l[i] = lr[(size_t)min(s0 + i, p.S - 1) * p.l_ss];
#pragma unroll
        for (int i = 0; i < kB; ++i) L = fmaxf(L, l[i] * p.lse_mul);
    }
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    float wsum = 0.f;
    if (L != -INFINITY) {
        for (int s0 = 0; s0 < p.S; s0 += kB) {
            float l[kB];
            f32x4 v[kB];
#pragma unroll
            for (int i = 0; i < kB; ++i) {
                const size_t s = (size_t)min(s0 + i, p.S - 1);
                l[i] = lr[s * p.l_ss];
                v[i] = *(const f32x4 *)(orow + s * p.o_ss);
            }
            // an empty part (weight 0: lse = -inf) is selected away, whatever
            // its output holds
#pragma unroll
            for (int i = 0; i < kB; ++i) {
                const float w = s0 + i < p.S ? __builtin_amdgcn_exp2f(l[i] * p.lse_mul - L) : 0.f;
                const bool use = w != 0.f;
                wsum += w;
                acc[0] = use ? fmaf(w, v[i][0], acc[0]) : acc[0];
                acc[1] = use ? fmaf(w, v[i][1], acc[1]) : acc[1];
                acc[2] = use ? fmaf(w, v[i][2], acc[2]) : acc[2];
                acc[3] = use ? fmaf(w, v[i][3], acc[3]) : acc[3];
            }
        }
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    if (OUT_BF16) {
        bf16x4 r = {(__bf16)(acc[0] * inv), (__bf16)(acc[1] * inv), (__bf16)(acc[2] * inv),
                    (__bf16)(acc[3] * inv)};
        *(bf16x4 *)((uint16_t *)p.out + row * p.Dv + d0) = r;
    } else {
        *(float4 *)((float *)p.out + row * p.Dv + d0) =
            make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
    }
}

} // namespace

int launch_merge(const MergeArgs &a, hipStream_t stream)
{
    if (a.Dv % 4 != 0 || a.Dv <= 0 || a.S <= 0 || a.rows <= 0) return -1;
    const long long threads = a.rows * (a.Dv / 4);
    const long long nblk = (threads + kMT - 1) / kMT;
    if (nblk > 0x7fffffffLL) return -1;
    dim3 grid((unsigned)nblk), block(kMT);
    if (a.out_bf16)
        hipLaunchKernelGGL(merge_kernel<true>, grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL(merge_kernel<false>, grid, block, 0, stream, a);
    return 0;
}

int launch_combine(const CombineArgs &a, hipStream_t stream)
{
    if (a.Dv % 4 != 0 || a.Dv <= 0 || a.Dv > 4 * kCT || a.S <= 0) return -1;
    dim3 grid((unsigned)((size_t)a.B * a.Hq)), block((a.Dv / 4 + 63) / 64 * 64);  // whole waves
    if (a.out_bf16)
        hipLaunchKernelGGL((combine_kernel<true>), grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((combine_kernel<false>), grid, block, 0, stream, a);
    return 0;
}

} // namespace gqa
