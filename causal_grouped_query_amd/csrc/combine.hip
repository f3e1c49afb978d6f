// combine.hip -- exact log-sum-exp merge of split-KV decode partials.
//
// Each split s of a row holds a normalised partial output o_s over its key
// chunk and lse_s = log2 of that chunk's softmax normaliser (in the scaled,
// base-2 units the partial kernels use).  Softmax over the union of chunks
// is recovered exactly (up to rounding) as
//     L = log2 sum_s 2^{lse_s},   o = sum_s 2^{lse_s - L} o_s,
// the same merge online softmax applies tile by tile ("A Visual Guide to
// Attention", section on sources and execution).  Empty chunks carry
// lse = -inf and weigh nothing; a row with no keys at all yields zeros.
// After the balanced (flat) decode a row has a variable number of pieces,
// recorded per stream by the partial kernel.
#include "launch.h"

namespace gqa {

namespace {

constexpr int kCT = 128;  // threads per row; each owns 4 output dims

template <bool OUT_BF16>
__global__ __launch_bounds__(kCT) void combine_kernel(CombineArgs p)
{
    const size_t row = blockIdx.x;  // b * Hq + head
    const float *lse = p.part_lse + row * p.S;
    const float *po = p.part_o + row * (size_t)p.S * p.Dv;
    int ns = p.S;
    if (p.counts) {
        const int b = (int)(row / p.Hq), head = (int)(row % p.Hq);
        const int w = (b * p.Hkv + head / p.G) * p.n_hblk + (head % p.G) / 32;
        ns = p.lens[b] > 0 ? p.counts[w] : 0;
    }

    float L = -INFINITY;
    for (int s = 0; s < ns; ++s) L = fmaxf(L, lse[s]);
    const int d0 = threadIdx.x * 4;
    if (d0 >= p.Dv) return;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    float wsum = 0.f;
    if (L != -INFINITY) {
        for (int s = 0; s < ns; ++s) {
            const float w = __builtin_amdgcn_exp2f(lse[s] - L);
            if (w == 0.f) continue;
            wsum += w;
            const float4 v = *(const float4 *)(po + (size_t)s * p.Dv + d0);
            acc[0] = fmaf(w, v.x, acc[0]);
            acc[1] = fmaf(w, v.y, acc[1]);
            acc[2] = fmaf(w, v.z, acc[2]);
            acc[3] = fmaf(w, v.w, acc[3]);
        }
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    if (OUT_BF16) {
        uint16_t *out = (uint16_t *)p.out + row * p.Dv + d0;
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        bf16x4 r = {(__bf16)(acc[0] * inv), (__bf16)(acc[1] * inv), (__bf16)(acc[2] * inv),
                    (__bf16)(acc[3] * inv)};
        *(bf16x4 *)out = r;
    } else {
        float *out = (float *)p.out + row * p.Dv + d0;
        *(float4 *)out = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
    }
}

} // namespace

int launch_combine(const CombineArgs &a, hipStream_t stream)
{
    if (a.Dv % 4 != 0 || a.Dv > 4 * kCT) return -1;
    dim3 grid((unsigned)((size_t)a.B * a.Hq)), block(kCT);
    if (a.out_bf16)
        hipLaunchKernelGGL(combine_kernel<true>, grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL(combine_kernel<false>, grid, block, 0, stream, a);
    return 0;
}

} // namespace gqa
