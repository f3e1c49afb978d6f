// f32_kernels.hip -- fp32 attention for small head dims (64, 128): the
// prefill/suffix forward and the split-KV decode partials, on the vector ALU.
//
// Same operation as the bf16 kernels (unified formula of the "Attention
// variants" page, query offset Tk - Tq of its minimal semantic
// implementation), kept in fp32 end to end so results hold to ~1e-6.  One
// wave handles one query row: lanes score 64 keys at a time against K rows
// read from LDS, the wave reduces max and sum with shuffles, and each lane
// accumulates the output dims d = lane and lane + 64.  Grouped heads read
// their KV head by address (g(a) = a / (Hq/Hkv)); nothing is copied.
#include "device_common.h"
#include "launch.h"

namespace gqa {

namespace {

constexpr int kKB = 64;  // keys per block

__device__ __forceinline__ float wave_max(float x)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
    return x;
}
__device__ __forceinline__ float wave_sum(float x)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

// Attends query row `qrow` (D floats) over keys [kbeg, kend) of one KV head.
// Keys j > last are masked.  Returns the un-normalised accumulators and the
// running max (natural-log units) and sum.
template <int D>
__device__ void attend_f32(const float *qrow, const float *kb, long long k_st, const float *vb,
                           long long v_st, int kbeg, int kend, float scale, float (&acc)[2],
                           float &m_run, float &l_run, float *sq, float *sk)
{
    const int lane = threadIdx.x & 63;
    for (int d = lane; d < D; d += 64) sq[d] = qrow[d];
    __syncthreads();
    acc[0] = acc[1] = 0.f;
    m_run = -INFINITY;
    l_run = 0.f;
    for (int k0 = kbeg; k0 < kend; k0 += kKB) {
        const int nk = min(kKB, kend - k0);
        // stage K rows of this block in LDS (row pitch D + 1 avoids bank aliasing)
        for (int idx = lane; idx < nk * D; idx += 64) {
            const int j = idx / D, d = idx % D;
            sk[j * (D + 1) + d] = kb[(size_t)(k0 + j) * k_st + d];
        }
        __syncthreads();
        float s = -INFINITY;
        if (lane < nk) {
            float dot = 0.f;
            for (int d = 0; d < D; ++d) dot = fmaf(sq[d], sk[lane * (D + 1) + d], dot);
            s = dot * scale;
        }
        const float mx = wave_max(s);
        const float m_new = fmaxf(m_run, mx);
        const float alpha = (m_run == -INFINITY) ? 0.f : expf(m_run - m_new);
        const float pj = (lane < nk) ? expf(s - m_new) : 0.f;
        l_run = l_run * alpha + wave_sum(pj);
        acc[0] *= alpha;
        acc[1] *= alpha;
        for (int j = 0; j < nk; ++j) {
            const float pb = __shfl(pj, j, 64);
            const float *vrow = vb + (size_t)(k0 + j) * v_st;
            acc[0] = fmaf(pb, vrow[lane], acc[0]);
            if (D > 64) acc[1] = fmaf(pb, vrow[lane + 64], acc[1]);
        }
        m_run = m_new;
        __syncthreads();
    }
}

template <int D>
__global__ __launch_bounds__(64) void fwd_f32_kernel(F32FwdArgs p)
{
    __shared__ float sq[D];
    __shared__ float sk[kKB * (D + 1)];
    debug_nanfill(sq);
    debug_nanfill(sk);
    const int i = blockIdx.x, a = blockIdx.y, b = blockIdx.z;
    const int g = a / p.G;
    const int lane = threadIdx.x;
    const int off = p.Tk - p.Tq;
    const int kend = p.causal ? min(p.Tk, off + i + 1) : p.Tk;
    const float *qrow = p.q + (((size_t)b * p.Hq + a) * p.Tq + i) * D;
    const float *kb = p.k + ((size_t)b * p.Hkv + g) * p.Tk * D;
    const float *vb = p.v + ((size_t)b * p.Hkv + g) * p.Tk * D;
    float acc[2], m, l;
    attend_f32<D>(qrow, kb, D, vb, D, 0, kend, p.scale, acc, m, l, sq, sk);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float *orow = p.out + (((size_t)b * p.Hq + a) * p.Tq + i) * D;
    orow[lane] = acc[0] * inv;
    if (D > 64) orow[lane + 64] = acc[1] * inv;
}

template <int D>
__global__ __launch_bounds__(64) void decode_f32_kernel(DecodeArgs p)
{
    __shared__ float sq[D];
    __shared__ float sk[kKB * (D + 1)];
    debug_nanfill(sq);
    debug_nanfill(sk);
    const int split = blockIdx.x, a = blockIdx.y, b = blockIdx.z;
    const int g = a / p.G;
    const int lane = threadIdx.x;
    int len = p.lens[b];
    len = len < 0 ? 0 : (len > p.Tmax ? p.Tmax : len);
    int kst = 0;  // sliding window: the last `window` keys only, rows kst ..
    if (p.window > 0 && len > p.window) {
        kst = len - p.window;
        len = p.window;
    }
    const int kbeg = split * p.chunk;
    const int kend = min(len, kbeg + p.chunk);
    const float *qrow = (const float *)p.q + ((size_t)b * p.Hq + a) * D;
    const float *kb = (const float *)p.k + (size_t)b * p.k_sb + (size_t)g * p.k_sh + (size_t)kst * p.k_st;
    const float *vb = (const float *)p.v + (size_t)b * p.v_sb + (size_t)g * p.v_sh + (size_t)kst * p.v_st;
    // p.c carries the plain scale for the fp32 path
    float acc[2], m, l;
    attend_f32<D>(qrow, kb, p.k_st, vb, p.v_st, kbeg, kend, p.c, acc, m, l, sq, sk);
    const size_t prow = ((size_t)b * p.Hq + a) * p.S + split;
    float *po = (float *)p.part_o + prow * D;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    po[lane] = acc[0] * inv;
    if (D > 64) po[lane + 64] = acc[1] * inv;
    if (lane == 0)
        p.part_lse[prow] = l > 0.f ? (m * 1.4426950408889634f + log2f(l)) : -INFINITY;
}

} // namespace

int launch_fwd_f32(const F32FwdArgs &a, int D, hipStream_t stream)
{
    dim3 grid(a.Tq, a.Hq, a.B), block(64);
    if (D == 64)
        hipLaunchKernelGGL(fwd_f32_kernel<64>, grid, block, 0, stream, a);
    else if (D == 128)
        hipLaunchKernelGGL(fwd_f32_kernel<128>, grid, block, 0, stream, a);
    else
        return -1;
    return 0;
}

int launch_decode_f32(const DecodeArgs &a, int D, hipStream_t stream)
{
    dim3 grid(a.S, a.Hq, a.B), block(64);
    if (D == 64)
        hipLaunchKernelGGL(decode_f32_kernel<64>, grid, block, 0, stream, a);
    else if (D == 128)
        hipLaunchKernelGGL(decode_f32_kernel<128>, grid, block, 0, stream, a);
    else
        return -1;
    return 0;
}

} // namespace gqa
