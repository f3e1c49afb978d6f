// f32_kernels.hip -- fp32 attention for small head dims (64, 128): the
// prefill/suffix forward and the split-KV decode partials, on the vector ALU.
//
// Same operation as the bf16 kernels (unified formula of the "Attention
// variants" page, query offset Tk - Tq of its minimal semantic
// implementation), kept in fp32 end to end so results hold to ~1e-6.
//
// The KV head is shared by its query group as in the bf16 kernels: a
// workgroup owns up to 32 query rows of ONE KV head -- Gt = min(G, 32) heads
// of the group times P = 32 / Gt consecutive positions (decode: the Gt heads
// of one position) -- and stages each 64-key K and V tile in LDS once for
// all of them.  Wave w takes rows w, w + 4, ...; for a row, lanes score the
// tile's keys (lane = key, the dot product over the LDS K row), the wave
// reduces max and sum with shuffles, and lane l accumulates output dims l
// and l + 64 from the LDS V rows.  Nothing is copied per query head.
#include "device_common.h"
#include "launch.h"

namespace gqa {

namespace {

constexpr int kKB = 64;           // keys per tile
constexpr int kRows = 32;         // query rows per workgroup
constexpr int kNW = 4;            // waves per workgroup
constexpr int kRW = kRows / kNW;  // rows per wave

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

template <int D>
struct F32Smem {
    float q[kRows][D];        // the workgroup's query rows
    float k[kKB][D + 1];      // K tile (row pitch D + 1: lane = key reads hit distinct banks)
    float v[kKB][D];          // V tile
};

// Rows of one workgroup over the keys [kb0, kb1) of one KV head (rows kb,
// vb, strides k_st, v_st).  Row r is valid if ok(r); its query is q_of(r)
// (D floats) and it sees the keys [first(r), last(r)].  Calls done(r, acc,
// m, l) with the un-normalised accumulators (dims lane, lane + 64), the
// running max (natural-log units) and sum.
template <int D, typename Ok, typename Q, typename First, typename Last, typename Done>
__device__ __forceinline__ void group_attend(F32Smem<D> &sm, const float *kb, long long k_st, const float *vb,
                                             long long v_st, int kb0, int kb1, float scale, Ok ok, Q q_of,
                                             First first, Last last, Done done)
{
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    for (int i = tid; i < kRows * D; i += 64 * kNW) {
        const int r = i / D, d = i % D;
        sm.q[r][d] = ok(r) ? q_of(r)[d] : 0.f;
    }
    float acc[kRW][2], m_run[kRW], l_run[kRW];
#pragma unroll
    for (int rr = 0; rr < kRW; ++rr) {
        acc[rr][0] = acc[rr][1] = 0.f;
        m_run[rr] = -INFINITY;
        l_run[rr] = 0.f;
    }
    constexpr int D4 = D / 4;
    for (int k0 = kb0; k0 < kb1; k0 += kKB) {
        const int nk = min(kKB, kb1 - k0);
        __syncthreads();  // the previous tile's readers are done (and the queries are staged)
        for (int i = tid; i < nk * D4; i += 64 * kNW) {
            const int j = i / D4, d = 4 * (i % D4);
            const float4 kv = *(const float4 *)(kb + (size_t)(k0 + j) * k_st + d);
            const float4 vv = *(const float4 *)(vb + (size_t)(k0 + j) * v_st + d);
            sm.k[j][d] = kv.x;
            sm.k[j][d + 1] = kv.y;
            sm.k[j][d + 2] = kv.z;
            sm.k[j][d + 3] = kv.w;
            *(float4 *)&sm.v[j][d] = vv;
        }
        __syncthreads();
#pragma unroll
        for (int rr = 0; rr < kRW; ++rr) {
            const int r = w + kNW * rr;
            if (!ok(r)) continue;
            const int lo = first(r), hi = last(r);
            if (k0 > hi || k0 + nk <= lo) continue;  // nothing of this tile is visible to the row
            const int key = k0 + lane;
            float s = -INFINITY;
            if (lane < nk && key >= lo && key <= hi) {
                float dot = 0.f;
#pragma unroll 8
                for (int d = 0; d < D; ++d) dot = fmaf(sm.q[r][d], sm.k[lane][d], dot);
                s = dot * scale;
            }
            const float mx = wave_max(s);
            const float m_new = fmaxf(m_run[rr], mx);
            const float alpha = (m_run[rr] == -INFINITY) ? 0.f : expf(m_run[rr] - m_new);
            const float pj = (s == -INFINITY) ? 0.f : expf(s - m_new);
            l_run[rr] = l_run[rr] * alpha + wave_sum(pj);
            acc[rr][0] *= alpha;
            acc[rr][1] *= alpha;
            for (int j = 0; j < nk; ++j) {
                const float pb = __shfl(pj, j, 64);
                acc[rr][0] = fmaf(pb, sm.v[j][lane], acc[rr][0]);
                if (D > 64) acc[rr][1] = fmaf(pb, sm.v[j][lane + 64], acc[rr][1]);
            }
            m_run[rr] = m_new;
        }
    }
#pragma unroll
    for (int rr = 0; rr < kRW; ++rr) {
        const int r = w + kNW * rr;
        if (ok(r)) done(r, acc[rr], m_run[rr], l_run[rr]);
    }
}

// grid (query tiles of P positions, Hkv * n_hblk, B)
template <int D>
__global__ __launch_bounds__(64 * kNW) void fwd_f32_kernel(F32FwdArgs p)
{
    __shared__ F32Smem<D> sm;
    debug_nanfill(sm);
    const int qt = blockIdx.x, b = blockIdx.z;
    const int kvh = blockIdx.y / p.n_hblk, hblk = blockIdx.y % p.n_hblk;
    const int lane = threadIdx.x & 63;
    const int Gt = p.Gt, P = p.P;
    const int off = p.Tk - p.Tq;
    auto head_of = [&](int r) { return kvh * p.G + hblk * Gt + r % Gt; };
    auto pos_of = [&](int r) { return qt * P + r / Gt; };
    auto ok = [&](int r) { return r < Gt * P && hblk * Gt + r % Gt < p.G && pos_of(r) < p.Tq; };
    auto q_of = [&](int r) { return p.q + (((size_t)b * p.Hq + head_of(r)) * p.Tq + pos_of(r)) * D; };
    auto first = [&](int) { return 0; };
    auto last = [&](int r) { return p.causal ? min(off + pos_of(r), p.Tk - 1) : p.Tk - 1; };
    const int maxpos = min(p.Tq - 1, qt * P + P - 1);
    const int kb1 = p.causal ? max(0, min(p.Tk, off + maxpos + 1)) : p.Tk;
    const float *kb = p.k + ((size_t)b * p.Hkv + kvh) * p.Tk * D;
    const float *vb = p.v + ((size_t)b * p.Hkv + kvh) * p.Tk * D;
    group_attend<D>(sm, kb, D, vb, D, 0, kb1, p.scale, ok, q_of, first, last,
                    [&](int r, const float (&acc)[2], float, float l) {
                        const float inv = l > 0.f ? 1.f / l : 0.f;
                        float *orow = p.out + (((size_t)b * p.Hq + head_of(r)) * p.Tq + pos_of(r)) * D;
                        orow[lane] = acc[0] * inv;
                        if (D > 64) orow[lane + 64] = acc[1] * inv;
                    });
}

// grid (S, Hkv * n_hblk, B): the Gt heads of a head block, one key chunk
template <int D>
__global__ __launch_bounds__(64 * kNW) void decode_f32_kernel(DecodeArgs p)
{
    __shared__ F32Smem<D> sm;
    debug_nanfill(sm);
    const int split = blockIdx.x, b = blockIdx.z;
    const int kvh = blockIdx.y / p.n_hblk, hblk = blockIdx.y % p.n_hblk;
    const int lane = threadIdx.x & 63;
    const int Gt = min(p.G, kRows);
    int len = p.lens[b];
    len = len < 0 ? 0 : (len > p.Tmax ? p.Tmax : len);
    int kst = 0;  // sliding window: the last `window` keys only, rows kst ..
    if (p.window > 0 && len > p.window) {
        kst = len - p.window;
        len = p.window;
    }
    const int kbeg = split * p.chunk;
    const int kend = min(len, kbeg + p.chunk);
    auto head_of = [&](int r) { return kvh * p.G + hblk * Gt + r; };
    auto ok = [&](int r) { return r < Gt && hblk * Gt + r < p.G; };
    auto q_of = [&](int r) { return (const float *)p.q + ((size_t)b * p.Hq + head_of(r)) * D; };
    auto first = [&](int) { return 0; };
    auto last = [&](int) { return kend - 1; };
    const float *kb = (const float *)p.k + (size_t)b * p.k_sb + (size_t)kvh * p.k_sh + (size_t)kst * p.k_st;
    const float *vb = (const float *)p.v + (size_t)b * p.v_sb + (size_t)kvh * p.v_sh + (size_t)kst * p.v_st;
    // p.c carries the plain scale for the fp32 path
    group_attend<D>(sm, kb, p.k_st, vb, p.v_st, kbeg, kend, p.c, ok, q_of, first, last,
                    [&](int r, const float (&acc)[2], float m, float l) {
                        const size_t prow = ((size_t)b * p.Hq + head_of(r)) * p.S + split;
                        float *po = (float *)p.part_o + prow * D;
                        const float inv = l > 0.f ? 1.f / l : 0.f;
                        po[lane] = acc[0] * inv;
                        if (D > 64) po[lane + 64] = acc[1] * inv;
                        if (lane == 0)
                            p.part_lse[prow] = l > 0.f ? (m * 1.4426950408889634f + log2f(l)) : -INFINITY;
                    });
}

} // namespace

// query rows of one workgroup: Gt heads of a group x P positions; P halves
// (down to 1) while the grid would have fewer than 512 workgroups, so a
// small problem still spreads over the device
static void f32_row_blocks(int G, int &Gt, int &P, int &n_hblk, long long positions = 1)
{
    Gt = G < kRows ? G : kRows;
    P = kRows / Gt;
    n_hblk = (G + Gt - 1) / Gt;
    while (P > 1 && positions * n_hblk / P < 512) P /= 2;
}

int launch_fwd_f32(const F32FwdArgs &a_in, int D, hipStream_t stream)
{
    F32FwdArgs a = a_in;
    f32_row_blocks(a.G, a.Gt, a.P, a.n_hblk, (long long)a.B * a.Hkv * a.Tq);
    const long long ny = (long long)a.Hkv * a.n_hblk;
    if (ny > 65535 || a.B > 65535) return -1;
    dim3 grid((unsigned)((a.Tq + a.P - 1) / a.P), (unsigned)ny, a.B), block(64 * kNW);
    if (D == 64)
        hipLaunchKernelGGL(fwd_f32_kernel<64>, grid, block, 0, stream, a);
    else if (D == 128)
        hipLaunchKernelGGL(fwd_f32_kernel<128>, grid, block, 0, stream, a);
    else
        return -1;
    return 0;
}

int launch_decode_f32(const DecodeArgs &a_in, int D, hipStream_t stream)
{
    DecodeArgs a = a_in;
    int Gt, P;
    f32_row_blocks(a.G, Gt, P, a.n_hblk);
    const long long ny = (long long)a.Hkv * a.n_hblk;
    if (ny > 65535 || a.B > 65535 || a.S > 0x7fffffff) return -1;
    dim3 grid(a.S, (unsigned)ny, a.B), block(64 * kNW);
    if (D == 64)
        hipLaunchKernelGGL(decode_f32_kernel<64>, grid, block, 0, stream, a);
    else if (D == 128)
        hipLaunchKernelGGL(decode_f32_kernel<128>, grid, block, 0, stream, a);
    else
        return -1;
    return 0;
}

} // namespace gqa
