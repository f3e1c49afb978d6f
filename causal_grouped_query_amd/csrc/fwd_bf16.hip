// fwd_bf16.hip -- prefill / suffix forward of causal grouped-query attention
// on gfx950, bf16 storage with fp32 accumulation.
//
// Computes o_a = softmax(Q_a K_{g(a)}^T * scale + M) V_{g(a)} (the unified
// formula of the "Attention variants" page) with the query offset Tk - Tq of
// that page's minimal semantic implementation.  Execution follows the tiled,
// online-softmax scheme the pages credit to FlashAttention ("A Visual Guide to
// Attention", section on sources and execution): exact up to rounding, no
// Tq x Tk matrix in HBM.
//
// gfx950 design
//  * One workgroup = 4 waves = 128 query rows that all read ONE KV head:
//    Gt query heads of the group x Pt positions (Gt * Pt = 128).  Each K/V
//    tile is staged in LDS once and used by the whole group of heads; there
//    is no repeat_interleave copy, the head map g(a) = a / (Hq/Hkv) is pure
//    addressing.
//  * A wave owns 32 query rows.  Scores are computed transposed,
//    S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: Q^T sits in registers as the
//    B operand for the whole key loop, K rows come from LDS as the A operand.
//    In the accumulator every lane holds one query column, so row max and row
//    sum are in-lane plus a single exchange with lane l^32.
//  * O^T = V^T P^T: P^T needs no data movement (see kperm in
//    device_common.h); V is transposed into LDS while staging so the A
//    operand is one 16-byte LDS read.
//  * Online softmax in base 2: scale*log2(e) is folded into one FMA per
//    score, exp via v_exp_f32.
//  * Grid order: tiles of one (batch, KV head, head block) are consecutive
//    on one XCD (the dispatcher deals workgroups round-robin over 8 XCDs, so
//    the remap keeps a KV head's K/V in one L2), heaviest causal tiles first.
//  * K/V tiles are double-buffered through registers: the global loads of
//    tile i+1 are in flight while tile i is computed.
#include "device_common.h"
#include "launch.h"

namespace gqa {

namespace {

constexpr int kNW = 4;        // waves per workgroup
constexpr int kBN = 64;       // keys per tile
constexpr int kThreads = 64 * kNW;

template <int D>
struct FwdSmem {
    static constexpr int KP = D + 8;    // K row pitch (elements), breaks bank aliasing
    static constexpr int VP = kBN + 8;  // V^T row pitch (elements)
    uint16_t k[kBN * KP];
    uint16_t vt[D * VP];
};

template <int D>
__global__ __launch_bounds__(kThreads) void fwd_bf16_kernel(FwdArgs p)
{
    constexpr int KP = FwdSmem<D>::KP;
    constexpr int VP = FwdSmem<D>::VP;
    constexpr int KS = D / 16;                            // MFMA k-steps over the head dim
    constexpr int DT = D / 32;                            // 32-row tiles of O^T
    constexpr int KCH = kBN * D / 8;                      // 16-byte chunks per K tile
    constexpr int KPT = (KCH + kThreads - 1) / kThreads;  // chunks per thread
    constexpr int VBL = (kBN / 4) * (D / 8);              // 4x8 V blocks per tile
    constexpr int VPT = (VBL + kThreads - 1) / kThreads;  // blocks per thread

    __shared__ __attribute__((aligned(16))) FwdSmem<D> sm;

    // ---- workgroup -> (unit, query tile), XCD-aware, heaviest first ----
    const int nblk = gridDim.x;
    const int L = blockIdx.x;
    const int xcd = L & 7, r = L >> 3;
    const int per = nblk >> 3, rem = nblk & 7;
    const int Lp = (xcd < rem) ? xcd * (per + 1) + r : rem * (per + 1) + (xcd - rem) * per + r;
    const int unit = Lp / p.n_qt;
    const int qt = p.n_qt - 1 - (Lp - unit * p.n_qt);
    const int hblk = unit % p.n_hblk;
    const int bk = unit / p.n_hblk;  // b * Hkv + kv head
    const int kvh = bk % p.Hkv;
    const int b = bk / p.Hkv;

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int col = lane & 31, hi = lane >> 5;
    const int head = kvh * p.G + hblk * p.Gt + (w % p.Gt);
    const int q0 = qt * p.Pt + (w / p.Gt) * 32;  // first query index of this wave
    const int off = p.Tk - p.Tq;                 // absolute position of query 0
    const int qi = q0 + col;                     // this lane's query
    const bool wave_active = q0 < p.Tq;

    // keys the workgroup needs: [0, kend)
    int kend = p.Tk;
    if (p.causal) kend = min(p.Tk, off + min(p.Tq, qt * p.Pt + p.Pt));
    const int ntiles = (kend + kBN - 1) / kBN;
    // last key any row of this wave can see
    const int wlast = p.causal ? off + min(q0 + 31, p.Tq - 1) : p.Tk - 1;
    // last key this lane's query can see
    const int lim = p.causal ? min(off + qi, p.Tk - 1) : p.Tk - 1;

    const uint16_t *kbase = p.k + (size_t)bk * p.Tk * D;
    const uint16_t *vbase = p.v + (size_t)bk * p.Tk * D;

    // ---- Q^T in registers (B operand), zero for rows past Tq ----
    u32x4 qreg[KS];
    {
        const bool ok = wave_active && qi < p.Tq;
        const uint16_t *qrow = p.q + (((size_t)b * p.Hq + head) * p.Tq + (ok ? qi : 0)) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 z = {0u, 0u, 0u, 0u};
            qreg[ks] = ok ? *(const u32x4 *)(qrow + 16 * ks + 8 * hi) : z;
        }
    }

    f32x16 o[DT];
#pragma unroll
    for (int i = 0; i < DT; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[i][e] = 0.f;
    float m_run = -INFINITY;  // running max of scaled scores (log2 units)
    float l_run = 0.f;        // this lane's half of the running sum

    u32x4 kpre[KPT];
    u32x4 vpre[VPT][4];

    auto load_tile = [&](int k0) {
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int c = tid + i * kThreads;
            const int row = c / (D / 8), cc = c % (D / 8);
            u32x4 z = {0u, 0u, 0u, 0u};
            kpre[i] = (c < KCH && k0 + row < p.Tk)
                          ? *(const u32x4 *)(kbase + (size_t)(k0 + row) * D + cc * 8)
                          : z;
        }
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int vb = tid + i * kThreads;
            const int db = vb % (D / 8), kb = vb / (D / 8);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int key = k0 + 4 * kb + j;
                u32x4 z = {0u, 0u, 0u, 0u};
                vpre[i][j] = (vb < VBL && key < p.Tk)
                                 ? *(const u32x4 *)(vbase + (size_t)key * D + db * 8)
                                 : z;
            }
        }
    };

    auto store_tile = [&]() {
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int c = tid + i * kThreads;
            const int row = c / (D / 8), cc = c % (D / 8);
            if (c < KCH) *(u32x4 *)(&sm.k[row * KP + cc * 8]) = kpre[i];
        }
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int vb = tid + i * kThreads;
            const int db = vb % (D / 8), kb = vb / (D / 8);
            if (vb < VBL) {
                u32x2 t8[8];
                transpose4x8(vpre[i], t8);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    *(u32x2 *)(&sm.vt[(db * 8 + e) * VP + 4 * kb]) = t8[e];
            }
        }
    };

    const float c = p.c;
    if (ntiles > 0) load_tile(0);

    for (int it = 0; it < ntiles; ++it) {
        const int k0 = it * kBN;
        __syncthreads();  // everyone is done reading the previous tile
        store_tile();
        __syncthreads();
        if (it + 1 < ntiles) load_tile(k0 + kBN);
        if (!wave_active || k0 > wlast) continue;

        // ---- S^T = K Q^T for 64 keys (two 32-key tiles) ----
        f32x16 s[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
            for (int e = 0; e < 16; ++e) s[t][e] = 0.f;
            const uint16_t *krow = &sm.k[(32 * t + kperm(col)) * KP + 8 * hi];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                s[t] = mfma32x32x16(*(const u32x4 *)(krow + 16 * ks), qreg[ks], s[t]);
        }

        // ---- mask (diagonal and ragged tiles only) ----
        const bool need_mask = (p.causal && k0 + kBN - 1 > off + q0) || (k0 + kBN > p.Tk);
        if (need_mask) {
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    if (k0 + acc_key(t, e, hi) > lim) s[t][e] = -INFINITY;
        }

        // ---- online softmax (base 2) ----
        float mx = s[0][0];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[t][e]);
        mx = fmaxf(mx, wave_swap_half(mx));
        const float m_new = fmaxf(m_run, mx * c);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < DT; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) o[i][e] *= alpha;

        u32x4 pb[4];
        float psum = 0.f;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                float pv[8];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    pv[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][8 * h + e], c, -m_use));
                u32x4 pk;
                pk.x = pack_bf16x2(pv[0], pv[1]);
                pk.y = pack_bf16x2(pv[2], pv[3]);
                pk.z = pack_bf16x2(pv[4], pv[5]);
                pk.w = pack_bf16x2(pv[6], pv[7]);
                psum = sum_bf16x8(pk, psum);
                pb[2 * t + h] = pk;
            }
        }
        l_run += psum;

        // ---- O^T += V^T P^T ----
#pragma unroll
        for (int st = 0; st < 4; ++st) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const u32x4 va = *(const u32x4 *)(&sm.vt[(32 * dt + col) * VP + 16 * st + 8 * hi]);
                o[dt] = mfma32x32x16(va, pb[st], o[dt]);
            }
        }
    }

    if (!wave_active || qi >= p.Tq) return;
    const float l_tot = l_run + wave_swap_half(l_run);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t *orow = p.out + (((size_t)b * p.Hq + head) * p.Tq + qi) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int d = 32 * dt + 8 * j + 4 * hi;
            u32x2 pk;
            pk.x = pack_bf16x2(o[dt][4 * j + 0] * inv, o[dt][4 * j + 1] * inv);
            pk.y = pack_bf16x2(o[dt][4 * j + 2] * inv, o[dt][4 * j + 3] * inv);
            *(u32x2 *)(orow + d) = pk;
        }
    }
}

} // namespace

int launch_fwd_bf16(const FwdArgs &a, int D, hipStream_t stream)
{
    const long long nblk = (long long)a.n_units * a.n_qt;
    if (nblk <= 0 || nblk > 0x7fffffffLL) return -1;
    dim3 grid((unsigned)nblk), block(kThreads);
    if (D == 128)
        hipLaunchKernelGGL(fwd_bf16_kernel<128>, grid, block, 0, stream, a);
    else if (D == 64)
        hipLaunchKernelGGL(fwd_bf16_kernel<64>, grid, block, 0, stream, a);
    else
        return -1;
    return 0;
}

int fwd_bf16_rows_per_block() { return 32 * kNW; }

} // namespace gqa
