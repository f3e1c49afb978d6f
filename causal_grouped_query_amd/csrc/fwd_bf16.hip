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
//    device_common.h); V stays row-major in LDS and its transposed A operand
//    comes from two ds_read_b64_tr_b16 per MFMA.
//  * K and V tiles go straight from HBM to LDS with global_load_lds (no
//    registers, no VALU), into a double-buffered, XOR-swizzled ring: tile
//    i+1 is in flight while tile i is computed; one barrier per tile.
//  * Online softmax in base 2: scale*log2(e) is folded into one FMA per
//    score, exp via v_exp_f32, the row sum via v_dot2 over the bf16-rounded
//    weights.  The running max is only moved (and O rescaled) when a tile's
//    max exceeds it by more than 2^8; weights then stay <= 256, which fp32
//    and bf16 hold exactly as well as weights <= 1, and the result is the
//    same softmax.
//  * Grid order: tiles of one (batch, KV head, head block) are consecutive
//    on one XCD (the dispatcher deals workgroups round-robin over 8 XCDs, so
//    the remap keeps a KV head's K/V in one L2), heaviest causal tiles first.
#include "device_common.h"
#include "launch.h"

namespace gqa {

namespace {

constexpr int kNW = 4;        // waves per workgroup
constexpr int kBN = 64;       // keys per tile
constexpr int kThreads = 64 * kNW;

template <int D>
struct FwdSmem {
    static constexpr int TILE = kBN * D;  // elements of one K or V tile (swizzled, unpadded)
    uint16_t k[2][TILE];
    uint16_t v[2][TILE];
};

template <int D>
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_kernel(FwdArgs p)
{
    constexpr int CPR = D / 8;                     // 16-byte chunks per row
    constexpr int KS = D / 16;                     // MFMA k-steps over the head dim
    constexpr int DT = D / 32;                     // 32-row tiles of O^T
    constexpr int NINS = kBN * CPR / kThreads;     // async copies per thread per tensor
    static_assert(kBN * CPR % kThreads == 0, "tile must split evenly over the workgroup");

    __shared__ __attribute__((aligned(1024))) FwdSmem<D> sm;

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

    // Async copy of keys [k0, k0 + 64) of K and V into ring slot `buf`.  LDS
    // chunk Lc = row * CPR + slot holds global chunk slot ^ swz(row); rows
    // past Tk re-read row Tk - 1 (in bounds; those keys are masked).
    auto issue_tile = [&](int k0, int buf) {
#pragma unroll
        for (int j = 0; j < NINS; ++j) {
            const int base = (j * kNW + w) * 64;  // first LDS chunk of this wave's copy
            const int Lc = base + lane;
            const int row = Lc / CPR, slot = Lc % CPR;
            const int c = slot ^ swz<CPR>(row);
            const size_t grow = (size_t)min(k0 + row, p.Tk - 1) * D + c * 8;
            g2lds16(kbase + grow, &sm.k[buf][base * 8]);
            g2lds16(vbase + grow, &sm.v[buf][base * 8]);
        }
    };

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
    float m_run = -INFINITY;  // running reference max of scaled scores (log2 units)
    float l_run = 0.f;        // this lane's half of the running sum

    // per-lane LDS offsets (elements) that do not depend on the tile
    int koff[2][KS];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int rr = 32 * t + kperm(col);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) koff[t][ks] = rr * D + (((2 * ks + hi) ^ swz<CPR>(rr)) * 8);
    }
    // V^T operand through transpose reads: lane = 16 g + i points at row
    // 16 st + 8 (g >> 1) + 4 h + (i >> 2), columns 32 dt + 16 (g & 1) + 4 (i & 3)
    const int vg = lane >> 4, vi = lane & 15;
    int voff[4][2];  // [st][h], column part added per dt
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int h = 0; h < 2; ++h) voff[st][h] = 16 * st + 8 * (vg >> 1) + 4 * h + (vi >> 2);

    const float c = p.c;
    if (ntiles > 0) issue_tile(0, 0);
    wait_vmem();
    __syncthreads();

    for (int it = 0; it < ntiles; ++it) {
        const int k0 = it * kBN;
        const int buf = it & 1;
        if (it + 1 < ntiles) issue_tile(k0 + kBN, buf ^ 1);

        if (wave_active && k0 <= wlast) {
            const uint16_t *ks_ = sm.k[buf];
            const uint16_t *vs_ = sm.v[buf];

            // ---- S^T = K Q^T for 64 keys (two 32-key tiles) ----
            f32x16 s[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
#pragma unroll
                for (int e = 0; e < 16; ++e) s[t][e] = 0.f;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    s[t] = mfma32x32x16(*(const u32x4 *)(ks_ + koff[t][ks]), qreg[ks], s[t]);
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

            // ---- online softmax (base 2, lazily rescaled) ----
            float mx = s[0][0];
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[t][e]);
            mx = fmaxf(mx, wave_swap_half(mx));
            const float mt = mx * c;
            if (__any(mt > m_run + 8.0f)) {
                // only lanes whose own max crossed the threshold move their
                // reference, so a row never depends on keys it cannot see
                const float m_new = (mt > m_run + 8.0f) ? mt : m_run;
                const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
                m_run = m_new;
                l_run *= alpha;
#pragma unroll
                for (int i = 0; i < DT; ++i)
#pragma unroll
                    for (int e = 0; e < 16; ++e) o[i][e] *= alpha;
            }
            const float m_use = (m_run == -INFINITY) ? 0.f : m_run;

            u32x4 pb[4];
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
                    l_run = sum_bf16x8(pk, l_run);
                    pb[2 * t + h] = pk;
                }
            }

            // ---- O^T += V^T P^T ----
#pragma unroll
            for (int st = 0; st < 4; ++st) {
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const int cb = 32 * dt + 16 * (vg & 1) + 4 * (vi & 3);  // column of this lane's chunk
                    u32x2 lo, hi2;
                    {
                        const int row = voff[st][0];
                        lo = lds_read_tr16(vs_ + row * D + (((cb >> 3) ^ swz<CPR>(row)) * 8) + (cb & 7));
                    }
                    {
                        const int row = voff[st][1];
                        hi2 = lds_read_tr16(vs_ + row * D + (((cb >> 3) ^ swz<CPR>(row)) * 8) + (cb & 7));
                    }
                    u32x4 va = {lo.x, lo.y, hi2.x, hi2.y};
                    o[dt] = mfma32x32x16(va, pb[st], o[dt]);
                }
            }
        }
        wait_vmem();
        __syncthreads();  // tile it+1 landed; everyone is done with slot `buf`
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
