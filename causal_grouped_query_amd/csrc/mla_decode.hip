// mla_decode.hip -- split-KV decode partials for the weight-absorbed MLA
// shape on gfx950: MQA over a shared 576-wide latent key (512 latent + 64
// rope dims) whose first 512 columns are the value ("Attention Architecture
// Evolution", MLA section and the absorbed score / value equations of its
// DSA section: the score is q_C' c_KV^T + q_R k_R^T, i.e. one 576-wide dot,
// and the output aggregates c_KV itself).
//
// A workgroup owns 128 query heads of one sequence and one key chunk; the
// key tile (32 keys x 576) is copied HBM -> LDS once with global_load_lds
// into a 3-deep ring and read by all 8 waves.  The per-wave register budget
// is the problem this layout solves: one wave holding Q^T for 32 heads over
// 576 dims (144 VGPRs) and O^T over 512 dims (256 accumulators) does not fit.
// Instead wave w = (head group hg = w & 3, half = w >> 2):
//   * computes the partial scores of its 32 heads over dims
//     [288*half, 288*half + 288) with v_mfma_f32_32x32x16_bf16 (18 steps),
//   * swaps partial scores with its partner wave (same heads, other half)
//     through LDS and adds them (both waves then hold the same full scores),
//   * runs the online softmax (identical in both waves),
//   * accumulates O^T for output dims [256*half, 256*half + 256) from V^T
//     transpose reads (ds_read_b64_tr_b16) of the same LDS key tile.
// Partial outputs and log-sum-exp values go to the workspace exactly as for
// the other decode kernels; combine.hip merges them.
#include "device_common.h"
#include "launch.h"

namespace gqa {

namespace {

constexpr int kTK = 32;      // keys per tile
constexpr int kDK = 576;     // key width (latent 512 + rope 64)
constexpr int kDV = 512;     // value width (the latent)
constexpr int kNW = 8;       // waves per workgroup
constexpr int kNT = 64 * kNW;
constexpr int kStages = 3;
#ifndef GQA_MLA_PREFETCH
#define GQA_MLA_PREFETCH 0  // LDS operand reads kept in flight ahead of the MFMAs (spills if > 0)
#endif
constexpr int kCPR = kDK / 8;              // 72 16-byte chunks per key row
constexpr int kKSH = kDK / 16 / 2;         // 18 MFMA k-steps per half
constexpr int kDTH = kDV / 32 / 2;         // 8 output tiles per half
static_assert(kTK * kCPR % 64 == 0, "tile is whole wave copies");

struct MlaSmem {
    uint16_t k[kStages][kTK * kDK];
    float xs[kNW][16 * 64];  // partial-score exchange, one f32x16 per lane per wave
};

__global__ __launch_bounds__(kNT, 2) void mla_decode_kernel(DecodeArgs p)
{
    constexpr int NCOPY = kTK * kCPR / 64;  // 36 wave-copies per tile, spread over 8 waves
    __shared__ __attribute__((aligned(1024))) MlaSmem sm;

    // chunk-major order, as in the other decode kernel
    const int nbk = p.B * p.Hkv;
    const int split = blockIdx.x / nbk;
    const int bk = blockIdx.x - split * nbk;  // b * Hkv + kv head
    const int hblk = blockIdx.y;
    const int kvh = bk % p.Hkv, b = bk / p.Hkv;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int col = lane & 31, hi = lane >> 5;
    const int hg = w & 3, half = w >> 2;
    const int hh = hblk * 128 + hg * 32 + col;  // head within the group
    const bool head_ok = hh < p.G;
    const int head = kvh * p.G + (head_ok ? hh : 0);

    int len = p.lens[b];
    len = len < 0 ? 0 : (len > p.Tmax ? p.Tmax : len);
    const int kbeg = split * p.chunk;
    const int kend = min(len, kbeg + p.chunk);
    const int ntiles = kend > kbeg ? (kend - kbeg + kTK - 1) / kTK : 0;

    const uint16_t *kb = (const uint16_t *)p.k + (size_t)b * p.k_sb + (size_t)kvh * p.k_sh;

    // wave copy j covers LDS chunks [64 j, 64 j + 64); waves take j = w, w + 8, ...
    // (36 copies: waves 0-3 do 5, waves 4-7 do 4; the count per wave is fixed)
    const int my_copies = (NCOPY - w + kNW - 1) / kNW;
    using Tile = PlaneTile<kTK>;
    auto issue_tile = [&](int k0, int slot) {
        for (int j = w; j < NCOPY; j += kNW) {
            int row, chunk;
            Tile::slot_source(j * 64 + lane, row, chunk);
            g2lds16(kb + (size_t)min(k0 + row, kend - 1) * p.k_st + chunk * 8, &sm.k[slot][j * 64 * 8]);
        }
    };

    // Q^T for this wave's heads over its half of the key dims
    u32x4 qreg[kKSH];
    {
        const uint16_t *qrow = (const uint16_t *)p.q + ((size_t)b * p.Hq + head) * kDK + 288 * half;
#pragma unroll
        for (int ks = 0; ks < kKSH; ++ks) {
            u32x4 z = {0u, 0u, 0u, 0u};
            qreg[ks] = head_ok ? *(const u32x4 *)(qrow + 16 * ks + 8 * hi) : z;
        }
#pragma unroll
        for (int ks = 0; ks < kKSH; ++ks) hold_reg(qreg[ks]);
    }

    f32x16 o[kDTH];
#pragma unroll
    for (int i = 0; i < kDTH; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[i][e] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    const int krow = kperm(col);
    const int kbase_even = Tile::offset(krow, hi);
    const int kbase_odd = Tile::offset(krow, 2 + hi);
    const int vg = lane >> 4, vi = lane & 15;
    const int vrow = 8 * (vg >> 1) + (vi >> 2), vchunk = 2 * (vg & 1) + ((vi >> 1) & 1);
    const int vb_h0 = Tile::offset(vrow, vchunk) + 8 * (vi & 1);      // rows 16 st + vrow
    const int vb_h1 = Tile::offset(vrow + 4, vchunk) + 8 * (vi & 1);  // rows 16 st + vrow + 4
    float *xs_mine = &sm.xs[w][0];
    const float *xs_peer = &sm.xs[w ^ 4][0];

#pragma unroll
    for (int s = 0; s < kStages - 1; ++s)
        if (s < ntiles) issue_tile(kbeg + s * kTK, s);

    const float c = p.c;
    for (int it = 0; it < ntiles; ++it) {
        const int k0 = kbeg + it * kTK;
        const int slot = it % kStages;
        // tile `it` must have landed; the next tile's copies may still fly
        if (it + kStages - 2 < ntiles) {
            if (my_copies == 5)
                wait_vmem_le<5>();
            else
                wait_vmem_le<4>();
        } else {
            wait_vmem();
        }
        lds_barrier();  // tile visible; the previous slot and exchange buffers are free
        if (it + kStages - 1 < ntiles) issue_tile(k0 + (kStages - 1) * kTK, (it + kStages - 1) % kStages);

        const char *ks_ = (const char *)sm.k[slot];
        f32x16 s;
#pragma unroll
        for (int e = 0; e < 16; ++e) s[e] = 0.f;
#pragma unroll
        for (int ks = 0; ks < kKSH; ++ks) {
            // chunk 36 half + 2 ks + hi lives in plane 9 half + ks / 2
            const int off_ = ((ks & 1) ? kbase_odd : kbase_even) + (9 * half + (ks >> 1)) * Tile::PLANE_BYTES;
            s = mfma32x32x16(*(const u32x4 *)(ks_ + off_), qreg[ks], s);
        }
#if GQA_MLA_PREFETCH
        // keep GQA_MLA_PREFETCH operand reads in flight ahead of the MFMAs
        __builtin_amdgcn_sched_group_barrier(0x100, GQA_MLA_PREFETCH, 0);
#pragma unroll
        for (int i = 0; i < kKSH - GQA_MLA_PREFETCH; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, GQA_MLA_PREFETCH, 0);
#endif
        // swap partial scores with the partner wave (same heads, other half)
#pragma unroll
        for (int e = 0; e < 16; e += 4) {
            f32x4 v4 = {s[e], s[e + 1], s[e + 2], s[e + 3]};
            *(f32x4 *)(xs_mine + e * 64 + 4 * lane) = v4;
        }
        lds_barrier();
#pragma unroll
        for (int e = 0; e < 16; e += 4) {
            // (fp addition commutes, so both waves get bit-identical sums)
            const f32x4 v4 = *(const f32x4 *)(xs_peer + e * 64 + 4 * lane);
            s[e] += v4[0];
            s[e + 1] += v4[1];
            s[e + 2] += v4[2];
            s[e + 3] += v4[3];
        }

        if (k0 + kTK > kend) {
#pragma unroll
            for (int e = 0; e < 16; ++e)
                if (k0 + acc_key(0, e, hi) >= kend) s[e] = -INFINITY;
        }

        float mx = s[0];
#pragma unroll
        for (int e = 1; e < 16; ++e) mx = fmaxf(mx, s[e]);
        mx = halves_max(mx);
        const float mt = mx * c;
        if (__any(mt > m_run + 8.0f)) {
            const float m_new = (mt > m_run + 8.0f) ? mt : m_run;
            const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int i = 0; i < kDTH; ++i)
#pragma unroll
                for (int e = 0; e < 16; ++e) o[i][e] *= alpha;
        }
        const float m_use = (m_run == -INFINITY) ? 0.f : m_run;

        u32x4 pb[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            float pv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                pv[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * h + e], c, -m_use));
            pb[h].x = pack_bf16x2(pv[0], pv[1]);
            pb[h].y = pack_bf16x2(pv[2], pv[3]);
            pb[h].z = pack_bf16x2(pv[4], pv[5]);
            pb[h].w = pack_bf16x2(pv[6], pv[7]);
            l_run = sum_bf16x8(pb[h], l_run);
        }

        // O^T (this half's 256 dims) += V^T P^T, V^T = transpose of the latent
        // prefix: output dims 256 half + 32 dt + ... live in plane 8 half + dt
#pragma unroll
        for (int st = 0; st < 2; ++st) {
#pragma unroll
            for (int dt = 0; dt < kDTH; ++dt) {
                const int o_ = (8 * half + dt) * Tile::PLANE_BYTES + 16 * st * 64;
                const u32x2 lo = lds_read_tr16(ks_ + vb_h0 + o_);
                const u32x2 hv = lds_read_tr16(ks_ + vb_h1 + o_);
                u32x4 va = {lo.x, lo.y, hv.x, hv.y};
                o[dt] = mfma32x32x16(va, pb[st], o[dt]);
            }
        }
#if GQA_MLA_PREFETCH
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * GQA_MLA_PREFETCH, 0);
#pragma unroll
        for (int i = 0; i < 2 * kDTH - GQA_MLA_PREFETCH; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, GQA_MLA_PREFETCH, 0);
#endif
    }

    if (!head_ok) return;
    const float l_tot = halves_sum(l_run);
    const size_t prow = ((size_t)b * p.Hq + head) * p.S + split;
    float *po = p.part_o + prow * kDV + 256 * half;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
    for (int dt = 0; dt < kDTH; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f32x4 v4 = {o[dt][4 * j] * inv, o[dt][4 * j + 1] * inv, o[dt][4 * j + 2] * inv,
                        o[dt][4 * j + 3] * inv};
            *(f32x4 *)(po + 32 * dt + 8 * j + 4 * hi) = v4;
        }
    if (half == 0 && hi == 0) p.part_lse[prow] = l_tot > 0.f ? m_run + __log2f(l_tot) : -INFINITY;
}

} // namespace

int launch_mla_decode(const DecodeArgs &a, hipStream_t stream)
{
    dim3 grid(a.S * a.B * a.Hkv, a.n_hblk), block(kNT);
    hipLaunchKernelGGL(mla_decode_kernel, grid, block, 0, stream, a);
    return 0;
}

} // namespace gqa
