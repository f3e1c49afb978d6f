// decode_bf16.hip -- split-KV single-token decode partials for grouped-query
// attention on gfx950 (bf16 storage, fp32 accumulation).
//
// Decode reads the whole KV stream once per step and is bound by that read
// ("Linear Attention and Sparse Attention" survey, 6.2 on decode; "Attention
// Architecture Evolution", Full Attention section).  The key axis of every
// sequence is cut into S chunks; each workgroup computes one chunk for all
// the query heads of one KV head (the GQA group shares the K/V tile in LDS),
// and writes a normalised partial output plus its log-sum-exp.  A second
// kernel (combine.hip) merges the S partials exactly (online-softmax merge,
// "A Visual Guide to Attention", section on sources and execution).
//
// Layout in a workgroup: NW waves, wave w owns query heads
// 32*(NW*hblk + w) + (0..31) of the group (columns of the MFMA, zero-padded
// when the group is smaller).  Scores are S^T = K Q^T (32 keys x 32 heads per
// v_mfma_f32_32x32x16_bf16), O^T = V^T P^T as in the prefill kernel.
// K/V tiles of 32 keys stream HBM -> LDS through global_load_lds into a
// STAGES-deep ring (STAGES-1 tiles in flight while one is computed); V^T
// comes from ds_read_b64_tr_b16.  (The absorbed-MLA shape has its own kernel,
// mla_decode.hip, whose register budget needs a different wave layout.)
#include "device_common.h"
#include "launch.h"

namespace gqa {

namespace {

constexpr int kTK = 32;  // keys per tile
#ifndef GQA_DEC_STAGES
#define GQA_DEC_STAGES 2  // K/V ring depth for the 128-dim kernel
#endif

template <int DK, int DV, int STAGES>
struct DecSmem {
    uint16_t k[STAGES][kTK * DK];
    uint16_t v[STAGES][kTK * DV];
};

template <int DK, int DV, int NW, int STAGES>
__global__ __launch_bounds__(64 * NW, (DK <= 128 ? 2 : 1)) void decode_bf16_kernel(DecodeArgs p)
{
    constexpr int NT = 64 * NW;
    constexpr int CPRK = DK / 8, CPRV = DV / 8;
    constexpr int KS = DK / 16;
    constexpr int DT = DV / 32;
    constexpr int KINS = kTK * CPRK / NT;                  // async copies per thread, K tile
    constexpr int VINS = kTK * CPRV / NT;                  // and V tile
    constexpr int NI = KINS + VINS;                        // vmem ops per thread per tile
    static_assert(kTK * CPRK % NT == 0 && kTK * CPRV % NT == 0, "tile must split evenly");
    static_assert(STAGES >= 2 && (STAGES - 2) * NI < 64, "ring depth");

    __shared__ __attribute__((aligned(1024))) DecSmem<DK, DV, STAGES> sm;

    // chunk-major order: every sequence's first chunk is dispatched before
    // any second chunk, so full chunks start first and the short / empty
    // ones of ragged lengths fill the tail
    const int nbk = p.B * p.Hkv;
    const int split = blockIdx.x / nbk;
    const int bk = blockIdx.x - split * nbk;  // b * Hkv + kv head
    const int hblk = blockIdx.y;
    const int kvh = bk % p.Hkv, b = bk / p.Hkv;

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31, hi = lane >> 5;
    const int hh = (hblk * NW + w) * 32 + col;  // head within the group
    const bool head_ok = hh < p.G;
    const int head = kvh * p.G + (head_ok ? hh : 0);

    int len = p.lens[b];
    len = len < 0 ? 0 : (len > p.Tmax ? p.Tmax : len);
    const int kbeg = split * p.chunk;
    const int kend = min(len, kbeg + p.chunk);
    const int ntiles = kend > kbeg ? (kend - kbeg + kTK - 1) / kTK : 0;

    const uint16_t *kb = (const uint16_t *)p.k + (size_t)b * p.k_sb + (size_t)kvh * p.k_sh;
    const uint16_t *vb = (const uint16_t *)p.v + (size_t)b * p.v_sb + (size_t)kvh * p.v_sh;

    // Async copy of keys [k0, k0 + 32) into ring slot `slot` (plane layout,
    // see PlaneTile); rows past the chunk end re-read its last key (in
    // bounds; masked below).
    using Tile = PlaneTile<kTK>;
    // per-lane byte offsets of each copy's source inside a tile (row, chunk)
    int krow_[KINS], vrow_[VINS];
    unsigned koff_[KINS], voff_[VINS];
#pragma unroll
    for (int j = 0; j < KINS; ++j) {
        int row, chunk;
        Tile::slot_source((j * NW + w) * 64 + lane, row, chunk);
        krow_[j] = row;
        koff_[j] = (unsigned)(row * p.k_st + chunk * 8) * 2u;
    }
#pragma unroll
    for (int j = 0; j < VINS; ++j) {
        int row, chunk;
        Tile::slot_source((j * NW + w) * 64 + lane, row, chunk);
        vrow_[j] = row;
        voff_[j] = (unsigned)(row * p.v_st + chunk * 8) * 2u;
    }
    auto issue_tile = [&](int k0, int slot) {
        if (k0 + kTK <= kend) {
            const uint16_t *k0p = kb + (size_t)k0 * p.k_st;
            const uint16_t *v0p = vb + (size_t)k0 * p.v_st;
#pragma unroll
            for (int j = 0; j < KINS; ++j) g2lds16(k0p, koff_[j], &sm.k[slot][(j * NW + w) * 64 * 8]);
#pragma unroll
            for (int j = 0; j < VINS; ++j) g2lds16(v0p, voff_[j], &sm.v[slot][(j * NW + w) * 64 * 8]);
        } else {
            // ragged last tile: rows past the chunk end re-read its last key
            // (in bounds; masked below)
#pragma unroll
            for (int j = 0; j < KINS; ++j) {
                const int row = min(k0 + krow_[j], kend - 1);
                g2lds16((const char *)(kb + (size_t)row * p.k_st) + (koff_[j] - (unsigned)(krow_[j] * p.k_st) * 2u),
                        &sm.k[slot][(j * NW + w) * 64 * 8]);
            }
#pragma unroll
            for (int j = 0; j < VINS; ++j) {
                const int row = min(k0 + vrow_[j], kend - 1);
                g2lds16((const char *)(vb + (size_t)row * p.v_st) + (voff_[j] - (unsigned)(vrow_[j] * p.v_st) * 2u),
                        &sm.v[slot][(j * NW + w) * 64 * 8]);
            }
        }
    };

    u32x4 qreg[KS];
    {
        const uint16_t *qrow = (const uint16_t *)p.q + ((size_t)b * p.Hq + head) * DK;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 z = {0u, 0u, 0u, 0u};
            qreg[ks] = head_ok ? *(const u32x4 *)(qrow + 16 * ks + 8 * hi) : z;
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) hold_reg(qreg[ks]);
    }

    f32x16 o[DT];
#pragma unroll
    for (int i = 0; i < DT; ++i)
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

    // prologue: fill all but one ring slot
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
        if (s < ntiles) issue_tile(kbeg + s * kTK, s);

    const float c = p.c;
    for (int it = 0; it < ntiles; ++it) {
        const int k0 = kbeg + it * kTK;
        const int slot = it % STAGES;
        if (it + STAGES - 2 < ntiles)
            wait_vmem_le<(STAGES - 2) * NI>();  // tile `it` landed, later ones may fly
        else
            wait_vmem();
        lds_barrier();  // tile visible to all waves; slot of tile it-1 is free
        if (it + STAGES - 1 < ntiles) issue_tile(k0 + (STAGES - 1) * kTK, (it + STAGES - 1) % STAGES);

        const char *ks_ = (const char *)sm.k[slot];
        f32x16 s;
#pragma unroll
        for (int e = 0; e < 16; ++e) s[e] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int off_ = ((ks & 1) ? kbase_odd : kbase_even) + (ks >> 1) * Tile::PLANE_BYTES;
            s = mfma32x32x16(*(const u32x4 *)(ks_ + off_), qreg[ks], s);
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

        // O^T += V^T P^T; V^T via transpose reads of the V tile
        const char *vs_ = (const char *)sm.v[slot];
#pragma unroll
        for (int st = 0; st < 2; ++st) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const int o_ = dt * Tile::PLANE_BYTES + 16 * st * 64;
                const u32x2 lo = lds_read_tr16(vs_ + vb_h0 + o_);
                const u32x2 hv = lds_read_tr16(vs_ + vb_h1 + o_);
                u32x4 va = {lo.x, lo.y, hv.x, hv.y};
                o[dt] = mfma32x32x16(va, pb[st], o[dt]);
            }
        }
    }

    if (!head_ok) return;
    const float l_tot = halves_sum(l_run);
    const size_t prow = ((size_t)b * p.Hq + head) * p.S + split;
    float *po = p.part_o + prow * DV;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f32x4 v4 = {o[dt][4 * j] * inv, o[dt][4 * j + 1] * inv, o[dt][4 * j + 2] * inv,
                        o[dt][4 * j + 3] * inv};
            *(f32x4 *)(po + 32 * dt + 8 * j + 4 * hi) = v4;
        }
    // empty chunk: o = 0 and lse = -inf, so it weighs nothing in the merge
    if (hi == 0) p.part_lse[prow] = l_tot > 0.f ? m_run + __log2f(l_tot) : -INFINITY;
}

template <int DK, int DV, int NW, int STAGES>
int launch_one(const DecodeArgs &a, hipStream_t stream)
{
    dim3 grid(a.S * a.B * a.Hkv, a.n_hblk), block(64 * NW);
    hipLaunchKernelGGL((decode_bf16_kernel<DK, DV, NW, STAGES>), grid, block, 0, stream, a);
    return 0;
}

} // namespace

int decode_bf16_key_tile() { return kTK; }

// Query heads one workgroup covers for a head-dim pair and group size.
int decode_bf16_heads_per_block(int Dk, int G)
{
    if (Dk == 576) return 128;
    (void)G;
    return 32;
}

int launch_decode_bf16(const DecodeArgs &a, int Dk, int Dv, hipStream_t stream)
{
    if (Dk == 128 && Dv == 128) return launch_one<128, 128, 1, GQA_DEC_STAGES>(a, stream);
    if (Dk == 64 && Dv == 64) return launch_one<64, 64, 1, 3>(a, stream);
    if (Dk == 576 && Dv == 512) {
        // the value must be the latent prefix of the key (v == k, same strides)
        const bool v_is_k_prefix =
            a.v == a.k && a.v_sb == a.k_sb && a.v_sh == a.k_sh && a.v_st == a.k_st;
        if (!v_is_k_prefix) return -1;
        return launch_mla_decode(a, stream);
    }
    return -1;
}

} // namespace gqa
