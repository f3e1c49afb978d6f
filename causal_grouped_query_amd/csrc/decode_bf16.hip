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
// The same kernel serves the weight-absorbed MLA shape of "Attention
// Architecture Evolution" (MLA section; absorbed score/value equations of its
// DSA section): MQA with a 576-wide key (512 latent + 64 rope) whose first
// 512 columns are the value; the caller passes v = k.
//
// Layout in a workgroup: NW waves, wave w owns query heads
// 32*(NW*hblk + w) + (0..31) of the group (columns of the MFMA, zero-padded
// when the group is smaller).  Scores are S^T = K Q^T (32 keys x 32 heads per
// v_mfma_f32_32x32x16_bf16), O^T = V^T P^T as in the prefill kernel.
#include "device_common.h"
#include "launch.h"

namespace gqa {

namespace {

constexpr int kTK = 32;  // keys per tile

template <int DK, int DV>
struct DecSmem {
    static constexpr int KP = DK + 8;
    static constexpr int VP = kTK + 8;
    uint16_t k[kTK * KP];
    uint16_t vt[DV * VP];
};

template <int DK, int DV, int NW, bool PREFETCH>
__global__ __launch_bounds__(64 * NW) void decode_bf16_kernel(DecodeArgs p)
{
    constexpr int NT = 64 * NW;
    constexpr int KP = DecSmem<DK, DV>::KP;
    constexpr int VP = DecSmem<DK, DV>::VP;
    constexpr int KS = DK / 16;
    constexpr int DT = DV / 32;
    constexpr int KCH = kTK * DK / 8;
    constexpr int KPT = (KCH + NT - 1) / NT;
    constexpr int VBL = (kTK / 4) * (DV / 8);
    constexpr int VPT = (VBL + NT - 1) / NT;

    __shared__ __attribute__((aligned(16))) DecSmem<DK, DV> sm;

    const int split = blockIdx.x;
    const int hblk = blockIdx.y;
    const int bk = blockIdx.z;  // b * Hkv + kv head
    const int kvh = bk % p.Hkv, b = bk / p.Hkv;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
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

    u32x4 qreg[KS];
    {
        const uint16_t *qrow = (const uint16_t *)p.q + ((size_t)b * p.Hq + head) * DK;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 z = {0u, 0u, 0u, 0u};
            qreg[ks] = head_ok ? *(const u32x4 *)(qrow + 16 * ks + 8 * hi) : z;
        }
    }

    f32x16 o[DT];
#pragma unroll
    for (int i = 0; i < DT; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[i][e] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    u32x4 kpre[KPT];
    u32x4 vpre[VPT][4];

    auto load_tile = [&](int k0) {
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int c = tid + i * NT;
            const int row = c / (DK / 8), cc = c % (DK / 8);
            u32x4 z = {0u, 0u, 0u, 0u};
            kpre[i] = (c < KCH && k0 + row < kend)
                          ? *(const u32x4 *)(kb + (size_t)(k0 + row) * p.k_st + cc * 8)
                          : z;
        }
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int vbk = tid + i * NT;
            const int db = vbk % (DV / 8), kq = vbk / (DV / 8);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int key = k0 + 4 * kq + j;
                u32x4 z = {0u, 0u, 0u, 0u};
                vpre[i][j] = (vbk < VBL && key < kend)
                                 ? *(const u32x4 *)(vb + (size_t)key * p.v_st + db * 8)
                                 : z;
            }
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int c = tid + i * NT;
            const int row = c / (DK / 8), cc = c % (DK / 8);
            if (c < KCH) *(u32x4 *)(&sm.k[row * KP + cc * 8]) = kpre[i];
        }
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int vbk = tid + i * NT;
            const int db = vbk % (DV / 8), kq = vbk / (DV / 8);
            if (vbk < VBL) {
                u32x2 t8[8];
                transpose4x8(vpre[i], t8);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    *(u32x2 *)(&sm.vt[(db * 8 + e) * VP + 4 * kq]) = t8[e];
            }
        }
    };

    const float c = p.c;
    if (PREFETCH && ntiles > 0) load_tile(kbeg);

    for (int it = 0; it < ntiles; ++it) {
        const int k0 = kbeg + it * kTK;
        if (!PREFETCH) load_tile(k0);
        __syncthreads();
        store_tile();
        __syncthreads();
        if (PREFETCH && it + 1 < ntiles) load_tile(k0 + kTK);

        f32x16 s;
#pragma unroll
        for (int e = 0; e < 16; ++e) s[e] = 0.f;
        const uint16_t *krow = &sm.k[kperm(col) * KP + 8 * hi];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) s = mfma32x32x16(*(const u32x4 *)(krow + 16 * ks), qreg[ks], s);

        if (k0 + kTK > kend) {
#pragma unroll
            for (int e = 0; e < 16; ++e)
                if (k0 + acc_key(0, e, hi) >= kend) s[e] = -INFINITY;
        }

        float mx = s[0];
#pragma unroll
        for (int e = 1; e < 16; ++e) mx = fmaxf(mx, s[e]);
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

        u32x4 pb[2];
        float psum = 0.f;
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
            psum = sum_bf16x8(pb[h], psum);
        }
        l_run += psum;

#pragma unroll
        for (int st = 0; st < 2; ++st) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const u32x4 va = *(const u32x4 *)(&sm.vt[(32 * dt + col) * VP + 16 * st + 8 * hi]);
                o[dt] = mfma32x32x16(va, pb[st], o[dt]);
            }
        }
    }

    if (!head_ok) return;
    const float l_tot = l_run + wave_swap_half(l_run);
    const size_t prow = ((size_t)b * p.Hq + head) * p.S + split;
    float *po = p.part_o + prow * DV;
    if (l_tot > 0.f) {
        const float inv = 1.f / l_tot;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                f32x4 v4 = {o[dt][4 * j] * inv, o[dt][4 * j + 1] * inv, o[dt][4 * j + 2] * inv,
                            o[dt][4 * j + 3] * inv};
                *(f32x4 *)(po + 32 * dt + 8 * j + 4 * hi) = v4;
            }
        if (hi == 0) p.part_lse[prow] = m_run + __log2f(l_tot);
    } else {
        // empty chunk: contributes nothing to the merge
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                f32x4 z = {0.f, 0.f, 0.f, 0.f};
                *(f32x4 *)(po + 32 * dt + 8 * j + 4 * hi) = z;
            }
        if (hi == 0) p.part_lse[prow] = -INFINITY;
    }
}

template <int DK, int DV, int NW, bool PF>
int launch_one(const DecodeArgs &a, hipStream_t stream)
{
    dim3 grid(a.S, a.n_hblk, a.B * a.Hkv), block(64 * NW);
    hipLaunchKernelGGL((decode_bf16_kernel<DK, DV, NW, PF>), grid, block, 0, stream, a);
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
    if (Dk == 128 && Dv == 128) return launch_one<128, 128, 1, true>(a, stream);
    if (Dk == 64 && Dv == 64) return launch_one<64, 64, 1, true>(a, stream);
    if (Dk == 576 && Dv == 512) return launch_one<576, 512, 4, false>(a, stream);
    return -1;
}

} // namespace gqa
