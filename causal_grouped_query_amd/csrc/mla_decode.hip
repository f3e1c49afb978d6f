// mla_decode.hip -- split-KV decode partials for the weight-absorbed MLA
// shape on gfx950: MQA over a shared 576-wide latent key (512 latent + 64
// rope dims) whose first 512 columns are the value ("Attention Architecture
// Evolution", MLA section and the absorbed score / value equations of its
// DSA section: the score is q_C' c_KV^T + q_R k_R^T, i.e. one 576-wide dot,
// and the output aggregates c_KV itself).
//
// A workgroup owns 128 query heads of one sequence and one key chunk; the
// key tile (32 keys x 576) is copied HBM -> LDS once with global_load_lds
// into a ring (4 deep, 3 for the top-k flavour, whose staged index list
// takes LDS) and read by all 8 waves.  Wave w owns 16 heads and works
// with v_mfma_f32_16x16x32_bf16, so its whole state fits one wave's share of
// the register file (2 waves per SIMD): Q^T over 576 dims (72 VGPRs) and O^T
// over 512 dims (128 accumulators).  Per tile and wave:
//   * scores S^T = K Q^T: 2 key blocks x 18 contraction steps,
//   * online softmax per head: each head is one accumulator column held by
//     the four lanes l, l^16, l^32, l^48 (reduced with permlane swaps),
//   * O^T += V^T P^T over 32 blocks of 16 output dims; the P^T operand is the
//     lane's own 8 weights (the contraction slots of lane group g are the
//     keys its score accumulators hold), and V^T comes from two
//     ds_read_b64_tr_b16 of the same LDS key tile.
// No scores are exchanged between waves, so the tile loop has one barrier.
// Partial outputs and log-sum-exp values go to the workspace exactly as for
// the other decode kernels; combine.hip merges them.
//
// Top-k sparse flavour (SPARSE = true; DeepSeek Sparse Attention on the
// absorbed MLA, "Attention Architecture Evolution", DSA section): the key
// axis a split walks is the list of selected cache positions instead of the
// positions themselves.  The workgroup copies its slice of the list HBM ->
// LDS first (the same asynchronous copy as the key tiles), then each row of
// a key tile is copied from the position its entry names.  An entry outside
// [0, len) (or past the slice) fetches a clamped, valid row and is masked to
// -inf, so it weighs nothing and never brings in memory past len.
// Everything after the copy is the dense kernel.
#include "device_common.h"
#include "launch.h"

namespace gqa {

namespace {

constexpr int kTK = 32;      // keys per tile
constexpr int kDK = 576;     // key width (latent 512 + rope 64)
constexpr int kDV = 512;     // value width (the latent)
#ifndef GQA_MLA_NW
#define GQA_MLA_NW 8
#endif
#ifndef GQA_MLA_STAGES
#define GQA_MLA_STAGES 4  // key-tile ring depth of the dense kernel
#endif
constexpr int kNW = GQA_MLA_NW;  // waves per workgroup
constexpr int kNT = 64 * kNW;
#ifndef GQA_MLA_NT
#define GQA_MLA_NT 0
#endif
// Non-temporal copies (device_common.h), off: unlike the GQA decode's
// stream they gained nothing here (absorbed MLA 187.0 vs 186.6 us) and
// slowed the top-k decode (batch 16 / 64: 47.1 vs 44.1, 75.4 vs 73.0 us;
// decode + combine, one box)
constexpr bool kCopyNT = GQA_MLA_NT;
constexpr int kHW = 16;      // heads per wave
constexpr int kStagesDense = GQA_MLA_STAGES;
constexpr int kStagesSparse = 3;  // the staged index list takes the rest of the LDS
constexpr int kBlocksPerCu = 8 / kNW;  // two waves per SIMD
static_assert(kNW == 4 || kNW == 8, "four or eight waves of 16 heads");
#ifndef GQA_MLA_PF
#define GQA_MLA_PF 6  // operand reads issued ahead of the MFMAs (0: compiler's choice)
#endif
constexpr int kCPR = kDK / 8;   // 72 16-byte chunks per key row
constexpr int kKS = kDK / 32;   // 18 contraction steps of 32 dims
constexpr int kDB = kDV / 16;   // 32 output blocks of 16 dims
constexpr int kMaxChunk = 4096;  // index-list entries one sparse workgroup stages
static_assert(kTK * kCPR % 64 == 0, "tile is whole wave copies");
constexpr int kCopiesMax = (kTK * kCPR / 64 + kNW - 1) / kNW;  // wave copies per tile, at most

template <int STAGES>
struct MlaSmem {
    uint16_t k[STAGES][kTK * kDK];
};

// The index mask of the DSA page is a scatter: a position listed twice is
// selected once.  Within a staged slice of n entries, every entry that
// repeats the position of an earlier entry of the slice is replaced by -1
// (selects nothing).  An open-addressing table of 2 * kMaxChunk slots maps
// each valid position to the smallest slice index listing it: an entry
// claims an empty slot, or lowers the index held by the slot of its
// position; afterwards an entry is kept iff its position's slot holds its
// own index.  Slots only ever hold entries of one position, so the result
// is deterministic.  All threads of the workgroup take part; ends with a
// barrier.
__device__ __forceinline__ void dedup_slice(int *sidx, unsigned *htab, int n, int len, int tid)
{
    constexpr unsigned kEmpty = 0xffffffffu, kMask = 2 * kMaxChunk - 1;
    auto home = [](int pos) { return ((unsigned)pos * 2654435761u) >> 19; };  // 13 bits: 2 * kMaxChunk slots
    for (int e = tid; e < n; e += kNT) {
        const int pos = sidx[e];
        if ((unsigned)pos >= (unsigned)len) continue;
        for (unsigned h = home(pos) & kMask;; h = (h + 1) & kMask) {
            const unsigned old = atomicCAS(&htab[h], kEmpty, (unsigned)e);
            if (old == kEmpty) break;  // claimed
            if (sidx[old] == pos) {    // this position's slot: keep the smaller index
                atomicMin(&htab[h], (unsigned)e);
                break;
            }
        }
    }
    __syncthreads();
    bool drop[(kMaxChunk + kNT - 1) / kNT];
#pragma unroll
    for (int r = 0; r < (kMaxChunk + kNT - 1) / kNT; ++r) {
        const int e = tid + r * kNT;
        drop[r] = false;
        if (e >= n) continue;
        const int pos = sidx[e];
        if ((unsigned)pos >= (unsigned)len) continue;
        for (unsigned h = home(pos) & kMask;; h = (h + 1) & kMask) {
            const unsigned v = htab[h];
            if (v == kEmpty) break;  // (not reached: the position was inserted along this probe path)
            if (sidx[v] == pos) {
                drop[r] = v != (unsigned)e;
                break;
            }
        }
    }
    __syncthreads();  // every lookup done before any entry is overwritten
#pragma unroll
    for (int r = 0; r < (kMaxChunk + kNT - 1) / kNT; ++r)
        if (drop[r]) sidx[tid + r * kNT] = -1;
    __syncthreads();
}

template <bool SPARSE>
__global__ __launch_bounds__(kNT, kBlocksPerCu) void mla_decode_kernel(DecodeArgs p)
{
    constexpr int NCOPY = kTK * kCPR / 64;  // 36 wave-copies per tile, spread over 8 waves
    constexpr int kStages = SPARSE ? kStagesSparse : kStagesDense;
    __shared__ __attribute__((aligned(1024))) MlaSmem<kStages> sm;
    __shared__ __attribute__((aligned(16))) int sidx[SPARSE ? kMaxChunk : 4];  // staged index slice
    // sparse: open-addressing set of the slice's positions (entry indices)
    __shared__ unsigned htab[SPARSE ? 2 * kMaxChunk : 1];
    debug_nanfill(sm);
    debug_nanfill(sidx);
    debug_nanfill(htab);

    // chunk-major order, as in the other decode kernel
    const int nbk = p.B * p.Hkv;
    const int split = blockIdx.x / nbk;
    const int bk = blockIdx.x - split * nbk;  // b * Hkv + kv head
    const int hblk = blockIdx.y;
    const int kvh = bk % p.Hkv, b = bk / p.Hkv;

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15, g = lane >> 4;
    const int hh = hblk * (kHW * kNW) + kHW * w + r16;  // head within the group
    const bool head_ok = hh < p.G;
    const int head = kvh * p.G + (head_ok ? hh : 0);

    int len = p.lens[b];
    len = len < 0 ? 0 : (len > p.Tmax ? p.Tmax : len);
    int kst = 0;  // dense with a sliding window: the last `window` keys, rows kst ..
    if (!SPARSE && p.window > 0 && len > p.window) {
        kst = len - p.window;
        len = p.window;
    }
    const int kbeg = split * p.chunk;
    // dense: cache positions [kbeg, kend); sparse: index-list entries
    const int kend = min(SPARSE ? p.topk : len, kbeg + p.chunk);
    int ntiles = kend > kbeg ? (kend - kbeg + kTK - 1) / kTK : 0;

    const uint16_t *kb = (const uint16_t *)p.k + (size_t)b * p.k_sb + (size_t)kvh * p.k_sh + (size_t)kst * p.k_st;

    // sparse: copy entries [kbeg, kbeg + 32 ntiles) of the list to LDS
    // (addresses clamped into the list; what lies past kend is never used
    // unmasked).  A sequence of length 0 has nothing to read.
    if constexpr (SPARSE) {
        if (len == 0) ntiles = 0;
        const int *il = p.idx + (size_t)b * p.topk;
        for (int e0 = w * 64; e0 < ntiles * kTK; e0 += kNT)
            g2lds4<kCopyNT>(il + min(kbeg + e0 + lane, p.topk - 1), &sidx[e0]);
        for (int i = tid; i < 2 * kMaxChunk; i += kNT) htab[i] = 0xffffffffu;
        wait_vmem();
        lds_barrier();  // the slice and the empty table are visible to every wave
        dedup_slice(sidx, htab, kend - kbeg, len, tid);
    }

    // wave copy j covers LDS chunks [64 j, 64 j + 64); waves take j = w, w + 8, ...
    // (36 copies: waves 0-3 do 5, waves 4-7 do 4; the count per wave is fixed)
    const int my_copies = (NCOPY - w + kNW - 1) / kNW;
    using Tile = PlaneTile<kTK, true>;
    // Copy j fills LDS slots 64 j + lane of the plane layout: tile row
    // 16 (j & 1) + lrow, chunk 4 (j >> 1) + lchunk, with the lane's row and
    // chunk inside a 16-row half-plane fixed (rows r and r + 16 share the
    // swizzle).  A copy is then a workgroup-uniform base plus a per-lane
    // unsigned 32-bit byte offset: for a full dense tile one fixed offset
    // serves every copy; otherwise the offset is the fetched row times the
    // row pitch plus the lane's chunk.  Dense offsets stay inside one tile,
    // under 2^31 since the host bounds the row pitch to 2^25 elements; a
    // top-k cache whose offsets from its first row could pass 2^32 takes
    // per-lane 64-bit addresses instead.  The copy loops stay rolled:
    // unrolled, their per-copy values stay live beside the 200 registers of
    // Q^T and O^T and the tile loop spills.
    const int lrow = lane >> 2;
    auto lane_chunk16 = [&]() { return (unsigned)(((lane & 3) ^ pswz16(lrow)) * 16); };
    const unsigned pitch = (unsigned)p.k_st * 2u;  // bytes between key rows
    // dense: offset of the lane's slot from its copy's base; sparse: its chunk
    const unsigned lane_off = SPARSE ? lane_chunk16() : (unsigned)lrow * pitch + lane_chunk16();
    const bool off32 = !SPARSE || (long long)p.Tmax * p.k_st * 2 + kDK * 2 < (1LL << 32);
    const unsigned ring_lds = lds_u32(&sm) + (unsigned)(w * 64 * 16);
    auto issue_tile = [&](int k0, int slot) {
        const unsigned dst = ring_lds + (unsigned)(slot * kTK * kDK * 2);
        if (!SPARSE && k0 + kTK <= kend) {
#pragma unroll 1
            for (int jj = 0; jj < kCopiesMax; ++jj) {
                const int j = w + kNW * jj;
                if (j < NCOPY)
                    g2lds16_at<kCopyNT>(kb + (size_t)(k0 + 16 * (j & 1)) * p.k_st + 32 * (j >> 1), lane_off,
                               dst + (unsigned)(jj * kNW * 64 * 16));
            }
        } else if (off32) {
            // sparse: rows named by the staged list; dense: the tail tile,
            // rows past kend re-read row kend - 1 (masked)
            const uint16_t *base = SPARSE ? kb : kb + (size_t)k0 * p.k_st;
#pragma unroll 1
            for (int jj = 0; jj < kCopiesMax; ++jj) {
                const int j = w + kNW * jj;
                if (j >= NCOPY) continue;
                const int row = 16 * (j & 1) + lrow;
                unsigned off;
                if (SPARSE) {
                    const int pos = min(max(sidx[k0 - kbeg + row], 0), len - 1);  // in range for any entry
                    off = (unsigned)pos * pitch + lane_off;
                } else {
                    off = lane_off + (unsigned)(min(row, kend - 1 - k0) - lrow) * pitch;
                }
                g2lds16_at<kCopyNT>(base + 32 * (j >> 1), off, dst + (unsigned)(jj * kNW * 64 * 16));
            }
        } else if constexpr (SPARSE) {
            unsigned lc = lane_chunk16();
            asm volatile("" : "+v"(lc));  // computed here: no 64-bit per-lane value lives across the loop
#pragma unroll 1
            for (int jj = 0; jj < kCopiesMax; ++jj) {
                const int j = w + kNW * jj;
                if (j >= NCOPY) continue;
                const int row = 16 * (j & 1) + lrow;
                const int pos = min(max(sidx[k0 - kbeg + row], 0), len - 1);
                g2lds16_at<kCopyNT>((const char *)(kb + (size_t)pos * p.k_st + 32 * (j >> 1)) + lc,
                           dst + (unsigned)(jj * kNW * 64 * 16));
            }
        }
    };

    // Q^T (B operand): head r16 of this wave, dims 32 ks + 8 g .. + 7
    u32x4 qreg[kKS];
    auto load_q = [&]() {
        const uint16_t *qrow = (const uint16_t *)p.q + ((size_t)b * p.Hq + head) * kDK + 8 * g;
#pragma unroll
        for (int ks = 0; ks < kKS; ++ks) {
            u32x4 z = {0u, 0u, 0u, 0u};
            qreg[ks] = head_ok ? *(const u32x4 *)(qrow + 32 * ks) : z;
        }
#pragma unroll
        for (int ks = 0; ks < kKS; ++ks) hold_reg(qreg[ks]);
    };
    // dense: the query first; sparse: after the first tiles' copies, so the
    // query latency overlaps theirs (the list copy already took one latency)
    if constexpr (!SPARSE) load_q();

    f32x4 o[kDB];
#pragma unroll
    for (int i = 0; i < kDB; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;

    // K operand (A): key row 16 t + r16, dims 32 ks + 8 g .. + 7 = chunk
    // 4 ks + g, i.e. plane ks, chunk g of the plane.  Rows r and r + 16 share
    // the swizzle, so block 1 is block 0 + 16 rows.
    const int kb0 = Tile::offset(r16, g);
    // V^T operand (A) by transpose reads: in 16-lane group g, lane 4 r + q
    // points at key 4 g + r (first read) or 16 + 4 g + r (second read), the
    // keys of contraction slots r and 4 + r (the lane's score elements),
    // dims 16 db + 4 q .. + 3: chunk 2 db + (q >> 1) (plane db >> 1, chunk
    // 2 (db & 1) + (q >> 1) of the plane), byte 8 (q & 1) inside it.
    const int vr = r16 >> 2, vq = r16 & 3;
    // (the second read is the first one 16 rows further down)
    int vb[2];  // [db & 1]
#pragma unroll
    for (int odd = 0; odd < 2; ++odd) vb[odd] = Tile::offset(4 * g + vr, 2 * odd + (vq >> 1)) + 8 * (vq & 1);

#pragma unroll
    for (int s = 0; s < kStages - 1; ++s)
        if (s < ntiles) issue_tile(kbeg + s * kTK, s);
    if constexpr (SPARSE) load_q();

    const float c = p.c;
    for (int it = 0; it < ntiles; ++it) {
        const int k0 = kbeg + it * kTK;
        const int slot = it % kStages;
        // tile `it` must have landed; the next tile's copies may still fly
        if (it + kStages - 2 < ntiles) {
            if (my_copies == kCopiesMax)
                wait_vmem_le<kCopiesMax * (kStages - 2)>();
            else
                wait_vmem_le<(kCopiesMax - 1) * (kStages - 2)>();
        } else {
            wait_vmem();
        }
        lds_barrier();  // tile visible; the slot of tile it-1 is free
        if (it + kStages - 1 < ntiles) issue_tile(k0 + (kStages - 1) * kTK, (it + kStages - 1) % kStages);

        const char *ks_ = (const char *)sm.k[slot];
        f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < kKS; ++ks) {
            s0 = mfma16x16x32(*(const u32x4 *)(ks_ + kb0 + ks * Tile::PLANE_BYTES), qreg[ks], s0);
            s1 = mfma16x16x32(*(const u32x4 *)(ks_ + kb0 + 16 * 64 + ks * Tile::PLANE_BYTES), qreg[ks], s1);
        }
#if GQA_MLA_PF
        __builtin_amdgcn_sched_group_barrier(0x100, GQA_MLA_PF, 0);
#pragma unroll
        for (int i = 0; i < 2 * kKS - GQA_MLA_PF; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, GQA_MLA_PF, 0);
#endif
        // element i of s0 / s1: key 4 g + i / 16 + 4 g + i, head r16
        if (SPARSE) {
            // entry k0 + j selects a key iff it lies in the slice and names a
            // position in [0, len)
            const int4 e0 = *(const int4 *)&sidx[k0 - kbeg + 4 * g];
            const int4 e1 = *(const int4 *)&sidx[k0 - kbeg + 16 + 4 * g];
            const int a0[4] = {e0.x, e0.y, e0.z, e0.w}, a1[4] = {e1.x, e1.y, e1.z, e1.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (k0 + 4 * g + i >= kend || (unsigned)a0[i] >= (unsigned)len) s0[i] = -INFINITY;
                if (k0 + 16 + 4 * g + i >= kend || (unsigned)a1[i] >= (unsigned)len) s1[i] = -INFINITY;
            }
        } else if (k0 + kTK > kend) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (k0 + 4 * g + i >= kend) s0[i] = -INFINITY;
                if (k0 + 16 + 4 * g + i >= kend) s1[i] = -INFINITY;
            }
        }

        float mx = fmaxf(fmaxf(s0[0], s0[1]), fmaxf(s0[2], s0[3]));
        mx = fmaxf(mx, fmaxf(fmaxf(s1[0], s1[1]), fmaxf(s1[2], s1[3])));
        const float mt = quarters_max(mx) * c;
        if (__any(mt > m_run + 8.0f)) {
            // only heads whose max crossed the threshold move their reference
            const float m_new = (mt > m_run + 8.0f) ? mt : m_run;
            const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int i = 0; i < kDB; ++i) o[i] *= alpha;
        }
        const float m_use = (m_run == -INFINITY) ? 0.f : m_run;

        u32x4 pb;
        {
            float pv[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pv[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[i], c, -m_use));
                pv[4 + i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[i], c, -m_use));
            }
            pb.x = pack_bf16x2(pv[0], pv[1]);
            pb.y = pack_bf16x2(pv[2], pv[3]);
            pb.z = pack_bf16x2(pv[4], pv[5]);
            pb.w = pack_bf16x2(pv[6], pv[7]);
            l_run = sum_bf16x8(pb, l_run);
        }

        // O^T += V^T P^T over the latent prefix of the tile
#pragma unroll
        for (int db = 0; db < kDB; ++db) {
            const int o_ = (db >> 1) * Tile::PLANE_BYTES;
            const u32x2 lo = lds_read_tr16(ks_ + vb[db & 1] + o_);
            const u32x2 hv = lds_read_tr16(ks_ + vb[db & 1] + 16 * 64 + o_);
            const u32x4 va = {lo.x, lo.y, hv.x, hv.y};
            o[db] = mfma16x16x32(va, pb, o[db]);
        }
#if GQA_MLA_PF
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * GQA_MLA_PF, 0);
#pragma unroll
        for (int i = 0; i < kDB - GQA_MLA_PF; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, GQA_MLA_PF, 0);
#endif
    }

    if (!head_ok) return;
    const float l_tot = quarters_sum(l_run);
    const size_t prow = ((size_t)b * p.Hq + head) * p.S + split;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    // element i of o[db]: output dim 16 db + 4 g + i, head r16
#pragma unroll
    for (int db = 0; db < kDB; ++db)
        store_partial4(p.part_o, prow * kDV + 4 * g + 16 * db, o[db][0] * inv, o[db][1] * inv, o[db][2] * inv,
                       o[db][3] * inv);
    if (g == 0) p.part_lse[prow] = l_tot > 0.f ? m_run + __log2f(l_tot) : -INFINITY;
}

} // namespace

int launch_mla_decode(const DecodeArgs &a, hipStream_t stream)
{
    dim3 grid(a.S * a.B * a.Hkv, a.n_hblk), block(kNT);
    hipLaunchKernelGGL(mla_decode_kernel<false>, grid, block, 0, stream, a);
    return 0;
}

int mla_topk_max_chunk() { return kMaxChunk; }
int mla_heads_per_block() { return kHW * kNW; }

int launch_mla_decode_topk(const DecodeArgs &a, hipStream_t stream)
{
    if (!a.idx || a.topk <= 0 || a.chunk <= 0 || a.chunk % kTK || a.chunk > kMaxChunk) return -1;
    dim3 grid(a.S * a.B * a.Hkv, a.n_hblk), block(kNT);
    hipLaunchKernelGGL(mla_decode_kernel<true>, grid, block, 0, stream, a);
    return 0;
}

} // namespace gqa
