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
//  * One workgroup = NW waves that all read ONE KV head: Gt query heads of
//    the group x Pt positions.  Each K/V tile is staged in LDS once and used
//    by the whole group of heads; there is no repeat_interleave copy, the
//    head map g(a) = a / (Hq/Hkv) is pure addressing.
//  * A wave owns 32 * NC query rows (NC column blocks of the MFMA); every
//    K operand and every V^T operand read from LDS feeds NC MFMAs, so LDS
//    reads and HBM/L2 -> LDS copies per FLOP fall as 1 / NC.  Scores are computed transposed,
//    S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: Q^T sits in registers as the
//    B operand for the whole key loop, K rows come from LDS as the A operand.
//    In the accumulator every lane holds one query column, so row max and row
//    sum are in-lane plus a single exchange with lane l^32.
//  * O^T = V^T P^T: P^T needs no data movement (see kperm in
//    device_common.h); V stays row-major in LDS and its transposed A operand
//    comes from two ds_read_b64_tr_b16 per MFMA.
//  * K and V tiles go straight from HBM to LDS with global_load_lds (no
//    registers, no VALU), into a STAGES-deep ring in the swizzled plane
//    layout of device_common.h (every LDS read of the loop is a base
//    register plus an immediate): tiles i+1 .. i+STAGES-1 are in flight while
//    tile i is computed; one barrier per tile.  Eight waves (256 query rows)
//    share each tile, one workgroup per CU with a 4-deep ring (128 KiB):
//    half the L2 -> LDS traffic per FLOP of two 4-wave workgroups per CU.
//  * Online softmax in base 2: scale*log2(e) is folded into one FMA per
//    score, exp via v_exp_f32, the row sum via v_dot2 over the bf16-rounded
//    weights.  The reference max is set from a lane's first visible tile
//    and moved (O rescaled) only when that lane's tile weights sum past
//    2^16, so the common tile computes no max at all; weights stay below
//    2^16, which fp32 and bf16 carry with the same relative precision as
//    weights <= 1, and the normalised result is the same softmax.
//  * Grid order: tiles of one (batch, KV head, head block) are consecutive
//    on one XCD (the dispatcher deals workgroups round-robin over 8 XCDs, so
//    the remap keeps a KV head's K/V in one L2), heaviest causal tiles first.
//  * Packed variable-length sequences (cu_seqlens) with an optional sliding
//    window are the same kernel (template flag VAR): per-sequence bounds,
//    strided token rows, a key loop that starts at the window's first tile
//    and a lower mask bound per lane.  Optional used lengths per sequence
//    turn the tail of each slot into padding (a right-padded batch): padded
//    keys are never read, padded query rows never written.
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace gqa {

namespace {

#ifndef GQA_FWD_NC
#define GQA_FWD_NC 1      // 32-row column blocks per wave
#endif
#ifndef GQA_FWD_NW
#define GQA_FWD_NW 8      // waves per workgroup
#endif
#ifndef GQA_FWD_STAGES
#define GQA_FWD_STAGES 4  // K/V ring depth
#endif
#ifndef GQA_FWD_PREFETCH
#define GQA_FWD_PREFETCH 4  // LDS operand reads kept in flight ahead of the MFMAs (0: compiler's choice)
#endif
// sum of one lane's weights in a tile past which its reference max moves
constexpr float kSumCap = 65536.0f;
constexpr int kNC = GQA_FWD_NC;
constexpr int kNW = GQA_FWD_NW;
#ifndef GQA_FWD_BN
#define GQA_FWD_BN 64     // keys per K/V tile
#endif
constexpr int kBN = GQA_FWD_BN;   // keys per tile
constexpr int kNT = kBN / 32;     // 32-key score tiles per key tile
constexpr int kStages = GQA_FWD_STAGES;
constexpr int kThreads = 64 * kNW;
constexpr int kWavesPerSimd = kNC == 1 ? 2 : 1;  // register budget: 256 or 512 per lane
// workgroups per CU that keep kWavesPerSimd waves on each of the 4 SIMDs
constexpr int kBlocksPerCu = (4 * kWavesPerSimd + kNW - 1) / kNW;
constexpr long long kResidentBlocks = 256LL * kBlocksPerCu;  // workgroups resident at once

template <int D>
struct FwdSmem {
    static constexpr int TILE = kBN * D;  // elements of one K or V tile (plane layout)
    uint16_t k[kStages][TILE];
    uint16_t v[kStages][TILE];
};

// VAR: packed variable-length sequences (cu_seqlens), strided tensors and an
// optional sliding window; false: the dense [B,H,T,D] problem (every VAR term
// below folds away).
// first token slot of packed sequence b, clamped to [0, total]
__device__ __forceinline__ int seq_start(const int *cu, int b, int total) { return min(max(cu[b], 0), total); }
// tokens of packed sequence b: its slot length, or the used length when
// given (clamped to the slot; the rest of the slot is padding).  The slot is
// clamped to [0, total), so offsets that disagree with the buffers never
// address a token outside them.
__device__ __forceinline__ int used_len(const int *cu, const int *used, int b, int total)
{
    const int s = seq_start(cu, b, total);
    const int n = min(max(cu[b + 1], s), total) - s;
    return used ? min(max(used[b], 0), n) : n;
}

// PART: key-shard mode for context parallelism (dense layout only): query i
// sits at key index q_minus_k + i of the given keys, and the normalised
// output goes out in fp32 together with its natural-log LSE, the partial
// result an exact log-sum-exp merge combines across shards.
template <int D, bool VAR, bool PART = false>
__global__ __launch_bounds__(kThreads, kBlocksPerCu) void fwd_bf16_kernel(FwdArgs p)
{
    constexpr int CPR = D / 8;                     // 16-byte chunks per row
    constexpr int KS = D / 16;                     // MFMA k-steps over the head dim
    constexpr int DT = D / 32;                     // 32-row tiles of O^T
    constexpr int NINS = kBN * CPR / kThreads;     // async copies per thread per tensor
    constexpr int ROWS = 32 * kNC;                 // query rows per wave
    static_assert(kBN * CPR % kThreads == 0, "tile must split evenly over the workgroup");
    static_assert(offsetof(FwdSmem<D>, v) == kStages * FwdSmem<D>::TILE * 2, "V ring follows the K ring");
    using Tile = PlaneTile<kBN>;

    __shared__ __attribute__((aligned(1024))) FwdSmem<D> sm;
    debug_nanfill(sm);

    // ---- workgroup -> (unit, query tile), heaviest first ----
    // Dense: all units carry the same work, so consecutive query tiles of a
    // unit go to one XCD (the dispatcher deals ids round-robin over 8 XCDs;
    // the remap keeps a KV head's K/V in one L2).  Varlen: units differ in
    // size, so ids run query-tile-major over all units and the round-robin
    // spreads every sequence over the XCDs (with a multiple of 8 units each
    // unit still stays on one XCD).
    const int nblk = gridDim.x;
    const int L = blockIdx.x;
    // A dense launch with fewer workgroups than items (one resident round)
    // loops over items; otherwise every workgroup takes one item.
    const long long items = (long long)p.n_units * p.n_qt;
    const bool looping = !VAR && nblk < items;
    for (int k = 0;; ++k) {
        int unit, qt;
        if (VAR) {
            // ids enumerate (flat query tile f, head unit u of the sequence); u
            // runs fastest so one tile's KV heads go to different XCDs.  f counts
            // the query tiles of all sequences in order (the grid is an upper
            // bound, there are no empty sequences' tiles in it); within a
            // sequence the last tiles (most keys) come first.
            const int u = L % p.n_units;
            const int f = L / p.n_units;
            const int lane0 = threadIdx.x & 63;
            int base = 0, bsel = -1, fb1 = 0;
            for (int b0 = 0; b0 < p.B; b0 += 64) {
                const int bb = b0 + lane0;
                const int nt = bb < p.B ? (used_len(p.cu_q, p.used_q, bb, p.total_q) + p.Pt - 1) / p.Pt : 0;
                int incl = nt;
#pragma unroll
                for (int o = 1; o < 64; o <<= 1) {
                    const int y = __shfl_up(incl, o);
                    if (lane0 >= o) incl += y;
                }
                const unsigned long long hit = __ballot(bb < p.B && base + incl > f);
                if (hit) {
                    const int Lh = __ffsll((long long)hit) - 1;
                    bsel = b0 + Lh;
                    fb1 = base + __shfl(incl, Lh);
                    break;
                }
                base += __shfl(incl, 63);
            }
            if (bsel < 0) return;  // past the last tile (whole workgroup, before any barrier)
            qt = fb1 - 1 - f;
            unit = __builtin_amdgcn_readfirstlane(bsel) * p.n_units + u;
            qt = __builtin_amdgcn_readfirstlane(qt);
        } else if (!looping) {
            const int xcd = L & 7, r = L >> 3;
            const int per = nblk >> 3, rem = nblk & 7;
            const int Lp = (xcd < rem) ? xcd * (per + 1) + r : rem * (per + 1) + (xcd - rem) * per + r;
            unit = Lp / p.n_qt;
            qt = p.n_qt - 1 - (Lp - unit * p.n_qt);
        } else {
            // XCD x (workgroups L = x mod 8, all resident) walks the contiguous
            // item range that the one-item-per-workgroup order gives it, in
            // snake order over its n workgroups: the j-th takes positions j,
            // 2n - 1 - j, 2n + j, ...  Within a unit the positions run from the
            // heaviest causal tile to the lightest, so the snake pairs heavy
            // with light and every workgroup gets about the same number of key
            // tiles, with no dispatch between its items.
            const int xcd = L & 7, j = L >> 3;
            const int nwx = (nblk >> 3) + ((nblk & 7) > xcd ? 1 : 0);
            const int per = (int)(items >> 3), rem = (int)(items & 7);
            const int cnt = per + (xcd < rem ? 1 : 0);
            const int start = xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per;
            const int pos = (k & 1) ? (k + 1) * nwx - 1 - j : k * nwx + j;
            if (pos >= cnt) break;
            const int Lp = start + pos;
            unit = Lp / p.n_qt;
            qt = p.n_qt - 1 - (Lp - unit * p.n_qt);
        }
        const int hblk = unit % p.n_hblk;
        const int bk = unit / p.n_hblk;  // b * Hkv + kv head
        const int kvh = bk % p.Hkv;
        const int b = bk / p.Hkv;

        // sequence bounds: the whole problem, or sequence b of the packed batch
        int Tq = p.Tq, Tk = p.Tk, sq0 = 0, sk0 = 0;
        if (VAR) {
            sq0 = seq_start(p.cu_q, b, p.total_q);
            sk0 = seq_start(p.cu_k, b, p.total_k);
            Tq = used_len(p.cu_q, p.used_q, b, p.total_q);
            Tk = used_len(p.cu_k, p.used_k, b, p.total_k);
            if (qt * p.Pt >= Tq) return;  // the whole workgroup (no barrier passed yet)
        }
        const int win = VAR ? p.window : 0;  // > 0: keys p-w+1 .. p only

        const int tid = threadIdx.x;
        const int lane = tid & 63;
        const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (uniform)
        const int col = lane & 31, hi = lane >> 5;
        const int head = kvh * p.G + hblk * p.Gt + (w % p.Gt);
        const int q0 = qt * p.Pt + (w / p.Gt) * ROWS;  // first query index of this wave
        const int off = PART ? p.q_minus_k : Tk - Tq;  // position of query 0, counted in keys
        const bool wave_active = q0 < Tq;

        // keys the workgroup needs: tiles [t0, t0 + ntiles)
        int kend = Tk;
        if (p.causal) kend = min(Tk, off + min(Tq, qt * p.Pt + p.Pt));
        const int t0 = win > 0 ? max(0, off + qt * p.Pt - win + 1) / kBN : 0;
        const int ntiles = max(0, (kend + kBN - 1) / kBN - t0);
        // last key any row of this wave can see
        const int wlast = p.causal ? off + min(q0 + ROWS - 1, Tq - 1) : Tk - 1;
        // window: first key the wave's lowest row can see, and the largest first
        // key of its rows (tiles starting below it need the lower mask)
        const int wfirst = off + q0 - win + 1;
        const int wlo_hi = off + min(q0 + ROWS - 1, Tq - 1) - win + 1;
        // last (and with a window first) key each of this lane's queries can see
        int lim[kNC], llo[kNC];
#pragma unroll
        for (int cb = 0; cb < kNC; ++cb) {
            lim[cb] = p.causal ? min(off + q0 + 32 * cb + col, Tk - 1) : Tk - 1;
            llo[cb] = off + q0 + 32 * cb + col - win + 1;
        }

        // K / V rows: [B,Hkv,T,D] contiguous, or strided tokens of sequence b
        const long long krs = VAR ? p.k_st : D, vrs = VAR ? p.v_st : D;  // elements between key rows
        const uint16_t *kbase = VAR ? p.k + (size_t)kvh * p.k_sh + (size_t)sk0 * p.k_st : p.k + (size_t)bk * p.Tk * D;
        const uint16_t *vbase = VAR ? p.v + (size_t)kvh * p.v_sh + (size_t)sk0 * p.v_st : p.v + (size_t)bk * p.Tk * D;

        // ---- async copies (plane layout, see PlaneTile) ----
        // Copy j of this wave fills 16-byte slots 64 (j * NW + w) + lane; the
        // source (row, chunk) of each slot is fixed, so its byte offset inside a
        // tile is computed once.  Rows past Tk re-read row Tk - 1 (in bounds,
        // masked).
        int grow_[NINS];
        unsigned goff_[NINS], gvoff_[NINS];  // byte offsets inside a K / V tile
#pragma unroll
        for (int j = 0; j < NINS; ++j) {
            int row, chunk;
            Tile::slot_source((j * kNW + w) * 64 + lane, row, chunk);
            grow_[j] = row;
            goff_[j] = (unsigned)(row * krs + chunk * 8) * 2u;
            gvoff_[j] = VAR ? (unsigned)(row * vrs + chunk * 8) * 2u : goff_[j];
        }
        // LDS byte address of this wave's first slot in K ring slot 0 (V slots
        // follow the K slots)
        const unsigned ring_lds = lds_u32(&sm) + (unsigned)(w * 64 * 16);
        constexpr unsigned kTileBytes = FwdSmem<D>::TILE * 2u;
        auto issue = [&](const uint16_t *src, unsigned dst, int k0, const unsigned (&offs)[NINS], long long rs) {
            if (k0 + kBN <= Tk) {
                const uint16_t *s0 = src + (size_t)k0 * rs;
#pragma unroll
                for (int j = 0; j < NINS; ++j) g2lds16_at(s0, offs[j], dst + (unsigned)(j * kNW * 64 * 16));
            } else {
#pragma unroll
                for (int j = 0; j < NINS; ++j) {
                    const int row = min(k0 + grow_[j], Tk - 1);
                    g2lds16_at((const char *)(src + (size_t)row * rs) + (offs[j] - (unsigned)(grow_[j] * rs) * 2u),
                               dst + (unsigned)(j * kNW * 64 * 16));
                }
            }
        };
        auto issue_kv = [&](int j, int slot) {  // tile t0 + j of the workgroup into ring slot `slot`
            issue(kbase, ring_lds + (unsigned)slot * kTileBytes, (t0 + j) * kBN, goff_, krs);
            issue(vbase, ring_lds + (unsigned)(kStages + slot) * kTileBytes, (t0 + j) * kBN, gvoff_, vrs);
        };

        // ---- Q^T in registers (B operands), zero for rows past Tq ----
        u32x4 qreg[kNC][KS];
#pragma unroll
        for (int cb = 0; cb < kNC; ++cb) {
            const int qi = q0 + 32 * cb + col;
            const bool ok = wave_active && qi < Tq;
            const uint16_t *qrow = VAR ? p.q + (size_t)head * p.q_sh + (size_t)(sq0 + (ok ? qi : 0)) * p.q_st
                                       : p.q + (((size_t)b * p.Hq + head) * p.Tq + (ok ? qi : 0)) * D;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                u32x4 z = {0u, 0u, 0u, 0u};
                qreg[cb][ks] = ok ? *(const u32x4 *)(qrow + 16 * ks + 8 * hi) : z;
            }
        }
#pragma unroll
        for (int cb = 0; cb < kNC; ++cb)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) hold_reg(qreg[cb][ks]);

        f32x16 o[kNC][DT];
#pragma unroll
        for (int cb = 0; cb < kNC; ++cb)
#pragma unroll
            for (int i = 0; i < DT; ++i)
#pragma unroll
                for (int e = 0; e < 16; ++e) o[cb][i][e] = 0.f;
        float m_run[kNC], l_run[kNC];  // running reference max (log2 units), this lane's half of the sum
#pragma unroll
        for (int cb = 0; cb < kNC; ++cb) {
            m_run[cb] = -INFINITY;
            l_run[cb] = 0.f;
        }

        // Per-lane LDS byte offsets; everything else in the tile loop is an
        // immediate.  K operand: row 32 t + kperm(col), chunk 2 ks + hi.
        const int krow = kperm(col);
        const int kb_even = Tile::offset(krow, hi);     // chunks with (2 ks + hi) & 3 = hi
        const int kb_odd = Tile::offset(krow, 2 + hi);  // and = 2 + hi
        // V^T operand through transpose reads: lane 16 g + i points at row
        // 16 st + 8 (g >> 1) + 4 h + (i >> 2), columns 32 dt + 16 (g & 1) + 4 (i & 3).
        const int vg = lane >> 4, vi = lane & 15;
        const int vrow = 8 * (vg >> 1) + (vi >> 2), vchunk = 2 * (vg & 1) + ((vi >> 1) & 1);
        const int vb_h0 = Tile::offset(vrow, vchunk) + 8 * (vi & 1);
        const int vb_h1 = Tile::offset(vrow + 4, vchunk) + 8 * (vi & 1);

        const float c = p.c;

        // Tile building blocks: S^T = K Q^T (each K operand feeds NC MFMAs);
        // mask on diagonal / ragged tiles and online softmax (VALU only); O^T +=
        // V^T P^T (each V^T operand feeds NC MFMAs).
        auto qk_body = [&](int it, f32x16 (&sc)[kNC][kNT]) {
            const char *ks_ = (const char *)sm.k[it % kStages];
#pragma unroll
            for (int cb = 0; cb < kNC; ++cb)
#pragma unroll
                for (int t = 0; t < kNT; ++t)
#pragma unroll
                    for (int e = 0; e < 16; ++e) sc[cb][t][e] = 0.f;
            // head-dim steps outermost: consecutive MFMAs share their Q^T
            // operand and alternate between the 32-key blocks' accumulators
            // (each accumulator still sums its steps in order, so the scores
            // are the same bits as with the key blocks outermost)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
                for (int t = 0; t < kNT; ++t) {
                    const int off_ = ((ks & 1) ? kb_odd : kb_even) + (ks >> 1) * Tile::PLANE_BYTES + t * 32 * 64;
                    const u32x4 a = *(const u32x4 *)(ks_ + off_);
#pragma unroll
                    for (int cb = 0; cb < kNC; ++cb) sc[cb][t] = mfma32x32x16(a, qreg[cb][ks], sc[cb][t]);
                }
            }
        };
        auto pv_body = [&](int it, const u32x4 (&pb)[kNC][2 * kNT]) {
            const char *vs_ = (const char *)sm.v[it % kStages];
#pragma unroll
            for (int st = 0; st < 2 * kNT; ++st) {
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const int o_ = dt * Tile::PLANE_BYTES + 16 * st * 64;
                    const u32x2 lo = lds_read_tr16(vs_ + vb_h0 + o_);
                    const u32x2 hv = lds_read_tr16(vs_ + vb_h1 + o_);
                    const u32x4 va = {lo.x, lo.y, hv.x, hv.y};
#pragma unroll
                    for (int cb = 0; cb < kNC; ++cb) o[cb][dt] = mfma32x32x16(va, pb[cb][st], o[cb][dt]);
                }
            }
        };
        // Operand-read schedule of NG MFMA groups (NC MFMAs each) fed by R LDS
        // reads per group: the reads of the next GQA_FWD_PREFETCH groups are
        // issued ahead of the MFMAs, so the LDS latency overlaps earlier MFMAs.
        auto read_schedule = [&](auto ng_, auto r_) {
    #if GQA_FWD_PREFETCH
            constexpr int NG = decltype(ng_)::value, R = decltype(r_)::value;
            constexpr int PF = GQA_FWD_PREFETCH < NG ? GQA_FWD_PREFETCH : NG;
            __builtin_amdgcn_sched_group_barrier(0x100, R * PF, 0);
#pragma unroll
            for (int i = 0; i < NG - PF; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, kNC, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, kNC * PF, 0);
    #endif
        };
        auto qk = [&](int it, f32x16 (&sc)[kNC][kNT]) {
            qk_body(it, sc);
            read_schedule(std::integral_constant<int, kNT * KS>{}, std::integral_constant<int, 1>{});
        };
        auto pv = [&](int it, const u32x4 (&pb)[kNC][2 * kNT]) {
            pv_body(it, pb);
            read_schedule(std::integral_constant<int, 2 * kNT * DT>{}, std::integral_constant<int, 2>{});
        };
        auto softmax = [&](int it, f32x16 (&sc)[kNC][kNT], u32x4 (&pb)[kNC][2 * kNT]) {
            const int k0 = (t0 + it) * kBN;
            const bool need_mask = (p.causal && k0 + kBN - 1 > off + q0) || (k0 + kBN > Tk) || (win > 0 && k0 < wlo_hi);
            if (need_mask) {
#pragma unroll
                for (int cb = 0; cb < kNC; ++cb)
#pragma unroll
                    for (int t = 0; t < kNT; ++t)
#pragma unroll
                        for (int e = 0; e < 16; ++e) {
                            const int key = k0 + acc_key(t, e, hi);
                            if (key > lim[cb] || (win > 0 && key < llo[cb])) sc[cb][t][e] = -INFINITY;
                        }
            }

            // online softmax (base 2).  The weights are formed against a
            // reference that moves rarely: it is set from the tile max on a
            // lane's first tile with a visible key, and afterwards it moves (and
            // the lane's O column is rescaled) only when the lane's tile weights
            // sum past kSumCap -- an overflow to inf shows up there too -- in
            // which case the weights are formed again against the moved
            // reference.  Weights then stay below 2^16, which fp32 and bf16 carry
            // with the same relative precision as weights <= 1, and the
            // normalised result is the same softmax.  A lane moves only on its
            // own scores, so a row never depends on keys it cannot see.  In the
            // common case the block is the weights alone, written for
            // instruction-level parallelism (its latency is exposed beside
            // another wave's MFMAs): four independent row-sum chains, one check.
            float ts[kNC];  // this lane's sum of the tile's weights
            auto weights = [&]() {
#pragma unroll
                for (int cb = 0; cb < kNC; ++cb) {
                    const float m_use = (m_run[cb] == -INFINITY) ? 0.f : m_run[cb];
                    float part[2 * kNT];
#pragma unroll
                    for (int t = 0; t < kNT; ++t) {
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            float pv[8];
#pragma unroll
                            for (int e = 0; e < 8; ++e)
                                pv[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[cb][t][8 * h + e], c, -m_use));
                            u32x4 pk;
                            pk.x = pack_bf16x2(pv[0], pv[1]);
                            pk.y = pack_bf16x2(pv[2], pv[3]);
                            pk.z = pack_bf16x2(pv[4], pv[5]);
                            pk.w = pack_bf16x2(pv[6], pv[7]);
                            part[2 * t + h] = sum_bf16x8(pk, 0.f);
                            pb[cb][2 * t + h] = pk;
                        }
                    }
                    float acc = part[0];
#pragma unroll
                    for (int i = 1; i < 2 * kNT; ++i) acc += part[i];
                    ts[cb] = acc;
                }
            };
            // move the reference of every lane whose tile max exceeds it by more
            // than 2^8 (the tile max as a tree of v_max3, log2 units)
            auto move_ref = [&]() {
#pragma unroll
                for (int cb = 0; cb < kNC; ++cb) {
                    constexpr int NV = 16 * kNT;
                    float m1[NV];
#pragma unroll
                    for (int t = 0; t < kNT; ++t)
#pragma unroll
                        for (int e = 0; e < 16; ++e) m1[16 * t + e] = sc[cb][t][e];
                    int n_ = NV;
#pragma unroll
                    for (int r = 0; r < 6; ++r) {
                        if (n_ == 1) break;
                        const int out = (n_ + 2) / 3;
#pragma unroll
                        for (int e = 0; e < out; ++e) {
                            const int a = 3 * e;
                            m1[e] = a + 2 < n_ ? vmax3(m1[a], m1[a + 1], m1[a + 2])
                                               : (a + 1 < n_ ? vmax(m1[a], m1[a + 1]) : m1[a]);
                        }
                        n_ = out;
                    }
                    const float mt = halves_vmax(m1[0]) * c;
                    const float m_new = (mt > m_run[cb] + 8.0f) ? mt : m_run[cb];
                    const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run[cb] - m_new);
                    m_run[cb] = m_new;
                    l_run[cb] *= alpha;
#pragma unroll
                    for (int i = 0; i < DT; ++i)
#pragma unroll
                        for (int e = 0; e < 16; ++e) o[cb][i][e] *= alpha;
                }
            };
            bool fresh = false;
#pragma unroll
            for (int cb = 0; cb < kNC; ++cb) fresh |= m_run[cb] == -INFINITY;
            if (__any(fresh)) move_ref();
            weights();
            bool big = false;
#pragma unroll
            for (int cb = 0; cb < kNC; ++cb) big |= !(ts[cb] <= kSumCap);
            if (__any(big)) {
                move_ref();
                weights();
            }
#pragma unroll
            for (int cb = 0; cb < kNC; ++cb) l_run[cb] += ts[cb];
        };

        // ring of kStages K/V slots, filled kStages - 1 tiles ahead
#pragma unroll
        for (int s_ = 0; s_ < kStages - 1; ++s_)
            if (s_ < ntiles) issue_kv(s_, s_);
        auto live = [&](int it) {  // tile t0 + it has keys this wave sees
            const int k0 = (t0 + it) * kBN;
            return wave_active && k0 <= wlast && (win <= 0 || k0 + kBN - 1 >= wfirst);
        };
        f32x16 sc[kNC][kNT];
        u32x4 pb[kNC][2 * kNT];
        for (int it = 0; it < ntiles; ++it) {
            if (it + kStages - 2 < ntiles)
                wait_vmem_le<(kStages - 2) * 2 * NINS>();  // tile it landed; later ones may fly
            else
                wait_vmem();
            lds_barrier();  // tile it visible; the slot of tile it-1 is free
            const int nx = it + kStages - 1;
            if (nx < ntiles) issue_kv(nx, nx % kStages);
            if (live(it)) {
                qk(it, sc);
                softmax(it, sc, pb);
                pv(it, pb);
            }
        }

        if (wave_active) {
            if constexpr (PART) {
#pragma unroll
                for (int cb = 0; cb < kNC; ++cb) {
                    const int qi = q0 + 32 * cb + col;
                    if (qi >= Tq) continue;
                    const float l_tot = halves_sum(l_run[cb]);
                    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
                    const size_t row = ((size_t)b * p.Hq + head) * p.Tq + qi;
                    float *orow = p.out_f32 + row * D;
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const f32x4 v4 = {o[cb][dt][4 * j] * inv, o[cb][dt][4 * j + 1] * inv,
                                              o[cb][dt][4 * j + 2] * inv, o[cb][dt][4 * j + 3] * inv};
                            *(f32x4 *)(orow + 32 * dt + 8 * j + 4 * hi) = v4;
                        }
                    // lse = ln(sum of exp(scale * s)) = ln 2 * (m + log2 l) in the
                    // kernel's base-2 units; no visible key: -inf (weighs nothing)
                    if (hi == 0) p.lse[row] = l_tot > 0.f ? 0.69314718055994531f * (m_run[cb] + __log2f(l_tot)) : -INFINITY;
                }
            } else {
#pragma unroll
                for (int cb = 0; cb < kNC; ++cb) {
                    const int qi = q0 + 32 * cb + col;
                    if (qi >= Tq) continue;
                    const float l_tot = halves_sum(l_run[cb]);
                    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
                    uint16_t *orow = VAR ? p.out + (size_t)head * p.o_sh + (size_t)(sq0 + qi) * p.o_st
                                         : p.out + (((size_t)b * p.Hq + head) * p.Tq + qi) * D;
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const int d = 32 * dt + 8 * j + 4 * hi;
                            u32x2 pk;
                            pk.x = pack_bf16x2(o[cb][dt][4 * j + 0] * inv, o[cb][dt][4 * j + 1] * inv);
                            pk.y = pack_bf16x2(o[cb][dt][4 * j + 2] * inv, o[cb][dt][4 * j + 3] * inv);
                            *(u32x2 *)(orow + d) = pk;
                        }
                    }
                }
            }
        }
        if (!looping) break;
        lds_barrier();  // every wave is done with the ring before the next item's copies
    }
}


} // namespace

int launch_fwd_bf16(const FwdArgs &a, int D, hipStream_t stream)
{
    const long long items = (long long)a.n_units * a.n_qt;
    if (items <= 0 || items > 0x7fffffffLL) return -1;
    // Dense D = 128 with more items than one resident round of workgroups
    // (one per CU on the 256 CUs of an MI355X): that round loops over the
    // items in the kernel's snake order, which gives every workgroup the
    // same number of key tiles when each XCD's share is whole units (same
    // causal profile) and an even number of items per workgroup (checked by
    // brute force over all such shapes up to 129 units x 199 query tiles).
    // Any other launch takes one item per workgroup, in dispatch order.
    const long long per_xcd = items / 8, nwx = kResidentBlocks / 8;
    const bool looping = D == 128 && !a.varlen && items > kResidentBlocks && items % 8 == 0 &&
                         per_xcd % a.n_qt == 0 && a.n_qt % 2 == 0 && per_xcd % nwx == 0 && (per_xcd / nwx) % 2 == 0;
    const long long nblk = looping ? kResidentBlocks : items;
    dim3 grid((unsigned)nblk), block(kThreads);
    if (D == 128 && !a.varlen)
        hipLaunchKernelGGL((fwd_bf16_kernel<128, false>), grid, block, 0, stream, a);
    else if (D == 64 && !a.varlen)
        hipLaunchKernelGGL((fwd_bf16_kernel<64, false>), grid, block, 0, stream, a);
    else if (D == 128)
        hipLaunchKernelGGL((fwd_bf16_kernel<128, true>), grid, block, 0, stream, a);
    else if (D == 64)
        hipLaunchKernelGGL((fwd_bf16_kernel<64, true>), grid, block, 0, stream, a);
    else
        return -1;
    return 0;
}

int launch_fwd_bf16_shard(const FwdArgs &a, int D, hipStream_t stream)
{
    const long long nblk = (long long)a.n_units * a.n_qt;
    if (nblk <= 0 || nblk > 0x7fffffffLL || a.varlen || !a.out_f32 || !a.lse) return -1;
    dim3 grid((unsigned)nblk), block(kThreads);
    if (D == 128)
        hipLaunchKernelGGL((fwd_bf16_kernel<128, false, true>), grid, block, 0, stream, a);
    else if (D == 64)
        hipLaunchKernelGGL((fwd_bf16_kernel<64, false, true>), grid, block, 0, stream, a);
    else
        return -1;
    return 0;
}

int fwd_bf16_waves_per_block() { return kNW; }
int fwd_bf16_rows_per_wave() { return 32 * kNC; }

} // namespace gqa
