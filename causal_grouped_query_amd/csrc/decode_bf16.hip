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
//
// Two schedules share this tile computation: decode_bf16_kernel cuts every
// sequence into S equal chunks (one workgroup each), decode_bf16_flat_kernel
// shares all key tiles of all sequences out evenly over a fixed number of
// workgroups (used for S >= 3; ragged lengths then cost no balance).
//
// The flat kernel also reads an FP8 cache (template flag F8): E4M3 codes
// with one fp32 scale per (b, h, t) row, the block-scaled FP8 form of
// "Attention Architecture Evolution" (DSA section) with a block of a whole
// row.  The raw tile (half the bytes) and its 64 row scales come in through
// the same copy ring, row-major with the 16-byte chunks of row r rotated by
// XOR with (r >> 1) so that the operand reads below spread over the LDS
// banks.  MFMA operands are read straight from the codes and converted
// exactly to bf16 in registers (v_cvt_scalef32_pk_bf16_fp8 with scale 1:
// every E4M3 value is a bf16 value): K rows as 8-byte reads, V^T with the
// 8-bit transpose read ds_read_b64_tr_b8 (in each 16-lane group, lane i
// receives byte i & 7 of the 8-byte chunks addressed by lanes 2 r + (i >> 3),
// r = 0..7, in that order; checked with an in-bounds probe).  Scores are
// multiplied by the key's scale; the value scale is folded into the bf16
// weight of the P V product, and the normaliser sums the unscaled fp32
// weights.
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace gqa {

namespace {

constexpr int kTK = 32;  // keys per tile
#ifndef GQA_DEC_NT
#define GQA_DEC_NT 1
#endif
// The KV rows are read once per call: non-temporal copies (device_common.h).
// After the forward kernel, whose output lines are still dirty in the
// caches, the GQA decode then streams at 216 instead of 234 us, 221 instead
// of 224 us alone, and the FP8 decode takes 111 instead of 124 us (one box).
constexpr bool kCopyNT = GQA_DEC_NT;
#ifndef GQA_DEC_LAST_PCT
#define GQA_DEC_LAST_PCT 10
#endif
constexpr long long kLastPct = GQA_DEC_LAST_PCT;  // share of the key tiles left to the pieces after the first round
#ifndef GQA_DEC_QUEUE_MIN_TILES
#define GQA_DEC_QUEUE_MIN_TILES 48
#endif
// the piece queue is used when the first round holds at least this many key
// tiles per workgroup (shorter decodes lose more to a ticket per piece than
// their tail costs: at 32 the ragged decode of 32 sequences was 3 us slower)
constexpr long long kQueueMinTiles = GQA_DEC_QUEUE_MIN_TILES;
#ifndef GQA_DEC_STAGES
#define GQA_DEC_STAGES 2  // K/V ring depth for the 128-dim kernel
#endif

template <int DK, int DV, int STAGES>
struct DecSmem {
    uint16_t k[STAGES][kTK * DK];
    uint16_t v[STAGES][kTK * DV];
};

// FP8 flat decode: a ring of raw tiles (codes and row scales)
template <int DK, int DV, int STAGES>
struct DecSmemF8 {
    uint8_t kq[STAGES][kTK * DK];
    uint8_t vq[STAGES][kTK * DV];
    float sc[STAGES][2 * kTK];  // key scales of the tile's 32 rows, then value scales
};

// E4M3 codes -> bf16, exact: 8 codes (bytes of x, then of y) to 8 bf16
__device__ __forceinline__ u32x4 e4m3x8_to_bf16(u32x2 c)
{
    u32x4 r;
    r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.x, 1.0f, false));
    r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.x, 1.0f, true));
    r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.y, 1.0f, false));
    r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.y, 1.0f, true));
    return r;
}

// 8-bit transpose read (ds_read_b64_tr_b8), lane layout in the header comment
__device__ __forceinline__ u32x2 lds_read_tr8(const void *lds_addr)
{
    typedef int i32x2 __attribute__((ext_vector_type(2)));
    i32x2 r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((GQA_LDS i32x2 *)lds_addr);
    return __builtin_bit_cast(u32x2, r);
}

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
    debug_nanfill(sm);

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
    int kst = 0;  // sliding window: the last `window` keys only, rows kst ..
    if (p.window > 0 && len > p.window) {
        kst = len - p.window;
        len = p.window;
    }
    const int kbeg = split * p.chunk;
    const int kend = min(len, kbeg + p.chunk);
    const int ntiles = kend > kbeg ? (kend - kbeg + kTK - 1) / kTK : 0;

    const uint16_t *kb = (const uint16_t *)p.k + (size_t)b * p.k_sb + (size_t)kvh * p.k_sh + (size_t)kst * p.k_st;
    const uint16_t *vb = (const uint16_t *)p.v + (size_t)b * p.v_sb + (size_t)kvh * p.v_sh + (size_t)kst * p.v_st;

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
            for (int j = 0; j < KINS; ++j) g2lds16<kCopyNT>(k0p, koff_[j], &sm.k[slot][(j * NW + w) * 64 * 8]);
#pragma unroll
            for (int j = 0; j < VINS; ++j) g2lds16<kCopyNT>(v0p, voff_[j], &sm.v[slot][(j * NW + w) * 64 * 8]);
        } else {
            // ragged last tile: rows past the chunk end re-read its last key
            // (in bounds; masked below)
#pragma unroll
            for (int j = 0; j < KINS; ++j) {
                const int row = min(k0 + krow_[j], kend - 1);
                g2lds16<kCopyNT>((const char *)(kb + (size_t)row * p.k_st) + (koff_[j] - (unsigned)(krow_[j] * p.k_st) * 2u),
                        &sm.k[slot][(j * NW + w) * 64 * 8]);
            }
#pragma unroll
            for (int j = 0; j < VINS; ++j) {
                const int row = min(k0 + vrow_[j], kend - 1);
                g2lds16<kCopyNT>((const char *)(vb + (size_t)row * p.v_st) + (voff_[j] - (unsigned)(vrow_[j] * p.v_st) * 2u),
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
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            store_partial4(p.part_o, prow * DV + 32 * dt + 8 * j + 4 * hi, o[dt][4 * j] * inv,
                           o[dt][4 * j + 1] * inv, o[dt][4 * j + 2] * inv, o[dt][4 * j + 3] * inv);
    // empty chunk: o = 0 and lse = -inf, so it weighs nothing in the merge
    if (hi == 0) p.part_lse[prow] = l_tot > 0.f ? m_run + __log2f(l_tot) : -INFINITY;
}

// ---------------------------------------------------------------------------
// Flat decode: the same tile computation, but the work is balanced instead of
// cut into fixed chunks per sequence.  All (batch, KV head, head block)
// streams are laid end to end as one sequence of T key tiles (stream w of
// batch b holds ceil(len_b / 32) tiles); workgroup i of the N that run takes
// the contiguous tiles [i T / N, (i+1) T / N).  Ragged lengths therefore cost
// nothing in balance, and each workgroup starts up once.  A workgroup writes
// one normalised partial (o, lse) for every stream piece it covers, into
// partial slot i - (first workgroup of that stream); the workgroup holding a
// stream's first tile marks the slots past the stream's last piece empty
// (lse = -inf), so the combine merges all S slots as for the chunked
// schedule.  N is
// capped so that no stream is cut into more than S pieces: consecutive cuts
// are at least floor(T / N) tiles apart, so a stream of n tiles has at most
// (n - 2) / floor(T / N) + 2 pieces.
template <int DK, int DV, int STAGES, bool F8>
__global__ __launch_bounds__(64, 2) void decode_bf16_flat_kernel(DecodeArgs p)
{
    constexpr int NT = 64;
    constexpr int EB = F8 ? 1 : 2;                  // bytes per cached element
    constexpr int CPRK = DK * EB / 16, CPRV = DV * EB / 16;  // 16-byte copies per row
    constexpr int KS = DK / 16;
    constexpr int DT = DV / 32;
    constexpr int KINS = kTK * CPRK / NT;
    constexpr int VINS = kTK * CPRV / NT;
    constexpr int NI = KINS + VINS + (F8 ? 1 : 0);  // + one copy of the tile's row scales
    static_assert(kTK * CPRK % NT == 0 && kTK * CPRV % NT == 0, "tile must split evenly");
    static_assert(STAGES >= 2 && (STAGES - 2) * NI < 64, "ring depth");

    using Smem = typename std::conditional<F8, DecSmemF8<DK, DV, STAGES>, DecSmem<DK, DV, STAGES>>::type;
    __shared__ __attribute__((aligned(1024))) Smem sm;
    debug_nanfill(sm);

    const int lane = threadIdx.x;
    const int col = lane & 31, hi = lane >> 5;
    const int H = p.Hkv * p.n_hblk;  // streams per batch
    // keys a sequence's query attends to: the clamped length, or with a
    // sliding window its last `window` keys
    auto eff_len = [&](int len) {
        len = len < 0 ? 0 : (len > p.Tmax ? p.Tmax : len);
        return (p.window > 0 && len > p.window) ? p.window : len;
    };
    auto ntile = [&](int len) { return (eff_len(len) + kTK - 1) / kTK; };

    // ---- total tiles T and the longest stream (every workgroup computes them) ----
    long long tsum = 0;
    int nmax = 0;
    for (int b0 = 0; b0 < p.B; b0 += 64) {
        const int n = b0 + lane < p.B ? ntile(p.lens[b0 + lane]) : 0;
        tsum += n;
        nmax = max(nmax, n);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        tsum += __shfl_xor(tsum, o);
        nmax = max(nmax, __shfl_xor(nmax, o));
    }
    const long long T = tsum * H;
    if (blockIdx.x == 0) {
        // rows of empty sequences get no piece: mark all their partial slots
        // empty (lse = -inf), so the combine writes zeros for them
        for (int b0 = 0; b0 < p.B; b0 += 64) {
            unsigned long long empty = __ballot(b0 + lane < p.B && ntile(p.lens[b0 + lane]) == 0);
            while (empty) {
                const int b = b0 + __ffsll((long long)empty) - 1;
                empty &= empty - 1;
                for (int i = lane; i < p.Hq * p.S; i += 64) p.part_lse[(size_t)b * p.Hq * p.S + i] = -INFINITY;
            }
        }
    }
    if (T == 0) return;
    const long long S2 = p.S - 2;  // the host uses this kernel only for S >= 3
    long long ne = T * S2 / ((nmax > 2 ? nmax - 2 : 0) + S2);
    ne = ne < 1 ? 1 : (ne > p.n_wg ? p.n_wg : ne);
    const long long N = ne;
    if ((long long)blockIdx.x >= N) return;
    // Piece sizes.  Every piece holds at least floor(T / N) >= m tiles,
    // m = floor((nmax - 2) / (S - 1)) + 1, and a stream of n tiles meets at
    // most floor((n - 2) / m) + 2 <= S pieces.  Equal pieces, one per
    // workgroup, unless the work is long enough for the queue: then the
    // first round (nl pieces, one per resident workgroup) takes the large
    // share and the pieces after it only ~kLastPct % of the tiles (never
    // below m tiles each), handed out through a device-wide counter
    // (below), so that compute units, and whole XCDs, that stream faster
    // take more of the small pieces and all of them finish closer together.
    // (The dispatcher alone cannot do this: it deals workgroups to the XCDs
    // round-robin, so every XCD gets the same share of the pieces.)
    const long long nl = p.n_first;
    const bool queue = p.queue && nl > 0 && N > nl && T >= nl * kQueueMinTiles;
    long long n1 = N, T1 = T;  // equal pieces: one region
    if (queue) {
        const long long m = (nmax > 2 ? (nmax - 2) / (p.S - 1) : 0) + 1;
        const long long n2 = N - nl;
        long long ts = (T * kLastPct + 99) / 100;
        if (ts < n2 * m) ts = n2 * m;
        if (ts * N <= T * n2) {  // small pieces no larger than equal ones
            n1 = nl;
            T1 = T - ts;
        }
    }
    auto bnd = [&](long long w) {  // first tile of piece w (w <= N)
        return w <= n1 ? w * T1 / n1 : T1 + (w - n1) * (T - T1) / (N - n1);
    };
    auto wg_of = [&](long long t) {  // piece whose range holds tile t
        long long x = t < T1 ? t * n1 / T1 : n1 + (t - T1) * (N - n1) / (T - T1);
        while (x + 1 < N && bnd(x + 1) <= t) ++x;
        return x;
    };

    // ---- cursors over (batch b, stream s of the batch, tile u of the stream) ----
    // (all fields are wave-uniform and kept in scalar registers, so the
    // length of the next batch is a scalar load: a vector load here would
    // make the compiler drain the copy ring with vmcnt(0) on every tile)
    struct Cur {
        int b, s, u, n;    // n = tiles per stream of batch b
        int len;           // keys batch b attends to (clamped, windowed)
        int kst;           // cache row of its first key (window start)
        long long base;    // global index of batch b's first tile
        int lens64, chunk; // lengths of batches 64 chunk + lane (one per lane)
    };
    auto uni = [](int x) { return __builtin_amdgcn_readfirstlane(x); };
    auto uni64 = [](long long x) {
        const unsigned lo32 = __builtin_amdgcn_readfirstlane((unsigned)x);
        const unsigned hi32 = __builtin_amdgcn_readfirstlane((unsigned)((unsigned long long)x >> 32));
        return (long long)(((unsigned long long)hi32 << 32) | lo32);
    };
    auto clamp_len = [&](int len) { return len < 0 ? 0 : (len > p.Tmax ? p.Tmax : len); };
    auto set_len = [&](Cur &c, int clamped) {  // window: the last `window` keys
        c.len = (p.window > 0 && clamped > p.window) ? p.window : clamped;
        c.kst = uni(clamped - c.len);
    };
    auto locate = [&](long long t) {
        Cur c;
        long long base = 0;
        for (int b0 = 0;; b0 += 64) {
            const int b = b0 + lane;
            const long long v = b < p.B ? (long long)ntile(p.lens[b]) * H : 0;
            long long incl = v;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const long long y = __shfl_up(incl, o);
                if (lane >= o) incl += y;
            }
            const unsigned long long hit = __ballot(b < p.B && base + incl > t);
            if (hit) {
                const int L = __ffsll((long long)hit) - 1;
                const long long incl_l = __shfl(incl, L), v_l = __shfl(v, L);
                c.b = uni(b0 + L);
                c.base = uni64(base + incl_l - v_l);
                c.n = uni((int)(v_l / H));
                const long long rel = t - c.base;
                c.s = uni((int)(rel / c.n));
                c.u = uni((int)(rel % c.n));
                c.chunk = uni(b0 >> 6);
                c.lens64 = b < p.B ? clamp_len(p.lens[b]) : 0;
                set_len(c, __builtin_amdgcn_readlane(c.lens64, L));
                return c;
            }
            base += __shfl(incl, 63);
        }
    };
    auto advance = [&](Cur &c) {
        if (++c.u < c.n) return;
        c.u = 0;
        if (++c.s < H) return;
        c.s = 0;
        c.base += (long long)H * c.n;
        do {
            c.b = uni(c.b + 1);
            if (c.b >= p.B) {  // past the last batch (only the copy cursor gets here)
                c.len = kTK;
                c.kst = 0;
            } else {
                if ((c.b >> 6) != c.chunk) {  // next 64 batches: one vector load
                    c.chunk = c.b >> 6;
                    const int bb = 64 * c.chunk + lane;
                    c.lens64 = bb < p.B ? clamp_len(p.lens[bb]) : 0;
                }
                set_len(c, __builtin_amdgcn_readlane(c.lens64, c.b & 63));
            }
            c.n = (c.len + kTK - 1) / kTK;
        } while (c.n == 0);
    };

    using Tile = PlaneTile<kTK>;
    // Source (row, 16-byte chunk) of each of this lane's copies: the bf16
    // tile in plane layout, or (F8) the raw tile row-major, slot q at byte
    // 16 q: row q / CPR, and position q % CPR holds chunk position ^ sw(row),
    // sw(row) = (row >> 1) mod CPR.
    auto src_of = [&](int q, int cpr, int &row, int &chunk) {
        if constexpr (F8) {
            row = q / cpr;
            chunk = (q % cpr) ^ ((row >> 1) & (cpr - 1));
        } else {
            (void)cpr;
            Tile::slot_source(q, row, chunk);
        }
    };
    int krow_[KINS], vrow_[VINS];
    unsigned koff_[KINS], voff_[VINS];
#pragma unroll
    for (int j = 0; j < KINS; ++j) {
        int row, chunk;
        src_of(j * 64 + lane, CPRK, row, chunk);
        krow_[j] = row;
        koff_[j] = F8 ? (unsigned)(row * p.k_st + chunk * 16) : (unsigned)(row * p.k_st + chunk * 8) * 2u;
    }
#pragma unroll
    for (int j = 0; j < VINS; ++j) {
        int row, chunk;
        src_of(j * 64 + lane, CPRV, row, chunk);
        vrow_[j] = row;
        voff_[j] = F8 ? (unsigned)(row * p.v_st + chunk * 16) : (unsigned)(row * p.v_st + chunk * 8) * 2u;
    }
    // LDS destinations of copy j (a wave writes 64 consecutive 16-byte slots)
    auto kdst = [&](int slot, int j) -> void * {
        if constexpr (F8) return &sm.kq[slot][j * 64 * 16];
        else return &sm.k[slot][j * 64 * 8];
    };
    auto vdst = [&](int slot, int j) -> void * {
        if constexpr (F8) return &sm.vq[slot][j * 64 * 16];
        else return &sm.v[slot][j * 64 * 8];
    };
    // copy the tile under cursor c into ring slot `slot`
    // element type of the cached rows: bf16, or one-byte codes
    using Elem = typename std::conditional<F8, uint8_t, uint16_t>::type;
    auto issue_tile = [&](const Cur &c, int slot) {
        const int kvh = c.s / p.n_hblk;
        const int len = c.len;
        const int k0 = c.u * kTK;
        const Elem *kb = (const Elem *)p.k + (size_t)c.b * p.k_sb + (size_t)kvh * p.k_sh + (size_t)c.kst * p.k_st;
        const Elem *vb = (const Elem *)p.v + (size_t)c.b * p.v_sb + (size_t)kvh * p.v_sh + (size_t)c.kst * p.v_st;
        if (k0 + kTK <= len) {
            const Elem *k0p = kb + (size_t)k0 * p.k_st;
            const Elem *v0p = vb + (size_t)k0 * p.v_st;
#pragma unroll
            for (int j = 0; j < KINS; ++j) g2lds16<kCopyNT>(k0p, koff_[j], kdst(slot, j));
#pragma unroll
            for (int j = 0; j < VINS; ++j) g2lds16<kCopyNT>(v0p, voff_[j], vdst(slot, j));
        } else {
            // ragged last tile: rows past the sequence end re-read its last
            // key (in bounds; masked below)
#pragma unroll
            for (int j = 0; j < KINS; ++j) {
                const int row = min(k0 + krow_[j], len - 1);
                g2lds16<kCopyNT>((const char *)(kb + (size_t)row * p.k_st) + (koff_[j] - (unsigned)(krow_[j] * p.k_st) * (unsigned)EB),
                        kdst(slot, j));
            }
#pragma unroll
            for (int j = 0; j < VINS; ++j) {
                const int row = min(k0 + vrow_[j], len - 1);
                g2lds16<kCopyNT>((const char *)(vb + (size_t)row * p.v_st) + (voff_[j] - (unsigned)(vrow_[j] * p.v_st) * (unsigned)EB),
                        vdst(slot, j));
            }
        }
        if constexpr (F8) {
            // row scales: lanes 0-31 the keys', 32-63 the values' (rows past
            // the sequence end re-read its last row)
            const int r = c.kst + min(k0 + (lane & 31), len - 1);
            const float *sp = lane < 32
                ? p.k_scale + (size_t)c.b * p.ks_sb + (size_t)kvh * p.ks_sh + (size_t)r * p.ks_st
                : p.v_scale + (size_t)c.b * p.vs_sb + (size_t)kvh * p.vs_sh + (size_t)r * p.vs_st;
            g2lds4<kCopyNT>(sp, &sm.sc[slot][0]);
        }
    };

    const int krow = kperm(col);
    const int kbase_even = Tile::offset(krow, hi);
    const int kbase_odd = Tile::offset(krow, 2 + hi);
    const int vg = lane >> 4, vi = lane & 15;
    const int vrow = 8 * (vg >> 1) + (vi >> 2), vchunk = 2 * (vg & 1) + ((vi >> 1) & 1);
    const int vb_h0 = Tile::offset(vrow, vchunk) + 8 * (vi & 1);
    const int vb_h1 = Tile::offset(vrow + 4, vchunk) + 8 * (vi & 1);
    // F8 operand reads from the raw (swizzled) tiles: K row krow, half hi;
    // V^T lane roles (group g = lane >> 4, i = lane & 15: r = i >> 1, h = i & 1)
    const int k8_base = krow * DK + 8 * hi;
    const int k8_sw = (krow >> 1) & (CPRK - 1);
    const int v8_row = 8 * (vg >> 1) + (vi >> 1);
    const int v8_h = vi & 1, v8_g1 = vg & 1;
    const float c = p.c;

    // The queue: workgroup i < nl takes first-round piece i and ends; the
    // dispatcher then starts the later workgroups of each XCD as its slots
    // free, and each of them takes piece nl + t for every ticket t it draws
    // from the counter until the tickets run out.  Workgroup 0 zeroes the
    // counter as it starts, before any slot frees, and itself draws after
    // its first piece until the tickets run out, so every piece is computed
    // whenever the others start.  A draw that still read the previous
    // call's value takes a piece past the end (none) or one that is drawn
    // again after the reset: the two compute the same values into the same
    // slots.
    if (queue && blockIdx.x == 0 && lane == 0)
        __hip_atomic_store(p.queue, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool draws = queue && (blockIdx.x == 0 || (long long)blockIdx.x >= nl);
    // (the ticket is unsigned: readfirstlane returns an int, and a stale
    // count of 2^31 or more must not become a negative piece index)
    auto draw = [&]() -> long long {
        unsigned t = 0;
        if (lane == 0) t = __hip_atomic_fetch_add(p.queue, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return nl + (long long)(unsigned)__builtin_amdgcn_readfirstlane((int)t);
    };
    const long long wi0 = (queue && (long long)blockIdx.x >= nl) ? draw() : (long long)blockIdx.x;
    for (long long wi = wi0; wi < N; wi = draws ? draw() : N) {
        const long long lo = bnd(wi), hi_t = bnd(wi + 1);
        if (lo >= hi_t) continue;
        const int ntl = (int)(hi_t - lo);  // tiles of this piece
        Cur dc = locate(lo);               // copy cursor (runs STAGES-1 tiles ahead)
        Cur cc = dc;                       // compute cursor
#pragma unroll
        for (int s = 0; s < STAGES - 1; ++s)
            if (s < ntl) {
                issue_tile(dc, s);
                advance(dc);
            }

        u32x4 qreg[KS];
        f32x16 o[DT];
        float m_run = -INFINITY, l_run = 0.f;
        bool head_ok = false;
        int head = 0;
        for (int it = 0; it < ntl; ++it) {
            const int slot = it % STAGES;
            if (it + STAGES - 2 < ntl)
                wait_vmem_le<(STAGES - 2) * NI>();  // tile `it` landed, later ones may fly
            else
                wait_vmem();
            lds_barrier();  // this wave's reads of the slot being refilled are complete
            if (it + STAGES - 1 < ntl) {
                issue_tile(dc, (it + STAGES - 1) % STAGES);
                advance(dc);
            }

            const int kvh = cc.s / p.n_hblk, hblk = cc.s % p.n_hblk;
            if (it == 0 || cc.u == 0) {
                // a new stream piece: its queries, fresh accumulators
                const int hh = hblk * 32 + col;
                head_ok = hh < p.G;
                head = kvh * p.G + (head_ok ? hh : 0);
                const uint16_t *qrow = (const uint16_t *)p.q + ((size_t)cc.b * p.Hq + head) * DK;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    u32x4 z = {0u, 0u, 0u, 0u};
                    qreg[ks] = head_ok ? *(const u32x4 *)(qrow + 16 * ks + 8 * hi) : z;
                }
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) hold_reg(qreg[ks]);
#pragma unroll
                for (int i = 0; i < DT; ++i)
#pragma unroll
                    for (int e = 0; e < 16; ++e) o[i][e] = 0.f;
                m_run = -INFINITY;
                l_run = 0.f;
            }
            const int kend = cc.len;
            const int k0 = cc.u * kTK;

            // element e of the score accumulator is key acc_key(0, e, hi): keys
            // 8 hi + 0..7 and 16 + 8 hi + 0..7 of the tile
            auto row_scales = [&](int base, float (&dst)[16]) {
                if constexpr (F8) {
                    const float *sc = &sm.sc[slot][base];
#pragma unroll
                    for (int e = 0; e < 16; ++e) dst[e] = sc[acc_key(0, e, hi)];
                }
            };

            f32x16 s;
#pragma unroll
            for (int e = 0; e < 16; ++e) s[e] = 0.f;
            if constexpr (F8) {
                // K operand: lane (col, hi) takes dims 16 ks + 8 hi .. + 7 of key
                // row krow: 8 codes of chunk ks, stored at position ks ^ sw(krow)
                const char *kq_ = (const char *)sm.kq[slot];
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const u32x2 c8 = *(const u32x2 *)(kq_ + k8_base + ((ks ^ k8_sw) << 4));
                    s = mfma32x32x16(e4m3x8_to_bf16(c8), qreg[ks], s);
                }
            } else {
                const char *ks_ = (const char *)sm.k[slot];
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const int off_ = ((ks & 1) ? kbase_odd : kbase_even) + (ks >> 1) * Tile::PLANE_BYTES;
                    s = mfma32x32x16(*(const u32x4 *)(ks_ + off_), qreg[ks], s);
                }
            }
            if constexpr (F8) {
                float ksc[16];  // the keys' row scales
                row_scales(0, ksc);
#pragma unroll
                for (int e = 0; e < 16; ++e) s[e] *= ksc[e];
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
                for (int i = 0; i < DT; ++i)
#pragma unroll
                    for (int e = 0; e < 16; ++e) o[i][e] *= alpha;
            }
            const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
            float vsc[16];  // F8: the values' row scales
            if constexpr (F8) row_scales(kTK, vsc);
            u32x4 pb[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                float pv[8];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    pv[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * h + e], c, -m_use));
                if constexpr (F8) {
                    // value scales ride on the weights; the normaliser takes the
                    // unscaled ones
#pragma unroll
                    for (int e = 0; e < 8; ++e) l_run += pv[e];
#pragma unroll
                    for (int e = 0; e < 8; ++e) pv[e] *= vsc[8 * h + e];
                }
                pb[h].x = pack_bf16x2(pv[0], pv[1]);
                pb[h].y = pack_bf16x2(pv[2], pv[3]);
                pb[h].z = pack_bf16x2(pv[4], pv[5]);
                pb[h].w = pack_bf16x2(pv[6], pv[7]);
                if constexpr (!F8) l_run = sum_bf16x8(pb[h], l_run);
            }
            if constexpr (F8) {
                // V^T operand of step st, dims 32 dt ..: in 16-lane group g, lane
                // 2 r + h points at key row 16 st + 8 (g >> 1) + r, dims
                // 32 dt + 16 (g & 1) + 8 h .. + 7 (chunk 2 dt + (g & 1), half h);
                // lane i then holds dim 32 dt + 16 (g & 1) + i of keys
                // 16 st + 8 (g >> 1) + 0..7, the keys of its P^T slice
                const char *vq_ = (const char *)sm.vq[slot];
#pragma unroll
                for (int st = 0; st < 2; ++st) {
                    const int row = 16 * st + v8_row;
                    const int sw = (row >> 1) & (CPRV - 1);
                    const char *rp = vq_ + row * DV + 8 * v8_h;
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt) {
                        const u32x2 c8 = lds_read_tr8(rp + (((2 * dt + v8_g1) ^ sw) << 4));
                        o[dt] = mfma32x32x16(e4m3x8_to_bf16(c8), pb[st], o[dt]);
                    }
                }
            } else {
                const char *vs_ = (const char *)sm.v[slot];
#pragma unroll
                for (int st = 0; st < 2; ++st) {
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt) {
                        const int o_ = dt * Tile::PLANE_BYTES + 16 * st * 64;
                        const u32x2 lo2 = lds_read_tr16(vs_ + vb_h0 + o_);
                        const u32x2 hv = lds_read_tr16(vs_ + vb_h1 + o_);
                        u32x4 va = {lo2.x, lo2.y, hv.x, hv.y};
                        o[dt] = mfma32x32x16(va, pb[st], o[dt]);
                    }
                }
            }

            if (cc.u == cc.n - 1 || it == ntl - 1) {
                // end of this workgroup's piece of the stream: write its partial
                const long long pw = cc.base + (long long)cc.s * cc.n;  // the stream's first tile
                const long long first = wg_of(pw);
                const int j = (int)(wi - first);
                if (head_ok) {
                    const float l_tot = halves_sum(l_run);
                    const size_t prow = ((size_t)cc.b * p.Hq + head) * p.S + j;
                    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj)
                            store_partial4(p.part_o, prow * DV + 32 * dt + 8 * jj + 4 * hi, o[dt][4 * jj] * inv,
                                           o[dt][4 * jj + 1] * inv, o[dt][4 * jj + 2] * inv, o[dt][4 * jj + 3] * inv);
                    if (hi == 0) p.part_lse[prow] = l_tot > 0.f ? m_run + __log2f(l_tot) : -INFINITY;
                }
                if (j == 0 && head_ok && hi == 0) {
                    // slots past the stream's last piece are empty for the combine
                    const int count = (int)(wg_of(pw + cc.n - 1) - wi + 1);
                    const size_t prow0 = ((size_t)cc.b * p.Hq + head) * p.S;
                    for (int q = count; q < p.S; ++q) p.part_lse[prow0 + q] = -INFINITY;
                }
            }
            advance(cc);
        }
    }
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
    if (Dk == 576) return mla_heads_per_block();
    (void)G;
    return 32;
}

int decode_bf16_flat_workgroups(int Dk)
{
    // 8 per compute unit on the 256 CUs of an MI355X.  The occupancy query
    // allows 5 resident 32 KiB-LDS workgroups per CU, but measured over 1280
    // .. 3200 workgroups the ragged GQA decode is fastest at 2048 (226 us)
    // and clearly slower at 1280 (258 us) and above 2048 (244 .. 251 us).
    (void)Dk;
#ifndef GQA_DEC_WG_PER_CU
#define GQA_DEC_WG_PER_CU 8
#endif
    return GQA_DEC_WG_PER_CU * 256;
}

int decode_bf16_flat_first_round(int Dk)
{
    // D = 128: per-workgroup clocks show four of these one-wave workgroups
    // (32 KiB of LDS each) resident per compute unit at a time, 1024 on the
    // chip.  D = 64 (24 KiB) fits more than four per CU, so the whole grid
    // is its first round (equal pieces, no queue).
#ifndef GQA_DEC_FIRST_PER_CU
#define GQA_DEC_FIRST_PER_CU 4
#endif
    return Dk == 128 ? GQA_DEC_FIRST_PER_CU * 256 : decode_bf16_flat_workgroups(Dk);
}

// FP8 flat decode: one resident round of workgroups.  At 16.5 KiB of LDS
// and two waves per SIMD, eight fit a compute unit; measured on the GQA
// decode workload, 6 and 8 per CU take 121 .. 129 us, 9 per CU (a second,
// partial round) 143 .. 148 us.
#ifndef GQA_DEC_F8_WG_PER_CU
#define GQA_DEC_F8_WG_PER_CU 8
#endif
int decode_fp8_flat_workgroups(int Dk)
{
    (void)Dk;
    return GQA_DEC_F8_WG_PER_CU * 256;
}

template <int DK, int DV, int STAGES, bool F8 = false>
int launch_flat(const DecodeArgs &a, hipStream_t stream)
{
    dim3 grid(a.n_wg), block(64);
    hipLaunchKernelGGL((decode_bf16_flat_kernel<DK, DV, STAGES, F8>), grid, block, 0, stream, a);
    return 0;
}

#ifndef GQA_DEC_F8_STAGES
#define GQA_DEC_F8_STAGES 2  // raw-tile ring depth of the FP8 flat decode (128-dim)
#endif

int launch_decode_fp8(const DecodeArgs &a, int Dk, int Dv, hipStream_t stream)
{
    if (!a.fp8 || a.n_wg <= 0 || a.S < 3 || !a.k_scale || !a.v_scale) return -1;
    if (Dk == 128 && Dv == 128) return launch_flat<128, 128, GQA_DEC_F8_STAGES, true>(a, stream);
    if (Dk == 64 && Dv == 64) return launch_flat<64, 64, 3, true>(a, stream);
    return -1;
}

int launch_decode_bf16(const DecodeArgs &a, int Dk, int Dv, hipStream_t stream)
{
    if (a.n_wg > 0) {
        if (a.S < 3) return -1;
        if (Dk == 128 && Dv == 128) return launch_flat<128, 128, GQA_DEC_STAGES>(a, stream);
        if (Dk == 64 && Dv == 64) return launch_flat<64, 64, 3>(a, stream);
        return -1;
    }
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
