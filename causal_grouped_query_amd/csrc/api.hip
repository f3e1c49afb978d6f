// api.hip -- exported C ABI of libgqa_attn.so (declared in include/gqa_attn.h).
//
// Every argument is validated here, on the host, before anything is
// launched; a rejected call touches no device memory and makes no HIP call.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "gqa_attn.h"
#include "launch.h"

#define GQA_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kMaxSplits = 1024;

bool finite_nonneg(float x) { return isfinite(x) && x >= 0.f; }

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// ceil(a / b) in 64-bit arithmetic (a >= 0, b > 0): sizes near INT_MAX must
// not overflow before the range checks that reject them
long long cdiv(long long a, long long b) { return (a + b - 1) / b; }

// scale * log2(e), kept strictly positive so that masked (-inf) scores stay
// -inf after scaling; a zero scale becomes 1e-30, which leaves every weight
// exactly equal in fp32 (uniform attention, as scale = 0 means).
float folded_scale(float scale) { return fmaxf(scale * kLog2e, 1e-30f); }

bool head_dims_fwd(int Dk, int Dv) { return Dk == Dv && (Dk == 64 || Dk == 128); }

bool head_dims_decode(int Dk, int Dv, int dtype)
{
    if (Dk == Dv && (Dk == 64 || Dk == 128)) return true;
    return dtype == GQA_BF16 && Dk == 576 && Dv == 512;
}

int check_common(int B, int Hq, int Hkv, int Dk, int Dv, float scale, int dtype)
{
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Dk <= 0 || Dv <= 0) return GQA_ERR_INVALID_ARG;
    if (Hq % Hkv != 0) return GQA_ERR_INVALID_ARG;
    if (!finite_nonneg(scale)) return GQA_ERR_INVALID_ARG;
    if (dtype != GQA_BF16 && dtype != GQA_F32) return GQA_ERR_INVALID_ARG;
    return GQA_OK;
}

// Debug builds (GQA_DEBUG_NANFILL=1): poison the split-KV workspace with
// NaN bit patterns before the partial kernels run, so a slot no kernel
// writes reaches the combine as NaN.  Nothing in normal builds.
#ifndef GQA_DEBUG_NANFILL
#define GQA_DEBUG_NANFILL 0
#endif
void debug_fill_workspace(void *ws, size_t bytes, hipStream_t st)
{
#if GQA_DEBUG_NANFILL
    (void)hipMemsetAsync(ws, 0xff, bytes, st);
#else
    (void)ws;
    (void)bytes;
    (void)st;
#endif
}

int launch_status(int rc)
{
    if (rc != 0) return GQA_ERR_UNSUPPORTED;
    return hipGetLastError() == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

// Splits when the caller leaves the choice to the library.  The choice
// depends only on the shape (it assumes the 256 compute units of an MI355X)
// so that the workspace size is known before any device call.
int default_splits(int B, int Hq, int Hkv, int Tmax, int Dk, int dtype)
{
    const int G = Hq / Hkv;
    if (Dk == 576) {
        // absorbed MLA: a workgroup covers 128 query heads of a sequence and
        // one of S equal key chunks; one workgroup per CU
        const long long groups = (long long)B * Hkv * cdiv(G, 128);
        long long s = (256 + groups - 1) / groups;
        const long long cap = cdiv(Tmax, 256);
        if (s > cap) s = cap;
        if (s < 1) s = 1;
        if (s > 64) s = 64;
        return (int)s;
    }
    const long long streams = (long long)B * Hkv * cdiv(G, 32);
    if (dtype == GQA_BF16) {
        // flat decode: S bounds the pieces any stream may be cut into.  The
        // kernel cuts its T key tiles into at most ~T (S-2) / (n_max + S - 4)
        // pieces (n_max tiles in the longest stream), and the pieces after
        // its first round hold no fewer than (n_max - 2) / (S - 1) tiles.
        // With every sequence full, T = streams * n_max, so S - 2 of twice
        // the pieces per stream keeps the grid full even when the lengths
        // are ragged, and four times that lets the last pieces shrink to
        // about a quarter of an even share (measured on the ragged GQA
        // decode, 512 streams: 34, whose smallest piece is that of 32, beats
        // 10, 16, 24, 48 and 64).
        const long long wgs = gqa::decode_bf16_flat_workgroups(Dk);
        long long s = 2 + 4 * ((2 * wgs + streams - 1) / streams);
        const long long cap = 2 + cdiv(Tmax, 32);
        if (s < 8) s = 8;
        if (s > cap) s = cap;
        if (s > 64) s = 64;
        return (int)(s < 3 ? 3 : s);
    }
    // fp32 path: one workgroup per (split, batch, KV head, 32 heads of its
    // group); ~2.5 workgroups
    // per resident slot if every sequence were full length, chunks of at
    // least 256 keys
    long long s = (3200 + streams - 1) / streams;
    const long long cap = cdiv(Tmax, 256);
    if (s > cap) s = cap;
    if (s < 1) s = 1;
    if (s > 64) s = 64;
    return (int)s;
}

// FP8 flat decode: one resident round of workgroups and equal pieces (no
// piece queue), so S only needs to keep the grid full when the lengths are
// ragged: S - 2 of twice the workgroups per stream (with every sequence
// full, T = streams * n_max).  Never above the bf16 default, so a workspace
// sized for that fits.
int fp8_default_splits(int B, int Hq, int Hkv, int Tmax, int Dk)
{
    const long long streams = (long long)B * Hkv * cdiv(Hq / Hkv, 32);
    const long long wgs = gqa::decode_fp8_flat_workgroups(Dk);
    long long s = 2 + (2 * wgs + streams - 1) / streams;
    const long long cap = 2 + cdiv(Tmax, 32);
    if (s < 8) s = 8;
    if (s > cap) s = cap;
    if (s > 64) s = 64;
    const int bf16 = default_splits(B, Hq, Hkv, Tmax, Dk, GQA_BF16);
    return (int)(s < 3 ? 3 : (s > bf16 ? bf16 : s));
}

// workspace: fp32 partial outputs [B, Hq, S, Dv], then fp32 partial
// log2-sum-exp [B, Hq, S], then (at the next 256-byte boundary) 256 bytes
// for the flat decode's piece counter
constexpr size_t kQueueBytes = 256;
size_t ws_bytes(int B, int Hq, int Dv, int S)
{
    const size_t rows = (size_t)B * Hq * S;
    size_t bytes = rows * Dv * sizeof(float) + rows * sizeof(float);
    return ((bytes + 255) & ~(size_t)255) + kQueueBytes;
}

// Workgroup geometry of the bf16 forward kernel: one wave owns one query
// head x rows_per_wave positions; a workgroup takes Gt heads of the group
// (largest power of two dividing both G and the wave count) x Pt positions.
// Tq is the (largest) query count per sequence.  False if the grid is too big.
bool fwd_geometry(gqa::FwdArgs &a, int B, int Hq, int Hkv, int Tq)
{
    const int G = Hq / Hkv;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.Tq = Tq;
    a.G = G;
    const int waves = gqa::fwd_bf16_waves_per_block();
    const int rpw = gqa::fwd_bf16_rows_per_wave();
    int gt = 1;
    while (gt * 2 <= waves && G % (gt * 2) == 0 && waves % (gt * 2) == 0) gt *= 2;
    a.Gt = gt;
    a.Pt = rpw * (waves / gt);
    a.n_hblk = G / gt;
    const long long n_qt = cdiv(Tq, a.Pt);
    const long long units = (long long)B * Hkv * a.n_hblk;
    if (units * n_qt > 0x7fffffffLL) return false;
    a.n_qt = (int)n_qt;
    a.n_units = (int)units;
    return true;
}

} // namespace

GQA_API const char *gqa_attn_strerror(int code)
{
    switch (code) {
    case GQA_OK: return "success";
    case GQA_ERR_INVALID_ARG: return "invalid argument";
    case GQA_ERR_UNSUPPORTED: return "unsupported head dimension / dtype combination";
    case GQA_ERR_WORKSPACE: return "workspace missing or too small";
    case GQA_ERR_HIP: return "HIP launch error";
    default: return "unknown error code";
    }
}

GQA_API int gqa_attn_fwd(const void *q, const void *k, const void *v, void *out, int B, int Hq,
                         int Hkv, int Tq, int Tk, int Dk, int Dv, float scale, int causal,
                         gqa_dtype dtype, void *stream)
{
    if (!q || !k || !v || !out) return GQA_ERR_INVALID_ARG;
    int rc = check_common(B, Hq, Hkv, Dk, Dv, scale, dtype);
    if (rc != GQA_OK) return rc;
    if (Tq <= 0 || Tk <= 0) return GQA_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1) return GQA_ERR_INVALID_ARG;
    if (causal && Tq > Tk) return GQA_ERR_INVALID_ARG;
    if (!head_dims_fwd(Dk, Dv)) return GQA_ERR_UNSUPPORTED;
    const int G = Hq / Hkv;
    hipStream_t st = (hipStream_t)stream;

    if (dtype == GQA_BF16) {
        if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 8))
            return GQA_ERR_INVALID_ARG;
        gqa::FwdArgs a = {};
        a.q = (const uint16_t *)q;
        a.k = (const uint16_t *)k;
        a.v = (const uint16_t *)v;
        a.out = (uint16_t *)out;
        a.Tk = Tk;
        if (!fwd_geometry(a, B, Hq, Hkv, Tq)) return GQA_ERR_UNSUPPORTED;
        a.causal = causal;
        a.c = folded_scale(scale);
        a.varlen = 0;
        (void)hipGetLastError();
        return launch_status(gqa::launch_fwd_bf16(a, Dk, st));
    }
    if (!aligned(q, 4) || !aligned(k, 4) || !aligned(v, 4) || !aligned(out, 4))
        return GQA_ERR_INVALID_ARG;
    if (Hq > 65535 || B > 65535) return GQA_ERR_UNSUPPORTED;
    gqa::F32FwdArgs a;
    a.q = (const float *)q;
    a.k = (const float *)k;
    a.v = (const float *)v;
    a.out = (float *)out;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.Tq = Tq;
    a.Tk = Tk;
    a.G = G;
    a.causal = causal;
    a.scale = scale;
    (void)hipGetLastError();
    return launch_status(gqa::launch_fwd_f32(a, Dk, st));
}

GQA_API int gqa_attn_fwd_varlen(const void *q, const void *k, const void *v, void *out,
                                const int *cu_seqlens_q, const int *cu_seqlens_k,
                                const int *seqused_q, const int *seqused_k, int num_seqs, int Hq,
                                int Hkv, int total_q, int total_k, int Dk, int Dv, long long q_sh, long long q_st,
                                long long k_sh, long long k_st, long long v_sh, long long v_st,
                                long long o_sh, long long o_st, float scale, int causal, int window,
                                gqa_dtype dtype, void *stream)
{
    if (!q || !k || !v || !out || !cu_seqlens_q || !cu_seqlens_k) return GQA_ERR_INVALID_ARG;
    int rc = check_common(num_seqs, Hq, Hkv, Dk, Dv, scale, dtype);
    if (rc != GQA_OK) return rc;
    if (total_q < 0 || total_k < 0) return GQA_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1) return GQA_ERR_INVALID_ARG;
    if (window < 0 || (window > 0 && !causal)) return GQA_ERR_INVALID_ARG;
    const long long in_strides[6] = {q_sh, q_st, k_sh, k_st, v_sh, v_st};
    for (long long st : in_strides)
        if (st <= 0 || st % 8 != 0) return GQA_ERR_INVALID_ARG;  // 16-byte rows
    if (o_sh <= 0 || o_st <= 0 || o_sh % 4 != 0 || o_st % 4 != 0) return GQA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 8) ||
        !aligned(cu_seqlens_q, 4) || !aligned(cu_seqlens_k, 4) || !aligned(seqused_q, 4) ||
        !aligned(seqused_k, 4))
        return GQA_ERR_INVALID_ARG;
    if (dtype != GQA_BF16 || !head_dims_fwd(Dk, Dv)) return GQA_ERR_UNSUPPORTED;
    // per-lane tile offsets are 32-bit: 63 rows of the larger key stride
    if (63LL * (k_st > v_st ? k_st : v_st) * 2 + 2LL * Dk >= (1LL << 31)) return GQA_ERR_UNSUPPORTED;

    gqa::FwdArgs a = {};
    a.q = (const uint16_t *)q;
    a.k = (const uint16_t *)k;
    a.v = (const uint16_t *)v;
    a.out = (uint16_t *)out;
    a.Tk = 0;  // per sequence, from cu_seqlens_k
    if (total_q == 0) return GQA_OK;  // no query token: nothing to write
    if (!fwd_geometry(a, num_seqs, Hq, Hkv, 1)) return GQA_ERR_UNSUPPORTED;
    // grid: (query tiles of all sequences) x (head units of one sequence);
    // sum_i ceil(Tq_i / Pt) <= total_q / Pt + num_seqs
    a.n_units = Hkv * a.n_hblk;
    const long long ntile_bound = (long long)total_q / a.Pt + num_seqs;
    if (ntile_bound * a.n_units > 0x7fffffffLL) return GQA_ERR_UNSUPPORTED;
    a.n_qt = (int)ntile_bound;
    a.causal = causal;
    a.c = folded_scale(scale);
    a.varlen = 1;
    a.total_q = total_q;
    a.total_k = total_k;
    a.cu_q = cu_seqlens_q;
    a.cu_k = cu_seqlens_k;
    a.used_q = seqused_q;  // null: the whole slot
    a.used_k = seqused_k;
    a.q_sh = q_sh;
    a.q_st = q_st;
    a.k_sh = k_sh;
    a.k_st = k_st;
    a.v_sh = v_sh;
    a.v_st = v_st;
    a.o_sh = o_sh;
    a.o_st = o_st;
    a.window = window;
    (void)hipGetLastError();
    return launch_status(gqa::launch_fwd_bf16(a, Dk, (hipStream_t)stream));
}

GQA_API int gqa_attn_fwd_shard(const void *q, const void *k, const void *v, float *out, float *lse, int B,
                               int Hq, int Hkv, int Tq, int Tk, int Dk, int Dv, long long q_pos0,
                               long long k_pos0, float scale, int causal, gqa_dtype dtype, void *stream)
{
    if (!q || !k || !v || !out || !lse) return GQA_ERR_INVALID_ARG;
    int rc = check_common(B, Hq, Hkv, Dk, Dv, scale, dtype);
    if (rc != GQA_OK) return rc;
    if (Tq <= 0 || Tk <= 0) return GQA_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1) return GQA_ERR_INVALID_ARG;
    if (q_pos0 < 0 || k_pos0 < 0) return GQA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(lse, 4))
        return GQA_ERR_INVALID_ARG;
    if (dtype != GQA_BF16 || !head_dims_fwd(Dk, Dv)) return GQA_ERR_UNSUPPORTED;
    // the kernel counts query positions in keys of the shard with 32-bit ints
    const long long qmk = q_pos0 - k_pos0;
    if (qmk > (1LL << 30) || qmk < -(1LL << 30)) return GQA_ERR_UNSUPPORTED;

    gqa::FwdArgs a = {};
    a.q = (const uint16_t *)q;
    a.k = (const uint16_t *)k;
    a.v = (const uint16_t *)v;
    a.Tk = Tk;
    if (!fwd_geometry(a, B, Hq, Hkv, Tq)) return GQA_ERR_UNSUPPORTED;
    a.causal = causal;
    a.c = folded_scale(scale);
    a.varlen = 0;
    a.q_minus_k = (int)qmk;
    a.out_f32 = out;
    a.lse = lse;
    (void)hipGetLastError();
    return launch_status(gqa::launch_fwd_bf16_shard(a, Dk, (hipStream_t)stream));
}

GQA_API int gqa_attn_merge(const float *o_parts, const float *lse_parts, void *out, int num_parts,
                           long long rows, int Dv, gqa_dtype out_dtype, void *stream)
{
    if (!o_parts || !lse_parts || !out) return GQA_ERR_INVALID_ARG;
    if (num_parts <= 0 || rows <= 0 || Dv <= 0) return GQA_ERR_INVALID_ARG;
    if (out_dtype != GQA_BF16 && out_dtype != GQA_F32) return GQA_ERR_INVALID_ARG;
    if (!aligned(o_parts, 16) || !aligned(lse_parts, 4) || !aligned(out, out_dtype == GQA_BF16 ? 8 : 16))
        return GQA_ERR_INVALID_ARG;
    if (Dv % 4 != 0 || Dv > 512) return GQA_ERR_UNSUPPORTED;
    if (rows * (Dv / 4) > (1LL << 40) || num_parts > kMaxSplits) return GQA_ERR_UNSUPPORTED;
    gqa::MergeArgs m;
    m.o = o_parts;
    m.lse = lse_parts;
    m.out = out;
    m.rows = rows;
    m.S = num_parts;
    m.Dv = Dv;
    m.out_bf16 = out_dtype == GQA_BF16;
    // gathered partials, part-major: o [S, rows, Dv], lse [S, rows], natural log
    m.o_rs = Dv;
    m.o_ss = rows * Dv;
    m.l_rs = 1;
    m.l_ss = rows;
    m.lse_mul = 1.4426950408889634f;  // log2(e)
    (void)hipGetLastError();
    return launch_status(gqa::launch_merge(m, (hipStream_t)stream));
}

GQA_API int gqa_attn_decode_splits(int B, int Hq, int Hkv, int Tmax, int Dk, int Dv, gqa_dtype dtype)
{
    int rc = check_common(B, Hq, Hkv, Dk, Dv, 1.f, dtype);
    if (rc != GQA_OK) return rc;
    if (Tmax <= 0) return GQA_ERR_INVALID_ARG;
    if (!head_dims_decode(Dk, Dv, dtype)) return GQA_ERR_UNSUPPORTED;
    return default_splits(B, Hq, Hkv, Tmax, Dk, dtype);
}

GQA_API int gqa_attn_decode_fp8_splits(int B, int Hq, int Hkv, int Tmax, int Dk, int Dv)
{
    int rc = check_common(B, Hq, Hkv, Dk, Dv, 1.f, GQA_BF16);
    if (rc != GQA_OK) return rc;
    if (Tmax <= 0) return GQA_ERR_INVALID_ARG;
    if (Dk != Dv || (Dk != 64 && Dk != 128)) return GQA_ERR_UNSUPPORTED;
    return fp8_default_splits(B, Hq, Hkv, Tmax, Dk);
}

// Top-k sparse decode: splits when the caller leaves the choice to the
// library.  A workgroup covers 128 heads of one sequence and one slice of the
// index list; aim at one workgroup per CU (256) with slices of at least 64
// entries, and never a slice longer than the kernel can stage.
static int topk_default_splits(int B, int Hq, int topk)
{
    const long long groups = (long long)B * cdiv(Hq, 128);
    long long s = (256 + groups - 1) / groups;
    const long long cap = cdiv(topk, 64);
    if (s > cap) s = cap;
    const long long need = cdiv(topk, gqa::mla_topk_max_chunk());
    if (s < need) s = need;
    if (s < 1) s = 1;
    return (int)s;
}

static int topk_shape_check(int B, int Hq, int topk, int Dk, int Dv, gqa_dtype dtype)
{
    int rc = check_common(B, Hq, 1, Dk, Dv, 1.f, dtype);
    if (rc != GQA_OK) return rc;
    if (topk <= 0) return GQA_ERR_INVALID_ARG;
    if (dtype != GQA_BF16 || Dk != 576 || Dv != 512) return GQA_ERR_UNSUPPORTED;
    if ((long long)topk > (long long)kMaxSplits * gqa::mla_topk_max_chunk()) return GQA_ERR_UNSUPPORTED;
    return GQA_OK;
}

GQA_API int gqa_attn_decode_topk_splits(int B, int Hq, int topk, int Dk, int Dv, gqa_dtype dtype)
{
    int rc = topk_shape_check(B, Hq, topk, Dk, Dv, dtype);
    if (rc != GQA_OK) return rc;
    return topk_default_splits(B, Hq, topk);
}

GQA_API int gqa_attn_decode_topk(const void *q, const void *kv, void *out, const int *seq_lens,
                                 const int *indices, int B, int Hq, int Tmax, int topk, int Dk, int Dv,
                                 long long kv_sb, long long kv_st, float scale, int num_splits,
                                 void *workspace, size_t workspace_bytes, gqa_dtype dtype, void *stream)
{
    if (!q || !kv || !out || !seq_lens || !indices) return GQA_ERR_INVALID_ARG;
    int rc = check_common(B, Hq, 1, Dk, Dv, scale, dtype);
    if (rc != GQA_OK) return rc;
    if (Tmax <= 0 || topk <= 0) return GQA_ERR_INVALID_ARG;
    if (kv_sb <= 0 || kv_st < Dk || kv_sb % 8 || kv_st % 8) return GQA_ERR_INVALID_ARG;
    if (num_splits < 0 || num_splits > kMaxSplits) return GQA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(kv, 16) || !aligned(out, 8) || !aligned(seq_lens, 4) ||
        !aligned(indices, 4))
        return GQA_ERR_INVALID_ARG;
    rc = topk_shape_check(B, Hq, topk, Dk, Dv, dtype);
    if (rc != GQA_OK) return rc;

    const int S = num_splits ? num_splits : topk_default_splits(B, Hq, topk);
    const int chunk = (int)(cdiv(cdiv(topk, S), 32) * 32);  // topk <= 1024 * 4096 (checked above)
    if (chunk > gqa::mla_topk_max_chunk()) return GQA_ERR_UNSUPPORTED;  // too few splits for topk
    const size_t need = ws_bytes(B, Hq, Dv, S);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 16)) return GQA_ERR_WORKSPACE;
    if ((long long)S * B > 0x7fffffffLL || cdiv(Hq, 128) > 65535) return GQA_ERR_UNSUPPORTED;

    gqa::DecodeArgs a = {};
    a.q = q;
    a.k = kv;
    a.v = kv;
    a.lens = seq_lens;
    a.part_o = (float *)workspace;
    a.part_lse = (float *)workspace + (size_t)B * Hq * S * Dv;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = 1;
    a.Tmax = Tmax;
    a.G = Hq;
    a.k_sb = a.v_sb = kv_sb;
    a.k_sh = a.v_sh = kv_sb;  // one KV head
    a.k_st = a.v_st = kv_st;
    a.S = S;
    a.chunk = chunk;
    a.n_hblk = (int)cdiv(Hq, gqa::mla_heads_per_block());
    a.c = folded_scale(scale);
    a.idx = indices;
    a.topk = topk;
    hipStream_t st = (hipStream_t)stream;
    debug_fill_workspace(workspace, need, st);
    (void)hipGetLastError();
    if (gqa::launch_mla_decode_topk(a, st) != 0) return GQA_ERR_UNSUPPORTED;
    gqa::CombineArgs c;
    c.part_o = a.part_o;
    c.part_lse = a.part_lse;
    c.out = out;
    c.B = B;
    c.Hq = Hq;
    c.S = S;
    c.Dv = Dv;
    c.out_bf16 = 1;
    return launch_status(gqa::launch_combine(c, st));
}

GQA_API int gqa_attn_decode_fp8(const void *q, const void *k, const void *v, const float *k_scale,
                                const float *v_scale, void *out, const int *seq_lens, int B, int Hq,
                                int Hkv, int Tmax, int Dk, int Dv, long long k_sb, long long k_sh,
                                long long k_st, long long v_sb, long long v_sh, long long v_st,
                                long long ks_sb, long long ks_sh, long long ks_st, long long vs_sb,
                                long long vs_sh, long long vs_st, float scale, int window,
                                int num_splits, void *workspace, size_t workspace_bytes, void *stream)
{
    if (!q || !k || !v || !k_scale || !v_scale || !out || !seq_lens) return GQA_ERR_INVALID_ARG;
    if (window < 0) return GQA_ERR_INVALID_ARG;
    int rc = check_common(B, Hq, Hkv, Dk, Dv, scale, GQA_BF16);
    if (rc != GQA_OK) return rc;
    if (Tmax <= 0) return GQA_ERR_INVALID_ARG;
    const long long cs[6] = {k_sb, k_sh, k_st, v_sb, v_sh, v_st};
    for (long long st : cs)
        if (st <= 0 || st % 16 != 0) return GQA_ERR_INVALID_ARG;  // 16-byte rows of codes
    if (k_st < Dk || v_st < Dv) return GQA_ERR_INVALID_ARG;      // rows may not overlap
    const long long ss[6] = {ks_sb, ks_sh, ks_st, vs_sb, vs_sh, vs_st};
    for (long long st : ss)
        if (st <= 0) return GQA_ERR_INVALID_ARG;
    if (num_splits < 0 || num_splits == 1 || num_splits == 2 || num_splits > kMaxSplits)
        return GQA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 8) || !aligned(k_scale, 4) ||
        !aligned(v_scale, 4) || !aligned(seq_lens, 4))
        return GQA_ERR_INVALID_ARG;
    if (Dk != Dv || (Dk != 64 && Dk != 128)) return GQA_ERR_UNSUPPORTED;
    // a 32-row tile is addressed with 32-bit byte offsets
    if (k_st > (1LL << 25) || v_st > (1LL << 25)) return GQA_ERR_UNSUPPORTED;

    const int S = num_splits ? num_splits : fp8_default_splits(B, Hq, Hkv, Tmax, Dk);
    const size_t need = ws_bytes(B, Hq, Dv, S);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 16)) return GQA_ERR_WORKSPACE;

    const int G = Hq / Hkv;
    gqa::DecodeArgs a = {};
    a.q = q;
    a.k = k;
    a.v = v;
    a.lens = seq_lens;
    a.part_o = (float *)workspace;
    a.part_lse = (float *)workspace + (size_t)B * Hq * S * Dv;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.Tmax = Tmax;
    a.G = G;
    a.k_sb = k_sb;
    a.k_sh = k_sh;
    a.k_st = k_st;
    a.v_sb = v_sb;
    a.v_sh = v_sh;
    a.v_st = v_st;
    a.S = S;
    a.chunk = 0;
    const int hpb = gqa::decode_bf16_heads_per_block(Dk, G);
    a.n_hblk = (int)cdiv(G, hpb);
    a.n_wg = gqa::decode_fp8_flat_workgroups(Dk);
    a.c = folded_scale(scale);
    a.fp8 = 1;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.ks_sb = ks_sb;
    a.ks_sh = ks_sh;
    a.ks_st = ks_st;
    a.vs_sb = vs_sb;
    a.vs_sh = vs_sh;
    a.vs_st = vs_st;
    a.window = window;
    hipStream_t st = (hipStream_t)stream;
    debug_fill_workspace(workspace, need, st);
    (void)hipGetLastError();
    if (gqa::launch_decode_fp8(a, Dk, Dv, st) != 0) return GQA_ERR_UNSUPPORTED;
    gqa::CombineArgs c;
    c.part_o = a.part_o;
    c.part_lse = a.part_lse;
    c.out = out;
    c.B = B;
    c.Hq = Hq;
    c.S = S;
    c.Dv = Dv;
    c.out_bf16 = 1;
    return launch_status(gqa::launch_combine(c, st));
}

GQA_API size_t gqa_attn_decode_workspace_size(int B, int Hq, int Dv, int num_splits)
{
    if (B <= 0 || Hq <= 0 || Dv <= 0 || num_splits <= 0 || num_splits > kMaxSplits) return 0;
    return ws_bytes(B, Hq, Dv, num_splits);
}

// Workspace layouts of the decode: the caller-sized one (fp32 partial
// outputs [B, Hq, S, Dv], then the fp32 partial LSE [B, Hq, S]) and the
// compact one of the allocation-free entry point (the same partials, then
// the LSE at the next 256-byte boundary); both end in the 256-byte piece
// counter region.
static size_t compact_ws_lse_offset(int B, int Hq, int Dv, int S, int dtype)
{
    const size_t rows = (size_t)B * Hq * S;
    const size_t o_bytes = rows * Dv * sizeof(float);
    return (o_bytes + 255) & ~(size_t)255;
}
static size_t compact_ws_bytes(int B, int Hq, int Dv, int S, int dtype)
{
    const size_t bytes = compact_ws_lse_offset(B, Hq, Dv, S, dtype) + (size_t)B * Hq * S * sizeof(float);
    return ((bytes + 255) & ~(size_t)255) + kQueueBytes;
}

static int decode_impl(const void *q, const void *k, const void *v, void *out, const int *seq_lens, int B,
                       int Hq, int Hkv, int Tmax, int Dk, int Dv, long long k_sb, long long k_sh,
                       long long k_st, long long v_sb, long long v_sh, long long v_st, float scale,
                       int window, int num_splits, void *workspace, size_t workspace_bytes, int dtype,
                       void *stream, bool compact = false, bool dry_run = false)
{
    if (!q || !k || !v || !out || !seq_lens) return GQA_ERR_INVALID_ARG;
    if (window < 0) return GQA_ERR_INVALID_ARG;
    int rc = check_common(B, Hq, Hkv, Dk, Dv, scale, dtype);
    if (rc != GQA_OK) return rc;
    if (Tmax <= 0) return GQA_ERR_INVALID_ARG;
    if (k_sb <= 0 || k_sh <= 0 || k_st <= 0 || v_sb <= 0 || v_sh <= 0 || v_st <= 0)
        return GQA_ERR_INVALID_ARG;
    if (k_st < Dk || v_st < Dv) return GQA_ERR_INVALID_ARG;  // rows may not overlap
    // the kernels address a 32-key tile with 32-bit byte offsets
    if (k_st > (1LL << 25) || v_st > (1LL << 25)) return GQA_ERR_UNSUPPORTED;
    if (num_splits < 0 || num_splits > kMaxSplits) return GQA_ERR_INVALID_ARG;
    if (!head_dims_decode(Dk, Dv, dtype)) return GQA_ERR_UNSUPPORTED;
    if (Dk == 576 && !(v == k && v_sb == k_sb && v_sh == k_sh && v_st == k_st))
        return GQA_ERR_UNSUPPORTED;  // absorbed MLA: the value is the key's latent prefix
    if (dtype == GQA_BF16) {
        if (k_sb % 8 || k_sh % 8 || k_st % 8 || v_sb % 8 || v_sh % 8 || v_st % 8)
            return GQA_ERR_INVALID_ARG;
        if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 8))
            return GQA_ERR_INVALID_ARG;
    } else {
        if (!aligned(q, 4) || !aligned(k, 4) || !aligned(v, 4) || !aligned(out, 16))
            return GQA_ERR_INVALID_ARG;
    }
    if (!aligned(seq_lens, 4)) return GQA_ERR_INVALID_ARG;

    const int S = num_splits ? num_splits : default_splits(B, Hq, Hkv, Tmax, Dk, dtype);
    const size_t need = compact ? compact_ws_bytes(B, Hq, Dv, S, dtype) : ws_bytes(B, Hq, Dv, S);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 16)) return GQA_ERR_WORKSPACE;

    const int G = Hq / Hkv;
    const int tile = dtype == GQA_BF16 ? gqa::decode_bf16_key_tile() : 64;
    const int Teff = (window > 0 && window < Tmax) ? window : Tmax;  // keys any query can see
    const long long chunk_ll = cdiv(cdiv(Teff, S), tile) * tile;
    if (chunk_ll > 0x7fffffffLL) return GQA_ERR_UNSUPPORTED;
    const int chunk = (int)chunk_ll;

    gqa::DecodeArgs a = {};
    a.q = q;
    a.k = k;
    a.v = v;
    a.lens = seq_lens;
    a.part_o = (float *)workspace;
    a.part_lse = compact ? (float *)((char *)workspace + compact_ws_lse_offset(B, Hq, Dv, S, dtype))
                         : (float *)workspace + (size_t)B * Hq * S * Dv;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.Tmax = Tmax;
    a.G = G;
    a.k_sb = k_sb;
    a.k_sh = k_sh;
    a.k_st = k_st;
    a.v_sb = v_sb;
    a.v_sh = v_sh;
    a.v_st = v_st;
    a.S = S;
    a.chunk = chunk;
    a.n_wg = 0;
    a.window = window;
    hipStream_t st = (hipStream_t)stream;

    if (dtype == GQA_BF16) {
        const int hpb = gqa::decode_bf16_heads_per_block(Dk, G);
        a.n_hblk = (int)cdiv(G, hpb);
        if ((long long)B * Hkv * S > 0x7fffffffLL || a.n_hblk > 65535) return GQA_ERR_UNSUPPORTED;
        if (Dk <= 128 && S >= 3) {
            // flat decode (balanced over all sequences); S bounds the pieces per stream
            a.n_wg = gqa::decode_bf16_flat_workgroups(Dk);
            a.n_first = gqa::decode_bf16_flat_first_round(Dk);
            a.queue = (unsigned *)((char *)workspace + need - kQueueBytes);
        }
        a.c = folded_scale(scale);
        if (dry_run) return GQA_OK;
        debug_fill_workspace(workspace, need, st);
        (void)hipGetLastError();
        rc = gqa::launch_decode_bf16(a, Dk, Dv, st);
    } else {
        if (Hq > 65535 || B > 65535) return GQA_ERR_UNSUPPORTED;
        a.n_hblk = (int)cdiv(G, 32);  // 32 query heads of the group per workgroup
        a.c = scale;  // the fp32 path works in natural-log units
        if (dry_run) return GQA_OK;
        debug_fill_workspace(workspace, need, st);
        (void)hipGetLastError();
        rc = gqa::launch_decode_f32(a, Dk, st);
    }
    if (rc != 0) return GQA_ERR_UNSUPPORTED;
    gqa::CombineArgs c;
    c.part_o = a.part_o;
    c.part_lse = a.part_lse;
    c.out = out;
    c.B = B;
    c.Hq = Hq;
    c.S = S;
    c.Dv = Dv;
    c.out_bf16 = dtype == GQA_BF16;
    return launch_status(gqa::launch_combine(c, st));
}

GQA_API int gqa_attn_decode(const void *q, const void *k, const void *v, void *out,
                            const int *seq_lens, int B, int Hq, int Hkv, int Tmax, int Dk, int Dv,
                            long long k_sb, long long k_sh, long long k_st, long long v_sb,
                            long long v_sh, long long v_st, float scale, int num_splits,
                            void *workspace, size_t workspace_bytes, gqa_dtype dtype, void *stream)
{
    return decode_impl(q, k, v, out, seq_lens, B, Hq, Hkv, Tmax, Dk, Dv, k_sb, k_sh, k_st, v_sb, v_sh, v_st,
                       scale, 0, num_splits, workspace, workspace_bytes, dtype, stream);
}

GQA_API int gqa_attn_decode_window(const void *q, const void *k, const void *v, void *out,
                                   const int *seq_lens, int B, int Hq, int Hkv, int Tmax, int Dk,
                                   int Dv, long long k_sb, long long k_sh, long long k_st,
                                   long long v_sb, long long v_sh, long long v_st, float scale,
                                   int window, int num_splits, void *workspace,
                                   size_t workspace_bytes, gqa_dtype dtype, void *stream)
{
    return decode_impl(q, k, v, out, seq_lens, B, Hq, Hkv, Tmax, Dk, Dv, k_sb, k_sh, k_st, v_sb, v_sh, v_st,
                       scale, window, num_splits, workspace, workspace_bytes, dtype, stream);
}

// ---- allocation-free decode ----
//
// The scratch of gqa_attn_decode_noalloc: one array per GPU for the life of
// the process.  In host code `scratch` names a host-side stand-in, not the
// device array, so it is never passed to a kernel or a copy: its device
// address is looked up once per device (hipGetSymbolAddress, with that device
// current) and kept in scratch_dev[].  Every call on a device uses the same
// array, so calls that overlap on one GPU race on it.  Nothing in it has to
// start at zero: the partial kernels write every slot the combine reads.
namespace {

constexpr size_t kScratchBytes = (size_t)GQA_DECODE_NOALLOC_MAX_SCRATCH;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
void *scratch_dev[kMaxDevices];
std::mutex scratch_mu;

// device address of this device's scratch array, or null on a HIP error
void *scratch_for_current_device()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_dev[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
        scratch_dev[dev] = ptr;
    }
    return scratch_dev[dev];
}

} // namespace

GQA_API size_t gqa_attn_decode_noalloc_scratch_bytes(int B, int Hq, int Dv, int num_splits, gqa_dtype dtype)
{
    if (B <= 0 || Hq <= 0 || Dv <= 0 || num_splits <= 0 || num_splits > kMaxSplits) return 0;
    if (dtype != GQA_BF16 && dtype != GQA_F32) return 0;
    return compact_ws_bytes(B, Hq, Dv, num_splits, dtype);
}

GQA_API int gqa_attn_decode_noalloc(const void *q, const void *k, const void *v, void *out,
                                    const int *seq_lens, int B, int Hq, int Hkv, int Tmax, int Dk, int Dv,
                                    long long k_sb, long long k_sh, long long k_st, long long v_sb,
                                    long long v_sh, long long v_st, float scale, int num_splits,
                                    gqa_dtype dtype, void *stream)
{
    // every argument is checked before the first HIP call (a dry run with a
    // stand-in workspace address that is never used); a shape whose partials
    // do not fit the scratch returns GQA_ERR_WORKSPACE
    int rc = decode_impl(q, k, v, out, seq_lens, B, Hq, Hkv, Tmax, Dk, Dv, k_sb, k_sh, k_st, v_sb, v_sh, v_st,
                         scale, 0, num_splits, (void *)(uintptr_t)256, kScratchBytes, dtype, stream, true, true);
    if (rc != GQA_OK) return rc;
    void *ws = scratch_for_current_device();
    if (!ws) return GQA_ERR_HIP;
    return decode_impl(q, k, v, out, seq_lens, B, Hq, Hkv, Tmax, Dk, Dv, k_sb, k_sh, k_st, v_sb, v_sh, v_st,
                       scale, 0, num_splits, ws, kScratchBytes, dtype, stream, true);
}
