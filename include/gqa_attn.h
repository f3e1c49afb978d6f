/*
 * gqa_attn.h -- C ABI of the MI355X (gfx950) causal grouped-query attention
 * library, libgqa_attn.so.
 *
 * The operation is dense softmax attention with grouped KV heads,
 *
 *     o_a = softmax( Q_a K_{g(a)}^T * scale + M ) V_{g(a)},
 *     g(a) = floor(a / (Hq / Hkv)),
 *
 * as written in the unified-notation section of the "Attention variants"
 * page (wineandchord.com, 注意力家族) and, for each of the MHA / MQA / GQA
 * limits, in the Dense Softmax family section of "Attention Architecture
 * Evolution".  M is the causal mask: with Tq queries over Tk keys the queries
 * sit at absolute positions Tk-Tq .. Tk-1 (the suffix-decode convention of the
 * "Attention variants" minimal semantic implementation and its section on
 * masks and incremental positions), and query i sees key j iff
 * j <= Tk - Tq + i.  One entry point covers MHA (Hkv = Hq), MQA (Hkv = 1),
 * GQA, and the weight-absorbed MLA decode shape of "Attention Architecture
 * Evolution" (MLA section and the DSA section's absorbed equations), which is
 * MQA over a 576-wide shared latent key whose first 512 columns are the value.
 *
 * Conventions for every entry point
 *  - Pointers q, k, v, out, seq_lens, cu_seqlens and workspace are DEVICE pointers
 *    (hipMalloc'd or torch CUDA tensors).  The caller owns all buffers; the
 *    library never allocates, frees or synchronises.
 *  - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL is the
 *    default stream) and runs asynchronously.
 *  - dtype selects the element type of q, k, v and out: GQA_BF16 (bfloat16
 *    storage, fp32 accumulation, fp32 softmax, P rounded to bf16 for the PV
 *    product, output rounded to nearest-even) or GQA_F32 (fp32 throughout).
 *  - scale must be finite and >= 0 (1/sqrt(Dk) is the pages' choice; the
 *    absorbed MLA shape uses 1/sqrt(192)).
 *  - out must not alias any input.
 *  - All argument checks run on the host before anything is launched; on
 *    error nothing is enqueued and no device memory is touched.
 *
 * Supported head dims (anything else returns GQA_ERR_UNSUPPORTED):
 *    gqa_attn_fwd:     (Dk, Dv) = (64, 64) or (128, 128), bf16 or fp32
 *    gqa_attn_fwd_varlen: (64, 64) or (128, 128), bf16
 *    gqa_attn_fwd_shard: (64, 64) or (128, 128), bf16 in, fp32 out + lse
 *    gqa_attn_decode:  (64, 64) or (128, 128), bf16 or fp32;
 *                      (576, 512) bf16 (the absorbed-MLA shape)
 *    gqa_attn_decode_topk: (576, 512) bf16
 *    gqa_attn_decode_fp8:  (64, 64) or (128, 128), FP8 E4M3 cache, bf16 q / out
 */
#ifndef GQA_ATTN_H
#define GQA_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type.  Callers pass it as an int; in C++ the enum has int as its
 * fixed underlying type, so an out-of-range value is a value the library
 * can reject (GQA_ERR_INVALID_ARG) rather than undefined behaviour. */
#ifdef __cplusplus
typedef enum gqa_dtype_e : int { GQA_BF16 = 0, GQA_F32 = 1 } gqa_dtype;
#else
typedef enum { GQA_BF16 = 0, GQA_F32 = 1 } gqa_dtype;
#endif

enum {
    GQA_OK = 0,
    GQA_ERR_INVALID_ARG = -1, /* null pointer, dim <= 0, Hq % Hkv != 0, causal with
                                 Tq > Tk, non-finite or negative scale, bad stride */
    GQA_ERR_UNSUPPORTED = -2, /* (Dk, Dv, dtype) combination not built */
    GQA_ERR_WORKSPACE = -3,   /* workspace null or smaller than required */
    GQA_ERR_HIP = -4          /* a HIP launch reported an error */
};

/*
 * Prefill / suffix forward.
 *
 *   q   [B, Hq,  Tq, Dk]   contiguous, row-major
 *   k   [B, Hkv, Tk, Dk]   contiguous
 *   v   [B, Hkv, Tk, Dv]   contiguous
 *   out [B, Hq,  Tq, Dv]   contiguous, written in full
 *
 * causal = 1: query i (position Tk - Tq + i) attends to keys 0 .. Tk - Tq + i;
 * requires Tq <= Tk (the pages' semantic implementation asserts it).
 * causal = 0: every query attends to all Tk keys (cross attention; any Tq).
 * Returns GQA_OK or a negative GQA_ERR_* code.
 */
int gqa_attn_fwd(const void *q, const void *k, const void *v, void *out, int B, int Hq, int Hkv,
                 int Tq, int Tk, int Dk, int Dv, float scale, int causal, gqa_dtype dtype, void *stream);

/*
 * Forward over packed variable-length sequences, with an optional sliding
 * window.  The "Attention variants" page (section on masks and incremental
 * positions) lists padding / packed-segment masks and sliding-window
 * patterns among the masks a real implementation has to handle; cu_seqlens
 * marks packed sequence boundaries ("Attention Architecture Evolution", GDN
 * code section); SWA keeps direct access to the most recent w positions ("A
 * Visual Guide to Attention", section on which positions are visible).
 *
 * num_seqs sequences are stored back to back along the token axis.
 * cu_seqlens_q / cu_seqlens_k: DEVICE int32 arrays of num_seqs + 1
 * non-decreasing offsets; sequence i owns query tokens cu_seqlens_q[i] ..
 * cu_seqlens_q[i+1]-1 and key tokens cu_seqlens_k[i] .. cu_seqlens_k[i+1]-1.
 * Element (h, t, d) of each tensor sits at ptr + h*X_sh + t*X_st + d
 * (element strides; d is unit-stride): q (Hq heads, Dk), k (Hkv, Dk),
 * v (Hkv, Dv), out (Hq, Dv).  [total, H, D] row-major has X_sh = D,
 * X_st = H*D; [H, total, D] has X_sh = total*D, X_st = D.  Tokens attend only
 * within their own sequence; inside a sequence with Tq_i queries and Tk_i
 * keys the rules of gqa_attn_fwd apply (query j at position Tk_i - Tq_i + j).
 * causal = 1 with window = w > 0: query at position p sees keys
 * max(0, p-w+1) .. p (the w most recent positions, its own included).
 * window = 0: no window.  A query with no visible key (causal and
 * Tq_i > Tk_i: the first Tq_i - Tk_i queries) gets a zero row.
 *
 * Padding (the same page's padding masks): seqused_q / seqused_k, DEVICE
 * int32 arrays of num_seqs entries or NULL.  When given, sequence i uses only
 * the first min(max(seqused[i], 0), slot length) tokens of its slot and the
 * rest is padding: padded keys are never read, padded query rows of out are
 * never written (left as they were), and Tq_i / Tk_i above are the used
 * lengths.  A right-padded batch [B, Tpad, H, D] is cu_seqlens = 0, Tpad,
 * 2*Tpad, ... with seqused = the true lengths.  NULL: every slot is used.
 *
 * total_q / total_k are the token slots of q and out / of k and v (the
 * buffers' token extents, normally cu_seqlens_q[num_seqs] and
 * cu_seqlens_k[num_seqs]); total_q sizes the grid (sum_i ceil(Tq_i / tile)
 * <= total_q / tile + num_seqs), and total_q = 0 returns GQA_OK with nothing
 * enqueued.  The offsets are device data and cannot be checked on the host;
 * the kernel clamps every sequence's slot to [0, total_q) / [0, total_k),
 * so offsets that disagree with the buffers never address a token outside
 * them (such a sequence is cut short, and with overlapping or decreasing
 * offsets some query rows may be left unwritten).  Used query rows of out
 * are written in full; out must not overlap itself or the inputs.
 * Requirements (else GQA_ERR_INVALID_ARG): q, k, v 16-byte aligned, out 8,
 * cu and seqused arrays 4; q/k/v head and token strides positive multiples of 8
 * elements, out strides positive multiples of 4; window >= 0 and only with
 * causal = 1; total_q, total_k >= 0.  bf16 only, (Dk, Dv) = (64, 64) or (128, 128); fp32 and other
 * dims return GQA_ERR_UNSUPPORTED, as do key / value token strides st with
 * 126 * st + 2 * Dk >= 2^31 (tile offsets are 32-bit byte offsets).
 */
int gqa_attn_fwd_varlen(const void *q, const void *k, const void *v, void *out, const int *cu_seqlens_q,
                        const int *cu_seqlens_k, const int *seqused_q, const int *seqused_k,
                        int num_seqs, int Hq, int Hkv, int total_q, int total_k, int Dk,
                        int Dv, long long q_sh, long long q_st, long long k_sh, long long k_st, long long v_sh,
                        long long v_st, long long o_sh, long long o_st, float scale, int causal, int window,
                        gqa_dtype dtype, void *stream);

/*
 * Forward over one shard of the key axis, for sequence (context) parallelism:
 * when one device cannot hold the context, each device keeps a slice of the
 * keys and attends over it, and the partial results are merged exactly
 * (Ring / Context Parallel in the causal-mainline section of the
 * long-context research ledger page; the merge is the online-softmax
 * rescaling of "A Visual Guide to Attention", section on sources and
 * execution).
 *
 *   q   [B, Hq,  Tq, Dk] bf16, contiguous; query i sits at absolute position
 *       q_pos0 + i
 *   k   [B, Hkv, Tk, Dk] bf16, contiguous; key j of the shard sits at
 *       absolute position k_pos0 + j
 *   v   [B, Hkv, Tk, Dv] bf16, contiguous
 *   out [B, Hq,  Tq, Dv] fp32: the softmax-normalised output over the
 *       shard's visible keys (written in full)
 *   lse [B, Hq,  Tq] fp32: natural log of the shard's softmax normaliser,
 *       ln sum_j exp(scale * q.k_j); a query that sees no key of the shard
 *       gets a zero row and lse = -inf
 * causal = 1: key j is visible iff k_pos0 + j <= q_pos0 + i (any Tq, Tk);
 * causal = 0: every key.  gqa_attn_merge combines the shards' (out, lse).
 * Requirements: q_pos0, k_pos0 >= 0 and |q_pos0 - k_pos0| <= 2^30
 * (else GQA_ERR_INVALID_ARG / GQA_ERR_UNSUPPORTED); q, k, v, out 16-byte
 * aligned, lse 4.  bf16 only, (Dk, Dv) = (64, 64) or (128, 128).
 */
int gqa_attn_fwd_shard(const void *q, const void *k, const void *v, float *out, float *lse, int B,
                       int Hq, int Hkv, int Tq, int Tk, int Dk, int Dv, long long q_pos0,
                       long long k_pos0, float scale, int causal, gqa_dtype dtype, void *stream);

/*
 * Exact log-sum-exp merge of num_parts partial results of the same rows
 * (e.g. the gathered outputs of gqa_attn_fwd_shard on every device):
 *   L = ln sum_s exp(lse_s),   out = sum_s exp(lse_s - L) * o_s.
 *   o_parts   fp32 [num_parts, rows, Dv], part-major, contiguous, 16-byte aligned
 *   lse_parts fp32 [num_parts, rows], natural log; -inf marks an empty part
 *   out       [rows, Dv], out_dtype GQA_BF16 (RNE) or GQA_F32
 * A row whose parts are all empty gets zeros.  Dv a multiple of 4, at most
 * 512; num_parts 1 .. 1024.
 */
int gqa_attn_merge(const float *o_parts, const float *lse_parts, void *out, int num_parts,
                   long long rows, int Dv, gqa_dtype out_dtype, void *stream);

/*
 * Split count the decode entry point uses when called with num_splits = 0.
 * It depends on the shape only (not on the device or on seq_lens), so the
 * workspace can be sized before any device call.  Host-only; returns >= 1,
 * or a negative GQA_ERR_* code for invalid or unsupported arguments.
 */
int gqa_attn_decode_splits(int B, int Hq, int Hkv, int Tmax, int Dk, int Dv, gqa_dtype dtype);

/*
 * Bytes of device workspace gqa_attn_decode needs for num_splits splits
 * (num_splits >= 1): fp32 partial outputs [B, Hq, S, Dv] followed by fp32
 * partial log-sum-exp values [B, Hq, S], rounded up to 256 bytes, and a
 * 256-byte region for the balanced schedule's piece counter (the kernel
 * zeroes it itself).  Returns 0 for invalid arguments.
 */
size_t gqa_attn_decode_workspace_size(int B, int Hq, int Dv, int num_splits);

/*
 * Single-token decode over a KV cache, split over the key axis with a
 * log-sum-exp combine.  A decode step reads the whole cached history and is
 * bound by that KV stream ("Linear Attention 与 Sparse Attention 梳理",
 * section 6.2 on decode; "Attention variants", KV Cache 成本 section, whose
 * cache-size formula is the read per step); partial results over key blocks
 * merge exactly by the online-softmax rescaling ("A Visual Guide to
 * Attention", section on sources and execution), which is what the combine
 * pass applies to the per-split (output, log-sum-exp) pairs.
 *
 *   q        [B, Hq, 1, Dk]  contiguous
 *   k, v     KV cache: element (b, h, t, d) at k[b*k_sb + h*k_sh + t*k_st + d]
 *            (element strides; d is unit-stride; t < Tmax).  For the
 *            absorbed-MLA shape pass v = k with the same strides and
 *            Dv = 512 < Dk = 576: the value is the latent prefix of each key.
 *            (For (576, 512) any other v returns GQA_ERR_UNSUPPORTED.)
 *            Strides must be multiples of 8 elements and the base pointers
 *            16-byte aligned.
 *   out      [B, Hq, 1, Dv]  contiguous
 *   seq_lens device int32[B]: sequence b has keys 0 .. seq_lens[b]-1 and its
 *            query sits at position seq_lens[b]-1 (sees all of them).  Values
 *            are read on the device: 0 gives a zero output row; values above
 *            Tmax are clamped to Tmax.  Cache slots at t >= seq_lens[b] are
 *            never read into the result (they may hold anything, NaN included).
 *   num_splits  number of key-axis splits, 1 .. 1024, or 0 for the value of
 *            gqa_attn_decode_splits().  For bf16 with Dk = Dv <= 128 and
 *            num_splits >= 3 the work is balanced over all sequences instead
 *            (the key tiles of all sequences are shared out over the
 *            workgroups; on long decodes the last ~10 % in smaller pieces
 *            that workgroups take at run time through a counter in the
 *            workspace) and num_splits bounds how many pieces one
 *            sequence's keys may be cut into; otherwise each sequence's keys
 *            are cut into num_splits equal chunks.  The result is the same
 *            attention either way (exact log-sum-exp merge).
 *   workspace   device buffer of at least
 *            gqa_attn_decode_workspace_size(B, Hq, Dv, splits) bytes, 256-byte
 *            aligned; contents on entry are ignored.  Two calls that share a
 *            workspace must be ordered on one stream.
 */
int gqa_attn_decode(const void *q, const void *k, const void *v, void *out, const int *seq_lens,
                    int B, int Hq, int Hkv, int Tmax, int Dk, int Dv, long long k_sb, long long k_sh,
                    long long k_st, long long v_sb, long long v_sh, long long v_st, float scale,
                    int num_splits, void *workspace, size_t workspace_bytes, gqa_dtype dtype,
                    void *stream);

/*
 * Single-token decode over an FP8 KV cache.  The cache holds OCP FP8 E4M3
 * codes (one byte per element: sign, 4 exponent bits with bias 7, 3 mantissa
 * bits, no infinities) with one fp32 scale per (b, h, t) row, the
 * block-scaled FP8 form the "Attention Architecture Evolution" page shows
 * for the DSA indexer's key cache (one scale per block of 128 features: a
 * whole row for the head dims here); the "Attention variants" page lists
 * the scale granularity of quantised K/V among the deployment concerns.
 * Element (b, h, t, d) stands for e4m3(code) * scale[b, h, t]; the result
 * is attention over those values, as gqa_attn_decode computes it for bf16.
 *
 *   q        [B, Hq, 1, Dk] bf16, contiguous, 16-byte aligned
 *   k, v     codes: element (b, h, t, d) at k[b*k_sb + h*k_sh + t*k_st + d]
 *            (strides in elements = bytes, positive multiples of 16;
 *            k_st >= Dk, v_st >= Dv; 16-byte aligned bases)
 *   k_scale, v_scale  fp32, the scale of row (b, h, t) at
 *            k_scale[b*ks_sb + h*ks_sh + t*ks_st] (strides > 0)
 *   out      [B, Hq, 1, Dv] bf16, contiguous
 *   seq_lens, workspace: as for gqa_attn_decode (workspace of
 *            gqa_attn_decode_workspace_size(B, Hq, Dv, splits) bytes)
 *   window   0, or w >= 1: a sliding window as for gqa_attn_decode_window
 *            (the last min(seq_lens[b], w) rows only)
 *   num_splits  0 (the value of gqa_attn_decode_fp8_splits(), which is never
 *            above gqa_attn_decode_splits(..., GQA_BF16)) or 3 .. 1024: the
 *            bound on the pieces one sequence's keys are cut into by the
 *            balanced schedule; 1 and 2 return GQA_ERR_INVALID_ARG.
 * Rows at t >= seq_lens[b] are never read (codes and scales there may hold
 * anything).  Codes of rows that are read must not be NaN.
 * Supported: Dk = Dv = 64 or 128 (else GQA_ERR_UNSUPPORTED), row strides up
 * to 2^25 bytes.  Same error rules as gqa_attn_decode.
 */
int gqa_attn_decode_fp8(const void *q, const void *k, const void *v, const float *k_scale,
                        const float *v_scale, void *out, const int *seq_lens, int B, int Hq, int Hkv,
                        int Tmax, int Dk, int Dv, long long k_sb, long long k_sh, long long k_st,
                        long long v_sb, long long v_sh, long long v_st, long long ks_sb,
                        long long ks_sh, long long ks_st, long long vs_sb, long long vs_sh,
                        long long vs_st, float scale, int window, int num_splits, void *workspace,
                        size_t workspace_bytes, void *stream);

/*
 * Split count gqa_attn_decode_fp8 uses when called with num_splits = 0
 * (shape only, host-only): 3 .. 64 and never above gqa_attn_decode_splits(B,
 * Hq, Hkv, Tmax, Dk, Dv, GQA_BF16), so a workspace sized for that value
 * fits; or a negative GQA_ERR_* code.  The FP8 decode runs one resident
 * round of workgroups with equal pieces, so it needs fewer split slots
 * than the bf16 decode's balanced schedule.
 */
int gqa_attn_decode_fp8_splits(int B, int Hq, int Hkv, int Tmax, int Dk, int Dv);

/*
 * Split count gqa_attn_decode_topk uses when called with num_splits = 0
 * (shape only, host-only): >= 1, or a negative GQA_ERR_* code.
 */
int gqa_attn_decode_topk_splits(int B, int Hq, int topk, int Dk, int Dv, gqa_dtype dtype);

/*
 * Top-k sparse single-token decode on the absorbed-MLA cache: DeepSeek Sparse
 * Attention ("Attention Architecture Evolution", DSA section).  An indexer
 * (not part of this library) selects for each sequence's query a list of
 * cached positions; the main attention keeps only those (the page's index
 * mask: -inf everywhere except 0 at the selected positions, added to the
 * absorbed scores q_C' c_KV^T + q_R k_R^T before the softmax), and the output
 * aggregates the selected latent rows.
 *
 *   q        [B, Hq, 1, Dk]  contiguous (one KV head shared by all Hq heads)
 *   kv       latent cache, element (b, t, d) at kv[b*kv_sb + t*kv_st + d]
 *            (d unit-stride, t < Tmax); the value is its first Dv columns.
 *            Strides multiples of 8 elements, kv_st >= Dk, kv 16-byte aligned.
 *   out      [B, Hq, 1, Dv]  contiguous, written in full
 *   seq_lens device int32[B]: valid cache length of sequence b (clamped to
 *            [0, Tmax] on the device).
 *   indices  device int32[B, topk], row-major: the selected positions of
 *            sequence b.  Entries outside [0, seq_lens[b]) select nothing
 *            (use -1 to pad a shorter selection); such entries are never
 *            used as addresses.  The order of the list does not matter.  A
 *            sequence with no valid entry gets a zero output row.  The
 *            page's mask is a scatter, so a position listed twice is
 *            selected once: the list is cut into num_splits slices of
 *            ceil(topk / num_splits) entries rounded up to a multiple of 32,
 *            and inside a slice an entry that repeats an earlier entry's
 *            position selects nothing.  A top-k lists distinct positions;
 *            a list whose repeats fall in different slices counts such a
 *            position once per slice (num_splits = 1, possible for lists of
 *            up to 4096 entries, applies the mask's rule to any list).
 *   num_splits  slices of the index list, 1 .. 1024, or 0 for
 *            gqa_attn_decode_topk_splits(); each slice may hold at most 4096
 *            entries (else GQA_ERR_UNSUPPORTED).
 *   workspace   device buffer of gqa_attn_decode_workspace_size(B, Hq, Dv,
 *            splits) bytes (same layout and rules as for gqa_attn_decode).
 * Supported: bf16, (Dk, Dv) = (576, 512); anything else GQA_ERR_UNSUPPORTED.
 * Same error rules as gqa_attn_decode (host checks, nothing enqueued on error).
 */
int gqa_attn_decode_topk(const void *q, const void *kv, void *out, const int *seq_lens,
                         const int *indices, int B, int Hq, int Tmax, int topk, int Dk, int Dv,
                         long long kv_sb, long long kv_st, float scale, int num_splits,
                         void *workspace, size_t workspace_bytes, gqa_dtype dtype, void *stream);

/*
 * gqa_attn_decode with a sliding window ("A Visual Guide to Attention",
 * section on which positions are visible: sliding-window attention keeps
 * direct access to the most recent w positions; the "Attention variants"
 * page lists sliding-window masks among those an implementation handles).
 * window = w >= 1: the query of sequence b (position seq_lens[b] - 1) sees
 * keys max(0, seq_lens[b] - w) .. seq_lens[b] - 1 of the cache (rows before
 * them are never read); window = 0: no window (exactly gqa_attn_decode);
 * window < 0: GQA_ERR_INVALID_ARG.  Every other argument, rule and
 * supported shape as for gqa_attn_decode.  (A rolling cache that keeps only
 * the last w rows needs no window: pass its fill level as seq_lens.)
 */
int gqa_attn_decode_window(const void *q, const void *k, const void *v, void *out,
                           const int *seq_lens, int B, int Hq, int Hkv, int Tmax, int Dk, int Dv,
                           long long k_sb, long long k_sh, long long k_st, long long v_sb,
                           long long v_sh, long long v_st, float scale, int window, int num_splits,
                           void *workspace, size_t workspace_bytes, gqa_dtype dtype, void *stream);

/*
 * gqa_attn_decode for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, rules, shapes and result as gqa_attn_decode, without the
 * workspace: the split partials live in a device array the library holds
 * for the life of the process, one per GPU, of GQA_DECODE_NOALLOC_MAX_SCRATCH
 * bytes.  The call allocates nothing; its first call on a device looks up
 * that device's array (hipGetSymbolAddress) with the device current.
 *
 * A shape needs gqa_attn_decode_noalloc_scratch_bytes(B, Hq, Dv, S, dtype)
 * bytes of it for S splits (num_splits, or gqa_attn_decode_splits() when 0):
 * B*Hq*S fp32 partial outputs of Dv values plus B*Hq*S fp32 log-sum-exp
 * values (at the next 256-byte boundary), rounded up to 256 bytes, plus 256
 * bytes for the piece counter.  A shape that needs more returns
 * GQA_ERR_WORKSPACE with nothing enqueued (e.g. B = 64, Hq = 32, Dv = 128,
 * S = 32 needs 33.8 MB; the absorbed-MLA B = 16, Hq = 128, Dv = 512,
 * S = 16 needs 67.2 MB).
 *
 * Calls on one GPU share its array: calls that overlap in time on that GPU
 * (different streams, or other processes' threads sharing this library
 * instance) race and corrupt each other's partials; order them on one
 * stream.  The array keeps the last call's contents; nothing in it needs to
 * start zeroed (every slot a call's combine reads is written by that call,
 * and the piece counter is zeroed by the call's own partial kernel).
 */
#define GQA_DECODE_NOALLOC_MAX_SCRATCH (96u << 20)
size_t gqa_attn_decode_noalloc_scratch_bytes(int B, int Hq, int Dv, int num_splits, gqa_dtype dtype);
int gqa_attn_decode_noalloc(const void *q, const void *k, const void *v, void *out, const int *seq_lens,
                            int B, int Hq, int Hkv, int Tmax, int Dk, int Dv, long long k_sb,
                            long long k_sh, long long k_st, long long v_sb, long long v_sh,
                            long long v_st, float scale, int num_splits, gqa_dtype dtype, void *stream);

/* Static, thread-safe description of a GQA_* return code. */
const char *gqa_attn_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* GQA_ATTN_H */
