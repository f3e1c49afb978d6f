// launch.h -- internal kernel argument blocks and launchers of libgqa_attn.so.
// Host code in api.hip validates every argument before calling these.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

// Store 4 consecutive normalised partial values (fp32) at element e of a
// split-partial row.  The partials stay in fp32 until the combine: a second
// bf16 rounding before the output's own would double the rounding error of
// large outputs.
__device__ __forceinline__ void store_partial4(void *po, size_t e, float a, float b, float c, float d)
{
    typedef float f4 __attribute__((ext_vector_type(4)));
    *(f4 *)((float *)po + e) = f4{a, b, c, d};
}

// Prefill / suffix forward (contiguous [B,H,T,D] tensors).
struct FwdArgs {
    const uint16_t *q;  // bf16 bits
    const uint16_t *k;
    const uint16_t *v;
    uint16_t *out;
    int B, Hq, Hkv, Tq, Tk;
    int G;       // Hq / Hkv
    int Gt;      // query heads per workgroup (divides G and the wave count)
    int Pt;      // query positions per workgroup (Gt * Pt = rows per workgroup)
    int n_hblk;  // G / Gt
    int n_qt;    // ceil(Tq / Pt)
    int n_units; // B * Hkv * n_hblk
    int causal;
    float c;     // scale * log2(e), > 0
    // packed variable-length mode (varlen != 0): B sequences, sequence b owns
    // the slots of query tokens cu_q[b] .. cu_q[b+1]-1 and key tokens
    // cu_k[b] .. cu_k[b+1]-1, of which the first used_q[b] / used_k[b]
    // (clamped to the slot; all of it when the pointer is null) are tokens and
    // the rest padding; element (h, t, d) of q sits at q + h*q_sh + t*q_st + d
    // (likewise k, v, out); n_qt = bound on the query tiles of all sequences;
    // window > 0: keys p-w+1 .. p only
    int varlen;
    int total_q, total_k;  // token slots of q / out and of k / v: every range is clamped to them
    const int *cu_q, *cu_k;
    const int *used_q, *used_k;
    long long q_sh, q_st, k_sh, k_st, v_sh, v_st, o_sh, o_st;
    int window;
    // key-shard mode (context parallelism): query i sits at key index
    // q_minus_k + i of this shard; fp32 outputs [B, Hq, Tq, Dv] and
    // natural-log LSE [B, Hq, Tq] instead of out
    int q_minus_k;
    float *out_f32, *lse;
};

int launch_fwd_bf16(const FwdArgs &a, int D, hipStream_t stream);
// Key-shard forward (a.q_minus_k, a.out_f32, a.lse; dense layout).
int launch_fwd_bf16_shard(const FwdArgs &a, int D, hipStream_t stream);
int fwd_bf16_waves_per_block();
int fwd_bf16_rows_per_wave();

// Split-KV decode partials over a strided cache.
struct DecodeArgs {
    const void *q;       // [B, Hq, 1, Dk] contiguous
    const void *k;       // cache, element strides below
    const void *v;
    const int *lens;     // device int32 [B]
    float *part_o;       // [B, Hq, S, Dv] normalised partial outputs (fp32)
    float *part_lse;     // [B, Hq, S] fp32, base-2 log-sum-exp of scaled scores
    int B, Hq, Hkv, Tmax, G;
    long long k_sb, k_sh, k_st;
    long long v_sb, v_sh, v_st;
    int S;               // splits (flat kernel: most partials any stream may need)
    int chunk;           // keys per split (multiple of the key tile)
    int n_hblk;          // head blocks per KV head
    float c;             // scale * log2(e)
    int n_wg;            // > 0: balanced (flat) schedule with this many workgroups
    int n_first;         // flat schedule: workgroups resident at once (the first
                         // round); with `queue` set, long decodes hand the pieces
                         // past the first round out through the counter
    unsigned *queue;     // piece counter in the workspace (reset by workgroup 0)
    // top-k sparse decode (absorbed MLA): idx [B, topk] int32 cache positions;
    // the key axis of the split is the index list, entries outside
    // [0, lens[b]) select nothing
    const int *idx;
    int topk;
    // FP8 E4M3 cache (fp8 != 0): k / v hold one-byte codes (strides in
    // elements = bytes); the value of (b, h, t, d) is code * scale[b, h, t]
    int fp8;
    const float *k_scale, *v_scale;
    long long ks_sb, ks_sh, ks_st, vs_sb, vs_sh, vs_st;
    // sliding window (> 0): the query at position len - 1 sees only the
    // last min(len, window) keys, rows len - that .. len - 1 of the cache
    int window;
};

int launch_decode_bf16(const DecodeArgs &a, int Dk, int Dv, hipStream_t stream);
// Flat decode over an FP8 E4M3 cache (a.fp8 = 1, a.n_wg > 0, a.S >= 3).
int launch_decode_fp8(const DecodeArgs &a, int Dk, int Dv, hipStream_t stream);
// Absorbed-MLA shape (Dk 576, Dv 512, V = latent prefix of K), 128 heads per block.
int launch_mla_decode(const DecodeArgs &a, hipStream_t stream);
// The same over the positions listed in a.idx; chunk <= mla_topk_max_chunk().
int launch_mla_decode_topk(const DecodeArgs &a, hipStream_t stream);
int mla_topk_max_chunk();
int mla_heads_per_block();
int decode_bf16_key_tile();
// Flat (balanced) decode for Dk = Dv <= 128: workgroups to launch, and how
// many of them are resident at once (the first round).
int decode_bf16_flat_workgroups(int Dk);
int decode_bf16_flat_first_round(int Dk);
int decode_fp8_flat_workgroups(int Dk);
int decode_bf16_heads_per_block(int Dk, int G);

// fp32 VALU paths (small head dims; exactness-first).
struct F32FwdArgs {
    const float *q, *k, *v;
    float *out;
    int B, Hq, Hkv, Tq, Tk, G, causal;
    float scale;
    int Gt, P, n_hblk;  // set by the launcher: heads x positions per workgroup, head blocks
};
int launch_fwd_f32(const F32FwdArgs &a, int D, hipStream_t stream);
int launch_decode_f32(const DecodeArgs &a, int D, hipStream_t stream);

// Log-sum-exp combine of the decode partials into the output.
struct CombineArgs {
    const float *part_o;  // [B, Hq, S, Dv] fp32
    const float *part_lse;
    void *out;           // [B, Hq, 1, Dv], bf16 or fp32
    int B, Hq, S, Dv;
    int out_bf16;
};
int launch_combine(const CombineArgs &a, hipStream_t stream);

// Exact LSE merge of S partial results of `rows` rows: part s of row r has
// its output at o + r*o_rs + s*o_ss (Dv fp32) and its lse at
// lse + r*l_rs + s*l_ss, natural log times lse_mul = log2(e), or base 2
// with lse_mul = 1.
struct MergeArgs {
    const float *o;
    const float *lse;
    void *out;         // [rows, Dv], bf16 or fp32
    long long rows;
    int S, Dv;
    int out_bf16;
    long long o_rs, o_ss, l_rs, l_ss;
    float lse_mul;
};
int launch_merge(const MergeArgs &a, hipStream_t stream);

} // namespace gqa
