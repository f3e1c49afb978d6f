"""Python binding of libgqa_attn.so: causal grouped-query attention on MI355X.

Argument marshalling only: every step of the attention runs in the HIP
kernels of the library.  PyTorch supplies device memory and the current
stream.  There is no fallback: if the library is missing, every call raises.

    attention(q, k, v, scale=None, causal=True)       prefill / suffix forward
    attention_varlen(q, k, v, cu_q, cu_k, scale=None, causal=True, window=0)
                                                      packed variable-length forward, sliding window
    decode(q, k_cache, v_cache, seq_lens, scale=None) split-KV single-token decode
    decode_noalloc(q, k_cache, v_cache, seq_lens, out) the same decode with no device allocation
    decode_topk(q, kv_cache, seq_lens, indices)       top-k sparse (DSA) decode, absorbed MLA
    decode_fp8(q, k_codes, v_codes, k_scale, v_scale, seq_lens)
                                                      decode over an FP8 E4M3 cache with row scales
    attention_shard(q, k, v, q_pos0, k_pos0)          one key shard: fp32 partial output + LSE
    merge(o_parts, lse_parts)                         exact LSE merge of partial results

Shapes follow the C header include/gqa_attn.h: q [B,Hq,Tq,Dk], k [B,Hkv,Tk,Dk],
v [B,Hkv,Tk,Dv]; decode caches [B,Hkv,Tmax,D] with any element strides whose
last dim is unit-stride (for the absorbed-MLA shape pass v_cache = k_cache[..., :512]).
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = [
    "LIB_PATH", "GQA_BF16", "GQA_F32", "GQAError", "lib", "attention", "attention_varlen", "check_cu_seqlens",
    "decode",
    "decode_splits", "decode_workspace_size", "decode_noalloc", "decode_noalloc_scratch_bytes", "decode_topk", "decode_topk_splits", "check_topk_distinct", "decode_fp8", "decode_fp8_splits", "attention_shard", "merge", "strerror",
]

# The library to load: the in-tree build, or another build of it (e.g. the
# NaN-fill debug build) named by GQA_ATTN_LIB.
LIB_PATH = os.environ.get("GQA_ATTN_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgqa_attn.so")
GQA_BF16, GQA_F32 = 0, 1
GQA_OK, GQA_ERR_INVALID_ARG, GQA_ERR_UNSUPPORTED, GQA_ERR_WORKSPACE, GQA_ERR_HIP = 0, -1, -2, -3, -4

EXPORTS = ("gqa_attn_fwd", "gqa_attn_fwd_varlen", "gqa_attn_decode", "gqa_attn_decode_splits",
           "gqa_attn_decode_workspace_size", "gqa_attn_decode_topk", "gqa_attn_decode_topk_splits",
           "gqa_attn_decode_fp8", "gqa_attn_decode_fp8_splits", "gqa_attn_fwd_shard", "gqa_attn_merge", "gqa_attn_decode_window",
           "gqa_attn_decode_noalloc", "gqa_attn_decode_noalloc_scratch_bytes", "gqa_attn_strerror")

_lib = None


class GQAError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {strerror(code)} (code {code})")


def lib() -> ctypes.CDLL:
    """Load the in-tree HIP library (built by causal_grouped_query_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m causal_grouped_query_amd.build` "
                "(there is no CPU fallback)")
        L = ctypes.CDLL(LIB_PATH)
        P, I, LL, F, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong, ctypes.c_float, ctypes.c_size_t
        L.gqa_attn_fwd.restype = I
        L.gqa_attn_fwd.argtypes = [P, P, P, P, I, I, I, I, I, I, I, F, I, I, P]
        L.gqa_attn_fwd_varlen.restype = I
        L.gqa_attn_fwd_varlen.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, LL, LL, LL, LL, LL, LL, LL, LL,
                                          F, I, I, I, P]
        L.gqa_attn_decode_splits.restype = I
        L.gqa_attn_decode_splits.argtypes = [I, I, I, I, I, I, I]
        L.gqa_attn_decode_workspace_size.restype = SZ
        L.gqa_attn_decode_workspace_size.argtypes = [I, I, I, I]
        L.gqa_attn_decode.restype = I
        L.gqa_attn_decode.argtypes = [P, P, P, P, P, I, I, I, I, I, I, LL, LL, LL, LL, LL, LL, F, I, P, SZ,
                                      I, P]
        L.gqa_attn_decode_topk_splits.restype = I
        L.gqa_attn_decode_topk_splits.argtypes = [I, I, I, I, I, I]
        L.gqa_attn_decode_topk.restype = I
        L.gqa_attn_decode_topk.argtypes = [P, P, P, P, P, I, I, I, I, I, I, LL, LL, F, I, P, SZ, I, P]
        L.gqa_attn_decode_fp8.restype = I
        L.gqa_attn_decode_fp8_splits.restype = I
        L.gqa_attn_decode_fp8_splits.argtypes = [I, I, I, I, I, I]
        L.gqa_attn_decode_fp8.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I] + [LL] * 12 + [F, I, I, P, SZ, P]
        L.gqa_attn_decode_window.restype = I
        L.gqa_attn_decode_window.argtypes = [P, P, P, P, P, I, I, I, I, I, I, LL, LL, LL, LL, LL, LL, F, I, I, P,
                                             SZ, I, P]
        L.gqa_attn_fwd_shard.restype = I
        L.gqa_attn_fwd_shard.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, LL, LL, F, I, I, P]
        L.gqa_attn_merge.restype = I
        L.gqa_attn_merge.argtypes = [P, P, P, I, LL, I, I, P]
        L.gqa_attn_decode_noalloc.restype = I
        L.gqa_attn_decode_noalloc.argtypes = [P, P, P, P, P, I, I, I, I, I, I, LL, LL, LL, LL, LL, LL, F, I, I, P]
        L.gqa_attn_decode_noalloc_scratch_bytes.restype = SZ
        L.gqa_attn_decode_noalloc_scratch_bytes.argtypes = [I, I, I, I, I]
        L.gqa_attn_strerror.restype = ctypes.c_char_p
        L.gqa_attn_strerror.argtypes = [I]
        _lib = L
    return _lib


def strerror(code: int) -> str:
    return lib().gqa_attn_strerror(int(code)).decode()


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return GQA_BF16
    if t.dtype == torch.float32:
        return GQA_F32
    raise ValueError(f"unsupported dtype {t.dtype}: use bfloat16 or float32")


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check_cuda(*ts):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must be on a HIP device (torch 'cuda')")


def attention(q, k, v, scale: float | None = None, causal: bool = True, out=None):
    """o = softmax(q k^T * scale + causal mask) v, KV head g(a) = a // (Hq // Hkv).

    q [B,Hq,Tq,Dk], k [B,Hkv,Tk,Dk], v [B,Hkv,Tk,Dv]: contiguous, same dtype
    (bfloat16 or float32) on one device.  Queries sit at positions Tk-Tq..Tk-1.
    """
    import torch
    _check_cuda(q, k, v)
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, H, T, D]")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share a dtype")
    B, Hq, Tq, Dk = q.shape
    Bk, Hkv, Tk, Dk2 = k.shape
    Bv, Hkv2, Tk2, Dv = v.shape
    if not (B == Bk == Bv and Hkv == Hkv2 and Tk == Tk2 and Dk == Dk2):
        raise ValueError("inconsistent q/k/v shapes")
    if scale is None:
        scale = 1.0 / math.sqrt(Dk)
    if out is None:
        out = torch.empty((B, Hq, Tq, Dv), dtype=q.dtype, device=q.device)
    elif out.shape != (B, Hq, Tq, Dv) or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous [B,Hq,Tq,Dv] tensor of q's dtype")
    rc = lib().gqa_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, Hq, Hkv, Tq, Tk,
                            Dk, Dv, float(scale), int(bool(causal)), _dtype_code(q), _stream())
    if rc != GQA_OK:
        raise GQAError(rc, "gqa_attn_fwd")
    return out


def _token_strides(t, name):
    """(head stride, token stride) in elements of a [total, H, D] tensor view."""
    if t.dim() != 3 or t.stride(2) != 1:
        raise ValueError(f"{name} must be a 3-D [total, H, D] tensor with unit-stride D")
    return t.stride(1), t.stride(0)


def check_cu_seqlens(cu, total: int, name: str = "cu_seqlens") -> None:
    """Host-side check of packed-sequence offsets (a list, array or CPU
    tensor): non-decreasing, starting at or above 0, ending at or below
    `total` token slots.  Raises ValueError otherwise."""
    vals = [int(x) for x in (cu.tolist() if hasattr(cu, "tolist") else cu)]
    if len(vals) < 2:
        raise ValueError(f"{name} needs num_seqs + 1 >= 2 offsets")
    if vals[0] < 0:
        raise ValueError(f"{name}[0] = {vals[0]} is negative")
    for i in range(len(vals) - 1):
        if vals[i + 1] < vals[i]:
            raise ValueError(f"{name} decreases at {i}: {vals[i]} -> {vals[i + 1]}")
    if vals[-1] > total:
        raise ValueError(f"{name}[-1] = {vals[-1]} exceeds the {total} token slots of the tensor")


def attention_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, scale: float | None = None, causal: bool = True,
                     window: int = 0, out=None, seqused_q=None, seqused_k=None, validate: bool = False):
    """Packed variable-length forward.  q [total_q, Hq, Dk], k [total_k, Hkv, Dk],
    v [total_k, Hkv, Dv] (any strides with unit-stride D), bfloat16; sequence i
    owns tokens cu_seqlens[i] .. cu_seqlens[i+1]-1 (int32 device tensors of
    num_seqs + 1 offsets).  window = w > 0 (causal only): each query sees its
    w most recent positions.  cu_seqlens_q[-1] must equal q.shape[0].
    seqused_q / seqused_k (int32 device tensors of num_seqs entries, optional):
    only the first seqused[i] tokens of slot i are used, the rest is padding;
    padded query rows of out are not written.  Returns out [total_q, Hq, Dv].
    The kernel clamps every sequence to the tensors' token extents; with
    validate=True the offsets are also copied to the host and checked
    (check_cu_seqlens), which synchronises with the device.
    """
    import torch
    _check_cuda(q, k, v, cu_seqlens_q, cu_seqlens_k)
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share a dtype")
    if cu_seqlens_q.dtype != torch.int32 or cu_seqlens_k.dtype != torch.int32:
        raise ValueError("cu_seqlens must be int32")
    if cu_seqlens_q.dim() != 1 or cu_seqlens_q.shape != cu_seqlens_k.shape or cu_seqlens_q.numel() < 2:
        raise ValueError("cu_seqlens_q / cu_seqlens_k must be 1-D with the same num_seqs + 1 entries")
    if not (cu_seqlens_q.is_contiguous() and cu_seqlens_k.is_contiguous()):
        raise ValueError("cu_seqlens must be contiguous")
    used = []
    for u in (seqused_q, seqused_k):
        if u is None:
            used.append(None)
            continue
        _check_cuda(u)
        if u.dtype != torch.int32 or u.dim() != 1 or u.numel() != cu_seqlens_q.numel() - 1 or not u.is_contiguous():
            raise ValueError("seqused must be a contiguous int32 tensor of num_seqs entries")
        used.append(u.data_ptr())
    q_sh, q_st = _token_strides(q, "q")
    k_sh, k_st = _token_strides(k, "k")
    v_sh, v_st = _token_strides(v, "v")
    total_q, Hq, Dk = q.shape
    _, Hkv, Dk2 = k.shape
    Dv = v.shape[2]
    if Dk != Dk2 or v.shape[1] != Hkv or v.shape[0] != k.shape[0]:
        raise ValueError("inconsistent q/k/v shapes")
    n = cu_seqlens_q.numel() - 1
    if validate:
        check_cu_seqlens(cu_seqlens_q.cpu(), total_q, "cu_seqlens_q")
        check_cu_seqlens(cu_seqlens_k.cpu(), k.shape[0], "cu_seqlens_k")
    if scale is None:
        scale = 1.0 / math.sqrt(Dk)
    if out is None:
        out = torch.empty((total_q, Hq, Dv), dtype=q.dtype, device=q.device)
    elif out.shape != (total_q, Hq, Dv) or out.dtype != q.dtype:
        raise ValueError("out must be a [total_q, Hq, Dv] tensor of q's dtype")
    if total_q == 0:
        return out  # no query token (an empty tensor has no storage to pass)
    o_sh, o_st = _token_strides(out, "out")
    rc = lib().gqa_attn_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                   cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), used[0], used[1], n, Hq, Hkv,
                                   total_q, k.shape[0], Dk, Dv, q_sh, q_st, k_sh, k_st, v_sh, v_st, o_sh, o_st,
                                   float(scale), int(bool(causal)), int(window), _dtype_code(q), _stream())
    if rc != GQA_OK:
        raise GQAError(rc, "gqa_attn_fwd_varlen")
    return out


def decode_splits(B: int, Hq: int, Hkv: int, Tmax: int, Dk: int, Dv: int, dtype_code: int) -> int:
    s = lib().gqa_attn_decode_splits(B, Hq, Hkv, Tmax, Dk, Dv, dtype_code)
    if s < 0:
        raise GQAError(s, "gqa_attn_decode_splits")
    return s


def decode_workspace_size(B: int, Hq: int, Dv: int, num_splits: int) -> int:
    return int(lib().gqa_attn_decode_workspace_size(B, Hq, Dv, num_splits))


def _decode_shapes(q, k_cache, v_cache, seq_lens):
    """Checks shared by the decode wrappers; returns B, Hq, Hkv, Tmax, Dk, Dv."""
    import torch
    _check_cuda(q, k_cache, v_cache, seq_lens)
    if q.dim() != 4 or q.shape[2] != 1 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [B, Hq, 1, Dk] tensor")
    if k_cache.dim() != 4 or v_cache.dim() != 4:
        raise ValueError("caches must be 4-D [B, Hkv, Tmax, D]")
    if k_cache.stride(3) != 1 or v_cache.stride(3) != 1:
        raise ValueError("the head dim of each cache must be unit-stride")
    if not (q.dtype == k_cache.dtype == v_cache.dtype):
        raise ValueError("q and caches must share a dtype")
    if seq_lens.dtype != torch.int32 or seq_lens.dim() != 1 or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must be a contiguous int32 tensor [B]")
    B, Hq, _, Dk = q.shape
    Bk, Hkv, Tmax, Dk2 = k_cache.shape
    Bv, Hkv2, Tmax2, Dv = v_cache.shape
    if not (B == Bk == Bv == seq_lens.shape[0] and Hkv == Hkv2 and Tmax == Tmax2 and Dk == Dk2):
        raise ValueError("inconsistent q / cache / seq_lens shapes")
    return B, Hq, Hkv, Tmax, Dk, Dv


def decode(q, k_cache, v_cache, seq_lens, scale: float | None = None, num_splits: int = 0, out=None,
           workspace=None, window: int = 0):
    """Single-token decode: q [B,Hq,1,Dk] over caches [B,Hkv,Tmax,D] holding seq_lens[b] keys.

    seq_lens: int32 device tensor [B].  Cache slots at or past seq_lens[b] are
    never read into the result.  num_splits = 0 lets the library choose.
    window = w > 0: only the last min(seq_lens[b], w) keys (sliding window).
    """
    import torch
    B, Hq, Hkv, Tmax, Dk, Dv = _decode_shapes(q, k_cache, v_cache, seq_lens)
    code = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(Dk)
    S = num_splits if num_splits else decode_splits(B, Hq, Hkv, Tmax, Dk, Dv, code)
    need = decode_workspace_size(B, Hq, Dv, S)
    if need == 0:
        raise GQAError(GQA_ERR_INVALID_ARG, "gqa_attn_decode_workspace_size")
    if workspace is None:
        workspace = torch.empty((need,), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((B, Hq, 1, Dv), dtype=q.dtype, device=q.device)
    elif out.shape != (B, Hq, 1, Dv) or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous [B,Hq,1,Dv] tensor of q's dtype")
    ks, vs = k_cache.stride(), v_cache.stride()
    if window:
        rc = lib().gqa_attn_decode_window(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), out.data_ptr(),
                                          seq_lens.data_ptr(), B, Hq, Hkv, Tmax, Dk, Dv, ks[0], ks[1], ks[2],
                                          vs[0], vs[1], vs[2], float(scale), int(window), int(S),
                                          workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                          code, _stream())
        where = "gqa_attn_decode_window"
    else:
        rc = lib().gqa_attn_decode(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), out.data_ptr(),
                                   seq_lens.data_ptr(), B, Hq, Hkv, Tmax, Dk, Dv, ks[0], ks[1], ks[2], vs[0],
                                   vs[1], vs[2], float(scale), int(S), workspace.data_ptr(),
                                   workspace.numel() * workspace.element_size(), code, _stream())
        where = "gqa_attn_decode"
    if rc != GQA_OK:
        raise GQAError(rc, where)
    return out


def decode_noalloc(q, k_cache, v_cache, seq_lens, out, scale: float | None = None, num_splits: int = 0):
    """decode() through gqa_attn_decode_noalloc: the split partials live in
    the library's per-GPU scratch array, so the call allocates nothing (out
    is the caller's [B,Hq,1,Dv] tensor).  Calls that overlap on one GPU race
    on that array; a shape whose partials exceed it raises GQAError
    (GQA_ERR_WORKSPACE)."""
    B, Hq, Hkv, Tmax, Dk, Dv = _decode_shapes(q, k_cache, v_cache, seq_lens)
    code = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(Dk)
    _check_cuda(out)
    if out.shape != (B, Hq, 1, Dv) or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous [B,Hq,1,Dv] tensor of q's dtype")
    ks, vs = k_cache.stride(), v_cache.stride()
    rc = lib().gqa_attn_decode_noalloc(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), out.data_ptr(),
                                       seq_lens.data_ptr(), B, Hq, Hkv, Tmax, Dk, Dv, ks[0], ks[1], ks[2], vs[0],
                                       vs[1], vs[2], float(scale), int(num_splits), code, _stream())
    if rc != GQA_OK:
        raise GQAError(rc, "gqa_attn_decode_noalloc")
    return out


def decode_noalloc_scratch_bytes(B: int, Hq: int, Dv: int, num_splits: int, dtype_code: int) -> int:
    """Bytes of the per-GPU scratch a decode_noalloc shape needs (0: invalid)."""
    return int(lib().gqa_attn_decode_noalloc_scratch_bytes(B, Hq, Dv, num_splits, dtype_code))


def decode_fp8_splits(B: int, Hq: int, Hkv: int, Tmax: int, Dk: int, Dv: int) -> int:
    """Split count decode_fp8 uses with num_splits = 0 (never above
    decode_splits(..., GQA_BF16), so a workspace sized for that fits)."""
    s = lib().gqa_attn_decode_fp8_splits(B, Hq, Hkv, Tmax, Dk, Dv)
    if s < 0:
        raise GQAError(s, "gqa_attn_decode_fp8_splits")
    return s


def decode_topk_splits(B: int, Hq: int, topk: int, Dk: int, Dv: int, dtype_code: int) -> int:
    s = lib().gqa_attn_decode_topk_splits(B, Hq, topk, Dk, Dv, dtype_code)
    if s < 0:
        raise GQAError(s, "gqa_attn_decode_topk_splits")
    return s


def check_topk_distinct(indices, seq_lens) -> None:
    """Host-side check that no row of a top-k list (CPU tensor or array
    [B, topk]) names a valid position twice; raises ValueError otherwise."""
    import numpy as np
    idx = np.asarray(indices.cpu() if hasattr(indices, "cpu") else indices)
    lens = np.asarray(seq_lens.cpu() if hasattr(seq_lens, "cpu") else seq_lens)
    for b in range(idx.shape[0]):
        row = idx[b][(idx[b] >= 0) & (idx[b] < lens[b])]
        if np.unique(row).size != row.size:
            raise ValueError(f"indices row {b} lists a position more than once")


def decode_topk(q, kv_cache, seq_lens, indices, Dv: int = 512, scale: float | None = None,
                num_splits: int = 0, out=None, workspace=None, validate: bool = False):
    """Top-k sparse decode on the absorbed-MLA cache: q [B,Hq,1,Dk] attends
    only to the cache positions listed in indices [B, topk] (int32; entries
    outside [0, seq_lens[b]) select nothing).  kv_cache [B,1,Tmax,Dk] (or
    [B,Tmax,Dk]); the value is its first Dv columns.  Returns [B,Hq,1,Dv].
    A position repeated inside one slice of the list counts once; repeats
    across slices count once per slice (see the C header).  validate=True
    checks on the host that no row repeats a position (synchronises)."""
    import torch
    _check_cuda(q, kv_cache, seq_lens, indices)
    if q.dim() != 4 or q.shape[2] != 1 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [B, Hq, 1, Dk] tensor")
    kv = kv_cache[:, 0] if kv_cache.dim() == 4 else kv_cache
    if kv.dim() != 3 or (kv_cache.dim() == 4 and kv_cache.shape[1] != 1) or kv.stride(2) != 1:
        raise ValueError("kv_cache must be [B, 1, Tmax, Dk] or [B, Tmax, Dk] with a unit-stride last dim")
    if q.dtype != kv.dtype:
        raise ValueError("q and the cache must share a dtype")
    if seq_lens.dtype != torch.int32 or seq_lens.dim() != 1 or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must be a contiguous int32 tensor [B]")
    if indices.dtype != torch.int32 or indices.dim() != 2 or not indices.is_contiguous():
        raise ValueError("indices must be a contiguous int32 tensor [B, topk]")
    B, Hq, _, Dk = q.shape
    if kv.shape[0] != B or kv.shape[2] != Dk or seq_lens.shape[0] != B or indices.shape[0] != B:
        raise ValueError("inconsistent q / cache / seq_lens / indices shapes")
    Tmax, topk = kv.shape[1], indices.shape[1]
    if validate:
        check_topk_distinct(indices, seq_lens)
    code = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(Dk)
    S = num_splits if num_splits else decode_topk_splits(B, Hq, topk, Dk, Dv, code)
    need = decode_workspace_size(B, Hq, Dv, S)
    if need == 0:
        raise GQAError(GQA_ERR_INVALID_ARG, "gqa_attn_decode_workspace_size")
    if workspace is None:
        workspace = torch.empty((need,), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((B, Hq, 1, Dv), dtype=q.dtype, device=q.device)
    elif out.shape != (B, Hq, 1, Dv) or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous [B,Hq,1,Dv] tensor of q's dtype")
    rc = lib().gqa_attn_decode_topk(q.data_ptr(), kv.data_ptr(), out.data_ptr(), seq_lens.data_ptr(),
                                    indices.data_ptr(), B, Hq, Tmax, topk, Dk, Dv, kv.stride(0), kv.stride(1),
                                    float(scale), int(S), workspace.data_ptr(),
                                    workspace.numel() * workspace.element_size(), code, _stream())
    if rc != GQA_OK:
        raise GQAError(rc, "gqa_attn_decode_topk")
    return out


def decode_fp8(q, k_codes, v_codes, k_scale, v_scale, seq_lens, scale: float | None = None, num_splits: int = 0,
               out=None, workspace=None, window: int = 0):
    """Single-token decode over an FP8 E4M3 cache: k_codes / v_codes
    [B,Hkv,Tmax,D] (uint8 or float8_e4m3fn storage, unit-stride last dim),
    k_scale / v_scale [B,Hkv,Tmax] float32 row scales; element (b,h,t,d)
    stands for e4m3(code) * scale[b,h,t].  q [B,Hq,1,D] bfloat16.  Returns
    [B,Hq,1,D] bfloat16."""
    import torch
    _check_cuda(q, k_codes, v_codes, k_scale, v_scale, seq_lens)
    if q.dim() != 4 or q.shape[2] != 1 or not q.is_contiguous() or q.dtype != torch.bfloat16:
        raise ValueError("q must be a contiguous bfloat16 [B, Hq, 1, D] tensor")
    for c in (k_codes, v_codes):
        if c.dim() != 4 or c.element_size() != 1 or c.stride(3) != 1:
            raise ValueError("code caches must be 4-D one-byte tensors with a unit-stride last dim")
    for sc in (k_scale, v_scale):
        if sc.dim() != 3 or sc.dtype != torch.float32:
            raise ValueError("scales must be float32 [B, Hkv, Tmax]")
    if seq_lens.dtype != torch.int32 or seq_lens.dim() != 1 or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must be a contiguous int32 tensor [B]")
    B, Hq, _, Dk = q.shape
    _, Hkv, Tmax, Dk2 = k_codes.shape
    Dv = v_codes.shape[3]
    if (k_codes.shape[0] != B or Dk2 != Dk or v_codes.shape[:3] != k_codes.shape[:3]
            or k_scale.shape != k_codes.shape[:3] or v_scale.shape != k_codes.shape[:3]
            or seq_lens.shape[0] != B):
        raise ValueError("inconsistent q / code / scale / seq_lens shapes")
    if scale is None:
        scale = 1.0 / math.sqrt(Dk)
    S = num_splits if num_splits else decode_fp8_splits(B, Hq, Hkv, Tmax, Dk, Dv)
    need = decode_workspace_size(B, Hq, Dv, S)
    if need == 0:
        raise GQAError(GQA_ERR_INVALID_ARG, "gqa_attn_decode_workspace_size")
    if workspace is None:
        workspace = torch.empty((need,), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((B, Hq, 1, Dv), dtype=q.dtype, device=q.device)
    elif out.shape != (B, Hq, 1, Dv) or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous [B,Hq,1,Dv] bfloat16 tensor")
    ks, vs, kss, vss = k_codes.stride(), v_codes.stride(), k_scale.stride(), v_scale.stride()
    rc = lib().gqa_attn_decode_fp8(q.data_ptr(), k_codes.data_ptr(), v_codes.data_ptr(), k_scale.data_ptr(),
                                   v_scale.data_ptr(), out.data_ptr(), seq_lens.data_ptr(), B, Hq, Hkv, Tmax, Dk,
                                   Dv, ks[0], ks[1], ks[2], vs[0], vs[1], vs[2], kss[0], kss[1], kss[2], vss[0],
                                   vss[1], vss[2], float(scale), int(window), int(S), workspace.data_ptr(),
                                   workspace.numel() * workspace.element_size(), _stream())
    if rc != GQA_OK:
        raise GQAError(rc, "gqa_attn_decode_fp8")
    return out


def attention_shard(q, k, v, q_pos0: int, k_pos0: int, scale: float | None = None, causal: bool = True,
                    out=None, lse=None):
    """Forward over one shard of the keys (context parallelism): q [B,Hq,Tq,Dk]
    at absolute positions q_pos0 + i, k / v [B,Hkv,Tk,D] at k_pos0 + j, all
    contiguous bfloat16.  Returns (out fp32 [B,Hq,Tq,Dv], lse fp32 [B,Hq,Tq],
    natural log, -inf where the shard holds no visible key)."""
    import torch
    _check_cuda(q, k, v)
    for t in (q, k, v):
        if t.dim() != 4 or not t.is_contiguous() or t.dtype != torch.bfloat16:
            raise ValueError("q, k, v must be contiguous 4-D bfloat16 tensors")
    B, Hq, Tq, Dk = q.shape
    _, Hkv, Tk, _ = k.shape
    Dv = v.shape[3]
    if scale is None:
        scale = 1.0 / math.sqrt(Dk)
    if out is None:
        out = torch.empty((B, Hq, Tq, Dv), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq, Tq), dtype=torch.float32, device=q.device)
    if (out.shape != (B, Hq, Tq, Dv) or out.dtype != torch.float32 or not out.is_contiguous()
            or lse.shape != (B, Hq, Tq) or lse.dtype != torch.float32 or not lse.is_contiguous()):
        raise ValueError("out must be fp32 [B,Hq,Tq,Dv] and lse fp32 [B,Hq,Tq], contiguous")
    rc = lib().gqa_attn_fwd_shard(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, Hq,
                                  Hkv, Tq, Tk, Dk, Dv, int(q_pos0), int(k_pos0), float(scale), int(bool(causal)),
                                  GQA_BF16, _stream())
    if rc != GQA_OK:
        raise GQAError(rc, "gqa_attn_fwd_shard")
    return out, lse


def merge(o_parts, lse_parts, out_dtype=None, out=None):
    """Exact log-sum-exp merge: o_parts fp32 [S, ..., Dv], lse_parts fp32
    [S, ...] (natural log) -> [..., Dv] (bfloat16 by default, or float32)."""
    import torch
    _check_cuda(o_parts, lse_parts)
    if o_parts.dtype != torch.float32 or lse_parts.dtype != torch.float32:
        raise ValueError("partials must be float32")
    if not (o_parts.is_contiguous() and lse_parts.is_contiguous()) or o_parts.shape[:-1] != lse_parts.shape:
        raise ValueError("o_parts [S, ..., Dv] and lse_parts [S, ...] must be contiguous and agree")
    S, Dv = o_parts.shape[0], o_parts.shape[-1]
    rows = lse_parts[0].numel()
    out_dtype = torch.bfloat16 if out_dtype is None else out_dtype
    code = {torch.bfloat16: GQA_BF16, torch.float32: GQA_F32}[out_dtype]
    if out is None:
        out = torch.empty(o_parts.shape[1:], dtype=out_dtype, device=o_parts.device)
    elif out.shape != o_parts.shape[1:] or out.dtype != out_dtype or not out.is_contiguous():
        raise ValueError("out must be contiguous with the shape of one part")
    rc = lib().gqa_attn_merge(o_parts.data_ptr(), lse_parts.data_ptr(), out.data_ptr(), S, rows, Dv, code, _stream())
    if rc != GQA_OK:
        raise GQAError(rc, "gqa_attn_merge")
    return out
