"""Python face of the fp64 CPU oracle (gqa_oracle.c).

TEST INFRASTRUCTURE ONLY.  The test suite, the smoke check and the
benchmark's CPU-baseline leg are the only callers allowed; the HIP library
and its Python binding never import this module, and this module imports
nothing from them.

The oracle computes the dense softmax attention of the unified formula
o_a = softmax(Q_a K_{g(a)}^T * scale + M) V_{g(a)} ("Attention variants"
page, unified-notation section), row by row in fp64, with the query position
offset Tk - Tq of that page's minimal semantic implementation.  See the header
of gqa_oracle.c for the step list.  Around that one definition:

  attention / probs       dense, causal or not, decode lengths, sliding window
  attention_varlen        packed sequences (cu_seqlens), padding (seqused)
  attention_e4m3kv        an FP8 E4M3 cache with one scale per row
  attention_shard         one key shard at absolute positions (partial + lse)
  decode_topk             DSA top-k selection on the absorbed MLA cache
  lse_merge               exact merge of partial results
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gqa_oracle.c")
_LIB = os.path.join(_HERE, "libgqa_oracle.so")

BF16, F32, F64 = 0, 1, 2

_lib = None


def build(force: bool = True) -> str:
    """Compile gqa_oracle.c with gcc (plain -O2, IEEE semantics, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.run(
            ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", _SRC, "-o", tmp, "-lm"],
            check=True,
        )
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build(force=False)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        LLP = ctypes.POINTER(ctypes.c_longlong)
        I = ctypes.c_int
        lib.oracle_attention.restype = I
        lib.oracle_attention.argtypes = [
            P, LLP, I, P, LLP, I, P, LLP, I, P,
            I, I, I, I, I, I, I, ctypes.c_double, I, I, P, ctypes.c_longlong, P, P, I,
        ]
        lib.oracle_probs.restype = I
        lib.oracle_probs.argtypes = [
            P, LLP, I, P, LLP, I, P, LLP, I, P,
            I, I, I, I, I, I, I, ctypes.c_double, I, I, I, I, I, P, P,
        ]
        lib.oracle_attention_e4m3kv.restype = I
        lib.oracle_attention_e4m3kv.argtypes = [
            P, LLP, I, P, LLP, P, LLP, P, LLP, P, LLP, P,
            I, I, I, I, I, I, I, ctypes.c_double, I, P, ctypes.c_longlong, P, P, I,
        ]
        lib.oracle_attention_shard.restype = I
        lib.oracle_attention_shard.argtypes = [
            P, LLP, I, P, LLP, I, P, LLP, I,
            I, I, I, I, I, I, I, ctypes.c_double, I, ctypes.c_longlong, ctypes.c_longlong,
            P, ctypes.c_longlong, P, P, I,
        ]
        lib.oracle_e4m3_table.restype = None
        lib.oracle_e4m3_table.argtypes = [P]
        lib.oracle_lse_merge.restype = None
        lib.oracle_lse_merge.argtypes = [P, P, I, ctypes.c_longlong, I, P, P]
        lib.oracle_max_threads.restype = I
        lib.oracle_max_threads.argtypes = []
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().oracle_max_threads())


class _Operand:
    """A 4-D input seen as (pointer, element strides, storage code)."""

    def __init__(self, x):
        self.keep = x
        try:
            import torch
        except ImportError:  # pragma: no cover
            torch = None
        if torch is not None and isinstance(x, torch.Tensor):
            if x.device.type != "cpu":
                raise ValueError("oracle operands must live in host memory")
            if x.dim() != 4:
                raise ValueError("oracle operands are 4-D (b, h, t, d)")
            codes = {torch.bfloat16: BF16, torch.float32: F32, torch.float64: F64}
            if x.dtype not in codes:
                raise ValueError(f"unsupported oracle dtype {x.dtype}")
            self.code = codes[x.dtype]
            self.ptr = x.data_ptr()
            self.strides = (ctypes.c_longlong * 4)(*x.stride())
            self.shape = tuple(x.shape)
            return
        a = np.asarray(x)
        if a.ndim != 4:
            raise ValueError("oracle operands are 4-D (b, h, t, d)")
        codes = {np.dtype(np.float32): F32, np.dtype(np.float64): F64}
        if a.dtype not in codes:
            raise ValueError(f"unsupported oracle dtype {a.dtype}")
        self.keep = a
        self.code = codes[a.dtype]
        self.ptr = a.ctypes.data
        self.strides = (ctypes.c_longlong * 4)(*(s // a.itemsize for s in a.strides))
        self.shape = a.shape


def _lens_arg(kv_lens, B):
    if kv_lens is None:
        return None, None
    arr = np.ascontiguousarray(np.asarray(kv_lens, dtype=np.int32))
    if arr.shape != (B,):
        raise ValueError("kv_lens must have one entry per sequence")
    return arr, arr.ctypes.data


def attention(q, k, v, scale: float, causal: bool, kv_lens=None, rows=None, threads: int = 0,
              with_lse: bool = False, window: int = 0):
    """fp64 attention.  q [B,Hq,Tq,Dk], k [B,Hkv,Tk,Dk], v [B,Hkv,Tk,Dv].

    kv_lens: optional per-sequence key counts (a decode cache of capacity Tk);
    rows: optional flat row ids ((b*Hq)+a)*Tq+i to compute only those rows;
    window: 0, or (causal only) a sliding window of w positions: the query at
    position p sees keys max(0, p-w+1) .. p.
    Returns out [B,Hq,Tq,Dv] (or [len(rows), Dv]) in fp64, plus lse if asked.
    """
    Q, K, V = _Operand(q), _Operand(k), _Operand(v)
    B, Hq, Tq, Dk = Q.shape
    Bk, Hkv, Tk, Dk2 = K.shape
    Bv, Hkv2, Tk2, Dv = V.shape
    if not (B == Bk == Bv and Hkv == Hkv2 and Tk == Tk2 and Dk == Dk2):
        raise ValueError("inconsistent q/k/v shapes")
    lens, lens_ptr = _lens_arg(kv_lens, B)
    if rows is None:
        out = np.empty((B, Hq, Tq, Dv), dtype=np.float64)
        lse = np.empty((B, Hq, Tq), dtype=np.float64)
        rows_arr, rows_ptr, nrows = None, None, 0
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nrows = rows_arr.size
        out = np.empty((nrows, Dv), dtype=np.float64)
        lse = np.empty((nrows,), dtype=np.float64)
        rows_ptr = rows_arr.ctypes.data
    rc = _load().oracle_attention(
        Q.ptr, Q.strides, Q.code, K.ptr, K.strides, K.code, V.ptr, V.strides, V.code, lens_ptr,
        B, Hq, Hkv, Tq, Tk, Dk, Dv, float(scale), int(bool(causal)), int(window), rows_ptr, nrows,
        out.ctypes.data, lse.ctypes.data, int(threads),
    )
    if rc != 0:
        raise ValueError("oracle rejected the problem (shapes, head grouping or Tq > Tk with causal)")
    return (out, lse) if with_lse else out


def attention_shard(q, k, v, scale: float, causal: bool, q_pos0: int, k_pos0: int, rows=None,
                    threads: int = 0):
    """fp64 attention of q over one shard of the keys (context parallelism).

    Query i sits at absolute position q_pos0 + i, key j of the shard at
    k_pos0 + j; causal: key j is visible iff k_pos0 + j <= q_pos0 + i.  A
    query with no visible key in the shard gets a zero row and lse = -inf.
    Returns (out [B,Hq,Tq,Dv] or [len(rows), Dv], lse natural log), the
    partial result that lse_merge combines across shards.
    """
    Q, K, V = _Operand(q), _Operand(k), _Operand(v)
    B, Hq, Tq, Dk = Q.shape
    _, Hkv, Tk, _ = K.shape
    Dv = V.shape[3]
    if rows is None:
        out = np.empty((B, Hq, Tq, Dv), dtype=np.float64)
        lse = np.empty((B, Hq, Tq), dtype=np.float64)
        rows_ptr, nrows = None, 0
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nrows = rows_arr.size
        out = np.empty((nrows, Dv), dtype=np.float64)
        lse = np.empty((nrows,), dtype=np.float64)
        rows_ptr = rows_arr.ctypes.data
    rc = _load().oracle_attention_shard(
        Q.ptr, Q.strides, Q.code, K.ptr, K.strides, K.code, V.ptr, V.strides, V.code,
        B, Hq, Hkv, Tq, Tk, Dk, Dv, float(scale), int(bool(causal)), int(q_pos0), int(k_pos0),
        rows_ptr, nrows, out.ctypes.data, lse.ctypes.data, int(threads),
    )
    if rc != 0:
        raise ValueError("oracle rejected the problem")
    return out, lse


def e4m3_table() -> np.ndarray:
    """Values of the 256 FP8 E4M3 codes (NaN for the two NaN codes)."""
    out = np.empty(256, dtype=np.float64)
    _load().oracle_e4m3_table(out.ctypes.data)
    return out


def _host_u8_4d(x, name):
    """A 4-D array of one-byte codes (torch uint8 / float8_e4m3fn or numpy
    uint8) as (pointer, element strides, keep-alive, shape)."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            if x.device.type != "cpu" or x.dim() != 4 or x.element_size() != 1:
                raise ValueError(f"{name}: a 4-D one-byte host tensor is required")
            return x.data_ptr(), (ctypes.c_longlong * 4)(*x.stride()), x, tuple(x.shape)
    except ImportError:  # pragma: no cover
        pass
    a = np.asarray(x)
    if a.ndim != 4 or a.dtype != np.uint8:
        raise ValueError(f"{name}: a 4-D uint8 array is required")
    return a.ctypes.data, (ctypes.c_longlong * 4)(*(st // 1 for st in a.strides)), a, a.shape


def _host_f32_3d(x, name):
    try:
        import torch
        if isinstance(x, torch.Tensor):
            if x.device.type != "cpu" or x.dim() != 3 or x.dtype != torch.float32:
                raise ValueError(f"{name}: a 3-D float32 host tensor is required")
            return x.data_ptr(), (ctypes.c_longlong * 3)(*x.stride()), x, tuple(x.shape)
    except ImportError:  # pragma: no cover
        pass
    a = np.asarray(x)
    if a.ndim != 3 or a.dtype != np.float32:
        raise ValueError(f"{name}: a 3-D float32 array is required")
    return a.ctypes.data, (ctypes.c_longlong * 3)(*(st // 4 for st in a.strides)), a, a.shape


def attention_e4m3kv(q, k_codes, k_scale, v_codes, v_scale, scale: float, causal: bool, kv_lens=None,
                     rows=None, threads: int = 0):
    """fp64 attention over an FP8 E4M3 cache with one scale per row.

    k_codes [B,Hkv,Tk,Dk] and v_codes [B,Hkv,Tk,Dv] hold E4M3 codes (uint8
    or float8_e4m3fn storage); k_scale / v_scale [B,Hkv,Tk] float32.  Element
    (b,h,t,d) stands for e4m3(code) * scale[b,h,t], formed exactly in fp64;
    everything else is attention() (q as bf16 / fp32 / fp64).
    """
    Q = _Operand(q)
    kp, ks, kkeep, kshape = _host_u8_4d(k_codes, "k_codes")
    vp, vs, vkeep, vshape = _host_u8_4d(v_codes, "v_codes")
    ksp, kss, kskeep, ksshape = _host_f32_3d(k_scale, "k_scale")
    vsp, vss, vskeep, vsshape = _host_f32_3d(v_scale, "v_scale")
    B, Hq, Tq, Dk = Q.shape
    _, Hkv, Tk, Dk2 = kshape
    Dv = vshape[3]
    if (kshape[0] != B or vshape[:3] != kshape[:3] or Dk != Dk2 or ksshape != kshape[:3]
            or vsshape != kshape[:3]):
        raise ValueError("inconsistent q / code / scale shapes")
    lens, lens_ptr = _lens_arg(kv_lens, B)
    if rows is None:
        out = np.empty((B, Hq, Tq, Dv), dtype=np.float64)
        rows_ptr, nrows = None, 0
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nrows = rows_arr.size
        out = np.empty((nrows, Dv), dtype=np.float64)
        rows_ptr = rows_arr.ctypes.data
    rc = _load().oracle_attention_e4m3kv(
        Q.ptr, Q.strides, Q.code, kp, ks, ksp, kss, vp, vs, vsp, vss, lens_ptr,
        B, Hq, Hkv, Tq, Tk, Dk, Dv, float(scale), int(bool(causal)), rows_ptr, nrows,
        out.ctypes.data, None, int(threads),
    )
    if rc != 0:
        raise ValueError("oracle rejected the problem")
    return out


def probs(q, k, v, scale: float, causal: bool, b: int, a: int, i: int, kv_lens=None, window: int = 0):
    """The probability row P_j over all Tk keys (zeros where masked) and the output row."""
    Q, K, V = _Operand(q), _Operand(k), _Operand(v)
    B, Hq, Tq, Dk = Q.shape
    _, Hkv, Tk, _ = K.shape
    Dv = V.shape[3]
    lens, lens_ptr = _lens_arg(kv_lens, B)
    p = np.empty((Tk,), dtype=np.float64)
    o = np.empty((Dv,), dtype=np.float64)
    rc = _load().oracle_probs(
        Q.ptr, Q.strides, Q.code, K.ptr, K.strides, K.code, V.ptr, V.strides, V.code, lens_ptr,
        B, Hq, Hkv, Tq, Tk, Dk, Dv, float(scale), int(bool(causal)), int(window), b, a, i,
        p.ctypes.data, o.ctypes.data,
    )
    if rc != 0:
        raise ValueError("oracle rejected the problem")
    return p, o


def attention_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, scale: float, causal: bool, window: int = 0,
                     threads: int = 0, seqused_q=None, seqused_k=None):
    """fp64 attention over packed variable-length sequences.

    q [total_q, Hq, Dk], k [total_k, Hkv, Dk], v [total_k, Hkv, Dv] hold the
    tokens of all sequences back to back; sequence i owns query tokens
    cu_seqlens_q[i] .. cu_seqlens_q[i+1]-1 and key tokens cu_seqlens_k[i] ..
    cu_seqlens_k[i+1]-1 (the packed-boundary reading of cu_seqlens on the
    "Attention Architecture Evolution" page).  Tokens never attend across
    sequences.  Within a sequence the rules of attention() apply (query j sits
    at position Tk_i - Tq_i + j; causal; optional window); a query with no
    visible key (Tq_i > Tk_i) gets a zero row.  Each sequence is computed by
    attention() on strided views of its own tokens.  Returns out
    [total_q, Hq, Dv] in fp64.

    Padding ("Attention variants", masks section, lists padding masks beside
    packed-segment masks): with seqused_q / seqused_k given, sequence i uses
    only the first min(seqused[i], slot length) tokens of its slot; the rest
    are padding.  Padded keys are invisible, padded query rows are not part of
    the result (returned as zeros), and the causal offset is taken between the
    used lengths.  A right-padded batch [B, Tpad, H, D] is then cu_seqlens =
    0, Tpad, 2 Tpad, ... with seqused = the true lengths.
    """
    cq = [int(x) for x in cu_seqlens_q]
    ck = [int(x) for x in cu_seqlens_k]
    if len(cq) != len(ck) or len(cq) < 2:
        raise ValueError("cu_seqlens_q / cu_seqlens_k must have the same length >= 2")

    def used(cu, u):  # token count of each sequence, padding excluded
        n = [max(cu[i + 1] - cu[i], 0) for i in range(len(cu) - 1)]
        if u is None:
            return n
        u = [int(x) for x in u]
        if len(u) != len(n):
            raise ValueError("seqused must hold one length per sequence")
        return [min(max(a, 0), b) for a, b in zip(u, n)]

    nq, nk = used(cq, seqused_q), used(ck, seqused_k)
    total_q, Hq, _ = q.shape
    Dv = v.shape[2]
    out = np.zeros((total_q, Hq, Dv), dtype=np.float64)

    def view(x, s, e):  # tokens s..e-1 as a [1, H, T, D] strided view
        try:
            import torch
            if isinstance(x, torch.Tensor):
                return x[s:e].permute(1, 0, 2).unsqueeze(0)
        except ImportError:  # pragma: no cover
            pass
        return np.asarray(x)[s:e].transpose(1, 0, 2)[None]

    for i in range(len(cq) - 1):
        tq, tk = nq[i], nk[i]
        qe, ke = cq[i] + tq, ck[i] + tk  # ends of the used tokens
        if tq <= 0 or tk <= 0:
            continue  # no query row, or no key: rows stay zero
        qs = cq[i]
        if causal and tq > tk:
            # the first tq - tk queries sit before key 0: zero rows
            qs = cq[i] + (tq - tk)
        o = attention(view(q, qs, qe), view(k, ck[i], ke), view(v, ck[i], ke), scale, causal,
                      threads=threads, window=window)
        out[qs:qe] = o[0].transpose(1, 0, 2)
    return out


def decode_topk(q, kv, kv_lens, indices, scale: float, Dv: int, threads: int = 0):
    """fp64 single-token decode over a selected subset of the cached keys.

    DeepSeek Sparse Attention on the absorbed MLA ("Attention Architecture
    Evolution", DSA section): an indexer picks for each query token a set J
    of cached positions, and the main attention keeps only those: the index
    mask is -inf everywhere except 0 at the listed positions, added to the
    scores before the softmax.  Written, as the page's production target
    describes it, as a gather of the listed latent rows followed by ordinary
    attention over them (masked keys carry weight exactly 0, so the two
    orders give the same result).

    q [B, Hq, 1, Dk]; kv [B, 1, Tmax, Dk] is the latent cache, whose first Dv
    columns are the value (MLA: V is the latent prefix of K); kv_lens [B]
    valid cache lengths; indices [B, topk] integer positions.  J_b is the SET
    of listed positions inside [0, kv_lens[b]) (the mask is a scatter, so a
    repeated position counts once; entries outside the range, such as -1
    padding, select nothing).  An empty J_b gives a zero row.  Returns
    [B, Hq, 1, Dv] in fp64.
    """
    try:
        import torch
        is_torch = isinstance(kv, torch.Tensor)
    except ImportError:  # pragma: no cover
        is_torch = False
    B, Hq, one, Dk = q.shape
    if one != 1 or kv.shape[0] != B or kv.shape[1] != 1 or kv.shape[3] != Dk or not 0 < Dv <= Dk:
        raise ValueError("decode_topk: q [B,Hq,1,Dk], kv [B,1,Tmax,Dk], 0 < Dv <= Dk")
    def host(x):  # torch tensor or array-like -> int64 numpy
        return np.asarray(x.cpu() if hasattr(x, "cpu") else x, dtype=np.int64)

    idx, lens = host(indices), host(kv_lens)
    if idx.ndim != 2 or idx.shape[0] != B or lens.shape != (B,):
        raise ValueError("decode_topk: indices [B, topk], kv_lens [B]")
    Tmax = kv.shape[2]
    out = np.zeros((B, Hq, 1, Dv), dtype=np.float64)
    for b in range(B):
        n = min(max(int(lens[b]), 0), Tmax)
        J = sorted({int(j) for j in idx[b] if 0 <= j < n})
        if not J:
            continue
        sel = torch.as_tensor(J) if is_torch else np.asarray(J)
        kj = kv[b:b + 1, :, sel, :]        # gathered [1, 1, |J|, Dk]
        vj = kj[..., :Dv]
        out[b:b + 1] = attention(q[b:b + 1], kj, vj, scale, False, threads=threads)
    return out


def lse_merge(o_parts, lse_parts):
    """Exact merge of partial results over disjoint key ranges.

    o_parts [S, R, Dv], lse_parts [S, R] (natural log, -inf for empty parts).
    """
    o_parts = np.ascontiguousarray(o_parts, dtype=np.float64)
    lse_parts = np.ascontiguousarray(lse_parts, dtype=np.float64)
    S, R, Dv = o_parts.shape
    out = np.empty((R, Dv), dtype=np.float64)
    lse = np.empty((R,), dtype=np.float64)
    _load().oracle_lse_merge(o_parts.ctypes.data, lse_parts.ctypes.data, S, R, Dv,
                             out.ctypes.data, lse.ctypes.data)
    return out, lse
