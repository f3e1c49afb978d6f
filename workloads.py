"""Seeded synthetic inputs for the attention workloads.

This module only draws inputs: it holds none of the attention arithmetic, so
that the HIP path and the fp64 oracle can both be fed from it without sharing
any computation.

Recipe (the same for every workload and size):
  * a CPU ``torch.Generator`` seeded with the workload's seed draws q, then k,
    then v with ``randn`` in fp32 (N(0,1)), each cast by round-to-nearest-even
    to the workload's storage type (bf16 or fp32);
  * decode lengths come from a second CPU generator seeded with seed + 1000:
    ``randint(lo, hi + 1, (B,))``, i.e. uniform on [lo, hi] inclusive;
  * decode caches have capacity Tmax; for parity runs every cache slot at a
    position >= len_b is overwritten with NaN, because those slots are not
    part of the input and must not reach the output;
  * the weight-absorbed MLA shape draws only q and k: the value is the first
    512 columns of the 576-wide key (latent 512 + rope 64), taken as a view;
  * packed variable-length workloads draw all tokens of all sequences at once
    in the [total, H, D] layout; cu_seqlens are the running sums of the
    listed lengths;
  * FP8 decode caches: after q, the generator draws the key values, then
    the value values, as ``randn * 64`` clamped to the E4M3 range +-448 and
    cast by torch to float8_e4m3fn (round to nearest even; the codes are
    kept as bytes), then the key scales, then the value scales, one per
    (b, h, t) row, as 2^u with u uniform on [-8, -5] (so dequantised values
    are about N(0, 1)); rows at or past len_b hold the NaN code 0x7F and a
    NaN scale in parity runs;
  * top-k sparse decode draws the selected positions from a third CPU
    generator seeded with seed + 2000: for each sequence the first
    min(topk, len_b) entries of ``randperm(len_b)`` (distinct positions in
    random order, as a top-k over indexer scores returns them), padded
    with -1 when len_b < topk.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import torch

_DT = {"bf16": torch.bfloat16, "f32": torch.float32}


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str  # "fwd", "decode", "fp8_decode", "mla_decode", "mla_topk_decode", "fwd+decode", "fwd_varlen", "fwd_shard"
    B: int
    Hq: int
    Hkv: int
    Tq: int
    Tk: int  # forward: key length; decode: cache capacity Tmax
    Dk: int
    Dv: int
    dtype: str
    seed: int
    scale: float
    causal: bool = True
    len_lo: int = 0  # decode lengths, inclusive range
    len_hi: int = 0
    extra: dict = field(default_factory=dict)

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads of the headline comparison.
TINY_F32 = Workload("tiny_fp32_gqa_b1_hq4_hkv2_t128_d64", "fwd+decode", 1, 4, 2, 128, 128, 64, 64,
                    "f32", 0, 1.0 / 8.0, len_lo=128, len_hi=128)
GQA_PREFILL = Workload("gqa_prefill_b4_hq32_hkv8_t4096_d128", "fwd", 4, 32, 8, 4096, 4096, 128, 128,
                       "bf16", 1, 1.0 / math.sqrt(128))
GQA_DECODE = Workload("gqa_decode_b64_hq32_hkv8_tmax8192_d128", "decode", 64, 32, 8, 1, 8192, 128, 128,
                      "bf16", 2, 1.0 / math.sqrt(128), len_lo=1024, len_hi=8192)
MQA_SUFFIX = Workload("mqa_suffix_prefill_b8_hq64_hkv1_tq512_tk16384_d128", "fwd", 8, 64, 1, 512, 16384,
                      128, 128, "bf16", 3, 1.0 / math.sqrt(128))
MLA_DECODE = Workload("mla_absorbed_decode_b16_hq128_tk32768_dk576_dv512", "mla_decode", 16, 128, 1, 1,
                      32768, 576, 512, "bf16", 4, 1.0 / math.sqrt(192), len_lo=32768, len_hi=32768)

ALL = [TINY_F32, GQA_PREFILL, GQA_DECODE, MQA_SUFFIX, MLA_DECODE]

# Sliding-window prefill over packed sequences of mixed lengths (GQA 32q / 8kv,
# d128, window 4096: the GQA + SWA pairing the pages name for Mistral 7B).
# B = number of packed sequences; Tq = Tk = the longest one.
SWA_VARLEN = Workload("swa_varlen_prefill_hq32_hkv8_d128_w4096_16k_tokens", "fwd_varlen", 8, 32, 8, 8192, 8192,
                      128, 128, "bf16", 5, 1.0 / math.sqrt(128),
                      extra={"lens": (8192, 4096, 2048, 1024, 512, 256, 128, 128), "window": 4096})


def varlen_inputs(w: Workload):
    """Packed tokens for a fwd_varlen workload (CPU): q [total, Hq, Dk],
    k [total, Hkv, Dk], v [total, Hkv, Dv] (drawn q, k, v in that order) and
    cu_seqlens int32 [B + 1] (the same offsets for queries and keys)."""
    lens = list(w.extra["lens"])
    total = sum(lens)
    g = torch.Generator("cpu").manual_seed(w.seed)
    q = _randn(g, (total, w.Hq, w.Dk), w.dtype)
    k = _randn(g, (total, w.Hkv, w.Dk), w.dtype)
    v = _randn(g, (total, w.Hkv, w.Dv), w.dtype)
    cu = torch.tensor([0] + [sum(lens[: i + 1]) for i in range(len(lens))], dtype=torch.int32)
    return q, k, v, cu


# DeepSeek Sparse Attention decode on the absorbed MLA cache: each query keeps
# the 2048 cached positions an indexer selected (the DeepSeek-V3.2 setting);
# cache lengths uniform on [4096, 32768].
MLA_TOPK = Workload("mla_dsa_topk2048_decode_b16_hq128_tk32768_dk576_dv512", "mla_topk_decode", 16, 128, 1, 1,
                    32768, 576, 512, "bf16", 6, 1.0 / math.sqrt(192), len_lo=4096, len_hi=32768,
                    extra={"topk": 2048})


# The same top-k decode at batch 64 (a serving batch: one workgroup per
# sequence and head block already fills the device).
MLA_TOPK_B64 = Workload("mla_dsa_topk2048_decode_b64_hq128_tk32768_dk576_dv512", "mla_topk_decode", 64, 128, 1,
                        1, 32768, 576, 512, "bf16", 9, 1.0 / math.sqrt(192), len_lo=4096, len_hi=32768,
                        extra={"topk": 2048})


# The GQA decode shape over an FP8 E4M3 cache with one scale per row.
GQA_DECODE_FP8 = Workload("gqa_decode_fp8kv_b64_hq32_hkv8_tmax8192_d128", "fp8_decode", 64, 32, 8, 1, 8192, 128, 128,
                          "bf16", 7, 1.0 / math.sqrt(128), len_lo=1024, len_hi=8192)


# One device's share of the MQA suffix shape under sequence (context)
# parallelism over 8 devices: the 512 queries (positions 15872..16383) and
# one 2048-key shard; Tk is the shard length.
CP_SHARD = Workload("context_parallel_shard_mqa_b8_hq64_hkv1_tq512_tk2048_of_16384_d128", "fwd_shard", 8, 64, 1,
                    512, 2048, 128, 128, "bf16", 8, 1.0 / math.sqrt(128),
                    extra={"shards": 8, "q_pos0": 16384 - 512})


def _randn(gen: torch.Generator, shape, dtype: str) -> torch.Tensor:
    return torch.randn(*shape, generator=gen, dtype=torch.float32).to(_DT[dtype])


def fwd_inputs(w: Workload):
    """q [B,Hq,Tq,Dk], k [B,Hkv,Tk,Dk], v [B,Hkv,Tk,Dv] on the CPU."""
    g = torch.Generator("cpu").manual_seed(w.seed)
    q = _randn(g, (w.B, w.Hq, w.Tq, w.Dk), w.dtype)
    k = _randn(g, (w.B, w.Hkv, w.Tk, w.Dk), w.dtype)
    v = _randn(g, (w.B, w.Hkv, w.Tk, w.Dv), w.dtype)
    return q, k, v


def decode_lengths(w: Workload) -> torch.Tensor:
    g = torch.Generator("cpu").manual_seed(w.seed + 1000)
    return torch.randint(w.len_lo, w.len_hi + 1, (w.B,), generator=g, dtype=torch.int32)


def _nan_tail(cache: torch.Tensor, lens: torch.Tensor) -> None:
    for b, n in enumerate(lens.tolist()):
        cache[b, :, n:, :] = float("nan")


def decode_inputs(w: Workload, nan_tail: bool = True):
    """q [B,Hq,1,Dk], k/v caches [B,Hkv,Tmax,D], lengths int32 [B] (CPU).

    For the MLA shape, v is the view k[..., :Dv] of the shared latent.
    """
    g = torch.Generator("cpu").manual_seed(w.seed)
    q = _randn(g, (w.B, w.Hq, 1, w.Dk), w.dtype)
    k = _randn(g, (w.B, w.Hkv, w.Tk, w.Dk), w.dtype)
    if w.kind in ("mla_decode", "mla_topk_decode"):
        v = None
    else:
        v = _randn(g, (w.B, w.Hkv, w.Tk, w.Dv), w.dtype)
    lens = decode_lengths(w)
    if nan_tail:
        _nan_tail(k, lens)
        if v is not None:
            _nan_tail(v, lens)
    if v is None:
        v = k[..., : w.Dv]
    return q, k, v, lens


def topk_indices(w: Workload, lens: torch.Tensor) -> torch.Tensor:
    """Selected positions int32 [B, topk] (CPU) for a top-k decode workload."""
    topk = w.extra["topk"]
    g = torch.Generator("cpu").manual_seed(w.seed + 2000)
    idx = torch.full((w.B, topk), -1, dtype=torch.int32)
    for b, n in enumerate(lens.tolist()):
        sel = torch.randperm(n, generator=g)[:topk]
        idx[b, : sel.numel()] = sel.to(torch.int32)
    return idx


def fp8_decode_inputs(w: Workload, nan_tail: bool = True):
    """q [B,Hq,1,Dk] bf16; key / value codes uint8 [B,Hkv,Tmax,D]; key / value
    row scales float32 [B,Hkv,Tmax]; lengths int32 [B] (all CPU)."""
    g = torch.Generator("cpu").manual_seed(w.seed)
    q = _randn(g, (w.B, w.Hq, 1, w.Dk), "bf16")

    def codes(d):
        x = torch.randn(w.B, w.Hkv, w.Tk, d, generator=g, dtype=torch.float32).mul_(64.0).clamp_(-448.0, 448.0)
        return x.to(torch.float8_e4m3fn).view(torch.uint8)

    kc = codes(w.Dk)
    vc = codes(w.Dv)
    ks = torch.exp2(torch.rand(w.B, w.Hkv, w.Tk, generator=g, dtype=torch.float32).mul_(3.0).sub_(8.0))
    vs = torch.exp2(torch.rand(w.B, w.Hkv, w.Tk, generator=g, dtype=torch.float32).mul_(3.0).sub_(8.0))
    lens = decode_lengths(w)
    if nan_tail:
        for b, n in enumerate(lens.tolist()):
            kc[b, :, n:] = 0x7F
            vc[b, :, n:] = 0x7F
            ks[b, :, n:] = float("nan")
            vs[b, :, n:] = float("nan")
    return q, kc, vc, ks, vs, lens
