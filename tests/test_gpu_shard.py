"""GPU parity of the key-shard forward (gqa_attn_fwd_shard) and the LSE merge
(gqa_attn_merge) against the fp64 oracle: the single-GPU part of sequence /
context parallelism (each device's shard result, and the exact merge that
follows the exchange of partial results).

Tolerances: outputs as for every bf16-input path (max |err| <= 2e-2, mean
<= 2e-3); LSE max |err| <= 1e-2 (the normaliser sums bf16-rounded weights);
merging fp32 partials into fp32, max |err| <= 1e-5.
"""
import numpy as np
import pytest
import torch

import causal_grouped_query_amd as gqa
from oracle import oracle as O

pytestmark = pytest.mark.gpu


def _rand(shape, seed):
    g = torch.Generator("cpu").manual_seed(seed)
    return torch.randn(*shape, generator=g, dtype=torch.float32).to(torch.bfloat16)


def _check(gpu, ref, what, tmax=2e-2, tmean=2e-3):
    g = gpu.detach().double().cpu().numpy().reshape(ref.shape)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(g), fin), f"{what}: finite pattern differs"
    assert np.array_equal(g[~fin], ref[~fin]), f"{what}: infinite entries differ"
    d = np.abs(g[fin] - ref[fin]) if fin.any() else np.zeros(1)
    print(f"{what} max_abs={d.max():.3e} mean_abs={d.mean():.3e}", flush=True)
    assert d.max() <= tmax and d.mean() <= tmean, f"{what}: max {d.max():.3e} mean {d.mean():.3e}"


@pytest.mark.parametrize("q_pos0,k_pos0", [
    (1000, 0),      # every key of the shard is in the past: all visible
    (1000, 900),    # the shard crosses the queries' positions (diagonal)
    (1000, 1100),   # partly in the future: the first queries see nothing
    (100, 5000),    # entirely in the future: zero rows, lse = -inf
])
@pytest.mark.parametrize("Hq,Hkv,D", [(32, 8, 128), (16, 1, 128), (8, 2, 64)])
def test_shard_matches_oracle(q_pos0, k_pos0, Hq, Hkv, D):
    B, Tq, Tk = 2, 200, 300
    q = _rand((B, Hq, Tq, D), 500)
    k = _rand((B, Hkv, Tk, D), 501)
    v = _rand((B, Hkv, Tk, D), 502)
    scale = 1.0 / np.sqrt(D)
    out, lse = gqa.attention_shard(q.cuda(), k.cuda(), v.cuda(), q_pos0, k_pos0, scale=scale, causal=True)
    ref, ref_lse = O.attention_shard(q, k, v, scale, True, q_pos0, k_pos0)
    _check(out, ref, f"shard out q0={q_pos0} k0={k_pos0} {Hq}/{Hkv} D{D}")
    _check(lse, ref_lse, f"shard lse q0={q_pos0} k0={k_pos0}", tmax=1e-2, tmean=2e-3)
    if k_pos0 > q_pos0 + Tq:
        assert torch.all(out == 0) and torch.all(torch.isneginf(lse))


def test_shard_noncausal():
    q = _rand((1, 8, 70, 128), 510)
    k = _rand((1, 2, 130, 128), 511)
    v = _rand((1, 2, 130, 128), 512)
    out, lse = gqa.attention_shard(q.cuda(), k.cuda(), v.cuda(), 0, 10**6, scale=0.1, causal=False)
    ref, ref_lse = O.attention_shard(q, k, v, 0.1, False, 0, 10**6)
    _check(out, ref, "shard non-causal")
    _check(lse, ref_lse, "shard non-causal lse", tmax=1e-2)


def test_merge_matches_oracle_merge():
    """Random fp32 partials with some empty parts (lse = -inf) and a row
    whose parts are all empty."""
    S, rows, Dv = 5, 300, 128
    g = torch.Generator("cpu").manual_seed(520)
    o = torch.randn(S, rows, Dv, generator=g)
    lse = torch.randn(S, rows, generator=g) * 4
    lse[1, ::3] = -float("inf")
    lse[:, 7] = -float("inf")
    ref, _ = O.lse_merge(o.permute(0, 1, 2).numpy().astype(np.float64), lse.numpy().astype(np.float64))
    ref[7] = 0.0  # the merge of nothing is a zero row
    out32 = gqa.merge(o.cuda(), lse.cuda(), out_dtype=torch.float32)
    _check(out32, ref, "merge fp32", tmax=1e-5, tmean=1e-6)
    out16 = gqa.merge(o.cuda(), lse.cuda())
    _check(out16, ref, "merge bf16", tmax=2e-2, tmean=2e-3)


@pytest.mark.parametrize("nshard", [2, 4, 7])
def test_context_parallel_shards_merge_to_full_attention(nshard):
    """A causal prefill (B2, 32 / 8 heads, 1024 positions) with its keys cut
    into shards as devices of a context-parallel group would hold them: each
    shard's partial result for all queries, merged, equals full causal
    attention."""
    B, Hq, Hkv, T, D = 2, 32, 8, 1024, 128
    q = _rand((B, Hq, T, D), 530)
    k = _rand((B, Hkv, T, D), 531)
    v = _rand((B, Hkv, T, D), 532)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    cuts = np.linspace(0, T, nshard + 1).astype(int)
    outs, lses = [], []
    for a, b in zip(cuts[:-1], cuts[1:]):
        o, l = gqa.attention_shard(qd, kd[:, :, a:b].contiguous(), vd[:, :, a:b].contiguous(), 0, int(a),
                                   causal=True)
        outs.append(o)
        lses.append(l)
    merged = gqa.merge(torch.stack(outs), torch.stack(lses))
    rng = np.random.default_rng(533)
    rows = sorted(set(rng.integers(0, B * Hq * T, 400).tolist()) | {0, T - 1, B * Hq * T - 1})
    ref = O.attention(q, k, v, 1.0 / np.sqrt(D), True, rows=rows)
    got = merged.reshape(B * Hq * T, D)[rows]
    _check(got, ref, f"context parallel, {nshard} shards")


@pytest.mark.parametrize("Dv,S", [(512, 3), (64, 9), (128, 1)])
def test_merge_other_widths(Dv, S):
    rows = 257
    g = torch.Generator("cpu").manual_seed(540 + Dv)
    o = torch.randn(S, rows, Dv, generator=g)
    lse = torch.randn(S, rows, generator=g) * 3
    if S > 1:
        lse[0, 5:9] = -float("inf")
    ref, _ = O.lse_merge(o.numpy().astype(np.float64), lse.numpy().astype(np.float64))
    out = gqa.merge(o.cuda(), lse.cuda(), out_dtype=torch.float32)
    _check(out, ref, f"merge Dv={Dv} S={S}", tmax=1e-5, tmean=1e-6)
