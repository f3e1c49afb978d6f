"""GPU parity of the top-k sparse (DSA) decode on the absorbed-MLA cache
(gqa_attn_decode_topk) against the fp64 oracle.

Tolerance as for every bf16 path: max |err| <= 2e-2, mean |err| <= 2e-3.
Cases: selections shorter and longer than a 32-entry tile, lists padded with
-1 and with positions past the sequence's length, sequences with no valid
entry and of length 0, cache slots past the length holding NaN, 1 .. many
slices of the list, a partial second 128-head block, the full-size workload
(every row), and the all-positions selection against the dense MLA decode.
"""
import numpy as np
import pytest
import torch

import causal_grouped_query_amd as gqa
import workloads as W
from oracle import oracle as O

pytestmark = pytest.mark.gpu

TMAX, TMEAN = 2e-2, 2e-3
SCALE = 1.0 / np.sqrt(192.0)


def _rand(shape, seed):
    g = torch.Generator("cpu").manual_seed(seed)
    return torch.randn(*shape, generator=g, dtype=torch.float32).to(torch.bfloat16)


def _check(gpu, ref, what):
    g = gpu.detach().double().cpu().numpy().reshape(ref.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    d = np.abs(g - ref)
    print(f"{what} max_abs={d.max():.3e} mean_abs={d.mean():.3e}", flush=True)
    assert d.max() <= TMAX and d.mean() <= TMEAN, f"{what}: max {d.max():.3e} mean {d.mean():.3e}"


def _problem(B, Hq, Tmax, lens, topk, seed, extra_invalid=0):
    q = _rand((B, Hq, 1, 576), seed)
    kv = _rand((B, 1, Tmax, 576), seed + 1)
    for b, n in enumerate(lens):
        kv[b, :, n:, :] = float("nan")
    rng = np.random.default_rng(seed + 2)
    idx = np.full((B, topk), -1, dtype=np.int32)
    for b, n in enumerate(lens):
        m = min(n, topk - extra_invalid)
        sel = rng.permutation(n)[:m]
        junk = rng.integers(n, n + 1000, extra_invalid)   # past the length: select nothing
        row = np.concatenate([sel, junk, np.full(topk - m - extra_invalid, -1)]).astype(np.int32)
        idx[b] = rng.permutation(row)
    return q, kv, np.asarray(lens, dtype=np.int32), idx


def _run(q, kv, lens, idx, splits=0):
    return gqa.decode_topk(q.cuda(), kv.cuda(), torch.from_numpy(lens).cuda(), torch.from_numpy(idx).cuda(),
                           scale=SCALE, num_splits=splits)


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 0])
def test_topk_decode_small(splits):
    q, kv, lens, idx = _problem(3, 128, 700, [700, 37, 300], 100, 200, extra_invalid=5)
    out = _run(q, kv, lens, idx, splits)
    ref = O.decode_topk(q, kv, lens, idx, SCALE, 512)
    _check(out, ref, f"topk small S={splits}")


@pytest.mark.parametrize("Hq", [16, 160])
def test_topk_decode_head_counts(Hq):
    q, kv, lens, idx = _problem(2, Hq, 400, [400, 129], 250, 210)
    out = _run(q, kv, lens, idx)
    ref = O.decode_topk(q, kv, lens, idx, SCALE, 512)
    _check(out, ref, f"topk Hq={Hq}")


def test_topk_decode_empty_selections_and_sequences():
    """Sequence 0: only invalid entries; sequence 1: length 0; sequence 2:
    a single valid entry (its output is that latent row, up to rounding)."""
    B, Hq, Tmax, topk = 3, 128, 96, 40
    q = _rand((B, Hq, 1, 576), 220)
    kv = _rand((B, 1, Tmax, 576), 221)
    lens = np.array([50, 0, 96], dtype=np.int32)
    kv[0, :, 50:] = float("nan")
    kv[1] = float("nan")
    idx = np.full((B, topk), -1, dtype=np.int32)
    idx[0, :10] = np.arange(50, 60)      # all past the length
    idx[1, :5] = np.arange(5)            # length 0: nothing valid
    idx[2, 17] = 61
    out = _run(q, kv, lens, idx, 2)
    ref = O.decode_topk(q, kv, lens, idx, SCALE, 512)
    assert torch.all(out[:2] == 0)
    _check(out, ref, "topk empty / single")


@pytest.mark.parametrize("splits", [1, 3])
def test_topk_reference_moves_out_of_order(splits):
    """Scores that climb by ~60 in log2 units along the cache, visited in the
    random order of a selection list: a head's reference max moves whenever a
    later entry names a much larger score (the rescale path, in any order)."""
    B, Hq, T, topk = 2, 128, 900, 640
    lens = np.array([900, 700], dtype=np.int32)
    q = _rand((B, Hq, 1, 576), 240)
    kv = _rand((B, 1, T, 576), 241).float()
    qd = q.float()[:, 0, 0, :]
    qd = qd / qd.norm(dim=-1, keepdim=True)
    kv = (kv + torch.linspace(0.0, 25.0, T)[None, None, :, None] * qd[:, None, None, :]).to(torch.bfloat16)
    for b, n in enumerate(lens):
        kv[b, :, n:, :] = float("nan")
    rng = np.random.default_rng(242)
    idx = np.stack([rng.permutation(int(n))[:topk] for n in lens]).astype(np.int32)
    out = _run(q, kv, lens, idx, splits)
    ref = O.decode_topk(q, kv, lens, idx, SCALE, 512)
    _check(out, ref, f"topk ramp S={splits}")


def test_topk_all_positions_equals_dense_mla_decode():
    """Selecting every position in order with the same slicing gives the
    dense MLA decode bit for bit (same tiles, same arithmetic)."""
    B, Hq, T = 2, 128, 512
    q = _rand((B, Hq, 1, 576), 230).cuda()
    kv = _rand((B, 1, T, 576), 231).cuda()
    lens = torch.full((B,), T, dtype=torch.int32, device="cuda")
    idx = torch.arange(T, dtype=torch.int32, device="cuda").repeat(B, 1).contiguous()
    for S in (1, 4):
        sparse = gqa.decode_topk(q, kv, lens, idx, scale=SCALE, num_splits=S)
        dense = gqa.decode(q, kv, kv[..., :512], lens, scale=SCALE, num_splits=S)
        assert torch.equal(sparse, dense), f"S={S}"


def test_topk_workload_full_size():
    """The benchmarked DSA workload (B16, 128 heads, top-2048 of caches up to
    32768), every output row against the oracle."""
    w = W.MLA_TOPK
    q, k, _, lens = W.decode_inputs(w)
    idx = W.topk_indices(w, lens)
    out = gqa.decode_topk(q.cuda(), k.cuda(), lens.cuda(), idx.cuda(), scale=w.scale)
    ref = O.decode_topk(q, k, lens, idx, w.scale, w.Dv)
    _check(out, ref, "topk workload")


def _with_repeats(lens, topk, n_distinct, seed):
    """Index rows of n_distinct positions each, filled up to topk with repeats
    of positions already listed, shuffled."""
    rng = np.random.default_rng(seed)
    idx = np.full((len(lens), topk), -1, dtype=np.int32)
    for b, n in enumerate(lens):
        sel = rng.permutation(n)[:min(n, n_distinct)]
        rep = rng.choice(sel, topk - sel.size)
        idx[b] = rng.permutation(np.concatenate([sel, rep])).astype(np.int32)
    return idx


@pytest.mark.parametrize("splits", [1, 0])
def test_topk_repeated_positions_in_one_slice_count_once(splits):
    """The page's index mask is a scatter: a position listed twice is selected
    once.  With one slice (splits=1) every repeat is inside it; with the
    default split the repeats of each slice are drawn from that slice's own
    positions.  Either way the result is the oracle's set semantics."""
    lens, topk = [500, 300, 37], 256
    q, kv, lens_a, _ = _problem(3, 128, 512, lens, topk, 71)
    if splits == 1:
        idx = _with_repeats(lens, topk, 100, 72)
    else:
        S = gqa.decode_topk_splits(3, 128, topk, 576, 512, gqa.GQA_BF16)
        chunk = -(-topk // S)
        chunk = -(-chunk // 32) * 32
        idx = np.full((3, topk), -1, dtype=np.int32)
        rng = np.random.default_rng(73)
        nsl = -(-topk // chunk)
        for b, n in enumerate(lens):
            perm = rng.permutation(n)
            for si, s0 in enumerate(range(0, topk, chunk)):  # each slice: its own disjoint positions, repeated
                m = min(chunk, topk - s0)
                own = perm[si * n // nsl:(si + 1) * n // nsl][: max(1, m // 2)]
                idx[b, s0:s0 + m] = rng.permutation(np.concatenate([own, rng.choice(own, m - own.size)]))
            used = [set(idx[b, s0:s0 + chunk].tolist()) for s0 in range(0, topk, chunk)]
            assert all(not (used[i] & used[j]) for i in range(nsl) for j in range(i))  # no cross-slice repeats
    assert any(np.unique(r[r >= 0]).size < (r >= 0).sum() for r in idx)  # the rows do repeat
    out = _run(q, kv, lens_a, idx, splits)
    _check(out, O.decode_topk(q, kv, lens_a, idx, SCALE, 512), f"repeats within slices, splits={splits}")
    with pytest.raises(ValueError):
        gqa.decode_topk(q.cuda(), kv.cuda(), torch.from_numpy(lens_a).cuda(), torch.from_numpy(idx).cuda(),
                        scale=SCALE, num_splits=splits, validate=True)


def test_topk_repeats_across_slices_count_once_per_slice():
    """The documented rule for a list whose repeats fall in different slices
    (a top-k never produces one): such a position counts once per slice.
    Checked against the oracle on an expanded cache in which every list
    entry is a row of its own (set semantics there = per-entry weights)."""
    lens, topk, splits = [400, 250], 128, 2  # slices of 64 entries
    q, kv, lens_a, _ = _problem(2, 128, 448, lens, topk, 81)
    rng = np.random.default_rng(82)
    idx = np.zeros((2, topk), dtype=np.int32)
    for b, n in enumerate(lens):
        sel = rng.permutation(n)[:64]
        idx[b, :64] = sel
        idx[b, 64:] = rng.permutation(sel)  # every position once in each slice
    out = _run(q, kv, lens_a, idx, splits)
    kv_exp = torch.stack([kv[b, :, torch.from_numpy(idx[b]).long()] for b in range(2)])  # [2, 1, topk, 576]
    idx_exp = np.tile(np.arange(topk, dtype=np.int32), (2, 1))
    ref = O.decode_topk(q, kv_exp, np.full(2, topk, dtype=np.int32), idx_exp, SCALE, 512)
    _check(out, ref, "repeats across slices")
