"""GPU parity on seeded random shapes: every entry point against the fp64
oracle, same tolerances as the targeted modules (bf16: max |err| <= 2e-2,
mean <= 2e-3; fp32: 1e-5).

The targeted modules pick their shapes case by case; this sweep draws them
from a seeded generator instead: group sizes that are not powers of two
(3, 5, 7), several KV heads, query and key counts on and off the tile edges,
causal and non-causal, sliding windows, split counts from one to more
pieces than tiles, empty and one-key sequences, fp32 and bf16.  Each case
prints its parameters before it runs, so a failure names its shape.
"""
import math

import numpy as np
import pytest
import torch

import causal_grouped_query_amd as gqa
import workloads as W
from oracle import oracle as O

pytestmark = pytest.mark.gpu

TOL = {"bf16": (2e-2, 2e-3), "f32": (1e-5, 1e-5)}
DT = {"bf16": torch.bfloat16, "f32": torch.float32}
N_CASES = 24


def _rand(shape, g, dtype="bf16"):
    return torch.randn(*shape, generator=g, dtype=torch.float32).to(DT[dtype])


def _check(gpu, ref, dtype, what):
    g = gpu.detach().double().cpu().numpy().reshape(ref.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    d = np.abs(g - ref)
    tmax, tmean = TOL[dtype]
    print(f"{what} max_abs={d.max():.3e} mean_abs={d.mean():.3e}", flush=True)
    assert d.max() <= tmax and d.mean() <= tmean, f"{what}: max {d.max():.3e} mean {d.mean():.3e}"


def _heads(rng):
    Hkv = int(rng.choice([1, 2, 3]))
    G = int(rng.choice([1, 2, 3, 4, 5, 7, 8, 16]))
    return Hkv * G, Hkv


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    gqa.lib()
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_forward(i):
    rng = np.random.default_rng(5000 + i)
    Hq, Hkv = _heads(rng)
    B = int(rng.integers(1, 4))
    D = int(rng.choice([64, 128]))
    causal = bool(rng.integers(0, 2))
    Tq = int(rng.integers(1, 300))
    Tk = Tq + int(rng.integers(0, 300)) if causal else int(rng.integers(1, 500))
    dtype = "f32" if i % 3 == 0 else "bf16"
    what = f"fwd B={B} Hq={Hq} Hkv={Hkv} Tq={Tq} Tk={Tk} D={D} causal={causal} {dtype}"
    print(what, flush=True)
    g = torch.Generator("cpu").manual_seed(6000 + i)
    q, k, v = _rand((B, Hq, Tq, D), g, dtype), _rand((B, Hkv, Tk, D), g, dtype), _rand((B, Hkv, Tk, D), g, dtype)
    scale = 1.0 / math.sqrt(D)
    out = gqa.attention(q.cuda(), k.cuda(), v.cuda(), scale=scale, causal=causal)
    ref = O.attention(q, k, v, scale, causal)
    _check(out, ref, dtype, what)


@pytest.mark.parametrize("i", range(8))
def test_random_forward_many_tiles(i):
    """Longer sequences (several query tiles and key tiles per workgroup,
    several head blocks), checked on sampled rows: tile and head-block
    edges of the first and last heads plus 400 random rows."""
    rng = np.random.default_rng(20000 + i)
    Hkv = int(rng.choice([1, 2, 4]))
    Hq = Hkv * int(rng.choice([1, 2, 3, 4, 6, 8, 12, 16, 32]))
    B = int(rng.integers(1, 3))
    D = int(rng.choice([64, 128]))
    causal = bool(rng.integers(0, 4))
    Tq = int(rng.integers(300, 2500))
    Tk = Tq + int(rng.integers(0, 1500)) if causal else int(rng.integers(200, 3000))
    dtype = "f32" if i % 4 == 0 else "bf16"
    what = f"fwd rows B={B} Hq={Hq} Hkv={Hkv} Tq={Tq} Tk={Tk} D={D} causal={causal} {dtype}"
    print(what, flush=True)
    g = torch.Generator("cpu").manual_seed(21000 + i)
    q, k, v = _rand((B, Hq, Tq, D), g, dtype), _rand((B, Hkv, Tk, D), g, dtype), _rand((B, Hkv, Tk, D), g, dtype)
    scale = 1.0 / math.sqrt(D)
    out = gqa.attention(q.cuda(), k.cuda(), v.cuda(), scale=scale, causal=causal)
    n = B * Hq * Tq
    edges = [(b * Hq + a) * Tq + p for b in range(B) for a in (0, Hq - 1) for p in (0, 63, 64, 255, 256, Tq - 1)
             if p < Tq]
    rows = np.unique(np.concatenate([rng.integers(0, n, 400), [0, n - 1], edges]))
    ref = O.attention(q, k, v, scale, causal, rows=rows.tolist())
    _check(out.reshape(n, D)[torch.from_numpy(rows).cuda()], ref, dtype, what)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_decode(i):
    rng = np.random.default_rng(7000 + i)
    Hq, Hkv = _heads(rng)
    B = int(rng.integers(1, 6))
    D = int(rng.choice([64, 128]))
    T = int(rng.integers(1, 1500))
    lens = [int(rng.integers(0, T + 1)) for _ in range(B)]
    lens[int(rng.integers(0, B))] = T  # one full-length sequence
    window = int(rng.choice([0, 0, 1, 33, int(rng.integers(1, T + 1))]))
    splits = int(rng.choice([0, 1, 2, 3, 5, 9, 40]))
    dtype = "f32" if i % 4 == 0 else "bf16"
    what = f"decode B={B} Hq={Hq} Hkv={Hkv} T={T} lens={lens} D={D} w={window} S={splits} {dtype}"
    print(what, flush=True)
    g = torch.Generator("cpu").manual_seed(8000 + i)
    q, k, v = _rand((B, Hq, 1, D), g, dtype), _rand((B, Hkv, T, D), g, dtype), _rand((B, Hkv, T, D), g, dtype)
    scale = 1.0 / math.sqrt(D)
    ref = O.attention(q, k, v, scale, True, kv_lens=lens, window=window)
    for b, n in enumerate(lens):  # cache slots past the length are never read
        k[b, :, n:] = float("nan")
        v[b, :, n:] = float("nan")
    out = gqa.decode(q.cuda(), k.cuda(), v.cuda(), torch.tensor(lens, dtype=torch.int32).cuda(), scale=scale,
                     num_splits=splits, window=window)
    _check(out, ref, dtype, what)


@pytest.mark.parametrize("i", range(12))
def test_random_varlen(i):
    rng = np.random.default_rng(9000 + i)
    Hq, Hkv = _heads(rng)
    D = int(rng.choice([64, 128]))
    causal = bool(rng.integers(0, 3))  # mostly causal
    n = int(rng.integers(1, 7))
    lens_k = [int(rng.integers(0, 400)) for _ in range(n)]
    lens_k[0] = max(lens_k[0], 1)  # at least one key in the batch
    lens_q = [int(rng.integers(0, lk + 1)) if causal else int(rng.integers(0, 300)) for lk in lens_k]
    window = int(rng.choice([0, 0, 1, 17, 128])) if causal else 0
    what = f"varlen Hq={Hq} Hkv={Hkv} D={D} causal={causal} w={window} q={lens_q} k={lens_k}"
    print(what, flush=True)
    cq, ck = [0] + np.cumsum(lens_q).tolist(), [0] + np.cumsum(lens_k).tolist()
    g = torch.Generator("cpu").manual_seed(9500 + i)
    q, k, v = _rand((max(cq[-1], 1), Hq, D), g), _rand((max(ck[-1], 1), Hkv, D), g), _rand((max(ck[-1], 1), Hkv, D), g)
    q, k, v = q[:cq[-1]], k[:ck[-1]], v[:ck[-1]]
    if cq[-1] == 0:
        return  # nothing to compute (the no-query case has a test of its own)
    scale = 1.0 / math.sqrt(D)
    out = gqa.attention_varlen(q.cuda(), k.cuda(), v.cuda(), torch.tensor(cq, dtype=torch.int32).cuda(),
                               torch.tensor(ck, dtype=torch.int32).cuda(), scale=scale, causal=causal, window=window)
    ref = O.attention_varlen(q, k, v, cq, ck, scale, causal, window=window)
    _check(out, ref, "bf16", what)


@pytest.mark.parametrize("i", range(8))
def test_random_fp8_decode(i):
    rng = np.random.default_rng(10000 + i)
    Hq, Hkv = _heads(rng)
    B = int(rng.integers(1, 5))
    D = int(rng.choice([64, 128]))
    T = int(rng.integers(1, 1200))
    lens = [int(rng.integers(0, T + 1)) for _ in range(B)]
    splits = int(rng.choice([0, 3, 4, 11]))
    what = f"fp8 decode B={B} Hq={Hq} Hkv={Hkv} T={T} lens={lens} D={D} S={splits}"
    print(what, flush=True)
    w = W.GQA_DECODE_FP8.scaled(B=B, Hq=Hq, Hkv=Hkv, Tk=T, Dk=D, Dv=D, seed=10500 + i, len_lo=0, len_hi=0)
    q, kc, vc, ks, vs, _ = W.fp8_decode_inputs(w, nan_tail=False)
    for b, n in enumerate(lens):
        ks[b, :, n:] = float("nan")
        vs[b, :, n:] = float("nan")
    scale = 1.0 / math.sqrt(D)
    out = gqa.decode_fp8(q.cuda(), kc.cuda(), vc.cuda(), ks.cuda(), vs.cuda(),
                         torch.tensor(lens, dtype=torch.int32).cuda(), scale=scale, num_splits=splits)
    ref = O.attention_e4m3kv(q, kc, ks, vc, vs, scale, True, kv_lens=lens)
    _check(out, ref, "bf16", what)


@pytest.mark.parametrize("i", range(8))
def test_random_mla_and_topk(i):
    rng = np.random.default_rng(11000 + i)
    Hq = int(rng.choice([16, 64, 128, 136, 256]))
    B = int(rng.integers(1, 4))
    T = int(rng.integers(1, 2000))
    lens = [int(rng.integers(0, T + 1)) for _ in range(B)]
    lens[0] = T
    splits = int(rng.choice([0, 1, 3, 6]))
    topk = int(rng.integers(1, 700))
    what = f"mla/top-k B={B} Hq={Hq} T={T} lens={lens} S={splits} topk={topk}"
    print(what, flush=True)
    g = torch.Generator("cpu").manual_seed(11500 + i)
    q, kv = _rand((B, Hq, 1, 576), g), _rand((B, 1, T, 576), g)
    scale = 1.0 / math.sqrt(192.0)
    # dense absorbed-MLA decode
    ref = O.attention(q, kv, kv[..., :512], scale, True, kv_lens=lens)
    for b, n in enumerate(lens):
        kv[b, :, n:] = float("nan")
    kvd = kv.cuda()
    lens_d = torch.tensor(lens, dtype=torch.int32).cuda()
    out = gqa.decode(q.cuda(), kvd, kvd[..., :512], lens_d, scale=scale, num_splits=splits)
    _check(out, ref, "bf16", "dense " + what)
    # top-k: distinct positions in random order, -1 padding and out-of-range entries
    idx = np.full((B, topk), -1, dtype=np.int32)
    for b, n in enumerate(lens):
        m = min(n, int(rng.integers(0, topk + 1)))
        sel = rng.permutation(n)[:m]
        junk = rng.integers(n, n + 50, int(rng.integers(0, topk - m + 1)))
        row = np.concatenate([sel, junk]).astype(np.int32)
        idx[b, :row.size] = row
        idx[b] = rng.permutation(idx[b])
    ts = int(rng.choice([0, 1, 2, 5]))
    out = gqa.decode_topk(q.cuda(), kvd, lens_d, torch.from_numpy(idx).cuda(), scale=scale, num_splits=ts)
    kv_ref = kv.clone()
    for b, n in enumerate(lens):
        kv_ref[b, :, n:] = 0.0  # (never selected; the oracle reads only listed positions in range)
    ref = O.decode_topk(q, kv_ref, np.asarray(lens, dtype=np.int32), idx, scale, 512)
    _check(out, ref, "bf16", f"top-k S={ts} " + what)
