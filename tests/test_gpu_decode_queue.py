"""The balanced bf16 decode of a long decode (more pieces than resident
workgroups, and at least 48 key tiles per resident workgroup): one round of
workgroups takes large first pieces, and the later workgroups draw the rest
from a counter kept in the last 256 bytes of the workspace (zeroed by the
kernel itself).

Checked against the fp64 oracle:
  * whatever the counter holds on entry (0, a mid-range ticket, a value past
    the end, all ones), with the rest of the workspace NaN-filled;
  * two shapes back to back on one workspace, then the first one again (the
    counter left by one call is the next call's stale value);
  * the full-size ragged GQA decode at split counts that change the piece
    sizes of the small last pieces, every output row compared with the
    equal-chunk schedule (S = 2, no queue) and sampled rows with the oracle;
  * seeded random long decodes: group sizes 1 to 48 (two head blocks),
    1 to 8 KV heads, head dims 128 (queued) and 64 (equal pieces), sliding
    windows, split counts 3 to 64, empty and one-key sequences, NaN past
    every sequence's end; sampled rows against the oracle (GQA_QUEUE_CASES
    cases, default 4, plus seed 7020: head dim 64 with more workgroups
    resident than the first round, which once let a draw before the
    counter's reset read a stale count of 2^31 or more as a negative piece
    index).

Each case first checks, with the kernel's own piece-count rule, that the
queue is used (more pieces than the first round of 1024 workgroups, and at
least 48 tiles per first-round workgroup).  Tolerance as for every bf16
path: max |err| <= 2e-2, mean |err| <= 2e-3.
"""
import math
import os

import numpy as np
import pytest
import torch

import causal_grouped_query_amd as gqa
import workloads as W
from oracle import oracle as O

pytestmark = pytest.mark.gpu

FIRST_ROUND = 1024   # workgroups resident at once (4 per CU x 256 CUs)
MAX_PIECES = 2048    # pieces of the balanced schedule at most
MIN_TILES = 48       # key tiles per first-round workgroup for the queue


def _queued(lens, Hkv, Tmax, S, G=4, window=0, D=128):
    """Whether the balanced decode uses its queue (host replica of the
    kernel's rule: T key tiles, n_max in the longest stream, N pieces; head
    dim 64 fits more than 1024 workgroups at once and takes equal pieces)."""
    if D != 128:
        return False
    eff = [min(max(int(n), 0), Tmax) for n in lens]
    if window > 0:
        eff = [min(n, window) for n in eff]
    tiles = [(n + 31) // 32 for n in eff]
    H = Hkv * ((G + 31) // 32)
    T = sum(tiles) * H
    nmax = max(tiles)
    if T == 0:
        return False
    N = max(1, min(T * (S - 2) // ((nmax - 2 if nmax > 2 else 0) + S - 2), MAX_PIECES))
    return N > FIRST_ROUND and T >= FIRST_ROUND * MIN_TILES


def _rand(shape, seed):
    g = torch.Generator("cpu").manual_seed(seed)
    return torch.randn(*shape, generator=g, dtype=torch.float32).to(torch.bfloat16)


def _check(gpu, ref, what):
    g = gpu.detach().double().cpu().numpy().reshape(ref.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    d = np.abs(g - ref)
    print(f"{what} max_abs={d.max():.3e} mean_abs={d.mean():.3e}", flush=True)
    assert d.max() <= 2e-2 and d.mean() <= 2e-3, f"{what}: max {d.max():.3e} mean {d.mean():.3e}"


def _case(seed, B=48, Hq=32, Hkv=8, T=8192, D=128):
    rng = np.random.default_rng(seed)
    lens = rng.integers(T // 2, T + 1, size=B)
    lens[0], lens[-1] = T, 1
    q, k, v = _rand((B, Hq, 1, D), seed + 1), _rand((B, Hkv, T, D), seed + 2), _rand((B, Hkv, T, D), seed + 3)
    return q, k, v, [int(x) for x in lens]


@pytest.fixture(scope="module")
def case900():
    q, k, v, lens = _case(900)
    ref = O.attention(q, k, v, 1.0 / np.sqrt(q.shape[-1]), True, kv_lens=lens)
    return (q.cuda(), k.cuda(), v.cuda(), torch.tensor(lens, dtype=torch.int32).cuda()), lens, ref


def _workspace(nbytes, counter):
    ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")
    ws[nbytes - 256:nbytes - 252] = torch.tensor([counter], dtype=torch.int64).view(torch.uint8)[:4].cuda()
    return ws


@pytest.mark.parametrize("counter", [0, 7, 500, 1 << 31, 0xFFFFFFFF])
def test_queue_any_counter_on_entry(case900, counter):
    (q, k, v, lens_d), lens, ref = case900
    B, Hq, _, D = q.shape
    S = 32
    assert _queued(lens, 8, 8192, S)
    ws = _workspace(gqa.decode_workspace_size(B, Hq, D, S), counter)
    out = gqa.decode(q, k, v, lens_d, num_splits=S, workspace=ws)
    _check(out, ref, f"queued decode, counter {counter:#x} on entry")


def test_queue_back_to_back_shapes_share_a_workspace():
    a = _case(910)
    b = _case(920, B=40, T=7000)
    S = 24
    for lens, Tm in ((a[3], 8192), (b[3], 7000)):
        assert _queued(lens, 8, Tm, S)
    nbytes = max(gqa.decode_workspace_size(x[0].shape[0], 32, 128, S) for x in (a, b))
    ws = _workspace(nbytes, 0xFFFFFFFF)
    for name, (q, k, v, lens) in (("first", a), ("second", b), ("first again", a)):
        out = gqa.decode(q.cuda(), k.cuda(), v.cuda(), torch.tensor(lens, dtype=torch.int32).cuda(),
                         num_splits=S, workspace=ws)
        ref = O.attention(q, k, v, 1.0 / np.sqrt(128), True, kv_lens=lens)
        _check(out, ref, f"queued decode, {name} shape on a shared workspace")


def test_queue_full_size_split_counts():
    w = W.GQA_DECODE
    q, k, v, lens = W.decode_inputs(w, nan_tail=True)
    qd, kd, vd, ld = q.cuda(), k.cuda(), v.cuda(), lens.cuda()
    base = gqa.decode(qd, kd, vd, ld, scale=w.scale, num_splits=2)  # equal chunks, no queue
    rows = sorted({0, w.B * w.Hq - 1, *np.random.default_rng(930).integers(0, w.B * w.Hq, 40).tolist()})
    ref = O.attention(q, k, v, w.scale, True, kv_lens=lens.tolist(), rows=rows)
    for S in (3, 8, 16, 32, 48, 64):
        queued = _queued(lens.tolist(), w.Hkv, w.Tk, S)
        out = gqa.decode(qd, kd, vd, ld, scale=w.scale, num_splits=S)
        torch.cuda.synchronize()
        d = (out.float() - base.float()).abs()
        print(f"S={S} queue={queued}: vs equal chunks max {d.max().item():.3e}", flush=True)
        assert torch.isfinite(out).all() and d.max().item() <= 2e-2 and d.mean().item() <= 2e-3
        got = out.reshape(-1, w.Dv)[torch.tensor(rows, device="cuda")]
        _check(got, ref, f"full-size GQA decode S={S} (queue {queued}), sampled rows")
    assert _queued(lens.tolist(), w.Hkv, w.Tk, 32) and not _queued(lens.tolist(), w.Hkv, w.Tk, 3)


def _random_long_decode(seed):
    rng = np.random.default_rng(seed)
    D = int(rng.choice([64, 128]))
    G = int(rng.choice([1, 2, 3, 4, 8, 16, 48]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    Tmax = int(rng.choice([2048, 4096, 8192, 12000]))
    window = int(rng.choice([0, 0, 0, 700, 3000]))
    S = int(rng.integers(3, 65))
    lo = int(rng.choice([1, Tmax // 4, Tmax // 2]))
    eff = (lo + Tmax) / 2 if window == 0 else min(window, (lo + Tmax) / 2)
    tiles_per_seq = Hkv * ((G + 31) // 32) * max(eff / 32, 1)
    B = int(math.ceil(1.5 * FIRST_ROUND * MIN_TILES / tiles_per_seq))
    if B * Hkv * Tmax * D * 4 > (3 << 30):  # keep the host cache small: long sequences instead
        window, lo, Tmax = 0, 4096, 8192
        B = int(math.ceil(1.5 * FIRST_ROUND * MIN_TILES / (Hkv * ((G + 31) // 32) * 192)))
    lens = rng.integers(lo, Tmax + 1, size=B)
    lens[rng.integers(0, B)] = 0
    lens[rng.integers(0, B)] = 1
    lens[0] = Tmax
    return dict(B=B, Hq=G * Hkv, Hkv=Hkv, Tmax=Tmax, D=D, window=window, S=S, lens=[int(x) for x in lens])


@pytest.mark.parametrize("seed", sorted({*range(7000, 7000 + int(os.environ.get("GQA_QUEUE_CASES", "4"))), 7020}))
def test_queue_random_long_decodes(seed):
    c = _random_long_decode(seed)
    B, Hq, Hkv, Tmax, D, window, S, lens = (c[k] for k in ("B", "Hq", "Hkv", "Tmax", "D", "window", "S", "lens"))
    G = Hq // Hkv
    print(f"seed {seed}: B={B} Hq={Hq} Hkv={Hkv} Tmax={Tmax} D={D} window={window} S={S}", flush=True)
    assert _queued(lens, Hkv, Tmax, S, G=G, window=window, D=D) == (D == 128)
    g = torch.Generator("cpu").manual_seed(seed)
    q = torch.randn(B, Hq, 1, D, generator=g).to(torch.bfloat16)
    k = torch.randn(B, Hkv, Tmax, D, generator=g).to(torch.bfloat16)
    v = torch.randn(B, Hkv, Tmax, D, generator=g).to(torch.bfloat16)
    for b, n in enumerate(lens):
        k[b, :, n:] = float("nan")
        v[b, :, n:] = float("nan")
    lens_t = torch.tensor(lens, dtype=torch.int32)
    out = gqa.decode(q.cuda(), k.cuda(), v.cuda(), lens_t.cuda(), num_splits=S, window=window)
    torch.cuda.synchronize()
    rng = np.random.default_rng(seed + 1)
    rows = sorted({0, B * Hq - 1, *(b * Hq for b in range(B) if lens[b] <= 1),
                   *rng.integers(0, B * Hq, 48).tolist()})
    ref = O.attention(q, k, v, 1.0 / np.sqrt(D), True, kv_lens=lens, rows=rows, window=window)
    got = out.reshape(-1, D)[torch.tensor(rows, device="cuda")]
    _check(got, ref, f"random long decode seed {seed}")
