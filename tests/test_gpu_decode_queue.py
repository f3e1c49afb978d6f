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
    equal-chunk schedule (S = 2, no queue) and sampled rows with the oracle.

Each case first checks, with the kernel's own piece-count rule, that the
queue is used (more pieces than the first round of 1024 workgroups, and at
least 48 tiles per first-round workgroup).  Tolerance as for every bf16
path: max |err| <= 2e-2, mean |err| <= 2e-3.
"""
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


def _queued(lens, Hkv, Tmax, S, G=4):
    """Whether the balanced decode uses its queue (host replica of the
    kernel's rule: T key tiles, n_max in the longest stream, N pieces)."""
    tiles = [(min(max(int(n), 0), Tmax) + 31) // 32 for n in lens]
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
