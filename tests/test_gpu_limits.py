"""GPU parity at the size limits of each entry point (sampled outputs
against the fp64 oracle; same tolerance as every bf16 path).

Long caches stress the 32-bit in-tile offsets and the balanced decode's
tile arithmetic (one stream of 32768 tiles), long prefills the grid and
causal-tile arithmetic, many packed sequences the device-side tile search,
and long top-k lists the index slicing (slices of at most 4096 entries).
A top-k cache whose row offsets pass 2^32 bytes (4.4 GB) takes the MLA
kernel's 64-bit copy addresses.
"""
import numpy as np
import pytest
import torch

import causal_grouped_query_amd as gqa
from oracle import oracle as O

pytestmark = pytest.mark.gpu

TMAX, TMEAN = 2e-2, 2e-3


def _rand(shape, seed, dtype=torch.bfloat16):
    g = torch.Generator("cpu").manual_seed(seed)
    return torch.randn(*shape, generator=g, dtype=torch.float32).to(dtype)


def _check(gpu, ref, what):
    g = gpu.detach().double().cpu().numpy().reshape(ref.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    d = np.abs(g - ref)
    print(f"{what} max_abs={d.max():.3e} mean_abs={d.mean():.3e}", flush=True)
    assert d.max() <= TMAX and d.mean() <= TMEAN, f"{what}: max {d.max():.3e} mean {d.mean():.3e}"


@pytest.mark.parametrize("splits", [2, 0])
def test_decode_one_million_keys(splits):
    """B1, 8 query heads on one KV head, a full cache of 2^20 keys (chunked
    schedule with 2 splits, and the balanced schedule)."""
    T, D = 1 << 20, 128
    q = _rand((1, 8, 1, D), 400)
    k = _rand((1, 1, T, D), 401)
    v = _rand((1, 1, T, D), 402)
    lens = torch.tensor([T], dtype=torch.int32)
    out = gqa.decode(q.cuda(), k.cuda(), v.cuda(), lens.cuda(), num_splits=splits)
    ref = O.attention(q, k, v, 1.0 / np.sqrt(D), True, kv_lens=[T])
    _check(out, ref, f"decode 2^20 keys S={splits}")


def test_fp8_decode_one_million_keys():
    T, D = 1 << 20, 128
    g = torch.Generator("cpu").manual_seed(410)
    q = torch.randn(1, 8, 1, D, generator=g).to(torch.bfloat16)
    kc = (torch.randn(1, 1, T, D, generator=g) * 64).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
    vc = (torch.randn(1, 1, T, D, generator=g) * 64).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
    ks = torch.exp2(torch.rand(1, 1, T, generator=g) * 3 - 8)
    vs = torch.exp2(torch.rand(1, 1, T, generator=g) * 3 - 8)
    lens = torch.tensor([T - 77], dtype=torch.int32)
    out = gqa.decode_fp8(q.cuda(), kc.cuda(), vc.cuda(), ks.cuda(), vs.cuda(), lens.cuda())
    ref = O.attention_e4m3kv(q, kc, ks, vc, vs, 1.0 / np.sqrt(D), True, kv_lens=[T - 77])
    _check(out, ref, "fp8 decode 2^20 keys")


def test_prefill_64k_tokens_sampled():
    """B1, 4 query heads on one KV head, 65536 causal positions; rows at the
    start, around tile edges and at the end of the sequence."""
    T, D = 1 << 16, 128
    q = _rand((1, 4, T, D), 420)
    k = _rand((1, 1, T, D), 421)
    v = _rand((1, 1, T, D), 422)
    out = gqa.attention(q.cuda(), k.cuda(), v.cuda(), causal=True)
    pos = [0, 1, 31, 32, 255, 256, 4095, 4096, 40000, T - 257, T - 256, T - 2, T - 1]
    rows = [a * T + p for a in range(4) for p in pos]
    ref = O.attention(q, k, v, 1.0 / np.sqrt(D), True, rows=rows)
    got = out.reshape(4 * T, D)[rows]
    _check(got, ref, "prefill 64k")


def test_mla_decode_128k_keys():
    T = 1 << 17
    q = _rand((2, 128, 1, 576), 430)
    kv = _rand((2, 1, T, 576), 431)
    lens = torch.tensor([T, T - 1000], dtype=torch.int32)
    kvd = kv.cuda()
    out = gqa.decode(q.cuda(), kvd, kvd[..., :512], lens.cuda(), scale=1.0 / np.sqrt(192.0))
    ref = O.attention(q, kv, kv[..., :512], 1.0 / np.sqrt(192.0), True, kv_lens=[T, T - 1000])
    _check(out, ref, "MLA decode 128k")


def test_varlen_two_thousand_sequences():
    """2000 packed sequences of 1..96 tokens with a window of 40: the device
    search over cu_seqlens walks 32 chunks of 64 sequences."""
    rng = np.random.default_rng(440)
    lens = rng.integers(1, 97, 2000).tolist()
    cu = [0] + np.cumsum(lens).tolist()
    q = _rand((cu[-1], 8, 64), 441)
    k = _rand((cu[-1], 2, 64), 442)
    v = _rand((cu[-1], 2, 64), 443)
    cud = torch.tensor(cu, dtype=torch.int32, device="cuda")
    out = gqa.attention_varlen(q.cuda(), k.cuda(), v.cuda(), cud, cud, causal=True, window=40)
    ref = O.attention_varlen(q, k, v, cu, cu, 1.0 / 8.0, True, window=40)
    _check(out, ref, "varlen 2000 sequences")


@pytest.mark.parametrize("topk,splits", [(16384, 4), (16384, 0), (20000, 5)])
def test_topk_long_selection(topk, splits):
    """Selections of 16k / 20k positions of a 65536-key cache: four or five
    slices of up to 4096 entries, and the library's choice."""
    T = 1 << 16
    q = _rand((2, 128, 1, 576), 450)
    kv = _rand((2, 1, T, 576), 451)
    lens = torch.tensor([T, 30000], dtype=torch.int32)
    rng = np.random.default_rng(452)
    idx = np.full((2, topk), -1, dtype=np.int32)
    for b, n in enumerate(lens.tolist()):
        sel = rng.permutation(n)[:topk]
        idx[b, :sel.size] = sel
    out = gqa.decode_topk(q.cuda(), kv.cuda(), lens.cuda(), torch.from_numpy(idx).cuda(),
                          scale=1.0 / np.sqrt(192.0), num_splits=splits)
    ref = O.decode_topk(q, kv, lens, idx, 1.0 / np.sqrt(192.0), 512)
    _check(out, ref, f"top-{topk} S={splits}")


def test_topk_cache_past_4gib():
    """Top-k decode on a 3.8M-row latent cache (4.4 GB): selected rows past
    2^32 bytes from the cache start take the 64-bit per-lane copy path.  Only
    the rows the kernel can read are written (the selected ones, the first
    and the last); the reference runs on those rows alone."""
    T, topk = 3_800_000, 256
    q = _rand((1, 128, 1, 576), 470)
    rng = np.random.default_rng(471)
    far = rng.choice(np.arange(3_730_000, T - 1), 160, replace=False)
    near = rng.choice(np.arange(1, 100_000), 80, replace=False)
    sel = np.concatenate([far, near, [0, T - 1]]).astype(np.int32)
    idx = np.concatenate([rng.permutation(sel), np.full(topk - sel.size, -1, np.int32)]).astype(np.int32)
    rows = _rand((sel.size, 576), 472)
    kvd = torch.empty((1, 1, T, 576), dtype=torch.bfloat16, device="cuda")
    kvd[0, 0, torch.from_numpy(sel).long().cuda()] = rows.cuda()
    out = gqa.decode_topk(q.cuda(), kvd, torch.tensor([T], dtype=torch.int32).cuda(),
                          torch.from_numpy(idx[None]).cuda(), scale=1.0 / np.sqrt(192.0), num_splits=2)
    compact = rows.reshape(1, 1, sel.size, 576)
    pos_of = {int(p): i for i, p in enumerate(sel)}
    cidx = np.array([[pos_of.get(int(p), -1) for p in idx]], dtype=np.int32)
    ref = O.decode_topk(q, compact, np.array([sel.size], dtype=np.int32), cidx, 1.0 / np.sqrt(192.0), 512)
    _check(out, ref, "top-k over a 4.4 GB cache")
    del kvd
