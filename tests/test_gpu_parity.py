"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Tolerances (written here, applied element by element to GPU output widened
to fp64 minus the oracle's fp64 output):
  bf16 storage, fp32 accumulation: max |err| <= 2e-2 and mean |err| <= 2e-3
  fp32 throughout:                 max |err| <= 1e-5
Small and mid-size cases compare every element and span several tiles with
ragged tails; the five headline workloads are run at full size with the
launch configuration the benchmark times and checked on sampled rows.
"""
import math
import zlib

import numpy as np
import pytest
import torch

import causal_grouped_query_amd as gqa
import workloads as W
from oracle import oracle as O

pytestmark = pytest.mark.gpu

TOL = {"bf16": (2e-2, 2e-3), "f32": (1e-5, 1e-5)}
DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def _err(gpu, ref):
    g = gpu.detach().double().cpu().numpy().reshape(ref.shape)
    d = np.abs(g - ref)
    assert np.isfinite(g).all(), "non-finite output"
    return float(d.max()), float(d.mean())


def _check(gpu, ref, dtype, what=""):
    mx, mean = _err(gpu, ref)
    tmax, tmean = TOL[dtype]
    print(f"{what} max_abs={mx:.3e} mean_abs={mean:.3e}", flush=True)
    assert mx <= tmax and mean <= tmean, f"{what}: max {mx:.3e} mean {mean:.3e}"


def _rand(shape, seed, dtype):
    g = torch.Generator("cpu").manual_seed(seed)
    return torch.randn(*shape, generator=g, dtype=torch.float32).to(DT[dtype])


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    gqa.lib()
    yield
    torch.cuda.synchronize()


# ------------------------------------------------------------------ worked example

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
def test_head_mapping_example_fwd_and_decode(dtype, D):
    """q = k = 0 and v = 1 / 7 for the two KV heads give [1, 1, 7, 7] exactly
    (the worked example of the Attention variants page, widened to D dims)."""
    q = torch.zeros(1, 4, 1, D, dtype=DT[dtype], device="cuda")
    k = torch.zeros(1, 2, 1, D, dtype=DT[dtype], device="cuda")
    v = torch.tensor([1.0, 7.0]).view(1, 2, 1, 1).expand(1, 2, 1, D).contiguous().to(DT[dtype]).cuda()
    out = gqa.attention(q, k, v)
    assert out[0, :, 0, :].float().cpu().tolist() == [[1.0] * D, [1.0] * D, [7.0] * D, [7.0] * D]
    lens = torch.ones(1, dtype=torch.int32, device="cuda")
    dec = gqa.decode(q, k, v, lens)
    assert dec[0, :, 0, :].float().cpu().tolist() == [[1.0] * D, [1.0] * D, [7.0] * D, [7.0] * D]


# ------------------------------------------------------------------ forward, full compare

FWD_CASES = [
    # B, Hq, Hkv, Tq, Tk, D, causal
    (2, 8, 2, 300, 300, 128, True),    # GQA G=4, several tiles, ragged tail
    (1, 4, 4, 257, 257, 128, True),    # MHA
    (2, 8, 1, 130, 130, 64, True),     # MQA, D=64
    (1, 6, 2, 200, 200, 128, True),    # G=3 (odd group)
    (2, 16, 2, 77, 333, 128, True),    # suffix queries, G=8 (two head blocks)
    (1, 8, 2, 1, 500, 128, True),      # one decode step through the forward entry
    (1, 4, 2, 100, 40, 128, False),    # cross attention, Tq > Tk
    (1, 4, 2, 64, 64, 64, True),       # exact tile multiples
    (2, 64, 1, 33, 1100, 128, True),   # MQA suffix, G=64
    (1, 2, 1, 5, 7, 64, True),         # smaller than one tile
    (1, 40, 1, 50, 70, 64, True),      # G=40: a full and a ragged block of query heads
]


@pytest.mark.parametrize("case", FWD_CASES, ids=lambda c: "B{}_Hq{}_Hkv{}_Tq{}_Tk{}_D{}_{}".format(
    *c[:6], "causal" if c[6] else "full"))
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fwd_matches_oracle(case, dtype):
    B, Hq, Hkv, Tq, Tk, D, causal = case
    seed = zlib.crc32(repr(case).encode()) % 10000
    q, k, v = (_rand((B, Hq, Tq, D), seed, dtype), _rand((B, Hkv, Tk, D), seed + 1, dtype),
               _rand((B, Hkv, Tk, D), seed + 2, dtype))
    scale = 1.0 / math.sqrt(D)
    out = gqa.attention(q.cuda(), k.cuda(), v.cuda(), scale=scale, causal=causal)
    torch.cuda.synchronize()
    ref = O.attention(q, k, v, scale, causal)
    _check(out, ref, dtype, f"fwd {case} {dtype}")


def test_fwd_scale_variants():
    B, Hq, Hkv, T, D = 1, 4, 2, 150, 128
    q, k, v = _rand((B, Hq, T, D), 5, "bf16"), _rand((B, Hkv, T, D), 6, "bf16"), _rand((B, Hkv, T, D), 7, "bf16")
    for scale in [0.0, 0.02, 0.3]:
        out = gqa.attention(q.cuda(), k.cuda(), v.cuda(), scale=scale, causal=True)
        _check(out, O.attention(q, k, v, scale, True), "bf16", f"scale {scale}")


@pytest.mark.parametrize("slope", [60.0, -60.0, 200.0])
def test_fwd_growing_and_falling_logits(slope):
    """Scores that rise (or fall) along the key axis by tens to hundreds of
    log2 units: a rising row makes the kernel move its reference max many
    times mid-row (each move rescales O), a falling row never moves it after
    the first tile.  Both must still match the oracle."""
    B, Hq, Hkv, T, D = 1, 4, 1, 700, 128
    g = torch.Generator("cpu").manual_seed(17)
    q = (torch.ones(B, Hq, T, D) + 0.1 * torch.randn(B, Hq, T, D, generator=g)).to(torch.bfloat16)
    ramp = torch.linspace(0.0, 1.0, T).view(1, 1, T, 1)
    # q.k_j * scale * log2(e) grows by about `slope` over the row
    k = (ramp * slope / (D * 0.0884 * 1.4427) + 0.05 * torch.randn(B, Hkv, T, D, generator=g)).to(torch.bfloat16)
    v = torch.randn(B, Hkv, T, D, generator=g).to(torch.bfloat16)
    scale = 1.0 / math.sqrt(D)
    out = gqa.attention(q.cuda(), k.cuda(), v.cuda(), scale=scale, causal=True)
    _check(out, O.attention(q, k, v, scale, True), "bf16", f"logit slope {slope}")


# ------------------------------------------------------------------ stated invariants on the GPU

def test_future_perturbation_is_bit_identical():
    """Rows at positions <= P must not change, bit for bit, when every key and
    value after P is replaced (future keys get exactly zero weight)."""
    B, Hq, Hkv, T, D = 2, 8, 2, 320, 128
    q, k, v = _rand((B, Hq, T, D), 11, "bf16"), _rand((B, Hkv, T, D), 12, "bf16"), _rand((B, Hkv, T, D), 13, "bf16")
    base = gqa.attention(q.cuda(), k.cuda(), v.cuda())
    for P in [0, 63, 64, 200]:
        k2, v2 = k.clone(), v.clone()
        k2[:, :, P + 1:] = _rand(k2[:, :, P + 1:].shape, 20 + P, "bf16") * 30
        v2[:, :, P + 1:] = _rand(v2[:, :, P + 1:].shape, 40 + P, "bf16") * 30
        out = gqa.attention(q.cuda(), k2.cuda(), v2.cuda())
        assert torch.equal(out[:, :, : P + 1], base[:, :, : P + 1])


def test_decode_equals_last_row_of_prefill():
    B, Hq, Hkv, T, D = 2, 8, 2, 277, 128
    q, k, v = _rand((B, Hq, T, D), 14, "bf16"), _rand((B, Hkv, T, D), 15, "bf16"), _rand((B, Hkv, T, D), 16, "bf16")
    full = gqa.attention(q.cuda(), k.cuda(), v.cuda())
    step = gqa.attention(q[:, :, -1:].contiguous().cuda(), k.cuda(), v.cuda())
    lens = torch.full((B,), T, dtype=torch.int32, device="cuda")
    dec = gqa.decode(q[:, :, -1:].contiguous().cuda(), k.cuda(), v.cuda(), lens)
    assert (step.float() - full[:, :, -1:].float()).abs().max().item() <= 2e-2
    assert (dec.float() - full[:, :, -1:].float()).abs().max().item() <= 2e-2


def test_constant_values_give_constant_output():
    B, Hq, Hkv, T, D = 1, 8, 2, 333, 128
    q, k = _rand((B, Hq, T, D), 17, "bf16") * 3, _rand((B, Hkv, T, D), 18, "bf16")
    v = torch.ones((B, Hkv, T, D), dtype=torch.bfloat16)
    out = gqa.attention(q.cuda(), k.cuda(), v.cuda())
    assert torch.all(out.float() == 1.0)
    lens = torch.tensor([T], dtype=torch.int32, device="cuda")
    dec = gqa.decode(q[:, :, -1:].contiguous().cuda(), k.cuda(), v.cuda(), lens)
    assert torch.all(dec.float() == 1.0)


# ------------------------------------------------------------------ decode

DEC_CASES = [
    # B, Hq, Hkv, Tmax, D, lens
    (5, 8, 2, 700, 128, [1, 31, 32, 33, 700]),
    (3, 32, 8, 1500, 128, [1024, 1100, 1499]),
    (2, 4, 4, 300, 64, [64, 299]),
    (2, 16, 1, 260, 128, [200, 65]),
    (1, 6, 2, 100, 64, [100]),
    (2, 40, 1, 300, 64, [300, 17]),    # G=40: two head blocks
]


@pytest.mark.parametrize("case", DEC_CASES, ids=lambda c: "B{}_Hq{}_Hkv{}_Tmax{}_D{}".format(*c[:5]))
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("splits", [1, 2, 0, 9, 1024])
def test_decode_matches_oracle(case, dtype, splits):
    B, Hq, Hkv, Tmax, D, lens = case
    seed = zlib.crc32(repr(case).encode()) % 10000
    q = _rand((B, Hq, 1, D), seed, dtype)
    k = _rand((B, Hkv, Tmax, D), seed + 1, dtype)
    v = _rand((B, Hkv, Tmax, D), seed + 2, dtype)
    for b, n in enumerate(lens):  # cache slots past the length hold NaN
        k[b, :, n:] = float("nan")
        v[b, :, n:] = float("nan")
    scale = 1.0 / math.sqrt(D)
    lt = torch.tensor(lens, dtype=torch.int32)
    out = gqa.decode(q.cuda(), k.cuda(), v.cuda(), lt.cuda(), scale=scale, num_splits=splits)
    torch.cuda.synchronize()
    ref = O.attention(q, k, v, scale, True, kv_lens=lens)
    _check(out, ref, dtype, f"decode {case} {dtype} S={splits}")


# The balanced decode (bf16, splits >= 3) lays the key tiles of all sequences
# end to end and shares them out evenly: these cases cross the 64-batch
# length chunks its cursors load, mix empty and full sequences, and take
# the smallest and largest piece bounds.
FLAT_CASES = [
    # B, Hq, Hkv, Tmax, D, lens (None: seeded random in [0, Tmax], zeros included)
    (130, 8, 2, 96, 128, None),
    (70, 4, 1, 200, 64, None),
    (4, 8, 2, 2000, 128, [0, 2000, 0, 1]),
    (1, 64, 1, 1000, 128, [999]),
]


@pytest.mark.parametrize("case", FLAT_CASES, ids=lambda c: "B{}_Hq{}_Hkv{}_Tmax{}_D{}".format(*c[:5]))
@pytest.mark.parametrize("splits", [3, 0, 64, 1024])
def test_flat_decode_matches_oracle(case, splits):
    B, Hq, Hkv, Tmax, D, lens = case
    seed = zlib.crc32(repr(case).encode()) % 10000
    if lens is None:
        g = torch.Generator().manual_seed(seed)
        lens = torch.randint(0, Tmax + 1, (B,), generator=g).tolist()
        lens[::7] = [0] * len(lens[::7])
        lens[1::11] = [Tmax] * len(lens[1::11])
    q = _rand((B, Hq, 1, D), seed, "bf16")
    k = _rand((B, Hkv, Tmax, D), seed + 1, "bf16")
    v = _rand((B, Hkv, Tmax, D), seed + 2, "bf16")
    for b, n in enumerate(lens):
        k[b, :, n:] = float("nan")
        v[b, :, n:] = float("nan")
    scale = 1.0 / math.sqrt(D)
    out = gqa.decode(q.cuda(), k.cuda(), v.cuda(), torch.tensor(lens, dtype=torch.int32).cuda(), scale=scale,
                     num_splits=splits)
    torch.cuda.synchronize()
    ref = O.attention(q, k, v, scale, True, kv_lens=lens)
    empty = [b for b, n in enumerate(lens) if n == 0]
    assert torch.all(out[empty] == 0)
    keep = [b for b, n in enumerate(lens) if n > 0]
    _check(out[keep], ref[keep], "bf16", f"flat decode {case[:5]} S={splits}")


def test_decode_strided_cache_view():
    """Caches with a larger capacity are read through strides, not copies."""
    B, Hq, Hkv, Tcap, Tmax, D = 2, 8, 2, 512, 300, 128
    kfull = _rand((B, Hkv, Tcap, D), 50, "bf16")
    vfull = _rand((B, Hkv, Tcap, D), 51, "bf16")
    q = _rand((B, Hq, 1, D), 52, "bf16")
    kv, vv = kfull.cuda()[:, :, :Tmax], vfull.cuda()[:, :, :Tmax]
    lens = [300, 123]
    out = gqa.decode(q.cuda(), kv, vv, torch.tensor(lens, dtype=torch.int32).cuda())
    ref = O.attention(q, kfull[:, :, :Tmax], vfull[:, :, :Tmax], 1 / math.sqrt(D), True, kv_lens=lens)
    _check(out, ref, "bf16", "strided decode")


def test_decode_zero_length_row_is_zero():
    B, Hq, Hkv, Tmax, D = 2, 4, 2, 64, 128
    q = _rand((B, Hq, 1, D), 53, "bf16").cuda()
    k = _rand((B, Hkv, Tmax, D), 54, "bf16").cuda()
    lens = torch.tensor([0, 64], dtype=torch.int32, device="cuda")
    out = gqa.decode(q, k, k, lens)
    assert torch.all(out[0] == 0)
    assert torch.isfinite(out[1].float()).all()


@pytest.mark.parametrize("Hq", [128, 16, 160])
@pytest.mark.parametrize("splits", [1, 3, 0])
def test_mla_absorbed_decode_matches_oracle(Hq, splits):
    """Absorbed MLA: one 576-wide latent key per token, value = its first 512
    columns (a view of the same cache), scale 1/sqrt(192)."""
    B, Tmax = 2, 700
    lens = [700, 333]
    q = _rand((B, Hq, 1, 576), 60 + Hq, "bf16")
    k = _rand((B, 1, Tmax, 576), 61 + Hq, "bf16")
    for b, n in enumerate(lens):
        k[b, :, n:] = float("nan")
    kd = k.cuda()
    scale = 1.0 / math.sqrt(192)
    out = gqa.decode(q.cuda(), kd, kd[..., :512], torch.tensor(lens, dtype=torch.int32).cuda(), scale=scale,
                     num_splits=splits)
    ref = O.attention(q, k, k[..., :512], scale, True, kv_lens=lens)
    _check(out, ref, "bf16", f"mla Hq={Hq} S={splits}")


@pytest.mark.parametrize("splits", [1, 3])
@pytest.mark.parametrize("rising", [True, False])
def test_mla_decode_reference_moves(splits, rising):
    """Absorbed MLA whose scores climb (or fall) by ~60 in log2 units along
    the sequence: every key is pulled toward the query direction by a ramp,
    so a head's running reference max has to move many times mid-chunk (the
    rescale path), or never after the first tile."""
    B, Hq, Tmax = 2, 128, 900
    lens = [900, 517]
    q = _rand((B, Hq, 1, 576), 91, "bf16")
    k = _rand((B, 1, Tmax, 576), 92, "bf16").float()
    qd = q.float()[:, 0, 0, :]  # head 0's direction, shared by all heads of the draw
    qd = qd / qd.norm(dim=-1, keepdim=True)
    ramp = torch.linspace(0.0, 25.0, Tmax) if rising else torch.linspace(25.0, 0.0, Tmax)
    k = (k + ramp[None, None, :, None] * qd[:, None, None, :]).to(torch.bfloat16)
    for b, n in enumerate(lens):
        k[b, :, n:] = float("nan")
    kd = k.cuda()
    scale = 1.0 / math.sqrt(192)
    out = gqa.decode(q.cuda(), kd, kd[..., :512], torch.tensor(lens, dtype=torch.int32).cuda(), scale=scale,
                     num_splits=splits)
    ref = O.attention(q, k, k[..., :512], scale, True, kv_lens=lens)
    _check(out, ref, "bf16", f"mla ramp rising={rising} S={splits}")


def test_mla_decode_empty_and_short_sequences():
    """Absorbed MLA with an empty sequence (zero output) and sequences shorter
    than one 32-key tile, several splits (most of them empty)."""
    B, Hq, Tmax = 3, 128, 96
    lens = [0, 5, 40]
    q = _rand((B, Hq, 1, 576), 71, "bf16")
    k = _rand((B, 1, Tmax, 576), 72, "bf16")
    for b, n in enumerate(lens):
        k[b, :, n:] = float("nan")
    kd = k.cuda()
    scale = 1.0 / math.sqrt(192)
    out = gqa.decode(q.cuda(), kd, kd[..., :512], torch.tensor(lens, dtype=torch.int32).cuda(), scale=scale,
                     num_splits=3)
    assert torch.all(out[0] == 0)
    ref = O.attention(q[1:], k[1:], k[1:, ..., :512], scale, True, kv_lens=lens[1:])
    _check(out[1:], ref, "bf16", "mla short / empty")


def _forward_loops(B, Hq, Hkv, T, rows_per_wave=32, waves=8, resident=256):
    """Host replica of the launcher's rule for the looping forward (dense,
    D = 128): one resident round of workgroups walks the items when every
    XCD's share is whole units with an even number of items per workgroup."""
    G = Hq // Hkv
    gt = 1
    while gt * 2 <= waves and G % (gt * 2) == 0 and waves % (gt * 2) == 0:
        gt *= 2
    pt = rows_per_wave * (waves // gt)
    n_qt = -(-T // pt)
    items = B * Hkv * (G // gt) * n_qt
    per, nwx = items // 8, resident // 8
    return (items > resident and items % 8 == 0 and per % n_qt == 0 and n_qt % 2 == 0
            and per % nwx == 0 and (per // nwx) % 2 == 0)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("B,T", [(8, 512), (4, 1024)])
def test_forward_looping_round(B, T, causal):
    """Shapes on which one resident round of workgroups loops over two items
    each (snake order within each XCD's range), compared in full."""
    Hq, Hkv, D = 32, 8, 128
    assert _forward_loops(B, Hq, Hkv, T)
    q, k, v = _rand((B, Hq, T, D), 60 + T, "bf16"), _rand((B, Hkv, T, D), 61 + T, "bf16"), _rand((B, Hkv, T, D), 62 + T, "bf16")
    out = gqa.attention(q.cuda(), k.cuda(), v.cuda(), causal=causal)
    _check(out, O.attention(q, k, v, 1.0 / math.sqrt(D), causal), "bf16", f"looping forward B={B} T={T} causal={causal}")


# ------------------------------------------------------------------ headline workloads, full size

def _sample_rows(B, Hq, Tq, n, seed, extra_pos=()):
    rng = np.random.default_rng(seed)
    rows = set()
    for b in {0, B - 1}:
        for a in {0, Hq - 1, Hq // 2}:
            for i in {0, Tq - 1, *[p for p in extra_pos if p < Tq]}:
                rows.add((b * Hq + a) * Tq + i)
    while len(rows) < n:
        rows.add(int(rng.integers(0, B * Hq * Tq)))
    return sorted(rows)


def _check_rows(out, rows, ref, dtype, what):
    flat = out.reshape(-1, out.shape[-1])
    got = flat[torch.tensor(rows, device=out.device)]
    _check(got, ref, dtype, what)


def test_workload_tiny_fp32_fwd_and_decode():
    w = W.TINY_F32
    q, k, v = W.fwd_inputs(w)
    out = gqa.attention(q.cuda(), k.cuda(), v.cuda(), scale=w.scale)
    _check(out, O.attention(q, k, v, w.scale, True), "f32", "tiny fp32 prefill")
    ql = q[:, :, -1:].contiguous()
    step = gqa.attention(ql.cuda(), k.cuda(), v.cuda(), scale=w.scale)
    ref_step = O.attention(ql, k, v, w.scale, True)
    _check(step, ref_step, "f32", "tiny fp32 decode via forward")
    lens = torch.full((w.B,), w.Tk, dtype=torch.int32, device="cuda")
    dec = gqa.decode(ql.cuda(), k.cuda(), v.cuda(), lens, scale=w.scale)
    _check(dec, ref_step, "f32", "tiny fp32 decode via split-KV")


@pytest.mark.parametrize("w", [W.GQA_PREFILL, W.MQA_SUFFIX], ids=lambda w: w.name)
def test_workload_prefill_full_size_sampled(w):
    q, k, v = W.fwd_inputs(w)
    out = gqa.attention(q.cuda(), k.cuda(), v.cuda(), scale=w.scale)
    torch.cuda.synchronize()
    rows = _sample_rows(w.B, w.Hq, w.Tq, 96, w.seed, extra_pos=(31, 32, 63, 64, 127, 128, 2047, 2048))
    ref = O.attention(q, k, v, w.scale, True, rows=rows)
    _check_rows(out, rows, ref, w.dtype, w.name)


@pytest.mark.parametrize("w", [W.GQA_DECODE, W.MLA_DECODE], ids=lambda w: w.name)
def test_workload_decode_full_size_sampled(w):
    q, k, v, lens = W.decode_inputs(w, nan_tail=True)
    kd = k.cuda()
    vd = kd[..., : w.Dv] if w.kind == "mla_decode" else v.cuda()
    out = gqa.decode(q.cuda(), kd, vd, lens.cuda(), scale=w.scale)
    torch.cuda.synchronize()
    rows = _sample_rows(w.B, w.Hq, 1, 48 if w.kind == "mla_decode" else 128, w.seed)
    ref = O.attention(q, k, v, w.scale, True, kv_lens=lens.tolist(), rows=rows)
    _check_rows(out, rows, ref, w.dtype, w.name)


@pytest.mark.parametrize("kind", ["gqa", "mla"])
def test_decode_large_values(kind):
    """Values eight times larger than N(0,1).  Every bf16 path's rounding
    (the weights of the P V product, the output) grows with |o|, so the bar
    here is eight times the N(0,1) one; and the split decode must add no
    error of its own through its partials: on the GQA shape its error is
    held to that of the forward kernel on the same query rows (one pass, no
    partials)."""
    if kind == "gqa":
        B, Hq, Hkv, T, D, Dv = 8, 32, 8, 3000, 128, 128
        q, k = _rand((B, Hq, 1, D), 91, "bf16"), _rand((B, Hkv, T, D), 92, "bf16")
        v = (_rand((B, Hkv, T, Dv), 93, "bf16").float() * 8).to(torch.bfloat16)
        lens = [3000, 1, 17, 2048, 999, 64, 2500, 1500]
        scale = 1.0 / math.sqrt(D)
    else:
        B, Hq, T = 4, 128, 3000
        q = _rand((B, Hq, 1, 576), 94, "bf16")
        k = (_rand((B, 1, T, 576), 95, "bf16").float() * 8).to(torch.bfloat16)  # the value is K's latent prefix
        v = k[..., :512]
        lens = [3000, 2999, 100, 1]
        scale = 0.02
    kd = k.cuda()
    vd = kd[..., :512] if kind == "mla" else v.cuda()
    lt = torch.tensor(lens, dtype=torch.int32)
    out = gqa.decode(q.cuda(), kd, vd, lt.cuda(), scale=scale)
    torch.cuda.synchronize()
    ref = O.attention(q, k, v, scale, True, kv_lens=lens)
    mx, mean = _err(out, ref)
    print(f"{kind} decode, |v| x 8: max_abs={mx:.3e} mean_abs={mean:.3e}", flush=True)
    assert mx <= 8 * 2e-2 and mean <= 8 * 2e-3
    if kind == "gqa":
        fmx, fmean = 0.0, 0.0
        for b, n in enumerate(lens):  # the same rows through the forward kernel: Tq = 1 over n keys
            o1 = gqa.attention(q[b:b + 1].cuda(), k[b:b + 1, :, :n].contiguous().cuda(),
                               v[b:b + 1, :, :n].contiguous().cuda(), scale=scale)
            e1 = _err(o1, ref[b:b + 1])
            fmx, fmean = max(fmx, e1[0]), fmean + e1[1] / B
        print(f"forward on the same rows: max_abs={fmx:.3e} mean_abs={fmean:.3e}", flush=True)
        assert mx <= 1.25 * fmx + 1e-3 and mean <= 1.25 * fmean + 1e-4
