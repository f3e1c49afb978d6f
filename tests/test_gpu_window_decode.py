"""GPU parity of the sliding-window decode (gqa_attn_decode_window, and the
window of gqa_attn_decode_fp8) against the fp64 oracle: the query of
sequence b (position len_b - 1) sees only the last min(len_b, w) keys.

Rows before the window and past the length hold NaN, so a kernel that read
any of them would fail.  Tolerances as for the decode paths: bf16 max
<= 2e-2, mean <= 2e-3; fp32 max <= 1e-5.
"""
import numpy as np
import pytest
import torch

import causal_grouped_query_amd as gqa
import workloads as W
from oracle import oracle as O

pytestmark = pytest.mark.gpu

LENS = [700, 37, 0, 1, 300, 64, 65]


def _rand(shape, seed, dtype):
    g = torch.Generator("cpu").manual_seed(seed)
    return torch.randn(*shape, generator=g, dtype=torch.float32).to(dtype)


def _check(gpu, ref, what, tmax, tmean):
    g = gpu.detach().double().cpu().numpy().reshape(ref.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    d = np.abs(g - ref)
    print(f"{what} max_abs={d.max():.3e} mean_abs={d.mean():.3e}", flush=True)
    assert d.max() <= tmax and d.mean() <= tmean, f"{what}: max {d.max():.3e} mean {d.mean():.3e}"


def _nan_outside_window(x, lens, w):
    for b, n in enumerate(lens):
        x[b, :, n:] = float("nan")
        if w:
            x[b, :, :max(0, n - w)] = float("nan")


@pytest.mark.parametrize("window", [1, 7, 64, 100, 5000])
@pytest.mark.parametrize("splits", [1, 2, 3, 0])
def test_window_decode_bf16(window, splits):
    B, Hq, Hkv, T, D = len(LENS), 32, 8, 700, 128
    q = _rand((B, Hq, 1, D), 600, torch.bfloat16)
    k = _rand((B, Hkv, T, D), 601, torch.bfloat16)
    v = _rand((B, Hkv, T, D), 602, torch.bfloat16)
    ref = O.attention(q, k, v, 1.0 / np.sqrt(D), True, kv_lens=LENS, window=window)
    _nan_outside_window(k, LENS, window)
    _nan_outside_window(v, LENS, window)
    lens = torch.tensor(LENS, dtype=torch.int32).cuda()
    out = gqa.decode(q.cuda(), k.cuda(), v.cuda(), lens, num_splits=splits, window=window)
    _check(out, ref, f"window decode bf16 w={window} S={splits}", 2e-2, 2e-3)


@pytest.mark.parametrize("window,D", [(3, 64), (50, 64), (1000, 64), (40, 128)])
def test_window_decode_f32(window, D):
    B, Hq, Hkv, T = len(LENS), 8, 2, 700
    q = _rand((B, Hq, 1, D), 610, torch.float32)
    k = _rand((B, Hkv, T, D), 611, torch.float32)
    v = _rand((B, Hkv, T, D), 612, torch.float32)
    ref = O.attention(q, k, v, 1.0 / np.sqrt(D), True, kv_lens=LENS, window=window)
    _nan_outside_window(k, LENS, window)
    _nan_outside_window(v, LENS, window)
    out = gqa.decode(q.cuda(), k.cuda(), v.cuda(), torch.tensor(LENS, dtype=torch.int32).cuda(),
                     scale=1.0 / np.sqrt(D), window=window)
    _check(out, ref, f"window decode fp32 w={window}", 1e-5, 1e-5)


@pytest.mark.parametrize("window", [33, 256])
def test_window_decode_mla(window):
    lens = [700, 37, 0, 300]
    q = _rand((4, 128, 1, 576), 620, torch.bfloat16)
    kv = _rand((4, 1, 700, 576), 621, torch.bfloat16)
    scale = 1.0 / np.sqrt(192.0)
    ref = O.attention(q, kv, kv[..., :512], scale, True, kv_lens=lens, window=window)
    _nan_outside_window(kv, lens, window)
    kvd = kv.cuda()
    out = gqa.decode(q.cuda(), kvd, kvd[..., :512], torch.tensor(lens, dtype=torch.int32).cuda(), scale=scale,
                     window=window)
    _check(out, ref, f"window decode MLA w={window}", 2e-2, 2e-3)


@pytest.mark.parametrize("window", [1, 100, 5000])
def test_window_decode_fp8(window):
    w = W.GQA_DECODE_FP8.scaled(B=len(LENS), Tk=700, seed=630, len_lo=0, len_hi=0)
    q, kc, vc, ks, vs, _ = W.fp8_decode_inputs(w, nan_tail=False)
    # row scales 2^-6 / 2^-5: dequantised values about N(0, 1), and exact in
    # the bf16 weight the value scale rides on.  (With window 1 the output
    # is one dequantised row, no average: the absolute bar assumes values of
    # unit size; the generator's random scales are covered where outputs
    # are averages.)
    ks.fill_(2.0 ** -6)
    vs.fill_(2.0 ** -6)
    vs[:, :, 1::2] = 2.0 ** -5
    # reference: each sequence's query over its visible rows only (the last
    # min(len, window) keys, all visible), a zero row for an empty sequence
    ref = np.zeros((w.B, w.Hq, 1, w.Dv))
    for b, n in enumerate(LENS):
        lo = max(0, n - window)
        if n > lo:
            ref[b:b + 1] = O.attention_e4m3kv(q[b:b + 1], kc[b:b + 1, :, lo:n].contiguous(), ks[b:b + 1, :, lo:n].contiguous(),
                                              vc[b:b + 1, :, lo:n].contiguous(), vs[b:b + 1, :, lo:n].contiguous(),
                                              w.scale, False)
    for b, n in enumerate(LENS):
        lo = max(0, n - window)
        kc[b, :, n:] = 0x7F
        vc[b, :, n:] = 0x7F
        kc[b, :, :lo] = 0x7F
        vc[b, :, :lo] = 0x7F
        ks[b, :, n:] = float("nan")
        ks[b, :, :lo] = float("nan")
    out = gqa.decode_fp8(q.cuda(), kc.cuda(), vc.cuda(), ks.cuda(), vs.cuda(),
                         torch.tensor(LENS, dtype=torch.int32).cuda(), scale=w.scale, window=window)
    _check(out, ref, f"window decode fp8 w={window}", 2e-2, 2e-3)
