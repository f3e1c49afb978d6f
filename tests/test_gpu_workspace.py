"""The decode combine reads every split slot of a row (empty ones too, with
weight 0) and must select empty slots away whatever they hold.  Each decode
entry point runs with a workspace pre-filled with 0xFF bytes (NaN in fp32 and
in bf16) against the fp64 oracle; ragged lengths leave many slots empty.
Split counts above 64 take the combine's second pass over slots (one lane
per slot, 64 at a time).  Tolerance as for every bf16 path: max |err| <=
2e-2, mean |err| <= 2e-3; fp32: max |err| <= 1e-5.
"""
import numpy as np
import pytest
import torch

import causal_grouped_query_amd as gqa
import workloads as W
from oracle import oracle as O

pytestmark = pytest.mark.gpu

LENS = [700, 37, 0, 1, 300, 64, 65, 2]


def _rand(shape, seed):
    g = torch.Generator("cpu").manual_seed(seed)
    return torch.randn(*shape, generator=g, dtype=torch.float32).to(torch.bfloat16)


def _check(gpu, ref, what):
    g = gpu.detach().double().cpu().numpy().reshape(ref.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    d = np.abs(g - ref)
    print(f"{what} max_abs={d.max():.3e} mean_abs={d.mean():.3e}", flush=True)
    assert d.max() <= 2e-2 and d.mean() <= 2e-3, f"{what}: max {d.max():.3e} mean {d.mean():.3e}"


def _nan_ws(nbytes):
    return torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("splits", [0, 2, 9, 40, 100, 300, 1024])
def test_gqa_decode_nan_workspace(splits):
    B, Hq, Hkv, T, D = len(LENS), 32, 8, 700, 128
    q, k, v = _rand((B, Hq, 1, D), 800), _rand((B, Hkv, T, D), 801), _rand((B, Hkv, T, D), 802)
    S = splits or gqa.decode_splits(B, Hq, Hkv, T, D, D, gqa.GQA_BF16)
    ws = _nan_ws(gqa.decode_workspace_size(B, Hq, D, S))
    out = gqa.decode(q.cuda(), k.cuda(), v.cuda(), torch.tensor(LENS, dtype=torch.int32).cuda(), num_splits=S,
                     workspace=ws)
    ref = O.attention(q, k, v, 1.0 / np.sqrt(D), True, kv_lens=LENS)
    _check(out, ref, f"gqa decode, NaN workspace, S={S}")


def test_mla_and_topk_decode_nan_workspace():
    lens = [700, 37, 0, 300]
    q, kv = _rand((4, 128, 1, 576), 810), _rand((4, 1, 700, 576), 811)
    lens_d = torch.tensor(lens, dtype=torch.int32).cuda()
    kvd = kv.cuda()
    scale = 1.0 / np.sqrt(192.0)
    S = 6
    out = gqa.decode(q.cuda(), kvd, kvd[..., :512], lens_d, scale=scale, num_splits=S,
                     workspace=_nan_ws(gqa.decode_workspace_size(4, 128, 512, S)))
    _check(out, O.attention(q, kv, kv[..., :512], scale, True, kv_lens=lens), "mla decode, NaN workspace")
    rng = np.random.default_rng(812)
    idx = np.full((4, 300), -1, dtype=np.int32)
    for b, n in enumerate(lens):
        sel = rng.permutation(n)[:rng.integers(0, 301)]
        idx[b, :sel.size] = sel
    St = 5
    out = gqa.decode_topk(q.cuda(), kvd, lens_d, torch.from_numpy(idx).cuda(), scale=scale, num_splits=St,
                          workspace=_nan_ws(gqa.decode_workspace_size(4, 128, 512, St)))
    _check(out, O.decode_topk(q, kv, torch.tensor(lens), idx, scale, 512), "top-k decode, NaN workspace")


def test_fp8_decode_nan_workspace():
    w = W.GQA_DECODE_FP8.scaled(B=len(LENS), Tk=700, seed=820, len_lo=0, len_hi=0)
    q, kc, vc, ks, vs, _ = W.fp8_decode_inputs(w, nan_tail=False)
    # power-of-two row scales: the rows of length 1 and 2 are (averages of)
    # single dequantised values of size up to ~10, where a random scale's
    # bf16 rounding in the weight alone uses most of the absolute bar (that
    # case has its own tests); this test is about the workspace
    ks.fill_(2.0 ** -6)
    vs.fill_(2.0 ** -6)
    vs[:, :, 1::2] = 2.0 ** -5
    S = 12
    out = gqa.decode_fp8(q.cuda(), kc.cuda(), vc.cuda(), ks.cuda(), vs.cuda(), torch.tensor(LENS, dtype=torch.int32).cuda(),
                         scale=w.scale, num_splits=S, workspace=_nan_ws(gqa.decode_workspace_size(w.B, w.Hq, w.Dv, S)))
    ref = O.attention_e4m3kv(q, kc, ks, vc, vs, w.scale, True, kv_lens=LENS)
    _check(out, ref, "fp8 decode, NaN workspace")


@pytest.mark.parametrize("splits", [3, 130])
def test_f32_decode_nan_workspace(splits):
    B, Hq, Hkv, T, D = len(LENS), 8, 2, 700, 64
    g = torch.Generator("cpu").manual_seed(830)
    q = torch.randn(B, Hq, 1, D, generator=g)
    k = torch.randn(B, Hkv, T, D, generator=g)
    v = torch.randn(B, Hkv, T, D, generator=g)
    out = gqa.decode(q.cuda(), k.cuda(), v.cuda(), torch.tensor(LENS, dtype=torch.int32).cuda(), scale=0.125,
                     num_splits=splits, workspace=_nan_ws(gqa.decode_workspace_size(B, Hq, D, splits)))
    ref = O.attention(q, k, v, 0.125, True, kv_lens=LENS)
    d = np.abs(out.double().cpu().numpy() - ref)
    print(f"fp32 decode, NaN workspace, S={splits} max_abs={d.max():.3e}", flush=True)
    assert np.isfinite(out.cpu().numpy()).all() and d.max() <= 1e-5
