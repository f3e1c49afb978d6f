"""GPU parity of the FP8-cache decode (gqa_attn_decode_fp8) against the fp64
oracle, which dequantises every E4M3 code exactly (code value x row scale).

Tolerance as for every bf16 path: max |err| <= 2e-2, mean |err| <= 2e-3.
Cases: GQA / MHA / MQA groups, D = 64 and 128, lengths of 0, 1, a partial
tile and the full cache, NaN codes and NaN scales in every row past the
length, several split bounds, cache and scale tensors stored [B, T, H, D]
(strided views), and the full-size workload on sampled rows.
"""
import numpy as np
import pytest
import torch

import causal_grouped_query_amd as gqa
import workloads as W
from oracle import oracle as O

pytestmark = pytest.mark.gpu

TMAX, TMEAN = 2e-2, 2e-3


def _check(gpu, ref, what):
    g = gpu.detach().double().cpu().numpy().reshape(ref.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    d = np.abs(g - ref)
    print(f"{what} max_abs={d.max():.3e} mean_abs={d.mean():.3e}", flush=True)
    assert d.max() <= TMAX and d.mean() <= TMEAN, f"{what}: max {d.max():.3e} mean {d.mean():.3e}"


def _inputs(B, Hq, Hkv, T, D, lens, seed):
    w = W.GQA_DECODE_FP8.scaled(B=B, Hq=Hq, Hkv=Hkv, Tk=T, Dk=D, Dv=D, seed=seed, len_lo=0, len_hi=0)
    q, kc, vc, ks, vs, _ = W.fp8_decode_inputs(w, nan_tail=False)
    lens_t = torch.tensor(lens, dtype=torch.int32)
    for b, n in enumerate(lens):
        kc[b, :, n:] = 0x7F
        vc[b, :, n:] = 0x7F
        ks[b, :, n:] = float("nan")
        vs[b, :, n:] = float("nan")
    return q, kc, vc, ks, vs, lens_t


def _gpu(q, kc, vc, ks, vs, lens, scale, splits=0):
    return gqa.decode_fp8(q.cuda(), kc.cuda(), vc.cuda(), ks.cuda(), vs.cuda(), lens.cuda(), scale=scale,
                          num_splits=splits)


@pytest.mark.parametrize("splits", [3, 5, 0])
@pytest.mark.parametrize("Hq,Hkv,D", [(32, 8, 128), (8, 8, 128), (16, 1, 128), (8, 2, 64)])
def test_fp8_decode_matches_oracle(Hq, Hkv, D, splits):
    lens = [700, 37, 0, 1, 64]
    q, kc, vc, ks, vs, lens_t = _inputs(len(lens), Hq, Hkv, 700, D, lens, 300 + Hq + D)
    scale = 1.0 / np.sqrt(D)
    out = _gpu(q, kc, vc, ks, vs, lens_t, scale, splits)
    ref = O.attention_e4m3kv(q, kc, ks, vc, vs, scale, True, kv_lens=lens)
    assert torch.all(out[2] == 0), "a sequence of length 0 gives a zero row"
    _check(out, ref, f"fp8 decode Hq={Hq} Hkv={Hkv} D={D} S={splits}")


def test_fp8_decode_strided_bthd_storage():
    """Codes stored [B, T, H, D] and scales [B, T, H], passed as strided
    [B, H, T, D] / [B, H, T] views."""
    B, Hq, Hkv, T, D = 3, 16, 4, 300, 128
    lens = [300, 129, 31]
    q, kc, vc, ks, vs, lens_t = _inputs(B, Hq, Hkv, T, D, lens, 310)
    to_bthd = lambda x: x.transpose(1, 2).contiguous().cuda().transpose(1, 2)
    out = gqa.decode_fp8(q.cuda(), to_bthd(kc), to_bthd(vc), to_bthd(ks), to_bthd(vs), lens_t.cuda(),
                         scale=0.09)
    ref = O.attention_e4m3kv(q, kc, ks, vc, vs, 0.09, True, kv_lens=lens)
    _check(out, ref, "fp8 decode strided")


def test_fp8_decode_workload_full_size_sampled():
    """The benchmarked FP8 workload at full size (B64, 32 / 8 heads, caches
    of up to 8192 rows with NaN tails), 4 heads of every sequence."""
    w = W.GQA_DECODE_FP8
    q, kc, vc, ks, vs, lens = W.fp8_decode_inputs(w)
    out = _gpu(q, kc, vc, ks, vs, lens, w.scale)
    rng = np.random.default_rng(11)
    rows = [b * w.Hq + int(a) for b in range(w.B) for a in rng.choice(w.Hq, 4, replace=False)]
    ref = O.attention_e4m3kv(q, kc, ks, vc, vs, w.scale, True, kv_lens=lens.tolist(), rows=rows)
    got = out.reshape(w.B * w.Hq, w.Dv)[rows]
    _check(got, ref, "fp8 workload")
