"""GPU: the allocation-free decode (gqa_attn_decode_noalloc) against the
workspace decode (gqa_attn_decode) on the same inputs, through the C ABI.

Both run the same kernels with the same split count, so the outputs must
agree bit for bit; each is also held to the bf16 / fp32 tolerances against
the fp64 oracle.  Two calls in a row on one device, the second smaller than
the first, check that the scratch array's stale contents from the first
call never reach the second.  Cache slots past each length hold NaN.
"""
import math

import numpy as np
import pytest
import torch

import causal_grouped_query_amd as gqa
from oracle import oracle as O

pytestmark = pytest.mark.gpu

TOL = {torch.bfloat16: (2e-2, 2e-3), torch.float32: (1e-5, 1e-5)}


def _inputs(B, Hq, Hkv, Tmax, D, Dv, dtype, seed, mla=False):
    g = torch.Generator("cpu").manual_seed(seed)
    q = torch.randn(B, Hq, 1, D, generator=g).to(dtype)
    k = torch.randn(B, Hkv, Tmax, D, generator=g).to(dtype)
    v = k[..., :Dv] if mla else torch.randn(B, Hkv, Tmax, Dv, generator=g).to(dtype)
    lens = torch.randint(1, Tmax + 1, (B,), generator=g, dtype=torch.int32)
    for b in range(B):  # slots past the length are not input: NaN
        k[b, :, lens[b]:] = float("nan")
        if not mla:
            v[b, :, lens[b]:] = float("nan")
    return q, k, v, lens


def _run_pair(q, k, v, lens, S, mla=False):
    dev = torch.device("cuda:0")
    qd, kd, ld = q.to(dev), k.to(dev), lens.to(dev)
    vd = kd[..., : v.shape[-1]] if mla else v.to(dev)
    B, Hq, _, D = q.shape
    Dv = v.shape[-1]
    scale = 1.0 / math.sqrt(192 if mla else D)
    out_ref = torch.empty((B, Hq, 1, Dv), dtype=q.dtype, device=dev)
    gqa.decode(qd, kd, vd, ld, scale=scale, num_splits=S, out=out_ref)
    out = torch.full((B, Hq, 1, Dv), float("nan"), dtype=q.dtype, device=dev)
    gqa.decode_noalloc(qd, kd, vd, ld, out, scale=scale, num_splits=S)
    torch.cuda.synchronize()
    return out.cpu(), out_ref.cpu(), scale


def _check(q, k, v, lens, S, mla=False):
    out, out_ref, scale = _run_pair(q, k, v, lens, S, mla)
    bits = torch.int16 if out.dtype == torch.bfloat16 else torch.int32
    assert torch.equal(out.view(bits), out_ref.view(bits)), "noalloc differs from the workspace decode"
    ref = O.attention(q, k, v, scale, True, kv_lens=lens.tolist())
    err = np.abs(out.double().numpy() - ref)
    tmax, tmean = TOL[q.dtype]
    assert np.isfinite(out.double().numpy()).all()
    assert err.max() <= tmax and err.mean() <= tmean, (err.max(), err.mean())


@pytest.mark.parametrize("S", [0, 2, 9])
def test_noalloc_matches_decode_twice_shrinking_bf16(S):
    # first call: 64 sequences of up to 4096 keys; second: 3 sequences of up to 300
    _check(*_inputs(64, 32, 8, 4096, 128, 128, torch.bfloat16, 1), S)
    _check(*_inputs(3, 8, 2, 300, 128, 128, torch.bfloat16, 2), S)


def test_noalloc_matches_decode_twice_shrinking_f32():
    _check(*_inputs(8, 16, 4, 1000, 64, 64, torch.float32, 3), 0)
    _check(*_inputs(2, 4, 2, 130, 64, 64, torch.float32, 4), 0)


def test_noalloc_absorbed_mla_then_gqa():
    # the absorbed-MLA shape (V = latent prefix of K), then a small GQA decode
    _check(*_inputs(4, 128, 1, 2048, 576, 512, torch.bfloat16, 5, mla=True), 0, mla=True)
    _check(*_inputs(2, 8, 2, 100, 128, 128, torch.bfloat16, 6), 0)


def test_noalloc_rejects_shapes_beyond_the_scratch():
    dev = torch.device("cuda:0")
    q = torch.zeros(1024, 128, 1, 576, dtype=torch.bfloat16, device=dev)
    kv = torch.zeros(1024, 1, 8, 576, dtype=torch.bfloat16, device=dev)
    lens = torch.ones(1024, dtype=torch.int32, device=dev)
    out = torch.empty(1024, 128, 1, 512, dtype=torch.bfloat16, device=dev)
    need = gqa.decode_noalloc_scratch_bytes(1024, 128, 512, 16, gqa.GQA_BF16)
    assert need > (64 << 20)
    with pytest.raises(gqa.GQAError) as e:
        gqa.decode_noalloc(q, kv, kv[..., :512], lens, out, scale=0.07, num_splits=16)
    assert e.value.code == gqa.GQA_ERR_WORKSPACE
