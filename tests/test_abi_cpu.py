"""Host-side checks of the C ABI (no GPU needed).

The library must load, export every entry point include/gqa_attn.h
declares, and reject bad arguments on the host with the documented codes
before anything touches the device.  Pointers here are fake but aligned
addresses: a rejected call never dereferences them, and no call below is a
valid one (a valid call would launch a kernel).
"""
import os
import re

import pytest

import causal_grouped_query_amd as gqa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gqa_attn.h")

FAKE = 0x10000  # aligned stand-in address; never dereferenced
BF16, F32 = gqa.GQA_BF16, gqa.GQA_F32
INVALID, UNSUP, WS = gqa.GQA_ERR_INVALID_ARG, gqa.GQA_ERR_UNSUPPORTED, gqa.GQA_ERR_WORKSPACE


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gqa_attn_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    import subprocess
    declared = _declared_functions()
    assert set(declared) == set(gqa.EXPORTS)
    L = gqa.lib()
    for name in declared:
        assert hasattr(L, name), name
    nm = subprocess.run(["nm", "-D", "--defined-only", gqa.LIB_PATH], capture_output=True, text=True,
                        check=True).stdout
    exported = set(re.findall(r"\bT (gqa_attn_\w+)", nm))
    assert exported == set(declared)


def test_strerror_strings():
    assert gqa.strerror(0) == "success"
    for code in (INVALID, UNSUP, WS, gqa.GQA_ERR_HIP):
        assert gqa.strerror(code) and gqa.strerror(code) != "unknown error code"
    assert gqa.strerror(-99) == "unknown error code"


def _fwd(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, B=1, Hq=4, Hkv=2, Tq=8, Tk=8, Dk=128, Dv=128, scale=0.1,
             causal=1, dtype=BF16)
    a.update(kw)
    return gqa.lib().gqa_attn_fwd(a["q"], a["k"], a["v"], a["out"], a["B"], a["Hq"], a["Hkv"], a["Tq"],
                                  a["Tk"], a["Dk"], a["Dv"], a["scale"], a["causal"], a["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), INVALID), (dict(k=0), INVALID), (dict(v=0), INVALID), (dict(out=0), INVALID),
    (dict(B=0), INVALID), (dict(Hq=0), INVALID), (dict(Hkv=-1), INVALID), (dict(Tq=0), INVALID),
    (dict(Tk=0), INVALID), (dict(Hq=6, Hkv=4), INVALID), (dict(Tq=9, Tk=8), INVALID),
    (dict(scale=float("nan")), INVALID), (dict(scale=float("inf")), INVALID), (dict(scale=-1.0), INVALID),
    (dict(causal=2), INVALID), (dict(dtype=7), INVALID), (dict(q=FAKE + 2), INVALID),
    (dict(Dk=96, Dv=96), UNSUP), (dict(Dk=128, Dv=64), UNSUP), (dict(Dk=576, Dv=512), UNSUP),
    (dict(Dk=256, Dv=256, dtype=F32), UNSUP),
])
def test_fwd_rejects_on_host(kw, code):
    assert _fwd(**kw) == code


def _fwd_varlen(**kw):
    H, D = 4, 128
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, cq=FAKE, ck=FAKE, uq=None, uk=None, n=2, Hq=H, Hkv=2, maxq=16, maxk=16,
             Dk=D, Dv=D,
             qsh=D, qst=H * D, ksh=D, kst=2 * D, vsh=D, vst=2 * D, osh=D, ost=H * D, scale=0.1, causal=1,
             window=0, dtype=BF16)
    a.update(kw)
    return gqa.lib().gqa_attn_fwd_varlen(a["q"], a["k"], a["v"], a["out"], a["cq"], a["ck"], a["uq"], a["uk"],
                                         a["n"], a["Hq"],
                                         a["Hkv"], a["maxq"], a["maxk"], a["Dk"], a["Dv"], a["qsh"], a["qst"],
                                         a["ksh"],
                                         a["kst"], a["vsh"], a["vst"], a["osh"], a["ost"], a["scale"],
                                         a["causal"], a["window"], a["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), INVALID), (dict(cq=0), INVALID), (dict(ck=0), INVALID), (dict(n=0), INVALID),
    (dict(maxq=-1), INVALID), (dict(maxk=-1), INVALID), (dict(Hq=6, Hkv=4), INVALID), (dict(causal=2), INVALID),
    (dict(window=-1), INVALID), (dict(window=4, causal=0), INVALID), (dict(qst=100), INVALID),
    (dict(kst=0), INVALID), (dict(vsh=-8), INVALID), (dict(ost=6), INVALID), (dict(k=FAKE + 8), INVALID),
    (dict(cq=FAKE + 2), INVALID), (dict(uq=FAKE + 2), INVALID), (dict(uk=FAKE + 1), INVALID),
    (dict(scale=float("nan")), INVALID),
    (dict(dtype=F32), UNSUP), (dict(Dk=96, Dv=96), UNSUP), (dict(Dk=576, Dv=512), UNSUP),
    (dict(kst=1 << 25), UNSUP), (dict(vst=1 << 25), UNSUP),
])
def test_fwd_varlen_rejects_on_host(kw, code):
    assert _fwd_varlen(**kw) == code


def _dec(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, lens=FAKE, B=2, Hq=8, Hkv=2, Tmax=64, Dk=128, Dv=128,
             ksb=2 * 64 * 128, ksh=64 * 128, kst=128, vsb=2 * 64 * 128, vsh=64 * 128, vst=128, scale=0.1,
             S=0, ws=FAKE, wsb=1 << 30, dtype=BF16)
    a.update(kw)
    return gqa.lib().gqa_attn_decode(a["q"], a["k"], a["v"], a["out"], a["lens"], a["B"], a["Hq"], a["Hkv"],
                                     a["Tmax"], a["Dk"], a["Dv"], a["ksb"], a["ksh"], a["kst"], a["vsb"],
                                     a["vsh"], a["vst"], a["scale"], a["S"], a["ws"], a["wsb"], a["dtype"],
                                     None)


@pytest.mark.parametrize("kw,code", [
    (dict(lens=0), INVALID), (dict(q=0), INVALID), (dict(Tmax=0), INVALID), (dict(Hq=6, Hkv=4), INVALID),
    (dict(kst=0), INVALID), (dict(kst=100), INVALID), (dict(vst=64), INVALID), (dict(ksh=-8), INVALID),
    (dict(S=-1), INVALID), (dict(S=1025), INVALID), (dict(scale=float("nan")), INVALID),
    (dict(k=FAKE + 8), INVALID), (dict(lens=FAKE + 2), INVALID),
    (dict(Dk=96, Dv=96), UNSUP), (dict(Dk=576, Dv=512, dtype=F32, kst=576, vst=576), UNSUP),
    # absorbed MLA: the value must be the key's latent prefix (same pointer and strides)
    (dict(Dk=576, Dv=512, kst=576, vst=576, v=FAKE + 4096), UNSUP),
    (dict(Dk=576, Dv=512, kst=576, vst=512), UNSUP),
    (dict(ws=0), WS), (dict(wsb=100), WS), (dict(ws=FAKE + 4), WS),
])
def test_decode_rejects_on_host(kw, code):
    assert _dec(**kw) == code


def test_workspace_size_and_splits():
    assert gqa.decode_workspace_size(2, 4, 128, 0) == 0
    assert gqa.decode_workspace_size(2, 4, 128, 1025) == 0
    n = gqa.decode_workspace_size(64, 32, 128, 16)
    assert n == 64 * 32 * 16 * 129 * 4 + 256  # partials, lse, the piece counter's 256 bytes
    # the split choice depends only on the shape
    s = gqa.decode_splits(64, 32, 8, 8192, 128, 128, BF16)
    assert 1 <= s <= 1024 and s == gqa.decode_splits(64, 32, 8, 8192, 128, 128, BF16)
    assert gqa.decode_splits(16, 128, 1, 32768, 576, 512, BF16) >= 1
    with pytest.raises(gqa.GQAError):
        gqa.decode_splits(16, 128, 1, 32768, 576, 512, F32)
    # every default split count fits a workspace the size function accepts
    for shape in [(1, 4, 2, 128, 64, 64, F32), (64, 32, 8, 8192, 128, 128, BF16), (16, 128, 1, 32768, 576, 512, BF16)]:
        B, Hq, Hkv, T, Dk, Dv, dt = shape
        assert gqa.decode_workspace_size(B, Hq, Dv, gqa.decode_splits(*shape)) > 0


def test_fp8_split_count():
    # one resident round, equal pieces: 2 + ceil(4096 / streams) within 8 .. 64,
    # and never above the bf16 default, so a workspace sized for that fits
    assert gqa.decode_fp8_splits(64, 32, 8, 8192, 128, 128) == 10
    for B, Hkv, T in [(1, 8, 8192), (8, 8, 8192), (16, 8, 8192), (64, 8, 8192), (128, 8, 8192), (64, 8, 100),
                      (4096, 8, 8192), (3, 1, 64)]:
        s8 = gqa.decode_fp8_splits(B, 32, Hkv, T, 128, 128)
        sb = gqa.decode_splits(B, 32, Hkv, T, 128, 128, BF16)
        assert 3 <= s8 <= 64 and s8 <= sb, (B, Hkv, T, s8, sb)
    with pytest.raises(gqa.GQAError):
        gqa.decode_fp8_splits(64, 32, 8, 8192, 576, 512)
    with pytest.raises(gqa.GQAError):
        gqa.decode_fp8_splits(64, 30, 8, 8192, 128, 128)
    with pytest.raises(gqa.GQAError):
        gqa.decode_fp8_splits(64, 32, 8, 0, 128, 128)


def test_python_binding_rejects_cpu_tensors():
    import torch
    q = torch.zeros(1, 2, 4, 64)
    with pytest.raises(ValueError):
        gqa.attention(q, q[:, :1], q[:, :1])


def _topk(**kw):
    a = dict(q=FAKE, kv=FAKE, out=FAKE, lens=FAKE, idx=FAKE, B=2, Hq=128, Tmax=4096, topk=2048, Dk=576, Dv=512,
             ksb=4096 * 576, kst=576, scale=0.07, S=0, ws=FAKE, wsb=1 << 30, dtype=BF16)
    a.update(kw)
    return gqa.lib().gqa_attn_decode_topk(a["q"], a["kv"], a["out"], a["lens"], a["idx"], a["B"], a["Hq"],
                                          a["Tmax"], a["topk"], a["Dk"], a["Dv"], a["ksb"], a["kst"], a["scale"],
                                          a["S"], a["ws"], a["wsb"], a["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), INVALID), (dict(kv=0), INVALID), (dict(idx=0), INVALID), (dict(lens=0), INVALID),
    (dict(out=0), INVALID), (dict(B=0), INVALID), (dict(topk=0), INVALID), (dict(Tmax=0), INVALID),
    (dict(kst=512), INVALID), (dict(kst=580), INVALID), (dict(ksb=0), INVALID), (dict(S=-1), INVALID),
    (dict(S=1025), INVALID), (dict(idx=FAKE + 2), INVALID), (dict(kv=FAKE + 8), INVALID),
    (dict(scale=float("inf")), INVALID),
    (dict(dtype=F32), UNSUP), (dict(Dk=128, Dv=128), UNSUP), (dict(topk=10000, S=2), UNSUP),
    (dict(ws=0), WS), (dict(wsb=1024), WS),
])
def test_decode_topk_rejects_on_host(kw, code):
    assert _topk(**kw) == code


def test_decode_topk_default_splits():
    # one 128-head workgroup per (sequence, slice): about 256 workgroups,
    # slices of >= 64 entries, never more than 4096 entries per slice
    assert gqa.decode_topk_splits(16, 128, 2048, 576, 512, BF16) == 16
    assert gqa.decode_topk_splits(1, 128, 2048, 576, 512, BF16) == 32
    assert gqa.decode_topk_splits(512, 128, 2048, 576, 512, BF16) == 1
    assert gqa.decode_topk_splits(512, 128, 100000, 576, 512, BF16) == 25
    assert gqa.lib().gqa_attn_decode_topk_splits(2, 128, 64, 128, 128, BF16) == UNSUP


def _f8(**kw):
    D, H, T = 128, 8, 64
    a = dict(q=FAKE, k=FAKE, v=FAKE, ks=FAKE, vs=FAKE, out=FAKE, lens=FAKE, B=2, Hq=32, Hkv=H, Tmax=T, Dk=D, Dv=D,
             ksb=H * T * D, ksh=T * D, kst=D, vsb=H * T * D, vsh=T * D, vst=D, ssb=H * T, ssh=T, sst=1,
             tsb=H * T, tsh=T, tst=1, scale=0.1, win=0, S=0, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return gqa.lib().gqa_attn_decode_fp8(a["q"], a["k"], a["v"], a["ks"], a["vs"], a["out"], a["lens"], a["B"],
                                         a["Hq"], a["Hkv"], a["Tmax"], a["Dk"], a["Dv"], a["ksb"], a["ksh"], a["kst"],
                                         a["vsb"], a["vsh"], a["vst"], a["ssb"], a["ssh"], a["sst"], a["tsb"],
                                         a["tsh"], a["tst"], a["scale"], a["win"], a["S"], a["ws"], a["wsb"],
                                         None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), INVALID), (dict(k=0), INVALID), (dict(ks=0), INVALID), (dict(vs=0), INVALID),
    (dict(lens=0), INVALID), (dict(Hq=30), INVALID), (dict(Tmax=0), INVALID), (dict(kst=120), INVALID),
    (dict(kst=64), INVALID), (dict(vsh=8), INVALID), (dict(sst=0), INVALID), (dict(tsh=-1), INVALID),
    (dict(S=1), INVALID), (dict(S=2), INVALID), (dict(S=1025), INVALID), (dict(ks=FAKE + 2), INVALID),
    (dict(k=FAKE + 8), INVALID), (dict(scale=float("nan")), INVALID), (dict(win=-1), INVALID),
    (dict(Dk=96, Dv=96), UNSUP), (dict(Dk=128, Dv=64), UNSUP), (dict(kst=1 << 26), UNSUP),
    (dict(ws=0), WS), (dict(wsb=4096), WS),
])
def test_decode_fp8_rejects_on_host(kw, code):
    assert _f8(**kw) == code


def _shard(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, lse=FAKE, B=1, Hq=8, Hkv=2, Tq=64, Tk=64, Dk=128, Dv=128,
             qp=100, kp=0, scale=0.1, causal=1, dtype=BF16)
    a.update(kw)
    return gqa.lib().gqa_attn_fwd_shard(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                                        a["Tq"], a["Tk"], a["Dk"], a["Dv"], a["qp"], a["kp"], a["scale"],
                                        a["causal"], a["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), INVALID), (dict(lse=0), INVALID), (dict(out=0), INVALID), (dict(Tq=0), INVALID),
    (dict(Tk=-1), INVALID), (dict(causal=3), INVALID), (dict(qp=-1), INVALID), (dict(kp=-5), INVALID),
    (dict(out=FAKE + 8), INVALID), (dict(lse=FAKE + 2), INVALID), (dict(Hq=7), INVALID),
    (dict(dtype=F32), UNSUP), (dict(Dk=96, Dv=96), UNSUP), (dict(qp=(1 << 31) + 5), UNSUP),
])
def test_fwd_shard_rejects_on_host(kw, code):
    assert _shard(**kw) == code


@pytest.mark.parametrize("args,code", [
    ((0, FAKE, FAKE, 2, 10, 128, BF16), INVALID), ((FAKE, FAKE, FAKE, 0, 10, 128, BF16), INVALID),
    ((FAKE, FAKE, FAKE, 2, 0, 128, BF16), INVALID), ((FAKE, FAKE, FAKE, 2, 10, 128, 7), INVALID),
    ((FAKE + 4, FAKE, FAKE, 2, 10, 128, BF16), INVALID), ((FAKE, FAKE, FAKE, 2, 10, 130, BF16), UNSUP),
    ((FAKE, FAKE, FAKE, 2, 10, 1024, F32), UNSUP), ((FAKE, FAKE, FAKE, 2000, 10, 128, BF16), UNSUP),
])
def test_merge_rejects_on_host(args, code):
    assert gqa.lib().gqa_attn_merge(*args, None) == code


def test_decode_window_rejects_on_host():
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, 2, 8, 2, 64, 128, 128, 2 * 64 * 128, 64 * 128, 128, 2 * 64 * 128,
            64 * 128, 128, 0.1]
    L = gqa.lib()
    assert L.gqa_attn_decode_window(*args, -1, 0, FAKE, 1 << 30, BF16, None) == INVALID
    assert L.gqa_attn_decode_window(*args, 4, 0, 0, 1 << 30, BF16, None) == WS
    assert L.gqa_attn_decode_window(*(args[:9] + [96, 96] + args[11:]), 4, 0, FAKE, 1 << 30, BF16, None) == UNSUP


def test_decode_noalloc_rejects_on_host():
    """gqa_attn_decode_noalloc checks every argument before its first HIP
    call: rejected calls here never reach the device (there is none)."""
    D, H, T, B, Hq = 128, 2, 64, 2, 8
    L = gqa.lib()

    def call(q=FAKE, Hq_=Hq, Hkv=H, Dk=D, Dv=D, S=0, dtype=BF16, B_=B, k=FAKE, v=FAKE, kst=D):
        return L.gqa_attn_decode_noalloc(q, k, v, FAKE, FAKE, B_, Hq_, Hkv, T, Dk, Dv, Hkv * T * kst, T * kst, kst,
                                         Hkv * T * kst, T * kst, kst, 0.1, S, dtype, None)
    assert call(q=0) == INVALID
    assert call(Hq_=6, Hkv=4) == INVALID
    assert call(S=-1) == INVALID
    assert call(S=1025) == INVALID
    assert call(dtype=7) == INVALID
    assert call(Dk=96, Dv=96) == UNSUP
    # absorbed-MLA shape whose partials exceed the scratch: B = 1024 sequences
    # of 128 heads, 16 splits of 512 bf16 values
    assert call(B_=1024, Hq_=128, Hkv=1, Dk=576, Dv=512, S=16, kst=576) == WS
    assert call(B_=4096, Hq_=32, Hkv=8, S=64, dtype=F32) == WS


def test_decode_noalloc_scratch_sizes():
    # fp32 partials, then the fp32 lse at the next 256-byte boundary, rounded
    # up to 256 bytes, then 256 bytes for the piece counter
    rows = 64 * 32 * 10
    assert gqa.decode_noalloc_scratch_bytes(64, 32, 128, 10, BF16) == rows * 128 * 4 + rows * 4 + 256
    rows = 16 * 128 * 16
    assert gqa.decode_noalloc_scratch_bytes(16, 128, 512, 16, BF16) == rows * 512 * 4 + rows * 4 + 256
    assert gqa.decode_noalloc_scratch_bytes(16, 128, 512, 16, BF16) <= 96 << 20  # the absorbed-MLA workload fits
    # the GQA decode at its default split count fits too
    s = gqa.decode_splits(64, 32, 8, 8192, 128, 128, BF16)
    assert gqa.decode_noalloc_scratch_bytes(64, 32, 128, s, BF16) <= 96 << 20
    assert gqa.decode_noalloc_scratch_bytes(1, 1, 3, 1, F32) == 512 + 256
    assert gqa.decode_noalloc_scratch_bytes(0, 32, 128, 10, BF16) == 0
    assert gqa.decode_noalloc_scratch_bytes(1, 32, 128, 10, 9) == 0


@pytest.mark.parametrize("cu,total,ok", [
    ([0, 5, 9], 9, True), ([0, 0, 0], 0, True), ([2, 5, 9], 9, True), ([0, 5, 9], 12, True),
    ([0, 5, 10], 9, False), ([-1, 5, 9], 9, False), ([0, 6, 5], 9, False), ([0], 9, False),
])
def test_check_cu_seqlens(cu, total, ok):
    """The binding's optional host check of packed offsets: non-decreasing,
    at or above 0, ending inside the tensor."""
    if ok:
        gqa.check_cu_seqlens(cu, total)
    else:
        with pytest.raises(ValueError):
            gqa.check_cu_seqlens(cu, total)


def test_check_topk_distinct():
    import numpy as np
    lens = np.array([10, 5])
    gqa.check_topk_distinct(np.array([[1, 2, 3, -1], [0, 4, 7, 7]]), lens)  # 7 >= 5 selects nothing
    with pytest.raises(ValueError):
        gqa.check_topk_distinct(np.array([[1, 2, 1, -1], [0, 1, 2, 3]]), lens)
