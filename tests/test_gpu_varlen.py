"""GPU parity of the packed variable-length / sliding-window forward
(gqa_attn_fwd_varlen) against the fp64 oracle.

Tolerance as for every bf16 path: max |err| <= 2e-2, mean |err| <= 2e-3
(GPU output widened to fp64 minus the oracle's fp64 output).  Cases cover
sequences shorter than, equal to and just past the 64-key tile and the
256-query workgroup tile, suffix sequences (fewer queries than keys), more
queries than keys (zero rows), empty sequences, non-causal cross attention,
both packed layouts ([total, H, D] and [H, total, D] views), MHA / GQA / MQA,
D = 64 and 128, windows from 1 to wider than every sequence, and the
full-size sliding-window workload on sampled rows.
"""
import numpy as np
import pytest
import torch

import causal_grouped_query_amd as gqa
import workloads as W
from oracle import oracle as O

pytestmark = pytest.mark.gpu

TMAX, TMEAN = 2e-2, 2e-3


def _rand(shape, seed):
    g = torch.Generator("cpu").manual_seed(seed)
    return torch.randn(*shape, generator=g, dtype=torch.float32).to(torch.bfloat16)


def _check(gpu, ref, what):
    g = gpu.detach().double().cpu().numpy().reshape(ref.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    d = np.abs(g - ref)
    print(f"{what} max_abs={d.max():.3e} mean_abs={d.mean():.3e}", flush=True)
    assert d.max() <= TMAX and d.mean() <= TMEAN, f"{what}: max {d.max():.3e} mean {d.mean():.3e}"


def _cu(lens):
    return [0] + np.cumsum(lens).tolist()


def _run(lens_q, lens_k, Hq, Hkv, D, causal, window, seed, layout="thd"):
    cq, ck = _cu(lens_q), _cu(lens_k)
    q = _rand((cq[-1], Hq, D), seed)
    k = _rand((ck[-1], Hkv, D), seed + 1)
    v = _rand((ck[-1], Hkv, D), seed + 2)
    scale = 1.0 / np.sqrt(D)
    if layout == "thd":
        qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
        out = None
    else:  # [H, total, D] storage, passed as a [total, H, D] view
        qd = q.permute(1, 0, 2).contiguous().cuda().permute(1, 0, 2)
        kd = k.permute(1, 0, 2).contiguous().cuda().permute(1, 0, 2)
        vd = v.permute(1, 0, 2).contiguous().cuda().permute(1, 0, 2)
        out = torch.empty((Hq, cq[-1], D), dtype=torch.bfloat16, device="cuda").permute(1, 0, 2)
    cqd = torch.tensor(cq, dtype=torch.int32, device="cuda")
    ckd = torch.tensor(ck, dtype=torch.int32, device="cuda")
    res = gqa.attention_varlen(qd, kd, vd, cqd, ckd, scale=scale, causal=causal, window=window, out=out)
    ref = O.attention_varlen(q, k, v, cq, ck, scale, causal, window=window)
    return res, ref, (q, k, v, cq, ck)


LENS = [1, 63, 64, 65, 200, 129, 300, 257]


@pytest.mark.parametrize("window", [0, 1, 7, 64, 100, 5000])
def test_varlen_window_gqa_d128(window):
    res, ref, _ = _run(LENS, LENS, 8, 2, 128, True, window, 10)
    _check(res, ref, f"varlen gqa w={window}")


@pytest.mark.parametrize("window", [0, 33, 300])
def test_varlen_suffix_sequences(window):
    """Fewer queries than keys: queries sit at the end of their sequence."""
    res, ref, _ = _run([5, 100, 1, 64, 70], [300, 100, 17, 200, 450], 8, 2, 128, True, window, 20)
    _check(res, ref, f"varlen suffix w={window}")


def test_varlen_more_queries_than_keys_and_empty_sequences():
    """Causal with Tq_i > Tk_i: the first Tq_i - Tk_i queries see no key (zero
    rows); empty sequences in between contribute nothing."""
    lens_q, lens_k = [10, 0, 3, 0, 90], [4, 0, 3, 5, 60]
    res, ref, _ = _run(lens_q, lens_k, 4, 2, 128, True, 0, 30)
    assert torch.all(res[:6] == 0)
    _check(res, ref, "varlen Tq>Tk / empty")


def test_varlen_noncausal_cross_attention():
    res, ref, _ = _run([7, 130, 64], [90, 30, 200], 8, 4, 128, False, 0, 40)
    _check(res, ref, "varlen non-causal")


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (16, 1), (8, 2)])
@pytest.mark.parametrize("layout", ["thd", "htd"])
def test_varlen_head_groups_layouts_d64(Hq, Hkv, layout):
    res, ref, _ = _run([70, 1, 256, 130], [70, 1, 256, 130], Hq, Hkv, 64, True, 50, 50, layout)
    _check(res, ref, f"varlen d64 {Hq}/{Hkv} {layout}")


def test_varlen_sequences_are_independent_and_window_hides_old_keys():
    """Bit-identical outputs when (a) another sequence's keys and values change
    and (b) keys / values older than every query's window change."""
    lens = [100, 300]
    w = 40
    res, _, (q, k, v, cq, ck) = _run(lens, lens, 4, 2, 128, True, w, 60)
    k2, v2 = k.clone(), v.clone()
    k2[:100] = _rand((100, 2, 128), 61)       # sequence 0 changes entirely
    v2[:100] = _rand((100, 2, 128), 62)
    k2[100:100 + 50] = _rand((50, 2, 128), 63)  # sequence 1: keys 0..49, older than the
    v2[100:100 + 50] = _rand((50, 2, 128), 64)  # window of queries at positions >= 89
    cqd = torch.tensor(cq, dtype=torch.int32, device="cuda")
    ckd = torch.tensor(ck, dtype=torch.int32, device="cuda")
    res2 = gqa.attention_varlen(q.cuda(), k2.cuda(), v2.cuda(), cqd, ckd, causal=True, window=w)
    first_unaffected = 100 + 50 + w - 1  # queries of sequence 1 at positions >= 50 + w - 1
    assert torch.equal(res[first_unaffected:], res2[first_unaffected:])


def test_varlen_dense_problem_matches_dense_entry():
    """One sequence of the dense problem through both entry points: identical
    results (same kernel arithmetic, different addressing)."""
    B, Hq, Hkv, T, D = 2, 8, 2, 333, 128
    q = _rand((B, Hq, T, D), 70).cuda()
    k = _rand((B, Hkv, T, D), 71).cuda()
    v = _rand((B, Hkv, T, D), 72).cuda()
    dense = gqa.attention(q, k, v, causal=True)
    cu = torch.tensor([0, T, 2 * T], dtype=torch.int32, device="cuda")
    pk = lambda x: x.permute(0, 2, 1, 3).reshape(B * T, x.shape[1], D)
    var = gqa.attention_varlen(pk(q), pk(k), pk(v), cu, cu, causal=True)
    assert torch.equal(var, pk(dense))


def test_swa_varlen_workload_full_size_sampled():
    """The benchmarked sliding-window workload at full size, checked on
    sampled rows of every sequence (first, last, around the window edge)."""
    w = W.SWA_VARLEN
    q, k, v, cu = W.varlen_inputs(w)
    cud = cu.cuda()
    out = gqa.attention_varlen(q.cuda(), k.cuda(), v.cuda(), cud, cud, scale=w.scale, causal=True,
                               window=w.extra["window"])
    win = w.extra["window"]
    cul = cu.tolist()
    rng = np.random.default_rng(5)
    for i in range(len(cul) - 1):
        s0, n = cul[i], cul[i + 1] - cul[i]
        pos = sorted({0, n - 1, min(win - 1, n - 1), min(win, n - 1), *rng.integers(0, n, 6).tolist()})
        heads = [0, w.Hq - 1, int(rng.integers(0, w.Hq))]
        view = lambda x: x[s0:s0 + n].permute(1, 0, 2).unsqueeze(0)
        rows = [a * n + p for a in heads for p in pos]
        ref = O.attention(view(q), view(k), view(v), w.scale, True, rows=rows, window=win)
        got = torch.stack([out[s0 + p, a] for a in heads for p in pos])
        _check(got, ref, f"swa workload seq {i} (len {n})")


def test_varlen_many_short_sequences():
    """More than 64 sequences (the tile search walks cu_seqlens in chunks of
    64), lengths 0..40 including empty ones, window 9."""
    rng = np.random.default_rng(7)
    lens = rng.integers(0, 41, 150).tolist()
    lens[3] = 0
    res, ref, _ = _run(lens, lens, 8, 2, 128, True, 9, 80)
    _check(res, ref, "varlen 150 sequences")


def test_varlen_no_query_tokens_is_a_no_op():
    q = torch.empty((0, 4, 128), dtype=torch.bfloat16, device="cuda")
    k = _rand((10, 2, 128), 90).cuda()
    cq = torch.tensor([0, 0], dtype=torch.int32, device="cuda")
    ck = torch.tensor([0, 10], dtype=torch.int32, device="cuda")
    out = gqa.attention_varlen(q, k, k, cq, ck)
    assert out.shape == (0, 4, 128)


@pytest.mark.parametrize("causal,window,used_q,used_k", [
    (True, 0, [300, 1, 0, 129, 64], [300, 1, 7, 129, 64]),
    (True, 50, [300, 200, 65, 2, 256], [300, 200, 65, 2, 256]),
    (True, 0, [10, 64, 1, 0, 33], [290, 64, 100, 8, 300]),     # suffix queries inside padded slots
    (True, 0, [90, 3, 256], [40, 3, 0]),                        # more queries than keys: zero rows
    (False, 0, [17, 300, 0], [300, 5, 44]),
])
def test_varlen_right_padded_batch(causal, window, used_q, used_k):
    """A right-padded batch [B, Tpad, H, D] through cu_seqlens = multiples of
    Tpad and the used lengths: padded keys hold NaN and are never read, padded
    query rows keep what out held before (a sentinel), used rows match the
    oracle."""
    B, Tpad, Hq, Hkv, D = len(used_q), 300, 8, 2, 128
    seed = 100 + sum(used_q)
    q = _rand((B * Tpad, Hq, D), seed)
    k = _rand((B * Tpad, Hkv, D), seed + 1)
    v = _rand((B * Tpad, Hkv, D), seed + 2)
    cu = [i * Tpad for i in range(B + 1)]
    keep_q = np.zeros(B * Tpad, dtype=bool)
    keep_k = np.zeros(B * Tpad, dtype=bool)
    for i in range(B):
        keep_q[cu[i]:cu[i] + used_q[i]] = True
        keep_k[cu[i]:cu[i] + used_k[i]] = True
    kd, vd = k.clone(), v.clone()
    kd[~keep_k] = float("nan")
    vd[~keep_k] = float("nan")
    cud = torch.tensor(cu, dtype=torch.int32, device="cuda")
    uq = torch.tensor(used_q, dtype=torch.int32, device="cuda")
    uk = torch.tensor(used_k, dtype=torch.int32, device="cuda")
    out = torch.full((B * Tpad, Hq, D), 7.0, dtype=torch.bfloat16, device="cuda")
    gqa.attention_varlen(q.cuda(), kd.cuda(), vd.cuda(), cud, cud, causal=causal, window=window, out=out,
                         seqused_q=uq, seqused_k=uk)
    ref = O.attention_varlen(q, k, v, cu, cu, 1.0 / np.sqrt(D), causal, window=window,
                             seqused_q=used_q, seqused_k=used_k)
    got = out.cpu()
    assert torch.all(got[torch.from_numpy(~keep_q)] == 7.0), "padded query rows were written"
    _check(got[torch.from_numpy(keep_q)], ref[keep_q], f"padded batch causal={causal} w={window}")


def test_varlen_padding_equals_packed():
    """The padded batch and the packed batch of the same tokens give
    bit-identical rows (same arithmetic, different addressing)."""
    Tpad, lens = 260, [260, 70, 129, 1]
    B, Hq, Hkv, D = len(lens), 4, 1, 64
    q = _rand((B * Tpad, Hq, D), 120).cuda()
    k = _rand((B * Tpad, Hkv, D), 121).cuda()
    v = _rand((B * Tpad, Hkv, D), 122).cuda()
    cu = torch.tensor([i * Tpad for i in range(B + 1)], dtype=torch.int32, device="cuda")
    used = torch.tensor(lens, dtype=torch.int32, device="cuda")
    pad = gqa.attention_varlen(q, k, v, cu, cu, causal=True, window=33, seqused_q=used, seqused_k=used)
    idx = torch.cat([torch.arange(i * Tpad, i * Tpad + n) for i, n in enumerate(lens)]).cuda()
    cp = torch.tensor([0] + np.cumsum(lens).tolist(), dtype=torch.int32, device="cuda")
    packed = gqa.attention_varlen(q[idx], k[idx], v[idx], cp, cp, causal=True, window=33)
    assert torch.equal(pad[idx], packed)


def test_multi_token_decode_over_padded_cache():
    """Incremental decode with several new tokens per sequence (the query
    count differs from the cache length, as the masks section of the
    "Attention variants" page calls out): a [B, Tmax, Hkv, D] cache with
    per-sequence fill levels, 4 queries per sequence at its last positions,
    expressed as packed slots (cu_seqlens = multiples of Tmax) with used
    lengths."""
    B, Tmax, Hq, Hkv, D, nq = 5, 600, 32, 8, 128, 4
    lens = [600, 4, 257, 31, 100]
    q = _rand((B * nq, Hq, D), 700)
    kc = _rand((B, Tmax, Hkv, D), 701)
    vc = _rand((B, Tmax, Hkv, D), 702)
    for b, n in enumerate(lens):
        kc[b, n:] = float("nan")
        vc[b, n:] = float("nan")
    cu_q = torch.arange(0, (B + 1) * nq, nq, dtype=torch.int32)
    cu_k = torch.arange(0, (B + 1) * Tmax, Tmax, dtype=torch.int32)
    used_k = torch.tensor(lens, dtype=torch.int32)
    out = gqa.attention_varlen(q.cuda(), kc.reshape(B * Tmax, Hkv, D).cuda(), vc.reshape(B * Tmax, Hkv, D).cuda(),
                               cu_q.cuda(), cu_k.cuda(), causal=True, seqused_k=used_k.cuda())
    kflat, vflat = kc.reshape(B * Tmax, Hkv, D), vc.reshape(B * Tmax, Hkv, D)
    ref = O.attention_varlen(q, kflat, vflat, cu_q.tolist(), cu_k.tolist(), 1.0 / np.sqrt(D), True,
                             seqused_k=lens)
    _check(out, ref, "multi-token decode, padded cache")


@pytest.mark.parametrize("cq_bad,ck_bad,cq_eff,ck_eff", [
    # last offsets past the tensors' 300 query / 420 key slots
    ([0, 100, 500], [0, 150, 700], [0, 100, 300], [0, 150, 420]),
    # a decreasing offset: the second sequence is empty
    ([0, 200, 100], [0, 300, 250], [0, 200, 200], [0, 300, 300]),
    # a negative first offset
    ([-50, 120, 300], [-10, 200, 420], [0, 120, 300], [0, 200, 420]),
])
def test_varlen_offsets_clamped_to_the_buffers(cq_bad, ck_bad, cq_eff, ck_eff):
    """Offsets that disagree with the tensors' token extents are clamped in
    the kernel: the result is that of the clamped layout, and no token
    outside q / k / v / out is addressed."""
    Hq, Hkv, D = 8, 2, 128
    q, k, v = _rand((300, Hq, D), 41), _rand((420, Hkv, D), 42), _rand((420, Hkv, D), 43)
    scale = 1.0 / np.sqrt(D)
    out = torch.zeros((300, Hq, D), dtype=torch.bfloat16, device="cuda")
    cqd = torch.tensor(cq_bad, dtype=torch.int32, device="cuda")
    ckd = torch.tensor(ck_bad, dtype=torch.int32, device="cuda")
    gqa.attention_varlen(q.cuda(), k.cuda(), v.cuda(), cqd, ckd, scale=scale, causal=True, out=out)
    torch.cuda.synchronize()
    ref = O.attention_varlen(q, k, v, cq_eff, ck_eff, scale, True)
    rows = [t for i in range(2) for t in range(cq_eff[i], cq_eff[i + 1])]  # tokens of non-empty sequences
    _check(out[rows], ref[rows], f"clamped offsets {cq_bad} / {ck_bad}")
    with pytest.raises(ValueError):
        gqa.attention_varlen(q.cuda(), k.cuda(), v.cuda(), cqd, ckd, scale=scale, causal=True, validate=True)
