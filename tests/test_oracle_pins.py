"""Pins for the fp64 oracle: facts fixed by the pages and by mathematics.

Each test checks the oracle against something other than its own formula:
the worked example the "Attention variants" page prints, invariants the
pages state (decode equals the last row of the causal prefill, softmax rows
sum to one, future keys get no weight, MHA/MQA are limits of GQA), closed
forms, and PyTorch's own scaled-dot-product attention run on the CPU in
float64 as an independent library routine.  A plausible slip anywhere in the
oracle (dropped scale, wrong head index, square mask on a suffix, a
transposed operand, a missing normaliser) fails at least one of them.
"""
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *rest = line.split()
            vals[key] = [float(x) for x in rest]
    return vals


def _rand(shape, seed, dtype=torch.float64):
    g = torch.Generator("cpu").manual_seed(seed)
    return torch.randn(*shape, generator=g, dtype=torch.float64).to(dtype)


# ---------------------------------------------------------------- worked example

def test_head_mapping_worked_example():
    """The page's head-mapping self-test: q=k=0, v=[1,7] per KV head -> [1,1,7,7]."""
    g = _read_golden("head_mapping_attention_variants.txt")
    q = np.array(g["q_values"]).reshape([int(x) for x in g["q_shape"]])
    k = np.array(g["k_values"]).reshape([int(x) for x in g["k_shape"]])
    v = np.array(g["v_values"]).reshape([int(x) for x in g["v_shape"]])
    out = O.attention(q, k, v, 1.0 / math.sqrt(q.shape[-1]), True)
    assert out.ravel().tolist() == g["expected"]


@pytest.mark.parametrize("Hq,vals,expected", [
    (8, [1.0, 7.0], [1, 1, 1, 1, 7, 7, 7, 7]),
    (8, [1.0, 3.0, 5.0, 7.0], [1, 1, 3, 3, 5, 5, 7, 7]),
    (4, [1.0, 3.0, 5.0, 7.0], [1, 3, 5, 7]),
    (4, [2.0], [2, 2, 2, 2]),
])
def test_head_mapping_extensions(Hq, vals, expected):
    Hkv = len(vals)
    q = np.zeros((1, Hq, 1, 1))
    k = np.zeros((1, Hkv, 1, 1))
    v = np.array(vals).reshape(1, Hkv, 1, 1)
    assert O.attention(q, k, v, 1.0, True).ravel().tolist() == [float(x) for x in expected]


# ---------------------------------------------------------------- stated invariants

def test_decode_is_last_row_pages_self_test_shapes():
    """The page's self-test: q (2,4,5,8), k,v (2,2,5,8) from seed 0; one-step decode
    equals the last row of the full causal output, and the output has q's shape."""
    torch.manual_seed(0)
    q = torch.randn(2, 4, 5, 8).double()
    k, v = torch.randn(2, 2, 5, 8).double(), torch.randn(2, 2, 5, 8).double()
    full = O.attention(q, k, v, 1 / math.sqrt(8), True)
    step = O.attention(q[:, :, -1:].contiguous(), k, v, 1 / math.sqrt(8), True)
    assert full.shape == tuple(q.shape)
    np.testing.assert_allclose(step, full[:, :, -1:], rtol=0, atol=1e-14)


@pytest.mark.parametrize("Tq", [1, 2, 7, 16, 33])
def test_suffix_queries_match_rows_of_full_prefill(Tq):
    """Queries at positions Tk-Tq..Tk-1 see the same keys as those rows of the full
    causal prefill (a square mask applied to a suffix would fail this)."""
    Tk = 33
    q = _rand((2, 6, Tk, 16), 1)
    k = _rand((2, 3, Tk, 16), 2)
    v = _rand((2, 3, Tk, 12), 3)
    full = O.attention(q, k, v, 0.25, True)
    suf = O.attention(q[:, :, Tk - Tq:].contiguous(), k, v, 0.25, True)
    np.testing.assert_allclose(suf, full[:, :, Tk - Tq:], rtol=0, atol=1e-14)


def test_probabilities_sum_to_one_and_future_is_zero():
    Tq, Tk = 9, 20
    q = _rand((1, 4, Tq, 8), 4)
    k = _rand((1, 2, Tk, 8), 5)
    v = _rand((1, 2, Tk, 8), 6)
    for a in range(4):
        for i in range(Tq):
            p, o = O.probs(q, k, v, 0.5, True, 0, a, i)
            pos = Tk - Tq + i
            assert abs(p.sum() - 1.0) < 1e-12
            assert np.all(p[pos + 1:] == 0.0)
            assert np.all(p[: pos + 1] > 0.0)
            # the output row is the probability-weighted sum of the KV head's values
            g = a // 2
            np.testing.assert_allclose(o, p @ v[0, g].numpy(), rtol=0, atol=1e-12)


def test_future_keys_and_values_have_no_effect():
    Tq = Tk = 24
    q = _rand((2, 4, Tq, 8), 7)
    k = _rand((2, 2, Tk, 8), 8)
    v = _rand((2, 2, Tk, 8), 9)
    base = O.attention(q, k, v, 0.3, True)
    for i in [0, 5, 17]:
        k2, v2 = k.clone(), v.clone()
        k2[:, :, i + 1:] = _rand(k2[:, :, i + 1:].shape, 10 + i) * 50
        v2[:, :, i + 1:] = _rand(v2[:, :, i + 1:].shape, 20 + i) * 50
        out = O.attention(q, k2, v2, 0.3, True)
        np.testing.assert_array_equal(out[:, :, : i + 1], base[:, :, : i + 1])


def test_decode_lengths_ignore_cache_tail():
    """A decode cache of capacity Tmax with len_b valid keys: the slots past len_b
    (here NaN) never reach the output, and the result equals a fresh forward over
    exactly len_b keys with the query at position len_b - 1."""
    B, Hq, Hkv, Tmax, D = 3, 4, 2, 40, 8
    q = _rand((B, Hq, 1, D), 11)
    k = _rand((B, Hkv, Tmax, D), 12)
    v = _rand((B, Hkv, Tmax, D), 13)
    lens = [1, 17, 40]
    for b, n in enumerate(lens):
        k[b, :, n:] = float("nan")
        v[b, :, n:] = float("nan")
    out = O.attention(q, k, v, 0.4, True, kv_lens=lens)
    assert np.isfinite(out).all()
    for b, n in enumerate(lens):
        ref = O.attention(q[b:b + 1], k[b:b + 1, :, :n].contiguous(), v[b:b + 1, :, :n].contiguous(),
                          0.4, True)
        np.testing.assert_array_equal(out[b:b + 1], ref)


def test_gqa_equals_mha_on_expanded_kv_and_mqa_limit():
    """GQA is MHA run on K/V whose heads are repeated G times (the expansion is a
    copy, not arithmetic); MQA is the Hkv=1 limit."""
    B, Hq, T, D = 2, 8, 13, 8
    q = _rand((B, Hq, T, D), 14)
    for Hkv in [1, 2, 4, 8]:
        k = _rand((B, Hkv, T, D), 15 + Hkv)
        v = _rand((B, Hkv, T, D), 25 + Hkv)
        G = Hq // Hkv
        ke = k.repeat_interleave(G, dim=1).contiguous()
        ve = v.repeat_interleave(G, dim=1).contiguous()
        np.testing.assert_array_equal(O.attention(q, k, v, 0.35, True), O.attention(q, ke, ve, 0.35, True))


# ---------------------------------------------------------------- closed forms

def test_zero_query_gives_prefix_mean():
    """q = 0 makes every visible key equally likely: o_i = mean(v[0..p_i])."""
    Tq, Tk = 7, 19
    q = torch.zeros((1, 2, Tq, 4), dtype=torch.float64)
    k = _rand((1, 1, Tk, 4), 30)
    v = _rand((1, 1, Tk, 5), 31)
    out = O.attention(q, k, v, 1.0, True)
    csum = np.cumsum(v[0, 0].numpy(), axis=0)
    for i in range(Tq):
        pos = Tk - Tq + i
        np.testing.assert_allclose(out[0, 0, i], csum[pos] / (pos + 1), rtol=0, atol=1e-13)
        np.testing.assert_allclose(out[0, 1, i], csum[pos] / (pos + 1), rtol=0, atol=1e-13)


def test_single_key_and_constant_values():
    q = _rand((2, 4, 1, 6), 32)
    k = _rand((2, 2, 1, 6), 33)
    v = _rand((2, 2, 1, 3), 34)
    out = O.attention(q, k, v, 0.7, True)
    np.testing.assert_array_equal(out, v.repeat_interleave(2, dim=1).numpy())
    # V == 1 everywhere gives an all-ones output for any scores
    q = _rand((2, 4, 11, 6), 35)
    k = _rand((2, 2, 11, 6), 36)
    ones = torch.ones((2, 2, 11, 3), dtype=torch.float64)
    np.testing.assert_allclose(O.attention(q, k, ones, 0.9, True), 1.0, rtol=0, atol=1e-14)


def test_identical_keys_noncausal_is_mean_of_values():
    k = _rand((1, 1, 1, 6), 37).repeat(1, 1, 10, 1).contiguous()
    q = _rand((1, 3, 4, 6), 38)
    v = _rand((1, 1, 10, 7), 39)
    out = O.attention(q, k, v, 0.5, False)
    np.testing.assert_allclose(out, np.broadcast_to(v.numpy().mean(axis=2, keepdims=True), out.shape),
                               rtol=0, atol=1e-13)


def test_dominant_key_selects_its_value():
    """One key aligned with the query and scaled far above the rest takes all the
    weight; a dropped scale or sign error would not."""
    D, Tk = 8, 12
    q = torch.zeros((1, 1, 1, D), dtype=torch.float64)
    q[..., 0] = 1.0
    k = _rand((1, 1, Tk, D), 40) * 0.1
    k[0, 0, 5, 0] = 400.0
    v = _rand((1, 1, Tk, 4), 41)
    out = O.attention(q, k, v, 0.5, False)
    np.testing.assert_allclose(out[0, 0, 0], v[0, 0, 5].numpy(), rtol=0, atol=1e-12)
    # with a negative alignment the same key gets no weight at all
    k[0, 0, 5, 0] = -400.0
    p, _ = O.probs(q, k, v, 0.5, False, 0, 0, 0)
    assert p[5] < 1e-80


def test_scale_enters_only_as_product_with_scores():
    q = _rand((1, 2, 5, 8), 42)
    k = _rand((1, 1, 9, 8), 43)
    v = _rand((1, 1, 9, 8), 44)
    a = O.attention(q, k, v, 0.5, True)
    b = O.attention(q * 2.0, k, v, 0.25, True)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)


def test_linearity_in_values():
    q = _rand((1, 4, 6, 8), 45)
    k = _rand((1, 2, 10, 8), 46)
    v = _rand((1, 2, 10, 8), 47)
    w = _rand((1, 2, 10, 8), 48)
    lhs = O.attention(q, k, 2.0 * v - 3.0 * w, 0.3, True)
    rhs = 2.0 * O.attention(q, k, v, 0.3, True) - 3.0 * O.attention(q, k, w, 0.3, True)
    np.testing.assert_allclose(lhs, rhs, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- library routine

def _sdpa_reference(q, k, v, scale, causal):
    """torch's scaled_dot_product_attention, CPU float64, with the query offset
    Tk - Tq expressed as an explicit boolean mask."""
    Tq, Tk = q.shape[2], k.shape[2]
    mask = None
    if causal:
        qpos = torch.arange(Tk - Tq, Tk)[:, None]
        kpos = torch.arange(Tk)[None, :]
        mask = kpos <= qpos
    return F.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=scale,
                                          enable_gqa=(q.shape[1] != k.shape[1]))


@pytest.mark.parametrize("B,Hq,Hkv,Tq,Tk,Dk,Dv,causal", [
    (1, 4, 2, 17, 17, 16, 16, True),     # square causal GQA, ragged length
    (2, 8, 2, 5, 29, 16, 16, True),      # suffix queries (decode-like chunk)
    (2, 6, 6, 1, 31, 8, 8, True),        # MHA single-step decode
    (1, 8, 1, 9, 40, 32, 32, True),      # MQA suffix
    (2, 4, 2, 12, 7, 16, 16, False),     # cross attention, Tq > Tk
    (1, 8, 1, 1, 23, 72, 64, True),      # absorbed-MLA shape family: Dk != Dv
])
def test_matches_torch_sdpa_float64(B, Hq, Hkv, Tq, Tk, Dk, Dv, causal):
    q = _rand((B, Hq, Tq, Dk), 50)
    k = _rand((B, Hkv, Tk, Dk), 51)
    v = _rand((B, Hkv, Tk, Dv), 52)
    scale = 1.0 / math.sqrt(Dk) * 1.3
    ours = O.attention(q, k, v, scale, causal)
    ref = _sdpa_reference(q, k, v, scale, causal).numpy()
    np.testing.assert_allclose(ours, ref, rtol=0, atol=1e-12)


def test_mla_value_is_latent_view_of_key():
    """Absorbed MLA decode: one 576-wide key = [512 latent | 64 rope]; the value is the
    latent part.  The score is the latent dot plus the rope dot, so splitting the
    query/key into the two parts and summing the two score matrices must give the
    same attention as the single wide dot."""
    B, Hq, T = 2, 8, 19
    q = _rand((B, Hq, 1, 576), 53)
    kc = _rand((B, 1, T, 576), 54)
    v = kc[..., :512]
    scale = 1.0 / math.sqrt(192)
    ours = O.attention(q, kc, v, scale, True)
    # independent route: scores as latent-dot + rope-dot, softmax via torch, sum via matmul
    s_lat = torch.einsum("bhqd,bkd->bhqk", q[..., :512], kc[:, 0, :, :512])
    s_rope = torch.einsum("bhqd,bkd->bhqk", q[..., 512:], kc[:, 0, :, 512:])
    p = torch.softmax((s_lat + s_rope) * scale, dim=-1)
    ref = torch.einsum("bhqk,bkd->bhqd", p, kc[:, 0, :, :512]).numpy()
    np.testing.assert_allclose(ours, ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- split-KV merge

@pytest.mark.parametrize("cuts", [[0, 64], [0, 1, 64], [0, 20, 21, 50, 64], list(range(0, 65, 8))])
def test_lse_merge_of_partitions_equals_full(cuts):
    """Attention over all keys equals the log-sum-exp merge of attention over any
    partition of the keys (non-causal, so each part is a plain slice)."""
    q = _rand((1, 4, 3, 16), 60)
    k = _rand((1, 2, 64, 16), 61)
    v = _rand((1, 2, 64, 16), 62)
    full, full_lse = O.attention(q, k, v, 0.25, False, with_lse=True)
    parts, lses = [], []
    for a, b in zip(cuts[:-1], cuts[1:]):
        o, l = O.attention(q, k[:, :, a:b].contiguous(), v[:, :, a:b].contiguous(), 0.25, False,
                           with_lse=True)
        parts.append(o.reshape(-1, 16))
        lses.append(l.reshape(-1))
    merged, merged_lse = O.lse_merge(np.stack(parts), np.stack(lses))
    np.testing.assert_allclose(merged, full.reshape(-1, 16), rtol=0, atol=1e-13)
    np.testing.assert_allclose(merged_lse, full_lse.reshape(-1), rtol=0, atol=1e-13)


def test_lse_is_log_of_partition_function():
    q = _rand((1, 2, 1, 8), 63)
    k = _rand((1, 1, 10, 8), 64)
    v = _rand((1, 1, 10, 8), 65)
    _, lse = O.attention(q, k, v, 0.5, False, with_lse=True)
    s = (q[0, :, 0] @ k[0, 0].T) * 0.5
    np.testing.assert_allclose(lse.ravel(), torch.logsumexp(s, dim=-1).numpy(), rtol=0, atol=1e-13)
    # an empty part merges as nothing
    merged, _ = O.lse_merge(np.stack([np.ones((1, 3)), np.full((1, 3), 5.0)]),
                            np.stack([np.array([0.0]), np.array([-np.inf])]))
    np.testing.assert_array_equal(merged, np.ones((1, 3)))


def test_empty_visible_set_is_zero_row():
    q = _rand((2, 2, 1, 4), 66)
    k = _rand((2, 1, 5, 4), 67)
    v = _rand((2, 1, 5, 4), 68)
    out, lse = O.attention(q, k, v, 1.0, True, kv_lens=[0, 3], with_lse=True)
    assert np.all(out[0] == 0.0) and np.all(np.isneginf(lse[0]))
    assert np.all(np.isfinite(out[1]))


def test_bf16_inputs_are_widened_exactly():
    x = _rand((1, 2, 6, 8), 69, torch.float32).to(torch.bfloat16)
    k = _rand((1, 1, 6, 8), 70, torch.float32).to(torch.bfloat16)
    v = _rand((1, 1, 6, 8), 71, torch.float32).to(torch.bfloat16)
    a = O.attention(x, k, v, 0.3, True)
    b = O.attention(x.double(), k.double(), v.double(), 0.3, True)
    np.testing.assert_array_equal(a, b)


def test_rows_subset_matches_full():
    q = _rand((2, 4, 9, 8), 72)
    k = _rand((2, 2, 12, 8), 73)
    v = _rand((2, 2, 12, 8), 74)
    full = O.attention(q, k, v, 0.4, True).reshape(-1, 8)
    rows = [0, 5, 17, 35, 71]
    np.testing.assert_array_equal(O.attention(q, k, v, 0.4, True, rows=rows), full[rows])


def test_rejects_bad_problems():
    q = np.zeros((1, 3, 2, 4))
    k = np.zeros((1, 2, 2, 4))
    with pytest.raises(ValueError):
        O.attention(q, k, k, 1.0, True)  # Hq % Hkv != 0
    q = np.zeros((1, 2, 5, 4))
    k = np.zeros((1, 1, 3, 4))
    with pytest.raises(ValueError):
        O.attention(q, k, k, 1.0, True)  # causal with Tq > Tk


# ---------------------------------------------------------------- sliding window
# "A Visual Guide to Attention", section on which positions are visible: SWA
# keeps direct access to the most recent w positions.  Reading: keys
# max(0, p-w+1) .. p for the query at position p (the current position counts).

@pytest.mark.parametrize("Tq,Tk", [(13, 13), (4, 19)])
def test_window_at_least_all_keys_is_full_causal(Tq, Tk):
    q = _rand((2, 4, Tq, 8), 80)
    k = _rand((2, 2, Tk, 8), 81)
    v = _rand((2, 2, Tk, 8), 82)
    full = O.attention(q, k, v, 0.5, True)
    for w in (Tk, Tk + 5):
        np.testing.assert_array_equal(O.attention(q, k, v, 0.5, True, window=w), full)


def test_window_of_one_returns_own_value():
    """Each query sees only the key at its own position: P = 1 there."""
    Tq, Tk = 6, 11
    q = _rand((1, 4, Tq, 8), 83)
    k = _rand((1, 2, Tk, 8), 84)
    v = _rand((1, 2, Tk, 5), 85)
    out = O.attention(q, k, v, 0.7, True, window=1)
    for a in range(4):
        np.testing.assert_array_equal(out[0, a], v[0, a // 2, Tk - Tq:].numpy())


@pytest.mark.parametrize("w", [2, 3, 8])
def test_zero_query_gives_window_mean(w):
    """q = 0: uniform weights over the visible keys, i.e. the mean of
    v[max(0, p-w+1) .. p]."""
    Tq, Tk = 7, 12
    q = torch.zeros((1, 2, Tq, 4), dtype=torch.float64)
    k = _rand((1, 1, Tk, 4), 86)
    v = _rand((1, 1, Tk, 3), 87)
    out = O.attention(q, k, v, 1.0, True, window=w)
    for i in range(Tq):
        p = Tk - Tq + i
        lo = max(0, p - w + 1)
        exp = v[0, 0, lo:p + 1].numpy().mean(axis=0)
        np.testing.assert_allclose(out[0, 0, i], exp, rtol=0, atol=1e-13)
        np.testing.assert_allclose(out[0, 1, i], exp, rtol=0, atol=1e-13)


def test_window_probabilities_vanish_outside_and_sum_to_one():
    Tq, Tk, w = 5, 16, 6
    q = _rand((1, 2, Tq, 8), 88)
    k = _rand((1, 1, Tk, 8), 89)
    v = _rand((1, 1, Tk, 8), 90)
    for i in range(Tq):
        p_row, _ = O.probs(q, k, v, 0.6, True, 0, 1, i, window=w)
        pos = Tk - Tq + i
        inside = (np.arange(Tk) >= pos - w + 1) & (np.arange(Tk) <= pos)
        assert np.all(p_row[~inside] == 0.0)
        assert np.all(p_row[inside] > 0.0)
        assert abs(p_row.sum() - 1.0) < 1e-12


@pytest.mark.parametrize("B,Hq,Hkv,Tq,Tk,w", [
    (2, 4, 2, 9, 9, 3), (1, 8, 1, 5, 21, 4), (2, 6, 6, 17, 17, 16), (1, 2, 1, 1, 30, 7),
])
def test_window_matches_explicit_mask(B, Hq, Hkv, Tq, Tk, w):
    """Independent masked softmax (torch SDPA, CPU float64) with the band mask
    p-w < j <= p written out."""
    q = _rand((B, Hq, Tq, 8), 91)
    k = _rand((B, Hkv, Tk, 8), 92)
    v = _rand((B, Hkv, Tk, 6), 93)
    qpos = torch.arange(Tk - Tq, Tk)[:, None]
    kpos = torch.arange(Tk)[None, :]
    mask = (kpos <= qpos) & (kpos > qpos - w)
    ref = F.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=0.45,
                                         enable_gqa=(Hq != Hkv)).numpy()
    np.testing.assert_allclose(O.attention(q, k, v, 0.45, True, window=w), ref, rtol=0, atol=1e-12)


def test_window_needs_causal_and_positive_width():
    q = np.zeros((1, 2, 3, 4))
    k = np.zeros((1, 1, 3, 4))
    with pytest.raises(ValueError):
        O.attention(q, k, k, 1.0, False, window=2)
    with pytest.raises(ValueError):
        O.attention(q, k, k, 1.0, True, window=-1)


# ---------------------------------------------------------------- packed variable length
# "Attention Architecture Evolution", GDN section: cu_seqlens only marks the
# boundaries of packed sequences; "Attention variants", masks section: a real
# implementation needs padding / packed-segment masks.  Reading: tokens attend
# only within their own sequence.

def _packed_mask_reference(q, k, v, cq, ck, scale, causal, w, uq=None, uk=None):
    """Whole packed problem as one masked softmax over all tokens (independent
    of the per-sequence slicing): allowed(i, j) iff same sequence, neither
    token is padding (index within the sequence >= its used length) and the
    causal / window rules hold inside it.  Rows with no allowed key are zero."""
    tq, tk = cq[-1], ck[-1]
    seq_q = np.searchsorted(cq, np.arange(tq), side="right") - 1
    seq_k = np.searchsorted(ck, np.arange(tk), side="right") - 1
    same = seq_q[:, None] == seq_k[None, :]
    lq = np.arange(tq) - np.asarray(cq)[seq_q]           # index within its sequence
    lk = np.arange(tk) - np.asarray(ck)[seq_k]
    nq = np.diff(cq) if uq is None else np.asarray(uq)
    nk = np.diff(ck) if uk is None else np.asarray(uk)
    Tq_i = nq[seq_q]
    Tk_i = nk[seq_q]
    pos = (Tk_i - Tq_i + lq)[:, None]
    allowed = same & (lq < Tq_i)[:, None] & (lk < nk[seq_k])[None, :]
    if causal:
        allowed &= lk[None, :] <= pos
        if w > 0:
            allowed &= lk[None, :] > pos - w
    Hq, Hkv = q.shape[1], k.shape[1]
    out = np.zeros((tq, Hq, v.shape[2]))
    qq, kk, vv = q.numpy(), k.numpy(), v.numpy()
    for a in range(Hq):
        g = a // (Hq // Hkv)
        s = scale * qq[:, a, :] @ kk[:, g, :].T
        s = np.where(allowed, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        has = np.isfinite(m[:, 0])
        e = np.where(allowed, np.exp(s - np.where(np.isfinite(m), m, 0.0)), 0.0)
        l = e.sum(axis=1, keepdims=True)
        pm = np.divide(e, l, out=np.zeros_like(e), where=l > 0)
        out[:, a, :] = pm @ vv[:, g, :]
        out[~has, a, :] = 0.0
    return out


@pytest.mark.parametrize("causal,w", [(True, 0), (True, 3), (False, 0)])
def test_varlen_equals_block_diagonal_mask(causal, w):
    lens_q = [5, 1, 9, 4]
    lens_k = [5, 6, 9, 11]          # sequence 1 and 3: suffix queries
    cq = np.concatenate([[0], np.cumsum(lens_q)]).tolist()
    ck = np.concatenate([[0], np.cumsum(lens_k)]).tolist()
    q = _rand((cq[-1], 4, 8), 94)
    k = _rand((ck[-1], 2, 8), 95)
    v = _rand((ck[-1], 2, 6), 96)
    ours = O.attention_varlen(q, k, v, cq, ck, 0.55, causal, window=w)
    ref = _packed_mask_reference(q, k, v, cq, ck, 0.55, causal, w)
    np.testing.assert_allclose(ours, ref, rtol=0, atol=1e-12)


def test_varlen_more_queries_than_keys_gives_zero_rows():
    """Causal, Tq_i > Tk_i: the first Tq_i - Tk_i queries sit before key 0 and
    see nothing (zero rows); the rest follow the suffix rule."""
    cq, ck = [0, 6], [0, 4]
    q = _rand((6, 2, 8), 97)
    k = _rand((4, 1, 8), 98)
    v = _rand((4, 1, 8), 99)
    ours = O.attention_varlen(q, k, v, cq, ck, 0.5, True)
    assert np.all(ours[:2] == 0.0)
    ref = _packed_mask_reference(q, k, v, cq, ck, 0.5, True, 0)
    np.testing.assert_allclose(ours, ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- padding
# "Attention variants", masks section: padding masks.  Reading: sequence i
# uses the first seqused[i] tokens of its slot; padded keys are invisible,
# padded query rows are not computed (zero in the oracle's result).

@pytest.mark.parametrize("causal,w", [(True, 0), (True, 4), (False, 0)])
def test_padding_equals_explicit_padding_mask(causal, w):
    Tpad, lens_q, lens_k = 12, [12, 3, 0, 7], [12, 9, 5, 7]
    cu = [i * Tpad for i in range(5)]
    q = _rand((4 * Tpad, 4, 8), 110)
    k = _rand((4 * Tpad, 2, 8), 111)
    v = _rand((4 * Tpad, 2, 6), 112)
    ours = O.attention_varlen(q, k, v, cu, cu, 0.5, causal, window=w, seqused_q=lens_q, seqused_k=lens_k)
    ref = _packed_mask_reference(q, k, v, cu, cu, 0.5, causal, w, lens_q, lens_k)
    np.testing.assert_allclose(ours, ref, rtol=0, atol=1e-12)


def test_padding_content_is_ignored_and_matches_packed():
    """A right-padded batch gives the packed batch of the same tokens, and
    nothing in the padding changes any used row."""
    Tpad, lens = 10, [10, 4, 7]
    cu = [0, 10, 20, 30]
    q = _rand((30, 2, 8), 113)
    k = _rand((30, 1, 8), 114)
    v = _rand((30, 1, 8), 115)
    pad = O.attention_varlen(q, k, v, cu, cu, 0.6, True, seqused_q=lens, seqused_k=lens)
    idx = np.concatenate([np.arange(c, c + n) for c, n in zip(cu, lens)])
    cp = [0] + np.cumsum(lens).tolist()
    packed = O.attention_varlen(q[idx], k[idx], v[idx], cp, cp, 0.6, True)
    np.testing.assert_array_equal(pad[idx], packed)
    keep = np.zeros(30, dtype=bool)
    keep[idx] = True
    assert np.all(pad[~keep] == 0.0)
    q2, k2, v2 = q.clone(), k.clone(), v.clone()
    for t in np.flatnonzero(~keep):
        q2[t], k2[t], v2[t] = 1e3, -1e3, float("nan")
    pad2 = O.attention_varlen(q2, k2, v2, cu, cu, 0.6, True, seqused_q=lens, seqused_k=lens)
    np.testing.assert_array_equal(pad2, pad)


def test_seqused_longer_than_slot_is_clamped():
    cu = [0, 5, 9]
    q = _rand((9, 2, 8), 116)
    k = _rand((9, 2, 8), 117)
    v = _rand((9, 2, 8), 118)
    a = O.attention_varlen(q, k, v, cu, cu, 0.5, True, seqused_q=[50, 4], seqused_k=[5, 99])
    b = O.attention_varlen(q, k, v, cu, cu, 0.5, True)
    np.testing.assert_array_equal(a, b)


# ---------------------------------------------------------------- DSA top-k decode
# "Attention Architecture Evolution", DSA section: the indexer's top-k
# positions become a mask that is -inf except at the selected positions
# (scattered zeros), added to the absorbed MLA scores before the softmax.

def _dsa_dense_mask_reference(q, kv, lens, idx, scale, Dv):
    """The page's reference order: dense scores over every cached position,
    plus an index mask built by scattering zeros into -inf, softmax, then the
    latent aggregation (independent of the gather in the oracle)."""
    qq, kk = q.double().numpy(), kv.double().numpy()
    B, Hq = qq.shape[0], qq.shape[1]
    out = np.zeros((B, Hq, 1, Dv))
    for b in range(B):
        n = int(lens[b])
        s = scale * qq[b, :, 0, :] @ kk[b, 0, :n, :].T          # [Hq, n]
        mask = np.full(n, -np.inf)
        sel = [int(j) for j in idx[b] if 0 <= j < n]
        mask[sel] = 0.0
        s = s + mask[None, :]
        if not sel:
            continue
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        p = e / e.sum(axis=1, keepdims=True)
        out[b, :, 0, :] = p @ kk[b, 0, :n, :Dv]
    return out


def test_dsa_topk_equals_dense_scores_plus_index_mask():
    B, Hq, Tmax, Dk, Dv = 3, 4, 40, 24, 16
    q = _rand((B, Hq, 1, Dk), 130)
    kv = _rand((B, 1, Tmax, Dk), 131)
    lens = [40, 17, 33]
    rng = np.random.default_rng(132)
    idx = np.stack([rng.choice(n, 9, replace=False) for n in lens])
    ours = O.decode_topk(q, kv, lens, idx, 0.3, Dv)
    ref = _dsa_dense_mask_reference(q, kv, lens, idx, 0.3, Dv)
    np.testing.assert_allclose(ours, ref, rtol=0, atol=1e-12)


def test_dsa_all_positions_selected_is_dense_decode():
    B, Hq, Tmax, Dk, Dv = 2, 6, 30, 16, 12
    q = _rand((B, Hq, 1, Dk), 133)
    kv = _rand((B, 1, Tmax, Dk), 134)
    lens = [30, 11]
    rng = np.random.default_rng(135)
    idx = np.full((B, 30), -1)
    for b, n in enumerate(lens):
        idx[b, :n] = rng.permutation(n)
    ours = O.decode_topk(q, kv, lens, idx, 0.25, Dv)
    dense = O.attention(q, kv, kv[..., :Dv], 0.25, True, kv_lens=lens)
    np.testing.assert_allclose(ours, dense, rtol=0, atol=1e-12)


def test_dsa_single_selected_position_returns_its_latent():
    q = _rand((2, 3, 1, 16), 136)
    kv = _rand((2, 1, 20, 16), 137)
    idx = np.array([[7, -1, 25], [-3, 19, 19]])          # one valid position each
    ours = O.decode_topk(q, kv, [20, 20], idx, 0.5, 10)
    np.testing.assert_array_equal(ours[0, :, 0], np.broadcast_to(kv[0, 0, 7, :10].double().numpy(), (3, 10)))
    np.testing.assert_array_equal(ours[1, :, 0], np.broadcast_to(kv[1, 0, 19, :10].double().numpy(), (3, 10)))


def test_dsa_invalid_duplicate_and_order_of_indices():
    """Entries outside [0, len) select nothing, a repeated position counts
    once (the mask is a scatter), the list order does not matter, and an
    empty selection gives a zero row."""
    q = _rand((2, 4, 1, 16), 138)
    kv = _rand((2, 1, 24, 16), 139)
    lens = [24, 10]
    base = np.array([[3, 9, 20, 1], [0, 4, 9, 2]])
    noisy = np.array([[20, -1, 3, 9, 3, 24, 1, 1], [9, 10, 2, 4, -7, 0, 0, 4]])
    a = O.decode_topk(q, kv, lens, base, 0.4, 16)
    b = O.decode_topk(q, kv, lens, noisy, 0.4, 16)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-14)
    empty = O.decode_topk(q, kv, lens, np.array([[-1, 30], [10, 11]]), 0.4, 16)
    assert np.all(empty == 0.0)


# ---------------------------------------------------------------- FP8 E4M3 cache
# "Attention Architecture Evolution", DSA section: FP8 keys with per-block
# scales; "Attention variants": scale granularity of quantised K/V.  The
# value of a cached element is e4m3(code) * scale of its row.

def test_e4m3_decoder_matches_format_and_library():
    """All 256 codes against torch's independent float8_e4m3fn decoding, plus
    closed forms of the OCP E4M3 format."""
    t = O.e4m3_table()
    lib = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(t, lib)                      # NaN positions must agree too
    assert t[0x38] == 1.0 and t[0x7E] == 448.0 and t[0x01] == 2.0 ** -9 and t[0x08] == 2.0 ** -6
    assert t[0x07] == 7 * 2.0 ** -9 and t[0x00] == 0.0 and np.signbit(t[0x80]) and t[0x80] == 0.0
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF]) and np.isfinite(np.delete(t, [0x7F, 0xFF])).all()
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0)                             # codes order the values
    np.testing.assert_array_equal(t[0x80:0xFF], -pos)          # sign bit negates


def _fp8_problem(B, Hq, Hkv, T, D, seed):
    g = torch.Generator("cpu").manual_seed(seed)
    q = torch.randn(B, Hq, 1, D, generator=g, dtype=torch.float64).to(torch.bfloat16)
    def codes():
        x = (torch.randn(B, Hkv, T, D, generator=g) * 64).clamp(-448, 448)
        return x.to(torch.float8_e4m3fn).view(torch.uint8)
    kc, vc = codes(), codes()
    ks = torch.exp2(-8 + 3 * torch.rand(B, Hkv, T, generator=g))
    vs = torch.exp2(-8 + 3 * torch.rand(B, Hkv, T, generator=g))
    return q, kc, ks, vc, vs


def _dequant_with_library(codes, sc):
    return codes.view(torch.float8_e4m3fn).to(torch.float64) * sc.double()[..., None]


def test_e4m3kv_attention_is_attention_of_dequantised_cache():
    """Against attention() on a cache dequantised with torch's decoder, for
    strided (transposed-storage) codes and scales and ragged lengths."""
    B, Hq, Hkv, T, D = 2, 4, 2, 37, 16
    q, kc, ks, vc, vs = _fp8_problem(B, Hq, Hkv, T, D, 140)
    kc_t = kc.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)   # [B,T,H,D] storage
    ks_t = ks.permute(0, 2, 1).contiguous().permute(0, 2, 1)
    lens = [37, 9]
    ours = O.attention_e4m3kv(q, kc_t, ks_t, vc, vs, 0.3, True, kv_lens=lens)
    ref = O.attention(q, _dequant_with_library(kc, ks), _dequant_with_library(vc, vs), 0.3, True, kv_lens=lens)
    np.testing.assert_allclose(ours, ref, rtol=0, atol=1e-13)


def test_e4m3kv_scales_act_linearly():
    """Scaling every key scale by c is scaling the softmax scale by c; scaling
    every value scale by c scales the output by c."""
    q, kc, ks, vc, vs = _fp8_problem(1, 4, 1, 25, 16, 141)
    base = O.attention_e4m3kv(q, kc, ks, vc, vs, 0.2, True)
    np.testing.assert_allclose(O.attention_e4m3kv(q, kc, ks * 4, vc, vs, 0.05, True), base, rtol=0, atol=1e-13)
    np.testing.assert_allclose(O.attention_e4m3kv(q, kc, ks, vc, vs * 8, 0.2, True), 8 * base, rtol=0, atol=1e-12)
    # a row scale enters only its own key: doubling key 3's value scale moves
    # the output by exactly p_3 * v_3 (probabilities from the dense form)
    vs2 = vs.clone()
    vs2[0, 0, 3] *= 2
    moved = O.attention_e4m3kv(q, kc, ks, vc, vs2, 0.2, True)
    K = _dequant_with_library(kc, ks)
    V = _dequant_with_library(vc, vs)
    for a in range(4):
        p_row, _ = O.probs(q, K, V, 0.2, True, 0, a, 0)
        np.testing.assert_allclose(moved[0, a, 0] - base[0, a, 0], p_row[3] * V[0, 0, 3].numpy(), rtol=0, atol=1e-12)


# ---------------------------------------------------------------- key shards
# Sequence / context parallelism (the long-context research ledger page,
# causal-mainline section: Ring / Context Parallel when one device cannot hold
# the context): each device attends over its slice of the key axis and the
# partial results are merged exactly.  A shard's keys sit at absolute
# positions k_pos0 + j, the queries at q_pos0 + i; causal visibility
# compares absolute positions.

def _shard_mask_reference(q, k, v, scale, q_pos0, k_pos0):
    """Explicit causal mask on absolute positions, numpy fp64 (independent of
    the oracle's visible-range arithmetic)."""
    qq, kk, vv = q.double().numpy(), k.double().numpy(), v.double().numpy()
    B, Hq, Tq, _ = qq.shape
    Hkv, Tk = kk.shape[1], kk.shape[2]
    allowed = (k_pos0 + np.arange(Tk))[None, :] <= (q_pos0 + np.arange(Tq))[:, None]
    out = np.zeros((B, Hq, Tq, vv.shape[3]))
    lse = np.full((B, Hq, Tq), -np.inf)
    for b in range(B):
        for a in range(Hq):
            g = a // (Hq // Hkv)
            s = np.where(allowed, scale * qq[b, a] @ kk[b, g].T, -np.inf)
            m = s.max(axis=1)
            has = np.isfinite(m)
            e = np.exp(s - np.where(has, m, 0.0)[:, None])
            l = e.sum(axis=1)
            out[b, a, has] = (e[has] / l[has, None]) @ vv[b, g]
            lse[b, a, has] = m[has] + np.log(l[has])
    return out, lse


@pytest.mark.parametrize("q_pos0,k_pos0", [(40, 0), (40, 30), (40, 45), (10, 55), (100, 3)])
def test_shard_equals_explicit_position_mask(q_pos0, k_pos0):
    q = _rand((2, 4, 9, 8), 150)
    k = _rand((2, 2, 21, 8), 151)
    v = _rand((2, 2, 21, 8), 152)
    out, lse = O.attention_shard(q, k, v, 0.4, True, q_pos0, k_pos0)
    ref, ref_lse = _shard_mask_reference(q, k, v, 0.4, q_pos0, k_pos0)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-12)


@pytest.mark.parametrize("cuts", [[0, 70], [0, 25, 70], [0, 1, 33, 34, 69, 70], [0, 50, 60, 70]])
def test_merged_causal_shards_equal_full_attention(cuts):
    """Causal suffix attention (Tq = 12 queries at positions 58..69 over 70
    keys) equals the LSE merge of the shards' partial results, for shards
    before, across and after the queries' positions."""
    Tq, Tk = 12, 70
    q = _rand((1, 4, Tq, 16), 153)
    k = _rand((1, 1, Tk, 16), 154)
    v = _rand((1, 1, Tk, 16), 155)
    full, full_lse = O.attention(q, k, v, 0.3, True, with_lse=True)
    parts, lses = [], []
    for a, b in zip(cuts[:-1], cuts[1:]):
        o, l = O.attention_shard(q, k[:, :, a:b].contiguous(), v[:, :, a:b].contiguous(), 0.3, True,
                                 Tk - Tq, a)
        parts.append(o.reshape(-1, 16))
        lses.append(l.reshape(-1))
    merged, merged_lse = O.lse_merge(np.stack(parts), np.stack(lses))
    np.testing.assert_allclose(merged, full.reshape(-1, 16), rtol=0, atol=1e-13)
    np.testing.assert_allclose(merged_lse, full_lse.reshape(-1), rtol=0, atol=1e-13)


def test_future_shard_gives_zero_rows_and_no_weight():
    q = _rand((1, 2, 5, 8), 156)
    k = _rand((1, 1, 6, 8), 157)
    out, lse = O.attention_shard(q, k, k, 0.5, True, 10, 15)   # keys 15..20, queries 10..14
    assert np.all(out == 0.0) and np.all(np.isneginf(lse))
