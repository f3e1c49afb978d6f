"""Host-side check of the dense bf16 forward's looping schedule (no GPU).

When a dense D = 128 forward has more items (head-block unit x query tile)
than one resident round of workgroups, the host launches that one round
(256 workgroups of 8 waves, one per CU) and each workgroup walks items in a
snake order inside its XCD's contiguous share.  The host takes that path
only when its divisibility conditions hold.  This test restates both the
host condition and the kernel's item arithmetic in plain Python. It checks
that every item of a qualifying shape is taken exactly once, and that the
causal key-tile counts per workgroup stay within 2 % of their mean (the
two headline forward shapes exactly equal).
"""
import math
import random

import pytest

WAVES, ROWS_PER_WAVE, BN, RESIDENT = 8, 32, 64, 256


def geometry(B, Hq, Hkv, Tq):
    G = Hq // Hkv
    gt = 1
    while gt * 2 <= WAVES and G % (gt * 2) == 0 and WAVES % (gt * 2) == 0:
        gt *= 2
    Pt = ROWS_PER_WAVE * (WAVES // gt)
    return B * Hkv * (G // gt), math.ceil(Tq / Pt), Pt


def host_loops(n_units, n_qt):
    items = n_units * n_qt
    per_xcd, nwx = items // 8, RESIDENT // 8
    return (items > RESIDENT and items % 8 == 0 and per_xcd % n_qt == 0 and n_qt % 2 == 0
            and per_xcd % nwx == 0 and (per_xcd // nwx) % 2 == 0)


def workgroup_items(L, nblk, items, n_qt):
    """(unit, query tile) pairs workgroup L takes, in order."""
    xcd, j = L & 7, L >> 3
    nwx = (nblk >> 3) + (1 if (nblk & 7) > xcd else 0)
    per, rem = items >> 3, items & 7
    cnt = per + (1 if xcd < rem else 0)
    start = xcd * (per + 1) if xcd < rem else rem * (per + 1) + (xcd - rem) * per
    out, k = [], 0
    while True:
        pos = (k + 1) * nwx - 1 - j if k & 1 else k * nwx + j
        if pos >= cnt:
            return out
        Lp = start + pos
        unit = Lp // n_qt
        out.append((unit, n_qt - 1 - (Lp - unit * n_qt)))
        k += 1


def key_tiles(qt, Pt, Tq, Tk):
    off = Tk - Tq
    kend = min(Tk, off + min(Tq, qt * Pt + Pt))
    return (kend + BN - 1) // BN


def check(B, Hq, Hkv, Tq, Tk):
    n_units, n_qt, Pt = geometry(B, Hq, Hkv, Tq)
    if not host_loops(n_units, n_qt):
        return None
    items = n_units * n_qt
    seen = [0] * items
    loads = []
    for L in range(RESIDENT):
        its = workgroup_items(L, RESIDENT, items, n_qt)
        for u, qt in its:
            assert 0 <= u < n_units and 0 <= qt < n_qt
            seen[u * n_qt + qt] += 1
        loads.append(sum(key_tiles(qt, Pt, Tq, Tk) for _, qt in its))
    assert all(c == 1 for c in seen), (B, Hq, Hkv, Tq, Tk)
    mean = sum(loads) / len(loads)
    return max(loads) / mean - 1.0, min(loads) / mean - 1.0


@pytest.mark.parametrize("shape,exact", [
    ((4, 32, 8, 4096, 4096), True),     # GQA prefill: 260 key tiles per workgroup
    ((8, 64, 1, 512, 16384), False),    # MQA suffix: loops, nearly flat causal profile
])
def test_headline_shapes_loop_and_balance(shape, exact):
    r = check(*shape)
    assert r is not None, "the host must take the looping path for this shape"
    hi, lo = r
    if exact:
        assert hi == 0.0 and lo == 0.0
    assert hi <= 0.02 and lo >= -0.02


def test_random_qualifying_shapes_cover_every_item_once():
    rng = random.Random(7)
    qualified = 0
    for _ in range(600):
        Hkv = rng.choice([1, 2, 4, 8])
        G = rng.choice([1, 2, 4, 8, 16])
        B = rng.randint(1, 64)
        Tq = 64 * rng.randint(1, 128)
        Tk = Tq + 64 * rng.choice([0, 0, 0, 4, 32])
        r = check(B, Hkv * G, Hkv, Tq, Tk)
        if r is None:
            continue
        qualified += 1
        hi, lo = r
        assert hi <= 0.02 and lo >= -0.02, (B, Hkv * G, Hkv, Tq, Tk, r)
    assert qualified >= 20


def test_small_or_indivisible_shapes_keep_one_item_per_workgroup():
    assert check(1, 8, 8, 256, 256) is None        # fewer items than one round
    assert check(4, 32, 8, 4032, 4032) is None     # odd number of query tiles per unit
    assert check(1, 32, 2, 4096, 4096) is None     # an XCD's share is not whole units
