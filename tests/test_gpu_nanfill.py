"""GPU parity under the NaN-fill debug build (libgqa_attn_nanfill.so).

That build fills every kernel's LDS buffers (K/V rings, staged index lists,
hash tables) and the split-KV workspace with NaN bit patterns before first
use, so a kernel that reads a ring slot, list entry or partial slot that no
copy or kernel wrote turns its output into NaN, which the oracle comparison
rejects.  Each kernel family runs here on cases from the parity modules,
through the same C ABI, against the same oracle and tolerances.
"""
import os

import pytest

import causal_grouped_query_amd as gqa
import test_gpu_fp8 as F8
import test_gpu_parity as P
import test_gpu_shard as SH
import test_gpu_topk as TK
import test_gpu_varlen as VL
import test_gpu_window_decode as WD

pytestmark = pytest.mark.gpu

NANFILL_LIB = os.path.join(os.path.dirname(os.path.abspath(gqa.__file__)), "libgqa_attn_nanfill.so")


@pytest.fixture(scope="module", autouse=True)
def _nanfill_library():
    if not os.path.exists(NANFILL_LIB):
        pytest.skip("the NaN-fill debug build is missing (causal_grouped_query_amd.build makes it)")
    saved_path, saved_lib = gqa.LIB_PATH, gqa._lib
    gqa.LIB_PATH, gqa._lib = NANFILL_LIB, None
    gqa.lib()
    yield
    gqa.LIB_PATH, gqa._lib = saved_path, saved_lib


@pytest.mark.parametrize("case", [P.FWD_CASES[0], P.FWD_CASES[4], P.FWD_CASES[6], P.FWD_CASES[9]])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_nanfill_fwd(case, dtype):
    P.test_fwd_matches_oracle(case, dtype)


@pytest.mark.parametrize("case", [P.DEC_CASES[0], P.DEC_CASES[2]])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("splits", [1, 2, 0, 1024])
def test_nanfill_decode(case, dtype, splits):
    P.test_decode_matches_oracle(case, dtype, splits)


@pytest.mark.parametrize("case", [P.FLAT_CASES[0], P.FLAT_CASES[2]])
@pytest.mark.parametrize("splits", [3, 0])
def test_nanfill_flat_decode(case, splits):
    P.test_flat_decode_matches_oracle(case, splits)


@pytest.mark.parametrize("splits", [1, 3, 0])
def test_nanfill_mla(splits):
    P.test_mla_absorbed_decode_matches_oracle(128, splits)
    P.test_mla_decode_empty_and_short_sequences()


def test_nanfill_varlen():
    VL.test_varlen_window_gqa_d128(64)
    VL.test_varlen_more_queries_than_keys_and_empty_sequences()
    VL.test_varlen_head_groups_layouts_d64(8, 2, "thd")


def test_nanfill_shard_and_merge():
    SH.test_shard_matches_oracle(1000, 900, 32, 8, 128)
    SH.test_merge_matches_oracle_merge()


@pytest.mark.parametrize("splits", [1, 3, 0])
def test_nanfill_topk(splits):
    TK.test_topk_decode_small(splits)


def test_nanfill_topk_repeats_and_empty():
    TK.test_topk_decode_empty_selections_and_sequences()
    TK.test_topk_repeated_positions_in_one_slice_count_once(0)


@pytest.mark.parametrize("splits", [3, 0])
def test_nanfill_fp8(splits):
    F8.test_fp8_decode_matches_oracle(32, 8, 128, splits)


def test_nanfill_window_decode():
    WD.test_window_decode_bf16(100, 0)
    WD.test_window_decode_f32(50, 64)
    WD.test_window_decode_mla(33)
