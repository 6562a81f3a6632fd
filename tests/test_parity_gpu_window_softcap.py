"""GPU parity of the sliding window and the logit softcap (TileOPs "Attention
Operators", GQADenseFwdOp stages 5 and 6; GQAPagedFwdOp takes the same two
parameters) against the fp64 oracle, with the comparison rule of
tests/parity.py.  The cases cover every schedule (8-wave prefill, 3-wave
stream-K decode, split decode, 4-wave D = 256), windows that start inside a
key tile, windows that leave whole splits or whole workgroups empty, rows
that see nothing, and caps small enough that most logits saturate."""
import numpy as np
import pytest
import torch

import oracle
import softmax_attention_amd as mi
from softmax_attention_amd import workloads
from tests.parity import check_full
from tests.test_parity_gpu import (DEV, _reset_split, dense_case, padding_mask,
                                   paged_case, run_dense, say)

pytestmark = pytest.mark.gpu

__all__ = ["_reset_split"]  # the autouse fixture that restores the split plan


# ---------------------------------------------------------------- dense


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("wl", [0, 100, 257])
def test_dense_causal_left_window(D, wl):
    dense_case(2, 700, 700, 16, 4, D, window=(wl, -1), seed=100 + wl, what=f"win{wl}")


def test_dense_rectangular_two_sided_window_with_mask():
    mask = padding_mask(2, 900, [900, 611])
    dense_case(2, 300, 900, 8, 8, 64, dtype=torch.float16, causal=False, window=(64, 32),
               mask=mask, seed=101, what="two_sided")


def test_dense_window_rows_that_see_nothing():
    # Sq > Skv, non-causal, narrow window: the first rows sit far left of key 0
    dense_case(1, 200, 60, 4, 2, 128, causal=False, window=(3, 5), seed=102, what="empty_rows")


@pytest.mark.parametrize("split_keys", [128, 512])
def test_dense_forced_splits_before_the_window(split_keys):
    # splits wholly left of every row's window write empty partials
    dense_case(1, 64, 3000, 8, 2, 128, window=(200, -1), split_keys=split_keys, seed=103,
               what="split_window")


@pytest.mark.parametrize("cap", [2.0, 50.0])
@pytest.mark.parametrize("D", [64, 128, 256])
def test_dense_softcap(cap, D):
    dense_case(2, 333, 333, 8, 2, D, softcap=cap, sigma=2.0, seed=104, what=f"cap{cap}")


def test_dense_softcap_with_window_mask_and_negative_scale():
    mask = padding_mask(2, 500, [500, 317])
    dense_case(2, 200, 500, 8, 4, 128, causal=False, scale=-0.3, softcap=1.5,
               window=(150, 10), mask=mask, seed=105, what="cap_window_neg")


def test_dense_softcap_zero_scale_gives_the_mean():
    dense_case(1, 130, 130, 4, 2, 64, scale=0.0, softcap=3.0, seed=106, what="cap_zero_scale")


def test_dense_window_wider_than_the_keys_is_no_window():
    q, k, v = workloads.dense_inputs(1, 100, 100, 8, 2, 128, seed=107)
    o1, l1 = run_dense(q, k, v, scale=None, causal=True)
    o2, l2 = run_dense(q, k, v, scale=None, causal=True, window=(100, 1 << 30))
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_dense_decode_shaped_window_streamk():
    dense_case(5, 1, 3000, 16, 4, 64, dtype=torch.float16, window=(700, -1), softcap=20.0,
               seed=108, what="sk_dense_window")


# ---------------------------------------------------------------- paged


@pytest.mark.parametrize("page_size", [16, 64])
@pytest.mark.parametrize("wl", [0, 31, 256, 5000])
def test_paged_decode_window_streamk(page_size, wl):
    lens = [1, 0, 64, 65, 1000, 513, 2047, 300]
    paged_case(len(lens), 1, 32, 8, 128, lens, page_size, window=(wl, -1), seed=110,
               what=f"sk_win{wl}")


@pytest.mark.parametrize("split_keys", [128, 1024])
def test_paged_decode_window_fixed_splits(split_keys):
    lens = [1, 0, 64, 65, 1000, 513, 2047, 300]
    paged_case(len(lens), 1, 32, 8, 128, lens, 64, window=(300, -1), softcap=5.0,
               split_keys=split_keys, seed=111, what="split_win")


@pytest.mark.parametrize("D", [64, 128, 256])
def test_paged_decode_softcap_head_dims(D):
    paged_case(4, 1, 16, 4, D, [700, 33, 1, 1500], 32, softcap=10.0, seed=112,
               what=f"cap_d{D}")


def test_paged_chunked_prefill_window_softcap_wide_group():
    paged_case(3, 37, 24, 2, 256, [900, 37, 20], 64, window=(128, -1), softcap=30.0, seed=113,
               what="chunked_win_cap")


def test_paged_prefill_window_multiple_row_blocks():
    paged_case(2, 150, 8, 2, 128, [150, 1200], 16, window=(90, -1), split_keys=256, seed=114,
               what="prefill_win_rb")


def test_paged_noncausal_two_sided_window_fp16():
    paged_case(3, 2, 8, 2, 128, [400, 2, 90], 64, dtype=torch.float16, causal=False,
               window=(40, 1), scale=0.2, seed=115, what="paged_two_sided")


# ---------------------------------------------------------------- full size


def test_full_size_causal_gqa_prefill_window_softcap():
    w = workloads.make(2)
    say(f"{w.name} window=(1023, -1) softcap=50")
    o, lse = run_dense(w.q, w.k, w.v, scale=w.scale, causal=True, window=(1023, -1),
                       softcap=50.0)
    # every output row (the window leaves ~44 % of the pairs: ~10 s of oracle)
    o_ref, lse_ref = oracle.attn_dense(w.q, w.k, w.v, scale=w.scale, causal=True,
                                       window=(1023, -1), softcap=50.0)
    check_full(o, lse, o_ref, lse_ref, w.name)


def test_full_size_paged_decode_window():
    w = workloads.make(3)
    say(f"{w.name} window=(2047, -1)")
    o, lse = mi.attn_fwd_paged(w.q.to(DEV), w.k_cache.to(DEV), w.v_cache.to(DEV),
                               w.real_seqlen_kv.to(DEV), w.block_table.to(DEV), w.page_size,
                               window=(2047, -1))
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_paged(w.q, w.k_cache, w.v_cache, w.real_seqlen_kv,
                                       w.block_table, w.page_size, window=(2047, -1))
    check_full(o, lse, o_ref, lse_ref, w.name)
