"""Pins of the oracle's paged attention over FP8 E4M3FN pools.

Sources on the pages: TileOPs "Attention Operators", GQAPrefillPagedWithKVCache
FwdOp (an FP8 pool carries one key and one value dequantization scale; the
chunk is appended to the pool, then attended to) and GQAVarlenFwdOp (FP8
dequantization: each scale multiplies its tensor).  Reading: an FP8 pool
element stands for decode(code) * scale, and attention runs on those values.

Independent checks: a 16-bit pool holding the decoded values exactly (power of
two scales keep them bf16-representable) gives the same bits through the
16-bit path; the value scale multiplies the output and leaves the LSE; the key
scale acts as a factor on the score scale; a NaN code reaches exactly the rows
that see its key; the append is the FP8 write followed by the FP8 read.
"""
import numpy as np
import pytest
import torch

import oracle
from softmax_attention_amd import workloads


def fp8_pools(num_pages, ps, Hkv, D, seed):
    g = torch.Generator().manual_seed(seed)
    codes = torch.randint(0, 256, (2, num_pages, ps, Hkv, D), generator=g, dtype=torch.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3C  # no NaN codes unless a test plants one
    return codes[0].numpy(), codes[1].numpy()


def decoded_bf16(codes, scale):
    table = torch.tensor([oracle.e4m3_decode(c) * scale for c in range(256)], dtype=torch.float64)
    vals = table[torch.from_numpy(codes.astype(np.int64))]
    out = vals.to(torch.bfloat16)
    assert torch.equal(out.to(torch.float64), vals)  # exactly representable
    return out


def case(seed, B=3, Hq=4, Hkv=2, D=16, ps=16, max_pages=4, sq=(1, 5, 0)):
    g = torch.Generator().manual_seed(seed)
    num_pages = B * max_pages + 1
    bt = torch.randperm(num_pages, generator=g)[:B * max_pages].view(B, max_pages).to(torch.int32)
    lens = [int(x) for x in torch.randint(6, max_pages * ps + 1, (B,), generator=g)]
    lens = [max(L, s) for L, s in zip(lens, sq)]
    tq = sum(sq)
    q = workloads.dense_inputs(1, max(tq, 1), 1, Hq, Hkv, D, seed=seed)[0][0][:tq]
    cu = np.concatenate([[0], np.cumsum(sq)]).astype(np.int32)
    kp, vp = fp8_pools(num_pages, ps, Hkv, D, seed + 1)
    return q, kp, vp, lens, bt, ps, cu


@pytest.mark.parametrize("k_scale,v_scale", [(1.0, 1.0), (0.25, 4.0), (2.0, 0.125)])
@pytest.mark.parametrize("causal", [True, False])
def test_fp8_pool_equals_a_16bit_pool_of_its_values(k_scale, v_scale, causal):
    q, kp, vp, lens, bt, ps, cu = case(11)
    o8, l8 = oracle.attn_paged_varlen(q, kp, vp, lens, bt, ps, cu, causal=causal, cache_fp8=True,
                                      k_scale=k_scale, v_scale=v_scale)
    o16, l16 = oracle.attn_paged_varlen(q, decoded_bf16(kp, k_scale), decoded_bf16(vp, v_scale),
                                        lens, bt, ps, cu, causal=causal)
    assert np.array_equal(o8, o16) and np.array_equal(l8, l16)


def test_value_scale_multiplies_the_output_only():
    q, kp, vp, lens, bt, ps, cu = case(12)
    o1, l1 = oracle.attn_paged_varlen(q, kp, vp, lens, bt, ps, cu, cache_fp8=True)
    vs = float(np.float32(0.37))  # the scale travels as float32
    o2, l2 = oracle.attn_paged_varlen(q, kp, vp, lens, bt, ps, cu, cache_fp8=True, v_scale=vs)
    np.testing.assert_allclose(o2, vs * o1, rtol=1e-12, atol=1e-15)
    assert np.array_equal(l1, l2)


def test_key_scale_acts_on_the_score_scale():
    q, kp, vp, lens, bt, ps, cu = case(13)
    alpha = 0.3
    o1, l1 = oracle.attn_paged_varlen(q, kp, vp, lens, bt, ps, cu, cache_fp8=True, k_scale=0.37,
                                      scale=alpha)
    a2 = float(np.float32(alpha * 0.37))
    o2, l2 = oracle.attn_paged_varlen(q, kp, vp, lens, bt, ps, cu, cache_fp8=True, scale=a2)
    np.testing.assert_allclose(o1, o2, rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(l1, l2, rtol=1e-5, atol=1e-6)


def test_nan_code_reaches_the_rows_that_see_its_key():
    # one request, a 5-query causal chunk at the end of 20 keys: query i sees
    # keys 0 .. 15 + i, so a NaN in key 17 reaches queries 2, 3, 4 only
    q, kp, vp, _, bt, ps, _ = case(14, B=1, sq=(5,))
    lens, cu = [20], np.array([0, 5], np.int32)
    page, slot = int(bt[0, 17 // ps]), 17 % ps
    kp = kp.copy()
    kp[page, slot, 1, 3] = 0x7F
    o, lse = oracle.attn_paged_varlen(q, kp, vp, lens, bt, ps, cu, cache_fp8=True)
    Hq = q.shape[1]
    for i in range(5):
        for h in range(Hq):
            sees = i >= 2 and h // (Hq // 2) == 1  # KV head 1 serves query heads 2, 3
            assert np.isnan(o[i, h]).all() == sees and np.isnan(lse[h, i]) == sees, (i, h)
            if not sees:
                assert np.isfinite(o[i, h]).all() and np.isfinite(lse[h, i])


def test_rejects_scales_that_are_not_finite_and_positive():
    q, kp, vp, lens, bt, ps, cu = case(15)
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        with pytest.raises(ValueError):
            oracle.attn_paged_varlen(q, kp, vp, lens, bt, ps, cu, cache_fp8=True, k_scale=bad)
        with pytest.raises(ValueError):
            oracle.attn_paged_varlen(q, kp, vp, lens, bt, ps, cu, cache_fp8=True, v_scale=bad)


@pytest.mark.parametrize("causal,cap", [(True, None), (False, 3.0)])
def test_fp8_append_is_the_fp8_write_then_the_fp8_read(causal, cap):
    ps, Hq, Hkv, D = 16, 4, 2, 16
    sq, before = [3, 0, 18, 1], [5, 9, 14, 0]
    B, max_pages = len(sq), 3
    num_pages = B * max_pages + 2
    bt = torch.randperm(num_pages, generator=torch.Generator().manual_seed(16))[:B * max_pages]
    bt = bt.view(B, max_pages).to(torch.int32)
    kp, vp = fp8_pools(num_pages, ps, Hkv, D, 17)
    tq = sum(sq)
    q, kn, vn = workloads.dense_inputs(1, tq, tq, Hq, Hkv, D, seed=18)
    q, kn, vn = q[0], kn[0] * 8, vn[0] * 8
    cu = np.concatenate([[0], np.cumsum(sq)]).astype(np.int32)
    ks, vs = 0.7, 1.3
    o, lse, nk, nv = oracle.attn_paged_append(q, kn, vn, kp, vp, before, bt, ps, cu,
                                              causal=causal, softcap=cap, cache_fp8=True,
                                              k_scale=ks, v_scale=vs)
    slots = [int(bt[b, (before[b] + i) // ps]) * ps + (before[b] + i) % ps
             for b in range(B) for i in range(sq[b])]
    wk, wv = oracle.kv_write(kn, vn, kp, vp, torch.tensor(slots, dtype=torch.int64),
                             cache_fp8=True, k_scale=ks, v_scale=vs)
    assert np.array_equal(nk.reshape(wk.shape), wk) and np.array_equal(nv.reshape(wv.shape), wv)
    after = [before[b] + sq[b] for b in range(B)]
    o_p, lse_p = oracle.attn_paged_varlen(q, wk, wv, after, bt, ps, cu, causal=causal,
                                          softcap=cap, cache_fp8=True, k_scale=ks, v_scale=vs)
    assert np.array_equal(o, o_p) and np.array_equal(lse, lse_p)
