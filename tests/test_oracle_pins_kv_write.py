"""Pins of the oracle's paged KV write, its FP8 E4M3FN codec, and the paged
prefill with append.

Sources on the pages: TileOPs "Attention Operators", PagedKVCacheWriteFwdOp
(each token's rows go to the pool row its slot names, page * page_size +
offset, -1 skipping it; nothing outside the named slots changes; an FP8 pool
stores row / scale cast to E4M3FN, NaN preserved, finite overflow and
infinities saturated to the largest finite magnitude of the same sign) and
GQAPrefillPagedWithKVCacheFwdOp (the chunk's keys and values are appended
after each request's cached ones, cache_seqlens counting them before the
append, and the chunk's queries attend to the cache).

Independent checks: torch's float8_e4m3fn conversion (a library routine; it
rounds to nearest even but turns overflow into NaN, so it is compared only
inside the finite range), the format's closed-form values, and for the append
the plain write and the plain packed-query paged call composed here with the
slots derived from the page-table rule.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from softmax_attention_amd import workloads


# ---------------------------------------------------------------- E4M3FN codec


def test_decoder_matches_torch_on_every_code():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = np.array([oracle.e4m3_decode(c) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan) and nan.sum() == 2  # 0x7f and 0xff
    assert np.array_equal(ours[~nan], ref[~nan])


def test_closed_form_values():
    assert oracle.e4m3_decode(0x38) == 1.0
    assert oracle.e4m3_decode(0x7E) == 448.0             # 1.110b * 2^8
    assert oracle.e4m3_decode(0x08) == 2.0 ** -6         # smallest normal
    assert oracle.e4m3_decode(0x01) == 2.0 ** -9         # smallest subnormal
    assert oracle.e4m3_decode(0x80) == 0.0 and math.copysign(1, oracle.e4m3_decode(0x80)) < 0


def test_every_finite_code_round_trips():
    for c in range(256):
        if (c & 0x7F) == 0x7F:
            continue
        assert oracle.e4m3_encode(oracle.e4m3_decode(c)) == c, hex(c)


def test_encoder_matches_torch_rounding_inside_the_finite_range():
    g = torch.Generator().manual_seed(7)
    x = torch.cat([torch.randn(20000, generator=g) * s for s in (1e-3, 0.05, 1.0, 30.0, 200.0)])
    x = x[x.abs() < 448]
    # the midpoints between neighbouring codes, where ties go to the even code
    vals = np.array([oracle.e4m3_decode(c) for c in range(0x7E)])
    mids = torch.tensor((vals[1:] + vals[:-1]) / 2, dtype=torch.float32)
    x = torch.cat([x, mids, -mids])
    ref = x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = np.array([oracle.e4m3_encode(float(v)) for v in x.numpy()], dtype=np.uint8)
    assert np.array_equal(ours, ref)


def test_saturation_and_nan():
    for v, code in ((448.0, 0x7E), (463.9, 0x7E), (500.0, 0x7E), (1e30, 0x7E), (math.inf, 0x7E),
                    (-500.0, 0xFE), (-math.inf, 0xFE)):
        assert oracle.e4m3_encode(v) == code, v
    assert oracle.e4m3_encode(math.nan) & 0x7F == 0x7F


# ---------------------------------------------------------------- KV write


def pools(num_pages, ps, Hkv, D, seed, fp8=False):
    g = torch.Generator().manual_seed(seed)
    if fp8:
        kp = torch.randint(0, 256, (num_pages, ps, Hkv, D), generator=g, dtype=torch.uint8)
        vp = torch.randint(0, 256, (num_pages, ps, Hkv, D), generator=g, dtype=torch.uint8)
        return kp.numpy(), vp.numpy()
    kp = torch.randn(num_pages, ps, Hkv, D, generator=g).to(torch.bfloat16)
    vp = torch.randn(num_pages, ps, Hkv, D, generator=g).to(torch.bfloat16)
    return kp, vp


def bits(t):
    return t.view(torch.int16).numpy().view(np.uint16)


def test_write_puts_each_row_at_its_slot_and_nothing_else():
    Hkv, D, ps, P = 2, 16, 16, 6
    kp, vp = pools(P, ps, Hkv, D, seed=1)
    k, v = (torch.randn(5, Hkv, D).to(torch.bfloat16) for _ in range(2))
    slots = torch.tensor([17, -1, 0, 95, 40], dtype=torch.int64)
    nk, nv = oracle.kv_write(k, v, kp, vp, slots)
    ek, ev = bits(kp).reshape(-1, Hkv, D).copy(), bits(vp).reshape(-1, Hkv, D).copy()
    for n, sl in enumerate(slots.tolist()):
        if sl >= 0:
            ek[sl], ev[sl] = bits(k[n]), bits(v[n])
    assert np.array_equal(nk.reshape(-1, Hkv, D), ek) and np.array_equal(nv.reshape(-1, Hkv, D), ev)
    # the skipped token left no trace
    assert not any(np.array_equal(nk.reshape(-1, Hkv, D)[r], bits(k[1])) for r in range(P * ps))


@pytest.mark.parametrize("k_scale,v_scale", [(1.0, 1.0), (0.37, 2.5)])
def test_fp8_write_stores_the_scaled_row_as_e4m3(k_scale, v_scale):
    Hkv, D, ps, P = 2, 32, 16, 4
    kp, vp = pools(P, ps, Hkv, D, seed=2, fp8=True)
    g = torch.Generator().manual_seed(3)
    k = (torch.randn(6, Hkv, D, generator=g) * 40).to(torch.bfloat16)
    v = (torch.randn(6, Hkv, D, generator=g) * 40).to(torch.bfloat16)
    k[0, 0, :4] = torch.tensor([1e4, -1e4, float("nan"), 0.0])
    slots = torch.tensor([3, 60, -1, 7, 8, 9], dtype=torch.int64)
    nk, nv = oracle.kv_write(k, v, kp, vp, slots, cache_fp8=True, k_scale=k_scale,
                             v_scale=v_scale)
    for n, sl in enumerate(slots.tolist()):
        if sl < 0:
            continue
        for src, scale, pool in ((k, k_scale, nk), (v, v_scale, nv)):
            x = src[n].to(torch.float32) / torch.tensor(scale, dtype=torch.float32)
            want = x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            big = x.abs().numpy() >= 464  # torch turns these into NaN; the pages saturate
            want = np.where(big, np.where(x.numpy() > 0, 0x7E, 0xFE), want)
            got = pool.reshape(-1, Hkv, D)[sl]
            nan = np.isnan(x.numpy())
            assert np.array_equal(got[~nan], want[~nan]) and np.all(got[nan] & 0x7F == 0x7F)
    assert nk.reshape(-1, Hkv, D)[3][0, 0] == 0x7E and nk.reshape(-1, Hkv, D)[3][0, 1] == 0xFE


def test_write_refuses_slots_outside_the_pool():
    kp, vp = pools(2, 16, 1, 8, seed=4)
    k = torch.zeros(1, 1, 8, dtype=torch.bfloat16)
    for bad in (32, -2):
        with pytest.raises(ValueError):
            oracle.kv_write(k, k, kp, vp, torch.tensor([bad], dtype=torch.int64))


# ---------------------------------------------------------------- append


@pytest.mark.parametrize("causal,cap", [(True, None), (False, 3.0)])
def test_append_equals_write_then_packed_paged_attention(causal, cap):
    ps, Hq, Hkv, D = 16, 4, 2, 16
    sq = [3, 0, 18, 1]
    before = [5, 9, 14, 0]
    B = len(sq)
    max_pages = 3
    num_pages = B * max_pages + 2
    bt = torch.randperm(num_pages, generator=torch.Generator().manual_seed(5))[:B * max_pages]
    bt = bt.view(B, max_pages).to(torch.int32)
    kp, vp = pools(num_pages, ps, Hkv, D, seed=6)
    tq = sum(sq)
    q, kn, vn = workloads.dense_inputs(1, tq, tq, Hq, Hkv, D, seed=7)
    q, kn, vn = q[0], kn[0], vn[0]
    cu = np.concatenate([[0], np.cumsum(sq)]).astype(np.int32)
    o, lse, nk, nv = oracle.attn_paged_append(q, kn, vn, kp, vp, before, bt, ps, cu,
                                              causal=causal, softcap=cap)
    # the slots from the page-table rule, written with the plain write
    slots = []
    for b in range(B):
        for i in range(sq[b]):
            pos = before[b] + i
            slots.append(int(bt[b, pos // ps]) * ps + pos % ps)
    wk, wv = oracle.kv_write(kn, vn, kp, vp, torch.tensor(slots, dtype=torch.int64))
    assert np.array_equal(nk.reshape(wk.shape), wk) and np.array_equal(nv.reshape(wv.shape), wv)
    after = [before[b] + sq[b] for b in range(B)]
    kt = torch.from_numpy(wk.view(np.int16)).view(torch.bfloat16)
    vt = torch.from_numpy(wv.view(np.int16)).view(torch.bfloat16)
    o_p, lse_p = oracle.attn_paged_varlen(q, kt, vt, after, bt, ps, cu, causal=causal,
                                          softcap=cap)
    assert np.array_equal(o, o_p) and np.array_equal(lse, lse_p)


def test_append_of_a_whole_prompt_equals_dense_causal_prefill():
    # an empty cache plus a chunk of S tokens is plain causal self-attention
    ps, Hq, Hkv, D, S = 16, 4, 1, 16, 40
    bt = torch.tensor([[2, 0, 3]], dtype=torch.int32)
    kp, vp = pools(4, ps, Hkv, D, seed=8)
    q, k, v = workloads.dense_inputs(1, S, S, Hq, Hkv, D, seed=9)
    o, lse, _, _ = oracle.attn_paged_append(q[0], k[0], v[0], kp, vp, [0], bt, ps, [0, S])
    o_d, lse_d = oracle.attn_dense(q, k, v, causal=True)
    assert np.array_equal(o, o_d[0]) and np.array_equal(lse, lse_d[0])
