"""Pins of the oracle's packed (THD) calls and attention sinks.

Sources on the pages: TileOPs "Attention Operators", GQAVarlenFwdOp (packed
q/k/v [total, heads, dim], requests delimited by cu_seqlens_q / cu_seqlens_kv,
the causal mask bottom-right aligned per request) and GQAPagedFwdOp (packed
queries over a paged cache, cache_seqlens counting each request's keys, its
queries included); both: optional float32 sinks, one logit per query head
added to the softmax denominator only, neither scaled nor softcapped, -inf
disabling a sink, +inf zeroing the head's output, and a row with no visible
key returning zero whatever its sink.

None of these re-types the oracle's per-request bookkeeping or its sink
line: a packed call is compared request by request with the plain dense and
paged calls on sliced tensors (bitwise), a sink is checked against the closed
form it implies for the unsunk result, and a torch fp64 reference appends the
sink as one more score column and drops it after the softmax.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from softmax_attention_amd import workloads


def packed_inputs(sq, skv, Hq, Hkv, D, seed, dtype=torch.bfloat16):
    tq, tk = sum(sq), sum(skv)
    q, k, v = workloads.dense_inputs(1, tq, max(tk, 1), Hq, Hkv, D, dtype=dtype, seed=seed)
    cu_q = np.concatenate([[0], np.cumsum(sq)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(skv)]).astype(np.int32)
    return q[0], k[0, :tk], v[0, :tk], cu_q, cu_k


VARLEN_CASES = [  # sq, skv, causal, window, softcap
    ([3, 1, 7, 0, 5], [9, 4, 7, 6, 0], True, None, None),
    ([4, 6], [4, 2], True, None, None),              # request 2: Sq > Skv, leading rows empty
    ([5, 2, 8], [11, 2, 30], False, (3, 2), 2.5),
    ([1, 1, 1, 1], [17, 1, 0, 40], True, (8, -1), None),
]


@pytest.mark.parametrize("case", range(len(VARLEN_CASES)))
def test_varlen_equals_per_request_dense_calls(case):
    sq, skv, causal, window, cap = VARLEN_CASES[case]
    Hq, Hkv, D = 4, 2, 8
    q, k, v, cu_q, cu_k = packed_inputs(sq, skv, Hq, Hkv, D, seed=70 + case)
    o, lse = oracle.attn_varlen(q, k, v, cu_q, cu_k, causal=causal, window=window, softcap=cap)
    for b in range(len(sq)):
        a, e = cu_q[b], cu_q[b + 1]
        if a == e:
            continue
        ka, ke = cu_k[b], cu_k[b + 1]
        o_d, lse_d = oracle.attn_dense(q[None, a:e], k[None, ka:ke], v[None, ka:ke],
                                       causal=causal, window=window, softcap=cap)
        assert np.array_equal(o[a:e], o_d[0]), b
        assert np.array_equal(lse[:, a:e], lse_d[0]), b


def test_varlen_with_equal_blocks_equals_the_batched_call():
    B, S, Hq, Hkv, D = 3, 6, 4, 1, 8
    q, k, v = workloads.dense_inputs(B, S, S, Hq, Hkv, D, seed=75)
    cu = np.arange(0, (B + 1) * S, S, dtype=np.int32)
    o, lse = oracle.attn_varlen(q.reshape(B * S, Hq, D), k.reshape(B * S, Hkv, D),
                                v.reshape(B * S, Hkv, D), cu, cu)
    o_b, lse_b = oracle.attn_dense(q, k, v)
    assert np.array_equal(o, o_b.reshape(B * S, Hq, D))
    assert np.array_equal(lse, lse_b.transpose(1, 0, 2).reshape(Hq, B * S))


def paged_setup(lens, Hkv, D, ps, seed, n_extra=3):
    B = len(lens)
    max_pages = max(1, max((L + ps - 1) // ps for L in lens))
    n_phys = B * max_pages + n_extra
    cap = max_pages * ps
    _, kd, vd = workloads.dense_inputs(B, 1, cap, Hkv, Hkv, D, seed=seed)
    kd, vd = kd.clone(), vd.clone()
    for b, L in enumerate(lens):
        kd[b, L:] = float("nan")
        vd[b, L:] = float("nan")
    g = torch.Generator().manual_seed(seed)
    bt = torch.randperm(n_phys, generator=g)[:B * max_pages].view(B, max_pages).to(torch.int32)
    kc = workloads.scatter_to_pages(kd, bt, ps, n_phys, fill=float("nan"))
    vc = workloads.scatter_to_pages(vd, bt, ps, n_phys, fill=float("nan"))
    return kd, vd, kc, vc, bt


@pytest.mark.parametrize("causal,window,cap", [(True, None, None), (False, (5, 3), 4.0),
                                               (True, (16, -1), None)])
def test_paged_varlen_equals_per_request_dense_calls(causal, window, cap):
    sq = [3, 0, 1, 9, 2]
    lens = [40, 7, 1, 9, 100]
    Hq, Hkv, D, ps = 6, 2, 8, 16
    kd, vd, kc, vc, bt = paged_setup(lens, Hkv, D, ps, seed=76)
    q, _, _ = workloads.dense_inputs(1, sum(sq), 1, Hq, Hkv, D, seed=77)
    q = q[0]
    cu_q = np.concatenate([[0], np.cumsum(sq)]).astype(np.int32)
    o, lse = oracle.attn_paged_varlen(q, kc, vc, lens, bt, ps, cu_q, causal=causal,
                                      window=window, softcap=cap)
    assert not np.isnan(o).any()
    for b in range(len(sq)):
        a, e = cu_q[b], cu_q[b + 1]
        if a == e:
            continue
        L = lens[b]
        o_d, lse_d = oracle.attn_dense(q[None, a:e], kd[b:b + 1, :L], vd[b:b + 1, :L],
                                       causal=causal, window=window, softcap=cap)
        assert np.array_equal(o[a:e], o_d[0]) and np.array_equal(lse[:, a:e], lse_d[0]), b


def test_paged_varlen_with_equal_query_counts_equals_the_paged_call():
    lens = [33, 64, 5]
    B, Sq, Hq, Hkv, D, ps = 3, 2, 4, 2, 8, 16
    _, _, kc, vc, bt = paged_setup(lens, Hkv, D, ps, seed=78)
    q, _, _ = workloads.dense_inputs(B, Sq, 1, Hq, Hkv, D, seed=79)
    cu_q = np.arange(0, (B + 1) * Sq, Sq, dtype=np.int32)
    o, lse = oracle.attn_paged_varlen(q.reshape(B * Sq, Hq, D), kc, vc, lens, bt, ps, cu_q)
    o_p, lse_p = oracle.attn_paged(q, kc, vc, torch.tensor(lens, dtype=torch.int32), bt, ps)
    assert np.array_equal(o, o_p.reshape(B * Sq, Hq, D))
    assert np.array_equal(lse, lse_p.transpose(1, 0, 2).reshape(Hq, B * Sq))


# ---------------------------------------------------------------- sinks


def test_disabled_sinks_change_nothing():
    q, k, v, cu_q, cu_k = packed_inputs([4, 3], [6, 9], 4, 2, 8, seed=80)
    o, lse = oracle.attn_varlen(q, k, v, cu_q, cu_k)
    o_s, lse_s = oracle.attn_varlen(q, k, v, cu_q, cu_k, sinks=np.full(4, -np.inf, np.float32))
    assert np.array_equal(o, o_s) and np.array_equal(lse, lse_s)


@pytest.mark.parametrize("scale,cap", [(None, None), (0.5, 1.0), (2.0, None)])
def test_sink_scales_the_output_by_its_share_of_the_denominator(scale, cap):
    # with the sink only in the denominator: lse_s = ln(e^lse + e^sink) and
    # o_s = o e^(lse - lse_s).  Sinks above the cap (3.0 > 1.0) and with a
    # scale != 1 show that the sink is used as given.
    sinks = np.array([3.0, -2.0, 0.25, 7.5], np.float32)
    q, k, v, cu_q, cu_k = packed_inputs([5, 2, 3], [5, 8, 1], 4, 2, 16, seed=81)
    o, lse = oracle.attn_varlen(q, k, v, cu_q, cu_k, scale=scale, softcap=cap)
    o_s, lse_s = oracle.attn_varlen(q, k, v, cu_q, cu_k, scale=scale, softcap=cap, sinks=sinks)
    for h in range(4):
        s = float(sinks[h])
        for t in range(o.shape[0]):
            want = max(lse[h, t], s) + math.log(math.exp(lse[h, t] - max(lse[h, t], s)) +
                                                math.exp(s - max(lse[h, t], s)))
            assert lse_s[h, t] == pytest.approx(want, rel=1e-14, abs=1e-14)
            np.testing.assert_allclose(o_s[t, h], o[t, h] * math.exp(lse[h, t] - want),
                                       rtol=1e-13, atol=1e-15)


def test_infinite_sink_zeroes_the_output():
    q, k, v, cu_q, cu_k = packed_inputs([3, 2], [3, 4], 2, 1, 8, seed=82)
    o, lse = oracle.attn_varlen(q, k, v, cu_q, cu_k, sinks=np.array([np.inf, 0.0], np.float32))
    assert np.all(o[:, 0] == 0) and np.all(lse[0] == np.inf)
    assert np.all(np.isfinite(lse[1]))


def test_row_without_visible_keys_is_zero_whatever_its_sink():
    # request 0 has 4 queries and 2 keys: its first 2 rows see nothing
    q, k, v, cu_q, cu_k = packed_inputs([4], [2], 3, 1, 8, seed=83)
    sinks = np.array([1.5, -np.inf, np.inf], np.float32)
    o, lse = oracle.attn_varlen(q, k, v, cu_q, cu_k, sinks=sinks)
    assert np.all(o[:2] == 0)
    assert np.array_equal(lse[:, :2], np.array([[1.5, 1.5], [-np.inf, -np.inf],
                                                [np.inf, np.inf]]))


def torch_sink_reference(q, k, v, cu_q, cu_k, scale, sinks):
    """fp64 torch on the CPU, request by request: causal scores, one extra
    column holding the sink, softmax, the extra column dropped before P.V."""
    o = torch.zeros(q.shape, dtype=torch.float64)
    lse = torch.zeros(q.shape[1], q.shape[0], dtype=torch.float64)
    Hq, Hkv = q.shape[1], k.shape[1]
    for b in range(len(cu_q) - 1):
        a, e, ka, ke = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        qb = q[a:e].to(torch.float64).transpose(0, 1)                      # [H, Sq, D]
        kb = k[ka:ke].to(torch.float64).transpose(0, 1).repeat_interleave(Hq // Hkv, 0)
        vb = v[ka:ke].to(torch.float64).transpose(0, 1).repeat_interleave(Hq // Hkv, 0)
        Sq, Skv = e - a, ke - ka
        z = torch.matmul(qb, kb.transpose(-1, -2).contiguous()) * scale
        hide = torch.triu(torch.ones(Sq, Skv, dtype=torch.bool), diagonal=Skv - Sq + 1)
        z = z.masked_fill(hide, float("-inf"))
        col = torch.tensor(sinks, dtype=torch.float64)[:, None, None].expand(Hq, Sq, 1)
        zs = torch.cat([z, col], dim=-1)
        p = torch.softmax(zs, dim=-1)[..., :Skv]
        o[a:e] = torch.matmul(p, vb).transpose(0, 1)
        lse[:, a:e] = torch.logsumexp(zs, dim=-1)
    return o.numpy(), lse.numpy()


def test_matches_torch_reference_with_a_sink_column():
    sinks = np.array([0.5, -1.0, 2.0, 0.0], np.float32)
    q, k, v, cu_q, cu_k = packed_inputs([6, 3, 8], [6, 10, 20], 4, 2, 16, seed=84)
    o, lse = oracle.attn_varlen(q, k, v, cu_q, cu_k, scale=0.25, sinks=sinks)
    o_t, lse_t = torch_sink_reference(q, k, v, cu_q, cu_k, 0.25, sinks)
    np.testing.assert_allclose(o, o_t, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lse_t, rtol=1e-12, atol=1e-12)


def test_malformed_offsets_are_rejected():
    q, k, v, cu_q, cu_k = packed_inputs([2, 2], [2, 2], 2, 1, 8, seed=85)
    for bad_q, bad_k in (([1, 2, 4], cu_k), ([0, 3, 2], cu_k), ([0, 2, 5], cu_k),
                         (cu_q, [0, 2, 3])):
        with pytest.raises(ValueError):
            oracle.attn_varlen(q, k, v, np.array(bad_q, np.int32), np.array(bad_k, np.int32))
