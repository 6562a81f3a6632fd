"""GPU parity of packed (THD) calls and attention sinks (TileOPs "Attention
Operators", GQAVarlenFwdOp and GQAPagedFwdOp) against the fp64 oracle, with
the comparison rule of tests/parity.py.  Requests of very different lengths
share one launch (row blocks past a short request, requests without queries
or keys, queries before the cache start), over every schedule (8-wave
prefill, stream-K and split decode, 4-wave D = 256), with sinks that are
finite, disabled (-inf) and +inf."""
import numpy as np
import pytest
import torch

import oracle
import softmax_attention_amd as mi
from softmax_attention_amd import workloads
from tests.parity import check_rows
from tests.test_parity_gpu import DEV, _reset_split, say

pytestmark = pytest.mark.gpu

__all__ = ["_reset_split"]  # the autouse fixture that restores the split plan


def packed(sq, skv, Hq, Hkv, D, seed, dtype):
    tq, tk = sum(sq), sum(skv)
    q, k, v = workloads.dense_inputs(1, max(tq, 1), max(tk, 1), Hq, Hkv, D, dtype=dtype,
                                     seed=seed)
    cu_q = torch.tensor(np.concatenate([[0], np.cumsum(sq)]), dtype=torch.int32)
    cu_k = torch.tensor(np.concatenate([[0], np.cumsum(skv)]), dtype=torch.int32)
    return q[0, :tq], k[0, :tk], v[0, :tk], cu_q, cu_k


def make_sinks(Hq, seed, special=True):
    g = torch.Generator().manual_seed(seed)
    s = (torch.randn(Hq, generator=g) * 2.0).to(torch.float32)
    if special:
        s[0] = float("-inf")
        s[Hq - 1] = float("inf")
    return s


def compare(o, lse, o_ref, lse_ref, what):
    o_np = o.detach().cpu().to(torch.float64).numpy()
    lse_np = lse.detach().cpu().numpy().astype(np.float64)
    return check_rows(o_np, lse_np.T, o_ref, lse_ref.T, what)


def varlen_case(sq, skv, Hq, Hkv, D, *, dtype=torch.bfloat16, causal=True, window=None,
                softcap=None, sinks=None, scale=None, split_keys=0, seed=0, what=""):
    say(f"varlen {what} sq={sq} skv={skv} Hq={Hq} Hkv={Hkv} D={D} {dtype} causal={causal} "
        f"window={window} softcap={softcap} sinks={sinks is not None} split_keys={split_keys}")
    q, k, v, cu_q, cu_k = packed(sq, skv, Hq, Hkv, D, seed, dtype)
    mi.set_split_keys(split_keys)
    o, lse = mi.attn_fwd_varlen(q.to(DEV), k.to(DEV), v.to(DEV), cu_q.to(DEV), cu_k.to(DEV),
                                causal=causal, window=window, softcap=softcap, scale=scale,
                                sinks=None if sinks is None else sinks.to(DEV))
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_varlen(q, k, v, cu_q, cu_k, causal=causal, window=window,
                                        softcap=softcap, scale=scale, sinks=sinks)
    return compare(o, lse, o_ref, lse_ref, what)


def test_varlen_prefill_ragged_requests():
    varlen_case([700, 1, 0, 333, 64], [700, 1, 0, 333, 64], 16, 4, 128, seed=200,
                what="prefill")


def test_varlen_chunked_with_window_fp16():
    # request 3 has more queries than keys: its first rows see nothing
    varlen_case([100, 7, 0, 50], [300, 7, 40, 20], 8, 2, 64, dtype=torch.float16,
                window=(64, -1), seed=201, what="chunked_window")


def test_varlen_noncausal_two_sided_window_softcap():
    varlen_case([90, 300, 2], [400, 100, 3], 8, 8, 128, causal=False, window=(40, 25),
                softcap=3.0, seed=202, what="noncausal")


@pytest.mark.parametrize("D", [64, 128])
def test_varlen_decode_streamk_with_sinks(D):
    varlen_case([1, 1, 0, 1, 1], [3000, 1, 50, 0, 777], 32, 8, D, sinks=make_sinks(32, 203),
                seed=203, what="decode_sinks")


@pytest.mark.parametrize("split_keys", [0, 256])
def test_varlen_sinks_prefill_and_splits(split_keys):
    varlen_case([200, 40, 1], [1000, 40, 500], 8, 2, 128, sinks=make_sinks(8, 204),
                split_keys=split_keys, seed=204, what="sinks_split")


def test_varlen_d256_sinks_softcap():
    varlen_case([37, 5, 60], [900, 5, 61], 24, 2, 256, sinks=make_sinks(24, 205),
                softcap=30.0, seed=205, what="d256")


def test_varlen_equal_blocks_equal_the_batched_call():
    say("varlen with equal blocks vs the batched dense call")
    B, S, Hq, Hkv, D = 3, 300, 8, 2, 128
    q, k, v = workloads.dense_inputs(B, S, S, Hq, Hkv, D, seed=206)
    cu = torch.arange(0, (B + 1) * S, S, dtype=torch.int32)
    o_v, l_v = mi.attn_fwd_varlen(q.reshape(B * S, Hq, D).to(DEV), k.reshape(B * S, Hkv, D).to(DEV),
                                  v.reshape(B * S, Hkv, D).to(DEV), cu.to(DEV), cu.to(DEV))
    o_d, l_d = mi.attn_fwd_dense(q.to(DEV), k.to(DEV), v.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(o_v, o_d.reshape(B * S, Hq, D))
    assert torch.equal(l_v, l_d.transpose(0, 1).reshape(Hq, B * S))


# ---------------------------------------------------------------- paged


def paged_varlen_case(sq, lens, Hq, Hkv, D, page_size, *, dtype=torch.bfloat16, causal=True,
                      window=None, softcap=None, sinks=None, split_keys=0, seed=0, what=""):
    say(f"paged_varlen {what} sq={sq} lens={lens} Hq={Hq} Hkv={Hkv} D={D} page={page_size} "
        f"window={window} softcap={softcap} sinks={sinks is not None} split_keys={split_keys}")
    B = len(sq)
    max_pages = max(1, max((L + page_size - 1) // page_size for L in lens)) + 1
    n_phys = B * max_pages + 3
    _, kd, vd = workloads.dense_inputs(B, 1, max_pages * page_size, Hkv, Hkv, D, dtype=dtype,
                                       seed=seed)
    kd, vd = kd.clone(), vd.clone()
    for b, L in enumerate(lens):
        kd[b, L:] = float("nan")
        vd[b, L:] = float("nan")
    g = torch.Generator().manual_seed(seed + 1)
    bt = torch.randperm(n_phys, generator=g)[:B * max_pages].view(B, max_pages).to(torch.int32)
    kc = workloads.scatter_to_pages(kd, bt, page_size, n_phys, fill=float("nan"))
    vc = workloads.scatter_to_pages(vd, bt, page_size, n_phys, fill=float("nan"))
    q, _, _ = workloads.dense_inputs(1, max(sum(sq), 1), 1, Hq, Hkv, D, dtype=dtype,
                                     seed=seed + 2)
    q = q[0, :sum(sq)]
    cu_q = torch.tensor(np.concatenate([[0], np.cumsum(sq)]), dtype=torch.int32)
    lens_t = torch.tensor(lens, dtype=torch.int32)
    mi.set_split_keys(split_keys)
    o, lse = mi.attn_fwd_paged_varlen(q.to(DEV), kc.to(DEV), vc.to(DEV), lens_t.to(DEV),
                                      bt.to(DEV), cu_q.to(DEV), page_size, causal=causal,
                                      window=window, softcap=softcap,
                                      sinks=None if sinks is None else sinks.to(DEV))
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_paged_varlen(q, kc, vc, lens_t, bt, page_size, cu_q,
                                              causal=causal, window=window, softcap=softcap,
                                              sinks=sinks)
    return compare(o, lse, o_ref, lse_ref, what)


@pytest.mark.parametrize("page_size", [16, 64])
def test_paged_varlen_mixed_prefill_and_decode(page_size):
    paged_varlen_case([1, 37, 0, 1, 5], [900, 37, 20, 1, 2000], 16, 4, 128, page_size,
                      softcap=20.0, sinks=make_sinks(16, 210), seed=210, what="mixed")


def test_paged_varlen_decode_streamk_window_sinks():
    lens = [1, 0, 64, 65, 1000, 513, 2047, 300]
    paged_varlen_case([1] * len(lens), lens, 32, 8, 128, 64, window=(255, -1),
                      sinks=make_sinks(32, 211), seed=211, what="decode")


def test_paged_varlen_split_decode_sinks():
    lens = [1, 0, 64, 65, 1000, 513, 2047, 300]
    paged_varlen_case([1] * len(lens), lens, 32, 8, 64, 32, sinks=make_sinks(32, 212),
                      split_keys=128, seed=212, what="split")


def test_paged_varlen_d256_wide_group():
    paged_varlen_case([37, 3, 20], [900, 37, 20], 24, 2, 256, 64, sinks=make_sinks(24, 213),
                      seed=213, what="d256")


def test_paged_varlen_equal_counts_equal_the_paged_call():
    say("paged varlen with equal query counts vs the paged call")
    w = workloads.make(3)
    q = w.q.to(DEV)
    kc, vc = w.k_cache.to(DEV), w.v_cache.to(DEV)
    lens, bt = w.real_seqlen_kv.to(DEV), w.block_table.to(DEV)
    cu = torch.arange(0, w.B + 1, dtype=torch.int32, device=DEV)
    o_v, l_v = mi.attn_fwd_paged_varlen(q.reshape(w.B, w.Hq, w.D), kc, vc, lens, bt, cu,
                                        w.page_size)
    o_p, l_p = mi.attn_fwd_paged(q, kc, vc, lens, bt, w.page_size)
    torch.cuda.synchronize()
    assert torch.equal(o_v, o_p.reshape(w.B, w.Hq, w.D))
    assert torch.equal(l_v, l_p.reshape(w.B, w.Hq).T)


def test_full_size_paged_varlen_decode_sinks():
    w = workloads.make(3)
    sinks = make_sinks(w.Hq, 214, special=False)
    say(f"{w.name} packed queries with sinks")
    cu = torch.arange(0, w.B + 1, dtype=torch.int32)
    q = w.q.reshape(w.B, w.Hq, w.D)
    o, lse = mi.attn_fwd_paged_varlen(q.to(DEV), w.k_cache.to(DEV), w.v_cache.to(DEV),
                                      w.real_seqlen_kv.to(DEV), w.block_table.to(DEV),
                                      cu.to(DEV), w.page_size, sinks=sinks.to(DEV))
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_paged_varlen(q, w.k_cache, w.v_cache, w.real_seqlen_kv,
                                              w.block_table, w.page_size, cu, sinks=sinks)
    compare(o, lse, o_ref, lse_ref, w.name)
