"""GPU parity of the paged KV-cache write and the paged prefill with append
(TileOPs "Attention Operators", PagedKVCacheWriteFwdOp and
GQAPrefillPagedWithKVCacheFwdOp) against the oracle: pools are compared byte
for byte (the write is integer work: copies, and FP8 codes the oracle derives
in the same float32 precision), attention outputs with the rule of
tests/parity.py."""
import numpy as np
import pytest
import torch

import oracle
import softmax_attention_amd as mi
from softmax_attention_amd import workloads
from tests.parity import check_rows
from tests.test_parity_gpu import DEV, _reset_split, say

pytestmark = pytest.mark.gpu

__all__ = ["_reset_split"]


def pool_bytes(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.uint8).numpy().reshape(-1)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_write_16bit_pools(dtype):
    say(f"kv write 16-bit {dtype}")
    P, ps, Hkv, D, T = 12, 16, 4, 128, 70
    g = torch.Generator().manual_seed(300)
    kp = torch.randn(P, ps, Hkv, D, generator=g).to(dtype)
    vp = torch.randn(P, ps, Hkv, D, generator=g).to(dtype)
    k = torch.randn(T, Hkv, D, generator=g).to(dtype)
    v = torch.randn(T, Hkv, D, generator=g).to(dtype)
    slots = torch.randperm(P * ps, generator=g)[:T].to(torch.int64)
    slots[::7] = -1
    kd, vd = kp.to(DEV), vp.to(DEV)
    mi.kv_cache_write(k.to(DEV), v.to(DEV), kd, vd, slots.to(DEV))
    torch.cuda.synchronize()
    ek, ev = oracle.kv_write(k, v, kp, vp, slots)
    assert np.array_equal(pool_bytes(kd), ek.view(np.uint8).reshape(-1))
    assert np.array_equal(pool_bytes(vd), ev.view(np.uint8).reshape(-1))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("k_scale,v_scale", [(1.0, 1.0), (0.37, 2.5)])
def test_write_fp8_pools(dtype, k_scale, v_scale):
    say(f"kv write fp8 {dtype} scales {k_scale} {v_scale}")
    P, ps, Hkv, D, T = 8, 16, 2, 64, 40
    g = torch.Generator().manual_seed(301)
    kp = torch.randint(0, 256, (P, ps, Hkv, D), generator=g, dtype=torch.uint8)
    vp = torch.randint(0, 256, (P, ps, Hkv, D), generator=g, dtype=torch.uint8)
    big = 3e4 if dtype == torch.bfloat16 else 6e4
    k = (torch.randn(T, Hkv, D, generator=g) * 40).to(dtype)
    v = (torch.randn(T, Hkv, D, generator=g) * 0.01).to(dtype)  # subnormal range too
    k[0, 0, :6] = torch.tensor([big, -big, float("nan"), float("inf"), float("-inf"), -0.0])
    # the midpoints between codes (ties to even) and the saturation edge
    vals = np.array([oracle.e4m3_decode(c) for c in range(0x7E)])
    mids = torch.tensor((vals[1:] + vals[:-1]) / 2 * k_scale, dtype=torch.float32).to(dtype)
    k[1:1 + (len(mids) + D - 1) // D].view(-1)[:len(mids)] = mids
    slots = torch.randperm(P * ps, generator=g)[:T].to(torch.int64)
    slots[3] = -1
    kd = kp.to(DEV).view(torch.float8_e4m3fn)
    vd = vp.to(DEV).view(torch.float8_e4m3fn)
    ks = torch.tensor([k_scale], dtype=torch.float32, device=DEV)
    vs = torch.tensor([v_scale], dtype=torch.float32, device=DEV)
    mi.kv_cache_write(k.to(DEV), v.to(DEV), kd, vd, slots.to(DEV), k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    ek, ev = oracle.kv_write(k, v, kp.numpy(), vp.numpy(), slots, cache_fp8=True,
                             k_scale=k_scale, v_scale=v_scale)
    assert np.array_equal(pool_bytes(kd), ek.reshape(-1))
    assert np.array_equal(pool_bytes(vd), ev.reshape(-1))


def test_write_skips_slots_outside_the_pool():
    say("kv write: slots past the pool are skipped")
    P, ps, Hkv, D = 4, 16, 1, 64
    g = torch.Generator().manual_seed(302)
    kp = torch.randn(P, ps, Hkv, D, generator=g).to(torch.bfloat16)
    k = torch.randn(3, Hkv, D, generator=g).to(torch.bfloat16)
    slots = torch.tensor([5, P * ps, 9], dtype=torch.int64)
    kd, vd = kp.to(DEV), kp.clone().to(DEV)
    mi.kv_cache_write(k.to(DEV), k.to(DEV), kd, vd, slots.to(DEV))
    torch.cuda.synchronize()
    ek, _ = oracle.kv_write(k, k, kp, kp, torch.tensor([5, -1, 9], dtype=torch.int64))
    assert np.array_equal(pool_bytes(kd), ek.view(np.uint8).reshape(-1))


# ---------------------------------------------------------------- append


def append_case(sq, before, Hq, Hkv, D, ps, *, dtype=torch.bfloat16, causal=True, softcap=None,
                seed=0, what=""):
    say(f"append {what} sq={sq} before={before} Hq={Hq} Hkv={Hkv} D={D} page={ps} "
        f"causal={causal} softcap={softcap}")
    B = len(sq)
    max_pages = max((b + s + ps - 1) // ps for b, s in zip(before, sq)) + 1
    num_pages = B * max_pages + 3
    g = torch.Generator().manual_seed(seed)
    bt = torch.randperm(num_pages, generator=g)[:B * max_pages].view(B, max_pages)
    bt = bt.to(torch.int32)
    kp = torch.randn(num_pages, ps, Hkv, D, generator=g).to(dtype)
    vp = torch.randn(num_pages, ps, Hkv, D, generator=g).to(dtype)
    tq = sum(sq)
    q, kn, vn = workloads.dense_inputs(1, max(tq, 1), max(tq, 1), Hq, Hkv, D, dtype=dtype,
                                       seed=seed + 1)
    q, kn, vn = q[0, :tq], kn[0, :tq], vn[0, :tq]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(sq)]), dtype=torch.int32)
    lens = torch.tensor(before, dtype=torch.int32)
    kd, vd = kp.to(DEV), vp.to(DEV)
    o, lse = mi.attn_fwd_paged_append(q.to(DEV), kn.to(DEV), vn.to(DEV), kd, vd, lens.to(DEV),
                                      bt.to(DEV), cu.to(DEV), ps, causal=causal,
                                      softcap=softcap)
    torch.cuda.synchronize()
    o_ref, lse_ref, ek, ev = oracle.attn_paged_append(q, kn, vn, kp, vp, lens, bt, ps, cu,
                                                      causal=causal, softcap=softcap)
    assert np.array_equal(pool_bytes(kd), ek.view(np.uint8).reshape(-1))
    assert np.array_equal(pool_bytes(vd), ev.view(np.uint8).reshape(-1))
    o_np = o.detach().cpu().to(torch.float64).numpy()
    check_rows(o_np, lse.cpu().numpy().astype(np.float64).T, o_ref, lse_ref.T, what)


def test_append_mixed_requests():
    append_case([3, 0, 18, 1], [5, 9, 14, 0], 8, 2, 128, 16, seed=310, what="mixed")


def test_append_long_chunks_across_pages_fp16_softcap():
    append_case([300, 45], [700, 0], 16, 4, 64, 64, dtype=torch.float16, softcap=5.0,
                seed=311, what="long")


def test_append_decode_tokens_streamk():
    lens = [0, 63, 64, 511, 1000, 3, 2047]
    append_case([1] * len(lens), lens, 32, 8, 128, 64, seed=312, what="decode")


def test_append_d256_wide_group_noncausal():
    append_case([37, 5], [200, 61], 24, 2, 256, 32, causal=False, seed=313, what="d256")


def test_full_size_append_of_the_last_token_equals_paged_decode():
    # appending each request's last cached row at its own position rewrites
    # the same bytes, so the call must equal the plain decode over the cache
    w = workloads.make(3)
    say(f"{w.name}: append of each request's last token")
    kc, vc = w.k_cache.to(DEV), w.v_cache.to(DEV)
    lens, bt = w.real_seqlen_kv.to(DEV), w.block_table.to(DEV)
    o_p, l_p = mi.attn_fwd_paged(w.q.to(DEV), kc, vc, lens, bt, w.page_size)
    last = (w.real_seqlen_kv - 1).long()
    rows = (w.block_table.long()[torch.arange(w.B), last // w.page_size] * w.page_size +
            last % w.page_size)
    kn, vn = w.k_cache[rows].to(DEV), w.v_cache[rows].to(DEV)
    before = (w.real_seqlen_kv - 1).to(DEV)
    cu = torch.arange(w.B + 1, dtype=torch.int32, device=DEV)
    o_a, l_a = mi.attn_fwd_paged_append(w.q.reshape(w.B, w.Hq, w.D).to(DEV), kn, vn, kc, vc,
                                        before, bt, cu, w.page_size)
    torch.cuda.synchronize()
    assert torch.equal(o_a, o_p.reshape(w.B, w.Hq, w.D))
    assert torch.equal(l_a, l_p.reshape(w.B, w.Hq).T)
    assert torch.equal(kc.cpu(), w.k_cache) and torch.equal(vc.cpu(), w.v_cache)
