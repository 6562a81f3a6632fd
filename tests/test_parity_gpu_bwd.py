"""GPU parity of the attention backward (TileOPs "Attention Operators",
GQABwdOp) against the fp64 oracle.  The GPU forward supplies o and lse; both
sides then take the same q, k, v, o, do and lse.  Tolerance (derived in the
design notes from the arithmetic: 16-bit P and dS operands, FP32
accumulation, 16-bit outputs): |g - g_ref| <= 2e-2 * rms(g_ref) + 1e-2 * |g_ref|
per element, for each of dq, dk, dv; no NaN."""
import numpy as np
import pytest
import torch

import oracle
import softmax_attention_amd as mi
from softmax_attention_amd import workloads
from tests.test_parity_gpu import DEV, say

pytestmark = pytest.mark.gpu


def check_grad(g, ref, what):
    g = g.detach().cpu().to(torch.float64).numpy()
    assert g.shape == ref.shape, (what, g.shape, ref.shape)
    assert not np.isnan(g).any(), f"{what}: NaN"
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    err = np.abs(g - ref)
    rel_rms = float(np.sqrt(np.mean(err ** 2))) / max(rms, 1e-30)
    assert rel_rms <= 1e-2, f"{what}: RMS error {rel_rms:.2e} of the reference RMS"
    bound = 0.1 * rms + 1e-2 * np.abs(ref)
    bad = err > bound
    if bad.any():
        idx = np.argwhere(bad)[:5].tolist()
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} out of tolerance, first "
                             f"{idx}, max err {err.max():.3e}, rms(ref) {rms:.3e}")
    return float(err.max() / max(rms, 1e-30))


def bwd_case(B, Sq, Skv, Hq, Hkv, D, *, dtype=torch.bfloat16, causal=True, scale=None, seed=0,
             what=""):
    say(f"bwd {what} B={B} Sq={Sq} Skv={Skv} Hq={Hq} Hkv={Hkv} D={D} {dtype} causal={causal} "
        f"scale={scale}")
    q, k, v = workloads.dense_inputs(B, Sq, Skv, Hq, Hkv, D, dtype=dtype, seed=seed)
    do = workloads.dense_inputs(B, Sq, Sq, Hq, Hkv, D, dtype=dtype, seed=seed + 1)[0]
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    o, lse = mi.attn_fwd_dense(qd, kd, vd, scale=scale, causal=causal)
    dq, dk, dv = mi.attn_bwd(qd, kd, vd, o, dod, lse, scale=scale, causal=causal)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attn_bwd(q, k, v, o.cpu(), do, lse.cpu(), scale=scale, causal=causal)
    return [check_grad(dq, rq, what + " dq"), check_grad(dk, rk, what + " dk"),
            check_grad(dv, rv, what + " dv")]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_causal_gqa_ragged(D, dtype):
    bwd_case(2, 200, 200, 8, 2, D, dtype=dtype, seed=400, what="causal")


def test_noncausal_rectangular():
    bwd_case(2, 70, 300, 6, 3, 128, causal=False, seed=401, what="noncausal")


def test_causal_fewer_queries_than_keys():
    bwd_case(1, 90, 333, 8, 8, 64, seed=402, what="chunk")


def test_causal_rows_that_see_nothing():
    # Sq > Skv: the first rows have lse = -inf and contribute nothing
    bwd_case(1, 150, 100, 4, 2, 128, seed=403, what="empty_rows")


@pytest.mark.parametrize("scale", [0.3, -0.2])
def test_explicit_scales(scale):
    bwd_case(1, 64, 64, 4, 1, 64, scale=scale, seed=404, what=f"scale{scale}")


def test_group_of_eight_many_blocks():
    bwd_case(1, 520, 520, 16, 2, 128, seed=405, what="g8")


def test_is_deterministic():
    say("bwd twice, same bits")
    q, k, v = workloads.dense_inputs(1, 300, 300, 8, 2, 128, seed=406)
    do = workloads.dense_inputs(1, 300, 300, 8, 2, 128, seed=407)[0]
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    o, lse = mi.attn_fwd_dense(qd, kd, vd)
    a = mi.attn_bwd(qd, kd, vd, o, dod, lse)
    b = mi.attn_bwd(qd, kd, vd, o, dod, lse)
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(a, b))


def test_larger_causal_gqa():
    bwd_case(1, 1024, 1024, 16, 4, 128, seed=408, what="s1024")


@pytest.mark.parametrize("Sq,Skv", [(0, 40), (40, 0)])
def test_empty_side_gives_zero_gradients(Sq, Skv):
    # no query: dk = dv = 0; no key: dq = 0 (written by a fill kernel, over
    # whatever the allocator handed out, several calls in a row)
    say(f"bwd empty side Sq={Sq} Skv={Skv}")
    q, k, v = workloads.dense_inputs(2, max(Sq, 1), max(Skv, 1), 4, 2, 64, seed=404)
    q, k, v = q[:, :Sq].to(DEV), k[:, :Skv].to(DEV), v[:, :Skv].to(DEV)
    o = torch.zeros_like(q)
    lse = torch.full((2, 4, Sq), float("-inf"), device=DEV)
    for _ in range(3):
        torch.empty(1 << 24, dtype=torch.uint8, device=DEV).fill_(0xFF)  # recycle dirty memory
        dq, dk, dv = mi.attn_bwd(q, k, v, o, q, lse)
        torch.cuda.synchronize()
        for g in (dq, dk, dv):
            assert g.numel() == 0 or bool((g == 0).all())
