"""Pins of the oracle's attention backward (TileOPs "Attention Operators",
GQABwdOp: dq, dk, dv from q, k, v, o, do and lse).

Independent checks: torch.autograd through a plain fp64 torch attention (a
library routine; with o and lse passed exactly, the gradients agree to
rounding), central finite differences of the oracle's own forward (which
shares no code path with its backward), closed forms for rows that see one key
or equal scores, and the GQA invariant that a KV head's gradient is the sum of
the MHA gradients of its query heads.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from softmax_attention_amd import workloads


def torch_forward(q, k, v, scale, causal):
    """fp64 torch attention on BSHD tensors with repeat_interleave GQA; returns
    (o [B,Sq,Hq,D], lse [B,Hq,Sq])."""
    Hq, Hkv = q.shape[2], k.shape[2]
    Sq, Skv = q.shape[1], k.shape[1]
    qh = q.transpose(1, 2)
    kh = k.transpose(1, 2).repeat_interleave(Hq // Hkv, dim=1)
    vh = v.transpose(1, 2).repeat_interleave(Hq // Hkv, dim=1)
    s = torch.matmul(qh, kh.transpose(-1, -2)) * scale
    if causal:
        hide = torch.triu(torch.ones(Sq, Skv, dtype=torch.bool), diagonal=Skv - Sq + 1)
        s = s.masked_fill(hide, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    return torch.matmul(torch.softmax(s, dim=-1), vh).transpose(1, 2), lse


def autograd_case(B, Sq, Skv, Hq, Hkv, D, causal, seed, scale=None):
    q, k, v = workloads.dense_inputs(B, Sq, Skv, Hq, Hkv, D, seed=seed)
    do = workloads.dense_inputs(B, Sq, Sq, Hq, Hkv, D, seed=seed + 1)[0]
    alpha = oracle.resolve_scale(scale, D)
    qf, kf, vf = (x.to(torch.float64).requires_grad_() for x in (q, k, v))
    o, lse = torch_forward(qf, kf, vf, alpha, causal)
    (o * do.to(torch.float64)).sum().backward()
    dq, dk, dv = oracle.attn_bwd(q, k, v, o.detach(), do, lse.detach(), scale=scale,
                                 causal=causal)
    return (dq, dk, dv), (qf.grad.numpy(), kf.grad.numpy(), vf.grad.numpy())


@pytest.mark.parametrize("B,Sq,Skv,Hq,Hkv,D,causal", [(2, 9, 9, 4, 2, 16, True),
                                                     (1, 6, 15, 6, 3, 8, True),
                                                     (2, 11, 7, 4, 4, 8, False),
                                                     (1, 12, 12, 8, 1, 32, True)])
def test_matches_torch_autograd(B, Sq, Skv, Hq, Hkv, D, causal):
    ours, ref = autograd_case(B, Sq, Skv, Hq, Hkv, D, causal, seed=90)
    for a, r in zip(ours, ref):
        np.testing.assert_allclose(a, r, rtol=1e-10, atol=1e-12)


def test_matches_torch_autograd_with_explicit_scale():
    ours, ref = autograd_case(1, 8, 8, 4, 2, 16, True, seed=91, scale=0.3)
    for a, r in zip(ours, ref):
        np.testing.assert_allclose(a, r, rtol=1e-10, atol=1e-12)


def test_central_differences_of_the_oracle_forward():
    # L = sum(O * dO) on the oracle's forward; q, k, v hold small integers /
    # 16 so that x +- 2^-6 stays exact in bf16.  Central differences are
    # exact up to the h^2 term.
    B, S, Hq, Hkv, D = 1, 5, 2, 1, 4
    rng = np.random.default_rng(92)
    mk = lambda shape: torch.from_numpy(rng.integers(-8, 9, shape).astype(np.float32) / 16)
    q, k, v = mk((B, S, Hq, D)), mk((B, S, Hkv, D)), mk((B, S, Hkv, D))
    do = mk((B, S, Hq, D)).to(torch.bfloat16)
    q, k, v = (x.to(torch.bfloat16) for x in (q, k, v))
    o, lse = oracle.attn_dense(q, k, v, scale=0.5, causal=True)
    dq, dk, dv = oracle.attn_bwd(q, k, v, o, do, lse, scale=0.5, causal=True)
    dof = do.to(torch.float64).numpy()
    h = 2.0 ** -6

    def loss(q_, k_, v_):
        return float((oracle.attn_dense(q_, k_, v_, scale=0.5, causal=True)[0] * dof).sum())

    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for idx in [(0, 2, 0, 1), (0, 4, x.shape[2] - 1, 3), (0, 0, 0, 0)]:
            xp, xm = x.clone(), x.clone()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert g[idx] == pytest.approx(fd, rel=2e-3, abs=2e-4), (name, idx)


def test_row_that_sees_one_key_has_zero_dq():
    # causal row 0 sees key 0 only: P = 1, O = v_0, so dS = dO.v_0 - dO.o = 0
    q, k, v = workloads.dense_inputs(1, 6, 6, 2, 1, 16, seed=93)
    do = workloads.dense_inputs(1, 6, 6, 2, 1, 16, seed=94)[0]
    o, lse = oracle.attn_dense(q, k, v, causal=True)
    dq, _, _ = oracle.attn_bwd(q, k, v, o, do, lse, causal=True)
    assert np.all(np.abs(dq[0, 0]) < 1e-15)


def test_equal_scores_give_the_averaged_dv():
    # alpha = 0: P_ij = 1 / (i + 1) for j <= i, so dv_j = sum_{i >= j} dO_i / (i + 1)
    S, D = 7, 8
    q, k, v = workloads.dense_inputs(1, S, S, 1, 1, D, seed=95)
    do = workloads.dense_inputs(1, S, S, 1, 1, D, seed=96)[0]
    o, lse = oracle.attn_dense(q, k, v, scale=0.0, causal=True)
    _, dk, dv = oracle.attn_bwd(q, k, v, o, do, lse, scale=0.0, causal=True)
    dof = do.to(torch.float64).numpy()[0, :, 0]
    for j in range(S):
        want = sum(dof[i] / (i + 1) for i in range(j, S))
        np.testing.assert_allclose(dv[0, j, 0], want, rtol=1e-13, atol=1e-14)
    assert np.all(dk == 0)  # alpha = 0 multiplies every dk


def test_gqa_gradient_is_the_sum_over_its_query_heads():
    B, S, Hq, Hkv, D = 1, 8, 6, 2, 8
    q, k, v = workloads.dense_inputs(B, S, S, Hq, Hkv, D, seed=97)
    do = workloads.dense_inputs(B, S, S, Hq, Hkv, D, seed=98)[0]
    o, lse = oracle.attn_dense(q, k, v, causal=True)
    dq, dk, dv = oracle.attn_bwd(q, k, v, o, do, lse, causal=True)
    g = Hq // Hkv
    kr, vr = k.repeat_interleave(g, dim=2), v.repeat_interleave(g, dim=2)
    dq_m, dk_m, dv_m = oracle.attn_bwd(q, kr, vr, o, do, lse, causal=True)
    assert np.array_equal(dq, dq_m)
    np.testing.assert_allclose(dk, dk_m.reshape(B, S, Hkv, g, D).sum(axis=3), rtol=1e-13,
                               atol=1e-14)
    np.testing.assert_allclose(dv, dv_m.reshape(B, S, Hkv, g, D).sum(axis=3), rtol=1e-13,
                               atol=1e-14)


def test_rows_that_see_nothing_contribute_nothing():
    q, k, v = workloads.dense_inputs(1, 6, 3, 2, 1, 8, seed=99)  # Sq > Skv: rows 0-2 empty
    do = workloads.dense_inputs(1, 6, 6, 2, 1, 8, seed=100)[0]
    o, lse = oracle.attn_dense(q, k, v, causal=True)
    assert np.all(np.isneginf(lse[:, :, :3]))
    dq, dk, dv = oracle.attn_bwd(q, k, v, o, do, lse, causal=True)
    assert np.all(dq[0, :3] == 0)
    do2 = do.clone()
    do2[:, :3] = 0
    _, dk2, dv2 = oracle.attn_bwd(q, k, v, o, do2, lse, causal=True)
    assert np.array_equal(dk, dk2) and np.array_equal(dv, dv2)
