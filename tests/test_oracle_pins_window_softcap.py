"""Pins of the oracle's sliding window and logit softcap.

Sources on the pages: TileOPs "Attention Operators", GQADenseFwdOp stage 5
(visible iff (not causal or j <= p_i) and (w_L = -1 or j >= p_i - w_L) and
(w_R = -1 or j <= p_i + w_R)) and stage 6 (logit c tanh(Z / c) for a softcap
c > 0, Z for c = 0, -inf for hidden keys); the init parameters (-1 = an
unlimited window side; None or 0 disables the cap; a negative cap is an
error); GQAPagedFwdOp takes the same two parameters per request.

None of these re-types the oracle's visibility test or its logit line: a
windowed row is compared with the plain (window-free, non-causal) oracle on
the slice of keys the window admits, special cases have closed forms computed
here with math.tanh, and a torch fp64 reference builds the band from
triangular masks.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from softmax_attention_amd import workloads


def f64(x: torch.Tensor) -> np.ndarray:
    return x.to(torch.float64).numpy()


def admitted(p, Skv, causal, wl, wr):
    """Keys [lo, hi] a query at position p may see, before the padding mask."""
    lo = 0 if wl == -1 else max(0, p - wl)
    hi = Skv - 1
    if causal:
        hi = min(hi, p)
    if wr != -1:
        hi = min(hi, p + wr)
    return lo, hi


CASES = [  # Sq, Skv, causal, (w_L, w_R), masked
    (9, 9, True, (3, -1), False),
    (9, 9, True, (0, -1), False),
    (5, 13, True, (4, 2), False),     # w_R is inert under the causal rule
    (7, 12, False, (2, 3), False),
    (7, 12, False, (-1, 0), False),
    (12, 7, False, (1, 1), False),    # Sq > Skv: some rows see nothing
    (6, 11, False, (5, -1), True),
    (8, 8, True, (2, -1), True),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_windowed_row_equals_attention_over_its_key_slice(case):
    Sq, Skv, causal, (wl, wr), masked = CASES[case]
    B, Hq, Hkv, D = 2, 4, 2, 8
    q, k, v = workloads.dense_inputs(B, Sq, Skv, Hq, Hkv, D, seed=40 + case)
    mask = None
    if masked:
        mask = torch.rand(B, Skv, generator=torch.Generator().manual_seed(case)) > 0.3
    o, lse = oracle.attn_dense(q, k, v, causal=causal, window=(wl, wr), key_padding_mask=mask)
    n_empty = 0
    for b in range(B):
        for i in range(Sq):
            lo, hi = admitted(i + Skv - Sq, Skv, causal, wl, wr)
            keep = None if mask is None else mask[b:b + 1, lo:hi + 1]
            if hi < lo or (keep is not None and not bool(keep.any())):
                assert np.all(o[b, i] == 0) and np.all(lse[b, :, i] == -np.inf)
                n_empty += 1
                continue
            o_s, lse_s = oracle.attn_dense(q[b:b + 1, i:i + 1], k[b:b + 1, lo:hi + 1],
                                           v[b:b + 1, lo:hi + 1], causal=False,
                                           key_padding_mask=keep)
            # same visible keys in the same order: bitwise equal
            assert np.array_equal(o[b, i], o_s[0, 0])
            assert np.array_equal(lse[b, :, i], lse_s[0, :, 0])
    if Sq > Skv:
        assert n_empty > 0


def test_zero_left_window_returns_the_value_row_at_the_query_position():
    B, Sq, Skv, Hq, Hkv, D = 1, 6, 10, 4, 2, 8
    q, k, v = workloads.dense_inputs(B, Sq, Skv, Hq, Hkv, D, seed=50)
    o, lse = oracle.attn_dense(q, k, v, causal=True, window=(0, -1), scale=0.5)
    qf, kf, vf = f64(q), f64(k), f64(v)
    for i in range(Sq):
        p = i + Skv - Sq
        for h in range(Hq):
            assert np.array_equal(o[0, i, h], vf[0, p, h // 2])
            z = 0.5 * float(np.dot(qf[0, i, h], kf[0, p, h // 2]))
            assert lse[0, h, i] == pytest.approx(z, rel=1e-15, abs=1e-15)


def test_zero_right_window_without_causal_equals_causal():
    q, k, v = workloads.dense_inputs(2, 5, 9, 4, 1, 8, seed=51)
    o_c, lse_c = oracle.attn_dense(q, k, v, causal=True)
    o_w, lse_w = oracle.attn_dense(q, k, v, causal=False, window=(-1, 0))
    assert np.array_equal(o_c, o_w) and np.array_equal(lse_c, lse_w)


def test_windows_wider_than_the_sequence_change_nothing():
    q, k, v = workloads.dense_inputs(2, 6, 9, 4, 2, 8, seed=52)
    for causal in (True, False):
        o, lse = oracle.attn_dense(q, k, v, causal=causal)
        o_w, lse_w = oracle.attn_dense(q, k, v, causal=causal, window=(9, 9))
        assert np.array_equal(o, o_w) and np.array_equal(lse, lse_w)
    # a window that admits fewer keys does change the result: row 0 sits at
    # p = 3, and w_L = 2 drops its key 0
    o, _ = oracle.attn_dense(q, k, v, causal=False)
    o_w, _ = oracle.attn_dense(q, k, v, causal=False, window=(2, -1))
    assert not np.array_equal(o[:, 0], o_w[:, 0])


def test_paged_window_sits_at_each_requests_own_position():
    B, Sq, Hq, Hkv, D, ps = 3, 3, 4, 2, 8, 16
    cap = 48
    q, kd, vd = workloads.dense_inputs(B, Sq, cap, Hq, Hkv, D, seed=53)
    bt = torch.randperm(12, generator=torch.Generator().manual_seed(6))[:B * 3].view(B, 3)
    bt = bt.to(torch.int32)
    kc = workloads.scatter_to_pages(kd, bt, ps, 12, fill=float("nan"))
    vc = workloads.scatter_to_pages(vd, bt, ps, 12, fill=float("nan"))
    lens = torch.tensor([40, 3, 21], dtype=torch.int32)
    for causal, win in ((True, (5, -1)), (False, (2, 1))):
        o_p, lse_p = oracle.attn_paged(q, kc, vc, lens, bt, ps, causal=causal, window=win,
                                       softcap=7.5)
        for b in range(B):
            L = int(lens[b])
            o_d, lse_d = oracle.attn_dense(q[b:b + 1], kd[b:b + 1, :L], vd[b:b + 1, :L],
                                           causal=causal, window=win, softcap=7.5)
            assert np.array_equal(o_p[b:b + 1], o_d) and np.array_equal(lse_p[b:b + 1], lse_d)


# ---------------------------------------------------------------- softcap


def small_int_inputs(shape_q, shape_kv, seed):
    rng = np.random.default_rng(seed)
    mk = lambda s: torch.from_numpy(rng.integers(-3, 4, s).astype(np.float32)).to(torch.bfloat16)
    return mk(shape_q), mk(shape_kv), mk(shape_kv)


@pytest.mark.parametrize("cap", [0.5, 3.0, 50.0])
def test_softcap_single_visible_key_has_the_capped_logit_as_lse(cap):
    q, k, v = small_int_inputs((1, 3, 2, 4), (1, 3, 1, 4), seed=60)
    o, lse = oracle.attn_dense(q, k, v, causal=True, scale=0.75, softcap=cap)
    qf, kf, vf = f64(q), f64(k), f64(v)
    for h in range(2):
        z = 0.75 * float(np.dot(qf[0, 0, h], kf[0, 0, 0]))
        assert lse[0, h, 0] == pytest.approx(cap * math.tanh(z / cap), rel=1e-15, abs=1e-15)
        assert np.array_equal(o[0, 0, h], vf[0, 0, 0])


@pytest.mark.parametrize("cap", [0.25, 2.0, 30.0])
def test_softcap_two_keys_closed_form(cap):
    q, k, v = small_int_inputs((1, 2, 3, 4), (1, 2, 3, 4), seed=61)
    o, lse = oracle.attn_dense(q, k, v, causal=True, scale=0.5, softcap=cap)
    qf, kf, vf = f64(q), f64(k), f64(v)
    for h in range(3):
        z = [0.5 * float(np.dot(qf[0, 1, h], kf[0, j, h])) for j in range(2)]
        L = [cap * math.tanh(x / cap) for x in z]
        top = max(L)
        den = sum(math.exp(x - top) for x in L)
        w = [math.exp(x - top) / den for x in L]
        assert lse[0, h, 1] == pytest.approx(top + math.log(den), rel=1e-14, abs=1e-14)
        np.testing.assert_allclose(o[0, 1, h], w[0] * vf[0, 0, h] + w[1] * vf[0, 1, h],
                                   rtol=1e-14, atol=1e-14)


def test_softcap_of_zero_scores_gives_the_mean():
    q, k, v = workloads.dense_inputs(1, 6, 6, 2, 1, 8, seed=62)
    o, lse = oracle.attn_dense(q, k, v, causal=True, scale=0.0, softcap=1.5)
    vf = f64(v)
    for i in range(6):
        np.testing.assert_allclose(o[0, i, 0], vf[0, :i + 1, 0].mean(axis=0), rtol=1e-14,
                                   atol=1e-15)
        assert lse[0, 0, i] == pytest.approx(math.log(i + 1), rel=1e-15)


def test_huge_softcap_approaches_no_cap():
    # c tanh(z / c) = z - z^3 / (3 c^2) + ...: at c = 1e6 the logits move by < 1e-10
    q, k, v = workloads.dense_inputs(2, 7, 7, 4, 2, 16, seed=63)
    o, lse = oracle.attn_dense(q, k, v, causal=True)
    o_c, lse_c = oracle.attn_dense(q, k, v, causal=True, softcap=1e6)
    np.testing.assert_allclose(o_c, o, rtol=0, atol=1e-9)
    np.testing.assert_allclose(lse_c, lse, rtol=0, atol=1e-9)
    assert not np.array_equal(lse_c, lse)


def test_capped_logits_bound_the_lse():
    # every logit lies in [-c, c] (tanh rounds to +-1 for large scores), so
    # ln n - c <= lse <= ln n + c for n visible keys
    q, k, v = workloads.dense_inputs(1, 10, 10, 2, 1, 32, seed=64)
    q = q * 8
    cap = float(np.float32(0.8))  # the cap is passed as a float32
    _, lse = oracle.attn_dense(q, k, v, causal=True, softcap=cap)
    for i in range(10):
        n = math.log(i + 1)
        assert n - cap - 1e-15 <= lse[0, 0, i] <= n + cap + 1e-15


# ---------------------------------------------------------------- torch reference


def torch_band_reference(q, k, v, scale, causal, wl, wr, cap):
    """fp64 torch on the CPU: the window as a band of two triangular masks
    (diagonal offsets Skv - Sq - w_L and Skv - Sq + w_R), torch.tanh for the
    cap, torch.softmax / logsumexp for the rest."""
    qf = q.to(torch.float64).transpose(1, 2)
    kf = k.to(torch.float64).transpose(1, 2)
    vf = v.to(torch.float64).transpose(1, 2)
    g = qf.shape[1] // kf.shape[1]
    kf = kf.repeat_interleave(g, dim=1)
    vf = vf.repeat_interleave(g, dim=1)
    Sq, Skv = qf.shape[2], kf.shape[2]
    z = torch.matmul(qf, kf.transpose(-1, -2).contiguous()) * scale
    if cap:
        z = cap * torch.tanh(z / cap)
    ones = torch.ones(Sq, Skv, dtype=torch.bool)
    keep = ones.clone()
    if causal:
        keep &= torch.tril(ones, diagonal=Skv - Sq)
    if wr != -1:
        keep &= torch.tril(ones, diagonal=Skv - Sq + wr)
    if wl != -1:
        keep &= torch.triu(ones, diagonal=Skv - Sq - wl)
    z = z.masked_fill(~keep, float("-inf"))
    return (torch.matmul(torch.softmax(z, dim=-1), vf).transpose(1, 2).numpy(),
            torch.logsumexp(z, dim=-1).numpy())


@pytest.mark.parametrize("Sq,Skv,causal,wl,wr,cap", [(16, 16, True, 5, -1, 20.0),
                                                     (8, 24, True, 3, 0, 0.0),
                                                     (12, 20, False, 4, 6, 5.0),
                                                     (20, 20, False, -1, 2, 1.0)])
def test_matches_torch_band_reference(Sq, Skv, causal, wl, wr, cap):
    q, k, v = workloads.dense_inputs(2, Sq, Skv, 4, 2, 16, seed=65)
    o, lse = oracle.attn_dense(q, k, v, scale=0.25, causal=causal, window=(wl, wr),
                               softcap=cap)
    o_t, lse_t = torch_band_reference(q, k, v, 0.25, causal, wl, wr, cap)
    ok = np.isfinite(lse_t)
    assert np.array_equal(np.isfinite(lse), ok)
    np.testing.assert_allclose(lse[ok], lse_t[ok], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(o[ok.transpose(0, 2, 1)], o_t[ok.transpose(0, 2, 1)],
                               rtol=1e-12, atol=1e-12)


def test_invalid_window_and_cap_are_rejected():
    q, k, v = workloads.dense_inputs(1, 2, 2, 2, 1, 8, seed=66)
    for kw in (dict(window=(-2, -1)), dict(window=(-1, -3)), dict(softcap=-1.0),
               dict(softcap=float("nan")), dict(softcap=float("inf"))):
        with pytest.raises(ValueError):
            oracle.attn_dense(q, k, v, **kw)
