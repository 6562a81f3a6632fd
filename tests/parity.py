"""Comparison rule between the HIP path and the fp64 oracle.

Floating point: |o - o_ref| <= 1e-2 + 1e-2 |o_ref| for the 16-bit output
(converted exactly to double) and |lse - lse_ref| <= 2e-3.  Special values
match exactly: where the oracle's row is empty (lse_ref = -inf) the HIP path
must return lse = -inf and o = +-0, where a +inf sink takes the row (lse_ref =
+inf) lse = +inf and o = +-0; no NaN anywhere.
"""
from __future__ import annotations

import numpy as np
import torch

O_ATOL = 1e-2
O_RTOL = 1e-2
LSE_ATOL = 2e-3


def to_np64(x: torch.Tensor) -> np.ndarray:
    return x.detach().to("cpu").to(torch.float64).numpy()


def check_rows(o: np.ndarray, lse: np.ndarray, o_ref: np.ndarray, lse_ref: np.ndarray,
               what: str = "") -> dict:
    """o/o_ref [..., D], lse/lse_ref [...] (matching leading shapes)."""
    assert o.shape == o_ref.shape, (o.shape, o_ref.shape)
    assert lse.shape == lse_ref.shape, (lse.shape, lse_ref.shape)
    assert not np.isnan(o).any(), f"{what}: NaN in o"
    assert not np.isnan(lse).any(), f"{what}: NaN in lse"
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), empty), \
        f"{what}: -inf LSE pattern differs ({int(np.isneginf(lse).sum())} vs {int(empty.sum())})"
    assert np.all(o[empty] == 0.0), f"{what}: empty rows must output zeros"
    # a +inf sink takes all the weight: +inf LSE and zero output, exactly
    full = np.isposinf(lse_ref)
    assert np.array_equal(np.isposinf(lse), full), f"{what}: +inf LSE pattern differs"
    assert np.all(o[full] == 0.0), f"{what}: rows with a +inf sink must output zeros"
    err_o = np.abs(o - o_ref)
    bound = O_ATOL + O_RTOL * np.abs(o_ref)
    bad = err_o > bound
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} o elements out of tolerance; first "
                             f"{idx.tolist()}; max err {float(err_o.max()):.3e}")
    fin = np.isfinite(lse_ref)
    err_l = np.abs(lse[fin] - lse_ref[fin])
    if err_l.size and err_l.max() > LSE_ATOL:
        raise AssertionError(f"{what}: lse max err {float(err_l.max()):.3e} > {LSE_ATOL}")
    return {"max_err_o": float(err_o.max()) if err_o.size else 0.0,
            "max_err_lse": float(err_l.max()) if err_l.size else 0.0,
            "empty_rows": int(empty.sum())}


def check_full(o_gpu: torch.Tensor, lse_gpu: torch.Tensor, o_ref: np.ndarray,
               lse_ref: np.ndarray, what: str = "") -> dict:
    """Whole outputs: o [B,Sq,Hq,D], lse [B,Hq,Sq]."""
    o = to_np64(o_gpu)
    lse = lse_gpu.detach().cpu().numpy().astype(np.float64)
    # put lse in [B, Sq, Hq] order so empty-row masks line up with o
    return check_rows(o, lse.transpose(0, 2, 1), o_ref, lse_ref.transpose(0, 2, 1), what)


def check_sampled(o_gpu: torch.Tensor, lse_gpu: torch.Tensor, rows, o_ref: np.ndarray,
                  lse_ref: np.ndarray, what: str = "") -> dict:
    """Selected rows (b, i, h) against oracle rows o_ref [n, D], lse_ref [n]."""
    rows = np.asarray(rows, dtype=np.int64).reshape(-1, 3)
    b, i, h = rows[:, 0], rows[:, 1], rows[:, 2]
    oc = o_gpu.detach().cpu()
    o = to_np64(oc[torch.from_numpy(b), torch.from_numpy(i), torch.from_numpy(h)])
    lse_all = lse_gpu.detach().cpu().numpy().astype(np.float64)
    lse = lse_all[b, h, i]
    return check_rows(o, lse, o_ref, lse_ref, what)
