"""A seeded sweep of GPU parity cases against the fp64 oracle, beyond the
hand-picked ones: random group sizes (1 to 16), head dims, dtypes, lengths
with ragged tails, causal or not, windows, softcaps, padding masks, page sizes,
packed requests, FP8 pools and the backward, each drawn from a fixed seed so
that a failure names a reproducible case.  The comparison rules are
tests/parity.py's (forward) and the backward tests' (gradients)."""
import numpy as np
import pytest
import torch

from tests.test_parity_gpu import _reset_split, dense_case, padding_mask, paged_case
from tests.test_parity_gpu_bwd import bwd_case
from tests.test_parity_gpu_fp8_cache import fp8_case
from tests.test_parity_gpu_varlen_sinks import make_sinks, paged_varlen_case, varlen_case

pytestmark = pytest.mark.gpu

__all__ = ["_reset_split"]  # the autouse fixture that restores the split plan

GROUPS = [(4, 4), (8, 2), (12, 4), (6, 2), (16, 1), (5, 5), (8, 8), (16, 2)]


def draw(seed):
    rng = np.random.default_rng(seed)
    Hq, Hkv = GROUPS[rng.integers(len(GROUPS))]
    D = int(rng.choice([64, 128, 256], p=[0.4, 0.45, 0.15]))
    dtype = torch.bfloat16 if rng.random() < 0.6 else torch.float16
    causal = bool(rng.random() < 0.7)
    window = None
    if rng.random() < 0.35:
        window = (int(rng.integers(-1, 200)), int(rng.integers(-1, 60)) if not causal else -1)
    softcap = float(rng.choice([10.0, 30.0])) if rng.random() < 0.3 else None
    return rng, Hq, Hkv, D, dtype, causal, window, softcap


@pytest.mark.parametrize("seed", range(40))
def test_sweep_dense(seed):
    rng, Hq, Hkv, D, dtype, causal, window, softcap = draw(1000 + seed)
    B = int(rng.integers(1, 4))
    Sq = int(rng.integers(1, 300))
    Skv = int(rng.integers(1, 400)) if rng.random() < 0.5 else Sq
    mask = None
    if rng.random() < 0.3:
        mask = padding_mask(B, Skv, [int(x) for x in rng.integers(0, Skv + 1, B)])
    split = int(rng.choice([0, 0, 64, 128]))
    dense_case(B, Sq, Skv, Hq, Hkv, D, dtype=dtype, causal=causal, mask=mask, window=window,
               softcap=softcap, split_keys=split, seed=seed, what=f"sweep{seed}")


@pytest.mark.parametrize("seed", range(30))
def test_sweep_paged(seed):
    rng, Hq, Hkv, D, dtype, causal, window, softcap = draw(2000 + seed)
    B = int(rng.integers(1, 6))
    Sq = int(rng.choice([1, 1, 3, 40]))
    lens = [int(x) for x in rng.integers(Sq, 1500, B)]
    page = int(rng.choice([16, 32, 64, 128]))
    split = int(rng.choice([0, 0, 128]))
    paged_case(B, Sq, Hq, Hkv, D, lens, page, dtype=dtype, causal=causal, window=window,
               softcap=softcap, split_keys=split, seed=seed, what=f"sweep{seed}")


@pytest.mark.parametrize("seed", range(30))
def test_sweep_varlen(seed):
    rng, Hq, Hkv, D, dtype, causal, window, softcap = draw(3000 + seed)
    n = int(rng.integers(1, 6))
    sq = [int(x) for x in rng.integers(0, 90, n)]
    skv = [int(x) for x in rng.integers(0, 300, n)]
    sinks = make_sinks(Hq, 3000 + seed) if rng.random() < 0.5 else None
    if rng.random() < 0.5:
        varlen_case(sq, skv, Hq, Hkv, D, dtype=dtype, causal=causal, window=window,
                    softcap=softcap, sinks=sinks, seed=seed, what=f"sweep{seed}")
    else:
        lens = [max(a, b) for a, b in zip(sq, skv)]
        page = int(rng.choice([16, 64]))
        paged_varlen_case(sq, lens, Hq, Hkv, D, page, dtype=dtype, causal=causal, window=window,
                          softcap=softcap, sinks=sinks, seed=seed, what=f"sweep{seed}")


@pytest.mark.parametrize("seed", range(12))
def test_sweep_fp8_pools(seed):
    rng, Hq, Hkv, D, dtype, causal, window, softcap = draw(4000 + seed)
    D = 64 if D == 64 else 128  # FP8 pools: D = 64 or 128
    n = int(rng.integers(1, 7))
    sq = [int(x) for x in rng.integers(0, 3, n)] if rng.random() < 0.6 else \
        [int(x) for x in rng.integers(0, 50, n)]
    lens = [max(s_, int(x)) for s_, x in zip(sq, rng.integers(0, 2500, n))]
    page = int(rng.choice([16, 32, 64]))
    # pool scales as a quantizer would pick them (codes of sigma 40 dequantize to
    # values of sigma 0.4 to 2): the comparison rule's absolute term assumes
    # O(1) values, as the 16-bit cases have
    ks, vs = float(rng.uniform(0.01, 0.05)), float(rng.uniform(0.01, 0.05))
    split = int(rng.choice([0, 0, 256]))
    fp8_case(sq, lens, Hq, Hkv, D, page, dtype=dtype, causal=causal, window=window,
             softcap=softcap, split_keys=split, ks=ks, vs=vs, seed=4000 + seed,
             what=f"sweep{seed}")


@pytest.mark.parametrize("seed", range(8))
def test_sweep_backward(seed):
    rng = np.random.default_rng(5000 + seed)
    Hq, Hkv = GROUPS[rng.integers(len(GROUPS))]
    D = int(rng.choice([64, 128]))
    dtype = torch.bfloat16 if rng.random() < 0.6 else torch.float16
    causal = bool(rng.random() < 0.7)
    B = int(rng.integers(1, 3))
    Sq = int(rng.integers(1, 260))
    Skv = int(rng.integers(1, 260)) if rng.random() < 0.4 else Sq
    bwd_case(B, Sq, Skv, Hq, Hkv, D, dtype=dtype, causal=causal, seed=5000 + seed,
             what=f"sweep{seed}")
