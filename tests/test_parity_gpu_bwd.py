"""GPU parity of the attention backward (TileOPs "Attention Operators",
GQABwdOp) against the fp64 oracle.

Inputs: q, k, v, do seeded; o and lse are the ORACLE's forward output, o
rounded to the dtype and lse to float32, and both the GPU and the oracle's
backward take exactly those tensors -- so a forward error cannot cancel a
backward one, and the comparison sees the backward's arithmetic alone.

Tolerance, derived from that arithmetic.  The GPU computes P = exp(alpha s -
lse), dP = dO.v, D_i = <dO_i, o_i> and dS = P (dP - D) in FP32, rounds P and
dS to the 16-bit dtype (unit roundoff u = 2^-8 for bf16, 2^-11 for fp16) as
MFMA operands, accumulates the products dv = P^T dO, dk = alpha dS^T q and
dq = alpha dS k in FP32, and rounds each gradient to the dtype.  Each summed
term thus carries a relative error of at most u from the operand rounding,
FP32 work adds errors far below 2^-14 of the magnitudes entering it, and the
final rounding adds u |g|.  Below the dtype's smallest normal value (2^-14
for fp16) a rounding error is bounded in absolute terms instead, by eta = half
the subnormal spacing (2^-25 for fp16, 2^-134 for bf16), once per rounded
operand and once for the output.  So, per element,

    |g - g_ref| <= u A_round + 2^-14 A_fp32 + eta (A_count + 1) + u |g_ref|,

with A_round the sum of the absolute values of the element's terms (e.g.
sum_i P_ij |dO_id| for dv), A_fp32 the same with |dS| replaced by
P (|dO|.|v| + |D|), which bounds the FP32 error of dS even where dP - D
cancels, and A_count the same with each rounded operand (P or dS) replaced
by 1 on the visible pairs.  These magnitudes are computed here in fp64 from
the same inputs (they set the bound only; the expected values are the
oracle's)."""
import numpy as np
import pytest
import torch

import oracle
import softmax_attention_amd as mi
from softmax_attention_amd import workloads
from tests.test_parity_gpu import DEV, say

pytestmark = pytest.mark.gpu

FP32_SLACK = 2.0 ** -14


def unit_roundoff(dtype):
    return 2.0 ** -8 if dtype == torch.bfloat16 else 2.0 ** -11


def subnormal_half_step(dtype):
    return 2.0 ** -134 if dtype == torch.bfloat16 else 2.0 ** -25


def term_magnitudes(q, k, v, o, do, lse, scale, causal):
    """(dq, dk, dv) term magnitudes: A_round, A_fp32 and A_count of each
    gradient element, fp64, in the BSHD layouts of the gradients."""
    B, Sq, Hq, D = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    alpha = oracle.resolve_scale(scale, D)
    f = lambda t: t.to(torch.float64).permute(0, 2, 1, 3).contiguous()  # BHSD
    qf, of, dof = f(q), f(o), f(do)
    kf = f(k).repeat_interleave(G, dim=1)
    vf = f(v).repeat_interleave(G, dim=1)
    lsef = lse.to(torch.float64)
    s = alpha * torch.matmul(qf, kf.transpose(-1, -2).contiguous())
    i = torch.arange(Sq)[:, None]
    j = torch.arange(Skv)[None, :]
    vis = (j <= i + Skv - Sq) if causal else torch.ones(Sq, Skv, dtype=torch.bool)
    arg = s - lsef[..., None]
    live = vis & torch.isfinite(lsef)[..., None]
    P = torch.where(live, torch.exp(arg), torch.zeros_like(s))
    ones = live.to(torch.float64)
    dP = torch.matmul(dof, vf.transpose(-1, -2).contiguous())
    Drow = (dof * of).sum(-1)
    dS = P * (dP - Drow[..., None])
    dS_f32 = P * (torch.matmul(dof.abs(), vf.abs().transpose(-1, -2).contiguous())
                  + Drow.abs()[..., None])
    a = abs(alpha)

    def per_kv(x):  # [B, Hq, Skv, D] -> summed over each KV head's G query heads, BSHD
        return x.view(B, Hkv, G, Skv, D).sum(2).permute(0, 2, 1, 3).contiguous()

    dq_r = a * torch.matmul(dS.abs(), kf.abs())
    dq_f = a * torch.matmul(dS_f32, kf.abs())
    dk_r = per_kv(a * torch.matmul(dS.abs().transpose(-1, -2).contiguous(), qf.abs()))
    dk_f = per_kv(a * torch.matmul(dS_f32.transpose(-1, -2).contiguous(), qf.abs()))
    dv_r = per_kv(torch.matmul(P.transpose(-1, -2).contiguous(), dof.abs()))
    dq_c = a * torch.matmul(ones, kf.abs())
    dk_c = per_kv(a * torch.matmul(ones.transpose(-1, -2).contiguous(), qf.abs()))
    dv_c = per_kv(torch.matmul(ones.transpose(-1, -2).contiguous(), dof.abs()))
    bshd = lambda x: x.permute(0, 2, 1, 3).contiguous().numpy()
    return ((bshd(dq_r), bshd(dq_f), bshd(dq_c)), (dk_r.numpy(), dk_f.numpy(), dk_c.numpy()),
            (dv_r.numpy(), dv_r.numpy(), dv_c.numpy()))


def check_grad(g, ref, mags, u, eta, what):
    g = g.detach().cpu().to(torch.float64).numpy()
    assert g.shape == ref.shape, (what, g.shape, ref.shape)
    assert not np.isnan(g).any(), f"{what}: NaN"
    a_round, a_f32, a_count = mags
    err = np.abs(g - ref)
    bound = u * a_round + FP32_SLACK * a_f32 + eta * (a_count + 1.0) + u * np.abs(ref)
    bad = err > bound
    if bad.any():
        idx = np.argwhere(bad)[:5].tolist()
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} out of tolerance, first "
                             f"{idx}, max err {err.max():.3e}")
    # how much of the bound the worst element used
    return float(np.max(err / np.maximum(bound, 1e-300))) if err.size else 0.0


def bwd_case(B, Sq, Skv, Hq, Hkv, D, *, dtype=torch.bfloat16, causal=True, scale=None, seed=0,
             what=""):
    say(f"bwd {what} B={B} Sq={Sq} Skv={Skv} Hq={Hq} Hkv={Hkv} D={D} {dtype} causal={causal} "
        f"scale={scale}")
    q, k, v = workloads.dense_inputs(B, Sq, Skv, Hq, Hkv, D, dtype=dtype, seed=seed)
    do = workloads.dense_inputs(B, Sq, Sq, Hq, Hkv, D, dtype=dtype, seed=seed + 1)[0]
    # the oracle's forward, rounded as a forward call would hand it over
    o64, lse64 = oracle.attn_dense(q, k, v, scale=scale, causal=causal)
    o = torch.from_numpy(o64).to(dtype)
    lse = torch.from_numpy(np.ascontiguousarray(lse64)).to(torch.float32)
    dq, dk, dv = mi.attn_bwd(q.to(DEV), k.to(DEV), v.to(DEV), o.to(DEV), do.to(DEV),
                             lse.to(DEV), scale=scale, causal=causal)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attn_bwd(q, k, v, o, do, lse, scale=scale, causal=causal)
    mq, mk, mv = term_magnitudes(q, k, v, o, do, lse, scale, causal)
    u, eta = unit_roundoff(dtype), subnormal_half_step(dtype)
    used = [check_grad(dq, rq, mq, u, eta, what + " dq"),
            check_grad(dk, rk, mk, u, eta, what + " dk"),
            check_grad(dv, rv, mv, u, eta, what + " dv")]
    say(f"bwd {what}: worst element used {max(used):.2f} of its bound")
    return used


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


@pytest.mark.parametrize("causal", [True, False])
def test_more_key_blocks_than_cus(causal):
    # 64 KV heads x 5 key blocks = 320 dk/dv workgroups: the first wave (one
    # per CU) walks its row tiles down, the rest walk up; G = 3 makes a tile
    # step cross head boundaries in both directions
    bwd_case(1, 40, 600, 192, 64, 64, causal=causal, seed=409, what=f"waves causal={causal}")


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
