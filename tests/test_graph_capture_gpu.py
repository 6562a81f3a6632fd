"""HIP-graph capture of the library's calls: a torch.cuda.CUDAGraph records
the paged decode (stream-K attention + merge), a dense causal prefill, the
FP8-pool decode and the backward on one stream, and every replay -- with the
program's own eager work and synchronisations in between, and new inputs
copied into the captured buffers -- must give the eager call's bits.  (The
library allocates its workspace on a call's first use, so each shape runs
once eagerly before capture; its kernels record no memset nodes.)"""
import pytest
import torch

import softmax_attention_amd as mi
from softmax_attention_amd import workloads
from tests.test_parity_gpu import DEV, say

pytestmark = pytest.mark.gpu


def small_decode(seed):
    g = torch.Generator().manual_seed(seed)
    B, Hq, Hkv, D, ps, n_phys = 6, 16, 4, 128, 64, 64
    lens = torch.randint(1, 900, (B,), generator=g).to(torch.int32)
    bt = torch.randperm(n_phys, generator=g)[:B * 10].view(B, 10).to(torch.int32)
    q = torch.randn(B, 1, Hq, D, generator=g).to(torch.bfloat16)
    kc = torch.randn(n_phys * ps, Hkv, D, generator=g).to(torch.bfloat16)
    vc = torch.randn(n_phys * ps, Hkv, D, generator=g).to(torch.bfloat16)
    return [t.to(DEV) for t in (q, kc, vc, lens, bt)] + [ps]


def check_replays(run, inputs, fresh, n=3):
    """run() reads the tensors in `inputs` and returns outputs; fresh(i) gives
    new values for them.  Capture once, then replay n times against eager."""
    run()  # first use: workspace, occupancy queries
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            outs = run()
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    for i in range(n):
        for dst, src in zip(inputs, fresh(i)):
            dst.copy_(src)
        torch.empty(1 << 22, device=DEV).uniform_()  # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in outs]
        want = run()
        torch.cuda.synchronize()
        for a, b in zip(got, want):
            assert torch.equal(a, b), f"replay {i} differs from the eager call"


def test_graph_paged_decode():
    say("graph: paged decode")
    q, kc, vc, lens, bt, ps = small_decode(500)
    fresh = lambda i: [torch.randn_like(q.float(), generator=None).to(q.dtype)]
    check_replays(lambda: mi.attn_fwd_paged(q, kc, vc, lens, bt, ps), [q], fresh)


def test_graph_fp8_decode():
    say("graph: FP8 pool decode")
    q, kc, vc, lens, bt, ps = small_decode(501)
    k8, v8 = kc.to(torch.float8_e4m3fn), vc.to(torch.float8_e4m3fn)
    ks = torch.tensor([0.5], device=DEV)
    vs = torch.tensor([2.0], device=DEV)
    q3 = q.reshape(q.shape[0], q.shape[2], q.shape[3]).contiguous()
    cu = torch.arange(0, q3.shape[0] + 1, dtype=torch.int32, device=DEV)
    fresh = lambda i: [torch.randn_like(q3.float()).to(q3.dtype)]
    check_replays(lambda: mi.attn_fwd_paged_varlen(q3, k8, v8, lens, bt, cu, ps, max_seqlen_q=1,
                                                   k_scale=ks, v_scale=vs), [q3], fresh)


def test_graph_prefill_and_backward():
    say("graph: dense prefill + backward")
    q, k, v = (t.to(DEV) for t in workloads.dense_inputs(1, 300, 300, 8, 2, 128, seed=502))
    do = workloads.dense_inputs(1, 300, 300, 8, 2, 128, seed=503)[0].to(DEV)

    def run():
        o, lse = mi.attn_fwd_dense(q, k, v, causal=True)
        dq, dk, dv = mi.attn_bwd(q, k, v, o, do, lse, causal=True)
        return [o, lse, dq, dk, dv]

    fresh = lambda i: [torch.randn_like(q.float()).to(q.dtype), torch.randn_like(do.float()).to(do.dtype)]
    check_replays(run, [q, do], fresh)


def big_decode(seed):
    # more requests and a longer cache than small_decode: needs a larger
    # split-KV workspace than anything before it
    g = torch.Generator().manual_seed(seed)
    B, Hq, Hkv, D, ps, n_phys = 64, 32, 8, 128, 64, 1200
    lens = torch.randint(500, 1200, (B,), generator=g).to(torch.int32)
    bt = torch.randint(0, n_phys, (B, 19), generator=g).to(torch.int32)
    q = torch.randn(B, 1, Hq, D, generator=g).to(torch.bfloat16)
    kc = torch.randn(n_phys * ps, Hkv, D, generator=g).to(torch.bfloat16)
    vc = torch.randn(n_phys * ps, Hkv, D, generator=g).to(torch.bfloat16)
    return [t.to(DEV) for t in (q, kc, vc, lens, bt)] + [ps]


def test_graph_replays_after_the_workspace_grew():
    # a graph captured while the workspace was small keeps its address; an
    # eager call that grows the workspace must not free it under the graph
    say("graph: replay after the workspace grew")
    mi.release_workspace()
    q, kc, vc, lens, bt, ps = small_decode(504)
    run = lambda: mi.attn_fwd_paged(q, kc, vc, lens, bt, ps)
    want = [t.clone() for t in run()]
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            outs = run()
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    bq, bkc, bvc, blens, bbt, bps = big_decode(505)
    for i in range(3):
        big = mi.attn_fwd_paged(bq, bkc, bvc, blens, bbt, bps)  # grows the workspace (once)
        torch.cuda.synchronize()
        torch.empty(1 << 24, dtype=torch.uint8, device=DEV).fill_(0xFF)  # reuse freed memory
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, want):
            assert torch.equal(a, b), f"replay {i} after growth differs from the eager call"
        assert not torch.isnan(big[0]).any()


def test_calls_on_two_streams_share_the_workspace_safely():
    # two decode calls in flight on two streams at once: the second waits for
    # the first's use of the workspace, so each equals its single-stream result
    say("workspace shared by two streams")
    a = small_decode(506)
    b = big_decode(507)
    ref_a = [t.clone() for t in mi.attn_fwd_paged(*a)]
    ref_b = [t.clone() for t in mi.attn_fwd_paged(*b)]
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    for i in range(4):
        with torch.cuda.stream(s1):
            out_b = mi.attn_fwd_paged(*b)
        with torch.cuda.stream(s2):
            out_a = mi.attn_fwd_paged(*a)
        torch.cuda.synchronize()
        for x, y in zip(out_a, ref_a):
            assert torch.equal(x, y), f"round {i}: stream 2's call differs"
        for x, y in zip(out_b, ref_b):
            assert torch.equal(x, y), f"round {i}: stream 1's call differs"
