"""The allocation-free paged entry point (attn_fwd_paged_noalloc): the same
kernels as attn_fwd_paged with the split-KV partials in the library's fixed
per-GPU scratch.  Its outputs must equal attn_fwd_paged's (bitwise: same
kernels, same plan) and the oracle's (the parity rule), on two calls in a row
of which the second is smaller; a call beyond the scratch is refused; and the
call can be captured in a HIP graph with no eager call before it."""
import pytest
import torch

import oracle
import softmax_attention_amd as mi
from softmax_attention_amd import workloads
from tests.parity import check_full

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(msg):
    print(f"[case] {msg}", flush=True)


def decode_inputs(B, Hq, Hkv, D, page, lens, seed, dtype=torch.bfloat16, Sq=1):
    g = torch.Generator().manual_seed(seed)
    max_pages = max(1, -(-max(lens) // page))
    n_phys = B * max_pages + 2
    bt = torch.randperm(n_phys, generator=g)[:B * max_pages].view(B, max_pages).to(torch.int32)
    q = torch.randn(B, Sq, Hq, D, generator=g).to(dtype)
    kc = torch.randn(n_phys * page, Hkv, D, generator=g).to(dtype)
    vc = torch.randn(n_phys * page, Hkv, D, generator=g).to(dtype)
    return q, kc, vc, torch.tensor(lens, dtype=torch.int32), bt, page


def check_against_both(inp, what):
    q, kc, vc, lens, bt, page = inp
    dq, dkc, dvc, dl, dbt = (t.to(DEV) for t in (q, kc, vc, lens, bt))
    o = torch.full_like(dq, float("nan"))
    lse = torch.full((q.shape[0], q.shape[2], q.shape[1]), float("nan"), device=DEV)
    mi.attn_fwd_paged_noalloc(dq, dkc, dvc, dl, dbt, page, out=o, lse=lse)
    o_ref_gpu, lse_ref_gpu = mi.attn_fwd_paged(dq, dkc, dvc, dl, dbt, page)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref_gpu) and torch.equal(lse, lse_ref_gpu), \
        f"{what}: differs from attn_fwd_paged"
    o_ref, lse_ref = oracle.attn_paged(q, kc, vc, lens, bt, page)
    stats = check_full(o, lse, o_ref, lse_ref, what)
    say(f"{what}: {stats}")


def test_noalloc_matches_paged_on_two_calls_the_second_smaller():
    g = torch.Generator().manual_seed(700)
    lens = torch.randint(1, 3000, (64,), generator=g).tolist()
    lens[5] = 0
    say("noalloc call 1: B=64 Hq=32 Hkv=8 D=128 page 64")
    check_against_both(decode_inputs(64, 32, 8, 128, 64, lens, 701), "noalloc big")
    say("noalloc call 2: B=5 Hq=16 Hkv=4 D=64 page 16")
    check_against_both(decode_inputs(5, 16, 4, 64, 16, [900, 1, 0, 37, 250], 702,
                                     dtype=torch.float16), "noalloc small")


def test_noalloc_chunked_prefill_split_plan():
    # several queries per request: the split plan (fixed splits + merge), whose
    # partials also live in the scratch
    say("noalloc chunked prefill, split plan")
    check_against_both(decode_inputs(3, 8, 2, 128, 64, [700, 40, 1500], 703, Sq=16),
                       "noalloc chunked")


def test_noalloc_refuses_a_call_beyond_its_scratch():
    # 2048 requests x 8 KV heads of partials need more than the 32 MiB
    say("noalloc refusal beyond the scratch")
    B, Hq, Hkv, D, page = 2048, 32, 8, 128, 64
    q = torch.zeros(B, 1, Hq, D, dtype=torch.bfloat16, device=DEV)
    kc = torch.zeros(page, Hkv, D, dtype=torch.bfloat16, device=DEV)
    lens = torch.ones(B, dtype=torch.int32, device=DEV)
    bt = torch.zeros(B, 1, dtype=torch.int32, device=DEV)
    o = torch.full_like(q, 7.0)
    with pytest.raises(ValueError, match="scratch"):
        mi.attn_fwd_paged_noalloc(q, kc, kc, lens, bt, page, out=o, lse=None)
    torch.cuda.synchronize()
    assert bool((o == 7.0).all()), "a refused call must enqueue nothing"


def test_noalloc_captures_without_a_prior_call():
    # no workspace to grow: the very first call can sit in a captured graph;
    # replays with fresh queries (and eager work between them) match eager calls
    say("noalloc under graph capture")
    q, kc, vc, lens, bt, page = (t.to(DEV) if isinstance(t, torch.Tensor) else t
                                 for t in decode_inputs(7, 16, 4, 128, 64,
                                                        [300, 5, 1200, 64, 65, 0, 999], 704))
    o = torch.empty_like(q)
    lse = torch.empty((q.shape[0], q.shape[2], 1), device=DEV)
    graph = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            mi.attn_fwd_paged_noalloc(q, kc, vc, lens, bt, page, out=o, lse=lse)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    g = torch.Generator().manual_seed(705)
    for i in range(3):
        q.copy_(torch.randn(q.shape, generator=g).to(q.dtype))
        torch.empty(1 << 22, device=DEV).uniform_()
        graph.replay()
        torch.cuda.synchronize()
        want_o, want_l = mi.attn_fwd_paged(q, kc, vc, lens, bt, page)
        torch.cuda.synchronize()
        assert torch.equal(o, want_o) and torch.equal(lse, want_l), f"replay {i} differs"
