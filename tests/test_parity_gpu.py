"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Every case runs the same seeded inputs through libmiattn on the GPU and
through the CPU oracle, and applies the comparison rule in tests/parity.py.
Small cases span several key tiles, several row blocks and a ragged tail and
are compared element by element; the five full-size workloads run in the
launch configuration the benchmark times and are compared element by element
on every output row too (the oracle runs them whole, on all host threads).
"""
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


@pytest.fixture(autouse=True)
def _reset_split():
    mi.set_split_keys(0)
    yield
    mi.set_split_keys(0)


def run_dense(q, k, v, *, scale, causal, mask=None, window=None, softcap=None):
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    md = None if mask is None else mask.to(DEV)
    o, lse = mi.attn_fwd_dense(qd, kd, vd, scale=scale, causal=causal, key_padding_mask=md,
                               window=window, softcap=softcap)
    torch.cuda.synchronize()
    return o, lse


def dense_case(B, Sq, Skv, Hq, Hkv, D, *, dtype=torch.bfloat16, causal=True, scale=None,
               mask=None, seed=0, sigma=1.0, window=None, softcap=None, split_keys=0, what=""):
    say(f"dense {what} B={B} Sq={Sq} Skv={Skv} Hq={Hq} Hkv={Hkv} D={D} {dtype} "
        f"causal={causal} scale={scale} mask={mask is not None} window={window} "
        f"softcap={softcap} split_keys={split_keys}")
    q, k, v = workloads.dense_inputs(B, Sq, Skv, Hq, Hkv, D, dtype=dtype, seed=seed, sigma=sigma)
    mi.set_split_keys(split_keys)
    o, lse = run_dense(q, k, v, scale=scale, causal=causal, mask=mask, window=window,
                       softcap=softcap)
    o_ref, lse_ref = oracle.attn_dense(q, k, v, scale=scale, causal=causal, key_padding_mask=mask,
                                       window=window, softcap=softcap)
    return check_full(o, lse, o_ref, lse_ref, what)


def padding_mask(B, Skv, lengths):
    return torch.arange(Skv)[None, :] < torch.tensor(lengths)[:, None]


# ---------------------------------------------------------------- dense


def test_tiny_workload_full():
    w = workloads.make(1)
    say(w.name)
    o, lse = run_dense(w.q, w.k, w.v, scale=w.scale, causal=w.causal)
    o_ref, lse_ref = oracle.attn_dense(w.q, w.k, w.v, scale=w.scale, causal=w.causal)
    check_full(o, lse, o_ref, lse_ref, w.name)


@pytest.mark.parametrize("D", [64, 128, 256])
def test_lse_of_a_row_dominated_by_one_key(D):
    # Every row sees one key at score 0 in the first key tile, one key at
    # score 3.46875 (2^(3.46875 log2 e) = 32.097 relative to the first tile's
    # max, below the lazy-max threshold, so that P is not 1) in the second,
    # and keys at -30 elsewhere.  Rounded to bf16, P = 32.097 becomes 32: a
    # denominator of rounded P would be 33 instead of 33.097 and the lse off
    # by 2.9e-3, beyond the 2e-3 bound.
    Skv, Sq = 260, 70
    q = torch.zeros(1, Sq, 2, D)
    q[..., 0] = 1.0
    b = torch.full((Skv,), -30.0)
    b[0] = 0.0
    b[130] = 3.46875
    k = torch.zeros(1, Skv, 1, D)
    k[0, :, 0, 0] = b
    v = workloads.dense_inputs(1, 1, Skv, 1, 1, D, seed=41)[2]
    q, k = q.to(torch.bfloat16), k.to(torch.bfloat16)
    say(f"row dominated by one key D={D}")
    o, lse = run_dense(q, k, v, scale=1.0, causal=False)
    o_ref, lse_ref = oracle.attn_dense(q, k, v, scale=1.0, causal=False)
    check_full(o, lse, o_ref, lse_ref, f"dominant key D={D}")


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_dense_causal_gqa_ragged(D, dtype):
    # 300 rows x 4 heads = 1200 packed rows -> 10 row blocks, a ragged last one;
    # 300 keys -> a partial last key tile for every tile width
    dense_case(1, 300, 300, 8, 2, D, dtype=dtype, causal=True, seed=D, what="causal_gqa")


@pytest.mark.parametrize("D", [64, 128, 256])
def test_dense_noncausal_key_padding(D):
    mask = padding_mask(3, 333, [333, 1, 170])
    dense_case(3, 97, 333, 4, 4, D, dtype=torch.float16, causal=False, scale=0.125, mask=mask,
               seed=7, sigma=0.5, what="mha_padding")


def test_dense_causal_with_random_mask_and_empty_rows():
    g = torch.Generator().manual_seed(9)
    mask = torch.rand(2, 260, generator=g) > 0.7
    mask[1, :] = False  # batch 1: every row empty
    mask[0, 0] = False  # causal row 0 of batch 0 sees only key 0: empty too
    dense_case(2, 260, 260, 6, 3, 128, causal=True, mask=mask, seed=10, what="random_mask")


@pytest.mark.parametrize("Sq,Skv", [(1, 1000), (77, 500), (129, 129), (200, 64), (50, 0),
                                    (5, 3)])
def test_dense_rectangular_and_degenerate(Sq, Skv):
    # Sq < Skv: chunked prefill / decode rows; Sq > Skv: the first Sq - Skv
    # rows see no key; Skv = 0: every row is empty
    dense_case(2, Sq, Skv, 8, 2, 128, causal=True, seed=11, what="rect")


@pytest.mark.parametrize("scale", [0.0, -0.3, 2.5])
def test_dense_explicit_scales(scale):
    dense_case(1, 130, 130, 4, 1, 64, causal=True, scale=scale, seed=12, what="scale")


@pytest.mark.parametrize("G", [1, 4, 12, 16])
def test_dense_group_sizes(G):
    dense_case(1, 70, 150, 2 * G, 2, 128, causal=True, seed=13, what=f"group{G}")


@pytest.mark.parametrize("split_keys", [64, 256])
def test_dense_forced_split_matches_oracle(split_keys):
    mi.set_split_keys(split_keys)
    dense_case(2, 150, 700, 8, 2, 128, causal=True, seed=14, what=f"split{split_keys}")
    mask = padding_mask(2, 700, [650, 3])
    dense_case(2, 150, 700, 8, 2, 64, dtype=torch.float16, causal=False, mask=mask, seed=15,
               what=f"split{split_keys}_mask")


def test_dense_zero_batch_or_queries_is_a_no_op():
    q = torch.zeros(0, 4, 2, 64, dtype=torch.bfloat16, device=DEV)
    k = torch.zeros(0, 4, 2, 64, dtype=torch.bfloat16, device=DEV)
    o, lse = mi.attn_fwd_dense(q, k, k)
    assert o.shape == q.shape and lse.shape == (0, 2, 4)
    q = torch.zeros(1, 0, 2, 64, dtype=torch.bfloat16, device=DEV)
    k = torch.zeros(1, 4, 2, 64, dtype=torch.bfloat16, device=DEV)
    o, lse = mi.attn_fwd_dense(q, k, k)
    assert o.shape == q.shape


def test_dense_writes_exactly_its_output():
    # guard bands around o and lse stay untouched; every element is written
    say("guard bands")
    B, S, Hq, Hkv, D = 1, 190, 4, 2, 128
    q, k, v = workloads.dense_inputs(B, S, S, Hq, Hkv, D, seed=16)
    n_o = B * S * Hq * D
    guard = 4096
    obuf = torch.full((n_o + 2 * guard,), float("nan"), dtype=torch.bfloat16, device=DEV)
    lbuf = torch.full((B * Hq * S + 2 * guard,), float("nan"), dtype=torch.float32, device=DEV)
    o = obuf[guard:guard + n_o].view(B, S, Hq, D)
    lse = lbuf[guard:guard + B * Hq * S].view(B, Hq, S)
    inputs = [x.to(DEV) for x in (q, k, v)]
    before = [x.clone() for x in inputs]
    mi.attn_fwd_dense(*inputs, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.isnan(obuf[:guard]).all() and torch.isnan(obuf[guard + n_o:]).all()
    assert torch.isnan(lbuf[:guard]).all() and torch.isnan(lbuf[guard + B * Hq * S:]).all()
    assert not torch.isnan(o).any() and not torch.isnan(lse).any()
    for a, b in zip(inputs, before):
        assert torch.equal(a, b)
    o_ref, lse_ref = oracle.attn_dense(q, k, v)
    check_full(o, lse, o_ref, lse_ref, "guard")


def test_dense_is_deterministic():
    q, k, v = (x.to(DEV) for x in workloads.dense_inputs(2, 257, 257, 8, 2, 128, seed=17))
    o1, l1 = mi.attn_fwd_dense(q, k, v)
    o2, l2 = mi.attn_fwd_dense(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# ---------------------------------------------------------------- paged


def paged_case(B, Sq, Hq, Hkv, D, lens, page_size, *, dtype=torch.bfloat16, causal=True,
               scale=None, seed=0, split_keys=0, window=None, softcap=None, what=""):
    say(f"paged {what} B={B} Sq={Sq} Hq={Hq} Hkv={Hkv} D={D} page={page_size} lens={lens} "
        f"split_keys={split_keys} window={window} softcap={softcap}")
    cap = max(max(lens), 1)
    max_pages = (cap + page_size - 1) // page_size + 1
    n_phys = B * max_pages + 3
    q, kd, vd = workloads.dense_inputs(B, Sq, max_pages * page_size, Hq, Hkv, D, dtype=dtype,
                                       seed=seed)
    g = torch.Generator().manual_seed(seed + 1000)
    bt = torch.randperm(n_phys, generator=g)[:B * max_pages].view(B, max_pages).to(torch.int32)
    # rows past each request's length and pages nobody maps hold NaN: a read
    # of any of them would poison the output
    kd, vd = kd.clone(), vd.clone()
    for b, L in enumerate(lens):
        kd[b, L:] = float("nan")
        vd[b, L:] = float("nan")
    kc = workloads.scatter_to_pages(kd, bt, page_size, n_phys, fill=float("nan"))
    vc = workloads.scatter_to_pages(vd, bt, page_size, n_phys, fill=float("nan"))
    lens_t = torch.tensor(lens, dtype=torch.int32)
    mi.set_split_keys(split_keys)
    o, lse = mi.attn_fwd_paged(q.to(DEV), kc.to(DEV), vc.to(DEV), lens_t.to(DEV), bt.to(DEV),
                               page_size, causal=causal, scale=scale, window=window,
                               softcap=softcap)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_paged(q, kc, vc, lens_t, bt, page_size, causal=causal,
                                       scale=scale, window=window, softcap=softcap)
    return check_full(o, lse, o_ref, lse_ref, what)


@pytest.mark.parametrize("page_size", [16, 64, 256])
@pytest.mark.parametrize("split_keys", [0, 128, 1024])
def test_paged_decode(page_size, split_keys):
    lens = [1, 0, 64, 65, 1000, 513, 2047, 300]
    paged_case(len(lens), 1, 32, 8, 128, lens, page_size, split_keys=split_keys, seed=21,
               what="decode")


@pytest.mark.parametrize("page_size", [16, 64])
def test_streamk_decode_fewer_tiles_than_workgroups(page_size):
    # 6 key tiles in all for several hundred workgroups: most workgroups get
    # an empty share, and the merge must skip their slots
    paged_case(3, 1, 4, 2, 128, [5, 0, 40], page_size, seed=31, what="sk_tiny")


@pytest.mark.parametrize("piece", [0, 1, 64])
def test_streamk_plan_piece_weights(piece):
    # the plan weighs each piece of a unit `piece` tiles on top of its tiles;
    # any weight must still cover every tile once and let the merge find
    # every partial: long and short requests, one without keys, and a tiny
    # batch with more workgroups than weight
    mi.set_streamk_piece(piece)
    try:
        paged_case(8, 1, 32, 8, 128, [1, 0, 64, 65, 1000, 513, 2047, 300], 64, seed=23,
                   what=f"piece {piece}")
        paged_case(3, 1, 4, 2, 128, [5, 0, 40], 16, seed=24, what=f"piece {piece} tiny")
        paged_case(6, 1, 16, 4, 64, [3, 700, 1, 0, 1500, 64], 32, dtype=torch.float16,
                   window=(200, -1), seed=25, what=f"piece {piece} window")
    finally:
        mi.set_streamk_piece(-1)


def test_streamk_decode_many_requests():
    # more batch entries than the plan kernel's 1024 threads (chunked prefix),
    # lengths 0..120 including zeros
    g = torch.Generator().manual_seed(32)
    lens = torch.randint(0, 121, (1500,), generator=g).tolist()
    lens[7] = 0
    lens[1499] = 0
    paged_case(len(lens), 1, 4, 1, 64, lens, 32, dtype=torch.float16, seed=33, what="sk_many")


def test_streamk_dense_decode():
    say("dense decode-shaped call (stream-K over dense K/V)")
    B, Sq, Skv, Hq, Hkv, D = 5, 1, 3000, 16, 4, 64
    q, k, v = workloads.dense_inputs(B, Sq, Skv, Hq, Hkv, D, dtype=torch.float16, seed=34)
    mi.set_split_keys(0)
    o, lse = mi.attn_fwd_dense(q.to(DEV), k.to(DEV), v.to(DEV), causal=True)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_dense(q, k, v, causal=True)
    check_full(o, lse, o_ref, lse_ref, "sk_dense")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Hkv", [1, 2, 3, 6])
@pytest.mark.parametrize("page_size", [16, 64])
def test_paired_and_single_head_decode(D, Hkv, page_size):
    # an even KV head count runs the paired decode (one workgroup reads two
    # adjacent heads' rows), an odd one the one-head decode; both against the
    # oracle, over lengths with empty, one-key and ragged requests
    lens = [0, 1, 33, 511, 1200, 64, 2500]
    paged_case(len(lens), 1, 4 * Hkv, Hkv, D, lens, page_size, seed=60 + Hkv + D,
               what=f"decode Hkv={Hkv} D={D}")


def rising_scores_case(Sq, Skv, Hq, Hkv, D, step, what):
    # q = e_0, k_j = b_j e_0 with b_j = step * (j // 64) + N(0, 0.25): every
    # 64 keys the scores jump by `step`, so unmasked tiles whose exponentials
    # against a running max set on earlier keys would exceed the 2^24 range
    # take the tile max (and raise the running max), and the others do not
    g = torch.Generator().manual_seed(70 + D)
    q = torch.zeros(1, Sq, Hq, D)
    q[..., 0] = 1.0
    b = step * (torch.arange(Skv) // 64).float() + 0.5 * torch.randn(Skv, generator=g)
    k = torch.zeros(1, Skv, Hkv, D)
    k[0, :, :, 0] = b[:, None]
    k[0, :, :, 1:] = 0.1 * torch.randn(Skv, Hkv, D - 1, generator=g)
    v = torch.randn(1, Skv, Hkv, D, generator=g)
    q, k, v = q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)
    say(f"rising scores {what} Sq={Sq} Skv={Skv} Hq={Hq} Hkv={Hkv} D={D} step={step}")
    o, lse = run_dense(q, k, v, scale=1.0, causal=False)
    o_ref, lse_ref = oracle.attn_dense(q, k, v, scale=1.0, causal=False)
    check_full(o, lse, o_ref, lse_ref, f"rising {what}")


@pytest.mark.parametrize("step", [3.0, 9.0, 40.0])
@pytest.mark.parametrize("D", [64, 128, 256])
def test_rising_scores_across_tiles(D, step):
    # prefill-shaped (the 8-wave schedule at D = 128, the streaming ones at
    # D = 64 and 256) and decode-shaped (stream-K) calls
    rising_scores_case(70, 700, 2, 1, D, step, "prefill")
    rising_scores_case(1, 1500, 8, 2, D, step, "decode")


@pytest.mark.parametrize("D", [64, 128, 256])
def test_paged_decode_head_dims(D):
    paged_case(4, 1, 16, 4, D, [700, 33, 1, 1500], 32, seed=22, what=f"decode_d{D}")


def test_paged_decode_fp16_noncausal_scale():
    paged_case(3, 2, 8, 2, 128, [400, 2, 90], 64, dtype=torch.float16, causal=False,
               scale=0.2, seed=23, what="fp16_noncausal")


@pytest.mark.parametrize("split_keys", [0, 512])
def test_paged_chunked_prefill_wide_group(split_keys):
    # group 12, D = 256, Sq > 1 new queries at the end of each cache; a
    # request shorter than Sq has empty leading rows
    paged_case(3, 37, 24, 2, 256, [900, 37, 20], 64, split_keys=split_keys, seed=24,
               what="chunked_g12")


def test_paged_prefill_multiple_row_blocks():
    paged_case(2, 150, 8, 2, 128, [150, 1200], 16, split_keys=256, seed=25, what="prefill_rb")


def test_paged_equals_dense_on_gpu():
    say("paged vs dense, same keys")
    B, Sq, Skv, Hq, Hkv, D, ps = 2, 64, 512, 8, 2, 128, 64
    q, kd, vd = workloads.dense_inputs(B, Sq, Skv, Hq, Hkv, D, seed=26)
    bt = torch.randperm(16, generator=torch.Generator().manual_seed(1))[:16].view(2, 8)
    bt = bt.to(torch.int32)
    kc = workloads.scatter_to_pages(kd, bt, ps, 16)
    vc = workloads.scatter_to_pages(vd, bt, ps, 16)
    lens = torch.full((B,), Skv, dtype=torch.int32)
    o_p, l_p = mi.attn_fwd_paged(q.to(DEV), kc.to(DEV), vc.to(DEV), lens.to(DEV), bt.to(DEV), ps)
    o_d, l_d = mi.attn_fwd_dense(q.to(DEV), kd.to(DEV), vd.to(DEV))
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_dense(q, kd, vd)
    check_full(o_p, l_p, o_ref, lse_ref, "paged")
    check_full(o_d, l_d, o_ref, lse_ref, "dense")


# ---------------------------------------------------------------- full-size workloads


def test_full_size_causal_gqa_prefill():
    # every one of the 262,144 output rows against the oracle (~25 s of host
    # threads), in the benchmark's launch configuration
    w = workloads.make(2)
    say(w.name)
    o, lse = run_dense(w.q, w.k, w.v, scale=w.scale, causal=True)
    say(f"{w.name}: oracle on {oracle.num_threads()} host threads")
    o_ref, lse_ref = oracle.attn_dense(w.q, w.k, w.v, scale=w.scale, causal=True)
    stats = check_full(o, lse, o_ref, lse_ref, w.name)
    say(f"{w.name}: {stats}")


def test_full_size_paged_decode():
    w = workloads.make(3)
    say(w.name)
    o, lse = mi.attn_fwd_paged(w.q.to(DEV), w.k_cache.to(DEV), w.v_cache.to(DEV),
                               w.real_seqlen_kv.to(DEV), w.block_table.to(DEV), w.page_size)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_paged(w.q, w.k_cache, w.v_cache, w.real_seqlen_kv,
                                       w.block_table, w.page_size)
    stats = check_full(o, lse, o_ref, lse_ref, w.name)
    say(f"{w.name}: {stats}")


def test_full_size_mha_key_padding():
    w = workloads.make(4)
    say(w.name)
    o, lse = run_dense(w.q, w.k, w.v, scale=w.scale, causal=False, mask=w.key_padding_mask)
    o_ref, lse_ref = oracle.attn_dense(w.q, w.k, w.v, scale=w.scale, causal=False,
                                       key_padding_mask=w.key_padding_mask)
    stats = check_full(o, lse, o_ref, lse_ref, w.name)
    say(f"{w.name}: {stats}")


def test_full_size_wide_group_chunked_prefill():
    w = workloads.make(5)
    say(w.name)
    o, lse = mi.attn_fwd_paged(w.q.to(DEV), w.k_cache.to(DEV), w.v_cache.to(DEV),
                               w.real_seqlen_kv.to(DEV), w.block_table.to(DEV), w.page_size,
                               scale=w.scale)
    torch.cuda.synchronize()
    say(f"{w.name}: oracle on {oracle.num_threads()} host threads")
    o_ref, lse_ref = oracle.attn_paged(w.q, w.k_cache, w.v_cache, w.real_seqlen_kv,
                                       w.block_table, w.page_size, scale=w.scale)
    stats = check_full(o, lse, o_ref, lse_ref, w.name)
    say(f"{w.name}: {stats}")


def test_refusals_name_the_limit():
    q = torch.zeros(1, 4, 6, 96, dtype=torch.bfloat16, device=DEV)
    k = torch.zeros(1, 4, 2, 96, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError, match="D=96"):
        mi.attn_fwd_dense(q, k, k)
    q = torch.zeros(1, 4, 5, 64, dtype=torch.bfloat16, device=DEV)
    k = torch.zeros(1, 4, 2, 64, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError, match="not divisible"):
        mi.attn_fwd_dense(q, k, k)
