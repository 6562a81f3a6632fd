"""The C ABI on the CPU: the library loads, exports every symbol its header
declares, and refuses invalid arguments with a message naming the limit --
all before any HIP call, so no GPU is needed (TileOPs "Attention Operators",
GQADenseFwdOp: a refusal names the limit; RL-Kernel "Standard Softmax
Attention", Known Limitations: Hq must be divisible by Hkv)."""
import ctypes
import math
import os
import re

import pytest

import softmax_attention_amd as mi
from softmax_attention_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "miattn.h")

NAN = float("nan")
FAKE = 0x10000  # a 16-byte aligned non-null address; never dereferenced on refusal


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(?:miattn_status|void|const char\s*\*)\s*(\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(binding.EXPORTS), names
    L = ctypes.CDLL(binding.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n


# ctypes kind of each C parameter type the header uses
_KINDS = {"int": "i32", "float": "f32", "int64_t": "i64", "miattn_dtype": "i32",
          "miattn_cache_dtype": "i32"}


def declared_prototypes():
    """{name: [parameter kind, ...]} for every function include/miattn.h declares;
    a kind is 'ptr' for any pointer, else the ctypes width of the scalar."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    protos = {}
    for m in re.finditer(r"\b(?:miattn_status|void|const char\s*\*)\s*(\w+)\s*\(([^)]*)\)\s*;",
                         text):
        params = [p.strip() for p in m.group(2).split(",")]
        kinds = []
        for prm in params:
            if prm in ("void", ""):
                continue
            if "*" in prm:
                kinds.append("ptr")
                continue
            typ = " ".join(prm.replace("const ", "").split()[:-1])
            kinds.append(_KINDS[typ])
        protos[m.group(1)] = kinds
    return protos


def _kind(ct):
    if ct in (ctypes.c_int, ctypes.c_int32):
        return "i32"
    if ct is ctypes.c_float:
        return "f32"
    if ct in (ctypes.c_int64, ctypes.c_longlong):
        return "i64"
    if ct is ctypes.c_void_p or ct is ctypes.c_char_p or issubclass(ct, ctypes._Pointer):
        return "ptr"
    raise AssertionError(f"unexpected ctypes type {ct}")


def test_binding_argtypes_match_the_header_prototypes():
    # the binding passes exactly the arguments the header declares, in order:
    # a caller built against the header and the binding agree on every slot
    protos = declared_prototypes()
    L = mi.lib()
    for name, kinds in protos.items():
        got = [_kind(t) for t in getattr(L, name).argtypes]
        assert got == kinds, (name, got, kinds)


def test_headline_entry_points_have_the_contract_signatures():
    # attn_fwd_dense(q, k, v, B, Hq, Hkv, Sq, Skv, D, scale, causal,
    #                key_padding_mask, o, lse, dtype, stream) and
    # attn_fwd_paged(q, k_cache, v_cache, real_seqlen_kv, block_table,
    #                page_size, causal, o, lse, B, Sq, Hq, Hkv, D, max_pages,
    #                num_phys_pages, scale, dtype, stream)
    protos = declared_prototypes()
    assert protos["attn_fwd_dense"] == ["ptr"] * 3 + ["i32"] * 6 + ["f32", "i32"] + \
        ["ptr"] * 3 + ["i32", "ptr"]
    assert protos["attn_fwd_paged"] == ["ptr"] * 5 + ["i32"] * 2 + ["ptr"] * 2 + \
        ["i32"] * 7 + ["f32", "i32", "ptr"]
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    dense_sig = re.search(r"attn_fwd_dense\(([^)]*)\)", text).group(1)
    names = [p.split()[-1].lstrip("*") for p in dense_sig.split(",")]
    assert names == ["q", "k", "v", "B", "Hq", "Hkv", "Sq", "Skv", "D", "scale", "causal",
                     "key_padding_mask", "o", "lse", "dtype", "stream"], names
    paged_sig = re.search(r"attn_fwd_paged\(([^)]*)\)", text).group(1)
    names = [p.split()[-1].lstrip("*") for p in paged_sig.split(",")]
    assert names == ["q", "k_cache", "v_cache", "real_seqlen_kv", "block_table", "page_size",
                     "causal", "o", "lse", "B", "Sq", "Hq", "Hkv", "D", "max_pages",
                     "num_phys_pages", "scale", "dtype", "stream"], names


def dense(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, B=1, Hq=8, Hkv=2, Sq=4, Skv=4, D=128, scale=NAN, causal=1,
             wl=-1, wr=-1, softcap=0.0, mask=None, o=FAKE, lse=None, dtype=0, stream=None)
    ex = any(x in kw for x in ("wl", "wr", "softcap"))
    a.update(kw)
    L = mi.lib()
    head = (a["q"], a["k"], a["v"], a["B"], a["Hq"], a["Hkv"], a["Sq"], a["Skv"], a["D"],
            a["scale"], a["causal"], a["mask"], a["o"], a["lse"])
    if ex:
        st = L.attn_fwd_dense_ex(*head, a["wl"], a["wr"], a["softcap"], a["dtype"], a["stream"])
    else:
        st = L.attn_fwd_dense(*head, a["dtype"], a["stream"])
    return st, L.miattn_last_error().decode()


def paged(**kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, lens=FAKE, bt=FAKE, page_size=64, causal=1, wl=-1,
             wr=-1, softcap=0.0, o=FAKE, lse=None, B=2, Sq=1, Hq=8, Hkv=2, D=128, max_pages=4,
             n_phys=8, scale=NAN, dtype=0, stream=None)
    ex = any(x in kw for x in ("wl", "wr", "softcap"))
    a.update(kw)
    L = mi.lib()
    head = (a["q"], a["kc"], a["vc"], a["lens"], a["bt"], a["page_size"], a["causal"], a["o"],
            a["lse"], a["B"], a["Sq"], a["Hq"], a["Hkv"], a["D"], a["max_pages"], a["n_phys"],
            a["scale"])
    if ex:
        st = L.attn_fwd_paged_ex(*head, a["wl"], a["wr"], a["softcap"], a["dtype"], a["stream"])
    else:
        st = L.attn_fwd_paged(*head, a["dtype"], a["stream"])
    return st, L.miattn_last_error().decode()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(Hq=30, Hkv=8), 1, "Hq (30) not divisible by Hkv (8)"),
    (dict(D=96), 2, "D=96 unsupported"),
    (dict(D=0), 1, "D=0"),
    (dict(B=-1), 1, "B=-1"),
    (dict(Sq=-3), 1, "Sq=-3"),
    (dict(Skv=-2), 1, "Skv=-2"),
    (dict(Hkv=0), 1, "head counts"),
    (dict(dtype=7), 2, "dtype 7"),
    (dict(scale=math.inf), 1, "scale must be finite"),
    (dict(q=None), 1, "must not be NULL"),
    (dict(o=None), 1, "must not be NULL"),
    (dict(k=None), 1, "k and v"),
    (dict(q=FAKE + 8), 1, "q not 16-byte aligned"),
    (dict(k=FAKE + 2), 1, "k not 16-byte aligned"),
    (dict(o=FAKE + 4), 1, "o not 16-byte aligned"),
    (dict(lse=FAKE + 2), 1, "lse not 4-byte aligned"),
    (dict(causal=2), 1, "causal=2"),
    (dict(wl=-2), 1, "window_left=-2"),
    (dict(wr=-5), 1, "window_right=-5"),
    (dict(softcap=-1.0), 1, "softcap"),
    (dict(softcap=NAN), 1, "softcap"),
    (dict(softcap=math.inf), 1, "softcap"),
    (dict(B=0, softcap=-1.0), 1, "softcap"),  # checked before the empty-call exit
])
def test_dense_refusals(kw, status, needle):
    st, msg = dense(**kw)
    assert st == status and needle in msg, (st, msg)


def test_dense_empty_calls_are_ok_without_touching_the_device():
    assert dense(B=0, q=None, o=None)[0] == 0
    assert dense(Sq=0, q=None, o=None)[0] == 0


@pytest.mark.parametrize("kw,status,needle", [
    (dict(page_size=0), 1, "page_size must be > 0"),
    (dict(page_size=48), 2, "page_size=48 unsupported"),
    (dict(page_size=8), 2, "page_size=8 unsupported"),
    (dict(max_pages=0), 1, "max_pages"),
    (dict(n_phys=-1), 1, "num_phys_pages"),
    (dict(lens=None), 1, "must not be NULL"),
    (dict(bt=None), 1, "must not be NULL"),
    (dict(kc=FAKE + 8), 1, "k_cache not 16-byte aligned"),
    (dict(bt=FAKE + 2), 1, "4-byte aligned"),
    (dict(Hq=12, Hkv=8), 1, "not divisible"),
    (dict(D=512), 2, "D=512 unsupported"),
    (dict(max_pages=1 << 30, page_size=64), 2, "exceeds"),
    (dict(wl=-3), 1, "window_left=-3"),
    (dict(wr=-4), 1, "window_right=-4"),
    (dict(softcap=-0.5), 1, "softcap"),
    (dict(B=-2), 1, "B=-2"),
    (dict(Sq=-1), 1, "Sq=-1"),
    (dict(Hkv=-1), 1, "head counts"),
    (dict(o=FAKE + 4), 1, "o not 16-byte aligned"),
    (dict(lse=FAKE + 1), 1, "lse not 4-byte aligned"),
    (dict(vc=FAKE + 8), 1, "v_cache not 16-byte aligned"),
    (dict(causal=3), 1, "causal=3"),
    (dict(dtype=5), 2, "dtype 5"),
    (dict(scale=-math.inf), 1, "scale must be finite"),
])
def test_paged_refusals(kw, status, needle):
    st, msg = paged(**kw)
    assert st == status and needle in msg, (st, msg)


def varlen(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, cq=FAKE, ck=FAKE, B=2, tq=6, tk=9, mq=4, mk=5, Hq=8,
             Hkv=2, D=128, scale=NAN, causal=1, wl=-1, wr=-1, softcap=0.0, sinks=None, o=FAKE,
             lse=None, dtype=0, stream=None)
    a.update(kw)
    L = mi.lib()
    st = L.attn_fwd_varlen(a["q"], a["k"], a["v"], a["cq"], a["ck"], a["B"], a["tq"], a["tk"],
                           a["mq"], a["mk"], a["Hq"], a["Hkv"], a["D"], a["scale"], a["causal"],
                           a["wl"], a["wr"], a["softcap"], a["sinks"], a["o"], a["lse"],
                           a["dtype"], a["stream"])
    return st, L.miattn_last_error().decode()


def paged_varlen(**kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, lens=FAKE, bt=FAKE, cq=FAKE, page_size=64, causal=1,
             wl=-1, wr=-1, softcap=0.0, sinks=None, o=FAKE, lse=None, B=2, tq=5, mq=4, Hq=8,
             Hkv=2, D=128, max_pages=4, n_phys=8, scale=NAN, dtype=0, cache=0, ks=None, vs=None,
             stream=None)
    a.update(kw)
    L = mi.lib()
    st = L.attn_fwd_paged_varlen(a["q"], a["kc"], a["vc"], a["lens"], a["bt"], a["cq"],
                                 a["page_size"], a["causal"], a["wl"], a["wr"], a["softcap"],
                                 a["sinks"], a["o"], a["lse"], a["B"], a["tq"], a["mq"], a["Hq"],
                                 a["Hkv"], a["D"], a["max_pages"], a["n_phys"], a["scale"],
                                 a["dtype"], a["cache"], a["ks"], a["vs"], a["stream"])
    return st, L.miattn_last_error().decode()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(cq=None), 1, "cu_seqlens_q and cu_seqlens_kv must not be NULL"),
    (dict(ck=None), 1, "must not be NULL"),
    (dict(cq=FAKE + 2), 1, "4-byte aligned"),
    (dict(tq=-1), 1, "total_q=-1"),
    (dict(mk=-1), 1, "Skv=-1"),
    (dict(sinks=FAKE + 1), 1, "sinks not 4-byte aligned"),
    (dict(Hq=6, Hkv=4), 1, "not divisible"),
    (dict(softcap=-2.0), 1, "softcap"),
    (dict(k=None), 1, "k and v"),
    (dict(D=80), 2, "D=80"),
])
def test_varlen_refusals(kw, status, needle):
    st, msg = varlen(**kw)
    assert st == status and needle in msg, (st, msg)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(cq=None), 1, "cu_seqlens_q must not be NULL"),
    (dict(cq=FAKE + 2), 1, "cu_seqlens_q not 4-byte aligned"),
    (dict(tq=-3), 1, "total_q=-3"),
    (dict(page_size=24), 2, "page_size=24"),
    (dict(lens=None), 1, "must not be NULL"),
    (dict(sinks=FAKE + 2), 1, "sinks not 4-byte aligned"),
    (dict(cache=1), 2, "cache_dtype 1 must equal dtype 0"),
    (dict(cache=-1), 1, "cache_dtype -1 unknown"),
    (dict(cache=7), 1, "cache_dtype 7 unknown"),
    (dict(cache=2), 1, "an FP8 pool needs 4-byte aligned k_scale and v_scale"),
    (dict(cache=2, ks=FAKE, vs=FAKE + 2), 1, "an FP8 pool needs"),
    (dict(cache=2, ks=FAKE, vs=FAKE, D=256, Hq=8, Hkv=2), 2, "FP8 pools: D=256"),
])
def test_paged_varlen_refusals(kw, status, needle):
    st, msg = paged_varlen(**kw)
    assert st == status and needle in msg, (st, msg)


def test_varlen_empty_calls_are_ok_without_touching_the_device():
    assert varlen(B=0, q=None, o=None, cq=None, ck=None)[0] == 0
    assert varlen(tq=0, q=None, o=None)[0] == 0
    assert varlen(mq=0, q=None, o=None)[0] == 0
    assert paged_varlen(tq=0, q=None, o=None)[0] == 0


def kvw(**kw):
    a = dict(k=FAKE, v=FAKE, kp=FAKE, vp=FAKE, sl=FAKE, tokens=4, Hkv=2, D=128, num_slots=64,
             dtype=0, cache=0, ks=None, vs=None, stream=None)
    a.update(kw)
    L = mi.lib()
    st = L.kv_cache_write(a["k"], a["v"], a["kp"], a["vp"], a["sl"], a["tokens"], a["Hkv"],
                          a["D"], a["num_slots"], a["dtype"], a["cache"], a["ks"], a["vs"],
                          a["stream"])
    return st, L.miattn_last_error().decode()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(tokens=-1), 1, "tokens=-1"),
    (dict(D=0), 1, "must be positive"),
    (dict(num_slots=-5), 1, "num_slots"),
    (dict(dtype=3), 2, "dtype 3"),
    (dict(cache=1), 2, "cache_dtype 1 must equal dtype 0"),
    (dict(cache=-1), 1, "cache_dtype -1 unknown"),
    (dict(cache=7), 1, "cache_dtype 7 unknown"),
    (dict(Hkv=1, D=12), 2, "multiple of 8"),
    (dict(sl=None), 1, "must not be NULL"),
    (dict(k=FAKE + 8), 1, "16-byte aligned"),
    (dict(kp=FAKE + 8), 1, "16-byte aligned"),
    (dict(sl=FAKE + 4), 1, "8-byte aligned"),
    (dict(cache=2), 1, "needs 4-byte aligned k_scale"),
    (dict(cache=2, ks=FAKE, vs=FAKE, kp=FAKE + 4), 1, "8-byte aligned"),
])
def test_kv_write_refusals(kw, status, needle):
    st, msg = kvw(**kw)
    assert st == status and needle in msg, (st, msg)


def test_kv_write_without_tokens_is_ok_without_touching_the_device():
    assert kvw(tokens=0, k=None, v=None, kp=None, vp=None, sl=None)[0] == 0


def append_call(**kw):
    a = dict(q=FAKE, kn=FAKE, vn=FAKE, kc=FAKE, vc=FAKE, lens=FAKE, bt=FAKE, cq=FAKE,
             page_size=64, causal=1, softcap=0.0, o=FAKE, lse=None, B=2, tq=5, mq=4, Hq=8,
             Hkv=2, D=128, max_pages=4, n_phys=8, scale=NAN, dtype=0, cache=0, ks=None, vs=None,
             stream=None)
    a.update(kw)
    L = mi.lib()
    st = L.attn_fwd_paged_append(a["q"], a["kn"], a["vn"], a["kc"], a["vc"], a["lens"],
                                 a["bt"], a["cq"], a["page_size"], a["causal"], a["softcap"],
                                 a["o"], a["lse"], a["B"], a["tq"], a["mq"], a["Hq"], a["Hkv"],
                                 a["D"], a["max_pages"], a["n_phys"], a["scale"], a["dtype"],
                                 a["cache"], a["ks"], a["vs"], a["stream"])
    return st, L.miattn_last_error().decode()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(kn=None), 1, "k_new and v_new must not be NULL"),
    (dict(vn=FAKE + 2), 1, "16-byte aligned"),
    (dict(cq=None), 1, "cu_seqlens_q must not be NULL"),
    (dict(page_size=20), 2, "page_size=20"),
    (dict(softcap=-3.0), 1, "softcap"),
    (dict(cache=2, ks=None, vs=FAKE), 1, "an FP8 pool needs"),
])
def test_paged_append_refusals(kw, status, needle):
    st, msg = append_call(**kw)
    assert st == status and needle in msg, (st, msg)


def test_python_binding_maps_refusals_to_value_error():
    import torch
    st, _ = dense(Hq=5, Hkv=2)
    with pytest.raises(ValueError, match="not divisible"):
        binding._check(st)
    st, _ = dense(D=32)
    with pytest.raises(ValueError, match="D=32"):
        binding._check(st)
    q = torch.zeros(1, 2, 4, 64, dtype=torch.bfloat16)
    k = torch.zeros(1, 2, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="dtype"):
        mi.attn_fwd_dense(q.float(), k.float(), k.float())
    with pytest.raises(ValueError, match="GPU"):
        mi.attn_fwd_dense(q, k, k)


def test_binding_fails_loudly_without_the_library(monkeypatch, tmp_path):
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        binding.lib()


def test_binding_checks_caller_outputs():
    # a caller-supplied out / lse must match what the kernels write in full
    import torch
    like = torch.zeros(2, 3, 4, 64, dtype=torch.bfloat16)
    assert binding._output(None, like).shape == like.shape
    ok = torch.empty_like(like)
    assert binding._output(ok, like) is ok
    for bad, needle in ((torch.empty(2, 3, 4, 32, dtype=torch.bfloat16), "out must be"),
                        (torch.empty(2, 3, 4, 64, dtype=torch.float32), "out must be"),
                        (torch.empty(2, 3, 64, 4, dtype=torch.bfloat16).transpose(2, 3),
                         "contiguous"),
                        (torch.empty(2, 3, 4, 64, dtype=torch.bfloat16, device="meta"),
                         "device")):
        with pytest.raises(ValueError, match=needle):
            binding._output(bad, like)
    dev = like.device
    assert binding._lse_output(None, (2, 4, 3), dev, False) is None
    assert binding._lse_output(None, (2, 4, 3), dev, True).dtype == torch.float32
    for bad, needle in ((torch.empty(2, 4, 2), "lse must be"),
                        (torch.empty(2, 4, 3, dtype=torch.float64), "lse must be"),
                        (torch.empty(2, 3, 4).transpose(1, 2), "contiguous"),
                        (torch.empty(2, 4, 3, device="meta"), "device")):
        with pytest.raises(ValueError, match=needle):
            binding._lse_output(bad, (2, 4, 3), dev, True)
