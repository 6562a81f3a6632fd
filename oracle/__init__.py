"""fp64 CPU oracle for grouped-query softmax attention forward -- TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or calls it, and this package uses
nothing from the product path: inputs arrive as plain 16-bit bit patterns and
integer arrays, results leave as float64 numpy arrays.

The arithmetic lives in ``attn_oracle.c`` (plain C, fp64, fixed summation
order); this module only compiles it with gcc and marshals arguments.  See the
header of ``attn_oracle.c`` for the definition it follows and its sources on
the pages (TileOPs "Attention Operators" GQADenseFwdOp stages 1 and 4-7 and
MHADecodePagedWithKVCacheFwdOp; RL-Kernel "Standard Softmax Attention";
MATE "QSA" Core Attention for the natural-log LSE and empty rows).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

BF16 = 0
FP16 = 1

# -ffp-contract=off and no fast-math keep every sum in the written order.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra"]


def build() -> str:
    """Compile the oracle with gcc into oracle/liboracle.so (always rebuilds)."""
    tmp = _LIB + ".tmp"
    subprocess.run(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64, f32 = ctypes.c_int, ctypes.c_int64, ctypes.c_float
        lib.oracle_decode.argtypes = [ctypes.c_uint16, i32]
        lib.oracle_decode.restype = ctypes.c_double
        lib.oracle_resolve_scale.argtypes = [f32, i32]
        lib.oracle_resolve_scale.restype = ctypes.c_double
        win = [i32, i32, f32]  # window_left, window_right, softcap
        lib.oracle_attn_dense.argtypes = [P, P, P, i32, i32, i32, i32, i32, i32, i32, f32, i32,
                                          *win, P, P, P]
        lib.oracle_attn_dense_rows.argtypes = [P, P, P, i32, i32, i32, i32, i32, i32, i32, f32,
                                               i32, *win, P, P, i64, P, P]
        lib.oracle_attn_paged.argtypes = [P, P, P, P, P, i32, i32, *win, i32, i32, i32, i32, i32,
                                          i32, f32, i32, P, P]
        lib.oracle_attn_paged_rows.argtypes = [P, P, P, P, P, i32, i32, *win, i32, i32, i32, i32,
                                               i32, i32, f32, i32, P, i64, P, P]
        lib.oracle_attn_varlen.argtypes = [P, P, P, i32, P, P, i32, i32, i32, i32, i32, i32, f32,
                                           i32, *win, P, P, P]
        lib.oracle_attn_paged_varlen.argtypes = [P, P, P, P, P, i32, P, i32, *win, P, i32, i32,
                                                 i32, i32, i32, i32, f32, i32, P, P]
        lib.oracle_attn_bwd.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, i32, i32, i32, f32,
                                        i32, P, P, P]
        lib.oracle_e4m3_decode.argtypes = [i32]
        lib.oracle_e4m3_decode.restype = ctypes.c_double
        lib.oracle_e4m3_encode.argtypes = [ctypes.c_double]
        lib.oracle_kv_write.argtypes = [P, P, i32, P, i32, i32, i32, i64, i32, f32, f32, P, P]
        lib.oracle_attn_paged_varlen_fp8.argtypes = [P, P, P, f32, f32, P, P, i32, P, i32, *win,
                                                     P, i32, i32, i32, i32, i32, i32, f32, i32,
                                                     P, P]
        lib.oracle_attn_paged_append.argtypes = [P, P, P, P, P, i32, f32, f32, P, P, i32, P, i32,
                                                 f32, i32, i32, i32, i32, i32, i32, i32, f32, i32,
                                                 P, P]
        for name in ("oracle_attn_dense", "oracle_attn_dense_rows", "oracle_attn_paged",
                     "oracle_attn_paged_rows", "oracle_attn_varlen", "oracle_attn_paged_varlen",
                     "oracle_e4m3_encode", "oracle_kv_write", "oracle_attn_paged_append",
                     "oracle_attn_paged_varlen_fp8",
                     "oracle_attn_bwd",
                     "oracle_num_threads"):
            getattr(lib, name).restype = i32
        _lib = lib
    return _lib


def _bits(x) -> np.ndarray:
    """16-bit bit patterns of a bf16/fp16 torch tensor (CPU copy) or uint16 array."""
    if isinstance(x, np.ndarray):
        assert x.dtype == np.uint16
        return np.ascontiguousarray(x)
    import torch
    assert x.dtype in (torch.bfloat16, torch.float16), x.dtype
    return np.ascontiguousarray(x.detach().cpu().contiguous().view(torch.int16).numpy()
                                .view(np.uint16))


def _dtype_code(x) -> int:
    if isinstance(x, np.ndarray):
        raise TypeError("pass dtype explicitly for raw bit arrays")
    import torch
    return BF16 if x.dtype == torch.bfloat16 else FP16


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _scale_arg(scale) -> float:
    return float("nan") if scale is None else float(scale)


def _opt_args(window, softcap):
    """(window_left, window_right, softcap) as the C entry points take them:
    -1 for an unlimited side, 0.0 for no cap (None and 0 both disable it)."""
    wl, wr = (-1, -1) if window is None else (int(window[0]), int(window[1]))
    return wl, wr, 0.0 if softcap is None else float(softcap)


def decode(bits: int, dtype: int) -> float:
    """Exact value of one 16-bit pattern (BF16 or FP16 code)."""
    return _load().oracle_decode(bits, dtype)


def resolve_scale(scale, D: int) -> float:
    """alpha as the oracle applies it: None -> float(1/sqrt(D)), else verbatim."""
    return _load().oracle_resolve_scale(_scale_arg(scale), D)


def num_threads() -> int:
    return _load().oracle_num_threads()


def _as_mask(mask, B, Skv):
    if mask is None:
        return None
    import torch
    if isinstance(mask, torch.Tensor):
        mask = mask.detach().cpu().numpy()
    m = np.ascontiguousarray(np.asarray(mask).astype(np.uint8))
    assert m.shape == (B, Skv), m.shape
    return m


def attn_dense(q, k, v, *, scale=None, causal=True, key_padding_mask=None, dtype=None,
               window=None, softcap=None):
    """o [B,Sq,Hq,D] float64, lse [B,Hq,Sq] float64 for a dense call.

    q [B,Sq,Hq,D], k/v [B,Skv,Hkv,D]: bf16/fp16 torch tensors (or uint16 bit
    arrays with ``dtype`` given).  window = (w_L, w_R), -1 = unlimited side;
    softcap None or 0 = no cap."""
    dt = _dtype_code(q) if dtype is None else dtype
    qb, kb, vb = _bits(q), _bits(k), _bits(v)
    B, Sq, Hq, D = qb.shape
    _, Skv, Hkv, _ = kb.shape
    m = _as_mask(key_padding_mask, B, Skv)
    o = np.zeros((B, Sq, Hq, D), np.float64)
    lse = np.zeros((B, Hq, Sq), np.float64)
    rc = _load().oracle_attn_dense(_ptr(qb), _ptr(kb), _ptr(vb), dt, B, Hq, Hkv, Sq, Skv, D,
                                   _scale_arg(scale), int(bool(causal)),
                                   *_opt_args(window, softcap),
                                   None if m is None else _ptr(m), _ptr(o), _ptr(lse))
    if rc != 0:
        raise ValueError(f"oracle_attn_dense rejected the call (rc={rc})")
    return o, lse


def _sel_array(rows) -> np.ndarray:
    sel = np.ascontiguousarray(np.asarray(rows, dtype=np.int32).reshape(-1, 3))
    return sel


def attn_dense_rows(q, k, v, rows, *, scale=None, causal=True, key_padding_mask=None,
                    dtype=None, window=None, softcap=None):
    """Selected rows (b, i, h) of a dense call: o [n, D], lse [n]."""
    dt = _dtype_code(q) if dtype is None else dtype
    qb, kb, vb = _bits(q), _bits(k), _bits(v)
    B, Sq, Hq, D = qb.shape
    _, Skv, Hkv, _ = kb.shape
    m = _as_mask(key_padding_mask, B, Skv)
    sel = _sel_array(rows)
    n = sel.shape[0]
    o = np.zeros((n, D), np.float64)
    lse = np.zeros((n,), np.float64)
    rc = _load().oracle_attn_dense_rows(_ptr(qb), _ptr(kb), _ptr(vb), dt, B, Hq, Hkv, Sq, Skv,
                                        D, _scale_arg(scale), int(bool(causal)),
                                        *_opt_args(window, softcap),
                                        None if m is None else _ptr(m), _ptr(sel), n, _ptr(o),
                                        _ptr(lse))
    if rc != 0:
        raise ValueError(f"oracle_attn_dense_rows rejected the call (rc={rc})")
    return o, lse


def _paged_args(q, k_cache, v_cache, real_seqlen_kv, block_table):
    qb, kb, vb = _bits(q), _bits(k_cache), _bits(v_cache)
    B, Sq, Hq, D = qb.shape
    Hkv = kb.shape[-2]
    import torch
    lens = real_seqlen_kv.detach().cpu().numpy() if isinstance(real_seqlen_kv, torch.Tensor) \
        else np.asarray(real_seqlen_kv)
    bt = block_table.detach().cpu().numpy() if isinstance(block_table, torch.Tensor) \
        else np.asarray(block_table)
    lens = np.ascontiguousarray(lens.astype(np.int32))
    bt = np.ascontiguousarray(bt.astype(np.int32))
    assert lens.shape == (B,) and bt.ndim == 2 and bt.shape[0] == B
    return qb, kb, vb, lens, bt, B, Sq, Hq, Hkv, D


def attn_paged(q, k_cache, v_cache, real_seqlen_kv, block_table, page_size, *, causal=True,
               scale=None, dtype=None, window=None, softcap=None):
    """o [B,Sq,Hq,D], lse [B,Hq,Sq] (float64) for a paged call.

    k_cache/v_cache: [pages*page_size, Hkv, D] or [pages, page_size, Hkv, D]."""
    dt = _dtype_code(q) if dtype is None else dtype
    qb, kb, vb, lens, bt, B, Sq, Hq, Hkv, D = _paged_args(q, k_cache, v_cache, real_seqlen_kv,
                                                          block_table)
    o = np.zeros((B, Sq, Hq, D), np.float64)
    lse = np.zeros((B, Hq, Sq), np.float64)
    rc = _load().oracle_attn_paged(_ptr(qb), _ptr(kb), _ptr(vb), _ptr(lens), _ptr(bt),
                                   int(page_size), int(bool(causal)),
                                   *_opt_args(window, softcap), B, Sq, Hq, Hkv, D,
                                   bt.shape[1], _scale_arg(scale), dt, _ptr(o), _ptr(lse))
    if rc != 0:
        raise ValueError(f"oracle_attn_paged rejected the call (rc={rc})")
    return o, lse


def attn_paged_rows(q, k_cache, v_cache, real_seqlen_kv, block_table, page_size, rows, *,
                    causal=True, scale=None, dtype=None, window=None, softcap=None):
    """Selected rows (b, i, h) of a paged call: o [n, D], lse [n]."""
    dt = _dtype_code(q) if dtype is None else dtype
    qb, kb, vb, lens, bt, B, Sq, Hq, Hkv, D = _paged_args(q, k_cache, v_cache, real_seqlen_kv,
                                                          block_table)
    sel = _sel_array(rows)
    n = sel.shape[0]
    o = np.zeros((n, D), np.float64)
    lse = np.zeros((n,), np.float64)
    rc = _load().oracle_attn_paged_rows(_ptr(qb), _ptr(kb), _ptr(vb), _ptr(lens), _ptr(bt),
                                        int(page_size), int(bool(causal)),
                                        *_opt_args(window, softcap), B, Sq, Hq, Hkv, D,
                                        bt.shape[1], _scale_arg(scale), dt, _ptr(sel), n,
                                        _ptr(o), _ptr(lse))
    if rc != 0:
        raise ValueError(f"oracle_attn_paged_rows rejected the call (rc={rc})")
    return o, lse


def _i32(x) -> np.ndarray:
    import torch
    if isinstance(x, torch.Tensor):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(x).astype(np.int32))


def _sinks(sinks, Hq):
    if sinks is None:
        return None
    import torch
    if isinstance(sinks, torch.Tensor):
        sinks = sinks.detach().cpu().numpy()
    a = np.ascontiguousarray(np.asarray(sinks, dtype=np.float32))
    assert a.shape == (Hq,), a.shape
    return a


def attn_varlen(q, k, v, cu_seqlens_q, cu_seqlens_kv, *, scale=None, causal=True, window=None,
                softcap=None, sinks=None, dtype=None):
    """Packed (THD) call: q [total_q,Hq,D], k/v [total_kv,Hkv,D], cu_seqlens [B+1]
    (int), sinks [Hq] float32 or None.  Returns o [total_q,Hq,D] and lse
    [Hq,total_q] (float64)."""
    dt = _dtype_code(q) if dtype is None else dtype
    qb, kb, vb = _bits(q), _bits(k), _bits(v)
    total_q, Hq, D = qb.shape
    total_kv, Hkv, _ = kb.shape
    cq, ck = _i32(cu_seqlens_q), _i32(cu_seqlens_kv)
    B = cq.shape[0] - 1
    sk = _sinks(sinks, Hq)
    o = np.zeros((total_q, Hq, D), np.float64)
    lse = np.zeros((Hq, total_q), np.float64)
    rc = _load().oracle_attn_varlen(_ptr(qb), _ptr(kb), _ptr(vb), dt, _ptr(cq), _ptr(ck), B,
                                    total_q, total_kv, Hq, Hkv, D, _scale_arg(scale),
                                    int(bool(causal)), *_opt_args(window, softcap),
                                    None if sk is None else _ptr(sk), _ptr(o), _ptr(lse))
    if rc != 0:
        raise ValueError(f"oracle_attn_varlen rejected the call (rc={rc})")
    return o, lse


def attn_paged_varlen(q, k_cache, v_cache, cache_seqlens, block_table, page_size, cu_seqlens_q,
                      *, causal=True, scale=None, window=None, softcap=None, sinks=None,
                      cache_fp8=False, k_scale=1.0, v_scale=1.0, dtype=None):
    """Packed-query paged call: q [total_q,Hq,D] delimited by cu_seqlens_q [B+1];
    k_cache/v_cache [pages*page_size,Hkv,D] or [pages,page_size,Hkv,D] (16-bit,
    or with cache_fp8 E4M3FN codes dequantized by k_scale / v_scale);
    cache_seqlens [B] (each request's keys, its queries included);
    block_table [B,max_pages].  Returns o [total_q,Hq,D], lse [Hq,total_q]."""
    dt = _dtype_code(q) if dtype is None else dtype
    if cache_fp8:
        return _attn_paged_varlen_fp8(q, k_cache, v_cache, cache_seqlens, block_table,
                                      page_size, cu_seqlens_q, causal, scale, window, softcap,
                                      sinks, float(k_scale), float(v_scale), dt)
    qb, kb, vb = _bits(q), _bits(k_cache), _bits(v_cache)
    total_q, Hq, D = qb.shape
    Hkv = kb.shape[-2]
    lens, bt, cq = _i32(cache_seqlens), _i32(block_table), _i32(cu_seqlens_q)
    B = cq.shape[0] - 1
    assert lens.shape == (B,) and bt.ndim == 2 and bt.shape[0] == B
    sk = _sinks(sinks, Hq)
    o = np.zeros((total_q, Hq, D), np.float64)
    lse = np.zeros((Hq, total_q), np.float64)
    rc = _load().oracle_attn_paged_varlen(_ptr(qb), _ptr(kb), _ptr(vb), _ptr(lens), _ptr(bt),
                                          int(page_size), _ptr(cq), int(bool(causal)),
                                          *_opt_args(window, softcap),
                                          None if sk is None else _ptr(sk), B, total_q, Hq, Hkv,
                                          D, bt.shape[1], _scale_arg(scale), dt, _ptr(o),
                                          _ptr(lse))
    if rc != 0:
        raise ValueError(f"oracle_attn_paged_varlen rejected the call (rc={rc})")
    return o, lse


def _codes(x) -> np.ndarray:
    """uint8 E4M3FN codes of a uint8 / float8_e4m3fn tensor or array."""
    if isinstance(x, np.ndarray):
        assert x.dtype == np.uint8
        return np.ascontiguousarray(x)
    import torch
    return np.ascontiguousarray(x.detach().cpu().contiguous().view(torch.uint8).numpy())


def _attn_paged_varlen_fp8(q, k_cache, v_cache, cache_seqlens, block_table, page_size,
                           cu_seqlens_q, causal, scale, window, softcap, sinks, k_scale,
                           v_scale, dt):
    qb, kb, vb = _bits(q), _codes(k_cache), _codes(v_cache)
    total_q, Hq, D = qb.shape
    Hkv = kb.shape[-2]
    lens, bt, cq = _i32(cache_seqlens), _i32(block_table), _i32(cu_seqlens_q)
    B = cq.shape[0] - 1
    assert lens.shape == (B,) and bt.ndim == 2 and bt.shape[0] == B
    sk = _sinks(sinks, Hq)
    o = np.zeros((total_q, Hq, D), np.float64)
    lse = np.zeros((Hq, total_q), np.float64)
    rc = _load().oracle_attn_paged_varlen_fp8(_ptr(qb), _ptr(kb), _ptr(vb), k_scale, v_scale,
                                              _ptr(lens), _ptr(bt), int(page_size), _ptr(cq),
                                              int(bool(causal)), *_opt_args(window, softcap),
                                              None if sk is None else _ptr(sk), B, total_q, Hq,
                                              Hkv, D, bt.shape[1], _scale_arg(scale), dt,
                                              _ptr(o), _ptr(lse))
    if rc != 0:
        raise ValueError(f"oracle_attn_paged_varlen_fp8 rejected the call (rc={rc})")
    return o, lse


def _f64(x) -> np.ndarray:
    import torch
    if isinstance(x, torch.Tensor):
        x = x.detach().cpu().to(torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def attn_bwd(q, k, v, o, do, lse, *, scale=None, causal=True, dtype=None):
    """Gradients of the dense call: q/do [B,Sq,Hq,D] and k/v [B,Skv,Hkv,D] as
    bf16/fp16 tensors (or uint16 patterns with ``dtype``); o [B,Sq,Hq,D] and
    lse [B,Hq,Sq] as any floats (taken exactly, as float64).  Returns dq, dk, dv
    (float64)."""
    dt = _dtype_code(q) if dtype is None else dtype
    qb, kb, vb, dob = _bits(q), _bits(k), _bits(v), _bits(do)
    B, Sq, Hq, D = qb.shape
    _, Skv, Hkv, _ = kb.shape
    of, lf = _f64(o), _f64(lse)
    assert of.shape == (B, Sq, Hq, D) and lf.shape == (B, Hq, Sq)
    dq = np.zeros((B, Sq, Hq, D), np.float64)
    dk = np.zeros((B, Skv, Hkv, D), np.float64)
    dv = np.zeros((B, Skv, Hkv, D), np.float64)
    rc = _load().oracle_attn_bwd(_ptr(qb), _ptr(kb), _ptr(vb), _ptr(of), _ptr(dob), _ptr(lf), dt,
                                 B, Hq, Hkv, Sq, Skv, D, _scale_arg(scale), int(bool(causal)),
                                 _ptr(dq), _ptr(dk), _ptr(dv))
    if rc != 0:
        raise ValueError(f"oracle_attn_bwd rejected the call (rc={rc})")
    return dq, dk, dv


def e4m3_encode(x: float) -> int:
    """E4M3FN code of x (nearest, ties to even; NaN kept; |x| > 448 -> +-448)."""
    return _load().oracle_e4m3_encode(float(x))


def e4m3_decode(code: int) -> float:
    return _load().oracle_e4m3_decode(int(code))


def kv_write(k, v, k_pool, v_pool, slot_mapping, *, cache_fp8=False, k_scale=1.0,
             v_scale=1.0, dtype=None):
    """Scatter k/v [tokens,Hkv,D] into copies of the pools ([num_slots,Hkv,D] or
    [pages,page_size,Hkv,D]: uint16 bit patterns, or uint8 E4M3FN codes when
    cache_fp8); slot_mapping int64 [tokens], -1 skips.  Returns the new pools
    as numpy arrays of the pools' shapes."""
    dt = _dtype_code(k) if dtype is None else dtype
    kb, vb = _bits(k), _bits(v)
    tokens, Hkv, D = kb.shape
    import torch
    def pool_np(p):
        if isinstance(p, torch.Tensor):
            p = p.detach().cpu()
            p = p.view(torch.uint8) if cache_fp8 else p.view(torch.int16)
            p = p.numpy().view(np.uint8 if cache_fp8 else np.uint16)
        return np.ascontiguousarray(np.array(p, copy=True))
    kp, vp = pool_np(k_pool), pool_np(v_pool)
    num_slots = kp.size // (Hkv * D)
    sl = slot_mapping.detach().cpu().numpy() if isinstance(slot_mapping, torch.Tensor) \
        else np.asarray(slot_mapping)
    sl = np.ascontiguousarray(sl.astype(np.int64))
    rc = _load().oracle_kv_write(_ptr(kb), _ptr(vb), dt, _ptr(sl), tokens, Hkv, D, num_slots,
                                 int(bool(cache_fp8)), float(k_scale), float(v_scale), _ptr(kp),
                                 _ptr(vp))
    if rc != 0:
        raise ValueError(f"oracle_kv_write rejected the call (rc={rc})")
    return kp, vp


def attn_paged_append(q, k_new, v_new, k_cache, v_cache, cache_seqlens, block_table, page_size,
                      cu_seqlens_q, *, causal=True, softcap=None, scale=None, cache_fp8=False,
                      k_scale=1.0, v_scale=1.0, dtype=None):
    """Prefill with append: writes k_new/v_new [total_q,Hkv,D] at each request's
    positions cache_seqlens[b] + i (copies of the pools: 16-bit, or with cache_fp8
    E4M3FN codes of value / scale), then attends the packed queries to
    cache_seqlens[b] + Sq_b keys.  Returns o [total_q,Hq,D], lse [Hq,total_q] and
    the two updated pools (uint16, or uint8 codes, numpy arrays)."""
    dt = _dtype_code(q) if dtype is None else dtype
    qb, kb, vb = _bits(q), _bits(k_new), _bits(v_new)
    if cache_fp8:
        kc, vc = np.array(_codes(k_cache), copy=True), np.array(_codes(v_cache), copy=True)
    else:
        kc, vc = np.array(_bits(k_cache), copy=True), np.array(_bits(v_cache), copy=True)
    total_q, Hq, D = qb.shape
    Hkv = kb.shape[1]
    lens, bt, cq = _i32(cache_seqlens), _i32(block_table), _i32(cu_seqlens_q)
    B = cq.shape[0] - 1
    num_pages = kc.size // (page_size * Hkv * D)
    o = np.zeros((total_q, Hq, D), np.float64)
    lse = np.zeros((Hq, total_q), np.float64)
    rc = _load().oracle_attn_paged_append(_ptr(qb), _ptr(kb), _ptr(vb), _ptr(kc), _ptr(vc),
                                          int(bool(cache_fp8)), float(k_scale), float(v_scale),
                                          _ptr(lens), _ptr(bt), int(page_size), _ptr(cq),
                                          int(bool(causal)),
                                          0.0 if softcap is None else float(softcap), B,
                                          total_q, Hq, Hkv, D, bt.shape[1], num_pages,
                                          _scale_arg(scale), dt, _ptr(o), _ptr(lse))
    if rc != 0:
        raise ValueError(f"oracle_attn_paged_append rejected the call (rc={rc})")
    return o, lse, kc, vc


__all__ = ["BF16", "FP16", "build", "decode", "resolve_scale", "num_threads", "attn_dense",
           "attn_dense_rows", "attn_paged", "attn_paged_rows", "attn_varlen",
           "attn_paged_varlen", "e4m3_encode", "e4m3_decode", "kv_write", "attn_paged_append",
           "attn_bwd"]
