"""ctypes binding of libmiattn (include/miattn.h): argument marshalling only.

Every step of the attention runs in the library's HIP kernels; torch supplies
device memory and the current stream.  There is no fallback: if the library is
missing or a call is refused, an exception says why.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmiattn.so")

MIATTN_OK, MIATTN_ERR_INVALID_ARG, MIATTN_ERR_UNSUPPORTED, MIATTN_ERR_HIP = 0, 1, 2, 3
MIATTN_BF16, MIATTN_FP16 = 0, 1
MIATTN_CACHE_BF16, MIATTN_CACHE_FP16, MIATTN_CACHE_FP8_E4M3 = 0, 1, 2

# every symbol include/miattn.h declares
EXPORTS = ("attn_fwd_dense", "attn_fwd_dense_ex", "attn_fwd_paged", "attn_fwd_paged_ex",
           "attn_fwd_paged_noalloc",
           "attn_fwd_varlen", "attn_fwd_paged_varlen", "kv_cache_write", "attn_fwd_paged_append",
           "attn_bwd", "miattn_last_error", "miattn_release_workspace", "miattn_set_split_keys",
           "miattn_set_streamk_piece", "miattn_profile_start", "miattn_profile_stop")

_lib = None


class MiattnError(RuntimeError):
    """A HIP runtime failure reported by libmiattn."""


def lib() -> ctypes.CDLL:
    """Load libmiattn.so (built in-tree by softmax_attention_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m softmax_attention_amd.build` "
                "(or __graft_entry__.build()) first")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        L.attn_fwd_dense.argtypes = [P, P, P, i32, i32, i32, i32, i32, i32, f32, i32, P, P, P,
                                     i32, P]
        L.attn_fwd_dense.restype = i32
        L.attn_fwd_dense_ex.argtypes = [P, P, P, i32, i32, i32, i32, i32, i32, f32, i32, P, P,
                                        P, i32, i32, f32, i32, P]
        L.attn_fwd_dense_ex.restype = i32
        L.attn_fwd_paged.argtypes = [P, P, P, P, P, i32, i32, P, P, i32, i32, i32, i32, i32, i32,
                                     i32, f32, i32, P]
        L.attn_fwd_paged.restype = i32
        L.attn_fwd_paged_ex.argtypes = [P, P, P, P, P, i32, i32, P, P, i32, i32, i32, i32, i32,
                                        i32, i32, f32, i32, i32, f32, i32, P]
        L.attn_fwd_paged_ex.restype = i32
        L.attn_fwd_paged_noalloc.argtypes = L.attn_fwd_paged.argtypes
        L.attn_fwd_paged_noalloc.restype = i32
        L.attn_fwd_varlen.argtypes = [P, P, P, P, P, i32, i32, i32, i32, i32, i32, i32, i32, f32,
                                      i32, i32, i32, f32, P, P, P, i32, P]
        L.attn_fwd_varlen.restype = i32
        L.attn_fwd_paged_varlen.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, f32, P, P, P,
                                            i32, i32, i32, i32, i32, i32, i32, i32, f32, i32,
                                            i32, P, P, P]
        L.attn_fwd_paged_varlen.restype = i32
        i64 = ctypes.c_int64
        L.kv_cache_write.argtypes = [P, P, P, P, P, i32, i32, i32, i64, i32, i32, P, P, P]
        L.kv_cache_write.restype = i32
        L.attn_fwd_paged_append.argtypes = [P, P, P, P, P, P, P, P, i32, i32, f32, P, P, i32,
                                            i32, i32, i32, i32, i32, i32, i32, f32, i32, i32, P,
                                            P, P]
        L.attn_fwd_paged_append.restype = i32
        L.attn_bwd.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, i32, i32, f32, i32, P, P, P,
                               i32, P]
        L.attn_bwd.restype = i32
        L.miattn_last_error.argtypes = []
        L.miattn_last_error.restype = ctypes.c_char_p
        L.miattn_release_workspace.argtypes = []
        L.miattn_release_workspace.restype = i32
        L.miattn_set_split_keys.argtypes = [i32]
        L.miattn_set_split_keys.restype = None
        L.miattn_set_streamk_piece.argtypes = [i32]
        L.miattn_set_streamk_piece.restype = None
        L.miattn_profile_start.argtypes = []
        L.miattn_profile_start.restype = None
        L.miattn_profile_stop.argtypes = [ctypes.POINTER(ctypes.c_double),
                                          ctypes.POINTER(ctypes.c_int),
                                          ctypes.POINTER(ctypes.c_double),
                                          ctypes.POINTER(ctypes.c_int)]
        L.miattn_profile_stop.restype = i32
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status == MIATTN_OK:
        return
    msg = lib().miattn_last_error().decode()
    if status in (MIATTN_ERR_INVALID_ARG, MIATTN_ERR_UNSUPPORTED):
        raise ValueError(msg)
    raise MiattnError(msg)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MIATTN_BF16
    if t.dtype == torch.float16:
        return MIATTN_FP16
    raise ValueError(f"dtype {t.dtype} unsupported (bfloat16, float16)")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _scale(scale) -> float:
    return math.nan if scale is None else float(scale)


def _window(window) -> Tuple[int, int]:
    if window is None:
        return -1, -1
    wl, wr = window
    return int(wl), int(wr)


def _softcap(softcap) -> float:
    return 0.0 if softcap is None else float(softcap)


def _stream() -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _output(out: Optional[torch.Tensor], like: torch.Tensor) -> torch.Tensor:
    """The caller's output tensor, checked against the shape, dtype and device
    the kernels write (they write it in full, as dense row-major), or a new
    one."""
    if out is None:
        return torch.empty_like(like)
    if tuple(out.shape) != tuple(like.shape) or out.dtype != like.dtype:
        raise ValueError(f"out must be {like.dtype} {tuple(like.shape)}, got {out.dtype} "
                         f"{tuple(out.shape)}")
    if out.device != like.device or not out.is_contiguous():
        raise ValueError("out must be contiguous and on the queries' device")
    return out


def _lse_output(lse: Optional[torch.Tensor], shape, device, return_lse: bool):
    """The caller's float32 LSE tensor of `shape` (checked), a new one, or None."""
    if not return_lse:
        return None
    if lse is None:
        return torch.empty(shape, dtype=torch.float32, device=device)
    if lse.dtype != torch.float32 or tuple(lse.shape) != tuple(shape):
        raise ValueError(f"lse must be float32 {tuple(shape)}, got {lse.dtype} "
                         f"{tuple(lse.shape)}")
    if lse.device != device or not lse.is_contiguous():
        raise ValueError("lse must be contiguous and on the queries' device")
    return lse


def attn_fwd_dense(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, scale=None,
                   causal: bool = True, window=None, softcap=None,
                   key_padding_mask: Optional[torch.Tensor] = None,
                   out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                   return_lse: bool = True) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Dense attention forward on the current stream.

    q [B,Sq,Hq,D], k/v [B,Skv,Hkv,D] (bf16 or fp16, CUDA); window (w_L, w_R),
    -1 = unlimited side, None = no window; softcap None or 0 = plain logits;
    key_padding_mask [B,Skv] bool (True = keep).  Returns (o [B,Sq,Hq,D],
    lse [B,Hq,Sq] fp32)."""
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be rank 4 (BSHD)")
    if k.shape != v.shape or k.shape[0] != q.shape[0] or k.shape[3] != q.shape[3]:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)} k {tuple(k.shape)} "
                         f"v {tuple(v.shape)}")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share one dtype")
    code = _dtype_code(q)
    if not (q.is_cuda and k.device == q.device and v.device == q.device):
        raise ValueError("q, k, v must be on one GPU device")
    q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
    B, Sq, Hq, D = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    mask = None
    if key_padding_mask is not None:
        if tuple(key_padding_mask.shape) != (B, Skv):
            raise ValueError(f"key_padding_mask must be [B, Skv] = [{B}, {Skv}]")
        mask = key_padding_mask.to(device=q.device, dtype=torch.bool).contiguous()
        mask = mask.view(torch.uint8)
    o = _output(out, q)
    lse = _lse_output(lse, (B, Hq, Sq), q.device, return_lse)
    if window is None and not softcap:
        st = lib().attn_fwd_dense(_ptr(q), _ptr(k), _ptr(v), B, Hq, Hkv, Sq, Skv, D,
                                  _scale(scale), int(bool(causal)), _ptr(mask), _ptr(o),
                                  _ptr(lse), code, _stream())
    else:
        st = lib().attn_fwd_dense_ex(_ptr(q), _ptr(k), _ptr(v), B, Hq, Hkv, Sq, Skv, D,
                                     _scale(scale), int(bool(causal)), _ptr(mask), _ptr(o),
                                     _ptr(lse), *_window(window), _softcap(softcap), code,
                                     _stream())
    _check(st)
    return o, lse


def _paged_geometry(q, k_cache, v_cache, real_seqlen_kv, block_table, page_size):
    """Checks of a uniform paged call; returns (n_pages, Hkv, D, B, Sq, Hq)."""
    if q.dim() != 4:
        raise ValueError("q must be rank 4 (BSHD)")
    if k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache must have one shape")
    if k_cache.dim() == 4:
        if k_cache.shape[1] != page_size:
            raise ValueError("rank-4 caches must be [pages, page_size, Hkv, D]")
        n_pages = k_cache.shape[0]
    elif k_cache.dim() == 3:
        if k_cache.shape[0] % page_size != 0:
            raise ValueError("flat cache rows must be a multiple of page_size")
        n_pages = k_cache.shape[0] // page_size
    else:
        raise ValueError("caches must be rank 3 or 4")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("q and the caches must share one dtype")
    if real_seqlen_kv.dtype != torch.int32 or block_table.dtype != torch.int32:
        raise ValueError("real_seqlen_kv and block_table must be int32")
    _dtype_code(q)
    if not all(t.is_cuda and t.device == q.device
               for t in (q, k_cache, v_cache, real_seqlen_kv, block_table)):
        raise ValueError("q, the caches, real_seqlen_kv and block_table must be on one GPU device")
    B, Sq, Hq, D = q.shape
    Hkv = k_cache.shape[-2]
    if k_cache.shape[-1] != D:
        raise ValueError("head dim of the caches differs from q")
    if block_table.dim() != 2 or block_table.shape[0] != B or real_seqlen_kv.shape != (B,):
        raise ValueError("block_table must be [B, max_pages] and real_seqlen_kv [B]")
    return n_pages, Hkv, D, B, Sq, Hq


def attn_fwd_paged(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                   real_seqlen_kv: torch.Tensor, block_table: torch.Tensor, page_size: int, *,
                   causal: bool = True, scale=None, window=None, softcap=None,
                   out: Optional[torch.Tensor] = None,
                   lse: Optional[torch.Tensor] = None, return_lse: bool = True
                   ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Paged attention forward on the current stream.

    q [B,Sq,Hq,D]; k_cache/v_cache [pages*page_size, Hkv, D] or
    [pages, page_size, Hkv, D]; real_seqlen_kv int32 [B] (cache length, the Sq
    query tokens included); block_table int32 [B, max_pages]; window and
    softcap as for attn_fwd_dense, the window placed at each request's own
    query positions."""
    n_pages, Hkv, D, B, Sq, Hq = _paged_geometry(q, k_cache, v_cache, real_seqlen_kv,
                                                 block_table, page_size)
    code = _dtype_code(q)
    q = q.contiguous()
    k_cache, v_cache = k_cache.contiguous(), v_cache.contiguous()
    real_seqlen_kv, block_table = real_seqlen_kv.contiguous(), block_table.contiguous()
    o = _output(out, q)
    lse = _lse_output(lse, (B, Hq, Sq), q.device, return_lse)
    args = (_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(real_seqlen_kv), _ptr(block_table),
            int(page_size), int(bool(causal)), _ptr(o), _ptr(lse), B, Sq, Hq, Hkv, D,
            block_table.shape[1], n_pages, _scale(scale))
    if window is None and not softcap:
        st = lib().attn_fwd_paged(*args, code, _stream())
    else:
        st = lib().attn_fwd_paged_ex(*args, *_window(window), _softcap(softcap), code, _stream())
    _check(st)
    return o, lse


def attn_fwd_paged_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                           real_seqlen_kv: torch.Tensor, block_table: torch.Tensor,
                           page_size: int, *, out: torch.Tensor, lse: Optional[torch.Tensor],
                           causal: bool = True, scale=None) -> None:
    """attn_fwd_paged through the library's allocation-free entry point: the
    caller passes out (and lse, or None) already allocated; the split-KV
    partials go to the library's fixed per-GPU scratch (calls that overlap on
    one GPU race on it)."""
    if out is None:
        raise ValueError("out must be given: this entry point allocates nothing")
    n_pages, Hkv, D, B, Sq, Hq = _paged_geometry(q, k_cache, v_cache, real_seqlen_kv,
                                                 block_table, page_size)
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache),
                    ("real_seqlen_kv", real_seqlen_kv), ("block_table", block_table)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous: this entry point allocates nothing")
    o = _output(out, q)
    if lse is not None:
        lse = _lse_output(lse, (B, Hq, Sq), q.device, True)
    _check(lib().attn_fwd_paged_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache),
                                        _ptr(real_seqlen_kv), _ptr(block_table), int(page_size),
                                        int(bool(causal)), _ptr(o), _ptr(lse), B, Sq, Hq, Hkv, D,
                                        block_table.shape[1], n_pages, _scale(scale),
                                        _dtype_code(q), _stream()))


def _offsets(cu: torch.Tensor, device, name: str) -> torch.Tensor:
    if cu.dtype != torch.int32 or cu.dim() != 1 or cu.numel() < 1:
        raise ValueError(f"{name} must be a 1-D int32 tensor [B + 1]")
    if not (cu.is_cuda and cu.device == device):
        raise ValueError(f"{name} must be on the queries' GPU device")
    return cu.contiguous()


def _max_len(cu: torch.Tensor) -> int:
    # one device -> host read when the caller does not pass the maximum
    return int((cu[1:] - cu[:-1]).max().item()) if cu.numel() > 1 else 0


def _sinks_arg(sinks, Hq: int, device):
    if sinks is None:
        return None
    if sinks.dtype != torch.float32 or tuple(sinks.shape) != (Hq,):
        raise ValueError(f"sinks must be float32 [Hq] = [{Hq}]")
    if not (sinks.is_cuda and sinks.device == device):
        raise ValueError("sinks must be on the queries' GPU device")
    return sinks.contiguous()


def attn_fwd_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                    cu_seqlens_q: torch.Tensor, cu_seqlens_kv: torch.Tensor, *,
                    max_seqlen_q: Optional[int] = None, max_seqlen_kv: Optional[int] = None,
                    scale=None, causal: bool = True, window=None, softcap=None,
                    sinks: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                    lse: Optional[torch.Tensor] = None, return_lse: bool = True
                    ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Packed (THD) attention forward on the current stream.

    q [total_q,Hq,D], k/v [total_kv,Hkv,D]; cu_seqlens_q/kv int32 [B+1];
    sinks float32 [Hq] or None.  Returns (o [total_q,Hq,D], lse [Hq,total_q]).
    Without max_seqlen_q/kv the maxima are read from the offsets (a sync)."""
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k, v must be rank 3 (THD)")
    if k.shape != v.shape or k.shape[2] != q.shape[2]:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)} k {tuple(k.shape)} "
                         f"v {tuple(v.shape)}")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share one dtype")
    code = _dtype_code(q)
    if not (q.is_cuda and k.device == q.device and v.device == q.device):
        raise ValueError("q, k, v must be on one GPU device")
    cq = _offsets(cu_seqlens_q, q.device, "cu_seqlens_q")
    ck = _offsets(cu_seqlens_kv, q.device, "cu_seqlens_kv")
    if cq.numel() != ck.numel():
        raise ValueError("cu_seqlens_q and cu_seqlens_kv must both be [B + 1]")
    q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
    total_q, Hq, D = q.shape
    total_kv, Hkv = k.shape[0], k.shape[1]
    B = cq.numel() - 1
    mq = _max_len(cq) if max_seqlen_q is None else int(max_seqlen_q)
    mk = _max_len(ck) if max_seqlen_kv is None else int(max_seqlen_kv)
    sk = _sinks_arg(sinks, Hq, q.device)
    o = _output(out, q)
    lse = _lse_output(lse, (Hq, total_q), q.device, return_lse)
    st = lib().attn_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(cq), _ptr(ck), B, total_q,
                               total_kv, mq, mk, Hq, Hkv, D, _scale(scale), int(bool(causal)),
                               *_window(window), _softcap(softcap), _ptr(sk), _ptr(o),
                               _ptr(lse), code, _stream())
    _check(st)
    return o, lse


def _pool_kind(q, k_cache, v_cache, k_scale, v_scale):
    """(cache dtype code, k_scale, v_scale) of a pool pair: 16-bit pools of q's
    dtype, or torch.float8_e4m3fn pools with float32 [1] scales on q's device."""
    if k_cache.dtype != v_cache.dtype:
        raise ValueError("k and v pools must share one dtype")
    if k_cache.dtype == torch.float8_e4m3fn:
        for name, sc in (("k_scale", k_scale), ("v_scale", v_scale)):
            if sc is None or sc.dtype != torch.float32 or sc.numel() != 1 or sc.device != q.device:
                raise ValueError(f"an FP8 pool needs {name}: float32 [1] on the GPU")
        return MIATTN_CACHE_FP8_E4M3, k_scale.contiguous(), v_scale.contiguous()
    if k_cache.dtype != q.dtype:
        raise ValueError("q and 16-bit pools must share one dtype")
    return _dtype_code(q), None, None


def attn_fwd_paged_varlen(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                          cache_seqlens: torch.Tensor, block_table: torch.Tensor,
                          cu_seqlens_q: torch.Tensor, page_size: int, *,
                          max_seqlen_q: Optional[int] = None, causal: bool = True, scale=None,
                          window=None, softcap=None, sinks: Optional[torch.Tensor] = None,
                          k_scale: Optional[torch.Tensor] = None,
                          v_scale: Optional[torch.Tensor] = None,
                          out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                          return_lse: bool = True
                          ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Paged attention over packed queries on the current stream.

    q [total_q,Hq,D] delimited by cu_seqlens_q int32 [B+1]; caches, block_table
    and page_size as for attn_fwd_paged (torch.float8_e4m3fn pools take
    k_scale/v_scale float32 [1] on the device: element = code * scale);
    cache_seqlens int32 [B] (each request's keys, its queries included).
    Returns (o [total_q,Hq,D], lse [Hq,total_q])."""
    if q.dim() != 3:
        raise ValueError("q must be rank 3 (THD)")
    if k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache must have one shape")
    if k_cache.dim() == 4:
        if k_cache.shape[1] != page_size:
            raise ValueError("rank-4 caches must be [pages, page_size, Hkv, D]")
        n_pages = k_cache.shape[0]
    elif k_cache.dim() == 3:
        if k_cache.shape[0] % page_size != 0:
            raise ValueError("flat cache rows must be a multiple of page_size")
        n_pages = k_cache.shape[0] // page_size
    else:
        raise ValueError("caches must be rank 3 or 4")
    cache, k_scale, v_scale = _pool_kind(q, k_cache, v_cache, k_scale, v_scale)
    if cache_seqlens.dtype != torch.int32 or block_table.dtype != torch.int32:
        raise ValueError("cache_seqlens and block_table must be int32")
    code = _dtype_code(q)
    if not all(t.is_cuda and t.device == q.device
               for t in (q, k_cache, v_cache, cache_seqlens, block_table)):
        raise ValueError("q, the caches, cache_seqlens and block_table must be on one GPU device")
    cq = _offsets(cu_seqlens_q, q.device, "cu_seqlens_q")
    total_q, Hq, D = q.shape
    Hkv = k_cache.shape[-2]
    B = cq.numel() - 1
    if k_cache.shape[-1] != D:
        raise ValueError("head dim of the caches differs from q")
    if block_table.dim() != 2 or block_table.shape[0] != B or cache_seqlens.shape != (B,):
        raise ValueError("block_table must be [B, max_pages] and cache_seqlens [B]")
    mq = _max_len(cq) if max_seqlen_q is None else int(max_seqlen_q)
    sk = _sinks_arg(sinks, Hq, q.device)
    q = q.contiguous()
    k_cache, v_cache = k_cache.contiguous(), v_cache.contiguous()
    cache_seqlens, block_table = cache_seqlens.contiguous(), block_table.contiguous()
    o = _output(out, q)
    lse = _lse_output(lse, (Hq, total_q), q.device, return_lse)
    st = lib().attn_fwd_paged_varlen(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cache_seqlens),
                                     _ptr(block_table), _ptr(cq), int(page_size),
                                     int(bool(causal)), *_window(window), _softcap(softcap),
                                     _ptr(sk), _ptr(o), _ptr(lse), B,
                                     total_q, mq, Hq, Hkv, D, block_table.shape[1], n_pages,
                                     _scale(scale), code, cache, _ptr(k_scale), _ptr(v_scale),
                                     _stream())
    _check(st)
    return o, lse


def _pool_geometry(k_pages: torch.Tensor, Hkv: int, D: int) -> int:
    """Rows (num_slots) of a pool [num_slots,Hkv,D] or [pages,page_size,Hkv,D]."""
    if k_pages.dim() not in (3, 4) or tuple(k_pages.shape[-2:]) != (Hkv, D):
        raise ValueError(f"pools must be [rows, {Hkv}, {D}] or [pages, page_size, {Hkv}, {D}]")
    return k_pages.numel() // (Hkv * D)


def kv_cache_write(k: torch.Tensor, v: torch.Tensor, k_pages: torch.Tensor,
                   v_pages: torch.Tensor, slot_mapping: torch.Tensor, *,
                   k_scale: Optional[torch.Tensor] = None,
                   v_scale: Optional[torch.Tensor] = None) -> None:
    """Scatter k/v [tokens,Hkv,D] into the pools at slot_mapping (int64 [tokens],
    -1 skips), on the current stream.  Pools of torch.float8_e4m3fn store
    value / scale (k_scale/v_scale float32 [1] on the device)."""
    if k.dim() != 3 or k.shape != v.shape:
        raise ValueError("k and v must be [tokens, Hkv, D] of one shape")
    if k.dtype != v.dtype:
        raise ValueError("k and v must share one dtype")
    code = _dtype_code(k)
    tokens, Hkv, D = k.shape
    if k_pages.shape != v_pages.shape or k_pages.dtype != v_pages.dtype:
        raise ValueError("k_pages and v_pages must have one shape and dtype")
    fp8 = k_pages.dtype == torch.float8_e4m3fn
    if not fp8 and k_pages.dtype != k.dtype:
        raise ValueError("a 16-bit pool must have the dtype of k and v")
    cache = MIATTN_CACHE_FP8_E4M3 if fp8 else code
    if slot_mapping.dtype != torch.int64 or tuple(slot_mapping.shape) != (tokens,):
        raise ValueError("slot_mapping must be int64 [tokens]")
    dev = k.device
    if not all(t.is_cuda and t.device == dev for t in (k, v, k_pages, v_pages, slot_mapping)):
        raise ValueError("k, v, the pools and slot_mapping must be on one GPU device")
    if not (k_pages.is_contiguous() and v_pages.is_contiguous()):
        raise ValueError("the pools must be contiguous (they are written in place)")
    if fp8:
        for name, sc in (("k_scale", k_scale), ("v_scale", v_scale)):
            if sc is None or sc.dtype != torch.float32 or sc.numel() != 1 or sc.device != dev:
                raise ValueError(f"an FP8 pool needs {name}: float32 [1] on the GPU")
    k, v, slot_mapping = k.contiguous(), v.contiguous(), slot_mapping.contiguous()
    num_slots = _pool_geometry(k_pages, Hkv, D)
    _check(lib().kv_cache_write(_ptr(k), _ptr(v), _ptr(k_pages), _ptr(v_pages),
                                _ptr(slot_mapping), tokens, Hkv, D, num_slots, code, cache,
                                _ptr(k_scale) if fp8 else None, _ptr(v_scale) if fp8 else None,
                                _stream()))


def attn_fwd_paged_append(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                          k_cache: torch.Tensor, v_cache: torch.Tensor,
                          cache_seqlens: torch.Tensor, block_table: torch.Tensor,
                          cu_seqlens_q: torch.Tensor, page_size: int, *,
                          max_seqlen_q: Optional[int] = None, causal: bool = True, scale=None,
                          softcap=None, k_scale: Optional[torch.Tensor] = None,
                          v_scale: Optional[torch.Tensor] = None,
                          out: Optional[torch.Tensor] = None,
                          lse: Optional[torch.Tensor] = None, return_lse: bool = True
                          ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Paged prefill with append on the current stream: writes k_new/v_new
    [total_q,Hkv,D] after each request's cache_seqlens[b] cached keys (pools
    written in place: 16-bit, or torch.float8_e4m3fn storing value / scale with
    k_scale/v_scale float32 [1]), then attends the packed queries q
    [total_q,Hq,D] to cache_seqlens[b] + Sq_b keys.  Returns (o [total_q,Hq,D],
    lse [Hq,total_q])."""
    if q.dim() != 3 or k_new.dim() != 3 or k_new.shape != v_new.shape:
        raise ValueError("q, k_new, v_new must be rank 3 (THD), k_new and v_new of one shape")
    if k_new.shape[0] != q.shape[0] or k_new.shape[2] != q.shape[2]:
        raise ValueError("k_new/v_new must have q's token count and head dim")
    if k_new.dtype != q.dtype or v_new.dtype != q.dtype:
        raise ValueError("q, k_new, v_new must share one dtype")
    cache, k_scale, v_scale = _pool_kind(q, k_cache, v_cache, k_scale, v_scale)
    if not (k_cache.is_contiguous() and v_cache.is_contiguous()):
        raise ValueError("the pools must be contiguous (they are written in place)")
    code = _dtype_code(q)
    dev = q.device
    if not all(t.is_cuda and t.device == dev for t in (q, k_new, v_new, k_cache, v_cache,
                                                       cache_seqlens, block_table)):
        raise ValueError("all tensors must be on one GPU device")
    if cache_seqlens.dtype != torch.int32 or block_table.dtype != torch.int32:
        raise ValueError("cache_seqlens and block_table must be int32")
    cq = _offsets(cu_seqlens_q, dev, "cu_seqlens_q")
    total_q, Hq, D = q.shape
    Hkv = k_new.shape[1]
    B = cq.numel() - 1
    if block_table.dim() != 2 or block_table.shape[0] != B or cache_seqlens.shape != (B,):
        raise ValueError("block_table must be [B, max_pages] and cache_seqlens [B]")
    num_slots = _pool_geometry(k_cache, Hkv, D)
    if num_slots % page_size != 0:
        raise ValueError("pool rows must be a multiple of page_size")
    mq = _max_len(cq) if max_seqlen_q is None else int(max_seqlen_q)
    q, k_new, v_new = q.contiguous(), k_new.contiguous(), v_new.contiguous()
    cache_seqlens, block_table = cache_seqlens.contiguous(), block_table.contiguous()
    o = _output(out, q)
    lse = _lse_output(lse, (Hq, total_q), dev, return_lse)
    _check(lib().attn_fwd_paged_append(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
                                       _ptr(v_cache), _ptr(cache_seqlens), _ptr(block_table),
                                       _ptr(cq), int(page_size), int(bool(causal)),
                                       _softcap(softcap), _ptr(o),
                                       _ptr(lse), B, total_q, mq, Hq,
                                       Hkv, D, block_table.shape[1], num_slots // page_size,
                                       _scale(scale), code, cache, _ptr(k_scale),
                                       _ptr(v_scale), _stream()))
    return o, lse


def attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
             do: torch.Tensor, lse: torch.Tensor, *, scale=None, causal: bool = True
             ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Attention backward on the current stream: q/o/do [B,Sq,Hq,D], k/v
    [B,Skv,Hkv,D] (bf16 or fp16), lse [B,Hq,Sq] fp32 from attn_fwd_dense.
    Returns (dq, dk, dv) in the input dtype."""
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        if t.dim() != 4:
            raise ValueError(f"{name} must be rank 4 (BSHD)")
    if o.shape != q.shape or do.shape != q.shape or k.shape != v.shape:
        raise ValueError("o and do must have q's shape, v k's shape")
    if k.shape[0] != q.shape[0] or k.shape[3] != q.shape[3]:
        raise ValueError("q and k must agree on B and D")
    if any(t.dtype != q.dtype for t in (k, v, o, do)):
        raise ValueError("q, k, v, o, do must share one dtype")
    code = _dtype_code(q)
    B, Sq, Hq, D = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, Sq):
        raise ValueError(f"lse must be float32 [B, Hq, Sq] = [{B}, {Hq}, {Sq}]")
    dev = q.device
    if not all(t.is_cuda and t.device == dev for t in (q, k, v, o, do, lse)):
        raise ValueError("all tensors must be on one GPU device")
    q, k, v, o, do, lse = (t.contiguous() for t in (q, k, v, o, do, lse))
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    _check(lib().attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), B, Hq, Hkv,
                          Sq, Skv, D, _scale(scale), int(bool(causal)), _ptr(dq), _ptr(dk),
                          _ptr(dv), code, _stream()))
    return dq, dk, dv


def set_split_keys(keys_per_split: int) -> None:
    """Keys per split-KV partition (0 = automatic)."""
    lib().miattn_set_split_keys(int(keys_per_split))


def set_streamk_piece(tiles: int) -> None:
    """Stream-K decode plan weight of starting a piece, in key tiles (tests;
    a negative value restores the default)."""
    lib().miattn_set_streamk_piece(int(tiles))


def release_workspace() -> None:
    _check(lib().miattn_release_workspace())


def profile_start() -> None:
    lib().miattn_profile_start()


def profile_stop() -> dict:
    """Summed kernel durations (ms) and launch counts since profile_start()."""
    a_ms, m_ms = ctypes.c_double(), ctypes.c_double()
    a_n, m_n = ctypes.c_int(), ctypes.c_int()
    _check(lib().miattn_profile_stop(ctypes.byref(a_ms), ctypes.byref(a_n), ctypes.byref(m_ms),
                                     ctypes.byref(m_n)))
    return {"attn_ms": a_ms.value, "attn_launches": a_n.value, "merge_ms": m_ms.value,
            "merge_launches": m_n.value}
