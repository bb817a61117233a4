"""Exact attention forward for AMD MI355X (gfx950): Python binding of libfa.so.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI of ``include/fa.h``.  PyTorch supplies device memory
and the current stream.  The calls mirror the interface described on
"FlashAttention 常用接口简单介绍" (§3.1-§3.4):

* ``fwd(q, k, v, ...)``            -> (out, softmax_lse)   dense [B, S, H, D]
* ``fwd_varlen(q, k, v, cu_q, cu_k, max_q, max_k, ...)``   packed sequences
* ``fwd_kvcache(q, k_cache, v_cache, cache_seqlens, block_table=None, ...)``
* ``combine(out_partial, lse_partial)``
* ``bwd(dout, q, k, v, out, lse, ...)`` -> (dq, dk, dv)    gradients of ``fwd``
* ``bwd_varlen(dout, q, k, v, out, lse, cu_q, cu_k, max_q, max_k, ...)``  of ``fwd_varlen``
* ``attention(q, k, v, ...)``      -> out, differentiable (``fwd`` + ``bwd``)
* ``attention_varlen(q, k, v, cu_q, cu_k, max_q, max_k, ...)`` -> out, differentiable

There is no fallback: if libfa.so is missing or a tensor is not on the GPU the
call raises.
"""

from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["fwd", "fwd_varlen", "fwd_kvcache", "fwd_kvcache_noalloc", "combine", "bwd", "bwd_varlen", "attention", "attention_varlen", "kvcache_workspace_size",
           "kvcache_num_splits", "kvcache_noalloc_max_bytes", "bwd_workspace_size", "library_path", "load_library", "FaError"]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libfa.so")
_lib = None

FA_OK, FA_ERR_INVALID_ARGUMENT, FA_ERR_UNSUPPORTED, FA_ERR_WORKSPACE_TOO_SMALL, FA_ERR_HIP = range(5)
_DTYPES = {torch.float16: 0, torch.bfloat16: 1}


class FaError(RuntimeError):
    """A libfa call returned FA_ERR_HIP (or an unknown status)."""


class _Opts(ctypes.Structure):
    _fields_ = [("softmax_scale", ctypes.c_float), ("causal", ctypes.c_int),
                ("window_left", ctypes.c_int), ("window_right", ctypes.c_int),
                ("softcap", ctypes.c_float), ("alibi_slopes", ctypes.c_void_p), ("finite_cache", ctypes.c_int)]


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libfa.so (built by ``exact_attention_forward_fa_amd.build``), or the
    library the environment variable FA_LIBRARY names (the debug builds)."""
    global _lib
    if _lib is not None:
        return _lib
    _lib = bind_library(os.environ.get("FA_LIBRARY") or _LIB_PATH)
    return _lib


def bind_library(path: str):
    """ctypes handle of a build of the library at path, with the argument types set
    (load_library keeps one as the library every call uses)."""
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m exact_attention_forward_fa_amd.build`")
    lib = ctypes.CDLL(path)
    P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    I64P = ctypes.POINTER(ctypes.c_int64)
    OP = ctypes.POINTER(_Opts)
    lib.fa_fwd.argtypes = [I, P, P, P, P, P, I, I, I, I, I, I, I64P, I64P, I64P, I64P, OP, P]
    lib.fa_fwd.restype = I
    lib.fa_fwd_fp8.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I64P, I64P, I64P, I64P, F, F, F, OP, P]
    lib.fa_fwd_fp8.restype = I
    lib.fa_fwd_varlen.argtypes = [I, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I64P, I64P, I64P, I64P, OP, P]
    lib.fa_fwd_varlen.restype = I
    lib.fa_kvcache_workspace_size.argtypes = [I, I, I, I, I]
    lib.fa_kvcache_workspace_size.restype = Z
    lib.fa_kvcache_num_splits.argtypes = [I, I, I, I]
    lib.fa_kvcache_num_splits.restype = I
    lib.fa_fwd_kvcache.argtypes = [I, P, P, P, P, P, I, I, I, I, P, Z, P, P, I, I, I, I, I, OP, P]
    lib.fa_fwd_kvcache.restype = I
    lib.fa_fwd_kvcache_append.argtypes = [I, P, P, P, P, P, I, I, I, I, P, P, I, I64P, I64P, P, Z, P, P,
                                          I, I, I, I, I, OP, P]
    lib.fa_fwd_kvcache_append.restype = I
    lib.fa_kvcache_noalloc_max_bytes.argtypes = []
    lib.fa_kvcache_noalloc_max_bytes.restype = Z
    lib.fa_fwd_kvcache_noalloc.argtypes = [I, P, P, P, P, P, I, I, I, I, P, P, I, I, I, I, I, OP, P]
    lib.fa_fwd_kvcache_noalloc.restype = I
    lib.fa_combine.argtypes = [P, P, I, I, I, I, I, I64P, I64P, I, P, I64P, P, P]
    lib.fa_combine.restype = I
    lib.fa_bwd_workspace_size.argtypes = [I, I, I]
    lib.fa_bwd_workspace_size.restype = Z
    lib.fa_bwd.argtypes = [I, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I64P, I64P, I64P, I64P, I64P, OP, P, Z, P]
    lib.fa_bwd.restype = I
    lib.fa_bwd_varlen.argtypes = [I, P, P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I,
                                  I64P, I64P, I64P, I64P, I64P, OP, P, Z, P]
    lib.fa_bwd_varlen.restype = I
    lib.fa_status_string.argtypes = [I]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_last_error.argtypes = []
    lib.fa_last_error.restype = ctypes.c_char_p
    return lib


def _check(status: int):
    if status == FA_OK:
        return
    lib = load_library()
    msg = f"{lib.fa_status_string(status).decode()}: {lib.fa_last_error().decode()}"
    if status == FA_ERR_INVALID_ARGUMENT:
        raise ValueError(msg)
    if status in (FA_ERR_UNSUPPORTED, FA_ERR_WORKSPACE_TOO_SMALL):
        raise NotImplementedError(msg)
    raise FaError(msg)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _strides(t, dims):
    arr = (ctypes.c_int64 * len(dims))(*[t.stride(d) for d in dims])
    return arr


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _opts(softmax_scale, causal, window_size, softcap, alibi_slopes, device, Hq, finite_cache=False):
    if alibi_slopes is not None:
        if alibi_slopes.dtype != torch.float32 or not alibi_slopes.is_cuda or not alibi_slopes.is_contiguous():
            raise ValueError("alibi_slopes must be a contiguous float32 CUDA tensor")
        if alibi_slopes.device != device:
            raise ValueError("alibi_slopes must be on the same device as q")
        if alibi_slopes.numel() < Hq:
            raise ValueError(f"alibi_slopes holds {alibi_slopes.numel()} slopes for {Hq} query heads")
    if softmax_scale is not None and not float(softmax_scale) > 0.0:
        raise ValueError("softmax_scale must be positive (None selects 1/sqrt(head_dim))")
    o = _Opts(0.0 if softmax_scale is None else float(softmax_scale), int(bool(causal)),
              int(window_size[0]), int(window_size[1]), float(softcap),
              None if alibi_slopes is None else alibi_slopes.data_ptr(), int(bool(finite_cache)))
    return ctypes.byref(o), o


def _check_out(out, shape, dtype, device, name="out"):
    """A caller-supplied output: its shape, dtype and device must be those the call writes
    (the C ABI sees only a pointer and strides, so a wrong size would write out of bounds)."""
    if out is None:
        return
    if tuple(out.shape) != tuple(shape) or out.dtype != dtype or out.device != device:
        raise ValueError(f"{name} must be a {dtype} tensor of shape {tuple(shape)} on {device}, got "
                         f"{out.dtype} {tuple(out.shape)} on {out.device}")
    if out.stride(-1) != 1:
        raise ValueError(f"{name}: head_dim must be contiguous")


def _check_lse(lse, shape, device):
    if lse is None:
        return
    if tuple(lse.shape) != tuple(shape) or lse.dtype != torch.float32 or lse.device != device \
            or not lse.is_contiguous():
        raise ValueError(f"lse must be a contiguous float32 tensor of shape {tuple(shape)} on {device}")


def _need_gpu(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must be on the GPU")
    dev = ts[0].device
    for t in ts:
        if t is not None and t.device != dev:
            raise ValueError("all tensors must be on the same device")


def _unsupported_kwargs(dropout_p=0.0, return_attn_probs=False):
    if dropout_p:
        raise NotImplementedError("dropout_p != 0 is not part of this forward")
    if return_attn_probs:
        raise NotImplementedError("return_attn_probs is not supported")


def fwd(q, k, v, softmax_scale=None, causal=False, window_size=(-1, -1), softcap=0.0, alibi_slopes=None,
        out=None, lse=None, dropout_p=0.0, deterministic=False, return_attn_probs=False,
        q_descale=1.0, k_descale=1.0, v_descale=1.0):
    """Dense forward.  q [B,Sq,Hq,D], k/v [B,Sk,Hkv,D] fp16/bf16 on the GPU (D stride 1).

    Returns (out [B,Sq,Hq,D], softmax_lse [B,Hq,Sq] float32).  ``deterministic``
    is accepted and ignored: the forward is deterministic.

    float8_e4m3fn q, k, v (D 64 or 128) run the fp8 kernel and return bf16
    out; ``q_descale`` / ``k_descale`` / ``v_descale`` are per-tensor factors
    of the dequantised values (1 for a direct conversion).
    """
    _unsupported_kwargs(dropout_p, return_attn_probs)
    if q.dtype == torch.float8_e4m3fn:
        return _fwd_fp8(q, k, v, softmax_scale, causal, window_size, softcap, alibi_slopes, out, lse,
                        q_descale, k_descale, v_descale)
    if q.dtype not in _DTYPES or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share dtype float16 or bfloat16")
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4 or k.shape != v.shape:
        raise ValueError("expected q [B,Sq,Hq,D] and k, v [B,Sk,Hkv,D]")
    if q.stride(-1) != 1 or k.stride(-1) != 1 or v.stride(-1) != 1:
        raise ValueError("head_dim must be contiguous")
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    if k.shape[0] != B or k.shape[3] != D:
        raise ValueError("batch / head_dim mismatch")
    _check_out(out, q.shape, q.dtype, q.device)
    _check_lse(lse, (B, Hq, Sq), q.device)
    _need_gpu(q, k, v, out, lse)
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    if lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    lib = load_library()
    ob, keep = _opts(softmax_scale, causal, window_size, softcap, alibi_slopes, q.device, Hq)
    _check(lib.fa_fwd(_DTYPES[q.dtype], _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                      B, Sq, Sk, Hq, Hkv, D, _strides(q, (0, 1, 2)), _strides(k, (0, 1, 2)),
                      _strides(v, (0, 1, 2)), _strides(out, (0, 1, 2)), ob, _stream(q.device)))
    return out, lse


def _fwd_fp8(q, k, v, softmax_scale, causal, window_size, softcap, alibi_slopes, out, lse,
             q_descale, k_descale, v_descale):
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must all be float8_e4m3fn")
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4 or k.shape != v.shape:
        raise ValueError("expected q [B,Sq,Hq,D] and k, v [B,Sk,Hkv,D]")
    if q.stride(-1) != 1 or k.stride(-1) != 1 or v.stride(-1) != 1:
        raise ValueError("head_dim must be contiguous")
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    if k.shape[0] != B or k.shape[3] != D:
        raise ValueError("batch / head_dim mismatch")
    _check_out(out, q.shape, torch.bfloat16, q.device)     # fp8 inputs give a bfloat16 out
    _check_lse(lse, (B, Hq, Sq), q.device)
    _need_gpu(q, k, v, out, lse)
    if out is None:
        out = torch.empty((B, Sq, Hq, D), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    lib = load_library()
    ob, keep = _opts(softmax_scale, causal, window_size, softcap, alibi_slopes, q.device, Hq)
    _check(lib.fa_fwd_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Sq, Sk, Hq, Hkv, D,
                          _strides(q, (0, 1, 2)), _strides(k, (0, 1, 2)), _strides(v, (0, 1, 2)),
                          _strides(out, (0, 1, 2)), float(q_descale), float(k_descale), float(v_descale),
                          ob, _stream(q.device)))
    return out, lse


def fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, softmax_scale=None,
               causal=False, window_size=(-1, -1), softcap=0.0, alibi_slopes=None, out=None, lse=None,
               dropout_p=0.0, deterministic=False, return_attn_probs=False):
    """Packed forward.  q [total_q,Hq,D], k/v [total_k,Hkv,D], cu_seqlens int32 [B+1] on the GPU.

    Returns (out [total_q,Hq,D], softmax_lse [Hq,total_q] float32).
    """
    _unsupported_kwargs(dropout_p, return_attn_probs)
    if q.dtype not in _DTYPES or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share dtype float16 or bfloat16")
    if cu_seqlens_q.dtype != torch.int32 or cu_seqlens_k.dtype != torch.int32:
        raise ValueError("cu_seqlens must be int32")
    if q.dim() != 3 or k.dim() != 3 or k.shape != v.shape:
        raise ValueError("expected q [total_q,Hq,D] and k, v [total_k,Hkv,D]")
    if q.stride(-1) != 1 or k.stride(-1) != 1 or v.stride(-1) != 1:
        raise ValueError("head_dim must be contiguous")
    total_q, Hq, D = q.shape
    total_k, Hkv = k.shape[0], k.shape[1]
    if k.shape[2] != D:
        raise ValueError("head_dim mismatch")
    if cu_seqlens_q.dim() != 1 or cu_seqlens_k.dim() != 1:
        raise ValueError("cu_seqlens must be 1-D [B+1]")
    B = cu_seqlens_q.numel() - 1
    if cu_seqlens_k.numel() != B + 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
    _check_out(out, q.shape, q.dtype, q.device)
    _check_lse(lse, (Hq, total_q), q.device)
    _need_gpu(q, k, v, cu_seqlens_q, cu_seqlens_k, out, lse)
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    if lse is None:
        lse = torch.empty((Hq, total_q), dtype=torch.float32, device=q.device)
    lib = load_library()
    ob, keep = _opts(softmax_scale, causal, window_size, softcap, alibi_slopes, q.device, Hq)
    _check(lib.fa_fwd_varlen(_DTYPES[q.dtype], _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                             _ptr(cu_seqlens_q.contiguous()), _ptr(cu_seqlens_k.contiguous()), B,
                             int(max_seqlen_q), int(max_seqlen_k), total_q, total_k, Hq, Hkv, D,
                             _strides(q, (0, 1)), _strides(k, (0, 1)), _strides(v, (0, 1)),
                             _strides(out, (0, 1)), ob, _stream(q.device)))
    return out, lse


def kvcache_workspace_size(B, Sq, Hq, D, num_splits) -> int:
    return int(load_library().fa_kvcache_workspace_size(B, Sq, Hq, D, num_splits))


def kvcache_num_splits(B, Hkv, max_seqlen_k, num_splits=0) -> int:
    return int(load_library().fa_kvcache_num_splits(B, Hkv, max_seqlen_k, num_splits))


def _kvcache_shapes(q, k_cache, v_cache, cache_seqlens, block_table):
    """Shapes of a KV-cache call, checked; returns (B, Sq, Hq, D, Hkv, page, nblocks,
    block-table stride, cache capacity)."""
    if cache_seqlens.dtype != torch.int32:
        raise ValueError("cache_seqlens must be int32")
    for t in (q, k_cache, v_cache):
        if not t.is_contiguous():
            raise ValueError("q, k_cache and v_cache must be contiguous")
    if q.dim() != 4 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("expected q [B,Sq,Hq,D] and k_cache, v_cache of one shape [B,Smax,Hkv,D] or "
                         "[num_pages,page_size,Hkv,D]")
    B, Sq, Hq, D = q.shape
    Hkv = k_cache.shape[2]
    if k_cache.shape[3] != D:
        raise ValueError(f"cache head_dim {k_cache.shape[3]} differs from q's {D}")
    if cache_seqlens.dim() != 1 or cache_seqlens.numel() != B or not cache_seqlens.is_contiguous():
        raise ValueError(f"cache_seqlens must be contiguous int32 [B={B}]")
    if block_table is not None:
        if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.stride(1) != 1:
            raise ValueError("block_table must be int32 [B, max_pages] with unit last stride")
        if block_table.shape[0] != B:
            raise ValueError(f"block_table has {block_table.shape[0]} rows for B={B} sequences")
        page, nblocks, bts = k_cache.shape[1], k_cache.shape[0], block_table.stride(0)
        if block_table.shape[0] > 1 and bts < block_table.shape[1]:
            raise ValueError("block_table rows overlap")
        smax_bound = bts * page
    else:
        if k_cache.shape[0] != B:
            raise ValueError(f"dense k_cache has batch {k_cache.shape[0]}, q has {B}")
        page, nblocks, bts = 0, k_cache.shape[1], 0
        smax_bound = nblocks
    return B, Sq, Hq, D, Hkv, page, nblocks, bts, smax_bound


def fwd_kvcache(q, k_cache, v_cache, cache_seqlens, block_table=None, num_splits=0, softmax_scale=None,
                causal=False, window_size=(-1, -1), softcap=0.0, alibi_slopes=None, workspace=None,
                out=None, lse=None, k=None, v=None, cache_leftpad=None, cache_batch_idx=None,
                return_softmax_lse=True, finite_cache=False):
    """Decode against a dense [B,Smax,Hkv,D] cache, or a page pool [P,page,Hkv,D] with block_table int32 [B,maxp].

    Split-KV over ``num_splits`` chunks (0 = library heuristic) followed by the
    LSE combine.  Returns (out [B,Sq,Hq,D], softmax_lse [B,Hq,Sq]).

    With ``k`` and ``v`` ([B,S_new,Hkv,D]) the new tokens are first written into
    the caches in place at positions cache_seqlens[b] + t, and the queries
    attend to cache_seqlens[b] + S_new tokens; ``cache_seqlens`` itself is left
    unchanged.

    ``finite_cache=True`` promises that the K and V values of every attended
    token are finite; the decode
    at head_dim 32 or 64 may then read several adjacent kv heads as one work item
    (faster, but a non-finite value in one head would reach its neighbours).
    """
    if (k is None) != (v is None):
        raise ValueError("k and v must be given together")
    if cache_leftpad is not None or cache_batch_idx is not None:
        raise NotImplementedError("cache_leftpad / cache_batch_idx are not supported")
    if q.dtype not in _DTYPES or k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("q and the caches must share dtype float16 or bfloat16")
    B, Sq, Hq, D, Hkv, page, nblocks, bts, smax_bound = _kvcache_shapes(q, k_cache, v_cache, cache_seqlens,
                                                                         block_table)
    if k is not None:
        if k.dtype != q.dtype or v.dtype != q.dtype:
            raise ValueError("k and v must share the dtype of q")
        if k.dim() != 4 or k.shape != v.shape or k.shape[0] != B or k.shape[2] != Hkv or k.shape[3] != D:
            raise ValueError("k and v must be [B, S_new, Hkv, D]")
        if k.stride(-1) != 1 or v.stride(-1) != 1:
            raise ValueError("head_dim of k and v must be contiguous")
    _check_out(out, q.shape, q.dtype, q.device)
    if out is not None and not out.is_contiguous():
        raise ValueError("out must be contiguous")
    _check_lse(lse, (B, Hq, Sq), q.device)
    _need_gpu(q, k_cache, v_cache, cache_seqlens, block_table, k, v, out, lse, workspace)
    lib = load_library()
    ns = int(lib.fa_kvcache_num_splits(B, Hkv, smax_bound, int(num_splits)))
    need = int(lib.fa_kvcache_workspace_size(B, Sq, Hq, D, ns))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the device of q")
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    ob, keep = _opts(softmax_scale, causal, window_size, softcap, alibi_slopes, q.device, Hq, finite_cache)
    if k is None:
        _check(lib.fa_fwd_kvcache(_DTYPES[q.dtype], _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cache_seqlens),
                                  _ptr(block_table), bts, page, nblocks, ns, _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _ptr(out), _ptr(lse),
                                  B, Sq, Hq, Hkv, D, ob, _stream(q.device)))
    else:
        _check(lib.fa_fwd_kvcache_append(_DTYPES[q.dtype], _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                         _ptr(cache_seqlens), _ptr(block_table), bts, page, nblocks, ns,
                                         _ptr(k), _ptr(v), k.shape[1], _strides(k, (0, 1, 2)),
                                         _strides(v, (0, 1, 2)), _ptr(workspace),
                                         workspace.numel() * workspace.element_size(), _ptr(out), _ptr(lse),
                                         B, Sq, Hq, Hkv, D, ob, _stream(q.device)))
    return (out, lse) if return_softmax_lse else out


def fwd_kvcache_noalloc(q, k_cache, v_cache, cache_seqlens, out, lse, block_table=None, num_splits=0,
                        softmax_scale=None, causal=False, window_size=(-1, -1), softcap=0.0, alibi_slopes=None,
                        finite_cache=False):
    """``fwd_kvcache`` (without new keys) through the entry point that allocates
    nothing: the decode workspace is the library's static device array, and the
    caller passes ``out`` [B,Sq,Hq,D] and ``lse`` [B,Hq,Sq].  Calls that overlap
    in time on one GPU share that array and race.  Returns (out, lse)."""
    if out is None or lse is None:
        raise ValueError("fwd_kvcache_noalloc writes into caller-given out and lse")
    if q.dtype not in _DTYPES or k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("q and the caches must share dtype float16 or bfloat16")
    B, Sq, Hq, D, Hkv, page, nblocks, bts, _ = _kvcache_shapes(q, k_cache, v_cache, cache_seqlens, block_table)
    _check_out(out, q.shape, q.dtype, q.device)
    if not out.is_contiguous():
        raise ValueError("out must be contiguous")
    _check_lse(lse, (B, Hq, Sq), q.device)
    _need_gpu(q, k_cache, v_cache, cache_seqlens, block_table, out, lse)
    lib = load_library()
    ob, keep = _opts(softmax_scale, causal, window_size, softcap, alibi_slopes, q.device, Hq, finite_cache)
    _check(lib.fa_fwd_kvcache_noalloc(_DTYPES[q.dtype], _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cache_seqlens),
                                      _ptr(block_table), bts, page, nblocks, int(num_splits), _ptr(out), _ptr(lse),
                                      B, Sq, Hq, Hkv, D, ob, _stream(q.device)))
    return out, lse


def kvcache_noalloc_max_bytes() -> int:
    """Size of the static decode workspace behind ``fwd_kvcache_noalloc``."""
    return int(load_library().fa_kvcache_noalloc_max_bytes())


def combine(out_partial, lse_partial, out_dtype=None, out=None, lse=None):
    """Merge split partials: out_partial [B,S,H,D,n] and lse_partial [B,S,H,n] float32 (any strides).

    Returns (out [B,S,H,D] in out_dtype (default float16), lse [B,S,H] float32).
    """
    if out_partial.dtype != torch.float32 or lse_partial.dtype != torch.float32:
        raise ValueError("partials must be float32")
    B, S, H, D, n = out_partial.shape
    if tuple(lse_partial.shape) != (B, S, H, n):
        raise ValueError("lse_partial must be [B,S,H,num_splits]")
    out_dtype = out_dtype or (out.dtype if out is not None else torch.float16)
    if out_dtype not in _DTYPES:
        raise ValueError("out_dtype must be float16 or bfloat16")
    _check_out(out, (B, S, H, D), out_dtype, out_partial.device)
    if lse is not None and (tuple(lse.shape) != (B, S, H) or lse.dtype != torch.float32
                            or lse.device != out_partial.device or not lse.is_contiguous()):
        raise ValueError(f"lse must be a contiguous float32 tensor of shape {(B, S, H)}")
    _need_gpu(out_partial, lse_partial, out, lse)
    if out is None:
        out = torch.empty((B, S, H, D), dtype=out_dtype, device=out_partial.device)
    if lse is None:
        lse = torch.empty((B, S, H), dtype=torch.float32, device=out_partial.device)
    lib = load_library()
    _check(lib.fa_combine(_ptr(out_partial), _ptr(lse_partial), B, S, H, D, n,
                          _strides(out_partial, (0, 1, 2, 3, 4)), _strides(lse_partial, (0, 1, 2, 3)),
                          _DTYPES[out.dtype], _ptr(out), _strides(out, (0, 1, 2)), _ptr(lse),
                          _stream(out_partial.device)))
    return out, lse


def bwd_workspace_size(B: int, Sq: int, Hq: int) -> int:
    """Bytes of device workspace ``bwd`` needs (the float32 row sums dout·out)."""
    return int(load_library().fa_bwd_workspace_size(B, Sq, Hq))


def bwd(dout, q, k, v, out, lse, softmax_scale=None, causal=False, window_size=(-1, -1), softcap=0.0,
        alibi_slopes=None, dq=None, dk=None, dv=None, workspace=None, deterministic=True):
    """Gradients of ``fwd``: returns (dq [B,Sq,Hq,D], dk, dv [B,Sk,Hkv,D]) for the
    gradient ``dout`` of ``out``.  ``out`` and ``lse`` are what ``fwd`` returned
    for the same q, k, v and options.  D is 32, 64, 96, 128 or 256.  The kernels are
    deterministic (``deterministic`` is accepted for interface parity)."""
    _need_gpu(dout, q, k, v, out, lse)
    if q.dtype not in _DTYPES or any(t.dtype != q.dtype for t in (k, v, out, dout)):
        raise ValueError("dout, q, k, v, out must share dtype float16 or bfloat16")
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4 or k.shape != v.shape or out.shape != q.shape \
            or dout.shape != q.shape:
        raise ValueError("expected q, out, dout [B,Sq,Hq,D] and k, v [B,Sk,Hkv,D]")
    if any(t.stride(-1) != 1 for t in (dout, q, k, v, out)):
        raise ValueError("head_dim must be contiguous")
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    if k.shape[0] != B or k.shape[3] != D:
        raise ValueError("batch / head_dim mismatch")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, Sq) or not lse.is_contiguous():
        raise ValueError("lse must be contiguous float32 [B, Hq, Sq]")
    for name, t, shape in (("dq", dq, q.shape), ("dk", dk, k.shape), ("dv", dv, k.shape)):
        if t is not None and (t.shape != shape or t.dtype != q.dtype or not t.is_contiguous()
                              or t.device != q.device):
            raise ValueError(f"{name} must be a contiguous tensor like its input")
    dq = torch.empty(q.shape, dtype=q.dtype, device=q.device) if dq is None else dq
    dk = torch.empty(k.shape, dtype=q.dtype, device=q.device) if dk is None else dk
    dv = torch.empty(k.shape, dtype=q.dtype, device=q.device) if dv is None else dv
    lib = load_library()
    need = int(lib.fa_bwd_workspace_size(B, Sq, Hq))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    ob, keep = _opts(softmax_scale, causal, window_size, softcap, alibi_slopes, q.device, Hq)
    _check(lib.fa_bwd(_DTYPES[q.dtype], _ptr(dout), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                      _ptr(dq), _ptr(dk), _ptr(dv), B, Sq, Sk, Hq, Hkv, D,
                      _strides(q, (0, 1, 2)), _strides(k, (0, 1, 2)), _strides(v, (0, 1, 2)),
                      _strides(out, (0, 1, 2)), _strides(dout, (0, 1, 2)), ob,
                      _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(q.device)))
    return dq, dk, dv


def bwd_varlen(dout, q, k, v, out, lse, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
               softmax_scale=None, causal=False, window_size=(-1, -1), softcap=0.0, alibi_slopes=None,
               dq=None, dk=None, dv=None, workspace=None, deterministic=True):
    """Gradients of ``fwd_varlen``: returns (dq [total_q,Hq,D], dk, dv [total_k,Hkv,D]).
    ``out`` and ``lse`` ([Hq, total_q]) are what ``fwd_varlen`` returned."""
    _need_gpu(dout, q, k, v, out, lse, cu_seqlens_q, cu_seqlens_k)
    if q.dtype not in _DTYPES or any(t.dtype != q.dtype for t in (k, v, out, dout)):
        raise ValueError("dout, q, k, v, out must share dtype float16 or bfloat16")
    if cu_seqlens_q.dtype != torch.int32 or cu_seqlens_k.dtype != torch.int32:
        raise ValueError("cu_seqlens must be int32")
    if q.dim() != 3 or k.dim() != 3 or k.shape != v.shape or out.shape != q.shape or dout.shape != q.shape:
        raise ValueError("expected q, out, dout [total_q,Hq,D] and k, v [total_k,Hkv,D]")
    if any(t.stride(-1) != 1 for t in (dout, q, k, v, out)):
        raise ValueError("head_dim must be contiguous")
    total_q, Hq, D = q.shape
    total_k, Hkv = k.shape[0], k.shape[1]
    B = cu_seqlens_q.numel() - 1
    if cu_seqlens_k.numel() != B + 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (Hq, total_q) or not lse.is_contiguous():
        raise ValueError("lse must be contiguous float32 [Hq, total_q]")
    for name, t, shape in (("dq", dq, q.shape), ("dk", dk, k.shape), ("dv", dv, k.shape)):
        if t is not None and (t.shape != shape or t.dtype != q.dtype or not t.is_contiguous()
                              or t.device != q.device):
            raise ValueError(f"{name} must be a contiguous tensor like its input")
    dq = torch.empty(q.shape, dtype=q.dtype, device=q.device) if dq is None else dq
    dk = torch.empty(k.shape, dtype=q.dtype, device=q.device) if dk is None else dk
    dv = torch.empty(k.shape, dtype=q.dtype, device=q.device) if dv is None else dv
    lib = load_library()
    need = int(lib.fa_bwd_workspace_size(1, total_q, Hq))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    ob, keep = _opts(softmax_scale, causal, window_size, softcap, alibi_slopes, q.device, Hq)
    _check(lib.fa_bwd_varlen(_DTYPES[q.dtype], _ptr(dout), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                             _ptr(dq), _ptr(dk), _ptr(dv), _ptr(cu_seqlens_q.contiguous()),
                             _ptr(cu_seqlens_k.contiguous()), B, int(max_seqlen_q), int(max_seqlen_k),
                             total_q, total_k, Hq, Hkv, D, _strides(q, (0, 1)), _strides(k, (0, 1)),
                             _strides(v, (0, 1)), _strides(out, (0, 1)), _strides(dout, (0, 1)), ob,
                             _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(q.device)))
    return dq, dk, dv


class _Attention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, softmax_scale, causal, window_size, softcap, alibi_slopes):
        out, lse = fwd(q, k, v, softmax_scale=softmax_scale, causal=causal, window_size=window_size,
                       softcap=softcap, alibi_slopes=alibi_slopes)
        ctx.save_for_backward(q, k, v, out, lse)
        ctx.opts = (softmax_scale, causal, window_size, softcap, alibi_slopes)
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k, v, out, lse = ctx.saved_tensors
        softmax_scale, causal, window_size, softcap, alibi_slopes = ctx.opts
        dq, dk, dv = bwd(dout.contiguous(), q, k, v, out, lse, softmax_scale=softmax_scale, causal=causal,
                         window_size=window_size, softcap=softcap, alibi_slopes=alibi_slopes)
        return dq, dk, dv, None, None, None, None, None


def attention(q, k, v, softmax_scale=None, causal=False, window_size=(-1, -1), softcap=0.0, alibi_slopes=None):
    """Differentiable dense attention: ``fwd`` forward, ``bwd`` backward (weights
    recomputed from the saved lse).  Returns out [B, Sq, Hq, D]."""
    return _Attention.apply(q, k, v, softmax_scale, causal, tuple(window_size), softcap, alibi_slopes)


class _AttentionVarlen(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, softmax_scale, causal,
                window_size, softcap, alibi_slopes):
        out, lse = fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                              softmax_scale=softmax_scale, causal=causal, window_size=window_size,
                              softcap=softcap, alibi_slopes=alibi_slopes)
        ctx.save_for_backward(q, k, v, out, lse, cu_seqlens_q, cu_seqlens_k)
        ctx.opts = (max_seqlen_q, max_seqlen_k, softmax_scale, causal, window_size, softcap, alibi_slopes)
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k, v, out, lse, cu_q, cu_k = ctx.saved_tensors
        max_q, max_k, softmax_scale, causal, window_size, softcap, alibi_slopes = ctx.opts
        dq, dk, dv = bwd_varlen(dout.contiguous(), q, k, v, out, lse, cu_q, cu_k, max_q, max_k,
                                softmax_scale=softmax_scale, causal=causal, window_size=window_size,
                                softcap=softcap, alibi_slopes=alibi_slopes)
        return dq, dk, dv, None, None, None, None, None, None, None, None, None


def attention_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, softmax_scale=None,
                     causal=False, window_size=(-1, -1), softcap=0.0, alibi_slopes=None):
    """Differentiable packed attention: ``fwd_varlen`` forward, ``bwd_varlen``
    backward.  Returns out [total_q, Hq, D]."""
    return _AttentionVarlen.apply(q, k, v, cu_seqlens_q, cu_seqlens_k, int(max_seqlen_q), int(max_seqlen_k),
                                  softmax_scale, causal, tuple(window_size), softcap, alibi_slopes)
