"""varlen_paged_kv_amd: varlen attention over a paged KV cache on MI355X (gfx950).

Thin Python binding over libvpk.so (C ABI in include/vpk.h).  PyTorch supplies
device memory and the current HIP stream; every step of the computation (the
in-place append, the page gather, both MFMA contractions, the online softmax,
the split merge) runs in the library's HIP kernels.  There is no fallback: if
the library is missing or the tensors are not on a GPU, the calls raise.

    out, lse = attn_varlen_paged_fwd(q, cu_seqlens_q, k_new, v_new, cu_seqlens_knew,
                                     k_cache, v_cache, block_table, cache_seqlens,
                                     page_size, causal, scale, kv_scale)
"""
from __future__ import annotations

import ctypes
import math
from typing import Optional, Sequence

import numpy as np
import torch

from . import _lib
from ._lib import VpkDims, VpkHostIndex, VpkHostPages

__all__ = ["attn_varlen_paged_fwd_noalloc", "set_workspace", "workspace_bytes_upper_bound", "library_memory", "attn_varlen_paged_fwd", "attn_varlen_paged_list_fwd", "kv_cache_append", "VpkError", "set_option", "abi_version",
           "timing_enable", "timing_reset", "timing_read", "device_error", "plan_debug", "Plan",
           "KERNEL_ATTENTION", "KERNEL_APPEND", "KERNEL_ATTENTION_DECODE", "KERNEL_MERGE", "KERNEL_ROPE",
           "KERNEL_ATTENTION_MIXED", "KERNEL_ATTENTION_PROB8",
           "attn_varlen_paged_rope_fwd", "attn_varlen_paged_qkv_prob_fwd"]

# kernel ids of the timing API: the prefill-mode attention grid, the standalone
# append, the decode-mode attention grid, the split merge, the rotary copies,
# the mixed attention grid (both kinds of items in one launch), the fp8
# QKV-Prob attention grid
KERNEL_ATTENTION, KERNEL_APPEND, KERNEL_ATTENTION_DECODE, KERNEL_MERGE, KERNEL_ROPE, KERNEL_ATTENTION_MIXED = \
    0, 1, 2, 3, 4, 5
KERNEL_ATTENTION_PROB8 = 6


class VpkError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_lib.STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status
        self.msg = msg


def _check(status: int):
    if status != _lib.VPK_SUCCESS:
        raise VpkError(status, _lib.load().vpk_last_error().decode(errors="replace"))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t: Optional[torch.Tensor], name: str, dtypes) -> Optional[torch.Tensor]:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise VpkError(_lib.VPK_ERROR_INVALID_VALUE, f"{name} must be a GPU tensor")
    if t.dtype not in dtypes:
        raise VpkError(_lib.VPK_ERROR_INVALID_VALUE, f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise VpkError(_lib.VPK_ERROR_INVALID_VALUE, f"{name} must be contiguous")
    return t


def _out_lse(out, lse, Tq, Hq, D, device):
    """Validate caller-supplied outputs: out bf16 [Tq, Hq, D], lse fp32 [Hq, Tq], contiguous, on q's device
    (the kernels write them densely with these shapes)."""
    if out is not None:
        out = _dev(out, "out", _BF16)
        if tuple(out.shape) != (Tq, Hq, D):
            raise VpkError(_lib.VPK_ERROR_INVALID_VALUE, f"out has shape {tuple(out.shape)}, expected {(Tq, Hq, D)}")
        if out.device != device:
            raise VpkError(_lib.VPK_ERROR_INVALID_VALUE, f"out is on {out.device}, q on {device}")
    if lse is not None:
        lse = _dev(lse, "lse", (torch.float32,))
        if tuple(lse.shape) != (Hq, Tq):
            raise VpkError(_lib.VPK_ERROR_INVALID_VALUE, f"lse has shape {tuple(lse.shape)}, expected {(Hq, Tq)}")
        if lse.device != device:
            raise VpkError(_lib.VPK_ERROR_INVALID_VALUE, f"lse is on {lse.device}, q on {device}")
    return out, lse


def _same_device(device, **tensors):
    for name, t in tensors.items():
        if t is not None and t.device != device:
            raise VpkError(_lib.VPK_ERROR_INVALID_VALUE, f"{name} is on {t.device}, q on {device}")


def _length(name, n, expected):
    if n != expected:
        raise VpkError(_lib.VPK_ERROR_INVALID_VALUE, f"{name} has {n} entries, expected {expected}")


def _host_i32(x) -> Optional[np.ndarray]:
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


_BF16 = (torch.bfloat16,)
_I32 = (torch.int32,)
_FP8 = (torch.uint8, torch.float8_e4m3fn)


def _stream_handle(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(int(stream.cuda_stream))


# Device workspace of each (device, stream) the binding has called on: a torch
# uint8 tensor registered with vpk_set_workspace, so that PyTorch owns the
# library's scratch memory (split partials, error flag, rope copies).
_WORKSPACES = {}
# set to False to leave streams without a caller workspace (the library then uses its own)
AUTO_WORKSPACE = True


def workspace_bytes_upper_bound(dims: VpkDims, rope: bool = False, num_cus: int = 0) -> int:
    """Device bytes that suffice for the workspace of any call with these sizes."""
    return int(_lib.load().vpk_workspace_bytes_upper_bound(ctypes.byref(dims), int(num_cus), int(bool(rope))))


def set_workspace(buf: Optional[torch.Tensor], stream=None):
    """Use ``buf`` (a contiguous device tensor, 256-byte aligned) as the workspace of the calls on
    ``stream``; None goes back to the library's own.  The binding manages one per stream by itself;
    this is for callers that bring their own."""
    h = _stream_handle(stream)
    if buf is None:
        _check(_lib.load().vpk_set_workspace(h, None, 0))
        return
    if not buf.is_cuda or not buf.is_contiguous():
        raise VpkError(_lib.VPK_ERROR_INVALID_VALUE, "the workspace must be a contiguous GPU tensor")
    _check(_lib.load().vpk_set_workspace(h, ctypes.c_void_p(buf.data_ptr()), buf.numel() * buf.element_size()))


def library_memory():
    """(device bytes, pinned host bytes) the library holds on its own (fallback workspaces, plan buffers)."""
    d, h = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check(_lib.load().vpk_library_memory(ctypes.byref(d), ctypes.byref(h)))
    return d.value, h.value


def _ensure_workspace(dims: VpkDims, device, stream_handle, rope: bool = False, extra: int = 0):
    """Register a torch-allocated workspace of at least the bound for this call's sizes (plus ``extra``
    bytes) on its stream (grown by replacing it: the old tensor goes back to torch's allocator in the
    stream's order)."""
    if not AUTO_WORKSPACE:
        return
    need = workspace_bytes_upper_bound(dims, rope) + int(extra)
    key = (device.index, stream_handle.value)
    cur = _WORKSPACES.get(key)
    if cur is not None and cur.numel() >= need:
        return
    size = max(need + need // 4, 1 << 20)
    size = (size + 4095) // 4096 * 4096
    ext = torch.cuda.ExternalStream(stream_handle.value, device=device) if stream_handle.value else None
    if ext is not None:
        with torch.cuda.stream(ext):
            buf = torch.empty(size, dtype=torch.uint8, device=device)
    else:
        buf = torch.empty(size, dtype=torch.uint8, device=device)
    _check(_lib.load().vpk_set_workspace(stream_handle, ctypes.c_void_p(buf.data_ptr()), size))
    _WORKSPACES[key] = buf


def _host_index(cu_q, cu_kn, cache_lens, block_table):
    keep = [_host_i32(cu_q), _host_i32(cu_kn), _host_i32(cache_lens), _host_i32(block_table)]
    hi = VpkHostIndex(*[None if a is None else a.ctypes.data for a in keep])
    return hi, keep


def attn_varlen_paged_fwd(q: torch.Tensor, cu_seqlens_q: torch.Tensor,
                          k_new: Optional[torch.Tensor] = None, v_new: Optional[torch.Tensor] = None,
                          cu_seqlens_knew: Optional[torch.Tensor] = None,
                          k_cache: Optional[torch.Tensor] = None, v_cache: Optional[torch.Tensor] = None,
                          block_table: Optional[torch.Tensor] = None,
                          cache_seqlens: Optional[torch.Tensor] = None,
                          page_size: int = 0, causal: bool = True, scale: Optional[float] = None,
                          kv_scale: Optional[Sequence[float]] = None, *,
                          out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                          return_lse: bool = True, host_index: Optional[dict] = None,
                          stream=None):
    """Append k_new/v_new into the paged cache (if both are given), then attend.

    Shapes: q [Tq, Hq, D] bf16; k_new/v_new [Tn, Hkv, D] bf16; caches
    [P, S, Hkv, D] bf16 or fp8 e4m3fn (uint8 / float8_e4m3fn); block_table
    [B, max_pages] int32; cu_seqlens_* [B + 1] int32; cache_seqlens [B] int32.
    ``host_index`` may hold host copies (CPU tensors or arrays) under the keys
    cu_seqlens_q, cu_seqlens_knew, cache_seqlens, block_table; missing ones are
    read back from the device by the library (a blocking copy).
    Returns (out [Tq, Hq, D] bf16, lse [Hq, Tq] fp32 or None).
    """
    return _attn_dense(q, cu_seqlens_q, k_new, v_new, cu_seqlens_knew, k_cache, v_cache, block_table,
                       cache_seqlens, page_size, causal, scale, kv_scale, out, lse, return_lse, host_index,
                       stream, None)


def attn_varlen_paged_fwd_noalloc(q: torch.Tensor, cu_seqlens_q: torch.Tensor,
                                  k_new: Optional[torch.Tensor] = None, v_new: Optional[torch.Tensor] = None,
                                  cu_seqlens_knew: Optional[torch.Tensor] = None,
                                  k_cache: Optional[torch.Tensor] = None, v_cache: Optional[torch.Tensor] = None,
                                  block_table: Optional[torch.Tensor] = None,
                                  cache_seqlens: Optional[torch.Tensor] = None,
                                  page_size: int = 0, causal: bool = True, scale: Optional[float] = None,
                                  kv_scale: Optional[Sequence[float]] = None, *,
                                  out: torch.Tensor, lse: Optional[torch.Tensor] = None,
                                  host_index: dict, stream=None):
    """attn_varlen_paged_fwd through the allocation-free entry point: the caller passes ``out`` (and
    ``lse`` to get it) and host copies of every index array in ``host_index``; the library's
    static device scratch holds the work list and the split partials.  Returns (out, lse)."""
    if out is None:
        raise VpkError(_lib.VPK_ERROR_INVALID_VALUE, "the allocation-free call writes into a given out")
    return _attn_dense(q, cu_seqlens_q, k_new, v_new, cu_seqlens_knew, k_cache, v_cache, block_table,
                       cache_seqlens, page_size, causal, scale, kv_scale, out, lse, lse is not None, host_index,
                       stream, None, noalloc=True)


def attn_varlen_paged_rope_fwd(q: torch.Tensor, cu_seqlens_q: torch.Tensor,
                               k_new: Optional[torch.Tensor] = None, v_new: Optional[torch.Tensor] = None,
                               cu_seqlens_knew: Optional[torch.Tensor] = None,
                               k_cache: Optional[torch.Tensor] = None, v_cache: Optional[torch.Tensor] = None,
                               block_table: Optional[torch.Tensor] = None,
                               cache_seqlens: Optional[torch.Tensor] = None,
                               page_size: int = 0, causal: bool = True, scale: Optional[float] = None,
                               kv_scale: Optional[Sequence[float]] = None, *,
                               rope_cos: torch.Tensor, rope_sin: torch.Tensor,
                               rotary_dim: Optional[int] = None, interleaved: bool = False,
                               out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                               return_lse: bool = True, host_index: Optional[dict] = None,
                               stream=None):
    """attn_varlen_paged_fwd with the query rows and new key rows turned by
    rotary embedding first (new token j at Lc + j, query row i at Lk - Lq + i).

    rope_cos / rope_sin: device float32 [max_positions, rotary_dim / 2];
    rotary_dim defaults to twice their width.  q and k_new are not modified;
    the cache stores the turned keys.
    """
    return _attn_dense(q, cu_seqlens_q, k_new, v_new, cu_seqlens_knew, k_cache, v_cache, block_table,
                       cache_seqlens, page_size, causal, scale, kv_scale, out, lse, return_lse, host_index,
                       stream, _rope_args(rope_cos, rope_sin, rotary_dim, interleaved))


def _rope_args(rope_cos, rope_sin, rotary_dim, interleaved):
    """(VpkRope, cos, sin): the C struct and the tensors it points into."""
    rope_cos = _dev(rope_cos, "rope_cos", (torch.float32,))
    rope_sin = _dev(rope_sin, "rope_sin", (torch.float32,))
    if rope_cos is None or rope_sin is None:
        raise VpkError(_lib.VPK_ERROR_INVALID_VALUE, "rope_cos and rope_sin must both be given")
    if rope_cos.dim() != 2 or tuple(rope_sin.shape) != tuple(rope_cos.shape):
        raise VpkError(_lib.VPK_ERROR_INVALID_VALUE, "rope_cos / rope_sin must both be [max_positions, rotary_dim / 2]")
    if rotary_dim is None:
        rotary_dim = 2 * rope_cos.shape[1]
    if 2 * rope_cos.shape[1] != rotary_dim:
        raise VpkError(_lib.VPK_ERROR_INVALID_VALUE, "rope tables must have rotary_dim / 2 columns")
    rope = _lib.VpkRope(_ptr(rope_cos), _ptr(rope_sin), rope_cos.shape[0], int(rotary_dim), int(bool(interleaved)))
    return rope, rope_cos, rope_sin


def attn_varlen_paged_qkv_prob_fwd(q: torch.Tensor, cu_seqlens_q: torch.Tensor,
                                   k_new: Optional[torch.Tensor] = None, v_new: Optional[torch.Tensor] = None,
                                   cu_seqlens_knew: Optional[torch.Tensor] = None,
                                   k_cache: Optional[torch.Tensor] = None, v_cache: Optional[torch.Tensor] = None,
                                   block_table: Optional[torch.Tensor] = None,
                                   cache_seqlens: Optional[torch.Tensor] = None,
                                   page_size: int = 0, causal: bool = True, scale: Optional[float] = None,
                                   kv_scale: Optional[Sequence[float]] = None, *,
                                   q_scale: float, p_scale: float = 1.0 / 448.0,
                                   rope_cos: Optional[torch.Tensor] = None, rope_sin: Optional[torch.Tensor] = None,
                                   rotary_dim: Optional[int] = None, interleaved: bool = False,
                                   out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                                   return_lse: bool = True, host_index: Optional[dict] = None,
                                   stream=None):
    """attn_varlen_paged_fwd in fp8 "QKV-Prob" form (fp8 cache only): the query
    rows are quantised to e4m3fn with ``q_scale``, the softmax output to
    e4m3fn with ``p_scale`` before the second product, and both products run
    on fp8 matrix cores.  ``rope_cos`` / ``rope_sin`` (optional) turn the
    query rows and new key rows first, as attn_varlen_paged_rope_fwd does.
    Returns (out, lse)."""
    rope = None
    if rope_cos is not None or rope_sin is not None:
        rope = _rope_args(rope_cos, rope_sin, rotary_dim, interleaved)
    return _attn_dense(q, cu_seqlens_q, k_new, v_new, cu_seqlens_knew, k_cache, v_cache, block_table,
                       cache_seqlens, page_size, causal, scale, kv_scale, out, lse, return_lse, host_index,
                       stream, rope, prob8=(float(q_scale), float(p_scale)))


def _attn_dense(q, cu_seqlens_q, k_new, v_new, cu_seqlens_knew, k_cache, v_cache, block_table, cache_seqlens,
                page_size, causal, scale, kv_scale, out, lse, return_lse, host_index, stream, rope, noalloc=False,
                prob8=None):
    lib = _lib.load()
    q = _dev(q, "q", _BF16)
    cu_seqlens_q = _dev(cu_seqlens_q, "cu_seqlens_q", _I32)
    k_new = _dev(k_new, "k_new", _BF16)
    v_new = _dev(v_new, "v_new", _BF16)
    cu_seqlens_knew = _dev(cu_seqlens_knew, "cu_seqlens_knew", _I32)
    fp8 = k_cache is not None and k_cache.dtype in _FP8
    k_cache = _dev(k_cache, "k_cache", _FP8 if fp8 else _BF16)
    v_cache = _dev(v_cache, "v_cache", _FP8 if fp8 else _BF16)
    block_table = _dev(block_table, "block_table", _I32)
    cache_seqlens = _dev(cache_seqlens, "cache_seqlens", _I32)
    if q.dim() != 3:
        raise VpkError(_lib.VPK_ERROR_INVALID_VALUE, "q must be [total_q, num_q_heads, head_dim]")
    Tq, Hq, D = q.shape
    B = cu_seqlens_q.numel() - 1
    Hkv = (k_new if k_new is not None else k_cache).shape[-2]
    Tn = 0 if k_new is None else k_new.shape[0]
    P = 0 if k_cache is None else k_cache.shape[0]
    for name, t, shp in (("k_new", k_new, (Tn, Hkv, D)), ("v_new", v_new, (Tn, Hkv, D)),
                         ("k_cache", k_cache, (P, page_size, Hkv, D)),
                         ("v_cache", v_cache, (P, page_size, Hkv, D))):
        if t is not None and tuple(t.shape) != shp:
            raise VpkError(_lib.VPK_ERROR_INVALID_VALUE, f"{name} has shape {tuple(t.shape)}, expected {shp}")
    _same_device(q.device, cu_seqlens_q=cu_seqlens_q, k_new=k_new, v_new=v_new, cu_seqlens_knew=cu_seqlens_knew,
                 k_cache=k_cache, v_cache=v_cache, block_table=block_table, cache_seqlens=cache_seqlens)
    if cu_seqlens_q.dim() != 1 or B < 0:
        raise VpkError(_lib.VPK_ERROR_INVALID_VALUE, "cu_seqlens_q must be [batch + 1]")
    if cu_seqlens_knew is not None:
        _length("cu_seqlens_knew", cu_seqlens_knew.numel(), B + 1)
    if cache_seqlens is not None:
        _length("cache_seqlens", cache_seqlens.numel(), B)
    if block_table is not None:
        if block_table.dim() != 2:
            raise VpkError(_lib.VPK_ERROR_INVALID_VALUE, "block_table must be [batch, max_pages_per_seq]")
        _length("block_table rows", block_table.shape[0], B)
    maxp = 0 if block_table is None else block_table.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out, lse = _out_lse(out, lse, Tq, Hq, D, q.device)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((Hq, Tq), dtype=torch.float32, device=q.device)
    dims = VpkDims(B, Tq, Tn, Hq, Hkv, D, P, maxp,
                   _lib.VPK_DTYPE_FP8_E4M3FN if fp8 else _lib.VPK_DTYPE_BF16)
    ks = None
    if fp8:
        if kv_scale is None:
            raise VpkError(_lib.VPK_ERROR_INVALID_VALUE, "kv_scale is required for an fp8 cache")
        ks = (ctypes.c_float * 2)(float(kv_scale[0]), float(kv_scale[1]))
    h = host_index or {}
    hi, keep = _host_index(h.get("cu_seqlens_q"), h.get("cu_seqlens_knew"),
                           h.get("cache_seqlens"), h.get("block_table"))
    for name, a, n in (("host cu_seqlens_q", keep[0], B + 1), ("host cu_seqlens_knew", keep[1], B + 1),
                       ("host cache_seqlens", keep[2], B), ("host block_table", keep[3], B * maxp)):
        if a is not None:
            _length(name, a.size, n)
    args = (ctypes.byref(dims), _ptr(q), _ptr(cu_seqlens_q), _ptr(k_new), _ptr(v_new), _ptr(cu_seqlens_knew),
            _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(cache_seqlens), int(page_size),
            int(bool(causal)), float(scale), ks)
    sh = _stream_handle(stream)
    tail = (_ptr(out), _ptr(lse), ctypes.byref(hi), sh)
    if noalloc:
        st = lib.attn_varlen_paged_fwd_noalloc(*args, *tail)
        del keep
        _check(st)
        return out, lse
    extra = 0
    if prob8 is not None and AUTO_WORKSPACE:
        # room for the decode-mode rows' kept scores (from the host lengths)
        sq = hi
        if keep[0] is None or (cu_seqlens_knew is not None and keep[1] is None) or \
                (cache_seqlens is not None and keep[2] is None):
            lens = [None if t is None else _host_i32(t) for t in (cu_seqlens_q, cu_seqlens_knew, cache_seqlens)]
            sq = VpkHostIndex(*[None if a is None else a.ctypes.data for a in lens], None)
        extra = int(lib.vpk_qkv_prob_score_bytes(ctypes.byref(dims), ctypes.byref(sq)))
    _ensure_workspace(dims, q.device, sh, rope is not None, extra)
    if prob8 is not None:
        qp = (ctypes.c_float * 2)(*prob8)
        st = lib.attn_varlen_paged_qkv_prob_fwd(*args, qp, None if rope is None else ctypes.byref(rope[0]), *tail)
    elif rope is None:
        st = lib.attn_varlen_paged_fwd(*args, *tail)
    else:
        st = lib.attn_varlen_paged_rope_fwd(*args, ctypes.byref(rope[0]), *tail)
    del keep
    _check(st)
    return out, lse


def attn_varlen_paged_list_fwd(q: torch.Tensor, q_start, q_len, k_new=None, v_new=None, cu_seqlens_knew=None,
                               k_cache=None, v_cache=None, kv_indptr=None, kv_indices=None, cache_seqlens=None,
                               page_size: int = 0, causal: bool = True, scale: Optional[float] = None,
                               kv_scale=None, *, out: Optional[torch.Tensor] = None,
                               lse: Optional[torch.Tensor] = None, return_lse: bool = True,
                               kv_indices_host=None, stream=None):
    """The page-list form: sequence b's query rows are q[q_start[b] : q_start[b] + q_len[b]]
    (anywhere in q, not overlapping), its page ids kv_indices[kv_indptr[b] : kv_indptr[b + 1]].

    q_start, q_len, cu_seqlens_knew, cache_seqlens and kv_indptr are host arrays
    (numpy or CPU tensors); kv_indices is a device int32 tensor (kv_indices_host
    an optional host copy for page-id range checks).  ``out`` rows that no
    sequence names are left as they are (a new ``out`` starts as zeros).
    Returns (out [Tq, Hq, D] bf16, lse [Hq, Tq] fp32 or None).
    """
    lib = _lib.load()
    q = _dev(q, "q", _BF16)
    k_new = _dev(k_new, "k_new", _BF16)
    v_new = _dev(v_new, "v_new", _BF16)
    fp8 = k_cache is not None and k_cache.dtype in _FP8
    k_cache = _dev(k_cache, "k_cache", _FP8 if fp8 else _BF16)
    v_cache = _dev(v_cache, "v_cache", _FP8 if fp8 else _BF16)
    kv_indices = _dev(kv_indices, "kv_indices", _I32)
    if q.dim() != 3:
        raise VpkError(_lib.VPK_ERROR_INVALID_VALUE, "q must be [total_q, num_q_heads, head_dim]")
    Tq, Hq, D = q.shape
    qs, ql = _host_i32(q_start), _host_i32(q_len)
    B = qs.size
    Hkv = (k_new if k_new is not None else k_cache).shape[-2]
    Tn = 0 if k_new is None else k_new.shape[0]
    P = 0 if k_cache is None else k_cache.shape[0]
    for name, t, shp in (("k_new", k_new, (Tn, Hkv, D)), ("v_new", v_new, (Tn, Hkv, D)),
                         ("k_cache", k_cache, (P, page_size, Hkv, D)),
                         ("v_cache", v_cache, (P, page_size, Hkv, D))):
        if t is not None and tuple(t.shape) != shp:
            raise VpkError(_lib.VPK_ERROR_INVALID_VALUE, f"{name} has shape {tuple(t.shape)}, expected {shp}")
    _same_device(q.device, k_new=k_new, v_new=v_new, k_cache=k_cache, v_cache=v_cache, kv_indices=kv_indices)
    _length("q_len", ql.size, B)
    for name, a, n in (("cu_seqlens_knew", cu_seqlens_knew, B + 1), ("cache_seqlens", cache_seqlens, B),
                       ("kv_indptr", kv_indptr, B + 1)):
        if a is not None:
            _length(name, _host_i32(a).size, n)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out, lse = _out_lse(out, lse, Tq, Hq, D, q.device)
    if out is None:
        out = torch.zeros_like(q)
    if lse is None and return_lse:
        lse = torch.full((Hq, Tq), float("nan"), dtype=torch.float32, device=q.device)
    dims = VpkDims(B, Tq, Tn, Hq, Hkv, D, P, 0, _lib.VPK_DTYPE_FP8_E4M3FN if fp8 else _lib.VPK_DTYPE_BF16)
    ks = None
    if fp8:
        if kv_scale is None:
            raise VpkError(_lib.VPK_ERROR_INVALID_VALUE, "kv_scale is required for an fp8 cache")
        ks = (ctypes.c_float * 2)(float(kv_scale[0]), float(kv_scale[1]))
    keep = [qs, ql, _host_i32(cu_seqlens_knew), _host_i32(cache_seqlens), _host_i32(kv_indptr),
            _host_i32(kv_indices_host)]
    hp = VpkHostPages(*[None if a is None else a.ctypes.data for a in keep])
    sh = _stream_handle(stream)
    wdims = VpkDims(*[getattr(dims, f) for f, _ in VpkDims._fields_])
    wdims.max_pages_per_seq = int(np.diff(keep[4]).max()) if keep[4] is not None and B else 0
    _ensure_workspace(wdims, q.device, sh)
    st = lib.attn_varlen_paged_list_fwd(ctypes.byref(dims), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
                                        _ptr(v_cache), _ptr(kv_indices), int(page_size), int(bool(causal)),
                                        float(scale), ks, _ptr(out), _ptr(lse), ctypes.byref(hp), sh)
    del keep
    _check(st)
    return out, lse


class Plan:
    """A prepared call (vpk_plan_create / vpk_plan_run): the work list of one set
    of lengths, built once in device memory; run() launches without host work
    and can be captured into a graph.

    Plan(cu_seqlens_q, num_q_heads, num_kv_heads, head_dim, cu_seqlens_knew=None,
         cache_seqlens=None, block_table=None, page_size=0, num_pages=0,
         max_pages_per_seq=0, cache_dtype="bf16" | "fp8", causal=True)
    The index arrays are host arrays (numpy or CPU tensors); block_table is
    optional here (page-id range checks).  A plan is for one device: create it
    with that device current.
    """

    def __init__(self, cu_seqlens_q, num_q_heads: int, num_kv_heads: int, head_dim: int, *,
                 cu_seqlens_knew=None, cache_seqlens=None, block_table=None, page_size: int = 0,
                 num_pages: int = 0, max_pages_per_seq: int = 0, cache_dtype: str = "bf16",
                 causal: bool = True):
        lib = _lib.load()
        self._h = None
        cu_q = _host_i32(cu_seqlens_q)
        cu_kn = _host_i32(cu_seqlens_knew)
        cl = _host_i32(cache_seqlens)
        B = cu_q.size - 1
        self.batch = B
        self.has_new = cu_kn is not None
        self.has_cache = cl is not None
        self.fp8 = self.has_cache and cache_dtype == "fp8"
        self.total_q = int(cu_q[-1])
        self.total_knew = int(cu_kn[-1]) if self.has_new else 0
        self.num_q_heads, self.num_kv_heads, self.head_dim = num_q_heads, num_kv_heads, head_dim
        self.page_size = int(page_size) if self.has_cache else 0
        self.num_pages = int(num_pages) if self.has_cache else 0
        self.max_pages = int(max_pages_per_seq) if self.has_cache else 0
        dims = VpkDims(B, self.total_q, self.total_knew, num_q_heads, num_kv_heads, head_dim,
                       self.num_pages, self.max_pages,
                       _lib.VPK_DTYPE_FP8_E4M3FN if self.fp8 else _lib.VPK_DTYPE_BF16)
        hi, keep = _host_index(cu_q, cu_kn, cl, block_table)
        h = ctypes.c_void_p()
        st = lib.vpk_plan_create(ctypes.byref(dims), ctypes.byref(hi), int(self.has_new),
                                 int(self.has_cache), self.page_size, int(bool(causal)), ctypes.byref(h))
        del keep
        _check(st)
        self._h = h

    def run(self, q, k_new=None, v_new=None, k_cache=None, v_cache=None, block_table=None, *,
            scale: Optional[float] = None, kv_scale=None, out=None, lse=None, return_lse: bool = True,
            stream=None):
        """Enqueue the planned call with these buffers; returns (out, lse).

        kv_scale (fp8 plans): a host pair (k_scale, v_scale), read now, or a
        device float32 tensor of 2 elements, read by the kernels when they run
        (vpk_plan_run_device_scale: a captured graph follows later values)."""
        lib = _lib.load()
        q = _dev(q, "q", _BF16)
        k_new = _dev(k_new, "k_new", _BF16)
        v_new = _dev(v_new, "v_new", _BF16)
        k_cache = _dev(k_cache, "k_cache", _FP8 if self.fp8 else _BF16)
        v_cache = _dev(v_cache, "v_cache", _FP8 if self.fp8 else _BF16)
        block_table = _dev(block_table, "block_table", _I32)
        Hq, Hkv, D = self.num_q_heads, self.num_kv_heads, self.head_dim
        for name, t, shp in (("q", q, (self.total_q, Hq, D)),
                             ("k_new", k_new, (self.total_knew, Hkv, D)),
                             ("v_new", v_new, (self.total_knew, Hkv, D)),
                             ("k_cache", k_cache, (self.num_pages, self.page_size, Hkv, D)),
                             ("v_cache", v_cache, (self.num_pages, self.page_size, Hkv, D))):
            if t is not None and tuple(t.shape) != shp:
                raise VpkError(_lib.VPK_ERROR_INVALID_VALUE, f"{name} has shape {tuple(t.shape)}, expected {shp}")
        if block_table is not None and tuple(block_table.shape) != (self.batch, self.max_pages):
            raise VpkError(_lib.VPK_ERROR_INVALID_VALUE,
                           f"block_table has shape {tuple(block_table.shape)}, expected {(self.batch, self.max_pages)}")
        _same_device(q.device, k_new=k_new, v_new=v_new, k_cache=k_cache, v_cache=v_cache, block_table=block_table)
        if scale is None:
            scale = 1.0 / math.sqrt(D)
        out, lse = _out_lse(out, lse, self.total_q, Hq, D, q.device)
        if out is None:
            out = torch.empty_like(q)
        if lse is None and return_lse:
            lse = torch.empty((Hq, self.total_q), dtype=torch.float32, device=q.device)
        if isinstance(kv_scale, torch.Tensor) and kv_scale.is_cuda:
            ksd = _dev(kv_scale, "kv_scale", (torch.float32,))
            if ksd.numel() != 2:
                raise VpkError(_lib.VPK_ERROR_INVALID_VALUE, "a device kv_scale holds 2 floats")
            st = lib.vpk_plan_run_device_scale(self._h, _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
                                               _ptr(v_cache), _ptr(block_table), float(scale), _ptr(ksd),
                                               _ptr(out), _ptr(lse), _stream_handle(stream))
            _check(st)
            return out, lse
        ks = None
        if self.fp8:
            if kv_scale is None:
                raise VpkError(_lib.VPK_ERROR_INVALID_VALUE, "kv_scale is required for an fp8 cache")
            ks = (ctypes.c_float * 2)(float(kv_scale[0]), float(kv_scale[1]))
        st = lib.vpk_plan_run(self._h, _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                              _ptr(block_table), float(scale), ks, _ptr(out), _ptr(lse),
                              _stream_handle(stream))
        _check(st)
        return out, lse

    def device_error(self, stream=None) -> int:
        f = ctypes.c_int32(0)
        _check(_lib.load().vpk_plan_device_error(self._h, _stream_handle(stream), ctypes.byref(f)))
        return int(f.value)

    def close(self):
        if self._h is not None:
            h, self._h = self._h, None
            _check(_lib.load().vpk_plan_destroy(h))

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def kv_cache_append(k_new, v_new, cu_seqlens_knew, k_cache, v_cache, block_table, cache_seqlens,
                    page_size: int, kv_scale=None, *, host_index: Optional[dict] = None, stream=None):
    """Store k_new/v_new into the paged cache at positions [Lc, Lc + Ln) of each sequence."""
    lib = _lib.load()
    fp8 = k_cache.dtype in _FP8
    k_new = _dev(k_new, "k_new", _BF16)
    v_new = _dev(v_new, "v_new", _BF16)
    cu_seqlens_knew = _dev(cu_seqlens_knew, "cu_seqlens_knew", _I32)
    k_cache = _dev(k_cache, "k_cache", _FP8 if fp8 else _BF16)
    v_cache = _dev(v_cache, "v_cache", _FP8 if fp8 else _BF16)
    block_table = _dev(block_table, "block_table", _I32)
    cache_seqlens = _dev(cache_seqlens, "cache_seqlens", _I32)
    if k_new.dim() != 3:
        raise VpkError(_lib.VPK_ERROR_INVALID_VALUE, "k_new must be [total_knew, num_kv_heads, head_dim]")
    Tn, Hkv, D = k_new.shape
    B = cu_seqlens_knew.numel() - 1
    _same_device(k_new.device, v_new=v_new, cu_seqlens_knew=cu_seqlens_knew, k_cache=k_cache, v_cache=v_cache,
                 block_table=block_table, cache_seqlens=cache_seqlens)
    for name, t, shp in (("v_new", v_new, (Tn, Hkv, D)), ("k_cache", k_cache, (k_cache.shape[0], page_size, Hkv, D)),
                         ("v_cache", v_cache, (k_cache.shape[0], page_size, Hkv, D))):
        if tuple(t.shape) != shp:
            raise VpkError(_lib.VPK_ERROR_INVALID_VALUE, f"{name} has shape {tuple(t.shape)}, expected {shp}")
    _length("cache_seqlens", cache_seqlens.numel(), B)
    if block_table.dim() != 2:
        raise VpkError(_lib.VPK_ERROR_INVALID_VALUE, "block_table must be [batch, max_pages_per_seq]")
    _length("block_table rows", block_table.shape[0], B)
    if fp8 and kv_scale is None:
        raise VpkError(_lib.VPK_ERROR_INVALID_VALUE, "kv_scale is required for an fp8 cache")
    dims = VpkDims(B, 0, Tn, Hkv, Hkv, D, k_cache.shape[0], block_table.shape[1],
                   _lib.VPK_DTYPE_FP8_E4M3FN if fp8 else _lib.VPK_DTYPE_BF16)
    ks = None
    if fp8:
        ks = (ctypes.c_float * 2)(float(kv_scale[0]), float(kv_scale[1]))
    h = host_index or {}
    hi, keep = _host_index(None, h.get("cu_seqlens_knew"), h.get("cache_seqlens"), h.get("block_table"))
    sh = _stream_handle(stream)
    _ensure_workspace(dims, k_new.device, sh)
    st = lib.kv_cache_append(ctypes.byref(dims), _ptr(k_new), _ptr(v_new), _ptr(cu_seqlens_knew),
                             _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(cache_seqlens),
                             int(page_size), ks, ctypes.byref(hi), sh)
    del keep
    _check(st)


def set_option(name: str, value: int):
    _check(_lib.load().vpk_set_option(name.encode(), int(value)))


def abi_version() -> int:
    return int(_lib.load().vpk_abi_version())


def timing_enable(on: bool = True):
    _check(_lib.load().vpk_timing_enable(1 if on else 0))


def timing_reset():
    _check(_lib.load().vpk_timing_reset())


def timing_read(kernel: int):
    """(total milliseconds, launches) of one kernel since the last reset."""
    ms = ctypes.c_double(0)
    n = ctypes.c_int64(0)
    _check(_lib.load().vpk_timing_read(int(kernel), ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def device_error(stream=None) -> int:
    f = ctypes.c_int32(0)
    _check(_lib.load().vpk_device_error(_stream_handle(stream), ctypes.byref(f)))
    return f.value


def plan_debug(*, batch, num_q_heads, num_kv_heads, head_dim, cu_seqlens_q, cu_seqlens_knew=None,
               cache_seqlens=None, block_table=None, page_size=1, causal=True, num_cus=256,
               has_cache=None, num_pages=None, kv_cache_dtype="bf16", capacity=None):
    """Host-only view of the attention work list: int32 array [n_items, 8] and the queue count."""
    lib = _lib.load()
    cu_q = _host_i32(cu_seqlens_q)
    cu_kn = _host_i32(cu_seqlens_knew)
    cl = _host_i32(cache_seqlens)
    bt = _host_i32(block_table)
    has_cache = (cl is not None) if has_cache is None else has_cache
    has_new = cu_kn is not None
    maxp = bt.shape[1] if bt is not None else (1 << 20)
    if num_pages is None:
        num_pages = (int(bt.max()) + 1) if bt is not None and bt.size else (1 << 20)
    dims = VpkDims(batch, int(cu_q[-1]), int(cu_kn[-1]) if has_new else 0, num_q_heads,
                   num_kv_heads, head_dim, num_pages if has_cache else 0, maxp,
                   _lib.VPK_DTYPE_FP8_E4M3FN if kv_cache_dtype == "fp8" else _lib.VPK_DTYPE_BF16)
    hi, keep = _host_index(cu_q, cu_kn, cl, bt)
    cap = capacity if capacity is not None else 1 << 16
    while True:
        buf = np.zeros((cap, 8), np.int32)
        n = ctypes.c_int32(0)
        nq = ctypes.c_int32(0)
        st = lib.vpk_plan_debug(ctypes.byref(dims), ctypes.byref(hi), int(has_cache), int(has_new),
                                int(page_size), int(bool(causal)), int(num_cus),
                                buf.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), cap,
                                ctypes.byref(n), ctypes.byref(nq))
        if st == _lib.VPK_ERROR_CAPACITY and n.value > cap and capacity is None:
            cap = n.value
            continue
        _check(st)
        del keep
        return buf[:n.value].copy(), nq.value
