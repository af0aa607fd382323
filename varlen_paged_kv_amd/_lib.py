"""ctypes loader and signatures for libvpk.so (the C ABI declared in include/vpk.h)."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libvpk.so")

VPK_SUCCESS = 0
VPK_ERROR_INVALID_VALUE = 1
VPK_ERROR_NOT_SUPPORTED = 2
VPK_ERROR_CAPACITY = 3
VPK_ERROR_HIP = 4
VPK_ERROR_OUT_OF_MEMORY = 5

VPK_DTYPE_BF16 = 1
VPK_DTYPE_FP8_E4M3FN = 2

STATUS_NAMES = {
    0: "VPK_SUCCESS", 1: "VPK_ERROR_INVALID_VALUE", 2: "VPK_ERROR_NOT_SUPPORTED",
    3: "VPK_ERROR_CAPACITY", 4: "VPK_ERROR_HIP", 5: "VPK_ERROR_OUT_OF_MEMORY",
}

# every symbol include/vpk.h declares
EXPORTS = (
    "attn_varlen_paged_fwd", "kv_cache_append", "vpk_last_error", "vpk_abi_version",
    "vpk_set_option", "vpk_timing_enable", "vpk_timing_reset", "vpk_timing_read",
    "vpk_device_error", "vpk_plan_debug", "vpk_plan_create", "vpk_plan_run", "vpk_plan_device_error",
    "vpk_plan_destroy", "attn_varlen_paged_list_fwd", "attn_varlen_paged_rope_fwd",
    "vpk_plan_run_device_scale", "vpk_set_workspace", "vpk_workspace_bytes_upper_bound", "vpk_library_memory",
    "attn_varlen_paged_fwd_noalloc", "attn_varlen_paged_qkv_prob_fwd", "vpk_qkv_prob_score_bytes",
)


class VpkHostPages(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("q_start", "q_len", "cu_seqlens_knew", "cache_seqlens",
                                                "kv_indptr", "kv_indices")]


class VpkDims(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("total_q", ctypes.c_int32),
        ("total_knew", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
        ("kv_cache_dtype", ctypes.c_int32),
    ]


class VpkRope(ctypes.Structure):
    _fields_ = [("cos", ctypes.c_void_p), ("sin", ctypes.c_void_p), ("max_positions", ctypes.c_int32),
                ("rotary_dim", ctypes.c_int32), ("interleaved", ctypes.c_int32)]


class VpkHostIndex(ctypes.Structure):
    _fields_ = [
        ("cu_seqlens_q", ctypes.c_void_p),
        ("cu_seqlens_knew", ctypes.c_void_p),
        ("cache_seqlens", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
    ]


_lib = None


def load() -> ctypes.CDLL:
    """Load libvpk.so (built in-tree by varlen_paged_kv_amd/build.py); raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libvpk.so not found at {LIB_PATH}: build it with "
                          "`python varlen_paged_kv_amd/build.py` (there is no fallback path)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
    P = ctypes.POINTER
    lib.attn_varlen_paged_fwd.restype = i32
    lib.attn_varlen_paged_fwd.argtypes = [
        P(VpkDims), vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, f32, P(f32), vp, vp,
        P(VpkHostIndex), vp]
    lib.attn_varlen_paged_fwd_noalloc.restype = i32
    lib.attn_varlen_paged_fwd_noalloc.argtypes = lib.attn_varlen_paged_fwd.argtypes
    lib.kv_cache_append.restype = i32
    lib.kv_cache_append.argtypes = [P(VpkDims), vp, vp, vp, vp, vp, vp, vp, i32, P(f32),
                                    P(VpkHostIndex), vp]
    lib.vpk_last_error.restype = ctypes.c_char_p
    lib.vpk_last_error.argtypes = []
    lib.vpk_abi_version.restype = i32
    lib.vpk_abi_version.argtypes = []
    lib.vpk_set_option.restype = i32
    lib.vpk_set_option.argtypes = [ctypes.c_char_p, ctypes.c_int64]
    lib.vpk_timing_enable.restype = i32
    lib.vpk_timing_enable.argtypes = [i32]
    lib.vpk_timing_reset.restype = i32
    lib.vpk_timing_reset.argtypes = []
    lib.vpk_timing_read.restype = i32
    lib.vpk_timing_read.argtypes = [i32, P(ctypes.c_double), P(ctypes.c_int64)]
    lib.vpk_device_error.restype = i32
    lib.vpk_device_error.argtypes = [vp, P(i32)]
    lib.vpk_plan_debug.restype = i32
    lib.vpk_plan_debug.argtypes = [P(VpkDims), P(VpkHostIndex), i32, i32, i32, i32, i32,
                                   P(i32), i32, P(i32), P(i32)]
    lib.attn_varlen_paged_rope_fwd.restype = i32
    lib.attn_varlen_paged_rope_fwd.argtypes = [P(VpkDims), vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, f32,
                                               P(f32), P(VpkRope), vp, vp, P(VpkHostIndex), vp]
    lib.attn_varlen_paged_qkv_prob_fwd.restype = i32
    lib.attn_varlen_paged_qkv_prob_fwd.argtypes = [P(VpkDims), vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, f32,
                                                   P(f32), P(f32), P(VpkRope), vp, vp, P(VpkHostIndex), vp]
    lib.attn_varlen_paged_list_fwd.restype = i32
    lib.attn_varlen_paged_list_fwd.argtypes = [P(VpkDims), vp, vp, vp, vp, vp, vp, i32, i32, f32, P(f32), vp, vp,
                                               P(VpkHostPages), vp]
    lib.vpk_plan_create.restype = i32
    lib.vpk_plan_create.argtypes = [P(VpkDims), P(VpkHostIndex), i32, i32, i32, i32, P(vp)]
    lib.vpk_plan_run.restype = i32
    lib.vpk_plan_run.argtypes = [vp, vp, vp, vp, vp, vp, vp, f32, P(f32), vp, vp, vp]
    lib.vpk_plan_run_device_scale.restype = i32
    lib.vpk_plan_run_device_scale.argtypes = [vp, vp, vp, vp, vp, vp, vp, f32, vp, vp, vp, vp]
    lib.vpk_plan_device_error.restype = i32
    lib.vpk_plan_device_error.argtypes = [vp, vp, P(i32)]
    lib.vpk_plan_destroy.restype = i32
    lib.vpk_plan_destroy.argtypes = [vp]
    lib.vpk_set_workspace.restype = i32
    lib.vpk_set_workspace.argtypes = [vp, vp, ctypes.c_size_t]
    lib.vpk_workspace_bytes_upper_bound.restype = ctypes.c_size_t
    lib.vpk_workspace_bytes_upper_bound.argtypes = [P(VpkDims), i32, i32]
    lib.vpk_qkv_prob_score_bytes.restype = ctypes.c_size_t
    lib.vpk_qkv_prob_score_bytes.argtypes = [P(VpkDims), P(VpkHostIndex)]
    lib.vpk_library_memory.restype = i32
    lib.vpk_library_memory.argtypes = [P(ctypes.c_size_t), P(ctypes.c_size_t)]
    _lib = lib
    return lib
