"""ctypes binding of libfmha.so: the C ABI of include/fmha.h, argument marshalling only.

The functions keep the C names.  Pointers may be passed as integers or as any object
with ``data_ptr()`` (a torch tensor); nothing here computes any part of the attention.
Loading fails with an exception when the HIP library has not been built: there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfmha.so")

DTYPES = {"f16": 0, "bf16": 1, "f8e4m3": 2}
MASKS = {"none": 0, "residual": 1, "causal_qbegin": 2, "causal_qend": 3}
STATUS = {0: "FMHA_OK", 1: "FMHA_ERR_NULL_POINTER", 2: "FMHA_ERR_INVALID_SHAPE", 3: "FMHA_ERR_UNSUPPORTED",
          4: "FMHA_ERR_MISALIGNED", 5: "FMHA_ERR_INVALID_ARGUMENT", 6: "FMHA_ERR_HIP", 7: "FMHA_ERR_SCRATCH_TOO_SMALL"}
# every symbol include/fmha.h declares
EXPORTS = ("fmha_fwd", "fmha_fwd_splitkv", "fmha_fwd_splitkv_noalloc", "fmha_fwd_splitkv_workspace_size",
           "fmha_fwd_splitkv_paged", "fmha_paged_kv_append", "fmha_bwd", "fmha_bwd_workspace_size", "fmha_status_string", "fmha_version")


class FmhaError(RuntimeError):
    def __init__(self, status: int):
        super().__init__(f"{STATUS.get(status, status)}: {fmha_status_string(status)}")
        self.status = status


class fmha_varlen(ctypes.Structure):
    _fields_ = [("cu_seqlens_q", ctypes.c_void_p), ("cu_seqlens_k", ctypes.c_void_p),
                ("total_length_q", ctypes.c_int32), ("total_length_k", ctypes.c_int32)]


class fmha_paged_kv(ctypes.Structure):
    _fields_ = [("block_table", ctypes.c_void_p), ("seqlens_k", ctypes.c_void_p), ("max_pages_per_seq", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int32), ("kv_dtype", ctypes.c_int)]


_lib: Optional[ctypes.CDLL] = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m head_attention_03_amd.build` "
                          "(there is no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    lib.fmha_fwd.restype = ctypes.c_int
    lib.fmha_fwd.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_void_p] + [ctypes.c_int32] * 6 + [
        ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.POINTER(fmha_varlen), ctypes.c_void_p]
    lib.fmha_fwd_splitkv.restype = ctypes.c_int
    lib.fmha_fwd_splitkv.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_void_p] + [ctypes.c_int32] * 6 + [
        ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.POINTER(fmha_varlen), ctypes.c_void_p,
        ctypes.c_size_t, ctypes.c_void_p]
    lib.fmha_fwd_splitkv_noalloc.restype = ctypes.c_int
    lib.fmha_fwd_splitkv_noalloc.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_void_p] + [ctypes.c_int32] * 6 + [
        ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.POINTER(fmha_varlen), ctypes.c_void_p]
    lib.fmha_fwd_splitkv_workspace_size.restype = ctypes.c_size_t
    lib.fmha_fwd_splitkv_workspace_size.argtypes = [ctypes.c_int32] * 6 + [ctypes.POINTER(fmha_varlen)]
    lib.fmha_fwd_splitkv_paged.restype = ctypes.c_int
    lib.fmha_fwd_splitkv_paged.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_void_p] + [ctypes.c_int32] * 6 + [
        ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.POINTER(fmha_paged_kv), ctypes.c_void_p,
        ctypes.c_size_t, ctypes.c_void_p]
    lib.fmha_paged_kv_append.restype = ctypes.c_int
    lib.fmha_paged_kv_append.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int32] * 4 + [
        ctypes.POINTER(fmha_paged_kv), ctypes.c_void_p]
    lib.fmha_bwd.restype = ctypes.c_int
    lib.fmha_bwd.argtypes = [ctypes.c_void_p] * 9 + [ctypes.c_int32] * 6 + [
        ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.POINTER(fmha_varlen), ctypes.c_void_p, ctypes.c_size_t,
        ctypes.c_void_p]
    lib.fmha_bwd_workspace_size.restype = ctypes.c_size_t
    lib.fmha_bwd_workspace_size.argtypes = [ctypes.c_int32] * 6 + [ctypes.c_int, ctypes.POINTER(fmha_varlen)]
    lib.fmha_status_string.restype = ctypes.c_char_p
    lib.fmha_status_string.argtypes = [ctypes.c_int]
    lib.fmha_version.restype = ctypes.c_int32
    lib.fmha_version.argtypes = []
    _lib = lib
    return lib


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if hasattr(x, "data_ptr"):
        return int(x.data_ptr())
    return int(x)


def _stream(s) -> Optional[int]:
    if s is None:
        return None
    if hasattr(s, "cuda_stream"):
        return int(s.cuda_stream)
    return int(s)


def make_varlen(cu_seqlens_q, cu_seqlens_k, total_length_q: int, total_length_k: int) -> fmha_varlen:
    return fmha_varlen(_ptr(cu_seqlens_q), _ptr(cu_seqlens_k), int(total_length_q), int(total_length_k))


def fmha_fwd(q, k, v, o, lse, B: int, Sq: int, Sk: int, H: int, H_kv: int, D: int, scale: float, mask, dtype,
             o_scale: float = 1.0, varlen: Optional[fmha_varlen] = None, stream=None) -> int:
    """Call the C entry point; returns the fmha_status code.  ``mask``/``dtype`` take enum values or names."""
    lib = load()
    mask = MASKS[mask] if isinstance(mask, str) else int(mask)
    dtype = DTYPES[dtype] if isinstance(dtype, str) else int(dtype)
    vl = ctypes.byref(varlen) if varlen is not None else None
    return int(lib.fmha_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(Sq), int(Sk), int(H),
                            int(H_kv), int(D), float(scale), mask, dtype, float(o_scale), vl, _stream(stream)))


def fmha_fwd_splitkv(q, k, v, o, lse, B: int, Sq: int, Sk: int, H: int, H_kv: int, D: int, scale: float, mask,
                     dtype, o_scale: float = 1.0, varlen: Optional[fmha_varlen] = None, workspace=None,
                     workspace_bytes: int = 0, stream=None) -> int:
    """Call the split-KV C entry point; returns the fmha_status code."""
    lib = load()
    mask = MASKS[mask] if isinstance(mask, str) else int(mask)
    dtype = DTYPES[dtype] if isinstance(dtype, str) else int(dtype)
    vl = ctypes.byref(varlen) if varlen is not None else None
    return int(lib.fmha_fwd_splitkv(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(Sq), int(Sk), int(H),
                                    int(H_kv), int(D), float(scale), mask, dtype, float(o_scale), vl, _ptr(workspace),
                                    int(workspace_bytes), _stream(stream)))


def fmha_fwd_splitkv_noalloc(q, k, v, o, lse, B: int, Sq: int, Sk: int, H: int, H_kv: int, D: int, scale: float,
                             mask, dtype, o_scale: float = 1.0, varlen: Optional[fmha_varlen] = None,
                             stream=None) -> int:
    """Call the allocation-free split-KV C entry point (library-owned scratch); returns the fmha_status code."""
    lib = load()
    mask = MASKS[mask] if isinstance(mask, str) else int(mask)
    dtype = DTYPES[dtype] if isinstance(dtype, str) else int(dtype)
    vl = ctypes.byref(varlen) if varlen is not None else None
    return int(lib.fmha_fwd_splitkv_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(Sq), int(Sk),
                                            int(H), int(H_kv), int(D), float(scale), mask, dtype, float(o_scale), vl,
                                            _stream(stream)))


def fmha_fwd_splitkv_workspace_size(B: int, Sq: int, Sk: int, H: int, H_kv: int, D: int,
                                    varlen: Optional[fmha_varlen] = None) -> int:
    vl = ctypes.byref(varlen) if varlen is not None else None
    return int(load().fmha_fwd_splitkv_workspace_size(int(B), int(Sq), int(Sk), int(H), int(H_kv), int(D), vl))


def make_paged_kv(block_table, seqlens_k, max_pages_per_seq: int, page_size: int, num_pages: int,
                  kv_dtype) -> fmha_paged_kv:
    """``kv_dtype``: the cache's element type (name or enum value): the call's dtype, or "f8e4m3"."""
    kv = DTYPES[kv_dtype] if isinstance(kv_dtype, str) else int(kv_dtype)
    return fmha_paged_kv(_ptr(block_table), _ptr(seqlens_k), int(max_pages_per_seq), int(page_size), int(num_pages), kv)


def fmha_fwd_splitkv_paged(q, k_cache, v_cache, o, lse, B: int, Sq: int, Sk: int, H: int, H_kv: int, D: int,
                           scale: float, mask, dtype, o_scale: float = 1.0, paged: Optional[fmha_paged_kv] = None,
                           workspace=None, workspace_bytes: int = 0, stream=None) -> int:
    """Call the paged-cache split-KV C entry point; returns the fmha_status code."""
    lib = load()
    mask = MASKS[mask] if isinstance(mask, str) else int(mask)
    dtype = DTYPES[dtype] if isinstance(dtype, str) else int(dtype)
    pk = ctypes.byref(paged) if paged is not None else None
    return int(lib.fmha_fwd_splitkv_paged(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(o), _ptr(lse), int(B), int(Sq),
                                          int(Sk), int(H), int(H_kv), int(D), float(scale), mask, dtype,
                                          float(o_scale), pk, _ptr(workspace), int(workspace_bytes), _stream(stream)))


def fmha_paged_kv_append(k_cache, v_cache, k_new, v_new, B: int, S_new: int, H_kv: int, D: int,
                         paged: Optional[fmha_paged_kv] = None, stream=None) -> int:
    """Call the paged-cache append C entry point; returns the fmha_status code."""
    lib = load()
    pk = ctypes.byref(paged) if paged is not None else None
    return int(lib.fmha_paged_kv_append(_ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new), int(B), int(S_new),
                                        int(H_kv), int(D), pk, _stream(stream)))


def fmha_bwd(q, k, v, o, dout, lse, dq, dk, dv, B: int, Sq: int, Sk: int, H: int, H_kv: int, D: int, scale: float,
             mask, dtype, varlen: Optional[fmha_varlen] = None, workspace=None, workspace_bytes: int = 0,
             stream=None) -> int:
    """Call the backward C entry point; returns the fmha_status code."""
    lib = load()
    mask = MASKS[mask] if isinstance(mask, str) else int(mask)
    dtype = DTYPES[dtype] if isinstance(dtype, str) else int(dtype)
    vl = ctypes.byref(varlen) if varlen is not None else None
    return int(lib.fmha_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                            int(B), int(Sq), int(Sk), int(H), int(H_kv), int(D), float(scale), mask, dtype, vl,
                            _ptr(workspace), int(workspace_bytes), _stream(stream)))


def fmha_bwd_workspace_size(B: int, Sq: int, Sk: int, H: int, H_kv: int, D: int, dtype,
                            varlen: Optional[fmha_varlen] = None) -> int:
    dtype = DTYPES[dtype] if isinstance(dtype, str) else int(dtype)
    vl = ctypes.byref(varlen) if varlen is not None else None
    return int(load().fmha_bwd_workspace_size(int(B), int(Sq), int(Sk), int(H), int(H_kv), int(D), dtype, vl))


def fmha_status_string(status: int) -> str:
    return load().fmha_status_string(int(status)).decode()


def fmha_version() -> int:
    return int(load().fmha_version())


def check(status: int) -> None:
    if status != 0:
        raise FmhaError(status)
