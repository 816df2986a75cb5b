"""ctypes binding over the C ABI in include/splitkv.h (argument marshalling only).

Every function here has the name of the C entry point it calls and does no
arithmetic of the method: buffers are passed as raw pointers (a torch tensor's
``data_ptr()`` or a plain integer), streams as HIP stream handles. A non-OK
status raises :class:`SplitKVError` carrying the status and the library's
detail message. The library must have been built (``python -m
split_kv_flash_amd.build``); there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
import re
from ctypes import POINTER, c_char_p, c_float, c_int32, c_int64, c_size_t, c_void_p
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libsplitkv.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "splitkv.h")

SK_OK, SK_ERR_INVALID_ARG, SK_ERR_UNSUPPORTED, SK_ERR_WORKSPACE_TOO_SMALL, SK_ERR_LAUNCH, SK_ERR_HIP = range(6)
SK_F32, SK_F16, SK_BF16 = 0, 1, 2
SK_KV_CONTIGUOUS, SK_KV_PAGED, SK_KV_INDEXED = 0, 1, 2
DTYPES = {"f32": SK_F32, "f16": SK_F16, "bf16": SK_BF16}


class SkDesc(ctypes.Structure):
    _fields_ = [
        ("batch", c_int32), ("num_q_heads", c_int32), ("num_kv_heads", c_int32),
        ("head_dim_qk", c_int32), ("head_dim_v", c_int32), ("kv_shared", c_int32),
        ("scale", c_float), ("q_dtype", c_int32), ("kv_dtype", c_int32), ("layout", c_int32),
        ("max_seq_len", c_int32), ("page_size", c_int32), ("max_pages_per_seq", c_int32),
        ("num_pages", c_int64), ("stride_seq", c_int64), ("stride_pos", c_int64),
        ("stride_head", c_int64),
    ]


class SkPlan(ctypes.Structure):
    _fields_ = [("n_splits", c_int32), ("chunk", c_int32)]

    def __repr__(self):
        return f"SkPlan(n_splits={self.n_splits}, chunk={self.chunk})"


class SkKernelInfo(ctypes.Structure):
    _fields_ = [("lds_bytes", c_int32), ("vgprs", c_int32), ("block", c_int32),
                ("grid_x", c_int32), ("grid_y", c_int32), ("grid_z", c_int32)]


class SplitKVError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[{status}] {message}")
        self.status = status
        self.message = message


_lib = None


def lib() -> ctypes.CDLL:
    """Load libsplitkv.so (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m split_kv_flash_amd.build` "
            "(the HIP library is required; there is no CPU fallback)")
    L = ctypes.CDLL(LIB_PATH)
    PD, PP = POINTER(SkDesc), POINTER(SkPlan)
    L.attn_decode_plan.argtypes = [PD, c_int32, c_int64, c_int32, c_int32, PP]
    L.attn_decode_plan.restype = c_int32
    L.attn_decode_workspace_bytes.argtypes = [PD, PP]
    L.attn_decode_workspace_bytes.restype = c_size_t
    L.attn_decode_splitk.argtypes = [PD, PP, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                     c_void_p, c_size_t, c_void_p]
    L.attn_decode_splitk.restype = c_int32
    L.attn_decode_combine.argtypes = [PD, PP, c_void_p, c_void_p, c_size_t, c_void_p, c_void_p,
                                      c_void_p]
    L.attn_decode_combine.restype = c_int32
    L.attn_decode_status_string.argtypes = [c_int32]
    L.attn_decode_status_string.restype = c_char_p
    L.attn_decode_last_error.argtypes = []
    L.attn_decode_last_error.restype = c_char_p
    L.attn_decode_kernel_info.argtypes = [PD, PP, POINTER(SkKernelInfo)]
    L.attn_decode_kernel_info.restype = c_int32
    L.attn_decode_workspace_init.argtypes = [PD, PP, c_void_p, c_size_t, c_void_p]
    L.attn_decode_workspace_init.restype = c_int32
    L.attn_decode.argtypes = [PD, PP, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                              c_size_t, c_void_p, c_void_p, c_void_p]
    L.attn_decode.restype = c_int32
    L.attn_decode_combine_project.argtypes = [PD, PP, c_void_p, c_void_p, c_size_t, c_void_p,
                                              c_int32, c_int32, c_void_p, c_void_p, c_void_p]
    L.attn_decode_combine_project.restype = c_int32
    L.attn_query_tiles.argtypes = [PD, PP, c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                                   c_void_p, c_size_t, c_void_p, c_void_p, c_void_p]
    L.attn_query_tiles.restype = c_int32
    L.attn_query_tiles_plan.argtypes = [PD, c_int32, c_int32, c_int64, c_int32, c_int32, PP]
    L.attn_query_tiles_plan.restype = c_int32
    L.attn_query_tiles_workspace_bytes.argtypes = [PD, PP, c_int32]
    L.attn_query_tiles_workspace_bytes.restype = c_size_t
    L.attn_decode_read_probe.argtypes = [c_void_p, c_size_t, c_int32, c_void_p, c_void_p]
    L.attn_decode_read_probe.restype = c_int32
    L.attn_decode_one_launch.argtypes = L.attn_decode.argtypes
    L.attn_decode_one_launch.restype = c_int32
    L.attn_decode_no_alloc.argtypes = [PD, PP, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                       c_void_p, c_void_p, c_void_p]
    L.attn_decode_no_alloc.restype = c_int32
    _lib = L
    return L


def header_functions() -> list:
    """Names of the functions include/splitkv.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_\w+)\s*\(", text)))


def _ptr(x) -> Optional[int]:
    """Device address of a tensor (None for NULL; an int passes through as an
    address). A host tensor is refused: the kernels would fault on it."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not getattr(x, "is_cuda", False):
        raise SplitKVError(SK_ERR_INVALID_ARG, "tensor arguments must live on the GPU")
    return x.data_ptr()


def _check(status: int):
    if status != SK_OK:
        raise SplitKVError(status, attn_decode_last_error() or attn_decode_status_string(status))


def attn_decode_status_string(status: int) -> str:
    return lib().attn_decode_status_string(status).decode()


def attn_decode_last_error() -> str:
    return lib().attn_decode_last_error().decode()


def attn_decode_plan(desc: SkDesc, max_seq_len: int, total_tokens: int, cu_count: int,
                     n_splits_requested: int = 0) -> SkPlan:
    plan = SkPlan()
    _check(lib().attn_decode_plan(ctypes.byref(desc), int(max_seq_len), int(total_tokens),
                                  int(cu_count), int(n_splits_requested), ctypes.byref(plan)))
    return plan


def attn_decode_workspace_bytes(desc: SkDesc, plan: SkPlan) -> int:
    n = lib().attn_decode_workspace_bytes(ctypes.byref(desc), ctypes.byref(plan))
    if n == 0:
        raise SplitKVError(SK_ERR_INVALID_ARG, attn_decode_last_error())
    return int(n)


def attn_decode_splitk(desc: SkDesc, plan: SkPlan, q, k, v, block_table, seq_lens, workspace,
                       workspace_bytes: int, stream: int) -> None:
    _check(lib().attn_decode_splitk(ctypes.byref(desc), ctypes.byref(plan), _ptr(q), _ptr(k),
                                    _ptr(v), _ptr(block_table), _ptr(seq_lens), _ptr(workspace),
                                    int(workspace_bytes), stream))


def attn_decode_combine(desc: SkDesc, plan: SkPlan, seq_lens, workspace, workspace_bytes: int,
                        out, lse, stream: int) -> None:
    _check(lib().attn_decode_combine(ctypes.byref(desc), ctypes.byref(plan), _ptr(seq_lens),
                                     _ptr(workspace), int(workspace_bytes), _ptr(out), _ptr(lse),
                                     stream))


def attn_decode_workspace_init(desc: SkDesc, plan: SkPlan, workspace, workspace_bytes: int,
                               stream: int) -> None:
    _check(lib().attn_decode_workspace_init(ctypes.byref(desc), ctypes.byref(plan),
                                            _ptr(workspace), int(workspace_bytes), stream))


def attn_decode(desc: SkDesc, plan: SkPlan, q, k, v, block_table, seq_lens, workspace,
                workspace_bytes: int, out, lse, stream: int) -> None:
    _check(lib().attn_decode(ctypes.byref(desc), ctypes.byref(plan), _ptr(q), _ptr(k), _ptr(v),
                             _ptr(block_table), _ptr(seq_lens), _ptr(workspace),
                             int(workspace_bytes), _ptr(out), _ptr(lse), stream))


def attn_decode_one_launch(desc: SkDesc, plan: SkPlan, q, k, v, block_table, seq_lens, workspace,
                           workspace_bytes: int, out, lse, stream: int) -> None:
    _check(lib().attn_decode_one_launch(ctypes.byref(desc), ctypes.byref(plan), _ptr(q), _ptr(k),
                                        _ptr(v), _ptr(block_table), _ptr(seq_lens),
                                        _ptr(workspace), int(workspace_bytes), _ptr(out),
                                        _ptr(lse), stream))


def attn_decode_no_alloc(desc: SkDesc, plan: SkPlan, q, k, v, block_table, seq_lens, out, lse,
                         stream: int) -> None:
    _check(lib().attn_decode_no_alloc(ctypes.byref(desc), ctypes.byref(plan), _ptr(q), _ptr(k),
                                      _ptr(v), _ptr(block_table), _ptr(seq_lens), _ptr(out),
                                      _ptr(lse), stream))


# Bytes of the library's per-device scratch behind attn_decode_no_alloc
# (SK_NO_ALLOC_SCRATCH_BYTES in include/splitkv.h).
SK_NO_ALLOC_SCRATCH_BYTES = 64 << 20


def attn_decode_combine_project(desc: SkDesc, plan: SkPlan, seq_lens, workspace,
                                workspace_bytes: int, w_proj, w_dtype: int, proj_dim: int, out,
                                lse, stream: int) -> None:
    _check(lib().attn_decode_combine_project(ctypes.byref(desc), ctypes.byref(plan),
                                             _ptr(seq_lens), _ptr(workspace), int(workspace_bytes),
                                             _ptr(w_proj), int(w_dtype), int(proj_dim), _ptr(out),
                                             _ptr(lse), stream))


def attn_query_tiles_plan(desc: SkDesc, q_len: int, max_seq_len: int, total_tokens: int,
                          cu_count: int, n_splits_requested: int = 0) -> SkPlan:
    plan = SkPlan()
    _check(lib().attn_query_tiles_plan(ctypes.byref(desc), int(q_len), int(max_seq_len),
                                       int(total_tokens), int(cu_count), int(n_splits_requested),
                                       ctypes.byref(plan)))
    return plan


def attn_query_tiles_workspace_bytes(desc: SkDesc, plan: SkPlan, q_len: int) -> int:
    n = lib().attn_query_tiles_workspace_bytes(ctypes.byref(desc), ctypes.byref(plan), int(q_len))
    if n == 0:
        raise SplitKVError(SK_ERR_INVALID_ARG, attn_decode_last_error())
    return int(n)


def attn_query_tiles(desc: SkDesc, plan: SkPlan, q_len: int, q, k, v, seq_lens, workspace,
                     workspace_bytes: int, out, lse, stream: int) -> None:
    _check(lib().attn_query_tiles(ctypes.byref(desc), ctypes.byref(plan), int(q_len), _ptr(q),
                                  _ptr(k), _ptr(v), _ptr(seq_lens), _ptr(workspace),
                                  int(workspace_bytes), _ptr(out), _ptr(lse), stream))


def attn_decode_read_probe(buf, nbytes: int, workgroups: int, scratch, stream: int) -> None:
    _check(lib().attn_decode_read_probe(_ptr(buf), int(nbytes), int(workgroups), _ptr(scratch),
                                        stream))


def attn_decode_kernel_info(desc: SkDesc, plan: SkPlan) -> SkKernelInfo:
    info = SkKernelInfo()
    _check(lib().attn_decode_kernel_info(ctypes.byref(desc), ctypes.byref(plan), ctypes.byref(info)))
    return info
