"""Paged grouped-query attention for MI355X (gfx950).

A thin ctypes binding over ``libpaged_attn.so`` (C ABI in
``include/paged_attn.h``).  It only marshals torch tensors into pointers,
sizes and strides; every step of the attention runs in the library's HIP
kernels.  PyTorch supplies device memory (including the split-KV workspace)
and the stream.  There is no fallback: if the library is missing or no GPU
is present, calls raise.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpaged_attn.so")

PATH_AUTO = 0
PATH_SPLIT_DECODE = 1
PATH_PREFILL = 2

ATTN_OK = 0


class attn_paged_dims(ctypes.Structure):
    _fields_ = [
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
        ("num_tokens", ctypes.c_int64),
        ("q_stride_token", ctypes.c_int64),
        ("q_stride_head", ctypes.c_int64),
        ("o_stride_token", ctypes.c_int64),
        ("o_stride_head", ctypes.c_int64),
        ("kv_stride_page", ctypes.c_int64),
        ("kv_stride_slot", ctypes.c_int64),
        ("kv_stride_head", ctypes.c_int64),
        ("kv_stride_kv", ctypes.c_int64),
        ("bt_stride", ctypes.c_int64),
    ]


class attn_paged_plan(ctypes.Structure):
    _fields_ = [
        ("path", ctypes.c_int32),
        ("pages_per_split", ctypes.c_int32),
        ("max_splits", ctypes.c_int32),
        ("grid_x", ctypes.c_int32),
        ("grid_y", ctypes.c_int32),
        ("grid_z", ctypes.c_int32),
        ("block_threads", ctypes.c_int32),
        ("workspace_bytes", ctypes.c_size_t),
    ]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libpaged_attn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("libpaged_attn.so is not built (%s); run paged_kv_gqa_fwd_amd/build.py" % path)
    lib = ctypes.CDLL(path)
    p, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    dims_p = ctypes.POINTER(attn_paged_dims)
    fwd_args = [p, p, p, p, p, p, i32, i32, ctypes.c_float, i32, dims_p, p, sz, p]
    lib.attn_paged_fwd.argtypes = fwd_args
    lib.attn_paged_fwd.restype = ctypes.c_int
    lib.attn_paged_fwd_ex.argtypes = fwd_args + [i32, i32]
    lib.attn_paged_fwd_ex.restype = ctypes.c_int
    lib.attn_paged_make_plan.argtypes = [dims_p, i32, i32, i32, i32, ctypes.POINTER(attn_paged_plan)]
    lib.attn_paged_make_plan.restype = ctypes.c_int
    lib.attn_paged_workspace_bytes.argtypes = [dims_p, i32, i32, ctypes.POINTER(ctypes.c_size_t)]
    lib.attn_paged_workspace_bytes.restype = ctypes.c_int
    lib.attn_status_string.argtypes = [ctypes.c_int]
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_kernel_timing_enable.argtypes = [i32]
    lib.attn_kernel_timing_enable.restype = ctypes.c_int
    lib.attn_kernel_timing_read.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i32),
                                            ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i32)]
    lib.attn_kernel_timing_read.restype = ctypes.c_int
    lib.attn_version.restype = ctypes.c_int
    _lib = lib
    return lib


class AttnError(RuntimeError):
    def __init__(self, status: int):
        msg = load_library().attn_status_string(status).decode()
        super().__init__("paged attention call failed: status %d (%s)" % (status, msg))
        self.status = status


def make_dims(q: torch.Tensor, kv_pool: torch.Tensor, block_table: torch.Tensor,
              out: Optional[torch.Tensor] = None) -> attn_paged_dims:
    """Sizes and element strides from the tensors (q/out [T, Hq, D]; kv_pool a
    [NP, P, Hkv, 2, D] view; block_table [B, MP])."""
    if q.dim() != 3 or kv_pool.dim() != 5 or block_table.dim() != 2:
        raise ValueError("expected q [T, Hq, D], kv_pool [NP, P, Hkv, 2, D], block_table [B, MP]")
    if kv_pool.shape[3] != 2:
        raise ValueError("kv_pool dim 3 must be 2 (K, V)")
    out = q if out is None else out
    T, hq, d = q.shape
    npg, P, hkv, _, d2 = kv_pool.shape
    if d2 != d or tuple(out.shape) != (T, hq, d):
        raise ValueError("head_dim / output shape mismatch")
    if q.stride(2) != 1 or out.stride(2) != 1 or kv_pool.stride(4) != 1:
        raise ValueError("head_dim axis must be contiguous")
    s = kv_pool.stride()
    return attn_paged_dims(
        num_q_heads=hq, num_kv_heads=hkv, head_dim=d, page_size=P, num_pages=npg,
        max_pages_per_seq=block_table.shape[1], num_tokens=T,
        q_stride_token=q.stride(0), q_stride_head=q.stride(1),
        o_stride_token=out.stride(0), o_stride_head=out.stride(1),
        kv_stride_page=s[0], kv_stride_slot=s[1], kv_stride_head=s[2], kv_stride_kv=s[3],
        bt_stride=block_table.stride(0))


def make_plan(dims: attn_paged_dims, n_seqs: int, max_q: int, path: int = PATH_AUTO,
              pages_per_split: int = 0) -> attn_paged_plan:
    plan = attn_paged_plan()
    rc = load_library().attn_paged_make_plan(ctypes.byref(dims), n_seqs, max_q, path,
                                             pages_per_split, ctypes.byref(plan))
    if rc != ATTN_OK:
        raise AttnError(rc)
    return plan


_ws_cache = {}


def _workspace(nbytes: int, device) -> torch.Tensor:
    key = (str(device),)
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        _ws_cache[key] = buf
    return buf


def _check_device_tensor(name, t, dtype):
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if t.device.type != "cuda":
        raise ValueError("%s must be a GPU tensor (the library has no CPU path)" % name)


def paged_attention(q: torch.Tensor, kv_pool: torch.Tensor, block_table: torch.Tensor,
                    seq_lens: torch.Tensor, cu_q: torch.Tensor, max_q: int, scale: float,
                    causal: bool = True, out: Optional[torch.Tensor] = None,
                    path: int = PATH_AUTO, pages_per_split: int = 0,
                    workspace: Optional[torch.Tensor] = None,
                    stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """Paged GQA attention forward through ``attn_paged_fwd_ex``.

    q [T, Hq, D] bf16, kv_pool [NP, P, Hkv, 2, D] bf16 view, block_table
    [B, MP] int32, seq_lens [B] int32, cu_q [B+1] int32 (all on the GPU).
    Returns ``out`` (allocated as zeros when not given).
    """
    lib = load_library()
    for name, t, dt in (("q", q, torch.bfloat16), ("kv_pool", kv_pool, torch.bfloat16),
                        ("block_table", block_table, torch.int32), ("seq_lens", seq_lens, torch.int32),
                        ("cu_q", cu_q, torch.int32)):
        _check_device_tensor(name, t, dt)
    if out is None:
        out = torch.zeros_like(q)
    _check_device_tensor("out", out, torch.bfloat16)
    if not (seq_lens.is_contiguous() and cu_q.is_contiguous() and block_table.stride(1) == 1):
        raise ValueError("seq_lens / cu_q must be contiguous and block_table rows contiguous")
    n_seqs = seq_lens.numel()
    if cu_q.numel() != n_seqs + 1 or block_table.shape[0] < n_seqs:
        raise ValueError("cu_q must have n_seqs + 1 entries and block_table >= n_seqs rows")
    dims = make_dims(q, kv_pool, block_table, out)
    plan = make_plan(dims, n_seqs, max_q, path, pages_per_split)
    ws_ptr, ws_bytes = None, 0
    if plan.workspace_bytes:
        if workspace is None:
            workspace = _workspace(plan.workspace_bytes, q.device)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    st = stream if stream is not None else torch.cuda.current_stream(q.device)
    rc = lib.attn_paged_fwd_ex(out.data_ptr(), q.data_ptr(), kv_pool.data_ptr(),
                               block_table.data_ptr(), seq_lens.data_ptr(), cu_q.data_ptr(),
                               n_seqs, int(max_q), float(scale), int(bool(causal)),
                               ctypes.byref(dims), ws_ptr, ws_bytes, ctypes.c_void_p(st.cuda_stream),
                               int(path), int(pages_per_split))
    if rc != ATTN_OK:
        raise AttnError(rc)
    return out


def kernel_timing_enable(on: bool) -> None:
    load_library().attn_kernel_timing_enable(1 if on else 0)


def kernel_timing_read():
    """(main_ms_total, main_launches, combine_ms_total, combine_launches)."""
    lib = load_library()
    mm, cm = ctypes.c_double(), ctypes.c_double()
    mn, cn = ctypes.c_int32(), ctypes.c_int32()
    rc = lib.attn_kernel_timing_read(ctypes.byref(mm), ctypes.byref(mn), ctypes.byref(cm), ctypes.byref(cn))
    if rc != ATTN_OK:
        raise AttnError(rc)
    return mm.value, mn.value, cm.value, cn.value
