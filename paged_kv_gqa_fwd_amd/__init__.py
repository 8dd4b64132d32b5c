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
PATH_SPLIT_DECODE = 1   # split-KV kernel + combine kernel
PATH_PREFILL = 2
PATH_SPLIT_FUSED = 3    # split-KV kernel whose last split per (sequence, KV head) merges
PATH_SPLIT_BALANCED = 4  # split-KV over equal page ranges of the whole batch + combine kernel
KV_BF16 = 0
KV_FP8_E4M3 = 1         # OCP e4m3 codes with per-tensor K and V scales

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


class attn_quant_dims(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("seq_len", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("q_stride", ctypes.c_int64 * 3),
        ("k_stride", ctypes.c_int64 * 3),
        ("v_stride", ctypes.c_int64 * 3),
        ("o_stride", ctypes.c_int64 * 3),
    ]


class attn_quant_layout(ctypes.Structure):
    _fields_ = [
        ("workspace_bytes", ctypes.c_size_t),
        ("off_mk", ctypes.c_size_t), ("off_sv", ctypes.c_size_t), ("off_sq", ctypes.c_size_t),
        ("off_sk", ctypes.c_size_t), ("off_qi", ctypes.c_size_t), ("off_ki", ctypes.c_size_t),
        ("off_vt", ctypes.c_size_t), ("off_ksum", ctypes.c_size_t), ("off_vmax", ctypes.c_size_t),
        ("blocks", ctypes.c_int32),
        ("chunks", ctypes.c_int32),
        ("vt_stride", ctypes.c_int32),
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
        ("counter_bytes", ctypes.c_size_t),
    ]


class attn_paged_options(ctypes.Structure):
    _fields_ = [
        ("sinks", ctypes.c_void_p),
        ("window", ctypes.c_int32),
        ("path_hint", ctypes.c_int32),
        ("pages_per_split", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("k_scale", ctypes.c_float),
        ("v_scale", ctypes.c_float),
    ]


class attn_kv_new_dims(ctypes.Structure):
    _fields_ = [
        ("k_stride_token", ctypes.c_int64),
        ("k_stride_head", ctypes.c_int64),
        ("v_stride_token", ctypes.c_int64),
        ("v_stride_head", ctypes.c_int64),
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
    opt_p = ctypes.POINTER(attn_paged_options)
    lib.attn_paged_make_plan_opt.argtypes = [dims_p, i32, i32, opt_p, ctypes.POINTER(attn_paged_plan)]
    lib.attn_paged_make_plan_opt.restype = ctypes.c_int
    lib.attn_paged_fwd_opt.argtypes = [p, p, p, p, p, p, i32, i32, ctypes.c_float, i32, dims_p, opt_p, p, sz, p]
    lib.attn_paged_fwd_opt.restype = ctypes.c_int
    lib.attn_paged_fwd_noalloc.argtypes = [p, p, p, p, p, p, i32, i32, ctypes.c_float, i32, dims_p, opt_p, p]
    lib.attn_paged_fwd_noalloc.restype = ctypes.c_int
    lib.attn_paged_make_plan.restype = ctypes.c_int
    lib.attn_paged_workspace_bytes.argtypes = [dims_p, i32, i32, ctypes.POINTER(ctypes.c_size_t)]
    lib.attn_paged_workspace_bytes.restype = ctypes.c_int
    nd_p = ctypes.POINTER(attn_kv_new_dims)
    lib.attn_paged_kv_write.argtypes = [p, p, p, p, p, p, i32, i32, dims_p, nd_p, p]
    lib.attn_paged_kv_write.restype = ctypes.c_int
    lib.attn_paged_fwd_write.argtypes = [p, p, p, p, p, p, p, p, i32, i32, ctypes.c_float, i32, dims_p, nd_p,
                                         p, sz, p]
    lib.attn_paged_fwd_write.restype = ctypes.c_int
    lib.attn_paged_kv_write_opt.argtypes = [p, p, p, p, p, p, i32, i32, dims_p, nd_p, ctypes.POINTER(attn_paged_options), p]
    lib.attn_paged_kv_write_opt.restype = ctypes.c_int
    lib.attn_paged_fwd_write_opt.argtypes = [p, p, p, p, p, p, p, p, i32, i32, ctypes.c_float, i32, dims_p, nd_p,
                                             ctypes.POINTER(attn_paged_options), p, sz, p]
    lib.attn_paged_fwd_write_opt.restype = ctypes.c_int
    lib.attn_workspace_clear.argtypes = [p, sz, p]
    lib.attn_workspace_clear.restype = ctypes.c_int
    lib.attn_status_string.argtypes = [ctypes.c_int]
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_kernel_timing_enable.argtypes = [i32]
    lib.attn_kernel_timing_enable.restype = ctypes.c_int
    dp, ip = ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i32)
    lib.attn_kernel_timing_read.argtypes = [dp, ip, dp, ip, dp, ip, dp, ip]
    lib.attn_kernel_timing_read.restype = ctypes.c_int
    lib.attn_stream_read.argtypes = [p, sz, p, i32, i32, p]
    lib.attn_stream_read.restype = ctypes.c_int
    qd_p = ctypes.POINTER(attn_quant_dims)
    lib.attn_quant_layout_of.argtypes = [qd_p, ctypes.POINTER(attn_quant_layout)]
    lib.attn_quant_layout_of.restype = ctypes.c_int
    lib.attn_quant_prep.argtypes = [p, p, p, qd_p, p, sz, p]
    lib.attn_quant_prep.restype = ctypes.c_int
    lib.attn_quant_attend.argtypes = [p, qd_p, ctypes.c_float, i32, p, sz, p]
    lib.attn_quant_attend.restype = ctypes.c_int
    lib.attn_quant_fwd.argtypes = [p, p, p, p, qd_p, ctypes.c_float, i32, p, sz, p]
    lib.attn_quant_fwd.restype = ctypes.c_int
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
              pages_per_split: int = 0, window: int = 0, kv_dtype: int = 0) -> attn_paged_plan:
    plan = attn_paged_plan()
    opt = attn_paged_options(None, int(window), int(path), int(pages_per_split), int(kv_dtype), 1.0, 1.0)
    rc = load_library().attn_paged_make_plan_opt(ctypes.byref(dims), n_seqs, max_q, ctypes.byref(opt),
                                                 ctypes.byref(plan))
    if rc != ATTN_OK:
        raise AttnError(rc)
    return plan


class _CachedWorkspace:
    """One workspace per (device, stream), grown on demand.  `clean` counts
    the leading bytes known to be zero: the fused split path needs its
    counter bytes zero on entry and leaves them zero, while partials written
    by any split call dirty everything past that call's counter bytes."""

    def __init__(self):
        self.buf = None
        self.clean = 0


_ws_cache = {}


def _workspace(nbytes: int, device, stream: torch.cuda.Stream) -> _CachedWorkspace:
    """The cached workspace of `stream`.  Calls on one stream run in order, so
    they may share it; each stream has its own, so that calls on different
    streams never overwrite each other's partials.  A grown buffer is
    allocated with `stream` current: the caching allocator then hands the
    old one to later allocations only in that stream's order, after the
    kernels already queued on it."""
    key = (str(device), int(stream.cuda_stream))
    ws = _ws_cache.setdefault(key, _CachedWorkspace())
    if ws.buf is None or ws.buf.numel() < nbytes:
        ws.buf = None
        with torch.cuda.stream(stream):
            ws.buf = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
        ws.clean = ws.buf.numel()
    return ws


def workspace_clear(workspace: torch.Tensor, nbytes: int, stream=None) -> None:
    """Zero the first ``nbytes`` of a workspace (``attn_workspace_clear``)."""
    st = stream if stream is not None else torch.cuda.current_stream(workspace.device)
    rc = load_library().attn_workspace_clear(workspace.data_ptr(), int(nbytes), ctypes.c_void_p(st.cuda_stream))
    if rc != ATTN_OK:
        raise AttnError(rc)


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
                    stream: Optional[torch.cuda.Stream] = None,
                    sinks: Optional[torch.Tensor] = None, window: int = 0,
                    k_scale: float = 1.0, v_scale: float = 1.0) -> torch.Tensor:
    """Paged GQA attention forward through ``attn_paged_fwd_opt``.

    sinks: optional f32 [Hq] GPU tensor of per-q-head sink logits; window:
    0 = none, W > 0 = each query sees only its last W key positions.  A uint8
    kv_pool is an fp8 (OCP e4m3) cache: K = k_scale * e4m3, V = v_scale * e4m3.

    q [T, Hq, D] bf16, kv_pool [NP, P, Hkv, 2, D] bf16 view, block_table
    [B, MP] int32, seq_lens [B] int32, cu_q [B+1] int32 (all on the GPU).
    Returns ``out`` (allocated as zeros when not given).  Without
    ``workspace`` a cached per-device buffer is used (its merge counters are
    kept zero); a caller-supplied ``workspace`` must have its first
    ``plan.counter_bytes`` bytes zero on the fused split path (see
    ``workspace_clear``).
    """
    lib = load_library()
    kv_dtype = KV_FP8_E4M3 if kv_pool.dtype == torch.uint8 else KV_BF16
    for name, t, dt in (("q", q, torch.bfloat16), ("kv_pool", kv_pool, torch.uint8 if kv_dtype else torch.bfloat16),
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
    plan = make_plan(dims, n_seqs, max_q, path, pages_per_split, window, kv_dtype)
    sinks_ptr = None
    if sinks is not None:
        _check_device_tensor("sinks", sinks, torch.float32)
        if sinks.numel() != q.shape[1] or not sinks.is_contiguous():
            raise ValueError("sinks must be a contiguous f32 tensor with one entry per q head")
        sinks_ptr = sinks.data_ptr()
    opt = attn_paged_options(sinks_ptr, int(window), int(path), int(pages_per_split), kv_dtype, float(k_scale),
                             float(v_scale))
    ws_ptr, ws_bytes, cached = None, 0, None
    st = stream if stream is not None else torch.cuda.current_stream(q.device)
    if plan.workspace_bytes:
        if workspace is None:
            cached = _workspace(plan.workspace_bytes, q.device, st)
            workspace = cached.buf
            if cached.clean < plan.counter_bytes:
                workspace_clear(workspace, plan.counter_bytes, st)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    rc = lib.attn_paged_fwd_opt(out.data_ptr(), q.data_ptr(), kv_pool.data_ptr(),
                                block_table.data_ptr(), seq_lens.data_ptr(), cu_q.data_ptr(),
                                n_seqs, int(max_q), float(scale), int(bool(causal)),
                                ctypes.byref(dims), ctypes.byref(opt), ws_ptr, ws_bytes,
                                ctypes.c_void_p(st.cuda_stream))
    if rc != ATTN_OK:
        raise AttnError(rc)
    if cached is not None:
        cached.clean = plan.counter_bytes
    return out


NOALLOC_SCRATCH_BYTES = 64 << 20   # ATTN_NOALLOC_SCRATCH_BYTES


def paged_attention_noalloc(q: torch.Tensor, kv_pool: torch.Tensor, block_table: torch.Tensor,
                            seq_lens: torch.Tensor, cu_q: torch.Tensor, max_q: int, scale: float,
                            out: torch.Tensor, causal: bool = True, path: int = PATH_AUTO,
                            pages_per_split: int = 0, stream: Optional[torch.cuda.Stream] = None,
                            sinks: Optional[torch.Tensor] = None, window: int = 0,
                            k_scale: float = 1.0, v_scale: float = 1.0) -> torch.Tensor:
    """``attn_paged_fwd_noalloc``: the paged call with no workspace; its
    partials live in the library's per-GPU scratch array.  ``out`` must be
    given (nothing is allocated here either).  Calls that overlap in time on
    one GPU race on the shared scratch."""
    lib = load_library()
    kv_dtype = KV_FP8_E4M3 if kv_pool.dtype == torch.uint8 else KV_BF16
    for name, t, dt in (("q", q, torch.bfloat16), ("kv_pool", kv_pool, torch.uint8 if kv_dtype else torch.bfloat16),
                        ("block_table", block_table, torch.int32), ("seq_lens", seq_lens, torch.int32),
                        ("cu_q", cu_q, torch.int32), ("out", out, torch.bfloat16)):
        _check_device_tensor(name, t, dt)
    n_seqs = seq_lens.numel()
    dims = make_dims(q, kv_pool, block_table, out)
    sinks_ptr = sinks.data_ptr() if sinks is not None else None
    opt = attn_paged_options(sinks_ptr, int(window), int(path), int(pages_per_split), kv_dtype, float(k_scale),
                             float(v_scale))
    st = stream if stream is not None else torch.cuda.current_stream(q.device)
    rc = lib.attn_paged_fwd_noalloc(out.data_ptr(), q.data_ptr(), kv_pool.data_ptr(), block_table.data_ptr(),
                                    seq_lens.data_ptr(), cu_q.data_ptr(), n_seqs, int(max_q), float(scale),
                                    int(bool(causal)), ctypes.byref(dims), ctypes.byref(opt),
                                    ctypes.c_void_p(st.cuda_stream))
    if rc != ATTN_OK:
        raise AttnError(rc)
    return out


def _new_kv_dims(k_new: torch.Tensor, v_new: torch.Tensor) -> attn_kv_new_dims:
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        _check_device_tensor(name, t, torch.bfloat16)
        if t.dim() != 3 or t.stride(2) != 1:
            raise ValueError("%s must be [T, Hkv, D] with D contiguous" % name)
    return attn_kv_new_dims(k_new.stride(0), k_new.stride(1), v_new.stride(0), v_new.stride(1))


def _pool_dtype(kv_pool: torch.Tensor) -> int:
    if kv_pool.dtype == torch.uint8:
        return KV_FP8_E4M3
    _check_device_tensor("kv_pool", kv_pool, torch.bfloat16)
    return KV_BF16


def kv_write(kv_pool: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, block_table: torch.Tensor,
             seq_lens: torch.Tensor, cu_q: torch.Tensor, max_q: int, q_like: Optional[torch.Tensor] = None,
             stream: Optional[torch.cuda.Stream] = None, k_scale: float = 1.0, v_scale: float = 1.0) -> None:
    """The KV-cache write (``attn_paged_kv_write_opt``): the new K/V rows
    k_new / v_new [T, Hkv, D] go to key positions L - n .. L - 1 of each
    sequence (as e4m3 codes of x / scale into a uint8 fp8 cache).  ``q_like``
    ([T, Hq, D]) supplies the q-head count of the dims (one q head per KV
    head is described when absent)."""
    lib = load_library()
    kv_dtype = _pool_dtype(kv_pool)
    if q_like is not None:
        dims = make_dims(q_like, kv_pool, block_table, q_like)
    else:
        # no q: describe packed [T, Hkv, D] rows with one q head per KV head
        T, hkv, d = k_new.shape
        s = kv_pool.stride()
        dims = attn_paged_dims(
            num_q_heads=hkv, num_kv_heads=kv_pool.shape[2], head_dim=d, page_size=kv_pool.shape[1],
            num_pages=kv_pool.shape[0], max_pages_per_seq=block_table.shape[1], num_tokens=T,
            q_stride_token=hkv * d, q_stride_head=d, o_stride_token=hkv * d, o_stride_head=d,
            kv_stride_page=s[0], kv_stride_slot=s[1], kv_stride_head=s[2], kv_stride_kv=s[3],
            bt_stride=block_table.stride(0))
    nd = _new_kv_dims(k_new, v_new)
    opt = attn_paged_options(None, 0, 0, 0, kv_dtype, float(k_scale), float(v_scale))
    st = stream if stream is not None else torch.cuda.current_stream(kv_pool.device)
    rc = lib.attn_paged_kv_write_opt(kv_pool.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), block_table.data_ptr(),
                                     seq_lens.data_ptr(), cu_q.data_ptr(), seq_lens.numel(), int(max_q),
                                     ctypes.byref(dims), ctypes.byref(nd), ctypes.byref(opt),
                                     ctypes.c_void_p(st.cuda_stream))
    if rc != ATTN_OK:
        raise AttnError(rc)


def paged_attention_write(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, kv_pool: torch.Tensor,
                          block_table: torch.Tensor, seq_lens: torch.Tensor, cu_q: torch.Tensor, max_q: int,
                          scale: float, causal: bool = True, out: Optional[torch.Tensor] = None,
                          stream: Optional[torch.cuda.Stream] = None, k_scale: float = 1.0,
                          v_scale: float = 1.0, path: int = PATH_AUTO, pages_per_split: int = 0,
                          sinks: Optional[torch.Tensor] = None, window: int = 0) -> torch.Tensor:
    """The cache write then attention in one call (``attn_paged_fwd_write_opt``;
    on the split paths the write runs inside the attention launch)."""
    lib = load_library()
    _check_device_tensor("q", q, torch.bfloat16)
    kv_dtype = _pool_dtype(kv_pool)
    if out is None:
        out = torch.zeros_like(q)
    dims = make_dims(q, kv_pool, block_table, out)
    nd = _new_kv_dims(k_new, v_new)
    plan = make_plan(dims, seq_lens.numel(), max_q, path, pages_per_split, window, kv_dtype)
    sinks_ptr = None
    if sinks is not None:
        _check_device_tensor("sinks", sinks, torch.float32)
        sinks_ptr = sinks.data_ptr()
    opt = attn_paged_options(sinks_ptr, int(window), int(path), int(pages_per_split), kv_dtype, float(k_scale),
                             float(v_scale))
    st = stream if stream is not None else torch.cuda.current_stream(q.device)
    ws_ptr, ws_bytes, cached = None, 0, None
    if plan.workspace_bytes:
        cached = _workspace(plan.workspace_bytes, q.device, st)
        if cached.clean < plan.counter_bytes:
            workspace_clear(cached.buf, plan.counter_bytes, st)
        ws_ptr, ws_bytes = cached.buf.data_ptr(), cached.buf.numel()
    rc = lib.attn_paged_fwd_write_opt(out.data_ptr(), q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(),
                                      kv_pool.data_ptr(), block_table.data_ptr(), seq_lens.data_ptr(),
                                      cu_q.data_ptr(), seq_lens.numel(), int(max_q), float(scale),
                                      int(bool(causal)), ctypes.byref(dims), ctypes.byref(nd), ctypes.byref(opt),
                                      ws_ptr, ws_bytes, ctypes.c_void_p(st.cuda_stream))
    if rc != ATTN_OK:
        raise AttnError(rc)
    if cached is not None:
        cached.clean = plan.counter_bytes
    return out


def stream_read(buf: torch.Tensor, grid: int = 512, sink: Optional[torch.Tensor] = None,
                stream: Optional[torch.cuda.Stream] = None, depth: int = 4) -> torch.Tensor:
    """Read the bytes of a contiguous GPU tensor once through
    ``attn_stream_read`` (the plain HBM read stream used as the on-box read
    ceiling).  Returns the sink (uint32 [grid * 256], overwritten)."""
    lib = load_library()
    if not (buf.is_cuda and buf.is_contiguous()):
        raise ValueError("buf must be a contiguous GPU tensor")
    nbytes = buf.numel() * buf.element_size()
    if sink is None:
        sink = torch.empty(grid * 256, dtype=torch.int32, device=buf.device)
    if sink.numel() < grid * 256 or not sink.is_cuda:
        raise ValueError("sink must be a GPU tensor of at least grid * 256 int32")
    st = stream if stream is not None else torch.cuda.current_stream(buf.device)
    rc = lib.attn_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), int(grid), int(depth),
                              ctypes.c_void_p(st.cuda_stream))
    if rc != ATTN_OK:
        raise AttnError(rc)
    return sink


def kernel_timing_enable(on: bool) -> None:
    load_library().attn_kernel_timing_enable(1 if on else 0)


def kernel_timing_read():
    """(main_ms_total, main_launches, combine_ms_total, combine_launches,
    prep_ms_total, prep_launches, write_ms_total, write_launches)."""
    lib = load_library()
    v = [ctypes.c_double(), ctypes.c_int32(), ctypes.c_double(), ctypes.c_int32(),
         ctypes.c_double(), ctypes.c_int32(), ctypes.c_double(), ctypes.c_int32()]
    rc = lib.attn_kernel_timing_read(*[ctypes.byref(x) for x in v])
    if rc != ATTN_OK:
        raise AttnError(rc)
    return tuple(x.value for x in v)


# ---------------------------------------------------------------- quantised path
def make_quant_dims(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                    out: Optional[torch.Tensor] = None) -> attn_quant_dims:
    """Sizes and element strides of dense [B, N, H, D] q / k / v / out."""
    out = q if out is None else out
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        if t.dim() != 4 or tuple(t.shape) != tuple(q.shape):
            raise ValueError("%s must be [B, N, H, D] like q" % name)
        if t.stride(3) != 1:
            raise ValueError("head_dim axis of %s must be contiguous" % name)
    B, N, H, D = q.shape
    dims = attn_quant_dims(batch=B, seq_len=N, num_heads=H, head_dim=D)
    for field, t in (("q_stride", q), ("k_stride", k), ("v_stride", v), ("o_stride", out)):
        arr = getattr(dims, field)
        for i in range(3):
            arr[i] = t.stride(i)
    return dims


def quant_layout(dims: attn_quant_dims) -> attn_quant_layout:
    lay = attn_quant_layout()
    rc = load_library().attn_quant_layout_of(ctypes.byref(dims), ctypes.byref(lay))
    if rc != ATTN_OK:
        raise AttnError(rc)
    return lay


def quant_prep(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
               workspace: Optional[torch.Tensor] = None,
               stream: Optional[torch.cuda.Stream] = None):
    """Quantisation steps (``attn_quant_prep``); returns (workspace, layout)."""
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_device_tensor(name, t, torch.bfloat16)
    dims = make_quant_dims(q, k, v)
    lay = quant_layout(dims)
    if workspace is None:
        workspace = torch.empty(lay.workspace_bytes, dtype=torch.uint8, device=q.device)
    st = stream if stream is not None else torch.cuda.current_stream(q.device)
    rc = lib.attn_quant_prep(q.data_ptr(), k.data_ptr(), v.data_ptr(), ctypes.byref(dims),
                             workspace.data_ptr(), workspace.numel(), ctypes.c_void_p(st.cuda_stream))
    if rc != ATTN_OK:
        raise AttnError(rc)
    return workspace, lay


def quant_attend(q_shape_like: torch.Tensor, workspace: torch.Tensor, scale: float,
                 causal: bool = False, out: Optional[torch.Tensor] = None,
                 stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """Fused quantised attention loop (``attn_quant_attend``) from a prepared
    workspace; ``q_shape_like`` gives the [B, N, H, D] shape and device."""
    lib = load_library()
    if out is None:
        out = torch.empty(q_shape_like.shape, dtype=torch.bfloat16, device=q_shape_like.device)
    _check_device_tensor("out", out, torch.bfloat16)
    _check_device_tensor("workspace", workspace, torch.uint8)
    dims = make_quant_dims(out, out, out, out)
    st = stream if stream is not None else torch.cuda.current_stream(out.device)
    rc = lib.attn_quant_attend(out.data_ptr(), ctypes.byref(dims), float(scale), int(bool(causal)),
                               workspace.data_ptr(), workspace.numel(), ctypes.c_void_p(st.cuda_stream))
    if rc != ATTN_OK:
        raise AttnError(rc)
    return out


def quant_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: float,
                    causal: bool = False, out: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None,
                    stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """Quantised attention in one call (``attn_quant_fwd``): q, k, v dense
    bf16 [B, N, H, D] on the GPU; returns out bf16 [B, N, H, D]."""
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_device_tensor(name, t, torch.bfloat16)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    _check_device_tensor("out", out, torch.bfloat16)
    dims = make_quant_dims(q, k, v, out)
    lay = quant_layout(dims)
    st = stream if stream is not None else torch.cuda.current_stream(q.device)
    if workspace is None:
        cached = _workspace(lay.workspace_bytes, q.device, st)
        cached.clean = 0   # the quantised intermediates overwrite it
        workspace = cached.buf
    rc = lib.attn_quant_fwd(out.data_ptr(), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                            ctypes.byref(dims), float(scale), int(bool(causal)), workspace.data_ptr(),
                            workspace.numel() * workspace.element_size(), ctypes.c_void_p(st.cuda_stream))
    if rc != ATTN_OK:
        raise AttnError(rc)
    return out


def quant_workspace_views(workspace: torch.Tensor, lay: attn_quant_layout, shape):
    """Typed views of the quantised intermediates inside a workspace."""
    B, N, H, D = shape
    def view(off, n, dtype):
        nbytes = n * torch.tensor([], dtype=dtype).element_size()
        return workspace[off:off + nbytes].view(dtype)
    return {
        "mk": view(lay.off_mk, B * H * D, torch.float32).view(B, H, D),
        "sv": view(lay.off_sv, B * H * D, torch.float32).view(B, H, D),
        "sq": view(lay.off_sq, B * H * lay.blocks, torch.float32).view(B, H, lay.blocks),
        "sk": view(lay.off_sk, B * H * lay.blocks, torch.float32).view(B, H, lay.blocks),
        "qi": view(lay.off_qi, B * N * H * D, torch.int8).view(B, N, H, D),
        "ki": view(lay.off_ki, B * N * H * D, torch.int8).view(B, N, H, D),
        "vt": view(lay.off_vt, B * H * D * lay.vt_stride, torch.uint8).view(B, H, D, lay.vt_stride),
    }
