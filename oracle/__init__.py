"""CPU fp64 oracle for paged grouped-query attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never imports,
links or calls it, and it shares no code with the HIP kernels: the C source
next to this file is compiled by ``gcc`` on its own.

``paged_attn`` is masked softmax attention written out as its definition
(see the header of ``paged_attn_oracle.c`` for the formula and the pages it
follows); ``kv_write`` is the cache write that precedes it, a plain scatter.  ``quant_prep`` / ``quant_attn`` emulate the int8 Q.K / fp8 P.V
quantised variant step by step (``quant_oracle.c``); the rounding of the
softmax weights to fp8 inside the fused loop is a reading ("parity
unpinned" by the page, which names that step but not its arithmetic); the
oracle's arithmetic for that reading is pinned by the tests against a
full-row computation and the closed form of the online recurrence.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRCS = [os.path.join(_HERE, "paged_attn_oracle.c"), os.path.join(_HERE, "quant_oracle.c")]
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, no fast-math, OpenMP)."""
    srcs = [s for s in _SRCS if os.path.exists(s)]
    stale = force or not os.path.exists(_LIB_PATH) or any(
        os.path.getmtime(s) > os.path.getmtime(_LIB_PATH) for s in srcs)
    if stale:
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-o", tmp] + srcs + ["-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB_PATH)
        p, i64, i32, f64 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
        lib.oracle_paged_attn.restype = ctypes.c_int
        lib.oracle_paged_attn.argtypes = [
            p, p, p, i64, i64, p, i64, i64, i64, i64, p, i64, p, p,
            i32, i32, i32, i32, i32, f64, i32, p, i64, i32]
        lib.oracle_paged_attn_ex.restype = ctypes.c_int
        lib.oracle_paged_attn_ex.argtypes = lib.oracle_paged_attn.argtypes + [p, i64, i32, f64, f64]
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_quant_prep.restype = ctypes.c_int
        lib.oracle_quant_prep.argtypes = [p, p, p, i32, i32, i32, i32, p, p, p, p, p, p, p, i32]
        lib.oracle_quant_attn.restype = ctypes.c_int
        lib.oracle_quant_attn.argtypes = [p, p, p, p, p, p, i32, i32, i32, i32, f64, i32, i32, p, p, i32]
        lib.oracle_e4m3_encode.restype = ctypes.c_uint8
        lib.oracle_e4m3_encode.argtypes = [f64]
        lib.oracle_e4m3_encode_array.restype = None
        lib.oracle_e4m3_encode_array.argtypes = [p, p, i64]
        lib.oracle_e4m3_decode.restype = ctypes.c_double
        lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        _lib = lib
    return _lib


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def _ptr(t: torch.Tensor) -> int:
    return t.data_ptr()


def paged_attn(q, kv_pool, block_table, seq_lens, cu_q, scale: float, causal: bool,
               row_mask=None, chunk_keys: int = 0, nthreads: int = 0, return_lse: bool = False,
               sinks=None, window: int = 0, k_scale: float = 1.0, v_scale: float = 1.0):
    """fp64 masked softmax attention over a paged KV cache.

    sinks : optional per-q-head sink logits [Hq] (joins the normalisation,
            no value row); window : W > 0 keeps only keys j >= pos - W + 1.
    A uint8 kv_pool holds OCP e4m3 codes: K = k_scale * e4m3(code),
    V = v_scale * e4m3(code).

    q         : bf16 [T, Hq, D] CPU tensor (D contiguous, other strides free)
    kv_pool   : bf16 [NP, P, Hkv, 2, D] CPU tensor view (index 3: 0 = K, 1 = V)
    block_table, seq_lens, cu_q : int32 CPU tensors
    Returns fp64 numpy [T, Hq, D] (rows not covered by cu_q are zero), and
    the natural-log lse [T, Hq] when ``return_lse``.
    """
    lib = _load()
    assert q.dtype == torch.bfloat16 and kv_pool.dtype in (torch.bfloat16, torch.uint8)
    kv_fp8 = kv_pool.dtype == torch.uint8
    assert q.device.type == "cpu" and kv_pool.device.type == "cpu"
    assert q.dim() == 3 and q.stride(2) == 1
    assert kv_pool.dim() == 5 and kv_pool.stride(4) == 1 and kv_pool.shape[3] == 2
    T, hq, d = q.shape
    _, P, hkv, _, d2 = kv_pool.shape
    assert d2 == d
    bt = block_table.to(torch.int32).contiguous()
    sl = seq_lens.to(torch.int32).contiguous()
    cq = cu_q.to(torch.int32).contiguous()
    n_seqs = sl.numel()
    out = np.zeros((T, hq, d), dtype=np.float64)
    lse = np.full((T, hq), -np.inf, dtype=np.float64)
    rm = None
    if row_mask is not None:
        rm = np.ascontiguousarray(np.asarray(row_mask, dtype=np.uint8))
        assert rm.shape == (T,)
    st = kv_pool.stride()
    sk = None
    if sinks is not None:
        sk = np.ascontiguousarray(np.asarray(sinks, dtype=np.float64))
        assert sk.shape == (hq,)
    rc = lib.oracle_paged_attn_ex(
        out.ctypes.data, lse.ctypes.data, _ptr(q), q.stride(0), q.stride(1),
        _ptr(kv_pool), st[0], st[1], st[2], st[3], _ptr(bt), bt.stride(0), _ptr(sl), _ptr(cq),
        n_seqs, hq, hkv, d, P, float(scale), int(bool(causal)),
        rm.ctypes.data if rm is not None else None, int(chunk_keys), int(nthreads),
        sk.ctypes.data if sk is not None else None, int(window), int(kv_fp8), float(k_scale), float(v_scale))
    if rc != 0:
        raise RuntimeError("oracle_paged_attn failed with status %d" % rc)
    return (out, lse) if return_lse else out


def e4m3_quantize(x: torch.Tensor, scale: float) -> torch.Tensor:
    """uint8 OCP e4m3 codes of x * (1 / scale), the reciprocal and the product
    rounded to f32 (the quantised path's reading of "value / scale"), then the
    encoder above (round to nearest even, saturating at +-448)."""
    inv = np.float32(1.0) / np.float32(scale)
    y = np.ascontiguousarray((x.float().numpy() * inv).astype(np.float32))
    out = np.zeros(y.shape, dtype=np.uint8)
    _load().oracle_e4m3_encode_array(y.ctypes.data, out.ctypes.data, y.size)
    return torch.from_numpy(out)


def kv_write(kv_pool, k_new, v_new, block_table, seq_lens, cu_q, k_scale=None, v_scale=None):
    """The KV-cache write that runs just before attention (metrale blueprint
    graph.json: node l3.attn.kv_write precedes l3.attn.attend), into the paged
    layout of kern-kernels examples/decode.json (buffers kv / table / seq /
    cuq).  Returns a new pool; the input pool is not modified.

    For sequence b with n = cu_q[b+1] - cu_q[b] new tokens and L = seq_lens[b]
    keys in all (the new ones included), new token i (row t = cu_q[b] + i) is
    key position pos = L - n + i: its K row k_new[t, g, :] and V row
    v_new[t, g, :] of every KV head g go to page block_table[b][pos // P],
    slot pos % P.  Tokens with pos < 0 (more new tokens than keys) have no
    place in the cache and are not written.

    kv_pool: bf16 [NP, P, Hkv, 2, D] CPU view; k_new, v_new: bf16 [T, Hkv, D].
    A uint8 pool is an fp8 cache: the rows are stored as e4m3_quantize(row,
    k_scale) and e4m3_quantize(row, v_scale).
    """
    pool = kv_pool.clone()
    if pool.dtype == torch.uint8:
        k_new = e4m3_quantize(k_new, k_scale)
        v_new = e4m3_quantize(v_new, v_scale)
    P = pool.shape[1]
    bt = block_table.to(torch.int64)
    for b in range(seq_lens.numel()):
        t0, t1, L = int(cu_q[b]), int(cu_q[b + 1]), int(seq_lens[b])
        n = t1 - t0
        for i in range(n):
            pos = L - n + i
            if pos < 0:
                continue
            page, slot = int(bt[b, pos // P]), pos % P
            pool[page, slot, :, 0, :] = k_new[t0 + i]
            pool[page, slot, :, 1, :] = v_new[t0 + i]
    return pool


QBLOCK = 64  # tokens per int8 scale block


def e4m3_encode(x: float) -> int:
    """OCP E4M3 code of x (round to nearest even, saturating at +-448)."""
    return int(_load().oracle_e4m3_encode(float(x)))


def e4m3_decode(code: int) -> float:
    return float(_load().oracle_e4m3_decode(int(code) & 0xFF))


def quant_prep(q, k, v, nthreads: int = 0) -> dict:
    """Quantisation steps of the int8/fp8 attention variant.

    q, k, v: bf16 [B, N, H, D] CPU tensors (made contiguous here).
    Returns numpy arrays: mk f32 [B,H,D]; qi, ki int8 [B,N,H,D];
    sq, sk f32 [B,H,ceil(N/64)]; vq uint8 e4m3 codes [B,H,D,N]; sv f32 [B,H,D].
    """
    lib = _load()
    q, k, v = (t.contiguous() for t in (q, k, v))
    assert q.dtype == k.dtype == v.dtype == torch.bfloat16 and q.shape == k.shape == v.shape
    B, N, H, D = q.shape
    NB = (N + QBLOCK - 1) // QBLOCK
    r = {"mk": np.zeros((B, H, D), np.float32), "qi": np.zeros((B, N, H, D), np.int8),
         "sq": np.zeros((B, H, NB), np.float32), "ki": np.zeros((B, N, H, D), np.int8),
         "sk": np.zeros((B, H, NB), np.float32), "vq": np.zeros((B, H, D, N), np.uint8),
         "sv": np.zeros((B, H, D), np.float32)}
    rc = lib.oracle_quant_prep(_ptr(q), _ptr(k), _ptr(v), B, N, H, D, r["mk"].ctypes.data,
                               r["qi"].ctypes.data, r["sq"].ctypes.data, r["ki"].ctypes.data,
                               r["sk"].ctypes.data, r["vq"].ctypes.data, r["sv"].ctypes.data,
                               int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_quant_prep failed with status %d" % rc)
    r["shape"] = (B, N, H, D)
    return r


def quant_attn(prep: dict, scale: float, causal: bool, quant_p: bool = True, row_mask=None,
               nthreads: int = 0) -> np.ndarray:
    """Quantised attention from ``quant_prep`` outputs; fp64 [B, N, H, D]."""
    lib = _load()
    B, N, H, D = prep["shape"]
    out = np.zeros((B, N, H, D), np.float64)
    rm = None
    if row_mask is not None:
        rm = np.ascontiguousarray(np.asarray(row_mask, dtype=np.uint8))
        assert rm.shape == (N,)
    arrs = [np.ascontiguousarray(prep[x]) for x in ("qi", "sq", "ki", "sk", "vq", "sv")]
    rc = lib.oracle_quant_attn(*[a.ctypes.data for a in arrs], B, N, H, D, float(scale),
                               int(bool(causal)), int(bool(quant_p)),
                               rm.ctypes.data if rm is not None else None, out.ctypes.data,
                               int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_quant_attn failed with status %d" % rc)
    return out
