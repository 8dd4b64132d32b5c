"""Shared helpers for the parity tests (imported by test modules only)."""
from __future__ import annotations

import sys

import numpy as np
import torch

# Tolerances for the bf16 path against the fp64 oracle.
MAX_ABS = 2e-2
REL_RMS = 5e-3


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def oracle_for(oracle_mod, case, row_mask=None, nthreads: int = 16):
    """Run the oracle on a CPU copy of ``case``."""
    c = case if case.q.device.type == "cpu" else case.to("cpu")
    return oracle_mod.paged_attn(c.q, c.kv, c.block_table, c.seq_lens, c.cu_q, c.scale, c.causal,
                                 row_mask=row_mask, nthreads=nthreads)


def run_gpu(case, path: int = 0, pages_per_split: int = 0, out=None):
    import paged_kv_gqa_fwd_amd as pa
    g = case if case.q.device.type == "cuda" else case.to("cuda")
    log("  gpu call: %s B=%d max_q=%d Hq=%d Hkv=%d D=%d path=%d pps=%d" % (
        case.name, case.n_seqs, case.max_q, case.num_q_heads, case.num_kv_heads, case.head_dim,
        path, pages_per_split))
    res = pa.paged_attention(g.q, g.kv, g.block_table, g.seq_lens, g.cu_q, max(case.max_q, 1),
                             case.scale, case.causal, out=out, path=path,
                             pages_per_split=pages_per_split)
    torch.cuda.synchronize()
    return res


def compare(got: torch.Tensor, ref: np.ndarray, rows=None, max_abs: float = MAX_ABS,
            rel_rms: float = REL_RMS, what: str = ""):
    """Element-wise comparison of the bf16 kernel output with the fp64 oracle
    over the written rows (optionally a row subset)."""
    g = got.detach().float().cpu().double().numpy()
    T = ref.shape[0]
    g = g[:T]
    if rows is not None:
        g, ref = g[rows], ref[rows]
    assert np.isfinite(g).all(), "%s: non-finite output" % what
    err = np.abs(g - ref)
    ma = float(err.max()) if err.size else 0.0
    denom = float(np.linalg.norm(ref))
    rr = float(np.linalg.norm(g - ref)) / denom if denom > 0 else float(np.linalg.norm(g))
    log("  %s: max_abs=%.3e rel_rms=%.3e" % (what, ma, rr))
    assert ma <= max_abs, "%s: max-abs error %.4g > %.4g" % (what, ma, max_abs)
    assert rr <= rel_rms, "%s: rel-RMS error %.4g > %.4g" % (what, rr, rel_rms)
    return ma, rr


def sub_case_rows(case, seq_ids):
    """A CPU PagedCase restricted to ``seq_ids`` (pages gathered into a small
    pool, block table renumbered) plus the token rows those sequences own."""
    import dataclasses
    bt = case.block_table.cpu()
    sl = case.seq_lens.cpu().tolist()
    cu = case.cu_q.cpu().tolist()
    P = case.kv.shape[1]
    pages, new_bt_rows, q_rows, q_lens, kv_lens = [], [], [], [], []
    for b in seq_ids:
        npg = (sl[b] + P - 1) // P
        ids = bt[b, :npg].tolist()
        row = list(range(len(pages), len(pages) + npg))
        pages.extend(ids)
        new_bt_rows.append(row + [-1] * (bt.shape[1] - npg))
        q_rows.extend(range(cu[b], cu[b + 1]))
        q_lens.append(cu[b + 1] - cu[b])
        kv_lens.append(sl[b])
    idx = torch.tensor(pages, dtype=torch.long, device=case.kv.device)
    kv = case.kv.index_select(0, idx).cpu().contiguous()
    q = case.q[torch.tensor(q_rows, dtype=torch.long, device=case.q.device)].cpu()
    cu_new = [0]
    for n in q_lens:
        cu_new.append(cu_new[-1] + n)
    sub = dataclasses.replace(
        case, q=q, pool_storage=kv, kv=kv, block_table=torch.tensor(new_bt_rows, dtype=torch.int32),
        seq_lens=torch.tensor(kv_lens, dtype=torch.int32), cu_q=torch.tensor(cu_new, dtype=torch.int32),
        q_lens=q_lens, kv_lens=kv_lens)
    return sub, q_rows


def dit_sample_rows(n_tokens: int, seed: int = 5) -> np.ndarray:
    """A seeded sample of one in sixteen token rows of the DiT shape (random
    rows plus both ends and the 64- and 256-row tile boundaries)."""
    k = -(-n_tokens // 16)
    pick = set(torch.randperm(n_tokens, generator=torch.Generator().manual_seed(seed))[:k].tolist())
    pick |= {0, 1, 63, 64, 127, 128, 255, 256, n_tokens - 51, n_tokens - 50, n_tokens - 1}
    return np.array(sorted(pick), dtype=np.int64)
