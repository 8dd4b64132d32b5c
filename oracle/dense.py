"""Dense fp64 form of the paged attention oracle -- TEST INFRASTRUCTURE ONLY.

Only ``tests/`` (and, through them, nothing else) may import this module; the
product library never imports, links or calls it, and it shares no code with
the HIP kernels.

It computes the same definition as ``oracle_paged_attn`` in
``paged_attn_oracle.c`` -- masked softmax attention over a paged KV cache
(Mojo SM100MHA2Q docs: attention over a KV cache, causal or unmasked, ragged
lengths, grouped q heads; kern-kernels examples/decode.json: the pool, block
table, lengths and cumulative query offsets) -- but takes the library's fp64
matrix product as the step that forms the scores and the weighted sum of V:

  for each sequence b (n = cu_q[b+1] - cu_q[b] queries, L = seq_lens[b] keys)
    K_b, V_b = the pool rows of keys 0 .. L-1, gathered through block_table[b]
    for each q head h (KV head g = h / G):
      S = scale * Q_h K_g^T                      (fp64 matmul, one row per query)
      S[i, j] = -inf where j >= vis_i,  vis_i = causal ? clamp(L - n + i + 1, 0, L) : L
      W = exp(S - rowmax S),  out = (W V_g) / rowsum W   (rows with vis_i = 0 give 0)

Every bf16 input is widened exactly to fp64.  Query rows are independent, so
they are processed in chunks that bound the score matrix's memory, and keys
that no row of a chunk sees (weight exactly 0) are left out of its products;
nothing else is blocked or reordered.  This form exists for the full-size parity
checks, where the per-key loop of the C oracle takes minutes; it is pinned
against that C oracle (an independent implementation of the same definition)
and against the closed forms in tests/test_oracle_pins.py.
"""
from __future__ import annotations

import math

import numpy as np
import torch


def paged_attn_rows(q, kv_pool, block_table, seq_lens, cu_q, scale: float, causal: bool, rows=None,
                    max_scores: int = 1 << 25):
    """fp64 attention for the token rows ``rows`` (all written rows if None).

    q: bf16 [T, Hq, D] CPU; kv_pool: bf16 [NP, P, Hkv, 2, D] CPU view (index 3:
    0 = K, 1 = V); block_table, seq_lens, cu_q: int32 CPU tensors.
    Returns (rows, out): the sorted int64 row indices and fp64 [len(rows), Hq, D].
    """
    assert q.dtype == torch.bfloat16 and kv_pool.dtype == torch.bfloat16
    assert q.device.type == "cpu" and kv_pool.device.type == "cpu"
    T, hq, d = q.shape
    _, P, hkv, two, d2 = kv_pool.shape
    assert two == 2 and d2 == d and hq % hkv == 0
    G = hq // hkv
    cu = [int(x) for x in cu_q.tolist()]
    sl = [int(x) for x in seq_lens.tolist()]
    B = len(sl)
    written = cu[B]
    if rows is None:
        want = np.arange(written, dtype=np.int64)
    else:
        want = np.unique(np.asarray(rows, dtype=np.int64))
        assert want.size == 0 or (want[0] >= 0 and want[-1] < written)
    out = np.zeros((want.size, hq, d), dtype=np.float64)
    bt = block_table.to(torch.int64)
    for b in range(B):
        q0, q1, L = cu[b], cu[b + 1], sl[b]
        n = q1 - q0
        lo_i, hi_i = np.searchsorted(want, q0), np.searchsorted(want, q1)
        if hi_i == lo_i or L == 0:
            continue   # no requested row, or no key: rows stay zero
        tok = want[lo_i:hi_i]
        i = tok - q0
        vis = np.clip(L - n + i + 1, 0, L) if causal else np.full(i.shape, L)
        npg = math.ceil(L / P)
        kvb = kv_pool[bt[b, :npg]].reshape(npg * P, hkv, 2, d)[:L]      # bf16 [L, Hkv, 2, D]
        qb = q[torch.from_numpy(tok)].double()                            # [ni, Hq, D]
        vis_t = torch.from_numpy(vis)
        key_idx = torch.arange(L)
        chunk = max(1, max_scores // L)     # query rows per score matrix
        for g in range(hkv):
            K = kvb[:, g, 0, :].double()
            V = kvb[:, g, 1, :].double()
            for hh in range(G):
                h = g * G + hh
                for c0 in range(0, tok.size, chunk):
                    c1 = min(tok.size, c0 + chunk)
                    vc = vis_t[c0:c1]
                    # keys no row of the chunk sees have weight exactly 0: leave them out
                    kmax = max(1, int(vc.max()))
                    S = (qb[c0:c1, h, :] @ K[:kmax].T) * scale            # [nc, kmax]
                    if causal and int(vc.min()) < kmax:
                        S.masked_fill_(key_idx[None, :kmax] >= vc[:, None], -math.inf)
                    has = vc > 0
                    m = S.max(dim=1).values
                    m = torch.where(has, m, torch.zeros_like(m))          # rows with no key: all -inf
                    W = torch.exp(S - m[:, None])
                    l = W.sum(dim=1)
                    O = (W @ V[:kmax]) / torch.where(has, l, torch.ones_like(l))[:, None]
                    O[~has] = 0.0
                    out[lo_i + c0:lo_i + c1, h, :] = O.numpy()
    return want, out
