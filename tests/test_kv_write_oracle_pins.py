"""Pins for the oracle's KV-cache write (CPU only).

The write is the step that runs just before attention (metrale blueprint
graph.json: l3.attn.kv_write, then l3.attn.attend): the step's new K/V rows
go to the slots of key positions L - n .. L - 1 of each sequence.  The pins
tie it to things other than its own scatter:

* only those slots change, every other pool byte stays bitwise the same;
* decode: attention after the write equals the log-sum-exp merge of the
  attention over the L - 1 older keys (the oracle's lse output) with the
  closed-form contribution of the one new key -- so the new token is the
  newest key, seen by its own query;
* prefill chunk: attention after the write equals brute-force dense
  attention over [older keys gathered from the untouched pool] + [new rows
  in order], with bottom-right causal masking;
* tokens without a place in the cache (n > L) are dropped, the last L kept.
"""
import math

import numpy as np
import pytest
import torch

import workloads


def _f64(t):
    return t.float().double().numpy()


def test_only_the_new_slots_change(oracle_mod):
    case = workloads.make_case("w1", 701, [1, 3, 70], [5, 64, 200], 8, 2, 16, causal=True, extra_pages=3)
    k_new, v_new = workloads.new_kv_tokens(case, 11)
    pool = oracle_mod.kv_write(case.kv, k_new, v_new, case.block_table, case.seq_lens, case.cu_q)
    changed = (pool != case.kv).any(dim=4).any(dim=3).any(dim=2)   # [NP, P]
    expect = torch.zeros_like(changed)
    P = case.kv.shape[1]
    for b, (n, L) in enumerate(zip(case.q_lens, case.kv_lens)):
        for pos in range(L - n, L):
            expect[int(case.block_table[b, pos // P]), pos % P] = True
    assert torch.equal(changed, expect)
    # the input pool is left as it was
    assert not torch.equal(pool, case.kv)


def test_decode_write_is_the_newest_key(oracle_mod):
    """out(L keys) = (e^lse_old out_old + e^s_new v_new) / (e^lse_old + e^s_new)."""
    case = workloads.make_case("w2", 702, [1, 1, 1], [1, 65, 300], 8, 2, 32, causal=True, scale=0.2)
    k_new, v_new = workloads.new_kv_tokens(case, 12)
    written = oracle_mod.kv_write(case.kv, k_new, v_new, case.block_table, case.seq_lens, case.cu_q)
    after = oracle_mod.paged_attn(case.q, written, case.block_table, case.seq_lens, case.cu_q,
                                  case.scale, True)
    older_lens = case.seq_lens - 1
    old_out, old_lse = oracle_mod.paged_attn(case.q, case.kv, case.block_table, older_lens, case.cu_q,
                                             case.scale, True, return_lse=True)
    q = _f64(case.q)
    G = 8 // 2
    for t in range(3):
        for h in range(8):
            kn, vn = _f64(k_new[t, h // G]), _f64(v_new[t, h // G])
            s_new = case.scale * float(q[t, h] @ kn)
            if math.isinf(old_lse[t, h]):          # L = 1: the new key is the only key
                expect = vn
            else:
                a, c = math.exp(old_lse[t, h] - s_new), 1.0
                expect = (a * old_out[t, h] + c * vn) / (a + c)
            np.testing.assert_allclose(after[t, h], expect, rtol=0, atol=1e-12)


def test_prefill_chunk_equals_dense_attention(oracle_mod):
    """Chunks of 3 and 70 new tokens on top of 61 and 130 cached keys."""
    q_lens, kv_lens = [3, 70], [64, 200]
    case = workloads.make_case("w3", 703, q_lens, kv_lens, 4, 2, 16, causal=True, scale=0.3)
    k_new, v_new = workloads.new_kv_tokens(case, 13)
    written = oracle_mod.kv_write(case.kv, k_new, v_new, case.block_table, case.seq_lens, case.cu_q)
    after = oracle_mod.paged_attn(case.q, written, case.block_table, case.seq_lens, case.cu_q,
                                  case.scale, True)
    q = _f64(case.q)
    P = case.kv.shape[1]
    t0 = 0
    for b, (n, L) in enumerate(zip(q_lens, kv_lens)):
        old = L - n
        K = np.zeros((L, 2, 16))
        V = np.zeros((L, 2, 16))
        for j in range(old):                     # older keys: untouched pool
            pg = int(case.block_table[b, j // P])
            K[j], V[j] = _f64(case.kv[pg, j % P, :, 0]), _f64(case.kv[pg, j % P, :, 1])
        K[old:], V[old:] = _f64(k_new[t0:t0 + n]), _f64(v_new[t0:t0 + n])
        for i in range(n):
            for h in range(4):
                s = case.scale * (K[:old + i + 1, h // 2] @ q[t0 + i, h])
                w = np.exp(s - s.max())
                np.testing.assert_allclose(after[t0 + i, h], (w / w.sum()) @ V[:old + i + 1, h // 2],
                                           rtol=0, atol=1e-12)
        t0 += n


def test_tokens_beyond_the_cache_are_dropped(oracle_mod):
    """n = 10 new tokens but L = 6 keys: tokens 4..9 take positions 0..5."""
    case = workloads.make_case("w4", 704, [10], [6], 2, 1, 8, causal=True)
    k_new, v_new = workloads.new_kv_tokens(case, 14)
    pool = oracle_mod.kv_write(case.kv, k_new, v_new, case.block_table, case.seq_lens, case.cu_q)
    pg = int(case.block_table[0, 0])
    assert torch.equal(pool[pg, :6, :, 0], k_new[4:])
    assert torch.equal(pool[pg, :6, :, 1], v_new[4:])
    assert torch.equal(pool[pg, 6:], case.kv[pg, 6:])
