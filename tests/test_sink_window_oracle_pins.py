"""Pins for the oracle's attention-sink and sliding-window variants (CPU only).

Readings (the pages only name the features): a sink is one logit per q head,
in the units of the scaled scores, that joins the softmax normalisation and
carries no value row; a window W > 0 keeps only keys j >= pos - W + 1 for a
query at position pos.  Each pin ties the oracle to something other than its
own code:

* brute force: numpy dense attention with an explicit extra score column for
  the sink (value row 0) and an explicit [lo, vis) mask;
* closed forms: one visible key and a sink give V sigma(s - sink); W = 1 under
  causal masking gives the query's own V row; the sink rescales the no-sink
  output by 1 / (1 + e^(sink - lse));
* invariants: a -inf sink and a window >= L change nothing (bitwise); a
  decode row with window W equals the same row over a sequence cut to its last
  W keys (page-aligned cut: shifted block table, bitwise).
"""
import math

import numpy as np
import pytest
import torch

import workloads


def _f64(t):
    return t.float().double().numpy()


def _dense(case):
    kv, P = case.kv, case.kv.shape[1]
    res = []
    for b, L in enumerate(case.kv_lens):
        K = np.zeros((L, kv.shape[2], kv.shape[4]))
        V = np.zeros_like(K)
        for j in range(L):
            pg = int(case.block_table[b, j // P])
            K[j], V[j] = _f64(kv[pg, j % P, :, 0]), _f64(kv[pg, j % P, :, 1])
        res.append((K, V))
    return res


def brute(case, sinks=None, window=0):
    q = _f64(case.q)
    T, hq, d = q.shape
    G = hq // case.num_kv_heads
    out = np.zeros((T, hq, d))
    t0 = 0
    for (n, L), (K, V) in zip(zip(case.q_lens, case.kv_lens), _dense(case)):
        for i in range(n):
            pos = L - n + i
            vis = min(max(pos + 1, 0), L) if case.causal else L
            lo = max(0, pos - window + 1) if window > 0 else 0
            for h in range(hq):
                s = [case.scale * float(K[j, h // G] @ q[t0 + i, h]) for j in range(lo, vis)]
                vals = [V[j, h // G] for j in range(lo, vis)]
                if sinks is not None:
                    s.append(float(sinks[h]))
                    vals.append(np.zeros(d))
                if not s or max(s) == -math.inf:
                    continue
                s = np.array(s)
                w = np.exp(s - s.max())
                out[t0 + i, h] = (w / w.sum()) @ np.array(vals)
        t0 += n
    return out


def _run(oracle_mod, case, **kw):
    return oracle_mod.paged_attn(case.q, case.kv, case.block_table, case.seq_lens, case.cu_q,
                                 case.scale, case.causal, **kw)


CASES = [
    dict(q_lens=[1, 1, 1], kv_lens=[1, 70, 200], hq=8, hkv=2, d=16, causal=True, window=50),
    dict(q_lens=[5, 40], kv_lens=[5, 130], hq=6, hkv=1, d=8, causal=True, window=64),
    dict(q_lens=[7, 2], kv_lens=[70, 9], hq=4, hkv=2, d=16, causal=False, window=20),
    dict(q_lens=[10, 4], kv_lens=[6, 64], hq=4, hkv=2, d=8, causal=True, window=3),   # n > L rows
    dict(q_lens=[3], kv_lens=[129], hq=2, hkv=1, d=8, causal=True, window=1),
]


@pytest.mark.parametrize("idx", range(len(CASES)))
@pytest.mark.parametrize("with_sink", [False, True])
@pytest.mark.parametrize("with_window", [False, True])
def test_brute_force(oracle_mod, idx, with_sink, with_window):
    c = dict(CASES[idx])
    W = c.pop("window") if with_window else 0
    c.pop("window", None)
    case = workloads.make_case("sw", 720 + idx, c["q_lens"], c["kv_lens"], c["hq"], c["hkv"], c["d"],
                               causal=c["causal"], scale=0.4)
    sinks = None
    if with_sink:
        sinks = np.linspace(-3.0, 5.0, c["hq"])
        sinks[0] = -math.inf          # a head without a sink
    got = _run(oracle_mod, case, sinks=sinks, window=W)
    np.testing.assert_allclose(got, brute(case, sinks, W), rtol=0, atol=1e-12)


def test_neutral_settings_change_nothing(oracle_mod):
    case = workloads.make_case("sw-n", 730, [3, 1], [100, 300], 8, 2, 32, causal=True)
    base, lse0 = _run(oracle_mod, case, return_lse=True)
    for kw in (dict(sinks=np.full(8, -np.inf)), dict(window=300), dict(window=10 ** 6), dict(window=0)):
        got, lse = _run(oracle_mod, case, return_lse=True, **kw)
        assert np.array_equal(got, base) and np.array_equal(lse, lse0), kw


def test_sink_rescales_by_lse(oracle_mod):
    case = workloads.make_case("sw-l", 731, [1, 20], [50, 90], 4, 2, 16, causal=True, scale=0.3)
    base, lse = _run(oracle_mod, case, return_lse=True)
    sinks = np.array([-1.0, 0.5, 2.0, 6.0])
    got, lse_s = _run(oracle_mod, case, sinks=sinks, return_lse=True)
    np.testing.assert_allclose(got, base / (1.0 + np.exp(sinks[None, :, None] - lse[:, :, None])),
                               rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse_s, np.logaddexp(lse, sinks[None, :]), rtol=0, atol=1e-12)


def test_one_key_and_a_sink_closed_form(oracle_mod):
    case = workloads.make_case("sw-1", 732, [1], [1], 2, 1, 8, causal=True, scale=0.7)
    q, k, v = _f64(case.q[0]), _f64(case.kv[int(case.block_table[0, 0]), 0, 0, 0]), \
        _f64(case.kv[int(case.block_table[0, 0]), 0, 0, 1])
    sinks = np.array([0.25, -2.0])
    got = _run(oracle_mod, case, sinks=sinks)
    for h in range(2):
        s = 0.7 * float(q[h] @ k)
        np.testing.assert_allclose(got[0, h], v / (1.0 + math.exp(sinks[h] - s)), rtol=0, atol=1e-14)


def test_window_one_gives_own_value_row(oracle_mod):
    case = workloads.make_case("sw-w1", 733, [4], [70], 2, 1, 8, causal=True)
    got = _run(oracle_mod, case, window=1)
    P = case.kv.shape[1]
    for i in range(4):
        pos = 70 - 4 + i
        v = _f64(case.kv[int(case.block_table[0, pos // P]), pos % P, 0, 1])
        assert np.array_equal(got[i, 0], v) and np.array_equal(got[i, 1], v)


def test_window_equals_cut_sequence(oracle_mod):
    """Decode with W = 128 equals the same query over only the last 128 keys:
    L = 320 (keys 192..319) and L = 256 (keys 128..255), cut at page borders,
    so the cut sequence is the block table shifted by 3 and 2 pages."""
    case = workloads.make_case("sw-c", 734, [1, 1], [320, 256], 8, 2, 16, causal=True)
    got = _run(oracle_mod, case, window=128)
    bt = case.block_table.clone()
    bt[0, :2] = case.block_table[0, 3:5]      # keys 192..319 -> positions 0..127
    bt[1, :2] = case.block_table[1, 2:4]      # keys 128..255 -> positions 0..127
    got_cut = oracle_mod.paged_attn(case.q, case.kv, bt, torch.tensor([128, 128], dtype=torch.int32),
                                    case.cu_q, case.scale, True)
    assert np.array_equal(got, got_cut)
