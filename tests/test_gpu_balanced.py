"""GPU parity of the balanced split-decode path (ATTN_PATH_SPLIT_BALANCED)
against the fp64 oracle, through the C ABI.

The path cuts the pages the whole batch needs into equal ranges, one
workgroup per (KV head, range); a range can end inside one sequence and go
on into the next.  These cases force short ranges over short, ragged
sequences so that ranges cross many sequence boundaries, hold several
pieces of one sequence, start mid-sequence and skip sequences with no page,
and check:

* every written row within the bf16 bar (max-abs 2e-2, rel-RMS 5e-3) of the
  oracle, with poisoned memory a correct kernel never reads;
* sinks, a window and an fp8 cache through the same path;
* rows of sequences with L = 0 come out as zeros, rows outside cu_q are
  untouched, and two runs give the same bits.
"""
import math

import numpy as np
import pytest
import torch

import workloads
from parity_util import compare, log, oracle_for

pytestmark = pytest.mark.gpu

PATH_BALANCED = 4


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_gqa_fwd_amd as pa
    pa.load_library()


def _ragged(seed, n_seqs, hq, hkv, d, max_q=1, lmax=700, window=0):
    """Short ragged sequences, including L = 0, L = 1, page edges, n = 0 and n > L."""
    g = torch.Generator().manual_seed(seed)
    special = [0, 1, 63, 64, 65, 128, 129]
    kv_lens, q_lens = [], []
    for i in range(n_seqs):
        L = special[i] if i < len(special) else int(torch.randint(0, lmax + 1, (1,), generator=g))
        n = int(torch.randint(0, max_q + 1, (1,), generator=g)) if max_q > 1 else (0 if i == 9 else 1)
        if i == 10:
            n, L = max_q, min(L, max_q - 1) if max_q > 1 else 0    # n > L (rows without keys)
        kv_lens.append(L)
        q_lens.append(n)
    return workloads.make_case("bal-%d" % seed, seed, q_lens, kv_lens, hq, hkv, d, causal=True,
                               table_cols=math.ceil(lmax / 64) + 1, poison=True)


def _gpu(case, pps, out=None, **kw):
    import paged_kv_gqa_fwd_amd as pa
    g = case if case.q.device.type == "cuda" else case.to("cuda")
    log("  gpu balanced call: %s B=%d max_q=%d Hq=%d Hkv=%d D=%d least range=%d %s" % (
        case.name, case.n_seqs, case.max_q, case.num_q_heads, case.num_kv_heads, case.head_dim, pps, kw))
    res = pa.paged_attention(g.q, g.kv, g.block_table, g.seq_lens, g.cu_q, max(case.max_q, 1), case.scale,
                             case.causal, out=out, path=PATH_BALANCED, pages_per_split=pps, **kw)
    torch.cuda.synchronize()
    return res


@pytest.mark.parametrize("pps", [0, 1, 2, 5, 13, 1000])
def test_ragged_decode_ranges_cross_sequences(oracle_mod, pps):
    case = _ragged(901, 40, 32, 8, 128)
    compare(_gpu(case, pps), oracle_for(oracle_mod, case), what="ragged decode, least range %d" % pps)


@pytest.mark.parametrize("pps", [1, 3, 7])
def test_multi_row_d256(oracle_mod, pps):
    """24/4 heads (G = 6), D 256, up to 2 query tokens per sequence (12 rows)."""
    case = _ragged(902, 30, 24, 4, 256, max_q=2)
    compare(_gpu(case, pps), oracle_for(oracle_mod, case), what="multi-row D256, least range %d" % pps)


def test_gqa8_four_tokens(oracle_mod):
    """64/8 heads (G = 8) with 2 query tokens: 16 rows, the MFMA tile's width."""
    case = _ragged(903, 20, 64, 8, 128, max_q=2)
    compare(_gpu(case, 3), oracle_for(oracle_mod, case), what="G8 x 2 tokens")


@pytest.mark.parametrize("window,pps", [(100, 2), (64, 1), (1, 3)])
def test_window_and_sinks(oracle_mod, window, pps):
    case = _ragged(904, 36, 32, 8, 128)
    sinks = torch.linspace(-2.0, 4.0, 32)
    sinks[3] = -math.inf
    ref = oracle_mod.paged_attn(case.q, case.kv, case.block_table, case.seq_lens, case.cu_q, case.scale,
                                case.causal, sinks=sinks.double().numpy(), window=window)
    compare(_gpu(case, pps, window=window, sinks=sinks.cuda()), ref,
            what="window %d + sinks, least range %d" % (window, pps))


@pytest.mark.parametrize("pps", [0, 2])
def test_fp8_cache(oracle_mod, pps):
    case8 = workloads.fp8_pool_case(_ragged(905, 40, 32, 8, 128))
    ref = oracle_mod.paged_attn(case8.q, case8.kv, case8.block_table, case8.seq_lens, case8.cu_q, case8.scale,
                                case8.causal, k_scale=0.5, v_scale=0.5)
    compare(_gpu(case8, pps, k_scale=0.5, v_scale=0.5), ref, what="fp8 cache, least range %d" % pps)


def test_empty_sequences_zero_and_rows_outside_untouched():
    import paged_kv_gqa_fwd_amd as pa
    case = workloads.make_case("bal-e", 906, [1, 1, 1, 1], [0, 200, 0, 70], 32, 8, 128, poison=True)
    g = case.to("cuda")
    T = case.q.shape[0]
    out = torch.full((T + 3, 32, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    _gpu(g, 1, out=out[:T])
    o = out.float().cpu()
    assert not o[0].abs().sum().item() and not o[2].abs().sum().item()   # L = 0: zeros
    assert torch.isfinite(o[:T]).all()
    assert (o[T:] == 7.0).all()                                          # rows past cu_q untouched


def test_max_sequences_and_determinism(oracle_mod):
    """1024 sequences (the path's limit) of 1..300 keys; two runs, same bits."""
    g = torch.Generator().manual_seed(907)
    lens = [int(x) for x in torch.randint(1, 301, (1024,), generator=g)]
    case = workloads.make_case("bal-1024", 907, [1] * 1024, lens, 8, 2, 128, table_cols=5)
    a = _gpu(case, 0).clone()
    b = _gpu(case, 0).clone()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    rows = list(range(0, 1024, 37))
    mask = np.zeros(case.q.shape[0], dtype=np.uint8)
    mask[rows] = 1
    compare(a, oracle_for(oracle_mod, case, row_mask=mask), rows=rows, what="1024 sequences (sampled rows)")


def test_decode_batch_auto_is_balanced(oracle_mod):
    """The automatic plan of the decode batch is this path; whole batch against the oracle."""
    import paged_kv_gqa_fwd_amd as pa
    case = workloads.decode_batch()
    g = case.to("cuda")
    out = torch.empty_like(g.q)
    plan = pa.make_plan(pa.make_dims(g.q, g.kv, g.block_table, out), case.n_seqs, 1)
    assert plan.path == PATH_BALANCED
    res = pa.paged_attention(g.q, g.kv, g.block_table, g.seq_lens, g.cu_q, 1, case.scale, True, out=out)
    torch.cuda.synchronize()
    compare(res, oracle_for(oracle_mod, case), what="decode batch, automatic (balanced) plan")
