"""GPU parity of the split-key prefill, through the C ABI.

A prefill grid too small to fill the GPU (at most 64 (tile, KV head,
sequence) items, the tiny mixed call among them) has each item's keys split
into runs of pages_per_split pages from row 0's window start -- the page
ranges and (O, m, l) partial layout of the split-decode path (decode.json
manifest, ops.decode.impl scratch: partial / stats) -- and the combine
kernel merges the partials; the prefill path with a forced pages_per_split
takes the same route at any size.  Every case holds every written row to
the bf16 bar (max-abs 2e-2, rel-RMS 5e-3) against the fp64 oracle, with NaN
/ inf poison in the slots past L and in unused pages: both head dims,
causal and unmasked (Mojo SM100MHA2Q docs, MaskType), windows and sinks, an
fp8 cache, rows that see no key of a split or none at all (n > L, L = 0),
splits of 1 to 5 pages and the automatic choice.
"""
import math

import pytest
import torch

import workloads
from parity_util import compare, log

pytestmark = pytest.mark.gpu

PATH_AUTO, PATH_PREFILL = 0, 2

# (D, G, Hkv, q_lens, kv_lens, causal)
SHAPES = [
    (256, 6, 4, [32, 32], [300, 700], True),           # the tiny mixed call's shape
    (128, 4, 2, [70, 9, 0], [391, 649, 300], True),    # odd pages, an empty query run
    (128, 8, 1, [40], [40], False),
    (256, 2, 2, [40, 7, 30], [40, 7, 900], True),      # n = L: early rows see few keys
    (256, 4, 1, [90, 5], [1000, 3], True),             # n > L
    (128, 2, 3, [20, 1], [0, 129], True),              # L = 0
]


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_gqa_fwd_amd as pa
    pa.load_library()


def _case(i, d, G, hkv, q_lens, kv_lens, causal):
    return workloads.make_case("pfsplit%d-D%d" % (i, d), 2500 + i, q_lens, kv_lens, G * hkv, hkv, d, causal=causal,
                               table_cols=max(max(kv_lens), 1) // 64 + 2, extra_pages=2, poison=True)


def _run(case, path, pps, **kw):
    import paged_kv_gqa_fwd_amd as pa
    g = case.to("cuda")
    mq = max(case.max_q, 1)
    plan = pa.make_plan(pa.make_dims(g.q, g.kv, g.block_table), case.n_seqs, mq, path, pps, kw.get("window", 0),
                        1 if g.kv.dtype == torch.uint8 else 0)
    log("  gpu split prefill: %s path=%d pps=%d -> splits=%d pages/split=%d grid=%d %s" % (
        case.name, path, pps, plan.max_splits, plan.pages_per_split, plan.grid_x * plan.grid_y * plan.grid_z,
        {k: v for k, v in kw.items() if k != "sinks"}))
    out = pa.paged_attention(g.q, g.kv, g.block_table, g.seq_lens, g.cu_q, mq, case.scale, case.causal, path=path,
                             pages_per_split=pps, **kw)
    torch.cuda.synchronize()
    return out, plan


@pytest.mark.parametrize("i", range(len(SHAPES)))
@pytest.mark.parametrize("pps", [1, 2, 3, 5])
def test_forced_splits(oracle_mod, i, pps):
    d, G, hkv, q_lens, kv_lens, causal = SHAPES[i]
    case = _case(i, d, G, hkv, q_lens, kv_lens, causal)
    ref = oracle_mod.paged_attn(case.q, case.kv, case.block_table, case.seq_lens, case.cu_q, case.scale, causal)
    out, plan = _run(case, PATH_PREFILL, pps)
    mp = case.block_table.shape[1]   # the table's columns bound the pages a split layout covers
    assert plan.path == PATH_PREFILL and plan.max_splits == -(-mp // pps)
    assert torch.isfinite(out.float()).all()
    compare(out, ref, what="%s pps=%d" % (case.name, pps))


def test_tiny_mixed_takes_splits(oracle_mod):
    """The tiny mixed call (16 items): the automatic plan splits its keys."""
    case = workloads.tiny_mixed()
    out, plan = _run(case, PATH_AUTO, 0)
    assert plan.path == PATH_PREFILL and plan.max_splits > 1
    ref = oracle_mod.paged_attn(case.q, case.kv, case.block_table, case.seq_lens, case.cu_q, case.scale, True)
    compare(out, ref, what="tiny mixed, automatic splits")


@pytest.mark.parametrize("d", [128, 256])
def test_splits_window_sinks_noncausal(oracle_mod, d):
    case = _case(10 + d, d, 4, 2, [50, 20], [800, 20], False)
    g = torch.Generator().manual_seed(d)
    sinks = (torch.randn(case.num_q_heads, generator=g) * 2).float()
    sinks[0] = -math.inf
    for window, pps in ((0, 2), (100, 1), (64, 3), (1, 2), (300, 0)):
        ref = oracle_mod.paged_attn(case.q, case.kv, case.block_table, case.seq_lens, case.cu_q, case.scale, False,
                                    sinks=sinks.double().numpy(), window=window)
        out, plan = _run(case, PATH_PREFILL if pps else PATH_AUTO, pps, window=window, sinks=sinks.cuda())
        compare(out, ref, what="D=%d window=%d pps=%d splits=%d with sinks" % (d, window, pps, plan.max_splits))


@pytest.mark.parametrize("d", [128, 256])
def test_splits_fp8_cache(oracle_mod, d):
    case = workloads.fp8_pool_case(_case(20 + d, d, 4, 2, [40, 33], [500, 900], True))
    ref = oracle_mod.paged_attn(case.q, case.kv, case.block_table, case.seq_lens, case.cu_q, case.scale, True,
                                k_scale=0.5, v_scale=0.5)
    for path, pps in ((PATH_AUTO, 0), (PATH_PREFILL, 2)):
        out, plan = _run(case, path, pps, k_scale=0.5, v_scale=0.5)
        assert plan.path == PATH_PREFILL and plan.max_splits > 1
        compare(out, ref, what="fp8 cache D=%d path=%d pps=%d" % (d, path, pps))
