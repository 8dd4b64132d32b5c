"""GPU parity of the short-sequence body: the split-decode kernels with two
or four blocks of 16 packed rows (17 to 64 rows G x n per (sequence, KV
head)), the cheaper body that short query runs take instead of the prefill
tile (Mojo SM100MHA2Q docs, struct summary: short sequences are routed to a
cheaper body at runtime), through the C ABI.

Every case holds every written row to the bf16 bar (max-abs 2e-2, rel-RMS
5e-3) against the fp64 oracle, with NaN / inf poison in the slots past L
and in unused pages.  Mixed short batches cover G x n from 17 to 64 with
L = 0, 1, 63, 65 (n > L rows that see no key or only part of the chunk),
both head dims, every split path (automatic balanced, fixed splits, the
single-launch merge), windows, sinks and an fp8 cache; the same inputs
through the prefill path agree with the oracle too.
"""
import math
import random

import pytest
import torch

import workloads
from parity_util import compare, log

pytestmark = pytest.mark.gpu

PATH_AUTO, PATH_SPLIT, PATH_PREFILL, PATH_FUSED, PATH_BALANCED = 0, 1, 2, 3, 4


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_gqa_fwd_amd as pa
    pa.load_library()


def _mixed(seed, G, hkv, d, n_max, causal=True, extra=()):
    """A short mixed batch: every G x n from 17 to 64 that n_max allows,
    against L = 0, 1, 63, 65 and longer contexts (several pages, a page
    edge), plus n = 0 and n > L."""
    rng = random.Random(seed)
    ns = [n for n in range(1, n_max + 1) if 17 <= G * n <= 64] or [n_max]
    q_lens, kv_lens = [], []
    for i, L in enumerate([0, 1, 63, 65, 64, 129, 700, 2000] + list(extra)):
        n = ns[i % len(ns)]
        q_lens.append(n)
        kv_lens.append(L)
    q_lens += [0, max(ns)]          # an empty sequence, and one more long run
    kv_lens += [300, rng.randint(150, 1200)]
    return workloads.make_case("short-G%d-D%d" % (G, d), seed, q_lens, kv_lens, G * hkv, hkv, d, causal=causal,
                               table_cols=math.ceil(max(kv_lens) / 64) + 1, extra_pages=2, poison=True)


def _run(case, path=PATH_AUTO, pps=0, **kw):
    import paged_kv_gqa_fwd_amd as pa
    g = case.to("cuda")
    mq = max(case.max_q, 1)
    plan = pa.make_plan(pa.make_dims(g.q, g.kv, g.block_table), case.n_seqs, mq, path, pps, kw.get("window", 0),
                        1 if g.kv.dtype == torch.uint8 else 0)
    log("  gpu short-body call: %s B=%d max_q=%d G=%d D=%d path=%d->%d pps=%d %s" % (
        case.name, case.n_seqs, mq, case.num_q_heads // case.num_kv_heads, case.head_dim, path, plan.path, pps,
        {k: v for k, v in kw.items() if k != "sinks"}))
    res = pa.paged_attention(g.q, g.kv, g.block_table, g.seq_lens, g.cu_q, mq, case.scale, case.causal, path=path,
                             pages_per_split=pps, **kw)
    torch.cuda.synchronize()
    return res, plan.path


SHAPES = [(4, 2, 128, 16), (6, 4, 256, 10), (8, 2, 256, 8), (8, 1, 128, 8), (5, 3, 128, 12)]


@pytest.mark.parametrize("G,hkv,d,n_max", SHAPES, ids=["G%d-hkv%d-D%d" % s[:3] for s in SHAPES])
@pytest.mark.parametrize("path,pps", [(PATH_AUTO, 0), (PATH_SPLIT, 1), (PATH_SPLIT, 3), (PATH_FUSED, 2),
                                      (PATH_BALANCED, 1)])
def test_short_mixed_batches(oracle_mod, G, hkv, d, n_max, path, pps):
    case = _mixed(1300 + G * 10 + d, G, hkv, d, n_max)
    ref = oracle_mod.paged_attn(case.q, case.kv, case.block_table, case.seq_lens, case.cu_q, case.scale, True)
    out, taken = _run(case, path, pps)
    assert taken != PATH_PREFILL and G * case.max_q > 16
    compare(out, ref, what="%s path=%d pps=%d" % (case.name, path, pps))


@pytest.mark.parametrize("d", [128, 256])
def test_short_body_equals_prefill_within_bar(oracle_mod, d):
    """The same short batch through the prefill kernel: both within the bar
    of the oracle (and so of each other)."""
    case = _mixed(1400 + d, 8, 2, d, 8)
    ref = oracle_mod.paged_attn(case.q, case.kv, case.block_table, case.seq_lens, case.cu_q, case.scale, True)
    short, t1 = _run(case)
    pre, t2 = _run(case, PATH_PREFILL)
    assert t1 == PATH_BALANCED and t2 == PATH_PREFILL
    compare(short, ref, what="short body D=%d" % d)
    compare(pre, ref, what="prefill D=%d" % d)


@pytest.mark.parametrize("d", [128, 256])
def test_short_body_noncausal_window_sinks(oracle_mod, d):
    case = _mixed(1500 + d, 6, 2, d, 10, causal=False)
    g = torch.Generator().manual_seed(d)
    sinks = (torch.randn(case.num_q_heads, generator=g) * 2).float()
    sinks[1] = -math.inf
    for window, path in ((0, PATH_AUTO), (100, PATH_AUTO), (64, PATH_SPLIT), (1, PATH_BALANCED)):
        ref = oracle_mod.paged_attn(case.q, case.kv, case.block_table, case.seq_lens, case.cu_q, case.scale, False,
                                    sinks=sinks.double().numpy(), window=window)
        out, _ = _run(case, path, 0, window=window, sinks=sinks.cuda())
        compare(out, ref, what="non-causal D=%d window=%d path=%d with sinks" % (d, window, path))


@pytest.mark.parametrize("d", [128, 256])
def test_short_body_fp8_cache(oracle_mod, d):
    case = workloads.fp8_pool_case(_mixed(1600 + d, 8, 2, d, 8))
    ref = oracle_mod.paged_attn(case.q, case.kv, case.block_table, case.seq_lens, case.cu_q, case.scale, True,
                                k_scale=0.5, v_scale=0.5)
    for path, pps in ((PATH_AUTO, 0), (PATH_SPLIT, 2)):
        out, taken = _run(case, path, pps, k_scale=0.5, v_scale=0.5)
        assert taken != PATH_PREFILL
        compare(out, ref, what="fp8 cache D=%d path=%d" % (d, path))


def test_short_body_random_sweep(oracle_mod):
    """Seeded random short batches: G 1-8, n up to 64 / G, D 128 / 256,
    ragged L (0, 1, page edges, a few pages), causal or not, every split
    path."""
    rng = random.Random(1777)
    for it in range(40):
        d = rng.choice([128, 256])
        G = rng.choice([2, 3, 4, 6, 8])
        hkv = rng.choice([1, 2, 4])
        nmax = 64 // G
        B = rng.randint(1, 9)
        q_lens = [rng.randint(0, nmax) for _ in range(B)]
        q_lens[0] = max(q_lens[0], 17 // G + 1) if 17 // G + 1 <= nmax else nmax
        kv_lens = [rng.choice([0, 1, 63, 64, 65, rng.randint(1, 400), rng.randint(400, 1500)]) for _ in range(B)]
        if max(kv_lens) == 0:
            kv_lens[0] = 77
        causal = rng.random() < 0.75
        path = rng.choice([PATH_AUTO, PATH_SPLIT, PATH_FUSED, PATH_BALANCED])
        pps = 0 if path == PATH_AUTO else rng.choice([0, 1, 2, 5])
        case = workloads.make_case("short-rnd%d" % it, 1700 + it, q_lens, kv_lens, G * hkv, hkv, d, causal=causal,
                                   table_cols=math.ceil(max(kv_lens) / 64) + 1, poison=True)
        ref = oracle_mod.paged_attn(case.q, case.kv, case.block_table, case.seq_lens, case.cu_q, case.scale, causal)
        out, _ = _run(case, path, pps)
        compare(out, ref, what="random short %d (G=%d D=%d path=%d pps=%d)" % (it, G, d, path, pps))
