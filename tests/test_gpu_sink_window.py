"""GPU parity of attention sinks and the sliding window (attn_paged_fwd_opt)
against the fp64 oracle, on the split-decode path (both merge forms) and the
prefill path, through the C ABI.

Tolerance: the bf16 bar (max-abs 2e-2, rel-RMS 5e-3 over every written row).
"""
import math

import numpy as np
import pytest
import torch

import workloads
from parity_util import compare, log

pytestmark = pytest.mark.gpu

PATH_AUTO, PATH_SPLIT, PATH_PREFILL, PATH_FUSED = 0, 1, 2, 3
INT32_MAX = 2 ** 31 - 1


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_gqa_fwd_amd as pa
    pa.load_library()


def _sinks(hq, seed):
    g = torch.Generator().manual_seed(seed)
    s = torch.rand(hq, generator=g) * 6.0 - 2.0      # logits in [-2, 4)
    s[0] = -math.inf                                  # one head without a sink
    return s


def _oracle(oracle_mod, case, sinks, window, **kw):
    return oracle_mod.paged_attn(case.q, case.kv, case.block_table, case.seq_lens, case.cu_q, case.scale,
                                 case.causal, sinks=None if sinks is None else sinks.double().numpy(),
                                 window=window, **kw)


def _gpu(case, sinks, window, path=PATH_AUTO, pps=0):
    import paged_kv_gqa_fwd_amd as pa
    g = case if case.q.device.type == "cuda" else case.to("cuda")
    log("  gpu call: %s window=%d sinks=%s path=%d pps=%d" % (case.name, window, sinks is not None, path, pps))
    out = pa.paged_attention(g.q, g.kv, g.block_table, g.seq_lens, g.cu_q, max(case.max_q, 1), case.scale,
                             case.causal, path=path, pages_per_split=pps, window=window,
                             sinks=None if sinks is None else sinks.cuda())
    torch.cuda.synchronize()
    return out


DECODE = [  # (window, with sinks)
    (1000, True), (1000, False), (0, True), (64, True), (1, False),
]


@pytest.mark.parametrize("window,with_sinks", DECODE)
def test_decode(oracle_mod, window, with_sinks):
    case = workloads.decode_batch(n_seqs=12, seed=811)
    sinks = _sinks(32, 1) if with_sinks else None
    ref = _oracle(oracle_mod, case, sinks, window)
    outs = {}
    for path, pps in ((PATH_AUTO, 0), (PATH_SPLIT, 3), (PATH_FUSED, 3), (PATH_SPLIT, 1000)):
        outs[(path, pps)] = _gpu(case, sinks, window, path, pps).clone()
        compare(outs[(path, pps)], ref, what="decode W=%d sinks=%s path=%d pps=%d" % (window, with_sinks, path, pps))
    # the single-launch merge gives the two-kernel path's bits
    assert torch.equal(outs[(PATH_FUSED, 3)].view(torch.int16), outs[(PATH_SPLIT, 3)].view(torch.int16))


def test_long_decode_window_d256(oracle_mod):
    """4 x 16384 keys, 16/2 heads, D 256, window 5000 (split plan covers it)."""
    case = workloads.long_decode(n_seqs=4, ctx=16384, seed=812)
    sinks = _sinks(16, 2)
    compare(_gpu(case, sinks, 5000), _oracle(oracle_mod, case, sinks, 5000), what="long decode W=5000")


@pytest.mark.parametrize("window,with_sinks", [(300, True), (300, False), (0, True), (1, True), (64, False)])
def test_chunked_prefill(oracle_mod, window, with_sinks):
    """Chunks of 100..300 tokens on 0..700 cached keys, 24/4 heads, D 256:
    rows of one chunk have different window starts."""
    case = workloads.chunked_prefill(n_seqs=3, q_lo=100, q_hi=300, ctx_hi=700, seed=813)
    sinks = _sinks(24, 3) if with_sinks else None
    compare(_gpu(case, sinks, window), _oracle(oracle_mod, case, sinks, window),
            what="chunked prefill W=%d sinks=%s" % (window, with_sinks))


def test_prefill_d128_noncausal_window(oracle_mod):
    """Non-causal D 128, 1000 tokens, 8 heads: keys [pos - W + 1, L)."""
    case = workloads.dit_self_attn(n_tokens=1000, heads=8)
    sinks = _sinks(8, 4)
    compare(_gpu(case, sinks, 200), _oracle(oracle_mod, case, sinks, 200), what="non-causal W=200")


def test_rows_without_keys_and_with_sinks(oracle_mod):
    """n > L rows see no key (zeros with or without a sink); L = 0 sequences."""
    case = workloads.make_case("sw-e", 814, [10, 1, 3], [6, 0, 200], 8, 2, 128, causal=True, poison=True)
    sinks = _sinks(8, 5)
    for window in (0, 4):
        for path in (PATH_AUTO, PATH_PREFILL):
            out = _gpu(case, sinks, window, path)
            compare(out, _oracle(oracle_mod, case, sinks, window), what="edge W=%d path=%d" % (window, path))
            assert not out[:4].float().abs().sum().item()       # rows with pos < 0


def test_neutral_options_are_bitwise_neutral():
    case = workloads.decode_batch(n_seqs=6, seed=815).to("cuda")
    chunk = workloads.chunked_prefill(n_seqs=2, q_lo=100, q_hi=200, ctx_hi=300, seed=816).to("cuda")
    for c in (case, chunk):
        base = _gpu(c, None, 0).clone()
        neutral = _gpu(c, torch.full((c.num_q_heads,), -math.inf), INT32_MAX).clone()
        assert torch.equal(base.view(torch.int16), neutral.view(torch.int16)), c.name
