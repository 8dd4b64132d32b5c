"""GPU checks of attn_paged_fwd_noalloc, the entry point that allocates
nothing (its split-KV partials live in the library's per-GPU scratch array).

Each call goes through the C ABI and is compared with attn_paged_fwd_opt (the
entry point it is a variant of) on the same inputs, to the bf16 path's bar
(max-abs 2e-2, relative RMS 5e-3; bitwise where both take the same plan),
and with the fp64 oracle.  Calls follow one another on the same GPU with
shrinking inputs, so each one starts from the scratch contents the previous
call left behind.
"""
import ctypes

import numpy as np
import pytest
import torch

import workloads
from parity_util import compare, log, oracle_for

pytestmark = pytest.mark.gpu

PATH_AUTO, PATH_SPLIT, PATH_FUSED = 0, 1, 3


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_gqa_fwd_amd as pa
    pa.load_library()


def _noalloc(case, out, path=PATH_AUTO, pps=0):
    """One attn_paged_fwd_noalloc call on the current stream."""
    import paged_kv_gqa_fwd_amd as pa
    lib = pa.load_library()
    dims = pa.make_dims(case.q, case.kv, case.block_table, out)
    opt = pa.attn_paged_options(None, 0, path, pps, pa.KV_BF16, 1.0, 1.0)
    st = torch.cuda.current_stream()
    log("  noalloc call: %s B=%d max_q=%d path=%d pps=%d" % (case.name, case.n_seqs, case.max_q, path, pps))
    rc = lib.attn_paged_fwd_noalloc(out.data_ptr(), case.q.data_ptr(), case.kv.data_ptr(),
                                    case.block_table.data_ptr(), case.seq_lens.data_ptr(), case.cu_q.data_ptr(),
                                    case.n_seqs, max(case.max_q, 1), case.scale, int(case.causal),
                                    ctypes.byref(dims), ctypes.byref(opt), ctypes.c_void_p(st.cuda_stream))
    assert rc == 0, "attn_paged_fwd_noalloc returned %d" % rc
    torch.cuda.synchronize()
    return out


def _with_workspace(case, path=PATH_AUTO, pps=0):
    import paged_kv_gqa_fwd_amd as pa
    out = pa.paged_attention(case.q, case.kv, case.block_table, case.seq_lens, case.cu_q, max(case.max_q, 1),
                             case.scale, case.causal, path=path, pages_per_split=pps)
    torch.cuda.synchronize()
    return out


def _check(case, path=PATH_AUTO, pps=0, bitwise=False, oracle_mod=None):
    ref_out = _with_workspace(case, path, pps)
    out = torch.full_like(case.q, float("nan"))
    _noalloc(case, out, path, pps)
    if bitwise:
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), "%s: not bitwise equal" % case.name
    compare(out, ref_out.float().cpu().double().numpy(), what="%s noalloc vs workspace entry" % case.name)
    if oracle_mod is not None:
        compare(out, oracle_for(oracle_mod, case.to("cpu")), what="%s noalloc vs oracle" % case.name)


def test_noalloc_two_calls_shrinking(oracle_mod):
    """The decode batch (balanced split path, partials in the scratch), then a
    smaller batch whose partials overwrite only the front of the scratch."""
    big = workloads.decode_batch(device="cuda")
    _check(big, oracle_mod=oracle_mod)
    small = workloads.decode_batch(device="cuda", n_seqs=5, seed=611, lo=64, hi=900, poison=True)
    _check(small, oracle_mod=oracle_mod)


def test_noalloc_same_plan_is_bitwise_equal(oracle_mod):
    """Forced fixed-size splits take the same plan on both entry points:
    bitwise-equal outputs, the second call smaller than the first."""
    a = workloads.long_decode(device="cuda", n_seqs=16, ctx=8192, seed=612)
    _check(a, path=PATH_SPLIT, pps=16, bitwise=True)
    b = workloads.long_decode(device="cuda", n_seqs=3, ctx=1000, seed=613, poison=True)
    _check(b, path=PATH_SPLIT, pps=2, bitwise=True, oracle_mod=oracle_mod)


def test_noalloc_single_launch_merge_counters_start_at_zero(oracle_mod):
    """The single-launch merge keeps its counters at the front of the
    scratch; a balanced call first fills those bytes with partials, so the
    entry point must clear them before the merge path runs (twice, the
    second call smaller)."""
    fill = workloads.decode_batch(device="cuda", n_seqs=32, seed=614)
    _noalloc(fill, torch.empty_like(fill.q))
    c1 = workloads.decode_batch(device="cuda", n_seqs=12, seed=615)
    _check(c1, path=PATH_FUSED, pps=3, bitwise=True, oracle_mod=oracle_mod)
    c2 = workloads.decode_batch(device="cuda", n_seqs=4, seed=616, lo=100, hi=700)
    _check(c2, path=PATH_FUSED, pps=1, bitwise=True, oracle_mod=oracle_mod)


def test_noalloc_prefill(oracle_mod):
    """Prefill-shaped calls in the scratch (over the partials an earlier call
    left there): a ragged batch of 512 or more workgroups keeps its
    launch-order table there, a grid of at most 128 items its split-key
    partials.  Same plan on both entry points: bitwise equal."""
    import paged_kv_gqa_fwd_amd as pa
    fill = workloads.decode_batch(device="cuda", n_seqs=32, seed=620)
    _noalloc(fill, torch.empty_like(fill.q))
    big = workloads.chunked_prefill(device="cuda", n_seqs=4, q_lo=900, q_hi=1500, ctx_hi=1500, seed=619)
    small = workloads.chunked_prefill(device="cuda", n_seqs=2, q_lo=100, q_hi=300, ctx_hi=500, seed=617)
    for case, split in ((big, False), (small, True)):
        plan = pa.make_plan(pa.make_dims(case.q, case.kv, case.block_table), case.n_seqs, case.max_q)
        assert plan.workspace_bytes > 0 and (plan.max_splits > 1) == split
        _check(case, bitwise=True, oracle_mod=oracle_mod if split else None)


def test_noalloc_rejects_plans_past_the_scratch():
    """Partials larger than the scratch array: ATTN_ERR_WORKSPACE, nothing
    launched, out untouched."""
    import paged_kv_gqa_fwd_amd as pa
    case = workloads.decode_batch(device="cuda", n_seqs=200, seed=618, lo=64, hi=8192)
    out = torch.full_like(case.q, 3.0)
    lib = pa.load_library()
    dims = pa.make_dims(case.q, case.kv, case.block_table, out)
    opt = pa.attn_paged_options(None, 0, PATH_SPLIT, 1, pa.KV_BF16, 1.0, 1.0)
    rc = lib.attn_paged_fwd_noalloc(out.data_ptr(), case.q.data_ptr(), case.kv.data_ptr(),
                                    case.block_table.data_ptr(), case.seq_lens.data_ptr(), case.cu_q.data_ptr(),
                                    case.n_seqs, 1, case.scale, 1, ctypes.byref(dims), ctypes.byref(opt),
                                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert rc == -6
    assert torch.all(out == 3.0)
