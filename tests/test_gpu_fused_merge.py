"""GPU tests of the single-launch split path (the last split of each
(sequence, KV head) merges the partials, counted with an i32 per pair).

* Same bits as the two-kernel path (split kernel + combine kernel): both run
  one merge arithmetic in split order.
* Within the bf16 tolerance of the fp64 oracle.
* The merge counters are zero again after every call, so repeated calls,
  calls with other sizes and calls after the two-kernel path (whose
  partials reuse those bytes) stay correct.
"""
import pytest
import torch

import workloads
from parity_util import compare, log, oracle_for, run_gpu

pytestmark = pytest.mark.gpu

PATH_SPLIT, PATH_FUSED = 1, 3


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_gqa_fwd_amd as pa
    pa.load_library()


def _bits(t):
    return t.view(torch.int16).cpu()


def _cached_counters(case):
    """The counter bytes of the binding's cached workspace for this case (one
    per (device, stream); the tests run on the current stream)."""
    import paged_kv_gqa_fwd_amd as pa
    key = (str(torch.device("cuda", torch.cuda.current_device())), int(torch.cuda.current_stream().cuda_stream))
    ws = pa._ws_cache[key]
    return ws.buf


@pytest.mark.parametrize("pps", [1, 3, 16])
def test_fused_equals_two_kernel_bitwise(oracle_mod, pps):
    case = workloads.decode_batch(n_seqs=12, seed=601).to("cuda")
    two = run_gpu(case, path=PATH_SPLIT, pages_per_split=pps).clone()
    one = run_gpu(case, path=PATH_FUSED, pages_per_split=pps).clone()
    assert torch.equal(_bits(one), _bits(two)), "fused merge differs from the combine kernel (pps=%d)" % pps
    compare(one, oracle_for(oracle_mod, case), what="fused decode pps=%d" % pps)


def test_fused_long_decode_d256(oracle_mod):
    """D 256, G 8, 4 sequences at context 16384 with 1% outlier keys."""
    case = workloads.long_decode(device="cuda", n_seqs=4, ctx=16384, seed=602)
    two = run_gpu(case, path=PATH_SPLIT, pages_per_split=8).clone()
    one = run_gpu(case, path=PATH_FUSED, pages_per_split=8).clone()
    assert torch.equal(_bits(one), _bits(two))
    compare(one, oracle_for(oracle_mod, case), what="fused long decode")


def test_fused_counters_return_to_zero(oracle_mod):
    import paged_kv_gqa_fwd_amd as pa
    a = workloads.decode_batch(n_seqs=20, seed=603).to("cuda")
    b = workloads.decode_batch(n_seqs=5, seed=604).to("cuda")
    ref_a, ref_b = oracle_for(oracle_mod, a), oracle_for(oracle_mod, b)
    dims = pa.make_dims(a.q, a.kv, a.block_table, a.q)
    plan_a = pa.make_plan(dims, a.n_seqs, 1, PATH_FUSED, 2)
    assert plan_a.counter_bytes > 0
    for i in range(3):
        compare(run_gpu(a, path=PATH_FUSED, pages_per_split=2), ref_a, what="fused call %d" % i)
        buf = _cached_counters(a)
        assert not buf[:plan_a.counter_bytes].any(), "merge counters not zero after call %d" % i
    # a smaller batch, a different split size, then the two-kernel path
    # (whose partials overwrite the counter bytes), then fused again
    compare(run_gpu(b, path=PATH_FUSED, pages_per_split=5), ref_b, what="fused, other sizes")
    compare(run_gpu(a, path=PATH_SPLIT, pages_per_split=1), ref_a, what="two-kernel in between")
    compare(run_gpu(a, path=PATH_FUSED, pages_per_split=3), ref_a, what="fused after two-kernel")
    assert not _cached_counters(a)[:plan_a.counter_bytes].any()


def test_fused_caller_workspace_and_clear(oracle_mod):
    import paged_kv_gqa_fwd_amd as pa
    case = workloads.decode_batch(n_seqs=9, seed=605).to("cuda")
    dims = pa.make_dims(case.q, case.kv, case.block_table, case.q)
    plan = pa.make_plan(dims, case.n_seqs, 1, PATH_FUSED, 4)
    C = plan.counter_bytes
    ws = torch.full((plan.workspace_bytes + 512,), 0xAB, dtype=torch.uint8, device="cuda")
    log("  workspace_clear of %d bytes" % C)
    pa.workspace_clear(ws, C)
    torch.cuda.synchronize()
    assert not ws[:C].any() and bool((ws[C:] == 0xAB).all())
    out = pa.paged_attention(case.q, case.kv, case.block_table, case.seq_lens, case.cu_q, 1,
                             case.scale, case.causal, path=PATH_FUSED, pages_per_split=4, workspace=ws)
    torch.cuda.synchronize()
    compare(out, oracle_for(oracle_mod, case), what="fused, caller workspace")
    assert not ws[:C].any()


def test_fused_empty_and_short_sequences(oracle_mod):
    """Sequences with L = 0, L = 1 and a tail page, several splits each."""
    case = workloads.make_case("fused-edge", 606, [1, 1, 1, 1, 1], [0, 1, 65, 700, 129], 32, 8, 128,
                               causal=True).to("cuda")
    two = run_gpu(case, path=PATH_SPLIT, pages_per_split=1).clone()
    one = run_gpu(case, path=PATH_FUSED, pages_per_split=1).clone()
    assert torch.equal(_bits(one), _bits(two))
    compare(one, oracle_for(oracle_mod, case), what="fused edge lengths")
