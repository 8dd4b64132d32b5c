"""GPU tests of the KV-cache write (attn_paged_kv_write) and of the write
followed by attention in one call (attn_paged_fwd_write), through the C ABI.

* The written pool is bit-exact against the oracle's scatter (every byte of
  the pool, poisoned unused slots included: a byte move has one right answer).
* Attention after the write is within the bf16 tolerance of the oracle's
  attention over the oracle-written pool.
* A call that fails validation launches nothing (the pool is untouched).
"""
import pytest
import torch

import workloads
from parity_util import compare, log, oracle_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_gqa_fwd_amd as pa
    pa.load_library()


def _bits(t):
    return t.contiguous().view(torch.int16).cpu()


CASE_NAMES = ["decode 16 seqs, D 128", "chunks across pages, D 256", "two-layer pool, 32-token chunks",
              "n > L and L = 0", "fused QKV views, poisoned pool"]


def _case(idx):
    """(name, case, layout of the new K/V rows); built on demand (test collection stays fast)."""
    if idx == 0:
        c, layout = workloads.decode_batch(n_seqs=16, seed=801), "separate"
    elif idx == 1:
        c, layout = workloads.chunked_prefill(n_seqs=3, q_lo=100, q_hi=300, ctx_hi=700, seed=802), "separate"
    elif idx == 2:
        c, layout = workloads.tiny_mixed(seed=803), "separate"
    elif idx == 3:
        c, layout = workloads.make_case("w-edge", 804, [10, 3, 0, 1], [6, 0, 5, 1], 8, 2, 128,
                                        causal=True, poison=True), "separate"
    else:
        c, layout = workloads.make_case("w-fused", 805, [1, 40, 2], [70, 129, 64], 24, 4, 256,
                                        causal=True, poison=True), "fused_qkv"
    return CASE_NAMES[idx], c, layout


@pytest.mark.parametrize("idx", range(5), ids=CASE_NAMES)
def test_kv_write_bit_exact(oracle_mod, idx):
    import paged_kv_gqa_fwd_amd as pa
    name, case, layout = _case(idx)
    k_new, v_new = workloads.new_kv_tokens(case, 900 + idx, layout=layout)
    expect = oracle_mod.kv_write(case.kv, k_new.cpu(), v_new.cpu(), case.block_table, case.seq_lens, case.cu_q)
    g = case.to("cuda")
    log("  gpu kv write: %s T=%d Hkv=%d D=%d" % (name, case.q.shape[0], case.num_kv_heads, case.head_dim))
    pa.kv_write(g.kv, k_new.cuda(), v_new.cuda(), g.block_table, g.seq_lens, g.cu_q, max(case.max_q, 1),
                q_like=g.q)
    torch.cuda.synchronize()
    assert torch.equal(_bits(g.kv), _bits(expect)), "%s: pool differs from the oracle's write" % name


@pytest.mark.parametrize("idx", range(5), ids=CASE_NAMES)
def test_write_then_attend(oracle_mod, idx):
    import dataclasses
    import paged_kv_gqa_fwd_amd as pa
    name, case, layout = _case(idx)
    k_new, v_new = workloads.new_kv_tokens(case, 900 + idx, layout=layout)
    written = oracle_mod.kv_write(case.kv, k_new.cpu(), v_new.cpu(), case.block_table, case.seq_lens, case.cu_q)
    ref = oracle_for(oracle_mod, dataclasses.replace(case, kv=written))
    g = case.to("cuda")
    log("  gpu write + attend: %s" % name)
    out = pa.paged_attention_write(g.q, k_new.cuda(), v_new.cuda(), g.kv, g.block_table, g.seq_lens, g.cu_q,
                                   max(case.max_q, 1), case.scale, case.causal)
    torch.cuda.synchronize()
    assert torch.equal(_bits(g.kv), _bits(written))
    compare(out, ref, what="write + attend: %s" % name)


def test_two_layer_pool_other_layer_untouched():
    """The manifest's pool holds two layers; writing layer 1 leaves layer 0."""
    import paged_kv_gqa_fwd_amd as pa
    case = workloads.tiny_mixed(seed=806)
    k_new, v_new = workloads.new_kv_tokens(case, 906)
    before = case.pool_storage.clone()
    g = case.to("cuda")
    pa.kv_write(g.kv, k_new.cuda(), v_new.cuda(), g.block_table, g.seq_lens, g.cu_q, case.max_q, q_like=g.q)
    torch.cuda.synchronize()
    after = g.pool_storage.cpu()
    changed = (after.view(torch.int16) != before.view(torch.int16))
    # only bytes inside the written view's slots may change
    view_mask = torch.zeros_like(before, dtype=torch.bool)
    view_mask.as_strided(case.kv.shape, case.kv.stride(), case.kv.storage_offset()).fill_(True)
    assert not (changed & ~view_mask).any()


def test_failed_validation_writes_nothing():
    import paged_kv_gqa_fwd_amd as pa
    case = workloads.decode_batch(n_seqs=4, seed=807).to("cuda")
    k_new, v_new = workloads.new_kv_tokens(case, 907)
    before = case.kv.clone()
    with pytest.raises(pa.AttnError):
        pa.paged_attention_write(case.q, k_new, v_new, case.kv, case.block_table, case.seq_lens, case.cu_q, 1,
                                 float("nan"), True)
    torch.cuda.synchronize()
    assert torch.equal(_bits(case.kv), _bits(before))
