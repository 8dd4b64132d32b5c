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


# ------------------------------------------------ the write fused into the split-decode launch
def _launches(fn):
    """(result, attention launches, write launches) of fn() from the library's
    per-launch timing (a fused call launches no separate write kernel)."""
    import paged_kv_gqa_fwd_amd as pa
    torch.cuda.synchronize()
    pa.kernel_timing_read()
    pa.kernel_timing_enable(True)
    res = fn()
    torch.cuda.synchronize()
    pa.kernel_timing_enable(False)
    _, main_n, _, _, _, _, _, write_n = pa.kernel_timing_read()
    return res, main_n, write_n


FUSED = [
    # name, q_lens, kv_lens, hq, hkv, d, path, pps, window, new-row layout
    ("decode D128 balanced", [1] * 12, None, 32, 8, 128, 0, 0, 0, "separate"),
    ("decode D256 fixed splits", [1] * 6, None, 16, 2, 256, 1, 3, 0, "separate"),
    ("decode D128 single-launch merge", [1] * 9, None, 24, 4, 128, 3, 2, 0, "fused_qkv"),
    ("short runs D128 n<=8, L=0/1/63/65", [8, 3, 1, 8, 5, 2], [0, 1, 63, 65, 700, 130], 16, 4, 128, 0, 0, 0,
     "separate"),
    ("short runs D256 n<=4, page-crossing", [4, 4, 2, 3], [66, 129, 64, 1000], 24, 4, 256, 4, 1, 0, "fused_qkv"),
    ("decode D128 window 100", [1] * 7, None, 32, 8, 128, 0, 0, 100, "separate"),
]


@pytest.mark.parametrize("idx", range(len(FUSED)), ids=[f[0] for f in FUSED])
def test_fused_write_then_attend(oracle_mod, idx):
    """The split paths take the new K/V rows inside the attention launch: the
    whole pool bit-exact against ORACLE-W (poisoned slots and unused pages
    included) and the attention within the bf16 bar of ORACLE-P over the
    written pool, with one launch and no separate write kernel."""
    import dataclasses
    import paged_kv_gqa_fwd_amd as pa
    name, q_lens, kv_lens, hq, hkv, d, path, pps, window, layout = FUSED[idx]
    if kv_lens is None:
        g = torch.Generator().manual_seed(810 + idx)
        kv_lens = torch.randint(1, 1500, (len(q_lens),), generator=g).tolist()
    case = workloads.make_case("fw-%d" % idx, 810 + idx, q_lens, kv_lens, hq, hkv, d, causal=True,
                               extra_pages=2, poison=True, table_cols=max(kv_lens) // 64 + 2)
    k_new, v_new = workloads.new_kv_tokens(case, 910 + idx, layout=layout)
    written = oracle_mod.kv_write(case.kv, k_new.cpu(), v_new.cpu(), case.block_table, case.seq_lens, case.cu_q)
    c_ref = dataclasses.replace(case, kv=written)
    ref = oracle_mod.paged_attn(c_ref.q, c_ref.kv, c_ref.block_table, c_ref.seq_lens, c_ref.cu_q, c_ref.scale,
                                True, window=window)
    g = case.to("cuda")
    log("  gpu fused write + attend: %s" % name)
    out, n_main, n_write = _launches(lambda: pa.paged_attention_write(
        g.q, k_new.cuda(), v_new.cuda(), g.kv, g.block_table, g.seq_lens, g.cu_q, max(case.max_q, 1), case.scale,
        True, path=path, pages_per_split=pps, window=window))
    assert (n_main, n_write) == (1, 0), "expected one fused launch, got %d attention + %d write" % (n_main, n_write)
    assert torch.equal(_bits(g.pool_storage), _bits(_written_storage(case, written)))
    compare(out, ref, what="fused write + attend: %s" % name)


def _written_storage(case, written_view):
    """The pool allocation with the oracle's written view copied in (the view
    may not cover the whole allocation)."""
    st = case.pool_storage.clone()
    st.as_strided(case.kv.shape, case.kv.stride(),
                  case.kv.storage_offset() - case.pool_storage.storage_offset()).copy_(written_view)
    return st


def test_fused_write_fp8_cache(oracle_mod):
    """Over an fp8 cache the fused write stores the e4m3 codes of x / scale
    (bit-exact against ORACLE-W) and attends to their decoded values."""
    import dataclasses
    import paged_kv_gqa_fwd_amd as pa
    case = workloads.fp8_pool_case(workloads.make_case("fw-f8", 830, [1] * 10 + [6],
                                                       [900, 1, 63, 64, 65, 300, 2000, 129, 5, 77, 190], 32, 8,
                                                       128, causal=True, extra_pages=2, poison=True))
    k_new, v_new = workloads.new_kv_tokens(case, 930)
    written = oracle_mod.kv_write(case.kv, k_new.cpu(), v_new.cpu(), case.block_table, case.seq_lens, case.cu_q,
                                  k_scale=0.5, v_scale=0.25)
    ref = oracle_mod.paged_attn(case.q, written, case.block_table, case.seq_lens, case.cu_q, case.scale, True,
                                k_scale=0.5, v_scale=0.25)
    g = case.to("cuda")
    out, n_main, n_write = _launches(lambda: pa.paged_attention_write(
        g.q, k_new.cuda(), v_new.cuda(), g.kv, g.block_table, g.seq_lens, g.cu_q, max(case.max_q, 1), case.scale,
        True, k_scale=0.5, v_scale=0.25))
    assert (n_main, n_write) == (1, 0)
    assert torch.equal(g.pool_storage.cpu(), _written_storage(case, written))
    compare(out, ref, what="fused write + attend, fp8 cache")


def test_unfusable_write_takes_two_launches(oracle_mod):
    """Rows that need the prefill kernel keep the separate write kernel."""
    import paged_kv_gqa_fwd_amd as pa
    case = workloads.chunked_prefill(n_seqs=2, q_lo=100, q_hi=200, ctx_hi=300, seed=840)
    k_new, v_new = workloads.new_kv_tokens(case, 940)
    written = oracle_mod.kv_write(case.kv, k_new.cpu(), v_new.cpu(), case.block_table, case.seq_lens, case.cu_q)
    g = case.to("cuda")
    _, n_main, n_write = _launches(lambda: pa.paged_attention_write(
        g.q, k_new.cuda(), v_new.cuda(), g.kv, g.block_table, g.seq_lens, g.cu_q, max(case.max_q, 1), case.scale,
        True))
    assert (n_main, n_write) == (1, 1)
    assert torch.equal(g.pool_storage.cpu(), _written_storage(case, written))
