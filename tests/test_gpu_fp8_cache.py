"""GPU parity of attention over an fp8 (OCP e4m3) paged KV cache against the
fp64 oracle (same codes, same per-tensor scales), through the C ABI: the
split-decode paths and the prefill path (through its bf16 staging pool).

Tolerance: the bf16 bar (max-abs 2e-2, rel-RMS 5e-3).  The dequantisation
is exact (every e4m3 value is a bf16 value; the scales enter the scores and
the output in f32), so the error budget is the bf16 path's.
"""
import math

import pytest
import torch

import workloads
from parity_util import compare, log

pytestmark = pytest.mark.gpu

PATH_AUTO, PATH_SPLIT, PATH_PREFILL, PATH_FUSED = 0, 1, 2, 3


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_gqa_fwd_amd as pa
    pa.load_library()


def _check(oracle_mod, case8, ks, vs, what, path=PATH_AUTO, pps=0, window=0, sinks=None):
    import paged_kv_gqa_fwd_amd as pa
    ref = oracle_mod.paged_attn(case8.q, case8.kv, case8.block_table, case8.seq_lens, case8.cu_q, case8.scale,
                                case8.causal, k_scale=ks, v_scale=vs, window=window,
                                sinks=None if sinks is None else sinks.double().numpy())
    g = case8.to("cuda")
    log("  gpu fp8 call: %s path=%d pps=%d W=%d" % (what, path, pps, window))
    out = pa.paged_attention(g.q, g.kv, g.block_table, g.seq_lens, g.cu_q, max(case8.max_q, 1), case8.scale,
                             case8.causal, path=path, pages_per_split=pps, window=window, k_scale=ks, v_scale=vs,
                             sinks=None if sinks is None else sinks.cuda())
    torch.cuda.synchronize()
    compare(out, ref, what=what)
    return out


@pytest.mark.parametrize("path,pps", [(PATH_AUTO, 0), (PATH_SPLIT, 1), (PATH_SPLIT, 1000), (PATH_FUSED, 3)])
def test_decode_batch_fp8(oracle_mod, path, pps):
    case8 = workloads.fp8_pool_case(workloads.decode_batch(n_seqs=12, seed=821))
    _check(oracle_mod, case8, 0.5, 0.5, "decode fp8 path=%d pps=%d" % (path, pps), path, pps)


def test_long_decode_fp8_d256(oracle_mod):
    case8 = workloads.fp8_pool_case(workloads.long_decode(n_seqs=4, ctx=8192, seed=822), mult=8.0)
    _check(oracle_mod, case8, 0.125, 0.125, "long decode fp8 D256")


def test_tiny_mixed_rows_fp8(oracle_mod):
    """Several query rows per sequence (6 heads x 2 tokens = 12 packed rows), the
    two-layer pool, poisoned tails, another K scale (V kept at unit size, the
    scale the absolute tolerance is stated for)."""
    base = workloads.make_case("f8-multi", 823, [2, 1, 2], [130, 64, 1], 24, 4, 256, causal=True, poison=True,
                               layers=2, layer=1)
    case8 = workloads.fp8_pool_case(base)
    _check(oracle_mod, case8, 0.3, 0.5, "fp8 multi-row")


def test_fp8_with_window_and_sinks(oracle_mod):
    case8 = workloads.fp8_pool_case(workloads.decode_batch(n_seqs=6, seed=824))
    sinks = torch.linspace(-1.0, 3.0, 32)
    sinks[0] = -math.inf
    _check(oracle_mod, case8, 0.5, 0.5, "fp8 W=700 sinks", window=700, sinks=sinks)


def test_fp8_equals_bf16_on_exact_values():
    """With power-of-two scales the dequantised cache is exactly a bf16 cache:
    the fp8 kernel must give the bf16 kernel's bits."""
    import dataclasses
    import paged_kv_gqa_fwd_amd as pa
    case8 = workloads.fp8_pool_case(workloads.decode_batch(n_seqs=8, seed=825)).to("cuda")
    vals = case8.pool_storage.view(torch.float8_e4m3fn).to(torch.bfloat16)
    kvb = vals.as_strided(case8.kv.shape, case8.kv.stride(), case8.kv.storage_offset())
    kvb[:, :, :, 0] *= 0.5
    kvb[:, :, :, 1] *= 0.25
    caseb = dataclasses.replace(case8, pool_storage=vals, kv=kvb)
    a = pa.paged_attention(case8.q, case8.kv, case8.block_table, case8.seq_lens, case8.cu_q, 1, case8.scale, True,
                           k_scale=0.5, v_scale=0.25)
    b = pa.paged_attention(caseb.q, caseb.kv, caseb.block_table, caseb.seq_lens, caseb.cu_q, 1, caseb.scale, True)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_every_code_decodes_exactly():
    """Each sequence has one key, so out = its V row: the 254 non-NaN codes
    (NaN codes replaced by 0) must come out as torch's e4m3 decoding, exactly
    (as values: the code of -0 comes out as +0, the sum P.V starting at +0)."""
    import paged_kv_gqa_fwd_amd as pa
    case = workloads.make_case("f8-codes", 827, [1, 1], [1, 1], 2, 2, 128, causal=True)
    case8 = workloads.fp8_pool_case(case)
    codes = torch.arange(256, dtype=torch.int32)
    codes[(codes & 0x7F) == 0x7F] = 0
    for b in range(2):
        pg = int(case8.block_table[b, 0])
        for g in range(2):
            case8.kv[pg, 0, g, 1] = codes[128 * b:128 * b + 128].to(torch.uint8)
    g8 = case8.to("cuda")
    out = pa.paged_attention(g8.q, g8.kv, g8.block_table, g8.seq_lens, g8.cu_q, 1, case8.scale, True,
                             k_scale=1.0, v_scale=1.0)
    torch.cuda.synchronize()
    expect = codes.to(torch.uint8).view(torch.float8_e4m3fn).to(torch.bfloat16).view(2, 128)
    for b in range(2):
        for h in range(2):
            assert torch.equal(out[b, h].cpu().float(), expect[b].float()), (b, h)


# ---------------------------------------------- prefill over an fp8 cache
# The prefill kernel reads an fp8 cache through a bf16 staging pool: the
# pages it reads are decoded (exactly) into the workspace first, k_scale joins
# the score scale and v_scale the output.

@pytest.mark.parametrize("d", [128, 256])
def test_fp8_prefill_chunks(oracle_mod, d):
    """Chunked-prefill shapes (prior context + new tokens, causal, poisoned
    slots) at both head dims, against the oracle on the same codes."""
    case = workloads.make_case("f8-pf-%d" % d, 826 + d, [150, 37, 300], [700, 40, 300], 24 if d == 256 else 32,
                               4 if d == 256 else 8, d, causal=True, extra_pages=2, poison=True)
    _check(oracle_mod, workloads.fp8_pool_case(case), 0.5, 0.5, "fp8 prefill D=%d" % d)


def test_fp8_prefill_noncausal_window_sinks(oracle_mod):
    case = workloads.make_case("f8-pf-w", 828, [90, 200], [333, 200], 12, 3, 128, causal=False, extra_pages=1,
                               poison=True)
    g = torch.Generator().manual_seed(4)
    sinks = (torch.randn(12, generator=g) * 2).float()
    sinks[2] = -math.inf
    case8 = workloads.fp8_pool_case(case, mult=4.0)
    _check(oracle_mod, case8, 0.25, 0.5, "fp8 prefill non-causal", path=PATH_PREFILL)
    _check(oracle_mod, case8, 0.25, 0.5, "fp8 prefill window 77 + sinks", path=PATH_PREFILL, window=77, sinks=sinks)
    _check(oracle_mod, case8, -0.25, 0.5, "fp8 prefill negative k_scale", path=PATH_PREFILL)


def test_fp8_prefill_manifest_pool(oracle_mod):
    """The manifest's two-layer pool (layer 1), 32-token chunks at G 6: the
    automatic plan takes the prefill kernel through the staging pool."""
    _check(oracle_mod, workloads.fp8_pool_case(workloads.tiny_mixed(seed=829)), 0.5, 1.0, "fp8 tiny mixed")


def test_fp8_prefill_equals_bf16_prefill_bitwise():
    """With unit scales the staged pages are exactly the bf16 pool of the
    decoded codes, so the prefill output must be the bf16 prefill's bits."""
    import dataclasses
    import paged_kv_gqa_fwd_amd as pa
    case8 = workloads.fp8_pool_case(workloads.chunked_prefill(n_seqs=3, q_lo=100, q_hi=260, ctx_hi=500,
                                                              seed=830)).to("cuda")
    vals = case8.pool_storage.view(torch.float8_e4m3fn).to(torch.bfloat16)
    kvb = vals.as_strided(case8.kv.shape, case8.kv.stride(), case8.kv.storage_offset())
    caseb = dataclasses.replace(case8, pool_storage=vals, kv=kvb)
    a = pa.paged_attention(case8.q, case8.kv, case8.block_table, case8.seq_lens, case8.cu_q, case8.max_q,
                           case8.scale, True, k_scale=1.0, v_scale=1.0)
    b = pa.paged_attention(caseb.q, caseb.kv, caseb.block_table, caseb.seq_lens, caseb.cu_q, caseb.max_q,
                           caseb.scale, True)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("big", [False, True])
def test_fp8_write_bit_exact(oracle_mod, big):
    """The quantising write gives the oracle's codes bit for bit (the product
    x * (1/scale) in f32 on both sides; with large rows the codes saturate)."""
    import paged_kv_gqa_fwd_amd as pa
    base = workloads.chunked_prefill(n_seqs=2, q_lo=40, q_hi=90, ctx_hi=300, seed=828)
    case8 = workloads.fp8_pool_case(base)
    k_new, v_new = workloads.new_kv_tokens(base, 48, layout="fused_qkv")
    if big:
        k_new = k_new * 300.0
    ks, vs = 0.37, 0.5
    expect = oracle_mod.kv_write(case8.kv, k_new, v_new, case8.block_table, case8.seq_lens, case8.cu_q,
                                 k_scale=ks, v_scale=vs)
    g8 = case8.to("cuda")
    pa.kv_write(g8.kv, k_new.cuda(), v_new.cuda(), g8.block_table, g8.seq_lens, g8.cu_q, case8.max_q, q_like=g8.q,
                k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    assert torch.equal(g8.kv.cpu(), expect)


def test_fp8_write_then_attend(oracle_mod):
    import paged_kv_gqa_fwd_amd as pa
    base = workloads.decode_batch(n_seqs=10, seed=829)
    case8 = workloads.fp8_pool_case(base)
    k_new, v_new = workloads.new_kv_tokens(base, 49)
    ks, vs = 0.5, 0.5
    written = oracle_mod.kv_write(case8.kv, k_new, v_new, case8.block_table, case8.seq_lens, case8.cu_q,
                                  k_scale=ks, v_scale=vs)
    ref = oracle_mod.paged_attn(case8.q, written, case8.block_table, case8.seq_lens, case8.cu_q, case8.scale, True,
                                k_scale=ks, v_scale=vs)
    g8 = case8.to("cuda")
    out = pa.paged_attention_write(g8.q, k_new.cuda(), v_new.cuda(), g8.kv, g8.block_table, g8.seq_lens, g8.cu_q, 1,
                                   case8.scale, True, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    assert torch.equal(g8.kv.cpu(), written)
    compare(out, ref, what="fp8 write + attend")
