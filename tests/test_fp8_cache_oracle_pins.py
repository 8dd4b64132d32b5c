"""Pins for the oracle over an fp8 (OCP e4m3) KV cache (CPU only).

Reading: the pool holds e4m3 codes with one scale for K and one for V,
K = k_scale * e4m3(code), V = v_scale * e4m3(code).  The pins tie the fp8
oracle to the bf16 oracle and to torch's float8_e4m3fn decoding:

* with power-of-two scales every dequantised value is exactly a bf16 value,
  so the fp8 oracle must equal the bf16 oracle on a bf16 pool holding those
  values, bitwise;
* scaling: k_scale multiplies the scores (so k_scale = c with scale s equals
  k_scale = 1 with scale c s) and v_scale multiplies the output;
* brute force over torch-decoded codes (numpy dense attention).
"""
import numpy as np
import pytest
import torch

import workloads


def _decoded_bf16_case(case8, k_scale, v_scale):
    """bf16 pool holding k_scale / v_scale times torch's decoding of every code."""
    import dataclasses
    vals = case8.pool_storage.view(torch.float8_e4m3fn).float()
    kv = case8.kv
    st = dataclasses.replace(case8, pool_storage=vals.to(torch.bfloat16))
    view = st.pool_storage.as_strided(kv.shape, kv.stride(), kv.storage_offset() - case8.pool_storage.storage_offset())
    view[:, :, :, 0] *= k_scale
    view[:, :, :, 1] *= v_scale
    return dataclasses.replace(st, kv=view)


def _run(oracle_mod, case, **kw):
    return oracle_mod.paged_attn(case.q, case.kv, case.block_table, case.seq_lens, case.cu_q, case.scale,
                                 case.causal, **kw)


@pytest.mark.parametrize("ks,vs", [(1.0, 1.0), (0.5, 0.25), (0.125, 2.0)])
def test_equals_bf16_oracle_on_exact_values(oracle_mod, ks, vs):
    base = workloads.make_case("f8", 740, [1, 3, 20], [65, 300, 128], 8, 2, 64, causal=True, scale=0.3)
    case8 = workloads.fp8_pool_case(base)
    got = _run(oracle_mod, case8, k_scale=ks, v_scale=vs)
    ref = _run(oracle_mod, _decoded_bf16_case(case8, ks, vs))
    assert np.array_equal(got, ref)


def test_k_scale_is_a_score_scale_and_v_scale_an_output_scale(oracle_mod):
    import dataclasses
    case8 = workloads.fp8_pool_case(workloads.make_case("f8s", 741, [1, 5], [100, 70], 4, 1, 32, causal=True,
                                                        scale=0.2))
    a = _run(oracle_mod, case8, k_scale=0.37, v_scale=1.0)
    b = _run(oracle_mod, dataclasses.replace(case8, scale=0.2 * 0.37), k_scale=1.0, v_scale=1.0)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-13)
    c = _run(oracle_mod, case8, k_scale=0.37, v_scale=3.0)
    np.testing.assert_allclose(c, 3.0 * a, rtol=1e-13, atol=1e-13)


def test_brute_force_over_torch_decoding(oracle_mod):
    case8 = workloads.fp8_pool_case(workloads.make_case("f8b", 742, [1, 4], [70, 9], 4, 2, 16, causal=True,
                                                        scale=0.25))
    ks, vs = 0.3, 0.7
    got = _run(oracle_mod, case8, k_scale=ks, v_scale=vs)
    kvf = case8.kv.view(torch.float8_e4m3fn).double()       # torch's decoding of the codes
    q = case8.q.double()
    P = case8.kv.shape[1]
    t0 = 0
    for b, (n, L) in enumerate(zip(case8.q_lens, case8.kv_lens)):
        idx = [(int(case8.block_table[b, j // P]), j % P) for j in range(L)]
        K = torch.stack([kvf[p, s, :, 0] for p, s in idx]) * ks       # [L, Hkv, D]
        V = torch.stack([kvf[p, s, :, 1] for p, s in idx]) * vs
        for i in range(n):
            vis = L - n + i + 1
            for h in range(4):
                s = 0.25 * (K[:vis, h // 2] @ q[t0 + i, h])
                w = torch.softmax(s, dim=0)
                np.testing.assert_allclose(got[t0 + i, h], (w @ V[:vis, h // 2]).numpy(), rtol=0, atol=1e-12)
        t0 += n


def test_quantize_matches_torch_e4m3(oracle_mod):
    """e4m3_quantize(x, s) equals torch's float8_e4m3fn conversion of the f32
    product x * (1/s) wherever that product is inside [-448, 448] (torch has no
    saturation; the oracle saturates, pinned by the encoder's own pins)."""
    g = torch.Generator().manual_seed(5)
    x = (torch.randn(4096, generator=g) * 3).to(torch.bfloat16)
    for s in (1.0, 0.25, 0.037, 3.0):
        got = oracle_mod.e4m3_quantize(x, s)
        y = x.float() * (torch.tensor(1.0, dtype=torch.float32) / torch.tensor(s, dtype=torch.float32))
        inside = y.abs() <= 448
        ref = y.to(torch.float8_e4m3fn).view(torch.uint8)
        assert torch.equal(got[inside], ref[inside]), s


def test_fp8_write_then_attend_is_quantised_attention(oracle_mod):
    """The fp8 write stores the quantised new rows: attention over the written
    fp8 cache equals attention over a bf16 cache that holds the dequantised
    rows (power-of-two scales keep every dequantised value a bf16 value)."""
    import dataclasses
    base = workloads.make_case("f8w", 743, [1, 3], [70, 129], 8, 2, 32, causal=True, scale=0.3)
    case8 = workloads.fp8_pool_case(base)
    k_new, v_new = workloads.new_kv_tokens(base, 44)
    ks, vs = 0.5, 0.25
    w8 = oracle_mod.kv_write(case8.kv, k_new, v_new, case8.block_table, case8.seq_lens, case8.cu_q,
                             k_scale=ks, v_scale=vs)
    got = oracle_mod.paged_attn(case8.q, w8, case8.block_table, case8.seq_lens, case8.cu_q, case8.scale, True,
                                k_scale=ks, v_scale=vs)
    kq = oracle_mod.e4m3_quantize(k_new, ks).view(torch.float8_e4m3fn).float() * ks
    vq = oracle_mod.e4m3_quantize(v_new, vs).view(torch.float8_e4m3fn).float() * vs
    cb = _decoded_bf16_case(case8, ks, vs)
    wb = oracle_mod.kv_write(cb.kv, kq.to(torch.bfloat16), vq.to(torch.bfloat16), cb.block_table, cb.seq_lens,
                             cb.cu_q)
    ref = oracle_mod.paged_attn(cb.q, wb, cb.block_table, cb.seq_lens, cb.cu_q, cb.scale, True)
    assert np.array_equal(got, ref)
