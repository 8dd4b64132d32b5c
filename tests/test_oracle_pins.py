"""Pins for the fp64 paged-attention oracle (CPU only).

Each test ties the oracle to something other than itself: a brute-force
dense computation, torch's scaled_dot_product_attention in float64, closed
forms, invariants of the mathematics, and the paged layout printed in the
decode.json manifest (kern-kernels examples).  A plausible mistake in the
oracle -- a dropped scale, a wrong sign, a wrong KV-head index, top-left
instead of bottom-right causal alignment, a mis-strided page -- fails at
least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16_np(t):
    return t.float().double().numpy()


def _dense_kv(case):
    """Per sequence, K and V as dense fp64 [L, Hkv, D] arrays gathered through the table."""
    kv = case.kv
    P = kv.shape[1]
    res = []
    for b, L in enumerate(case.kv_lens):
        ks, vs = [], []
        for j in range(L):
            pg = int(case.block_table[b, j // P])
            ks.append(_bf16_np(kv[pg, j % P, :, 0, :]))
            vs.append(_bf16_np(kv[pg, j % P, :, 1, :]))
        res.append((np.array(ks).reshape(L, kv.shape[2], -1), np.array(vs).reshape(L, kv.shape[2], -1)))
    return res


def brute_force(case):
    """Explicit score matrix, explicit mask, np.exp softmax (no online update)."""
    q = _bf16_np(case.q)
    T, hq, d = q.shape
    hkv = case.kv.shape[2]
    G = hq // hkv
    out = np.zeros((T, hq, d))
    dense = _dense_kv(case)
    t0 = 0
    for b, (n, L) in enumerate(zip(case.q_lens, case.kv_lens)):
        K, V = dense[b]
        for h in range(hq):
            g = h // G
            S = case.scale * (q[t0:t0 + n, h, :] @ K[:, g, :].T)     # [n, L]
            pos = L - n + np.arange(n)[:, None]
            key = np.arange(L)[None, :]
            mask = (key <= pos) if case.causal else np.ones((n, L), bool)
            S = np.where(mask, S, -np.inf)
            for i in range(n):
                if not mask[i].any():
                    continue
                w = np.exp(S[i] - S[i].max())
                out[t0 + i, h] = (w / w.sum()) @ V[:, g, :]
        t0 += n
    return out


def run_oracle(oracle_mod, case, **kw):
    return oracle_mod.paged_attn(case.q, case.kv, case.block_table, case.seq_lens, case.cu_q,
                                 case.scale, case.causal, **kw)


SMALL_CASES = [
    dict(q_lens=[1, 1, 1], kv_lens=[1, 63, 200], hq=8, hkv=2, d=8, causal=True),
    dict(q_lens=[5, 17, 64], kv_lens=[5, 80, 129], hq=6, hkv=1, d=16, causal=True),
    dict(q_lens=[3, 40], kv_lens=[65, 128], hq=4, hkv=4, d=128, causal=True),
    dict(q_lens=[7, 2], kv_lens=[70, 9], hq=12, hkv=3, d=32, causal=False),
    dict(q_lens=[10, 4], kv_lens=[6, 64], hq=4, hkv=2, d=8, causal=True),   # n > L: 4 rows see nothing
]


@pytest.mark.parametrize("idx", range(len(SMALL_CASES)))
def test_oracle_matches_brute_force(oracle_mod, idx):
    c = SMALL_CASES[idx]
    case = workloads.make_case("bf", 1000 + idx, c["q_lens"], c["kv_lens"], c["hq"], c["hkv"], c["d"],
                               causal=c["causal"], page_size=64, extra_pages=2)
    got = run_oracle(oracle_mod, case)
    exp = brute_force(case)
    np.testing.assert_allclose(got, exp, rtol=0, atol=1e-12)


def test_oracle_matches_torch_sdpa_f64(oracle_mod):
    """Library routine: float64 SDPA with K/V repeated G times and an explicit
    bottom-right boolean mask, over an identity block table."""
    n, L, hq, hkv, d = 24, 150, 12, 3, 64
    case = workloads.make_case("sdpa", 77, [n], [L], hq, hkv, d, causal=True, scale=0.21)
    # identity table: relocate pages to be in order
    P = 64
    npg = math.ceil(L / P)
    kv_ident = torch.stack([case.kv[int(case.block_table[0, i])] for i in range(npg)])
    bt = torch.arange(npg, dtype=torch.int32).view(1, -1)
    got = oracle_mod.paged_attn(case.q, kv_ident, bt, case.seq_lens, case.cu_q, case.scale, True)
    K = kv_ident[:, :, :, 0, :].reshape(-1, hkv, d)[:L].double()   # [L, Hkv, D]
    V = kv_ident[:, :, :, 1, :].reshape(-1, hkv, d)[:L].double()
    G = hq // hkv
    Kr = K.repeat_interleave(G, dim=1).permute(1, 0, 2)            # [Hq, L, D]
    Vr = V.repeat_interleave(G, dim=1).permute(1, 0, 2)
    Q = case.q.double().permute(1, 0, 2)                           # [Hq, n, D]
    pos = (L - n + torch.arange(n))[:, None]
    mask = torch.arange(L)[None, :] <= pos
    ref = torch.nn.functional.scaled_dot_product_attention(Q, Kr, Vr, attn_mask=mask, scale=case.scale)
    np.testing.assert_allclose(got, ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def test_constant_v_gives_that_row(oracle_mod):
    case = workloads.make_case("cv", 5, [3, 1], [100, 300], 8, 2, 32, causal=True)
    row = torch.randn(32, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    case.kv[:, :, :, 1, :] = row
    got = run_oracle(oracle_mod, case)
    np.testing.assert_allclose(got, np.broadcast_to(row.double().numpy(), got.shape), rtol=0, atol=1e-13)


def test_single_visible_key_gives_its_v_row_exactly(oracle_mod):
    # causal, n == L: query 0 sees only key 0; and a sequence with L = 1
    case = workloads.make_case("one", 6, [4, 1], [4, 1], 4, 2, 16, causal=True)
    got = run_oracle(oracle_mod, case)
    for b, t in ((0, 0), (1, 4)):
        pg = int(case.block_table[b, 0])
        for h in range(4):
            v = case.kv[pg, 0, h // 2, 1, :].double().numpy()
            assert np.array_equal(got[t, h], v)


def test_two_keys_closed_form(oracle_mod):
    """Two visible keys: out = V0 + sigmoid(s1 - s0) (V1 - V0)."""
    case = workloads.make_case("two", 8, [1], [2], 1, 1, 8, causal=True, scale=0.5)
    q = torch.zeros(1, 1, 8)
    q[0, 0, 0] = 1.5
    case.q.copy_(q.to(torch.bfloat16))
    pg = int(case.block_table[0, 0])
    case.kv[pg, 0, 0, 0, :] = 0
    k1 = torch.zeros(8)
    k1[0] = 2.0
    case.kv[pg, 1, 0, 0, :] = k1.to(torch.bfloat16)
    v0 = case.kv[pg, 0, 0, 1, :].double().numpy()
    v1 = case.kv[pg, 1, 0, 1, :].double().numpy()
    s = 0.5 * 1.5 * 2.0
    expect = v0 + (v1 - v0) / (1.0 + math.exp(-s))
    got = run_oracle(oracle_mod, case)
    np.testing.assert_allclose(got[0, 0], expect, rtol=0, atol=1e-14)


def test_scale_zero_gives_mean_of_visible_rows(oracle_mod):
    case = workloads.make_case("z", 9, [3], [70], 2, 1, 16, causal=True, scale=0.0)
    got = run_oracle(oracle_mod, case)
    dense = _dense_kv(case)[0][1]   # V [L, Hkv, D]
    for i in range(3):
        vis = 70 - 3 + i + 1
        np.testing.assert_allclose(got[i, 0], dense[:vis, 0].mean(0), rtol=0, atol=1e-13)


def test_page_relocation_is_bitwise_invariant(oracle_mod):
    case = workloads.make_case("perm", 10, [2, 9], [130, 190], 8, 2, 32, causal=True, extra_pages=3)
    base = run_oracle(oracle_mod, case)
    NP = case.kv.shape[0]
    pi = torch.randperm(NP, generator=torch.Generator().manual_seed(1))
    kv2 = torch.empty_like(case.kv)
    kv2[pi] = case.kv                     # pool'[pi(i)] = pool[i]
    bt = case.block_table.clone()
    valid = bt >= 0
    bt[valid] = pi[bt[valid].long()].to(torch.int32)
    got = oracle_mod.paged_attn(case.q, kv2, bt, case.seq_lens, case.cu_q, case.scale, True)
    assert np.array_equal(got, base)


@pytest.mark.parametrize("chunk", [1, 7, 64, 100])
def test_split_combine_equals_single_pass(oracle_mod, chunk):
    case = workloads.make_case("split", 11, [1, 6, 20], [257, 64, 300], 8, 2, 64, causal=True)
    one, lse1 = run_oracle(oracle_mod, case, return_lse=True)
    spl, lse2 = run_oracle(oracle_mod, case, chunk_keys=chunk, return_lse=True)
    np.testing.assert_allclose(spl, one, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse2, lse1, rtol=1e-12, atol=1e-12)


def test_gqa_equals_mha_with_repeated_kv(oracle_mod):
    hq, hkv, d = 12, 3, 32
    G = hq // hkv
    case = workloads.make_case("gqa", 12, [4, 1], [90, 33], hq, hkv, d, causal=True)
    got = run_oracle(oracle_mod, case)
    kv_rep = case.kv.repeat_interleave(G, dim=2).contiguous()     # [NP, P, Hq, 2, D]
    mha = oracle_mod.paged_attn(case.q, kv_rep, case.block_table, case.seq_lens, case.cu_q,
                                case.scale, True)
    assert np.array_equal(got, mha)


def test_decode_causal_equals_noncausal(oracle_mod):
    case = workloads.make_case("dec", 13, [1, 1, 1], [5, 64, 129], 4, 1, 16, causal=True)
    a = run_oracle(oracle_mod, case)
    b = oracle_mod.paged_attn(case.q, case.kv, case.block_table, case.seq_lens, case.cu_q,
                              case.scale, False)
    assert np.array_equal(a, b)


def test_causal_prefix_rows_equal_dense_prefix(oracle_mod):
    """With n == L, causal row i equals non-causal attention over keys 0..i."""
    n = 70
    case = workloads.make_case("pre", 14, [n], [n], 2, 1, 16, causal=True)
    full = run_oracle(oracle_mod, case)
    for i in (0, 1, 63, 64, 69):
        sub = workloads.make_case("pre", 14, [n], [n], 2, 1, 16, causal=True)
        # same tensors, but query i alone against a sequence truncated to i+1 keys
        q1 = case.q[i:i + 1].clone()
        got = oracle_mod.paged_attn(q1, case.kv, case.block_table, torch.tensor([i + 1], dtype=torch.int32),
                                    torch.tensor([0, 1], dtype=torch.int32), case.scale, False)
        assert np.array_equal(got[0], full[i])
        del sub


def test_manifest_layout_offsets_and_strides():
    """The tiny mixed workload reproduces the decode.json manifest's buffers:
    pool [22,2,64,4,2,256] with layer 1 used, K at +262144 B, V at +262656 B,
    and the K tensormap's byte strides (slot 4096, head 1024, page 524288)."""
    g = json.load(open(os.path.join(GOLDEN, "decode_manifest_layout.json")))
    case = workloads.tiny_mixed()
    assert list(case.pool_storage.shape) == g["buffers"]["kv"]["shape"]
    assert list(case.q.shape) == g["buffers"]["q"]["shape"]
    assert list(case.block_table.shape) == g["buffers"]["table"]["shape"]
    esz = 2
    k_off = (case.kv.storage_offset() - case.pool_storage.storage_offset()) * esz
    assert k_off == g["call_args_byte_offsets"]["k"]
    v_off = k_off + case.kv.stride(3) * esz
    assert v_off == g["call_args_byte_offsets"]["v"]
    ks = g["k_tensormap"]["strides_bytes"]
    assert case.kv.stride(1) * esz == ks[0]
    assert case.kv.stride(2) * esz == ks[1]
    assert case.kv.stride(0) * esz == ks[2]
    # q tensormap: 6 adjacent q heads per KV head (group 6), token stride 6144 elements
    qs = g["q_tensormap"]["strides_bytes"]
    assert qs[0] == case.q.stride(1) * esz * 1          # next q head in the group
    assert qs[1] == case.q.stride(1) * esz * 6          # next KV head's group
    assert qs[2] == case.q.stride(0) * esz              # next token
    assert case.q.stride(0) == g["pack_scalars"]["q_token_stride_elems"]
    assert g["pack_scalars"]["q_heads"] // g["pack_scalars"]["kv_heads"] == g["pack_scalars"]["group"]
    assert g["pack_scalars"]["max_kv_len"] == g["pack_scalars"]["table_cols"] * 64


def test_manifest_group_divide_constant():
    """The manifest's fast divide-by-6 (magic 0xAAAAAAAB, shift 2) maps q head h
    to h // 6 for every head index, consistent with contiguous head groups."""
    g = json.load(open(os.path.join(GOLDEN, "decode_manifest_layout.json")))["pack_scalars"]
    magic = g["group_div_magic_i32"] & 0xFFFFFFFF
    for h in range(1 << 16):
        assert ((h * magic) >> 32) >> g["group_div_shift"] == h // g["group"]


def test_manifest_scale_log2e_constant():
    """The manifest packs float32(scale * log2(e)) for scale 1/16 = 1/sqrt(256)."""
    g = json.load(open(os.path.join(GOLDEN, "decode_manifest_layout.json")))["pack_scalars"]
    bits = g["scale_log2e_f32_bits_i32"] & 0xFFFFFFFF
    want = np.float32((1.0 / math.sqrt(g["head_dim"])) * math.log2(math.e))
    assert int(np.array([want], np.float32).view(np.uint32)[0]) == bits


def test_oracle_reads_two_layer_pool_view(oracle_mod):
    """The strided layer-1 view of the manifest pool equals a contiguous copy."""
    case = workloads.tiny_mixed()
    a = run_oracle(oracle_mod, case)
    kvc = case.kv.contiguous()
    b = oracle_mod.paged_attn(case.q, kvc, case.block_table, case.seq_lens, case.cu_q, case.scale, True)
    assert np.array_equal(a, b)
    assert np.isfinite(a).all()


def test_rows_without_visible_keys_are_zero(oracle_mod):
    case = workloads.make_case("nv", 15, [6], [3], 2, 1, 8, causal=True)
    got, lse = run_oracle(oracle_mod, case, return_lse=True)
    # positions L - n + i = -3..2: rows 0..2 see nothing
    assert np.all(got[:3] == 0) and np.all(np.isneginf(lse[:3]))
    assert np.all(np.isfinite(lse[3:]))


def test_poisoned_unused_memory_is_never_read(oracle_mod):
    case = workloads.make_case("poi", 16, [3, 1], [77, 130], 4, 2, 16, causal=True,
                               extra_pages=2, poison=True)
    got = run_oracle(oracle_mod, case)
    assert np.isfinite(got).all()


def test_head_major_layout_is_same_attention(oracle_mod):
    """The head-major pool view holds the same (page, slot, head, K/V) values as
    a contiguous copy, and the oracle reads it identically."""
    case = workloads.make_case("hm", 17, [2, 1], [90, 200], 8, 2, 16, causal=True, layout="head_major")
    assert case.kv.stride(3) == 64 * 16 and case.kv.stride(1) == 16
    a = run_oracle(oracle_mod, case)
    b = oracle_mod.paged_attn(case.q, case.kv.contiguous(), case.block_table, case.seq_lens, case.cu_q,
                              case.scale, True)
    assert np.array_equal(a, b)


# ------------------------------------------------ dense (matmul) form of the oracle
DENSE_CASES = SMALL_CASES + [
    dict(q_lens=[0, 33, 1, 130], kv_lens=[0, 200, 64, 300], hq=24, hkv=4, d=256, causal=True),
    dict(q_lens=[50], kv_lens=[50], hq=8, hkv=8, d=128, causal=False),
    dict(q_lens=[9, 3], kv_lens=[0, 2], hq=8, hkv=1, d=128, causal=True),   # L = 0 and n > L rows
]


@pytest.mark.parametrize("idx", range(len(DENSE_CASES)))
def test_dense_form_matches_c_oracle(oracle_mod, idx):
    """The matmul form (oracle/dense.py) against the C loop: two independent
    implementations of the definition agree to fp64 rounding on every row,
    also over a poisoned pool (unused pages and slots past L never read)."""
    from oracle import dense
    c = DENSE_CASES[idx]
    case = workloads.make_case("dense", 2000 + idx, c["q_lens"], c["kv_lens"], c["hq"], c["hkv"], c["d"],
                               causal=c["causal"], extra_pages=2, poison=True)
    ref = run_oracle(oracle_mod, case)
    rows, got = dense.paged_attn_rows(case.q, case.kv, case.block_table, case.seq_lens, case.cu_q,
                                      case.scale, case.causal)
    assert np.array_equal(rows, np.arange(sum(c["q_lens"])))
    assert np.isfinite(got).all()
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)
    # a row subset gives the same rows (to rounding: its products are shaped differently)
    pick = rows[::3]
    r2, g2 = dense.paged_attn_rows(case.q, case.kv, case.block_table, case.seq_lens, case.cu_q,
                                   case.scale, case.causal, rows=pick[::-1])
    assert np.array_equal(r2, pick)
    np.testing.assert_allclose(g2, got[pick], rtol=0, atol=1e-13)


def test_dense_form_chunked_rows_and_two_layer_pool(oracle_mod):
    """Row chunks (a tiny score budget) and the manifest's two-layer pool view
    change nothing."""
    from oracle import dense
    case = workloads.tiny_mixed()
    ref = run_oracle(oracle_mod, case)
    _, a = dense.paged_attn_rows(case.q, case.kv, case.block_table, case.seq_lens, case.cu_q,
                                 case.scale, case.causal)
    _, b = dense.paged_attn_rows(case.q, case.kv, case.block_table, case.seq_lens, case.cu_q,
                                 case.scale, case.causal, max_scores=1000)
    np.testing.assert_allclose(a, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(b, a, rtol=0, atol=1e-13)


def test_dense_form_closed_forms():
    """Closed forms: a single visible key gives its V row exactly; constant V
    gives that row; scale 0 gives the mean of the visible V rows."""
    from oracle import dense
    case = workloads.make_case("onek", 6, [4, 1], [4, 1], 4, 2, 16, causal=True)
    _, got = dense.paged_attn_rows(case.q, case.kv, case.block_table, case.seq_lens, case.cu_q,
                                   case.scale, True)
    for b, t in ((0, 0), (1, 4)):
        pg = int(case.block_table[b, 0])
        for h in range(4):
            assert np.array_equal(got[t, h], case.kv[pg, 0, h // 2, 1, :].double().numpy())
    case = workloads.make_case("cv", 5, [3, 1], [100, 300], 8, 2, 32, causal=True)
    row = torch.randn(32, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    case.kv[:, :, :, 1, :] = row
    _, got = dense.paged_attn_rows(case.q, case.kv, case.block_table, case.seq_lens, case.cu_q,
                                   case.scale, True)
    np.testing.assert_allclose(got, np.broadcast_to(row.double().numpy(), got.shape), rtol=0, atol=1e-13)
    case = workloads.make_case("s0", 8, [5], [70], 4, 1, 16, causal=True)
    _, got = dense.paged_attn_rows(case.q, case.kv, case.block_table, case.seq_lens, case.cu_q, 0.0, True)
    dk = _dense_kv(case)[0][1][:, 0, :]     # V rows [L, D]
    for i in range(5):
        vis = 70 - 5 + i + 1
        np.testing.assert_allclose(got[i, 0], dk[:vis].mean(axis=0), rtol=0, atol=1e-13)
