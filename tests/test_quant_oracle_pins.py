"""Pins of the quantised-attention oracle (CPU only).

The oracle (oracle/quant_oracle.c) emulates the int8 Q.K / fp8 P.V variant
named by the SageAttention2 block-24 baseline page (phase_timings and
fused_mainloop_phases).  These tests tie it to things other than itself:

* the fp8 encoder/decoder against torch's float8_e4m3fn conversion over every
  bf16 input pattern (library routine), plus the documented saturation;
* the int8 block quantiser against the error bound |x - s q| <= s/2, the
  amax-hits-127 property and the all-zero block;
* K-mean smoothing against its defining invariance: a per-channel offset
  added to every key changes nothing (bitwise), and the mean moves by it;
* the whole pipeline, with the fp8 rounding of the weights switched off,
  against the plain attention oracle on inputs every quantiser represents
  exactly;
* with the weight rounding on, against a full-row numpy computation on rows
  whose maximum sits in the first key tile (so the running maximum never
  moves), and against the closed form of the online recurrence on rows whose
  running maximum moves from tile to tile (weights rounded to e4m3 by a
  nearest-value search over the decoded code grid);
* closed forms: a single visible key gives its dequantised V row exactly.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def _rand_bf16(shape, seed, scale=1.0, offset=None):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(*shape, generator=g) * scale
    if offset is not None:
        x = x + offset
    return x.to(torch.bfloat16)


# ------------------------------------------------------------------ fp8 codec
def test_e4m3_encoder_matches_torch_on_all_bf16_patterns():
    bits = torch.arange(0, 1 << 16, dtype=torch.int32).to(torch.int16)
    x = bits.view(torch.bfloat16).float()
    ok = torch.isfinite(x) & (x.abs() < 464.0)
    xs = x[ok]
    ref = xs.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = np.array([oracle.e4m3_encode(float(v)) for v in xs.tolist()], dtype=np.uint8)
    # torch keeps the sign of a zero result; so does the oracle
    assert np.array_equal(ours, ref)


def test_e4m3_saturates_above_448():
    for v in (464.0, 480.0, 1e4, 3e38):
        assert oracle.e4m3_encode(v) == 0x7E
        assert oracle.e4m3_encode(-v) == 0xFE
    assert oracle.e4m3_decode(0x7E) == 448.0


def test_e4m3_decoder_matches_torch():
    codes = [c for c in range(256) if c not in (0x7F, 0xFF)]
    ref = torch.tensor(codes, dtype=torch.uint8).view(torch.float8_e4m3fn).float().tolist()
    assert [oracle.e4m3_decode(c) for c in codes] == ref
    assert np.isnan(oracle.e4m3_decode(0x7F))


# --------------------------------------------------------------- int8 blocks
def test_int8_codes_round_half_to_even_like_torch_round():
    """Exact ties: blocks whose amax is 127 * 2^e have a power-of-two scale,
    so x * (1/s) is exact and every x placed at (k + 1/2) * s is a true tie.
    The codes must equal torch.round (half to even) plus the +-127 clamp;
    rounding ties away from zero, or truncating, fails here.  Q is quantised
    as it is (no smoothing), so the Q codes are checked."""
    B, H, D = 1, 2, 128
    N = 64 * 4
    q = torch.zeros(B, N, H, D)
    g = torch.Generator().manual_seed(7)
    for blk, e in enumerate((0, -1, 1, -3)):
        s = 2.0 ** e
        j0 = 64 * blk
        for h in range(H):
            k = torch.randint(-126, 126, (64, D), generator=g).float()
            x = (k + 0.5) * s                       # every element a tie
            x[0, 0] = 127.0 * s                     # the block's amax: scale = s exactly
            x[1, :8] = torch.tensor([0.5, -0.5, 1.5, -1.5, 2.5, -2.5, 126.5, -126.5]) * s
            q[0, j0:j0 + 64, h, :] = x
    qb = q.to(torch.bfloat16)
    assert torch.equal(qb.float(), q), "the ties must be exact bf16 values"
    kz = torch.zeros_like(qb)
    vz = torch.zeros_like(qb)
    p = oracle.quant_prep(qb, kz, vz)
    for blk, e in enumerate((0, -1, 1, -3)):
        s = 2.0 ** e
        assert p["sq"][0, :, blk].tolist() == [s] * H
        x = q[0, 64 * blk:64 * blk + 64].permute(1, 0, 2)            # [H, 64, D]
        want = torch.clamp(torch.round(x / s), -127, 127).to(torch.int8).numpy()
        got = p["qi"][0, 64 * blk:64 * blk + 64].transpose(1, 0, 2)   # [H, 64, D]
        assert np.array_equal(got, want), "block %d" % blk
    # the hand-placed ties: 0.5 -> 0, 1.5 -> 2, 2.5 -> 2, 126.5 -> 126
    assert p["qi"][0, 1, 0, :8].tolist() == [0, 0, 2, -2, 2, -2, 126, -126]


def test_int8_block_error_bound_and_amax():
    B, N, H, D = 1, 200, 3, 128     # 4 blocks, the last one 8 rows
    q = _rand_bf16((B, N, H, D), 1, scale=3.0)
    k = _rand_bf16((B, N, H, D), 2)
    v = _rand_bf16((B, N, H, D), 3)
    p = oracle.quant_prep(q, k, v)
    qf = q.float().numpy()
    for blk in range(4):
        j0, j1 = 64 * blk, min(N, 64 * blk + 64)
        for h in range(H):
            s = float(p["sq"][0, h, blk])
            x = qf[0, j0:j1, h, :]
            codes = p["qi"][0, j0:j1, h, :].astype(np.float64)
            # half a step, plus the f32 rounding of x * (1/s) (|x/s| <= 127)
            assert np.abs(x - s * codes).max() <= s * (0.5 + 1e-5)
            assert np.abs(codes).max() == 127
            assert np.isclose(s, np.abs(x).max() / 127, rtol=1e-6)


def test_int8_zero_block_has_unit_scale():
    B, N, H, D = 1, 128, 1, 128
    q = torch.zeros((B, N, H, D), dtype=torch.bfloat16)
    q[0, 64:] = _rand_bf16((64, 1, 128), 4)
    k = _rand_bf16((B, N, H, D), 5)
    v = _rand_bf16((B, N, H, D), 6)
    p = oracle.quant_prep(q, k, v)
    assert p["sq"][0, 0, 0] == 1.0
    assert not p["qi"][0, :64].any()


# ------------------------------------------------------------- K-mean smoothing
def test_k_mean_removes_per_channel_offset_bitwise():
    B, N, H, D = 1, 256, 2, 128
    g = torch.Generator().manual_seed(7)
    # small integers: every sum, mean (N a power of two) and difference is exact
    k = torch.randint(-8, 9, (B, N, H, D), generator=g).to(torch.bfloat16)
    c = torch.randint(-100, 101, (1, 1, H, D), generator=g).to(torch.float32)
    k2 = (k.float() + c).to(torch.bfloat16)
    assert torch.equal(k2.float(), k.float() + c)
    q = _rand_bf16((B, N, H, D), 8)
    v = _rand_bf16((B, N, H, D), 9)
    p1 = oracle.quant_prep(q, k, v)
    p2 = oracle.quant_prep(q, k2, v)
    assert np.array_equal(p2["mk"] - p1["mk"], c[0].numpy())
    for key in ("ki", "sk", "qi", "sq", "vq", "sv"):
        assert np.array_equal(p1[key], p2[key]), key
    o1 = oracle.quant_attn(p1, 0.088, causal=False)
    o2 = oracle.quant_attn(p2, 0.088, causal=False)
    assert np.array_equal(o1, o2)


# ------------------------------------------- pipeline vs the plain attention oracle
def _exact_inputs(N, H, D, seed):
    """Q, K integer-valued with |x| <= 127 and every 64-row block reaching 127
    (so the int8 scale is exactly 1), K with per-channel mean exactly 0 (its
    second half is the negated first half), and V on the e4m3 grid with every
    channel reaching 448 (fp8 scale exactly 1).  N is a multiple of 128."""
    g = torch.Generator().manual_seed(seed)
    q = torch.randint(-127, 128, (1, N, H, D), generator=g).float()
    half = torch.randint(-127, 128, (1, N // 2, H, D), generator=g).float()
    for blk in range(N // 128):
        half[0, 64 * blk, :, 1] = 127.0
    k = torch.cat([half, -half], dim=1)
    for blk in range(N // 64):
        q[0, 64 * blk, :, 0] = 127.0
    codes = torch.randint(0, 256, (1, N, H, D), generator=g)
    codes[(codes & 0x7F) == 0x7F] = 0x38
    v = codes.to(torch.uint8).view(torch.float8_e4m3fn).float()
    v[0, 3, :, :] = 448.0
    return q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)


def _plain_oracle_dense(q, k, v, scale, causal):
    """The paged fp64 oracle on dense [1, N, H, D] inputs (identity block table)."""
    _, N, H, D = q.shape
    P = 64
    NP = (N + P - 1) // P
    pool = torch.zeros((NP * P, H, 2, D), dtype=torch.bfloat16)
    pool[:N, :, 0] = k[0]
    pool[:N, :, 1] = v[0]
    pool = pool.view(NP, P, H, 2, D)
    bt = torch.arange(NP, dtype=torch.int32).view(1, NP)
    out = oracle.paged_attn(q[0].contiguous(), pool, bt, torch.tensor([N], dtype=torch.int32),
                            torch.tensor([0, N], dtype=torch.int32), scale, causal)
    return out[None]


@pytest.mark.parametrize("causal", [False, True])
def test_pipeline_without_weight_rounding_equals_plain_attention(causal):
    N, H, D = 256, 2, 128
    q, k, v = _exact_inputs(N, H, D, 11)
    p = oracle.quant_prep(q, k, v)
    assert np.all(p["sq"] == 1.0) and np.all(p["sk"] == 1.0) and np.all(p["sv"] == 1.0)
    assert np.all(p["mk"] == 0.0)
    assert np.array_equal(p["qi"].astype(np.float32), q.float().numpy())
    assert np.array_equal(p["ki"].astype(np.float32), k.float().numpy())
    scale = 2e-5
    got = oracle.quant_attn(p, scale, causal, quant_p=False)
    ref = _plain_oracle_dense(q, k, v, scale, causal)
    assert np.abs(got - ref).max() <= 1e-10 * max(1.0, np.abs(ref).max())


def test_weight_rounding_matches_full_row_numpy_when_max_is_in_first_tile():
    N, H, D = 256, 1, 128
    g = torch.Generator().manual_seed(12)
    q = (torch.randn(1, N, H, D, generator=g).abs() + 0.5).to(torch.bfloat16)
    k = torch.randn(1, N, H, D, generator=g)
    k[0, 5] = 4.0                     # key 5 (first tile) scores highest for every query
    k = k.to(torch.bfloat16)
    v = _rand_bf16((1, N, H, D), 13)
    p = oracle.quant_prep(q, k, v)
    scale = 0.05
    got = oracle.quant_attn(p, scale, causal=False, quant_p=True)
    # full-row computation from the quantised operands
    qi = p["qi"][0, :, 0, :].astype(np.int64)
    ki = p["ki"][0, :, 0, :].astype(np.int64)
    sq = np.repeat(p["sq"][0, 0].astype(np.float64), 64)[:N]
    sk = np.repeat(p["sk"][0, 0].astype(np.float64), 64)[:N]
    s = (qi @ ki.T).astype(np.float64) * sq[:, None] * sk[None, :] * scale
    assert np.all(np.argmax(s, axis=1) < 64)
    w = np.exp(s - s.max(axis=1, keepdims=True))
    wq = _e4m3_nearest(448.0 * w)
    vdec = torch.from_numpy(p["vq"][0, 0]).view(torch.float8_e4m3fn).double().numpy()  # [D, N]
    ref = (wq @ vdec.T) * p["sv"][0, 0].astype(np.float64)[None, :] / (448.0 * w.sum(axis=1, keepdims=True))
    assert np.abs(got[0, :, 0, :] - ref).max() <= 1e-12 * np.abs(ref).max()


def _e4m3_nearest(x):
    """Round non-negative doubles to the nearest e4m3 value (ties to the even
    code), by search over the grid of every positive code as torch decodes it.
    Direct from the double: torch's own conversion of a double goes through
    float first, and that double rounding can move a value that lies just off
    a tie onto it."""
    codes = np.arange(0, 0x7F)
    grid = torch.from_numpy(codes.astype(np.uint8)).view(torch.float8_e4m3fn).double().numpy()
    x = np.minimum(np.asarray(x, dtype=np.float64), 448.0)
    hi = np.clip(np.searchsorted(grid, x, side="left"), 1, len(grid) - 1)
    lo = hi - 1
    dl, dh = x - grid[lo], grid[hi] - x
    pick = np.where(dl < dh, lo, np.where(dh < dl, hi, np.where(codes[lo] % 2 == 0, lo, hi)))
    return grid[pick]


def _moving_max_closed_form(p, scale, causal, b=0, h=0, tile=64, final_max_only=False):
    """The online recurrence of the fused loop written in closed form.

    Keys are taken in ascending 64-key tiles.  With m_t the running maximum
    after tile t (the cumulative maximum of the per-tile maxima over the
    row's visible keys) and m_T its final value, the recurrence (rescale O
    and l by exp(m_old - m_new), add e4m3(448 exp(s - m_t)) V and
    exp(s - m_t)) sums to
        O = sum_t exp(m_t - m_T) sum_{j in t} dec(e4m3(448 exp(s_j - m_t))) V_j
        l = sum_j exp(s_j - m_T),   out = O s_v / (448 l).
    No rescaling happens here, so a wrong rescale factor, an l that sums the
    rounded weights or a non-cumulative maximum in the oracle shows.
    final_max_only rounds every weight against m_T instead (the schedule
    without an online maximum), to show that the pin sees the difference."""
    # the C library's exp (as the oracle uses), elementwise: numpy's own
    # vectorised exp differs from it in the last bit for a few percent of
    # arguments, which can move a weight across an e4m3 rounding boundary
    cexp = np.frompyfunc(math.exp, 1, 1)
    N = p["qi"].shape[1]
    qi = p["qi"][b, :, h, :].astype(np.int64)
    ki = p["ki"][b, :, h, :].astype(np.int64)
    sq = np.repeat(p["sq"][b, h].astype(np.float64), 64)[:N]
    sk = np.repeat(p["sk"][b, h].astype(np.float64), 64)[:N]
    s = (qi @ ki.T).astype(np.float64) * sq[:, None] * sk[None, :] * scale
    vdec = torch.from_numpy(p["vq"][b, h]).view(torch.float8_e4m3fn).double().numpy()[:, :N]  # [D, N]
    out = np.zeros((N, vdec.shape[0]))
    moves = np.zeros(N, dtype=np.int64)
    for i in range(N):
        vis = i + 1 if causal else N
        row = s[i, :vis]
        ntile = (vis + tile - 1) // tile
        tmax = np.array([row[t * tile:(t + 1) * tile].max() for t in range(ntile)])
        m = np.maximum.accumulate(tmax)
        moves[i] = len(np.unique(m)) - 1
        mT = m[-1]
        o = np.zeros(vdec.shape[0])
        for t in range(ntile):
            mt = mT if final_max_only else m[t]
            w = cexp(row[t * tile:(t + 1) * tile] - mt).astype(np.float64)
            wq = _e4m3_nearest(448.0 * w)
            o += math.exp(mt - mT) * (vdec[:, t * tile:t * tile + len(w)] @ wq)
        l = cexp(row - mT).astype(np.float64).sum()
        out[i] = o * p["sv"][b, h].astype(np.float64) / (448.0 * l)
    return out, moves


@pytest.mark.parametrize("causal", [False, True])
def test_weight_rounding_with_moving_max_matches_closed_form(causal):
    N, H, D = 300, 2, 128                  # five key tiles, the last one ragged (44 keys)
    g = torch.Generator().manual_seed(21)
    q = (torch.randn(1, N, H, D, generator=g).abs() + 0.5).to(torch.bfloat16)
    k = torch.randn(1, N, H, D, generator=g)
    for t in range(5):                     # one key per tile scores higher the later its tile
        k[0, 64 * t + 7] += 0.5 * (t + 1)
    k = k.to(torch.bfloat16)
    v = _rand_bf16((1, N, H, D), 22)
    p = oracle.quant_prep(q, k, v)
    scale = 0.05
    got = oracle.quant_attn(p, scale, causal=causal, quant_p=True)
    for h in range(H):
        ref, moves = _moving_max_closed_form(p, scale, causal, h=h)
        assert (moves >= 2).mean() > 0.5     # the running maximum moves on most rows
        assert np.abs(got[0, :, h, :] - ref).max() <= 1e-12 * np.abs(ref).max()
        # rounding every weight against the final maximum is a different
        # result, far outside the comparison above
        alt, _ = _moving_max_closed_form(p, scale, causal, h=h, final_max_only=True)
        assert np.abs(alt - ref).max() > 1e-6 * np.abs(ref).max()


def test_single_visible_key_gives_dequantised_v_row():
    N, H, D = 70, 2, 128
    q = _rand_bf16((1, N, H, D), 14)
    k = _rand_bf16((1, N, H, D), 15)
    v = _rand_bf16((1, N, H, D), 16)
    p = oracle.quant_prep(q, k, v)
    out = oracle.quant_attn(p, 0.088, causal=True)
    vdec = torch.from_numpy(p["vq"][0]).view(torch.float8_e4m3fn).double().numpy()  # [H, D, N]
    for h in range(H):
        exp_row = vdec[h, :, 0] * p["sv"][0, h].astype(np.float64)
        assert np.array_equal(out[0, 0, h], exp_row)


def test_weight_rounding_error_is_small_but_visible():
    """The fp8 rounding of the weights moves the result by a few 1e-3..1e-2
    (relative RMS) -- the reason the emulation matters for a 1e-2 bar."""
    N, H, D = 300, 2, 128
    q = _rand_bf16((1, N, H, D), 17)
    k = _rand_bf16((1, N, H, D), 18, offset=1.0)
    v = _rand_bf16((1, N, H, D), 19)
    p = oracle.quant_prep(q, k, v)
    a = oracle.quant_attn(p, D ** -0.5, False, quant_p=True)
    b = oracle.quant_attn(p, D ** -0.5, False, quant_p=False)
    rel = np.linalg.norm(a - b) / np.linalg.norm(b)
    assert 1e-3 < rel < 5e-2
