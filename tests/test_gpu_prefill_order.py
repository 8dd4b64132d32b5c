"""GPU checks of the prefill launch order, through the C ABI.

A ragged prefill batch (two or more sequences and 512 or more workgroups)
first runs a one-workgroup sort of the grid's (tile, KV head, sequence)
items by the pages each one streams, and the prefill workgroups then take
their items in that order, most pages first.  Every item writes only its
own output rows, so the order changes no bit of the result: each case's
batch output equals, bit for bit, the same sequences called one at a time
(one sequence keeps the grid order; its keys in one pass), and matches the fp64 oracle to the bf16
bar (max-abs 2e-2, rel-RMS 5e-3) on every row of the short sequences and a
seeded quarter of the long ones.  Cases cover both head dims, causal,
unmasked and windowed masks (Mojo SM100MHA2Q docs, MaskType), an empty
query run, an odd number of KV heads (the heads of a pair then straddle the
XCD deal), poisoned tails, and an fp8 cache read through the staging pool.
"""
import numpy as np
import pytest
import torch

import workloads
from parity_util import compare, log, sub_case_rows

pytestmark = pytest.mark.gpu

PATH_PREFILL = 2

# (D, G, Hkv, q_lens, kv_lens, causal, window): every grid holds >= 512 workgroups
CASES = [
    (256, 6, 4, [900, 40, 700, 1, 0], [2500, 40, 900, 1800, 600], True, 0),    # 43 tiles x 4 x 5
    (128, 4, 8, [2048, 300, 5], [3000, 300, 4000], True, 0),                 # 32 tiles x 8 x 3
    (128, 2, 8, [3000, 1400, 128], [3000, 2000, 128], False, 300),           # 24 tiles x 8 x 3
    (256, 3, 8, [1400, 90], [5000, 120], True, 700),                         # 33 tiles x 8 x 2
    (256, 2, 3, [1400, 30, 500, 1, 0, 900, 64, 200],
     [2000, 30, 600, 1000, 100, 900, 4000, 250], True, 0),                   # 22 tiles x 3 x 8 (Hkv odd)
]


def _grid(d, G, hkv, q_lens):
    bm = 256 if d == 128 else 128
    return -(-max(q_lens) * G // bm) * hkv * len(q_lens)


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_gqa_fwd_amd as pa
    pa.load_library()


def _call(case, window, kw, one_pass=False):
    import paged_kv_gqa_fwd_amd as pa
    g = case.to("cuda")
    # one_pass: a split size past every page keeps a small grid's keys in one
    # pass (no split-key partials), the arithmetic of the batch's workgroups
    out = pa.paged_attention(g.q, g.kv, g.block_table, g.seq_lens, g.cu_q, max(case.max_q, 1), case.scale,
                             case.causal, path=PATH_PREFILL, window=window,
                             pages_per_split=(1 << 30) if one_pass else 0, **kw)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("i", range(len(CASES)))
@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_ordered_batch_equals_single_calls(oracle_mod, i, fp8):
    import paged_kv_gqa_fwd_amd as pa
    d, G, hkv, q_lens, kv_lens, causal, window = CASES[i]
    assert _grid(d, G, hkv, q_lens) >= 512
    case = workloads.make_case("pforder%d-D%d" % (i, d), 2300 + i, q_lens, kv_lens, G * hkv, hkv, d, causal=causal,
                               table_cols=max(kv_lens) // 64 + 2, extra_pages=2, poison=True)
    kw = {}
    if fp8:
        case = workloads.fp8_pool_case(case)
        kw = {"k_scale": 0.5, "v_scale": 0.5}
    plan = pa.make_plan(pa.make_dims(case.q, case.kv, case.block_table), case.n_seqs, case.max_q, PATH_PREFILL,
                        0, window, 1 if fp8 else 0)
    assert plan.grid_x * plan.grid_y * plan.grid_z >= 512 and plan.workspace_bytes > 0
    log("  gpu ordered prefill: %s fp8=%s window=%d grid=%d" % (
        case.name, fp8, window, plan.grid_x * plan.grid_y * plan.grid_z))
    out = _call(case, window, kw)
    assert torch.isfinite(out.float()).all()
    # the same sequences one at a time (grid order): bit-for-bit equal rows
    cu = case.cu_q.tolist()
    for b in range(case.n_seqs):
        if cu[b + 1] == cu[b]:
            continue
        sub, rows = sub_case_rows(case, [b])
        one = _call(sub, window, kw, one_pass=True)
        got = out[cu[b]:cu[b + 1]]
        assert torch.equal(got.view(torch.int16), one[:len(rows)].view(torch.int16)), \
            "%s: sequence %d differs from its own call" % (case.name, b)
    # the oracle on a sample: short sequences whole, a quarter of the rest
    rng = np.random.default_rng(2400 + i)
    mask = np.zeros(case.q.shape[0], dtype=bool)
    for b in range(case.n_seqs):
        n = cu[b + 1] - cu[b]
        if n <= 128:
            mask[cu[b]:cu[b + 1]] = True
        else:
            mask[cu[b] + rng.choice(n, n // 4, replace=False)] = True
            mask[[cu[b], cu[b + 1] - 1]] = True
    ref = oracle_mod.paged_attn(case.q, case.kv, case.block_table, case.seq_lens, case.cu_q, case.scale, causal,
                                row_mask=mask, window=window, **kw)
    compare(out, ref, rows=np.nonzero(mask)[0], what="%s fp8=%s window=%d" % (case.name, fp8, window))


@pytest.mark.parametrize("ci", [0, 4])
def test_order_table_is_a_permutation_most_pages_first(ci):
    """The order table in the caller's workspace (its first bytes on a bf16
    cache): a permutation of the grid's items whose streamed pages
    (1 + ceil(last visible key / 64) for an item with rows, 0 without; no
    window) never increase along the launch order, with the KV heads of each
    (tile, sequence) pair in adjacent places."""
    import paged_kv_gqa_fwd_amd as pa
    d, G, hkv, q_lens, kv_lens, causal, window = CASES[ci]
    assert window == 0
    case = workloads.make_case("pforder-table%d" % ci, 2350 + ci, q_lens, kv_lens, G * hkv, hkv, d, causal=causal,
                               table_cols=max(kv_lens) // 64 + 2)
    plan = pa.make_plan(pa.make_dims(case.q, case.kv, case.block_table), case.n_seqs, case.max_q, PATH_PREFILL)
    items = plan.grid_x * plan.grid_y * plan.grid_z
    assert plan.workspace_bytes == -(-items * 4 // 256) * 256
    g = case.to("cuda")
    ws = torch.full((plan.workspace_bytes,), 0xFF, dtype=torch.uint8, device="cuda")
    log("  gpu ordered prefill with a caller workspace: grid=%d" % items)
    pa.paged_attention(g.q, g.kv, g.block_table, g.seq_lens, g.cu_q, case.max_q, case.scale, causal,
                       path=PATH_PREFILL, workspace=ws)
    torch.cuda.synchronize()
    order = ws[:items * 4].view(torch.int32).cpu().numpy()
    assert np.array_equal(np.sort(order), np.arange(items))
    bm = 128 if d == 256 else 256

    def pages(item):
        tile, rest = item % plan.grid_x, item // plan.grid_x
        b = rest // plan.grid_y
        n, L = q_lens[b], kv_lens[b]
        R = n * G
        if tile * bm >= R:
            return 0
        last = (min(R, tile * bm + bm) - 1) // G
        vis = min(max(L - n + last + 1, 0), L)
        return 1 + -(-vis // 64)

    work = np.array([pages(int(i)) for i in order])
    assert (np.diff(work) <= 0).all(), "launch order is not most pages first"
    assert work[-1] == 0 and work[0] > 1     # items without rows last
    # heads side by side: places hkv k .. hkv k + hkv - 1 hold one (tile, sequence) pair, heads 0 .. hkv-1
    pairs = order.reshape(-1, hkv)
    tile, rest = pairs % plan.grid_x, pairs // plan.grid_x
    assert (tile == tile[:, :1]).all() and (rest // hkv == rest[:, :1] // hkv).all()
    assert (rest % hkv == np.arange(hkv)[None, :]).all()
