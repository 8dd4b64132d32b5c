"""GPU parity on grids that cross the XCD-run renumbering of workgroups.

Grid-order prefill launches (one sequence, or fewer than 512 workgroups)
renumber every full run of 256 workgroup ids so that each XCD takes 32
consecutive grid items, and keep the ids past the last full run in grid
order; the quantised loop does the same with runs of 512 ids (64 items per
XCD).  These shapes have both a renumbered part and a tail in grid order,
and every output row is checked: against the dense fp64 form of ORACLE-P
(bf16 bar: max-abs 2e-2, rel-RMS 5e-3), or against ORACLE-Q (rel-RMS 1e-2).
"""
import numpy as np
import pytest
import torch

import workloads
from parity_util import compare, log, run_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_gqa_fwd_amd as pa
    pa.load_library()


PREFILL = [
    # name, tokens, q heads, kv heads, head_dim, causal -> workgroups (full runs of 256 + tail)
    ("non-causal D128 MHA, 16 tiles x 20 heads", 4000, 20, 20, 128, False),   # 320 = 256 + 64
    ("causal D128 G4, 63 tiles x 8 heads", 4000, 32, 8, 128, True),           # 504 = 256 + 248
    ("causal D256 G6, 188 tiles x 4 heads", 4000, 24, 4, 256, True),          # 752 = 512 + 240
]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,n,hq,hkv,d,causal", PREFILL, ids=[p[0] for p in PREFILL])
def test_prefill_grid_order_runs_all_rows(name, n, hq, hkv, d, causal):
    from oracle import dense
    case = workloads.make_case("grid-order " + name, 3100 + d + hkv, [n], [n], hq, hkv, d, causal=causal,
                               k_channel_offset_var=2.0, poison=True, device="cuda")
    out = run_gpu(case, path=2).cpu()
    c = case.to("cpu")
    del case
    torch.cuda.empty_cache()
    log("  dense fp64 oracle over %d token rows" % n)
    rows, ref = dense.paged_attn_rows(c.q, c.kv, c.block_table, c.seq_lens, c.cu_q, c.scale, c.causal)
    assert rows.size == n
    compare(out[torch.from_numpy(rows)], ref, what="%s, all %d token rows" % (name, n))


@pytest.mark.timeout(600)
def test_quant_grid_order_runs_all_rows(oracle_mod):
    """8000 tokens x 9 heads: 63 query tiles x 9 heads = 567 workgroups (one
    renumbered run of 512 and a tail of 55 in grid order); every row."""
    import paged_kv_gqa_fwd_amd as pa
    from test_gpu_quant import _check_prep, _compare
    q, k, v = workloads.dense_qkv(3300, 1, 8000, 9, k_channel_offset_var=2.0, device="cuda")
    prep = _check_prep(q, k, v, oracle_mod, "grid-order quant")
    scale = 128 ** -0.5
    out = pa.quant_attention(q, k, v, scale, False)
    torch.cuda.synchronize()
    log("  quantised oracle over all 8000 tokens x 9 heads")
    ref = oracle_mod.quant_attn(prep, scale, False)
    _compare(out, ref, "quant 8000 x 9 heads, all rows")
    assert np.isfinite(ref).all()
