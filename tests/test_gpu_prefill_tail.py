"""GPU parity of the prefill kernel's last-tile handling, through the C ABI.

The prefill kernel loads every slot of a page, also those past a
sequence's last key, and zeroes the V rows past the last key in LDS once
the last tile has landed (their scores are masked; a non-finite V row would
still turn a zero weight into NaN).  At head_dim 128 a tile is two pages,
and a tile whose second page lies past the workgroup's last visible key
re-reads the first page into that slot (its V rows zeroed too).  These
cases put the last key at page edges and inside pages, make the number of
visible pages odd and even, and poison the slots past L and the unused
pages with NaN / inf, on the bf16 pool and through the fp8 staging pool,
causal, unmasked and windowed (Mojo SM100MHA2Q docs, MaskType; kern-kernels
examples/decode.json, buffers.kv: pages of 64 slots).  The grids are small,
so each case runs both with its keys split (the automatic plan: every split's
last page is a last tile) and in one pass.

Tolerance: the bf16 bar (max-abs 2e-2, rel-RMS 5e-3 over every written row).
"""
import pytest
import torch

import workloads
from parity_util import compare, log

pytestmark = pytest.mark.gpu

PATH_PREFILL = 2

# (D, G, Hkv, q_lens, kv_lens, causal, window)
CASES = [
    (128, 4, 2, [70], [391], True, 0),             # 7 pages (odd): a tile's second page past the end
    (128, 4, 2, [64], [384], True, 0),             # 6 pages, last one full
    (128, 4, 2, [40, 9], [129, 649], True, 0),     # one key into a page; ragged batch
    (128, 1, 3, [300], [365], True, 0),            # several query tiles
    (128, 4, 2, [20], [129], False, 0),
    (128, 4, 2, [100], [1000], True, 200),         # window: the loop starts mid-sequence
    (256, 6, 2, [30, 50], [130, 1050], True, 0),
    (256, 6, 2, [64], [127], True, 0),             # 63 keys into the last page
    (256, 4, 2, [20], [129], False, 0),
    (256, 4, 1, [90], [1000], True, 130),
    (256, 2, 2, [40, 0, 7], [40, 300, 7], True, 0),  # n = L, an empty query run
]


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_gqa_fwd_amd as pa
    pa.load_library()


def _case(i, d, G, hkv, q_lens, kv_lens, causal):
    return workloads.make_case("pftail%d-D%d" % (i, d), 2100 + i, q_lens, kv_lens, G * hkv, hkv, d, causal=causal,
                               table_cols=max(kv_lens) // 64 + 2, extra_pages=2, poison=True)


@pytest.mark.parametrize("i", range(len(CASES)))
@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
@pytest.mark.parametrize("one_pass", [False, True], ids=["auto", "one_pass"])
def test_prefill_last_tile(oracle_mod, i, fp8, one_pass):
    import paged_kv_gqa_fwd_amd as pa
    d, G, hkv, q_lens, kv_lens, causal, window = CASES[i]
    case = _case(i, d, G, hkv, q_lens, kv_lens, causal)
    kw = {}
    if fp8:
        case = workloads.fp8_pool_case(case)
        kw = {"k_scale": 0.5, "v_scale": 0.5}
    ref = oracle_mod.paged_attn(case.q, case.kv, case.block_table, case.seq_lens, case.cu_q, case.scale, causal,
                                window=window, **kw)
    g = case.to("cuda")
    # these grids are small, so the automatic plan splits their keys; a
    # split size past every page keeps them in one pass
    log("  gpu prefill call: %s fp8=%s window=%d one_pass=%s" % (case.name, fp8, window, one_pass))
    out = pa.paged_attention(g.q, g.kv, g.block_table, g.seq_lens, g.cu_q, max(case.max_q, 1), case.scale, causal,
                             path=PATH_PREFILL, window=window, pages_per_split=(1 << 30) if one_pass else 0, **kw)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    compare(out, ref, what="%s fp8=%s window=%d one_pass=%s" % (case.name, fp8, window, one_pass))
