"""Seeded random sweep of the paged attention paths against the fp64 oracle,
through the C ABI.

Each case draws its shapes and options from a fixed-seed generator: head_dim
128 or 256; group sizes 1 to 8; ragged batches with empty sequences, single
keys, page-edge and multi-page lengths, n > L; causal or not; a sliding
window; attention sinks; an fp8 cache on the decode paths; every decode path
(automatic, fixed split with several least range sizes, single-launch merge,
balanced) and the prefill path.  Tail slots and unused pages are poisoned
with NaN / inf.  Every written row is held to the bf16 bar (max-abs 2e-2,
rel-RMS 5e-3).
"""
import math
import random

import pytest
import torch

import workloads
from parity_util import compare, log

pytestmark = pytest.mark.gpu

N_CASES = 200


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_gqa_fwd_amd as pa
    pa.load_library()


def _draw(rng: random.Random, it: int):
    d = rng.choice([128, 256])
    prefill = rng.random() < 0.4
    hkv = rng.choice([1, 2, 4] if prefill else [1, 2, 4, 8])
    G = rng.choice([1, 4, 6] if prefill else [1, 4, 6, 8])
    B = rng.randint(1, 8 if prefill else 12)
    q_lens, kv_lens = [], []
    for _ in range(B):
        L = rng.choice([0, 1, rng.randint(1, 64), rng.randint(60, 70), rng.randint(100, 600 if prefill else 900)])
        n = rng.randint(0, min(L + 2, 150)) if prefill else rng.choice([0, 1, 1, 1, 2])
        q_lens.append(n)
        kv_lens.append(L)
    if max(kv_lens) == 0:          # the pool needs at least one page
        kv_lens[0] = rng.randint(1, 200)
    if sum(q_lens) == 0:
        q_lens[0] = 1
    path = 2 if prefill else rng.choice([0, 1, 3, 4])
    return dict(d=d, hkv=hkv, hq=hkv * G, q_lens=q_lens, kv_lens=kv_lens,
                causal=rng.random() < 0.8, window=rng.choice([0, 0, 0, rng.randint(1, 300)]),
                sinks=rng.random() < 0.25, fp8=(not prefill) and rng.random() < 0.3, path=path,
                pps=0 if path in (0, 2) else rng.choice([0, 1, 2, 3, 7]), seed=rng.randint(1, 10 ** 6), it=it)


@pytest.mark.parametrize("block", range(4))
def test_random_cases(oracle_mod, block):
    import paged_kv_gqa_fwd_amd as pa
    rng = random.Random(9100 + block)
    for it in range(N_CASES // 4):
        c = _draw(rng, it)
        log("case %s" % c)
        case = workloads.make_case("rnd%d-%d" % (block, it), c["seed"], c["q_lens"], c["kv_lens"], c["hq"], c["hkv"],
                                   c["d"], causal=c["causal"], table_cols=math.ceil(max(c["kv_lens"]) / 64) + 1,
                                   poison=True)
        kw = {}
        if c["fp8"]:
            case = workloads.fp8_pool_case(case)
            kw = dict(k_scale=0.5, v_scale=0.5)
        sinks = None
        if c["sinks"]:
            g = torch.Generator().manual_seed(c["seed"])
            sinks = (torch.randn(c["hq"], generator=g) * 2).float()
            sinks[0] = -math.inf
        ref = oracle_mod.paged_attn(case.q, case.kv, case.block_table, case.seq_lens, case.cu_q, case.scale,
                                    case.causal, sinks=None if sinks is None else sinks.double().numpy(),
                                    window=c["window"], **kw)
        gc = case.to("cuda")
        res = pa.paged_attention(gc.q, gc.kv, gc.block_table, gc.seq_lens, gc.cu_q, max(case.max_q, 1), case.scale,
                                 case.causal, path=c["path"], pages_per_split=c["pps"], window=c["window"],
                                 sinks=None if sinks is None else sinks.cuda(), **kw)
        torch.cuda.synchronize()
        compare(res, ref, what="random case %d/%d" % (block, it))
