"""CPU-only checks of the C ABI: the library loads, exports every function the
header declares, and rejects invalid arguments before launching anything.
No call here reaches a kernel launch (every call fails validation, plans, or
is the n_seqs == 0 no-op), so no GPU is needed."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "paged_attn.h")

OK, E_NULL, E_SHAPE, E_UNSUP, E_STRIDE, E_ALIGN, E_WS, E_HIP = 0, -1, -2, -3, -4, -5, -6, -7
FAKE = 0x10000   # 16-byte aligned, never dereferenced


@pytest.fixture(scope="module")
def pa():
    import paged_kv_gqa_fwd_amd as mod
    from paged_kv_gqa_fwd_amd import build as b
    if not os.path.exists(mod.LIB_PATH):
        b.build()
    mod.load_library()
    return mod


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(attn_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_entry_points():
    fns = header_functions()
    for name in ("attn_paged_fwd", "attn_paged_fwd_ex", "attn_paged_make_plan",
                 "attn_paged_workspace_bytes", "attn_status_string", "attn_quant_fwd",
                 "attn_quant_prep", "attn_quant_attend", "attn_quant_layout_of",
                 "attn_workspace_clear", "attn_paged_kv_write", "attn_paged_fwd_write",
                 "attn_paged_fwd_opt", "attn_paged_make_plan_opt", "attn_paged_kv_write_opt",
                 "attn_paged_fwd_write_opt"):
        assert name in fns


def test_library_exports_every_header_function(pa):
    lib = ctypes.CDLL(pa.LIB_PATH)
    missing = [f for f in header_functions() if not hasattr(lib, f)]
    assert not missing, missing


def dims(**kw):
    import paged_kv_gqa_fwd_amd as mod
    d = dict(num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=64, num_pages=100,
             max_pages_per_seq=16, num_tokens=64, q_stride_token=32 * 128, q_stride_head=128,
             o_stride_token=32 * 128, o_stride_head=128, kv_stride_page=64 * 8 * 2 * 128,
             kv_stride_slot=8 * 2 * 128, kv_stride_head=2 * 128, kv_stride_kv=128, bt_stride=16)
    d.update(kw)
    return mod.attn_paged_dims(**d)


def call(pa, d, n_seqs=4, max_q=1, out=FAKE, q=FAKE, kv=FAKE, bt=FAKE, sl=FAKE, cq=FAKE,
         scale=0.1, causal=1, ws=None, ws_bytes=0, path=0, pps=0):
    lib = pa.load_library()
    return lib.attn_paged_fwd_ex(out, q, kv, bt, sl, cq, n_seqs, max_q, scale, causal,
                                 ctypes.byref(d) if d is not None else None, ws, ws_bytes, None,
                                 path, pps)


@pytest.mark.parametrize("kw,expect", [
    (dict(head_dim=64), E_UNSUP),
    (dict(head_dim=192), E_UNSUP),
    (dict(page_size=32), E_UNSUP),
    (dict(num_q_heads=30), E_SHAPE),
    (dict(num_kv_heads=0), E_SHAPE),
    (dict(num_pages=0), E_SHAPE),
    (dict(max_pages_per_seq=0), E_SHAPE),
    (dict(q_stride_head=100), E_STRIDE),
    (dict(q_stride_head=120), E_STRIDE),
    (dict(q_stride_token=128), E_STRIDE),
    (dict(o_stride_head=0), E_STRIDE),
    (dict(kv_stride_kv=64), E_STRIDE),
    (dict(kv_stride_slot=-256), E_STRIDE),
    (dict(bt_stride=8), E_STRIDE),
])
def test_invalid_dims_rejected(pa, kw, expect):
    assert call(pa, dims(**kw)) == expect


def test_null_dims(pa):
    assert call(pa, None) == E_NULL


@pytest.mark.parametrize("which", ["out", "q", "kv", "bt", "sl", "cq"])
def test_null_pointers(pa, which):
    assert call(pa, dims(), **{which: None}) == E_NULL


@pytest.mark.parametrize("which,val", [("out", FAKE + 2), ("q", FAKE + 8), ("kv", FAKE + 4),
                                       ("bt", FAKE + 1), ("sl", FAKE + 2), ("cq", FAKE + 3)])
def test_misaligned_pointers(pa, which, val):
    assert call(pa, dims(), **{which: val}) == E_ALIGN


def test_bad_sizes(pa):
    assert call(pa, dims(), n_seqs=-1) == E_SHAPE
    assert call(pa, dims(), n_seqs=70000) == E_SHAPE
    assert call(pa, dims(), max_q=0) == E_SHAPE
    assert call(pa, dims(), max_q=65) == E_SHAPE         # > num_tokens
    assert call(pa, dims(), scale=float("nan")) == E_SHAPE
    assert call(pa, dims(), scale=float("inf")) == E_SHAPE
    assert call(pa, dims(), path=7) == E_SHAPE
    assert call(pa, dims(), pps=-1) == E_SHAPE


def test_forced_split_path_row_limit(pa):
    # G = 4; max_q = 17 -> 68 packed rows > 64 (four blocks of 16): the split
    # kernels cannot take it; up to 64 rows they plan (the short-sequence body)
    assert call(pa, dims(), max_q=17, path=1) == E_UNSUP
    assert call(pa, dims(), max_q=17, path=4) == E_UNSUP
    import paged_kv_gqa_fwd_amd as mod
    for mq in (1, 4, 5, 8, 9, 16):
        p = mod.make_plan(dims(), 4, mq, mod.PATH_AUTO)
        assert p.path == mod.PATH_SPLIT_BALANCED, (mq, p.path)
    assert mod.make_plan(dims(), 4, 17, mod.PATH_AUTO).path == mod.PATH_PREFILL


def test_workspace_checks(pa):
    import paged_kv_gqa_fwd_amd as mod
    d = dims(max_pages_per_seq=128, bt_stride=128)
    plan = mod.make_plan(d, 64, 1, mod.PATH_SPLIT_FUSED)
    assert plan.path == mod.PATH_SPLIT_FUSED and plan.max_splits > 1 and plan.workspace_bytes > 0
    assert call(pa, d, n_seqs=64, path=3) == E_WS                           # missing
    assert call(pa, d, n_seqs=64, path=3, ws=FAKE + 16, ws_bytes=1 << 30) == E_WS   # misaligned
    assert call(pa, d, n_seqs=64, path=3, ws=FAKE, ws_bytes=plan.workspace_bytes - 1) == E_WS
    assert call(pa, d, n_seqs=64) == E_WS             # the two-kernel split path needs one too


def test_zero_sequences_is_noop(pa):
    assert call(pa, dims(), n_seqs=0, out=None, q=None) == OK


def test_plan_paths_and_sizes(pa):
    import paged_kv_gqa_fwd_amd as mod
    # decode batch: 64 seqs, G=4, MP=128 -> split decode
    d = dims(max_pages_per_seq=128, bt_stride=128)
    assert mod.make_plan(d, 64, 1).path == mod.PATH_SPLIT_BALANCED
    p = mod.make_plan(d, 64, 1, mod.PATH_SPLIT_FUSED)
    assert p.path == mod.PATH_SPLIT_FUSED
    assert p.grid_z == p.max_splits and p.grid_x == 8 and p.grid_y == 64
    assert p.max_splits == -(-128 // p.pages_per_split)
    rows = 64 * 1 * 32 * p.max_splits
    # one i32 merge counter per (sequence, KV head), ahead of the partials
    assert p.counter_bytes == 64 * 8 * 4
    assert p.workspace_bytes >= p.counter_bytes + rows * 128 * 4 + rows * 8
    # the two-kernel split path: same splits, no counters
    pc = mod.make_plan(d, 64, 1, mod.PATH_SPLIT_DECODE)
    assert pc.path == mod.PATH_SPLIT_DECODE and pc.counter_bytes == 0
    assert (pc.pages_per_split, pc.max_splits) == (p.pages_per_split, p.max_splits)
    assert pc.workspace_bytes == p.workspace_bytes - p.counter_bytes
    # counters round up to 256 bytes
    assert mod.make_plan(d, 3, 1, mod.PATH_SPLIT_FUSED).counter_bytes == 256
    # many query rows -> prefill, no workspace
    d2 = dims(num_q_heads=24, num_kv_heads=4, head_dim=256, q_stride_token=24 * 256,
              q_stride_head=256, o_stride_token=24 * 256, o_stride_head=256, num_tokens=4096,
              kv_stride_page=64 * 4 * 2 * 256, kv_stride_slot=4 * 2 * 256, kv_stride_head=512,
              kv_stride_kv=256, max_pages_per_seq=192, bt_stride=192)
    p2 = mod.make_plan(d2, 8, 4096)
    assert p2.path == mod.PATH_PREFILL
    assert p2.grid_x == -(-4096 * 6 // 128) and p2.grid_y == 4 and p2.grid_z == 8
    # ... except the launch-order table of a ragged batch: one i32 per
    # workgroup, 256-byte aligned, from 512 workgroups and two sequences up
    assert p2.workspace_bytes == -(-p2.grid_x * 4 * 8 * 4 // 256) * 256
    assert mod.make_plan(d2, 1, 4096).workspace_bytes == 0          # one sequence: grid order
    p5 = mod.make_plan(d2, 2, 63 * 128 // 6)                       # 63 tiles x 4 x 2 = 504 ...
    assert p5.grid_x == 63 and p5.workspace_bytes == 0
    p5 = mod.make_plan(d2, 2, 63 * 128 // 6 + 1)                   # ... 64 tiles: 512 workgroups
    assert p5.grid_x == 64 and p5.workspace_bytes == 2048
    # forced split sizes are clamped to [1, MP]
    p3 = mod.make_plan(d, 64, 1, mod.PATH_SPLIT_DECODE, 1000)
    assert p3.pages_per_split == 128 and p3.max_splits == 1 and p3.workspace_bytes == 0
    p3f = mod.make_plan(d, 64, 1, mod.PATH_SPLIT_FUSED, 1000)
    assert p3f.max_splits == 1 and p3f.workspace_bytes == 0 and p3f.counter_bytes == 0
    p4 = mod.make_plan(d, 64, 1, mod.PATH_SPLIT_DECODE, 3)
    assert p4.pages_per_split == 3 and p4.max_splits == 43
    # long decode: 128 seqs x 512 pages, 2 KV heads -> about four rounds of workgroups
    # (1024 resident on 256 CUs at one per CU) from the splits
    d5 = dims(num_q_heads=16, num_kv_heads=2, head_dim=256, q_stride_token=16 * 256, q_stride_head=256,
              o_stride_token=16 * 256, o_stride_head=256, kv_stride_page=64 * 2 * 2 * 256,
              kv_stride_slot=2 * 2 * 256, kv_stride_head=512, kv_stride_kv=256,
              max_pages_per_seq=512, bt_stride=512, num_tokens=128)
    p5 = mod.make_plan(d5, 128, 1, mod.PATH_SPLIT_DECODE)
    assert p5.path == mod.PATH_SPLIT_DECODE and p5.grid_z * 2 * 128 >= 4 * 256


def test_prefill_rejects_slot_strides_past_32_bit_offsets(pa):
    """The prefill kernel addresses the 64 slots of a page with 32-bit byte
    offsets from the page base: a slot stride with (63 * stride + D) * 2 past
    2^32 - 1 is refused on that path (nothing launched), while the split-decode
    paths (64-bit addressing) still plan it.  A slot-outermost pool over many
    pages is such a layout."""
    import paged_kv_gqa_fwd_amd as mod
    D, hkv, hq = 128, 8, 32
    limit = ((1 << 32) - 1) // 2            # (63 s + D) <= limit elements
    s_ok = (limit - D) // 63 // 8 * 8       # largest multiple of 8 that fits
    s_bad = s_ok + 8
    assert (63 * s_ok + D) * 2 <= (1 << 32) - 1 < (63 * s_bad + D) * 2
    for s, expect in ((s_ok, OK), (s_bad, E_UNSUP)):
        d = dims(num_q_heads=hq, num_kv_heads=hkv, head_dim=D, kv_stride_slot=s, kv_stride_page=8,
                 kv_stride_head=2 * D, kv_stride_kv=D, num_tokens=4096)
        plan = mod.attn_paged_plan()
        opt = mod.attn_paged_options(None, 0, mod.PATH_PREFILL, 0, 0, 1.0, 1.0)
        rc = pa.load_library().attn_paged_make_plan_opt(ctypes.byref(d), 4, 64, ctypes.byref(opt),
                                                       ctypes.byref(plan))
        assert rc == expect, (s, rc)
        if expect != OK:
            # AUTO takes prefill for 64 tokens x G 4 > 64 rows: the call is refused
            # before any launch
            assert call(pa, d, n_seqs=4, max_q=64) == E_UNSUP
        # decode-shaped calls keep their 64-bit split path
        assert mod.make_plan(d, 4, 1).path == mod.PATH_SPLIT_BALANCED


def test_plan_balanced(pa):
    import paged_kv_gqa_fwd_amd as mod
    d = dims(max_pages_per_seq=128, bt_stride=128)        # 32/8 heads, D 128
    p = mod.make_plan(d, 64, 1)
    # one round of resident workgroups: 256 CUs x 2 per CU over 8 KV heads
    assert p.path == mod.PATH_SPLIT_BALANCED and (p.grid_x, p.grid_y, p.grid_z) == (8, 64, 1)
    assert p.counter_bytes == 0
    # pieces per sequence bounded by floor((MP - 1) / C_min) + 2
    assert p.max_splits == 127 // p.pages_per_split + 2
    rows = 64 * 32 * p.max_splits
    assert p.workspace_bytes == 256 + rows * 128 * 4 + rows * 8
    # the least range size caps the partials at 64 MiB plus one split's worth
    assert p.max_splits * 64 * 32 * 130 * 4 <= (64 << 20) + 64 * 32 * 130 * 4
    # a forced least range size
    p7 = mod.make_plan(d, 64, 1, mod.PATH_SPLIT_BALANCED, 7)
    assert p7.pages_per_split == 7 and p7.max_splits == 127 // 7 + 2
    # AUTO with a forced split size keeps the fixed-size split path
    assert mod.make_plan(d, 64, 1, mod.PATH_AUTO, 16).path == mod.PATH_SPLIT_DECODE
    # more than 1024 sequences: the fixed-size split path; forcing balanced is unsupported
    d_big = dims(max_pages_per_seq=128, bt_stride=128, num_tokens=2048)
    assert mod.make_plan(d_big, 1025, 1).path == mod.PATH_SPLIT_DECODE
    assert mod.make_plan(d_big, 1024, 1).path == mod.PATH_SPLIT_BALANCED
    lib = pa.load_library()
    plan = mod.attn_paged_plan()
    assert lib.attn_paged_make_plan(ctypes.byref(d_big), 1025, 1, mod.PATH_SPLIT_BALANCED, 0,
                                    ctypes.byref(plan)) == E_UNSUP
    # long decode, 2 KV heads at D 256 (one workgroup per CU): 128 ranges
    d5 = dims(num_q_heads=16, num_kv_heads=2, head_dim=256, q_stride_token=16 * 256, q_stride_head=256,
              o_stride_token=16 * 256, o_stride_head=256, kv_stride_page=64 * 2 * 2 * 256,
              kv_stride_slot=2 * 2 * 256, kv_stride_head=512, kv_stride_kv=256,
              max_pages_per_seq=512, bt_stride=512, num_tokens=128)
    p5 = mod.make_plan(d5, 128, 1)
    assert p5.path == mod.PATH_SPLIT_BALANCED and (p5.grid_x, p5.grid_y) == (2, 128)
    assert p5.max_splits == 511 // p5.pages_per_split + 2
    # with a window only the pages from row 0's window start count
    pw = mod.make_plan(d5, 128, 1, window=4096)
    mp_w = (4096 + 1 + 62) // 64 + 1      # 65 pages from row 0's window start
    assert pw.max_splits == (mp_w - 1) // pw.pages_per_split + 2
    # more packed rows than four 16-row MFMA blocks -> prefill
    assert mod.make_plan(d, 64, 16).path == mod.PATH_SPLIT_BALANCED   # 64 packed rows: the short body
    assert mod.make_plan(d, 64, 17).path == mod.PATH_PREFILL


def test_workspace_bytes_query(pa):
    lib = pa.load_library()
    n = ctypes.c_size_t(0)
    d = dims(max_pages_per_seq=128, bt_stride=128)
    assert lib.attn_paged_workspace_bytes(ctypes.byref(d), 64, 1, ctypes.byref(n)) == OK
    assert n.value == pa.make_plan(d, 64, 1).workspace_bytes
    assert lib.attn_paged_workspace_bytes(ctypes.byref(d), 64, 1, None) == E_NULL


def _nd(pa, ks=(8 * 128, 128), vs=(8 * 128, 128)):
    import paged_kv_gqa_fwd_amd as mod
    return mod.attn_kv_new_dims(ks[0], ks[1], vs[0], vs[1])


def test_kv_write_validates_before_launch(pa):
    lib = pa.load_library()
    d = dims()   # 32 q / 8 KV heads, D 128
    F = FAKE

    def w(nd, n_seqs=4, kv=F, k=F, v=F, max_q=1):
        return lib.attn_paged_kv_write(kv, k, v, F, F, F, n_seqs, max_q, ctypes.byref(d),
                                       ctypes.byref(nd) if nd is not None else None, None)
    assert w(None) == E_NULL
    assert w(_nd(pa, ks=(8 * 128, 100))) == E_STRIDE         # head stride not a multiple of 8
    assert w(_nd(pa, ks=(8 * 128, 64))) == E_STRIDE          # rows shorter than D
    assert w(_nd(pa, vs=(4 * 128, 128))) == E_STRIDE         # heads of a token overlap the next token
    assert w(_nd(pa), k=None) == E_NULL
    assert w(_nd(pa), v=F + 8) == E_ALIGN
    assert w(_nd(pa), max_q=0) == E_SHAPE
    assert w(_nd(pa), n_seqs=0, kv=None, k=None, v=None) == OK   # nothing to write


def test_fwd_write_validates_both_steps(pa):
    lib = pa.load_library()
    d = dims()
    F = FAKE

    def fw(nd, scale=0.1, out=F, ws=None, ws_bytes=0, n_seqs=4):
        return lib.attn_paged_fwd_write(out, F, F, F, F, F, F, F, n_seqs, 1, scale, 1, ctypes.byref(d),
                                        ctypes.byref(nd) if nd is not None else None, ws, ws_bytes, None)
    assert fw(None) == E_NULL                       # write step
    assert fw(_nd(pa), scale=float("nan")) == E_SHAPE   # attention step
    assert fw(_nd(pa), out=None) == E_NULL
    assert fw(_nd(pa), out=F + 2) == E_ALIGN


def test_options_validate_and_shrink_the_split_plan(pa):
    import paged_kv_gqa_fwd_amd as mod
    lib = pa.load_library()
    d = dims(max_pages_per_seq=128, bt_stride=128)
    plan = mod.attn_paged_plan()

    def opt(sinks=None, window=0, path=0, pps=0):
        return mod.attn_paged_options(sinks, window, path, pps)

    def fo(o, ws=None, ws_bytes=0):
        return lib.attn_paged_fwd_opt(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 64, 1, 0.1, 1, ctypes.byref(d),
                                      ctypes.byref(o) if o is not None else None, ws, ws_bytes, None)
    assert fo(None) == E_NULL
    assert lib.attn_paged_make_plan_opt(ctypes.byref(d), 64, 1, None, ctypes.byref(plan)) == E_NULL
    assert fo(opt(window=-1)) == E_SHAPE
    assert fo(opt(sinks=FAKE + 2), ws=FAKE, ws_bytes=1 << 30) == E_ALIGN
    # a window shrinks the pages each sequence's splits must cover
    full = mod.make_plan(d, 64, 1)
    win = mod.make_plan(d, 64, 1, window=256)     # rows see <= 256 keys: <= 5 pages from row 0's start
    assert win.max_splits * win.pages_per_split >= 5 and win.max_splits * win.pages_per_split < 128
    assert win.workspace_bytes < full.workspace_bytes
    # windows that reach past every key a table can hold change nothing
    same = mod.make_plan(d, 64, 1, window=128 * 64)
    assert (same.pages_per_split, same.max_splits, same.workspace_bytes) == \
        (full.pages_per_split, full.max_splits, full.workspace_bytes)


def test_fp8_cache_options_validate(pa):
    import paged_kv_gqa_fwd_amd as mod
    lib = pa.load_library()
    d = dims(max_pages_per_seq=128, bt_stride=128)   # kv strides: multiples of 16
    plan = mod.attn_paged_plan()

    def mp(o, dd=d, max_q=1):
        return lib.attn_paged_make_plan_opt(ctypes.byref(dd), 64, max_q, ctypes.byref(o), ctypes.byref(plan))

    def fo(o):
        return lib.attn_paged_fwd_opt(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 64, 1, 0.1, 1, ctypes.byref(d),
                                      ctypes.byref(o), FAKE, 1 << 30, None)
    f8 = lambda **kw: mod.attn_paged_options(kw.get("sinks"), kw.get("window", 0), kw.get("path", 0),
                                             kw.get("pps", 0), kw.get("dtype", 1), kw.get("ks", 1.0),
                                             kw.get("vs", 1.0))
    assert mp(f8()) == OK and plan.path == mod.PATH_SPLIT_BALANCED
    assert mp(f8(dtype=2)) == E_UNSUP
    assert mp(f8(), max_q=16) == OK                         # 64 packed rows: the short-sequence body
    # more rows take the prefill kernel, which reads the pages through a bf16
    # staging pool in the workspace: 64 seqs x 128 pages x 64 slots x 8 heads
    # x 2 x D 128 bf16, plus one i32 table entry per page, then the launch
    # order of the 1 x 8 x 64 workgroups
    for kw in (dict(path=2), dict()):
        assert mp(f8(**kw), max_q=17) == OK and plan.path == mod.PATH_PREFILL
        pages = 64 * 128
        assert plan.workspace_bytes == pages * 64 * 8 * 2 * 128 * 2 + pages * 4 + 512 * 4
    bf = mod.attn_paged_options(None, 0, 2, 0, 0, 1.0, 1.0)
    assert mp(bf) == OK and plan.workspace_bytes == 512 * 4  # a bf16 prefill: only the launch order
    assert mp(bf, dd=dims(max_pages_per_seq=128, bt_stride=128, num_kv_heads=4)) == OK
    assert plan.workspace_bytes == 0                        # 256 workgroups: grid order, no workspace
    assert mp(f8(), dd=dims(max_pages_per_seq=128, bt_stride=128, kv_stride_kv=136)) == E_STRIDE
    assert fo(f8(ks=float("inf"))) == E_SHAPE
    assert fo(f8(vs=float("nan"))) == E_SHAPE
    # a bf16 cache ignores the scales (a zeroed options struct stays valid)
    assert mp(mod.attn_paged_options(None, 0, 0, 0, 0, 0.0, 0.0)) == OK
    # the quantising write needs finite, nonzero scales
    nd = mod.attn_kv_new_dims(8 * 128, 128, 8 * 128, 128)
    for bad in (f8(ks=0.0), f8(vs=float("inf"))):
        assert lib.attn_paged_kv_write_opt(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 1, ctypes.byref(d),
                                           ctypes.byref(nd), ctypes.byref(bad), None) == E_SHAPE
    assert lib.attn_paged_kv_write_opt(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 1, ctypes.byref(d),
                                       ctypes.byref(nd), None, None) == E_NULL


def test_workspace_clear_validates(pa):
    lib = pa.load_library()
    assert lib.attn_workspace_clear(None, 0, None) == OK          # nothing to do
    assert lib.attn_workspace_clear(None, 256, None) == E_NULL
    assert lib.attn_workspace_clear(0x1002, 256, None) == E_ALIGN
    assert lib.attn_workspace_clear(0x1000, 6, None) == E_SHAPE


def test_status_strings(pa):
    lib = pa.load_library()
    for s in (OK, E_NULL, E_SHAPE, E_UNSUP, E_STRIDE, E_ALIGN, E_WS, E_HIP, 12345):
        assert lib.attn_status_string(s)
    assert lib.attn_version() >= 10000


def test_python_binding_refuses_cpu_tensors(pa):
    import torch
    q = torch.zeros(1, 8, 128, dtype=torch.bfloat16)
    kv = torch.zeros(2, 64, 2, 2, 128, dtype=torch.bfloat16)
    bt = torch.zeros(1, 2, dtype=torch.int32)
    with pytest.raises(ValueError):
        pa.paged_attention(q, kv, bt, torch.ones(1, dtype=torch.int32),
                           torch.tensor([0, 1], dtype=torch.int32), 1, 0.1)


# ---------------------------------------------------------------- quantised path
def _qdims(pa, B=1, N=300, H=2, D=128):
    d = pa.attn_quant_dims(batch=B, seq_len=N, num_heads=H, head_dim=D)
    for f in ("q_stride", "k_stride", "v_stride", "o_stride"):
        arr = getattr(d, f)
        arr[0], arr[1], arr[2] = N * H * D, H * D, D
    return d


def test_quant_layout_sizes(pa):
    import ctypes
    d = _qdims(pa)
    lay = pa.attn_quant_layout()
    assert pa.load_library().attn_quant_layout_of(ctypes.byref(d), ctypes.byref(lay)) == 0
    assert lay.blocks == 5 and lay.chunks == 2 and lay.vt_stride == 320
    offs = [lay.off_mk, lay.off_sv, lay.off_sq, lay.off_sk, lay.off_qi, lay.off_ki, lay.off_vt,
            lay.off_ksum, lay.off_vmax]
    assert all(o % 256 == 0 for o in offs) and offs == sorted(offs)
    # every region fits before the next one and inside the workspace
    sizes = [2 * 128 * 4, 2 * 128 * 4, 2 * 5 * 4, 2 * 5 * 4, 300 * 2 * 128, 300 * 2 * 128,
             2 * 128 * 320, 2 * 2 * 128 * 8, 2 * 2 * 128 * 4]
    ends = [o + s for o, s in zip(offs, sizes)]
    assert all(e <= n for e, n in zip(ends, offs[1:] + [lay.workspace_bytes]))


@pytest.mark.parametrize("field,value,status", [
    ("head_dim", 256, -3), ("seq_len", 0, -2), ("num_heads", 0, -2), ("batch", 40000, -2)])
def test_quant_layout_rejects(pa, field, value, status):
    import ctypes
    d = _qdims(pa)
    setattr(d, field, value)
    lay = pa.attn_quant_layout()
    assert pa.load_library().attn_quant_layout_of(ctypes.byref(d), ctypes.byref(lay)) == status


def test_quant_layout_rejects_bad_strides(pa):
    import ctypes
    d = _qdims(pa)
    d.k_stride[1] = 100          # not a multiple of 8
    lay = pa.attn_quant_layout()
    assert pa.load_library().attn_quant_layout_of(ctypes.byref(d), ctypes.byref(lay)) == -4
    d = _qdims(pa)
    d.o_stride[2] = 64           # heads overlap
    assert pa.load_library().attn_quant_layout_of(ctypes.byref(d), ctypes.byref(lay)) == -4


def test_quant_calls_validate_before_launch(pa):
    import ctypes
    lib = pa.load_library()
    d = _qdims(pa)
    # workspace missing / too small / misaligned: rejected on the host
    assert lib.attn_quant_fwd(0x1000, 0x1000, 0x1000, 0x1000, ctypes.byref(d), 0.1, 0, None, 0, None) == -6
    assert lib.attn_quant_prep(0x1000, 0x1000, 0x1000, ctypes.byref(d), 0x1000, 16, None) == -6
    assert lib.attn_quant_attend(0x1000, ctypes.byref(d), 0.1, 0, 0x1008, 1 << 30, None) == -6
    # null and misaligned tensors
    assert lib.attn_quant_fwd(None, 0x1000, 0x1000, 0x1000, ctypes.byref(d), 0.1, 0, 0x1000, 1 << 30, None) == -1
    assert lib.attn_quant_fwd(0x1008, 0x1000, 0x1000, 0x1000, ctypes.byref(d), 0.1, 0, 0x1000, 1 << 30, None) == -5
    # non-finite scale
    assert lib.attn_quant_fwd(0x1000, 0x1000, 0x1000, 0x1000, ctypes.byref(d), float("nan"), 0, 0x1000, 1 << 30, None) == -2


def test_stream_read_validation(pa):
    lib = pa.load_library()
    assert lib.attn_stream_read(None, 16, FAKE, 1, 4, None) == E_NULL
    assert lib.attn_stream_read(FAKE, 16, None, 1, 4, None) == E_NULL
    assert lib.attn_stream_read(FAKE + 8, 16, FAKE, 1, 4, None) == E_ALIGN     # buffer not 16-byte aligned
    assert lib.attn_stream_read(FAKE, 24, FAKE, 1, 4, None) == E_ALIGN         # not a multiple of 16 bytes
    assert lib.attn_stream_read(FAKE, 16, FAKE + 2, 1, 4, None) == E_ALIGN     # sink not 4-byte aligned
    assert lib.attn_stream_read(FAKE, 16, FAKE, 0, 4, None) == E_SHAPE
    assert lib.attn_stream_read(FAKE, 16, FAKE, 65536, 4, None) == E_SHAPE
    assert lib.attn_stream_read(FAKE, 16, FAKE, 1, 6, None) == E_SHAPE        # depth 4 or 8
    assert lib.attn_stream_read(FAKE, 0, FAKE, 1, 8, None) == OK               # nothing to read: no launch


def test_noalloc_validates_before_any_hip_call(pa):
    """attn_paged_fwd_noalloc: argument errors and plans whose partials exceed
    the scratch array are refused on the host, before any HIP call (so these
    run without a GPU); n_seqs = 0 is a no-op."""
    import paged_kv_gqa_fwd_amd as mod
    lib = pa.load_library()

    def noalloc(d, n_seqs=4, max_q=1, opt=None, **ptrs):
        p = dict(out=FAKE, q=FAKE, kv=FAKE, bt=FAKE, sl=FAKE, cq=FAKE)
        p.update(ptrs)
        return lib.attn_paged_fwd_noalloc(p["out"], p["q"], p["kv"], p["bt"], p["sl"], p["cq"], n_seqs, max_q,
                                          0.1, 1, ctypes.byref(d) if d is not None else None,
                                          ctypes.byref(opt) if opt is not None else None, None)

    assert noalloc(None) == E_NULL
    assert noalloc(dims(head_dim=64)) == E_UNSUP
    assert noalloc(dims(q_stride_head=100)) == E_STRIDE
    assert noalloc(dims(), q=None) == E_NULL
    assert noalloc(dims(), out=FAKE + 2) == E_ALIGN
    assert noalloc(dims(), n_seqs=0, out=None, q=None) == OK
    # 1024 sequences x 32 heads x 16 one-page splits x D 128 of f32 partials
    # (256 MiB) cannot fit the 64 MiB array
    big = dims(max_pages_per_seq=16, bt_stride=16, num_tokens=1024)
    opt = mod.attn_paged_options(None, 0, mod.PATH_SPLIT_DECODE, 1, 0, 1.0, 1.0)
    assert mod.make_plan(big, 1024, 1, mod.PATH_SPLIT_DECODE, 1).workspace_bytes > mod.NOALLOC_SCRATCH_BYTES
    assert noalloc(big, n_seqs=1024, opt=opt) == E_WS


def test_prefill_split_plan(pa):
    """Split-key prefill plans (host logic): a grid of at most 128 items has
    its keys split into floor(256 / items) runs of the split-decode layout,
    page runs rounded to a ring tile (two pages at head_dim 128), with the
    partials in the workspace; a forced pages_per_split on the prefill path
    splits any grid; a window bounds the pages a split layout covers."""
    import paged_kv_gqa_fwd_amd as mod
    # 2 seqs x 32 tokens, 24 / 4 heads, D 256: 2 tiles x 4 x 2 = 16 items, MP 11
    d = dims(num_q_heads=24, num_kv_heads=4, head_dim=256, q_stride_token=24 * 256, q_stride_head=256,
             o_stride_token=24 * 256, o_stride_head=256, num_tokens=64, kv_stride_page=64 * 4 * 2 * 256,
             kv_stride_slot=4 * 2 * 256, kv_stride_head=512, kv_stride_kv=256, max_pages_per_seq=11, bt_stride=11)
    p = mod.make_plan(d, 2, 32)
    assert p.path == mod.PATH_PREFILL and p.max_splits == 11 and p.pages_per_split == 1
    assert (p.grid_x, p.grid_y, p.grid_z) == (2 * 11, 4, 2)
    rows = 2 * 32 * 24 * 11
    assert p.workspace_bytes == -(-rows * 256 * 4 // 256) * 256 + -(-rows * 8 // 256) * 256
    # forced: 3 pages per split -> ceil(11 / 3) = 4 splits; one split past every page -> one pass
    p3 = mod.make_plan(d, 2, 32, mod.PATH_PREFILL, 3)
    assert (p3.max_splits, p3.pages_per_split, p3.grid_x) == (4, 3, 8)
    p1 = mod.make_plan(d, 2, 32, mod.PATH_PREFILL, 1 << 30)
    assert (p1.max_splits, p1.grid_x, p1.workspace_bytes) == (1, 2, 0)
    # a window of 64 keys: rows reach (64 + 32 + 62) // 64 + 1 = 3 pages -> 3 splits of one page
    pw = mod.make_plan(d, 2, 32, mod.PATH_AUTO, 0, 64)
    assert pw.max_splits == 3 and pw.pages_per_split == 1
    # head_dim 128 (tiles of 2 pages): 16 seqs x 17 tokens x G 4 = 68 rows = 1 tile x 8 heads x 16 seqs
    # = 128 items, MP 31: 2 splits of 16 pages (15.5 rounded up to a tile)
    d2 = dims(max_pages_per_seq=31, bt_stride=31, num_tokens=16 * 17)
    p2 = mod.make_plan(d2, 16, 17)
    assert p2.path == mod.PATH_PREFILL and p2.max_splits == 2 and p2.pages_per_split == 16 and p2.grid_x == 2
    # 129 items and more: one pass
    p4 = mod.make_plan(dims(max_pages_per_seq=31, bt_stride=31, num_tokens=17 * 17), 17, 17)
    assert p4.path == mod.PATH_PREFILL and p4.max_splits == 1 and p4.grid_x == 1
