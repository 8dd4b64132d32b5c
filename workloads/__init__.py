"""Seeded synthetic inputs for paged grouped-query attention.

This module only draws inputs: sequence lengths, page assignments, Q, the
paged K/V pool and the perturbations named by each workload.  It holds none of
the attention arithmetic, so both the HIP path and the CPU oracle can be fed
from it without sharing any of the method's code.

Draw order (fixed, so every workload is reproducible from its seed):
  lengths -> page permutation -> Q -> pool K/V -> perturbations
(perturbations = K outlier rows, per-channel K offsets).  Lengths and the page
permutation always come from a CPU ``torch.Generator``; Q and the pool come
from a generator on ``device`` seeded with the same seed, so the lengths and
page tables are identical whichever device draws the values.  Values are
float32 ``randn`` rounded to bfloat16 (round-to-nearest-even).

Pool layout: ``[num_pages, page_size, num_kv_heads, 2, head_dim]`` with index
3 selecting K (0) or V (1) -- the decode.json manifest's ``kv`` buffer
(kern-kernels examples, buffers.kv) with its layer axis taken out.  The tiny
mixed workload keeps that manifest's two-layer pool and uses layer 1, as its
``programs.decode`` call does (K at +262144 bytes, V at +262656 bytes).
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import torch

PAGE_SIZE = 64


@dataclasses.dataclass
class PagedCase:
    name: str
    q: torch.Tensor             # bf16 [T, Hq, D]
    pool_storage: torch.Tensor  # bf16, the whole allocation
    kv: torch.Tensor            # bf16 [NP, P, Hkv, 2, D] view into pool_storage
    block_table: torch.Tensor   # int32 [B, MP]
    seq_lens: torch.Tensor      # int32 [B]
    cu_q: torch.Tensor          # int32 [B + 1]
    q_lens: List[int]
    kv_lens: List[int]
    scale: float
    causal: bool
    seed: int

    @property
    def n_seqs(self) -> int:
        return len(self.kv_lens)

    @property
    def max_q(self) -> int:
        return max(self.q_lens) if self.q_lens else 0

    @property
    def num_q_heads(self) -> int:
        return self.q.shape[1]

    @property
    def num_kv_heads(self) -> int:
        return self.kv.shape[2]

    @property
    def head_dim(self) -> int:
        return self.q.shape[2]

    def to(self, device) -> "PagedCase":
        """Copy every tensor to ``device`` keeping the pool's strides."""
        storage = self.pool_storage.to(device)
        kv = storage.as_strided(self.kv.shape, self.kv.stride(),
                                self.kv.storage_offset() - self.pool_storage.storage_offset())
        return dataclasses.replace(
            self, q=self.q.to(device), pool_storage=storage, kv=kv,
            block_table=self.block_table.to(device), seq_lens=self.seq_lens.to(device),
            cu_q=self.cu_q.to(device))

    def kv_bytes(self) -> int:
        """K and V bytes that one pass must read (each visible key once per KV head)."""
        hkv, d = self.num_kv_heads, self.head_dim
        return sum(self.kv_lens) * hkv * 2 * d * 2


def _randn_bf16(shape, gen, device, chunk_rows: int = 1024, add=None) -> torch.Tensor:
    """float32 N(0,1) rounded to bf16, drawn in row chunks to bound peak memory."""
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(shape[0], -1)
    for r0 in range(0, shape[0], chunk_rows):
        r1 = min(shape[0], r0 + chunk_rows)
        x = torch.randn((r1 - r0, flat.shape[1]), generator=gen, device=device, dtype=torch.float32)
        if add is not None:
            x = (x.view((r1 - r0,) + tuple(shape[1:])) + add).view(r1 - r0, -1)
        flat[r0:r1] = x.to(torch.bfloat16)
    return out


def make_case(name: str, seed: int, q_lens, kv_lens, num_q_heads: int, num_kv_heads: int,
              head_dim: int, causal: bool = True, scale: Optional[float] = None,
              page_size: int = PAGE_SIZE, table_cols: Optional[int] = None, extra_pages: int = 0,
              table_fill: str = "neg1", layers: int = 1, layer: int = 0,
              k_outlier_p: float = 0.0, k_outlier_mult: float = 4.0,
              k_channel_offset_var: float = 0.0, poison: bool = False,
              device="cpu", num_pages: Optional[int] = None, chunk_pages: int = 1024,
              layout: str = "slot_major") -> PagedCase:
    """Build one seeded paged-attention input.

    q_lens / kv_lens: per-sequence new-query counts n_b and total KV lengths
    L_b (L_b counts the step's own tokens; queries sit at the tail).
    table_fill: "neg1" puts -1 in unused block-table columns, "valid" fills
    the whole table from the page permutation (the manifest's full table).
    poison: fill unused pool pages and the slots past L_b in each sequence's
    last page with NaN / +-inf (a correct kernel never lets them reach the
    output: it skips them, masks their scores or zeroes their V rows).
    layout: "slot_major" stores [page, layer, slot, kv_head, {K,V}, D] (the
    decode.json manifest's order); "head_major" stores [page, kv_head, {K,V},
    slot, D], so each (page, KV head) is one contiguous K block followed by
    its V block.  Either way ``kv`` is the [page, slot, kv_head, {K,V}, D] view.
    """
    cpu_gen = torch.Generator(device="cpu").manual_seed(seed)
    q_lens = [int(x) for x in q_lens]
    kv_lens = [int(x) for x in kv_lens]
    B = len(kv_lens)
    assert len(q_lens) == B
    for n, L in zip(q_lens, kv_lens):
        assert 0 <= n and 0 <= L
    pages_needed = [math.ceil(L / page_size) for L in kv_lens]
    mp = table_cols if table_cols is not None else max([1] + pages_needed)
    assert all(p <= mp for p in pages_needed)
    used = sum(pages_needed)
    if table_fill == "valid":
        np_total = num_pages if num_pages is not None else B * mp
        assert np_total >= B * mp
    else:
        np_total = num_pages if num_pages is not None else used + extra_pages
        assert np_total >= used
    # page permutation (second draw)
    perm = torch.randperm(np_total, generator=cpu_gen).to(torch.int32)
    table = torch.full((B, mp), -1, dtype=torch.int32)
    if table_fill == "valid":
        table[:] = perm[: B * mp].view(B, mp)
    else:
        off = 0
        for b, npg in enumerate(pages_needed):
            table[b, :npg] = perm[off: off + npg]
            off += npg
    hq, hkv, d = num_q_heads, num_kv_heads, head_dim
    T = sum(q_lens)
    dev_gen = torch.Generator(device=device).manual_seed(seed)
    q = _randn_bf16((max(T, 1), hq, d), dev_gen, device)[:T] if T > 0 else \
        torch.empty((0, hq, d), dtype=torch.bfloat16, device=device)
    # pool K/V, optionally with a per-(kv head, channel) K offset added before rounding
    offset = None
    if k_channel_offset_var > 0:
        off_gen = torch.Generator(device="cpu").manual_seed(seed + 7919)
        offset = torch.randn((hkv, d), generator=off_gen) * math.sqrt(k_channel_offset_var)
        kv_off = torch.zeros((1, hkv, 2, d))
        kv_off[0, :, 0, :] = offset
        offset_dev = kv_off.to(device)
    if layout == "slot_major":
        storage = torch.empty((np_total, layers, page_size, hkv, 2, d), dtype=torch.bfloat16, device=device)
        layer_views = [storage[:, l] for l in range(layers)]
    elif layout == "head_major":
        assert layers == 1
        storage = torch.empty((np_total, hkv, 2, page_size, d), dtype=torch.bfloat16, device=device)
        layer_views = [storage.permute(0, 3, 1, 2, 4)]
    else:
        raise ValueError("unknown layout %r" % layout)
    for l in range(layers):
        for p0 in range(0, np_total, chunk_pages):
            p1 = min(np_total, p0 + chunk_pages)
            vals = _randn_bf16((p1 - p0, page_size, hkv, 2, d), dev_gen, device, chunk_rows=p1 - p0,
                               add=offset_dev if (offset is not None and l == layer) else None)
            layer_views[l][p0:p1] = vals
    kv = layer_views[layer]
    if k_outlier_p > 0:
        # Bernoulli per pool slot: every page belongs to one sequence, so this is
        # an independent draw per (sequence, position); all KV heads' K rows scale.
        mask_gen = torch.Generator(device="cpu").manual_seed(seed + 104729)
        mask = torch.rand((np_total, page_size), generator=mask_gen) < k_outlier_p
        idx = mask.nonzero().to(device)
        if idx.numel():
            sel = kv[idx[:, 0], idx[:, 1], :, 0, :].float() * k_outlier_mult
            kv[idx[:, 0], idx[:, 1], :, 0, :] = sel.to(torch.bfloat16)
    if poison:
        used_pages = set()
        tb = table.tolist()
        for b, npg in enumerate(pages_needed):
            used_pages.update(tb[b][:npg])
            rem = kv_lens[b] % page_size
            if npg > 0 and rem:
                last = tb[b][npg - 1]
                kv[last, rem:, :, 0, :] = float("nan")
                kv[last, rem:, :, 1, :] = float("inf")
        for p in range(np_total):
            if p not in used_pages:
                kv[p, :, :, 0, :] = float("-inf")
                kv[p, :, :, 1, :] = float("nan")
    cu = [0]
    for n in q_lens:
        cu.append(cu[-1] + n)
    return PagedCase(
        name=name, q=q, pool_storage=storage, kv=kv, block_table=table.to(device),
        seq_lens=torch.tensor(kv_lens, dtype=torch.int32).to(device),
        cu_q=torch.tensor(cu, dtype=torch.int32).to(device), q_lens=q_lens, kv_lens=kv_lens,
        scale=float(scale if scale is not None else 1.0 / math.sqrt(d)), causal=causal, seed=seed)


def _uniform_ints(gen, lo: int, hi: int, n: int) -> List[int]:
    """n integers uniform on [lo, hi] inclusive."""
    return torch.randint(lo, hi + 1, (n,), generator=gen).tolist()


# ---------------------------------------------------------------------------
# Named workloads.  Seeds 101..105.  Each returns a PagedCase; ``scale_down``
# shrinks lengths (and batch) for parity runs the oracle finishes in seconds.
# ---------------------------------------------------------------------------

def tiny_mixed(device="cpu", seed: int = 101) -> PagedCase:
    """2 sequences x 32 query tokens, 24 q / 4 KV heads, head_dim 256, page 64,
    a 22-page two-layer pool and a [2, 11] block table that is a random
    permutation of all page ids, KV lengths uniform in [64, 704], scale 1/16,
    causal -- the decode.json manifest's buffers (q [64,24,256], kv
    [22,2,64,4,2,256], table [2,11], seq [2], cuq [3]) and its
    programs.decode call on layer 1."""
    gen = torch.Generator().manual_seed(seed)
    kv_lens = _uniform_ints(gen, 64, 704, 2)
    return make_case("tiny_mixed", seed, [32, 32], kv_lens, 24, 4, 256, causal=True,
                     scale=1.0 / 16, table_cols=11, table_fill="valid", num_pages=22,
                     layers=2, layer=1, device=device)


def decode_batch(device="cpu", seed: int = 102, n_seqs: int = 64, lo: int = 1024,
                 hi: int = 8192, poison: bool = False) -> PagedCase:
    """64 sequences x 1 query token, 32 q / 8 KV heads, head_dim 128, KV
    lengths uniform in [1024, 8192], shuffled pages of a shared pool, causal."""
    gen = torch.Generator().manual_seed(seed)
    kv_lens = _uniform_ints(gen, lo, hi, n_seqs)
    return make_case("decode_batch", seed, [1] * n_seqs, kv_lens, 32, 8, 128, causal=True,
                     table_cols=math.ceil(hi / PAGE_SIZE), device=device, poison=poison)


def long_decode(device="cpu", seed: int = 103, n_seqs: int = 128, ctx: int = 32768,
                poison: bool = False, layout: str = "head_major") -> PagedCase:
    """128 sequences x 1 query token at context 32768, 16 q / 2 KV heads,
    head_dim 256, K rows scaled x4 at 1% of positions, causal.  The pool is
    stored head-major within each page (contiguous K then V block per KV
    head), the layout the split kernel streams fastest at head_dim 256."""
    return make_case("long_decode", seed, [1] * n_seqs, [ctx] * n_seqs, 16, 2, 256, causal=True,
                     k_outlier_p=0.01, k_outlier_mult=4.0, device=device, poison=poison,
                     layout=layout)


def chunked_prefill(device="cpu", seed: int = 104, n_seqs: int = 8, q_lo: int = 512,
                    q_hi: int = 4096, ctx_lo: int = 0, ctx_hi: int = 8192) -> PagedCase:
    """8 sequences, new-query lengths uniform in [512, 4096] appended to prior
    cached context uniform in [0, 8192]; 24 q / 4 KV heads, head_dim 256, causal."""
    gen = torch.Generator().manual_seed(seed)
    q_lens = _uniform_ints(gen, q_lo, q_hi, n_seqs)
    prior = _uniform_ints(gen, ctx_lo, ctx_hi, n_seqs)
    kv_lens = [c + n for c, n in zip(prior, q_lens)]
    return make_case("chunked_prefill", seed, q_lens, kv_lens, 24, 4, 256, causal=True,
                     table_cols=math.ceil((q_hi + ctx_hi) / PAGE_SIZE), device=device)


def dit_self_attn(device="cpu", seed: int = 105, n_tokens: int = 37810, heads: int = 56) -> PagedCase:
    """One sequence of 37810 tokens, 56 heads (MHA), head_dim 128, non-causal,
    K with a per-(head, channel) offset drawn N(0, variance 2) -- stands in for
    the video-DiT block-24 activations of the GB10 SageAttention2 benchmark
    (shape [1, 37810, 56, 128]), which are not available."""
    return make_case("dit_self_attn", seed, [n_tokens], [n_tokens], heads, heads, 128,
                     causal=False, k_channel_offset_var=2.0, device=device)


def short_batch(device="cpu", seed: int = 106, n_seqs: int = 256, q_lo: int = 2, q_hi: int = 8,
                lo: int = 1024, hi: int = 8192) -> PagedCase:
    """Short multi-token runs (speculative decoding's verify step, small
    chunks): 256 sequences x n query tokens uniform in [2, 8] at the tail of
    KV lengths uniform in [1024, 8192], 32 q / 4 KV heads (G 8, so 16 to 64
    packed rows per sequence and KV head), head_dim 128, causal."""
    gen = torch.Generator().manual_seed(seed)
    q_lens = _uniform_ints(gen, q_lo, q_hi, n_seqs)
    kv_lens = _uniform_ints(gen, lo, hi, n_seqs)
    return make_case("short_batch", seed, q_lens, kv_lens, 32, 4, 128, causal=True,
                     table_cols=math.ceil(hi / PAGE_SIZE), device=device)


def new_kv_tokens(case: PagedCase, seed: int, layout: str = "separate"):
    """Seeded K and V rows for the step's new tokens: bf16 [T, Hkv, D] each
    (T = the q rows of the case).  layout "separate" gives two contiguous
    tensors; "fused_qkv" gives strided views into one [T, Hq + 2 Hkv, D]
    projection output (q heads first, then K heads, then V heads), as a fused
    QKV projection would leave them."""
    gen = torch.Generator(device="cpu").manual_seed(seed)
    T, hq, d = case.q.shape
    hkv = case.num_kv_heads
    dev = case.q.device
    if layout == "separate":
        k = _randn_bf16((T, hkv, d), gen, "cpu")
        v = _randn_bf16((T, hkv, d), gen, "cpu")
        return k.to(dev), v.to(dev)
    assert layout == "fused_qkv"
    qkv = _randn_bf16((T, hq + 2 * hkv, d), gen, "cpu").to(dev)
    return qkv[:, hq:hq + hkv, :], qkv[:, hq + hkv:, :]


def fp8_pool_case(case: PagedCase, mult: float = 2.0) -> PagedCase:
    """The same case over an fp8 KV cache: every pool element (bf16 x) becomes
    the OCP e4m3 code of mult * x (torch's float8_e4m3fn conversion; poisoned
    NaN slots stay NaN codes), stored as uint8 with the pool's layout and
    element strides.  The cache then holds K = k_scale * e4m3(code) with
    k_scale chosen by the caller (1 / mult keeps the bf16 case's scale)."""
    storage = (case.pool_storage.float() * mult).to(torch.float8_e4m3fn).view(torch.uint8)
    kv = storage.as_strided(case.kv.shape, case.kv.stride(),
                            case.kv.storage_offset() - case.pool_storage.storage_offset())
    return dataclasses.replace(case, name=case.name + "-fp8", pool_storage=storage, kv=kv)


def dense_from_case(case: PagedCase):
    """Dense [1, N, H, D] views (q, k, v) of a one-sequence self-attention case
    (n = L): the pages are gathered in block-table order, K and V stay
    interleaved (strided views)."""
    assert case.n_seqs == 1 and case.q_lens[0] == case.kv_lens[0]
    N = case.kv_lens[0]
    P = case.kv.shape[1]
    npg = (N + P - 1) // P
    idx = case.block_table[0, :npg].to(torch.long).to(case.kv.device)
    kv = case.kv.index_select(0, idx).reshape(npg * P, *case.kv.shape[2:])[:N]
    return case.q[None], kv[None, :, :, 0, :], kv[None, :, :, 1, :]


def dense_qkv(seed: int, batch: int, n: int, heads: int, head_dim: int = 128,
              k_channel_offset_var: float = 0.0, device="cpu"):
    """Seeded dense bf16 q, k, v [B, N, H, D] ~ N(0, 1); K optionally plus a
    per-(batch, head, channel) offset ~ N(0, k_channel_offset_var) added
    before rounding.  Draw order: q, k, v, offset (CPU generator)."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    shape = (batch, n, heads, head_dim)
    q = torch.randn(shape, generator=g)
    k = torch.randn(shape, generator=g)
    v = torch.randn(shape, generator=g)
    if k_channel_offset_var > 0:
        k = k + torch.randn((batch, 1, heads, head_dim), generator=g) * math.sqrt(k_channel_offset_var)
    return tuple(t.to(torch.bfloat16).to(device) for t in (q, k, v))


WORKLOADS = {
    "tiny_mixed": tiny_mixed,
    "decode_batch": decode_batch,
    "long_decode": long_decode,
    "chunked_prefill": chunked_prefill,
    "dit_self_attn": dit_self_attn,
    "short_batch": short_batch,
}
