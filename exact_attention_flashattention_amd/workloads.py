"""Seeded synthetic inputs for the attention workloads.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic. Both the CPU oracle tests and the GPU path consume the
tensors it returns, so both sides see exactly the same values.

Recipe (the same for every workload):
  * one CPU ``torch.Generator`` seeded with ``42 + index`` (index 1..5 below);
  * values drawn as i.i.d. N(0, 1) in float32 with ``torch.randn``;
  * bf16 workloads cast those float32 draws with torch's round-to-nearest-even;
  * draw order: q, then (decode only) seq_lens, then k, then v, then (paged
    decode only) the page permutation.

Layouts:
  * prefill, index 1: ``[B, H, N, d]`` (the head-major layout).
  * prefill, index 2 and 3: ``[B, N, H, d]`` (token-major; the output has the
    same layout with Hq heads).
  * decode: q and o ``[B, Hq, d]``; K/V pools ``[num_pages, page_size, Hkv, d]``
    (a page holds ``page_size`` consecutive tokens of one sequence, all KV
    heads); ``block_table`` int32 ``[B, max_pages_per_seq]`` maps a sequence's
    logical page to a physical page; ``seq_lens`` int32 ``[B]``. Unused table
    entries hold -1 and are never dereferenced.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

PAGE_SIZE = 16


@dataclasses.dataclass
class PrefillInputs:
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    B: int
    N: int
    Hq: int
    Hkv: int
    d: int
    scale: float
    causal: bool
    layout: str  # "BNHD" or "BHND"
    name: str = ""


@dataclasses.dataclass
class DecodeInputs:
    q: torch.Tensor            # [B, Hq, d]
    k_pages: torch.Tensor      # [num_pages, page_size, Hkv, d]
    v_pages: torch.Tensor      # [num_pages, page_size, Hkv, d]
    block_table: torch.Tensor  # int32 [B, max_pages_per_seq]
    seq_lens: torch.Tensor     # int32 [B]
    B: int
    Hq: int
    Hkv: int
    d: int
    page_size: int
    max_pages_per_seq: int
    scale: float
    name: str = ""

    @property
    def num_pages(self) -> int:
        return int(self.k_pages.shape[0])


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return g


def _randn(g: torch.Generator, shape, dtype: torch.dtype) -> torch.Tensor:
    x = torch.randn(*shape, generator=g, dtype=torch.float32)
    return x if dtype == torch.float32 else x.to(dtype)


def prefill_inputs(B: int, N: int, Hq: int, Hkv: int, d: int, *, seed: int,
                   dtype: torch.dtype = torch.bfloat16, layout: str = "BNHD",
                   causal: bool = True, scale: Optional[float] = None,
                   name: str = "") -> PrefillInputs:
    """Draw q, k, v for a prefill call, in that order, from one generator."""
    g = _gen(seed)
    if layout == "BNHD":
        qs, ks = (B, N, Hq, d), (B, N, Hkv, d)
    elif layout == "BHND":
        qs, ks = (B, Hq, N, d), (B, Hkv, N, d)
    else:
        raise ValueError(f"unknown layout {layout}")
    q = _randn(g, qs, dtype)
    k = _randn(g, ks, dtype)
    v = _randn(g, ks, dtype)
    return PrefillInputs(q, k, v, B, N, Hq, Hkv, d,
                         1.0 / math.sqrt(d) if scale is None else scale,
                         causal, layout, name)


def output_gradient(x: PrefillInputs, *, seed: int) -> torch.Tensor:
    """dL/do for a backward pass: i.i.d. N(0, 1) of q's shape and dtype, from
    its own generator (seeded separately, so the forward inputs are unchanged)."""
    g = _gen(seed)
    return _randn(g, tuple(x.q.shape), x.q.dtype)


def paged_decode_inputs(B: int, Hq: int, Hkv: int, d: int, seq_lens, *, seed: int,
                        page_size: int = PAGE_SIZE, permute: bool = True,
                        max_pages_per_seq: Optional[int] = None,
                        dtype: torch.dtype = torch.bfloat16,
                        scale: Optional[float] = None, name: str = "") -> DecodeInputs:
    """Draw a decode problem whose pool holds exactly the pages the sequences need.

    ``seq_lens`` is either a list of ints or a ``(low, high)`` tuple, in which
    case the lengths are drawn uniformly from the inclusive integer range with
    the same generator (after q). Sequence b owns ``ceil(L_b / page_size)``
    pages. With ``permute`` the physical page numbers are a seeded random
    permutation of the pool, handed out to the sequences in order; otherwise
    sequence b's pages are laid out consecutively (the identity table), which
    makes the pool byte-identical to a contiguous ``[B, L, Hkv, d]`` cache when
    every length is the same multiple of ``page_size``.
    """
    g = _gen(seed)
    q = _randn(g, (B, Hq, d), dtype)
    if isinstance(seq_lens, tuple):
        lo, hi = seq_lens
        lens = torch.randint(lo, hi + 1, (B,), generator=g, dtype=torch.int64).tolist()
    else:
        lens = [int(x) for x in seq_lens]
        assert len(lens) == B
    pages_per = [-(-L // page_size) for L in lens]
    total = sum(pages_per)
    mpps = max(1, max(pages_per)) if max_pages_per_seq is None else max_pages_per_seq
    assert mpps >= max(pages_per, default=0)
    k_pages = _randn(g, (max(total, 1), page_size, Hkv, d), dtype)
    v_pages = _randn(g, (max(total, 1), page_size, Hkv, d), dtype)
    if permute:
        order = torch.randperm(max(total, 1), generator=g).tolist()
    else:
        order = list(range(max(total, 1)))
    table = torch.full((B, mpps), -1, dtype=torch.int32)
    cursor = 0
    for b in range(B):
        n = pages_per[b]
        if n:
            table[b, :n] = torch.tensor(order[cursor:cursor + n], dtype=torch.int32)
        cursor += n
    return DecodeInputs(q, k_pages, v_pages, table,
                        torch.tensor(lens, dtype=torch.int32), B, Hq, Hkv, d,
                        page_size, mpps, 1.0 / math.sqrt(d) if scale is None else scale,
                        name)


@dataclasses.dataclass
class ChunkInputs:
    """A chunk of new tokens per sequence after a cached prefix (chunked
    prefill). The pool holds the prefix; the chunk's own K/V are k_new/v_new,
    which the append step writes into the pool before the attention runs."""
    q: torch.Tensor            # [T, Hq, d], sequence b owns rows cu_q[b] .. cu_q[b+1]-1
    k_new: torch.Tensor        # [T, Hkv, d]
    v_new: torch.Tensor        # [T, Hkv, d]
    k_pages: torch.Tensor      # [num_pages, page_size, Hkv, d]
    v_pages: torch.Tensor
    block_table: torch.Tensor  # int32 [B, max_pages_per_seq], pages for prefix + chunk
    cu_q: torch.Tensor         # int32 [B + 1]
    prefix_lens: torch.Tensor  # int32 [B], P_b
    seq_lens: torch.Tensor     # int32 [B], P_b + c_b
    B: int
    Hq: int
    Hkv: int
    d: int
    page_size: int
    max_pages_per_seq: int
    max_q_len: int
    scale: float
    name: str = ""

    @property
    def num_pages(self) -> int:
        return int(self.k_pages.shape[0])

    @property
    def total_q(self) -> int:
        return int(self.q.shape[0])


def chunked_prefill_inputs(B: int, Hq: int, Hkv: int, d: int, prefix_lens, chunk_lens, *,
                           seed: int, page_size: int = PAGE_SIZE, permute: bool = True,
                           max_pages_per_seq: Optional[int] = None,
                           dtype: torch.dtype = torch.bfloat16,
                           scale: Optional[float] = None, name: str = "") -> ChunkInputs:
    """Draw a chunked-prefill problem. ``prefix_lens`` and ``chunk_lens`` are
    lists of ints or inclusive ``(low, high)`` ranges drawn uniformly. The
    lengths fix every shape, so they are drawn first (prefix, then chunk),
    then q, k_new, v_new, the pool's K, the pool's V and the page permutation.
    Sequence b owns ceil((P_b + c_b) / page_size) pages; its chunk slots in the
    pool hold unrelated draws until the append overwrites them."""
    g = _gen(seed)

    def lengths(spec):
        if isinstance(spec, tuple):
            lo, hi = spec
            return torch.randint(lo, hi + 1, (B,), generator=g, dtype=torch.int64).tolist()
        out = [int(x) for x in spec]
        assert len(out) == B
        return out

    P = lengths(prefix_lens)
    c = lengths(chunk_lens)
    T = sum(c)
    q = _randn(g, (T, Hq, d), dtype)
    k_new = _randn(g, (T, Hkv, d), dtype)
    v_new = _randn(g, (T, Hkv, d), dtype)
    L = [p + n for p, n in zip(P, c)]
    pages_per = [-(-x // page_size) for x in L]
    total = max(sum(pages_per), 1)
    mpps = max(1, max(pages_per)) if max_pages_per_seq is None else max_pages_per_seq
    assert mpps >= max(pages_per, default=0)
    k_pages = _randn(g, (total, page_size, Hkv, d), dtype)
    v_pages = _randn(g, (total, page_size, Hkv, d), dtype)
    order = torch.randperm(total, generator=g).tolist() if permute else list(range(total))
    table = torch.full((B, mpps), -1, dtype=torch.int32)
    cursor = 0
    for b in range(B):
        n = pages_per[b]
        if n:
            table[b, :n] = torch.tensor(order[cursor:cursor + n], dtype=torch.int32)
        cursor += n
    cu = [0]
    for n in c:
        cu.append(cu[-1] + n)
    return ChunkInputs(q, k_new, v_new, k_pages, v_pages, table,
                       torch.tensor(cu, dtype=torch.int32), torch.tensor(P, dtype=torch.int32),
                       torch.tensor(L, dtype=torch.int32), B, Hq, Hkv, d, page_size, mpps,
                       max(c, default=0), 1.0 / math.sqrt(d) if scale is None else scale, name)


def poison_chunk_slots(x: ChunkInputs, value: float = float("nan")) -> None:
    """Fill every pool slot that is not part of a cached prefix with ``value``:
    the chunk slots (until the append writes them), the slots past each
    sequence's end, and pages no sequence references."""
    keep = torch.zeros(x.k_pages.shape[0], x.page_size, dtype=torch.bool)
    for b in range(x.B):
        for t in range(int(x.prefix_lens[b])):
            keep[int(x.block_table[b, t // x.page_size]), t % x.page_size] = True
    x.k_pages[~keep] = value
    x.v_pages[~keep] = value


@dataclasses.dataclass
class MlaDecodeInputs:
    """One decode step of absorbed multi-head latent attention: every token
    caches one row [latent (d_c) ; rotary key (d_r)] shared by all heads."""
    q: torch.Tensor            # [B, Hq, d_c + d_r]
    kv_pages: torch.Tensor     # [num_pages, page_size, d_c + d_r]
    block_table: torch.Tensor  # int32 [B, max_pages_per_seq]
    seq_lens: torch.Tensor     # int32 [B]
    B: int
    Hq: int
    d_c: int
    d_r: int
    page_size: int
    max_pages_per_seq: int
    scale: float
    name: str = ""

    @property
    def num_pages(self) -> int:
        return int(self.kv_pages.shape[0])


def mla_decode_inputs(B: int, Hq: int, d_c: int, d_r: int, seq_lens, *, seed: int,
                      page_size: int = PAGE_SIZE, permute: bool = True,
                      max_pages_per_seq: Optional[int] = None, dtype: torch.dtype = torch.bfloat16,
                      scale: Optional[float] = None, d_head: int = 128, name: str = "") -> MlaDecodeInputs:
    """Draw an absorbed-MLA decode problem: q, then (for a range) the lengths,
    then the cache rows and the page permutation, as for paged_decode_inputs.
    The default scale is 1 / sqrt(d_head + d_r), the score scale of the
    non-absorbed heads the latent stands for."""
    g = _gen(seed)
    dk = d_c + d_r
    q = _randn(g, (B, Hq, dk), dtype)
    if isinstance(seq_lens, tuple):
        lo, hi = seq_lens
        lens = torch.randint(lo, hi + 1, (B,), generator=g, dtype=torch.int64).tolist()
    else:
        lens = [int(x) for x in seq_lens]
        assert len(lens) == B
    pages_per = [-(-L // page_size) for L in lens]
    total = max(sum(pages_per), 1)
    mpps = max(1, max(pages_per)) if max_pages_per_seq is None else max_pages_per_seq
    assert mpps >= max(pages_per, default=0)
    kv = _randn(g, (total, page_size, dk), dtype)
    order = torch.randperm(total, generator=g).tolist() if permute else list(range(total))
    table = torch.full((B, mpps), -1, dtype=torch.int32)
    cursor = 0
    for b in range(B):
        n = pages_per[b]
        if n:
            table[b, :n] = torch.tensor(order[cursor:cursor + n], dtype=torch.int32)
        cursor += n
    return MlaDecodeInputs(q, kv, table, torch.tensor(lens, dtype=torch.int32), B, Hq, d_c, d_r, page_size,
                           mpps, 1.0 / math.sqrt(d_head + d_r) if scale is None else scale, name)


def poison_unused_mla_slots(x: MlaDecodeInputs, value: float = float("nan")) -> None:
    """Fill the slots past each sequence's end on its last page, and every page
    no sequence references, with ``value``."""
    used = torch.zeros(x.kv_pages.shape[0], dtype=torch.bool)
    for b in range(x.B):
        L = int(x.seq_lens[b])
        n = -(-L // x.page_size)
        for p in range(n):
            used[int(x.block_table[b, p])] = True
        if n and L % x.page_size:
            x.kv_pages[int(x.block_table[b, n - 1]), L % x.page_size:] = value
    x.kv_pages[~used] = value


def poison_unused_slots(x: DecodeInputs, value: float = float("nan")) -> None:
    """Fill the slots past each sequence's end on its last page with ``value``
    (and any pool page no sequence references). A correct kernel never lets
    them reach the output."""
    used = torch.zeros(x.k_pages.shape[0], dtype=torch.bool)
    for b in range(x.B):
        L = int(x.seq_lens[b])
        n = -(-L // x.page_size)
        for p in range(n):
            used[int(x.block_table[b, p])] = True
        if n and L % x.page_size:
            last = int(x.block_table[b, n - 1])
            x.k_pages[last, L % x.page_size:] = value
            x.v_pages[last, L % x.page_size:] = value
    x.k_pages[~used] = value
    x.v_pages[~used] = value


# The standard workloads. Index 1 is the small fp32 parity case; index 2 is
# the headline prefill; index 3 the MHA/MQA endpoints; 4 and 5 decode; 6 a
# chunk of new tokens after a long cached prefix (paged prefill + append); 7
# an absorbed-MLA decode (one shared 576-wide latent row per token).

def workload_1() -> PrefillInputs:
    return prefill_inputs(1, 128, 4, 2, 64, seed=43, dtype=torch.float32,
                          layout="BHND", scale=1.0 / 8.0,
                          name="causal GQA fwd fp32 B=1 Hq=4 Hkv=2 N=128 d=64 [B,H,N,d]")


def workload_2() -> PrefillInputs:
    return prefill_inputs(4, 4096, 32, 8, 128, seed=44,
                          name="causal GQA prefill bf16 B=4 Hq=32 Hkv=8 N=4096 d=128 [B,N,H,d]")


def workload_3(hkv: int) -> PrefillInputs:
    assert hkv in (16, 1)
    return prefill_inputs(8, 2048, 16, hkv, 64, seed=45,
                          name=f"causal prefill bf16 B=8 Hq=16 Hkv={hkv} N=2048 d=64 [B,N,H,d]")


def workload_4() -> DecodeInputs:
    return paged_decode_inputs(64, 32, 8, 128, [8192] * 64, seed=46, permute=False,
                               name="batched decode bf16 B=64 Hq=32 Hkv=8 d=128 ctx=8192 contiguous")


def workload_5() -> DecodeInputs:
    return paged_decode_inputs(4, 64, 8, 128, (98304, 131072), seed=47, permute=True,
                               max_pages_per_seq=131072 // PAGE_SIZE,
                               name="paged decode bf16 B=4 Hq=64 Hkv=8 d=128 seq_lens~U[98304,131072] page=16 permuted")


def workload_6() -> ChunkInputs:
    return chunked_prefill_inputs(4, 32, 8, 128, (6144, 14336), [2048] * 4, seed=48,
                                  name="chunked prefill bf16 B=4 Hq=32 Hkv=8 d=128 prefix~U[6144,14336] "
                                       "chunk=2048 page=16 permuted")


def workload_7() -> MlaDecodeInputs:
    return mla_decode_inputs(16, 128, 512, 64, (8192, 16384), seed=49,
                             name="MLA-absorbed decode bf16 B=16 Hq=128 d_c=512 d_r=64 "
                                  "seq_lens~U[8192,16384] page=16 permuted")
