"""Seeded synthetic inputs for document-masked attention.

This module is shared by the HIP path's drivers and by the tests that call the
oracle.  It holds no attention arithmetic: it only draws document lengths and
bf16 tensors from seeded numpy generators and describes which query rows and
which key range a caller hands to the attention calls.

Workload shapes follow the pages' setting of packed training sequences with
skewed document lengths (FlashCP paper, section 2.1 "Input Packing and Document
Mask" and its evaluation setup: 128K context, head dim 128, 16/32 heads), and
the 2 x CP chunking of section 2.2 (chunks i and 2N-1-i on worker i).

Recipes
-------
* Document lengths come from ``numpy.random.default_rng(seed)``, drawn one at a
  time.  Lognormal: ``L = clip(rint(rng.lognormal(ln(median), sigma)), lo, hi)``
  until the running sum reaches T; the last document is truncated so the sum is
  exactly T.  Bimodal (131072-token mix): two long documents, ``L1`` uniform on
  ``[16384, 22938]`` and ``L2 = 39322 - L1`` (30% of the tokens); short documents
  uniform on ``[128, 2048]`` fill the other 91750 tokens (last one truncated);
  then the document order is shuffled with ``rng.permutation``.
* Every tensor (Q, K, V, dO) is defined over global positions [0, T) and is
  drawn in blocks of ``BLOCK_ROWS`` positions; block b of tensor t comes from
  ``default_rng([seed, t, b]).standard_normal((rows, H, D), float32)`` and is
  rounded to bf16 with round-to-nearest-even.  Any row subset can therefore be
  regenerated without drawing the rest.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

BLOCK_ROWS = 4096
TENSOR_IDS = {"q": 1, "k": 2, "v": 3, "do": 4}


# ---------------------------------------------------------------- bf16 helpers
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round-to-nearest-even); returns the uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(b).astype(np.float64)


# ------------------------------------------------------------ document lengths
def lognormal_docs(seed: int, median: float, sigma: float, lo: int, hi: int, total: int) -> list[int]:
    rng = np.random.default_rng(seed)
    out: list[int] = []
    s = 0
    while s < total:
        x = rng.lognormal(math.log(median), sigma)
        n = int(np.clip(np.rint(x), lo, hi))
        n = min(n, total - s)
        out.append(n)
        s += n
    return out


def bimodal_docs(seed: int, total: int = 131072) -> list[int]:
    rng = np.random.default_rng(seed)
    long_total = int(round(0.3 * total))          # 39322 for 131072
    l1 = int(rng.integers(16384, long_total - 16384, endpoint=True))
    docs = [l1, long_total - l1]
    short_total = total - long_total
    s = 0
    shorts: list[int] = []
    while s < short_total:
        n = int(rng.integers(128, 2048, endpoint=True))
        n = min(n, short_total - s)
        shorts.append(n)
        s += n
    docs += shorts
    perm = rng.permutation(len(docs))
    return [docs[i] for i in perm]


def cu_from_lengths(lengths) -> np.ndarray:
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return cu


# --------------------------------------------------------------------- tensors
def _block(seed: int, tid: int, b: int, rows: int, h: int, d: int) -> np.ndarray:
    rng = np.random.default_rng([seed, tid, b])
    return f32_to_bf16_bits(rng.standard_normal((rows, h, d), dtype=np.float32))


def draw_tensor(seed: int, name: str, total_rows: int, h: int, d: int, positions=None,
                threads: int | None = None) -> np.ndarray:
    """bf16 bits of tensor ``name`` at the given global positions ([n, h, d]).

    ``positions=None`` means all of [0, total_rows)."""
    tid = TENSOR_IDS[name]
    nblk = (total_rows + BLOCK_ROWS - 1) // BLOCK_ROWS
    if positions is None:
        blocks = list(range(nblk))
    else:
        positions = np.asarray(positions, dtype=np.int64)
        if positions.size and (positions.min() < 0 or positions.max() >= total_rows):
            raise ValueError("position out of range")
        blocks = sorted(set((positions // BLOCK_ROWS).tolist()))

    def one(b):
        rows = min(BLOCK_ROWS, total_rows - b * BLOCK_ROWS)
        return b, _block(seed, tid, b, rows, h, d)

    nthr = threads or min(16, os.cpu_count() or 1)
    if len(blocks) > 1 and nthr > 1:
        with ThreadPoolExecutor(nthr) as ex:
            parts = dict(ex.map(one, blocks))
    else:
        parts = dict(one(b) for b in blocks)
    if positions is None:
        return np.concatenate([parts[b] for b in blocks], axis=0) if blocks else np.zeros((0, h, d), np.uint16)
    out = np.empty((positions.size, h, d), dtype=np.uint16)
    for b in blocks:
        sel = np.nonzero(positions // BLOCK_ROWS == b)[0]
        out[sel] = parts[b][positions[sel] - b * BLOCK_ROWS]
    return out


# ------------------------------------------------------------------- workloads
@dataclass
class Workload:
    """One attention problem: packed sequence, local query chunks, KV range."""
    name: str
    seed: int
    total: int                      # packed sequence length T
    lengths: list
    hq: int
    hkv: int
    d: int
    chunks: list                    # [(g_start, len)] local query rows, in order
    kv_lo: int
    kv_hi: int
    backward: bool = False
    kv_block: int = 0               # >0: the rank computes per-KV-block partials
    meta: dict = field(default_factory=dict)

    @property
    def cu_seqlens(self) -> np.ndarray:
        return cu_from_lengths(self.lengths)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def tq(self) -> int:
        return int(sum(n for _, n in self.chunks))

    @property
    def tkv(self) -> int:
        return self.kv_hi - self.kv_lo

    def local_positions(self) -> np.ndarray:
        return np.concatenate([np.arange(g, g + n, dtype=np.int64) for g, n in self.chunks]) \
            if self.chunks else np.zeros(0, np.int64)

    def q(self, local_rows=None) -> np.ndarray:
        pos = self.local_positions()
        if local_rows is not None:
            pos = pos[np.asarray(local_rows, dtype=np.int64)]
        return draw_tensor(self.seed, "q", self.total, self.hq, self.d, pos)

    def do(self, local_rows=None) -> np.ndarray:
        pos = self.local_positions()
        if local_rows is not None:
            pos = pos[np.asarray(local_rows, dtype=np.int64)]
        return draw_tensor(self.seed, "do", self.total, self.hq, self.d, pos)

    def k(self, kv_rows=None) -> np.ndarray:
        pos = np.arange(self.kv_lo, self.kv_hi, dtype=np.int64)
        if kv_rows is not None:
            pos = pos[np.asarray(kv_rows, dtype=np.int64)]
        return draw_tensor(self.seed, "k", self.total, self.hkv, self.d, pos)

    def v(self, kv_rows=None) -> np.ndarray:
        pos = np.arange(self.kv_lo, self.kv_hi, dtype=np.int64)
        if kv_rows is not None:
            pos = pos[np.asarray(kv_rows, dtype=np.int64)]
        return draw_tensor(self.seed, "v", self.total, self.hkv, self.d, pos)


def make_config(index: int, seed: int | None = None) -> Workload:
    """The five standard workloads; the canonical seed is the config index."""
    s = index if seed is None else seed
    if index == 1:
        lengths = [512, 1024, 256, 256]
        return Workload("fwd_T2048_docs4_h8x8_d64", s, 2048, lengths, 8, 8, 64, [(0, 2048)], 0, 2048)
    if index == 2:
        lengths = lognormal_docs(s, 1024, 1.2, 64, 32768, 32768)
        return Workload("fwd_T32768_lognormal1024_h32x8_d128", s, 32768, lengths, 32, 8, 128, [(0, 32768)], 0, 32768)
    if index == 3:
        total, cp, rank, chunk = 131072, 8, 3, 8192
        lengths = lognormal_docs(s, 2048, 1.5, 64, 131072, total)
        chunks = [(rank * chunk, chunk), ((2 * cp - 1 - rank) * chunk, chunk)]
        return Workload("cp8_rank3_T131072_lognormal2048_h32x8_d128", s, total, lengths, 32, 8, 128,
                        chunks, 0, total, kv_block=8192, meta={"cp": cp, "rank": rank, "chunk": chunk})
    if index == 4:
        lengths = lognormal_docs(s, 1024, 1.2, 64, 65536, 65536)
        return Workload("fwdbwd_T65536_lognormal1024_h32x8_d128", s, 65536, lengths, 32, 8, 128,
                        [(0, 65536)], 0, 65536, backward=True)
    if index == 5:
        lengths = bimodal_docs(s, 131072)
        return Workload("fwdbwd_T131072_bimodal_h64x8_d128", s, 131072, lengths, 64, 8, 128,
                        [(0, 131072)], 0, 131072, backward=True)
    raise ValueError(f"unknown config {index}")


def custom_workload(seed: int, lengths, hq: int, hkv: int, d: int, chunks=None, kv_lo: int = 0,
                    kv_hi: int | None = None, backward: bool = False, name: str = "custom") -> Workload:
    total = int(sum(lengths))
    return Workload(name, seed, total, list(map(int, lengths)), hq, hkv, d,
                    list(chunks) if chunks is not None else [(0, total)], kv_lo,
                    total if kv_hi is None else kv_hi, backward)


def sequence_zigzag_chunks(total: int, cp: int, rank: int) -> list:
    """Per-sequence 2 x CP sharding: the packed sequence cut into 2*cp equal
    chunks, rank r holding chunks r and 2*cp - 1 - r (FlashCP section 2.3, the
    sharding that Llama3 CP and Ring-Attn (Zigzag) start from).  ``total`` must
    be a multiple of 2*cp."""
    if total % (2 * cp):
        raise ValueError("total must be a multiple of 2 * cp")
    c = total // (2 * cp)
    return [(rank * c, c), ((2 * cp - 1 - rank) * c, c)]


def doc_piece_bounds(length: int, cp: int) -> list:
    """Boundaries of the 2*cp pieces of one document: piece i covers local rows
    [floor(i*L/(2cp)), floor((i+1)*L/(2cp))), so pieces differ by at most one
    row and a document shorter than 2*cp leaves some pieces empty."""
    n = 2 * cp
    return [(i * length) // n for i in range(n + 1)]


def per_doc_chunks(lengths, cp: int, rank: int) -> list:
    """Per-document 2 x CP sharding (Per-Doc CP and Ring-Attn (Zigzag) varlen,
    FlashCP section 2.3): every document cut into 2*cp pieces, rank r holding
    pieces r and 2*cp - 1 - r of each.  Returned in ascending position order
    (document by document), empty pieces dropped; adjacent pieces stay separate
    chunks."""
    out = []
    start = 0
    for length in map(int, lengths):
        b = doc_piece_bounds(length, cp)
        for i in (rank, 2 * cp - 1 - rank):
            if b[i + 1] > b[i]:
                out.append((start + b[i], b[i + 1] - b[i]))
        start += length
    return out


def random_plan(rng: np.random.Generator, total: int, n_ranks: int, n_cuts: int) -> list:
    """A random assignment of the sequence to workers: [0, total) cut at
    n_cuts random points, each piece given to a random worker (every worker
    gets at least one piece when there are enough); per worker the pieces in
    ascending order, adjacent ones kept separate.  Covers every token once."""
    cuts = sorted(set(int(x) for x in rng.integers(1, max(total, 2), size=n_cuts) if 0 < x < total))
    bounds = [0] + cuts + [total]
    pieces = [(bounds[i], bounds[i + 1] - bounds[i]) for i in range(len(bounds) - 1) if bounds[i + 1] > bounds[i]]
    owner = rng.integers(0, n_ranks, size=len(pieces))
    if len(pieces) >= n_ranks:
        owner[rng.permutation(len(pieces))[:n_ranks]] = np.arange(n_ranks)
    return [[p for p, o in zip(pieces, owner) if o == r] for r in range(n_ranks)]


FIG3_PATTERNS = ("1x131072", "16x8192", "bimodal131072")


def fig3_lengths(pattern: str, seed: int = 5) -> list:
    """Document lengths of the kernel-efficiency study (FlashCP Figure 3: one
    128K document vs sixteen 8K documents), plus the bimodal 131072-token mix."""
    if pattern == "1x131072":
        return [131072]
    if pattern == "16x8192":
        return [8192] * 16
    if pattern == "bimodal131072":
        return bimodal_docs(seed, 131072)
    raise ValueError(f"unknown pattern {pattern}")


def fig3_workload(pattern: str, sharding: str, cp: int, rank: int, hq: int = 32, hkv: int = 8, d: int = 128,
                  seed: int = 5, lengths=None) -> Workload:
    """One CP rank's forward under per-sequence or per-document 2 x CP sharding,
    attending the whole (all-gathered) KV range; ``lengths`` overrides the
    pattern's documents."""
    lengths = fig3_lengths(pattern, seed) if lengths is None else list(lengths)
    total = int(sum(lengths))
    if sharding == "per_sequence":
        chunks = sequence_zigzag_chunks(total, cp, rank)
    elif sharding == "per_doc":
        chunks = per_doc_chunks(lengths, cp, rank)
    else:
        raise ValueError(f"unknown sharding {sharding}")
    return Workload(f"{sharding}_cp{cp}_rank{rank}_{pattern}_h{hq}x{hkv}_d{d}", seed, total, lengths, hq, hkv, d,
                    chunks, 0, total, meta={"cp": cp, "rank": rank, "pattern": pattern, "sharding": sharding})


def random_lengths(rng: np.random.Generator, total: int, max_len: int, p_one: float = 0.15) -> list[int]:
    """Random document split of ``total`` tokens, with some length-1 documents."""
    out = []
    s = 0
    while s < total:
        n = 1 if rng.random() < p_one else int(rng.integers(1, max_len + 1))
        n = min(n, total - s)
        out.append(n)
        s += n
    return out
