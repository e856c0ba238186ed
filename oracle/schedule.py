"""Reference tile scheduler: which (Q tile, KV tile) pairs hold allowed pairs.

Test infrastructure only (see the package docstring).

The production guide ("Causal Attention Creates Rank Load Imbalance") asks for
kernels that skip blocks with no valid (query, key) pair and for logging the
effective QK block count; the FlashCP paper's sharding-aware communication
(section 3.2) sends a worker only the KV prefix its shards need.  This module
states those quantities from their definitions:

* Tiles: Q tiles of ``bq`` rows are anchored at each chunk's start and never
  cross a chunk boundary; KV tiles of ``bk`` keys are anchored at kv_lo; the
  last tile of each may be ragged.
* For each (Q tile, KV tile): count = number of allowed (row, key) pairs inside
  it.  SKIP iff count == 0; FULL iff count == rows x cols; else PARTIAL.
* Canonical order: chunk ascending, Q tile ascending, KV tile ascending.
* Per Q tile the non-skipped KV tiles, and inside them the FULL ones, are
  reported as intervals [kt_lo, kt_hi) and [kt_full_lo, kt_full_hi).  The
  functions below compute the sets and then check that each is an interval
  (raising otherwise).  Empty encodings: no non-skipped tile -> (0, 0, 0, 0);
  no FULL tile -> kt_full_lo = kt_full_hi = kt_hi.  The same for KV tiles over
  the global Q-tile index (chunks must be in ascending position order).
* LPT launch order: tiles by descending number of non-skipped partner tiles,
  ties by ascending index.
* Need interval of a chunk: the smallest and largest+1 key position that any
  row of the chunk may attend (checked to be contiguous); (0, 0) if none.
* Counters: (non-skipped tile pairs, FULL, PARTIAL, useful pairs).
"""
from __future__ import annotations

import numpy as np

from .attention import allowed_mask, doc_index, local_positions


def q_tiles(chunks, bq: int):
    """[(chunk, local_row0, global_row0, nrows)] in canonical order."""
    out = []
    l0 = 0
    for c, (g, n) in enumerate(chunks):
        for t in range(0, n, bq):
            out.append((c, l0 + t, g + t, min(bq, n - t)))
        l0 += n
    return out


def kv_tiles(kv_lo: int, kv_hi: int, bk: int):
    """[(c0, c1)] global key ranges of the KV tiles."""
    return [(c, min(c + bk, kv_hi)) for c in range(kv_lo, kv_hi, bk)]


def tile_pair_counts_bruteforce(cu_seqlens, chunks, kv_lo, kv_hi, bq, bk) -> np.ndarray:
    """Allowed-pair count of every tile pair, summed over the explicit mask."""
    pos = local_positions(chunks)
    mask = allowed_mask(cu_seqlens, pos, kv_lo, kv_hi)
    qt = q_tiles(chunks, bq)
    kt = kv_tiles(kv_lo, kv_hi, bk)
    out = np.zeros((len(qt), len(kt)), dtype=np.int64)
    for a, (_, l0, _, n) in enumerate(qt):
        for b, (c0, c1) in enumerate(kt):
            out[a, b] = int(mask[l0:l0 + n, c0 - kv_lo:c1 - kv_lo].sum())
    return out


def _row_intervals(cu_seqlens, pos, kv_lo, kv_hi):
    """Inclusive allowed-key interval [a_i, b_i] of each row.

    With documents stored contiguously, the keys of row i's document that are
    not after i are exactly the positions from the document start up to i."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    start = cu[doc_index(cu, pos)]
    a = np.maximum(start, kv_lo)
    b = np.minimum(pos, kv_hi - 1)
    return a, b


def tile_pair_counts(cu_seqlens, chunks, kv_lo, kv_hi, bq, bk, row_block: int = 8192) -> np.ndarray:
    """Same counts as the brute force, per row from its allowed interval (any size)."""
    pos = local_positions(chunks)
    qt = q_tiles(chunks, bq)
    kt = kv_tiles(kv_lo, kv_hi, bk)
    c0 = np.array([c for c, _ in kt], dtype=np.int64)
    c1 = np.array([e for _, e in kt], dtype=np.int64)
    tile_of_row = np.empty(pos.size, dtype=np.int64)
    for a, (_, l0, _, n) in enumerate(qt):
        tile_of_row[l0:l0 + n] = a
    out = np.zeros((len(qt), len(kt)), dtype=np.int64)
    a_all, b_all = _row_intervals(cu_seqlens, pos, kv_lo, kv_hi)
    for r0 in range(0, pos.size, row_block):
        a = a_all[r0:r0 + row_block, None]
        b = b_all[r0:r0 + row_block, None]
        cnt = np.maximum(0, np.minimum(b, c1[None, :] - 1) - np.maximum(a, c0[None, :]) + 1)
        np.add.at(out, tile_of_row[r0:r0 + row_block], cnt)
    return out


def classify(counts: np.ndarray, chunks, kv_lo, kv_hi, bq, bk) -> np.ndarray:
    """0 = SKIP, 1 = FULL, 2 = PARTIAL for every tile pair."""
    rows = np.array([n for *_, n in q_tiles(chunks, bq)], dtype=np.int64)
    cols = np.array([e - c for c, e in kv_tiles(kv_lo, kv_hi, bk)], dtype=np.int64)
    size = rows[:, None] * cols[None, :]
    cls = np.where(counts == 0, 0, np.where(counts == size, 1, 2))
    return cls.astype(np.int8)


def _interval(flags: np.ndarray, what: str):
    idx = np.nonzero(flags)[0]
    if idx.size == 0:
        return None
    lo, hi = int(idx[0]), int(idx[-1]) + 1
    if hi - lo != idx.size:
        raise AssertionError(f"{what} is not contiguous")
    return lo, hi


def _ranges(cls_rows: np.ndarray, what: str) -> np.ndarray:
    out = np.zeros((cls_rows.shape[0], 4), dtype=np.int32)
    for a in range(cls_rows.shape[0]):
        ns = _interval(cls_rows[a] != 0, what + " non-skipped set")
        if ns is None:
            continue
        fl = _interval(cls_rows[a] == 1, what + " FULL set")
        lo, hi = ns
        flo, fhi = fl if fl is not None else (hi, hi)
        out[a] = (lo, flo, fhi, hi)
    return out


def lpt_order(weights) -> np.ndarray:
    """Indices by descending weight, ties by ascending index."""
    w = np.asarray(weights, dtype=np.int64)
    return np.lexsort((np.arange(w.size), -w)).astype(np.int32)


def need_intervals(cu_seqlens, chunks, kv_lo, kv_hi) -> np.ndarray:
    """[n_chunks, 2] key interval each chunk's rows need (checked contiguous)."""
    out = np.zeros((len(chunks), 2), dtype=np.int32)
    for c, (g, n) in enumerate(chunks):
        pos = np.arange(g, g + n, dtype=np.int64)
        a, b = _row_intervals(cu_seqlens, pos, kv_lo, kv_hi)
        ok = a <= b
        if not ok.any():
            continue
        lo, hi = int(a[ok].min()), int(b[ok].max()) + 1
        covered = np.zeros(hi - lo, dtype=bool)
        for x, y in zip(a[ok], b[ok]):
            covered[x - lo:y - lo + 1] = True
        if not covered.all():
            raise AssertionError("need set is not contiguous")
        out[c] = (lo, hi)
    return out


def useful_pairs(cu_seqlens, chunks, kv_lo, kv_hi) -> int:
    """Number of allowed (row, key) pairs per head."""
    a, b = _row_intervals(cu_seqlens, local_positions(chunks), kv_lo, kv_hi)
    return int(np.maximum(0, b - a + 1).sum())


def schedule(cu_seqlens, chunks, kv_lo, kv_hi, bq, bk, counts=None) -> dict:
    """Everything the scheduler reports, in canonical order."""
    starts = [g for g, _ in chunks]
    if any(starts[i] + chunks[i][1] > starts[i + 1] for i in range(len(chunks) - 1)):
        raise ValueError("chunks must be disjoint and in ascending position order")
    if counts is None:
        counts = tile_pair_counts(cu_seqlens, chunks, kv_lo, kv_hi, bq, bk)
    cls = classify(counts, chunks, kv_lo, kv_hi, bq, bk)
    qdesc = _ranges(cls, "KV tiles of a Q tile")
    kvdesc = _ranges(cls.T, "Q tiles of a KV tile")
    nonskip = int((cls != 0).sum())
    full = int((cls == 1).sum())
    return {
        "qtile_desc": qdesc,
        "kvtile_desc": kvdesc,
        "lpt_q": lpt_order((cls != 0).sum(axis=1)),
        "lpt_kv": lpt_order((cls != 0).sum(axis=0)),
        "need": need_intervals(cu_seqlens, chunks, kv_lo, kv_hi),
        "counters": np.array([nonskip, full, nonskip - full, int(counts.sum())], dtype=np.int64),
        "classes": cls,
    }
