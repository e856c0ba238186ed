"""Reference for the KV exchange of sharding-aware context parallelism.

Test infrastructure only (see the package docstring).

FlashCP paper, section 3.1 (problem formulation) and 3.2 ("Dynamic
Sharding-aware Communication"), Eq. 4 and Eq. 5:

* A worker's input is split into document shards s_i with prefix length p_i
  (the tokens of the same document before the shard).  Here a shard is a
  maximal run of one worker's chunk inside one document.
* A query token attends only to the prefix of its own document, so the KV a
  worker needs is, over its tokens, the union of [document start, token].
* The static pattern sends the full KV: 4 x (sum_i d_i / N) x H x D x (N - 1)
  elements on the critical path (Eq. 4).
* The sharding-aware pattern sends, per worker, only the shards that are not
  the last shard of their document (the set S-hat; a document kept whole is
  its own last shard), packed into one continuous buffer; the volume is
  4 x max_j sum_{i in S-hat} x_ij s_i x H x D x (N - 1) (Eq. 5).  The factor 4
  is K and V, forward and backward.

Readings: H is the number of KV heads (K and V are what travel); positions not
needed by a worker hold zeros in its KV buffer (any finite value would do:
the mask gives them weight zero).
"""
from __future__ import annotations

import numpy as np

from .attention import doc_index, local_positions


def document_shards(cu_seqlens, chunks):
    """[(g_start, s, doc, p)] shards of one worker in its local order: each
    chunk cut at document boundaries; p = tokens of the document before it."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    out = []
    for g, n in chunks:
        pos = np.arange(g, g + n, dtype=np.int64)
        if n == 0:
            continue
        docs = doc_index(cu, pos)
        for dd in np.unique(docs):
            sel = pos[docs == dd]
            out.append((int(sel[0]), int(sel.size), int(dd), int(sel[0] - cu[dd])))
    return out


def is_last_shard(cu_seqlens, shard) -> bool:
    g, s, dd, _ = shard
    return g + s == int(cu_seqlens[dd + 1])


def sent_rows(cu_seqlens, chunks) -> int:
    """sum of s_i over the worker's shards in S-hat."""
    return sum(sh[1] for sh in document_shards(cu_seqlens, chunks) if not is_last_shard(cu_seqlens, sh))


def eq4_elements(total: int, n: int, h: int, d: int) -> float:
    """Eq. 4: the static full-KV pattern."""
    return 4.0 * total / n * h * d * (n - 1)


def eq5_elements(cu_seqlens, rank_chunks, h: int, d: int) -> float:
    """Eq. 5: the sharding-aware pattern (the largest worker's S-hat rows)."""
    n = len(rank_chunks)
    return 4.0 * max(sent_rows(cu_seqlens, ch) for ch in rank_chunks) * h * d * (n - 1)


def packed_send_buffer(kv_local: np.ndarray, cu_seqlens, chunks) -> np.ndarray:
    """The worker's continuous send buffer: rows of its S-hat shards, in its
    local order, no padding.  kv_local: [rows of the chunks concatenated, ...]."""
    pos = local_positions(chunks)
    keep = np.zeros(pos.size, dtype=bool)
    for g, s, dd, _ in document_shards(cu_seqlens, chunks):
        if not is_last_shard(cu_seqlens, (g, s, dd, 0)):
            keep |= (pos >= g) & (pos < g + s)
    return kv_local[keep]


def needed_positions(cu_seqlens, chunks, total: int) -> np.ndarray:
    """Boolean [total]: positions some token of the worker may attend."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    need = np.zeros(total, dtype=bool)
    pos = local_positions(chunks)
    if pos.size == 0:
        return need
    starts = cu[doc_index(cu, pos)]
    # prefix [start, token] of every token, as a difference array
    diff = np.zeros(total + 1, dtype=np.int64)
    np.add.at(diff, starts, 1)
    np.add.at(diff, pos + 1, -1)
    return np.cumsum(diff)[:total] > 0


def received_kv(kv_global: np.ndarray, cu_seqlens, chunks):
    """(kv_lo, kv_hi, buffer): the worker's KV over [kv_lo, kv_hi) = the span of
    its needed positions, holding the global rows where needed, zeros elsewhere."""
    total = kv_global.shape[0]
    need = needed_positions(cu_seqlens, chunks, total)
    idx = np.nonzero(need)[0]
    if idx.size == 0:
        return 0, 0, kv_global[:0].copy()
    lo, hi = int(idx[0]), int(idx[-1]) + 1
    buf = np.zeros_like(kv_global[lo:hi])
    buf[need[lo:hi]] = kv_global[lo:hi][need[lo:hi]]
    return lo, hi, buf
