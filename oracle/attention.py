"""fp64 reference for document-masked attention: forward, merge, backward.

Test infrastructure only (see the package docstring).

Conventions (readings where the pages are silent):
* Q, O, dO, dQ: [Tq, Hq, D], local query rows = the chunks concatenated in list
  order; chunk c covers global positions [g_start, g_start + len).
* K, V, dK, dV: [Tkv, Hkv, D]; row r holds global position kv_lo + r.
* LSE: [Hq, Tq], natural log of the sum of exp(score) over allowed keys.
* GQA: query head h reads KV head h // (Hq // Hkv) (contiguous groups).
* A row with no allowed key in [kv_lo, kv_hi) has O = 0 and LSE = -inf.
"""
from __future__ import annotations

import numpy as np


def doc_index(cu_seqlens, positions) -> np.ndarray:
    """Document id of each global position: d such that cu[d] <= p < cu[d+1]."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    pos = np.asarray(positions, dtype=np.int64)
    return np.searchsorted(cu, pos, side="right") - 1


def local_positions(chunks) -> np.ndarray:
    """Global position of every local query row (chunks concatenated in order)."""
    parts = [np.arange(g, g + n, dtype=np.int64) for g, n in chunks]
    return np.concatenate(parts) if parts else np.zeros(0, np.int64)


def allowed_mask(cu_seqlens, q_pos, kv_lo: int, kv_hi: int) -> np.ndarray:
    """Explicit boolean document mask [len(q_pos), kv_hi - kv_lo].

    FlashCP paper, section 2.1 / Figure 1(a): a query attends only to keys of
    its own document that are not after it (intra-document causal mask).  The
    diagonal is included: the shard workload of section 3.1 and the causal pair
    count L(L+1)/2 of the CP-variance article both count it.
    """
    kv_pos = np.arange(kv_lo, kv_hi, dtype=np.int64)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    dq = doc_index(cu_seqlens, q_pos)
    dk = doc_index(cu_seqlens, kv_pos)
    return (dq[:, None] == dk[None, :]) & (kv_pos[None, :] <= q_pos[:, None])


def _as64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def attention_forward(q, k, v, cu_seqlens, chunks, kv_lo: int, kv_hi: int, scale: float,
                      rows=None, row_block: int = 256):
    """O [n, Hq, D] and LSE [Hq, n] for local rows ``rows`` (default: all).

    Per row i and head h: s_ij = scale * q_i . k_j for allowed j (explicit mask);
    LSE = ln sum_j exp(s_ij) (max-subtracted); O = sum_j exp(s_ij - LSE) v_j.
    Rows are processed ``row_block`` at a time only to bound memory; every row
    sees the whole key range [kv_lo, kv_hi) with its explicit mask.
    """
    q = _as64(q)
    k = _as64(k)
    v = _as64(v)
    tq, hq, d = q.shape
    hkv = k.shape[1]
    if hq % hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    if k.shape[0] != kv_hi - kv_lo:
        raise ValueError("K rows must equal kv_hi - kv_lo")
    g = hq // hkv
    pos = local_positions(chunks)
    if pos.size != tq:
        raise ValueError("Q rows must equal the total chunk length")
    rows = np.arange(tq) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((rows.size, hq, d))
    lse = np.full((hq, rows.size), -np.inf)
    for r0 in range(0, rows.size, row_block):
        rr = rows[r0:r0 + row_block]
        mask = allowed_mask(cu_seqlens, pos[rr], kv_lo, kv_hi)
        any_allowed = mask.any(axis=1)
        for h in range(hq):
            kh = h // g
            s = scale * (q[rr, h, :] @ k[:, kh, :].T)
            s = np.where(mask, s, -np.inf)
            m = np.where(any_allowed, s.max(axis=1, initial=-np.inf), 0.0)
            e = np.where(mask, np.exp(s - m[:, None]), 0.0)
            tot = e.sum(axis=1)
            with np.errstate(divide="ignore"):
                row_lse = np.where(any_allowed, m + np.log(np.where(any_allowed, tot, 1.0)), -np.inf)
            p = np.where(any_allowed[:, None], e / np.where(any_allowed, tot, 1.0)[:, None], 0.0)
            out[r0:r0 + rr.size, h, :] = p @ v[:, kh, :]
            lse[h, r0:r0 + rr.size] = row_lse
    return out, lse


def lse_merge(o_parts, lse_parts):
    """Combine partial results computed over disjoint KV ranges.

    Production guide, "Core Principle: Split Q, Circulate KV" and the ring
    attention steps: partials are combined with the row maximum and the
    exponential sum.  For each row: m = max_p LSE_p; LSE = m + ln sum_p
    exp(LSE_p - m); O = sum_p exp(LSE_p - LSE) O_p.  If every partial is empty
    (m = -inf) the row is (O = 0, LSE = -inf).

    o_parts: [P, rows, Hq, D]; lse_parts: [P, Hq, rows].
    """
    o = _as64(o_parts)
    lse = _as64(lse_parts)
    m = lse.max(axis=0)                                   # [Hq, rows]
    finite = np.isfinite(m)
    m0 = np.where(finite, m, 0.0)
    w = np.where(np.isfinite(lse), np.exp(lse - m0[None]), 0.0)  # [P, Hq, rows]
    tot = w.sum(axis=0)
    with np.errstate(divide="ignore"):
        out_lse = np.where(finite, m0 + np.log(np.where(finite, tot, 1.0)), -np.inf)
    coef = np.where(finite[None], w / np.where(finite, tot, 1.0)[None], 0.0)  # exp(LSE_p - LSE)
    out = np.einsum("phr,prhd->rhd", coef, o)
    return out, out_lse


def attention_backward(q, k, v, do, cu_seqlens, chunks, kv_lo: int, kv_hi: int, scale: float,
                       dq_key_range=None, row_block: int = 256):
    """Exact gradients (dQ, dK, dV) of L = <dO, O> for the forward above.

    The pages name the attention backward (FlashCP paper, Figure 6 latency
    breakdown, "Attention BWD") without writing it; this is plain calculus on
    the forward's definition, using the oracle's own float64 O and LSE:

      P_ij = exp(s_ij - LSE_i)          (0 where the mask forbids (i, j))
      Delta_i = sum_d dO_id O_id
      dP_ij = dO_i . v_j
      dS_ij = P_ij (dP_ij - Delta_i)
      dQ_i = scale sum_j dS_ij k_j
      dK_j = scale sum_{i, h in group(j)} dS_ij q_i
      dV_j = sum_{i, h in group(j)} P_ij dO_i

    ``dq_key_range=(lo, hi)`` (global positions) restricts the sum for dQ to keys
    in [lo, hi): the share of dQ a call holding only those keys contributes.
    """
    q = _as64(q)
    k = _as64(k)
    v = _as64(v)
    do = _as64(do)
    tq, hq, d = q.shape
    hkv = k.shape[1]
    g = hq // hkv
    o, lse = attention_forward(q, k, v, cu_seqlens, chunks, kv_lo, kv_hi, scale, row_block=row_block)
    pos = local_positions(chunks)
    kv_pos = np.arange(kv_lo, kv_hi, dtype=np.int64)
    if dq_key_range is None:
        key_sel = np.ones(kv_pos.size, dtype=bool)
    else:
        key_sel = (kv_pos >= dq_key_range[0]) & (kv_pos < dq_key_range[1])
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for r0 in range(0, tq, row_block):
        rr = np.arange(r0, min(tq, r0 + row_block))
        mask = allowed_mask(cu_seqlens, pos[rr], kv_lo, kv_hi)
        for h in range(hq):
            kh = h // g
            s = scale * (q[rr, h, :] @ k[:, kh, :].T)
            l_row = lse[h, rr]
            safe = np.where(np.isfinite(l_row), l_row, 0.0)
            p = np.where(mask, np.exp(np.where(mask, s, 0.0) - safe[:, None]), 0.0)
            delta = (do[rr, h, :] * o[rr, h, :]).sum(axis=1)
            dp = do[rr, h, :] @ v[:, kh, :].T
            ds = p * (dp - delta[:, None])
            dq[rr, h, :] = scale * (ds[:, key_sel] @ k[key_sel, kh, :])
            dk[:, kh, :] += scale * (ds.T @ q[rr, h, :])
            dv[:, kh, :] += p.T @ do[rr, h, :]
    return dq, dk, dv
