"""Pins for the reference scheduler (CPU only): explicit-mask brute force,
the pages' closed-form workloads, contiguity of every reported interval, and
the LPT order definition."""
import numpy as np
import pytest

import oracle
from document_masked_attention_amd.workloads import random_lengths, cu_from_lengths, make_config


def _random_problem(rng):
    total = int(rng.integers(1, 160))
    lengths = random_lengths(rng, total, int(rng.integers(1, 60)), p_one=0.2)
    cu = cu_from_lengths(lengths)
    # ascending disjoint chunks
    cuts = np.sort(rng.choice(np.arange(total + 1), size=min(total + 1, 2 * int(rng.integers(1, 4))), replace=False))
    chunks = [(int(a), int(b - a)) for a, b in zip(cuts[::2], cuts[1::2]) if b > a]
    if not chunks:
        chunks = [(0, total)]
    lo = int(rng.integers(0, total))
    hi = int(rng.integers(lo + 1, total + 1))
    bq = int(rng.choice([1, 2, 3, 8, 16, 32]))
    bk = int(rng.choice([1, 4, 5, 16, 64]))
    return cu, chunks, lo, hi, bq, bk


def test_interval_counts_equal_explicit_mask_bruteforce():
    rng = np.random.default_rng(0)
    for _ in range(1500):
        cu, chunks, lo, hi, bq, bk = _random_problem(rng)
        a = oracle.tile_pair_counts_bruteforce(cu, chunks, lo, hi, bq, bk)
        b = oracle.tile_pair_counts(cu, chunks, lo, hi, bq, bk)
        assert np.array_equal(a, b)
        s = oracle.schedule(cu, chunks, lo, hi, bq, bk, counts=a)   # raises if a set is not an interval
        assert s["counters"][3] == oracle.useful_pairs(cu, chunks, lo, hi) == a.sum()
        cls = s["classes"]
        for t, (klo, kflo, kfhi, khi) in enumerate(s["qtile_desc"]):
            ns = np.nonzero(cls[t])[0]
            if ns.size == 0:
                assert (klo, kflo, kfhi, khi) == (0, 0, 0, 0)
                continue
            assert (klo, khi) == (ns[0], ns[-1] + 1)
            full = np.nonzero(cls[t] == 1)[0]
            if full.size:
                assert (kflo, kfhi) == (full[0], full[-1] + 1)
            else:
                assert kflo == kfhi == khi


def test_need_interval_bruteforce():
    rng = np.random.default_rng(1)
    for _ in range(500):
        cu, chunks, lo, hi, _, _ = _random_problem(rng)
        need = oracle.need_intervals(cu, chunks, lo, hi)
        for c, (g, n) in enumerate(chunks):
            m = oracle.allowed_mask(cu, np.arange(g, g + n), lo, hi).any(axis=0)
            keys = np.nonzero(m)[0] + lo
            want = (keys[0], keys[-1] + 1) if keys.size else (0, 0)
            assert tuple(need[c]) == want


def test_useful_pairs_match_shard_workload_formula():
    """FlashCP paper, section 3.1: a shard of length s with p same-document tokens
    before it has W = (2p + s + 1) s / 2 unmasked pairs (diagonal included)."""
    rng = np.random.default_rng(2)
    for _ in range(300):
        total = int(rng.integers(1, 400))
        lengths = random_lengths(rng, total, 120)
        cu = cu_from_lengths(lengths)
        cuts = np.sort(rng.choice(np.arange(total + 1), size=2, replace=False))
        chunks = [(int(cuts[0]), int(cuts[1] - cuts[0]))]
        g0, g1 = cuts
        w = 0
        for a, b in zip(cu[:-1], cu[1:]):
            s0, s1 = max(a, g0), min(b, g1)
            if s1 > s0:
                p, s = s0 - a, s1 - s0
                w += (2 * p + s + 1) * s // 2
        assert oracle.useful_pairs(cu, chunks, 0, total) == w


def test_causal_pair_count_closed_form():
    """CP-variance article, "Theory": a causal document of length L has L(L+1)/2 pairs."""
    w = make_config(1)
    want = sum(n * (n + 1) // 2 for n in w.lengths)
    assert want == 721920
    assert oracle.useful_pairs(w.cu_seqlens, w.chunks, w.kv_lo, w.kv_hi) == want
    s = oracle.schedule(w.cu_seqlens, w.chunks, w.kv_lo, w.kv_hi, 128, 64)
    assert s["counters"][3] == want


def test_lpt_order_definition():
    rng = np.random.default_rng(3)
    for _ in range(200):
        w = rng.integers(0, 5, size=int(rng.integers(0, 40)))
        got = oracle.lpt_order(w).tolist()
        assert got == sorted(range(len(w)), key=lambda i: (-int(w[i]), i))


def test_cp_rank_need_list_blocks():
    """The 2 x CP chunk of rank 3 at CP = 8 (chunks 3 and 12 of 16) needs KV from
    the start of its first row's document up to its own end."""
    w = make_config(3)
    need = oracle.need_intervals(w.cu_seqlens, w.chunks, w.kv_lo, w.kv_hi)
    cu = w.cu_seqlens
    for (g, n), (lo, hi) in zip(w.chunks, need):
        d = np.searchsorted(cu, g, side="right") - 1
        assert (lo, hi) == (cu[d], g + n)


def test_classify_counters_of_the_2048_token_workload_by_hand():
    """Tile classes of the 2048-token workload (documents 512, 1024, 256, 256) at
    128 x 64 tiles, derived from the mask definition without counting pairs
    (production guide, "Causal Attention Creates Rank Load Imbalance": skip
    blocks with no valid pair, log the effective block count).

    Every document boundary is a multiple of 128, so each Q tile [r0, r0 + 128)
    lies inside one document with start ds.  Its rows attend keys [ds, r1), so
    its non-skipped KV tiles are 64-key tiles ds/64 .. r1/64 - 1.  A KV tile
    [c0, c0 + 64) is FULL when every row sees every key: c0 >= ds and
    c0 + 63 <= r0, i.e. tiles ds/64 .. r0/64 - 1, (r0 - ds)/64 of them.  The two
    tiles over [r0, r0 + 128) hold the diagonal: key c0 + 1 is not seen by row
    c0, so they are PARTIAL.  FULL per document: 512 -> 0+2+4+6 = 12;
    1024 -> 0+2+...+14 = 56; 256 -> 0+2 = 2 (twice): 72.  PARTIAL: 16 Q tiles x
    2 = 32.  Non-skipped: 104.  Allowed pairs (CP-variance article, "Theory"):
    sum L(L+1)/2 = 721,920."""
    w = make_config(1)
    s = oracle.schedule(w.cu_seqlens, w.chunks, w.kv_lo, w.kv_hi, 128, 64)
    assert s["counters"].tolist() == [104, 72, 32, 721920]
    starts = [0, 512, 1536, 1792]
    want_q = []
    for t in range(16):
        r0 = 128 * t
        ds = max(x for x in starts if x <= r0)
        lo, hi = ds // 64, (r0 + 128) // 64
        full_hi = r0 // 64
        want_q.append((lo, lo, full_hi, hi) if full_hi > lo else (lo, hi, hi, hi))
    assert [tuple(r) for r in s["qtile_desc"].tolist()] == want_q
    # a KV tile [c0, c0 + 64) in a document [ds, de) is attended by Q tiles
    # c0 // 128 .. de/128 - 1; FULL for the ones that start at or after c0 + 64
    ends = [512, 1536, 1792, 2048]
    want_kv = []
    for j in range(32):
        c0 = 64 * j
        de = min(x for x in ends if x > c0)
        lo, hi = c0 // 128, de // 128
        flo = (c0 + 64 + 127) // 128
        want_kv.append((lo, flo, hi, hi) if flo < hi else (lo, hi, hi, hi))
    assert [tuple(r) for r in s["kvtile_desc"].tolist()] == want_kv


def test_classify_ragged_two_chunk_case_by_hand():
    """A case small enough to classify by hand: documents [0, 5), [5, 13),
    [13, 20); query chunks rows 3..8 (starting inside document 0, crossing into
    document 1) and rows 15..19 (inside document 2); KV range [2, 18) cutting
    documents 0 and 2; bq = 4, bk = 3, so the last Q tile of each chunk and the
    last KV tile are ragged.

    Q tiles (anchored at each chunk start): rows {3,4,5,6}, {7,8}, {15,16,17,18},
    {19}.  KV tiles (anchored at 2): [2,5) [5,8) [8,11) [11,14) [14,17) [17,18).
    Allowed keys per row (same document, not after the row, inside [2, 18)):
      3: 2-3   4: 2-4   5: 5   6: 5-6   7: 5-7   8: 5-8
      15: 13-15   16: 13-16   17: 13-17   18: 13-17   19: 13-17
    Allowed pairs per (Q tile, KV tile) and the tile size (rows x keys):
      tile {3..6}:   [2,5) 2+3 = 5 of 12 P;  [5,8) 1+2 = 3 of 12 P
      tile {7,8}:    [5,8) 3+3 = 6 of 6 F;   [8,11) 0+1 = 1 of 6 P
      tile {15..18}: [11,14) 4 of 12 P;  [14,17) 2+3+3+3 = 11 of 12 P;
                     [17,18) 0+0+1+1 = 2 of 4 P
      tile {19}:     [11,14) 1 of 3 P;   [14,17) 3 of 3 F;   [17,18) 1 of 1 F
    (P = PARTIAL, F = FULL; every other pair is SKIP)."""
    cu = [0, 5, 13, 20]
    chunks = [(3, 6), (15, 5)]
    s = oracle.schedule(cu, chunks, 2, 18, 4, 3)
    assert oracle.q_tiles(chunks, 4) == [(0, 0, 3, 4), (0, 4, 7, 2), (1, 6, 15, 4), (1, 10, 19, 1)]
    assert oracle.kv_tiles(2, 18, 3) == [(2, 5), (5, 8), (8, 11), (11, 14), (14, 17), (17, 18)]
    S, F, P = 0, 1, 2
    assert s["classes"].tolist() == [[P, P, S, S, S, S],
                                     [S, F, P, S, S, S],
                                     [S, S, S, P, P, P],
                                     [S, S, S, P, F, F]]
    # {kt_lo, kt_full_lo, kt_full_hi, kt_hi}; no FULL tile -> full_lo = full_hi = hi
    assert s["qtile_desc"].tolist() == [[0, 2, 2, 2], [1, 1, 2, 3], [3, 6, 6, 6], [3, 4, 6, 6]]
    assert s["kvtile_desc"].tolist() == [[0, 1, 1, 1], [0, 1, 2, 2], [1, 2, 2, 2],
                                         [2, 4, 4, 4], [2, 3, 4, 4], [2, 3, 4, 4]]
    # need: from the document start of the chunk's first row (clipped to kv_lo)
    # up to the chunk end (clipped to kv_hi)
    assert s["need"].tolist() == [[2, 9], [13, 18]]
    # 10 non-skipped, 3 FULL, 7 PARTIAL; allowed pairs 2+3+1+2+3+4+3+4+5+5+5 = 37
    assert s["counters"].tolist() == [10, 3, 7, 37]
    # LPT: by descending non-skipped count (Q tiles 2, 2, 3, 3; KV tiles 1, 2, 1, 2, 2, 2), ties ascending
    assert s["lpt_q"].tolist() == [2, 3, 0, 1]
    assert s["lpt_kv"].tolist() == [1, 3, 4, 5, 0, 2]
