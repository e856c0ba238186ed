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
