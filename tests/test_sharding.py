"""2 x CP chunk lists (FlashCP section 2.3: each document, or the whole
sequence, cut into 2N chunks, worker i holding chunks i and 2N-1-i), checked
on the CPU: exact partition, the assignment rule on hand-worked cases, and the
balance property that motivates the pattern, counted by the oracle."""
import numpy as np
import pytest

import oracle
from document_masked_attention_amd.workloads import (per_doc_chunks, sequence_zigzag_chunks, doc_piece_bounds,
                                                     fig3_workload, fig3_lengths, FIG3_PATTERNS, cu_from_lengths)


def _owner(lengths, cp):
    """Rank owning every global position, from the chunk lists of all ranks."""
    total = sum(lengths)
    own = np.full(total, -1)
    for r in range(cp):
        for g, n in per_doc_chunks(lengths, cp, r):
            assert n > 0 and np.all(own[g:g + n] == -1), "chunks overlap"
            own[g:g + n] = r
    return own


def test_hand_worked_pieces():
    # L = 10, cp = 2: four pieces [0,2) [2,5) [5,7) [7,10)
    assert doc_piece_bounds(10, 2) == [0, 2, 5, 7, 10]
    assert per_doc_chunks([10], 2, 0) == [(0, 2), (7, 3)]
    assert per_doc_chunks([10], 2, 1) == [(2, 3), (5, 2)]          # adjacent pieces stay two chunks
    # two documents, the second offset by the first's length
    assert per_doc_chunks([8, 4], 2, 1) == [(2, 2), (4, 2), (9, 1), (10, 1)]
    # a document shorter than 2cp leaves empty pieces, which are dropped
    assert per_doc_chunks([3], 2, 0) == [(2, 1)]                   # bounds 0,0,1,2,3: piece 0 empty
    assert per_doc_chunks([3], 2, 1) == [(0, 1), (1, 1)]
    assert sequence_zigzag_chunks(64, 4, 1) == [(8, 8), (48, 8)]
    with pytest.raises(ValueError):
        sequence_zigzag_chunks(60, 4, 0)


@pytest.mark.parametrize("cp", [1, 2, 3, 8])
def test_partition_and_rule(cp):
    rng = np.random.default_rng(cp)
    lengths = [int(x) for x in rng.integers(1, 300, size=40)] + [1, 2 * cp - 1, 2 * cp]
    own = _owner(lengths, cp)
    assert np.all(own >= 0), "a position is held by no rank"
    cu = cu_from_lengths(lengths)
    for di, length in enumerate(lengths):
        for t in range(length):                       # piece index of local row t, from floor(i L / 2cp) <= t
            piece = max(i for i in range(2 * cp) if (i * length) // (2 * cp) <= t)
            want = piece if piece < cp else 2 * cp - 1 - piece
            assert own[cu[di] + t] == want


@pytest.mark.parametrize("cp", [2, 4, 8])
def test_per_doc_balance_closed_form(cp):
    """Every document divisible into 2cp pieces of c rows gives every rank
    (2cp - 1) c^2 + c (c + 1) allowed pairs from it: piece i's rows see i*c
    earlier keys of the document plus a causal triangle."""
    lengths = [2 * cp * c for c in (1, 3, 8, 17, 64)]
    cu = cu_from_lengths(lengths)
    total = int(cu[-1])
    want = sum((2 * cp - 1) * (L // (2 * cp)) ** 2 + (L // (2 * cp)) * (L // (2 * cp) + 1) for L in lengths)
    for r in range(cp):
        assert oracle.useful_pairs(cu, per_doc_chunks(lengths, cp, r), 0, total) == want


def test_per_doc_balance_bruteforce_tiny():
    lengths = [12, 4, 8]
    cu = cu_from_lengths(lengths)
    pairs = []
    for r in range(2):
        chunks = per_doc_chunks(lengths, 2, r)
        pos = oracle.local_positions(chunks)
        pairs.append(int(oracle.allowed_mask(cu, pos, 0, 24).sum()))
    # hand count: c = 3, 1, 2 per piece -> 3*9+12, 3*1+2, 3*4+6 = 39 + 5 + 18
    assert pairs == [62, 62]


def test_per_sequence_imbalance_on_mixed_documents():
    """Whole-sequence chunks balance one causal document but not a mix of
    lengths: the pattern of the pages' motivation."""
    cu1 = cu_from_lengths([4096])
    p1 = [oracle.useful_pairs(cu1, sequence_zigzag_chunks(4096, 4, r), 0, 4096) for r in range(4)]
    assert len(set(p1)) == 1
    lengths = [3000, 200, 300, 596]
    cu = cu_from_lengths(lengths)
    ps = [oracle.useful_pairs(cu, sequence_zigzag_chunks(4096, 4, r), 0, 4096) for r in range(4)]
    pd = [oracle.useful_pairs(cu, per_doc_chunks(lengths, 4, r), 0, 4096) for r in range(4)]
    assert max(ps) / np.mean(ps) > 1.5
    assert max(pd) / np.mean(pd) < 1.01


def test_study_workloads():
    for pattern in FIG3_PATTERNS:
        lengths = fig3_lengths(pattern)
        assert sum(lengths) == 131072
        for r in (0, 3, 7):
            a = fig3_workload(pattern, "per_doc", 8, r)
            b = fig3_workload(pattern, "per_sequence", 8, r)
            assert a.lengths == b.lengths == lengths and b.chunks == sequence_zigzag_chunks(131072, 8, r)
            assert len(a.chunks) <= 256
            if pattern == "1x131072":
                assert a.chunks == b.chunks
    assert len(fig3_workload("16x8192", "per_doc", 8, 3).chunks) == 32
