"""Pins of the Algorithm 1 planner oracle (FlashCP sections 3.1, 3.3, 3.4):
the shard workload against explicit-mask pair counts, two plans traced by
hand through the algorithm, the pages' limiting cases (two equal documents
stay whole, one dominant document goes Per-Doc), and the constraints every
plan must meet (Eq. 1 cover, Eq. 2 equal tokens, the target ratio), with the
ratio recounted from the explicit mask."""
import numpy as np
import pytest

import oracle
from document_masked_attention_amd.workloads import cu_from_lengths, lognormal_docs, bimodal_docs


def test_shard_workload_is_the_pair_count():
    rng = np.random.default_rng(0)
    for _ in range(200):
        p, s = int(rng.integers(0, 300)), int(rng.integers(0, 300))
        cu = cu_from_lengths([p + s + int(rng.integers(0, 5))])
        assert oracle.shard_workload(p, s) == oracle.useful_pairs(cu, [(p, s)], 0, int(cu[-1]))


def test_hand_traced_plans():
    # D = [5, 3, 2, 2], N = 2.  LPT by workload: d0 -> w0 (15), d1, d2, d3 -> w1
    # (6, 9, 12); tokens 5 / 7 against 6 / 6: w1 gives back d3; its head (1
    # token) fills w1 again (load 10), its tail (p = 1) goes to w0 (W = 2,
    # load 17); ratio 17 * 2 / 27.
    per_doc, whole, ratio = oracle.flashcp_plan([5, 3, 2, 2], 2, 1.5)
    assert per_doc == [] and whole == [[(0, 0, 5), (3, 1, 1)], [(1, 0, 3), (2, 0, 2), (3, 0, 1)]]
    assert ratio == 34 / 27
    # R = 1.2: 34/27 > 1.2, so d0 goes Per-Doc: pieces [0,1) [1,2) [2,3) [3,5);
    # w0 holds pieces 0 and 3 (W = 1 + 9), w1 pieces 1 and 2 (W = 2 + 3); token
    # targets 6 - 3 = 3 and 6 - 2 = 4.  d1 -> w1 (11), d2 -> w0 (13), d3 -> w1
    # (14); w1 gives back d3: head (1 token) to w1 (12), tail to w0 (15).
    chunks, per_doc, ratio = oracle.plan_chunks([5, 3, 2, 2], 2, 1.2)
    assert per_doc == [0] and ratio == 30 / 27
    assert chunks == [[(0, 1), (3, 2), (8, 2), (11, 1)], [(1, 2), (5, 3), (10, 1)]]


def test_two_equal_documents_stay_whole():
    """Figure 4(1): each document intact on its own worker, nothing exchanged."""
    cu = cu_from_lengths([4096, 4096])
    chunks, per_doc, ratio = oracle.plan_chunks([4096, 4096], 2, 1.01)
    assert per_doc == [] and ratio == 1.0 and chunks == [[(0, 4096)], [(4096, 4096)]]
    assert oracle.eq5_elements(cu, chunks, 8, 128) == 0


def test_dominant_document_goes_per_doc():
    """A document holding most tokens cannot be balanced whole (section 3.4,
    'Combine Per-Doc and Whole-Doc Sharding')."""
    lengths = [100] * 20 + [30000]
    chunks, per_doc, ratio = oracle.plan_chunks(lengths, 4, 1.05)
    assert per_doc == [20] and ratio <= 1.05


def _check_plan(lengths, n, r):
    chunks, per_doc, ratio = oracle.plan_chunks(lengths, n, r)
    cu = cu_from_lengths(lengths)
    total = int(cu[-1])
    held = np.zeros(total, dtype=np.int64)
    for ch in chunks:
        prev = -1
        for g, s in ch:
            assert s > 0 and g > prev
            held[g:g + s] += 1
            prev = g + s
    assert np.all(held == 1)                                         # Eq. 1: every token on one worker
    toks = [sum(s for _, s in ch) for ch in chunks]
    # Eq. 2: equal up to one token, unless Per-Doc rounding alone already
    # leaves more (each Per-Doc document shifts a worker by less than 2)
    assert max(toks) - min(toks) <= (1 if not per_doc else 1 + 2 * len(per_doc))
    loads = [oracle.useful_pairs(cu, ch, 0, total) for ch in chunks]    # recounted by the explicit mask
    assert ratio == oracle.imbalance_ratio(loads)
    nonempty = [i for i, L in enumerate(lengths) if L > 0]
    assert ratio <= r or sorted(per_doc) == sorted(nonempty)
    return chunks, per_doc, ratio


@pytest.mark.parametrize("n", [2, 3, 4, 8])
def test_random_plans_meet_the_constraints(n):
    rng = np.random.default_rng(n)
    for case in range(40):
        lengths = [int(x) for x in rng.integers(0, 600, size=int(rng.integers(1, 25)))]
        if rng.random() < 0.3:
            lengths.append(int(rng.integers(2000, 6000)))
        _check_plan(lengths, n, float(rng.choice([1.0, 1.02, 1.1, 1.5])))


def test_study_workloads_plan():
    for lengths in (bimodal_docs(5), lognormal_docs(3, 2048, 1.5, 64, 131072, 131072), [8192] * 16, [131072]):
        chunks, per_doc, ratio = oracle.plan_chunks(lengths, 8, 1.05)
        assert ratio <= 1.05
        assert all(sum(s for _, s in ch) == 16384 for ch in chunks)
    # sixteen equal documents: two whole documents per worker, nothing travels
    chunks, per_doc, _ = oracle.plan_chunks([8192] * 16, 8, 1.05)
    assert per_doc == [] and all(len(ch) <= 2 for ch in chunks)
