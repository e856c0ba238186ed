"""Pins of the KV-exchange oracle (FlashCP section 3.2, Eq. 4 and Eq. 5):
hand-worked plans, the pages' own limiting cases (a document kept whole needs
no communication; a single document sharded by sequence saves nothing), the
need set against the explicit mask, and the claim that only shards that are
not their document's last shard ever need to travel."""
import numpy as np
import pytest

import oracle
from document_masked_attention_amd.workloads import (cu_from_lengths, per_doc_chunks, sequence_zigzag_chunks,
                                                     random_plan)


def test_hand_worked_plan():
    # documents [0,6) [6,8) [8,12); worker 0: [0,4) and [10,12); worker 1: [4,10)
    cu = cu_from_lengths([6, 2, 4])
    plan = [[(0, 4), (10, 2)], [(4, 6)]]
    assert oracle.document_shards(cu, plan[0]) == [(0, 4, 0, 0), (10, 2, 2, 2)]
    assert oracle.document_shards(cu, plan[1]) == [(4, 2, 0, 4), (6, 2, 1, 0), (8, 2, 2, 0)]
    assert [oracle.is_last_shard(cu, s) for s in oracle.document_shards(cu, plan[1])] == [True, True, False]
    assert [oracle.sent_rows(cu, p) for p in plan] == [4, 2]
    h, d = 3, 5
    assert oracle.eq5_elements(cu, plan, h, d) == 4 * 4 * h * d * 1
    assert oracle.eq4_elements(12, 2, h, d) == 4 * 6 * h * d * 1
    kv = np.arange(12 * 2).reshape(12, 2)            # row p holds 2p, 2p + 1
    local1 = kv[4:10]
    assert np.array_equal(oracle.packed_send_buffer(local1, cu, plan[1]), kv[8:10])
    local0 = np.concatenate([kv[0:4], kv[10:12]])
    assert np.array_equal(oracle.packed_send_buffer(local0, cu, plan[0]), kv[0:4])
    # worker 1 needs [0,6) (doc 0 prefix of rows 4,5), [6,8), [8,10): all of [0,10)
    lo, hi, buf = oracle.received_kv(kv, cu, plan[1])
    assert (lo, hi) == (0, 10) and np.array_equal(buf, kv[0:10])
    # worker 0 needs [0,4) and [8,12): rows 4..7 are zero
    lo, hi, buf = oracle.received_kv(kv, cu, plan[0])
    assert (lo, hi) == (0, 12)
    want = kv.copy()
    want[4:8] = 0
    assert np.array_equal(buf, want)


def test_whole_documents_need_no_exchange():
    """Each document intact on one worker: no shard is sent (section 3.3, Figure 4(1))."""
    lengths = [300, 120, 77, 500, 3]
    cu = cu_from_lengths(lengths)
    plan = [[(0, 300), (420, 77)], [(300, 120), (497, 500)], [(997, 3)]]
    assert oracle.eq5_elements(cu, plan, 8, 128) == 0


@pytest.mark.parametrize("n", [2, 4, 8])
def test_one_document_sharded_by_sequence_saves_nothing(n):
    """One causal document in 2N chunks: worker 0 sends chunk 0 only (its
    chunk 2N-1 is the document's last shard), every other worker both chunks,
    so the largest send is T/N and Eq. 5 equals Eq. 4."""
    total = 2 * n * 64
    cu = cu_from_lengths([total])
    plan = [sequence_zigzag_chunks(total, n, r) for r in range(n)]
    assert [oracle.sent_rows(cu, p) for p in plan] == [64] + [128] * (n - 1)
    assert oracle.eq5_elements(cu, plan, 8, 128) == oracle.eq4_elements(total, n, 8, 128)


def test_needed_positions_match_the_mask():
    rng = np.random.default_rng(3)
    for case in range(30):
        lengths = [int(x) for x in rng.integers(0, 40, size=int(rng.integers(1, 8)))] + [int(rng.integers(1, 30))]
        cu = cu_from_lengths(lengths)
        total = int(cu[-1])
        plan = random_plan(rng, total, int(rng.integers(1, 5)), int(rng.integers(1, 9)))
        for chunks in plan:
            pos = oracle.local_positions(chunks)
            want = oracle.allowed_mask(cu, pos, 0, total).any(axis=0)
            assert np.array_equal(oracle.needed_positions(cu, chunks, total), want)


def test_only_non_last_shards_need_to_travel():
    """Every position a worker needs is its own or inside another worker's
    S-hat shards (the premise of Eq. 5)."""
    rng = np.random.default_rng(4)
    for case in range(40):
        lengths = [int(x) for x in rng.integers(1, 200, size=int(rng.integers(1, 12)))]
        cu = cu_from_lengths(lengths)
        total = int(cu[-1])
        n = int(rng.integers(2, 6))
        plan = random_plan(rng, total, n, int(rng.integers(n, 4 * n)))
        sent = np.zeros((n, total), dtype=bool)
        own = np.zeros((n, total), dtype=bool)
        for r, chunks in enumerate(plan):
            for g, s, dd, _ in oracle.document_shards(cu, chunks):
                own[r, g:g + s] = True
                if not oracle.is_last_shard(cu, (g, s, dd, 0)):
                    sent[r, g:g + s] = True
        assert np.all(own.sum(axis=0) == 1)
        for r, chunks in enumerate(plan):
            need = oracle.needed_positions(cu, chunks, total)
            avail = own[r] | np.delete(sent, r, axis=0).any(axis=0)
            assert not np.any(need & ~avail)


def test_per_doc_pieces_send_all_but_last_pieces():
    lengths = [64, 32, 128]
    cu = cu_from_lengths(lengths)
    plan = [per_doc_chunks(lengths, 4, r) for r in range(4)]
    # worker 0 holds piece 7 of each document (its last shard): sends only piece 0 of each
    assert oracle.sent_rows(cu, plan[0]) == 8 + 4 + 16
    for r in range(1, 4):
        assert oracle.sent_rows(cu, plan[r]) == 2 * (8 + 4 + 16)
