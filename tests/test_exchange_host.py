"""Host-side exchange planning of the library (send and receive row maps)
against the oracle, on the CPU: the maps are applied with numpy slicing here,
so this checks which rows travel and where they land (needed rows from the
oracle; zeros over the rest of each 128-row block that holds one, nothing
written elsewhere); the GPU copy of the same maps is checked in
test_gpu_exchange.py."""
import numpy as np
import pytest

import oracle
from document_masked_attention_amd import api
from placement_util import check_placement
from document_masked_attention_amd.workloads import (cu_from_lengths, per_doc_chunks, sequence_zigzag_chunks,
                                                     random_plan, lognormal_docs)


def _apply(maps, src, dst):
    for s, d, n in maps:
        dst[d:d + n] = 0 if s == -1 else src[s:s + n]
    return dst


def _plans():
    rng = np.random.default_rng(8)
    out = []
    lengths = [10]
    out.append((lengths, [per_doc_chunks(lengths, 2, r) for r in range(2)]))
    lengths = [6, 2, 4]
    out.append((lengths, [[(0, 4), (10, 2)], [(4, 6)]]))
    lengths = [64, 32, 128, 1, 7]
    out.append((lengths, [per_doc_chunks(lengths, 4, r) for r in range(4)]))
    out.append(([232], [sequence_zigzag_chunks(232 - 232 % 8, 4, r) for r in range(4)]))
    for case in range(25):
        lengths = [int(x) for x in rng.integers(0, 300, size=int(rng.integers(1, 15)))] + [int(rng.integers(1, 99))]
        total = sum(lengths)
        n = int(rng.integers(1, 7))
        out.append((lengths, random_plan(rng, total, n, int(rng.integers(0, 5 * n)))))
    lengths = lognormal_docs(5, 512, 1.2, 16, 8192, 16384)
    out.append((lengths, [per_doc_chunks(lengths, 8, r) for r in range(8)]))
    return out


@pytest.mark.parametrize("case", range(30))
def test_maps_against_oracle(case):
    lengths, plan = _plans()[case]
    cu = cu_from_lengths(lengths)
    total = int(cu[-1])
    if sum(n for ch in plan for _, n in ch) != total:          # the per-sequence case trims the tail
        lengths = [sum(n for ch in plan for _, n in ch)]
        cu = cu_from_lengths(lengths)
        total = int(cu[-1])
    kv = np.random.default_rng(case).integers(1, 1 << 30, size=(total, 3))   # nonzero rows
    packed = []
    for chunks in plan:
        local = kv[oracle.local_positions(chunks)]
        maps, rows = api.exchange_send_maps(cu, chunks)
        want = oracle.packed_send_buffer(local, cu, chunks)
        assert rows == oracle.sent_rows(cu, chunks) == want.shape[0]
        got = _apply(maps, local, np.zeros((rows, 3), kv.dtype))
        assert np.array_equal(got, want)
        packed.append(want)
    slot = max([p.shape[0] for p in packed] + [1])
    gathered = np.zeros((len(plan) * slot, 3), kv.dtype)
    for k, p in enumerate(packed):
        gathered[k * slot:k * slot + p.shape[0]] = p
    for r, chunks in enumerate(plan):
        m = api.exchange_recv_maps(cu, plan, r, slot)
        lo, hi, want = oracle.received_kv(kv, cu, chunks)
        assert (m["kv_lo"], m["kv_hi"]) == (lo, hi)
        dsts = [d for _, d, _ in m["remote"]]
        assert dsts == sorted(dsts)
        buf = _apply(m["remote"], gathered, np.full((hi - lo, 3), -1, kv.dtype))
        buf = _apply(m["local"], kv[oracle.local_positions(chunks)], buf)
        need = oracle.needed_positions(cu, chunks, total)[lo:hi]
        check_placement(buf, want, need, -1, f"rank {r}")


def test_planning_rejects_bad_plans():
    cu = cu_from_lengths([10, 6])
    good = [[(0, 8)], [(8, 8)]]
    api.exchange_recv_maps(cu, good, 0, 8)
    for bad, slot in (([[(0, 8)], [(9, 7)]], 8),          # position 8 held by nobody
                      ([[(0, 9)], [(8, 8)]], 8),          # position 8 held twice
                      ([[(8, 8)], [(0, 8)]], 0),          # slot smaller than a worker's send rows
                      ([[(4, 4), (0, 4)], [(8, 8)]], 8)):  # chunks out of order
        with pytest.raises(api.DocmaskError):
            api.exchange_recv_maps(cu, bad, 0, slot)
    with pytest.raises(api.DocmaskError):
        api.exchange_send_maps(cu, [(10, 7)])              # past the sequence end
    with pytest.raises(api.DocmaskError):
        api.exchange_recv_maps(cu, good, 2, 8)             # no such rank
