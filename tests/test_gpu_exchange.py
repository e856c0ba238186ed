"""KV exchange on the GPU: the row-copy kernel against numpy slicing, and the
whole single-GPU side of the sharding-aware exchange (pack the rows a worker
sends, place gathered rows at their positions) against the oracle, bit for
bit, followed by forward and backward over the placed KV against the oracle,
with every row the placement leaves untouched holding NaN."""
import numpy as np
import pytest
import torch

import oracle
from document_masked_attention_amd import api
from document_masked_attention_amd.workloads import (custom_workload, per_doc_chunks, random_plan, fig3_workload,
                                                     sequence_zigzag_chunks, draw_tensor)
from gpu_util import to_dev, bf16_to_np, f64, assert_close, O_TOL, LSE_TOL
from placement_util import check_placement

pytestmark = pytest.mark.gpu

NAN_BITS = 0x7FC0          # bf16 quiet NaN


def _random_maps(rng, src_rows, dst_rows, n):
    """Disjoint ascending destination runs; about one in five writes zeros (source -1)."""
    pts = np.sort(rng.choice(dst_rows + 1, size=min(2 * n, dst_rows + 1), replace=False))
    maps = []
    for j in range(0, len(pts) - 1, 2):
        d, e = int(pts[j]), int(pts[j + 1])
        length = min(e - d, src_rows)
        src = -1 if rng.random() < 0.2 else int(rng.integers(0, src_rows - length + 1))
        maps.append((src, d, length))
    return maps


@pytest.mark.parametrize("row_bytes", [16, 48, 256, 2048, 4096])
def test_copy_rows_random(row_bytes):
    rng = np.random.default_rng(row_bytes)
    for case in range(6):
        src_rows, dst_rows = int(rng.integers(1, 3000)), int(rng.integers(1, 3000))
        maps = _random_maps(rng, src_rows, dst_rows, int(rng.integers(0, 300)))
        zero, two = case % 2 == 0, case % 3 != 0
        print(f"[copy] row_bytes={row_bytes} case={case} maps={len(maps)} zero={zero} two={two}", flush=True)
        w = row_bytes // 4
        sk = torch.from_numpy(rng.integers(1, 1 << 30, size=(src_rows, w), dtype=np.int32)).cuda()
        sv = torch.from_numpy(rng.integers(1, 1 << 30, size=(src_rows, w), dtype=np.int32)).cuda() if two else None
        dk = torch.full((dst_rows, w), -5, dtype=torch.int32, device="cuda")
        dv = torch.full((dst_rows, w), -6, dtype=torch.int32, device="cuda") if two else None
        api.copy_rows(sk, sv, dk, dv, maps, zero)
        torch.cuda.synchronize()
        for src, dst, fill in ((sk, dk, -5), (sv, dv, -6)):
            if src is None:
                continue
            want = np.full((dst_rows, w), 0 if zero else fill, dtype=np.int32)
            s_np = src.cpu().numpy()
            for s, d, n in maps:
                want[d:d + n] = 0 if s == -1 else s_np[s:s + n]
            assert np.array_equal(dst.cpu().numpy(), want)


def test_copy_rows_zero_fill_only_and_large():
    d = torch.full((5000, 512), 7, dtype=torch.int32, device="cuda")
    api.copy_rows(d[:0], None, d, None, [], True)                       # no maps: zero everything
    torch.cuda.synchronize()
    assert int(d.abs().sum().item()) == 0
    # one long map over 2^20 + 3 rows of 2 KiB (several spans per block, ragged end)
    n = (1 << 20) + 3
    s = torch.arange(n * 512, dtype=torch.int32, device="cuda").view(n, 512)
    t = torch.empty((n + 10, 512), dtype=torch.int32, device="cuda")
    api.copy_rows(s, None, t, None, [(0, 10, n)], True)
    torch.cuda.synchronize()
    assert torch.equal(t[10:], s) and int(t[:10].abs().sum().item()) == 0


def _exchange(plan, lengths, hkv, d, seed):
    """Pack every worker's rows, gather (plain tensor copies), place them for
    each worker; returns the per-worker placements and maps."""
    from document_masked_attention_amd.workloads import cu_from_lengths
    cu = cu_from_lengths(lengths)
    total = int(cu[-1])
    kg = draw_tensor(seed, "k", total, hkv, d)
    vg = draw_tensor(seed, "v", total, hkv, d)
    packed, rows = [], []
    for chunks in plan:
        pos = oracle.local_positions(chunks)
        kl, vl = to_dev(kg[pos]), to_dev(vg[pos])
        maps, n = api.exchange_send_maps(cu, chunks)
        pk = torch.empty((n, hkv, d), dtype=torch.bfloat16, device="cuda")
        pv = torch.empty_like(pk)
        api.copy_rows(kl, vl, pk, pv, maps, False)
        torch.cuda.synchronize()
        assert np.array_equal(pk.view(torch.int16).cpu().numpy().view(np.uint16),
                              oracle.packed_send_buffer(kg[pos], cu, chunks))
        assert np.array_equal(pv.view(torch.int16).cpu().numpy().view(np.uint16),
                              oracle.packed_send_buffer(vg[pos], cu, chunks))
        packed.append((pk, pv, kl, vl))
        rows.append(n)
    slot = max(rows + [1])
    gk = torch.zeros((len(plan) * slot, hkv, d), dtype=torch.bfloat16, device="cuda")
    gv = torch.zeros_like(gk)
    for r, (pk, pv, _, _) in enumerate(packed):                     # stands in for the all-gather
        gk[r * slot:r * slot + pk.shape[0]] = pk
        gv[r * slot:r * slot + pv.shape[0]] = pv
    out = []
    for r, chunks in enumerate(plan):
        m = api.exchange_recv_maps(cu, plan, r, slot)
        lo, hi = m["kv_lo"], m["kv_hi"]
        # rows the placement must not write hold NaN: attention over the
        # placed KV then proves that no kernel reads them
        bk = torch.full((hi - lo, hkv, d), NAN_BITS, dtype=torch.int16, device="cuda").view(torch.bfloat16)
        bv = torch.full((hi - lo, hkv, d), NAN_BITS, dtype=torch.int16, device="cuda").view(torch.bfloat16)
        api.copy_rows(gk, gv, bk, bv, m["remote"], False)
        api.copy_rows(packed[r][2], packed[r][3], bk, bv, m["local"], False)
        torch.cuda.synchronize()
        need = oracle.needed_positions(cu, chunks, total)[lo:hi]
        for buf, glob in ((bk, kg), (bv, vg)):
            wlo, whi, want = oracle.received_kv(glob, cu, chunks)
            assert (wlo, whi) == (lo, hi)
            check_placement(buf.view(torch.int16).cpu().numpy().view(np.uint16), want, need, NAN_BITS, f"rank {r}")
        out.append((chunks, lo, hi, bk, bv))
    return cu, out


@pytest.mark.parametrize("kind", ["per_doc", "per_sequence", "random", "flashcp"])
def test_exchange_then_attention_small(kind):
    rng = np.random.default_rng({"per_doc": 1, "per_sequence": 2, "random": 3, "flashcp": 4}[kind])
    n = 4
    if kind == "flashcp":
        lengths = [int(x) for x in rng.integers(1, 200, size=10)] + [900]
        plan = oracle.plan_chunks(lengths, n, 1.05)[0]
    elif kind == "per_sequence":
        lengths = [int(x) for x in rng.integers(1, 200, size=6)]
        lengths[-1] += (-sum(lengths)) % (2 * n)
        plan = [sequence_zigzag_chunks(sum(lengths), n, r) for r in range(n)]
    elif kind == "per_doc":
        lengths = [int(x) for x in rng.integers(1, 300, size=7)] + [3]
        plan = [per_doc_chunks(lengths, n, r) for r in range(n)]
    else:
        lengths = [int(x) for x in rng.integers(0, 250, size=8)] + [5]
        plan = random_plan(rng, sum(lengths), n, 14)
    hq, hkv, d = 8, 2, 128
    seed = 40 + len(kind)
    print(f"[exchange] {kind} lengths={lengths} plan={[len(p) for p in plan]}", flush=True)
    cu, placed = _exchange(plan, lengths, hkv, d, seed)
    for r, (chunks, lo, hi, bk, bv) in enumerate(placed):
        if not chunks:
            continue
        w = custom_workload(seed, lengths, hq, hkv, d, chunks=chunks)
        q, do = w.q(), w.do()
        qd, dod = to_dev(q), to_dev(do)
        o, lse = api.attn_fwd(qd, bk, bv, cu, chunks, lo, hi, w.scale)
        dq, dk, dv = api.attn_bwd(qd, bk, bv, o, lse, dod, cu, chunks, lo, hi, w.scale)
        torch.cuda.synchronize()
        kg, vg = draw_tensor(seed, "k", w.total, hkv, d), draw_tensor(seed, "v", w.total, hkv, d)
        want_o, want_l = oracle.attention_forward(f64(q), f64(kg), f64(vg), cu, chunks, 0, w.total, w.scale)
        assert_close(bf16_to_np(o), want_o, O_TOL, f"rank {r} O")
        assert_close(lse.cpu().numpy(), want_l, LSE_TOL, f"rank {r} LSE")
        wq, wk, wv = oracle.attention_backward(f64(q), f64(kg), f64(vg), f64(do), cu, chunks, 0, w.total, w.scale)
        assert_close(dq.cpu().numpy(), wq, O_TOL, f"rank {r} dQ")
        assert_close(dk.cpu().numpy(), wk[lo:hi], O_TOL, f"rank {r} dK")
        assert_close(dv.cpu().numpy(), wv[lo:hi], O_TOL, f"rank {r} dV")


def test_exchange_study_plan_full_size():
    """CP = 8 per-document plan of the 16 x 8192 study workload (8 KV heads,
    D = 128): every worker's pack and placement bit-exact."""
    plan = [fig3_workload("16x8192", "per_doc", 8, r).chunks for r in range(8)]
    _exchange(plan, [8192] * 16, 8, 128, 5)


def test_exchange_flashcp_plan_bimodal():
    """The planner's CP = 8 plan of the bimodal 131072-token mix: every
    worker's pack and placement bit-exact."""
    from document_masked_attention_amd.workloads import bimodal_docs
    lengths = bimodal_docs(5)
    plan = oracle.plan_chunks(lengths, 8, 1.05)[0]
    _exchange(plan, lengths, 8, 128, 5)
