"""Per-document 2 x CP chunk lists on the GPU vs the fp64 oracle.

Every rank's rows under per-document sharding (pieces i and 2N-1-i of each
document, FlashCP section 2.3) go through the same entry points as any other
chunk list: small problems element by element (forward and backward, every
rank), the full-size study workloads on sampled rows, and the block-by-block
execution (one partial per contiguous KV block, merged) against the single
call and the oracle."""
import numpy as np
import pytest
import torch

import oracle
from document_masked_attention_amd import api
from document_masked_attention_amd.workloads import (custom_workload, per_doc_chunks, random_lengths, fig3_workload,
                                                     FIG3_PATTERNS)
from gpu_util import to_dev, bf16_to_np, f64, assert_close, O_TOL, LSE_TOL

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cp", [2, 4])
def test_small_every_rank_fwd_bwd(cp):
    rng = np.random.default_rng(70 + cp)
    lengths = random_lengths(rng, 900, 260, p_one=0.1) + [2 * cp - 1, 64 * 2 * cp]
    for r in range(cp):
        chunks = per_doc_chunks(lengths, cp, r)
        hq, hkv, d = [(8, 2, 128), (4, 1, 64)][r % 2]
        w = custom_workload(100 * cp + r, lengths, hq, hkv, d, chunks=chunks, backward=True)
        print(f"[shard] cp={cp} rank={r} chunks={len(chunks)} tq={w.tq} h={hq}/{hkv} d={d}", flush=True)
        q, k, v, do = w.q(), w.k(), w.v(), w.do()
        qd, kd, vd, dod = to_dev(q), to_dev(k), to_dev(v), to_dev(do)
        o, lse = api.attn_fwd(qd, kd, vd, w.cu_seqlens, chunks, 0, w.total, w.scale)
        dq, dk, dv = api.attn_bwd(qd, kd, vd, o, lse, dod, w.cu_seqlens, chunks, 0, w.total, w.scale)
        torch.cuda.synchronize()
        want_o, want_l = oracle.attention_forward(f64(q), f64(k), f64(v), w.cu_seqlens, chunks, 0, w.total, w.scale)
        assert_close(bf16_to_np(o), want_o, O_TOL, "O")
        assert_close(lse.cpu().numpy(), want_l, LSE_TOL, "LSE")
        wq, wk, wv = oracle.attention_backward(f64(q), f64(k), f64(v), f64(do), w.cu_seqlens, chunks, 0, w.total,
                                               w.scale)
        assert_close(dq.cpu().numpy(), wq, O_TOL, "dQ")
        assert_close(dk.cpu().numpy(), wk, O_TOL, "dK")
        assert_close(dv.cpu().numpy(), wv, O_TOL, "dV")


def _rows(w, n, seed):
    """Sampled local rows: the first and last row of every chunk (capped) and random ones."""
    starts = np.cumsum([0] + [c for _, c in w.chunks])[:-1]
    ends = starts + np.array([c for _, c in w.chunks]) - 1
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([starts[:24], ends[:24], rng.choice(w.tq, n, replace=False)]))


@pytest.mark.parametrize("pattern", FIG3_PATTERNS[1:])
def test_study_per_doc_sampled_rows(pattern):
    w = fig3_workload(pattern, "per_doc", 8, 3)
    print(f"[shard] {w.name} chunks={len(w.chunks)} tq={w.tq}", flush=True)
    q, k, v = w.q(), w.k(), w.v()
    o, lse = api.attn_fwd(to_dev(q), to_dev(k), to_dev(v), w.cu_seqlens, w.chunks, 0, w.total, w.scale)
    torch.cuda.synchronize()
    sel = _rows(w, 48, 11)
    want_o, want_l = oracle.attention_forward(f64(q), f64(k), f64(v), w.cu_seqlens, w.chunks, 0, w.total, w.scale,
                                              rows=sel)
    assert_close(bf16_to_np(o)[sel], want_o, O_TOL, "O")
    assert_close(lse.cpu().numpy()[:, sel], want_l, LSE_TOL, "LSE")


def test_blockwise_partials_merge():
    """Rank 3 of CP = 8 on 16 x 8192 documents, per-document pieces: one
    partial per 16384-key block, merged; equals the single call and the oracle."""
    w = fig3_workload("16x8192", "per_doc", 8, 3)
    q, k, v = w.q(), w.k(), w.v()
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    blk = w.total // 8
    po = torch.empty((8, w.tq, w.hq, w.d), dtype=torch.bfloat16, device="cuda")
    pl = torch.empty((8, w.hq, w.tq), dtype=torch.float32, device="cuda")
    for b in range(8):
        print(f"[shard] block {b}", flush=True)
        api.attn_fwd(qd, kd[b * blk:(b + 1) * blk], vd[b * blk:(b + 1) * blk], w.cu_seqlens, w.chunks, b * blk,
                     (b + 1) * blk, w.scale, out=po[b], lse=pl[b])
    o_m, l_m = api.lse_merge(po, pl)
    o1, l1 = api.attn_fwd(qd, kd, vd, w.cu_seqlens, w.chunks, 0, w.total, w.scale)
    torch.cuda.synchronize()
    o_np, l_np = bf16_to_np(o_m), l_m.cpu().numpy().astype(np.float64)
    assert_close(o_np, bf16_to_np(o1), O_TOL, "merged vs single-call O")
    assert_close(l_np, l1.cpu().numpy(), LSE_TOL, "merged vs single-call LSE")
    sel = _rows(w, 32, 12)
    want_o, want_l = oracle.attention_forward(f64(q), f64(k), f64(v), w.cu_seqlens, w.chunks, 0, w.total, w.scale,
                                              rows=sel)
    assert_close(o_np[sel], want_o, O_TOL, "merged O")
    assert_close(l_np[:, sel], want_l, LSE_TOL, "merged LSE")


@pytest.mark.parametrize("rank", [0, 5])
def test_flashcp_plan_sampled_rows(rank):
    """A worker of the CP = 8 Algorithm 1 plan of the bimodal mix (whole
    documents, head cuts, two Per-Doc documents): sampled rows vs the oracle."""
    from document_masked_attention_amd.workloads import bimodal_docs
    lengths = bimodal_docs(5)
    chunks = oracle.plan_chunks(lengths, 8, 1.05)[0][rank]
    w = custom_workload(5, lengths, 32, 8, 128, chunks=chunks)
    print(f"[shard] flashcp rank {rank} chunks={len(chunks)} tq={w.tq}", flush=True)
    q, k, v = w.q(), w.k(), w.v()
    o, lse = api.attn_fwd(to_dev(q), to_dev(k), to_dev(v), w.cu_seqlens, chunks, 0, w.total, w.scale)
    torch.cuda.synchronize()
    sel = _rows(w, 48, 13 + rank)
    want_o, want_l = oracle.attention_forward(f64(q), f64(k), f64(v), w.cu_seqlens, chunks, 0, w.total, w.scale,
                                              rows=sel)
    assert_close(bf16_to_np(o)[sel], want_o, O_TOL, "O")
    assert_close(lse.cpu().numpy()[:, sel], want_l, LSE_TOL, "LSE")
