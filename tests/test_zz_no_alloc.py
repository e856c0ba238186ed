"""docmask_attn_fwd_noalloc (the forward on the library's static scratch, no
workspace) against docmask_attn_fwd with a caller workspace: two calls in a
row on one GPU, the second with a smaller problem (and other head shape), each
bit-identical to the workspace forward and within tolerance of the oracle on
sampled rows."""
import numpy as np
import pytest
import torch

import oracle
from document_masked_attention_amd import api
from document_masked_attention_amd.workloads import custom_workload, random_lengths
from gpu_util import to_dev, bf16_to_np, f64, assert_close, O_TOL, LSE_TOL

pytestmark = pytest.mark.gpu


def _compare(w, tag):
    print(f"[noalloc] {tag}: T={w.total} tq={w.tq} h={w.hq}/{w.hkv} d={w.d} chunks={w.chunks} "
          f"kv=[{w.kv_lo},{w.kv_hi})", flush=True)
    q, k, v = w.q(), w.k(), w.v()
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    cu = torch.as_tensor(w.cu_seqlens, dtype=torch.int32, device="cuda")
    o_ref, l_ref = api.attn_fwd(qd, kd, vd, cu, w.chunks, w.kv_lo, w.kv_hi, w.scale)
    o = torch.full_like(o_ref, float("nan"))
    lse = torch.full_like(l_ref, float("nan"))
    api.attn_fwd_noalloc(qd, kd, vd, cu, w.chunks, w.kv_lo, w.kv_hi, w.scale, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), f"{tag}: O differs from the workspace forward"
    assert torch.equal(lse, l_ref), f"{tag}: LSE differs from the workspace forward"
    rows = np.unique(np.concatenate([np.linspace(0, w.tq - 1, 40).astype(int), [0, w.tq - 1]]))
    want_o, want_l = oracle.attention_forward(f64(q), f64(k), f64(v), w.cu_seqlens, w.chunks, w.kv_lo, w.kv_hi,
                                              w.scale, rows=rows)
    assert_close(bf16_to_np(o)[rows], want_o, O_TOL, f"{tag} O vs oracle")
    assert_close(lse.cpu().numpy()[:, rows], want_l, LSE_TOL, f"{tag} LSE vs oracle")


def test_noalloc_forward_two_calls_second_smaller():
    rng = np.random.default_rng(41)
    total = 9000
    big = custom_workload(41, random_lengths(rng, total, 3000, p_one=0.05), 16, 2, 128,
                          chunks=[(100, 4000), (5000, 3900)], kv_lo=0, kv_hi=total)
    small = custom_workload(42, random_lengths(rng, 700, 200, p_one=0.1), 8, 8, 64)
    _compare(big, "first call (larger)")
    _compare(small, "second call (smaller)")
    _compare(big, "third call (larger again)")


def test_noalloc_forward_graph_replays_after_other_calls():
    """Captured in a HIP graph (the callers this entry point is for), with an
    eager call on another problem between replays overwriting the shared
    scratch: every replay gives the eager result bit for bit, because each call
    writes every scratch region it reads before reading it."""
    rng = np.random.default_rng(43)
    w = custom_workload(43, random_lengths(rng, 3000, 900, p_one=0.05), 8, 2, 128)
    other = custom_workload(44, random_lengths(rng, 5000, 2500, p_one=0.05), 16, 4, 64,
                            chunks=[(0, 2000), (3000, 2000)], kv_lo=0, kv_hi=5000)
    print(f"[noalloc graph] T={w.total} h={w.hq}/{w.hkv} d={w.d}; other T={other.total} "
          f"h={other.hq}/{other.hkv} d={other.d}", flush=True)
    q, k, v = to_dev(w.q()), to_dev(w.k()), to_dev(w.v())
    cu = torch.as_tensor(w.cu_seqlens, dtype=torch.int32, device="cuda")
    oq, ok_, ov = to_dev(other.q()), to_dev(other.k()), to_dev(other.v())
    ocu = torch.as_tensor(other.cu_seqlens, dtype=torch.int32, device="cuda")
    o = torch.empty((w.tq, w.hq, w.d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.hq, w.tq), dtype=torch.float32, device="cuda")
    o2 = torch.empty((other.tq, other.hq, other.d), dtype=torch.bfloat16, device="cuda")
    lse2 = torch.empty((other.hq, other.tq), dtype=torch.float32, device="cuda")

    def run():
        api.attn_fwd_noalloc(q, k, v, cu, w.chunks, w.kv_lo, w.kv_hi, w.scale, out=o, lse=lse)

    run()
    torch.cuda.synchronize()
    ref_o, ref_l = o.clone(), lse.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()
    for rep in range(3):
        api.attn_fwd_noalloc(oq, ok_, ov, ocu, other.chunks, other.kv_lo, other.kv_hi, other.scale, out=o2, lse=lse2)
        o.zero_()
        lse.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), ref_o.view(torch.int16)), f"replay {rep}: O differs"
        assert torch.equal(lse, ref_l), f"replay {rep}: LSE differs"
