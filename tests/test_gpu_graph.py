"""The forward + backward enqueue only kernels on the caller's stream (no
allocation, no host synchronisation), so a caller can capture them in a HIP
graph.  Each replay, with eager work on the same buffers in between, must give
the eager results bit for bit (the kernels are deterministic)."""
import numpy as np
import pytest
import torch

from document_masked_attention_amd import api
from document_masked_attention_amd.workloads import custom_workload, random_lengths
from gpu_util import to_dev

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    rng = np.random.default_rng(77)
    w = custom_workload(77, random_lengths(rng, 700, 300, p_one=0.05), 8, 2, 128, backward=True)
    print(f"[graph] T={w.total} h={w.hq}/{w.hkv} d={w.d}", flush=True)
    q, k, v, do = to_dev(w.q()), to_dev(w.k()), to_dev(w.v()), to_dev(w.do())
    cu = torch.as_tensor(w.cu_seqlens, dtype=torch.int32, device="cuda")
    n_docs = cu.numel() - 1
    o = torch.empty((w.tq, w.hq, w.d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.hq, w.tq), dtype=torch.float32, device="cuda")
    dq = torch.empty((w.tq, w.hq, w.d), dtype=torch.float32, device="cuda")
    dk = torch.empty((w.tkv, w.hkv, w.d), dtype=torch.float32, device="cuda")
    dv = torch.empty_like(dk)
    wsf = torch.empty(api.workspace_size(api.OP_FWD, n_docs, w.chunks, w.kv_lo, w.kv_hi, w.hq, w.hkv, w.d),
                      dtype=torch.uint8, device="cuda")
    wsb = torch.empty(api.workspace_size(api.OP_BWD, n_docs, w.chunks, w.kv_lo, w.kv_hi, w.hq, w.hkv, w.d),
                      dtype=torch.uint8, device="cuda")

    def run():
        api.attn_fwd(q, k, v, cu, w.chunks, w.kv_lo, w.kv_hi, w.scale, out=o, lse=lse, workspace=wsf)
        api.attn_bwd(q, k, v, o, lse, do, cu, w.chunks, w.kv_lo, w.kv_hi, w.scale, dq=dq, dk=dk, dv=dv,
                     workspace=wsb)

    run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (o, lse, dq, dk, dv)]

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
        for t in (o, lse, dq, dk, dv):          # eager work on the same buffers between replays
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("O", "LSE", "dQ", "dK", "dV"), (o, lse, dq, dk, dv), ref):
            assert torch.equal(got, want), f"replay {rep}: {name} differs from the eager result"
    assert api.check_errors(wsb) == api.OK


def test_graph_cp_rank_pipeline():
    """One worker's whole single-GPU CP path in one graph: pack its sent KV
    rows, gather (the collective's stand-in, by the same row copy), place the
    KV it needs, forward per 256-key block + LSE merge, backward per block with
    the merged O/LSE (dQ shares added).  Replays equal the eager run bit for bit."""
    from document_masked_attention_amd.workloads import per_doc_chunks
    rng = np.random.default_rng(78)
    lengths = random_lengths(rng, 1200, 400, p_one=0.05)
    n_w, hq, hkv, d = 2, 8, 2, 128
    plan = [per_doc_chunks(lengths, n_w, r) for r in range(n_w)]
    w = custom_workload(78, lengths, hq, hkv, d, backward=True)
    cu_h = w.cu_seqlens
    cu = torch.as_tensor(cu_h, dtype=torch.int32, device="cuda")
    kg, vg = to_dev(w.k()), to_dev(w.v())
    sends = [api.exchange_send_maps(cu_h, ch) for ch in plan]
    slot = max(n for _, n in sends)
    locs = []
    for ch in plan:
        pos = torch.as_tensor(np.concatenate([np.arange(g, g + n) for g, n in ch]), device="cuda")
        locs.append((kg.index_select(0, pos).contiguous(), vg.index_select(0, pos).contiguous()))
    me = 1
    m = api.exchange_recv_maps(cu_h, plan, me, slot)
    lo, hi = m["kv_lo"], m["kv_hi"]
    chunks = plan[me]
    wr = custom_workload(78, lengths, hq, hkv, d, chunks=chunks, backward=True)
    q, do = to_dev(wr.q()), to_dev(wr.do())
    pk = [torch.empty((slot, hkv, d), dtype=torch.bfloat16, device="cuda") for _ in range(n_w)]
    pv = [torch.empty_like(t) for t in pk]
    gk = torch.zeros((n_w * slot, hkv, d), dtype=torch.bfloat16, device="cuda")
    gv = torch.zeros_like(gk)
    bk = torch.zeros((hi - lo, hkv, d), dtype=torch.bfloat16, device="cuda")
    bv = torch.zeros_like(bk)
    blk = 256
    blocks = [(x, min(x + blk, hi)) for x in range(lo, hi, blk)]
    po = torch.empty((len(blocks), wr.tq, hq, d), dtype=torch.bfloat16, device="cuda")
    pl = torch.empty((len(blocks), hq, wr.tq), dtype=torch.float32, device="cuda")
    om = torch.empty((wr.tq, hq, d), dtype=torch.bfloat16, device="cuda")
    lm = torch.empty((hq, wr.tq), dtype=torch.float32, device="cuda")
    dq = torch.empty((wr.tq, hq, d), dtype=torch.float32, device="cuda")
    dk = torch.empty((hi - lo, hkv, d), dtype=torch.float32, device="cuda")
    dv = torch.empty_like(dk)
    nd = cu.numel() - 1
    wsf = [torch.empty(api.workspace_size(api.OP_FWD, nd, chunks, a, b, hq, hkv, d), dtype=torch.uint8,
                       device="cuda") for a, b in blocks]
    wsb = torch.empty(max(api.workspace_size(api.OP_BWD, nd, chunks, a, b, hq, hkv, d) for a, b in blocks),
                      dtype=torch.uint8, device="cuda")
    print(f"[graph cp] T={w.total} worker {me}: chunks={len(chunks)} kv=[{lo},{hi}) blocks={len(blocks)}", flush=True)

    def run():
        for r in range(n_w):                                  # pack, then gather into the slots
            maps, n = sends[r]
            api.copy_rows(locs[r][0], locs[r][1], pk[r][:n], pv[r][:n], maps, False)
            api.copy_rows(pk[r][:n], pv[r][:n], gk[r * slot:r * slot + n], gv[r * slot:r * slot + n],
                          [(0, 0, n)] if n else [], False)
        api.copy_rows(gk, gv, bk, bv, m["remote"], False)
        api.copy_rows(locs[me][0], locs[me][1], bk, bv, m["local"], False)
        for i, (a, b) in enumerate(blocks):
            api.attn_fwd(q, bk[a - lo:b - lo], bv[a - lo:b - lo], cu, chunks, a, b, wr.scale, out=po[i], lse=pl[i],
                         workspace=wsf[i])
        api.lse_merge(po, pl, o_out=om, lse_out=lm)
        for i, (a, b) in enumerate(blocks):
            api.attn_bwd(q, bk[a - lo:b - lo], bv[a - lo:b - lo], om, lm, do, cu, chunks, a, b, wr.scale, dq=dq,
                         dk=dk[a - lo:b - lo], dv=dv[a - lo:b - lo], accumulate_dq=i > 0, delta_ready=i > 0,
                         workspace=wsb)

    run()
    torch.cuda.synchronize()
    outs = (bk, bv, om, lm, dq, dk, dv)
    ref = [t.clone() for t in outs]
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
        for t in outs + (gk, gv, po, pl):
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("placed K", "placed V", "O", "LSE", "dQ", "dK", "dV"), outs, ref):
            assert torch.equal(got, want), f"replay {rep}: {name} differs from the eager result"
