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
