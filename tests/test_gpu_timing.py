"""The library's kernel timer, which bench.py's roofline line reads: every
launch is counted in its kernel class, nothing is recorded while timing is
off, enabling clears the totals, and the summed kernel time of a call agrees
with stream events recorded around that call."""
import numpy as np
import pytest
import torch

from document_masked_attention_amd import api
from document_masked_attention_amd.workloads import custom_workload, random_lengths
from gpu_util import to_dev

pytestmark = pytest.mark.gpu


def _counts():
    return {c: api.timing_read(c) for c in range(api.N_KERNEL_CLASSES)}


def test_timer_counts_launches_and_matches_stream_events():
    rng = np.random.default_rng(31)
    w = custom_workload(31, random_lengths(rng, 24576, 6000, p_one=0.02), 32, 8, 128, backward=True)
    print(f"[timing] T={w.total} h={w.hq}/{w.hkv} d={w.d}", flush=True)
    q, k, v, do = to_dev(w.q()), to_dev(w.k()), to_dev(w.v()), to_dev(w.do())
    cu = torch.as_tensor(w.cu_seqlens, dtype=torch.int32, device="cuda")
    o, lse = api.attn_fwd(q, k, v, cu, w.chunks, w.kv_lo, w.kv_hi, w.scale)
    dq, dk, dv = api.attn_bwd(q, k, v, o, lse, do, cu, w.chunks, w.kv_lo, w.kv_hi, w.scale)
    torch.cuda.synchronize()

    api.timing_enable(True)
    assert all(n == 0 for _, n in _counts().values())
    api.attn_fwd(q, k, v, cu, w.chunks, w.kv_lo, w.kv_hi, w.scale, out=o, lse=lse)
    api.attn_bwd(q, k, v, o, lse, do, cu, w.chunks, w.kv_lo, w.kv_hi, w.scale, dq=dq, dk=dk, dv=dv)
    parts = torch.stack([o, o])
    lparts = torch.stack([lse, lse])
    api.lse_merge(parts, lparts)
    api.f32_to_bf16(dq)
    torch.cuda.synchronize()
    c = _counts()
    api.timing_enable(False)
    # one schedule build for the forward, two for the backward (query-major and key-major)
    want = {api.KERNEL_SCHEDULE: 3, api.KERNEL_FWD: 1, api.KERNEL_DELTA: 0, api.KERNEL_DKDV: 1, api.KERNEL_DQ: 1,
            api.KERNEL_MERGE: 1, api.KERNEL_CONVERT: 1, api.KERNEL_COPY: 0, api.KERNEL_HEAD: 1}
    assert {k_: n for k_, (_, n) in c.items()} == want
    assert all((ms > 0) == (want[k_] > 0) for k_, (ms, _) in c.items())

    # timing off: further launches are not recorded
    api.attn_fwd(q, k, v, cu, w.chunks, w.kv_lo, w.kv_hi, w.scale, out=o, lse=lse)
    torch.cuda.synchronize()
    assert api.timing_read(api.KERNEL_FWD)[1] == 1

    # the forward's kernel time (scheduler + attention) against events around the call, over several calls
    reps = 10
    api.timing_enable(True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        api.attn_fwd(q, k, v, cu, w.chunks, w.kv_lo, w.kv_hi, w.scale, out=o, lse=lse)
    e1.record()
    torch.cuda.synchronize()
    kern = api.timing_read(api.KERNEL_FWD)[0] + api.timing_read(api.KERNEL_SCHEDULE)[0]
    api.timing_enable(False)
    wall = e0.elapsed_time(e1)
    print(f"[timing] fwd kernels {kern / reps:.3f} ms, events around the calls {wall / reps:.3f} ms", flush=True)
    assert 0.8 * wall <= kern <= 1.02 * wall
