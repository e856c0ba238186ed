"""Helpers shared by the GPU parity tests (device transfer, comparisons and
the record of measured errors)."""
import json
import os
import time

import numpy as np
import torch

from document_masked_attention_amd.workloads import bf16_bits_to_f32, custom_workload, lognormal_docs

O_TOL = 2e-2      # max abs error on O, dQ, dK, dV (bf16 I/O)
LSE_TOL = 1e-3    # max abs error on the LSE

D64_LONG_LABEL = 6   # the parity table's row label of the workload below


def d64_long_workload():
    """Head size 64 at full size: 65536 tokens of lognormal(median 2048,
    sigma 1.3) documents clipped to [64, 32768] (seed 65: 17 documents, the
    longest 22,529 tokens), 16 query / 4 KV heads, forward and backward
    inputs."""
    return custom_workload(65, lognormal_docs(65, 2048, 1.3, 64, 32768, 65536), 16, 4, 64, backward=True)


def to_dev(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> torch.bfloat16 on the GPU."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def bf16_to_np(t: torch.Tensor) -> np.ndarray:
    """torch.bfloat16 (any device) -> float64 numpy."""
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32).__lshift__(16) \
        .view(np.float32).astype(np.float64)


def f64(bits: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(bits).astype(np.float64)


def assert_close(got, want, tol, what):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    inf_g, inf_w = np.isinf(got), np.isinf(want)
    assert np.array_equal(inf_g, inf_w), f"{what}: infinity pattern differs ({inf_g.sum()} vs {inf_w.sum()})"
    if inf_w.any():
        assert np.array_equal(got[inf_w], want[inf_w]), f"{what}: infinities of different sign"
    fin = ~inf_w
    assert not np.isnan(got).any(), f"{what}: NaN in result"
    err = np.abs(got[fin] - want[fin]).max() if fin.any() else 0.0
    assert err <= tol, f"{what}: max abs error {err:.3e} > {tol:.1e}"
    return err


def host_cores() -> int:
    return len(os.sched_getaffinity(0))


def gpu_ms(fn):
    """(result, milliseconds) of fn() between two events on the current stream."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    out = fn()
    e1.record()
    torch.cuda.synchronize()
    return out, e0.elapsed_time(e1)


def timed_s(fn):
    """(result, wall seconds) of fn() on the host."""
    t0 = time.perf_counter()
    out = fn()
    return out, time.perf_counter() - t0


def record(**row):
    """Append one row of measured parity errors (and timings) as a JSON line to
    the file named by DOCMASK_PARITY_LOG; nothing happens when it is unset."""
    path = os.environ.get("DOCMASK_PARITY_LOG")
    if not path:
        return
    row = {k: (float(v) if isinstance(v, (np.floating, np.integer)) else v) for k, v in row.items()}
    with open(path, "a") as f:
        f.write(json.dumps(row) + "\n")
