"""Benchmark of the document-masked attention hot path on one MI355X.

One step = one pass of the hot path over the 131072-token bimodal packed
sequence (64 query heads, 8 KV heads, head dim 128): tile scheduler, forward
(O, LSE), backward preprocess (Delta) and backward (dQ, dK, dV).  The inputs
are synthetic (seeded normal bf16, the bimodal document-length recipe) and
already resident in HBM when the timed region starts.

`value` is useful (unmasked) attention TFLOP/s of forward + backward:
forward 4*D*Hq*pairs, backward 10*D*Hq*pairs (five GEMM-shaped products per
allowed pair, the QK^T recompute included); pairs = allowed (row, key) pairs
per head.  The same run also times the forward alone and the backward alone
(mean, and the median of 20 calls); the forward of one CP rank (rank 3 of
CP = 8: 2 x CP chunks 3 and 12 of 16 x 8192, lognormal documents) three ways:
per-(chunk, KV block) calls plus the LSE merge of their bf16 or float32
partials, and one call over the rank's whole KV range (with --cp-backward
also its backward the same two ways); and the CPU oracle on a bounded sample.
`--study sharding` instead runs the 2 x CP sharding study (every worker of
CP = 8 under whole-sequence, per-document and Algorithm 1 plans, with their
KV exchange).
During the timed steps the library's event timer brackets every kernel
launch on its stream; the roofline line is the kernel with the largest share
of the step: its algorithmic flop per launch divided by its mean launch time.

    python bench.py [--gpus 1] [--steps 5] [--warmup 2] [--no-cpu-baseline] [--cp-backward] [--study sharding|length|power]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA (256 CU x 4096 flop/clk x 2.4 GHz)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
PROFILE_DIR = os.path.join(ROOT, "profiles")
WORKLOAD_TAG = "T131072_bimodal_h64x8_d128"
# sources each kernel class is compiled from (a counter summary taken on other sources is stale)
KERNEL_SOURCES = {"fwd_kernel": ["fwd.hip", "common.h", "kernels.h"],
                  "dkdv_kernel": ["bwd.hip", "common.h", "kernels.h"],
                  "dq_kernel": ["bwd.hip", "common.h", "kernels.h"]}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash(names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "document_masked_attention_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def pmc_file(kernel: str) -> str:
    return os.path.join(PROFILE_DIR, f"{kernel}_{WORKLOAD_TAG}_pmc.txt")


def read_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from its committed counter summary, or
    None if absent or taken on a different kernel source."""
    path = pmc_file(kernel)
    if kernel not in KERNEL_SOURCES or not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != kernel_source_hash(KERNEL_SOURCES[kernel]):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


MERGE_PMC = "merge_kernel_cp8_rank3_T131072_lognormal2048_h32x8_d128_pmc.txt"


def read_merge_traffic(key: str):
    """HBM bytes per merge pass (`merge_kernel` or `merge_kernel_f32`) from the
    committed counter summary, or None if absent or taken on other source."""
    path = os.path.join(PROFILE_DIR, MERGE_PMC)
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != kernel_source_hash(["merge.hip", "common.h", "kernels.h"]):
        return None
    try:
        return float(vals[f"{key}.hbm_bytes_per_pass"])
    except (KeyError, ValueError):
        return None


def cpu_model() -> str:
    """The host CPU's model name (first 'model name' line of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def blas_threads() -> int | None:
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        return None


def merge_bytes(lse_parts: np.ndarray, d: int) -> float:
    """The GPU merge's byte count for partials lse_parts [P, Hq, R]: every LSE
    read, the O rows of partials with a finite LSE read, O and LSE written."""
    p_c, hq, r = lse_parts.shape
    finite = int(np.isfinite(lse_parts).sum())
    return p_c * r * hq * 4 + finite * 2 * d + r * hq * (2 * d + 4)


def cpu_baseline(w, min_tokens: int = 10000, merge_rows: int = 8192):
    """The oracle, as it stands, on bounded samples of the same workloads, on
    this host's cores (its numpy uses the BLAS threads it finds):
      * fwd + bwd (the bench's value): whole documents covering the first
        `min_tokens` tokens of the 131072-token bimodal mix, KV head 0 with its
        query heads;
      * fwd only: the same sample;
      * lse_merge: the CP rank's (rank 3 of 8, chunks 3 and 12) partial shapes,
        4 and 7 partials, on `merge_rows` rows of each chunk (default: all
        8192, the GPU merge's whole workload) and all 32 heads,
        with seeded normal partial O (bf16 values) and LSE (all finite, like
        the GPU partials of that rank's canonical seed), bytes counted as the
        GPU merge counts them."""
    import oracle
    from document_masked_attention_amd.workloads import bf16_bits_to_f64, f32_to_bf16_bits, make_config
    cores = len(os.sched_getaffinity(0))
    cu = w.cu_seqlens
    end = int(cu[np.searchsorted(cu, min_tokens)])
    pos = np.arange(end)
    g = w.hq // w.hkv
    q = bf16_bits_to_f64(w.q(pos)[:, :g])
    k = bf16_bits_to_f64(w.k(pos)[:, :1])
    v = bf16_bits_to_f64(w.v(pos)[:, :1])
    do = bf16_bits_to_f64(w.do(pos)[:, :g])
    sub_cu = cu[cu <= end]
    pairs = oracle.useful_pairs(sub_cu, [(0, end)], 0, end)
    t0 = time.perf_counter()
    oracle.attention_backward(q, k, v, do, sub_cu, [(0, end)], 0, end, w.scale)   # runs its own forward
    dt = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.attention_forward(q, k, v, sub_cu, [(0, end)], 0, end, w.scale)
    dt_f = time.perf_counter() - t0
    # merge: the rank's partial shapes (blocks its chunks need), sampled rows
    w3 = make_config(3)
    need = oracle.need_intervals(w3.cu_seqlens, w3.chunks, w3.kv_lo, w3.kv_hi)
    rng = np.random.default_rng(3)
    m_bytes, m_secs, parts = 0.0, 0.0, []
    for (lo, hi) in need:
        p_c = int((hi + w3.kv_block - 1) // w3.kv_block - lo // w3.kv_block)
        parts.append(p_c)
        o_p = bf16_bits_to_f64(f32_to_bf16_bits(rng.standard_normal((p_c, merge_rows, w3.hq, w3.d), np.float32)))
        l_p = (3.0 * rng.standard_normal((p_c, w3.hq, merge_rows))).astype(np.float32).astype(np.float64)
        t0 = time.perf_counter()
        oracle.lse_merge(o_p, l_p)
        m_secs += time.perf_counter() - t0
        m_bytes += merge_bytes(l_p, w3.d)
    bl = blas_threads()
    return {"value": round(14.0 * w.d * g * pairs / dt / 1e12, 6), "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle",
            "sample": f"fwd+bwd, first {end} tokens ({len(sub_cu) - 1} whole documents) of the 131072-token "
                      f"bimodal mix, KV head 0 with its {g} query heads, float64 numpy, {dt:.1f} s; flop counted "
                      f"as the oracle executes it (14*D*Hq*pairs)",
            "seconds": round(dt, 2), "cpu": cpu_model(), "blas_threads": bl,
            "components": {
                "fwd": {"value": round(4.0 * w.d * g * pairs / dt_f / 1e12, 6), "unit": "TFLOP/s",
                        "seconds": round(dt_f, 2), "sample": "the same sample, forward only (4*D*Hq*pairs)"},
                "merge": {"value": round(m_bytes / m_secs / 1e9, 3), "unit": "GB/s", "seconds": round(m_secs, 2),
                          "bytes": int(m_bytes),
                          "sample": f"oracle.lse_merge on the CP rank's partial shapes ({parts} partials), "
                                    f"{merge_rows} rows per chunk, {w3.hq} heads, D={w3.d}; bytes as the GPU "
                                    f"merge counts them"}}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-merge", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run the f32->bf16 conversion over 1 GiB (reference for HBM byte counters)")
    ap.add_argument("--study", choices=["sharding", "length", "power"],
                    help="instead of the step benchmark: 'sharding' times every CP rank's forward under "
                         "per-sequence, per-document and Algorithm 1 sharding; 'length' times forward and "
                         "backward of one GPU's sequence from 32K to 1M tokens; 'power' samples board power and "
                         "clocks (amd-smi) while the forward, the backward, a bf16 GEMM and the matrix-core probe "
                         "run back to back")
    ap.add_argument("--cp", type=int, default=8, help="CP size of the sharding study")
    ap.add_argument("--cp-backward", action="store_true",
                    help="also time the CP rank's backward (per-block calls vs one call); off by default so that "
                         "the backward kernels' launches in a trace of this command are the step's alone")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU; multi-GPU runs are not part of it",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    if args.study == "sharding":
        study_sharding(args.cp, max(args.steps, 3))
        return
    if args.study == "length":
        study_length(max(args.steps, 3))
        return
    if args.study == "power":
        study_power()
        return

    import torch
    import oracle  # noqa: F401  (imported only for the cpu_baseline leg)
    from document_masked_attention_amd import api
    from document_masked_attention_amd.workloads import make_config

    api.lib()                                       # fail loudly if the library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def upload(bits):
        return torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)

    # ------------------------------------------------------------ workload
    w = make_config(5)
    log(f"[bench] workload {w.name}: generating inputs")
    t0 = time.time()
    q, k, v, do = upload(w.q()), upload(w.k()), upload(w.v()), upload(w.do())
    cu = torch.as_tensor(w.cu_seqlens, dtype=torch.int32, device=dev)
    log(f"[bench] inputs resident in HBM ({time.time() - t0:.1f} s)")
    sched = api.schedule(cu, w.chunks, w.kv_lo, w.kv_hi, 128, 64)
    counters = sched["counters"].cpu().numpy()
    pairs = int(counters[3])
    fwd_flop = 4.0 * w.d * w.hq * pairs
    bwd_flop = 10.0 * w.d * w.hq * pairs
    o = torch.empty_like(q)
    lse = torch.empty((w.hq, w.tq), dtype=torch.float32, device=dev)
    dq = torch.empty((w.tq, w.hq, w.d), dtype=torch.float32, device=dev)
    dk = torch.empty((w.tkv, w.hkv, w.d), dtype=torch.float32, device=dev)
    dv = torch.empty_like(dk)
    ws_f = torch.empty(api.workspace_size(api.OP_FWD, len(w.lengths), w.chunks, w.kv_lo, w.kv_hi, w.hq, w.hkv, w.d),
                       dtype=torch.uint8, device=dev)
    ws_b = torch.empty(api.workspace_size(api.OP_BWD, len(w.lengths), w.chunks, w.kv_lo, w.kv_hi, w.hq, w.hkv, w.d),
                       dtype=torch.uint8, device=dev)

    def fwd():
        api.attn_fwd(q, k, v, cu, w.chunks, w.kv_lo, w.kv_hi, w.scale, out=o, lse=lse, workspace=ws_f)

    def bwd():
        api.attn_bwd(q, k, v, o, lse, do, cu, w.chunks, w.kv_lo, w.kv_hi, w.scale, dq=dq, dk=dk, dv=dv,
                     workspace=ws_b)

    def step():
        fwd()
        bwd()

    def timed(fn, n):
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n            # ms per call

    for i in range(args.warmup):
        step()
        log(f"[bench] warmup step {i + 1}/{args.warmup} done")
    torch.cuda.synchronize()
    if api.check_errors(ws_f) != api.OK or api.check_errors(ws_b) != api.OK:
        raise RuntimeError("device-side input error")
    api.timing_enable(True)          # events around every kernel launch, on the launch stream
    ms_step = timed(step, args.steps)
    per_kernel = {}
    for kc in range(api.N_KERNEL_CLASSES):
        tot, n = api.timing_read(kc)
        if n:
            per_kernel[api.kernel_class_name(kc)] = {"launches": n, "total_ms": tot, "mean_ms": tot / n}
    api.timing_enable(False)
    log(f"[bench] {args.steps} timed steps: {ms_step:.3f} ms/step; per kernel "
        + ", ".join(f"{k} {v['mean_ms']:.3f} ms x{v['launches'] // args.steps}" for k, v in per_kernel.items()))
    ms_fwd = timed(fwd, args.steps)
    ms_bwd = timed(bwd, args.steps)
    log(f"[bench] fwd {ms_fwd:.3f} ms, bwd {ms_bwd:.3f} ms")

    def median_ms(fn, n=20):
        """Median over n calls, each between its own pair of events."""
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        torch.cuda.synchronize()
        for a, b in ev:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in ev]))

    med_fwd = median_ms(fwd)
    med_bwd = median_ms(bwd)
    log(f"[bench] median of 20: fwd {med_fwd:.3f} ms, bwd {med_bwd:.3f} ms")
    step()                                            # leave consistent outputs behind

    value = (fwd_flop + bwd_flop) / (ms_step * 1e-3) / 1e12
    # algorithmic flop per launch of each attention kernel (allowed pairs only):
    # forward QK^T + PV; dK/dV kernel QK^T recompute + dO V^T + P^T dO + dS^T Q;
    # dQ kernel QK^T recompute + dO V^T + dS K
    kernel_flop = {"fwd_kernel": 4.0 * w.d * w.hq * pairs, "dkdv_kernel": 8.0 * w.d * w.hq * pairs,
                   "dq_kernel": 6.0 * w.d * w.hq * pairs}
    dominant = max(kernel_flop, key=lambda k: per_kernel[k]["total_ms"])
    dom_ms = per_kernel[dominant]["mean_ms"]
    dom_tflops = kernel_flop[dominant] / (dom_ms * 1e-3) / 1e12
    t_, h_, d_ = w.tq, w.hq, w.d
    kernel_bytes = {   # compulsory HBM bytes per launch: each input read once, each output written once
        "fwd_kernel": 2 * t_ * h_ * d_ * 2 + 2 * w.tkv * w.hkv * d_ * 2 + t_ * h_ * 4,
        "dkdv_kernel": 2 * t_ * h_ * d_ * 2 + 2 * t_ * h_ * 4 + 2 * w.tkv * w.hkv * d_ * 2 + 2 * w.tkv * w.hkv * d_ * 4,
        "dq_kernel": 2 * t_ * h_ * d_ * 2 + 2 * t_ * h_ * 4 + 2 * w.tkv * w.hkv * d_ * 2 + t_ * h_ * d_ * 4,
    }
    traffic = read_traffic(dominant)
    result = {
        "metric": "useful attention TFLOP/s fwd & fwd+bwd (% bf16 MFMA peak); merge GB/s",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "seq_len": w.total, "documents": len(w.lengths), "seed": w.seed,
                   "q_heads": w.hq, "kv_heads": w.hkv, "head_dim": w.d, "pairs_per_head": pairs,
                   "value_is": "fwd+bwd useful TFLOP/s (fwd 4*D*Hq*pairs + bwd 10*D*Hq*pairs)"},
        "roofline": {"bound": "mfma", "kernel": dominant,
                     "achieved": round(dom_tflops, 3), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(dom_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": None if traffic is None else round(traffic),
                     "algorithmic_flop": kernel_flop[dominant],
                     "algorithmic_bytes": int(kernel_bytes[dominant]),
                     "launch_ms": round(dom_ms, 4)},
        "components": {
            "fwd": {"ms": round(ms_fwd, 4), "tflops": round(fwd_flop / (ms_fwd * 1e-3) / 1e12, 3),
                    "frac_of_peak": round(fwd_flop / (ms_fwd * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                    "median_of_20_ms": round(med_fwd, 4),
                    "median_frac_of_peak": round(fwd_flop / (med_fwd * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)},
            "bwd": {"ms": round(ms_bwd, 4), "tflops": round(bwd_flop / (ms_bwd * 1e-3) / 1e12, 3),
                    "frac_of_peak": round(bwd_flop / (ms_bwd * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                    "tflops_8d_count": round(0.8 * bwd_flop / (ms_bwd * 1e-3) / 1e12, 3),
                    "median_of_20_ms": round(med_bwd, 4),
                    "median_frac_of_peak": round(bwd_flop / (med_bwd * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)},
            "kernels": {k: {"launches_per_step": v["launches"] // args.steps, "mean_ms": round(v["mean_ms"], 4),
                            **({"tflops": round(kernel_flop[k] / (v["mean_ms"] * 1e-3) / 1e12, 3),
                                "frac_of_peak": round(kernel_flop[k] / (v["mean_ms"] * 1e-3) / 1e12
                                                      / PEAK_BF16_TFLOPS, 4)} if k in kernel_flop else {})}
                        for k, v in per_kernel.items()},
            "scheduler_counters": {"nonskip_tiles_128x64": int(counters[0]), "full": int(counters[1]),
                                   "partial": int(counters[2])},
        },
    }
    del o, lse, dq, dk, dv, q, k, v, do, ws_f, ws_b
    torch.cuda.empty_cache()

    if not args.no_merge:
        merge, cp_fwd, cp_bwd = bench_merge(api, torch, dev, upload, args.steps, args.cp_backward)
        result["components"]["merge"] = merge
        result["components"]["cp_rank_forward"] = cp_fwd
        if cp_bwd is not None:
            result["components"]["cp_rank_backward"] = cp_bwd
    if args.copy_calibration:
        # a streaming kernel of known size for scaling HBM byte counters: the
        # library's f32 -> bf16 conversion reads 1 GiB and writes 512 MiB
        a = torch.zeros(1 << 28, dtype=torch.float32, device=dev)
        b = torch.empty(1 << 28, dtype=torch.bfloat16, device=dev)
        for _ in range(3):
            api.f32_to_bf16(a, out=b)
        torch.cuda.synchronize()
        result["copy_calibration_bytes"] = {"kernel": "f32_to_bf16_kernel", "read": a.numel() * 4,
                                            "write": b.numel() * 2}
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle) ...")
        result["cpu_baseline"] = cpu_baseline(w)
        log(f"[bench] cpu baseline {result['cpu_baseline']['seconds']} s")
    print(json.dumps(result), flush=True)


def study_power(seconds: float = 4.0):
    """Board power and GFX clocks (amd-smi, sampled about every 0.3 s) while
    the step's forward, its backward and, as references of what the chip
    sustains on pure matrix work, a bf16 8192^3 GEMM (torch.matmul) and the
    library's matrix-core probe (back-to-back v_mfma_f32_32x32x16_bf16, then
    v_mfma_f32_16x16x32_bf16, on operands in registers, no memory traffic;
    N(0, 1) bf16 operands, and all zeros as a control for data-dependent
    power) each run back to back for `seconds`; one JSON line with the
    medians per phase."""
    import statistics
    import subprocess
    import threading
    import torch
    from document_masked_attention_amd import api
    from document_masked_attention_amd.workloads import make_config
    api.lib()
    dev = torch.device("cuda:0")
    samples, stop, phase = [], threading.Event(), ["idle"]

    def sampler():
        while not stop.is_set():
            try:
                r = subprocess.run(["amd-smi", "metric", "-g", "0", "-p", "-c", "--json"], capture_output=True,
                                   text=True, timeout=10)
                d = json.loads(r.stdout)
                g = d["gpu_data"][0] if isinstance(d, dict) and "gpu_data" in d else d[0]
                pw = g["power"]["socket_power"]
                clk = [v["clk"]["value"] for k_, v in g["clock"].items()
                       if k_.startswith("gfx") and isinstance(v, dict) and isinstance(v.get("clk"), dict)]
                samples.append((phase[0], float(pw["value"]), statistics.mean(clk)))
            except Exception as e:          # a sample that cannot be read is skipped, and said so
                log(f"[power] sample skipped: {e}")
            time.sleep(0.25)

    w = make_config(5)
    up = lambda b: torch.from_numpy(b.view(np.int16)).to(dev).view(torch.bfloat16)
    q, k, v, do = up(w.q()), up(w.k()), up(w.v()), up(w.do())
    cu = torch.as_tensor(w.cu_seqlens, dtype=torch.int32, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.hq, w.tq), dtype=torch.float32, device=dev)
    dq = torch.empty((w.tq, w.hq, w.d), dtype=torch.float32, device=dev)
    dk = torch.empty((w.tkv, w.hkv, w.d), dtype=torch.float32, device=dev)
    dv = torch.empty_like(dk)
    pairs = int(api.schedule(cu, w.chunks, 0, w.total, 128, 64)["counters"][3].item())
    a = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16)
    b = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16)
    probe_ops = torch.randn(1 << 20, device=dev, dtype=torch.bfloat16)
    probe_zero = torch.zeros(1 << 20, device=dev, dtype=torch.bfloat16)
    probe_wg, probe_iters = 2048, 1024         # 8 workgroups per CU over the run, 2 resident
    probe_out = torch.empty(256 * probe_wg, device=dev, dtype=torch.float32)
    probe_flop = float(api.PROBE_FLOP_PER_WAVE_ITER) * probe_iters * 4 * probe_wg
    legs = (("fwd", lambda: api.attn_fwd(q, k, v, cu, w.chunks, 0, w.total, w.scale, out=o, lse=lse),
             4.0 * w.d * w.hq * pairs),
            ("bwd", lambda: api.attn_bwd(q, k, v, o, lse, do, cu, w.chunks, 0, w.total, w.scale, dq=dq, dk=dk, dv=dv),
             10.0 * w.d * w.hq * pairs),
            ("gemm_bf16_8192", lambda: torch.matmul(a, b), 2.0 * 8192 ** 3),
            ("mfma_probe_randn", lambda: api.mfma_probe(probe_ops, probe_wg, probe_iters, out=probe_out), probe_flop),
            ("mfma_probe_zero", lambda: api.mfma_probe(probe_zero, probe_wg, probe_iters, out=probe_out), probe_flop),
            ("mfma16_probe_randn", lambda: api.mfma_probe(probe_ops, probe_wg, probe_iters, out=probe_out, shape=16),
             probe_flop),
            ("mfma16_probe_zero", lambda: api.mfma_probe(probe_zero, probe_wg, probe_iters, out=probe_out, shape=16),
             probe_flop))
    for _, fn, _ in legs:
        fn()
    torch.cuda.synchronize()
    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    time.sleep(1.0)
    result = {"study": "power", "workload": w.name, "phases": {}}
    for name, fn, flop in legs:
        phase[0] = name
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n, t0 = 0, time.time()
        e0.record()
        while time.time() - t0 < seconds:
            for _ in range(4):
                fn()
            n += 4
            torch.cuda.synchronize()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / n
        result["phases"][name] = {"calls": n, "ms_per_call": round(ms, 4),
                                  "tflops": round(flop / (ms * 1e-3) / 1e12, 1),
                                  "frac_of_peak": round(flop / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        log(f"[power] {name}: {n} calls, {ms:.3f} ms each")
        phase[0] = "idle"
        time.sleep(1.0)
    stop.set()
    th.join()
    for name in list(result["phases"]) + ["idle"]:
        sel = [(pw, c) for ph, pw, c in samples if ph == name]
        if sel:
            result["phases"].setdefault(name, {}).update({
                "samples": len(sel), "board_power_w_median": statistics.median(x for x, _ in sel),
                "board_power_w_max": max(x for x, _ in sel), "gfx_clock_mhz_median": round(statistics.median(c for _, c in sel), 1)})
    print(json.dumps(result), flush=True)


def bench_merge(api, torch, dev, upload, steps, cp_backward=False):
    """lse_merge of rank 3's per-block partials (CP = 8, chunks 3 and 12)."""
    from document_masked_attention_amd.workloads import make_config
    w = make_config(3)
    log(f"[bench] merge workload {w.name}: generating inputs")
    q, k, v = upload(w.q()), upload(w.k()), upload(w.v())
    cu = torch.as_tensor(w.cu_seqlens, dtype=torch.int32, device=dev)
    need = api.schedule(cu, w.chunks, w.kv_lo, w.kv_hi, 8192, 8192)["need"].cpu().numpy()
    blk = w.kv_block
    jobs = []
    fwd_calls = []
    row0 = 0
    total_bytes = 0.0
    dense_bytes = 0.0
    for ci, (g, n) in enumerate(w.chunks):
        blocks = list(range(need[ci, 0] // blk, (need[ci, 1] + blk - 1) // blk))
        po = torch.empty((len(blocks), n, w.hq, w.d), dtype=torch.bfloat16, device=dev)
        pl = torch.empty((len(blocks), w.hq, n), dtype=torch.float32, device=dev)
        for i, b in enumerate(blocks):
            api.attn_fwd(q[row0:row0 + n], k[blk * b:blk * (b + 1)], v[blk * b:blk * (b + 1)], cu, [(g, n)],
                         blk * b, blk * (b + 1), w.scale, out=po[i], lse=pl[i])
        oo = torch.empty((n, w.hq, w.d), dtype=torch.bfloat16, device=dev)
        lo = torch.empty((w.hq, n), dtype=torch.float32, device=dev)
        finite = int(torch.isfinite(pl).sum().item())
        p_c = len(blocks)
        total_bytes += p_c * n * w.hq * 4 + finite * 2 * w.d + n * w.hq * (2 * w.d + 4)
        dense_bytes += p_c * n * w.hq * (4 + 2 * w.d) + n * w.hq * (2 * w.d + 4)
        jobs.append((po, pl, oo, lo))
        fwd_calls.append((row0, g, n, blocks, po, pl))
        row0 += n
    torch.cuda.synchronize()

    # the rank's forward as the pages' ring schedule runs it: one call per
    # (chunk, KV block), partials merged afterwards (timed below on its own)
    def fwd_all():
        for r0, g, n, blocks, po, pl in fwd_calls:
            for i, b in enumerate(blocks):
                api.attn_fwd(q[r0:r0 + n], k[blk * b:blk * (b + 1)], v[blk * b:blk * (b + 1)], cu, [(g, n)],
                             blk * b, blk * (b + 1), w.scale, out=po[i], lse=pl[i])

    reps = max(steps, 5)
    fwd_all()
    torch.cuda.synchronize()
    api.timing_enable(True)
    f0 = torch.cuda.Event(enable_timing=True)
    f1 = torch.cuda.Event(enable_timing=True)
    f0.record()
    for _ in range(reps):
        fwd_all()
    f1.record()
    torch.cuda.synchronize()
    t_fwd, n_fwd = api.timing_read(api.KERNEL_FWD)
    t_sch, _ = api.timing_read(api.KERNEL_SCHEDULE)
    api.timing_enable(False)
    wall_ms = f0.elapsed_time(f1) / reps
    kern_ms = (t_fwd + t_sch) / reps
    pairs = int(api.schedule(cu, w.chunks, w.kv_lo, w.kv_hi, 128, 64)["counters"][3].item())
    flop = 4.0 * w.d * w.hq * pairs
    cp_fwd = {"workload": w.name, "calls_per_pass": n_fwd // reps, "pairs_per_head": pairs,
              "useful_tflop": round(flop / 1e12, 3), "kernel_ms": round(kern_ms, 4), "wall_ms": round(wall_ms, 4),
              "tflops_kernel": round(flop / (kern_ms * 1e-3) / 1e12, 2),
              "frac_of_peak": round(flop / (kern_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
              "note": "sum of the per-(chunk, 8192-key block) forward calls' scheduler and kernel time; "
                      "wall_ms includes host launch overhead"}

    def merge_all():
        for po, pl, oo, lo in jobs:
            api.lse_merge(po, pl, o_out=oo, lse_out=lo)

    merge_all()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(max(steps, 10)):
        merge_all()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / max(steps, 10)
    gbs = total_bytes / (ms * 1e-3) / 1e9
    parts = [j[0].shape[0] for j in jobs]
    # the same rows in one call over the whole KV range (no partials, no merge)
    o1 = torch.empty((w.tq, w.hq, w.d), dtype=torch.bfloat16, device=dev)
    l1 = torch.empty((w.hq, w.tq), dtype=torch.float32, device=dev)

    def fwd_one():
        api.attn_fwd(q, k, v, cu, w.chunks, w.kv_lo, w.kv_hi, w.scale, out=o1, lse=l1)

    fwd_one()
    torch.cuda.synchronize()
    api.timing_enable(True)
    for _ in range(reps):
        fwd_one()
    torch.cuda.synchronize()
    t1, _ = api.timing_read(api.KERNEL_FWD)
    t1s, _ = api.timing_read(api.KERNEL_SCHEDULE)
    api.timing_enable(False)
    one_ms = (t1 + t1s) / reps
    cp_fwd.update({"per_block_plus_merge_ms": round(kern_ms + ms, 4),
                   "single_call_kernel_ms": round(one_ms, 4),
                   "single_call_tflops": round(flop / (one_ms * 1e-3) / 1e12, 2),
                   "single_call_frac_of_peak": round(flop / (one_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)})
    # the same per-block calls with float32 partials, merged by lse_merge_f32
    jobs32 = []
    for r0, g, n, blocks, po, pl in fwd_calls:
        jobs32.append((r0, g, n, blocks, torch.empty(po.shape, dtype=torch.float32, device=dev), pl,
                       torch.empty((n, w.hq, w.d), dtype=torch.bfloat16, device=dev),
                       torch.empty((w.hq, n), dtype=torch.float32, device=dev)))

    def fwd_all32():
        for r0, g, n, blocks, po, pl, _, _ in jobs32:
            for i, b in enumerate(blocks):
                api.attn_fwd(q[r0:r0 + n], k[blk * b:blk * (b + 1)], v[blk * b:blk * (b + 1)], cu, [(g, n)],
                             blk * b, blk * (b + 1), w.scale, out=po[i], lse=pl[i], f32_out=True)

    def merge_all32():
        for _, _, _, _, po, pl, oo, lo in jobs32:
            api.lse_merge(po, pl, o_out=oo, lse_out=lo)

    fwd_all32()
    merge_all32()
    torch.cuda.synchronize()
    api.timing_enable(True)
    for _ in range(reps):
        fwd_all32()
    torch.cuda.synchronize()
    f32_fwd_ms = (api.timing_read(api.KERNEL_FWD)[0] + api.timing_read(api.KERNEL_SCHEDULE)[0]) / reps
    api.timing_enable(False)
    api.timing_enable(True)
    for _ in range(reps):
        merge_all32()
    torch.cuda.synchronize()
    f32_merge_ms = api.timing_read(api.KERNEL_MERGE)[0] / reps
    api.timing_enable(False)
    # the bf16 merge's bytes plus the second half of every float32 partial O row read
    bytes32 = total_bytes + sum(int(torch.isfinite(j[5]).sum().item()) * 2 * w.d for j in jobs32)
    cp_fwd.update({"f32_partials": {
        "fwd_kernel_ms": round(f32_fwd_ms, 4), "merge_ms": round(f32_merge_ms, 4),
        "total_ms": round(f32_fwd_ms + f32_merge_ms, 4), "merge_bytes": int(bytes32),
        "merge_GBps": round(bytes32 / (f32_merge_ms * 1e-3) / 1e9, 1),
        "merge_traffic": read_merge_traffic("merge_kernel_f32"),
        "note": "per-block forward calls writing float32 O, then lse_merge_f32 (bf16 output)"}})
    del jobs32
    merge = {"workload": w.name, "partials_per_chunk": parts, "ms": round(ms, 4), "bytes": int(total_bytes),
             "dense_bytes": int(dense_bytes), "GB/s": round(gbs, 1), "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
             "bound": "hbm", "traffic": read_merge_traffic("merge_kernel")}
    if not cp_backward:
        return merge, cp_fwd, None
    # the rank's backward as a ring schedule runs it: per-(chunk, KV block)
    # calls with the merged O and LSE (dQ shares accumulated, Delta formed by
    # the first call of each chunk), beside one call over the whole KV range
    merge_all()
    do_r = upload(w.do())
    dq_r = torch.empty((w.tq, w.hq, w.d), dtype=torch.float32, device=dev)
    dk_b = torch.empty((blk, w.hkv, w.d), dtype=torch.float32, device=dev)
    dv_b = torch.empty_like(dk_b)
    ws_c = {}
    for r0, g, n, blocks, _, _ in fwd_calls:
        ws_c[g] = torch.empty(max(api.workspace_size(api.OP_BWD, len(w.lengths), [(g, n)], blk * b, blk * (b + 1),
                                                     w.hq, w.hkv, w.d) for b in blocks), dtype=torch.uint8, device=dev)

    def bwd_all():
        for (r0, g, n, blocks, _, _), (_, _, oo, lo) in zip(fwd_calls, jobs):
            for i, b in enumerate(blocks):
                api.attn_bwd(q[r0:r0 + n], k[blk * b:blk * (b + 1)], v[blk * b:blk * (b + 1)], oo, lo,
                             do_r[r0:r0 + n], cu, [(g, n)], blk * b, blk * (b + 1), w.scale, dq=dq_r[r0:r0 + n],
                             dk=dk_b, dv=dv_b, accumulate_dq=i > 0, delta_ready=i > 0, workspace=ws_c[g])

    dq1 = torch.empty((w.tq, w.hq, w.d), dtype=torch.float32, device=dev)
    dk1 = torch.empty((w.tkv, w.hkv, w.d), dtype=torch.float32, device=dev)
    dv1 = torch.empty_like(dk1)

    def bwd_one():
        api.attn_bwd(q, k, v, o1, l1, do_r, cu, w.chunks, w.kv_lo, w.kv_hi, w.scale, dq=dq1, dk=dk1, dv=dv1)

    bwd_flop = 10.0 * w.d * w.hq * pairs
    legs = {}
    for name, fn in (("per_block", bwd_all), ("single_call", bwd_one)):
        fn()
        torch.cuda.synchronize()
        api.timing_enable(True)
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        kms = sum(api.timing_read(c)[0] for c in (api.KERNEL_SCHEDULE, api.KERNEL_DQ, api.KERNEL_DKDV)) / reps
        calls = api.timing_read(api.KERNEL_DKDV)[1] // reps
        api.timing_enable(False)
        legs[name] = {"kernel_ms": round(kms, 4), "calls_per_pass": calls,
                      "tflops": round(bwd_flop / (kms * 1e-3) / 1e12, 2),
                      "frac_of_peak": round(bwd_flop / (kms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    cp_bwd = {"workload": w.name, "useful_tflop": round(bwd_flop / 1e12, 3), **legs,
              "note": "scheduler + dQ + dK/dV kernel time; useful work 10*D*Hq*pairs"}
    del do_r, dq_r, dk_b, dv_b, dq1, dk1, dv1, ws_c
    return merge, cp_fwd, cp_bwd


FLASHCP_RATIO = 1.05         # target workload ratio of the planner in the sharding study


def study_plan(api, sharding, lengths, cp, hq, hkv, d, seed):
    """Every worker's chunk list under one sharding of the study."""
    from document_masked_attention_amd.workloads import fig3_workload
    if sharding == "flashcp":
        return api.plan_shards(lengths, cp, FLASHCP_RATIO)[0]
    return [fig3_workload("", sharding, cp, r, hq, hkv, d, seed, lengths=lengths).chunks for r in range(cp)]


def exchange_study(api, torch, dev, kf, vf, lengths, cp, hq, hkv, d, seed, reps):
    """Sharding-aware KV exchange of every worker (FlashCP section 3.2): rows
    sent (Eq. 5's terms) against the static full-KV pattern (Eq. 4), and the
    time of the two copies one GPU runs: packing the worker's sent rows, and
    placing the gathered rows plus its own at their positions."""
    from document_masked_attention_amd.workloads import fig3_workload, cu_from_lengths
    cu = cu_from_lengths(lengths)
    total = int(cu[-1])
    rb = hkv * d * 2                                   # bytes per KV row and tensor
    out = {}
    for sharding in ("per_sequence", "per_doc", "flashcp"):
        plan = study_plan(api, sharding, lengths, cp, hq, hkv, d, seed)
        send = [api.exchange_send_maps(cu, ch) for ch in plan]
        slot = max([n for _, n in send] + [1])
        gk = torch.zeros((cp * slot, hkv, d), dtype=torch.bfloat16, device=dev)
        gv = torch.zeros_like(gk)
        pack_ms, unpack_ms, pack_bytes, unpack_bytes, written_rows, span_rows = [], [], [], [], [], []
        locs = []
        for r, ch in enumerate(plan):
            pos = torch.as_tensor(np.concatenate([np.arange(g, g + n) for g, n in ch]), device=dev)
            kl, vl = kf.index_select(0, pos), vf.index_select(0, pos)
            locs.append((kl, vl))
            maps, n = send[r]
            dk, dv = gk[r * slot:r * slot + n], gv[r * slot:r * slot + n]

            def pack():
                api.copy_rows(kl, vl, dk, dv, maps, False)
            pack()
            torch.cuda.synchronize()
            api.timing_enable(True)
            for _ in range(reps):
                pack()
            torch.cuda.synchronize()
            pack_ms.append(api.timing_read(api.KERNEL_COPY)[0] / reps)
            api.timing_enable(False)
            pack_bytes.append(2 * 2 * n * rb)
        for r, ch in enumerate(plan):
            m = api.exchange_recv_maps(cu, plan, r, slot)
            span = m["kv_hi"] - m["kv_lo"]
            bk = torch.empty((span, hkv, d), dtype=torch.bfloat16, device=dev)
            bv = torch.empty_like(bk)
            kl, vl = locs[r]

            def place():
                api.copy_rows(gk, gv, bk, bv, m["remote"], False)
                api.copy_rows(kl, vl, bk, bv, m["local"], False)
            place()
            torch.cuda.synchronize()
            api.timing_enable(True)
            for _ in range(reps):
                place()
            torch.cuda.synchronize()
            unpack_ms.append(api.timing_read(api.KERNEL_COPY)[0] / reps)
            api.timing_enable(False)
            copied = sum(x[2] for x in m["remote"] if x[0] >= 0)
            zeros = sum(x[2] for x in m["remote"] if x[0] < 0)
            own = sum(x[2] for x in m["local"])
            unpack_bytes.append(2 * rb * (2 * copied + zeros + 2 * own))
            written_rows.append(copied + zeros + own)
            span_rows.append(span)
            del bk, bv
        sent = [n for _, n in send]
        eq4 = 4.0 * total / cp * hkv * d * (cp - 1) * 2
        eq5 = 4.0 * max(sent) * hkv * d * (cp - 1) * 2
        pb, pm = np.array(pack_bytes, float), np.array(pack_ms)
        ub, um = np.array(unpack_bytes, float), np.array(unpack_ms)
        out[sharding] = {
            "sent_rows_per_rank": sent, "eq4_bytes": eq4, "eq5_bytes": eq5, "eq5_over_eq4": round(eq5 / eq4, 4),
            "pack_ms_per_rank": [round(x, 4) for x in pm], "unpack_ms_per_rank": [round(x, 4) for x in um],
            "pack_GBps": round(float(pb.sum() / (pm.sum() * 1e-3) / 1e9), 1) if pm.sum() > 0 else None,
            "unpack_GBps": round(float(ub.sum() / (um.sum() * 1e-3) / 1e9), 1),
            "unpack_frac_of_hbm_peak": round(float(ub.sum() / (um.sum() * 1e-3) / 1e9 / PEAK_HBM_GBS), 4),
            "placed_rows_written": int(sum(written_rows)), "placed_range_rows": int(sum(span_rows)),
            "bytes_note": "pack: K and V sent rows read + written; place: gathered and own rows read + written, "
                          "zero rows written (the rest of each 128-row KV block holding a needed row)"}
        log(f"[study] exchange {sharding}: eq5/eq4 {eq5 / eq4:.3f}, pack {out[sharding]['pack_GBps']} GB/s, "
            f"place {out[sharding]['unpack_GBps']} GB/s")
        del gk, gv, locs
    return out


def study_length(reps: int):
    """Forward and backward of one GPU's packed sequence at 32K to 1M tokens
    (lognormal(2048, 1.5) documents up to 131072 tokens, 32 query / 8 KV heads,
    D = 128): kernel time by the library's event timer, useful TFLOP/s and the
    fraction of dense bf16 peak at each length."""
    import torch
    from document_masked_attention_amd import api
    from document_masked_attention_amd.workloads import custom_workload, lognormal_docs
    api.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    hq, hkv, d = 32, 8, 128
    out = {"study": "sequence length", "q_heads": hq, "kv_heads": hkv, "head_dim": d, "reps": reps,
           "documents": "lognormal(2048, 1.5), clip [64, 131072], seed 9", "lengths": []}

    def dev_bits(bits):
        return torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)

    for t in (1 << 15, 1 << 17, 1 << 19, 1 << 20):
        w = custom_workload(9, lognormal_docs(9, 2048, 1.5, 64, 131072, t), hq, hkv, d, backward=True)
        log(f"[study] length {t}: {len(w.lengths)} documents, generating inputs")
        q, k, v, do = dev_bits(w.q()), dev_bits(w.k()), dev_bits(w.v()), dev_bits(w.do())
        cu = torch.as_tensor(w.cu_seqlens, dtype=torch.int32, device=dev)
        pairs = int(api.schedule(cu, w.chunks, 0, t, 128, 64)["counters"][3].item())
        o, lse = api.attn_fwd(q, k, v, cu, w.chunks, 0, t, w.scale)
        dq, dk, dv = api.attn_bwd(q, k, v, o, lse, do, cu, w.chunks, 0, t, w.scale)
        torch.cuda.synchronize()
        api.timing_enable(True)
        for _ in range(reps):
            api.attn_fwd(q, k, v, cu, w.chunks, 0, t, w.scale, out=o, lse=lse)
        torch.cuda.synchronize()
        fwd_ms = (api.timing_read(api.KERNEL_FWD)[0] + api.timing_read(api.KERNEL_SCHEDULE)[0]) / reps
        api.timing_enable(False)
        api.timing_enable(True)
        for _ in range(reps):
            api.attn_bwd(q, k, v, o, lse, do, cu, w.chunks, 0, t, w.scale, dq=dq, dk=dk, dv=dv)
        torch.cuda.synchronize()
        bwd_ms = sum(api.timing_read(c)[0] for c in (api.KERNEL_SCHEDULE, api.KERNEL_DQ, api.KERNEL_DKDV)) / reps
        api.timing_enable(False)
        ff, bf = 4.0 * d * hq * pairs, 10.0 * d * hq * pairs
        row = {"tokens": t, "documents": len(w.lengths), "pairs_per_head": pairs,
               "fwd_ms": round(fwd_ms, 4), "fwd_tflops": round(ff / (fwd_ms * 1e-3) / 1e12, 1),
               "fwd_frac_of_peak": round(ff / (fwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
               "bwd_ms": round(bwd_ms, 4), "bwd_tflops": round(bf / (bwd_ms * 1e-3) / 1e12, 1),
               "bwd_frac_of_peak": round(bf / (bwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
               "resident_gib": round(sum(x.numel() * x.element_size() for x in (q, k, v, do, o, lse, dq, dk, dv))
                                     / 2 ** 30, 2)}
        out["lengths"].append(row)
        log(f"[study] length {t}: fwd {fwd_ms:.3f} ms ({row['fwd_frac_of_peak']:.3f}), "
            f"bwd {bwd_ms:.3f} ms ({row['bwd_frac_of_peak']:.3f})")
        del q, k, v, do, o, lse, dq, dk, dv
        torch.cuda.empty_cache()
    print(json.dumps(out), flush=True)


def study_sharding(cp: int, reps: int):
    """Kernel-efficiency study of 2 x CP sharding on one GPU (the single-GPU
    analogue of FlashCP Figure 3).  For every rank r of a CP group of size cp,
    the rank's forward is run three ways over the all-gathered KV range:

      per_sequence        chunks r and 2cp-1-r of the packed sequence, one call;
      per_doc             pieces r and 2cp-1-r of every document, one call;
      per_doc_blockwise   the same rows computed block by block, one call per
                          contiguous KV block of T/cp keys that the rows need,
                          then the partials merged (ring-style execution);
      flashcp             the library's Algorithm 1 plan (whole documents, head
                          cuts for equal tokens, Per-Doc for the longest ones
                          while the workload ratio exceeds 1.05), one call.

    Time per rank = the library's event timer summed over scheduler, forward
    and merge kernels; a CP step is as slow as its slowest rank."""
    import torch
    from document_masked_attention_amd import api
    from document_masked_attention_amd.workloads import (FIG3_PATTERNS, fig3_lengths, draw_tensor, cu_from_lengths,
                                                         Workload)
    api.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    hq, hkv, d, seed = 32, 8, 128, 5
    out = {"study": "2xCP sharding, one rank's forward over the all-gathered KV", "cp": cp, "q_heads": hq,
           "kv_heads": hkv, "head_dim": d, "reps": reps, "time": "scheduler + forward (+ merge) kernel ms",
           "patterns": {}}

    def dev_bits(bits):
        return torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)

    def lib_ms(classes):
        return sum(api.timing_read(c)[0] for c in classes) / reps

    for pattern in FIG3_PATTERNS:
        lengths = fig3_lengths(pattern, seed)
        total = int(sum(lengths))
        log(f"[study] {pattern}: {len(lengths)} documents, generating inputs")
        qf = dev_bits(draw_tensor(seed, "q", total, hq, d))
        kf = dev_bits(draw_tensor(seed, "k", total, hkv, d))
        vf = dev_bits(draw_tensor(seed, "v", total, hkv, d))
        cu = torch.as_tensor(cu_from_lengths(lengths), dtype=torch.int32, device=dev)
        blk = total // cp
        res = {s: {"per_rank_ms": [], "per_rank_wall_ms": [], "per_rank_pairs": [], "per_rank_chunks": []}
               for s in ("per_sequence", "per_doc", "per_doc_blockwise", "flashcp")}
        plans = {sh: study_plan(api, sh, lengths, cp, hq, hkv, d, seed) for sh in ("per_sequence", "per_doc", "flashcp")}
        scale = 1.0 / np.sqrt(d)
        # the GPU idled while the inputs were generated: bring its clocks up before timing rank 0
        wq = qf.index_select(0, torch.arange(16384, device=dev))
        t_end = time.time() + 1.0
        while time.time() < t_end:
            for _ in range(10):
                api.attn_fwd(wq, kf, vf, cu, [(0, 16384)], 0, total, scale)
            torch.cuda.synchronize()
        del wq
        for r in range(cp):
            for sharding in ("per_sequence", "per_doc", "flashcp"):
                w = Workload(f"{sharding}_cp{cp}_rank{r}_{pattern}", seed, total, lengths, hq, hkv, d,
                             plans[sharding][r], 0, total)
                pos = torch.as_tensor(w.local_positions(), device=dev)
                q = qf.index_select(0, pos)
                o = torch.empty((w.tq, hq, d), dtype=torch.bfloat16, device=dev)
                lse = torch.empty((hq, w.tq), dtype=torch.float32, device=dev)
                ws = torch.empty(api.workspace_size(api.OP_FWD, len(lengths), w.chunks, 0, total, hq, hkv, d),
                                 dtype=torch.uint8, device=dev)
                sched = api.schedule(cu, w.chunks, 0, total, 128, 64)
                pairs = int(sched["counters"][3].item())
                need = sched["need"].cpu().numpy()
                variants = [(sharding, None)]
                if sharding == "per_doc":
                    lo = int(need[:, 0][need[:, 1] > need[:, 0]].min())
                    hi = int(need[:, 1].max())
                    blocks = [b for b in range(cp) if b * blk < hi and (b + 1) * blk > lo]
                    po = torch.empty((len(blocks), w.tq, hq, d), dtype=torch.bfloat16, device=dev)
                    pl = torch.empty((len(blocks), hq, w.tq), dtype=torch.float32, device=dev)
                    variants.append(("per_doc_blockwise", blocks))

                for name, blocks in variants:
                    if blocks is None:
                        def run():
                            api.attn_fwd(q, kf, vf, cu, w.chunks, 0, total, scale, out=o, lse=lse, workspace=ws)
                    else:
                        def run():
                            for i, b in enumerate(blocks):
                                api.attn_fwd(q, kf[b * blk:(b + 1) * blk], vf[b * blk:(b + 1) * blk], cu, w.chunks,
                                             b * blk, (b + 1) * blk, scale, out=po[i], lse=pl[i])
                            api.lse_merge(po, pl, o_out=o, lse_out=lse)
                    run()
                    torch.cuda.synchronize()
                    api.timing_enable(True)
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record()
                    for _ in range(reps):
                        run()
                    e1.record()
                    torch.cuda.synchronize()
                    ms = lib_ms((api.KERNEL_SCHEDULE, api.KERNEL_FWD, api.KERNEL_MERGE))
                    api.timing_enable(False)
                    rr = res[name]
                    rr["per_rank_ms"].append(round(ms, 4))
                    rr["per_rank_wall_ms"].append(round(e0.elapsed_time(e1) / reps, 4))
                    rr["per_rank_pairs"].append(pairs)
                    rr["per_rank_chunks"].append(len(w.chunks))
                    if blocks is not None:
                        rr.setdefault("kv_blocks_per_rank", []).append(len(blocks))
                del q, o, lse, ws
                if sharding == "per_doc":
                    del po, pl
            log(f"[study] {pattern} rank {r}: " + ", ".join(f"{k} {v['per_rank_ms'][-1]:.3f} ms"
                                                            for k, v in res.items()))
        base = max(res["per_sequence"]["per_rank_ms"])
        for name, rr in res.items():
            ms = np.array(rr["per_rank_ms"])
            pr = np.array(rr["per_rank_pairs"], dtype=np.float64)
            flop = 4.0 * d * hq * pr
            rr.update({"max_ms": round(float(ms.max()), 4), "mean_ms": round(float(ms.mean()), 4),
                       "normalized_latency": round(float(ms.max()) / base, 4),
                       "pair_imbalance": round(float(pr.max() / pr.mean()), 4),
                       "mean_rank_tflops": round(float((flop / (ms * 1e-3)).mean() / 1e12), 2),
                       "mean_rank_frac_of_peak": round(float((flop / (ms * 1e-3)).mean() / 1e12 / PEAK_BF16_TFLOPS), 4)})
        out["patterns"][pattern] = {"documents": len(lengths), **res,
                                    "exchange": exchange_study(api, torch, dev, kf, vf, lengths, cp, hq, hkv, d,
                                                               seed, reps)}
        del qf, kf, vf
        torch.cuda.empty_cache()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
