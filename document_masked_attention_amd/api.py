"""Thin Python binding of libdocmask.so (C ABI in include/docmask.h).

Argument marshalling only: every step of the computation runs in the HIP
library.  PyTorch supplies device memory and the current HIP stream.  Tensors
must be on the current GPU; bf16 tensors may be given as torch.bfloat16 or as
16-bit integer views of the same bits.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

# DOCMASK_LIBRARY names another build of the same library (e.g. the
# host-sanitized one); by default the in-tree libdocmask.so
_LIB_PATH = os.environ.get("DOCMASK_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                               "libdocmask.so")
_lib = None

OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP, EDEVICE_INPUT, ESCRATCH = 0, -1, -2, -3, -4, -5, -6
NOALLOC_SCRATCH_BYTES = 4 << 20
OP_FWD, OP_BWD = 1, 2
ACCUMULATE_DQ = 1
DELTA_READY = 2
MAX_CHUNKS = 256
(KERNEL_SCHEDULE, KERNEL_FWD, KERNEL_DELTA, KERNEL_DKDV, KERNEL_DQ, KERNEL_MERGE,
 KERNEL_CONVERT, KERNEL_COPY, KERNEL_HEAD) = range(9)
N_KERNEL_CLASSES = 9

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t
_f32 = ctypes.c_float


class Chunk(ctypes.Structure):
    _fields_ = [("g_start", ctypes.c_int32), ("len", ctypes.c_int32)]


class RowMap(ctypes.Structure):
    _fields_ = [("src", ctypes.c_int32), ("dst", ctypes.c_int32), ("len", ctypes.c_int32)]


_SIGNATURES = {
    "docmask_workspace_size": (_sz, [ctypes.c_int, _i32, _vp, _i32, _i32, _i32, _i32, _i32, _i32]),
    "docmask_schedule_workspace_size": (_sz, [_vp, _i32, _i32, _i32, _i32, _i32]),
    "docmask_schedule": (ctypes.c_int, [_vp, _i32, _vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp,
                                        _vp, _vp, _sz, _vp]),
    "docmask_attn_fwd": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _f32,
                                        _vp, _vp, _vp, _sz, _vp]),
    "docmask_attn_bwd": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _i32,
                                        _i32, _f32, _vp, _vp, _vp, ctypes.c_int, _vp, _sz, _vp]),
    "lse_merge": (ctypes.c_int, [_vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp]),
    "lse_merge_f32": (ctypes.c_int, [_vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp]),
    "docmask_attn_fwd_noalloc": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                                                _f32, _vp, _vp, _vp]),
    "docmask_attn_fwd_f32out": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                                               _f32, _vp, _vp, _vp, _sz, _vp]),
    "docmask_check_errors": (ctypes.c_int, [_vp, _vp]),
    "docmask_f32_to_bf16": (ctypes.c_int, [_vp, _vp, _i64, _vp]),
    "docmask_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "docmask_timing_enable": (ctypes.c_int, [ctypes.c_int]),
    "docmask_timing_read": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_i64)]),
    "docmask_kernel_class_name": (ctypes.c_char_p, [ctypes.c_int]),
    "docmask_mfma_probe": (ctypes.c_int, [_vp, _i64, _i32, _i32, _i32, _vp, _vp]),
    "docmask_plan_shards": (ctypes.c_int, [_vp, _i32, _i32, ctypes.c_double, _vp, _i32, _vp, _vp,
                                           ctypes.POINTER(_i32), ctypes.POINTER(ctypes.c_double)]),
    "docmask_copy_rows": (ctypes.c_int, [_vp, _vp, _i64, _vp, _vp, _i64, _i64, _vp, _i32, ctypes.c_int, _vp]),
    "docmask_exchange_send_maps": (ctypes.c_int, [_vp, _i32, _vp, _i32, _vp, _i32, ctypes.POINTER(_i32),
                                                  ctypes.POINTER(_i64)]),
    "docmask_exchange_recv_maps": (ctypes.c_int, [_vp, _i32, _vp, _vp, _i32, _i32, _i64, ctypes.POINTER(_i32),
                                                  ctypes.POINTER(_i32), _vp, _i32, ctypes.POINTER(_i32), _vp, _i32,
                                                  ctypes.POINTER(_i32)]),
}


class DocmaskError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {strerror(status)} (status {status})")
        self.status = status


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                               "`python -m document_masked_attention_amd.build`")
        handle = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def lib_path() -> str:
    return _LIB_PATH


def strerror(status: int) -> str:
    return lib().docmask_strerror(status).decode()


def _check(status: int, what: str):
    if status != OK:
        raise DocmaskError(status, what)


def _chunks(chunks):
    n = len(chunks)
    arr = (Chunk * max(n, 1))()
    for i, (g, length) in enumerate(chunks):
        arr[i].g_start = int(g)
        arr[i].len = int(length)
    return arr, n


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _bits(t: torch.Tensor) -> torch.Tensor:
    if t.dtype == torch.bfloat16:
        return t
    if t.dtype in (torch.int16, torch.uint16):
        return t
    raise TypeError(f"expected bf16 data, got {t.dtype}")


def _dev_i32(x, device) -> torch.Tensor:
    if isinstance(x, torch.Tensor):
        if x.dtype != torch.int32 or x.device.type != "cuda":
            raise TypeError("cu_seqlens must be an int32 tensor on the GPU")
        return x
    return torch.as_tensor(x, dtype=torch.int32, device=device)


def workspace_size(op: int, n_docs: int, chunks, kv_lo: int, kv_hi: int, hq: int, hkv: int, d: int) -> int:
    arr, n = _chunks(chunks)
    return int(lib().docmask_workspace_size(op, n_docs, arr, n, kv_lo, kv_hi, hq, hkv, d))


def schedule_workspace_size(chunks, kv_lo: int, kv_hi: int, bq: int, bk: int) -> int:
    arr, n = _chunks(chunks)
    return int(lib().docmask_schedule_workspace_size(arr, n, kv_lo, kv_hi, bq, bk))


def schedule(cu_seqlens, chunks, kv_lo: int, kv_hi: int, bq: int, bk: int, device="cuda") -> dict:
    """Run the tile scheduler and return its outputs as device tensors."""
    cu = _dev_i32(cu_seqlens, device)
    n_qt = sum((n + bq - 1) // bq for _, n in chunks)
    n_kt = (kv_hi - kv_lo + bk - 1) // bk
    out = {
        "qtile_desc": torch.empty((n_qt, 4), dtype=torch.int32, device=cu.device),
        "kvtile_desc": torch.empty((n_kt, 4), dtype=torch.int32, device=cu.device),
        "need": torch.empty((len(chunks), 2), dtype=torch.int32, device=cu.device),
        "lpt_q": torch.empty(n_qt, dtype=torch.int32, device=cu.device),
        "lpt_kv": torch.empty(n_kt, dtype=torch.int32, device=cu.device),
        "counters": torch.empty(4, dtype=torch.int64, device=cu.device),
    }
    ws_bytes = schedule_workspace_size(chunks, kv_lo, kv_hi, bq, bk)
    if ws_bytes == 0:
        raise DocmaskError(EINVAL, "docmask_schedule_workspace_size")
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=cu.device)
    arr, n = _chunks(chunks)
    st = lib().docmask_schedule(_ptr(cu), cu.numel() - 1, arr, n, kv_lo, kv_hi, bq, bk,
                                _ptr(out["qtile_desc"]), _ptr(out["kvtile_desc"]), _ptr(out["need"]),
                                _ptr(out["lpt_q"]), _ptr(out["lpt_kv"]), _ptr(out["counters"]),
                                _ptr(ws), ws_bytes, _stream())
    _check(st, "docmask_schedule")
    out["workspace"] = ws
    return out


def attn_fwd(q, k, v, cu_seqlens, chunks, kv_lo: int, kv_hi: int, scale: float | None = None,
             out=None, lse=None, workspace=None, f32_out: bool = False):
    """O [Tq, Hq, D] (bf16; float32 with f32_out, for lse_merge_f32) and LSE
    [Hq, Tq] (float32) of document-masked attention."""
    q, k, v = _bits(q), _bits(k), _bits(v)
    tq, hq, d = q.shape
    hkv = k.shape[1]
    cu = _dev_i32(cu_seqlens, q.device)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    if out is None:
        out = torch.empty((tq, hq, d), dtype=torch.float32 if f32_out else torch.bfloat16, device=q.device)
    if (out.dtype == torch.float32) != f32_out:
        raise TypeError("out must be float32 exactly when f32_out is set")
    if lse is None:
        lse = torch.empty((hq, tq), dtype=torch.float32, device=q.device)
    n_docs = cu.numel() - 1
    ws_bytes = workspace_size(OP_FWD, n_docs, chunks, kv_lo, kv_hi, hq, hkv, d)
    if ws_bytes == 0:
        raise DocmaskError(EINVAL, "docmask_workspace_size")
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    arr, n = _chunks(chunks)
    fn = lib().docmask_attn_fwd_f32out if f32_out else lib().docmask_attn_fwd
    st = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(cu), n_docs, arr, n, kv_lo, kv_hi, hq, hkv, d,
            float(scale), _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(), _stream())
    _check(st, "docmask_attn_fwd_f32out" if f32_out else "docmask_attn_fwd")
    return out, lse


def attn_fwd_noalloc(q, k, v, cu_seqlens, chunks, kv_lo: int, kv_hi: int, scale: float | None = None, out=None,
                     lse=None):
    """docmask_attn_fwd_noalloc: the forward without a workspace (the library's
    static scratch); out and lse must be given when the caller cannot allocate."""
    q, k, v = _bits(q), _bits(k), _bits(v)
    tq, hq, d = q.shape
    hkv = k.shape[1]
    cu = _dev_i32(cu_seqlens, q.device)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    if out is None:
        out = torch.empty((tq, hq, d), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((hq, tq), dtype=torch.float32, device=q.device)
    arr, n = _chunks(chunks)
    st = lib().docmask_attn_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(cu), cu.numel() - 1, arr, n, kv_lo, kv_hi,
                                        hq, hkv, d, float(scale), _ptr(out), _ptr(lse), _stream())
    _check(st, "docmask_attn_fwd_noalloc")
    return out, lse


def attn_bwd(q, k, v, o, lse, d_o, cu_seqlens, chunks, kv_lo: int, kv_hi: int, scale: float | None = None,
             dq=None, dk=None, dv=None, accumulate_dq: bool = False, delta_ready: bool = False, workspace=None):
    """float32 dQ [Tq, Hq, D], dK and dV [Tkv, Hkv, D].

    ``delta_ready`` requires ``workspace`` from an earlier call with the same
    o, d_o, chunks and heads."""
    q, k, v, o, d_o = _bits(q), _bits(k), _bits(v), _bits(o), _bits(d_o)
    tq, hq, d = q.shape
    tkv, hkv, _ = k.shape
    cu = _dev_i32(cu_seqlens, q.device)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    if dq is None:
        dq = torch.empty((tq, hq, d), dtype=torch.float32, device=q.device)
    if dk is None:
        dk = torch.empty((tkv, hkv, d), dtype=torch.float32, device=q.device)
    if dv is None:
        dv = torch.empty((tkv, hkv, d), dtype=torch.float32, device=q.device)
    n_docs = cu.numel() - 1
    ws_bytes = workspace_size(OP_BWD, n_docs, chunks, kv_lo, kv_hi, hq, hkv, d)
    if ws_bytes == 0:
        raise DocmaskError(EINVAL, "docmask_workspace_size")
    if workspace is None or workspace.numel() < ws_bytes:
        if delta_ready:
            raise ValueError("delta_ready needs the workspace of an earlier call")
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    arr, n = _chunks(chunks)
    st = lib().docmask_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(d_o), _ptr(cu), n_docs, arr, n,
                                kv_lo, kv_hi, hq, hkv, d, float(scale), _ptr(dq), _ptr(dk), _ptr(dv),
                                (ACCUMULATE_DQ if accumulate_dq else 0) | (DELTA_READY if delta_ready else 0),
                                _ptr(workspace), workspace.numel(),
                                _stream())
    _check(st, "docmask_attn_bwd")
    return dq, dk, dv


def lse_merge(o_parts, lse_parts, o_out=None, lse_out=None):
    """Merge partials o_parts [P, rows, hq, d] (bf16, or float32 from
    attn_fwd(..., f32_out=True)), lse_parts [P, hq, rows]; bf16 output."""
    f32 = o_parts.dtype == torch.float32
    if not f32:
        o_parts = _bits(o_parts)
    n_parts, rows, hq, d = o_parts.shape
    if o_out is None:
        o_out = torch.empty((rows, hq, d), dtype=torch.bfloat16, device=o_parts.device)
    if lse_out is None:
        lse_out = torch.empty((hq, rows), dtype=torch.float32, device=o_parts.device)
    fn = lib().lse_merge_f32 if f32 else lib().lse_merge
    st = fn(_ptr(o_parts), _ptr(lse_parts), n_parts, rows, hq, d, _ptr(o_out), _ptr(lse_out), _stream())
    _check(st, "lse_merge_f32" if f32 else "lse_merge")
    return o_out, lse_out


def check_errors(workspace) -> int:
    """Synchronise and return the device-side input status of a workspace."""
    return int(lib().docmask_check_errors(_ptr(workspace), _stream()))


def f32_to_bf16(src: torch.Tensor, out=None) -> torch.Tensor:
    if out is None:
        out = torch.empty(src.shape, dtype=torch.bfloat16, device=src.device)
    st = lib().docmask_f32_to_bf16(_ptr(src), _ptr(out), src.numel(), _stream())
    _check(st, "docmask_f32_to_bf16")
    return out


def timing_enable(on: bool = True) -> None:
    """Start (clearing the totals) or stop per-kernel event timing."""
    _check(lib().docmask_timing_enable(1 if on else 0), "docmask_timing_enable")


def timing_read(kernel_class: int) -> tuple[float, int]:
    """(summed milliseconds, launches) of one kernel class since timing_enable(True)."""
    ms = ctypes.c_double(0.0)
    n = _i64(0)
    _check(lib().docmask_timing_read(kernel_class, ctypes.byref(ms), ctypes.byref(n)), "docmask_timing_read")
    return ms.value, int(n.value)


def kernel_class_name(kernel_class: int) -> str:
    return lib().docmask_kernel_class_name(kernel_class).decode()


PROBE_FLOP_PER_WAVE_ITER = 32768 * 16     # per wave and loop iteration, either shape (16 MFMAs of 32x32x16 or 32 of 16x16x32)


def mfma_probe(operands: torch.Tensor, n_workgroups: int, iters: int, out=None, shape: int = 32) -> torch.Tensor:
    """docmask_mfma_probe: back-to-back bf16 MFMAs (shape 32: 32 x 32 x 16,
    shape 16: 16 x 16 x 32) on `operands` (a bf16 device tensor) in
    n_workgroups x 4 waves; float32 [256 n_workgroups], one sum of
    accumulator elements per lane."""
    operands = _bits(operands)
    if out is None:
        out = torch.empty(256 * n_workgroups, dtype=torch.float32, device=operands.device)
    st = lib().docmask_mfma_probe(_ptr(operands), operands.numel(), n_workgroups, iters, shape, _ptr(out), _stream())
    _check(st, "docmask_mfma_probe")
    return out


# ----------------------------------------------------------------- KV exchange
def _host_i32(x):
    a = (ctypes.c_int32 * max(len(x), 1))()
    for i, v in enumerate(x):
        a[i] = int(v)
    return a


def _maps_arr(maps):
    n = len(maps)
    arr = (RowMap * max(n, 1))()
    for i, (s_, d_, l_) in enumerate(maps):
        arr[i].src, arr[i].dst, arr[i].len = int(s_), int(d_), int(l_)
    return arr, n


def _maps_list(arr, n):
    return [(arr[i].src, arr[i].dst, arr[i].len) for i in range(n)]


def copy_rows(src_k, src_v, dst_k, dst_v, maps, zero_gaps: bool):
    """dst[m.dst + t] = src[m.src + t] for every (src, dst, len) map, rows of
    the tensors' first dimension; K and V together or src_v = dst_v = None."""
    def row_bytes_of(t):
        return math.prod(t.shape[1:]) * t.element_size()

    row_bytes = row_bytes_of(src_k)
    for t in (src_k, src_v, dst_k, dst_v):
        if t is not None and not t.is_contiguous():
            raise ValueError("copy_rows needs contiguous tensors")
        if t is not None and row_bytes_of(t) != row_bytes:
            raise ValueError("source and destination rows differ in size")
    arr, n = _maps_arr(maps)
    _check(lib().docmask_copy_rows(_ptr(src_k), _ptr(src_v), src_k.shape[0], _ptr(dst_k), _ptr(dst_v),
                                   dst_k.shape[0], row_bytes, arr, n, 1 if zero_gaps else 0, _stream()),
           "docmask_copy_rows")


def exchange_send_maps(cu_seqlens_host, chunks):
    """(maps, send_rows): local KV rows -> packed send buffer for one worker."""
    cu = _host_i32(cu_seqlens_host)
    arr, n = _chunks(chunks)
    nm, rows = _i32(0), _i64(0)
    _check(lib().docmask_exchange_send_maps(cu, len(cu_seqlens_host) - 1, arr, n, None, 0, ctypes.byref(nm),
                                            ctypes.byref(rows)), "docmask_exchange_send_maps")
    out = (RowMap * max(nm.value, 1))()
    _check(lib().docmask_exchange_send_maps(cu, len(cu_seqlens_host) - 1, arr, n, out, nm.value, ctypes.byref(nm),
                                            ctypes.byref(rows)), "docmask_exchange_send_maps")
    return _maps_list(out, nm.value), int(rows.value)


def exchange_recv_maps(cu_seqlens_host, rank_chunks, rank: int, slot_rows: int):
    """dict(kv_lo, kv_hi, remote, local) for worker `rank` (see docmask.h)."""
    cu = _host_i32(cu_seqlens_host)
    flat = [c for ch in rank_chunks for c in ch]
    arr, _ = _chunks(flat)
    counts = _host_i32([len(ch) for ch in rank_chunks])
    lo, hi, nr, nl = _i32(0), _i32(0), _i32(0), _i32(0)
    args = (cu, len(cu_seqlens_host) - 1, arr, counts, len(rank_chunks), rank, slot_rows, ctypes.byref(lo),
            ctypes.byref(hi))
    _check(lib().docmask_exchange_recv_maps(*args, None, 0, ctypes.byref(nr), None, 0, ctypes.byref(nl)),
           "docmask_exchange_recv_maps")
    rem = (RowMap * max(nr.value, 1))()
    loc = (RowMap * max(nl.value, 1))()
    _check(lib().docmask_exchange_recv_maps(*args, rem, nr.value, ctypes.byref(nr), loc, nl.value, ctypes.byref(nl)),
           "docmask_exchange_recv_maps")
    return {"kv_lo": lo.value, "kv_hi": hi.value, "remote": _maps_list(rem, nr.value),
            "local": _maps_list(loc, nl.value)}


def plan_shards(doc_lengths, n_workers: int, target_ratio: float):
    """FlashCP planner: (per-worker chunk lists, Per-Doc document ids, ratio)."""
    lens = _host_i32(doc_lengths)
    n = len(doc_lengths)
    counts = (ctypes.c_int32 * n_workers)()
    npd, ratio = _i32(0), ctypes.c_double(0.0)
    pd = (ctypes.c_int32 * max(n, 1))()
    _check(lib().docmask_plan_shards(lens, n, n_workers, target_ratio, None, 0, counts, pd, ctypes.byref(npd),
                                     ctypes.byref(ratio)), "docmask_plan_shards")
    total = sum(counts)
    arr = (Chunk * max(total, 1))()
    _check(lib().docmask_plan_shards(lens, n, n_workers, target_ratio, arr, total, counts, pd, ctypes.byref(npd),
                                     ctypes.byref(ratio)), "docmask_plan_shards")
    out, k = [], 0
    for j in range(n_workers):
        out.append([(arr[k + i].g_start, arr[k + i].len) for i in range(counts[j])])
        k += counts[j]
    return out, [pd[i] for i in range(npd.value)], ratio.value
