"""The C-ABI library on the CPU: it loads, exports every function the public
header declares, and rejects bad arguments on the host before touching the GPU
(these calls never reach a HIP launch)."""
import ctypes
import os
import re

import pytest

from document_masked_attention_amd import api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "docmask.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(api.lib_path()):
        from document_masked_attention_amd import build
        build.build()
    return api.lib()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w]*\s*\**\s+\**([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_every_declared_symbol_is_exported(lib):
    names = _declared_functions()
    assert {"docmask_attn_fwd", "docmask_attn_bwd", "lse_merge", "docmask_schedule"} <= set(names)
    handle = ctypes.CDLL(api.lib_path())
    for n in names:
        assert hasattr(handle, n), n
    assert set(names) == set(api._SIGNATURES), "binding and header disagree"


FAKE = 0x10000            # an aligned, never dereferenced stand-in address
MIS = 0x10002             # misaligned


def _fwd(lib, q=FAKE, k=FAKE, v=FAKE, cu=FAKE, n_docs=3, chunks=((0, 100),), kv=(0, 100), hq=4, hkv=2, d=128,
         scale=0.1, o=FAKE, lse=FAKE, ws=FAKE, ws_bytes=16, n_chunks=None):
    arr, n = api._chunks(list(chunks))
    return lib.docmask_attn_fwd(q, k, v, cu, n_docs, arr, n if n_chunks is None else n_chunks, kv[0], kv[1], hq,
                                hkv, d, scale, o, lse, ws, ws_bytes, None)


def test_fwd_argument_validation(lib):
    assert _fwd(lib, d=96) == api.EUNSUPPORTED
    assert _fwd(lib, hq=6, hkv=4) == api.EINVAL
    assert _fwd(lib, hkv=0) == api.EINVAL
    assert _fwd(lib, n_docs=0) == api.EINVAL
    assert _fwd(lib, cu=None) == api.EINVAL
    assert _fwd(lib, kv=(50, 10)) == api.EINVAL
    assert _fwd(lib, kv=(-1, 10)) == api.EINVAL
    assert _fwd(lib, chunks=((10, 20), (5, 3))) == api.EINVAL          # not ascending
    assert _fwd(lib, chunks=((10, 20), (25, 3))) == api.EINVAL         # overlapping
    assert _fwd(lib, chunks=((0, -1),)) == api.EINVAL
    assert _fwd(lib, n_chunks=api.MAX_CHUNKS + 1) == api.EINVAL
    assert _fwd(lib, q=MIS) == api.EINVAL
    assert _fwd(lib, o=None) == api.EINVAL
    assert _fwd(lib, k=None) == api.EINVAL
    assert _fwd(lib, scale=float("nan")) == api.EINVAL
    assert _fwd(lib, scale=float("inf")) == api.EINVAL
    assert _fwd(lib, scale=0.0) == api.EINVAL                          # masked scores would become NaN
    assert _fwd(lib, scale=-0.1) == api.EINVAL                         # would reverse the softmax reference
    arr, n = api._chunks([(0, 100)])
    for bad_scale in (0.0, -0.1, float("nan")):
        assert lib.docmask_attn_fwd_f32out(FAKE, FAKE, FAKE, FAKE, 3, arr, n, 0, 100, 4, 2, 128, bad_scale, FAKE,
                                           FAKE, FAKE, 1 << 30, None) == api.EINVAL
    assert _fwd(lib, ws=None) == api.EWORKSPACE
    assert _fwd(lib, ws_bytes=16) == api.EWORKSPACE
    assert _fwd(lib, chunks=()) == api.OK                              # no query rows: nothing to do


def test_noalloc_forward_validation(lib):
    """Checked on the host before the static scratch is looked up."""
    def call(chunks=((0, 100),), scale=0.1, d=128, cu=FAKE, hq=4, hkv=2):
        arr, n = api._chunks(list(chunks))
        return lib.docmask_attn_fwd_noalloc(FAKE, FAKE, FAKE, cu, 3, arr, n, 0, 100, hq, hkv, d, scale, FAKE, FAKE,
                                            None)
    assert call(scale=0.0) == api.EINVAL
    assert call(scale=float("nan")) == api.EINVAL
    assert call(cu=None) == api.EINVAL
    assert call(d=96) == api.EUNSUPPORTED
    assert call(hq=6, hkv=4) == api.EINVAL
    assert call(chunks=()) == api.OK                                   # no query rows: nothing to do
    # the forward workspace of 2^22 query rows (>= 40 bytes per 32-row tile) exceeds the static scratch
    big = [(0, 1 << 22)]
    assert api.workspace_size(api.OP_FWD, 3, big, 0, 100, 16, 2, 128) > api.NOALLOC_SCRATCH_BYTES
    assert call(chunks=big, hq=16) == api.ESCRATCH
    assert "static scratch" in api.strerror(api.ESCRATCH)


def test_bwd_and_merge_validation(lib):
    arr, n = api._chunks([(0, 100)])
    args = [FAKE] * 7 + [3, arr, n, 0, 100, 4, 2, 128, 0.1, FAKE, FAKE, FAKE]
    assert lib.docmask_attn_bwd(*args, 0, FAKE, 16, None) == api.EWORKSPACE
    assert lib.docmask_attn_bwd(*args, 8, FAKE, 1 << 30, None) == api.EINVAL      # unknown flag
    bad = list(args)
    bad[16] = MIS                                                                 # misaligned dq
    assert lib.docmask_attn_bwd(*bad, 0, FAKE, 1 << 30, None) == api.EINVAL
    for bad_scale in (0.0, -0.1, float("nan"), float("-inf")):
        bad = list(args)
        bad[15] = bad_scale
        assert lib.docmask_attn_bwd(*bad, 0, FAKE, 1 << 30, None) == api.EINVAL
    assert lib.lse_merge(FAKE, FAKE, 0, 10, 4, 128, FAKE, FAKE, None) == api.EINVAL
    assert lib.lse_merge(FAKE, FAKE, 2, 10, 4, 32, FAKE, FAKE, None) == api.EUNSUPPORTED
    assert lib.lse_merge(MIS, FAKE, 2, 10, 4, 128, FAKE, FAKE, None) == api.EINVAL
    assert lib.lse_merge(FAKE, FAKE, 2, 0, 4, 128, FAKE, FAKE, None) == api.OK
    assert lib.docmask_f32_to_bf16(FAKE, FAKE, -1, None) == api.EINVAL
    assert lib.docmask_check_errors(None, None) == api.EINVAL


def test_workspace_sizes(lib):
    fwd = api.workspace_size(api.OP_FWD, 3, [(0, 4096)], 0, 4096, 32, 8, 128)
    bwd = api.workspace_size(api.OP_BWD, 3, [(0, 4096)], 0, 4096, 32, 8, 128)
    assert fwd > 0 and bwd > 32 * 4096 * 4                  # the backward holds Delta [Hq, Tq]
    assert api.workspace_size(api.OP_FWD, 3, [(0, 4096)], 0, 4096, 32, 8, 96) == 0
    assert api.workspace_size(7, 3, [(0, 4096)], 0, 4096, 32, 8, 128) == 0
    assert api.schedule_workspace_size([(0, 100)], 0, 100, 16, 16) > 0
    # the backward workspace grows with the KV range, Delta [Hq, Tq] does not
    small = api.workspace_size(api.OP_BWD, 3, [(0, 4096)], 0, 100, 32, 8, 128)
    assert 32 * 4096 * 4 < small < bwd
    assert api.schedule_workspace_size([(0, 100)], 0, 100, 0, 16) == 0


def test_strerror(lib):
    for s in (api.OK, api.EINVAL, api.EUNSUPPORTED, api.EWORKSPACE, api.EHIP, api.EDEVICE_INPUT, api.ESCRATCH):
        assert api.strerror(s)
    assert "unknown" in api.strerror(123)


def test_timing_controls(lib):
    names = {api.kernel_class_name(i) for i in range(api.N_KERNEL_CLASSES)}
    assert len(names) == api.N_KERNEL_CLASSES and "dkdv_kernel" in names and "fwd_kernel" in names
    assert api.kernel_class_name(api.N_KERNEL_CLASSES) == "unknown"
    api.timing_enable(True)
    assert api.timing_read(api.KERNEL_DKDV) == (0.0, 0)      # nothing launched
    api.timing_enable(False)
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    assert lib.docmask_timing_read(-1, ctypes.byref(ms), ctypes.byref(n)) == api.EINVAL
    assert lib.docmask_timing_read(api.N_KERNEL_CLASSES, ctypes.byref(ms), ctypes.byref(n)) == api.EINVAL
    assert lib.docmask_timing_read(0, None, ctypes.byref(n)) == api.EINVAL


def test_mfma_probe_validation(lib):
    probe = lib.docmask_mfma_probe
    assert probe(None, 1024, 1, 1, 32, FAKE, None) == api.EINVAL
    assert probe(FAKE, 1024, 1, 1, 32, None, None) == api.EINVAL
    assert probe(MIS, 1024, 1, 1, 32, FAKE, None) == api.EINVAL        # operands not 16-byte aligned
    assert probe(FAKE, 1024, 1, 1, 32, FAKE + 2, None) == api.EINVAL   # out not 4-byte aligned
    assert probe(FAKE, 120, 1, 1, 32, FAKE, None) == api.EINVAL        # fewer than 128 values
    assert probe(FAKE, 1028, 1, 1, 32, FAKE, None) == api.EINVAL       # not a multiple of 8
    assert probe(FAKE, 1024, 0, 1, 32, FAKE, None) == api.EINVAL
    assert probe(FAKE, 1024, 1, -1, 32, FAKE, None) == api.EINVAL
    for shape in (0, 8, 24, 64):                                       # only 32 and 16
        assert probe(FAKE, 1024, 1, 1, shape, FAKE, None) == api.EINVAL


def _copy(lib, maps=((0, 0, 4),), src_k=FAKE, src_v=FAKE, dst_k=FAKE, dst_v=FAKE, src_rows=10, dst_rows=10,
          row_bytes=64, zero=0):
    arr, n = api._maps_arr(list(maps))
    return lib.docmask_copy_rows(src_k, src_v, src_rows, dst_k, dst_v, dst_rows, row_bytes, arr, n, zero, None)


def test_copy_rows_validation(lib):
    assert _copy(lib, row_bytes=40) == api.EINVAL                       # not a multiple of 16
    assert _copy(lib, row_bytes=0) == api.EINVAL
    assert _copy(lib, maps=((0, 4, 4), (0, 2, 4))) == api.EINVAL        # destinations not ascending
    assert _copy(lib, maps=((0, 0, 4), (0, 3, 2))) == api.EINVAL        # overlapping destinations
    assert _copy(lib, maps=((8, 0, 4),)) == api.EINVAL                  # source past its end
    assert _copy(lib, maps=((0, 8, 4),)) == api.EINVAL                  # destination past its end
    assert _copy(lib, maps=((-2, 0, 4),)) == api.EINVAL                 # -1 is the only negative source (zeros)
    assert _copy(lib, maps=((-1, 8, 4),)) == api.EINVAL                 # zero run past the destination end
    assert _copy(lib, maps=((0, 0, -1),)) == api.EINVAL
    assert _copy(lib, src_v=None) == api.EINVAL                         # K and V must come together
    assert _copy(lib, dst_k=MIS) == api.EINVAL
    assert _copy(lib, src_k=None) == api.EINVAL
    assert _copy(lib, dst_rows=-1) == api.EINVAL
    assert _copy(lib, maps=()) == api.OK                                # nothing to write
    assert _copy(lib, maps=((0, 0, 0),)) == api.OK                      # empty map only
    assert _copy(lib, maps=(), dst_rows=0, zero=1) == api.OK
