"""Backward kernels on the GPU vs the fp64 oracle (exact gradients).

The GPU backward takes the GPU forward's O and LSE; the oracle uses its own
float64 forward.  Small problems are compared element by element.  At full
size, each sampled document is checked through a sub-problem the oracle can
afford: its last rows as the query chunk against the document's whole key
range.  dQ of those rows and dK/dV of the keys inside that tail depend only on
the tail rows (a key is attended only by rows at or after it in its document),
so the sub-problem's values are exact there."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
from document_masked_attention_amd import api
from document_masked_attention_amd.workloads import custom_workload, make_config, random_lengths, Workload
from gpu_util import (to_dev, f64, assert_close, O_TOL, gpu_ms, timed_s, record, host_cores,
                      d64_long_workload, D64_LONG_LABEL)

pytestmark = pytest.mark.gpu


def _gpu_fwd_bwd(w: Workload, q, k, v, do, accumulate=False, with_ms=False):
    qd, kd, vd, dod = to_dev(q), to_dev(k), to_dev(v), to_dev(do)
    o, lse = api.attn_fwd(qd, kd, vd, w.cu_seqlens, w.chunks, w.kv_lo, w.kv_hi, w.scale)
    (dq, dk, dv), ms = gpu_ms(lambda: api.attn_bwd(qd, kd, vd, o, lse, dod, w.cu_seqlens, w.chunks, w.kv_lo, w.kv_hi,
                                                   w.scale))
    out = (dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy())
    return (*out, ms) if with_ms else out


def _oracle_backward_by_head(q, k, v, do, cu, chunks, kv_lo, kv_hi, scale, tag):
    """oracle.attention_backward for one KV head and its G query heads, one
    oracle call per query head in parallel threads (BLAS threads shared out);
    dQ per head, dK and dV summed over the heads (each head's share of the
    group's gradient is exactly that head's call)."""
    from threadpoolctl import threadpool_limits
    g = q.shape[1]
    workers = max(1, min(g, host_cores()))

    def one(h):
        r, secs = timed_s(lambda: oracle.attention_backward(q[:, h:h + 1], k, v, do[:, h:h + 1], cu, chunks, kv_lo,
                                                             kv_hi, scale))
        print(f"[bwd] {tag}: oracle query head {h} done ({secs:.1f} s)", flush=True)
        return r

    with threadpool_limits(limits=max(1, host_cores() // workers)):
        with ThreadPoolExecutor(workers) as ex:
            res = list(ex.map(one, range(g)))
    return (np.concatenate([r[0] for r in res], axis=1), np.sum([r[1] for r in res], axis=0),
            np.sum([r[2] for r in res], axis=0))


def _check_small(w: Workload, tag):
    print(f"[bwd] {tag} T={w.total} h={w.hq}/{w.hkv} d={w.d} chunks={w.chunks} kv=[{w.kv_lo},{w.kv_hi})",
          flush=True)
    q, k, v, do = w.q(), w.k(), w.v(), w.do()
    dq, dk, dv = _gpu_fwd_bwd(w, q, k, v, do)
    wq, wk, wv = oracle.attention_backward(f64(q), f64(k), f64(v), f64(do), w.cu_seqlens, w.chunks, w.kv_lo,
                                           w.kv_hi, w.scale)
    assert_close(dq, wq, O_TOL, f"{tag} dQ")
    assert_close(dk, wk, O_TOL, f"{tag} dK")
    assert_close(dv, wv, O_TOL, f"{tag} dV")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("hq,hkv", [(4, 4), (4, 2), (6, 2), (8, 2), (12, 2), (8, 1), (16, 2), (32, 2)])
def test_small_random(d, hq, hkv):
    rng = np.random.default_rng(2000 + d + 10 * hq + hkv)
    total = int(rng.integers(300, 600))
    w = custom_workload(int(rng.integers(1 << 30)), random_lengths(rng, total, 180, p_one=0.1), hq, hkv, d,
                        backward=True)
    _check_small(w, f"small d={d} g={hq // hkv}")


def test_edge_documents():
    for lengths in ([1] * 40, [31, 1, 32, 33, 127, 128, 129, 1, 2], [300], [5, 0, 7, 250]):
        w = custom_workload(len(lengths), lengths, 4, 1, 128, backward=True)
        _check_small(w, f"edge {lengths[:5]}")


def test_chunks_and_kv_ranges():
    rng = np.random.default_rng(11)
    for case in range(4):
        total = int(rng.integers(400, 700))
        lengths = random_lengths(rng, total, 250)
        a = int(rng.integers(0, total // 3))
        b = int(rng.integers(a + 1, total // 2))
        c = int(rng.integers(total // 2, total - 1))
        lo = int(rng.integers(0, total // 2))
        hi = int(rng.integers(lo + 1, total + 1))
        w = custom_workload(case, lengths, 8, 2, [64, 128][case % 2], chunks=[(a, b - a), (c, total - c)],
                            kv_lo=lo, kv_hi=hi, backward=True)
        _check_small(w, f"chunks case {case}")


def test_split_kv_backward_sums_to_full():
    """Per-block calls with the merged O/LSE: exact dK/dV per block, dQ shares add up."""
    w = custom_workload(21, random_lengths(np.random.default_rng(21), 600, 250), 8, 2, 128, backward=True)
    q, k, v, do = w.q(), w.k(), w.v(), w.do()
    qd, kd, vd, dod = to_dev(q), to_dev(k), to_dev(v), to_dev(do)
    cu = w.cu_seqlens
    o, lse = api.attn_fwd(qd, kd, vd, cu, w.chunks, 0, w.total, w.scale)
    dq = torch.zeros((w.tq, w.hq, w.d), dtype=torch.float32, device="cuda")
    dk = torch.empty((w.total, w.hkv, w.d), dtype=torch.float32, device="cuda")
    dv = torch.empty_like(dk)
    cuts = [0, 128, 129, 333, 600]
    for x, y in zip(cuts[:-1], cuts[1:]):
        api.attn_bwd(qd, kd[x:y], vd[x:y], o, lse, dod, cu, w.chunks, x, y, w.scale, dq=dq, dk=dk[x:y],
                     dv=dv[x:y], accumulate_dq=True)
    torch.cuda.synchronize()
    wq, wk, wv = oracle.attention_backward(f64(q), f64(k), f64(v), f64(do), cu, w.chunks, 0, w.total, w.scale)
    assert_close(dq.cpu().numpy(), wq, O_TOL, "split dQ")
    assert_close(dk.cpu().numpy(), wk, O_TOL, "split dK")
    assert_close(dv.cpu().numpy(), wv, O_TOL, "split dV")


def test_split_kv_backward_document_heads_across_block_cuts():
    """KV blocks cut through the first 32 positions of documents, where the
    backward computes pairs in float32 (the head pass): each block's call
    takes only the pairs whose key is in its block, so the shares still sum
    to the oracle's gradients, and to one call over the whole range."""
    lengths = [10, 100, 40, 300, 150]                  # documents start at 0, 10, 110, 150, 450
    cuts = [0, 20, 130, 160, 470, 600]                 # cut inside the heads of the last four
    w = custom_workload(23, lengths, 8, 2, 128, backward=True)
    q, k, v, do = w.q(), w.k(), w.v(), w.do()
    qd, kd, vd, dod = to_dev(q), to_dev(k), to_dev(v), to_dev(do)
    cu = w.cu_seqlens
    o, lse = api.attn_fwd(qd, kd, vd, cu, w.chunks, 0, w.total, w.scale)
    dq1, dk1, dv1 = api.attn_bwd(qd, kd, vd, o, lse, dod, cu, w.chunks, 0, w.total, w.scale)
    dq = torch.zeros((w.tq, w.hq, w.d), dtype=torch.float32, device="cuda")
    dk = torch.empty((w.total, w.hkv, w.d), dtype=torch.float32, device="cuda")
    dv = torch.empty_like(dk)
    for x, y in zip(cuts[:-1], cuts[1:]):
        api.attn_bwd(qd, kd[x:y], vd[x:y], o, lse, dod, cu, w.chunks, x, y, w.scale, dq=dq, dk=dk[x:y],
                     dv=dv[x:y], accumulate_dq=True)
    torch.cuda.synchronize()
    wq, wk, wv = oracle.attention_backward(f64(q), f64(k), f64(v), f64(do), cu, w.chunks, 0, w.total, w.scale)
    for name, got, single, want in (("dQ", dq, dq1, wq), ("dK", dk, dk1, wk), ("dV", dv, dv1, wv)):
        assert_close(got.cpu().numpy(), want, O_TOL, f"split {name} vs oracle")
        assert_close(single.cpu().numpy(), want, O_TOL, f"single {name} vs oracle")
        # rows whose head is cut take Delta from the bf16 O instead of the head pass's own
        assert_close(got.cpu().numpy(), single.cpu().numpy(), 5e-3, f"split vs single {name}")


def test_split_kv_backward_ragged_last_block_delta_ready():
    """Split-KV backward whose second KV block is shorter than the first:
    Delta formed by the first call ([0, 8192)) and reused by the second
    ([8192, 12000), DOCMASK_DELTA_READY) through one workspace, dQ shares
    added; equal to one call over [0, 12000) and to the oracle on sampled rows
    and keys."""
    total = 12000
    w = custom_workload(31, random_lengths(np.random.default_rng(31), total, 5000), 8, 2, 128, backward=True)
    q, k, v, do = w.q(), w.k(), w.v(), w.do()
    qd, kd, vd, dod = to_dev(q), to_dev(k), to_dev(v), to_dev(do)
    cu = w.cu_seqlens
    print(f"[bwd] ragged split-KV with Delta reuse: {len(w.lengths)} documents, blocks [0,8192) [8192,{total})",
          flush=True)
    o, lse = api.attn_fwd(qd, kd, vd, cu, w.chunks, 0, total, w.scale)
    dq1, dk1, dv1 = api.attn_bwd(qd, kd, vd, o, lse, dod, cu, w.chunks, 0, total, w.scale)
    ws = torch.empty(api.workspace_size(api.OP_BWD, len(w.lengths), w.chunks, 0, 8192, w.hq, w.hkv, w.d),
                     dtype=torch.uint8, device="cuda")
    dq = torch.empty_like(dq1)
    dk = torch.empty_like(dk1)
    dv = torch.empty_like(dv1)
    for i, (x, y) in enumerate([(0, 8192), (8192, total)]):
        api.attn_bwd(qd, kd[x:y], vd[x:y], o, lse, dod, cu, w.chunks, x, y, w.scale, dq=dq, dk=dk[x:y],
                     dv=dv[x:y], accumulate_dq=i > 0, delta_ready=i > 0, workspace=ws)
    torch.cuda.synchronize()
    assert_close(dq.cpu().numpy(), dq1.cpu().numpy(), 1e-4, "split vs single dQ")
    assert_close(dk.cpu().numpy(), dk1.cpu().numpy(), 1e-5, "split vs single dK")
    assert_close(dv.cpu().numpy(), dv1.cpu().numpy(), 1e-5, "split vs single dV")
    rows = np.unique(np.concatenate([np.arange(0, total, 997), [total - 1]]))
    wq, _, _ = oracle.attention_backward(f64(q[rows]), f64(k), f64(v), f64(do[rows]), cu,
                                         [(int(r), 1) for r in rows], 0, total, w.scale)
    assert_close(dq.cpu().numpy()[rows], wq, O_TOL, "split dQ vs oracle")
    # dK / dV of the second block's keys: every row of their documents at or after them
    a = int(cu[np.searchsorted(cu, 8192, side="right") - 1])
    wq, wk, wv = oracle.attention_backward(f64(q[a:]), f64(k[a:]), f64(v[a:]), f64(do[a:]), cu, [(a, total - a)],
                                           a, total, w.scale)
    assert_close(dk.cpu().numpy()[8192:], wk[8192 - a:], O_TOL, "split dK vs oracle (second block)")
    assert_close(dv.cpu().numpy()[8192:], wv[8192 - a:], O_TOL, "split dV vs oracle (second block)")


@pytest.mark.parametrize("cfg,seed", [(4, None), (5, None), (4, 11), (4, 12), (4, 13), (5, 12)])
def test_full_size_sampled_documents(cfg, seed):
    """Canonical seeds (the config index) and the extra seeds 11-13."""
    w = make_config(cfg, seed)
    print(f"[bwd] config {cfg} seed {w.seed}: generating inputs", flush=True)
    q, k, v, do = w.q(), w.k(), w.v(), w.do()
    dq, dk, dv = _gpu_fwd_bwd(w, q, k, v, do)
    cu = w.cu_seqlens
    lengths = np.diff(cu)
    order = np.argsort(lengths, kind="stable")
    docs = sorted({int(order[0]), int(order[len(order) // 2]), int(order[-1]), int(order[-2])})
    rng = np.random.default_rng(cfg)
    g = w.hq // w.hkv
    errs = []
    for doc in docs:
        a, b = int(cu[doc]), int(cu[doc + 1])
        tail = min(b - a, 256)
        t0 = b - tail
        kvh = int(rng.integers(w.hkv))
        heads = np.arange(kvh * g, (kvh + 1) * g)
        print(f"[bwd] config {cfg} doc {doc} [{a},{b}) tail {tail} kv head {kvh}", flush=True)
        sq = f64(q[t0:b][:, heads])
        sdo = f64(do[t0:b][:, heads])
        sk = f64(k[a:b, kvh:kvh + 1])
        sv = f64(v[a:b, kvh:kvh + 1])
        wq, wk, wv = oracle.attention_backward(sq, sk, sv, sdo, cu, [(t0, tail)], a, b, w.scale)
        errs.append((assert_close(dq[t0:b][:, heads], wq, O_TOL, f"doc {doc} dQ"),
                     assert_close(dk[t0:b, kvh:kvh + 1], wk[t0 - a:], O_TOL, f"doc {doc} dK"),
                     assert_close(dv[t0:b, kvh:kvh + 1], wv[t0 - a:], O_TOL, f"doc {doc} dV")))
    e = np.max(errs, axis=0)
    record(config=cfg, seed=w.seed, check="backward, document tails",
           compared=f"last <= 256 rows and keys of {len(docs)} documents, one KV-head group each",
           err_dQ=e[0], err_dK=e[1], err_dV=e[2], cores=host_cores())


def _whole_document(w: Workload, q, k, v, do, grads, doc, kvh, label, what, ms=None):
    """dQ, dK, dV of one whole document on one KV-head group against the
    oracle sub-problem chunk = [a, b), KV = [a, b): exact, because a key is
    attended only by rows of its own document."""
    dq, dk, dv = grads
    cu = w.cu_seqlens
    g = w.hq // w.hkv
    a, b = int(cu[doc]), int(cu[doc + 1])
    heads = np.arange(kvh * g, (kvh + 1) * g)
    tag = f"{label} doc {doc} [{a},{b}) ({b - a} tokens) kv head {kvh}"
    print(f"[bwd] {tag}: oracle over the whole document", flush=True)
    (wq, wk, wv), secs = timed_s(lambda: _oracle_backward_by_head(
        f64(q[a:b][:, heads]), f64(k[a:b, kvh:kvh + 1]), f64(v[a:b, kvh:kvh + 1]), f64(do[a:b][:, heads]), cu,
        [(a, b - a)], a, b, w.scale, tag))
    eq = assert_close(dq[a:b][:, heads], wq, O_TOL, f"{tag} dQ")
    ek = assert_close(dk[a:b, kvh:kvh + 1], wk, O_TOL, f"{tag} dK")
    ev = assert_close(dv[a:b, kvh:kvh + 1], wv, O_TOL, f"{tag} dV")
    print(f"[bwd] {tag}: max abs error dQ {eq:.2e} dK {ek:.2e} dV {ev:.2e} (oracle {secs:.1f} s)", flush=True)
    record(config=label, seed=w.seed, check=f"backward, whole document of {b - a} tokens ({what})",
           compared=f"all {b - a} rows and keys, KV head {kvh} with its {g} query heads",
           err_dQ=eq, err_dK=ek, err_dV=ev, gpu_ms=None if ms is None else round(ms, 3), oracle_s=round(secs, 2),
           cores=host_cores())


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("cfg,ranks", [(4, (1,)), (5, (1, 2))])
def test_full_size_whole_long_documents(cfg, ranks):
    """Whole long documents of the full-size workloads (canonical seeds): the
    longest (and, for the 131072-token mix, the second-longest) document,
    every row and every key, one KV-head group; this covers the key-major
    work items' whole walks over the document's query blocks (production
    guide, "Step 1: Establish a Single-GPU Numerical Baseline": long
    sequences, not only short ones)."""
    w = make_config(cfg)
    print(f"[bwd] config {cfg} seed {w.seed}: generating inputs", flush=True)
    q, k, v, do = w.q(), w.k(), w.v(), w.do()
    *grads, ms = _gpu_fwd_bwd(w, q, k, v, do, with_ms=True)
    order = np.argsort(-np.diff(w.cu_seqlens), kind="stable")
    for rank in ranks:
        _whole_document(w, q, k, v, do, grads, int(order[rank - 1]), (3 * rank + cfg) % w.hkv, cfg,
                        f"rank {rank} by length", ms)


def _every_document_tail(w: Workload, q, k, v, do, grads, label):
    """Every document, every KV head: its last <= 256 rows and keys against
    the oracle sub-problem (exact there), so every short document is checked
    whole."""
    from threadpoolctl import threadpool_limits
    dq, dk, dv = grads
    cu = w.cu_seqlens
    g = w.hq // w.hkv
    jobs = [(doc, kvh) for doc in range(len(cu) - 1) for kvh in range(w.hkv)]

    def one(job):
        doc, kvh = job
        a, b = int(cu[doc]), int(cu[doc + 1])
        t0 = b - min(b - a, 256)
        heads = np.arange(kvh * g, (kvh + 1) * g)
        wq, wk, wv = oracle.attention_backward(f64(q[t0:b][:, heads]), f64(k[a:b, kvh:kvh + 1]),
                                               f64(v[a:b, kvh:kvh + 1]), f64(do[t0:b][:, heads]), cu,
                                               [(t0, b - t0)], a, b, w.scale)
        return (float(np.abs(dq[t0:b][:, heads] - wq).max()), float(np.abs(dk[t0:b, kvh:kvh + 1] - wk[t0 - a:]).max()),
                float(np.abs(dv[t0:b, kvh:kvh + 1] - wv[t0 - a:]).max()))

    errs, secs = timed_s(lambda: _map_oracle(one, jobs, threadpool_limits))
    e = np.max(np.array(errs), axis=0)
    print(f"[bwd] {label}: {len(jobs)} (document, KV head) tails, max abs error dQ {e[0]:.2e} dK {e[1]:.2e} "
          f"dV {e[2]:.2e} (oracle {secs:.1f} s)", flush=True)
    record(config=label, seed=w.seed, check="backward, every document tail on every KV head",
           compared=f"last <= 256 rows and keys of all {len(cu) - 1} documents x {w.hkv} KV-head groups",
           err_dQ=e[0], err_dK=e[1], err_dV=e[2], oracle_s=round(secs, 2), cores=host_cores())
    for name, err in zip(("dQ", "dK", "dV"), e):
        assert err <= O_TOL, f"{label}: {name} max abs error {err:.3e} > {O_TOL}"


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg", [4, 5])
def test_full_size_every_document_tail_every_kv_head(cfg):
    """Every document of the full-size workloads (canonical seeds) on every KV
    head -- the rows with the fewest keys, whose P and dS are the largest, are
    where rounding them to the bf16 matrix-core operands costs the most."""
    w = make_config(cfg)
    print(f"[bwd] config {cfg} seed {w.seed}: generating inputs", flush=True)
    q, k, v, do = w.q(), w.k(), w.v(), w.do()
    _every_document_tail(w, q, k, v, do, _gpu_fwd_bwd(w, q, k, v, do), cfg)


@pytest.mark.timeout(900)
def test_d64_long_documents():
    """Head size 64 at full size (the D = 64 kernels have their own LDS
    layouts and tile walks): the 65536-token lognormal mix whose longest
    document has 22,529 tokens, 16 query / 4 KV heads.  That document whole on
    one KV-head group, and every document's tail on every KV head."""
    w = d64_long_workload()
    print(f"[bwd] d64 long documents seed {w.seed}: generating inputs", flush=True)
    q, k, v, do = w.q(), w.k(), w.v(), w.do()
    *grads, ms = _gpu_fwd_bwd(w, q, k, v, do, with_ms=True)
    longest = int(np.argmax(np.diff(w.cu_seqlens)))
    _whole_document(w, q, k, v, do, grads, longest, 1, D64_LONG_LABEL, "the longest", ms)
    _every_document_tail(w, q, k, v, do, grads, D64_LONG_LABEL)


def _map_oracle(fn, jobs, threadpool_limits):
    """fn over jobs on the host cores, one BLAS thread per worker."""
    with threadpool_limits(limits=1):
        with ThreadPoolExecutor(max(1, host_cores())) as ex:
            return list(ex.map(fn, jobs))


def test_one_million_tokens_document_tails():
    """2^20 packed tokens: dQ/dK/dV of the last rows of the longest and the
    last document (64-bit offsets past 2^31 bytes in dQ)."""
    from document_masked_attention_amd.workloads import lognormal_docs
    total = 1 << 20
    w = custom_workload(21, lognormal_docs(21, 4096, 1.2, 64, 65536, total), 16, 2, 128, backward=True)
    print(f"[bwd] 2^20 tokens, {len(w.lengths)} documents: generating inputs", flush=True)
    q, k, v, do = w.q(), w.k(), w.v(), w.do()
    dq, dk, dv = _gpu_fwd_bwd(w, q, k, v, do)
    cu = w.cu_seqlens
    lengths = np.diff(cu)
    g = w.hq // w.hkv
    for doc in sorted({int(np.argmax(lengths)), len(lengths) - 1}):
        a, b = int(cu[doc]), int(cu[doc + 1])
        tail = min(b - a, 128)
        t0 = b - tail
        kvh = doc % w.hkv
        heads = np.arange(kvh * g, (kvh + 1) * g)
        print(f"[bwd] 2^20 doc {doc} [{a},{b}) tail {tail} kv head {kvh}", flush=True)
        wq, wk, wv = oracle.attention_backward(f64(q[t0:b][:, heads]), f64(k[a:b, kvh:kvh + 1]),
                                               f64(v[a:b, kvh:kvh + 1]), f64(do[t0:b][:, heads]), cu, [(t0, tail)],
                                               a, b, w.scale)
        assert_close(dq[t0:b][:, heads], wq, O_TOL, f"doc {doc} dQ")
        assert_close(dk[t0:b, kvh:kvh + 1], wk[t0 - a:], O_TOL, f"doc {doc} dK")
        assert_close(dv[t0:b, kvh:kvh + 1], wv[t0 - a:], O_TOL, f"doc {doc} dV")



@pytest.mark.timeout(900)
def test_cp_rank_split_backward():
    """Rank 3 of CP = 8 run as a ring rank runs it: per-(chunk, 8192-key block)
    backward calls with the merged O and LSE, dQ shares accumulated, Delta
    formed by each chunk's first call; equals the single call over the whole
    KV range, whose dQ on sampled rows matches the oracle."""
    w = make_config(3)
    q, k, v, do = w.q(), w.k(), w.v(), w.do()
    qd, kd, vd, dod = to_dev(q), to_dev(k), to_dev(v), to_dev(do)
    cu = w.cu_seqlens
    o1, l1 = api.attn_fwd(qd, kd, vd, cu, w.chunks, w.kv_lo, w.kv_hi, w.scale)
    dq1, dk1, dv1 = api.attn_bwd(qd, kd, vd, o1, l1, dod, cu, w.chunks, w.kv_lo, w.kv_hi, w.scale)
    need = api.schedule(cu, w.chunks, w.kv_lo, w.kv_hi, 8192, 8192)["need"].cpu().numpy()
    dq = torch.empty_like(dq1)
    dk = torch.zeros_like(dk1)
    dv = torch.zeros_like(dv1)
    row0 = 0
    for ci, (g, n) in enumerate(w.chunks):
        blocks = list(range(need[ci, 0] // 8192, (need[ci, 1] + 8191) // 8192))
        print(f"[cp bwd] chunk {g} blocks {blocks}", flush=True)
        rows = slice(row0, row0 + n)
        po = torch.empty((len(blocks), n, w.hq, w.d), dtype=torch.bfloat16, device="cuda")
        pl = torch.empty((len(blocks), w.hq, n), dtype=torch.float32, device="cuda")
        for i, b in enumerate(blocks):
            sl = slice(8192 * b, 8192 * (b + 1))
            api.attn_fwd(qd[rows], kd[sl], vd[sl], cu, [(g, n)], sl.start, sl.stop, w.scale, out=po[i], lse=pl[i])
        om, lm = api.lse_merge(po, pl)
        ws = torch.empty(api.workspace_size(api.OP_BWD, len(w.lengths), [(g, n)], 0, 8192, w.hq, w.hkv, w.d),
                         dtype=torch.uint8, device="cuda")
        dkb = torch.empty((8192, w.hkv, w.d), dtype=torch.float32, device="cuda")
        dvb = torch.empty_like(dkb)
        for i, b in enumerate(blocks):
            sl = slice(8192 * b, 8192 * (b + 1))
            api.attn_bwd(qd[rows], kd[sl], vd[sl], om, lm, dod[rows], cu, [(g, n)], sl.start, sl.stop, w.scale,
                         dq=dq[rows], dk=dkb, dv=dvb, accumulate_dq=i > 0, delta_ready=i > 0, workspace=ws)
            dk[sl] += dkb
            dv[sl] += dvb
        row0 += n
    torch.cuda.synchronize()
    assert_close(dq.cpu().numpy(), dq1.cpu().numpy(), O_TOL, "per-block vs single-call dQ")
    assert_close(dk.cpu().numpy(), dk1.cpu().numpy(), O_TOL, "per-block vs single-call dK")
    assert_close(dv.cpu().numpy(), dv1.cpu().numpy(), O_TOL, "per-block vs single-call dV")
    sel = np.unique(np.concatenate([np.arange(0, w.tq, 1021), [w.tq - 1]]))
    pos = w.local_positions()
    wq, _, _ = oracle.attention_backward(f64(q[sel]), f64(k), f64(v), f64(do[sel]), cu,
                                         [(int(pos[r]), 1) for r in sel], w.kv_lo, w.kv_hi, w.scale)
    assert_close(dq1.cpu().numpy()[sel], wq, O_TOL, "single-call dQ vs oracle")
    # dK / dV of sampled keys against the oracle: 64-key runs at the start of
    # each chunk's document (attended by every row of the chunk, the longest
    # walks over query blocks) and at each chunk's end.  On this rank a key is
    # attended only by the rank's rows of its own document at or after it, so
    # the sub-problem (those rows; keys from the document start to the chunk
    # end) is exact for the sampled keys.  One KV-head group each.
    dk1n, dv1n = dk1.cpu().numpy(), dv1.cpu().numpy()
    g = w.hq // w.hkv
    row0 = 0
    for ci, (gs, n) in enumerate(w.chunks):
        d = int(np.searchsorted(cu, gs, side="right") - 1)
        ds, de = int(cu[d]), int(cu[d + 1])
        assert gs + n <= de, "the sampled keys' attending rows are the chunk's own"
        for j0 in (ds, gs + n - 64):
            kvh = (ci + j0) % w.hkv
            heads = np.arange(kvh * g, (kvh + 1) * g)
            r0 = max(j0, gs)
            rows = slice(row0 + r0 - gs, row0 + n)
            keys = np.arange(ds, gs + n)
            tag = f"CP rank chunk {gs}: keys [{j0},{j0 + 64}) kv head {kvh}, {gs + n - r0} attending rows"
            print(f"[cp bwd] {tag}", flush=True)
            (_, wk, wv), secs = timed_s(lambda: _oracle_backward_by_head(
                f64(q[rows][:, heads]), f64(k[keys][:, kvh:kvh + 1]), f64(v[keys][:, kvh:kvh + 1]),
                f64(do[rows][:, heads]), cu, [(r0, gs + n - r0)], ds, gs + n, w.scale, tag))
            ek = assert_close(dk1n[j0:j0 + 64, kvh:kvh + 1], wk[j0 - ds:j0 - ds + 64], O_TOL, f"{tag} dK")
            ev = assert_close(dv1n[j0:j0 + 64, kvh:kvh + 1], wv[j0 - ds:j0 - ds + 64], O_TOL, f"{tag} dV")
            record(config=3, seed=w.seed, check=f"backward over the rank's whole KV range, 64 keys at {j0}",
                   compared=f"dK, dV of 64 keys (KV head {kvh}, {g} query heads, {gs + n - r0} attending rows)",
                   err_dK=ek, err_dV=ev, oracle_s=round(secs, 2), cores=host_cores())
        row0 += n
