"""Forward kernel and LSE merge on the GPU vs the fp64 oracle.

Small problems are compared element by element; the full-size workloads are
compared on sampled rows that the oracle computes against the full key range
(their explicit mask over every key), and the 2 x CP rank workload is run the
way a rank runs it: one partial per (chunk, 8192-key block), merged."""
import math

import numpy as np
import pytest
import torch

import oracle
from document_masked_attention_amd import api
from document_masked_attention_amd.workloads import custom_workload, make_config, random_lengths, Workload
from gpu_util import (to_dev, bf16_to_np, f64, assert_close, O_TOL, LSE_TOL, gpu_ms, timed_s, record,
                      host_cores, d64_long_workload, D64_LONG_LABEL)

pytestmark = pytest.mark.gpu


def _run_and_compare(w: Workload, rows=None, tag="", config=None):
    """GPU forward of the whole workload against the oracle on `rows` (all by
    default); with `config`, the measured errors and times are recorded."""
    print(f"[fwd] {tag} {w.name} seed={w.seed} T={w.total} tq={w.tq} h={w.hq}/{w.hkv} d={w.d} "
          f"chunks={w.chunks[:4]} kv=[{w.kv_lo},{w.kv_hi})", flush=True)
    q, k, v = w.q(), w.k(), w.v()
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    (o, lse), ms = gpu_ms(lambda: api.attn_fwd(qd, kd, vd, w.cu_seqlens, w.chunks, w.kv_lo, w.kv_hi, w.scale))
    o_np = bf16_to_np(o)
    lse_np = lse.cpu().numpy().astype(np.float64)
    sel = np.arange(w.tq) if rows is None else np.asarray(rows)
    (want_o, want_l), secs = timed_s(lambda: oracle.attention_forward(f64(q), f64(k), f64(v), w.cu_seqlens, w.chunks,
                                                                       w.kv_lo, w.kv_hi, w.scale, rows=sel))
    eo = assert_close(o_np[sel], want_o, O_TOL, f"{tag} O")
    el = assert_close(lse_np[:, sel], want_l, LSE_TOL, f"{tag} LSE")
    if config is not None:
        record(config=config, seed=w.seed, check="forward", compared=f"{sel.size} of {w.tq} rows, all heads",
               err_O=eo, err_LSE=el, gpu_ms=round(ms, 3), oracle_s=round(secs, 2), cores=host_cores())
    return q, k, v, o_np, lse_np


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("hq,hkv", [(4, 4), (4, 2), (6, 2), (8, 2), (12, 2), (8, 1), (16, 2), (32, 2)])
def test_small_random(d, hq, hkv):
    rng = np.random.default_rng(1000 + d + 10 * hq + hkv)
    total = int(rng.integers(300, 700))
    lengths = random_lengths(rng, total, 200, p_one=0.1)
    w = custom_workload(int(rng.integers(1 << 30)), lengths, hq, hkv, d)
    _run_and_compare(w, tag=f"small d={d} g={hq // hkv}")


def test_edge_documents():
    """Length-1 documents, boundaries at tile edges +-1, ragged tails."""
    for lengths in ([1] * 70, [31, 1, 32, 33, 63, 64, 65, 127, 128, 129, 1, 1, 2],
                    [64] * 5 + [1], [200], [1, 199], [5, 0, 7, 250]):
        for hq, hkv in ((4, 1), (8, 8)):
            w = custom_workload(sum(lengths) + hq, lengths, hq, hkv, 128)
            _run_and_compare(w, tag=f"edge {lengths[:6]}")


def test_whole_sequence_one_document_is_causal():
    w = custom_workload(77, [1000], 8, 2, 64)
    _run_and_compare(w, tag="one doc")


def test_chunks_and_kv_ranges():
    """Two-chunk query lists and KV ranges that cut documents, leaving rows empty."""
    rng = np.random.default_rng(5)
    for case in range(8):
        total = int(rng.integers(400, 900))
        lengths = random_lengths(rng, total, 300)
        a = int(rng.integers(0, total // 3))
        b = int(rng.integers(a + 1, total // 2))
        c = int(rng.integers(total // 2, total - 1))
        chunks = [(a, b - a), (c, total - c)]
        lo = int(rng.integers(0, total // 2))
        hi = int(rng.integers(lo + 1, total + 1))
        hq, hkv = [(4, 1), (8, 2), (4, 4)][case % 3]
        w = custom_workload(case, lengths, hq, hkv, [64, 128][case % 2], chunks=chunks, kv_lo=lo, kv_hi=hi)
        _run_and_compare(w, tag=f"chunks case {case}")


def test_first_token_outputs_its_value_row_exactly():
    lengths = [1, 17, 64, 3, 129, 1, 300]
    w = custom_workload(9, lengths, 8, 2, 128)
    q, k, v, o_np, _ = _run_and_compare(w, tag="first token")
    cu = w.cu_seqlens
    for a in cu[:-1]:
        for h in range(8):
            assert np.array_equal(o_np[a, h], f64(v)[a, h // 4]), f"row {a} head {h}"


def test_empty_kv_range_rows():
    """KV range that no row may attend: O = 0, LSE = -inf everywhere."""
    w = custom_workload(3, [100, 100], 4, 2, 64, chunks=[(0, 100)], kv_lo=100, kv_hi=200)
    _, _, _, o_np, lse_np = _run_and_compare(w, tag="empty kv")
    assert np.all(o_np == 0) and np.all(np.isneginf(lse_np))


def test_config1_full():
    _run_and_compare(make_config(1), tag="config 1", config=1)


def _sample_rows(w: Workload, n: int, seed: int):
    rng = np.random.default_rng(seed)
    cu = w.cu_seqlens
    pos = w.local_positions()
    firsts = np.nonzero(np.isin(pos, cu[:-1]))[0][:16]                # first rows of documents
    ends = np.nonzero(np.isin(pos + 1, cu[1:]))[0][:16]               # last rows of documents
    edges = np.arange(31, w.tq, 8192)[:8]
    rand = rng.choice(w.tq, size=n, replace=False)
    return np.unique(np.concatenate([firsts, ends, edges, rand, [0, w.tq - 1]]))


@pytest.mark.parametrize("cfg,seed", [(2, None), (4, None), (5, None), (2, 11), (2, 12), (2, 13), (4, 11), (4, 12),
                                      (4, 13), (5, 11)])
def test_full_size_sampled_rows(cfg, seed):
    """Canonical seeds (the config index) and the extra seeds 11-13."""
    w = make_config(cfg, seed)
    _run_and_compare(w, rows=_sample_rows(w, 128 if cfg < 5 else 64, cfg), tag=f"config {cfg} seed {w.seed} sampled",
                     config=cfg)


def _every_document_head(w: Workload, q, k, v, label):
    """GPU forward of the whole workload; every document's first <= 256 rows on
    every query head against the oracle over those rows and keys (exact: a row
    attends only earlier keys of its document).  Returns the largest errors."""
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    o, lse = api.attn_fwd(to_dev(q), to_dev(k), to_dev(v), w.cu_seqlens, w.chunks, w.kv_lo, w.kv_hi, w.scale)
    o = bf16_to_np(o)
    lse = lse.cpu().numpy()
    cu = w.cu_seqlens
    g = w.hq // w.hkv

    def one(job):
        doc, kvh = job
        a, b = int(cu[doc]), int(cu[doc + 1])
        n = min(b - a, 256)
        heads = np.arange(kvh * g, (kvh + 1) * g)
        wo, wl = oracle.attention_forward(f64(q[a:a + n][:, heads]), f64(k[a:a + n, kvh:kvh + 1]),
                                          f64(v[a:a + n, kvh:kvh + 1]), cu, [(a, n)], a, a + n, w.scale)
        return (float(np.abs(o[a:a + n][:, heads] - wo).max()), float(np.abs(lse[heads][:, a:a + n] - wl).max()))

    jobs = [(doc, kvh) for doc in range(len(cu) - 1) for kvh in range(w.hkv)]

    def run():
        with threadpool_limits(limits=1):
            with ThreadPoolExecutor(max(1, host_cores())) as ex:
                return list(ex.map(one, jobs))

    errs, secs = timed_s(run)
    e = np.max(np.array(errs), axis=0)
    print(f"[fwd] {label}: {len(jobs)} (document, KV head) heads, max abs error O {e[0]:.2e} LSE {e[1]:.2e} "
          f"(oracle {secs:.1f} s)", flush=True)
    record(config=label, seed=w.seed, check="forward, every document's first rows on every head",
           compared=f"first <= 256 rows of all {len(cu) - 1} documents, all {w.hq} heads",
           err_O=e[0], err_LSE=e[1], oracle_s=round(secs, 2), cores=host_cores())
    assert e[0] <= O_TOL, f"O max abs error {e[0]:.3e}"
    assert e[1] <= LSE_TOL, f"LSE max abs error {e[1]:.3e}"


@pytest.mark.timeout(600)
@pytest.mark.parametrize("cfg", [4, 5])
def test_full_size_every_document_head_every_head(cfg):
    """Every document of the full-size workloads (canonical seeds), every
    query head: its first <= 256 rows against the oracle over those rows and
    keys -- the rows with the fewest keys, whose probabilities are the largest."""
    w = make_config(cfg)
    print(f"[fwd] config {cfg} seed {w.seed}: every document's first rows", flush=True)
    _every_document_head(w, w.q(), w.k(), w.v(), cfg)


@pytest.mark.timeout(600)
def test_d64_long_documents():
    """Head size 64 at full size (the D = 64 kernels have their own LDS
    layouts and tile walks): the 65536-token lognormal mix with a
    22,529-token document, 16 query / 4 KV heads.  Sampled rows (first and
    last rows of documents among them) against the oracle over the whole
    key range, then every document's first <= 256 rows on every head."""
    w = d64_long_workload()
    _run_and_compare(w, rows=_sample_rows(w, 128, D64_LONG_LABEL), tag="d64 long documents sampled",
                     config=D64_LONG_LABEL)
    _every_document_head(w, w.q(), w.k(), w.v(), D64_LONG_LABEL)


@pytest.mark.parametrize("seed", [None, 11])
def test_cp_rank_partials_and_merge(seed):
    """Rank 3 of CP = 8: per-chunk partials over the 8192-key blocks the need
    list names, merged with lse_merge; sampled rows vs the oracle over the full
    key range; the merged result also equals the single full-range call."""
    w = make_config(3, seed)
    q, k, v = w.q(), w.k(), w.v()
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    cu = w.cu_seqlens
    sched = api.schedule(cu, w.chunks, w.kv_lo, w.kv_hi, 8192, 8192)
    need = sched["need"].cpu().numpy()
    row0 = 0
    for ci, (g, n) in enumerate(w.chunks):
        lo_b, hi_b = need[ci, 0] // 8192, (need[ci, 1] + 8191) // 8192
        blocks = list(range(lo_b, hi_b))
        print(f"[cp] chunk {g} blocks {blocks}", flush=True)
        parts_o = torch.empty((len(blocks), n, w.hq, w.d), dtype=torch.bfloat16, device="cuda")
        parts_l = torch.empty((len(blocks), w.hq, n), dtype=torch.float32, device="cuda")
        for i, b in enumerate(blocks):
            api.attn_fwd(qd[row0:row0 + n], kd[8192 * b:8192 * (b + 1)], vd[8192 * b:8192 * (b + 1)], cu,
                         [(g, n)], 8192 * b, 8192 * (b + 1), w.scale, out=parts_o[i], lse=parts_l[i])
        o_m, l_m = api.lse_merge(parts_o, parts_l)
        o_full, l_full = api.attn_fwd(qd[row0:row0 + n], kd, vd, cu, [(g, n)], w.kv_lo, w.kv_hi, w.scale)
        torch.cuda.synchronize()
        o_np, l_np = bf16_to_np(o_m), l_m.cpu().numpy().astype(np.float64)
        # merged vs single full-range call (both GPU): double rounding of bf16 partials only
        assert_close(o_np, bf16_to_np(o_full), O_TOL, "merged vs full-range O")
        assert_close(l_np, l_full.cpu().numpy(), LSE_TOL, "merged vs full-range LSE")
        rows = np.unique(np.concatenate([np.arange(0, n, 97), [n - 1]]))
        wq = f64(q[row0 + rows])
        (want_o, want_l), secs = timed_s(lambda: oracle.attention_forward(
            wq, f64(k), f64(v), cu, [(g + int(r), 1) for r in rows], w.kv_lo, w.kv_hi, w.scale))
        eo = assert_close(o_np[rows], want_o, O_TOL, f"chunk {g} merged O")
        el = assert_close(l_np[:, rows], want_l, LSE_TOL, f"chunk {g} merged LSE")
        record(config=3, seed=w.seed, check=f"per-block forward + lse_merge, chunk at {g} ({len(blocks)} partials)",
               compared=f"{rows.size} of {n} rows, all heads", err_O=eo, err_LSE=el, oracle_s=round(secs, 2),
               cores=host_cores())
        row0 += n


def test_merge_against_oracle_small():
    rng = np.random.default_rng(4)
    for d in (64, 128):
        p, rows, hq = 5, 77, 3
        o = rng.standard_normal((p, rows, hq, d)).astype(np.float32)
        lse = (3 * rng.standard_normal((p, hq, rows))).astype(np.float32)
        lse[1, 0, :10] = -np.inf                          # some empty partials
        lse[:, 1, 20:25] = -np.inf                        # rows with every partial empty
        o_b = torch.from_numpy(o).to(torch.bfloat16)
        o_m, l_m = api.lse_merge(o_b.cuda(), torch.from_numpy(lse).cuda())
        torch.cuda.synchronize()
        want_o, want_l = oracle.lse_merge(o_b.float().numpy().astype(np.float64), lse.astype(np.float64))
        assert_close(bf16_to_np(o_m), want_o, O_TOL, "merge O")
        assert_close(l_m.cpu().numpy(), want_l, LSE_TOL, "merge LSE")


@pytest.mark.parametrize("d", [64, 128])
def test_f32_output_rounds_to_the_bf16_output(d):
    """The float32-output forward computes the same values: rounding them to
    bf16 (the oracle's rounding) gives the bf16 forward's bits exactly."""
    rng = np.random.default_rng(300 + d)
    lengths = random_lengths(rng, 900, 300, p_one=0.1)
    w = custom_workload(77 + d, lengths, 8, 2, d, chunks=[(0, 400), (500, 400)], kv_lo=50, kv_hi=880)
    print(f"[fwd32] d={d} lengths={lengths[:6]}", flush=True)
    q, k, v = to_dev(w.q()), to_dev(w.k()), to_dev(w.v())
    o16, l16 = api.attn_fwd(q, k, v, w.cu_seqlens, w.chunks, w.kv_lo, w.kv_hi, w.scale)
    o32, l32 = api.attn_fwd(q, k, v, w.cu_seqlens, w.chunks, w.kv_lo, w.kv_hi, w.scale, f32_out=True)
    torch.cuda.synchronize()
    assert o32.dtype == torch.float32
    assert np.array_equal(oracle.round_to_bf16_bits(o32.cpu().numpy()),
                          o16.view(torch.int16).cpu().numpy().view(np.uint16))
    assert torch.equal(l16, l32)
    want_o, want_l = oracle.attention_forward(f64(w.q()), f64(w.k()), f64(w.v()), w.cu_seqlens, w.chunks, w.kv_lo,
                                              w.kv_hi, w.scale)
    assert_close(o32.cpu().numpy(), want_o, O_TOL, "O32")


def test_merge_f32_against_oracle_small():
    rng = np.random.default_rng(5)
    for d in (64, 128):
        for p in (1, 5, 11):                              # 11 partials: the batched path
            rows, hq = 77, 3
            o = rng.standard_normal((p, rows, hq, d)).astype(np.float32)
            lse = (3 * rng.standard_normal((p, hq, rows))).astype(np.float32)
            lse[0, 0, :10] = -np.inf
            lse[:, 1, 20:25] = -np.inf
            print(f"[merge32] d={d} parts={p}", flush=True)
            o_m, l_m = api.lse_merge(torch.from_numpy(o).cuda(), torch.from_numpy(lse).cuda())
            torch.cuda.synchronize()
            want_o, want_l = oracle.lse_merge(o.astype(np.float64), lse.astype(np.float64))
            assert_close(bf16_to_np(o_m), want_o, O_TOL, "merge32 O")
            assert_close(l_m.cpu().numpy(), want_l, LSE_TOL, "merge32 LSE")


def test_cp_rank_f32_partials_and_merge():
    """Rank 3 of CP = 8 with float32 partials: merged result against the
    oracle on sampled rows, no worse than the bf16 partials' merge."""
    w = make_config(3)
    q, k, v = w.q(), w.k(), w.v()
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    cu = w.cu_seqlens
    need = api.schedule(cu, w.chunks, w.kv_lo, w.kv_hi, 8192, 8192)["need"].cpu().numpy()
    row0 = 0
    for ci, (g, n) in enumerate(w.chunks):
        blocks = list(range(need[ci, 0] // 8192, (need[ci, 1] + 8191) // 8192))
        print(f"[cp32] chunk {g} blocks {blocks}", flush=True)
        p32 = torch.empty((len(blocks), n, w.hq, w.d), dtype=torch.float32, device="cuda")
        p16 = torch.empty((len(blocks), n, w.hq, w.d), dtype=torch.bfloat16, device="cuda")
        pl = torch.empty((len(blocks), w.hq, n), dtype=torch.float32, device="cuda")
        for i, b in enumerate(blocks):
            sl = slice(8192 * b, 8192 * (b + 1))
            api.attn_fwd(qd[row0:row0 + n], kd[sl], vd[sl], cu, [(g, n)], 8192 * b, 8192 * (b + 1), w.scale,
                         out=p32[i], lse=pl[i], f32_out=True)
            api.attn_fwd(qd[row0:row0 + n], kd[sl], vd[sl], cu, [(g, n)], 8192 * b, 8192 * (b + 1), w.scale,
                         out=p16[i], lse=pl[i])
        o32, l32 = api.lse_merge(p32, pl)
        o16, l16 = api.lse_merge(p16, pl)
        torch.cuda.synchronize()
        rows = np.unique(np.concatenate([np.arange(0, n, 97), [n - 1]]))
        want_o, want_l = oracle.attention_forward(f64(q[row0 + rows]), f64(k), f64(v), cu,
                                                  [(g + int(r), 1) for r in rows], w.kv_lo, w.kv_hi, w.scale)
        e32 = assert_close(bf16_to_np(o32)[rows], want_o, O_TOL, f"chunk {g} f32-partials O")
        e16 = assert_close(bf16_to_np(o16)[rows], want_o, O_TOL, f"chunk {g} bf16-partials O")
        assert_close(l32.cpu().numpy()[:, rows], want_l, LSE_TOL, f"chunk {g} LSE")
        print(f"[cp32] max abs error: float32 partials {e32:.2e}, bf16 partials {e16:.2e}", flush=True)
        assert e32 <= e16
        row0 += n


def test_max_chunks():
    """DOCMASK_MAX_CHUNKS query chunks of 1-9 rows each over 40 documents."""
    rng = np.random.default_rng(256)
    lengths = [int(x) for x in rng.integers(20, 120, size=40)]
    total = sum(lengths)
    starts = np.sort(rng.choice(np.arange(0, total - 10, 11), size=api.MAX_CHUNKS, replace=False))
    chunks = [(int(g), int(rng.integers(1, 10))) for g in starts]
    w = custom_workload(256, lengths, 8, 2, 64, chunks=chunks)
    assert len(w.chunks) == api.MAX_CHUNKS
    _run_and_compare(w, tag="256 chunks")


def test_one_million_tokens_sampled_rows():
    """2^20 packed tokens (lognormal documents up to 65536): 64-bit offsets
    past 2^31 bytes in Q and O; sampled rows against the oracle."""
    from document_masked_attention_amd.workloads import lognormal_docs
    total = 1 << 20
    w = custom_workload(20, lognormal_docs(20, 4096, 1.2, 64, 65536, total), 16, 2, 128)
    print(f"[fwd] 2^20 tokens, {len(w.lengths)} documents: generating inputs", flush=True)
    assert w.tq * w.hq * w.d * 2 > 2 ** 31
    q, k, v = w.q(), w.k(), w.v()
    o, lse = api.attn_fwd(to_dev(q), to_dev(k), to_dev(v), w.cu_seqlens, w.chunks, 0, w.total, w.scale)
    torch.cuda.synchronize()
    rows = _sample_rows(w, 48, 20)
    print(f"[fwd] 2^20 tokens: oracle on {rows.size} rows", flush=True)
    want_o, want_l = oracle.attention_forward(f64(q[rows]), f64(k), f64(v), w.cu_seqlens,
                                              [(int(r), 1) for r in rows], 0, w.total, w.scale)
    assert_close(bf16_to_np(o[torch.as_tensor(rows, device="cuda")]), want_o, O_TOL, "2^20 O")
    assert_close(lse[:, torch.as_tensor(rows, device="cuda")].cpu().numpy(), want_l, LSE_TOL, "2^20 LSE")


def _trend_inputs(lengths, slopes, hq, hkv, d, seed):
    """Q rows all close to one direction v and K rows drifting along v with the
    key's position in its document (slope per key, in units of v), plus noise:
    a row's scores then grow (slope > 0) or shrink (slope < 0) steadily along
    its document.  bf16 bit patterns, like the seeded generator's."""
    from document_masked_attention_amd.workloads import f32_to_bf16_bits
    rng = np.random.default_rng(seed)
    total = sum(lengths)
    v = rng.standard_normal(d).astype(np.float32)
    v /= np.linalg.norm(v)
    q = 0.3 * rng.standard_normal((total, hq, d)).astype(np.float32) + 4.0 * v
    k = 0.5 * rng.standard_normal((total, hkv, d)).astype(np.float32)
    pos = 0
    for n, slope in zip(lengths, slopes):
        k[pos:pos + n] += (slope * np.arange(n, dtype=np.float32))[:, None, None] * v
        pos += n
    vv = rng.standard_normal((total, hkv, d)).astype(np.float32)
    return f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(vv)


@pytest.mark.parametrize("d", [64, 128])
def test_scores_rising_along_the_document(d):
    """The forward forms a tile's exponentials against the running reference and
    takes the tile maximum (raising the reference, rescaling O) only when some
    lane's sum exceeds 2^15 or a row has no reference yet.  Steeply rising
    scores force that on nearly every tile (first document), gently rising
    ones after many accepted tiles (second), falling ones never after the
    first tile (third, exponentials underflowing to zero); all against the
    oracle, every row."""
    lengths, slopes = [700, 1500, 900], [0.9, 0.02, -0.05]
    hq, hkv = 8, 2
    q, k, v = _trend_inputs(lengths, slopes, hq, hkv, d, 50 + d)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    total = int(cu[-1])
    scale = 1.0 / math.sqrt(d)
    print(f"[fwd] rising scores d={d} lengths={lengths} slopes={slopes}", flush=True)
    o, lse = api.attn_fwd(to_dev(q), to_dev(k), to_dev(v), cu, [(0, total)], 0, total, scale)
    torch.cuda.synchronize()
    want_o, want_l = oracle.attention_forward(f64(q), f64(k), f64(v), cu, [(0, total)], 0, total, scale)
    # the steep document's scores span hundreds of natural-log units along a row
    assert want_l[:, cu[1] - 1].min() > want_l[:, 0].max() + 100
    assert_close(bf16_to_np(o), want_o, O_TOL, "rising scores O")
    assert_close(lse.cpu().numpy(), want_l, LSE_TOL, "rising scores LSE")
