"""Tile scheduler on the GPU vs the oracle's definition: bit-exact."""
import numpy as np
import pytest
import torch

import oracle
from document_masked_attention_amd import api
from document_masked_attention_amd.workloads import make_config, random_lengths, cu_from_lengths

pytestmark = pytest.mark.gpu


def _compare(cu, chunks, lo, hi, bq, bk, tag):
    want = oracle.schedule(cu, chunks, lo, hi, bq, bk)
    got = api.schedule(cu, chunks, lo, hi, bq, bk)
    torch.cuda.synchronize()
    assert api.check_errors(got["workspace"]) == api.OK, tag
    for key in ("qtile_desc", "kvtile_desc", "need", "lpt_q", "lpt_kv", "counters"):
        g = got[key].cpu().numpy()
        w = np.asarray(want[key])
        assert np.array_equal(g.reshape(w.shape), w), f"{tag}: {key} differs"


def test_random_small_problems():
    rng = np.random.default_rng(123)
    for case in range(150):
        total = int(rng.integers(1, 300))
        lengths = random_lengths(rng, total, int(rng.integers(1, 120)), p_one=0.2)
        cu = cu_from_lengths(lengths)
        k = int(rng.integers(1, 4))
        cuts = np.sort(rng.choice(np.arange(total + 1), size=min(total + 1, 2 * k), replace=False))
        chunks = [(int(a), int(b - a)) for a, b in zip(cuts[::2], cuts[1::2]) if b > a] or [(0, total)]
        lo = int(rng.integers(0, total))
        hi = int(rng.integers(lo + 1, total + 1))
        bq = int(rng.choice([1, 3, 16, 32, 64, 128]))
        bk = int(rng.choice([1, 5, 32, 64, 128]))
        _compare(cu, chunks, lo, hi, bq, bk, f"case {case}")


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("tiles", [(128, 64), (32, 64), (32, 128)])
def test_configs(cfg, tiles):
    w = make_config(cfg)
    _compare(w.cu_seqlens, w.chunks, w.kv_lo, w.kv_hi, tiles[0], tiles[1], f"config {cfg} tiles {tiles}")


def test_cp_rank_blocks():
    """Rank 3 of CP = 8: each chunk against each 8192-key block before it."""
    w = make_config(3)
    for g, n in w.chunks:
        for b in range(0, g // 8192 + 1):
            _compare(w.cu_seqlens, [(g, n)], 8192 * b, 8192 * (b + 1), 32, 64, f"chunk {g} block {b}")


def test_malformed_cu_seqlens_reported():
    cu = np.array([0, 10, 5, 40], dtype=np.int32)          # decreasing
    out = api.schedule(cu, [(0, 40)], 0, 40, 16, 16)
    assert api.check_errors(out["workspace"]) == api.EDEVICE_INPUT
    cu2 = np.array([0, 10, 20], dtype=np.int32)              # too short for the chunk
    out = api.schedule(cu2, [(0, 40)], 0, 40, 16, 16)
    assert api.check_errors(out["workspace"]) == api.EDEVICE_INPUT
