"""Pins for the oracle's forward pass and merge (CPU only).

Each test compares the oracle with something other than itself: a hand-derived
worked example, torch's own attention routine, textbook causal attention per
document, closed forms (first token, length-1 documents, uniform scores) and
the merge-partition invariant."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from document_masked_attention_amd.workloads import random_lengths, cu_from_lengths

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _num(x):
    table = {"0": 0.0, "ln2": math.log(2), "ln3": math.log(3), "ln5": math.log(5), "ln6": math.log(6),
             "-inf": -math.inf, "2/3 ln2": 2 / 3 * math.log(2), "ln3 - 1/3 ln2": math.log(3) - math.log(2) / 3}
    return table[x] if isinstance(x, str) else float(x)


def _load_tiny():
    with open(os.path.join(GOLD, "tiny_rational.json")) as f:
        g = json.load(f)
    arr = lambda key: np.array([_num(x) for x in g[key]]).reshape(-1, 1, 1)
    return g, arr("q"), arr("k"), arr("v"), arr("do")


def test_golden_tiny_forward():
    g, q, k, v, _ = _load_tiny()
    cu = g["cu_seqlens"]
    o, lse = oracle.attention_forward(q, k, v, cu, [(0, 4)], 0, 4, g["scale"])
    np.testing.assert_allclose(o[:, 0, 0], g["full"]["o"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[0], [_num(x) for x in g["full"]["lse"]], rtol=0, atol=1e-12)
    # key sub-ranges, including rows with no allowed key
    o2, l2 = oracle.attention_forward(q, k[2:], v[2:], cu, [(0, 4)], 2, 4, g["scale"])
    np.testing.assert_allclose(o2[:, 0, 0], g["keys_2_4"]["o"], atol=1e-12)
    assert np.array_equal(np.isinf(l2[0]), [True, True, False, False])
    np.testing.assert_allclose(l2[0, 2:], [_num(x) for x in g["keys_2_4"]["lse"][2:]], atol=1e-12)
    o1, l1 = oracle.attention_forward(q, k[:2], v[:2], cu, [(0, 4)], 0, 2, g["scale"])
    np.testing.assert_allclose(o1[:, 0, 0], g["keys_0_2"]["o"], atol=1e-12)
    # merging the two partials gives back the full-range values
    om, lm = oracle.lse_merge(np.stack([o1, o2]), np.stack([l1, l2]))
    np.testing.assert_allclose(om[:, 0, 0], g["full"]["o"], atol=1e-12)
    np.testing.assert_allclose(lm[0], [_num(x) for x in g["full"]["lse"]], atol=1e-12)
    # a chunk list holding only rows 2..3
    oc, lc = oracle.attention_forward(q[2:], k, v, cu, [(2, 2)], 0, 4, g["scale"])
    np.testing.assert_allclose(oc[:, 0, 0], g["full"]["o"][2:], atol=1e-12)
    assert oracle.useful_pairs(cu, [(0, 4)], 0, 4) == g["pairs"]


def _rand_case(seed, total, max_len, hq, hkv, d, p_one=0.15):
    rng = np.random.default_rng(seed)
    lengths = random_lengths(rng, total, max_len, p_one)
    q = rng.standard_normal((total, hq, d))
    k = rng.standard_normal((total, hkv, d))
    v = rng.standard_normal((total, hkv, d))
    return cu_from_lengths(lengths), lengths, q, k, v


def _torch_masked_sdpa(q, k, v, mask, scale):
    g = q.shape[1] // k.shape[1]
    tq = torch.from_numpy(q).permute(1, 0, 2)[None]
    tk = torch.from_numpy(k).repeat_interleave(g, dim=1).permute(1, 0, 2)[None]
    tv = torch.from_numpy(v).repeat_interleave(g, dim=1).permute(1, 0, 2)[None]
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.from_numpy(mask), scale=scale)
    return out[0].permute(1, 0, 2).numpy()


@pytest.mark.parametrize("seed,total,max_len,hq,hkv,d", [
    (0, 64, 16, 2, 2, 8), (1, 300, 80, 4, 1, 16), (2, 1000, 400, 8, 2, 32), (3, 2048, 900, 4, 4, 64)])
def test_library_sdpa_block_diagonal_causal(seed, total, max_len, hq, hkv, d):
    """torch's scaled_dot_product_attention with a block-diagonal causal mask."""
    cu, _, q, k, v = _rand_case(seed, total, max_len, hq, hkv, d)
    scale = 1 / math.sqrt(d)
    o, _ = oracle.attention_forward(q, k, v, cu, [(0, total)], 0, total, scale)
    docs = np.searchsorted(cu, np.arange(total), side="right") - 1
    mask = (docs[:, None] == docs[None, :]) & np.tri(total, dtype=bool)
    ref = _torch_masked_sdpa(q, k, v, mask, scale)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-10)


@pytest.mark.parametrize("seed", range(4))
def test_separate_per_document_causal(seed):
    """Packed doc-masked attention == textbook causal attention run per document."""
    cu, lengths, q, k, v = _rand_case(100 + seed, 700, 200, 4, 2, 16)
    scale = 0.3
    o, lse = oracle.attention_forward(q, k, v, cu, [(0, 700)], 0, 700, scale)
    for a, b in zip(cu[:-1], cu[1:]):
        tq = torch.from_numpy(q[a:b]).permute(1, 0, 2)[None]
        tk = torch.from_numpy(k[a:b]).repeat_interleave(2, dim=1).permute(1, 0, 2)[None]
        tv = torch.from_numpy(v[a:b]).repeat_interleave(2, dim=1).permute(1, 0, 2)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=scale)
        np.testing.assert_allclose(o[a:b], ref[0].permute(1, 0, 2).numpy(), rtol=0, atol=1e-10)
        # LSE of the last row of the document: log-sum-exp over the whole document
        s = scale * np.einsum("hd,jhd->hj", q[b - 1], np.repeat(k[a:b], 2, axis=1))
        np.testing.assert_allclose(lse[:, b - 1 - 0], np.log(np.exp(s).sum(axis=1)), rtol=0, atol=1e-10)


def test_first_token_and_length_one_documents():
    cu, lengths, q, k, v = _rand_case(7, 400, 60, 4, 2, 8, p_one=0.3)
    scale = 0.5
    o, lse = oracle.attention_forward(q, k, v, cu, [(0, 400)], 0, 400, scale)
    for a in cu[:-1]:
        for h in range(4):
            assert np.array_equal(o[a, h], v[a, h // 2])          # first token outputs its own V row
            assert abs(lse[h, a] - scale * float(np.dot(q[a, h], k[a, h // 2]))) < 1e-12
    # every document of length 1
    n = 50
    rng = np.random.default_rng(3)
    q1, k1, v1 = (rng.standard_normal((n, 2, 4)) for _ in range(3))
    o1, l1 = oracle.attention_forward(q1, k1, v1, np.arange(n + 1), [(0, n)], 0, n, 1.0)
    assert np.array_equal(o1, v1)


def test_uniform_scores_give_prefix_means():
    """q = 0 makes every allowed score 0: O_i is the mean of V over the allowed keys."""
    cu, lengths, _, k, v = _rand_case(11, 500, 120, 2, 1, 8)
    q = np.zeros((500, 2, 8))
    o, lse = oracle.attention_forward(q, k, v, cu, [(0, 500)], 0, 500, 1.0)
    for a, b in zip(cu[:-1], cu[1:]):
        cnt = np.arange(1, b - a + 1)
        mean = np.cumsum(v[a:b, 0], axis=0) / cnt[:, None]
        for h in range(2):
            np.testing.assert_allclose(o[a:b, h], mean, atol=1e-12)
            np.testing.assert_allclose(lse[h, a:b], np.log(cnt), atol=1e-12)


def test_document_permutation_equivariance():
    rng = np.random.default_rng(5)
    lengths = random_lengths(rng, 300, 70)
    cu = cu_from_lengths(lengths)
    q, k, v = (rng.standard_normal((300, 2, 8)) for _ in range(3))
    o, lse = oracle.attention_forward(q, k, v, cu, [(0, 300)], 0, 300, 0.4)
    perm = rng.permutation(len(lengths))
    idx = np.concatenate([np.arange(cu[i], cu[i + 1]) for i in perm])
    cu2 = cu_from_lengths([lengths[i] for i in perm])
    o2, l2 = oracle.attention_forward(q[idx], k[idx], v[idx], cu2, [(0, 300)], 0, 300, 0.4)
    np.testing.assert_allclose(o2, o[idx], atol=1e-12)
    np.testing.assert_allclose(l2, lse[:, idx], atol=1e-12)


@pytest.mark.parametrize("seed", range(6))
def test_merge_of_split_kv_equals_full(seed):
    rng = np.random.default_rng(200 + seed)
    total = int(rng.integers(50, 400))
    lengths = random_lengths(rng, total, 90)
    cu = cu_from_lengths(lengths)
    hq, hkv, d = 4, 2, 8
    q = rng.standard_normal((total, hq, d))
    k = rng.standard_normal((total, hkv, d))
    v = rng.standard_normal((total, hkv, d))
    # a chunk list of two ascending chunks and a KV range that may cut documents
    a = int(rng.integers(0, total // 2))
    b = int(rng.integers(a + 1, total))
    chunks = [(0, a), (b, total - b)] if a > 0 else [(b, total - b)]
    rows = np.concatenate([np.arange(g, g + n) for g, n in chunks])
    lo = int(rng.integers(0, total // 3))
    hi = int(rng.integers(lo + 1, total + 1))
    full_o, full_l = oracle.attention_forward(q[rows], k[lo:hi], v[lo:hi], cu, chunks, lo, hi, 0.35)
    cuts = sorted(set([lo, hi] + rng.integers(lo, hi, size=int(rng.integers(1, 5))).tolist()))
    parts = [oracle.attention_forward(q[rows], k[x:y], v[x:y], cu, chunks, x, y, 0.35)
             for x, y in zip(cuts[:-1], cuts[1:]) if y > x]
    om, lm = oracle.lse_merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    np.testing.assert_allclose(om, full_o, atol=1e-12)
    assert np.array_equal(np.isinf(lm), np.isinf(full_l))
    fin = np.isfinite(full_l)
    np.testing.assert_allclose(lm[fin], full_l[fin], atol=1e-12)
    assert np.all(om[~fin.T] == 0)


def test_merge_special_cases():
    rng = np.random.default_rng(9)
    o = rng.standard_normal((3, 5, 2, 4))
    lse = rng.standard_normal((3, 2, 5))
    om, lm = oracle.lse_merge(o[:1], lse[:1])                        # one partial: identity
    np.testing.assert_allclose(om, o[0], atol=1e-15)
    np.testing.assert_allclose(lm, lse[0], atol=1e-15)
    eq = np.repeat(lse[:1], 2, axis=0)                               # equal LSEs: average, LSE + ln 2
    om, lm = oracle.lse_merge(o[:2], eq)
    np.testing.assert_allclose(om, 0.5 * (o[0] + o[1]), atol=1e-15)
    np.testing.assert_allclose(lm, lse[0] + math.log(2), atol=1e-15)
    ninf = np.full((2, 2, 5), -np.inf)                               # all empty -> (0, -inf)
    om, lm = oracle.lse_merge(o[:2], ninf)
    assert np.all(om == 0) and np.all(np.isneginf(lm))
    mixed = lse[:2].copy()                                           # one empty partial: the other one
    mixed[1] = -np.inf
    om, lm = oracle.lse_merge(o[:2], mixed)
    np.testing.assert_allclose(om, o[0], atol=1e-15)
    np.testing.assert_allclose(lm, lse[0], atol=1e-15)
