"""Pins for the oracle's backward pass (CPU only): hand-derived gradients,
central finite differences, torch autograd through masked attention, and
invariants that hold for the exact gradient."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from document_masked_attention_amd.workloads import random_lengths, cu_from_lengths
from test_oracle_forward import _load_tiny, _num


def test_golden_tiny_backward():
    g, q, k, v, do = _load_tiny()
    dq, dk, dv = oracle.attention_backward(q, k, v, do, g["cu_seqlens"], [(0, 4)], 0, 4, g["scale"])
    np.testing.assert_allclose(dv[:, 0, 0], g["full"]["dv"], atol=1e-12)
    np.testing.assert_allclose(dk[:, 0, 0], g["full"]["dk"], atol=1e-12)
    np.testing.assert_allclose(dq[:, 0, 0], [_num(x) for x in g["full"]["dq"]], atol=1e-12)


def _case(seed, total, max_len, hq, hkv, d):
    rng = np.random.default_rng(seed)
    lengths = random_lengths(rng, total, max_len)
    cu = cu_from_lengths(lengths)
    q, do = (rng.standard_normal((total, hq, d)) for _ in range(2))
    k, v = (rng.standard_normal((total, hkv, d)) for _ in range(2))
    return cu, q, k, v, do


def _loss(q, k, v, do, cu, chunks, lo, hi, scale):
    o, _ = oracle.attention_forward(q, k, v, cu, chunks, lo, hi, scale)
    return float((o * do).sum())


@pytest.mark.parametrize("seed", range(3))
def test_central_finite_differences(seed):
    total, hq, hkv, d = 12, 4, 2, 3
    cu, q, k, v, do = _case(seed, total, 5, hq, hkv, d)
    rng = np.random.default_rng(seed)
    lo = int(rng.integers(0, 3))
    chunks = [(0, 5), (7, 5)]
    rows = np.r_[0:5, 7:12]
    q, do = q[rows], do[rows]
    k, v = k[lo:], v[lo:]
    scale = 0.7
    dq, dk, dv = oracle.attention_backward(q, k, v, do, cu, chunks, lo, total, scale)
    eps = 1e-6
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + eps
            lp = _loss(q, k, v, do, cu, chunks, lo, total, scale)
            x[idx] = old - eps
            lm = _loss(q, k, v, do, cu, chunks, lo, total, scale)
            x[idx] = old
            num[idx] = (lp - lm) / (2 * eps)
        err = np.abs(num - grad).max() / max(1.0, np.abs(grad).max())
        assert err < 1e-6, (name, err)


@pytest.mark.parametrize("seed,total,hq,hkv,d", [(0, 200, 4, 4, 8), (1, 500, 8, 2, 16), (2, 900, 8, 1, 32)])
def test_torch_autograd_masked_sdpa(seed, total, hq, hkv, d):
    cu, q, k, v, do = _case(seed, total, 150, hq, hkv, d)
    scale = 1 / math.sqrt(d)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, cu, [(0, total)], 0, total, scale)
    g = hq // hkv
    docs = np.searchsorted(cu, np.arange(total), side="right") - 1
    mask = torch.from_numpy((docs[:, None] == docs[None, :]) & np.tri(total, dtype=bool))
    tq = torch.from_numpy(q).requires_grad_()
    tk = torch.from_numpy(k).requires_grad_()
    tv = torch.from_numpy(v).requires_grad_()
    out = torch.nn.functional.scaled_dot_product_attention(
        tq.permute(1, 0, 2)[None], tk.repeat_interleave(g, 1).permute(1, 0, 2)[None],
        tv.repeat_interleave(g, 1).permute(1, 0, 2)[None], attn_mask=mask, scale=scale)
    (out[0].permute(1, 0, 2) * torch.from_numpy(do)).sum().backward()
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-10)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-10)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-10)


@pytest.mark.parametrize("seed", range(3))
def test_gradient_invariants(seed):
    total, hq, hkv, d = 600, 8, 2, 16
    cu, q, k, v, do = _case(50 + seed, total, 200, hq, hkv, d)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, cu, [(0, total)], 0, total, 0.25)
    g = hq // hkv
    for a, b in zip(cu[:-1], cu[1:]):
        # sum_j dS_ij = 0 for every row, so dK summed over a document vanishes
        np.testing.assert_allclose(dk[a:b].sum(axis=0), 0, atol=1e-10)
        # softmax rows sum to one: dV summed over a document is the group's dO sum
        want = do[a:b].reshape(b - a, hkv, g, d).sum(axis=(0, 2))
        np.testing.assert_allclose(dv[a:b].sum(axis=0), want, atol=1e-10)
    # scores are unchanged by Q -> aQ, K -> K/a
    assert abs((q * dq).sum() - (k * dk).sum()) < 1e-9 * max(1.0, abs((q * dq).sum()))


def test_split_kv_dq_shares_sum_to_full():
    total, hq, hkv, d = 300, 4, 2, 8
    cu, q, k, v, do = _case(77, total, 90, hq, hkv, d)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, cu, [(0, total)], 0, total, 0.3)
    cuts = [0, 37, 128, 129, 300]
    acc = np.zeros_like(dq)
    for x, y in zip(cuts[:-1], cuts[1:]):
        part, _, _ = oracle.attention_backward(q, k, v, do, cu, [(0, total)], 0, total, 0.3,
                                                dq_key_range=(x, y))
        acc += part
    np.testing.assert_allclose(acc, dq, atol=1e-12)
