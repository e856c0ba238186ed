"""The library's sharding planner (host code) against the Algorithm 1 oracle
on the CPU: identical chunk lists, Per-Doc documents and ratio (integer work,
compared exactly), and argument checks."""
import numpy as np
import pytest

import oracle
from document_masked_attention_amd import api
from document_masked_attention_amd.workloads import lognormal_docs, bimodal_docs


def _cases():
    rng = np.random.default_rng(21)
    out = [([5, 3, 2, 2], 2, 1.5), ([5, 3, 2, 2], 2, 1.2), ([4096, 4096], 2, 1.01), ([100] * 20 + [30000], 4, 1.05),
           ([], 3, 1.1), ([0, 0], 2, 1.0), ([7], 4, 1.0), ([1] * 9, 4, 1.0)]
    for case in range(120):
        n = int(rng.choice([1, 2, 3, 4, 5, 8, 16]))
        lengths = [int(x) for x in rng.integers(0, 900, size=int(rng.integers(1, 40)))]
        if rng.random() < 0.3:
            lengths.append(int(rng.integers(2000, 20000)))
        out.append((lengths, n, float(rng.choice([1.0, 1.01, 1.05, 1.2, 2.0]))))
    for seed in range(4):
        out.append((bimodal_docs(seed + 1), 8, 1.05))
        out.append((lognormal_docs(seed + 1, 2048, 1.5, 64, 131072, 131072), 8, 1.05))
        out.append((lognormal_docs(seed + 1, 1024, 1.2, 64, 65536, 65536), 4, 1.02))
    return out


@pytest.mark.parametrize("case", range(140))
def test_planner_matches_oracle(case):
    lengths, n, r = _cases()[case]
    got = api.plan_shards(lengths, n, r)
    want = oracle.plan_chunks(lengths, n, r)
    assert got[0] == want[0]
    assert got[1] == want[1]
    assert got[2] == want[2]


def test_planner_arguments():
    for args in (([5, -1], 2, 1.1), ([5], 0, 1.1), ([5], 2, 0.9), ([5], 2, float("nan")), ([2 ** 30, 2 ** 30], 2, 1.1)):
        with pytest.raises(api.DocmaskError):
            api.plan_shards(*args)
