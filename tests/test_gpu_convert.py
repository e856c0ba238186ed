"""The optional gradient convert (float32 -> bf16) on the GPU vs the oracle's
round-to-nearest-even definition, bit for bit (NaN: any NaN)."""
import numpy as np
import pytest
import torch

import oracle
from document_masked_attention_amd import api

pytestmark = pytest.mark.gpu


def _special():
    pats = [0x3F800000, 0x3F808000, 0x3F818000, 0x3F808001, 0x3F807FFF, 0x3FFF8000, 0x7F7FFFFF, 0x7F800000,
            0xFF800000, 0x00000000, 0x80000000, 0x00000001, 0x00008000, 0x00018000, 0x807FFFFF, 0x7FC00000,
            0xFFC00123]
    return np.array(pats, dtype=np.uint32).view(np.float32)


@pytest.mark.parametrize("n", [1, 7, 8, 4096 + 5, 1 << 20])
def test_convert_bitexact(n):
    print(f"[convert] n={n}", flush=True)
    rng = np.random.default_rng(n)
    x = (rng.standard_normal(n) * np.exp2(rng.integers(-30, 30, size=n))).astype(np.float32)
    sp = _special()
    x[: min(n, sp.size)] = sp[: min(n, sp.size)]
    src = torch.from_numpy(x).to("cuda")
    out = api.f32_to_bf16(src)
    torch.cuda.synchronize()
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    want = oracle.round_to_bf16_bits(x)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.all(((got[nan] & 0x7F80) == 0x7F80) & ((got[nan] & 0x007F) != 0))


def test_convert_gradients_within_tolerance_of_oracle_values():
    """bf16 copies of float32 gradients: within max(2e-2, half a bf16 ulp of the value)."""
    rng = np.random.default_rng(3)
    g = (rng.standard_normal(1 << 16) * 6).astype(np.float32)
    out = api.f32_to_bf16(torch.from_numpy(g).to("cuda")).float().cpu().numpy()
    ulp_half = np.exp2(np.floor(np.log2(np.maximum(np.abs(g), 1e-30))) - 8)
    assert np.all(np.abs(out - g) <= np.maximum(2e-2, ulp_half))
