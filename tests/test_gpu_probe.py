"""docmask_mfma_probe, the matrix-core rate probe of the power study: its
lanes really run the documented MFMAs per iteration on the documented
operand slots, for both shapes.  All-ones operands give 4096 per iteration in
every lane exactly (shape 32: 4 accumulators of 16 elements, each gaining 4 x
16 per iteration; shape 16: 8 accumulators of 4 elements, each gaining 4 x 32);
on random bf16 operands the sum of a wave's outputs, which covers each
accumulator's tile once whatever the output layout, equals the sum of the
products A_k B_k per iteration built from the lanes' operand registers in the
documented operand layout (float64 on the host)."""
import numpy as np
import pytest
import torch

from document_masked_attention_amd import api
from document_masked_attention_amd.workloads import bf16_bits_to_f64, f32_to_bf16_bits

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("shape", [32, 16])
def test_probe_all_ones_is_exact(shape):
    ops = torch.ones(1024, dtype=torch.bfloat16, device="cuda")
    for n_wg, iters in ((1, 0), (4, 1), (3, 37)):
        print(f"[probe] shape {shape} ones n_wg={n_wg} iters={iters}", flush=True)
        out = api.mfma_probe(ops, n_wg, iters, shape=shape)
        torch.cuda.synchronize()
        assert out.numel() == 256 * n_wg
        assert torch.all(out == 4096.0 * iters), (n_wg, iters, out.unique())


@pytest.mark.parametrize("shape", [32, 16])
def test_probe_random_operands_wave_sums(shape):
    rng = np.random.default_rng(9)
    n_ops, n_wg, iters = 4096 + 512, 2, 3          # the lanes' runs wrap around the buffer
    bits = f32_to_bf16_bits(rng.standard_normal(n_ops, dtype=np.float32))
    vals = bf16_bits_to_f64(bits)
    ops = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    print(f"[probe] shape {shape} random n_ops={n_ops} n_wg={n_wg} iters={iters}", flush=True)
    out = api.mfma_probe(ops, n_wg, iters, shape=shape).cpu().numpy().astype(np.float64)

    def run(gl, off):
        i = (128 * gl + off) % n_ops
        return vals[i:i + 8]

    m, kd, n_mfma = (32, 16, 16) if shape == 32 else (16, 32, 32)   # A is m x kd, B is kd x m
    for wave in range(4 * n_wg):
        gls = 64 * wave + np.arange(64)
        want, scale = 0.0, 0.0
        for k in range(n_mfma):
            a = np.zeros((m, kd))
            b = np.zeros((kd, m))
            for l in range(64):
                h, r = divmod(l, m)
                a[r, 8 * h:8 * h + 8] = run(gls[l], 8 * (k % 8))
                b[8 * h:8 * h + 8, r] = run(gls[l], 64 + 8 * ((3 * k) % 8))
            c = a @ b
            want += c.sum()
            scale += np.abs(c).sum()
        got = out[gls].sum()
        assert abs(got - iters * want) <= 1e-5 * iters * scale + 1e-6, (wave, got, iters * want)
