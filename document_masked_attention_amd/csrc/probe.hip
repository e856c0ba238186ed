// Matrix-core rate probe: a measurement aid for the roofline of the attention
// kernels, not a step of the attention computation.  Every wave runs
// back-to-back bf16 MFMAs -- v_mfma_f32_32x32x16_bf16 (the dK/dV kernel's) or
// v_mfma_f32_16x16x32_bf16 (the forward's and the dQ kernel's) -- on operands
// held in registers, with no memory traffic between its first loads and its
// one store, so its rate is what the matrix cores sustain on that data at the
// clock the chip holds under that load.
#include "docmask.h"
#include "common.h"

#include <type_traits>

namespace docmask {
namespace {

constexpr int kProbeSlots = 8;      // distinct A and B operand registers per lane

// Lane l of the grid (gl = global thread index) takes its operand registers
// from 8-value runs of `ops`: A slot j at (128 gl + 8 j) mod n, B slot j at
// (128 gl + 64 + 8 j) mod n.  MFMA k of an iteration multiplies A slot k mod 8
// by B slot 3k mod 8, so consecutive MFMAs never see the same operands: for
// SHAPE 32, 16 MFMAs of 32 x 32 x 16 into accumulator k mod 4; for SHAPE 16,
// 32 MFMAs of 16 x 16 x 32 into accumulator k mod 8 (the same 2^19 products
// per iteration).  The lane writes the sum of its accumulator elements.
template <int SHAPE>
__global__ __launch_bounds__(256, 2) void mfma_probe_kernel(const uint16_t* __restrict__ ops, int64_t n_ops,
                                                            int32_t iters, float* __restrict__ out) {
  constexpr int NM = SHAPE == 32 ? 16 : 32;         // MFMAs per iteration
  constexpr int NA = SHAPE == 32 ? 4 : 8;           // independent accumulators
  using Acc = typename std::conditional<SHAPE == 32, f32x16, f32x4>::type;
  const int64_t gl = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  // (128 gl + off) mod n for off < 128 <= n: one division, then at most one
  // subtraction
  const int64_t r0 = (gl * 128) % n_ops;
  auto at = [&](int off) { const int64_t i = r0 + off; return i >= n_ops ? i - n_ops : i; };
  bf16x8 a[kProbeSlots], b[kProbeSlots];
#pragma unroll
  for (int j = 0; j < kProbeSlots; ++j) {
    a[j] = *reinterpret_cast<const bf16x8*>(ops + at(8 * j));
    b[j] = *reinterpret_cast<const bf16x8*>(ops + at(64 + 8 * j));
  }
  Acc c[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i) c[i] = Acc{};
  for (int it = 0; it < iters; ++it) {
    static_for<NM>([&](auto kc) __attribute__((always_inline)) {
      constexpr int k = decltype(kc)::value;
      if constexpr (SHAPE == 32)
        c[k % NA] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[k % kProbeSlots], b[(3 * k) % kProbeSlots], c[k % NA],
                                                            0, 0, 0);
      else
        c[k % NA] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[k % kProbeSlots], b[(3 * k) % kProbeSlots], c[k % NA],
                                                            0, 0, 0);
    });
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NA; ++i)
#pragma unroll
    for (int e = 0; e < (SHAPE == 32 ? 16 : 4); ++e) s += c[i][e];
  out[gl] = s;
}

}  // namespace
}  // namespace docmask

using namespace docmask;

int docmask_mfma_probe(const void* operands, int64_t n_operands, int32_t n_workgroups, int32_t iters, int32_t shape,
                       float* out, hipStream_t stream) {
  if (!operands || !out || n_operands < 128 || n_operands % 8 != 0 || n_workgroups < 1 || iters < 0)
    return DOCMASK_EINVAL;
  if (shape != 32 && shape != 16) return DOCMASK_EINVAL;
  if ((reinterpret_cast<uintptr_t>(operands) & 15u) != 0 || (reinterpret_cast<uintptr_t>(out) & 3u) != 0)
    return DOCMASK_EINVAL;
  const uint16_t* ops = static_cast<const uint16_t*>(operands);
  if (shape == 32)
    hipLaunchKernelGGL(mfma_probe_kernel<32>, dim3((unsigned)n_workgroups), dim3(256), 0, stream, ops, n_operands, iters,
                       out);
  else
    hipLaunchKernelGGL(mfma_probe_kernel<16>, dim3((unsigned)n_workgroups), dim3(256), 0, stream, ops, n_operands, iters,
                       out);
  return hipGetLastError() == hipSuccess ? DOCMASK_OK : DOCMASK_EHIP;
}
