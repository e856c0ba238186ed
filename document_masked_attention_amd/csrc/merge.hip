// LSE merge: combine partial (O, LSE) results computed over disjoint KV ranges
// (production guide, "Core Principle: Split Q, Circulate KV": partials are
// combined with the row maximum and the exponential sum).  Per row and head:
//   m = max_p LSE_p,  LSE = m + ln sum_p exp(LSE_p - m),
//   O = sum_p exp(LSE_p - LSE) O_p;   every partial empty -> (0, -inf).
// Bandwidth bound: every thread streams one 16-byte slice (8 bf16) of one
// (row, head) from each partial whose LSE is finite, and writes one slice.
#include "kernels.h"

namespace docmask {

template <int D>
__global__ __launch_bounds__(256) void merge_kernel(MergeParams p) {
  constexpr int CPR = D / 8;                        // threads per (row, head)
  const size_t n_rh = (size_t)p.rows * p.hq;
  const size_t gid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t rh = gid / CPR;
  const int c = (int)(gid % CPR);
  if (rh >= n_rh) return;
  const int row = (int)(rh / p.hq), head = (int)(rh % p.hq);
  const size_t lse_stride = n_rh;                   // elements between partials
  const float* lp = p.lse_parts + (size_t)head * p.rows + row;
  float m = -INFINITY;
  for (int q = 0; q < p.n_parts; ++q) m = fmaxf(m, lp[q * lse_stride]);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float out_lse = -INFINITY;
  if (m != -INFINITY) {
    const float m2 = m * kLog2e;
    float s = 0.f;
    for (int q = 0; q < p.n_parts; ++q) s += __builtin_amdgcn_exp2f(__builtin_fmaf(lp[q * lse_stride], kLog2e, -m2));
    const float lse2 = m2 + __log2f(s);             // log2 of the merged sum
    out_lse = lse2 * kLn2;
    const uint16_t* op = p.o_parts + rh * D + 8 * c;
    const size_t o_stride = n_rh * D;
    for (int q = 0; q < p.n_parts; ++q) {
      const float lq = lp[q * lse_stride];
      if (lq == -INFINITY) continue;                // empty partial: weight 0, not read
      const float wgt = __builtin_amdgcn_exp2f(__builtin_fmaf(lq, kLog2e, -lse2));
      const uint4 raw = *reinterpret_cast<const uint4*>(op + q * o_stride);
      const uint32_t wds[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] += wgt * __uint_as_float(wds[i] << 16);
        acc[2 * i + 1] += wgt * __uint_as_float(wds[i] & 0xffff0000u);
      }
    }
  }
  uint4 outv;
  uint32_t* ow = reinterpret_cast<uint32_t*>(&outv);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16x2 two = __builtin_convertvector(f32x2{acc[2 * i], acc[2 * i + 1]}, bf16x2);
    ow[i] = *reinterpret_cast<const uint32_t*>(&two);
  }
  *reinterpret_cast<uint4*>(p.o_out + rh * D + 8 * c) = outv;
  if (c == 0) p.lse_out[(size_t)head * p.rows + row] = out_lse;
}

__global__ __launch_bounds__(256) void f32_to_bf16_kernel(const float* __restrict__ src, uint16_t* __restrict__ dst,
                                                          int64_t n) {
  const int64_t i0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (i0 + 8 <= n) {
    const float4 a = *reinterpret_cast<const float4*>(src + i0);
    const float4 b = *reinterpret_cast<const float4*>(src + i0 + 4);
    const bf16x2 p0 = __builtin_convertvector(f32x2{a.x, a.y}, bf16x2);
    const bf16x2 p1 = __builtin_convertvector(f32x2{a.z, a.w}, bf16x2);
    const bf16x2 p2 = __builtin_convertvector(f32x2{b.x, b.y}, bf16x2);
    const bf16x2 p3 = __builtin_convertvector(f32x2{b.z, b.w}, bf16x2);
    uint4 o;
    o.x = *reinterpret_cast<const uint32_t*>(&p0);
    o.y = *reinterpret_cast<const uint32_t*>(&p1);
    o.z = *reinterpret_cast<const uint32_t*>(&p2);
    o.w = *reinterpret_cast<const uint32_t*>(&p3);
    *reinterpret_cast<uint4*>(dst + i0) = o;
  } else {
    for (int64_t i = i0; i < n; ++i) {
      const __bf16 h = (__bf16)src[i];
      dst[i] = *reinterpret_cast<const uint16_t*>(&h);
    }
  }
}

hipError_t launch_merge(const MergeParams& p, int d, hipStream_t stream) {
  const long long threads = (long long)p.rows * p.hq * (d / 8);
  if (threads == 0) return hipSuccess;
  const long long blocks = (threads + 255) / 256;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  KernelTimer timer(KC_MERGE, stream);
  if (d == 128) hipLaunchKernelGGL(merge_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  else hipLaunchKernelGGL(merge_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_f32_to_bf16(const float* src, uint16_t* dst, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const long long blocks = ((n + 7) / 8 + 255) / 256;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  KernelTimer timer(KC_CONVERT, stream);
  hipLaunchKernelGGL(f32_to_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, src, dst, n);
  return hipGetLastError();
}

}  // namespace docmask
