// LSE merge: combine partial (O, LSE) results computed over disjoint KV ranges
// (production guide, "Core Principle: Split Q, Circulate KV": partials are
// combined with the row maximum and the exponential sum).  Per row and head:
//   m = max_p LSE_p,  LSE = m + ln sum_p exp(LSE_p - m),
//   O = sum_p exp(LSE_p - LSE) O_p;   every partial empty -> (0, -inf).
// Bandwidth bound: every thread streams one slice of 8 values of one (row,
// head) from each partial whose LSE is finite (16 bytes of bf16, or 32 bytes
// when the partials are float32), and writes one 16-byte bf16 slice.
#include "kernels.h"

namespace docmask {

// Weighted sum of the slices of partials [q0, q0 + QB) with LSE values lq
// (-inf: empty partial, weight 0, not read); all slices are requested before
// any is used.  op points at the thread's slice of partial 0 in 16-byte units
// (two units per slice for float32 partials); o_stride = units between partials.
template <int QB, bool F32>
__device__ __forceinline__ void merge_group(const u32x4* op, size_t o_stride, int q0, const float (&lq)[QB],
                                            float lse2, float (&acc)[8]) {
  constexpr int U = F32 ? 2 : 1;
  float wgt[QB];
  u32x4 raw[QB][U];
#pragma unroll
  for (int i = 0; i < QB; ++i) {
    wgt[i] = lq[i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(__builtin_fmaf(lq[i], kLog2e, -lse2));
#pragma unroll
    for (int j = 0; j < U; ++j) {
      raw[i][j] = u32x4{0u, 0u, 0u, 0u};
      if (lq[i] != -INFINITY) raw[i][j] = __builtin_nontemporal_load(op + (size_t)(q0 + i) * o_stride + j);
    }
  }
#pragma unroll
  for (int i = 0; i < QB; ++i)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (F32) {
        acc[k] += wgt[i] * __uint_as_float(raw[i][0][k]);
        acc[4 + k] += wgt[i] * __uint_as_float(raw[i][U - 1][k]);
      } else {
        acc[2 * k] += wgt[i] * __uint_as_float(raw[i][0][k] << 16);
        acc[2 * k + 1] += wgt[i] * __uint_as_float(raw[i][0][k] & 0xffff0000u);
      }
    }
}

template <int D, bool F32>
__global__ __launch_bounds__(256) void merge_kernel(MergeParams p) {
  constexpr int CPR = D / 8;                        // threads per (row, head)
  constexpr int QB = 8;                             // partials per batch of loads
  const size_t n_rh = (size_t)p.rows * p.hq;
  const size_t gid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t rh = gid / CPR;
  const int c = (int)(gid % CPR);
  if (rh >= n_rh) return;
  const int row = (int)(rh / p.hq), head = (int)(rh % p.hq);
  const size_t lse_stride = n_rh;                   // elements between partials
  const float* lp = p.lse_parts + (size_t)head * p.rows + row;
  const int np = p.n_parts;
  const u32x4* op = F32 ? reinterpret_cast<const u32x4*>(p.o_parts32 + rh * D + 8 * c)
                        : reinterpret_cast<const u32x4*>(p.o_parts + rh * D + 8 * c);
  const size_t o_stride = n_rh * D / (F32 ? 4 : 8);  // 16-byte units between partials
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float out_lse = -INFINITY;
  if (np <= QB) {
    // all LSE values in registers: one round of LSE loads, one of slices
    float lq[QB];
#pragma unroll
    for (int i = 0; i < QB; ++i) lq[i] = i < np ? lp[i * lse_stride] : -INFINITY;
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < QB; ++i) m = fmaxf(m, lq[i]);
    if (m != -INFINITY) {
      const float m2 = m * kLog2e;
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < QB; ++i) s += __builtin_amdgcn_exp2f(__builtin_fmaf(lq[i], kLog2e, -m2));
      const float lse2 = m2 + __log2f(s);           // log2 of the merged sum
      out_lse = lse2 * kLn2;
      merge_group<QB, F32>(op, o_stride, 0, lq, lse2, acc);
    }
  } else {
    float m = -INFINITY;
#pragma unroll 4
    for (int q = 0; q < np; ++q) m = fmaxf(m, lp[q * lse_stride]);
    if (m != -INFINITY) {
      const float m2 = m * kLog2e;
      float s = 0.f;
#pragma unroll 4
      for (int q = 0; q < np; ++q) s += __builtin_amdgcn_exp2f(__builtin_fmaf(lp[q * lse_stride], kLog2e, -m2));
      const float lse2 = m2 + __log2f(s);
      out_lse = lse2 * kLn2;
      for (int q0 = 0; q0 < np; q0 += QB) {
        float lq[QB];
#pragma unroll
        for (int i = 0; i < QB; ++i) lq[i] = q0 + i < np ? lp[(q0 + i) * lse_stride] : -INFINITY;
        merge_group<QB, F32>(op, o_stride, q0, lq, lse2, acc);
      }
    }
  }
  u32x4 outv;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16x2 two = __builtin_convertvector(f32x2{acc[2 * i], acc[2 * i + 1]}, bf16x2);
    outv[i] = __builtin_bit_cast(uint32_t, two);
  }
  __builtin_nontemporal_store(outv, reinterpret_cast<u32x4*>(p.o_out + rh * D + 8 * c));
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
  const bool f32 = p.o_parts32 != nullptr;
  if (d == 128 && f32) hipLaunchKernelGGL((merge_kernel<128, true>), dim3((unsigned)blocks), dim3(256), 0, stream, p);
  else if (d == 128) hipLaunchKernelGGL((merge_kernel<128, false>), dim3((unsigned)blocks), dim3(256), 0, stream, p);
  else if (f32) hipLaunchKernelGGL((merge_kernel<64, true>), dim3((unsigned)blocks), dim3(256), 0, stream, p);
  else hipLaunchKernelGGL((merge_kernel<64, false>), dim3((unsigned)blocks), dim3(256), 0, stream, p);
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
