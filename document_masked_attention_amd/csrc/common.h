// Internal definitions shared by the HIP kernels of libdocmask (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace docmask {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kMaxChunks = 256;
constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.442695040888963407f;

// Chunk list passed by value to the scheduler kernels (host array copied into
// the kernel arguments, so no host memory is referenced after the launch).
struct ChunkTable {
  int32_t n;
  int32_t g_start[kMaxChunks];
  int32_t len[kMaxChunks];
};

// Per-Q-tile plan written by the scheduler and read by the attention kernels.
enum QPlan { QP_LROW0 = 0, QP_GROW0, QP_NROWS, QP_DS0, QP_KT_LO, QP_KT_FLO, QP_KT_FHI, QP_KT_HI, QP_WORDS };

// Workspace header (first 256 bytes of every workspace).
struct WsHeader {
  int32_t device_error;  // nonzero: cu_seqlens malformed; attention kernels exit early
  int32_t pad[63];
};

// Start position of the document holding global position p:
// cu[d] with cu[d] <= p < cu[d+1].  Positions at or beyond cu[n_docs] map to
// the last document (never read memory outside cu[0..n_docs]).
__device__ __forceinline__ int32_t doc_start(const int32_t* __restrict__ cu, int32_t n_docs, int32_t p) {
  int lo = 0, hi = n_docs;  // invariant: cu[lo] <= p (assumed), answer in [lo, hi)
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (cu[mid] <= p) lo = mid; else hi = mid;
  }
  return cu[lo];
}

// End position of the document holding p: cu[d+1].
__device__ __forceinline__ int32_t doc_end(const int32_t* __restrict__ cu, int32_t n_docs, int32_t p) {
  int lo = 0, hi = n_docs;
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (cu[mid] <= p) lo = mid; else hi = mid;
  }
  return cu[lo + 1];
}

__host__ __device__ __forceinline__ int32_t ceil_div(int32_t a, int32_t b) { return (a + b - 1) / b; }

// Block index remap so that consecutive logical work items of a cluster land on
// the same XCD (the hardware hands workgroups to the 8 XCDs round-robin) while
// clusters themselves are dealt round-robin over the XCDs in logical order.
// A bijection on [0, n).
__device__ __forceinline__ int xcd_remap(int b, int n, int cluster) {
  const int per = 8 * cluster;
  const int full = (n / per) * per;
  if (b >= full) return b;
  const int xcd = b & 7;
  const int k = b >> 3;                 // k-th workgroup this XCD receives
  return ((k / cluster) * 8 + xcd) * cluster + (k % cluster);
}

__device__ __forceinline__ float wave_shfl_xor32(float x) {
  return __shfl_xor(x, 32, 64);
}

// max / sum of x over the lane pair (l, l ^ 32) with v_permlane32_swap: the
// swap leaves {x_l, x_(l^32)} in the two results of every lane.
__device__ __forceinline__ float pair_max32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// LDS transpose read (gfx950 ds_read_b64_tr_b16).  Within each group of 16
// lanes, output lane i gets element e (0..3) = the 16-bit value at
// (address supplied by lane 4e + i/4 of the group) + (i mod 4) elements.  So a
// lane that supplies the address of row R, column C of a row-major tile feeds
// row R's columns C..C+3 to four lanes; MFMA operands whose contraction index
// runs down the rows of a tile are read straight from the row-major tile.
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
__device__ __forceinline__ v4i16 lds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p));
}

// Two transpose reads assembled into one 8 x bf16 MFMA operand.
__device__ __forceinline__ bf16x8 tr_operand(const uint16_t* p0, const uint16_t* p1) {
  const v4i16 a = lds_read_tr16(p0);
  const v4i16 b = lds_read_tr16(p1);
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  const v8i16 c = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, c);
}

}  // namespace docmask
