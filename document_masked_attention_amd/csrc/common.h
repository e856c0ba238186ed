// Internal definitions shared by the HIP kernels of libdocmask (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace docmask {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));   // 16-byte staging register

constexpr int kMaxChunks = 256;

// Compile-time loop: f(std::integral_constant<int, i>) for i = 0 .. N-1, so that
// register arrays indexed by i are resolved before any loop transformation.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}
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

// Work-item placement.  Logical items are (rank, kv_head, head_block) with
// rank the LPT position of a tile.  Items are grouped in clusters of `cr`
// consecutive ranks x all head blocks of ONE KV head: neighbouring tiles of a
// document read overlapping K/V (query-major kernels) or Q/dO rows (key-major
// kernel), so a cluster should run at the same time on the same XCD and share
// its L2.  The hardware deals workgroups to the 8 XCDs round-robin, so
// physical block b runs on XCD b % 8; clusters are dealt to XCDs in logical
// order (keeping the LPT order across the chip).  A bijection on [0, n).
struct WorkItem {
  int rank, kvh, hb;
};
__device__ __forceinline__ WorkItem map_work(int b, int n_ranks, int hkv, int n_hb, int cr) {
  const int csize = cr * n_hb;                      // items per cluster
  const int per_rank = hkv * n_hb;
  const int n = n_ranks * per_rank;
  // XCD deal: the k-th block an XCD receives belongs to cluster (k / csize) * 8 + xcd
  int w = b;
  const int full = (n / (8 * csize)) * (8 * csize);
  if (b < full) {
    const int xcd = b & 7, k = b >> 3;
    w = ((k / csize) * 8 + xcd) * csize + (k % csize);
  }
  WorkItem it;
  const int full_ranks = (n_ranks / cr) * cr;
  if (w < full_ranks * per_rank) {
    const int ci = w / csize, within = w - ci * csize;
    const int rank_block = ci / hkv;
    it.kvh = ci - rank_block * hkv;
    it.rank = rank_block * cr + within / n_hb;
    it.hb = within % n_hb;
  } else {
    const int w2 = w - full_ranks * per_rank;
    it.rank = full_ranks + w2 / per_rank;
    const int rem = w2 % per_rank;
    it.kvh = rem / n_hb;
    it.hb = rem % n_hb;
  }
  return it;
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

// Row-major bf16 tiles in LDS that are read both as 16-byte row chunks (MFMA
// operands along the row; lane l reads row l mod 16 at chunk l / 16 (+ 4 s))
// and through transpose reads (operands down the columns; the lanes of group
// g = l / 16 name rows 4 g + (l mod 16) / 4 at column groups l mod 4 of 16
// consecutive columns).  The LDS serves a 16-byte read in 16-lane cycles and a
// transpose read in 32-lane cycles whose lane sets are not consecutive lanes;
// the layouts below were measured bank-conflict free for both patterns
// (SQ_LDS_BANK_CONFLICT), where the swizzle f(r) = 4 (r mod 4) + (r / 4 mod 4)
// conflicts on the 16-byte reads and f(r) = r mod 16 on the transpose reads.
// For D = 128 rows are unpadded and the 16 chunks of row r are stored at
// chunk position c ^ f(r), f a function of r mod 16 (the layout repeats every
// 16 rows):
//   f(r) = 2 ((r' ^ (r' >> 3)) mod 8),  r' = r mod 16.
// For D = 64 rows are padded to 80 elements (160 bytes) instead.
template <int D>
struct SwzTile {
  static constexpr int kRowElems = D == 128 ? 128 : D + 16;
  static constexpr int kElems(int rows) { return rows * kRowElems; }
  __device__ static __forceinline__ int f(int r) { const int q = r & 15; return ((q ^ (q >> 3)) & 7) << 1; }
  // element offset of (row r, column col); col % 4 == 0 for transpose reads
  __device__ static __forceinline__ int off(int r, int col) {
    if (D == 128) return r * 128 + (((col >> 3) ^ f(r)) << 3) + (col & 7);
    return r * kRowElems + col;
  }
};

// The same two read patterns on unpadded rows for both head sizes, so that a
// tile is a dense run of 16-byte chunks that direct global-to-LDS loads can
// fill (64 lanes write 1 KB contiguously).  Chunk c of row r sits at c ^ f(r):
//   D = 128 (16 chunks, a row spans all 64 banks): f(r) = 4 (r mod 4) + (r / 4 mod 4)
//   D = 64 (8 chunks, two rows share the banks): f(r) = 4 (r / 2 mod 2) + (r / 4 mod 4)
// For D = 64 the 16 rows of a chunk read split into two parities of 8 rows
// with distinct f, and rows 4a + e, 4a + e + 2 of a transpose read use
// opposite halves of the row's banks.
template <int D>
struct DenseTile {
  static_assert(D == 64 || D == 128, "head size");
  static constexpr int kChunks = D / 8;
  static constexpr int kElems(int rows) { return rows * D; }
  __device__ static __forceinline__ int f(int r) {
    return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
  }
  __device__ static __forceinline__ int off(int r, int col) { return r * D + (((col >> 3) ^ f(r)) << 3) + (col & 7); }
  // logical chunk stored at chunk position pos of row r
  __device__ static __forceinline__ int chunk_at(int r, int pos) { return pos ^ f(r); }
};

// Direct 16-byte global-to-LDS loads (inline assembly): lane l's 16 bytes
// land at M0 + 16 l, the LDS destination being wave-uniform.  Completion is
// counted by vmcnt.  The compiler neither tracks the LDS write (the caller
// waits with wait_vmem() or a counted vmcnt and a barrier before any wave
// reads the buffer) nor inserts conservative waits before unrelated LDS
// reads; the one wait state an LDS DMA needs after a scalar write of M0 is
// the s_nop.

// From a wave-uniform base (SGPRs) plus a 32-bit lane byte offset: no
// per-lane 64-bit address arithmetic.
__device__ __forceinline__ void lds_dma16_s(const void* ubase, uint32_t voff, void* lds_base) {
  const uint32_t lds_addr =
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds_base;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(ubase),
               "s"(lds_addr)
               : "memory", "m0");
}

// The same with the LDS destination given as a wave-uniform LDS byte address
// plus a compile-time offset (one scalar add into M0): the caller keeps one
// base register instead of one per destination.
template <uint32_t OFF>
__device__ __forceinline__ void lds_dma16_so(const void* ubase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_add_u32 m0, %2, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(ubase),
               "s"(lds_addr), "n"(OFF)
               : "memory", "m0", "scc");
}

// Direct 4-byte global-to-LDS load: lane l's dword lands at lds_base + 4 l.
__device__ __forceinline__ void lds_dma4(const void* gptr, void* lds_base) {
  const uint32_t lds_addr =
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds_base;
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(gptr), "s"(lds_addr)
               : "memory", "m0");
}

// Load of a word the kernel never writes (scheduler tables), through the
// constant address space so that a wave-uniform index becomes a scalar load.
__device__ __forceinline__ int32_t ld_const(const int32_t* base, size_t idx) {
  return ((const __attribute__((address_space(4))) int32_t*)(base))[idx];
}

// Wait until this wave's global loads (including direct-to-LDS ones) are done.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0f70); }   // vmcnt(0)

// Two transpose reads assembled into one 8 x bf16 MFMA operand.
__device__ __forceinline__ bf16x8 tr_operand(const uint16_t* p0, const uint16_t* p1) {
  const v4i16 a = lds_read_tr16(p0);
  const v4i16 b = lds_read_tr16(p1);
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  const v8i16 c = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, c);
}

}  // namespace docmask
