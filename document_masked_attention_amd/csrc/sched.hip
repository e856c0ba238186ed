// Tile scheduler kernels (integer only).
//
// Block skipping as the production guide ("Causal Attention Creates Rank Load
// Imbalance") asks for it, and the per-chunk KV need list, the single-GPU
// counterpart of the FlashCP paper's sharding-aware KV selection (section 3.2).
//
// Closed forms used here (documents are contiguous ranges of positions, so a
// row i may attend exactly the keys j with ds(i) <= j <= i, ds = start of i's
// document, FlashCP section 2.1):
//  * Q tile rows [r0, r1): the non-skipped keys are the single interval
//    [max(kv_lo, ds(r0)), min(kv_hi, r1)).
//  * KV tile keys [c0, c1) is FULL for rows [r0, r1) iff c1 - 1 <= r0 and c0
//    lies in the document of r1 - 1; the FULL tiles of a Q tile are therefore
//    one contiguous sub-range.
//  * KV tile [c0, c1) is attended by the rows [c0, end of doc(c1 - 1)).
//  * Chunk [g0, g1) needs keys [max(kv_lo, ds(g0)), min(kv_hi, g1)).
#include "kernels.h"

namespace docmask {

// cu_seqlens must start at 0, never decrease and reach every position used.
__global__ __launch_bounds__(1024) void validate_kernel(SchedParams p) {
  int bad = 0;
  if (threadIdx.x == 0) bad = (p.cu[0] != 0) || (p.cu[p.n_docs] < p.needed_end);
  for (int d = threadIdx.x; d < p.n_docs; d += blockDim.x) bad |= p.cu[d] > p.cu[d + 1];
  bad = __syncthreads_or(bad);
  if (threadIdx.x == 0) {
    p.err[0] = bad;
    if (p.counters)
      for (int i = 0; i < 4; ++i) p.counters[i] = 0ull;
  }
}

__device__ __forceinline__ void locate_tile(const ChunkTable& ch, int bq, int t, int& c, int& lrow0,
                                            int& grow0, int& nrows) {
  int acc_t = 0, acc_r = 0;
  for (c = 0; c < ch.n; ++c) {
    int nt = ceil_div(ch.len[c], bq);
    if (t < acc_t + nt) break;
    acc_t += nt;
    acc_r += ch.len[c];
  }
  int u = t - acc_t;
  lrow0 = acc_r + u * bq;
  grow0 = ch.g_start[c] + u * bq;
  nrows = min(bq, ch.len[c] - u * bq);
}

__global__ __launch_bounds__(256) void qtile_kernel(SchedParams p) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= p.n_qtiles) return;
  int c, lrow0, r0, nrows;
  locate_tile(p.ch, p.bq, t, c, lrow0, r0, nrows);
  const int r1 = r0 + nrows;
  const int ds0 = doc_start(p.cu, p.n_docs, r0);
  const int lo = max(p.kv_lo, ds0), hi = min(p.kv_hi, r1);
  int kt_lo = 0, kt_flo = 0, kt_fhi = 0, kt_hi = 0;
  if (lo < hi) {
    kt_lo = (lo - p.kv_lo) / p.bk;
    kt_hi = ceil_div(hi - p.kv_lo, p.bk);
    const int dsl = doc_start(p.cu, p.n_docs, r1 - 1);
    const int j_a = ceil_div(max(dsl - p.kv_lo, 0), p.bk);          // first tile with c0 >= ds(r1-1)
    const int j_b = (p.kv_hi <= r0 + 1) ? p.n_kvtiles                 // tiles with c1 - 1 <= r0
                                        : max(0, r0 + 1 - p.kv_lo) / p.bk;
    kt_flo = max(j_a, kt_lo);
    kt_fhi = min(j_b, kt_hi);
    if (kt_flo >= kt_fhi) kt_flo = kt_fhi = kt_hi;
    // keep every index inside [0, n_kvtiles] even for malformed cu_seqlens
    kt_lo = min(max(kt_lo, 0), p.n_kvtiles);
    kt_hi = min(max(kt_hi, kt_lo), p.n_kvtiles);
    kt_flo = min(max(kt_flo, kt_lo), kt_hi);
    kt_fhi = min(max(kt_fhi, kt_flo), kt_hi);
  }
  if (p.plan_q) {
    int* o = p.plan_q + (size_t)t * QP_WORDS;
    o[QP_LROW0] = lrow0; o[QP_GROW0] = r0; o[QP_NROWS] = nrows; o[QP_DS0] = ds0;
    o[QP_KT_LO] = kt_lo; o[QP_KT_FLO] = kt_flo; o[QP_KT_FHI] = kt_fhi; o[QP_KT_HI] = kt_hi;
  }
  if (p.qdesc) {
    int* o = p.qdesc + (size_t)t * 4;
    o[0] = kt_lo; o[1] = kt_flo; o[2] = kt_fhi; o[3] = kt_hi;
  }
  if (p.key_q) p.key_q[t] = kt_hi - kt_lo;
  if (p.counters) {
    long long pairs = 0;
    // rows of the tile, walking the documents they fall in
    int dlo = 0, dhi = p.n_docs;
    while (dhi - dlo > 1) {
      int mid = (dlo + dhi) >> 1;
      if (p.cu[mid] <= r0) dlo = mid; else dhi = mid;
    }
    int d = dlo;
    for (int i = r0; i < r1; ++i) {
      while (d + 1 < p.n_docs && p.cu[d + 1] <= i) ++d;
      const int a = max(p.cu[d], p.kv_lo), b = min(i, p.kv_hi - 1);
      if (b >= a) pairs += (long long)(b - a + 1);
    }
    const int nonskip = kt_hi - kt_lo, full = kt_fhi - kt_flo;
    if (nonskip) atomicAdd(&p.counters[0], (unsigned long long)nonskip);
    if (full) atomicAdd(&p.counters[1], (unsigned long long)full);
    if (nonskip - full) atomicAdd(&p.counters[2], (unsigned long long)(nonskip - full));
    if (pairs) atomicAdd(&p.counters[3], (unsigned long long)pairs);
  }
}

__global__ __launch_bounds__(256) void kvtile_kernel(SchedParams p) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= p.n_kvtiles) return;
  const int c0 = p.kv_lo + j * p.bk;
  const int c1 = min(c0 + p.bk, p.kv_hi);
  const int e_att = doc_end(p.cu, p.n_docs, c1 - 1);    // rows [c0, e_att) attend this tile
  const int e_full = doc_end(p.cu, p.n_docs, c0);       // FULL rows end inside doc(c0)
  int qt_lo = 0x7fffffff, qt_hi = -1, fq_lo = 0x7fffffff, fq_hi = -1;
  int tb = 0;
  for (int c = 0; c < p.ch.n; ++c) {
    const int g = p.ch.g_start[c], n = p.ch.len[c], nt = ceil_div(n, p.bq);
    const int a = max(g, c0), b = min(g + n, e_att);
    if (a < b) {
      qt_lo = min(qt_lo, tb + (a - g) / p.bq);
      qt_hi = max(qt_hi, tb + ceil_div(b - g, p.bq));
      const int fu_lo = ceil_div(max(c1 - 1 - g, 0), p.bq);
      const int fu_hi = (g + n <= e_full) ? nt : (e_full - g > 0 ? (e_full - g) / p.bq : 0);
      if (fu_lo < fu_hi) {
        fq_lo = min(fq_lo, tb + fu_lo);
        fq_hi = max(fq_hi, tb + fu_hi);
      }
    }
    tb += nt;
  }
  int d0 = 0, d1 = 0, d2 = 0, d3 = 0;
  if (qt_lo < qt_hi) {
    d0 = qt_lo; d3 = min(qt_hi, p.n_qtiles);
    d0 = min(d0, d3);
    if (fq_lo < fq_hi) { d1 = min(max(fq_lo, d0), d3); d2 = min(max(fq_hi, d1), d3); }
    else { d1 = d2 = d3; }
    if (d1 >= d2) d1 = d2 = d3;
  }
  if (p.kvdesc) {
    int* o = p.kvdesc + (size_t)j * 4;
    o[0] = d0; o[1] = d1; o[2] = d2; o[3] = d3;
  }
  if (p.key_kv) p.key_kv[j] = d3 - d0;
}

// Pairing of KV tiles into dK/dV work items.  Tiles with work that attend the
// same last query tile (the tiles of one document) form a run [r0, r1) whose
// work falls linearly along it (tile j is attended from its own position to
// the document end); tile r0 + i is paired with tile r1 - 1 - i, so every
// pair of a document holds about the same work, and the pairs of one document
// that run together read the same query rows at the same time (the dK/dV
// kernel walks the first tile from the document end down and the second one
// from its diagonal up).  A tile without work, and the middle tile of an odd
// run, is a work item alone.  Keys: 1 + ceil(work / 2) for a pair leader (the
// lower tile), 0 for the other tile of a pair (it runs inside its leader's
// work item).  One thread per run start walks the run.
__global__ __launch_bounds__(256) void kvpair_kernel(SchedParams p) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= p.n_kvtiles) return;
  const int4* __restrict__ desc = reinterpret_cast<const int4*>(p.kvdesc);
  int32_t* __restrict__ pair = p.kv_pair;
  int32_t* __restrict__ key = p.key_pair;
  const int4 dj = desc[j];
  const int wj = dj.w - dj.x;
  if (wj <= 0) {
    pair[j] = j;
    key[j] = 1;
    return;
  }
  if (j > 0) {
    const int4 dp = desc[j - 1];
    if (dp.w - dp.x > 0 && dp.w == dj.w) return;                    // not a run start
  }
  int e = j + 1;
  for (; e < p.n_kvtiles; ++e) {
    const int4 d = desc[e];
    if (d.w - d.x <= 0 || d.w != dj.w) break;
  }
  for (int a = j, b = e - 1; a <= b; ++a, --b) {
    const int4 da = desc[a], db = desc[b];
    pair[a] = b;
    pair[b] = a;
    const int w = a == b ? da.w - da.x : (da.w - da.x) + (db.w - db.x);
    key[a] = 1 + (w + 1) / 2;
    if (a != b) key[b] = 0;
  }
}

__global__ __launch_bounds__(256) void need_kernel(SchedParams p) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= p.ch.n) return;
  const int g0 = p.ch.g_start[c], g1 = g0 + p.ch.len[c];
  int lo = 0, hi = 0;
  if (g1 > g0) {
    lo = max(p.kv_lo, doc_start(p.cu, p.n_docs, g0));
    hi = min(p.kv_hi, g1);
    if (lo >= hi) lo = hi = 0;
  }
  p.need[2 * c] = lo;
  p.need[2 * c + 1] = hi;
}

// Stable counting sort of n tiles by descending key (keys in [0, max_key]):
// the LPT (longest processing time first) launch order, ties by index.
// One workgroup; `hist` holds max_key + 1 ints of workspace.  Every access to
// `hist` is an agent-scope atomic so that no wave reads a stale L1 copy.
__device__ __forceinline__ int ld_ag(int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_ag(int32_t* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ __launch_bounds__(1024) void lpt_kernel(const int32_t* __restrict__ keys, int32_t n,
                                                   int32_t max_key, int32_t* hist,
                                                   int32_t* __restrict__ order) {
  __shared__ int32_t scan[1024];
  __shared__ int32_t carry;
  const int tid = threadIdx.x;
  const int nk = max_key + 1;
  for (int k = tid; k < nk; k += 1024) st_ag(&hist[k], 0);
  __threadfence();
  __syncthreads();
  for (int i = tid; i < n; i += 1024) {
    int key = min(max(keys[i], 0), max_key);
    atomicAdd(&hist[key], 1);
  }
  __threadfence();
  __syncthreads();
  // exclusive scan over keys in descending order: start[k] = #tiles with key > k
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < nk; base += 1024) {
    const int idx = base + tid;                 // position in descending order
    const int key = max_key - idx;
    const int h = idx < nk ? ld_ag(&hist[key]) : 0;
    scan[tid] = h;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {  // Hillis-Steele inclusive scan
      int x = tid >= off ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += x;
      __syncthreads();
    }
    const int incl = scan[tid];
    const int c = carry;
    __syncthreads();
    if (idx < nk) st_ag(&hist[key], c + incl - h);
    if (tid == 1023) carry = c + incl;
    __syncthreads();
  }
  __threadfence();
  __syncthreads();
  // stable placement by one wave, 64 tiles at a time in index order
  if (tid < 64) {
    int bits = 0;
    while (bits < 31 && (1 << bits) <= max_key) ++bits;
    const unsigned long long lt = (1ull << tid) - 1ull;
    for (int base = 0; base < n; base += 64) {
      const int i = base + tid;
      const bool valid = i < n;
      const int key = valid ? min(max(keys[i], 0), max_key) : 0;
      unsigned long long m = __ballot(valid);
      for (int b = 0; b < bits; ++b) {
        const int bit = (key >> b) & 1;
        const unsigned long long ones = __ballot(valid && bit);
        m &= bit ? ones : ~ones;
      }
      const int rank = __popcll(m & lt);
      const int leader = valid ? __ffsll((long long)m) - 1 : 0;
      int pos0 = 0;
      if (valid && tid == leader) pos0 = atomicAdd(&hist[key], __popcll(m));
      pos0 = __shfl(pos0, leader, 64);
      if (valid && pos0 + rank < n) order[pos0 + rank] = i;
    }
  }
}

// The same ordering with the histogram in LDS (dynamic shared memory of
// max_key + 1 ints), for key ranges up to kLptLdsKeys: LDS atomics instead of
// contended global ones.
constexpr int kLptLdsKeys = 8192;
__global__ __launch_bounds__(1024) void lpt_lds_kernel(const int32_t* __restrict__ keys, int32_t n,
                                                       int32_t max_key, int32_t* __restrict__ order) {
  extern __shared__ int32_t lhist[];
  __shared__ int32_t scan[1024];
  __shared__ int32_t carry;
  const int tid = threadIdx.x;
  const int nk = max_key + 1;
  for (int k = tid; k < nk; k += 1024) lhist[k] = 0;
  __syncthreads();
  for (int i = tid; i < n; i += 1024) atomicAdd(&lhist[min(max(keys[i], 0), max_key)], 1);
  if (tid == 0) carry = 0;
  __syncthreads();
  // exclusive scan over keys in descending order: start[k] = #tiles with key > k
  for (int base = 0; base < nk; base += 1024) {
    const int idx = base + tid;
    const int key = max_key - idx;
    const int h = idx < nk ? lhist[key] : 0;
    scan[tid] = h;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int x = tid >= off ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += x;
      __syncthreads();
    }
    const int incl = scan[tid];
    const int c = carry;
    __syncthreads();
    if (idx < nk) lhist[key] = c + incl - h;
    if (tid == 1023) carry = c + incl;
    __syncthreads();
  }
  // stable placement: each wave takes 64 consecutive tiles in turn (chunk
  // order across waves is kept by a ticket so that ties stay in index order)
  if (tid < 64) {
    int bits = 0;
    while (bits < 31 && (1 << bits) <= max_key) ++bits;
    const unsigned long long lt = (1ull << tid) - 1ull;
    for (int base = 0; base < n; base += 64) {
      const int i = base + tid;
      const bool valid = i < n;
      const int key = valid ? min(max(keys[i], 0), max_key) : 0;
      unsigned long long m = __ballot(valid);
      for (int b = 0; b < bits; ++b) {
        const int bit = (key >> b) & 1;
        const unsigned long long ones = __ballot(valid && bit);
        m &= bit ? ones : ~ones;
      }
      const int rank = __popcll(m & lt);
      const int leader = valid ? __ffsll((long long)m) - 1 : 0;
      int pos0 = 0;
      if (valid && tid == leader) pos0 = atomicAdd(&lhist[key], __popcll(m));
      pos0 = __shfl(pos0, leader, 64);
      if (valid && pos0 + rank < n) order[pos0 + rank] = i;
    }
  }
}

// ---------------------------------------------------------------- host side
hipError_t launch_schedule(const SchedParams& p, int32_t* lpt_q, int32_t* lpt_kv, int32_t* hist,
                           hipStream_t stream) {
  KernelTimer timer(KC_SCHEDULE, stream);
  hipLaunchKernelGGL(validate_kernel, dim3(1), dim3(1024), 0, stream, p);
  if (p.n_qtiles > 0 && (p.plan_q || p.qdesc || p.key_q || p.counters))
    hipLaunchKernelGGL(qtile_kernel, dim3(ceil_div(p.n_qtiles, 256)), dim3(256), 0, stream, p);
  if (p.n_kvtiles > 0 && (p.kvdesc || p.key_kv))
    hipLaunchKernelGGL(kvtile_kernel, dim3(ceil_div(p.n_kvtiles, 256)), dim3(256), 0, stream, p);
  if (p.kv_pair && p.kvdesc && p.n_kvtiles > 0)
    hipLaunchKernelGGL(kvpair_kernel, dim3(ceil_div(p.n_kvtiles, 256)), dim3(256), 0, stream, p);
  if (p.need && p.ch.n > 0)
    hipLaunchKernelGGL(need_kernel, dim3(ceil_div(p.ch.n, 256)), dim3(256), 0, stream, p);
  // keys of Q tiles are KV-tile counts (<= n_kvtiles) and vice versa
  auto lpt = [&](const int32_t* keys, int32_t n, int32_t max_key, int32_t* order) {
    if (max_key + 1 <= kLptLdsKeys)
      hipLaunchKernelGGL(lpt_lds_kernel, dim3(1), dim3(1024), (size_t)(max_key + 1) * sizeof(int32_t), stream, keys,
                         n, max_key, order);
    else
      hipLaunchKernelGGL(lpt_kernel, dim3(1), dim3(1024), 0, stream, keys, n, max_key, hist, order);
  };
  if (lpt_q && p.n_qtiles > 0) lpt((const int32_t*)p.key_q, p.n_qtiles, p.n_kvtiles, lpt_q);
  // KV tiles (pair keys are <= 1 + n_qtiles when the tiles are paired)
  if (lpt_kv && p.n_kvtiles > 0) {
    if (p.kv_pair) lpt((const int32_t*)p.key_pair, p.n_kvtiles, p.n_qtiles + 1, lpt_kv);
    else lpt((const int32_t*)p.key_kv, p.n_kvtiles, p.n_qtiles, lpt_kv);
  }
  return hipGetLastError();
}

}  // namespace docmask
