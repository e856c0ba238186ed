// KV exchange of sharding-aware context parallelism, the part one GPU runs
// ("FlashCP", section 3.2 "Dynamic Sharding-aware Communication", Eq. 5).
//
// A worker sends only the KV of its document shards that are not the last
// shard of their document (a document kept whole on one worker counts as its
// own last shard): later shards of the same document, on other workers, need
// those rows as their prefix; nothing else is ever attended from elsewhere.
// The rows are compacted into one continuous buffer without per-document
// padding.  After the collective (not part of this library) a worker places
// the rows its chunks need, plus its own rows, at their global positions in
// the KV range [kv_lo, kv_hi) that the attention entry points take.
//
// Both directions are one primitive, a row copy driven by a map list:
// copy_rows_kernel streams 16-byte units; each workgroup takes a contiguous
// span of destination units, finds the first map that reaches it (binary
// search over the map table in LDS), and every thread walks the maps forward
// as its units advance.  A map with source -1 writes zero rows; gap rows
// (covered by no map) are zeroed or left alone.  Bandwidth bound: copied rows
// are read once, every written row is written once.
//
// The attention kernels read KV in whole tiles of at most kZeroBlock rows
// counted from kv_lo, and give keys outside a query's document weight zero,
// so the placement writes zeros over the rows of those tiles that no chunk
// needs (finite values for the masked keys) and leaves the rest of the range
// untouched.
#include "docmask.h"
#include "kernels.h"

#include <algorithm>
#include <cstring>
#include <vector>

namespace docmask {
namespace {

constexpr int kCopyMaps = 128;      // maps per launch (kernel-argument table)
constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 8;      // 16-byte units per thread per span

struct CopyTable {
  int32_t n;
  int32_t dst_lo[kCopyMaps];        // destination rows [dst_lo, dst_hi), relative to the launch's first row
  int32_t dst_hi[kCopyMaps];
  int32_t src[kCopyMaps];           // source row of dst_lo; -1: zero rows
};

struct CopyParams {
  const u32x4* src_k;
  const u32x4* src_v;               // null: one tensor (or no map)
  u32x4* dst_k;
  u32x4* dst_v;
  int64_t row_units;                // 16-byte units per row
  int64_t row0;                     // first destination row of this launch
  int64_t n_units;                  // units of this launch's destination rows
  int32_t zero_gaps;
};

__global__ __launch_bounds__(kCopyThreads) void copy_rows_kernel(CopyParams p, CopyTable t) {
  __shared__ int32_t s_lo[kCopyMaps], s_hi[kCopyMaps], s_src[kCopyMaps];
  const int n = t.n;
  for (int i = threadIdx.x; i < n; i += kCopyThreads) {
    s_lo[i] = t.dst_lo[i];
    s_hi[i] = t.dst_hi[i];
    s_src[i] = t.src[i];
  }
  __syncthreads();
  const int64_t ru = p.row_units;
  const int64_t span = (int64_t)kCopyThreads * kCopyUnroll;
  const int64_t dst0 = p.row0 * ru;
  const bool two = p.dst_v != nullptr;            // a source V exists whenever a map does
  for (int64_t c0 = (int64_t)blockIdx.x * span; c0 < p.n_units; c0 += (int64_t)gridDim.x * span) {
    const int64_t r_first = c0 / ru;
    int lo = 0, hi = n;                             // first map ending after the span's first row
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (s_hi[mid] > r_first) hi = mid;
      else lo = mid + 1;
    }
    int i = lo;
    u32x4 a[kCopyUnroll], b[kCopyUnroll];
    bool st[kCopyUnroll];
#pragma unroll
    for (int k = 0; k < kCopyUnroll; ++k) {
      const int64_t u = c0 + k * kCopyThreads + threadIdx.x;
      const bool valid = u < p.n_units;
      while (i < n && (int64_t)s_hi[i] * ru <= u) ++i;
      const bool covered = valid && i < n && (int64_t)s_lo[i] * ru <= u;
      a[k] = u32x4{0u, 0u, 0u, 0u};
      b[k] = u32x4{0u, 0u, 0u, 0u};
      if (covered && s_src[i] >= 0) {                 // src -1: a run of zero rows
        const int64_t s = (int64_t)s_src[i] * ru + (u - (int64_t)s_lo[i] * ru);
        a[k] = __builtin_nontemporal_load(p.src_k + s);
        if (two) b[k] = __builtin_nontemporal_load(p.src_v + s);
      }
      st[k] = valid && (covered || p.zero_gaps);
    }
#pragma unroll
    for (int k = 0; k < kCopyUnroll; ++k) {
      if (!st[k]) continue;
      const int64_t d = dst0 + c0 + k * kCopyThreads + threadIdx.x;
      __builtin_nontemporal_store(a[k], p.dst_k + d);
      if (two) __builtin_nontemporal_store(b[k], p.dst_v + d);
    }
  }
}

}  // namespace

// maps: sorted by dst, disjoint, len > 0, in bounds (checked by the caller).
hipError_t launch_copy_rows(const void* src_k, const void* src_v, void* dst_k, void* dst_v, int64_t dst_rows,
                            int64_t row_bytes, const docmask_rowmap* maps, int32_t n_maps, bool zero_gaps,
                            hipStream_t stream) {
  CopyParams p;
  p.src_k = static_cast<const u32x4*>(src_k);
  p.src_v = static_cast<const u32x4*>(src_v);
  p.dst_k = static_cast<u32x4*>(dst_k);
  p.dst_v = static_cast<u32x4*>(dst_v);
  p.row_units = row_bytes / 16;
  p.zero_gaps = zero_gaps ? 1 : 0;
  const int32_t n_batches = n_maps == 0 ? (zero_gaps ? 1 : 0) : (n_maps + kCopyMaps - 1) / kCopyMaps;
  for (int32_t bi = 0; bi < n_batches; ++bi) {
    const int32_t first = bi * kCopyMaps, last = std::min(n_maps, first + kCopyMaps);
    int64_t row0, row1;
    if (zero_gaps) {
      row0 = bi == 0 ? 0 : maps[first].dst;
      row1 = last == n_maps ? dst_rows : maps[last].dst;
    } else {
      row0 = maps[first].dst;
      row1 = (int64_t)maps[last - 1].dst + maps[last - 1].len;
    }
    if (row1 <= row0) continue;
    CopyTable t;
    std::memset(&t, 0, sizeof(t));
    t.n = last - first;
    for (int32_t i = first; i < last; ++i) {
      t.dst_lo[i - first] = (int32_t)(maps[i].dst - row0);
      t.dst_hi[i - first] = (int32_t)(maps[i].dst - row0 + maps[i].len);
      t.src[i - first] = maps[i].src;
    }
    p.row0 = row0;
    p.n_units = (row1 - row0) * p.row_units;
    const int64_t span = (int64_t)kCopyThreads * kCopyUnroll;
    const int64_t blocks = std::min<int64_t>((p.n_units + span - 1) / span, 1 << 20);
    KernelTimer timer(KC_COPY, stream);
    hipLaunchKernelGGL(copy_rows_kernel, dim3((unsigned)blocks), dim3(kCopyThreads), 0, stream, p, t);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace docmask

// ------------------------------------------------------------ host planning
namespace {

using docmask::launch_copy_rows;

constexpr int32_t kZeroBlock = 128;   // largest KV tile of the attention kernels (rows from kv_lo)

struct Piece {
  int32_t g;       // global start
  int32_t len;
  int32_t local;   // row in the owner's local layout (chunks concatenated)
};

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_cu(const int32_t* cu, int32_t n_docs) {
  if (!cu || n_docs < 1 || cu[0] != 0) return false;
  for (int32_t i = 0; i < n_docs; ++i)
    if (cu[i + 1] < cu[i]) return false;
  return true;
}

// chunks ascending, disjoint, non-negative, inside [0, total)
bool valid_chunks(const docmask_chunk* c, int32_t n, int32_t total) {
  if (n < 0 || (n > 0 && !c)) return false;
  int64_t prev_end = 0;
  for (int32_t i = 0; i < n; ++i) {
    if (c[i].len < 0 || c[i].g_start < prev_end || (int64_t)c[i].g_start + c[i].len > total) return false;
    prev_end = (int64_t)c[i].g_start + c[i].len;
  }
  return true;
}

int32_t doc_start_of(const int32_t* cu, int32_t n_docs, int32_t pos) {
  const int32_t* it = std::upper_bound(cu, cu + n_docs + 1, pos);
  return *(it - 1);
}

int32_t doc_end_of(const int32_t* cu, int32_t n_docs, int32_t pos) {
  return *std::upper_bound(cu, cu + n_docs + 1, pos);
}

// Rows of one worker that the exchange sends, coalesced where contiguous both
// in the local layout and in global positions; packed in this order.
std::vector<Piece> send_pieces(const int32_t* cu, int32_t n_docs, const docmask_chunk* chunks, int32_t n_chunks) {
  std::vector<Piece> out;
  int32_t local = 0;
  for (int32_t c = 0; c < n_chunks; ++c) {
    const int32_t g = chunks[c].g_start, end = g + chunks[c].len;
    for (int32_t p = g; p < end;) {
      const int32_t doc_end = doc_end_of(cu, n_docs, p);
      const int32_t q = std::min(end, doc_end);
      if (q < doc_end) {                               // not the document's last shard
        const Piece pc{p, q - p, local + (p - g)};
        if (!out.empty() && out.back().g + out.back().len == pc.g && out.back().local + out.back().len == pc.local)
          out.back().len += pc.len;
        else
          out.push_back(pc);
      }
      p = q;
    }
    local += chunks[c].len;
  }
  return out;
}

int64_t rows_of(const std::vector<Piece>& v) {
  int64_t s = 0;
  for (const Piece& p : v) s += p.len;
  return s;
}

}  // namespace

extern "C" {

int docmask_copy_rows(const void* src_k, const void* src_v, int64_t src_rows, void* dst_k, void* dst_v,
                      int64_t dst_rows, int64_t row_bytes, const docmask_rowmap* maps, int32_t n_maps,
                      int zero_gaps, hipStream_t stream) {
  if (row_bytes <= 0 || row_bytes % 16 || src_rows < 0 || dst_rows < 0 || n_maps < 0) return DOCMASK_EINVAL;
  if (src_rows > INT32_MAX || dst_rows > INT32_MAX) return DOCMASK_EINVAL;
  if (n_maps > 0 && !maps) return DOCMASK_EINVAL;
  std::vector<docmask_rowmap> m;
  m.reserve(n_maps);
  int64_t prev_end = 0;
  bool reads = false;
  for (int32_t i = 0; i < n_maps; ++i) {
    const docmask_rowmap r = maps[i];
    if (r.len < 0 || r.src < -1 || r.dst < prev_end) return DOCMASK_EINVAL;
    if ((r.src >= 0 && (int64_t)r.src + r.len > src_rows) || (int64_t)r.dst + r.len > dst_rows)
      return DOCMASK_EINVAL;
    prev_end = (int64_t)r.dst + r.len;
    if (r.len > 0) {
      m.push_back(r);
      reads = reads || r.src >= 0;
    }
  }
  const bool writes = dst_rows > 0 && (!m.empty() || zero_gaps);
  if (!writes) return DOCMASK_OK;                 // empty tensors may come with null pointers
  if ((src_v == nullptr) != (dst_v == nullptr) && !(!reads && src_v == nullptr)) return DOCMASK_EINVAL;
  if (!dst_k || !aligned16(dst_k) || (dst_v && !aligned16(dst_v))) return DOCMASK_EINVAL;
  if (reads && (!src_k || !aligned16(src_k) || (src_v && !aligned16(src_v)))) return DOCMASK_EINVAL;
  const hipError_t e = launch_copy_rows(src_k, src_v, dst_k, dst_v, dst_rows, row_bytes, m.data(),
                                        (int32_t)m.size(), zero_gaps != 0, stream);
  return e == hipSuccess ? DOCMASK_OK : DOCMASK_EHIP;
}

int docmask_exchange_send_maps(const int32_t* cu_seqlens, int32_t n_docs, const docmask_chunk* chunks,
                               int32_t n_chunks, docmask_rowmap* maps, int32_t max_maps, int32_t* n_maps,
                               int64_t* send_rows) {
  if (!n_maps || !send_rows || !valid_cu(cu_seqlens, n_docs)) return DOCMASK_EINVAL;
  if (!valid_chunks(chunks, n_chunks, cu_seqlens[n_docs])) return DOCMASK_EINVAL;
  const std::vector<Piece> pcs = send_pieces(cu_seqlens, n_docs, chunks, n_chunks);
  *n_maps = (int32_t)pcs.size();
  *send_rows = rows_of(pcs);
  if (!maps) return DOCMASK_OK;
  if (max_maps < (int32_t)pcs.size()) return DOCMASK_EINVAL;
  int32_t packed = 0;
  for (size_t i = 0; i < pcs.size(); ++i) {
    maps[i] = docmask_rowmap{pcs[i].local, packed, pcs[i].len};
    packed += pcs[i].len;
  }
  return DOCMASK_OK;
}

int docmask_exchange_recv_maps(const int32_t* cu_seqlens, int32_t n_docs, const docmask_chunk* all_chunks,
                               const int32_t* rank_n_chunks, int32_t n_ranks, int32_t rank, int64_t slot_rows,
                               int32_t* kv_lo, int32_t* kv_hi, docmask_rowmap* remote, int32_t max_remote,
                               int32_t* n_remote, docmask_rowmap* local, int32_t max_local, int32_t* n_local) {
  if (!kv_lo || !kv_hi || !n_remote || !n_local || !rank_n_chunks || !valid_cu(cu_seqlens, n_docs))
    return DOCMASK_EINVAL;
  if (n_ranks < 1 || rank < 0 || rank >= n_ranks || slot_rows < 0) return DOCMASK_EINVAL;
  const int32_t total = cu_seqlens[n_docs];
  // every rank's list valid; together they cover [0, total) exactly once
  std::vector<int32_t> off(n_ranks + 1, 0);
  for (int32_t k = 0; k < n_ranks; ++k) {
    if (rank_n_chunks[k] < 0) return DOCMASK_EINVAL;
    off[k + 1] = off[k] + rank_n_chunks[k];
  }
  if (off[n_ranks] > 0 && !all_chunks) return DOCMASK_EINVAL;
  std::vector<std::pair<int32_t, int32_t>> cover;
  for (int32_t k = 0; k < n_ranks; ++k) {
    if (!valid_chunks(all_chunks + off[k], rank_n_chunks[k], total)) return DOCMASK_EINVAL;
    for (int32_t c = off[k]; c < off[k + 1]; ++c)
      if (all_chunks[c].len > 0) cover.emplace_back(all_chunks[c].g_start, all_chunks[c].len);
  }
  std::sort(cover.begin(), cover.end());
  int64_t pos = 0;
  for (const auto& c : cover) {
    if (c.first != pos) return DOCMASK_EINVAL;
    pos += c.second;
  }
  if (pos != total) return DOCMASK_EINVAL;

  // the rank's need intervals: [document start of a chunk's first row, chunk end), merged
  const docmask_chunk* mine = all_chunks + off[rank];
  const int32_t n_mine = rank_n_chunks[rank];
  std::vector<std::pair<int32_t, int32_t>> need;
  for (int32_t c = 0; c < n_mine; ++c) {
    if (mine[c].len == 0) continue;
    const int32_t lo = doc_start_of(cu_seqlens, n_docs, mine[c].g_start), hi = mine[c].g_start + mine[c].len;
    if (!need.empty() && lo <= need.back().second) need.back().second = std::max(need.back().second, hi);
    else need.emplace_back(lo, hi);
  }
  *kv_lo = need.empty() ? 0 : need.front().first;
  *kv_hi = need.empty() ? 0 : need.back().second;

  std::vector<docmask_rowmap> rem;
  for (int32_t k = 0; k < n_ranks; ++k) {
    if (k == rank) continue;
    const std::vector<Piece> pcs = send_pieces(cu_seqlens, n_docs, all_chunks + off[k], rank_n_chunks[k]);
    if (rows_of(pcs) > slot_rows) return DOCMASK_EINVAL;
    int64_t packed = 0;
    size_t ni = 0;
    for (const Piece& pc : pcs) {
      const int32_t a = pc.g, b = pc.g + pc.len;
      while (ni < need.size() && need[ni].second <= a) ++ni;
      for (size_t j = ni; j < need.size() && need[j].first < b; ++j) {
        const int32_t x = std::max(a, need[j].first), y = std::min(b, need[j].second);
        if (y > x) {
          const int64_t src = (int64_t)k * slot_rows + packed + (x - a);
          if (src + (y - x) > INT32_MAX) return DOCMASK_EINVAL;
          rem.push_back(docmask_rowmap{(int32_t)src, x - *kv_lo, y - x});
        }
      }
      packed += pc.len;
    }
  }
  // zero runs: rows of the kZeroBlock-row blocks (from kv_lo) that meet a need
  // interval and that neither another worker's rows nor this worker's own fill
  {
    std::vector<std::pair<int64_t, int64_t>> held;             // destination rows written by copies
    for (const docmask_rowmap& r : rem) held.emplace_back(r.dst, (int64_t)r.dst + r.len);
    for (int32_t c = 0; c < n_mine; ++c)
      if (mine[c].len > 0) held.emplace_back(mine[c].g_start - *kv_lo, (int64_t)mine[c].g_start - *kv_lo + mine[c].len);
    std::sort(held.begin(), held.end());
    const int64_t span = (int64_t)*kv_hi - *kv_lo;
    std::vector<std::pair<int64_t, int64_t>> blocks;
    for (const auto& nd : need) {
      const int64_t a = (nd.first - *kv_lo) / kZeroBlock * kZeroBlock;
      const int64_t b = std::min<int64_t>(((int64_t)nd.second - *kv_lo + kZeroBlock - 1) / kZeroBlock * kZeroBlock, span);
      if (!blocks.empty() && a <= blocks.back().second) blocks.back().second = std::max(blocks.back().second, b);
      else blocks.emplace_back(a, b);
    }
    size_t hi_i = 0;
    for (const auto& bl : blocks) {
      int64_t pos = bl.first;
      while (hi_i < held.size() && held[hi_i].second <= pos) ++hi_i;
      for (size_t t = hi_i; pos < bl.second; ++t) {
        const int64_t next = t < held.size() ? std::min(held[t].first, bl.second) : bl.second;
        if (next > pos) rem.push_back(docmask_rowmap{-1, (int32_t)pos, (int32_t)(next - pos)});
        if (t >= held.size()) break;
        pos = std::max(pos, held[t].second);
      }
    }
  }
  std::sort(rem.begin(), rem.end(), [](const docmask_rowmap& x, const docmask_rowmap& y) { return x.dst < y.dst; });
  *n_remote = (int32_t)rem.size();
  *n_local = 0;
  for (int32_t c = 0; c < n_mine; ++c) *n_local += mine[c].len > 0;
  if (remote) {
    if (max_remote < (int32_t)rem.size()) return DOCMASK_EINVAL;
    std::copy(rem.begin(), rem.end(), remote);
  }
  if (local) {
    if (max_local < *n_local) return DOCMASK_EINVAL;
    int32_t row = 0, j = 0;
    for (int32_t c = 0; c < n_mine; ++c) {
      if (mine[c].len > 0) local[j++] = docmask_rowmap{row, mine[c].g_start - *kv_lo, mine[c].len};
      row += mine[c].len;
    }
  }
  return DOCMASK_OK;
}

}  // extern "C"
