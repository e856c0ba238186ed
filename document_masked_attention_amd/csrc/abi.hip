// Host side of the C ABI declared in include/docmask.h: argument validation
// (before anything is enqueued), workspace layout and kernel launches.
#include "docmask.h"
#include "kernels.h"

#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>

using namespace docmask;

// Scratch of docmask_attn_fwd_noalloc: the forward's workspace (error word,
// tile plans, LPT keys and order, histogram) as one static device array, so
// that entry point never allocates.  Each GPU the library runs on holds its
// own copy until the process ends.  Host code never passes this name to a
// kernel (on the host it is only a stand-in for the symbol): it uses the
// device address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[DOCMASK_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

struct Problem {
  int64_t tq = 0;          // local query rows
  int32_t tkv = 0;
  int32_t needed_end = 0;  // largest position + 1 touched
  int32_t group = 1;
};

// Shape checks shared by every attention entry point (no pointers).
int check_shape(int32_t n_docs, const docmask_chunk* chunks, int32_t n_chunks, int32_t kv_lo, int32_t kv_hi,
                int32_t hq, int32_t hkv, int32_t d, Problem* pr) {
  if (n_docs < 1) return DOCMASK_EINVAL;
  if (n_chunks < 0 || n_chunks > DOCMASK_MAX_CHUNKS) return DOCMASK_EINVAL;
  if (n_chunks > 0 && !chunks) return DOCMASK_EINVAL;
  if (kv_lo < 0 || kv_hi < kv_lo) return DOCMASK_EINVAL;
  if (hq < 1 || hkv < 1 || hq % hkv != 0) return DOCMASK_EINVAL;
  if (d != 64 && d != 128) return DOCMASK_EUNSUPPORTED;
  int64_t tq = 0, end = kv_hi, prev_end = 0;
  for (int i = 0; i < n_chunks; ++i) {
    const int64_t g = chunks[i].g_start, n = chunks[i].len;
    if (g < 0 || n < 0 || g + n > INT32_MAX) return DOCMASK_EINVAL;
    if (i > 0 && g < prev_end) return DOCMASK_EINVAL;   // ascending and disjoint
    prev_end = g + n;
    tq += n;
    if (n > 0 && g + n > end) end = g + n;
  }
  if (tq > INT32_MAX) return DOCMASK_EINVAL;
  if (tq * hq > INT32_MAX) return DOCMASK_EINVAL;      // LSE index range
  pr->tq = tq;
  pr->tkv = kv_hi - kv_lo;
  pr->needed_end = (int32_t)end;
  pr->group = hq / hkv;
  return DOCMASK_OK;
}

int64_t count_qtiles(const docmask_chunk* chunks, int32_t n_chunks, int32_t bq) {
  int64_t n = 0;
  for (int i = 0; i < n_chunks; ++i) n += (chunks[i].len + (int64_t)bq - 1) / bq;
  return n;
}

ChunkTable make_table(const docmask_chunk* chunks, int32_t n_chunks) {
  ChunkTable t;
  std::memset(&t, 0, sizeof(t));
  t.n = n_chunks;
  for (int i = 0; i < n_chunks; ++i) {
    t.g_start[i] = chunks[i].g_start;
    t.len[i] = chunks[i].len;
  }
  return t;
}

// Workspace layout of one entry point (byte offsets; 0 = region absent).
struct Layout {
  size_t plan_q = 0, key_q = 0, lpt_q = 0, kvdesc = 0, key_kv = 0, lpt_kv = 0, kv_pair = 0, key_pair = 0, plan_q2 = 0,
         hist = 0, delta = 0, total = 0;
  int64_t n_qt = 0, n_kt = 0, n_qt2 = 0, n_kt2 = 0;
};

Layout fwd_layout(const docmask_chunk* chunks, int32_t n_chunks, const Problem& pr) {
  Layout L;
  const int bq = fwd_rows_per_tile(pr.group);
  L.n_qt = count_qtiles(chunks, n_chunks, bq);
  L.n_kt = (pr.tkv + (int64_t)kFwdBK - 1) / kFwdBK;
  size_t off = kAlign;                                   // header
  L.plan_q = off; off = align_up(off + (size_t)L.n_qt * QP_WORDS * 4);
  L.key_q = off;  off = align_up(off + (size_t)L.n_qt * 4);
  L.lpt_q = off;  off = align_up(off + (size_t)L.n_qt * 4);
  L.hist = off;   off = align_up(off + (size_t)(L.n_kt + 1) * 4);
  L.total = off;
  return L;
}

Layout bwd_layout(const docmask_chunk* chunks, int32_t n_chunks, const Problem& pr, int32_t hq) {
  // dK/dV pass: 32-row query blocks x 128-key tiles; dQ pass: forward-style tiles
  Layout L;
  L.n_qt = count_qtiles(chunks, n_chunks, kBwdBQ);
  L.n_kt = (pr.tkv + (int64_t)kBwdBK - 1) / kBwdBK;
  L.n_qt2 = count_qtiles(chunks, n_chunks, dq_rows_per_tile(pr.group));
  L.n_kt2 = (pr.tkv + (int64_t)kDqBK - 1) / kDqBK;
  // Delta first, right after the header: its offset depends on nothing but
  // the header, so a later call with DOCMASK_DELTA_READY over a KV block of a
  // different length finds it where the earlier call stored it
  size_t off = kAlign;
  L.delta = off;  off = align_up(off + (size_t)hq * pr.tq * 4);
  L.plan_q = off; off = align_up(off + (size_t)L.n_qt * QP_WORDS * 4);
  L.kvdesc = off; off = align_up(off + (size_t)L.n_kt * 4 * 4);
  L.key_kv = off; off = align_up(off + (size_t)L.n_kt * 4);
  L.lpt_kv = off; off = align_up(off + (size_t)L.n_kt * 4);
  L.kv_pair = off; off = align_up(off + (size_t)L.n_kt * 4);
  L.key_pair = off; off = align_up(off + (size_t)L.n_kt * 4);
  L.plan_q2 = off; off = align_up(off + (size_t)L.n_qt2 * QP_WORDS * 4);
  L.key_q = off;  off = align_up(off + (size_t)L.n_qt2 * 4);
  L.lpt_q = off;  off = align_up(off + (size_t)L.n_qt2 * 4);
  const int64_t hist_n = (L.n_qt > L.n_kt2 ? L.n_qt : L.n_kt2) + 2;
  L.hist = off;   off = align_up(off + (size_t)hist_n * 4);
  L.total = off;
  return L;
}

Layout sched_layout(int64_t n_qt, int64_t n_kt) {
  Layout L;
  L.n_qt = n_qt;
  L.n_kt = n_kt;
  size_t off = kAlign;
  L.key_q = off;  off = align_up(off + (size_t)n_qt * 4);
  L.key_kv = off; off = align_up(off + (size_t)n_kt * 4);
  L.hist = off;   off = align_up(off + (size_t)((n_qt > n_kt ? n_qt : n_kt) + 1) * 4);
  L.total = off;
  return L;
}

template <typename T>
T* at(void* ws, size_t off) { return reinterpret_cast<T*>(static_cast<char*>(ws) + off); }

int hip_status(hipError_t e) { return e == hipSuccess ? DOCMASK_OK : DOCMASK_EHIP; }

// Ranks (LPT-adjacent tiles) per XCD cluster.  With one rank per cluster the
// 8-way round-robin deal of workgroups puts KV head h's work items on XCD
// h mod 8 (for 8 KV heads, each XCD's L2 serves one head); larger clusters
// measured no faster on the 131072-token workload.
constexpr int kXcdCluster = 1;

}  // namespace

extern "C" {

size_t docmask_workspace_size(int op, int32_t n_docs, const docmask_chunk* chunks, int32_t n_chunks,
                              int32_t kv_lo, int32_t kv_hi, int32_t hq, int32_t hkv, int32_t d) {
  Problem pr;
  if (check_shape(n_docs, chunks, n_chunks, kv_lo, kv_hi, hq, hkv, d, &pr) != DOCMASK_OK) return 0;
  if (op == DOCMASK_OP_FWD) return fwd_layout(chunks, n_chunks, pr).total;
  if (op == DOCMASK_OP_BWD) return bwd_layout(chunks, n_chunks, pr, hq).total;
  return 0;
}

size_t docmask_schedule_workspace_size(const docmask_chunk* chunks, int32_t n_chunks, int32_t kv_lo,
                                       int32_t kv_hi, int32_t bq, int32_t bk) {
  Problem pr;
  if (bq < 1 || bk < 1) return 0;
  if (check_shape(1, chunks, n_chunks, kv_lo, kv_hi, 1, 1, 64, &pr) != DOCMASK_OK) return 0;
  return sched_layout(count_qtiles(chunks, n_chunks, bq), (pr.tkv + (int64_t)bk - 1) / bk).total;
}

int docmask_schedule(const int32_t* cu_seqlens_dev, int32_t n_docs, const docmask_chunk* chunks,
                     int32_t n_chunks, int32_t kv_lo, int32_t kv_hi, int32_t bq, int32_t bk,
                     int32_t* qtile_desc, int32_t* kvtile_desc, int32_t* need, int32_t* lpt_q,
                     int32_t* lpt_kv, int64_t* counters, void* workspace, size_t workspace_bytes,
                     hipStream_t stream) {
  Problem pr;
  if (bq < 1 || bk < 1 || !cu_seqlens_dev) return DOCMASK_EINVAL;
  int st = check_shape(n_docs, chunks, n_chunks, kv_lo, kv_hi, 1, 1, 64, &pr);
  if (st != DOCMASK_OK) return st;
  const int64_t n_qt = count_qtiles(chunks, n_chunks, bq);
  const int64_t n_kt = (pr.tkv + (int64_t)bk - 1) / bk;
  const Layout L = sched_layout(n_qt, n_kt);
  if (!workspace || workspace_bytes < L.total) return DOCMASK_EWORKSPACE;
  if (!aligned4(workspace)) return DOCMASK_EINVAL;
  SchedParams p;
  std::memset(&p, 0, sizeof(p));
  p.ch = make_table(chunks, n_chunks);
  p.kv_lo = kv_lo; p.kv_hi = kv_hi; p.bq = bq; p.bk = bk;
  p.n_qtiles = (int32_t)n_qt; p.n_kvtiles = (int32_t)n_kt;
  p.cu = cu_seqlens_dev; p.n_docs = n_docs; p.needed_end = pr.needed_end;
  p.qdesc = qtile_desc; p.kvdesc = kvtile_desc; p.need = need;
  p.key_q = at<int32_t>(workspace, L.key_q);
  p.key_kv = at<int32_t>(workspace, L.key_kv);
  p.counters = reinterpret_cast<unsigned long long*>(counters);
  p.err = at<int32_t>(workspace, 0);
  return hip_status(launch_schedule(p, lpt_q, lpt_kv, at<int32_t>(workspace, L.hist), stream));
}

// o (bf16) or o32 (float32): exactly one is the output of O
static int attn_fwd_impl(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_dev,
                         int32_t n_docs, const docmask_chunk* chunks, int32_t n_chunks, int32_t kv_lo, int32_t kv_hi,
                         int32_t hq, int32_t hkv, int32_t d, float softmax_scale, void* o, float* o32, float* lse,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
  Problem pr;
  int st = check_shape(n_docs, chunks, n_chunks, kv_lo, kv_hi, hq, hkv, d, &pr);
  if (st != DOCMASK_OK) return st;
  if (!cu_seqlens_dev || !std::isfinite(softmax_scale) || !(softmax_scale > 0.f)) return DOCMASK_EINVAL;
  if (pr.tq == 0) return DOCMASK_OK;
  void* out = o32 ? static_cast<void*>(o32) : o;
  if (!q || !out || !lse || !aligned16(q) || !aligned16(out) || !aligned4(lse)) return DOCMASK_EINVAL;
  if (pr.tkv > 0 && (!k || !v || !aligned16(k) || !aligned16(v))) return DOCMASK_EINVAL;
  const Layout L = fwd_layout(chunks, n_chunks, pr);
  if (!workspace || workspace_bytes < L.total) return DOCMASK_EWORKSPACE;
  if (!aligned16(workspace)) return DOCMASK_EINVAL;

  SchedParams sp;
  std::memset(&sp, 0, sizeof(sp));
  sp.ch = make_table(chunks, n_chunks);
  sp.kv_lo = kv_lo; sp.kv_hi = kv_hi; sp.bq = fwd_rows_per_tile(pr.group); sp.bk = kFwdBK;
  sp.n_qtiles = (int32_t)L.n_qt; sp.n_kvtiles = (int32_t)L.n_kt;
  sp.cu = cu_seqlens_dev; sp.n_docs = n_docs; sp.needed_end = pr.needed_end;
  sp.plan_q = at<int32_t>(workspace, L.plan_q);
  sp.key_q = at<int32_t>(workspace, L.key_q);
  sp.err = at<int32_t>(workspace, 0);
  int32_t* lpt = at<int32_t>(workspace, L.lpt_q);
  hipError_t e = launch_schedule(sp, lpt, nullptr, at<int32_t>(workspace, L.hist), stream);
  if (e != hipSuccess) return DOCMASK_EHIP;

  FwdParams fp;
  std::memset(&fp, 0, sizeof(fp));
  fp.q = static_cast<const uint16_t*>(q);
  fp.k = static_cast<const uint16_t*>(k);
  fp.v = static_cast<const uint16_t*>(v);
  fp.o = static_cast<uint16_t*>(o);
  fp.o32 = o32;
  fp.lse = lse;
  fp.cu = cu_seqlens_dev;
  fp.plan = sp.plan_q;
  fp.lpt = lpt;
  fp.err = sp.err;
  fp.n_docs = n_docs; fp.n_qtiles = (int32_t)L.n_qt; fp.hq = hq; fp.hkv = hkv; fp.group = pr.group;
  fp.kv_lo = kv_lo; fp.kv_hi = kv_hi; fp.tq = (int32_t)pr.tq; fp.xcd_cluster = kXcdCluster;
  fp.scale_log2 = (float)((double)softmax_scale * 1.4426950408889634);
  return hip_status(launch_fwd(fp, d, stream));
}

int docmask_attn_fwd(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_dev,
                     int32_t n_docs, const docmask_chunk* chunks, int32_t n_chunks, int32_t kv_lo,
                     int32_t kv_hi, int32_t hq, int32_t hkv, int32_t d, float softmax_scale, void* o,
                     float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return attn_fwd_impl(q, k, v, cu_seqlens_dev, n_docs, chunks, n_chunks, kv_lo, kv_hi, hq, hkv, d, softmax_scale,
                       o, nullptr, lse, workspace, workspace_bytes, stream);
}

// Device address of `scratch` on the current device, looked up on the first
// call on that device (with it current) and kept per device.
static int noalloc_scratch(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DOCMASK_EHIP;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DOCMASK_EHIP;
    addr[dev] = p;
  }
  *out = addr[dev];
  return DOCMASK_OK;
}

int docmask_attn_fwd_noalloc(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_dev,
                             int32_t n_docs, const docmask_chunk* chunks, int32_t n_chunks, int32_t kv_lo,
                             int32_t kv_hi, int32_t hq, int32_t hkv, int32_t d, float softmax_scale, void* o,
                             float* lse, hipStream_t stream) {
  Problem pr;
  int st = check_shape(n_docs, chunks, n_chunks, kv_lo, kv_hi, hq, hkv, d, &pr);
  if (st != DOCMASK_OK) return st;
  if (!cu_seqlens_dev || !std::isfinite(softmax_scale) || !(softmax_scale > 0.f)) return DOCMASK_EINVAL;
  if (pr.tq == 0) return DOCMASK_OK;
  const size_t need = fwd_layout(chunks, n_chunks, pr).total;
  if (need > DOCMASK_NOALLOC_SCRATCH_BYTES) return DOCMASK_ESCRATCH;
  void* ws = nullptr;
  st = noalloc_scratch(&ws);
  if (st != DOCMASK_OK) return st;
  // every region of the workspace the kernels read is written earlier in the
  // same call (the error word by the validation kernel), so the previous
  // call's contents need no clearing
  return attn_fwd_impl(q, k, v, cu_seqlens_dev, n_docs, chunks, n_chunks, kv_lo, kv_hi, hq, hkv, d, softmax_scale, o,
                       nullptr, lse, ws, DOCMASK_NOALLOC_SCRATCH_BYTES, stream);
}

int docmask_attn_fwd_f32out(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_dev,
                            int32_t n_docs, const docmask_chunk* chunks, int32_t n_chunks, int32_t kv_lo,
                            int32_t kv_hi, int32_t hq, int32_t hkv, int32_t d, float softmax_scale, float* o,
                            float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!o) return DOCMASK_EINVAL;
  return attn_fwd_impl(q, k, v, cu_seqlens_dev, n_docs, chunks, n_chunks, kv_lo, kv_hi, hq, hkv, d, softmax_scale,
                       nullptr, o, lse, workspace, workspace_bytes, stream);
}

int docmask_attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                     const void* d_o, const int32_t* cu_seqlens_dev, int32_t n_docs,
                     const docmask_chunk* chunks, int32_t n_chunks, int32_t kv_lo, int32_t kv_hi,
                     int32_t hq, int32_t hkv, int32_t d, float softmax_scale, float* dq, float* dk,
                     float* dv, int flags, void* workspace, size_t workspace_bytes,
                     hipStream_t stream) {
  Problem pr;
  int st = check_shape(n_docs, chunks, n_chunks, kv_lo, kv_hi, hq, hkv, d, &pr);
  if (st != DOCMASK_OK) return st;
  if (!cu_seqlens_dev || !std::isfinite(softmax_scale) || !(softmax_scale > 0.f)) return DOCMASK_EINVAL;
  if (flags & ~(DOCMASK_ACCUMULATE_DQ | DOCMASK_DELTA_READY)) return DOCMASK_EINVAL;
  if (pr.tq > 0 && (!q || !o || !lse || !d_o || !dq || !aligned16(q) || !aligned16(o) || !aligned16(d_o) ||
                    !aligned16(dq) || !aligned4(lse)))
    return DOCMASK_EINVAL;
  if (pr.tkv > 0 && (!k || !v || !dk || !dv || !aligned16(k) || !aligned16(v) || !aligned16(dk) || !aligned16(dv)))
    return DOCMASK_EINVAL;
  if (pr.tq == 0 && pr.tkv == 0) return DOCMASK_OK;
  const Layout L = bwd_layout(chunks, n_chunks, pr, hq);
  if (!workspace || workspace_bytes < L.total) return DOCMASK_EWORKSPACE;
  if (!aligned16(workspace)) return DOCMASK_EINVAL;

  // schedule of the dK/dV pass (KV-tile ranges, LPT over KV tiles)
  SchedParams sp;
  std::memset(&sp, 0, sizeof(sp));
  sp.ch = make_table(chunks, n_chunks);
  sp.kv_lo = kv_lo; sp.kv_hi = kv_hi; sp.bq = kBwdBQ; sp.bk = kBwdBK;
  sp.n_qtiles = (int32_t)L.n_qt; sp.n_kvtiles = (int32_t)L.n_kt;
  sp.cu = cu_seqlens_dev; sp.n_docs = n_docs; sp.needed_end = pr.needed_end;
  sp.plan_q = at<int32_t>(workspace, L.plan_q);
  sp.kvdesc = at<int32_t>(workspace, L.kvdesc);
  sp.key_kv = at<int32_t>(workspace, L.key_kv);
  sp.kv_pair = at<int32_t>(workspace, L.kv_pair);
  sp.key_pair = at<int32_t>(workspace, L.key_pair);
  sp.err = at<int32_t>(workspace, 0);
  int32_t* lpt_kv = at<int32_t>(workspace, L.lpt_kv);
  hipError_t e = launch_schedule(sp, nullptr, lpt_kv, at<int32_t>(workspace, L.hist), stream);
  if (e != hipSuccess) return DOCMASK_EHIP;
  // schedule of the dQ pass (forward-style Q-tile ranges, LPT over Q tiles)
  SchedParams sq = sp;
  sq.bq = dq_rows_per_tile(pr.group); sq.bk = kDqBK;
  sq.n_qtiles = (int32_t)L.n_qt2; sq.n_kvtiles = (int32_t)L.n_kt2;
  sq.plan_q = at<int32_t>(workspace, L.plan_q2);
  sq.kvdesc = nullptr;
  sq.key_kv = nullptr;
  sq.kv_pair = nullptr;
  sq.key_pair = nullptr;
  sq.key_q = at<int32_t>(workspace, L.key_q);
  int32_t* lpt_q = at<int32_t>(workspace, L.lpt_q);
  e = launch_schedule(sq, lpt_q, nullptr, at<int32_t>(workspace, L.hist), stream);
  if (e != hipSuccess) return DOCMASK_EHIP;

  BwdParams bp;
  std::memset(&bp, 0, sizeof(bp));
  bp.q = static_cast<const uint16_t*>(q);
  bp.k = static_cast<const uint16_t*>(k);
  bp.v = static_cast<const uint16_t*>(v);
  bp.o = static_cast<const uint16_t*>(o);
  bp.d_o = static_cast<const uint16_t*>(d_o);
  bp.lse = lse;
  bp.dq = dq; bp.dk = dk; bp.dv = dv;
  bp.delta = at<float>(workspace, L.delta);
  bp.cu = cu_seqlens_dev;
  bp.plan_kq = sp.plan_q;
  bp.kvdesc = sp.kvdesc;
  bp.lpt_kv = lpt_kv;
  bp.kv_pair = sp.kv_pair;
  bp.plan_q = sq.plan_q;
  bp.lpt_q = lpt_q;
  bp.err = sp.err;
  bp.n_docs = n_docs; bp.n_qtiles = (int32_t)L.n_qt; bp.n_kvtiles = (int32_t)L.n_kt;
  bp.n_qtiles_dq = (int32_t)L.n_qt2;
  bp.hq = hq; bp.hkv = hkv; bp.group = pr.group; bp.kv_lo = kv_lo; bp.kv_hi = kv_hi;
  bp.tq = (int32_t)pr.tq; bp.xcd_cluster = kXcdCluster;
  bp.xcd_cluster_q = kXcdCluster;
  bp.accumulate_dq = (flags & DOCMASK_ACCUMULATE_DQ) != 0;
  bp.scale = softmax_scale;
  bp.scale_log2 = (float)((double)softmax_scale * 1.4426950408889634);
  return hip_status(launch_bwd(bp, sp.ch, d, (flags & DOCMASK_DELTA_READY) != 0, stream));
}

// o_parts (bf16) or o_parts32 (float32): exactly one holds the partials
static int merge_impl(const void* o_parts, const float* o_parts32, const float* lse_parts, int32_t n_parts,
                      int32_t rows, int32_t hq, int32_t d, void* o_out, float* lse_out, hipStream_t stream) {
  if (n_parts < 1 || rows < 0 || hq < 1) return DOCMASK_EINVAL;
  if (d != 64 && d != 128) return DOCMASK_EUNSUPPORTED;
  if ((int64_t)rows * hq > INT32_MAX) return DOCMASK_EINVAL;
  if (rows == 0) return DOCMASK_OK;
  const void* parts = o_parts32 ? static_cast<const void*>(o_parts32) : o_parts;
  if (!parts || !lse_parts || !o_out || !lse_out) return DOCMASK_EINVAL;
  if (!aligned16(parts) || !aligned16(o_out) || !aligned4(lse_parts) || !aligned4(lse_out)) return DOCMASK_EINVAL;
  MergeParams p;
  p.o_parts = static_cast<const uint16_t*>(o_parts);
  p.o_parts32 = o_parts32;
  p.lse_parts = lse_parts;
  p.o_out = static_cast<uint16_t*>(o_out);
  p.lse_out = lse_out;
  p.n_parts = n_parts; p.rows = rows; p.hq = hq;
  return hip_status(launch_merge(p, d, stream));
}

int lse_merge(const void* o_parts, const float* lse_parts, int32_t n_parts, int32_t rows, int32_t hq,
              int32_t d, void* o_out, float* lse_out, hipStream_t stream) {
  return merge_impl(o_parts, nullptr, lse_parts, n_parts, rows, hq, d, o_out, lse_out, stream);
}

int lse_merge_f32(const float* o_parts, const float* lse_parts, int32_t n_parts, int32_t rows, int32_t hq,
                  int32_t d, void* o_out, float* lse_out, hipStream_t stream) {
  if (!o_parts) return DOCMASK_EINVAL;
  return merge_impl(nullptr, o_parts, lse_parts, n_parts, rows, hq, d, o_out, lse_out, stream);
}

int docmask_check_errors(const void* workspace, hipStream_t stream) {
  if (!workspace) return DOCMASK_EINVAL;
  if (hipStreamSynchronize(stream) != hipSuccess) return DOCMASK_EHIP;
  int32_t flag = 0;
  if (hipMemcpy(&flag, workspace, sizeof(flag), hipMemcpyDeviceToHost) != hipSuccess) return DOCMASK_EHIP;
  return flag ? DOCMASK_EDEVICE_INPUT : DOCMASK_OK;
}

int docmask_f32_to_bf16(const float* src, void* dst, int64_t n, hipStream_t stream) {
  if (n < 0) return DOCMASK_EINVAL;
  if (n == 0) return DOCMASK_OK;
  if (!src || !dst || !aligned16(src) || !aligned16(dst)) return DOCMASK_EINVAL;
  return hip_status(launch_f32_to_bf16(src, static_cast<uint16_t*>(dst), n, stream));
}

const char* docmask_strerror(int status) {
  switch (status) {
    case DOCMASK_OK: return "ok";
    case DOCMASK_EINVAL: return "invalid argument";
    case DOCMASK_EUNSUPPORTED: return "unsupported configuration (head_dim must be 64 or 128)";
    case DOCMASK_EWORKSPACE: return "workspace missing or too small";
    case DOCMASK_EHIP: return "HIP launch failed";
    case DOCMASK_EDEVICE_INPUT: return "malformed cu_seqlens (not starting at 0, decreasing, or too short)";
    case DOCMASK_ESCRATCH:
      return "problem too large for the allocation-free forward's static scratch (DOCMASK_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

}  // extern "C"
