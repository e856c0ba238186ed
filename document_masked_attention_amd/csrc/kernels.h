// Kernel parameter blocks and launchers (internal to libdocmask).
#pragma once

#include "common.h"
#include "docmask.h"
#include "timing.h"

namespace docmask {

struct SchedParams {
  ChunkTable ch;
  int32_t kv_lo, kv_hi, bq, bk, n_qtiles, n_kvtiles;
  const int32_t* cu;
  int32_t n_docs;
  int32_t needed_end;              // largest global position + 1 any call touches
  int32_t* plan_q;                 // [n_qtiles][QP_WORDS] or null
  int32_t* qdesc;                  // [n_qtiles][4] or null
  int32_t* kvdesc;                 // [n_kvtiles][4] or null
  int32_t* need;                   // [n_chunks][2] or null
  int32_t* key_q;                  // [n_qtiles] or null
  int32_t* key_kv;                 // [n_kvtiles] or null
  int32_t* kv_pair;                // [n_kvtiles] KV tile paired with each tile (itself if alone) or null
  int32_t* key_pair;               // [n_kvtiles] LPT key of the pair a tile leads (0: not a leader)
  unsigned long long* counters;    // [4] or null
  int32_t* err;                    // workspace error word
};

struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* o32;            // non-null: O written here as float32 (partials for the fp32 merge), o unused
  float* lse;
  const int32_t* cu;
  const int32_t* plan;   // [n_qtiles][QP_WORDS]
  const int32_t* lpt;    // [n_qtiles]
  const int32_t* err;
  int32_t n_docs, n_qtiles, hq, hkv, group, n_hb, kv_lo, kv_hi, tq, xcd_cluster;
  float scale_log2;      // softmax scale * log2(e)
};

struct MergeParams {
  const uint16_t* o_parts;   // [P][rows][hq][D] bf16, or
  const float* o_parts32;    // the same as float32 (non-null selects it)
  const float* lse_parts;    // [P][hq][rows]
  uint16_t* o_out;           // [rows][hq][D]
  float* lse_out;            // [hq][rows]
  int32_t n_parts, rows, hq;
};

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* d_o;
  const float* lse;
  float* dq;
  float* dk;
  float* dv;
  float* delta;           // [hq][tq] workspace
  const int32_t* cu;
  const int32_t* plan_kq; // [n_qtiles][QP_WORDS], 32-row query blocks (dK/dV kernel)
  const int32_t* kvdesc;  // [n_kvtiles][4] with bk = kBwdBK
  const int32_t* lpt_kv;  // [n_kvtiles] work items (pair leaders first, by descending work)
  const int32_t* kv_pair; // [n_kvtiles] partner tile of each KV tile (itself if alone)
  const int32_t* plan_q;  // [n_qtiles_dq][QP_WORDS], forward-style tiles (dQ kernel)
  const int32_t* lpt_q;   // [n_qtiles_dq]
  const int32_t* err;
  int32_t n_docs, n_qtiles, n_kvtiles, n_qtiles_dq, hq, hkv, group, n_hb, kv_lo, kv_hi, tq;
  int32_t xcd_cluster, xcd_cluster_q;   // ranks per XCD cluster (dK/dV, dQ)
  int32_t accumulate_dq;
  int32_t delta_ready;    // Delta supplied by the caller (else the dQ kernel computes and stores it)
  float scale;            // softmax scale
  float scale_log2;       // softmax scale * log2(e)
};

constexpr int kFwdBK = 64;
constexpr int kBwdBQ = 32;
constexpr int kBwdBK = 128;
constexpr int kDqBK = 64;
// Positions per document start whose pairs the backward evaluates in fp32 (the
// head pass): every allowed pair (i, j) with ds <= j <= i < ds + kBwdHead, ds
// the document start.  Must stay below kDqBK and kBwdBK, so that no FULL
// tile of either backward kernel holds such a pair (the kernels mask them
// out on their masked path).
constexpr int kBwdHead = 32;
static_assert(kBwdHead < kDqBK && kBwdHead < kBwdBK, "head pairs only in masked tiles");

hipError_t launch_schedule(const SchedParams& p, int32_t* lpt_q, int32_t* lpt_kv, int32_t* hist,
                           hipStream_t stream);
hipError_t launch_fwd(const FwdParams& p, int d, hipStream_t stream);
int fwd_rows_per_tile(int group);
hipError_t launch_merge(const MergeParams& p, int d, hipStream_t stream);
hipError_t launch_f32_to_bf16(const float* src, uint16_t* dst, int64_t n, hipStream_t stream);
hipError_t launch_bwd(const BwdParams& p, const ChunkTable& ch, int d, bool delta_ready, hipStream_t stream);
int dq_rows_per_tile(int group);
hipError_t launch_copy_rows(const void* src_k, const void* src_v, void* dst_k, void* dst_v, int64_t dst_rows,
                            int64_t row_bytes, const docmask_rowmap* maps, int32_t n_maps, bool zero_gaps,
                            hipStream_t stream);

}  // namespace docmask
