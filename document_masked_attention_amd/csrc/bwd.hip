// Backward kernels: exact gradients of <dO, O> for document-masked attention.
//
// The pages name the attention backward (FlashCP paper, Figure 6, "Attention
// BWD") without writing it out; this is the plain calculus of the forward:
//   P_ij = exp(s_ij - LSE_i)  (0 where the document mask forbids (i, j))
//   Delta_i = sum_d dO_id O_id
//   dV_j = sum_i P_ij dO_i,   dS_ij = P_ij (dO_i . v_j - Delta_i)
//   dK_j = scale sum_i dS_ij q_i,   dQ_i = scale sum_j dS_ij k_j
// with dK and dV summed over the query heads of each KV group.
//
// Two kernels, both deterministic (no atomics):
//
// * dkdv_kernel, key-major.  Work item = (KV tile of 128 keys, KV head);
//   8 waves x 16 keys, each wave keeping its K and V rows (MFMA B operands)
//   and its dK, dV accumulators in registers.  It walks every (32-row query
//   block, query head of the group) that attends the tile -- the scheduler's
//   per-KV-tile range -- with the Q and dO rows double-buffered in LDS:
//     S = Q K^T,  P = exp2(S c - LSE2),  dV^T += dO^T P,
//     dP = dO V^T,  dS = P (dP - Delta),  dK^T += Q^T dS
//   (v_mfma_f32_16x16x32_bf16; Q^T and dO^T come from the row-major tiles
//   through LDS transpose reads).
// * dq_kernel, query-major, shaped like the forward.  Work item = (query tile,
//   KV head, block of query heads), 8 waves; each wave owns 32 rows x 1 head
//   and walks the tile's KV range:
//     S^T = K Q^T,  dP^T = V dO^T,  dS^T = P^T (dP^T - Delta),  dQ^T += K^T dS^T
//   (v_mfma_f32_32x32x16_bf16; K^T through transpose reads).
#include "kernels.h"

#include <cstdlib>

namespace docmask {

// Delta = rowsum(dO * O) per (row, head), float32 from the bf16 inputs.
template <int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(const uint16_t* __restrict__ o,
                                                        const uint16_t* __restrict__ d_o,
                                                        float* __restrict__ delta, int32_t tq, int32_t hq) {
  constexpr int CPR = D / 8;
  const size_t gid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t rh = gid / CPR;
  const int c = (int)(gid % CPR);
  const size_t n_rh = (size_t)tq * hq;
  float acc = 0.f;
  if (rh < n_rh) {
    const uint4 a = *reinterpret_cast<const uint4*>(o + rh * D + 8 * c);
    const uint4 b = *reinterpret_cast<const uint4*>(d_o + rh * D + 8 * c);
    const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc += __uint_as_float(aw[i] << 16) * __uint_as_float(bw[i] << 16);
      acc += __uint_as_float(aw[i] & 0xffff0000u) * __uint_as_float(bw[i] & 0xffff0000u);
    }
  }
#pragma unroll
  for (int off = CPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (rh < n_rh && c == 0) {
    const int row = (int)(rh / hq), head = (int)(rh % hq);
    delta[(size_t)head * tq + row] = acc;
  }
}

__device__ __forceinline__ bf16x8 cvt8(float a0, float a1, float a2, float a3, float b0, float b1, float b2,
                                      float b3) {
  const bf16x2 p0 = __builtin_convertvector(f32x2{a0, a1}, bf16x2);
  const bf16x2 p1 = __builtin_convertvector(f32x2{a2, a3}, bf16x2);
  const bf16x2 p2 = __builtin_convertvector(f32x2{b0, b1}, bf16x2);
  const bf16x2 p3 = __builtin_convertvector(f32x2{b2, b3}, bf16x2);
  return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// ------------------------------------------------------------------ dK, dV
// HPI query heads of the group are processed per step: the K/V operand
// registers are shared, the heads' MFMA chains are independent, and each
// barrier covers HPI times the work.
template <int D, int HPI>
__global__ __launch_bounds__(512, 1) void dkdv_kernel(BwdParams p) {
  constexpr int BQ = kBwdBQ;            // 32 query rows per step
  constexpr int BK = kBwdBK;            // 128 keys per work item, 16 per wave
  constexpr int NKS = D / 32;           // k-steps over d (16x16x32)
  constexpr int NDB = D / 16;           // 16-wide d blocks of dK^T / dV^T
  constexpr int CPR = D / 8;            // 16-byte chunks per row
  using L = SwzTile<D, kSwzOctet>;      // Q / dO tile layout (row chunks + transpose reads)
  constexpr int TE = L::kElems(BQ);     // elements of one 32-row tile
  constexpr int NCH = 2 * HPI * BQ * CPR;   // 16-byte chunks staged per step (Q and dO of HPI heads)
  constexpr int CPT = (NCH + 511) / 512;    // chunks per thread
  __shared__ __attribute__((aligned(16))) uint16_t qd_s[2][2 * HPI][TE];   // [buf][2h: Q, 2h+1: dO]
  __shared__ __attribute__((aligned(16))) float lse_s[2][HPI][BQ];
  __shared__ __attribute__((aligned(16))) float dlt_s[2][HPI][BQ];

  if (p.err[0]) return;

  const WorkItem wi = map_work(blockIdx.x, p.n_kvtiles, p.hkv, 1, p.xcd_cluster);
  const int kvh = wi.kvh;
  const int tile = min(max(p.lpt_kv[wi.rank], 0), p.n_kvtiles - 1);
  const int32_t* kd = p.kvdesc + (size_t)tile * 4;
  const int qt_lo = kd[0], qt_flo = kd[1], qt_fhi = kd[2], qt_hi = kd[3];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, g = lane >> 4, i16 = lane & 15;
  const int tkv = p.kv_hi - p.kv_lo;
  const int key_l = tile * BK + 16 * wave + i16;    // this lane's key (local KV row)
  const bool key_ok = key_l < tkv;
  const int key_g = p.kv_lo + key_l;
  // rows that may attend this key: key_g <= i < end of its document
  const int key_end = key_ok ? doc_end(p.cu, p.n_docs, key_g) : key_g;
  const size_t kv_rstride = (size_t)p.hkv * D;
  const bool ragged = (tile + 1) * BK > tkv;

  // K and V rows of this lane's key as MFMA B operands: d = 32 s + 8 g .. +8
  bf16x8 kf[NKS], vf[NKS];
  {
    const int kl = min(key_l, tkv - 1);               // padding keys: any finite row, masked below
    const uint16_t* kr = p.k + (size_t)kl * kv_rstride + (size_t)kvh * D + 8 * g;
    const uint16_t* vr = p.v + (size_t)kl * kv_rstride + (size_t)kvh * D + 8 * g;
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      kf[s] = *reinterpret_cast<const bf16x8*>(kr + 32 * s);
      vf[s] = *reinterpret_cast<const bf16x8*>(vr + 32 * s);
    }
  }
  f32x4 dkacc[NDB], dvacc[NDB];
#pragma unroll
  for (int b = 0; b < NDB; ++b) { dkacc[b] = f32x4{}; dvacc[b] = f32x4{}; }

  const int n_hsteps = p.group / HPI;
  const int n_it = (qt_hi - qt_lo) * n_hsteps;
  // staging of one step: chunk u (< NCH) = tensor t (2h: Q, 2h+1: dO of head
  // h of the step), row, 16-byte column chunk; lse / Delta of the HPI heads
  auto load_step = [&](int it, u32x4 (&reg)[CPT], float& sc) __attribute__((always_inline)) {
    const int qt = qt_lo + it / n_hsteps;
    const int head0 = kvh * p.group + (it % n_hsteps) * HPI;
    const int32_t* pl = p.plan_kq + (size_t)qt * QP_WORDS;
    const int l_row0 = pl[QP_LROW0], nrows = pl[QP_NROWS];
    static_for<CPT>([&](auto jc) __attribute__((always_inline)) {
      constexpr int j = decltype(jc)::value;
      const int u = tid + 512 * j;
      if (NCH % 512 == 0 || u < NCH) {
        const int t = u / (BQ * CPR), rc = u % (BQ * CPR);
        const int row = rc / CPR, c = rc % CPR;
        const int rr = min(row, nrows - 1);         // padded rows: a real row, never used (P = 0)
        const size_t off = ((size_t)(l_row0 + rr) * p.hq + head0 + (t >> 1)) * D + 8 * c;
        reg[j] = *reinterpret_cast<const u32x4*>(((t & 1) ? p.d_o : p.q) + off);
      }
    });
    sc = 0.f;
    if (tid < 2 * HPI * BQ) {
      const int row = tid % BQ, h = (tid / BQ) % HPI;
      const bool is_lse = tid < HPI * BQ;
      if (row < nrows) {
        const size_t idx = (size_t)(head0 + h) * p.tq + l_row0 + row;
        if (is_lse) {
          const float lv = p.lse[idx];
          sc = lv == -INFINITY ? INFINITY : lv * kLog2e;   // empty row: P = 0
        } else {
          sc = p.delta[idx];
        }
      } else {
        sc = is_lse ? INFINITY : 0.f;                    // padded row: P = 0
      }
    }
  };
  auto store_step = [&](int buf, const u32x4 (&reg)[CPT], float sc) __attribute__((always_inline)) {
    static_for<CPT>([&](auto jc) __attribute__((always_inline)) {
      constexpr int j = decltype(jc)::value;
      const int u = tid + 512 * j;
      if (NCH % 512 == 0 || u < NCH) {
        const int t = u / (BQ * CPR), rc = u % (BQ * CPR);
        const int row = rc / CPR, c = rc % CPR;
        *reinterpret_cast<u32x4*>(&qd_s[buf][t][L::off(row, 8 * c)]) = reg[j];
      }
    });
    if (tid < HPI * BQ) lse_s[buf][tid / BQ][tid % BQ] = sc;
    else if (tid < 2 * HPI * BQ) dlt_s[buf][(tid / BQ) % HPI][tid % BQ] = sc;
  };

  // transpose-read source row/column of this lane inside a 32-row tile: query
  // rows {4g + e} (first read) and {16 + 4g + e} (second read), columns
  // 16 db + 4 (i16 % 4); the swizzle depends on the row modulo 16 only
  const int tr_row = 4 * g + (i16 >> 2), tr_col = 4 * (i16 & 3);

  if (n_it > 0) {
    u32x4 reg[CPT];
    float sc;
    load_step(0, reg, sc);
    store_step(0, reg, sc);
  }
  __syncthreads();
  for (int it = 0; it < n_it; ++it) {
    const int buf = it & 1;
    u32x4 reg[CPT];
    float sc;
    load_step(min(it + 1, n_it - 1), reg, sc);        // next step's rows in flight (last: a repeat)

    const int qt = qt_lo + it / n_hsteps;
    const int32_t* pl = p.plan_kq + (size_t)qt * QP_WORDS;
    const int g_row0 = pl[QP_GROW0], nrows = pl[QP_NROWS];
    const bool masked = qt < qt_flo || qt >= qt_fhi || ragged;
    // allowed rows of this key: key_g <= g_row0 + qr < key_end, qr < nrows
    const int lo = key_g - g_row0;
    const int hi = key_ok ? min(key_end - g_row0, nrows) : lo;

    bf16x8 pb[HPI], dsb[HPI];
#pragma unroll
    for (int h = 0; h < HPI; ++h) {
      const uint16_t* qs = qd_s[buf][2 * h];
      const uint16_t* dos = qd_s[buf][2 * h + 1];
      // S = Q K^T and dP = dO V^T: rows q = 16 mb + 4 g + r, column = this lane's key
      f32x4 sacc[2], dpacc[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        sacc[mb] = f32x4{};
        dpacc[mb] = f32x4{};
#pragma unroll
        for (int s = 0; s < NKS; ++s) {
          const int off = L::off(16 * mb + i16, 32 * s + 8 * g);
          const bf16x8 qa_ = *reinterpret_cast<const bf16x8*>(&qs[off]);
          const bf16x8 da_ = *reinterpret_cast<const bf16x8*>(&dos[off]);
          sacc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa_, kf[s], sacc[mb], 0, 0, 0);
          dpacc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(da_, vf[s], dpacc[mb], 0, 0, 0);
        }
      }
      const f32x4 l0 = *reinterpret_cast<const f32x4*>(&lse_s[buf][h][4 * g]);
      const f32x4 l1 = *reinterpret_cast<const f32x4*>(&lse_s[buf][h][16 + 4 * g]);
      const f32x4 d0 = *reinterpret_cast<const f32x4*>(&dlt_s[buf][h][4 * g]);
      const f32x4 d1 = *reinterpret_cast<const f32x4*>(&dlt_s[buf][h][16 + 4 * g]);
      float pv[8], dsv[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pv[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[0][r], p.scale_log2, -l0[r]));
        pv[4 + r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[1][r], p.scale_log2, -l1[r]));
      }
      if (masked) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int qr = 16 * (e >> 2) + 4 * g + (e & 3);
          if (qr < lo || qr >= hi) pv[e] = 0.f;
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        dsv[r] = pv[r] * (dpacc[0][r] - d0[r]);
        dsv[4 + r] = pv[4 + r] * (dpacc[1][r] - d1[r]);
      }
      pb[h] = cvt8(pv[0], pv[1], pv[2], pv[3], pv[4], pv[5], pv[6], pv[7]);
      dsb[h] = cvt8(dsv[0], dsv[1], dsv[2], dsv[3], dsv[4], dsv[5], dsv[6], dsv[7]);
    }
    // dV^T += dO^T P and dK^T += Q^T dS over the 32 rows of each head (one
    // k-step each): the A operands gather rows {4g + e, 16 + 4g + e} of
    // column 16 db + i16.  The schedule keeps the transpose reads two
    // (d block, head) groups ahead of the MFMAs that consume them.
    sched_reads_ahead<NDB * HPI, 4, 2>();
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int o0 = L::off(tr_row, 16 * db + tr_col), o1 = L::off(tr_row + 16, 16 * db + tr_col);
#pragma unroll
      for (int h = 0; h < HPI; ++h) {
        const uint16_t* qs = qd_s[buf][2 * h];
        const uint16_t* dos = qd_s[buf][2 * h + 1];
        const bf16x8 doT = tr_operand(dos + o0, dos + o1);
        const bf16x8 qT = tr_operand(qs + o0, qs + o1);
        dvacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(doT, pb[h], dvacc[db], 0, 0, 0);
        dkacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qT, dsb[h], dkacc[db], 0, 0, 0);
      }
    }
    store_step(buf ^ 1, reg, sc);
    __syncthreads();
  }

  // dK (scaled) and dV of this lane's key: d = 16 db + 4 g .. +4
  if (key_ok) {
    float* dkp = p.dk + (size_t)key_l * kv_rstride + (size_t)kvh * D + 4 * g;
    float* dvp = p.dv + (size_t)key_l * kv_rstride + (size_t)kvh * D + 4 * g;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      *reinterpret_cast<float4*>(dkp + 16 * db) =
          make_float4(dkacc[db][0] * p.scale, dkacc[db][1] * p.scale, dkacc[db][2] * p.scale, dkacc[db][3] * p.scale);
      *reinterpret_cast<float4*>(dvp + 16 * db) = make_float4(dvacc[db][0], dvacc[db][1], dvacc[db][2], dvacc[db][3]);
    }
  }
}

// ------------------------------------------------------------------ dQ
template <int D, int RB, int HB>
__global__ __launch_bounds__(512, 1) void dq_kernel(BwdParams p) {
  static_assert(RB * HB == 8, "eight waves per workgroup");
  constexpr int BK = kDqBK;
  using L = SwzTile<D, kSwzQuad>;       // K tile: row chunks and transpose reads
  constexpr int VS = D + 8;             // V tile: row chunks only (padded rows)
  constexpr int CPK = D / 8;
  constexpr int KPP = 512 / CPK;
  constexpr int KPASS = BK / KPP;
  constexpr int NKS = D / 16;
  constexpr int NDB = D / 32;
  __shared__ __attribute__((aligned(16))) uint16_t k_s[2][L::kElems(BK)];
  __shared__ __attribute__((aligned(16))) uint16_t v_s[2][BK * VS];

  if (p.err[0]) return;

  const WorkItem wi = map_work(blockIdx.x, p.n_qtiles_dq, p.hkv, p.n_hb, p.xcd_cluster_q);
  const int kvh = wi.kvh, hb = wi.hb;
  const int tile = min(max(p.lpt_q[wi.rank], 0), p.n_qtiles_dq - 1);
  const int32_t* pl = p.plan_q + (size_t)tile * QP_WORDS;
  const int l_row0 = pl[QP_LROW0], g_row0 = pl[QP_GROW0], nrows = pl[QP_NROWS];
  const int kt_lo = pl[QP_KT_LO], kt_flo = pl[QP_KT_FLO], kt_fhi = pl[QP_KT_FHI], kt_hi = pl[QP_KT_HI];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, hh = lane >> 5, ln = lane & 31;
  const int rb = wave / HB, hs = wave % HB;
  const int head = kvh * p.group + hb * HB + hs;
  const int qr = 32 * rb + ln;
  const bool row_ok = qr < nrows;
  const int gi = g_row0 + qr;
  const size_t o_off = ((size_t)(l_row0 + qr) * p.hq + head) * D;
  int a_lo = 0x40000000, a_w = 0;
  float lse2 = INFINITY, dlt = 0.f;
  if (row_ok) {
    const int lo = max(doc_start(p.cu, p.n_docs, gi), p.kv_lo), hi = min(gi, p.kv_hi - 1);
    if (hi >= lo) { a_lo = lo; a_w = hi - lo; }
    const float lv = p.lse[(size_t)head * p.tq + l_row0 + qr];
    lse2 = lv == -INFINITY ? INFINITY : lv * kLog2e;
    dlt = p.delta[(size_t)head * p.tq + l_row0 + qr];
  }
  bf16x8 qf[NKS], dof[NKS];
#pragma unroll
  for (int s = 0; s < NKS; ++s) {
    qf[s] = row_ok ? *reinterpret_cast<const bf16x8*>(p.q + o_off + 16 * s + 8 * hh) : bf16x8{};
    dof[s] = row_ok ? *reinterpret_cast<const bf16x8*>(p.d_o + o_off + 16 * s + 8 * hh) : bf16x8{};
  }
  f32x16 dqacc[NDB];
#pragma unroll
  for (int b = 0; b < NDB; ++b) dqacc[b] = f32x16{};

  const int tkv = p.kv_hi - p.kv_lo;
  const size_t kv_rstride = (size_t)p.hkv * D;
  const uint16_t* kbase = p.k + (size_t)kvh * D;
  const uint16_t* vbase = p.v + (size_t)kvh * D;
  const int kc = tid % CPK, kk0 = tid / CPK;
  auto load_rows = [&](const uint16_t* base, int kt, u32x4 (&reg)[KPASS]) __attribute__((always_inline)) {
#pragma unroll
    for (int pp = 0; pp < KPASS; ++pp) {
      const int key = min(kt * BK + kk0 + KPP * pp, tkv - 1);   // padding keys: masked, any finite row
      reg[pp] = *reinterpret_cast<const u32x4*>(base + (size_t)key * kv_rstride + 8 * kc);
    }
  };
  auto store_k = [&](uint16_t* lds, const u32x4 (&reg)[KPASS]) __attribute__((always_inline)) {
#pragma unroll
    for (int pp = 0; pp < KPASS; ++pp)
      *reinterpret_cast<u32x4*>(&lds[L::off(kk0 + KPP * pp, 8 * kc)]) = reg[pp];
  };
  auto store_v = [&](uint16_t* lds, const u32x4 (&reg)[KPASS]) __attribute__((always_inline)) {
#pragma unroll
    for (int pp = 0; pp < KPASS; ++pp)
      *reinterpret_cast<u32x4*>(&lds[(kk0 + KPP * pp) * VS + 8 * kc]) = reg[pp];
  };
  // transpose-read source row/column for the K^T operand (keys in the S^T
  // accumulator's permuted order, see the forward kernel)
  const int i16 = lane & 15;
  const int kt_row = 4 * hh + (i16 >> 2), kt_col = 16 * ((lane >> 4) & 1) + 4 * (i16 & 3);

  const int n = kt_hi - kt_lo;
  if (n > 0) {
    u32x4 kr[KPASS], vr[KPASS];
    load_rows(kbase, kt_lo, kr);
    load_rows(vbase, kt_lo, vr);
    store_k(k_s[0], kr);
    store_v(v_s[0], vr);
  }
  __syncthreads();
  for (int u = 0; u < n; ++u) {
    const int kt = kt_lo + u;
    const int buf = u & 1;
    u32x4 kr[KPASS], vr[KPASS];
    load_rows(kbase, min(kt + 1, kt_hi - 1), kr);    // the last tile again on the final step
    load_rows(vbase, min(kt + 1, kt_hi - 1), vr);
    const uint16_t* ks = k_s[buf];
    const uint16_t* vs = v_s[buf];
    const bool partial = kt < kt_flo || kt >= kt_fhi || (kt + 1) * BK > tkv;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 sacc = f32x16{}, dpacc = f32x16{};
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(&ks[L::off(32 * kb + ln, 16 * s + 8 * hh)]);
        const bf16x8 vf = *reinterpret_cast<const bf16x8*>(&vs[(32 * kb + ln) * VS + 16 * s + 8 * hh]);
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], sacc, 0, 0, 0);
        dpacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, dof[s], dpacc, 0, 0, 0);
      }
      // P^T and dS^T for keys 32 kb + 8 (r / 4) + 4 hh + r % 4 of this tile
      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r], p.scale_log2, -lse2));
        if (partial) {
          const unsigned rel = (unsigned)(p.kv_lo + kt * BK + 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3) - a_lo);
          if (rel > (unsigned)a_w) pr = 0.f;
        }
        ds[r] = pr * (dpacc[r] - dlt);
      }
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        const bf16x8 dsb = cvt8(ds[8 * k2], ds[8 * k2 + 1], ds[8 * k2 + 2], ds[8 * k2 + 3], ds[8 * k2 + 4],
                                ds[8 * k2 + 5], ds[8 * k2 + 6], ds[8 * k2 + 7]);
#pragma unroll
        for (int b = 0; b < NDB; ++b) {
          const int r0 = 32 * kb + 16 * k2 + kt_row;
          const bf16x8 kT = tr_operand(ks + L::off(r0, 32 * b + kt_col), ks + L::off(r0 + 8, 32 * b + kt_col));
          dqacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kT, dsb, dqacc[b], 0, 0, 0);
        }
      }
    }
    store_k(k_s[buf ^ 1], kr);
    store_v(v_s[buf ^ 1], vr);
    __syncthreads();
  }

  // dQ = scale * acc: lane's row, d = 32 b + 8 g + 4 hh .. +4 (added to dq for split-KV callers)
  if (row_ok) {
    float* dqp = p.dq + o_off + 4 * hh;
#pragma unroll
    for (int b = 0; b < NDB; ++b)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        float4 val = make_float4(dqacc[b][4 * g4] * p.scale, dqacc[b][4 * g4 + 1] * p.scale,
                                 dqacc[b][4 * g4 + 2] * p.scale, dqacc[b][4 * g4 + 3] * p.scale);
        float4* dst = reinterpret_cast<float4*>(dqp + 32 * b + 8 * g4);
        if (p.accumulate_dq) {
          const float4 old = *dst;
          val.x += old.x; val.y += old.y; val.z += old.z; val.w += old.w;
        }
        *dst = val;
      }
  }
}

// query heads per dK/dV step (overridable through DOCMASK_DKDV_HEADS for tuning)
static int dkdv_heads_per_step(int group) {
  int want = 2;
  if (const char* v = std::getenv("DOCMASK_DKDV_HEADS")) want = std::atoi(v);
  for (int h : {4, 2, 1})
    if (h <= want && group % h == 0) return h;
  return 1;
}

// query heads per dQ work item: as many heads of the GQA group as divide it (<= 8)
static int dq_heads_per_item(int group) {
  return (group % 8 == 0) ? 8 : (group % 4 == 0) ? 4 : (group % 2 == 0) ? 2 : 1;
}

int dq_rows_per_tile(int group) { return 32 * (8 / dq_heads_per_item(group)); }

hipError_t launch_bwd(const BwdParams& p, int d, bool delta_ready, hipStream_t stream) {
  const long long rh_threads = (long long)p.tq * p.hq * (d / 8);
  if (rh_threads > 0 && !delta_ready) {
    const long long blocks = (rh_threads + 255) / 256;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    KernelTimer timer(KC_DELTA, stream);
    if (d == 128)
      hipLaunchKernelGGL(bwd_delta_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, stream, p.o, p.d_o, p.delta,
                         p.tq, p.hq);
    else
      hipLaunchKernelGGL(bwd_delta_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, stream, p.o, p.d_o, p.delta,
                         p.tq, p.hq);
  }
  const long long nblk_kv = (long long)p.n_kvtiles * p.hkv;
  if (nblk_kv > 0) {
    if (nblk_kv > 0x7fffffffLL) return hipErrorInvalidValue;
    const int hpi = dkdv_heads_per_step(p.group);
    dim3 grid((unsigned)nblk_kv), block(512);
    KernelTimer timer(KC_DKDV, stream);
    if (d == 128) {
      if (hpi == 4) hipLaunchKernelGGL((dkdv_kernel<128, 4>), grid, block, 0, stream, p);
      else if (hpi == 2) hipLaunchKernelGGL((dkdv_kernel<128, 2>), grid, block, 0, stream, p);
      else hipLaunchKernelGGL((dkdv_kernel<128, 1>), grid, block, 0, stream, p);
    } else {
      if (hpi == 4) hipLaunchKernelGGL((dkdv_kernel<64, 4>), grid, block, 0, stream, p);
      else if (hpi == 2) hipLaunchKernelGGL((dkdv_kernel<64, 2>), grid, block, 0, stream, p);
      else hipLaunchKernelGGL((dkdv_kernel<64, 1>), grid, block, 0, stream, p);
    }
  }
  const int hb = dq_heads_per_item(p.group);
  BwdParams a = p;
  a.n_hb = p.group / hb;
  const long long nblk_q = (long long)p.n_qtiles_dq * p.hkv * a.n_hb;
  if (nblk_q > 0) {
    if (nblk_q > 0x7fffffffLL) return hipErrorInvalidValue;
    dim3 grid((unsigned)nblk_q), block(512);
    KernelTimer timer(KC_DQ, stream);
    if (d == 128) {
      if (hb == 8) hipLaunchKernelGGL((dq_kernel<128, 1, 8>), grid, block, 0, stream, a);
      else if (hb == 4) hipLaunchKernelGGL((dq_kernel<128, 2, 4>), grid, block, 0, stream, a);
      else if (hb == 2) hipLaunchKernelGGL((dq_kernel<128, 4, 2>), grid, block, 0, stream, a);
      else hipLaunchKernelGGL((dq_kernel<128, 8, 1>), grid, block, 0, stream, a);
    } else {
      if (hb == 8) hipLaunchKernelGGL((dq_kernel<64, 1, 8>), grid, block, 0, stream, a);
      else if (hb == 4) hipLaunchKernelGGL((dq_kernel<64, 2, 4>), grid, block, 0, stream, a);
      else if (hb == 2) hipLaunchKernelGGL((dq_kernel<64, 4, 2>), grid, block, 0, stream, a);
      else hipLaunchKernelGGL((dq_kernel<64, 8, 1>), grid, block, 0, stream, a);
    }
  }
  return hipGetLastError();
}

}  // namespace docmask
