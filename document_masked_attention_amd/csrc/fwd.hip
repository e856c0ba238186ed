// Forward kernel: document-masked attention, O and LSE, bf16 in / fp32 math.
//
// Computes, for every local query row i and head h (FlashCP paper, section 2.1:
// a query sees the keys of its own document that are not after it),
//   LSE_ih = ln sum_j exp(scale q_ih . k_j),  O_ih = sum_j exp(scale q_ih . k_j - LSE_ih) v_j
// over the allowed keys j in [kv_lo, kv_hi), with an online softmax over KV
// tiles (the row maximum and exponential sum of the production guide's
// "Core Principle: Split Q, Circulate KV", here applied tile by tile).
//
// Work item = (Q tile of 32*RB rows, KV head, block of HB query heads of that
// KV head's group); 4 waves of 64 lanes, wave w owns 32 rows x 1 head.  The
// scheduler's per-Q-tile KV range skips fully masked tiles; the mask is applied
// only on PARTIAL tiles.  K and V tiles (64 keys) are staged in LDS and shared
// by the 4 waves (GQA heads and/or row blocks).
//
// MFMA formulation (v_mfma_f32_32x32x16_bf16, wave64):
//   S^T[key][q] = K Q^T   (A = K rows from LDS, B = Q held in registers)
//   O^T[d][q]  += V^T P^T (A = V^T from LDS, B = P^T straight from the S^T
//                          accumulators, converted to bf16)
// With keys on the accumulator rows, a query's scores sit in one lane pair
// (lane and lane^32), so row max/sum are in-register plus one cross-half swap.
// The accumulator row order of S^T is {0-3, 8-11 | 4-7, 12-15} per 16 keys for
// the two lane halves; the V^T operand is gathered in that same key order from
// the row-major V tile with LDS transpose reads (ds_read_b64_tr_b16).
// K/V tiles are double-buffered in LDS (filled by direct global-to-LDS loads)
// with one barrier per tile; after a tile's softmax the MFMAs of the next
// tile's S^T and of this tile's PV run back to back, while the other wave on
// the SIMD works on its softmax.
#include "kernels.h"

#include <type_traits>

namespace docmask {

// Softmax reference.  A tile's exponentials are first formed against the
// running reference m (no tile maximum is taken); the tile is accepted when no
// lane's sum of them exceeds kAcceptSum, so every accepted value is at most
// 2^15 (rounded to bf16 with its usual 8-bit precision, far from fp32
// overflow in O and the row sum).  Otherwise (and while some row of the wave
// has no reference yet) the tile's maximum is taken, the reference raised to
// it, O and the sum rescaled, and the exponentials formed again.  Any
// reference gives the same result after the final division by the row sum.
constexpr float kAcceptSum = 32768.f;

template <int D, int RB, int HB>
__global__ __launch_bounds__(256, 2) void fwd_kernel(FwdParams p) {
  static_assert(RB * HB == 4, "four waves per workgroup");
  constexpr int BK = kFwdBK;
  constexpr int KSTR = D + 8;           // K row stride (bf16): 16-byte row reads hit distinct banks
  constexpr int VSTR = D + 32;          // V row stride: transpose reads of 4 rows hit distinct banks
  constexpr int CPK = D / 8;            // 16-byte chunks per key row
  constexpr int KCH = KSTR / 8, VCH = VSTR / 8;       // 16-byte slots per LDS row (data + padding)
  constexpr int WLK = BK * KCH / 64, WLV = BK * VCH / 64;   // direct loads (64 slots) per tile
  static_assert(BK * KCH % 64 == 0 && BK * VCH % 64 == 0, "tiles are whole direct loads");
  constexpr int DPK = (WLK + 3) / 4, DPV = (WLV + 3) / 4;   // per wave (the last may be idle)
  constexpr int NKS = D / 16;           // k-steps of QK^T
  constexpr int NDB = D / 32;           // 32-wide d blocks of O
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][BK * KSTR];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[2][BK * VSTR];

  if (p.err[0]) return;

  const WorkItem wi = map_work(blockIdx.x, p.n_qtiles, p.hkv, p.n_hb, p.xcd_cluster);
  const int kvh = wi.kvh, hb = wi.hb;
  const int tile = min(max(p.lpt[wi.rank], 0), p.n_qtiles - 1);
  const int32_t* pl = p.plan + (size_t)tile * QP_WORDS;
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
  // allowed keys of this row: [a_lo, a_lo + a_w] (global positions); empty rows never match
  int a_lo = 0x40000000, a_w = 0;
  if (row_ok) {
    const int lo = max(doc_start(p.cu, p.n_docs, gi), p.kv_lo), hi = min(gi, p.kv_hi - 1);
    if (hi >= lo) { a_lo = lo; a_w = hi - lo; }
  }

  bf16x8 qf[NKS];            // Q operand of this lane: row qr, d = 16 s + 8 hh .. +8, k-step s

  f32x16 oacc[NDB];
#pragma unroll
  for (int b = 0; b < NDB; ++b) oacc[b] = f32x16{};
  float m_run = -INFINITY;   // softmax reference (scale*log2(e) units)
  float l_run = 0.f;         // this lane half's share of the exp-sum

  const int tkv = p.kv_hi - p.kv_lo;
  const size_t kv_rstride = (size_t)p.hkv * D;
  const uint16_t* kbase = p.k + (size_t)kvh * D;
  const uint16_t* vbase = p.v + (size_t)kvh * D;

  // K and V tiles reach LDS by direct global-to-LDS loads (no staging
  // registers; completion by this wave's vmcnt, then a barrier).  A tile of
  // padded rows is a run of 16-byte slots; direct load j (of a wave: j = wave
  // + 4 i) fills slots 64 j .. 64 j + 63, and lane l's slot 64 j + l is row
  // q / CH, chunk q % CH (q = 64 j + l).  Padding slots load any real chunk
  // of the row (never read).  The tile base is wave-uniform; each lane adds a
  // 32-bit byte offset.  Padding keys of a ragged last tile read the last real
  // row instead: their scores are always masked (P = 0 exactly), so any
  // finite K/V row will do.
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t row_bytes = (uint32_t)(kv_rstride * sizeof(uint16_t));
  uint32_t krow[DPK], kchk[DPK], vrow[DPV], vchk[DPV];
#pragma unroll
  for (int i = 0; i < DPK; ++i) {
    const int q = (wave_u + 4 * i) * 64 + lane;
    krow[i] = (uint32_t)(q / KCH) * row_bytes;
    kchk[i] = 16u * (uint32_t)min(q % KCH, CPK - 1);
  }
#pragma unroll
  for (int i = 0; i < DPV; ++i) {
    const int q = (wave_u + 4 * i) * 64 + lane;
    vrow[i] = (uint32_t)(q / VCH) * row_bytes;
    vchk[i] = 16u * (uint32_t)min(q % VCH, CPK - 1);
  }
  // full tiles: uniform tile base + precomputed lane offsets; the ragged last
  // tile clamps the row part of the offset (a wave-uniform branch)
  auto issue_rows = [&](const uint16_t* base, int kt, uint16_t* lds, const uint32_t* row, const uint32_t* chk,
                        auto dp_c, auto wl_c) __attribute__((always_inline)) {
    constexpr int DP = decltype(dp_c)::value, WL = decltype(wl_c)::value;
    const uint16_t* tb = base + (size_t)kt * BK * kv_rstride;
    // load i of every wave exists when 4 (i + 1) <= WL (no branch); only the
    // last one may be idle on some waves
    auto one = [&](auto ic, uint32_t off) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value;
      if constexpr (4 * (i + 1) <= WL) lds_dma16_s(tb, off, lds + (wave_u + 4 * i) * 512);
      else if (wave_u + 4 * i < WL) lds_dma16_s(tb, off, lds + (wave_u + 4 * i) * 512);
    };
    if ((kt + 1) * BK <= tkv) {
      static_for<DP>([&](auto ic) __attribute__((always_inline)) {
        constexpr int i = decltype(ic)::value;
        one(ic, row[i] + chk[i]);
      });
    } else {
      const uint32_t lim = (uint32_t)(tkv - 1 - kt * BK) * row_bytes;
      static_for<DP>([&](auto ic) __attribute__((always_inline)) {
        constexpr int i = decltype(ic)::value;
        one(ic, min(row[i], lim) + chk[i]);
      });
    }
  };
  auto issue_k = [&](int kt, uint16_t* lds) __attribute__((always_inline)) {
    issue_rows(kbase, kt, lds, krow, kchk, std::integral_constant<int, DPK>{}, std::integral_constant<int, WLK>{});
  };
  auto issue_v = [&](int kt, uint16_t* lds) __attribute__((always_inline)) {
    issue_rows(vbase, kt, lds, vrow, vchk, std::integral_constant<int, DPV>{}, std::integral_constant<int, WLV>{});
  };
  // transpose-read source address of this lane inside a V tile (see lds_read_tr16)
  const int i16 = lane & 15;
  const int vt_off = (4 * hh + (i16 >> 2)) * VSTR + 16 * ((lane >> 4) & 1) + 4 * (i16 & 3);

  // S^T = K Q^T for the two 32-key blocks of the tile held in K buffer kb_
  auto compute_s = [&](const uint16_t* kl, f32x16 (&sacc)[2]) __attribute__((always_inline)) {
    constexpr int NT = 2 * NKS, PFS = 4;
    sacc[0] = f32x16{};
    sacc[1] = f32x16{};
    bf16x8 op[NT];
    auto load = [&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value;
      op[i] = *reinterpret_cast<const bf16x8*>(&kl[(32 * (i % 2) + ln) * KSTR + 16 * (i / 2) + 8 * hh]);
    };
    static_for<PFS>([&](auto ic) __attribute__((always_inline)) { load(ic); });
    static_for<NT>([&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value;
      if constexpr (i + PFS < NT) load(std::integral_constant<int, i + PFS>{});
      sacc[i % 2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[i], qf[i / 2], sacc[i % 2], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // Pipeline over the n tiles (index u = kt - kt_lo): K tile u lives in
  // k_lds[u & 1] and V tile u in v_lds[u & 1].  Step u computes S(u + 1) right
  // after the softmax of tile u, so K is staged two tiles ahead and V one.
  const int n = kt_hi - kt_lo;
  f32x16 s_cur[2];
  if (n > 0) {
    issue_k(kt_lo, k_lds[0]);
    issue_v(kt_lo, v_lds[0]);
    if (n > 1) issue_k(kt_lo + 1, k_lds[1]);
  }
  // the first tiles are in flight while the Q operands load
#pragma unroll
  for (int s = 0; s < NKS; ++s) {
    if (row_ok) qf[s] = *reinterpret_cast<const bf16x8*>(p.q + o_off + 16 * s + 8 * hh);
    else qf[s] = bf16x8{};
  }
  if (n > 0) {
    wait_vmem();
    __syncthreads();
    compute_s(k_lds[0], s_cur);
    __syncthreads();                  // every wave has read K tile 0 before it is overwritten
  }
  // the Q operands are in registers before any tile loads are in flight (a
  // first use inside the loop would wait for all of them)
#pragma unroll
  for (int s = 0; s < NKS; ++s) asm volatile("" ::"v"(qf[s]));
  // One pipeline step; `has_next` is a compile-time flag so that the steady-state
  // body has no branches between the next tile's MFMAs and this tile's softmax.
  auto step = [&](int u, auto has_next_c) __attribute__((always_inline)) {
    constexpr bool has_next = decltype(has_next_c)::value;
    const int kt = kt_lo + u;
    if (has_next) {
      // K tile u + 2 (if any) into the buffer K tile u left, V tile u + 1 into
      // the one V tile u - 1 left; in flight during this tile's math
      if (kt + 2 < kt_hi) issue_k(kt + 2, k_lds[u & 1]);
      issue_v(kt + 1, v_lds[(u + 1) & 1]);
    }

    // document mask on PARTIAL tiles and on the ragged last tile (its padding
    // keys lie beyond kv_hi even when every real pair is allowed)
    if (kt < kt_flo || kt >= kt_fhi || (kt + 1) * BK > tkv) {
      const int rel0 = p.kv_lo + kt * BK + 4 * hh - a_lo;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const unsigned rel = (unsigned)(rel0 + 32 * kb + 8 * (r >> 2) + (r & 3));
          if (rel > (unsigned)a_w) s_cur[kb][r] = -INFINITY;
        }
    }
    // online softmax (base 2) against the running reference (see kAcceptSum)
    float rs = 0.f;
    bf16x8 pf[4];
    auto exps = [&](float m_use) __attribute__((always_inline)) {
      float r_ = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[kb][r], p.scale_log2, -m_use));
          const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[kb][r + 1], p.scale_log2, -m_use));
          r_ += e0 + e1;
          const bf16x2 two = __builtin_convertvector(f32x2{e0, e1}, bf16x2);
          pf[2 * kb + (r >> 3)][r & 7] = two[0];
          pf[2 * kb + (r >> 3)][(r & 7) + 1] = two[1];
        }
      return r_;
    };
    bool redo = true;
    if (!__any(m_run == -INFINITY)) {
      rs = exps(m_run);
      redo = __any(rs > kAcceptSum);
    }
    if (redo) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s_cur[kb][r]);
      const float m_new = fmaxf(m_run, pair_max32(mx) * p.scale_log2);
      if (__any(m_new > m_run)) {
        const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int b = 0; b < NDB; ++b) oacc[b] *= alpha;
      }
      rs = exps(m_run == -INFINITY ? 0.f : m_run);
    }
    l_run += rs;
    // S of the next tile, into the registers this tile's softmax has just
    // read; those MFMAs and this tile's PV run back to back, at raised wave
    // priority so that the matrix core is fed first while the other wave of
    // the SIMD runs its softmax
    __builtin_amdgcn_s_setprio(1);
    if (has_next) compute_s(k_lds[(u + 1) & 1], s_cur);

    // O^T += V^T P^T, 16 keys per step; V^T comes from the row-major V tile
    // through transpose reads, in the accumulator's permuted key order
    const uint16_t* vl = v_lds[u & 1];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int b = 0; b < NDB; ++b) {
        const uint16_t* vp = vl + vt_off + 16 * s * VSTR + 32 * b;
        const bf16x8 vf = tr_operand(vp, vp + 8 * VSTR);
        oacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[s], oacc[b], 0, 0, 0);
      }
    __builtin_amdgcn_s_setprio(0);
    if (has_next) {
      wait_vmem();
      __syncthreads();
    }
  };
  for (int u = 0; u + 1 < n; ++u) step(u, std::true_type{});
  if (n > 0) step(n - 1, std::false_type{});

  // epilogue: normalise, write O (bf16, or float32 partials) and LSE (natural log)
  const float l_tot = pair_sum32(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (row_ok && p.o32) {
#pragma unroll
    for (int b = 0; b < NDB; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 val = make_float4(oacc[b][4 * g] * inv, oacc[b][4 * g + 1] * inv, oacc[b][4 * g + 2] * inv,
                                       oacc[b][4 * g + 3] * inv);
        *reinterpret_cast<float4*>(p.o32 + o_off + 32 * b + 8 * g + 4 * hh) = val;
      }
  } else if (row_ok) {
#pragma unroll
    for (int b = 0; b < NDB; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const bf16x2 lo2 = __builtin_convertvector(f32x2{oacc[b][4 * g] * inv, oacc[b][4 * g + 1] * inv}, bf16x2);
        const bf16x2 hi2 = __builtin_convertvector(f32x2{oacc[b][4 * g + 2] * inv, oacc[b][4 * g + 3] * inv}, bf16x2);
        uint2 val;
        val.x = *reinterpret_cast<const uint32_t*>(&lo2);
        val.y = *reinterpret_cast<const uint32_t*>(&hi2);
        *reinterpret_cast<uint2*>(p.o + o_off + 32 * b + 8 * g + 4 * hh) = val;
      }
  }
  if (row_ok) {
    if (hh == 0)
      p.lse[(size_t)head * p.tq + l_row0 + qr] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------- host side
hipError_t launch_fwd(const FwdParams& p, int d, hipStream_t stream) {
  // rows x heads per workgroup: as many GQA heads as divide the group (<= 4)
  const int hb = (p.group % 4 == 0) ? 4 : (p.group % 2 == 0 ? 2 : 1);
  FwdParams a = p;
  a.n_hb = p.group / hb;
  const long long nblk = (long long)p.n_qtiles * p.hkv * a.n_hb;
  if (nblk == 0) return hipSuccess;
  if (nblk > 0x7fffffffLL) return hipErrorInvalidValue;
  dim3 grid((unsigned)nblk), block(256);
  KernelTimer timer(KC_FWD, stream);
  if (d == 128) {
    if (hb == 4) hipLaunchKernelGGL((fwd_kernel<128, 1, 4>), grid, block, 0, stream, a);
    else if (hb == 2) hipLaunchKernelGGL((fwd_kernel<128, 2, 2>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((fwd_kernel<128, 4, 1>), grid, block, 0, stream, a);
  } else {
    if (hb == 4) hipLaunchKernelGGL((fwd_kernel<64, 1, 4>), grid, block, 0, stream, a);
    else if (hb == 2) hipLaunchKernelGGL((fwd_kernel<64, 2, 2>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((fwd_kernel<64, 4, 1>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

int fwd_rows_per_tile(int group) {
  const int hb = (group % 4 == 0) ? 4 : (group % 2 == 0 ? 2 : 1);
  return 32 * (4 / hb);
}

}  // namespace docmask
