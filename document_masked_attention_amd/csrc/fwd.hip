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
// MFMA formulation (v_mfma_f32_16x16x32_bf16, wave64; a wave's 32 rows are
// two 16-row halves):
//   S^T[key][q] = K Q^T   (A = 16 K rows from LDS, B = Q held in registers;
//                          every K operand feeds both halves)
//   O^T[d][q]  += V^T P^T (A = V^T from LDS, B = P^T straight from the S^T
//                          accumulators, converted to bf16)
// Lane l holds query row l mod 16 of each half and, per 16 keys, the four
// keys 4 (l / 16) .. +3; a row's scores sit in four lanes (l mod 16 equal),
// joined only for the tile maximum and the final sum.  P^T of 32 keys is the B
// operand in the key order {4 g .. 4 g + 3, 16 + 4 g .. 16 + 4 g + 3} for lane
// group g; the V^T operand is gathered in that same order from the row-major V
// tile with LDS transpose reads (ds_read_b64_tr_b16).  Against the 32 x 32 x 16
// instruction this moves half the accumulator data per product, which measured
// ~2% faster here at the same LDS traffic (the matrix cores take less power per
// product).
// K/V tiles are double-buffered in LDS (filled by direct global-to-LDS loads)
// with one barrier per tile; after a tile's softmax the MFMAs of the next
// tile's S^T and of this tile's PV run back to back as one stream of
// prefetched operands, while the other wave on the SIMD works on its softmax.
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
  using L = SwzTile<D>;                 // K and V tile layout: 16-byte row reads and transpose reads on distinct banks
  constexpr int CPK = D / 8;            // 16-byte chunks per key row
  constexpr int RE = L::kRowElems;      // LDS row length (bf16): D = 128 unpadded, D = 64 padded to 80
  constexpr int SK = RE / 8;            // 16-byte slots per LDS row
  constexpr int WL = BK * SK / 64;      // direct loads (64 slots) per K or V tile
  static_assert(BK * SK % 64 == 0, "tiles are whole direct loads");
  constexpr int DP = (WL + 3) / 4;      // per wave (the last may be idle)
  constexpr int NKS = D / 32;           // 32-wide k-steps of QK^T
  constexpr int NDB = D / 16;           // 16-wide d blocks of O
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][L::kElems(BK)];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[2][L::kElems(BK)];

  if (p.err[0]) return;

  const WorkItem wi = map_work(blockIdx.x, p.n_qtiles, p.hkv, p.n_hb, p.xcd_cluster);
  const int kvh = wi.kvh, hb = wi.hb;
  const int tile = min(max(p.lpt[wi.rank], 0), p.n_qtiles - 1);
  const int32_t* pl = p.plan + (size_t)tile * QP_WORDS;
  const int l_row0 = pl[QP_LROW0], g_row0 = pl[QP_GROW0], nrows = pl[QP_NROWS];
  const int kt_lo = pl[QP_KT_LO], kt_flo = pl[QP_KT_FLO], kt_fhi = pl[QP_KT_FHI], kt_hi = pl[QP_KT_HI];

  // Lane l works on rows 16 r + (l mod 16) of the wave's 32 (r = 0, 1: the two
  // 16-row halves) and, in every 16 x 16 accumulator, on the four rows of
  // group g = l / 16.
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, g4 = lane >> 4, i16 = lane & 15;
  const int rb = wave / HB, hs = wave % HB;
  const int head = kvh * p.group + hb * HB + hs;
  int qr[2], a_lo[2], a_w[2];
  bool row_ok[2];
  size_t o_off[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    qr[r] = 32 * rb + 16 * r + i16;
    row_ok[r] = qr[r] < nrows;
    o_off[r] = ((size_t)(l_row0 + qr[r]) * p.hq + head) * D;
    // allowed keys of this row: [a_lo, a_lo + a_w] (global positions); empty rows never match
    a_lo[r] = 0x40000000;
    a_w[r] = 0;
    if (row_ok[r]) {
      const int gi = g_row0 + qr[r];
      const int lo = max(doc_start(p.cu, p.n_docs, gi), p.kv_lo), hi = min(gi, p.kv_hi - 1);
      if (hi >= lo) { a_lo[r] = lo; a_w[r] = hi - lo; }
    }
  }

  bf16x8 qf[2][NKS];         // Q operand: row 16 r + l mod 16, d = 32 s + 8 g .. +8, k-step s

  f32x4 oacc[NDB][2];        // O^T: d = 16 b + 4 g + e, row 16 r + l mod 16
#pragma unroll
  for (int b = 0; b < NDB; ++b) oacc[b][0] = oacc[b][1] = f32x4{};
  float m_run[2] = {-INFINITY, -INFINITY};   // softmax reference per row (scale*log2(e) units)
  float l_run[2] = {0.f, 0.f};               // this lane's share of the row's exp-sum

  const int tkv = p.kv_hi - p.kv_lo;
  const size_t kv_rstride = (size_t)p.hkv * D;
  const uint16_t* kbase = p.k + (size_t)kvh * D;
  const uint16_t* vbase = p.v + (size_t)kvh * D;
  // K and V tiles reach LDS by direct global-to-LDS loads (no staging
  // registers; completion by this wave's vmcnt, then a barrier).  A tile is a
  // run of 16-byte slots, RE / 8 per row; direct load j (of a wave: j = wave
  // + 4 i) fills slots 64 j .. 64 j + 63, and lane l's slot q = 64 j + l is
  // position q % SK of row q / SK, which holds the row's chunk of that
  // position under the tile's swizzle (D = 128), or the same chunk (D = 64;
  // its padding slots load any real chunk of the row, never read).  K and V
  // tiles share the layout and so the lane offsets.  The tile base is
  // wave-uniform; each lane adds a 32-bit byte offset.  Padding keys of a
  // ragged last tile read the last real row instead: their scores are always
  // masked (P = 0 exactly), so any finite K/V row will do.
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t row_bytes = (uint32_t)(kv_rstride * sizeof(uint16_t));
  uint32_t lrow[DP], lchk[DP];
#pragma unroll
  for (int i = 0; i < DP; ++i) {
    const int q = (wave_u + 4 * i) * 64 + lane, r = q / SK, pos = q % SK;
    lrow[i] = (uint32_t)r * row_bytes;
    lchk[i] = 16u * (uint32_t)(D == 128 ? (pos ^ L::f(r)) : min(pos, CPK - 1));
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
    issue_rows(kbase, kt, lds, lrow, lchk, std::integral_constant<int, DP>{}, std::integral_constant<int, WL>{});
  };
  auto issue_v = [&](int kt, uint16_t* lds) __attribute__((always_inline)) {
    issue_rows(vbase, kt, lds, lrow, lchk, std::integral_constant<int, DP>{}, std::integral_constant<int, WL>{});
  };
  // LDS element offsets of this lane's reads in a tile.  K rows (S^T's A
  // operand): row 16 kb + (l mod 16), d = 32 s + 8 g .. +8, one offset per
  // k-step s (the swizzle repeats every 16 rows, so block kb adds 16 kb rows).
  // V^T (transpose reads, see lds_read_tr16): as the supplier of group g,
  // lane l names row 4 g + (l mod 16) / 4 and column 16 b + 4 (l mod 4), so
  // that lane l of the group receives rows 4 g .. 4 g + 3 of column
  // 16 b + (l mod 16); one offset per 16-column block b, the 32-key half t
  // and the second read (16 rows on) adding whole rows.
  int ko[NKS], vto[NDB];
#pragma unroll
  for (int s = 0; s < NKS; ++s) ko[s] = L::off(i16, 32 * s + 8 * g4);
#pragma unroll
  for (int b = 0; b < NDB; ++b) vto[b] = L::off(4 * g4 + (i16 >> 2), 16 * b + 4 * (i16 & 3));

  // S^T = K Q^T over the tile held in K buffer kl: 4 blocks of 16 keys x the
  // two 16-row halves, D / 32 k-steps; every K operand feeds both halves
  auto compute_s = [&](const uint16_t* kl, f32x4 (&sacc)[4][2]) __attribute__((always_inline)) {
    constexpr int NT = 4 * NKS, PFS = 4;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) sacc[kb][0] = sacc[kb][1] = f32x4{};
    bf16x8 op[NT];
    auto load = [&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value;
      op[i] = *reinterpret_cast<const bf16x8*>(&kl[ko[i / 4] + 16 * (i % 4) * RE]);
    };
    static_for<PFS>([&](auto ic) __attribute__((always_inline)) { load(ic); });
    static_for<NT>([&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value;
      if constexpr (i + PFS < NT) load(std::integral_constant<int, i + PFS>{});
      sacc[i % 4][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op[i], qf[0][i / 4], sacc[i % 4][0], 0, 0, 0);
      sacc[i % 4][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op[i], qf[1][i / 4], sacc[i % 4][1], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // Pipeline over the n tiles (index u = kt - kt_lo): K tile u lives in
  // k_lds[u & 1] and V tile u in v_lds[u & 1].  Step u computes S(u + 1) right
  // after the softmax of tile u, so K is staged two tiles ahead and V one.
  const int n = kt_hi - kt_lo;
  f32x4 s_cur[4][2];
  if (n > 0) {
    issue_k(kt_lo, k_lds[0]);
    issue_v(kt_lo, v_lds[0]);
    if (n > 1) issue_k(kt_lo + 1, k_lds[1]);
  }
  // the first tiles are in flight while the Q operands load
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      if (row_ok[r]) qf[r][s] = *reinterpret_cast<const bf16x8*>(p.q + o_off[r] + 32 * s + 8 * g4);
      else qf[r][s] = bf16x8{};
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
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int s = 0; s < NKS; ++s) asm volatile("" ::"v"(qf[r][s]));
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
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int rel0 = p.kv_lo + kt * BK + 4 * g4 - a_lo[r];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const unsigned rel = (unsigned)(rel0 + 16 * kb + e);
            if (rel > (unsigned)a_w[r]) s_cur[kb][r][e] = -INFINITY;
          }
      }
    }
    // online softmax (base 2) against the running reference (see kAcceptSum).
    // P^T of key block pair (2 t, 2 t + 1) is the B operand of k-step t of
    // PV, in the key order {4 g .. 4 g + 3, 16 + 4 g .. 16 + 4 g + 3}.
    float rs[2] = {0.f, 0.f};
    bf16x8 pf[2][2];
    auto exps = [&](const float (&m_use)[2]) __attribute__((always_inline)) {
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        float r_ = 0.f;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int e = 0; e < 4; e += 2) {
            const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[kb][r][e], p.scale_log2, -m_use[r]));
            const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[kb][r][e + 1], p.scale_log2, -m_use[r]));
            r_ += e0 + e1;
            const bf16x2 two = __builtin_convertvector(f32x2{e0, e1}, bf16x2);
            pf[kb >> 1][r][4 * (kb & 1) + e] = two[0];
            pf[kb >> 1][r][4 * (kb & 1) + e + 1] = two[1];
          }
        rs[r] = r_;
      }
    };
    bool redo = true;
    if (!__any(m_run[0] == -INFINITY || m_run[1] == -INFINITY)) {
      exps(m_run);
      redo = __any(rs[0] > kAcceptSum || rs[1] > kAcceptSum);
    }
    if (redo) {
      float m_new[2];
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int e = 0; e < 4; ++e) mx = fmaxf(mx, s_cur[kb][r][e]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));        // the row's four lanes (g = 0 .. 3)
        m_new[r] = fmaxf(m_run[r], pair_max32(mx) * p.scale_log2);
      }
      if (__any(m_new[0] > m_run[0] || m_new[1] > m_run[1])) {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const float alpha = m_new[r] == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run[r] - m_new[r]);
          m_run[r] = m_new[r];
          l_run[r] *= alpha;
#pragma unroll
          for (int b = 0; b < NDB; ++b) oacc[b][r] *= alpha;
        }
      }
      const float m_use[2] = {m_run[0] == -INFINITY ? 0.f : m_run[0], m_run[1] == -INFINITY ? 0.f : m_run[1]};
      exps(m_use);
    }
    l_run[0] += rs[0];
    l_run[1] += rs[1];
    // One stream of MFMA operands, each feeding both row halves: the K
    // fragments of the next tile's S (into the registers this tile's softmax
    // has just read), then the V^T fragments of this tile's PV (32 keys per
    // k-step, from the row-major V tile through transpose reads in P^T's key
    // order).  Every fragment is read PF slots ahead, across the S / PV
    // boundary too.  The block runs at raised wave priority so that the
    // matrix core is fed first while the other wave of the SIMD runs its
    // softmax.
    __builtin_amdgcn_s_setprio(1);
    {
      constexpr int NS = has_next ? 4 * NKS : 0, NSLOT = NS + 2 * NDB, PF = 4;
      const uint16_t* kl = k_lds[(u + 1) & 1];
      const uint16_t* vl = v_lds[u & 1];
      if (has_next) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) s_cur[kb][0] = s_cur[kb][1] = f32x4{};
      }
      bf16x8 opr[NSLOT];
      auto load = [&](auto ic) __attribute__((always_inline)) {
        constexpr int i = decltype(ic)::value;
        if constexpr (i < NS) {
          opr[i] = *reinterpret_cast<const bf16x8*>(&kl[ko[i / 4] + 16 * (i % 4) * RE]);
        } else {
          constexpr int t = (i - NS) / NDB, b = (i - NS) % NDB;
          const uint16_t* vp = vl + vto[b] + 32 * t * RE;
          opr[i] = tr_operand(vp, vp + 16 * RE);
        }
      };
      static_for<PF>([&](auto ic) __attribute__((always_inline)) { load(ic); });
      static_for<NSLOT>([&](auto ic) __attribute__((always_inline)) {
        constexpr int i = decltype(ic)::value;
        if constexpr (i + PF < NSLOT) load(std::integral_constant<int, i + PF>{});
        if constexpr (i < NS) {
          s_cur[i % 4][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(opr[i], qf[0][i / 4], s_cur[i % 4][0], 0, 0, 0);
          s_cur[i % 4][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(opr[i], qf[1][i / 4], s_cur[i % 4][1], 0, 0, 0);
        } else {
          constexpr int t = (i - NS) / NDB, b = (i - NS) % NDB;
          oacc[b][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(opr[i], pf[t][0], oacc[b][0], 0, 0, 0);
          oacc[b][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(opr[i], pf[t][1], oacc[b][1], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      });
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
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const float l_half = l_run[r] + __shfl_xor(l_run[r], 16);
    const float l_tot = pair_sum32(l_half);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (row_ok[r] && p.o32) {
#pragma unroll
      for (int b = 0; b < NDB; ++b) {
        const float4 val = make_float4(oacc[b][r][0] * inv, oacc[b][r][1] * inv, oacc[b][r][2] * inv,
                                       oacc[b][r][3] * inv);
        *reinterpret_cast<float4*>(p.o32 + o_off[r] + 16 * b + 4 * g4) = val;
      }
    } else if (row_ok[r]) {
#pragma unroll
      for (int b = 0; b < NDB; ++b) {
        const bf16x2 lo2 = __builtin_convertvector(f32x2{oacc[b][r][0] * inv, oacc[b][r][1] * inv}, bf16x2);
        const bf16x2 hi2 = __builtin_convertvector(f32x2{oacc[b][r][2] * inv, oacc[b][r][3] * inv}, bf16x2);
        uint2 val;
        val.x = *reinterpret_cast<const uint32_t*>(&lo2);
        val.y = *reinterpret_cast<const uint32_t*>(&hi2);
        *reinterpret_cast<uint2*>(p.o + o_off[r] + 16 * b + 4 * g4) = val;
      }
    }
    if (row_ok[r] && g4 == 0)
      p.lse[(size_t)head * p.tq + l_row0 + qr[r]] = l_tot > 0.f ? (m_run[r] + __log2f(l_tot)) * kLn2 : -INFINITY;
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
