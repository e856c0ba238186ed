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
// the two lane halves; V^T is stored in LDS in that same permuted key order so
// each lane fetches its 8 keys with one 16-byte read.
#include "kernels.h"

namespace docmask {

__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) { return (a & 0xffffu) | (b << 16); }
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xffff0000u); }

// Position (in units of 4 keys) of key group kg inside a 64-key V^T row: the
// two middle 4-key blocks of every 16 keys are swapped.
__device__ __forceinline__ int vt_pos4(int kg) { return (kg & ~3) | ((kg & 1) << 1) | ((kg >> 1) & 1); }

template <int D, int RB, int HB>
__global__ __launch_bounds__(256, 2) void fwd_kernel(FwdParams p) {
  static_assert(RB * HB == 4, "four waves per workgroup");
  constexpr int BK = kFwdBK;
  constexpr int KSTR = D + 8;           // K row stride in LDS (bf16 elements)
  constexpr int VSTR = BK + 8;          // V^T row stride
  constexpr int CPK = D / 8;            // 16-byte chunks per key row
  constexpr int KPP = 256 / CPK;        // keys per load pass
  constexpr int KPASS = BK / KPP;
  constexpr int VUNITS = 16 * CPK;      // (4 keys x 8 d) units per V tile
  constexpr int NKS = D / 16;           // k-steps of QK^T
  constexpr int NDB = D / 32;           // 32-wide d blocks of O
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[BK * KSTR];
  __shared__ __attribute__((aligned(16))) uint16_t vt_lds[D * VSTR];

  if (p.err[0]) return;

  const int w = xcd_remap(blockIdx.x, gridDim.x, p.xcd_cluster);
  const int per_tile = p.hkv * p.n_hb;
  const int rank = w / per_tile;
  const int rem = w - rank * per_tile;
  const int kvh = rem / p.n_hb;
  const int hb = rem - kvh * p.n_hb;
  const int tile = min(max(p.lpt[rank], 0), p.n_qtiles - 1);
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
  const int dsi = row_ok ? doc_start(p.cu, p.n_docs, gi) : 0;
  const size_t o_off = ((size_t)(l_row0 + qr) * p.hq + head) * D;

  // Q operand of this lane: row qr, d = 16 s + 8 hh .. +8, for every k-step s.
  bf16x8 qf[NKS];
#pragma unroll
  for (int s = 0; s < NKS; ++s) {
    if (row_ok) qf[s] = *reinterpret_cast<const bf16x8*>(p.q + o_off + 16 * s + 8 * hh);
    else qf[s] = bf16x8{};
  }

  f32x16 oacc[NDB];
#pragma unroll
  for (int b = 0; b < NDB; ++b) oacc[b] = f32x16{};
  float m_run = -INFINITY;   // running max of scale*log2(e)*s
  float l_run = 0.f;         // this lane half's share of the exp-sum

  const int tkv = p.kv_hi - p.kv_lo;
  const size_t kv_rstride = (size_t)p.hkv * D;
  const uint16_t* kbase = p.k + (size_t)kvh * D;
  const uint16_t* vbase = p.v + (size_t)kvh * D;

  // global -> register staging of one K/V tile
  uint4 kreg[KPASS];
  uint4 vreg[4];
  const int kc = tid % CPK, kk0 = tid / CPK;
  const int vkg = tid & 15, vc = tid >> 4;
  auto load_tile = [&](int kt) {
    const int key0 = kt * BK;
#pragma unroll
    for (int pp = 0; pp < KPASS; ++pp) {
      const int key = key0 + kk0 + KPP * pp;
      kreg[pp] = key < tkv ? *reinterpret_cast<const uint4*>(kbase + (size_t)key * kv_rstride + 8 * kc)
                           : make_uint4(0, 0, 0, 0);
    }
    if (tid < VUNITS) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = key0 + 4 * vkg + i;
        vreg[i] = key < tkv ? *reinterpret_cast<const uint4*>(vbase + (size_t)key * kv_rstride + 8 * vc)
                            : make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int pp = 0; pp < KPASS; ++pp)
      *reinterpret_cast<uint4*>(&k_lds[(kk0 + KPP * pp) * KSTR + 8 * kc]) = kreg[pp];
    if (tid < VUNITS) {
      const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&vreg[0]);
      const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&vreg[1]);
      const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&vreg[2]);
      const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&vreg[3]);
      const int col = 4 * vt_pos4(vkg);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int wd = e >> 1;
        uint2 val;
        if (e & 1) { val.x = pack_hi(w0[wd], w1[wd]); val.y = pack_hi(w2[wd], w3[wd]); }
        else       { val.x = pack_lo(w0[wd], w1[wd]); val.y = pack_lo(w2[wd], w3[wd]); }
        *reinterpret_cast<uint2*>(&vt_lds[(8 * vc + e) * VSTR + col]) = val;
      }
    }
  };

  if (kt_lo < kt_hi) load_tile(kt_lo);
  for (int kt = kt_lo; kt < kt_hi; ++kt) {
    __syncthreads();                 // previous tile fully consumed
    store_tile();
    __syncthreads();
    if (kt + 1 < kt_hi) load_tile(kt + 1);

    // S^T = K Q^T for the two 32-key blocks of the tile
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sacc[kb] = f32x16{};
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(&k_lds[(32 * kb + ln) * KSTR + 16 * s + 8 * hh]);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], sacc[kb], 0, 0, 0);
      }
    }
    // document mask on PARTIAL tiles and on the ragged last tile (its padding
    // keys lie beyond kv_hi even when every real pair is allowed)
    if (kt < kt_flo || kt >= kt_fhi || (kt + 1) * BK > tkv) {
      const int key0 = p.kv_lo + kt * BK + 4 * hh;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = key0 + 32 * kb + 8 * (r >> 2) + (r & 3);
          const bool ok = (j >= dsi) && (j <= gi) && (j < p.kv_hi);
          if (!ok) sacc[kb][r] = -INFINITY;
        }
    }
    // online softmax (base 2)
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
    mx = fmaxf(mx, wave_shfl_xor32(mx));
    const float m_new = fmaxf(m_run, mx * p.scale_log2);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][r], p.scale_log2, -m_use));
        sacc[kb][r] = e;
        rs += e;
      }
    l_run = l_run * alpha + rs;
#pragma unroll
    for (int b = 0; b < NDB; ++b) oacc[b] *= alpha;

    // O^T += V^T P^T, 16 keys per step
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int kb = s >> 1, base = 8 * (s & 1);
      bf16x8 pf;
#pragma unroll
      for (int i = 0; i < 8; i += 2) {
        const bf16x2 two = __builtin_convertvector(f32x2{sacc[kb][base + i], sacc[kb][base + i + 1]}, bf16x2);
        pf[i] = two[0];
        pf[i + 1] = two[1];
      }
#pragma unroll
      for (int b = 0; b < NDB; ++b) {
        const bf16x8 vf = *reinterpret_cast<const bf16x8*>(&vt_lds[(32 * b + ln) * VSTR + 16 * s + 8 * hh]);
        oacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, oacc[b], 0, 0, 0);
      }
    }
  }

  // epilogue: normalise, write O (bf16) and LSE (natural log)
  const float l_tot = l_run + wave_shfl_xor32(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (row_ok) {
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
