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
// Work item = (KV tile of 128 keys, KV head); 4 waves, wave w owns keys
// 32w..32w+31 and keeps their K and V rows, dK and dV in registers.  The item
// walks the query tiles (32 rows) that attend its keys -- the scheduler's
// per-KV-tile range -- for every query head of the group, recomputing P from
// the LSE.  MFMA layouts (v_mfma_f32_32x32x16_bf16):
//   S   [q][key]  = Q K^T    (A = Q rows from LDS, B = K in registers)
//   dV^T[d][key] += dO^T P   (A = dO^T from LDS, B = P from the S accumulators)
//   dP  [q][key]  = dO V^T   (A = dO rows from LDS, B = V in registers)
//   dK^T[d][key] += Q^T dS   (A = Q^T from LDS, B = dS from registers)
//   dQ  [q][d]    = dS K     (A = dS staged in LDS, B = K^T from LDS), added to
//                            the float32 dQ with atomics (several KV tiles
//                            contribute to one query row).
// Accumulator rows of S are ordered {0-3, 8-11 | 4-7, 12-15} per 16 queries
// for the two lane halves; Q^T and dO^T are stored in that permuted query
// order so each lane reads its 8 queries with one 16-byte load.
#include "kernels.h"

namespace docmask {

__device__ __forceinline__ uint32_t bpack_lo(uint32_t a, uint32_t b) { return (a & 0xffffu) | (b << 16); }
__device__ __forceinline__ uint32_t bpack_hi(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xffff0000u); }
__device__ __forceinline__ int perm_pos4(int g) { return (g & ~3) | ((g & 1) << 1) | ((g >> 1) & 1); }

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

__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ dst, int64_t n) {
  const int64_t i0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i0 + 4 <= n) *reinterpret_cast<float4*>(dst + i0) = make_float4(0.f, 0.f, 0.f, 0.f);
  else
    for (int64_t i = i0; i < n; ++i) dst[i] = 0.f;
}

template <int D>
__global__ __launch_bounds__(256, 1) void bwd_kernel(BwdParams p) {
  constexpr int BQ = kBwdBQ;            // 32 query rows per step
  constexpr int BK = kBwdBK;            // 128 keys per work item
  constexpr int NKS = D / 16;           // k-steps over d
  constexpr int NDB = D / 32;           // 32-wide d blocks
  constexpr int CPK = D / 8;            // 16-byte chunks per row
  constexpr int RSTR = D + 8;           // row-major Q / dO stride (bf16)
  constexpr int TSTR = BQ + 8;          // Q^T / dO^T stride
  constexpr int SSTR = BK + 8;          // dS stride
  constexpr int KTSTR = BK + 8;         // K^T stride
  constexpr int QUNITS = (BQ / 4) * CPK;   // (4 rows x 8 d) units of one 32-row block
  constexpr int WPD = 4 / NDB;          // waves per d block in the dQ step
  constexpr int KPW = BK / WPD;         // keys each wave sums in the dQ step
  __shared__ __attribute__((aligned(16))) uint16_t q_lds[BQ * RSTR];
  __shared__ __attribute__((aligned(16))) uint16_t do_lds[BQ * RSTR];
  __shared__ __attribute__((aligned(16))) uint16_t qt_lds[D * TSTR];
  __shared__ __attribute__((aligned(16))) uint16_t dot_lds[D * TSTR];
  __shared__ __attribute__((aligned(16))) uint16_t ds_lds[BQ * SSTR];
  __shared__ __attribute__((aligned(16))) uint16_t kt_lds[D * KTSTR];
  __shared__ float lse_lds[BQ], delta_lds[BQ];
  __shared__ int32_t dstart_lds[BQ];

  if (p.err[0]) return;

  const int w = xcd_remap(blockIdx.x, gridDim.x, p.xcd_cluster);
  const int rank = w / p.hkv;
  const int kvh = w - rank * p.hkv;
  const int tile = min(max(p.lpt_kv[rank], 0), p.n_kvtiles - 1);
  const int32_t* kd = p.kvdesc + (size_t)tile * 4;
  const int qt_lo = kd[0], qt_flo = kd[1], qt_fhi = kd[2], qt_hi = kd[3];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, hh = lane >> 5, ln = lane & 31;
  const int tkv = p.kv_hi - p.kv_lo;
  const int key_l = tile * BK + 32 * wave + ln;     // this lane's key, local KV row
  const bool key_ok = key_l < tkv;
  const int key_g = p.kv_lo + key_l;
  const size_t kv_rstride = (size_t)p.hkv * D;

  // K and V rows of this lane's key as MFMA B operands (d = 16 s + 8 hh ..)
  bf16x8 kf[NKS], vf[NKS];
  {
    const uint16_t* kr = p.k + (size_t)key_l * kv_rstride + (size_t)kvh * D + 8 * hh;
    const uint16_t* vr = p.v + (size_t)key_l * kv_rstride + (size_t)kvh * D + 8 * hh;
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      kf[s] = key_ok ? *reinterpret_cast<const bf16x8*>(kr + 16 * s) : bf16x8{};
      vf[s] = key_ok ? *reinterpret_cast<const bf16x8*>(vr + 16 * s) : bf16x8{};
    }
  }
  // K^T of the whole tile in LDS (natural key order) for the dQ step
  for (int u = tid; u < (BK / 4) * CPK; u += 256) {
    const int kg = u % (BK / 4), c = u / (BK / 4);
    uint4 r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kl = tile * BK + 4 * kg + i;
      r[i] = kl < tkv ? *reinterpret_cast<const uint4*>(p.k + (size_t)kl * kv_rstride + (size_t)kvh * D + 8 * c)
                      : make_uint4(0, 0, 0, 0);
    }
    const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&r[0]);
    const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&r[1]);
    const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&r[2]);
    const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&r[3]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint2 val;
      if (e & 1) { val.x = bpack_hi(w0[e >> 1], w1[e >> 1]); val.y = bpack_hi(w2[e >> 1], w3[e >> 1]); }
      else       { val.x = bpack_lo(w0[e >> 1], w1[e >> 1]); val.y = bpack_lo(w2[e >> 1], w3[e >> 1]); }
      *reinterpret_cast<uint2*>(&kt_lds[(8 * c + e) * KTSTR + 4 * kg]) = val;
    }
  }

  f32x16 dkacc[NDB], dvacc[NDB];
#pragma unroll
  for (int b = 0; b < NDB; ++b) { dkacc[b] = f32x16{}; dvacc[b] = f32x16{}; }

  // dQ step assignment: d block and key range of this wave
  const int dq_db = wave / WPD;
  const int dq_k0 = (wave % WPD) * KPW;

  for (int qt = qt_lo; qt < qt_hi; ++qt) {
    const int32_t* pl = p.plan_q + (size_t)qt * QP_WORDS;
    const int l_row0 = pl[QP_LROW0], g_row0 = pl[QP_GROW0], nrows = pl[QP_NROWS];
    // mask PARTIAL tiles and the ragged last KV tile (padding keys beyond kv_hi)
    const bool partial = qt < qt_flo || qt >= qt_fhi || (tile + 1) * BK > tkv;
    for (int hs = 0; hs < p.group; ++hs) {
      const int head = kvh * p.group + hs;
      __syncthreads();                     // previous step done with the LDS buffers
      // stage Q and dO rows (row-major and transposed) and the per-row scalars
      {
        const int which = tid / QUNITS;    // 0: Q, 1: dO (threads beyond 2*QUNITS idle)
        const int u = tid % QUNITS;
        if (which < 2) {
          const uint16_t* src = which == 0 ? p.q : p.d_o;
          uint16_t* rm = which == 0 ? q_lds : do_lds;
          uint16_t* tr = which == 0 ? qt_lds : dot_lds;
          const int rg = u % (BQ / 4), c = u / (BQ / 4);
          uint4 r[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int qr = 4 * rg + i;
            r[i] = qr < nrows ? *reinterpret_cast<const uint4*>(src + ((size_t)(l_row0 + qr) * p.hq + head) * D + 8 * c)
                              : make_uint4(0, 0, 0, 0);
            *reinterpret_cast<uint4*>(&rm[qr * RSTR + 8 * c]) = r[i];
          }
          const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&r[0]);
          const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&r[1]);
          const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&r[2]);
          const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&r[3]);
          const int col = 4 * perm_pos4(rg);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            uint2 val;
            if (e & 1) { val.x = bpack_hi(w0[e >> 1], w1[e >> 1]); val.y = bpack_hi(w2[e >> 1], w3[e >> 1]); }
            else       { val.x = bpack_lo(w0[e >> 1], w1[e >> 1]); val.y = bpack_lo(w2[e >> 1], w3[e >> 1]); }
            *reinterpret_cast<uint2*>(&tr[(8 * c + e) * TSTR + col]) = val;
          }
        }
        if (tid >= 224) {
          const int qr = tid - 224;
          float l2 = INFINITY, dl = 0.f;
          int dsr = 0;
          if (qr < nrows) {
            const float lv = p.lse[(size_t)head * p.tq + l_row0 + qr];
            l2 = lv == -INFINITY ? INFINITY : lv * kLog2e;   // empty row: P = 0
            dl = p.delta[(size_t)head * p.tq + l_row0 + qr];
            dsr = doc_start(p.cu, p.n_docs, g_row0 + qr);
          }
          lse_lds[qr] = l2;
          delta_lds[qr] = dl;
          dstart_lds[qr] = dsr;
        }
      }
      __syncthreads();

      // S = Q K^T (rows = queries, lanes = this wave's keys)
      f32x16 sacc = f32x16{};
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        const bf16x8 qa = *reinterpret_cast<const bf16x8*>(&q_lds[ln * RSTR + 16 * s + 8 * hh]);
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[s], sacc, 0, 0, 0);
      }
      // P = exp2(s * scale * log2e - LSE * log2e); masked pairs and padded rows give 0
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qr = 8 * (r >> 2) + 4 * hh + (r & 3);
        float e = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r], p.scale_log2, -lse_lds[qr]));
        if (partial) {
          const int gi = g_row0 + qr;
          const bool ok = key_ok && qr < nrows && key_g >= dstart_lds[qr] && key_g <= gi;
          if (!ok) e = 0.f;
        }
        sacc[r] = e;
      }
      bf16x8 pb[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
          const bf16x2 two = __builtin_convertvector(f32x2{sacc[8 * ks + i], sacc[8 * ks + i + 1]}, bf16x2);
          pb[ks][i] = two[0];
          pb[ks][i + 1] = two[1];
        }
      // dV^T += dO^T P
#pragma unroll
      for (int b = 0; b < NDB; ++b)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(&dot_lds[(32 * b + ln) * TSTR + 16 * ks + 8 * hh]);
          dvacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[ks], dvacc[b], 0, 0, 0);
        }
      // dP = dO V^T
      f32x16 dpacc = f32x16{};
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&do_lds[ln * RSTR + 16 * s + 8 * hh]);
        dpacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, vf[s], dpacc, 0, 0, 0);
      }
      // dS = P (dP - Delta)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qr = 8 * (r >> 2) + 4 * hh + (r & 3);
        dpacc[r] = sacc[r] * (dpacc[r] - delta_lds[qr]);
      }
      bf16x8 dsb[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
          const bf16x2 two = __builtin_convertvector(f32x2{dpacc[8 * ks + i], dpacc[8 * ks + i + 1]}, bf16x2);
          dsb[ks][i] = two[0];
          dsb[ks][i + 1] = two[1];
        }
      // dK^T += Q^T dS
#pragma unroll
      for (int b = 0; b < NDB; ++b)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(&qt_lds[(32 * b + ln) * TSTR + 16 * ks + 8 * hh]);
          dkacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, dsb[ks], dkacc[b], 0, 0, 0);
        }
      // stage dS [q][key] for the dQ step
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int qr = 16 * ks + 8 * (i >> 2) + 4 * hh + (i & 3);
          const __bf16 hv = dsb[ks][i];
          ds_lds[qr * SSTR + 32 * wave + ln] = *reinterpret_cast<const uint16_t*>(&hv);
        }
      __syncthreads();
      // dQ[q][d] += scale * dS K for this wave's d block and key range
      f32x16 dqacc = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KPW / 16; ++ks) {
        const int k0 = dq_k0 + 16 * ks + 8 * hh;
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&ds_lds[ln * SSTR + k0]);
        const bf16x8 b = *reinterpret_cast<const bf16x8*>(&kt_lds[(32 * dq_db + ln) * KTSTR + k0]);
        dqacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, dqacc, 0, 0, 0);
      }
      float* dqp = p.dq + (size_t)head * D + 32 * dq_db + ln;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qr = 8 * (r >> 2) + 4 * hh + (r & 3);
        if (qr < nrows) atomicAdd(dqp + (size_t)(l_row0 + qr) * p.hq * D, dqacc[r] * p.scale);
      }
    }
  }

  // dK (scaled) and dV of this lane's key: rows d = 32 b + 8 g + 4 hh .. +4
  if (key_ok) {
    float* dkp = p.dk + (size_t)key_l * kv_rstride + (size_t)kvh * D + 4 * hh;
    float* dvp = p.dv + (size_t)key_l * kv_rstride + (size_t)kvh * D + 4 * hh;
#pragma unroll
    for (int b = 0; b < NDB; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * b + 8 * g;
        *reinterpret_cast<float4*>(dkp + d0) =
            make_float4(dkacc[b][4 * g] * p.scale, dkacc[b][4 * g + 1] * p.scale, dkacc[b][4 * g + 2] * p.scale,
                        dkacc[b][4 * g + 3] * p.scale);
        *reinterpret_cast<float4*>(dvp + d0) =
            make_float4(dvacc[b][4 * g], dvacc[b][4 * g + 1], dvacc[b][4 * g + 2], dvacc[b][4 * g + 3]);
      }
  }
}

hipError_t launch_fill_zero(float* dst, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const long long blocks = ((n + 3) / 4 + 255) / 256;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, dst, n);
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdParams& p, int d, bool accumulate_dq, bool delta_ready, hipStream_t stream) {
  hipError_t e;
  if (!accumulate_dq) {
    e = launch_fill_zero(p.dq, (int64_t)p.tq * p.hq * d, stream);
    if (e != hipSuccess) return e;
  }
  const long long rh_threads = (long long)p.tq * p.hq * (d / 8);
  if (rh_threads > 0 && !delta_ready) {
    const long long blocks = (rh_threads + 255) / 256;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    if (d == 128)
      hipLaunchKernelGGL(bwd_delta_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, stream, p.o, p.d_o, p.delta,
                         p.tq, p.hq);
    else
      hipLaunchKernelGGL(bwd_delta_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, stream, p.o, p.d_o, p.delta,
                         p.tq, p.hq);
  }
  const long long nblk = (long long)p.n_kvtiles * p.hkv;
  if (nblk > 0) {
    if (nblk > 0x7fffffffLL) return hipErrorInvalidValue;
    if (d == 128) hipLaunchKernelGGL(bwd_kernel<128>, dim3((unsigned)nblk), dim3(256), 0, stream, p);
    else hipLaunchKernelGGL(bwd_kernel<64>, dim3((unsigned)nblk), dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace docmask
