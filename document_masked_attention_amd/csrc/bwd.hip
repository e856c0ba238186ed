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
// Three kernels, all deterministic (no atomics), launched in this order (the
// first two leave out each document's first kBwdHead x kBwdHead positions,
// which the third computes in fp32):
//
// * dq_kernel, query-major, shaped like the forward.  Work item = (query tile,
//   KV head, block of query heads), 4 waves, two workgroups per CU; each
//   wave owns 32 rows x 1 head (two 16-row halves).
//   It first forms Delta of its rows (unless the caller supplied it) from the
//   dO operands it holds and the O rows, and stores it; then it walks the
//   tile's KV range, 32 keys at a time:
//     S^T = K Q^T,  dP^T = V dO^T,  dS^T = P^T (dP^T - Delta),  dQ^T += K^T dS^T
//   (v_mfma_f32_16x16x32_bf16, every K, V and K^T operand feeding both row
//   halves; K^T through transpose reads; dS^T straight from the
//   accumulators, in the forward's permuted key order).  The operands of a
//   32-key step form one stream, each read two MFMA slots ahead, across the
//   softmax and into the next step (8% faster than reads placed by the
//   compiler, which waited on most of them).
// * dkdv_kernel, key-major.  Work item = (one or two KV tiles of 128 keys
//   of a document, paired by the scheduler, KV head); 4 waves x 32 keys (one
//   wave per SIMD), each lane keeping one key's K and V rows (MFMA B
//   operands) and its dK, dV accumulators in registers.  For each tile it
//   walks every (32-row query block, query head of the group) that attends
//   the tile -- the scheduler's per-KV-tile range -- with the Q and dO rows
//   staged in LDS:
//     S = Q K^T,  P = exp2(S c - LSE2),  dV^T += dO^T P,
//     dP = dO V^T,  dS = P (dP - Delta),  dK^T += Q^T dS
//   (v_mfma_f32_32x32x16_bf16; Q^T and dO^T come from the row-major tiles
//   through LDS transpose reads).
// * head_kernel: the pairs ds <= j <= i < ds + kBwdHead of every document
//   (ds its start) in fp32, added to dq, dk and dv (see there).
#include "kernels.h"


namespace docmask {

__device__ __forceinline__ bf16x8 cvt8(float a0, float a1, float a2, float a3, float b0, float b1, float b2,
                                      float b3) {
  const bf16x2 p0 = __builtin_convertvector(f32x2{a0, a1}, bf16x2);
  const bf16x2 p1 = __builtin_convertvector(f32x2{a2, a3}, bf16x2);
  const bf16x2 p2 = __builtin_convertvector(f32x2{b0, b1}, bf16x2);
  const bf16x2 p3 = __builtin_convertvector(f32x2{b2, b3}, bf16x2);
  return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// S and dP tiles of the dK/dV kernel: v_mfma_f32_32x32x16_bf16 with the
// accumulator in VGPRs and the B operand (the lane's K or V row) in AGPRs,
// written as inline assembly so that these tiles stay in VGPRs next to the
// dK / dV accumulators the compiler keeps in AGPRs (the vector ALU reads them
// without copies).  The compiler does not see these MFMAs, so it inserts no
// wait states for them: every vector instruction that reads or writes such a
// tile is issued at least 12 wait states (issued instructions or s_nop
// cycles) after the last MFMA that writes it, the latency this 8-pass MFMA
// needs on gfx950; dP's initial value (-Delta) comes straight from LDS reads.
__device__ __forceinline__ void mfma_v_zero(f32x16& c, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_v_acc(f32x16& c, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "a"(b));
}
// 12 wait states
__device__ __forceinline__ void mfma_v_settle() { asm volatile("s_nop 7\n\ts_nop 3"); }

// ------------------------------------------------------------------ dK, dV
// Work item = (pair of KV tiles of 128 keys, KV head), the tiles processed
// one after the other; four waves of 32 keys, one wave per SIMD.  Each lane
// keeps one key: its K and V rows are the MFMA B
// operands of S = Q K^T and dP = dO V^T (v_mfma_f32_32x32x16_bf16), whose
// output tiles hold 16 query rows {8 j + 4 h + r} of that key per lane.  In
// that register order P and dS are directly the B operands of dV^T += dO^T P
// and dK^T += Q^T dS, with the 16-row k-step visited as rows
// {4h .. 4h+3, 8+4h .. 8+4h+3} per half-wave h; the A operands dO^T and Q^T
// come from the row-major LDS tiles through transpose reads in the same row
// order.  dP starts from -Delta, so dS = P dP; P = exp2(S c - LSE2), with
// the scores of disallowed pairs set to -inf (only units outside the tile's
// FULL range, in a branch between pipeline regions).
//
// Per tile the work is a sequence of units (32-row query block, query head):
// the first tile of a pair walks its query blocks from the last one down, the
// second from its first one up, so that the work items of one document
// running at the same time read the same Q / dO rows together (L2 reuse).
// Units are software-pipelined: region u runs the softmax of unit u on the
// vector ALU while the matrix cores run dV / dK of unit u - 1 and S / dP of
// unit u + 1.  Two units form a staging step; steps go through a ring of four
// LDS buffers filled by direct global-to-LDS loads: step s + 3 is issued in
// the middle of step s, as soon as the barrier there frees the buffer of
// step s - 1.

template <int D>
__global__ __launch_bounds__(256, 1) void dkdv_kernel(BwdParams p) {
  constexpr int BQ = kBwdBQ;            // 32 query rows per unit
  constexpr int BK = kBwdBK;            // 128 keys per work item, 32 per wave
  constexpr int NKS = D / 16;           // k-steps of S and dP over d
  constexpr int NMB = D / 32;           // 32-wide d blocks of dK^T / dV^T
  constexpr int NBUF = 4;               // staging ring depth (steps)
  using L = DenseTile<D>;               // Q / dO tile layout (row chunks + transpose reads)
  constexpr int TE = L::kElems(BQ);
  constexpr int RPL = 512 / D;          // tile rows per direct load (64 lanes x 16 bytes)
  constexpr int WLT = BQ / RPL;         // direct loads per tile
  constexpr int DPW = 4 * WLT / 4;      // direct loads per wave per step (2 units x Q, dO = 4 tiles)
  constexpr int VM_PER_STEP = 1 + DPW;  // vector-memory instructions per wave per step
  constexpr int TB = 2 * TE;            // bytes per Q / dO tile
  constexpr int QDB = 4 * TB;           // bytes per staging step of tiles
  // Q / dO tiles of the ring: qd[g][2 j + 0: Q, 2 j + 1: dO] of unit j of the
  // step staged in buffer g; their LSE / Delta rows in sm[g]
  struct Small {
    float lse[2][BQ];       // LSE * log2(e); +inf: P = 0
    float ndl[2][BQ];       // -Delta
    float raw[256];         // loaded LSE / Delta words, one per thread
  };
  __shared__ __attribute__((aligned(16))) uint16_t qd[NBUF][4][TE];
  __shared__ __attribute__((aligned(16))) Small sm[NBUF];

  if (p.err[0]) return;

  // Work item: a pair of KV tiles (the lower one leads; the scheduler's
  // pairing), or one tile alone; a tile that is not a leader runs inside its
  // leader's work item.
  const WorkItem wi = map_work(blockIdx.x, p.n_kvtiles, p.hkv, 1, p.xcd_cluster);
  const int kvh = wi.kvh;
  const int lead = min(max(ld_const(p.lpt_kv, wi.rank), 0), p.n_kvtiles - 1);
  const int partner = min(max(ld_const(p.kv_pair, lead), 0), p.n_kvtiles - 1);
  if (partner < lead) return;
  const int n_parts = partner > lead ? 2 : 1;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, hh = lane >> 5, l32 = lane & 31;
  const int tkv = p.kv_hi - p.kv_lo;
  const size_t kv_rstride = (size_t)p.hkv * D;

  // Per-tile state, set at the start of each part: the tile's query-block
  // range, this lane's key, the walking direction over the query blocks.
  int tile = lead, qt_lo = 0, qt_flo = 0, qt_fhi = 0, qt_hi = 0, dir = -1;
  int key_l = 0, key_g = 0, key_row0 = 0, key_end = 0, n_units = 0, n_steps = 0;
  bool key_ok = false, ragged = false;
  bf16x8 kf[NKS], vf[NKS];        // K and V rows of this lane's key as B operands: d = 16 s + 8 hh .. +8
  f32x16 dkacc[NMB], dvacc[NMB];

  // LSE (wave 0) or Delta (wave 1) rows staged by this wave; waves 2 and 3
  // load the same words again, unused, so every wave issues the same number
  // of vector-memory instructions per step
  const float* ld_src = (wave & 1) ? p.delta : p.lse;
  // Unit sequence: unit u is (query block qt_hi - 1 - u / G when walking
  // down, qt_lo + u / G when walking up; head u % G of the group).  A
  // wave-uniform cursor walks it in order, two units per staged step; units
  // past the end repeat the last one (dummy units, P = 0).
  struct UnitInfo {
    int l_row0, g_row0, nrows, head, masked, dummy;
  };
  int cur_u = 0, cur_qt = 0, cur_hd = 0;
  auto next_unit = [&]() __attribute__((always_inline)) -> UnitInfo {
    UnitInfo ui;
    ui.dummy = cur_u >= n_units;
    const int qt = ui.dummy ? (dir < 0 ? qt_lo : qt_hi - 1) : cur_qt;
    ui.head = kvh * p.group + (ui.dummy ? p.group - 1 : cur_hd);
    ui.l_row0 = ld_const(p.plan_kq, (size_t)qt * QP_WORDS + QP_LROW0);
    ui.g_row0 = ld_const(p.plan_kq, (size_t)qt * QP_WORDS + QP_GROW0);
    ui.nrows = ld_const(p.plan_kq, (size_t)qt * QP_WORDS + QP_NROWS);
    // inside the tile's FULL range every (row, key) pair is allowed
    ui.masked = (qt < qt_flo || qt >= qt_fhi || ragged || ui.nrows < BQ) ? 1 : 0;
    ++cur_u;
    if (++cur_hd == p.group) { cur_hd = 0; cur_qt += dir; }
    return ui;
  };
  // lane byte offsets of the direct loads of a full unit (32 rows): row r of
  // the tile at r * Hq * D * 2 bytes, chunk position lane % (D/8) holding
  // chunk chunk_at(r, pos)
  const uint32_t row_b = (uint32_t)(p.hq * D * sizeof(uint16_t));
  uint32_t loff_full[DPW];
#pragma unroll
  for (int i = 0; i < DPW; ++i) {
    const int r = (wave + 4 * (i % (WLT / 4))) * RPL + lane / L::kChunks;
    loff_full[i] = (uint32_t)r * row_b + 16u * (uint32_t)L::chunk_at(r, lane % L::kChunks);
  }
  // Loads of the next step to stage (its two units come back in u0 / u1)
  // into buffer g, all direct global-to-LDS loads (no register is written
  // asynchronously): per wave first one dword per lane into raw[tid] (threads
  // 0..127: LSE then Delta of unit (tid / 32) % 2, row tid % 32 clamped to a
  // real row), then DPW 16-byte loads: load i covers tile t = i / (WLT / 4)
  // (Q, dO of unit 0, Q, dO of unit 1), rows RPL (wave + 4 (i % (WLT / 4))) ..,
  // lane -> row + lane / (D/8), chunk position lane % (D/8), from the tile's
  // uniform base plus a 32-bit lane offset.  Units with padded rows clamp the
  // row to the last real one (one wave-uniform branch).
  // LDS byte address of this wave's first direct-load slot in buffer 0
  const uint32_t qd_wave =
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)&qd[0][0][wave * RPL * D];
  auto issue = [&](auto g_c, UnitInfo& u0, UnitInfo& u1) __attribute__((always_inline)) {
    constexpr int g = decltype(g_c)::value;
    u0 = next_unit();
    u1 = next_unit();
    {
      const int j = (tid >> 5) & 1, row = tid & 31;
      const float* b0 = ld_src + (size_t)u0.head * p.tq + u0.l_row0;
      const float* b1 = ld_src + (size_t)u1.head * p.tq + u1.l_row0;
      lds_dma4((j ? b1 : b0) + min(row, (j ? u1.nrows : u0.nrows) - 1), &sm[g].raw[64 * wave]);
    }
    const uint16_t* tb[4] = {p.q + ((size_t)u0.l_row0 * p.hq + u0.head) * D,
                             p.d_o + ((size_t)u0.l_row0 * p.hq + u0.head) * D,
                             p.q + ((size_t)u1.l_row0 * p.hq + u1.head) * D,
                             p.d_o + ((size_t)u1.l_row0 * p.hq + u1.head) * D};
    if (u0.nrows == BQ && u1.nrows == BQ) {
      static_for<DPW>([&](auto ic) __attribute__((always_inline)) {
        constexpr int i = decltype(ic)::value;
        constexpr int t = i / (WLT / 4);
        lds_dma16_so<(uint32_t)(g * QDB + t * TB + 4 * (i % (WLT / 4)) * RPL * D * 2)>(tb[t], loff_full[i], qd_wave);
      });
    } else {
      static_for<DPW>([&](auto ic) __attribute__((always_inline)) {
        constexpr int i = decltype(ic)::value;
        constexpr int t = i / (WLT / 4);
        const int nrows = (t >> 1) ? u1.nrows : u0.nrows;
        const int r0 = (wave + 4 * (i % (WLT / 4))) * RPL;
        const int r = r0 + lane / L::kChunks;
        const uint32_t off =
            (uint32_t)min(r, nrows - 1) * row_b + 16u * (uint32_t)L::chunk_at(r, lane % L::kChunks);
        lds_dma16_so<(uint32_t)(g * QDB + t * TB + 4 * (i % (WLT / 4)) * RPL * D * 2)>(tb[t], off, qd_wave);
      });
    }
  };
  // LSE2 / -Delta of a staged step, from this thread's own loaded word:
  // padded rows and dummy units get LSE = +inf, Delta = 0 (P = 0); an empty
  // row (LSE = -inf) likewise gets P = 0
  auto finish = [&](int g, const UnitInfo& u0, const UnitInfo& u1) __attribute__((always_inline)) {
    Small& dst = sm[g];
    const float v = dst.raw[tid];
    const int j = (tid >> 5) & 1, row = tid & 31;
    const bool pad = row >= (j ? u1.nrows : u0.nrows) || (j ? u1.dummy : u0.dummy);
    if (tid < 64) {
      dst.lse[j][row] = (pad || v == -INFINITY) ? INFINITY : v * kLog2e;
    } else if (tid < 128) {
      dst.ndl[j][row] = pad ? 0.f : -v;
    }
  };
  // waits until at most `n` of this wave's vector-memory instructions are
  // outstanding (the memory clobber keeps LDS reads of the staged data after it)
  auto wait_vm = [&](auto n_c) __attribute__((always_inline)) {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(decltype(n_c)::value) : "memory");
  };

  // transpose-read source of this lane: row 4 (lane / 32) + (lane / 4) % 4 of
  // the k-step (second read: + 8), column 16 ((lane / 16) % 2) + 4 (lane % 4)
  // of the 32-wide d block
  const int tr_row = 4 * hh + ((lane >> 2) & 3), tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  // LDS reads of the ring use a lane byte offset inside a tile held in a
  // register plus a constant (buffer, tile, k-step) in the instruction's
  // 16-bit offset field; buffers at or above 64 KiB use a second copy of the
  // lane offsets advanced by 64 KiB.  Row reads: row l32, k-step sb.
  // Transpose reads: d block m, rows tr_row (+ 8); the 16-row k-step t of a
  // tile adds 16 rows (the swizzle repeats every 16 rows).
  const char* qd_b = reinterpret_cast<const char*>(&qd[0][0][0]);
  constexpr bool kTwoSets = NBUF * QDB > 65536;
  uint32_t ro_lo[NKS], ro_hi[NKS], tro_lo[NMB][2], tro_hi[NMB][2];
#pragma unroll
  for (int sb = 0; sb < NKS; ++sb) {
    ro_lo[sb] = 2u * (uint32_t)L::off(l32, 16 * sb + 8 * hh);
    ro_hi[sb] = ro_lo[sb] + 65536u;
  }
#pragma unroll
  for (int m = 0; m < NMB; ++m)
#pragma unroll
    for (int o = 0; o < 2; ++o) {
      tro_lo[m][o] = 2u * (uint32_t)L::off(8 * o + tr_row, 32 * m + tr_col);
      tro_hi[m][o] = tro_lo[m][o] + 65536u;
    }
  if constexpr (kTwoSets) {
    // separate registers (no re-adding of 64 KiB per read); the mask keeps
    // the values known non-negative so that constants fold into the offset
#pragma unroll
    for (int sb = 0; sb < NKS; ++sb) { asm volatile("" : "+v"(ro_hi[sb])); ro_hi[sb] &= 0x3ffffu; }
#pragma unroll
    for (int m = 0; m < NMB; ++m)
#pragma unroll
      for (int o = 0; o < 2; ++o) { asm volatile("" : "+v"(tro_hi[m][o])); tro_hi[m][o] &= 0x3ffffu; }
  }
  // address of buffer G, tile T, constant byte offset C, lane offset (lo, hi)
  auto qd_at = [&](auto g_c, auto t_c, auto c_c, uint32_t lo, uint32_t hi) __attribute__((always_inline)) {
    constexpr uint32_t off = decltype(g_c)::value * QDB + decltype(t_c)::value * TB + decltype(c_c)::value;
    if constexpr (!kTwoSets || off < 65536u - TB) return reinterpret_cast<const uint16_t*>(qd_b + lo + off);
    else return reinterpret_cast<const uint16_t*>(qd_b + hi + (off - 65536u));
  };

  // document mask of a unit on its S accumulators: scores of (row, this key)
  // pairs that are not allowed become -inf (P = 0).  Only units outside the
  // tile's FULL range need it; the caller branches on ui.masked.
  auto unit_mask = [&](const UnitInfo& ui, f32x16& sa) __attribute__((always_inline)) {
    // rows this pass takes: key_row0 <= g_row0 + qr < key_end, qr < nrows
    const int lo = key_row0 - ui.g_row0;
    const int hi = key_ok ? min(key_end - ui.g_row0, ui.nrows) : lo;
    const unsigned span = (unsigned)max(hi - lo, 0);
    mfma_v_settle();
#pragma unroll
    for (int e = 0; e < 16; ++e)
      if ((unsigned)(8 * (e >> 2) + 4 * hh + (e & 3) - lo) >= span) sa[e] = -INFINITY;
  };
  // One pipeline region, as NP slots in a fixed order (scheduling fences
  // between slots).  Slot k issues
  //   * MFMA k of dV / dK for unit A: d block m = k / 4, k-step t = (k / 2) % 2,
  //     dV (k even, A operand dO^T) or dK (k odd, A operand Q^T);
  //   * MFMA k of S / dP for unit B: k-step s = k / 2, S (k even, Q rows, from
  //     zero) or dP (k odd, dO rows, from -Delta);
  //   * the softmax of the elements of unit C that fall to slot k;
  // and the LDS reads of slot k + PF, so every operand has PF slots of
  // matrix work to arrive.
  constexpr int NP = 4 * NMB;           // == 2 * NKS: slots per region
  constexpr int PF = 1;                 // operand prefetch distance (slots): 1 measured faster than 2 or 3
  constexpr int EPS = 16 / NP;          // softmax elements per slot
  // Buffers GA (unit ja: dV / dK operands), GB (unit jb: S / dP operands)
  // and GC (unit jc: softmax LSE) are compile-time ring indices.
  auto region = [&](auto ga_c, auto ja_c, const bf16x8 (&pba)[2], const bf16x8 (&dsba)[2],
                    auto gb_c, auto jb_c, f32x16& sab, f32x16& dab,
                    auto gc_c, auto jc_c, const f32x16& sac, const f32x16& dac, bf16x8 (&pbc)[2],
                    bf16x8 (&dsbc)[2]) __attribute__((always_inline)) {
    constexpr int ja = decltype(ja_c)::value, jb = decltype(jb_c)::value, jc = decltype(jc_c)::value;
    using IC = std::integral_constant<int, 0>;
    bf16x8 opa[NP], opb[NP];
    auto load = [&](auto kc) __attribute__((always_inline)) {
      constexpr int k = decltype(kc)::value;
      constexpr int m = k / 4, t = (k / 2) % 2, sb = k / 2;
      // A: dO^T (k even) or Q^T (k odd) of unit ja; B: Q (k even) or dO (k odd) rows of unit jb
      using TA = std::integral_constant<int, 2 * ja + 1 - (k % 2)>;
      using TBt = std::integral_constant<int, 2 * jb + (k % 2)>;
      using CT = std::integral_constant<int, 16 * t * D * 2>;
      opa[k] = tr_operand(qd_at(ga_c, TA{}, CT{}, tro_lo[m][0], tro_hi[m][0]),
                          qd_at(ga_c, TA{}, CT{}, tro_lo[m][1], tro_hi[m][1]));
      opb[k] = *reinterpret_cast<const bf16x8*>(qd_at(gb_c, TBt{}, IC{}, ro_lo[sb], ro_hi[sb]));
    };
    const Small& stc = sm[decltype(gc_c)::value];
    const Small& stb = sm[decltype(gb_c)::value];
    f32x4 l4[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) l4[jj] = *reinterpret_cast<const f32x4*>(&stc.lse[jc][8 * jj + 4 * hh]);
    f32x16 ndb;                                   // -Delta of unit B's rows: dP starts from it
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(&stb.ndl[jb][8 * jj + 4 * hh]);
#pragma unroll
      for (int r = 0; r < 4; ++r) ndb[4 * jj + r] = d4[r];
    }
    static_for<PF>([&](auto kc) __attribute__((always_inline)) { load(kc); });
    float xv[16], pv[16], dsv[16];
    static_for<EPS>([&](auto ec) __attribute__((always_inline)) {
      constexpr int e = decltype(ec)::value;
      xv[e] = __builtin_fmaf(sac[e], p.scale_log2, -l4[e / 4][e % 4]);
    });
    static_for<NP>([&](auto kc) __attribute__((always_inline)) {
      constexpr int k = decltype(kc)::value;
      constexpr int m = k / 4, t = (k / 2) % 2, sb = k / 2;
      if constexpr (k % 2 == 0)
        dvacc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opa[k], pba[t], dvacc[m], 0, 0, 0);
      else
        dkacc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opa[k], dsba[t], dkacc[m], 0, 0, 0);
      if constexpr (k + PF < NP) load(std::integral_constant<int, k + PF>{});
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (k % 2 == 0) {
        if constexpr (sb == 0) mfma_v_zero(sab, opb[k], kf[sb]); else mfma_v_acc(sab, opb[k], kf[sb]);
      } else {
        if constexpr (sb == 0) dab = ndb;
        mfma_v_acc(dab, opb[k], vf[sb]);
      }
      // softmax elements, software-pipelined across slots so that no
      // instruction waits on one issued just before it: slot k forms the
      // exponent argument of its next slot's elements, exponentiates its own
      // and multiplies the previous slot's by dP
      static_for<EPS>([&](auto ec) __attribute__((always_inline)) {
        constexpr int e = k * EPS + decltype(ec)::value;
        if constexpr (e + EPS < 16) xv[e + EPS] = __builtin_fmaf(sac[e + EPS], p.scale_log2, -l4[(e + EPS) / 4][(e + EPS) % 4]);
        pv[e] = __builtin_amdgcn_exp2f(xv[e]);
        if constexpr (e >= EPS) dsv[e - EPS] = pv[e - EPS] * dac[e - EPS];
      });
      __builtin_amdgcn_sched_barrier(0);
    });
    static_for<EPS>([&](auto ec) __attribute__((always_inline)) {
      constexpr int e = 16 - EPS + decltype(ec)::value;
      dsv[e] = pv[e] * dac[e];
    });
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      pbc[t] = cvt8(pv[8 * t], pv[8 * t + 1], pv[8 * t + 2], pv[8 * t + 3], pv[8 * t + 4], pv[8 * t + 5],
                    pv[8 * t + 6], pv[8 * t + 7]);
      dsbc[t] = cvt8(dsv[8 * t], dsv[8 * t + 1], dsv[8 * t + 2], dsv[8 * t + 3], dsv[8 * t + 4], dsv[8 * t + 5],
                     dsv[8 * t + 6], dsv[8 * t + 7]);
    }
    asm volatile("" : "+v"(pbc[0]), "+v"(pbc[1]), "+v"(dsbc[0]), "+v"(dsbc[1]));
    __builtin_amdgcn_sched_barrier(0);
  };
  // S and dP (from -Delta) of unit j of buffer g, alone (pipeline start)
  auto sdp = [&](int g, int j, f32x16& sa, f32x16& da) __attribute__((always_inline)) {
    const uint16_t* qs = qd[g][2 * j];
    const uint16_t* dos = qd[g][2 * j + 1];
    f32x16 nd;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(&sm[g].ndl[j][8 * jj + 4 * hh]);
#pragma unroll
      for (int r = 0; r < 4; ++r) nd[4 * jj + r] = d4[r];
    }
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      const int off = L::off(l32, 16 * s + 8 * hh);
      const bf16x8 qa_ = *reinterpret_cast<const bf16x8*>(&qs[off]);
      const bf16x8 da_ = *reinterpret_cast<const bf16x8*>(&dos[off]);
      if (s == 0) {
        mfma_v_zero(sa, qa_, kf[s]);
        da = nd;
      } else {
        mfma_v_acc(sa, qa_, kf[s]);
      }
      mfma_v_acc(da, da_, vf[s]);
    }
    mfma_v_settle();
  };
  // dV^T += dO^T P and dK^T += Q^T dS for unit j of buffer g, alone (pipeline end)
  auto dvdk = [&](int g, int j, const bf16x8 (&pb)[2], const bf16x8 (&dsb)[2]) __attribute__((always_inline)) {
    const uint16_t* qs = qd[g][2 * j];
    const uint16_t* dos = qd[g][2 * j + 1];
#pragma unroll
    for (int m = 0; m < NMB; ++m) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int o0 = L::off(16 * t + tr_row, 32 * m + tr_col);
        const int o1 = L::off(16 * t + 8 + tr_row, 32 * m + tr_col);
        const bf16x8 doT = tr_operand(dos + o0, dos + o1);
        const bf16x8 qT = tr_operand(qs + o0, qs + o1);
        dvacc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(doT, pb[t], dvacc[m], 0, 0, 0);
        dkacc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qT, dsb[t], dkacc[m], 0, 0, 0);
      }
    }
  };

  for (int part = 0; part < n_parts; ++part) {
    // ---- tile of this part: the leader walks its query blocks from the
    // document end down, its partner from its diagonal up
    tile = part ? partner : lead;
    dir = part ? 1 : -1;
    qt_lo = ld_const(p.kvdesc, (size_t)tile * 4);
    qt_flo = ld_const(p.kvdesc, (size_t)tile * 4 + 1);
    qt_fhi = ld_const(p.kvdesc, (size_t)tile * 4 + 2);
    qt_hi = ld_const(p.kvdesc, (size_t)tile * 4 + 3);
    key_l = tile * BK + 32 * wave + l32;              // this lane's key (local KV row)
    key_ok = key_l < tkv;
    key_g = p.kv_lo + key_l;
    key_end = key_ok ? doc_end(p.cu, p.n_docs, key_g) : key_g;
    // a key among its document's first kBwdHead positions leaves the rows
    // among those positions to the head pass (fp32); its other rows are here
    key_row0 = key_g;
    if (key_ok) {
      const int ds = doc_start(p.cu, p.n_docs, key_g);
      if (key_g - ds < kBwdHead) key_row0 = ds + kBwdHead;
    }
    ragged = (tile + 1) * BK > tkv;
    {
      const int kl = min(key_l, tkv - 1);               // padding keys: any finite row, masked below
      const uint16_t* kr = p.k + (size_t)kl * kv_rstride + (size_t)kvh * D + 8 * hh;
      const uint16_t* vr = p.v + (size_t)kl * kv_rstride + (size_t)kvh * D + 8 * hh;
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        kf[s] = *reinterpret_cast<const bf16x8*>(kr + 16 * s);
        vf[s] = *reinterpret_cast<const bf16x8*>(vr + 16 * s);
      }
    }
#pragma unroll
    for (int m = 0; m < NMB; ++m) { dkacc[m] = f32x16{}; dvacc[m] = f32x16{}; }
    n_units = (qt_hi - qt_lo) * p.group;                // 0: no query row attends the tile (zero gradients)
    n_steps = (n_units + 1) >> 1;                       // the last step may hold one dummy unit
    cur_u = 0;
    cur_qt = dir < 0 ? qt_hi - 1 : qt_lo;
    cur_hd = 0;
    if (part) __syncthreads();                          // the previous tile's LDS reads are done

    if (n_units > 0) {
      // prologue: steps 0 and 1 staged, step 2 in flight; S / dP of unit 0.
      // Unit 1's tiles of buffer NBUF - 1 (the operands of the "previous
      // unit" of step 0, whose P and dS are zero) are cleared, so that
      // 0 * garbage cannot make a NaN.
      UnitInfo ic0, ic1, in0, in1, i20, i21;   // plan words of steps s, s + 1, s + 2
      issue(std::integral_constant<int, 0>{}, ic0, ic1);
      issue(std::integral_constant<int, 1>{}, in0, in1);
      issue(std::integral_constant<int, 2>{}, i20, i21);
      {
        uint4* z = reinterpret_cast<uint4*>(&qd[NBUF - 1][2][0]);
#pragma unroll
        for (int i = 0; i < 2 * TB / 16 / 256; ++i) z[tid + 256 * i] = uint4{0u, 0u, 0u, 0u};
      }
      wait_vm(std::integral_constant<int, VM_PER_STEP>{});
      finish(0, ic0, ic1);
      finish(1, in0, in1);
      // the key's document end and the K / V operands are in registers before
      // any later loads are in flight
      asm volatile("" ::"v"(key_end), "v"(key_row0));
#pragma unroll
      for (int s = 0; s < NKS; ++s) asm volatile("" ::"a"(kf[s]), "a"(vf[s]));
      __syncthreads();

      f32x16 sa[2], da[2];
      bf16x8 pb[2][2], dsb[2][2];
#pragma unroll
      for (int t = 0; t < 2; ++t) { pb[1][t] = bf16x8{}; dsb[1][t] = bf16x8{}; }   // unit -1: adds zero
      sdp(0, 0, sa[0], da[0]);
      if (ic0.masked) unit_mask(ic0, sa[0]);
      // Step s (buffer phase PH = s mod NBUF, a compile-time constant so that
      // every LDS address is a register plus an immediate): units 2s, 2s + 1.
      auto step = [&](int s, auto ph_c) __attribute__((always_inline)) {
        constexpr int ph = decltype(ph_c)::value;
        using GC = std::integral_constant<int, ph>;
        using GP = std::integral_constant<int, (ph + NBUF - 1) % NBUF>;
        using GN1 = std::integral_constant<int, (ph + 1) % NBUF>;
        using J0 = std::integral_constant<int, 0>;
        using J1 = std::integral_constant<int, 1>;
        // ---- region 2s: dV, dK (2s - 1) | S, dP (2s + 1) | softmax(2s)
        __builtin_amdgcn_sched_barrier(0);
        region(GP{}, J1{}, pb[1], dsb[1], GC{}, J1{}, sa[1], da[1], GC{}, J0{}, sa[0], da[0], pb[0], dsb[0]);
        if (ic1.masked) unit_mask(ic1, sa[1]);
        // ---- step s + 1 staged (its loads were issued four regions ago;
        // step s + 2's may still be in flight)
        if (s > 0) {
          wait_vm(std::integral_constant<int, VM_PER_STEP>{});
          finish(GN1::value, in0, in1);
        }
        __syncthreads();
        // ---- step s + 3 into the buffer of step s - 1, whose last reader
        // (region 2s, the previous unit's dV / dK) is behind the barrier
        UnitInfo i30, i31;
        issue(std::integral_constant<int, (ph + 3) % NBUF>{}, i30, i31);
        // ---- region 2s + 1: dV, dK (2s) | S, dP (2s + 2) | softmax(2s + 1)
        __builtin_amdgcn_sched_barrier(0);
        region(GC{}, J0{}, pb[0], dsb[0], GN1{}, J0{}, sa[0], da[0], GC{}, J1{}, sa[1], da[1], pb[1], dsb[1]);
        if (in0.masked) unit_mask(in0, sa[0]);
        ic0 = in0; ic1 = in1; in0 = i20; in1 = i21; i20 = i30; i21 = i31;
      };
      static_assert(NBUF == 4, "one unrolled step per buffer phase");
      for (int s = 0; s < n_steps; s += NBUF) {
        step(s, std::integral_constant<int, 0>{});
        if (s + 1 < n_steps) step(s + 1, std::integral_constant<int, 1>{});
        if (s + 2 < n_steps) step(s + 2, std::integral_constant<int, 2>{});
        if (s + 3 < n_steps) step(s + 3, std::integral_constant<int, 3>{});
      }
      // the last unit's dV, dK (a dummy unit adds zero)
      dvdk((n_steps - 1) & (NBUF - 1), 1, pb[1], dsb[1]);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // drain the clamped tail loads
    }

    // dK (scaled) and dV of this lane's key: d = 32 m + 8 j + 4 hh .. +4
    if (key_ok) {
      float* dkp = p.dk + (size_t)key_l * kv_rstride + (size_t)kvh * D + 4 * hh;
      float* dvp = p.dv + (size_t)key_l * kv_rstride + (size_t)kvh * D + 4 * hh;
#pragma unroll
      for (int m = 0; m < NMB; ++m)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int c = 32 * m + 8 * j;
          *reinterpret_cast<float4*>(dkp + c) =
              make_float4(dkacc[m][4 * j] * p.scale, dkacc[m][4 * j + 1] * p.scale, dkacc[m][4 * j + 2] * p.scale,
                          dkacc[m][4 * j + 3] * p.scale);
          *reinterpret_cast<float4*>(dvp + c) =
              make_float4(dvacc[m][4 * j], dvacc[m][4 * j + 1], dvacc[m][4 * j + 2], dvacc[m][4 * j + 3]);
        }
    }
  }
}

// ------------------------------------------------------------------ dQ
template <int D, int RB, int HB>
__global__ __launch_bounds__(256, 2) void dq_kernel(BwdParams p) {
  constexpr int NW = RB * HB;           // waves per workgroup (two workgroups per CU)
  static_assert(NW == 4, "four waves per workgroup");
  constexpr int BK = kDqBK;
  using L = SwzTile<D>;                 // K and V tiles (K: row chunks and transpose reads; V: row chunks)
  constexpr int CPK = D / 8;
  constexpr int NKS = D / 32;           // 32-wide k-steps of S^T and dP^T
  constexpr int NDB = D / 16;           // 16-wide d blocks of dQ
  // K and V tiles reach LDS by direct global-to-LDS loads: a tile is a run of
  // 16-byte slots (SK per row: the row's chunks plus any padding slots), and
  // direct load j fills slots 64 j .. 64 j + 63.  Lane l of load j maps slot
  // q = 64 j + l back to (row q / SK, stored position q % SK): chunk position
  // ^ f(row) for D = 128 (unpadded swizzled rows), the position itself for
  // D = 64; padding slots load any real chunk of the row (never read).  K and
  // V share the layout, so one set of lane offsets serves both.
  constexpr int SK = L::kRowElems / 8;
  constexpr int WK = BK * SK / 64;                          // direct loads per K or V tile
  constexpr int DK = (WK + NW - 1) / NW;                    // per wave (the last may be idle)
  static_assert(BK * SK % 64 == 0, "tiles are whole direct loads");
  constexpr int KTB = BK * SK * 16;                         // bytes per K or V tile
  __shared__ __attribute__((aligned(16))) uint16_t k_s[2][L::kElems(BK)];
  __shared__ __attribute__((aligned(16))) uint16_t v_s[2][L::kElems(BK)];

  if (p.err[0]) return;

  const WorkItem wi = map_work(blockIdx.x, p.n_qtiles_dq, p.hkv, p.n_hb, p.xcd_cluster_q);
  const int kvh = wi.kvh, hb = wi.hb;
  const int tile = min(max(p.lpt_q[wi.rank], 0), p.n_qtiles_dq - 1);
  const int32_t* pl = p.plan_q + (size_t)tile * QP_WORDS;
  const int l_row0 = pl[QP_LROW0], g_row0 = pl[QP_GROW0], nrows = pl[QP_NROWS];
  const int kt_lo = pl[QP_KT_LO], kt_flo = pl[QP_KT_FLO], kt_fhi = pl[QP_KT_FHI], kt_hi = pl[QP_KT_HI];

  // Lane l works on rows 16 r + (l mod 16) of the wave's 32 (r = 0, 1: the two
  // 16-row halves) and, in every 16 x 16 accumulator, on the four rows of
  // group g = l / 16.
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, g4 = lane >> 4, i16 = lane & 15;
  const int rb = wave / HB, hs = wave % HB;
  const int head = kvh * p.group + hb * HB + hs;
  int qr[2], gi[2];
  bool row_ok[2];
  size_t o_off[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    qr[r] = 32 * rb + 16 * r + i16;
    row_ok[r] = qr[r] < nrows;
    gi[r] = g_row0 + qr[r];
    o_off[r] = ((size_t)(l_row0 + qr[r]) * p.hq + head) * D;
  }
  const int tkv = p.kv_hi - p.kv_lo;
  const size_t kv_rstride = (size_t)p.hkv * D;
  const uint16_t* kbase = p.k + (size_t)kvh * D;
  const uint16_t* vbase = p.v + (size_t)kvh * D;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t row_bytes = (uint32_t)(kv_rstride * sizeof(uint16_t));
  // lane source offsets (bytes from the tile's first row) of this wave's loads
  uint32_t krow[DK], kchk[DK];
#pragma unroll
  for (int i = 0; i < DK; ++i) {
    const int q = (wave_u + NW * i) * 64 + lane, r = q / SK, pos = q % SK;
    krow[i] = (uint32_t)r * row_bytes;
    kchk[i] = 16u * (uint32_t)(D == 128 ? (pos ^ L::f(r)) : min(pos, CPK - 1));
  }
  const uint32_t k_wave = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)&k_s[0][0] + 1024u * wave_u;
  const uint32_t v_wave = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)&v_s[0][0] + 1024u * wave_u;
  // K and V tile kt into buffer BUF: uniform tile base + lane offsets; the
  // ragged last tile clamps the row part (padding keys read the last real row:
  // their scores are masked, any finite row will do)
  auto issue_tile = [&](int kt, auto buf_c) __attribute__((always_inline)) {
    constexpr int buf = decltype(buf_c)::value;
    const uint16_t* kb = kbase + (size_t)kt * BK * kv_rstride;
    const uint16_t* vb = vbase + (size_t)kt * BK * kv_rstride;
    const uint32_t lim = (uint32_t)max(tkv - 1 - kt * BK, 0) * row_bytes;
    static_for<DK>([&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value;
      if (NW * (i + 1) <= WK || wave_u + NW * i < WK)    // only the last load may be idle
        lds_dma16_so<(uint32_t)(buf * KTB + NW * 1024 * i)>(kb, min(krow[i], lim) + kchk[i], k_wave);
    });
    static_for<DK>([&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value;
      if (NW * (i + 1) <= WK || wave_u + NW * i < WK)
        lds_dma16_so<(uint32_t)(buf * KTB + NW * 1024 * i)>(vb, min(krow[i], lim) + kchk[i], v_wave);
    });
  };
  // the first K / V tile is in flight while the row operands load
  const int n = kt_hi - kt_lo;
  if (n > 0) issue_tile(kt_lo, std::integral_constant<int, 0>{});
  int a_lo[2], a_w[2];
  float lse2[2], dlt[2];
  bf16x8 qf[2][NKS], dof[2][NKS];      // row 16 r + l mod 16, d = 32 s + 8 g .. +8, k-step s
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    a_lo[r] = 0x40000000;
    a_w[r] = 0;
    lse2[r] = INFINITY;
    dlt[r] = 0.f;
    if (row_ok[r]) {
      // a row among its document's first kBwdHead positions attends only keys
      // among them: all of its pairs belong to the head pass (fp32)
      const int ds = doc_start(p.cu, p.n_docs, gi[r]);
      const int lo = max(ds, p.kv_lo), hi = min(gi[r], p.kv_hi - 1);
      if (hi >= lo && gi[r] - ds >= kBwdHead) { a_lo[r] = lo; a_w[r] = hi - lo; }
      const float lv = p.lse[(size_t)head * p.tq + l_row0 + qr[r]];
      lse2[r] = lv == -INFINITY ? INFINITY : lv * kLog2e;
      if (p.delta_ready) dlt[r] = p.delta[(size_t)head * p.tq + l_row0 + qr[r]];
    }
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      qf[r][s] = row_ok[r] ? *reinterpret_cast<const bf16x8*>(p.q + o_off[r] + 32 * s + 8 * g4) : bf16x8{};
      dof[r][s] = row_ok[r] ? *reinterpret_cast<const bf16x8*>(p.d_o + o_off[r] + 32 * s + 8 * g4) : bf16x8{};
    }
  }
  // Delta = rowsum(dO * O) for this row and head, unless the caller supplied
  // it: this lane's quarter of the row (d = 32 s + 8 g .. +8) from the dO
  // operands already in registers, then the sum over the row's four lanes.
  // Each (row, head) belongs to exactly one dQ work item, which stores it for
  // the dK/dV kernel that runs next.
  if (!p.delta_ready) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      float part = 0.f;
      if (row_ok[r]) {
#pragma unroll
        for (int s = 0; s < NKS; ++s) {
          const bf16x8 ov = *reinterpret_cast<const bf16x8*>(p.o + o_off[r] + 32 * s + 8 * g4);
#pragma unroll
          for (int e = 0; e < 8; ++e) part = __builtin_fmaf((float)ov[e], (float)dof[r][s][e], part);
        }
      }
      part += __shfl_xor(part, 16);
      dlt[r] = pair_sum32(part);
      if (row_ok[r] && g4 == 0) p.delta[(size_t)head * p.tq + l_row0 + qr[r]] = dlt[r];
    }
  }
  // dQ^T accumulators: d block b, row half r; lane group g holds d = 16 b + 4 g .. +3
  f32x4 dqacc[NDB][2];
#pragma unroll
  for (int b = 0; b < NDB; ++b) dqacc[b][0] = dqacc[b][1] = f32x4{};

  wait_vmem();
  __syncthreads();
  // K and V operand reads of S^T / dP^T: row 16 kb + (l mod 16), d = 32 s +
  // 8 g .. +8; one lane byte offset per k-step (the same in the K and V
  // tiles) plus a constant (buffer, 16-key block) in the instruction's offset
  // field (the swizzle repeats every 16 rows)
  constexpr int KRB = L::kRowElems * 2;                 // bytes per K row
  const char* kb_s = reinterpret_cast<const char*>(&k_s[0][0]);
  const char* vb_s = reinterpret_cast<const char*>(&v_s[0][0]);
  uint32_t ko[NKS];
#pragma unroll
  for (int s = 0; s < NKS; ++s) ko[s] = 2u * (uint32_t)L::off(i16, 32 * s + 8 * g4);
  // K^T operand of dQ^T += K^T dS^T (transpose reads, see lds_read_tr16): as
  // the supplier of group g, lane l names key row 4 g + (l mod 16) / 4 and
  // column 16 b + 4 (l mod 4), so lane l of the group receives keys 4 g ..
  // 4 g + 3 of column 16 b + (l mod 16).  The second read of a 32-key half
  // takes the keys 16 rows further (the dS^T operand's key order, as in the
  // forward).
  uint32_t kto[NDB];
#pragma unroll
  for (int b = 0; b < NDB; ++b) kto[b] = 2u * (uint32_t)L::off(4 * g4 + (i16 >> 2), 16 * b + 4 * (i16 & 3));
  // One KV tile (index u); the K / V buffer is a compile-time constant so
  // that LDS addresses fold into immediates.
  auto tile_step = [&](int u, auto buf_c) __attribute__((always_inline)) {
    constexpr int buf = decltype(buf_c)::value;
    constexpr int KB0 = buf * L::kElems(BK) * 2;          // byte offset of this K (and V) buffer
    const int kt = kt_lo + u;
    // the next tile into the other buffer (its last reader finished before
    // the previous barrier); in flight during this tile's math
    if (u + 1 < n) issue_tile(kt + 1, std::integral_constant<int, buf ^ 1>{});
    const bool partial = kt < kt_flo || kt >= kt_fhi || (kt + 1) * BK > tkv;
    // Each 32-key half t is one stream of LDS operands, each feeding the two
    // row halves: NSD slots of S^T / dP^T (slot j: k-step j / 4, key block
    // 2 t + (j / 2) % 2, a K row operand for j even and a V row operand for j
    // odd), the softmax, then NDB slots of dQ^T (K^T by transpose reads).
    // Every operand is read PF slots ahead, across the softmax and into the
    // next half's S^T / dP^T.
    constexpr int NSD = 4 * NKS, NH = NSD + NDB, PF = 2;
    bf16x8 opr[2 * NH];
    auto load = [&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value;
      constexpr int t = i / NH, j = i % NH;
      if constexpr (j < NSD) {
        constexpr int s = j / 4, kb = 2 * t + (j / 2) % 2;
        const char* base = j % 2 == 0 ? kb_s : vb_s;
        opr[i] = *reinterpret_cast<const bf16x8*>(base + ko[s] + (KB0 + 16 * kb * KRB));
      } else {
        constexpr int b = j - NSD;
        const char* kp = kb_s + kto[b] + (KB0 + 32 * t * KRB);
        opr[i] = tr_operand(reinterpret_cast<const uint16_t*>(kp), reinterpret_cast<const uint16_t*>(kp + 16 * KRB));
      }
    };
    static_for<PF>([&](auto ic) __attribute__((always_inline)) { load(ic); });
    static_for<2>([&](auto tc) __attribute__((always_inline)) {
      constexpr int t = decltype(tc)::value;
      // S^T and dP^T of the 32 keys 32 t .. +31 (16-key blocks kb = 2 t, 2 t + 1)
      // at raised wave priority (the other wave of the SIMD fills the gaps
      // with its vector work); dP^T starts from -Delta, so dS^T = P^T dP^T
      f32x4 sacc[2][2], dpacc[2][2];
#pragma unroll
      for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          sacc[k][r] = f32x4{};
          dpacc[k][r] = f32x4{-dlt[r], -dlt[r], -dlt[r], -dlt[r]};
        }
      __builtin_amdgcn_s_setprio(1);
      static_for<NSD>([&](auto jc) __attribute__((always_inline)) {
        constexpr int j = decltype(jc)::value, i = t * NH + j;
        if constexpr (i + PF < 2 * NH) load(std::integral_constant<int, i + PF>{});
        constexpr int s = j / 4, k = (j / 2) % 2;
        if constexpr (j % 2 == 0) {
          sacc[k][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(opr[i], qf[0][s], sacc[k][0], 0, 0, 0);
          sacc[k][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(opr[i], qf[1][s], sacc[k][1], 0, 0, 0);
        } else {
          dpacc[k][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(opr[i], dof[0][s], dpacc[k][0], 0, 0, 0);
          dpacc[k][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(opr[i], dof[1][s], dpacc[k][1], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      });
      __builtin_amdgcn_s_setprio(0);
      // document mask (PARTIAL and ragged tiles only, a wave-uniform branch):
      // masked scores become -inf, so P = 0
      if (partial) {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const int rel0 = p.kv_lo + kt * BK + 32 * t + 4 * g4 - a_lo[r];
#pragma unroll
          for (int k = 0; k < 2; ++k)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if ((unsigned)(rel0 + 16 * k + e) > (unsigned)a_w[r]) sacc[k][r][e] = -INFINITY;
        }
      }
      // P^T and dS^T of keys 32 t + 16 k + 4 g + e; the dS^T operand of row
      // half r in the key order {4 g .. 4 g + 3, 16 + 4 g .. 16 + 4 g + 3}
      bf16x8 dsb[2];
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        float ds[8];
#pragma unroll
        for (int k = 0; k < 2; ++k)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[k][r][e], p.scale_log2, -lse2[r]));
            ds[4 * k + e] = pr * dpacc[k][r][e];
          }
        dsb[r] = cvt8(ds[0], ds[1], ds[2], ds[3], ds[4], ds[5], ds[6], ds[7]);
      }
      __builtin_amdgcn_sched_barrier(0);
      static_for<NDB>([&](auto bc) __attribute__((always_inline)) {
        constexpr int b = decltype(bc)::value, i = t * NH + NSD + b;
        if constexpr (i + PF < 2 * NH) load(std::integral_constant<int, i + PF>{});
        dqacc[b][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(opr[i], dsb[0], dqacc[b][0], 0, 0, 0);
        dqacc[b][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(opr[i], dsb[1], dqacc[b][1], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      });
    });
    wait_vmem();
    __syncthreads();
  };
  for (int u = 0; u < n; u += 2) {
    tile_step(u, std::integral_constant<int, 0>{});
    if (u + 1 < n) tile_step(u + 1, std::integral_constant<int, 1>{});
  }

  // dQ = scale * acc: row 16 r + l mod 16, d = 16 b + 4 g .. +4 (added to dq for split-KV callers)
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    if (!row_ok[r]) continue;
#pragma unroll
    for (int b = 0; b < NDB; ++b) {
      float4 val = make_float4(dqacc[b][r][0] * p.scale, dqacc[b][r][1] * p.scale, dqacc[b][r][2] * p.scale,
                               dqacc[b][r][3] * p.scale);
      float4* dst = reinterpret_cast<float4*>(p.dq + o_off[r] + 16 * b + 4 * g4);
      if (p.accumulate_dq) {
        const float4 old = *dst;
        val.x += old.x; val.y += old.y; val.z += old.z; val.w += old.w;
      }
      *dst = val;
    }
  }
}

// ------------------------------------------------------------------ head pass
// The pairs (i, j) with ds <= j <= i < ds + kBwdHead of every document (ds its
// start) -- the rows with the fewest keys, whose P and dS are the largest --
// in fp32 throughout: the two kernels above leave them out, because rounding
// P and dS to the bf16 matrix-core operands costs the most there.  These rows
// also take their Delta from the pass's own P and dP when all their keys are
// in the call's KV range (the bf16 O that the other rows' Delta is formed
// from is least accurate for rows with few keys).  Workgroup =
// (document, KV head); it adds the pairs' dQ shares of the group's query heads
// into dq and their dK and dV (summed over those heads) into dk and dv, after
// both kernels have written them.  Only the pairs of this call count: rows in
// its chunks, keys in [kv_lo, kv_hi).  Disjoint outputs per workgroup: the
// result does not depend on the order in which workgroups run.
template <int D>
__global__ __launch_bounds__(256, 2) void head_kernel(BwdParams p, ChunkTable ch) {
  constexpr int H = kBwdHead;
  constexpr int DS = D + 4;             // LDS row stride (floats): 16-byte row reads of 16 rows on distinct banks
  constexpr int DG = D / 8;             // 8-wide d groups; 256 % DG == 0, so a thread keeps its d group
  constexpr int NT = (H * DG + 255) / 256;   // (row or key, d group) tasks per thread
  constexpr int NKS = D / 16;
  static_assert(H == 32, "the head block is one 32 x 32 MFMA tile");
  __shared__ __attribute__((aligned(16))) float ks[H][DS], vs[H][DS], qs[H][DS], dos[H][DS];
  __shared__ float ps[H][H + 1], dss[H][H + 1];
  __shared__ int rl[H];                 // local query row of head position t, -1 if not a row of this call
  __shared__ float lse2[H], dlt[H];

  if (p.err[0]) return;
  const int doc = blockIdx.x / p.hkv, kvh = blockIdx.x % p.hkv;
  const int a = p.cu[doc], b = p.cu[doc + 1];
  const int k0 = max(a, p.kv_lo), he = min(b, a + H), k1 = min(he, p.kv_hi);
  if (k1 <= k0) return;                 // no head key in this call's KV range
  const int nk = k1 - k0, nr = he - k0; // head keys [k0, k1); rows [k0, he) (a row before k0 has no such key)
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int dg0 = 8 * (tid % DG);       // this thread's d group

  if (tid < H) {
    int loc = -1;
    if (tid < nr) {
      const int g = k0 + tid;
      int off = 0;
      for (int c = 0; c < ch.n; ++c) {
        if (g >= ch.g_start[c] && g < ch.g_start[c] + ch.len[c]) { loc = off + g - ch.g_start[c]; break; }
        off += ch.len[c];
      }
    }
    rl[tid] = loc;
  }
  // K and V rows of the head keys (float: K for dQ, both for the S / dP
  // operands, converted back to bf16 exactly)
  for (int t = tid; t < H * DG; t += 256) {
    const int c = t / DG;
    float kf[8] = {}, vf[8] = {};
    if (c < nk) {
      const size_t off = ((size_t)(k0 + c - p.kv_lo) * p.hkv + kvh) * D + dg0;
      const bf16x8 kb = *reinterpret_cast<const bf16x8*>(p.k + off);
      const bf16x8 vb = *reinterpret_cast<const bf16x8*>(p.v + off);
#pragma unroll
      for (int e = 0; e < 8; ++e) { kf[e] = (float)kb[e]; vf[e] = (float)vb[e]; }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) { ks[c][dg0 + e] = kf[e]; vs[c][dg0 + e] = vf[e]; }
  }
  __syncthreads();
  bool any_row = false;
  for (int r = 0; r < nr; ++r) any_row |= rl[r] >= 0;
  if (!any_row) return;                 // no head row among this call's query rows

  // S and dP by v_mfma_f32_32x32x16_bf16 (exact bf16 products, fp32 sums):
  // wave 0 takes the 32 x 32 tile, lane l holding key column l % 32; all
  // operands come from the LDS rows.
  const int kcol = l32;

  float dka[NT][8], dva[NT][8];         // dK, dV of keys (tid + 256 i) / DG, summed over the group's heads
#pragma unroll
  for (int i = 0; i < NT; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) { dka[i][e] = 0.f; dva[i][e] = 0.f; }

  // Q and dO of this thread's fill tasks (row (tid + 256 i) / DG, its d
  // group), LSE and Delta of head position tid: loaded one head ahead, so
  // that their latency overlaps the previous head's work
  bf16x8 pq[NT], pd[NT];
  float plse = -INFINITY, pdlt = 0.f;
  auto prefetch = [&](int head) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int t = tid + 256 * i, r = min(t / DG, H - 1);
      const int lr = r < nr ? rl[r] : -1;
      pq[i] = bf16x8{};
      pd[i] = bf16x8{};
      if (lr >= 0 && t < H * DG) {
        const size_t off = ((size_t)lr * p.hq + head) * D + dg0;
        pq[i] = *reinterpret_cast<const bf16x8*>(p.q + off);
        pd[i] = *reinterpret_cast<const bf16x8*>(p.d_o + off);
      }
    }
    if (tid < H) {
      const int lr = tid < nr ? rl[tid] : -1;
      plse = -INFINITY;
      pdlt = 0.f;
      if (lr >= 0) {
        plse = p.lse[(size_t)head * p.tq + lr];
        pdlt = p.delta[(size_t)head * p.tq + lr];
      }
    }
  };
  prefetch(kvh * p.group);
  for (int hs = 0; hs < p.group; ++hs) {
    const int head = kvh * p.group + hs;
    // this head's Q and dO rows (float), LSE (base 2) and Delta into LDS
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int t = tid + 256 * i;
      if (t < H * DG) {
        const int r = t / DG;
#pragma unroll
        for (int e = 0; e < 8; ++e) { qs[r][dg0 + e] = (float)pq[i][e]; dos[r][dg0 + e] = (float)pd[i][e]; }
      }
    }
    if (tid < H) {
      lse2[tid] = plse == -INFINITY ? INFINITY : plse * kLog2e;
      dlt[tid] = pdlt;
    }
    __syncthreads();
    if (hs + 1 < p.group) prefetch(head + 1);
    f32x16 sacc = f32x16{}, pacc = f32x16{};
    if (wave == 0) {
      // A operands: this lane's row of the tile from the LDS rows (bf16
      // values, so the conversion back is exact)
      const int row = l32;
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        const float* qr_ = &qs[row][16 * s + 8 * hh];
        const float* dr_ = &dos[row][16 * s + 8 * hh];
        const float* kr_ = &ks[kcol][16 * s + 8 * hh];
        const float* vr_ = &vs[kcol][16 * s + 8 * hh];
        const bf16x8 qa = cvt8(qr_[0], qr_[1], qr_[2], qr_[3], qr_[4], qr_[5], qr_[6], qr_[7]);
        const bf16x8 da = cvt8(dr_[0], dr_[1], dr_[2], dr_[3], dr_[4], dr_[5], dr_[6], dr_[7]);
        const bf16x8 kb = cvt8(kr_[0], kr_[1], kr_[2], kr_[3], kr_[4], kr_[5], kr_[6], kr_[7]);
        const bf16x8 vb = cvt8(vr_[0], vr_[1], vr_[2], vr_[3], vr_[4], vr_[5], vr_[6], vr_[7]);
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kb, sacc, 0, 0, 0);
        pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da, vb, pacc, 0, 0, 0);
      }
    }
    if (wave == 0) {
      // element e of the tile: row 8 (e / 4) + 4 hh + e % 4, key kcol;
      // pairs outside the head triangle (key after row), or of rows not in
      // this call, get P = 0
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = 8 * (e >> 2) + 4 * hh + (e & 3);
        float pr = 0.f;
        if (r < nr && kcol < nk && kcol <= r && rl[r] >= 0)
          pr = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[e], p.scale_log2, -lse2[r]));
        ps[r][kcol] = pr;
        dss[r][kcol] = pacc[e];         // dP for now
      }
    }
    __syncthreads();
    // Delta of a head row whose keys all lie in this call's KV range: the
    // sum over them of P dP (= dO . O with O in fp32, not the bf16 O the
    // other rows' Delta comes from)
    if (tid < nr && rl[tid] >= 0 && a >= p.kv_lo && k0 + tid < p.kv_hi) {
      float acc = 0.f;
      for (int c = 0; c <= tid; ++c) acc = __builtin_fmaf(ps[tid][c], dss[tid][c], acc);
      dlt[tid] = acc;
    }
    __syncthreads();
    for (int t = tid; t < H * H; t += 256) {
      const int r = t / H, c = t % H;
      dss[r][c] = ps[r][c] * (dss[r][c] - dlt[r]);
    }
    __syncthreads();
    // dQ of the head rows (tid + 256 i) / DG: scale * sum_c dS[r][c] k_c,
    // added to dq (its old values load while the dK / dV sums run)
    float acc[NT][8];
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[i][e] = 0.f;
    {
      int rows_i[NT];                   // task rows, clamped (a clamped task's result is not written)
#pragma unroll
      for (int i = 0; i < NT; ++i) rows_i[i] = min((tid + 256 * i) / DG, H - 1);
#pragma unroll 4
      for (int c = 0; c < nk; ++c) {
        const f32x4 k0v = *reinterpret_cast<const f32x4*>(&ks[c][dg0]);
        const f32x4 k1v = *reinterpret_cast<const f32x4*>(&ks[c][dg0 + 4]);
#pragma unroll
        for (int i = 0; i < NT; ++i) {
          const float w = dss[rows_i[i]][c];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[i][e] = __builtin_fmaf(w, k0v[e], acc[i][e]);
            acc[i][4 + e] = __builtin_fmaf(w, k1v[e], acc[i][4 + e]);
          }
        }
      }
    }
    float* dqp[NT];
    float4 old[NT][2];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int r = (tid + 256 * i) / DG;
      const int lr = r < nr ? rl[r] : -1;   // r < nr <= H: not a clamped task
      dqp[i] = lr >= 0 ? p.dq + ((size_t)lr * p.hq + head) * D + dg0 : nullptr;
      if (dqp[i]) {
        old[i][0] = *reinterpret_cast<const float4*>(dqp[i]);
        old[i][1] = *reinterpret_cast<const float4*>(dqp[i] + 4);
      }
    }
    // dK and dV of the head keys (tid + 256 i) / DG: sums over the head rows
    {
      int keys_i[NT];                   // task keys, clamped (a clamped task's result is not written)
#pragma unroll
      for (int i = 0; i < NT; ++i) keys_i[i] = min((tid + 256 * i) / DG, H - 1);
#pragma unroll 4
      for (int r = 0; r < nr; ++r) {
        const f32x4 q0 = *reinterpret_cast<const f32x4*>(&qs[r][dg0]);
        const f32x4 q1 = *reinterpret_cast<const f32x4*>(&qs[r][dg0 + 4]);
        const f32x4 o0 = *reinterpret_cast<const f32x4*>(&dos[r][dg0]);
        const f32x4 o1 = *reinterpret_cast<const f32x4*>(&dos[r][dg0 + 4]);
#pragma unroll
        for (int i = 0; i < NT; ++i) {
          const float w = dss[r][keys_i[i]], pw = ps[r][keys_i[i]];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            dka[i][e] = __builtin_fmaf(w, q0[e], dka[i][e]);
            dka[i][4 + e] = __builtin_fmaf(w, q1[e], dka[i][4 + e]);
            dva[i][e] = __builtin_fmaf(pw, o0[e], dva[i][e]);
            dva[i][4 + e] = __builtin_fmaf(pw, o1[e], dva[i][4 + e]);
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      if (!dqp[i]) continue;
      const float4 n0 = make_float4(old[i][0].x + acc[i][0] * p.scale, old[i][0].y + acc[i][1] * p.scale,
                                    old[i][0].z + acc[i][2] * p.scale, old[i][0].w + acc[i][3] * p.scale);
      const float4 n1 = make_float4(old[i][1].x + acc[i][4] * p.scale, old[i][1].y + acc[i][5] * p.scale,
                                    old[i][1].z + acc[i][6] * p.scale, old[i][1].w + acc[i][7] * p.scale);
      *reinterpret_cast<float4*>(dqp[i]) = n0;
      *reinterpret_cast<float4*>(dqp[i] + 4) = n1;
    }
    __syncthreads();                    // before the next head's rows overwrite qs, dos, ps, dss
  }
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const int c = (tid + 256 * i) / DG;
    if (c >= nk) continue;              // c < nk <= H: not a clamped task
    const size_t off = ((size_t)(k0 + c - p.kv_lo) * p.hkv + kvh) * D + dg0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p.dk[off + e] += dka[i][e] * p.scale;
      p.dv[off + e] += dva[i][e];
    }
  }
}

// query heads per dQ work item: as many heads of the GQA group as divide it (<= 8)
static int dq_heads_per_item(int group) {
  return (group % 4 == 0) ? 4 : (group % 2 == 0) ? 2 : 1;
}

int dq_rows_per_tile(int group) { return 32 * (4 / dq_heads_per_item(group)); }

hipError_t launch_bwd(const BwdParams& p, const ChunkTable& ch, int d, bool delta_ready, hipStream_t stream) {
  // dQ first: unless the caller supplied Delta, its work items compute and
  // store it, and the dK/dV kernel reads it
  const int hb = dq_heads_per_item(p.group);
  BwdParams a = p;
  a.n_hb = p.group / hb;
  a.delta_ready = delta_ready ? 1 : 0;
  const long long nblk_q = (long long)p.n_qtiles_dq * p.hkv * a.n_hb;
  if (nblk_q > 0) {
    if (nblk_q > 0x7fffffffLL) return hipErrorInvalidValue;
    dim3 grid((unsigned)nblk_q), block(256);
    KernelTimer timer(KC_DQ, stream);
    if (d == 128) {
      if (hb == 4) hipLaunchKernelGGL((dq_kernel<128, 1, 4>), grid, block, 0, stream, a);
      else if (hb == 2) hipLaunchKernelGGL((dq_kernel<128, 2, 2>), grid, block, 0, stream, a);
      else hipLaunchKernelGGL((dq_kernel<128, 4, 1>), grid, block, 0, stream, a);
    } else {
      if (hb == 4) hipLaunchKernelGGL((dq_kernel<64, 1, 4>), grid, block, 0, stream, a);
      else if (hb == 2) hipLaunchKernelGGL((dq_kernel<64, 2, 2>), grid, block, 0, stream, a);
      else hipLaunchKernelGGL((dq_kernel<64, 4, 1>), grid, block, 0, stream, a);
    }
  }
  const long long nblk_kv = (long long)p.n_kvtiles * p.hkv;
  if (nblk_kv > 0) {
    if (nblk_kv > 0x7fffffffLL) return hipErrorInvalidValue;
    dim3 grid((unsigned)nblk_kv), block(256);
    KernelTimer timer(KC_DKDV, stream);
    if (d == 128) hipLaunchKernelGGL((dkdv_kernel<128>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((dkdv_kernel<64>), grid, block, 0, stream, p);
  }
  // the head pass adds to what both kernels wrote
  const long long nblk_h = (long long)p.n_docs * p.hkv;
  if (nblk_q > 0 && nblk_h > 0) {
    if (nblk_h > 0x7fffffffLL) return hipErrorInvalidValue;
    KernelTimer timer(KC_HEAD, stream);
    if (d == 128) hipLaunchKernelGGL((head_kernel<128>), dim3((unsigned)nblk_h), dim3(256), 0, stream, p, ch);
    else hipLaunchKernelGGL((head_kernel<64>), dim3((unsigned)nblk_h), dim3(256), 0, stream, p, ch);
  }
  return hipGetLastError();
}

}  // namespace docmask
