// Backward attention kernels.
//
// Gradients of L with respect to q, k, v given dO = dL/dO, for the operation
// of the forward kernel (paper-graph architecture page of arXiv 2411.13476,
// section 3.4: "Standard attention", Eq. 6 RoPE, "Mask construction").  With
// P the masked softmax, q', k' the rotated inputs and R(pos) the rotation:
//   dV_j  = sum_i P_ij dO_i                  Dv_i = dO_i . O_i
//   dP_ij = dO_i . v_j                       dS_ij = P_ij (dP_ij - Dv_i)
//   dq_i  = R(pos_i)^T  scale sum_j dS_ij k'_j
//   dk_j  = R(pos_j)^T  scale sum_i dS_ij q'_i
// Key gradients also sum over the query heads of a grouped-query group.
//
// Four kernels, all without atomics:
//   pre    per query row: Dv_i, and the anchor column's P_i0 and dS_i0; per
//          block of 64 rows, partial sums of dS_i0 q'_i and P_i0 dO_i;
//   dkdv   per (row b, kv head, key tile of 128): K and V stay in registers,
//          the live query tiles of the key-major plan stream through LDS;
//   dq     per (row b, query head, query tile of 128): the structure of the
//          forward kernel, recomputing S and dP from LSE; adds the anchor
//          column's term and un-rotates;
//   anchor per (row b, kv head): reduces the partial sums into dk_0, dv_0.
// A float32 atomic accumulation of dq across key tiles would move about
// 34 GB at 64K tokens x 32 heads and is limited by the L2 atomic rate, so dq
// is recomputed query-major instead (deterministic, no dq scratch).
#include "aa_internal.h"

namespace aa {

constexpr float kLog2e = 1.44269504088896340736f;

// ---------------------------------------------------------------------------
// pre: one workgroup per (row b, query head, block of kPreRows rows).
// D/8 lanes share one row, 8 features each.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void k_bwd_pre(
    const bf16* __restrict__ qr, const bf16* __restrict__ kr, const bf16* __restrict__ v,
    const bf16* __restrict__ o, const bf16* __restrict__ dout, const float* __restrict__ lse,
    int S, int Hq, int Hkv, int nblk, float scale, float* __restrict__ dvec,
    float* __restrict__ ds0, float* __restrict__ part_dk, float* __restrict__ part_dv) {
  constexpr int LPR = D / 8;                // lanes per row
  constexpr int RPP = 256 / LPR;            // rows per pass of the workgroup
  __shared__ float red_k[RPP][D + 4];
  __shared__ float red_v[RPP][D + 4];
  const int blk = blockIdx.x % nblk, b = blockIdx.x / nblk;
  const int hq = blockIdx.y;
  const int hkv = hq / (Hq / Hkv);
  const int tid = threadIdx.x;
  const int slot = tid / LPR, f0 = (tid % LPR) * 8;
  const size_t tok0 = (size_t)b * S;
  float k0[8], v0[8];
  {
    const bf16x8 kk = *(const bf16x8*)(kr + (tok0 * Hkv + hkv) * D + f0);
    const bf16x8 vv = *(const bf16x8*)(v + (tok0 * Hkv + hkv) * D + f0);
#pragma unroll
    for (int i = 0; i < 8; ++i) { k0[i] = (float)kk[i]; v0[i] = (float)vv[i]; }
  }
  float pk[8] = {0, 0, 0, 0, 0, 0, 0, 0}, pv[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int r0 = 0; r0 < kPreRows; r0 += RPP) {
    const int row = blk * kPreRows + r0 + slot;
    const bool valid = row < S;
    const size_t tok = tok0 + (valid ? row : S - 1);
    const size_t off = (tok * Hq + hq) * D + f0;
    const bf16x8 qv = *(const bf16x8*)(qr + off);
    const bf16x8 ov = *(const bf16x8*)(o + off);
    const bf16x8 dv = *(const bf16x8*)(dout + off);
    float d_o = 0.f, s0 = 0.f, dp0 = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float g = (float)dv[i];
      d_o += g * (float)ov[i];
      s0 += (float)qv[i] * k0[i];
      dp0 += g * v0[i];
    }
#pragma unroll
    for (int off2 = LPR / 2; off2 > 0; off2 >>= 1) {
      d_o += __shfl_xor(d_o, off2);
      s0 += __shfl_xor(s0, off2);
      dp0 += __shfl_xor(dp0, off2);
    }
    const float L = lse[((size_t)b * Hq + hq) * S + (valid ? row : S - 1)];
    float p0 = valid ? exp2f((s0 * scale - L) * kLog2e) : 0.f;
    const float dsv = p0 * (dp0 - d_o);
    if (valid && (tid % LPR) == 0) {
      dvec[((size_t)b * Hq + hq) * S + row] = d_o;
      ds0[((size_t)b * Hq + hq) * S + row] = dsv;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pk[i] += dsv * (float)qv[i];
      pv[i] += p0 * (float)dv[i];
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    red_k[slot][f0 + i] = pk[i];
    red_v[slot][f0 + i] = pv[i];
  }
  __syncthreads();
  for (int d = tid; d < D; d += 256) {
    float sk = 0.f, sv = 0.f;
    for (int r = 0; r < RPP; ++r) { sk += red_k[r][d]; sv += red_v[r][d]; }
    const size_t pidx = (((size_t)b * Hq + hq) * nblk + blk) * D + d;
    part_dk[pidx] = sk;
    part_dv[pidx] = sv;
  }
}

// ---------------------------------------------------------------------------
// dkdv: one workgroup (4 waves) per (row b, kv head, key tile of 128 keys);
// each wave owns 32 keys.  In this kernel the MFMA accumulators are laid out
// with keys as columns, so that P, dS (query x key) feed the B operand of
// dV^T = dO^T P and dK^T = Q^T dS directly.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256, 1) void k_bwd_dkdv(
    const bf16* __restrict__ qr, const bf16* __restrict__ kr, const bf16* __restrict__ v,
    const bf16* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ dvec,
    const float* __restrict__ table, const int32_t* __restrict__ pos,
    const int32_t* __restrict__ lo, const int32_t* __restrict__ hi,
    const int32_t* __restrict__ kptr, const int32_t* __restrict__ qidx,
    const uint8_t* __restrict__ qkind, const int32_t* __restrict__ status, int S, int Hq, int Hkv,
    int nk, float scale, bf16* __restrict__ dk, bf16* __restrict__ dv) {
  constexpr int BM = kDkvBM, BN = kDkvBN;
  constexpr int RST = D + 8;     // row-major tile stride (bf16)
  constexpr int TST = BM + 4;    // transposed tile stride (bf16)
  constexpr int NKK = D / 16;
  constexpr int NDB = D / 32;
  constexpr int NQB = BM / 32;   // 32-query blocks of a query tile
  constexpr int NQC = BM / 16;   // 16-query reduction steps
  constexpr int GROUPS = (BM / 4) * (D / 8);
  __shared__ __align__(16) bf16 Qs[BM * RST];
  __shared__ __align__(16) bf16 Qt[D * TST];
  __shared__ __align__(16) bf16 Gs[BM * RST];    // dO
  __shared__ __align__(16) bf16 Gt[D * TST];
  __shared__ float s_lse[BM], s_dv[BM];
  __shared__ int s_lo[BM], s_hi[BM];

  const int b = blockIdx.x / nk, kt = blockIdx.x % nk;
  const int hkv = blockIdx.y;
  const int group = Hq / Hkv;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int h = lane >> 5, col = lane & 31;
  const int key = kt * BN + wave * 32 + col;       // row-local key of this lane's column
  const bool kvalid = key < S;
  const size_t tok0 = (size_t)b * S;
  const size_t ktok = tok0 + (kvalid ? key : S - 1);
  const bool bad = status[0] != kStatusOk;
  const float scale_log2 = scale * kLog2e;

  // K^T and V^T operands: lane holds key `col`, features 16*kk + 8*h + i.
  bf16x8 kf[NKK], vf[NKK];
  {
    const bf16* kp = kr + (ktok * Hkv + hkv) * D + 8 * h;
    const bf16* vp = v + (ktok * Hkv + hkv) * D + 8 * h;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      kf[kk] = *(const bf16x8*)(kp + 16 * kk);
      vf[kk] = *(const bf16x8*)(vp + 16 * kk);
    }
  }
  f32x16 dka[NDB], dva[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) { dka[db][j] = 0.f; dva[db][j] = 0.f; }

  // Staging: each thread owns 4 consecutive query rows x 8 features of Q
  // and of dO; it writes them row-major and transposed.
  const int g_row = (tid / (D / 8)) * 4, g_f = (tid % (D / 8)) * 8;
  bf16x8 qreg[4], greg[4];
  float r_lse = 0.f, r_dv = 0.f;
  int r_lo = 1, r_hi = 0;
  const size_t q_row_stride = (size_t)Hq * D;

  auto gload = [&](int hq, int qt) {
    if (tid < GROUPS) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int q = min(qt * BM + g_row + r, S - 1);
        const size_t off = (tok0 + q) * q_row_stride + (size_t)hq * D + g_f;
        qreg[r] = *(const bf16x8*)(qr + off);
        greg[r] = *(const bf16x8*)(dout + off);
      }
    }
    if (tid < BM) {
      const int q = qt * BM + tid;
      const int qc = min(q, S - 1);
      r_lse = lse[((size_t)b * Hq + hq) * S + qc] * kLog2e;
      r_dv = dvec[((size_t)b * Hq + hq) * S + qc];
      r_lo = q < S ? lo[tok0 + qc] : 1;
      r_hi = q < S ? hi[tok0 + qc] : 0;
    }
  };
  auto lstore = [&]() {
    if (tid < GROUPS) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        *(bf16x8*)(Qs + (g_row + r) * RST + g_f) = qreg[r];
        *(bf16x8*)(Gs + (g_row + r) * RST + g_f) = greg[r];
      }
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        bf16x4 a, c;
        a[0] = qreg[0][dd]; a[1] = qreg[1][dd]; a[2] = qreg[2][dd]; a[3] = qreg[3][dd];
        c[0] = greg[0][dd]; c[1] = greg[1][dd]; c[2] = greg[2][dd]; c[3] = greg[3][dd];
        *(bf16x4*)(Qt + (g_f + dd) * TST + g_row) = a;
        *(bf16x4*)(Gt + (g_f + dd) * TST + g_row) = c;
      }
    }
    if (tid < BM) {
      s_lse[tid] = r_lse;
      s_dv[tid] = r_dv;
      s_lo[tid] = r_lo;
      s_hi[tid] = r_hi;
    }
  };

  const int e_begin = kptr[blockIdx.x], e_end = kptr[blockIdx.x + 1];
  // Work list: every q head of the group x every live, not anchor-only query tile.
  int e = e_begin, hi_q = hkv * group;
  auto advance = [&](int& ee, int& hh) {
    do {
      ++ee;
      if (ee >= e_end) { ee = e_begin; ++hh; }
    } while (hh < (hkv + 1) * group && qkind[ee] == kTileAnchor);
  };
  // first item
  if (e_begin < e_end) {
    while (e < e_end && qkind[e] == kTileAnchor) ++e;
    if (e >= e_end) hi_q = (hkv + 1) * group;   // nothing live besides the anchor
  } else {
    hi_q = (hkv + 1) * group;
  }
  if (hi_q < (hkv + 1) * group) gload(hi_q, qidx[e]);

  while (hi_q < (hkv + 1) * group) {
    const int qt = qidx[e];
    const bool need_mask = qkind[e] != kTileFull || kt == 0;
    __syncthreads();
    lstore();
    __syncthreads();
    int e_next = e, h_next = hi_q;
    advance(e_next, h_next);
    if (h_next < (hkv + 1) * group) gload(h_next, qidx[e_next]);

    // S = Q K^T and dP = dO V^T: columns = this wave's keys, rows = queries.
    f32x16 sp[NQB], dp[NQB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
#pragma unroll
      for (int j = 0; j < 16; ++j) { sp[qb][j] = 0.f; dp[qb][j] = 0.f; }
      const bf16* qa = Qs + (qb * 32 + col) * RST + 8 * h;
      const bf16* ga = Gs + (qb * 32 + col) * RST + 8 * h;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        sp[qb] = mfma32(*(const bf16x8*)(qa + 16 * kk), kf[kk], sp[qb]);
        dp[qb] = mfma32(*(const bf16x8*)(ga + 16 * kk), vf[kk], dp[qb]);
      }
    }
    // P = exp2(s * scale_log2 - lse_log2), dS = P (dP - Dv).
    bf16x8 pbv[NQC], dsb[NQC];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int qi = qb * 32 + 8 * (j >> 2) + 4 * h + (j & 3);   // tile-local query
        float p = exp2f(sp[qb][j] * scale_log2 - s_lse[qi]);
        if (need_mask) p = (key >= s_lo[qi] && key <= s_hi[qi]) ? p : 0.f;
        const float ds = p * (dp[qb][j] - s_dv[qi]);
        pbv[2 * qb + (j >> 3)][j & 7] = (bf16)p;
        dsb[2 * qb + (j >> 3)][j & 7] = (bf16)ds;
      }
    // dV^T += dO^T P ; dK^T += Q^T dS  (reduction over queries, accumulator
    // order of 16-query steps: rows 0-3, 8-11 in lanes 0-31; 4-7, 12-15 above)
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const bf16* gta = Gt + (32 * db + col) * TST + 4 * h;
      const bf16* qta = Qt + (32 * db + col) * TST + 4 * h;
#pragma unroll
      for (int c = 0; c < NQC; ++c) {
        const bf16x4 g0 = *(const bf16x4*)(gta + 16 * c), g1 = *(const bf16x4*)(gta + 16 * c + 8);
        const bf16x4 q0 = *(const bf16x4*)(qta + 16 * c), q1 = *(const bf16x4*)(qta + 16 * c + 8);
        bf16x8 ga, qa;
        ga[0] = g0[0]; ga[1] = g0[1]; ga[2] = g0[2]; ga[3] = g0[3];
        ga[4] = g1[0]; ga[5] = g1[1]; ga[6] = g1[2]; ga[7] = g1[3];
        qa[0] = q0[0]; qa[1] = q0[1]; qa[2] = q0[2]; qa[3] = q0[3];
        qa[4] = q1[0]; qa[5] = q1[1]; qa[6] = q1[2]; qa[7] = q1[3];
        dva[db] = mfma32(ga, pbv[c], dva[db]);
        dka[db] = mfma32(qa, dsb[c], dka[db]);
      }
    }
    e = e_next;
    hi_q = h_next;
  }

  // Epilogue: dK = R(pos)^T (scale * dK'), dV as accumulated.
  if (kvalid) {
    const int p = pos[ktok];
    const float* tb = table + (size_t)p * D;      // (D/2) pairs of {cos, sin}
    bf16* dkp = dk + (ktok * Hkv + hkv) * D;
    bf16* dvp = dv + (ktok * Hkv + hkv) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * db + 8 * g + 4 * h;     // features d0 .. d0+3 = pairs d0/2, d0/2+1
        bf16x4 wk, wv;
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
          const float c = tb[d0 + 2 * pr], s = tb[d0 + 2 * pr + 1];
          const float x0 = dka[db][4 * g + 2 * pr] * scale, x1 = dka[db][4 * g + 2 * pr + 1] * scale;
          wk[2 * pr] = (bf16)(bad ? NAN : x0 * c + x1 * s);
          wk[2 * pr + 1] = (bf16)(bad ? NAN : x1 * c - x0 * s);
          wv[2 * pr] = (bf16)(bad ? NAN : dva[db][4 * g + 2 * pr]);
          wv[2 * pr + 1] = (bf16)(bad ? NAN : dva[db][4 * g + 2 * pr + 1]);
        }
        *(bf16x4*)(dkp + d0) = wk;
        *(bf16x4*)(dvp + d0) = wv;
      }
  }
}

// ---------------------------------------------------------------------------
// dq: one workgroup (4 waves) per (row b, query head, query tile of 128);
// each wave owns 32 queries, as in the forward kernel.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256, 2) void k_bwd_dq(
    const bf16* __restrict__ qr, const bf16* __restrict__ kr, const bf16* __restrict__ v,
    const bf16* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ dvec,
    const float* __restrict__ ds0, const float* __restrict__ table,
    const int32_t* __restrict__ pos, const int32_t* __restrict__ lo,
    const int32_t* __restrict__ hi, const int32_t* __restrict__ qptr,
    const int32_t* __restrict__ kidx, const uint8_t* __restrict__ kkind,
    const int32_t* __restrict__ status, int S, int Hq, int Hkv, int nq, float scale,
    bf16* __restrict__ dq) {
  constexpr int BM = kFwdBM, BN = kFwdBN;
  constexpr int RST = D + 8;
  constexpr int TST = BN + 4;
  constexpr int NKK = D / 16;
  constexpr int NDB = D / 32;
  constexpr int NKB = BN / 32;
  constexpr int NKC = BN / 16;
  constexpr int GROUPS = (BN / 4) * (D / 8);
  __shared__ __align__(16) bf16 Ks[BN * RST];
  __shared__ __align__(16) bf16 Vs[BN * RST];
  __shared__ __align__(16) bf16 Kt[D * TST];

  const int tile = blockIdx.x;
  const int hq = blockIdx.y;
  const int b = tile / nq, qt = tile % nq;
  const int hkv = hq / (Hq / Hkv);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int h = lane >> 5, col = lane & 31;
  const int qrow = qt * BM + wave * 32 + col;
  const bool qvalid = qrow < S;
  const size_t tok0 = (size_t)b * S;
  const size_t tok = tok0 + (qvalid ? qrow : S - 1);
  int qlo = lo[tok], qhi = hi[tok];
  if (!qvalid) { qlo = 1; qhi = 0; }
  const bool bad = status[0] != kStatusOk;
  const float scale_log2 = scale * kLog2e;
  const size_t rowstat = ((size_t)b * Hq + hq) * S + (qvalid ? qrow : S - 1);
  const float lse2 = lse[rowstat] * kLog2e;
  const float dvi = dvec[rowstat];

  bf16x8 qf[NKK], gf[NKK];
  {
    const size_t off = (tok * Hq + hq) * D + 8 * h;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      qf[kk] = *(const bf16x8*)(qr + off + 16 * kk);
      gf[kk] = *(const bf16x8*)(dout + off + 16 * kk);
    }
  }
  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[db][j] = 0.f;

  const size_t kv_row_stride = (size_t)Hkv * D;
  const bf16* kbase = kr + tok0 * kv_row_stride + hkv * D;
  const bf16* vbase = v + tok0 * kv_row_stride + hkv * D;
  const int g_key = (tid / (D / 8)) * 4, g_f = (tid % (D / 8)) * 8;
  bf16x8 kreg[4], vreg[4];

  auto gload = [&](int kt) {
    if (tid < GROUPS) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = min(kt * BN + g_key + r, S - 1);
        kreg[r] = *(const bf16x8*)(kbase + key * kv_row_stride + g_f);
        vreg[r] = *(const bf16x8*)(vbase + key * kv_row_stride + g_f);
      }
    }
  };
  auto lstore = [&]() {
    if (tid < GROUPS) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        *(bf16x8*)(Ks + (g_key + r) * RST + g_f) = kreg[r];
        *(bf16x8*)(Vs + (g_key + r) * RST + g_f) = vreg[r];
      }
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        bf16x4 w;
        w[0] = kreg[0][dd]; w[1] = kreg[1][dd]; w[2] = kreg[2][dd]; w[3] = kreg[3][dd];
        *(bf16x4*)(Kt + (g_f + dd) * TST + g_key) = w;
      }
    }
  };

  int e = qptr[tile];
  const int e_end = qptr[tile + 1];
  if (e < e_end && kkind[e] == kTileAnchor) ++e;
  if (e < e_end) gload(kidx[e]);
  while (e < e_end) {
    const int kt = kidx[e];
    const bool need_mask = kkind[e] != kTileFull || kt == 0;
    __syncthreads();
    lstore();
    __syncthreads();
    if (e + 1 < e_end) gload(kidx[e + 1]);

    // S^T = K Q^T, dP^T = V dO^T: rows = keys, columns = this wave's queries.
    f32x16 st[NKB], dpt[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int j = 0; j < 16; ++j) { st[kb][j] = 0.f; dpt[kb][j] = 0.f; }
      const bf16* ka = Ks + (kb * 32 + col) * RST + 8 * h;
      const bf16* va = Vs + (kb * 32 + col) * RST + 8 * h;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        st[kb] = mfma32(*(const bf16x8*)(ka + 16 * kk), qf[kk], st[kb]);
        dpt[kb] = mfma32(*(const bf16x8*)(va + 16 * kk), gf[kk], dpt[kb]);
      }
    }
    bf16x8 dsb[NKC];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        float p = exp2f(st[kb][j] * scale_log2 - lse2);
        if (need_mask) {
          const int key = kt * BN + kb * 32 + 8 * (j >> 2) + 4 * h + (j & 3);
          p = (key >= qlo && key <= qhi) ? p : 0.f;
        }
        dsb[2 * kb + (j >> 3)][j & 7] = (bf16)(p * (dpt[kb][j] - dvi));
      }
    // dQ^T += K^T dS^T
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const bf16* ta = Kt + (32 * db + col) * TST + 4 * h;
#pragma unroll
      for (int c = 0; c < NKC; ++c) {
        const bf16x4 a0 = *(const bf16x4*)(ta + 16 * c), a1 = *(const bf16x4*)(ta + 16 * c + 8);
        bf16x8 a;
        a[0] = a0[0]; a[1] = a0[1]; a[2] = a0[2]; a[3] = a0[3];
        a[4] = a1[0]; a[5] = a1[1]; a[6] = a1[2]; a[7] = a1[3];
        acc[db] = mfma32(a, dsb[c], acc[db]);
      }
    }
    ++e;
  }

  // Epilogue: dq' = scale (acc + dS_i0 k'_0); dq = R(pos_i)^T dq'.
  if (qvalid) {
    const float a0 = ds0[rowstat];
    const bf16* k0 = kr + (tok0 * Hkv + hkv) * D;
    const int p = pos[tok];
    const float* tb = table + (size_t)p * D;
    bf16* dqp = dq + (tok * Hq + hq) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * db + 8 * g + 4 * h;
        const bf16x4 kz = *(const bf16x4*)(k0 + d0);
        bf16x4 w;
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
          const float c = tb[d0 + 2 * pr], s = tb[d0 + 2 * pr + 1];
          const float x0 = scale * (acc[db][4 * g + 2 * pr] + a0 * (float)kz[2 * pr]);
          const float x1 = scale * (acc[db][4 * g + 2 * pr + 1] + a0 * (float)kz[2 * pr + 1]);
          w[2 * pr] = (bf16)(bad ? NAN : x0 * c + x1 * s);
          w[2 * pr + 1] = (bf16)(bad ? NAN : x1 * c - x0 * s);
        }
        *(bf16x4*)(dqp + d0) = w;
      }
  }
}

// ---------------------------------------------------------------------------
// anchor: one workgroup per (row b, kv head); thread d sums the partials of
// the group's query heads and row blocks into dk_0[d], dv_0[d].  The anchor's
// position is 0, so R(0)^T = I.
// ---------------------------------------------------------------------------
__global__ void k_bwd_anchor(const float* __restrict__ part_dk, const float* __restrict__ part_dv,
                             const int32_t* __restrict__ status, int S, int Hq, int Hkv, int D,
                             int nblk, float scale, bf16* __restrict__ dk, bf16* __restrict__ dv) {
  const int b = blockIdx.x, hkv = blockIdx.y;
  const int group = Hq / Hkv;
  const bool bad = status[0] != kStatusOk;
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    float sk = 0.f, sv = 0.f;
    for (int hq = hkv * group; hq < (hkv + 1) * group; ++hq) {
      const float* pk = part_dk + ((size_t)b * Hq + hq) * nblk * D + d;
      const float* pv = part_dv + ((size_t)b * Hq + hq) * nblk * D + d;
      for (int n = 0; n < nblk; ++n) { sk += pk[(size_t)n * D]; sv += pv[(size_t)n * D]; }
    }
    const size_t off = ((size_t)b * S * Hkv + hkv) * D + d;
    dk[off] = (bf16)(bad ? NAN : sk * scale);
    dv[off] = (bf16)(bad ? NAN : sv);
  }
}

// ---------------------------------------------------------------- launchers
hipError_t launch_bwd_pre(const BwdArgs& a, hipStream_t st) {
  const dim3 grid(a.B * a.nblk, a.Hq);
  if (a.D == 128)
    hipLaunchKernelGGL(k_bwd_pre<128>, grid, dim3(256), 0, st, a.qr, a.kr, a.v, a.o, a.dout,
                       a.lse, a.S, a.Hq, a.Hkv, a.nblk, a.scale, a.dvec, a.ds0, a.part_dk,
                       a.part_dv);
  else
    hipLaunchKernelGGL(k_bwd_pre<64>, grid, dim3(256), 0, st, a.qr, a.kr, a.v, a.o, a.dout,
                       a.lse, a.S, a.Hq, a.Hkv, a.nblk, a.scale, a.dvec, a.ds0, a.part_dk,
                       a.part_dv);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv(const BwdArgs& a, const PlanBufs& pk, hipStream_t st) {
  const dim3 grid(a.B * pk.nk, a.Hkv);
  if (a.D == 128)
    hipLaunchKernelGGL(k_bwd_dkdv<128>, grid, dim3(256), 0, st, a.qr, a.kr, a.v, a.dout, a.lse,
                       a.dvec, a.table, a.tt.pos, a.tt.lo, a.tt.hi, pk.kptr, pk.qidx, pk.qkind,
                       a.status, a.S, a.Hq, a.Hkv, pk.nk, a.scale, a.dk, a.dv);
  else
    hipLaunchKernelGGL(k_bwd_dkdv<64>, grid, dim3(256), 0, st, a.qr, a.kr, a.v, a.dout, a.lse,
                       a.dvec, a.table, a.tt.pos, a.tt.lo, a.tt.hi, pk.kptr, pk.qidx, pk.qkind,
                       a.status, a.S, a.Hq, a.Hkv, pk.nk, a.scale, a.dk, a.dv);
  return hipGetLastError();
}

hipError_t launch_bwd_dq(const BwdArgs& a, const PlanBufs& pq, hipStream_t st) {
  const dim3 grid(a.B * pq.nq, a.Hq);
  if (a.D == 128)
    hipLaunchKernelGGL(k_bwd_dq<128>, grid, dim3(256), 0, st, a.qr, a.kr, a.v, a.dout, a.lse,
                       a.dvec, a.ds0, a.table, a.tt.pos, a.tt.lo, a.tt.hi, pq.qptr, pq.kidx,
                       pq.kkind, a.status, a.S, a.Hq, a.Hkv, pq.nq, a.scale, a.dq);
  else
    hipLaunchKernelGGL(k_bwd_dq<64>, grid, dim3(256), 0, st, a.qr, a.kr, a.v, a.dout, a.lse,
                       a.dvec, a.ds0, a.table, a.tt.pos, a.tt.lo, a.tt.hi, pq.qptr, pq.kidx,
                       pq.kkind, a.status, a.S, a.Hq, a.Hkv, pq.nq, a.scale, a.dq);
  return hipGetLastError();
}

hipError_t launch_bwd_anchor(const BwdArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_bwd_anchor, dim3(a.B, a.Hkv), dim3(128), 0, st, a.part_dk, a.part_dv,
                     a.status, a.S, a.Hq, a.Hkv, a.D, a.nblk, a.scale, a.dk, a.dv);
  return hipGetLastError();
}

}  // namespace aa
