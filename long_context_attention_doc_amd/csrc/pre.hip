// Backward preprocessing kernel (the first of the backward's kernels; the
// others are in bwd.hip, which states the gradients they compute).
//
// Per query row i of the tile grid: Dv_i = dO_i . O_i, and the anchor
// column's terms P_i0 = exp(scale q'_i . k'_0 - LSE_i), dP_i0 = dO_i . v_0,
// dS_i0 = P_i0 (dP_i0 - Dv_i) (paper-graph architecture page of
// arXiv 2411.13476, "Mask construction": every query sees the anchor).  Per
// block of 64 rows: the dK/dV kernel's query record and the partial sums of
// dS_i0 q'_i and P_i0 dO_i that the anchor reduction adds into dk_0, dv_0.
// Built with the compiler's default scheduler (a memory-bound kernel; the
// attention kernels use the iterative ILP one).
#include <type_traits>

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
    const void* __restrict__ o, int o_f32, const bf16* __restrict__ dout,
    const float* __restrict__ lse,
    const int32_t* __restrict__ lo, const int32_t* __restrict__ hi, int S, int Hq, int Hkv,
    int nblk, float scale, int anchor, int origin, float* __restrict__ dvec,
    float* __restrict__ ds0, float* __restrict__ part_dk, float* __restrict__ part_dv,
    float* __restrict__ qstats, const int32_t* __restrict__ tok_map,
    const int32_t* __restrict__ status, bf16* __restrict__ dq) {
  constexpr int LPR = D / 8;                // lanes per row
  constexpr int RPP = 256 / LPR;            // rows per pass of the workgroup
  __shared__ float red_k[RPP][D + 4];
  __shared__ float red_v[RPP][D + 4];
  // heads fastest: neighbouring workgroups read neighbouring D-wide pieces
  // of the same token rows
  const int hq = blockIdx.x % Hq;
  const int rb = blockIdx.x / Hq;
  const int blk = rb % nblk, b = rb / nblk;
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
  // Blocks follow the query tiles of the tile grid (rows origin + 64*blk ..).
  // With the grid after the anchor, block 0 also takes the anchor row in a
  // pass of its own (slot 0 only): its Dv, its anchor-column terms and its
  // dq, which no query tile covers.
  //
  // NP passes of RPP rows each: every pass's row loads are issued before the
  // first row is reduced (one memory latency per workgroup instead of one
  // per pass), with the O type a compile-time choice so that no branch
  // splits the loads.
  auto run = [&](auto o_is_f32, auto np_c, int r_first, bool arow) {
    constexpr bool OF32 = decltype(o_is_f32)::value;
    constexpr int NP = decltype(np_c)::value;
    using OVec = std::conditional_t<OF32, f32x4, bf16x8>;
    int row[NP];
    bool valid[NP];
    size_t tok[NP], otok[NP];
    bf16x8 qv[NP], dv[NP];
    OVec ov[NP][OF32 ? 2 : 1];
    float L[NP];
    int lov[NP], hiv[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      row[p] = arow ? (slot == 0 ? 0 : S) : origin + blk * kPreRows + r_first + p * RPP + slot;
      valid[p] = row[p] < S;
      tok[p] = tok0 + (valid[p] ? row[p] : S - 1);
      otok[p] = tok[p];
    }
    if (tok_map) {   // the caller's O and LSE rows (one branch around all the loads)
#pragma unroll
      for (int p = 0; p < NP; ++p) otok[p] = (size_t)tok_map[tok[p]];
    }
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const size_t off = (tok[p] * Hq + hq) * D + f0;
      qv[p] = *(const bf16x8*)(qr + off);
      dv[p] = *(const bf16x8*)(dout + off);
      const size_t oo = (otok[p] * Hq + hq) * D + f0;
      if constexpr (OF32) {
        ov[p][0] = ((const f32x4*)((const float*)o + oo))[0];
        ov[p][1] = ((const f32x4*)((const float*)o + oo))[1];
      } else {
        ov[p][0] = *(const bf16x8*)((const bf16*)o + oo);
      }
      L[p] = lse[((size_t)b * Hq + hq) * S + (otok[p] - tok0)];
      lov[p] = lo[tok[p]];
      hiv[p] = hi[tok[p]];
    }
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      float of[8];
      if constexpr (OF32) {
#pragma unroll
        for (int i = 0; i < 4; ++i) { of[i] = ov[p][0][i]; of[4 + i] = ov[p][1][i]; }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) of[i] = (float)ov[p][0][i];
      }
      float d_o = 0.f, s0 = 0.f, dp0 = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float g = (float)dv[p][i];
        d_o += g * of[i];
        s0 += (float)qv[p][i] * k0[i];
        dp0 += g * v0[i];
      }
#pragma unroll
      for (int off2 = LPR / 2; off2 > 0; off2 >>= 1) {
        d_o += __shfl_xor(d_o, off2);
        s0 += __shfl_xor(s0, off2);
        dp0 += __shfl_xor(dp0, off2);
      }
      // without an anchor there is no anchor column: its weight and dS are zero
      const float p0 = valid[p] && anchor ? __builtin_amdgcn_exp2f((s0 * scale - L[p]) * kLog2e) : 0.f;
      const float dsv = p0 * (dp0 - d_o);
      if (valid[p] && (tid % LPR) == 0) {
        dvec[((size_t)b * Hq + hq) * S + row[p]] = d_o;
        ds0[((size_t)b * Hq + hq) * S + row[p]] = dsv;
      }
      if (arow && valid[p]) {
        // dq of the anchor row: scale * dS_00 k'_0, position 0 (no rotation)
        bf16x8 w;
        const bool bad = status[0] != kStatusOk;
#pragma unroll
        for (int i = 0; i < 8; ++i) w[i] = (bf16)(bad ? NAN : scale * dsv * k0[i]);
        *(bf16x8*)(dq + (otok[p] * Hq + hq) * D + f0) = w;
      }
      if ((tid % LPR) == 0 && !arow) {
        // tile-aligned record for the dK/dV kernel; rows past S see nothing
        float* rec = qstats + (((size_t)b * Hq + hq) * nblk + blk) * 4 * kPreRows;
        const int rr = r_first + p * RPP + slot;
        rec[rr] = valid[p] ? L[p] * kLog2e : 0.f;
        rec[kPreRows + rr] = valid[p] ? d_o : 0.f;
        rec[2 * kPreRows + rr] = __int_as_float(valid[p] ? lov[p] : 1);
        rec[3 * kPreRows + rr] = __int_as_float(valid[p] ? hiv[p] : 0);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        pk[i] += dsv * (float)qv[p][i];
        pv[i] += p0 * (float)dv[p][i];
      }
    }
  };
  constexpr int kPasses = kPreRows / RPP;
  static_assert(kPasses * RPP == kPreRows, "whole passes per block");
  auto all = [&](auto o_is_f32) {
    if (origin && blk == 0) run(o_is_f32, std::integral_constant<int, 1>{}, 0, true);
    run(o_is_f32, std::integral_constant<int, kPasses>{}, 0, false);
  };
  if (o_f32) all(std::true_type{});
  else all(std::false_type{});
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


// ---------------------------------------------------------------- launcher
hipError_t launch_bwd_pre(const BwdArgs& a, hipStream_t st) {
  const long long blocks = (long long)a.Hq * a.B * a.nblk;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)blocks);
  if (a.D == 128)
    hipLaunchKernelGGL(k_bwd_pre<128>, grid, dim3(256), 0, st, a.qr, a.kr, a.v, a.o, a.o_f32, a.dout,
                       a.lse, a.tt.lo, a.tt.hi, a.S, a.Hq, a.Hkv, a.nblk, a.scale, a.anchor, a.origin,
                       a.dvec, a.ds0, a.part_dk, a.part_dv, a.qstats, a.tok_map, a.status, a.dq);
  else
    hipLaunchKernelGGL(k_bwd_pre<64>, grid, dim3(256), 0, st, a.qr, a.kr, a.v, a.o, a.o_f32, a.dout,
                       a.lse, a.tt.lo, a.tt.hi, a.S, a.Hq, a.Hkv, a.nblk, a.scale, a.anchor, a.origin,
                       a.dvec, a.ds0, a.part_dk, a.part_dv, a.qstats, a.tok_map, a.status, a.dq);
  return hipGetLastError();
}

}  // namespace aa
