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
// Four kernels, all without atomics (the first in pre.hip):
//   pre    per query row: Dv_i, and the anchor column's P_i0 and dS_i0; per
//          block of 64 rows, partial sums of dS_i0 q'_i and P_i0 dO_i;
//   dkdv   per (row b, kv head, key tile of 128): K in LDS and V in
//          registers for the whole kernel, the live query tiles of the
//          key-major plan stream through LDS;
//   dq     per (row b, query head, query tile of 128): the structure of the
//          forward kernel, recomputing S and dP from LSE; adds the anchor
//          column's term and un-rotates;
//   anchor per (row b, kv head): reduces the partial sums into dk_0, dv_0.
// A float32 atomic accumulation of dq across key tiles would move about
// 34 GB at 64K tokens x 32 heads and is limited by the L2 atomic rate, so dq
// is recomputed query-major instead (deterministic, no dq scratch).
#include <type_traits>

#include "aa_internal.h"

namespace aa {

constexpr float kLog2e = 1.44269504088896340736f;

// ---------------------------------------------------------------------------
// dkdv: one workgroup of four waves per (row b, kv head, key tile of 128 keys),
// two workgroups per CU.  Wave w owns keys [32w, 32w+32) of the tile for
// every query, so nothing is reduced across waves; a 64-query tile of the
// plan is taken as two 32-query halves.  The two waves that share a SIMD
// belong to different workgroups and are not held in step by a barrier.
//   * The workgroup's K rows sit in LDS with padded rows (B operand of
//     S = Q K^T, read row-wise only); the V operand (B of dP = dO V^T) stays
//     in registers.
//   * Q and dO half tiles go straight into double-buffered swizzled LDS, one
//     half ahead, the key tile's query tiles taken from the document's last
//     one down; row reads feed S and dP, transposing reads feed Q^T, dO^T.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256, 2) void k_bwd_dkdv(
    const bf16* __restrict__ qr, const bf16* __restrict__ kr, const bf16* __restrict__ v,
    const bf16* __restrict__ dout, const float* __restrict__ qstats,
    const float* __restrict__ table, const int32_t* __restrict__ pos,
    const int32_t* __restrict__ kptr, const int32_t* __restrict__ qpack,
    const int32_t* __restrict__ order_flags, const int32_t* __restrict__ status, int S, int Hq,
    int Hkv,
    int nk, int nblk, int n_items, float scale, int anchor, int origin,
    const int32_t* __restrict__ tok_map, bf16* __restrict__ dk, bf16* __restrict__ dv) {
  constexpr int BM = kDkvBM, BN = kDkvBN;    // plan tiles: 64 queries x 128 keys
  constexpr int BH = BM / 2;                 // queries per step
  constexpr int NKK = D / 16;
  constexpr int NDB = D / 32;
  static_assert(BN == 4 * 32 && BH == 32, "four waves of 32 keys, 32-query steps");
  using T = SwzTile<D>;
  // Two buffers, each holding a Q and a dO half tile back to back: a dO
  // read is then its Q read's address plus a constant (one address add for
  // both operands).
  __shared__ __align__(16) bf16 QG[2][2 * BH * D];
  __shared__ __align__(16) float s_st[2][4][BM];
  // This workgroup's keys (rotated), only ever read row-wise: rows padded by
  // 16 bytes instead of swizzled, so that 16 consecutive rows at one 16-byte
  // column still hit 16 distinct 4-bank groups and a lane's eight reads are
  // one base address plus immediate offsets.
  constexpr int KLD = D + 8;
  __shared__ __align__(16) bf16 Ks[BN * KLD];

  int hkv, ktile;   // ktile = b * nk + kt, in natural order: within a document the
                    // key tiles already go from the most query tiles to the fewest
  if (!work_head_rank(n_items / Hkv, Hkv, *order_flags, hkv, ktile)) return;
  const int b = ktile / nk, kt = ktile % nk;
  const int group = Hq / Hkv;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int h = lane >> 5, col = lane & 31;
  const int key = origin + kt * BN + wave * 32 + col;   // row-local key of this lane's column
  const bool kvalid = key < S;
  const size_t tok0 = (size_t)b * S;
  const size_t ktok = tok0 + (kvalid ? key : S - 1);
  const bool bad = status[0] != kStatusOk;
  const float scale_log2 = scale * kLog2e;

  // V operand: lane holds key `col`, features 16*kk + 8*h + i; K rows in LDS.
  bf16x8 vf[NKK];
  {
    const bf16* vp = v + (ktok * Hkv + hkv) * D + 8 * h;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) vf[kk] = *(const bf16x8*)(vp + 16 * kk);
    const size_t kv_row_stride = (size_t)Hkv * D;
    const bf16* kb0 = kr + tok0 * kv_row_stride + hkv * D;
    constexpr int NCH = D / 8;
#pragma unroll
    for (int u = 0; u < BN * NCH / 256; ++u) {
      const int idx = u * 256 + tid, r = idx / NCH, c = idx % NCH;
      const int krow = min(origin + kt * BN + r, S - 1);
      *(bf16x8*)(Ks + r * KLD + c * 8) = *(const bf16x8*)(kb0 + (size_t)krow * kv_row_stride + c * 8);
    }
  }
  f32x16 dka[NDB], dva[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) { dka[db][j] = 0.f; dva[db][j] = 0.f; }

  // Q and dO half tiles go straight into LDS; wave 0 also fetches the tile's
  // per-query record (LSE, Dv, visible-key interval).
  // Q and dO share a row stride, so one set of precomputed lane offsets
  // serves both.
  const size_t q_row_stride = (size_t)Hq * D;
  DirectTile<D, BH, 256> dl;
  dl.init(q_row_stride);
  auto issue = [&](int buf, int hq, int qt, int half) {
    const int row0 = origin + qt * BM + half * BH;
    dl.load_at(lds_addr(QG[0]) + buf * (4 * BH * D), qr + tok0 * q_row_stride + (size_t)hq * D,
               q_row_stride, row0, S - 1);
    dl.load_at(lds_addr(QG[0]) + buf * (4 * BH * D) + 2 * BH * D, dout + tok0 * q_row_stride + (size_t)hq * D,
               q_row_stride, row0, S - 1);
    if (wave == 0) {
      // the record index is wave-uniform: keep its arithmetic scalar
      const int ri = __builtin_amdgcn_readfirstlane((b * Hq + hq) * nblk + qt);
      const float* rec = qstats + (size_t)ri * (4 * BM);
      dma16(rec, 16 * lane, lds_ptr(lds_addr(&s_st[0][0][0]) + buf * (4 * BM * 4)));
    }
  };

  // Work list: every q head of the group x every live, not anchor-only query
  // tile x its two halves.
  const int e_begin = kptr[ktile], e_end = kptr[ktile + 1];
  const int h_end = (hkv + 1) * group;
  // The query tiles are taken from the document's last one down to the
  // diagonal: the workgroups of neighbouring key tiles then all start on
  // the same query tile and move down it in step, so each Q/dO tile is
  // fetched from HBM about once per XCD instead of once per staggered
  // workgroup (walking up from each diagonal, 64 concurrent workgroups
  // span about 4 MB of Q/dO, the size of an XCD's L2).
  auto first = [&](int& ee, int& hh) {
    ee = e_end - 1;
    hh = hkv * group;
    if (e_begin >= e_end) { hh = h_end; return; }
    while (ee >= e_begin && packed_kind(qpack[ee]) == kTileAnchor) --ee;
    if (ee < e_begin) hh = h_end;            // nothing live besides the anchor
  };
  auto advance = [&](int& ee, int& hh) {
    do {
      --ee;
      if (ee < e_begin) { ee = e_end - 1; ++hh; }
    } while (hh < h_end && packed_kind(qpack[ee]) == kTileAnchor);
  };

  int e, hq, half = 0;
  first(e, hq);
  if (hq < h_end) issue(0, hq, packed_idx(qpack[e]), 0);
  // one step per half tile; the buffer of a step is `cur` (unrolling the loop
  // by buffer would need a second set of address registers and spills)
  int kro = (32 * wave + col) * KLD + 8 * h;
  // Byte offsets inside a buffer of QG: row reads of (row col, chunk h),
  // the chunk 2kk + h being that offset XOR 32 kk (see tr_operand_x), and
  // the transposing reads' two pieces.
  const uint32_t o_row = 2u * T::chunk_off(col, h);
  uint32_t o_tr0, o_tr8;
  tr_lane_offsets<D>(o_tr0, o_tr8);
  const char* qg = (const char*)&QG[0][0];
  int cur = 0;
  while (hq < h_end) {
    const bool need_mask =
        packed_kind(qpack[e]) != kTileFull || (anchor && kt == 0 && origin == 0);
    int e1 = e, h1 = hq, half1 = half ^ 1;
    if (half1 == 0) advance(e1, h1);
    const int qt1 = h1 < h_end ? packed_idx(qpack[e1]) : 0;
    wait_direct_loads();
    __syncthreads();      // half tile in buffer `cur` visible; the other buffer free
    if (h1 < h_end) issue(cur ^ 1, h1, qt1, half1);
    // this lane's K row offset, re-declared live in every step so that the
    // eight reads below stay one register plus immediate offsets (hoisted out
    // of the loop they would take eight registers)
    asm volatile("" : "+v"(kro));
    // this step's buffer: the Q half tile, then the dO half tile
    constexpr uint32_t kBuf = 2 * 2 * BH * D, kG = 2 * BH * D;   // bytes
    uint32_t b_row = cur * kBuf + o_row, b_tr0 = cur * kBuf + o_tr0, b_tr8 = cur * kBuf + o_tr8;
    // opaque per step, so that the compiler keeps three registers and one
    // XOR per read instead of hoisting every XORed offset out of the loop
    asm volatile("" : "+v"(b_row), "+v"(b_tr0), "+v"(b_tr8));
    const float* stc = &s_st[cur][0][0] + half * BH;

    // S = Q K^T, dP = dO V^T for the 32 queries: columns = this wave's keys.
    f32x16 sp, dp;
#pragma unroll
    for (int j = 0; j < 16; ++j) { sp[j] = 0.f; dp[j] = 0.f; }
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const uint32_t o = b_row ^ (32u * kk);
      const bf16x8 kb = *(const bf16x8*)(Ks + kro + 16 * kk);
      sp = mfma32(*(const bf16x8*)(qg + o), kb, sp);
      dp = mfma32(*(const bf16x8*)(qg + o + kG), vf[kk], dp);
    }
    // P = exp2(s * scale_log2 - lse_log2), dS = P (dP - Dv).
    bf16x8 pb[2], db_[2];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int q0 = 8 * g + 4 * h;            // step-local queries q0 .. q0+3
      const f32x4 l4 = *(const f32x4*)(stc + q0);
      const f32x4 d4 = *(const f32x4*)(stc + BM + q0);
      float pv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) pv[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sp[4 * g + r], scale_log2, -l4[r]));
      if (need_mask) {
        // Read as float vectors and reinterpreted in registers: a typed
        // vector load keeps its type-based alias information, and without
        // it the compiler would first wait for the next half tile's direct
        // loads to land (they may write any LDS it cannot tell apart).
        const f32x4 lo4 = *(const f32x4*)(stc + 2 * BM + q0);
        const f32x4 hi4 = *(const f32x4*)(stc + 3 * BM + q0);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          pv[r] = ((int)(key >= __float_as_int(lo4[r])) & (int)(key <= __float_as_int(hi4[r]))) ? pv[r] : 0.f;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 4 * g + r;
        pb[j >> 3][j & 7] = (bf16)pv[r];
        db_[j >> 3][j & 7] = (bf16)(pv[r] * (dp[j] - d4[r]));
      }
    }
    // dV^T += dO^T P, dK^T += Q^T dS over the 32 queries.
#pragma unroll
    for (int dblk = 0; dblk < NDB; ++dblk)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        dva[dblk] = mfma32(tr_operand_x<D>(qg + kG, b_tr0, b_tr8, 16 * c, 32 * dblk), pb[c], dva[dblk]);
        dka[dblk] = mfma32(tr_operand_x<D>(qg, b_tr0, b_tr8, 16 * c, 32 * dblk), db_[c], dka[dblk]);
      }
    // Schedule of these products: the first three operands' reads, then each
    // MFMA followed by the reads of the operand three MFMAs later, so that
    // three operands are in flight behind every product (left to itself the
    // compiler reads each operand right before its MFMA and waits for it).
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);   // 6 LDS reads
#pragma unroll
    for (int i = 0; i < 4 * NDB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                        // 1 MFMA
      if (i + 3 < 4 * NDB) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // 2 LDS reads
    }
    e = e1; hq = h1; half = half1;
    cur ^= 1;
  }

  // Epilogue: dK = R(pos)^T (scale * dK'), dV as accumulated.
  if (kvalid) {
    const int pk = pos[ktok];
    const float* tb = table + (size_t)pk * D;      // (D/2) pairs of {cos, sin}
    const size_t otok = tok_map ? (size_t)tok_map[ktok] : ktok;   // the caller's dk, dv row
    bf16* dkp = dk + (otok * Hkv + hkv) * D;
    bf16* dvp = dv + (otok * Hkv + hkv) * D;
#pragma unroll
    for (int dblk = 0; dblk < NDB; ++dblk)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * dblk + 8 * g + 4 * h;
        const f32x4 cs = *(const f32x4*)(tb + d0);    // cos, sin of pairs d0/2, d0/2+1
        bf16x4 wk, wv;
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
          const float c = cs[2 * pr], s = cs[2 * pr + 1];
          const float x0 = dka[dblk][4 * g + 2 * pr] * scale, x1 = dka[dblk][4 * g + 2 * pr + 1] * scale;
          wk[2 * pr] = (bf16)(bad ? NAN : x0 * c + x1 * s);
          wk[2 * pr + 1] = (bf16)(bad ? NAN : x1 * c - x0 * s);
          wv[2 * pr] = (bf16)(bad ? NAN : dva[dblk][4 * g + 2 * pr]);
          wv[2 * pr + 1] = (bf16)(bad ? NAN : dva[dblk][4 * g + 2 * pr + 1]);
        }
        *(bf16x4*)(dkp + d0) = wk;
        *(bf16x4*)(dvp + d0) = wv;
      }
  }
}

// ---------------------------------------------------------------------------
// dq: one workgroup (4 waves) per (row b, query head, query tile of 128);
// each wave owns 32 queries, as in the forward kernel.  K and V tiles go
// straight into a ring of swizzled LDS buffers: row reads feed S^T = K Q^T
// and dP^T = V dO^T, transposing reads feed K^T in dQ^T = K^T dS^T.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kFwdThreads, kFwdBlocksPerCU) void k_bwd_dq(
    const bf16* __restrict__ qr, const bf16* __restrict__ kr, const bf16* __restrict__ v,
    const bf16* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ dvec,
    const float* __restrict__ ds0, const float* __restrict__ table,
    const int32_t* __restrict__ pos, const int32_t* __restrict__ lo,
    const int32_t* __restrict__ hi, const int32_t* __restrict__ qptr,
    const int32_t* __restrict__ kpack, const int32_t* __restrict__ order,
    const int32_t* __restrict__ status, int S, int Hq, int Hkv, int nq, int n_items, float scale,
    int anchor, int origin, const int32_t* __restrict__ tok_map, bf16* __restrict__ dq) {
  constexpr int BM = kFwdBM, BN = kFwdBN;
  constexpr int NKK = D / 16;
  constexpr int NDB = D / 32;
  constexpr int NKB = BN / 32;
  using T = SwzTile<D>;
  constexpr int NBUF = kFwdStages;
  // One LDS object per buffer: the compiler can then tell that reads of
  // one buffer do not alias the direct loads in flight into the other, and
  // does not wait for those loads before the reads.
  __shared__ __align__(16) bf16 Ks0[BN * D];
  __shared__ __align__(16) bf16 Ks1[BN * D];
  __shared__ __align__(16) bf16 Vs0[BN * D];
  __shared__ __align__(16) bf16 Vs1[BN * D];

  const int tiles_per_head = n_items / Hq;
  int hq, rank;
  if (!work_head_rank(tiles_per_head, Hq, order[tiles_per_head], hq, rank)) return;
  const int tile = order[rank];   // b * nq + qt
  const int b = tile / nq, qt = tile % nq;
  const int hkv = hq / (Hq / Hkv);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int h = lane >> 5, col = lane & 31;
  const int qrow = origin + qt * BM + wave * 32 + col;
  const bool qvalid = qrow < S;
  const size_t tok0 = (size_t)b * S;
  const size_t tok = tok0 + (qvalid ? qrow : S - 1);
  int qlo = lo[tok], qhi = hi[tok];
  if (!qvalid) { qlo = 1; qhi = 0; }
  const bool bad = status[0] != kStatusOk;
  const float scale_log2 = scale * kLog2e;
  const size_t rowstat = ((size_t)b * Hq + hq) * S + (qvalid ? qrow : S - 1);
  const size_t otok = tok_map ? (size_t)tok_map[tok] : tok;   // the caller's LSE and dq row
  const float nlse2 = -lse[((size_t)b * Hq + hq) * S + (otok - tok0)] * kLog2e;
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

  static_assert(NBUF == 2, "the unrolled tile loop assumes two buffers");
  const size_t kv_row_stride = (size_t)Hkv * D;
  const bf16* kbase = kr + tok0 * kv_row_stride + hkv * D;
  const bf16* vbase = v + tok0 * kv_row_stride + hkv * D;
  DirectTile<D, BN, kFwdThreads> dl;
  dl.init(kv_row_stride);
  auto issue = [&](int buf, int kt) {
    dl.load(buf ? Ks1 : Ks0, kbase, kv_row_stride, origin + kt * BN, S - 1);
    dl.load(buf ? Vs1 : Vs0, vbase, kv_row_stride, origin + kt * BN, S - 1);
  };

  int e_first = qptr[tile];
  const int e_end = qptr[tile + 1];
  if (e_first < e_end && packed_kind(kpack[e_first]) == kTileAnchor) ++e_first;
  const int n_tiles = e_end - e_first;
  if (n_tiles > 0) issue(0, packed_idx(kpack[e_first]));
  // Byte offsets inside a K/V tile: row reads of (row col, chunk h), chunk
  // 2kk + h being that offset XOR 32 kk (see tr_operand_x), and the
  // transposing reads' two pieces.
  const uint32_t o_row = 2u * T::chunk_off(col, h);
  uint32_t o_tr0, o_tr8;
  tr_lane_offsets<D>(o_tr0, o_tr8);
  // tile loop unrolled by two: every LDS address of a buffer is base + constant
  auto step = [&](auto bufc, int i) {
    constexpr int BUF = decltype(bufc)::value;
    const int ent = kpack[e_first + i];
    const int kt = packed_idx(ent);
    const bool need_mask = packed_kind(ent) != kTileFull || (anchor && kt == 0 && origin == 0);
    const int key0 = origin + kt * BN;   // the tile's first key (row-local)
    const bool more = i + 1 < n_tiles;
    const int ent_next = more ? kpack[e_first + i + 1] : 0;
    wait_direct_loads();
    __syncthreads();                 // tile i visible; the other buffer is free
    if (more) issue(BUF ^ 1, packed_idx(ent_next));
    const char* Kc = (const char*)(BUF ? Ks1 : Ks0);
    const char* Vc = (const char*)(BUF ? Vs1 : Vs0);
    // opaque per step, so that the compiler keeps three registers and one
    // XOR per read instead of hoisting every XORed offset out of the loop
    uint32_t b_row = o_row, b_tr0 = o_tr0, b_tr8 = o_tr8;
    asm volatile("" : "+v"(b_row), "+v"(b_tr0), "+v"(b_tr8));

    // One 32-key block at a time: S^T = K Q^T, dP^T = V dO^T (rows = keys,
    // columns = this wave's queries), dS^T, then dQ^T += K^T dS^T.
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      // a block none of the wave's queries may see contributes exactly zero
      const int k0 = key0 + 32 * kb;
      if (need_mask && !__builtin_amdgcn_ballot_w64(qlo <= k0 + 31 && qhi >= k0)) continue;
      f32x16 st, dpt;
#pragma unroll
      for (int j = 0; j < 16; ++j) { st[j] = 0.f; dpt[j] = 0.f; }
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const uint32_t o = (b_row ^ (32u * kk)) + 2u * 32 * kb * D;
        st = mfma32(*(const bf16x8*)(Kc + o), qf[kk], st);
        dpt = mfma32(*(const bf16x8*)(Vc + o), gf[kk], dpt);
      }
      // P^T = exp2(s * scale_log2 - lse_log2) in place of the scores
#pragma unroll
      for (int j = 0; j < 16; ++j) st[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(st[j], scale_log2, nlse2));
      if (need_mask) {
        const int a = qlo - k0 - 4 * h, z = qhi - k0 - 4 * h;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int off = 8 * (j >> 2) + (j & 3);
          st[j] = (off >= a && off <= z) ? st[j] : 0.f;
        }
      }
      bf16x8 dsb[2];
#pragma unroll
      for (int j = 0; j < 16; ++j) dsb[j >> 3][j & 7] = (bf16)(st[j] * (dpt[j] - dvi));
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int c = 0; c < 2; ++c)
          acc[db] = mfma32(tr_operand_x<D>(Kc, b_tr0, b_tr8, 32 * kb + 16 * c, 32 * db), dsb[c], acc[db]);
    }
  };
  for (int i = 0; i < n_tiles; i += 2) {
    step(std::integral_constant<int, 0>{}, i);
    if (i + 1 < n_tiles) step(std::integral_constant<int, 1>{}, i + 1);
  }

  // Epilogue: dq' = scale (acc + dS_i0 k'_0); dq = R(pos_i)^T dq'.
  if (qvalid) {
    const float a0 = ds0[rowstat];
    const bf16* k0 = kr + (tok0 * Hkv + hkv) * D;
    const int pq = pos[tok];
    const float* tb = table + (size_t)pq * D;
    bf16* dqp = dq + (otok * Hq + hq) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * db + 8 * g + 4 * h;
        const bf16x4 kz = *(const bf16x4*)(k0 + d0);
        const f32x4 cs = *(const f32x4*)(tb + d0);
        bf16x4 w;
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
          const float c = cs[2 * pr], s = cs[2 * pr + 1];
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
// anchor: one workgroup of 1024 threads per (row b, kv head).  Thread
// (part, d) sums every parts-th row-block partial of the group's query heads
// for feature d; the parts are then added in LDS.  The anchor's position is
// 0, so R(0)^T = I.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void k_bwd_anchor(
    const float* __restrict__ part_dk, const float* __restrict__ part_dv,
    const int32_t* __restrict__ status, int S, int Hq, int Hkv, int D, int nblk, float scale,
    const int32_t* __restrict__ tok_map, bf16* __restrict__ dk, bf16* __restrict__ dv) {
  __shared__ float red[2][1024];
  const int b = blockIdx.x / Hkv, hkv = blockIdx.x % Hkv;
  const int group = Hq / Hkv;
  const int parts = 1024 / D;
  const int d = threadIdx.x % D, part = threadIdx.x / D;
  const bool bad = status[0] != kStatusOk;
  // eight running sums per quantity: eight independent loads in flight per
  // thread instead of one dependent chain
  constexpr int U = 8;
  float ak[U], av[U];
#pragma unroll
  for (int u = 0; u < U; ++u) { ak[u] = 0.f; av[u] = 0.f; }
  for (int hq = hkv * group; hq < (hkv + 1) * group; ++hq) {
    const size_t base = ((size_t)b * Hq + hq) * nblk * D + d;
    int n = part;
    for (; n + (U - 1) * parts < nblk; n += U * parts) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        ak[u] += part_dk[base + (size_t)(n + u * parts) * D];
        av[u] += part_dv[base + (size_t)(n + u * parts) * D];
      }
    }
    for (; n < nblk; n += parts) {
      ak[0] += part_dk[base + (size_t)n * D];
      av[0] += part_dv[base + (size_t)n * D];
    }
  }
  float sk = 0.f, sv = 0.f;
#pragma unroll
  for (int u = 0; u < U; ++u) { sk += ak[u]; sv += av[u]; }
  red[0][threadIdx.x] = sk;
  red[1][threadIdx.x] = sv;
  __syncthreads();
  if (part == 0) {
    for (int q = 1; q < parts; ++q) {
      sk += red[0][q * D + d];
      sv += red[1][q * D + d];
    }
    const size_t atok = tok_map ? (size_t)tok_map[(size_t)b * S] : (size_t)b * S;
    const size_t off = (atok * Hkv + hkv) * D + d;
    dk[off] = (bf16)(bad ? NAN : sk * scale);
    dv[off] = (bf16)(bad ? NAN : sv);
  }
}

// ---------------------------------------------------------------- launchers
hipError_t launch_bwd_dkdv(const BwdArgs& a, const PlanBufs& pk, const PlanBufs& pq,
                           hipStream_t st) {
  const int n_items = a.B * pk.nk * a.Hkv;
  const int32_t* flags = pq.order + (size_t)a.B * pq.nq;   // the query-major plan's order flags
  const dim3 grid(padded_grid(n_items));
  if (a.D == 128)
    hipLaunchKernelGGL(k_bwd_dkdv<128>, grid, dim3(256), 0, st, a.qr, a.kr, a.v, a.dout,
                       a.qstats, a.table, a.tt.pos, pk.kptr, pk.qpack, flags, a.status, a.S,
                       a.Hq, a.Hkv, pk.nk, a.nblk, n_items, a.scale, a.anchor, pk.origin, a.tok_map,
                       a.dk, a.dv);
  else
    hipLaunchKernelGGL(k_bwd_dkdv<64>, grid, dim3(256), 0, st, a.qr, a.kr, a.v, a.dout,
                       a.qstats, a.table, a.tt.pos, pk.kptr, pk.qpack, flags, a.status, a.S,
                       a.Hq, a.Hkv, pk.nk, a.nblk, n_items, a.scale, a.anchor, pk.origin, a.tok_map,
                       a.dk, a.dv);
  return hipGetLastError();
}

hipError_t launch_bwd_dq(const BwdArgs& a, const PlanBufs& pq, hipStream_t st) {
  const int n_items = a.B * pq.nq * a.Hq;
  const dim3 grid(padded_grid(n_items));
  if (a.D == 128)
    hipLaunchKernelGGL(k_bwd_dq<128>, grid, dim3(kFwdThreads), 0, st, a.qr, a.kr, a.v, a.dout, a.lse,
                       a.dvec, a.ds0, a.table, a.tt.pos, a.tt.lo, a.tt.hi, pq.qptr, pq.kpack,
                       pq.order, a.status, a.S, a.Hq, a.Hkv, pq.nq, n_items, a.scale, a.anchor, pq.origin,
                       a.tok_map, a.dq);
  else
    hipLaunchKernelGGL(k_bwd_dq<64>, grid, dim3(kFwdThreads), 0, st, a.qr, a.kr, a.v, a.dout, a.lse,
                       a.dvec, a.ds0, a.table, a.tt.pos, a.tt.lo, a.tt.hi, pq.qptr, pq.kpack,
                       pq.order, a.status, a.S, a.Hq, a.Hkv, pq.nq, n_items, a.scale, a.anchor, pq.origin,
                       a.tok_map, a.dq);
  return hipGetLastError();
}

hipError_t launch_bwd_anchor(const BwdArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_bwd_anchor, dim3(a.B * a.Hkv), dim3(1024), 0, st, a.part_dk, a.part_dv,
                     a.status, a.S, a.Hq, a.Hkv, a.D, a.nblk, a.scale, a.tok_map, a.dk, a.dv);
  return hipGetLastError();
}

}  // namespace aa
