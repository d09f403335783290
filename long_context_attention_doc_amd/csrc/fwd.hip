// Forward attention kernel: flash-style online softmax over the live key tiles
// of the tile plan, bf16 MFMA (v_mfma_f32_32x32x16_bf16) with float32
// accumulation.
//
// What it computes (paper-graph architecture page of arXiv 2411.13476,
// section 3.4, "Standard attention" and "AnchorAttention: The Shared Anchor
// Design", "Mask construction"): for every query i of a packed row,
//   O_i = sum_j softmax_j(scale * q'_i . k'_j) v_j
// over the keys j the mask allows: the row's anchor (column 0) and the keys
// of i's own document that are not after i.  q', k' are the RoPE-rotated,
// bf16-rounded inputs.
//
// Work decomposition.  A workgroup of four 64-lane waves owns one
// (row b, query head, query tile of 128 rows); each wave owns 32 queries.
// The kernel computes the transposed score block S^T = K Q^T so that each
// lane's 32x32 accumulator column is one query: the softmax row statistics
// are then per lane, and the two lanes holding the same query (lane l and
// l + 32) combine with one v_permlane32_swap.
//   * Q^T (B operand) stays in registers for the whole key loop.  The RoPE
//     rotation of Q happens in its load (ROTATE_Q): the rotated rows are
//     formed once per work item and also written out for the backward.  K
//     is streamed (every query tile reads it again), so it is rotated once
//     by the RoPE pass before this kernel.
//   * K and V tiles go straight from global memory into a ring of LDS
//     buffers (direct buffer loads to LDS) in a row-major layout with an XOR swizzle; K
//     is read row-wise (A operand of S^T), V with transposing LDS reads
//     (A operand V^T of O^T = V^T P^T).  Up to kFwdStages-1 tiles are in
//     flight while the current tile is computed.
//   * P^T goes from the score accumulators straight into the B operand of
//     the second product; the transposed V^T reads deliver keys in the
//     accumulator's row order.
//   * The anchor column is folded in before the loop as the softmax's
//     starting point (m = s_i0, l = 1, acc = v_0); inside the loop column 0
//     is outside every query's document interval, so it is never counted
//     twice.  Key tiles that see only the anchor are skipped.
//   * The running maximum m is exact (the largest weight of every row is
//     exactly 1 before bf16 rounding), but the O rescale is skipped, wave by
//     wave, on tiles where no query's maximum grew; on long documents that
//     is most tiles.
#include <type_traits>

#include "aa_internal.h"

namespace aa {

template <int D, bool ROTATE_Q>
__global__ __launch_bounds__(kFwdThreads, kFwdBlocksPerCU) void k_fwd(
    const bf16* __restrict__ q_raw, const float* __restrict__ table, const int32_t* __restrict__ pos,
    int npos, bf16* __restrict__ qr, const bf16* __restrict__ kr, const bf16* __restrict__ v,
    const int32_t* __restrict__ lo, const int32_t* __restrict__ hi,
    const int32_t* __restrict__ qptr, const int32_t* __restrict__ kpack,
    const int32_t* __restrict__ order, const int32_t* __restrict__ status, int S, int Hq, int Hkv,
    int nq, int n_items, float scale_log2, int anchor, int origin, void* __restrict__ o,
    int o_f32, float* __restrict__ lse, const int32_t* __restrict__ tok_map) {
  constexpr int BM = kFwdBM, BN = kFwdBN;
  constexpr int NKK = D / 16;    // 16-wide reduction steps over d
  constexpr int NDB = D / 32;    // 32-row blocks of d in O^T
  constexpr int NKB = BN / 32;   // 32-key blocks of a key tile
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
  const size_t tok = (size_t)b * S + (qvalid ? qrow : S - 1);
  int qlo = lo[tok], qhi = hi[tok];
  if (!qvalid) { qlo = 1; qhi = 0; }
  const bool bad = status[0] != kStatusOk;

  // Q^T operand: lane holds query `col`, features 16*kk + 8*h + i.  With
  // ROTATE_Q the RoPE stage happens here: Q stays in registers for the
  // whole key loop, so it is rotated once, and the rotated rows are written
  // out for the backward.  The raw rows are loaded first, then the first K/V
  // tile is issued, then the rows' cos/sin values (their address needs the
  // position ID), so that the loads' latencies overlap (workgroups with few
  // key tiles gain).
  bf16x8 qf[NKK];
  const size_t qoff = (tok * Hq + hq) * D + 8 * h;
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) qf[kk] = *(const bf16x8*)((ROTATE_Q ? q_raw : qr) + qoff + 16 * kk);

  const size_t tok0 = (size_t)b * S;
  // K and V tiles are loaded straight into LDS, two buffers; the tile loop is
  // unrolled by two so that every LDS address of a buffer is base + constant.
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

  // Live key tiles e_first .. e_end-1 (only key tile 0 can be anchor-only).
  int e_first = qptr[tile];
  const int e_end = qptr[tile + 1];
  if (e_first < e_end && packed_kind(kpack[e_first]) == kTileAnchor) ++e_first;
  const int n_tiles = e_end - e_first;
  if (n_tiles > 0) issue(0, packed_idx(kpack[e_first]));

  if constexpr (ROTATE_Q) {
    const int p = min(max(pos[tok], 0), npos - 1);
    const float* tb = table + (size_t)p * D + 8 * h;     // row p, pair (8h)/2, {cos, sin}
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) qf[kk] = rope_rotate8(qf[kk], tb + 16 * kk);
    if (qvalid) {
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) *(bf16x8*)(qr + qoff + 16 * kk) = qf[kk];
    }
  }

  // Anchor column: s_i0 = q'_i . k'_0 (k'_0 = k_0, its position is 0).  Rows
  // without an anchor start from an empty softmax instead.
  float m, l;
  f32x16 acc[NDB];
  if (!anchor) {
    m = -INFINITY;
    l = 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[db][j] = 0.f;
  } else {
    const bf16* k0 = kr + (tok0 * Hkv + hkv) * D + 8 * h;
    float s0 = 0.f;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const bf16x8 kv = *(const bf16x8*)(k0 + 16 * kk);
#pragma unroll
      for (int i = 0; i < 8; ++i) s0 += (float)qf[kk][i] * (float)kv[i];
    }
    s0 += partner(s0);
    m = s0 * scale_log2;
    l = h == 0 ? 1.f : 0.f;          // each lane keeps half of the row sum
    const bf16* v0 = v + (tok0 * Hkv + hkv) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const bf16x4 w = *(const bf16x4*)(v0 + 32 * db + 8 * g + 4 * h);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[db][4 * g + r] = (float)w[r];
      }
  }

  auto step = [&](auto bufc, int i) {
    constexpr int BUF = decltype(bufc)::value;
    const int ent = kpack[e_first + i];
    const int kt = packed_idx(ent);
    // (at origin 0 key tile 0 holds the anchor column, which the softmax
    // start already counts)
    const bool need_mask = packed_kind(ent) != kTileFull || (anchor && kt == 0 && origin == 0);
    const int key0 = origin + kt * BN;   // the tile's first key (row-local)
    const bool more = i + 1 < n_tiles;
    const int ent_next = more ? kpack[e_first + i + 1] : 0;
    wait_direct_loads();
    __syncthreads();                 // tile i visible; the other buffer is free
    if (more) issue(BUF ^ 1, packed_idx(ent_next));
    const bf16* Kc = BUF ? Ks1 : Ks0;
    const bf16* Vc = BUF ? Vs1 : Vs0;

    // A 32-key block that none of the wave's queries may see (a document
    // edge or the causal diagonal inside a partial tile) has exactly zero
    // weights: every stage below skips it (wave-uniform branches), so its
    // score registers are never filled or read.
    bool live[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const int k0 = key0 + 32 * kb;
      live[kb] = !need_mask || __builtin_amdgcn_ballot_w64(qlo <= k0 + 31 && qhi >= k0) != 0;
    }

    // S^T = K Q^T for this wave's 32 queries and the BN keys of the tile.
    f32x16 st[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
      if (live[kb]) {
#pragma unroll
        for (int j = 0; j < 16; ++j) st[kb][j] = 0.f;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
          st[kb] = mfma32(*(const bf16x8*)(Kc + T::chunk_off(kb * 32 + col, 2 * kk + h)), qf[kk],
                          st[kb]);
      }
    if (need_mask) {
      // keys outside [qlo, qhi] (row-local) are masked
      const int a = qlo - key0 - 4 * h, z = qhi - key0 - 4 * h;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        if (live[kb]) {
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int off = kb * 32 + 8 * (j >> 2) + (j & 3);
            st[kb][j] = (off >= a && off <= z) ? st[kb][j] : -INFINITY;
          }
        }
    }
    // Tile maximum over the live blocks (raw scores; the scale is positive).
    // IEEE maximum needs no input canonicalisation and fuses into
    // three-input maxima.
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
      if (live[kb]) {
        float mk = st[kb][0];
#pragma unroll
        for (int j = 1; j < 15; j += 2)
          mk = __builtin_elementwise_maximum(__builtin_elementwise_maximum(mk, st[kb][j]),
                                             st[kb][j + 1]);
        mk = __builtin_elementwise_maximum(mk, st[kb][15]);
        mt = __builtin_elementwise_maximum(mt, mk);
      }
    mt = __builtin_elementwise_maximum(mt, partner(mt)) * scale_log2;
    const bool raise = mt > m;
    if (__builtin_amdgcn_ballot_w64(raise)) {
      const float m_new = raise ? mt : m;
      const float factor = raise ? __builtin_amdgcn_exp2f(m - m_new) : 1.f;  // m may be -inf
      m = m_new;
      l *= factor;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[db][j] *= factor;
    }

    // P^T = exp2(s * scale_log2 - m) as bf16 B operands, one per 16-key step,
    // and O^T += V^T P^T, over the live key blocks.  The row sum adds the
    // same bf16 weights that multiply V (pairwise dot products with ones),
    // so numerator and denominator see identical P.
    const float nm = m == -INFINITY ? 0.f : -m;   // a row that has seen no key yet
    const bf16x2 ones = {(bf16)1.f, (bf16)1.f};
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
      if (live[kb]) {
        bf16x8 pb[2];
#pragma unroll
        for (int j = 0; j < 16; ++j)
          pb[j >> 3][j & 7] = (bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(st[kb][j], scale_log2, nm));
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[c], pb[c], 0, 1), ones, l, false);
          l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[c], pb[c], 2, 3), ones, l, false);
          l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[c], pb[c], 4, 5), ones, l, false);
          l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[c], pb[c], 6, 7), ones, l, false);
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int c = 0; c < 2; ++c)
            acc[db] = mfma32(tr_operand<D>(Vc, 32 * kb + 16 * c, 32 * db), pb[c], acc[db]);
      }
  };
  for (int i = 0; i < n_tiles; i += 2) {
    step(std::integral_constant<int, 0>{}, i);
    if (i + 1 < n_tiles) step(std::integral_constant<int, 1>{}, i + 1);
  }

  // Epilogue: O = acc / l, LSE = (m + log2 l) * ln 2.
  const float lt = l + partner(l);
  const float inv = 1.f / lt;
  if (qvalid) {
    const size_t otok = tok_map ? (size_t)tok_map[tok] : tok;   // where this query's output goes
    const size_t orow = (otok * Hq + hq) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 w;
#pragma unroll
        for (int r = 0; r < 4; ++r) w[r] = bad ? NAN : acc[db][4 * g + r] * inv;
        const int d0 = 32 * db + 8 * g + 4 * h;
        if (o_f32) {
          *(f32x4*)((float*)o + orow + d0) = w;
        } else {
          bf16x4 wb;
#pragma unroll
          for (int r = 0; r < 4; ++r) wb[r] = (bf16)w[r];
          *(bf16x4*)((bf16*)o + orow + d0) = wb;
        }
      }
    if (h == 0) {
      const float val = (m + __log2f(lt)) * 0.69314718055994530942f;
      lse[((size_t)b * Hq + hq) * S + (otok - tok0)] = bad ? NAN : val;
    }
  }

  // The anchor row, outside a grid that starts after it: it sees only
  // itself, so O_0 = v_0 and LSE_0 = scale * q'_0 . k'_0 (position 0, so
  // q'_0, k'_0 are the inputs themselves).  Wave 0 of the row's first query
  // tile does it, one 8-feature piece per lane.
  if (origin && qt == 0 && wave == 0) {
    constexpr int NC = D / 8;
    const size_t otok = tok_map ? (size_t)tok_map[tok0] : tok0;
    float sp = 0.f;
    if (lane < NC) {
      const size_t qa = (tok0 * Hq + hq) * D + 8 * lane;
      bf16x8 qv = *(const bf16x8*)((ROTATE_Q ? q_raw : qr) + qa);
      if constexpr (ROTATE_Q) {
        qv = rope_rotate8(qv, table + 8 * lane);   // table row 0: the identity, bit for bit
        *(bf16x8*)(qr + qa) = qv;
      }
      const bf16x8 kv = *(const bf16x8*)(kr + (tok0 * Hkv + hkv) * D + 8 * lane);
#pragma unroll
      for (int i = 0; i < 8; ++i) sp += (float)qv[i] * (float)kv[i];
      const bf16x8 vv = *(const bf16x8*)(v + (tok0 * Hkv + hkv) * D + 8 * lane);
      const size_t orow = (otok * Hq + hq) * D + 8 * lane;
      if (o_f32) {
        f32x4 w0, w1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          w0[i] = bad ? NAN : (float)vv[i];
          w1[i] = bad ? NAN : (float)vv[4 + i];
        }
        ((f32x4*)((float*)o + orow))[0] = w0;
        ((f32x4*)((float*)o + orow))[1] = w1;
      } else {
        bf16x8 w = vv;
        if (bad) {
#pragma unroll
          for (int i = 0; i < 8; ++i) w[i] = (bf16)NAN;
        }
        *(bf16x8*)((bf16*)o + orow) = w;
      }
    }
#pragma unroll
    for (int off = NC / 2; off > 0; off >>= 1) sp += __shfl_xor(sp, off);
    if (lane == 0)
      lse[((size_t)b * Hq + hq) * S + (otok - tok0)] =
          bad ? NAN : sp * scale_log2 * 0.69314718055994530942f;
  }
}

hipError_t launch_fwd(const bf16* q_raw, const float* table, int npos, bf16* qr, const bf16* kr,
                      const bf16* v, TokenTables tt, const PlanBufs& pb, const int32_t* status,
                      int B, int S, int Hq, int Hkv, int D, float scale, int anchor, void* o,
                      int o_f32, float* lse, const int32_t* tok_map, hipStream_t st) {
  const float scale_log2 = scale * 1.44269504088896340736f;
  const int n_items = B * pb.nq * Hq;
  const dim3 grid(padded_grid(n_items));
#define AA_LAUNCH_FWD(DD, RQ)                                                                    \
  hipLaunchKernelGGL((k_fwd<DD, RQ>), grid, dim3(kFwdThreads), 0, st, q_raw, table, tt.pos, npos, qr, kr, \
                     v, tt.lo, tt.hi, pb.qptr, pb.kpack, pb.order, status, S, Hq, Hkv, pb.nq,     \
                     n_items, scale_log2, anchor, pb.origin, o, o_f32, lse, tok_map)
  if (D == 128) {
    if (q_raw) AA_LAUNCH_FWD(128, true);
    else AA_LAUNCH_FWD(128, false);
  } else {
    if (q_raw) AA_LAUNCH_FWD(64, true);
    else AA_LAUNCH_FWD(64, false);
  }
#undef AA_LAUNCH_FWD
  return hipGetLastError();
}

}  // namespace aa
