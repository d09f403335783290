// Internal declarations shared by the library's HIP translation units.
// Not part of the public ABI (see include/anchor_attn.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace aa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kStatusOk = 0;
constexpr int kStatusBadDocs = 2;

constexpr uint8_t kTileFull = 1;
constexpr uint8_t kTilePartial = 2;
constexpr uint8_t kTileAnchor = 3;

constexpr int kMaxHalfD = 64;   // D <= 128

// theta_p = base^(-2p/D) in float64, passed by value to the RoPE table kernel.
struct RopeTheta {
  double t[kMaxHalfD];
};

// Per-token tables written by the position kernel (row-local indices).
//   pos[t]: position ID; lo[t], hi[t]: the document keys query t may see
//   besides the anchor, as the closed interval [lo, hi] (empty for the anchor
//   itself: lo = 1, hi = 0).
struct TokenTables {
  int32_t* pos;
  int32_t* lo;
  int32_t* hi;
};

// Buffers of one tile plan.
struct PlanBufs {
  int BM, BN, nq, nk;
  size_t cap;          // B * nq * nk
  uint8_t* kinds;      // dense [B][nq][nk]
  int32_t* cntq;       // [B*nq]
  int32_t* cntk;       // [B*nk]
  int32_t* qptr;       // [B*nq + 1]
  int32_t* kidx;       // [cap]
  uint8_t* kkind;      // [cap]
  int32_t* kptr;       // [B*nk + 1]
  int32_t* qidx;       // [cap]
  uint8_t* qkind;      // [cap]
  int32_t* n_live;     // [1]
};

// ---------------------------------------------------------------- launchers
hipError_t launch_positions(const int32_t* cu, int n_seg, int B, int S, int causal, int mode,
                            TokenTables tt, int32_t* status, hipStream_t st);
hipError_t launch_plan(const int32_t* lo, const int32_t* hi, int B, int S, PlanBufs pb,
                       bool key_major, hipStream_t st);
hipError_t launch_rope_table(int S, int D, const RopeTheta& th, float* table, hipStream_t st);
hipError_t launch_rope_apply(const bf16* x, const int32_t* pos, const float* table, int B, int S,
                             int H, int D, bf16* x_rot, hipStream_t st);
hipError_t launch_fwd(const bf16* qr, const bf16* kr, const bf16* v, TokenTables tt,
                      const PlanBufs& pb, const int32_t* status, int B, int S, int Hq, int Hkv,
                      int D, float scale, bf16* o, float* lse, hipStream_t st);

struct BwdArgs {
  const bf16* qr;      // rotated q [B,S,Hq,D]
  const bf16* kr;      // rotated k [B,S,Hkv,D]
  const bf16* v;
  const bf16* o;
  const bf16* dout;
  const float* lse;    // [B,Hq,S]
  const float* table;  // RoPE cos/sin table [S][D/2][2]
  TokenTables tt;
  const int32_t* status;
  float* dvec;         // [B,Hq,S]   rowsum(dO * O)
  float* ds0;          // [B,Hq,S]   dS of the anchor column
  float* part_dk;      // [B,Hq,nblk,D] per-row-block sums for the anchor key
  float* part_dv;      // [B,Hq,nblk,D]
  int nblk;
  bf16* dq;
  bf16* dk;
  bf16* dv;
  int B, S, Hq, Hkv, D;
  float scale;
};
constexpr int kPreRows = 64;    // rows per block of the backward preprocess

hipError_t launch_bwd_pre(const BwdArgs& a, hipStream_t st);
hipError_t launch_bwd_dkdv(const BwdArgs& a, const PlanBufs& pk, hipStream_t st);
hipError_t launch_bwd_dq(const BwdArgs& a, const PlanBufs& pq, hipStream_t st);
hipError_t launch_bwd_anchor(const BwdArgs& a, hipStream_t st);

// ---------------------------------------------------------------- device helpers
// 32x32x16 bf16 MFMA.  Lane l: A row / B column l%32, reduction index
// 8*(l/32) + i for element i of the operand; C column l%32, C row
// 8*(j/4) + 4*(l/32) + j%4 for accumulator element j.
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// The value held by the lane 32 apart (the lane sharing this accumulator column).
__device__ __forceinline__ float partner(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  // lanes 0-31 receive x[l+32] in r[1]; lanes 32-63 receive x[l-32] in r[0]
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

// Tile shapes of the attention kernels.
constexpr int kFwdBM = 128, kFwdBN = 64;     // forward and dQ: query tile x key tile
constexpr int kDkvBM = 64, kDkvBN = 128;     // dK/dV: query tile x key tile

}  // namespace aa
