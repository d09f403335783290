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
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
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

// Interleaved chunks: per-chunk placement in the permuted row and per-row
// validity (k_chunk_layout), the permuted row's source tokens (k_chunk_tokens).
constexpr int kMaxChunksPerRow = 4096;
struct ChunkBufs {
  int32_t* new_start;  // [n_chunks] chunk start in the permuted row (row-local)
  int32_t* doc_start;  // [n_chunks] start of the chunk's document there
  int32_t* doc_end;    // [n_chunks] end (exclusive) of the chunk's document there
  int32_t* row_ok;     // [B] 1 when the row's chunks are valid
  int32_t* src;        // [B*S] permuted token -> original token
};

// Buffers of one tile plan.
// Tile (qt, kt) of a plan holds rows origin + qt*BM .. and keys
// origin + kt*BN .. (row-local, cut at S; nq = ceil(S/BM), nk = ceil(S/BN)).
// With origin 1 (rows that start with the shared anchor) no tile holds the
// anchor's query row or key column: every query sees the anchor column
// outside the tiles, and the anchor row sees only itself.
struct PlanBufs {
  int BM, BN, nq, nk;
  int origin;          // 0 or 1
  size_t cap;          // B * nq * nk
  uint8_t* kinds;      // dense [B][nq][nk]
  uint8_t* kinds_t;    // dense [B][nk][nq] (key-major copy)
  int32_t* cntq;       // [B*nq]
  int32_t* cntk;       // [B*nk]
  int32_t* qptr;       // [B*nq + 1]
  int32_t* kidx;       // [cap]
  uint8_t* kkind;      // [cap]
  int32_t* kpack;      // [cap] kidx | kkind << 24 (read with scalar loads), may be null
  int32_t* kptr;       // [B*nk + 1]
  int32_t* qidx;       // [cap]
  uint8_t* qkind;      // [cap]
  int32_t* qpack;      // [cap] qidx | qkind << 24, may be null
  int32_t* n_live;     // [1]
  int32_t* order;      // [B*nq + 1] work order of the query tiles, then its flags (kOrder*);
                       // null where no attention kernel runs on the plan
};

// ---------------------------------------------------------------- launchers
hipError_t launch_positions(const int32_t* cu, int n_seg, int B, int S, int causal, int mode,
                            int anchor, TokenTables tt, int32_t* status, hipStream_t st);
// Where a plan build gets its token tables: with cu (device cu_doc_lens) it
// computes them into tt (position IDs, key intervals) and checks the segment
// layout into status; with cu null it reads tt.
struct PlanSrc {
  const int32_t* cu;
  int n_seg, causal, mode;
  TokenTables tt;
  int32_t* status;
};
// Tile plans in one pass over the rows: a query-major plan pq (kinds,
// qptr/kidx/kkind/kpack, n_live, and the work order when pq->order is set)
// and/or a key-major plan pk (kinds_t, kptr/qidx/qkind/qpack; pk->cntk must
// be zero beforehand; n_live when pq is null).  Either may be null.
hipError_t launch_plans(const PlanSrc& src, int B, int S, int anchor, const PlanBufs* pq,
                        const PlanBufs* pk, hipStream_t st);
// Clears *status (when not null) and n int32 values at p.
hipError_t launch_clear(int32_t* status, int32_t* p, int n, hipStream_t st);
// The RoPE table.  It runs first in every attention call, so it also clears
// *status and the n_zero int32 values at zero (when not null).
hipError_t launch_rope_table(int S, int D, const RopeTheta& th, float* table, int32_t* status,
                             int32_t* zero, int n_zero, hipStream_t st);
hipError_t launch_chunk_layout(const int32_t* cu, const int32_t* chunk_doc, int n_chunks, int B,
                               int S, int causal, int mode, int anchor, ChunkBufs cb,
                               TokenTables tt, int32_t* status, hipStream_t st);
// y[p] = x[src[p]] for rows of H*D elements (one token's heads).
hipError_t launch_tile_order(const int32_t* cnt, int n, int32_t* order, hipStream_t st);
hipError_t launch_gather_rows(const bf16* x, const int32_t* src, int B, int S, int H, int D,
                              bf16* y, hipStream_t st);
hipError_t launch_rope_apply(const bf16* x, const int32_t* src, const int32_t* pos, const float* table, int npos, int B, int S,
                             int H, int D, bf16* x_rot, hipStream_t st);
// The forward.  With q_raw non-null it rotates Q itself as it loads it (from
// q_raw, positions tt.pos and the RoPE table of npos rows) and writes the
// rotated q to qr for the backward; otherwise it reads qr, rotated before.
// With tok_map non-null (rows permuted so that documents are contiguous) the
// output of position p goes to token tok_map[p] of o and lse.
// o is bf16, or float32 with o_f32.
hipError_t launch_fwd(const bf16* q_raw, const float* table, int npos, bf16* qr, const bf16* kr,
                      const bf16* v, TokenTables tt, const PlanBufs& pb, const int32_t* status,
                      int B, int S, int Hq, int Hkv, int D, float scale, int anchor, void* o,
                      int o_f32, float* lse, const int32_t* tok_map, hipStream_t st);

struct BwdArgs {
  const bf16* qr;      // rotated q [B,S,Hq,D]
  const bf16* kr;      // rotated k [B,S,Hkv,D]
  const bf16* v;
  const void* o;       // bf16, or float32 with o_f32
  const bf16* dout;
  const float* lse;    // [B,Hq,S]
  const float* table;  // RoPE cos/sin table [S][D/2][2]
  TokenTables tt;
  const int32_t* status;
  float* dvec;         // [B,Hq,S]   rowsum(dO * O)
  float* ds0;          // [B,Hq,S]   dS of the anchor column
  float* qstats;       // [B,Hq,nblk][4][kPreRows] per 64-query tile: LSE*log2(e), Dv, lo, hi
  float* part_dk;      // [B,Hq,nblk,D] per-row-block sums for the anchor key
  float* part_dv;      // [B,Hq,nblk,D]
  int nblk;
  bf16* dq;
  bf16* dk;
  bf16* dv;
  int B, S, Hq, Hkv, D;
  float scale;
  int anchor;          // 0: rows without a shared anchor (intra-document attention)
  int origin = 0;      // the tile grid's first row (PlanBufs::origin); blocks of the
                       // preprocess follow it
  // Rows permuted so that documents are contiguous: position p (over B*S) is
  // token tok_map[p] of the caller's o, lse, dq, dk, dv; qr, kr, v, dout and
  // the token tables are in permuted order.  Null: no permutation.
  const int32_t* tok_map = nullptr;
  int o_f32 = 0;
};
constexpr int kPreRows = 64;    // rows per block of the backward preprocess

hipError_t launch_bwd_pre(const BwdArgs& a, hipStream_t st);
hipError_t launch_bwd_dkdv(const BwdArgs& a, const PlanBufs& pk, const PlanBufs& pq,
                           hipStream_t st);
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

// RoPE (Eq. 6 of arXiv 2411.13476 as given on the paper-graph architecture
// page, section 3.4) of 8 consecutive features x[d0 .. d0+8), four adjacent
// pairs, of a token at table row p: tb = table + (p * (D/2) + d0/2) * 2 holds
// {cos, sin} of the four pair angles.  Float32 rotation, bf16 result (RNE).
// The RoPE pass and the forward's Q loads share this one definition, so a
// rotated vector is the same bits wherever it is formed.
__device__ __forceinline__ bf16x8 rope_rotate8(const bf16x8 xv, const float* tb) {
  const f32x4 cs01 = ((const f32x4*)tb)[0];   // cos0 sin0 cos1 sin1
  const f32x4 cs23 = ((const f32x4*)tb)[1];
  bf16x8 out;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float c = q < 2 ? cs01[2 * (q & 1)] : cs23[2 * (q & 1)];
    const float s = q < 2 ? cs01[2 * (q & 1) + 1] : cs23[2 * (q & 1) + 1];
    const float x0 = (float)xv[2 * q], x1 = (float)xv[2 * q + 1];
    out[2 * q] = (bf16)__builtin_fmaf(x0, c, -x1 * s);
    out[2 * q + 1] = (bf16)__builtin_fmaf(x0, s, x1 * c);
  }
  return out;
}

// ---------------------------------------------------------------- LDS tiles
// A [rows][D] bf16 tile in LDS, row-major with the 16-byte chunks of each row
// permuted by an XOR swizzle, so that both access patterns of the kernels are
// free of bank conflicts:
//   * row reads: 16 consecutive rows, the same 16-byte chunk (MFMA operand
//     whose reduction runs along the features);
//   * transposed reads (ds_read_b64_tr_b16): 4 consecutive rows x 4
//     consecutive chunks per 32 lanes (MFMA operand whose reduction runs
//     along the rows).
// For D = 128 a row is exactly one 256-byte bank row; the permutation swaps
// the two 2-bit fields of (row mod 16).  For D = 64 two rows share a bank row.
template <int D>
struct SwzTile {
  static constexpr int kChunks = D / 8;
  __device__ static __forceinline__ int swz(int row) {
    return D == 128 ? (((row & 3) << 2) | ((row >> 2) & 3)) : ((row >> 1) & 7);
  }
  // element offset of (row, 8-element chunk c)
  __device__ static __forceinline__ int chunk_off(int row, int c) {
    return row * D + ((c ^ swz(row)) & (kChunks - 1)) * 8;
  }
  // element offset of (row, feature f) for f a multiple of 4
  __device__ static __forceinline__ int off(int row, int f) {
    return chunk_off(row, f >> 3) + (f & 7);
  }
};

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// One 8-byte transposed LDS read: within each group of 16 lanes, lane t
// receives element t%4 of the 8-byte pieces addressed by lanes t/4 + 4*i,
// i = 0..3.
__device__ __forceinline__ i16x4 ds_read_tr(const bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

// MFMA operand whose reduction index runs over tile rows r0 .. r0+15 and
// whose row/column index is the feature f0 + (lane % 32), read from a
// row-major swizzled tile.  Element i of lane l holds
//   T[r0 + 8*(i/4) + 4*(l/32) + i%4][f0 + l%32],
// the row order of a 32x32 accumulator column, so that this operand pairs
// with B/A operands built directly from accumulator registers.
template <int D>
__device__ __forceinline__ bf16x8 tr_operand(const bf16* tile, int r0, int f0) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, t = lane & 15;
  const int row = r0 + 4 * (g >> 1) + (t >> 2);
  const int f = f0 + 16 * (g & 1) + 4 * (t & 3);
  // whole-vector casts: the two 4-element results become the two halves of
  // the operand without element-wise repacking
  const bf16x4 a = __builtin_bit_cast(bf16x4, ds_read_tr(tile + SwzTile<D>::off(row, f)));
  const bf16x4 b = __builtin_bit_cast(bf16x4, ds_read_tr(tile + SwzTile<D>::off(row + 8, f)));
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// The same operand addressed by XOR.  In a swizzled row the byte offset of
// chunk c is that of chunk (c mod 4) XOR 16 (c - c mod 4): the chunk's high
// bits only flip address bits of the chunk field that the row part (a
// multiple of 2D bytes) and the low chunk bits never touch.  So one register
// per lane and piece serves every 32-feature block f0 with one XOR, instead
// of one precomputed register per block.  o0, o8 (tr_lane_offsets): this
// lane's byte offsets of the two 8-row pieces for r0 = 0, f0 = 0.  b0, b8:
// o0, o8 plus the byte offset of the tile inside `tile`, which must be a
// multiple of 2D (a whole row) so that the XOR only meets the lane's own
// chunk bits.  r0 a multiple of 16, f0 of 32.
template <int D>
__device__ __forceinline__ void tr_lane_offsets(uint32_t& o0, uint32_t& o8) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, t = lane & 15;
  const int row = 4 * (g >> 1) + (t >> 2);
  const int f = 16 * (g & 1) + 4 * (t & 3);
  o0 = 2u * SwzTile<D>::off(row, f);
  o8 = 2u * SwzTile<D>::off(row + 8, f);
}
template <int D>
__device__ __forceinline__ bf16x8 tr_operand_x(const char* tile, uint32_t b0, uint32_t b8, int r0,
                                               int f0) {
  const uint32_t x = 2u * f0, rb = 2u * r0 * D;
  const bf16x4 a = __builtin_bit_cast(bf16x4, ds_read_tr((const bf16*)(tile + ((b0 ^ x) + rb))));
  const bf16x4 b = __builtin_bit_cast(bf16x4, ds_read_tr((const bf16*)(tile + ((b8 ^ x) + rb))));
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

typedef __attribute__((address_space(3))) void lds_void;

// 32-bit LDS address of a __shared__ location, and back.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(lds_void*)p;
}
__device__ __forceinline__ lds_void* lds_ptr(uint32_t a) { return (lds_void*)(uintptr_t)a; }

// Direct copy of 16 bytes per lane from global memory into LDS
// (buffer_load_dwordx4 ... lds): lane L reads base + voff and writes the 16
// bytes at lds + 16 L.  `base` must be wave-uniform (it is read into scalar
// registers).  The buffer form is used rather than global_load_lds: with a
// global-segment LDS load in flight the compiler assumes the LDS counter may
// complete out of order and waits for every outstanding LDS read
// (lgkmcnt(0)) before using any of them, so no operand read can be issued
// ahead of its MFMA; the buffer form counts only in the vector-memory
// counter and leaves the LDS reads' waits exact.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, lds_void* lds) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void* ub = (void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
  // raw buffer: stride 0, 2^31 - 1 bytes addressable from `base`, the data
  // format word of a plain dword buffer
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(ub, 0, 0x7fffffff, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, lds, 16, voff, 0, 0, 0);
}

// Direct global -> LDS copy (dma16 above) of a [ROWS][D] tile
// into the swizzled layout: lane L of a wave's instruction writes the 16
// bytes at LDS chunk base + L, so each lane fetches the logical chunk that
// the swizzle places there.  Global rows row0 .. row0+ROWS-1 are clamped to
// row_max.  Every thread of the NTHREADS-thread workgroup calls it; the data
// is visible after wait_direct_loads() and a workgroup barrier.
// DirectTile<D, ROWS, NTHREADS>::init() precomputes each lane's element
// offsets (row * row_stride + chunk * 8) inside a tile; load() adds the
// tile's first row (a wave-uniform base) and only re-derives clamped offsets
// for a tile that runs past row_max.
template <int D, int ROWS, int NTHREADS>
struct DirectTile {
  static constexpr int NCH = D / 8;
  static constexpr int ITERS = ROWS * NCH / NTHREADS;
  static_assert(ROWS * NCH % NTHREADS == 0, "tile must split evenly over the waves");
  uint32_t off[ITERS];   // byte offset of this lane's 16 bytes from the tile's first row
  __device__ __forceinline__ static void locate(int u, int& row, int& chunk) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int pc_idx = (wave * ITERS + u) * 64 + lane;
    row = pc_idx / NCH;
    chunk = ((pc_idx % NCH) ^ SwzTile<D>::swz(row)) & (NCH - 1);
  }
  __device__ __forceinline__ void init(size_t row_stride) {
#pragma unroll
    for (int u = 0; u < ITERS; ++u) {
      int row, chunk;
      locate(u, row, chunk);
      off[u] = (uint32_t)((row * row_stride + chunk * 8) * sizeof(bf16));
    }
  }
  // load() with the LDS tile given by its 32-bit address.  The compiler then
  // ties the copy to no __shared__ variable and inserts no wait for it before
  // LDS reads; the caller's wait_direct_loads() and barrier order the data.
  __device__ __forceinline__ void load_at(uint32_t lds_tile, const bf16* gbase, size_t row_stride,
                                          int row0, int row_max) const {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (row0 + ROWS - 1 <= row_max) {
      const char* tbase = (const char*)(gbase + (size_t)row0 * row_stride);
#pragma unroll
      for (int u = 0; u < ITERS; ++u)
        dma16(tbase, off[u], lds_ptr(lds_tile + (wave * ITERS + u) * 64 * 16));
    } else {
      const int rb = min(row0, row_max);
      const char* cbase = (const char*)(gbase + (size_t)rb * row_stride);
#pragma unroll
      for (int u = 0; u < ITERS; ++u) {
        int row, chunk;
        locate(u, row, chunk);
        const int r = min(row0 + row, row_max) - rb;
        dma16(cbase, (uint32_t)((r * row_stride + chunk * 8) * sizeof(bf16)),
              lds_ptr(lds_tile + (wave * ITERS + u) * 64 * 16));
      }
    }
  }
  // The tile base is uniform and the offsets are 32-bit, so every load takes
  // the buffer descriptor (scalar) + vector-offset form with its LDS address
  // in M0.
  __device__ __forceinline__ void load(bf16* lds_tile, const bf16* gbase, size_t row_stride,
                                       int row0, int row_max) const {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (row0 + ROWS - 1 <= row_max) {
      const char* tbase = (const char*)(gbase + (size_t)row0 * row_stride);
#pragma unroll
      for (int u = 0; u < ITERS; ++u)
        dma16(tbase, off[u], (lds_void*)(lds_tile + (wave * ITERS + u) * 64 * 8));
    } else {
      // Rows past row_max read row_max.  The offsets are unsigned, so they are
      // taken from min(row0, row_max): a tile may start past the last row
      // (the second half of a last query tile), and every offset stays >= 0.
      const int rb = min(row0, row_max);
      const char* cbase = (const char*)(gbase + (size_t)rb * row_stride);
#pragma unroll
      for (int u = 0; u < ITERS; ++u) {
        int row, chunk;
        locate(u, row, chunk);
        const int r = min(row0 + row, row_max) - rb;
        dma16(cbase, (uint32_t)((r * row_stride + chunk * 8) * sizeof(bf16)),
              (lds_void*)(lds_tile + (wave * ITERS + u) * 64 * 8));
      }
    }
  }
};

// Wait until this wave's direct-to-LDS loads (and other vector memory loads)
// have completed: s_waitcnt vmcnt(0).
__device__ __forceinline__ void wait_direct_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Wait until at most N of this wave's vector memory loads are outstanding
// (s_waitcnt vmcnt(N), N < 64; the count's high bits live in bits 15:14):
// every load issued before the last N is done.
template <int N>
__device__ __forceinline__ void wait_loads_but() {
  static_assert(N >= 0 && N < 64, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// ---------------------------------------------------------------- XCD-aware order
// The MI355X dispatcher deals consecutive workgroup ids round-robin to its
// 8 XCDs, each with a private L2.  Work items that share K/V or Q/dO tiles
// are neighbours in the natural order (tiles of one head and document), so a
// launch of padded_grid(total) workgroups maps id L to work item
// (L % 8) * per + L / 8: every XCD walks one contiguous slice of the items.
// Returns -1 for the padding workgroups (at most 7).
constexpr int kXcds = 8;
__host__ __device__ inline int xcd_per(int total) { return (total + kXcds - 1) / kXcds; }
__host__ __device__ inline int padded_grid(int total) { return xcd_per(total) * kXcds; }
__device__ __forceinline__ int xcd_work_item(int linear, int total) {
  const int w = (linear % kXcds) * xcd_per(total) + linear / kXcds;
  return w < total ? w : -1;
}

// Work order of a launch over H heads x T tiles.  The plan builder writes,
// for its T = B * nq query tiles, order[0 .. T) (the tiles in launch order)
// and order[T] (these flags):
//  kOrderLpt         the tiles go by descending live-tile count, ties by index
//                    (longest processing time first); else natural order.
//                    Chosen when the largest count exceeds 1.5x the mean.
//  kOrderInterleave  an XCD's slice of work items (H / 8 whole heads when H is
//                    a multiple of 8) is walked rank-major across its heads,
//                    so the first tiles of all its heads start together; else
//                    head after head.  Chosen when a head has at most
//                    kInterleaveMaxTiles tiles (about two rounds of an XCD's
//                    concurrent workgroups, where walking head after head
//                    starts the last head's long tiles late) or when the work
//                    is even (the heads' tiles of one token range then run
//                    together and their K/V rows are adjacent in HBM).  With
//                    many tiles per head and uneven work, head after head
//                    keeps one head's concurrent tiles on shared K/V in L2.
constexpr int kOrderLpt = 1, kOrderInterleave = 2;   // AA_ORDER_LPT, AA_ORDER_INTERLEAVE
constexpr int kInterleaveMaxTiles = 128;

// Workgroup -> (head, rank of its tile in the order), or false for a padding
// workgroup.  When H is a multiple of the XCD count each XCD walks whole
// heads (xcd_work_item), as described with kOrderInterleave.  Otherwise an
// XCD's slice would hold part of a head, and in longest-first order the
// first slice would get that head's long tiles and the next one its short
// tiles; there the workgroups take the items rank-major across heads in
// plain launch order, so that the dispatcher's round-robin deals every
// rank's tiles evenly over the XCDs.
__device__ __forceinline__ bool work_head_rank(int T, int H, int flags, int& head, int& rank) {
  const int n_items = T * H;
  if (H % kXcds != 0) {
    const int w = blockIdx.x;
    if (w >= n_items) return false;
    head = w % H;
    rank = w / H;
    return true;
  }
  const int w = xcd_work_item(blockIdx.x, n_items);
  if (w < 0) return false;
  if (flags & kOrderInterleave) {
    const int G = H / kXcds, slice = G * T;
    const int x = w / slice, u = w - x * slice;
    head = x * G + u % G;
    rank = u / G;
    return true;
  }
  head = w / T;
  rank = w - head * T;
  return true;
}

// Packed plan entries: tile index in the low 24 bits, kind in the high 8.
__host__ __device__ inline int pack_tile(int idx, int kind) { return idx | (kind << 24); }
__device__ __forceinline__ int packed_idx(int v) { return v & 0xffffff; }
__device__ __forceinline__ int packed_kind(int v) { return (unsigned)v >> 24; }

// Wait until at most `tiles` groups of PER vector-memory instructions issued
// after the one waited for are still outstanding (tiles <= 3).
template <int PER>
__device__ __forceinline__ void wait_all_but_tiles(int tiles) {
  if (tiles <= 0) wait_direct_loads();
  else if (tiles == 1) wait_loads_but<PER>();
  else if (tiles == 2) wait_loads_but<(2 * PER < 63 ? 2 * PER : 63)>();
  else wait_loads_but<(3 * PER < 63 ? 3 * PER : 63)>();
}

// Tile shapes of the attention kernels.
#ifndef AA_FWD_BN
#define AA_FWD_BN 64
#endif
#ifndef AA_FWD_STAGES
#define AA_FWD_STAGES 2
#endif
#ifndef AA_FWD_BM
#define AA_FWD_BM 128
#endif
constexpr int kFwdBM = AA_FWD_BM, kFwdBN = AA_FWD_BN;   // forward and dQ: query tile x key tile
constexpr int kFwdThreads = 2 * kFwdBM;                  // one wave per 32 queries
constexpr int kFwdBlocksPerCU = 512 / kFwdThreads;       // two waves per SIMD
constexpr int kFwdStages = AA_FWD_STAGES;         // K/V tiles in LDS (prefetch depth + 1)
constexpr int kDkvBM = 64, kDkvBN = 128;          // dK/dV: query tile x key tile

}  // namespace aa
