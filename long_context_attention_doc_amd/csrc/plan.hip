// Position IDs and the block-sparse tile plan.
//
// Position IDs follow the paper-graph architecture page of arXiv 2411.13476,
// section 3.4, "Intra-document attention with position ID reset (Figure 2,
// middle)": IDs restart at every document and a document's first token gets
// ID 1; the shared anchor (section 3.4, "AnchorAttention: The Shared Anchor
// Design") keeps ID 0.  The mask is the page's "Mask construction": every
// query sees its row's anchor, causal keys of its own document, nothing else.
//
// Because documents are contiguous segments, what query t sees besides the
// anchor is one closed interval of keys [lo[t], hi[t]] (row-local); the tile
// plan and the attention kernels use only these intervals.
//
// Two options follow the other paradigms of the page's Figure 2: continuous
// position IDs (the row-local index, as in the page's "Core design" of
// AnchorAttention and in standard intra-document attention), and rows
// without an anchor (intra-document attention, Figure 2 left and middle),
// where the row's first token is an ordinary document token and a query sees
// only its own document.
#include "aa_internal.h"

namespace aa {

// One thread per token: segment lookup by binary search over cu_doc_lens,
// position ID, visible-key interval, and validation of the segment layout.
// Every derived index is clamped into the row so that later kernels stay in
// bounds even when cu_doc_lens is invalid (the status word reports it).
// mode 0: reset (a document's first token gets 1); 1: continuous (row-local
// index).  anchor 0: no anchor, every token belongs to a document.
__global__ void k_positions(const int32_t* __restrict__ cu, int n_seg, int B, int S, int causal,
                            int mode, int anchor, int32_t* __restrict__ pos,
                            int32_t* __restrict__ lo, int32_t* __restrict__ hi,
                            int32_t* __restrict__ status) {
  const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long total = (long long)B * S;
  if (t < n_seg) {
    if (cu[t] >= cu[t + 1]) status[0] = kStatusBadDocs;
  }
  if (t == 0) {
    if (cu[0] != 0 || (long long)cu[n_seg] != total) status[0] = kStatusBadDocs;
  }
  if (t >= total) return;
  int a = 0, bnd = n_seg - 1;             // largest k with cu[k] <= t
  while (a < bnd) {
    const int mid = (a + bnd + 1) >> 1;
    if ((long long)cu[mid] <= t) a = mid; else bnd = mid - 1;
  }
  const long long s = cu[a], e = cu[a + 1];
  const long long rs = (t / S) * (long long)S;
  bool bad = !(s <= t && t < e && s >= rs && e <= rs + S);
  if (anchor) {
    if (t == rs && e != rs + 1) bad = true;        // the anchor is a segment of its own
    if (t == rs + 1 && s != t) bad = true;         // so the next segment starts right after it
  }
  if (bad) status[0] = kStatusBadDocs;
  const int local = (int)(t - rs);
  const int first = anchor ? 1 : 0;                // first row-local index of a document
  int p, l, h;
  if (anchor && t == rs) {
    p = 0; l = 1; h = 0;                           // anchor: sees only itself (column 0)
  } else {
    long long sl = s - rs, el = e - rs;            // row-local segment [sl, el)
    sl = sl < first ? first : (sl > local ? local : sl);
    el = el > S ? S : (el <= local ? local + 1 : el);
    p = mode == 0 ? (int)(local - sl + 1) : local;
    l = (int)sl;
    h = causal ? local : (int)(el - 1);
  }
  pos[t] = p;
  lo[t] = l;
  hi[t] = h;
}

// One workgroup per (row b, query tile qt): classify every key tile.
// A tile is live when some query row of it sees some key of it (the anchor
// column 0 is seen by every query); FULL when all BM x BN elements exist and
// are seen; ANCHOR when it is key tile 0 and only column 0 is seen; PARTIAL
// otherwise.  Also counts the live tiles of the query tile.
__global__ void k_tile_kinds(const int32_t* __restrict__ lo, const int32_t* __restrict__ hi,
                             int S, int BM, int BN, int nq, int nk, int anchor,
                             uint8_t* __restrict__ kinds, int32_t* __restrict__ cntq) {
  __shared__ int slo[256], shi[256];
  __shared__ int wcount[8];
  const int tile = blockIdx.x;            // b * nq + qt
  const int b = tile / nq, qt = tile % nq;
  const int r0 = qt * BM;
  const int nrows = min(BM, S - r0);
  for (int r = threadIdx.x; r < BM; r += blockDim.x) {
    if (r < nrows) {
      const size_t t = (size_t)b * S + r0 + r;
      slo[r] = lo[t];
      shi[r] = hi[t];
    }
  }
  __syncthreads();
  int cnt = 0;
  for (int kt = threadIdx.x; kt < nk; kt += blockDim.x) {
    const int c0 = kt * BN;
    const int c1 = min(S, c0 + BN) - 1;
    const bool cols_exist = (c0 + BN) <= S;
    bool any_live = false, any_doc = false, all_full = nrows == BM && cols_exist;
    for (int r = 0; r < nrows; ++r) {
      const int a = max(slo[r], c0), z = min(shi[r], c1);
      const int ndoc = z >= a ? z - a + 1 : 0;
      const int n = ndoc + (anchor && kt == 0 ? 1 : 0);
      any_live |= n > 0;
      any_doc |= ndoc > 0;
      all_full &= n == BN;
    }
    uint8_t kind = 0;
    if (any_live)
      kind = all_full ? kTileFull : ((anchor && kt == 0 && !any_doc) ? kTileAnchor : kTilePartial);
    kinds[(size_t)tile * nk + kt] = kind;
    cnt += kind != 0;
  }
  // block reduction of the live count
  for (int off = 32; off > 0; off >>= 1) cnt += __shfl_xor(cnt, off);
  if ((threadIdx.x & 63) == 0) wcount[threadIdx.x >> 6] = cnt;
  __syncthreads();
  if (threadIdx.x == 0) {
    int tot = 0;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) tot += wcount[w];
    cntq[tile] = tot;
  }
}

// Single-workgroup exclusive scan: ptr[i] = sum(cnt[0..i)), ptr[n] = total.
__global__ void k_scan(const int32_t* __restrict__ cnt, int n, int32_t* __restrict__ ptr,
                       int32_t* __restrict__ total_out) {
  __shared__ int buf[1024];
  __shared__ int carry;
  if (threadIdx.x == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < n; base += 1024) {
    const int i = base + threadIdx.x;
    const int x = i < n ? cnt[i] : 0;
    buf[threadIdx.x] = x;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int y = (int)threadIdx.x >= off ? buf[threadIdx.x - off] : 0;
      __syncthreads();
      buf[threadIdx.x] += y;
      __syncthreads();
    }
    if (i < n) ptr[i] = carry + buf[threadIdx.x] - x;
    __syncthreads();
    if (threadIdx.x == 1023) carry += buf[1023];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    ptr[n] = carry;
    if (total_out) total_out[0] = carry;
  }
}

// Transposed copy of the kind matrix: kinds_t[b][kt][qt] = kinds[b][qt][kt],
// 64 x 64 blocks through LDS.
__global__ void k_transpose_kinds(const uint8_t* __restrict__ kinds, int nq, int nk,
                                  uint8_t* __restrict__ kinds_t) {
  __shared__ uint8_t blk[64][65];
  const int b = blockIdx.z;
  const int q0 = blockIdx.y * 64, k0 = blockIdx.x * 64;
  const uint8_t* src = kinds + (size_t)b * nq * nk;
  uint8_t* dst = kinds_t + (size_t)b * nq * nk;
  for (int i = threadIdx.y; i < 64; i += blockDim.y) {
    const int q = q0 + i, k = k0 + threadIdx.x;
    blk[i][threadIdx.x] = (q < nq && k < nk) ? src[(size_t)q * nk + k] : 0;
  }
  __syncthreads();
  for (int i = threadIdx.y; i < 64; i += blockDim.y) {
    const int k = k0 + i, q = q0 + threadIdx.x;
    if (k < nk && q < nq) dst[(size_t)k * nq + q] = blk[threadIdx.x][i];
  }
}

// One wave per row of a dense [rows][n] kind matrix: number of live entries.
__global__ void k_row_count(const uint8_t* __restrict__ m, int rows, int n,
                            int32_t* __restrict__ cnt) {
  const int row = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const uint8_t* r = m + (size_t)row * n;
  int c = 0;
  for (int i0 = 0; i0 < n; i0 += 64) {
    const int i = i0 + lane;
    c += __popcll(__builtin_amdgcn_ballot_w64(i < n && r[i] != 0));
  }
  if (lane == 0) cnt[row] = c;
}

// One wave per row: the live entries of the row, ascending, at ptr[row].
__global__ void k_row_compact(const uint8_t* __restrict__ m, int rows, int n,
                              const int32_t* __restrict__ ptr, int32_t* __restrict__ idx,
                              uint8_t* __restrict__ kind, int32_t* __restrict__ pack) {
  const int row = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const uint8_t* r = m + (size_t)row * n;
  int w = ptr[row];
  for (int i0 = 0; i0 < n; i0 += 64) {
    const int i = i0 + lane;
    const uint8_t k = i < n ? r[i] : 0;
    const unsigned long long live = __builtin_amdgcn_ballot_w64(k != 0);
    if (k) {
      const int before = __popcll(live & ((1ull << lane) - 1ull));
      idx[w + before] = i;
      kind[w + before] = k;
      if (pack) pack[w + before] = pack_tile(i, k);
    }
    w += __popcll(live);
  }
}

// Work order of the n query tiles of a plan (the flags are described with
// kOrderLpt): order[0 .. n) and order[n].  Every workgroup holds all counts in
// LDS and derives the same flags; thread i writes tile i at its rank, the
// number of tiles that go before it.  Plans with more than kMaxLptTiles tiles
// keep the natural order, head after head.
constexpr int kMaxLptTiles = 16384;
__global__ __launch_bounds__(256) void k_tile_order(const int32_t* __restrict__ cnt, int n,
                                                   int32_t* __restrict__ order) {
  __shared__ int w[kMaxLptTiles];
  __shared__ int wmax[4], wsum[4];
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (n > kMaxLptTiles) {
    if (i < n) order[i] = i;
    if (i == 0) order[n] = 0;
    return;
  }
  int mx = 0, sm = 0;   // counts are at most nk and n * nk < 2^29 here
  for (int j = threadIdx.x; j < n; j += 256) {
    const int c = cnt[j];
    w[j] = c;
    mx = max(mx, c);
    sm += c;
  }
  for (int off = 32; off > 0; off >>= 1) {
    mx = max(mx, __shfl_xor(mx, off));
    sm += __shfl_xor(sm, off);
  }
  if ((threadIdx.x & 63) == 0) {
    wmax[threadIdx.x >> 6] = mx;
    wsum[threadIdx.x >> 6] = sm;
  }
  __syncthreads();
  mx = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
  const long long total = (long long)wsum[0] + wsum[1] + wsum[2] + wsum[3];
  const bool lpt = 2LL * mx * n > 3LL * total;
  const bool interleave = n <= kInterleaveMaxTiles || !lpt;
  if (i == 0) order[n] = (lpt ? kOrderLpt : 0) | (interleave ? kOrderInterleave : 0);
  if (i >= n) return;
  if (!lpt) {
    order[i] = i;
    return;
  }
  const int wi = w[i];
  int rank = 0;
  for (int j = 0; j < n; ++j) {
    const int wj = w[j];
    rank += (wj > wi) || (wj == wi && j < i);
  }
  order[rank] = i;
}

hipError_t launch_tile_order(const int32_t* cnt, int n, int32_t* order, hipStream_t st) {
  hipLaunchKernelGGL(k_tile_order, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, cnt, n,
                     order);
  return hipGetLastError();
}

hipError_t launch_positions(const int32_t* cu, int n_seg, int B, int S, int causal, int mode,
                            int anchor, TokenTables tt, int32_t* status, hipStream_t st) {
  const long long total = (long long)B * S;
  const long long n = total > n_seg ? total : n_seg;
  const int threads = 256;
  const unsigned blocks = (unsigned)((n + threads - 1) / threads);
  hipLaunchKernelGGL(k_positions, dim3(blocks), dim3(threads), 0, st, cu, n_seg, B, S, causal,
                     mode, anchor, tt.pos, tt.lo, tt.hi, status);
  return hipGetLastError();
}

hipError_t launch_plan(const int32_t* lo, const int32_t* hi, int B, int S, int anchor, PlanBufs pb,
                       bool key_major, hipStream_t st) {
  const int nq = pb.nq, nk = pb.nk;
  hipLaunchKernelGGL(k_tile_kinds, dim3(B * nq), dim3(256), 0, st, lo, hi, S, pb.BM, pb.BN, nq,
                     nk, anchor, pb.kinds, pb.cntq);
  hipLaunchKernelGGL(k_scan, dim3(1), dim3(1024), 0, st, pb.cntq, B * nq, pb.qptr, pb.n_live);
  hipLaunchKernelGGL(k_row_compact, dim3((B * nq + 3) / 4), dim3(256), 0, st, pb.kinds, B * nq, nk,
                     pb.qptr, pb.kidx, pb.kkind, pb.kpack);
  if (pb.order && !key_major)   // the key-major launches read the query-major plan's flags
    hipLaunchKernelGGL(k_tile_order, dim3((B * nq + 255) / 256), dim3(256), 0, st, pb.cntq, B * nq,
                       pb.order);
  if (key_major) {
    hipLaunchKernelGGL(k_transpose_kinds, dim3((nk + 63) / 64, (nq + 63) / 64, B), dim3(64, 4), 0,
                       st, pb.kinds, nq, nk, pb.kinds_t);
    hipLaunchKernelGGL(k_row_count, dim3((B * nk + 3) / 4), dim3(256), 0, st, pb.kinds_t, B * nk,
                       nq, pb.cntk);
    hipLaunchKernelGGL(k_scan, dim3(1), dim3(1024), 0, st, pb.cntk, B * nk, pb.kptr,
                       (int32_t*)nullptr);
    hipLaunchKernelGGL(k_row_compact, dim3((B * nk + 3) / 4), dim3(256), 0, st, pb.kinds_t, B * nk,
                       nq, pb.kptr, pb.qidx, pb.qkind, pb.qpack);
  }
  return hipGetLastError();
}

}  // namespace aa
