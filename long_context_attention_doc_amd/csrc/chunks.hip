// Interleaved document chunks (arch page of arXiv 2411.13476, section 5,
// "AnchorAttention with Interleaved Chunks", Figure 5 middle and right):
// documents are cut into chunks that are shuffled across a packed row, every
// document keeping the order of its own tokens.  The mask still lets a query
// see its anchor and the keys of its own document (in any chunk) that are not
// after it.
//
// The library turns this into the contiguous case by a permutation of each
// row: the anchor first, then every document's tokens in their own order,
// documents by ascending id.  The permutation keeps the order inside every
// document, so "same document and not after the query" is the same relation
// before and after it, and the block-sparse kernels run unchanged on the
// permuted row.  Q and K are gathered by the RoPE pass itself and V and dO
// (streamed through LDS tiles) by the gather below; every other access to a
// caller's tensor (O and LSE written by the forward and read by the backward,
// dq, dk, dv) goes through the permutation inside the kernels.
//
// k_chunk_layout sorts the chunks of a row by (document id, chunk index) in
// LDS and assigns every chunk its place in the permuted row; k_chunk_tokens
// then writes, per permuted token, its source token, position ID and visible
// key interval.
#include "aa_internal.h"

namespace aa {

// Inclusive scan of buf[0, n) in place with `op` (n <= 4 * blockDim.x,
// blockDim.x == 1024); part holds 1024 ints of scratch.
template <typename Op>
__device__ void block_scan_incl(int* buf, int n, Op op, int identity, int* part) {
  const int t = threadIdx.x;
  int v[4];
  int acc = identity;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int idx = 4 * t + k;
    acc = op(acc, idx < n ? buf[idx] : identity);
    v[k] = acc;
  }
  part[t] = acc;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int y = t >= off ? part[t - off] : identity;
    __syncthreads();
    part[t] = op(part[t], y);
    __syncthreads();
  }
  const int pre = t > 0 ? part[t - 1] : identity;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int idx = 4 * t + k;
    if (idx < n) buf[idx] = op(pre, v[k]);
  }
  __syncthreads();
}

struct OpAdd {
  __device__ int operator()(int a, int b) const { return a + b; }
};
struct OpMin {
  __device__ int operator()(int a, int b) const { return a < b ? a : b; }
};

// One workgroup of 1024 threads per row b.  Validates the row's chunks
// (they start at the row start, end at the row end, are non-empty; with an
// anchor the first is the one-token anchor with id -1 and no other has -1;
// without an anchor every id is >= 0; at most kMaxChunksPerRow of them) and,
// for a valid row, writes for every chunk c its start in the permuted row
// (row-local), and the start and end of its document there.
__global__ __launch_bounds__(1024) void k_chunk_layout(
    const int32_t* __restrict__ cu, const int32_t* __restrict__ chunk_doc, int n_chunks, int B,
    int S, int anchor, int32_t* __restrict__ new_start, int32_t* __restrict__ doc_start,
    int32_t* __restrict__ doc_end, int32_t* __restrict__ row_ok, int32_t* __restrict__ status) {
  __shared__ unsigned long long key[kMaxChunksPerRow];
  __shared__ int bstart[kMaxChunksPerRow];
  __shared__ int bdoc[kMaxChunksPerRow];
  __shared__ int bend[kMaxChunksPerRow];
  __shared__ int part[1024];
  __shared__ int s_c0, s_n, s_bad;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const long long rs = (long long)b * S, re = rs + S;
  if (tid == 0) {
    int lo = 0, hi = n_chunks;                   // first chunk starting at or after rs
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if ((long long)cu[mid] < rs) lo = mid + 1; else hi = mid;
    }
    const int c0 = lo;
    lo = c0; hi = n_chunks;                      // first boundary at or after re (cu[n_chunks] = B*S)
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if ((long long)cu[mid] < re) lo = mid + 1; else hi = mid;
    }
    const int c1 = lo;
    int bad = c0 >= n_chunks || (long long)cu[c0] != rs || (long long)cu[c1] != re || c1 <= c0 ||
              c1 - c0 > kMaxChunksPerRow;
    s_c0 = c0;
    s_n = bad ? 0 : c1 - c0;
    s_bad = bad;
  }
  __syncthreads();
  const int c0 = s_c0, n = s_n;
  int npow = 1;
  while (npow < n) npow <<= 1;
  for (int i = tid; i < npow; i += 1024) {
    if (i < n) {
      const int c = c0 + i;
      const int len = cu[c + 1] - cu[c];
      const int d = chunk_doc[c];
      const bool ok = len > 0 && (anchor ? (i == 0 ? (d == -1 && len == 1) : d >= 0) : d >= 0);
      if (!ok) s_bad = 1;                        // every writer stores the same value
      key[i] = ((unsigned long long)(unsigned)(d + 1) << 32) | (unsigned)i;
    } else {
      key[i] = ~0ull;
    }
  }
  __syncthreads();
  if (s_bad) {
    if (tid == 0) {
      row_ok[b] = 0;
      status[0] = kStatusBadDocs;
    }
    return;
  }
  // bitonic sort of the keys, ascending: documents by id, chunks in order
  for (int k = 2; k <= npow; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < npow; i += 1024) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const bool up = (i & k) == 0;
          const unsigned long long x = key[i], y = key[ixj];
          if ((x > y) == up) {
            key[i] = y;
            key[ixj] = x;
          }
        }
      }
      __syncthreads();
    }
  }
  // chunk starts in the permuted row: exclusive sum of the sorted lengths
  for (int i = tid; i < n; i += 1024) {
    const int c = c0 + (int)(unsigned)(key[i] & 0xffffffffull);
    bstart[i] = cu[c + 1] - cu[c];
    bdoc[i] = (int)(key[i] >> 32);
  }
  __syncthreads();
  block_scan_incl(bstart, n, OpAdd{}, 0, part);
  for (int i = tid; i < n; i += 1024) {
    const int c = c0 + (int)(unsigned)(key[i] & 0xffffffffull);
    bstart[i] -= cu[c + 1] - cu[c];              // inclusive -> exclusive
  }
  __syncthreads();
  // document ends: the start of the next document after i (S after the last),
  // as a minimum scan from the right over the document boundaries
  for (int i = tid; i < n; i += 1024) {
    const int j = n - 1 - i;                     // reversed index
    bend[i] = j == n - 1 ? S : (bdoc[j + 1] != bdoc[j] ? bstart[j + 1] : 0x7fffffff);
  }
  __syncthreads();
  block_scan_incl(bend, n, OpMin{}, 0x7fffffff, part);
  // document starts: the start of the document's first chunk.  Starts grow
  // with i, so it is the largest first-chunk start at or before i; written as
  // a minimum scan over negated values.
  int* bfirst = reinterpret_cast<int*>(key);     // keys are no longer needed after this copy
  int idx_keep[4];
  for (int k = 0; k < 4; ++k) {
    const int i = tid + 1024 * k;
    idx_keep[k] = i < n ? (int)(unsigned)(key[i] & 0xffffffffull) : 0;
  }
  __syncthreads();
  for (int k = 0; k < 4; ++k) {
    const int i = tid + 1024 * k;
    if (i < n) bfirst[i] = (i == 0 || bdoc[i - 1] != bdoc[i]) ? -bstart[i] : 0x7fffffff;
  }
  __syncthreads();
  block_scan_incl(bfirst, n, OpMin{}, 0x7fffffff, part);
  for (int k = 0; k < 4; ++k) {
    const int i = tid + 1024 * k;
    if (i < n) {
      const int c = c0 + idx_keep[k];
      new_start[c] = bstart[i];
      doc_start[c] = -bfirst[i];
      doc_end[c] = bend[n - 1 - i];
    }
  }
  if (tid == 0) row_ok[b] = 1;
}

// One thread per token t of the original stream: its chunk (binary search),
// its place p in the permuted row and, indexed by p, the source token, the
// position ID and the visible key interval (row-local, permuted order).  Also
// validates cu as k_positions does.  A row that failed validation keeps the
// identity order with every query masked.
__global__ void k_chunk_tokens(const int32_t* __restrict__ cu, const int32_t* __restrict__ chunk_doc,
                               int n_chunks, int B, int S, int causal, int mode, int anchor,
                               const int32_t* __restrict__ new_start,
                               const int32_t* __restrict__ doc_start,
                               const int32_t* __restrict__ doc_end,
                               const int32_t* __restrict__ row_ok, int32_t* __restrict__ src,
                               int32_t* __restrict__ pos, int32_t* __restrict__ lo,
                               int32_t* __restrict__ hi, int32_t* __restrict__ status) {
  const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long total = (long long)B * S;
  if (t < n_chunks && cu[t] >= cu[t + 1]) status[0] = kStatusBadDocs;
  if (t == 0 && (cu[0] != 0 || (long long)cu[n_chunks] != total)) status[0] = kStatusBadDocs;
  if (t >= total) return;
  int a = 0, bnd = n_chunks - 1;                 // largest c with cu[c] <= t
  while (a < bnd) {
    const int mid = (a + bnd + 1) >> 1;
    if ((long long)cu[mid] <= t) a = mid; else bnd = mid - 1;
  }
  const int c = a;
  const long long rs = (t / S) * (long long)S;
  const int local = (int)(t - rs);
  const bool ok = row_ok[t / S] != 0 && cu[c] <= t && t < cu[c + 1];
  if (!ok) {
    src[t] = (int32_t)t;
    pos[t] = 0;
    lo[t] = 1;
    hi[t] = 0;
    return;
  }
  int pl = new_start[c] + (int)(t - cu[c]);
  pl = pl < 0 ? 0 : (pl > S - 1 ? S - 1 : pl);
  const long long p = rs + pl;
  src[p] = (int32_t)t;
  if (anchor && chunk_doc[c] == -1) {
    pos[p] = 0;
    lo[p] = 1;
    hi[p] = 0;
  } else {
    const int ds = doc_start[c], de = doc_end[c];
    pos[p] = mode == 0 ? pl - ds + 1 : local;
    lo[p] = ds;
    hi[p] = causal ? pl : de - 1;
  }
}

// y[p] = x[src[p]] for rows of row_vecs 16-byte vectors (one token's heads).
__global__ void k_gather_rows(const bf16* __restrict__ x, const int32_t* __restrict__ src,
                              long long n_vec, int row_vecs, bf16* __restrict__ y) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_vec) return;
  const long long p = i / row_vecs;
  const int w = (int)(i % row_vecs);
  *(bf16x8*)(y + i * 8) = *(const bf16x8*)(x + ((long long)src[p] * row_vecs + w) * 8);
}

hipError_t launch_chunk_layout(const int32_t* cu, const int32_t* chunk_doc, int n_chunks, int B,
                               int S, int causal, int mode, int anchor, ChunkBufs cb,
                               TokenTables tt, int32_t* status, hipStream_t st) {
  hipLaunchKernelGGL(k_chunk_layout, dim3(B), dim3(1024), 0, st, cu, chunk_doc, n_chunks, B, S,
                     anchor, cb.new_start, cb.doc_start, cb.doc_end, cb.row_ok, status);
  const long long total = (long long)B * S;
  const long long n = total > n_chunks ? total : n_chunks;
  hipLaunchKernelGGL(k_chunk_tokens, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, cu,
                     chunk_doc, n_chunks, B, S, causal, mode, anchor, cb.new_start, cb.doc_start,
                     cb.doc_end, cb.row_ok, cb.src, tt.pos, tt.lo, tt.hi, status);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const bf16* x, const int32_t* src, int B, int S, int H, int D,
                              bf16* y, hipStream_t st) {
  const int row_vecs = H * D / 8;
  const long long n = (long long)B * S * row_vecs;
  hipLaunchKernelGGL(k_gather_rows, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, x, src, n,
                     row_vecs, y);
  return hipGetLastError();
}

}  // namespace aa
