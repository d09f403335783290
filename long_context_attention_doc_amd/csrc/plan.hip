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

// Token t's segment (binary search over cu_doc_lens), position ID and the
// closed interval [lo, hi] of keys it sees besides the anchor; *bad is set
// when the segment layout around t is invalid.  Every derived index is
// clamped into the row so that later kernels stay in bounds even then (the
// status word reports it).  mode 0: reset (a document's first token gets 1);
// 1: continuous (row-local index).  anchor 0: every token is a document token.
__device__ __forceinline__ void token_tables(long long t, const int32_t* __restrict__ cu, int n_seg,
                                             int S, int causal, int mode, int anchor, int& p,
                                             int& l, int& h, bool& bad) {
  int a = 0, bnd = n_seg - 1;             // largest k with cu[k] <= t
  while (a < bnd) {
    const int mid = (a + bnd + 1) >> 1;
    if ((long long)cu[mid] <= t) a = mid; else bnd = mid - 1;
  }
  const long long s = cu[a], e = cu[a + 1];
  const long long rs = (t / S) * (long long)S;
  bad = !(s <= t && t < e && s >= rs && e <= rs + S);
  if (anchor) {
    if (t == rs && e != rs + 1) bad = true;        // the anchor is a segment of its own
    if (t == rs + 1 && s != t) bad = true;         // so the next segment starts right after it
  }
  const int local = (int)(t - rs);
  const int first = anchor ? 1 : 0;                // first row-local index of a document
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
}

// The global checks of cu_doc_lens, spread over the threads of a launch:
// strictly increasing, from 0 to B*S.
__device__ __forceinline__ void check_offsets(long long g, const int32_t* __restrict__ cu, int n_seg,
                                              long long total, int32_t* __restrict__ status) {
  if (g < n_seg && cu[g] >= cu[g + 1]) status[0] = kStatusBadDocs;
  if (g == 0 && (cu[0] != 0 || (long long)cu[n_seg] != total)) status[0] = kStatusBadDocs;
}

// One thread per token: the token tables and the layout checks.
__global__ void k_positions(const int32_t* __restrict__ cu, int n_seg, int B, int S, int causal,
                            int mode, int anchor, int32_t* __restrict__ pos,
                            int32_t* __restrict__ lo, int32_t* __restrict__ hi,
                            int32_t* __restrict__ status) {
  const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long total = (long long)B * S;
  check_offsets(t, cu, n_seg, total, status);
  if (t >= total) return;
  int p, l, h;
  bool bad;
  token_tables(t, cu, n_seg, S, causal, mode, anchor, p, l, h, bad);
  if (bad) status[0] = kStatusBadDocs;
  pos[t] = p;
  lo[t] = l;
  hi[t] = h;
}

// Kind of the tile of query rows [r, r + nrows) (their intervals in slo/shi)
// and key tile kt of BN keys: live when some query row sees some key of it
// (the anchor column 0 is seen by every query); FULL when all BM x BN
// elements exist and are seen; ANCHOR when it is key tile 0 and only column
// 0 is seen; PARTIAL otherwise; 0 when dead.
__device__ __forceinline__ uint8_t tile_kind(const int* slo, const int* shi, int r, int nrows,
                                             int BM, int c0, int BN, int S, int anchor) {
  const int c1 = min(S, c0 + BN) - 1;
  const bool cols_exist = (c0 + BN) <= S;
  const bool anchor_col = anchor && c0 == 0;      // the tile starts at the anchor column
  bool any_live = false, any_doc = false, all_full = nrows == BM && cols_exist;
  for (int i = r; i < r + nrows; ++i) {
    const int a = max(slo[i], c0), z = min(shi[i], c1);
    const int ndoc = z >= a ? z - a + 1 : 0;
    const int n = ndoc + (anchor_col ? 1 : 0);
    any_live |= n > 0;
    any_doc |= ndoc > 0;
    all_full &= n == BN;
  }
  if (!any_live) return 0;
  return all_full ? kTileFull : ((anchor_col && !any_doc) ? kTileAnchor : kTilePartial);
}

// The same kind in O(log BM) for rows whose intervals are monotone: lo and hi
// non-decreasing over the rows, every row but the first one nonempty (lo <=
// hi; only the anchor row, a row's first token, is empty), and with an
// anchor no interval reaching column 0.  Every
// valid layout is: documents are contiguous segments, a query's interval
// starts at its document's first token and ends at itself (causal) or at its
// document's last token.  Then the rows that see a key at or after c0 are a
// suffix (hi rises) and those that see one at or before c1 a prefix (lo
// rises), so some row sees a key of the tile exactly when the first row of
// the suffix starts at or before c1; all rows see all of them exactly when
// the last row starts at or before the tile's first document key and the
// first row ends at or after its last key.
__device__ __forceinline__ uint8_t tile_kind_monotone(const int* slo, const int* shi, int r,
                                                      int nrows, int BM, int c0, int BN, int S,
                                                      int anchor) {
  if (nrows <= 0) return 0;
  const int c1 = min(S, c0 + BN) - 1;
  const bool cols_exist = (c0 + BN) <= S;
  const bool anchor_col = anchor && c0 == 0;
  // the first row may be the empty anchor row: it sees only column 0
  const int rf = r + (slo[r] > shi[r] ? 1 : 0);
  const int re = r + nrows;            // rows rf .. re-1 are nonempty
  // first row in [rf, re) with hi >= c0 (re if none)
  int a = rf, z = re;
  while (a < z) {
    const int m = (a + z) >> 1;
    if (shi[m] >= c0) z = m; else a = m + 1;
  }
  const bool any_doc = a < re && slo[a] <= c1 && c0 <= c1;
  const bool any_live = any_doc || anchor_col;
  if (!any_live) return 0;
  // every row sees every column: BM rows, BN columns, the first row not the
  // anchor row, lo of the last row at most the first document key of the tile
  // (c0 + 1 when column 0 is the anchor's), hi of the first row at least c1
  const bool all_full = nrows == BM && cols_exist && rf == r &&
                        slo[r + nrows - 1] <= c0 + (anchor_col ? 1 : 0) && shi[r] >= c1;
  return all_full ? kTileFull : ((anchor_col && !any_doc) ? kTileAnchor : kTilePartial);
}

// One workgroup per (row b, block of RB rows starting at origin + rb*RB):
// with cu given, the token tables of its rows (the first block of a row also
// those of the rows before origin) and its share of the layout checks;
// otherwise it reads them.  Then the kinds of every tile whose query tile
// lies in its rows, for up to two plans of the same origin: a query-major one
// (dense kinds row and live count of each of its query tiles) and a
// key-major one (dense key-major kinds, live counts of the key tiles added
// atomically to cntk, which must start at zero).  RB is a multiple of each
// plan's BM and at most 256.
struct KindsOut {
  int BM, BN, nq, nk;
  uint8_t* kinds;      // [B][nq][nk] (query-major) or [B][nk][nq] (key-major)
  int32_t* cnt;        // [B*nq] (query-major) or [B*nk] (key-major)
  int key_major;
};

__global__ __launch_bounds__(256) void k_plan_kinds(
    const int32_t* __restrict__ cu, int n_seg, int B, int S, int causal, int mode, int anchor,
    int32_t* __restrict__ pos, int32_t* __restrict__ lo, int32_t* __restrict__ hi,
    int32_t* __restrict__ status, int RB, int nrb, int origin, KindsOut p0, KindsOut p1) {
  __shared__ int slo[256], shi[256];
  __shared__ int wcount[4];
  const int b = blockIdx.x / nrb, rb = blockIdx.x % nrb;
  const int r0 = origin + rb * RB;
  const int nrows = max(0, min(RB, S - r0));
  const size_t tok0 = (size_t)b * S + r0;
  if (cu) {
    check_offsets((long long)blockIdx.x * blockDim.x + threadIdx.x, cu, n_seg, (long long)B * S,
                  status);
    // r < 0: the rows before the grid's origin, done by the row's first block
    for (int r = (rb == 0 ? -origin : 0) + (int)threadIdx.x; r < nrows; r += blockDim.x) {
      int p, l, h;
      bool bad;
      token_tables((long long)tok0 + r, cu, n_seg, S, causal, mode, anchor, p, l, h, bad);
      if (bad) status[0] = kStatusBadDocs;
      pos[tok0 + r] = p;
      lo[tok0 + r] = l;
      hi[tok0 + r] = h;
      if (r >= 0) {
        slo[r] = l;
        shi[r] = h;
      }
    }
  } else {
    for (int r = threadIdx.x; r < nrows; r += blockDim.x) {
      slo[r] = lo[tok0 + r];
      shi[r] = hi[tok0 + r];
    }
  }
  __syncthreads();
  // do this block's intervals allow the O(log BM) kinds?  (they do for every
  // valid layout; the per-row scan is kept for anything else)
  __shared__ int not_monotone;
  if (threadIdx.x == 0) not_monotone = 0;
  __syncthreads();
  for (int r = threadIdx.x; r < nrows; r += blockDim.x) {
    if (r + 1 < nrows && (slo[r] > slo[r + 1] || shi[r] > shi[r + 1] || slo[r + 1] > shi[r + 1]))
      not_monotone = 1;
    if (anchor && slo[r] < 1) not_monotone = 1;   // column 0 is the anchor's, never a document key
  }
  __syncthreads();
  const bool monotone = not_monotone == 0;
  for (int pl = 0; pl < 2; ++pl) {
    const KindsOut& P = pl ? p1 : p0;
    if (!P.kinds) continue;
    for (int sub = 0; sub < RB / P.BM; ++sub) {
      const int qt = rb * (RB / P.BM) + sub;
      if (qt >= P.nq) break;                      // uniform
      const int rr = sub * P.BM;
      const int n = max(0, min(P.BM, nrows - rr));
      int cnt = 0;
      for (int kt = threadIdx.x; kt < P.nk; kt += blockDim.x) {
        const uint8_t kind =
            monotone ? tile_kind_monotone(slo, shi, rr, n, P.BM, origin + kt * P.BN, P.BN, S, anchor)
                     : tile_kind(slo, shi, rr, n, P.BM, origin + kt * P.BN, P.BN, S, anchor);
        if (P.key_major) {
          P.kinds[((size_t)b * P.nk + kt) * P.nq + qt] = kind;
          if (kind) atomicAdd(P.cnt + (size_t)b * P.nk + kt, 1);
        } else {
          P.kinds[((size_t)b * P.nq + qt) * P.nk + kt] = kind;
          cnt += kind != 0;
        }
      }
      if (!P.key_major) {
        for (int off = 32; off > 0; off >>= 1) cnt += __shfl_xor(cnt, off);
        if ((threadIdx.x & 63) == 0) wcount[threadIdx.x >> 6] = cnt;
        __syncthreads();
        if (threadIdx.x == 0) P.cnt[(size_t)b * P.nq + qt] = wcount[0] + wcount[1] + wcount[2] + wcount[3];
        __syncthreads();
      }
    }
  }
}

// Clears the status word (when given) and n int32 counters.
__global__ void k_clear(int32_t* __restrict__ status, int32_t* __restrict__ p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i == 0 && status) status[0] = kStatusOk;
  if (i < n) p[i] = 0;
}

// Exclusive scan by one workgroup of NT threads: ptr[i] = sum(cnt[0..i)),
// ptr[n] = total (also to *total_out when not null).  buf: NT ints of LDS.
template <int NT>
__device__ void block_scan(const int32_t* __restrict__ cnt, int n, int32_t* __restrict__ ptr,
                           int32_t* __restrict__ total_out, int* buf) {
  int carry = 0;
  for (int base = 0; base < n; base += NT) {
    const int i = base + threadIdx.x;
    const int x = i < n ? cnt[i] : 0;
    buf[threadIdx.x] = x;
    __syncthreads();
    for (int off = 1; off < NT; off <<= 1) {
      const int y = (int)threadIdx.x >= off ? buf[threadIdx.x - off] : 0;
      __syncthreads();
      buf[threadIdx.x] += y;
      __syncthreads();
    }
    if (i < n) ptr[i] = carry + buf[threadIdx.x] - x;
    carry += buf[NT - 1];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    ptr[n] = carry;
    if (total_out) total_out[0] = carry;
  }
}

// Single-workgroup exclusive scan.
__global__ __launch_bounds__(1024) void k_scan(const int32_t* __restrict__ cnt, int n,
                                               int32_t* __restrict__ ptr,
                                               int32_t* __restrict__ total_out) {
  __shared__ int buf[1024];
  block_scan<1024>(cnt, n, ptr, total_out, buf);
}

// One wave per row: the live entries of the row, ascending, at ptr[row].
// The rows of two dense kind matrices (a plan's query-major and key-major
// ones) can go in one launch: waves past the first matrix's rows take the
// second's (rows2 = 0 for one matrix).
struct CompactRows {
  const uint8_t* m;       // [rows][n]
  int rows, n;
  const int32_t* ptr;
  int32_t* idx;
  uint8_t* kind;
  int32_t* pack;          // may be null
};
__global__ void k_row_compact(CompactRows a, CompactRows c) {
  int row = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= a.rows) {   // wave-uniform
    row -= a.rows;
    a = c;
    if (row >= a.rows) return;
  }
  const uint8_t* __restrict__ m = a.m;
  const int n = a.n;
  const int32_t* __restrict__ ptr = a.ptr;
  int32_t* __restrict__ idx = a.idx;
  uint8_t* __restrict__ kind = a.kind;
  int32_t* __restrict__ pack = a.pack;
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
// With ptr not null, the workgroup after the last one needed for the order
// also writes the plan's exclusive scan of the counts (ptr, *total_out), so a
// query-major plan needs no separate scan launch; with cnt2 not null, the
// workgroup after that one writes the exclusive scan of a second count array
// (the key-major plan's, ptr2, *total2).
constexpr int kMaxLptTiles = 16384;
__global__ __launch_bounds__(256) void k_tile_order(const int32_t* __restrict__ cnt, int n,
                                                   int32_t* __restrict__ order,
                                                   int32_t* __restrict__ ptr,
                                                   int32_t* __restrict__ total_out,
                                                   const int32_t* __restrict__ cnt2, int n2,
                                                   int32_t* __restrict__ ptr2,
                                                   int32_t* __restrict__ total2) {
  __shared__ int w[kMaxLptTiles];
  __shared__ int wmax[4], wsum[4];
  const int n_order = (n + 255) / 256;   // workgroups of the order
  if (ptr && (int)blockIdx.x == n_order) {
    block_scan<256>(cnt, n, ptr, total_out, w);
    return;
  }
  if (cnt2 && (int)blockIdx.x == n_order + (ptr ? 1 : 0)) {
    block_scan<256>(cnt2, n2, ptr2, total2, w);
    return;
  }
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
                     order, (int32_t*)nullptr, (int32_t*)nullptr, (const int32_t*)nullptr, 0,
                     (int32_t*)nullptr, (int32_t*)nullptr);
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

hipError_t launch_clear(int32_t* status, int32_t* p, int n, hipStream_t st) {
  const int blocks = n > 0 ? (n + 255) / 256 : 1;
  hipLaunchKernelGGL(k_clear, dim3(blocks), dim3(256), 0, st, status, p, n);
  return hipGetLastError();
}

hipError_t launch_plans(const PlanSrc& src, int B, int S, int anchor, const PlanBufs* pq,
                        const PlanBufs* pk, hipStream_t st) {
  KindsOut o[2] = {};
  int RB = 0;
  const int origin = pq ? pq->origin : pk->origin;
  if (pq) {
    o[0] = KindsOut{pq->BM, pq->BN, pq->nq, pq->nk, pq->kinds, pq->cntq, 0};
    RB = pq->BM;
  }
  if (pk) {
    o[1] = KindsOut{pk->BM, pk->BN, pk->nq, pk->nk, pk->kinds_t, pk->cntk, 1};
    RB = RB > pk->BM ? RB : pk->BM;
  }
  if (RB == 0 || RB > 256 || (pq && RB % pq->BM) || (pk && RB % pk->BM) ||
      (pq && pk && pq->origin != pk->origin))
    return hipErrorInvalidValue;
  const int nrb = (S + RB - 1) / RB;
  // the launch must cover the n_seg offsets it checks (RB <= 256 threads per
  // RB rows, and n_seg <= B*S)
  hipLaunchKernelGGL(k_plan_kinds, dim3(B * nrb), dim3(256), 0, st, src.cu, src.n_seg, B, S,
                     src.causal, src.mode, anchor, src.tt.pos, src.tt.lo, src.tt.hi, src.status, RB,
                     nrb, origin, o[0], o[1]);
  const int nq_rows = pq ? B * pq->nq : 0;   // query-major plan: B*nq rows of nk kinds
  const int nk_rows = pk ? B * pk->nk : 0;   // key-major plan: B*nk rows of nq kinds
  int32_t* const k_total = pq ? (int32_t*)nullptr : (pk ? pk->n_live : nullptr);
  if (pq && pq->order) {
    // the query-major work order, then both plans' scans, in one launch (the
    // scans take the workgroups after the order's)
    const unsigned grid = (unsigned)((nq_rows + 255) / 256) + 1 + (pk ? 1 : 0);
    hipLaunchKernelGGL(k_tile_order, dim3(grid), dim3(256), 0, st, pq->cntq, nq_rows, pq->order,
                       pq->qptr, pq->n_live, pk ? pk->cntk : (const int32_t*)nullptr, nk_rows,
                       pk ? pk->kptr : (int32_t*)nullptr, k_total);
  } else {
    if (pq) hipLaunchKernelGGL(k_scan, dim3(1), dim3(1024), 0, st, pq->cntq, nq_rows, pq->qptr, pq->n_live);
    if (pk) hipLaunchKernelGGL(k_scan, dim3(1), dim3(1024), 0, st, pk->cntk, nk_rows, pk->kptr, k_total);
  }
  // both plans' CSR in one launch, one wave per row
  CompactRows cq{}, ck{};
  if (pq) cq = CompactRows{pq->kinds, nq_rows, pq->nk, pq->qptr, pq->kidx, pq->kkind, pq->kpack};
  if (pk) ck = CompactRows{pk->kinds_t, nk_rows, pk->nq, pk->kptr, pk->qidx, pk->qkind, pk->qpack};
  const int rows = nq_rows + nk_rows;
  hipLaunchKernelGGL(k_row_compact, dim3((rows + 3) / 4), dim3(256), 0, st, cq, ck);
  return hipGetLastError();
}

}  // namespace aa
