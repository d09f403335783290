// C ABI of the AnchorAttention library: argument validation, workspace
// carving and the stream-ordered launch sequence of each entry point.
// The public contract is documented in include/anchor_attn.h.
#include <math.h>
#include <string.h>

#include <mutex>

#include "anchor_attn.h"
#include "aa_internal.h"

namespace aa {
namespace {

constexpr size_t kAlign = 256;

size_t up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct PlanLayout {
  int BM, BN, nq, nk;
  size_t cap;
  size_t kinds, kinds_t, cntq, cntk, qptr, kidx, kkind, kpack, kptr, qidx, qkind, qpack, n_live, order;
  size_t end;
};

PlanLayout plan_layout(int B, int S, int BM, int BN, size_t base) {
  PlanLayout p;
  p.BM = BM;
  p.BN = BN;
  p.nq = (S + BM - 1) / BM;
  p.nk = (S + BN - 1) / BN;
  p.cap = (size_t)B * p.nq * p.nk;
  size_t o = up(base);
  p.kinds = o;  o = up(o + p.cap);
  p.kinds_t = o; o = up(o + p.cap);
  p.cntq = o;   o = up(o + (size_t)B * p.nq * 4);
  p.cntk = o;   o = up(o + (size_t)B * p.nk * 4);
  p.qptr = o;   o = up(o + ((size_t)B * p.nq + 1) * 4);
  p.kidx = o;   o = up(o + p.cap * 4);
  p.kkind = o;  o = up(o + p.cap);
  p.kpack = o;  o = up(o + p.cap * 4);
  p.kptr = o;   o = up(o + ((size_t)B * p.nk + 1) * 4);
  p.qidx = o;   o = up(o + p.cap * 4);
  p.qkind = o;  o = up(o + p.cap);
  p.qpack = o;  o = up(o + p.cap * 4);
  p.n_live = o; o = up(o + 4);
  p.order = o;  o = up(o + ((size_t)B * p.nq + 1) * 4);
  p.end = o;
  return p;
}

// Where the attention kernels' tile grid starts in a row: after the anchor
// with AA_FLAG_GRID_AFTER_ANCHOR, else at the row's first token.
int grid_origin(int flags) { return (flags & AA_FLAG_GRID_AFTER_ANCHOR) ? 1 : 0; }

// origin: where the tile grid starts in a row (1 after a shared anchor).
PlanBufs plan_bufs(const PlanLayout& l, char* ws, int origin) {
  PlanBufs b;
  b.BM = l.BM; b.BN = l.BN; b.nq = l.nq; b.nk = l.nk; b.cap = l.cap;
  b.origin = origin;
  b.kinds = (uint8_t*)(ws + l.kinds);
  b.kinds_t = (uint8_t*)(ws + l.kinds_t);
  b.cntq = (int32_t*)(ws + l.cntq);
  b.cntk = (int32_t*)(ws + l.cntk);
  b.qptr = (int32_t*)(ws + l.qptr);
  b.kidx = (int32_t*)(ws + l.kidx);
  b.kkind = (uint8_t*)(ws + l.kkind);
  b.kpack = (int32_t*)(ws + l.kpack);
  b.kptr = (int32_t*)(ws + l.kptr);
  b.qidx = (int32_t*)(ws + l.qidx);
  b.qkind = (uint8_t*)(ws + l.qkind);
  b.qpack = (int32_t*)(ws + l.qpack);
  b.n_live = (int32_t*)(ws + l.n_live);
  b.order = (int32_t*)(ws + l.order);
  return b;
}

// Workspace of the attention entry points.
struct Layout {
  size_t status, pos, lo, hi, table, qrot, krot;
  PlanLayout pq;        // query-major plan of the forward and dq kernels
  PlanLayout pk;        // key-major plan of the dkdv kernel (backward only)
  size_t dvec, ds0, pdk, pdv, qstats;
  int nblk;
  size_t total;
};

Layout layout(int B, int S, int Hq, int Hkv, int D, bool bwd) {
  Layout L;
  const size_t T = (size_t)B * S;
  size_t o = 0;
  L.status = o; o = up(o + 4);
  L.pos = o;    o = up(o + T * 4);
  L.lo = o;     o = up(o + T * 4);
  L.hi = o;     o = up(o + T * 4);
  L.table = o;  o = up(o + (size_t)(S + 1) * D * 4);   // positions 0 .. S
  L.qrot = o;   o = up(o + T * Hq * D * 2);
  L.krot = o;   o = up(o + T * Hkv * D * 2);
  L.pq = plan_layout(B, S, kFwdBM, kFwdBN, o);
  o = L.pq.end;
  L.nblk = (S + kPreRows - 1) / kPreRows;
  if (bwd) {
    L.pk = plan_layout(B, S, kDkvBM, kDkvBN, o);
    o = L.pk.end;
    L.dvec = o; o = up(o + (size_t)B * Hq * S * 4);
    L.ds0 = o;  o = up(o + (size_t)B * Hq * S * 4);
    L.pdk = o;  o = up(o + (size_t)B * Hq * L.nblk * D * 4);
    L.pdv = o;  o = up(o + (size_t)B * Hq * L.nblk * D * 4);
    L.qstats = o; o = up(o + (size_t)B * Hq * L.nblk * 4 * kPreRows * 4);
  } else {
    L.pk = L.pq;
    L.dvec = L.ds0 = L.pdk = L.pdv = L.qstats = 0;
  }
  L.total = o;
  return L;
}

// Extra workspace of the interleaved-chunk entry points, after the Layout.
struct ChunkLayout {
  size_t new_start, doc_start, doc_end, row_ok, src, vperm, doperm;
  size_t total;
};

ChunkLayout chunk_layout(size_t base, int B, int S, int Hq, int Hkv, int D, int n_chunks,
                         bool bwd) {
  ChunkLayout C;
  const size_t T = (size_t)B * S;
  size_t o = up(base);
  C.new_start = o; o = up(o + (size_t)n_chunks * 4);
  C.doc_start = o; o = up(o + (size_t)n_chunks * 4);
  C.doc_end = o;   o = up(o + (size_t)n_chunks * 4);
  C.row_ok = o;    o = up(o + (size_t)B * 4);
  C.src = o;       o = up(o + T * 4);
  C.vperm = o;     o = up(o + T * Hkv * D * 2);   // V and dO stream through LDS tiles in
  C.doperm = 0;                                    // permuted order; everything else is
  if (bwd) {                                       // read or written at tok_map[p]
    C.doperm = o;  o = up(o + T * Hq * D * 2);
  }
  C.total = o;
  return C;
}

ChunkBufs chunk_bufs(const ChunkLayout& C, char* ws) {
  ChunkBufs cb;
  cb.new_start = (int32_t*)(ws + C.new_start);
  cb.doc_start = (int32_t*)(ws + C.doc_start);
  cb.doc_end = (int32_t*)(ws + C.doc_end);
  cb.row_ok = (int32_t*)(ws + C.row_ok);
  cb.src = (int32_t*)(ws + C.src);
  return cb;
}

bool shape_ok(int B, int S, int Hq, int Hkv, int D) {
  if (B < 1 || S < 1 || Hq < 1 || Hkv < 1 || Hq > 65535) return false;
  if (Hq % Hkv != 0) return false;
  if ((long long)B * S > 0x7fffffffLL) return false;
  (void)D;
  return true;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

__global__ void k_zero_status(int32_t* status) {
  if (threadIdx.x == 0) status[0] = kStatusOk;
}

RopeTheta make_theta(int D, double base) {
  RopeTheta th;
  for (int p = 0; p < kMaxHalfD; ++p) th.t[p] = p < D / 2 ? pow(base, -2.0 * p / D) : 0.0;
  return th;
}

#define AA_HIP(expr)                                  \
  do {                                                \
    if ((expr) != hipSuccess) return AA_EHIP;         \
  } while (0)

// Opt-in per-kernel timing: events recorded around every launch.  The state
// is per host thread, so calls made from other threads neither see nor
// disturb a profiling session; without one the library keeps no state.
struct Profiler {
  bool on = false;
  int cap = 0, used = 0;
  hipEvent_t* ev = nullptr;   // 2 * cap events
  int* id = nullptr;          // kernel id of each recorded launch
};
thread_local Profiler g_prof;

// Brackets one launcher call with profiling events when profiling is on.
#define AA_LAUNCH(kid, stream, expr)                                              \
  do {                                                                            \
    const bool _rec = g_prof.on && g_prof.used < g_prof.cap;                      \
    if (_rec) AA_HIP(hipEventRecord(g_prof.ev[2 * g_prof.used], (stream)));       \
    AA_HIP(expr);                                                                 \
    if (_rec) {                                                                   \
      AA_HIP(hipEventRecord(g_prof.ev[2 * g_prof.used + 1], (stream)));           \
      g_prof.id[g_prof.used++] = (kid);                                           \
    }                                                                             \
  } while (0)

// Positions, plan(s), RoPE table, rotated q and k: the prologue shared by
// the forward and the backward.
aa_status prologue(const Layout& L, char* ws, const void* q, const void* k,
                   const int32_t* cu, int n_seg, double rope_base, int causal, int flags, int B,
                   int S, int Hq, int Hkv, int D, bool bwd, hipStream_t st, bool rotate_q = true) {
  int32_t* status = (int32_t*)(ws + L.status);
  TokenTables tt{(int32_t*)(ws + L.pos), (int32_t*)(ws + L.lo), (int32_t*)(ws + L.hi)};
  const int mode = (flags & AA_FLAG_CONTINUOUS_POS) ? 1 : 0;
  const int anchor = (flags & AA_FLAG_NO_ANCHOR) ? 0 : 1;
  float* table = (float*)(ws + L.table);
  const int origin = grid_origin(flags);
  PlanBufs pq = plan_bufs(L.pq, ws, origin), pk = plan_bufs(L.pk, ws, origin);
  // Position IDs reach S when a document without an anchor fills a row under
  // reset IDs (its tokens count 1 .. S), so the table has S + 1 rows.  The
  // table kernel runs first: it also clears the status word and the
  // key-major plan's counters.
  AA_LAUNCH(AA_K_ROPE_TABLE, st,
            launch_rope_table(S + 1, D, make_theta(D, rope_base), table, status,
                              bwd ? pk.cntk : nullptr, B * pk.nk, st));
  // token tables and both plans (the key-major one when the workspace holds
  // the backward's layout) in one pass
  const PlanSrc src{cu, n_seg, causal, mode, tt, status};
  AA_LAUNCH(AA_K_PLAN, st, launch_plans(src, B, S, anchor, &pq, bwd ? &pk : nullptr, st));
  if (rotate_q)
    AA_LAUNCH(AA_K_ROPE, st,
              launch_rope_apply((const bf16*)q, nullptr, tt.pos, table, S + 1, B, S, Hq, D,
                                (bf16*)(ws + L.qrot), st));
  AA_LAUNCH(AA_K_ROPE, st,
            launch_rope_apply((const bf16*)k, nullptr, tt.pos, table, S + 1, B, S, Hkv, D,
                              (bf16*)(ws + L.krot), st));
  return AA_OK;
}

// The prologue of the interleaved-chunk entry points: the permuted layout of
// every row (token tables in permuted order), plan(s), RoPE table, q and k
// gathered and rotated in one pass, v gathered.
aa_status prologue_chunks(const Layout& L, const ChunkLayout& C, char* ws, const void* q,
                          const void* k, const void* v, const int32_t* cu,
                          const int32_t* chunk_doc, int n_chunks, double rope_base, int causal,
                          int flags, int B, int S, int Hq, int Hkv, int D, bool bwd,
                          hipStream_t st) {
  int32_t* status = (int32_t*)(ws + L.status);
  TokenTables tt{(int32_t*)(ws + L.pos), (int32_t*)(ws + L.lo), (int32_t*)(ws + L.hi)};
  const int mode = (flags & AA_FLAG_CONTINUOUS_POS) ? 1 : 0;
  const int anchor = (flags & AA_FLAG_NO_ANCHOR) ? 0 : 1;
  const ChunkBufs cb = chunk_bufs(C, ws);
  float* table = (float*)(ws + L.table);
  const int origin = grid_origin(flags);
  PlanBufs pq = plan_bufs(L.pq, ws, origin), pk = plan_bufs(L.pk, ws, origin);
  AA_LAUNCH(AA_K_ROPE_TABLE, st,
            launch_rope_table(S + 1, D, make_theta(D, rope_base), table, status,
                              bwd ? pk.cntk : nullptr, B * pk.nk, st));
  AA_LAUNCH(AA_K_CHUNKS, st,
            launch_chunk_layout(cu, chunk_doc, n_chunks, B, S, causal, mode, anchor, cb, tt,
                                status, st));
  // the plans from the permuted token tables the layout kernel wrote
  const PlanSrc src{nullptr, 0, causal, mode, tt, status};
  AA_LAUNCH(AA_K_PLAN, st, launch_plans(src, B, S, anchor, &pq, bwd ? &pk : nullptr, st));
  AA_LAUNCH(AA_K_ROPE, st,
            launch_rope_apply((const bf16*)q, cb.src, tt.pos, table, S + 1, B, S, Hq, D,
                              (bf16*)(ws + L.qrot), st));
  AA_LAUNCH(AA_K_ROPE, st,
            launch_rope_apply((const bf16*)k, cb.src, tt.pos, table, S + 1, B, S, Hkv, D,
                              (bf16*)(ws + L.krot), st));
  AA_LAUNCH(AA_K_GATHER, st,
            launch_gather_rows((const bf16*)v, cb.src, B, S, Hkv, D, (bf16*)(ws + C.vperm),
                             st));
  return AA_OK;
}

}  // namespace
}  // namespace aa

using namespace aa;

extern "C" {

const char* anchor_attn_strerror(aa_status s) {
  switch (s) {
    case AA_OK: return "ok";
    case AA_EINVAL: return "invalid argument (null pointer, size, alignment or head grouping)";
    case AA_EDOCS: return "cu_doc_lens violates the packed-segment layout";
    case AA_EUNSUPPORTED: return "unsupported head dimension or tile size";
    case AA_EWORKSPACE: return "workspace too small";
    case AA_EHIP: return "HIP runtime error or kernel launch failure";
  }
  return "unknown status";
}

const char* anchor_attn_version(void) { return "anchor_attn 0.1 gfx950"; }

size_t anchor_attn_workspace_size(int B, int S, int Hq, int Hkv, int D, int for_bwd) {
  if (!shape_ok(B, S, Hq, Hkv, D) || (D != 64 && D != 128)) return 0;
  return layout(B, S, Hq, Hkv, D, for_bwd != 0).total;
}

static bool flags_ok(int flags, int extra = 0) {
  return (flags & ~(AA_FLAG_CONTINUOUS_POS | AA_FLAG_NO_ANCHOR | extra)) == 0;
}

// Flags of the attention entry points: the grid after the anchor needs rows
// that have one.
static bool attn_flags_ok(int flags, int extra) {
  if ((flags & AA_FLAG_GRID_AFTER_ANCHOR) && (flags & AA_FLAG_NO_ANCHOR)) return false;
  return flags_ok(flags, extra | AA_FLAG_O_FP32 | AA_FLAG_GRID_AFTER_ANCHOR);
}

static aa_status fwd_impl(const void* q, const void* k, const void* v, const int32_t* cu_doc_lens,
                          int n_seg, double rope_base, int causal, int flags, int B, int S, int Hq,
                          int Hkv, int D, float softmax_scale, void* o, float* lse,
                          void* workspace, size_t ws_bytes, hipStream_t stream) {
  if (!q || !k || !v || !cu_doc_lens || !o || !lse || !workspace) return AA_EINVAL;
  if (!attn_flags_ok(flags, AA_FLAG_FWD_WORKSPACE)) return AA_EINVAL;
  if (!shape_ok(B, S, Hq, Hkv, D) || n_seg < B) return AA_EINVAL;
  if (D != 64 && D != 128) return AA_EUNSUPPORTED;
  if (!(rope_base > 0.0) || !isfinite(rope_base)) return AA_EINVAL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(lse, 4) || !aligned(cu_doc_lens, 4) || !aligned(workspace, kAlign))
    return AA_EINVAL;
  const Layout Lf = layout(B, S, Hq, Hkv, D, false);
  if (ws_bytes < Lf.total) return AA_EWORKSPACE;
  // A workspace that holds the backward's layout (of which the forward's is
  // a prefix) also gets the backward's key-major plan, built in the same pass
  // as the forward's plan, for a backward with AA_FLAG_FWD_WORKSPACE.
  const Layout Lb = layout(B, S, Hq, Hkv, D, true);
  const bool with_bwd_plan = ws_bytes >= Lb.total;
  const Layout& L = with_bwd_plan ? Lb : Lf;
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.f / sqrtf((float)D);
  char* ws = (char*)workspace;
  // the forward rotates Q as it loads it (and leaves the rotated q in the
  // workspace for the backward); the RoPE pass rotates K only
  aa_status s = prologue(L, ws, q, k, cu_doc_lens, n_seg, rope_base, causal, flags, B, S, Hq,
                         Hkv, D, with_bwd_plan, stream, /*rotate_q=*/false);
  if (s != AA_OK) return s;
  TokenTables tt{(int32_t*)(ws + L.pos), (int32_t*)(ws + L.lo), (int32_t*)(ws + L.hi)};
  const int anchor = (flags & AA_FLAG_NO_ANCHOR) ? 0 : 1;
  AA_LAUNCH(AA_K_FWD, stream,
            launch_fwd((const bf16*)q, (const float*)(ws + L.table), S + 1, (bf16*)(ws + L.qrot),
                       (const bf16*)(ws + L.krot), (const bf16*)v, tt, plan_bufs(L.pq, ws, grid_origin(flags)),
                       (const int32_t*)(ws + L.status), B, S, Hq, Hkv, D, scale, anchor, o,
                       (flags & AA_FLAG_O_FP32) ? 1 : 0, lse, nullptr, stream));
  return AA_OK;
}

static aa_status bwd_impl(const void* q, const void* k, const void* v, const void* o,
                          const float* lse, const void* dout, const int32_t* cu_doc_lens,
                          int n_seg, double rope_base, int causal, int flags, int B, int S, int Hq,
                          int Hkv, int D, float softmax_scale, void* dq, void* dk, void* dv,
                          void* workspace, size_t ws_bytes, hipStream_t stream) {
  if (!q || !k || !v || !o || !lse || !dout || !cu_doc_lens || !dq || !dk || !dv || !workspace)
    return AA_EINVAL;
  if (!attn_flags_ok(flags, AA_FLAG_FWD_WORKSPACE)) return AA_EINVAL;
  if (!shape_ok(B, S, Hq, Hkv, D) || n_seg < B) return AA_EINVAL;
  if (D != 64 && D != 128) return AA_EUNSUPPORTED;
  if (!(rope_base > 0.0) || !isfinite(rope_base)) return AA_EINVAL;
  const void* ptrs16[] = {q, k, v, o, dout, dq, dk, dv};
  for (const void* p : ptrs16)
    if (!aligned(p, 16)) return AA_EINVAL;
  if (!aligned(lse, 4) || !aligned(cu_doc_lens, 4) || !aligned(workspace, kAlign)) return AA_EINVAL;
  const Layout L = layout(B, S, Hq, Hkv, D, true);
  if (ws_bytes < L.total) return AA_EWORKSPACE;
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.f / sqrtf((float)D);
  char* ws = (char*)workspace;
  if (flags & AA_FLAG_FWD_WORKSPACE) {
    // the forward's status word, token tables, both plans, RoPE table and
    // rotated q, k are still in place (the forward built the key-major plan
    // too, the workspace holding the backward's layout): nothing to rebuild
  } else {
    aa_status s = prologue(L, ws, q, k, cu_doc_lens, n_seg, rope_base, causal, flags, B, S, Hq,
                           Hkv, D, true, stream);
    if (s != AA_OK) return s;
  }
  BwdArgs a;
  a.qr = (const bf16*)(ws + L.qrot);
  a.kr = (const bf16*)(ws + L.krot);
  a.v = (const bf16*)v;
  a.o = o;
  a.o_f32 = (flags & AA_FLAG_O_FP32) ? 1 : 0;
  a.dout = (const bf16*)dout;
  a.lse = lse;
  a.table = (const float*)(ws + L.table);
  a.tt = TokenTables{(int32_t*)(ws + L.pos), (int32_t*)(ws + L.lo), (int32_t*)(ws + L.hi)};
  a.status = (const int32_t*)(ws + L.status);
  a.dvec = (float*)(ws + L.dvec);
  a.ds0 = (float*)(ws + L.ds0);
  a.part_dk = (float*)(ws + L.pdk);
  a.part_dv = (float*)(ws + L.pdv);
  a.qstats = (float*)(ws + L.qstats);
  a.nblk = L.nblk;
  a.dq = (bf16*)dq;
  a.dk = (bf16*)dk;
  a.dv = (bf16*)dv;
  a.B = B; a.S = S; a.Hq = Hq; a.Hkv = Hkv; a.D = D;
  a.scale = scale;
  a.anchor = (flags & AA_FLAG_NO_ANCHOR) ? 0 : 1;
  a.origin = grid_origin(flags);
  AA_LAUNCH(AA_K_BWD_PRE, stream, launch_bwd_pre(a, stream));
  AA_LAUNCH(AA_K_BWD_DKDV, stream,
            launch_bwd_dkdv(a, plan_bufs(L.pk, ws, a.origin), plan_bufs(L.pq, ws, a.origin),
                            stream));
  AA_LAUNCH(AA_K_BWD_DQ, stream, launch_bwd_dq(a, plan_bufs(L.pq, ws, a.origin), stream));
  // without an anchor, key 0 is an ordinary key and dk/dv of it are complete
  if (a.anchor) AA_LAUNCH(AA_K_BWD_ANCHOR, stream, launch_bwd_anchor(a, stream));
  return AA_OK;
}

aa_status anchor_attn_fwd(const void* q, const void* k, const void* v, const int32_t* cu_doc_lens,
                          int n_seg, double rope_base, int causal, int B, int S, int Hq, int Hkv,
                          int D, float softmax_scale, void* o, float* lse, void* workspace,
                          size_t ws_bytes, hipStream_t stream) {
  return fwd_impl(q, k, v, cu_doc_lens, n_seg, rope_base, causal, 0, B, S, Hq, Hkv, D,
                  softmax_scale, o, lse, workspace, ws_bytes, stream);
}

aa_status anchor_attn_fwd_ex(const void* q, const void* k, const void* v,
                             const int32_t* cu_doc_lens, int n_seg, double rope_base, int causal,
                             int flags, int B, int S, int Hq, int Hkv, int D, float softmax_scale,
                             void* o, float* lse, void* workspace, size_t ws_bytes,
                             hipStream_t stream) {
  return fwd_impl(q, k, v, cu_doc_lens, n_seg, rope_base, causal, flags, B, S, Hq, Hkv, D,
                  softmax_scale, o, lse, workspace, ws_bytes, stream);
}

aa_status anchor_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                          const float* lse, const void* dout, const int32_t* cu_doc_lens,
                          int n_seg, double rope_base, int causal, int B, int S, int Hq, int Hkv,
                          int D, float softmax_scale, void* dq, void* dk, void* dv,
                          void* workspace, size_t ws_bytes, hipStream_t stream) {
  return bwd_impl(q, k, v, o, lse, dout, cu_doc_lens, n_seg, rope_base, causal, 0, B, S, Hq, Hkv,
                  D, softmax_scale, dq, dk, dv, workspace, ws_bytes, stream);
}

aa_status anchor_attn_bwd_ex(const void* q, const void* k, const void* v, const void* o,
                             const float* lse, const void* dout, const int32_t* cu_doc_lens,
                             int n_seg, double rope_base, int causal, int flags, int B, int S,
                             int Hq, int Hkv, int D, float softmax_scale, void* dq, void* dk,
                             void* dv, void* workspace, size_t ws_bytes, hipStream_t stream) {
  return bwd_impl(q, k, v, o, lse, dout, cu_doc_lens, n_seg, rope_base, causal, flags, B, S, Hq,
                  Hkv, D, softmax_scale, dq, dk, dv, workspace, ws_bytes, stream);
}

size_t anchor_attn_chunks_workspace_size(int B, int S, int Hq, int Hkv, int D, int n_chunks,
                                         int for_bwd) {
  if (!shape_ok(B, S, Hq, Hkv, D) || (D != 64 && D != 128) || n_chunks < B) return 0;
  const Layout L = layout(B, S, Hq, Hkv, D, for_bwd != 0);
  return chunk_layout(L.total, B, S, Hq, Hkv, D, n_chunks, for_bwd != 0).total;
}

static aa_status chunk_args_ok(const int32_t* cu, const int32_t* chunk_doc, int n_chunks, int flags,
                               int B, int S, int Hq, int Hkv, int D, double rope_base,
                               int extra_flags = 0) {
  if (!cu || !chunk_doc) return AA_EINVAL;
  if (!shape_ok(B, S, Hq, Hkv, D) || n_chunks < B) return AA_EINVAL;
  if (D != 64 && D != 128) return AA_EUNSUPPORTED;
  if (!(extra_flags ? attn_flags_ok(flags, 0) : flags_ok(flags))) return AA_EINVAL;
  if (!(rope_base > 0.0) || !isfinite(rope_base)) return AA_EINVAL;
  if (!aligned(cu, 4) || !aligned(chunk_doc, 4)) return AA_EINVAL;
  return AA_OK;
}

aa_status anchor_attn_fwd_chunks(const void* q, const void* k, const void* v,
                                 const int32_t* cu_chunks, const int32_t* chunk_doc, int n_chunks,
                                 double rope_base, int causal, int flags, int B, int S, int Hq,
                                 int Hkv, int D, float softmax_scale, void* o, float* lse,
                                 void* workspace, size_t ws_bytes, hipStream_t stream) {
  if (!q || !k || !v || !o || !lse || !workspace) return AA_EINVAL;
  const aa_status e = chunk_args_ok(cu_chunks, chunk_doc, n_chunks, flags, B, S, Hq, Hkv, D, rope_base,
                                    AA_FLAG_O_FP32);
  if (e != AA_OK) return e;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(lse, 4) || !aligned(workspace, kAlign))
    return AA_EINVAL;
  const Layout L = layout(B, S, Hq, Hkv, D, false);
  const ChunkLayout C = chunk_layout(L.total, B, S, Hq, Hkv, D, n_chunks, false);
  if (ws_bytes < C.total) return AA_EWORKSPACE;
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.f / sqrtf((float)D);
  char* ws = (char*)workspace;
  aa_status s = prologue_chunks(L, C, ws, q, k, v, cu_chunks, chunk_doc, n_chunks, rope_base,
                                causal, flags, B, S, Hq, Hkv, D, false, stream);
  if (s != AA_OK) return s;
  TokenTables tt{(int32_t*)(ws + L.pos), (int32_t*)(ws + L.lo), (int32_t*)(ws + L.hi)};
  const int anchor = (flags & AA_FLAG_NO_ANCHOR) ? 0 : 1;
  const int32_t* src = (const int32_t*)(ws + C.src);
  AA_LAUNCH(AA_K_FWD, stream,
            launch_fwd(nullptr, nullptr, 0, (bf16*)(ws + L.qrot), (const bf16*)(ws + L.krot),
                       (const bf16*)(ws + C.vperm), tt, plan_bufs(L.pq, ws, grid_origin(flags)),
                       (const int32_t*)(ws + L.status), B, S, Hq, Hkv, D, scale, anchor, o,
                       (flags & AA_FLAG_O_FP32) ? 1 : 0, lse, src, stream));
  return AA_OK;
}

aa_status anchor_attn_bwd_chunks(const void* q, const void* k, const void* v, const void* o,
                                 const float* lse, const void* dout, const int32_t* cu_chunks,
                                 const int32_t* chunk_doc, int n_chunks, double rope_base,
                                 int causal, int flags, int B, int S, int Hq, int Hkv, int D,
                                 float softmax_scale, void* dq, void* dk, void* dv,
                                 void* workspace, size_t ws_bytes, hipStream_t stream) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !workspace) return AA_EINVAL;
  const aa_status e = chunk_args_ok(cu_chunks, chunk_doc, n_chunks, flags, B, S, Hq, Hkv, D, rope_base,
                                    AA_FLAG_O_FP32);
  if (e != AA_OK) return e;
  const void* ptrs16[] = {q, k, v, o, dout, dq, dk, dv};
  for (const void* p : ptrs16)
    if (!aligned(p, 16)) return AA_EINVAL;
  if (!aligned(lse, 4) || !aligned(workspace, kAlign)) return AA_EINVAL;
  const Layout L = layout(B, S, Hq, Hkv, D, true);
  const ChunkLayout C = chunk_layout(L.total, B, S, Hq, Hkv, D, n_chunks, true);
  if (ws_bytes < C.total) return AA_EWORKSPACE;
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.f / sqrtf((float)D);
  char* ws = (char*)workspace;
  aa_status s = prologue_chunks(L, C, ws, q, k, v, cu_chunks, chunk_doc, n_chunks, rope_base,
                                causal, flags, B, S, Hq, Hkv, D, true, stream);
  if (s != AA_OK) return s;
  const int32_t* src = (const int32_t*)(ws + C.src);
  AA_LAUNCH(AA_K_GATHER, stream,
            launch_gather_rows((const bf16*)dout, src, B, S, Hq, D, (bf16*)(ws + C.doperm),
                             stream));
  BwdArgs a;
  a.qr = (const bf16*)(ws + L.qrot);
  a.kr = (const bf16*)(ws + L.krot);
  a.v = (const bf16*)(ws + C.vperm);
  a.o = o;
  a.o_f32 = (flags & AA_FLAG_O_FP32) ? 1 : 0;
  a.dout = (const bf16*)(ws + C.doperm);
  a.lse = lse;
  a.table = (const float*)(ws + L.table);
  a.tt = TokenTables{(int32_t*)(ws + L.pos), (int32_t*)(ws + L.lo), (int32_t*)(ws + L.hi)};
  a.status = (const int32_t*)(ws + L.status);
  a.dvec = (float*)(ws + L.dvec);
  a.ds0 = (float*)(ws + L.ds0);
  a.part_dk = (float*)(ws + L.pdk);
  a.part_dv = (float*)(ws + L.pdv);
  a.qstats = (float*)(ws + L.qstats);
  a.nblk = L.nblk;
  a.dq = (bf16*)dq;
  a.dk = (bf16*)dk;
  a.dv = (bf16*)dv;
  a.tok_map = src;
  a.B = B; a.S = S; a.Hq = Hq; a.Hkv = Hkv; a.D = D;
  a.scale = scale;
  a.anchor = (flags & AA_FLAG_NO_ANCHOR) ? 0 : 1;
  a.origin = grid_origin(flags);
  AA_LAUNCH(AA_K_BWD_PRE, stream, launch_bwd_pre(a, stream));
  AA_LAUNCH(AA_K_BWD_DKDV, stream,
            launch_bwd_dkdv(a, plan_bufs(L.pk, ws, a.origin), plan_bufs(L.pq, ws, a.origin),
                            stream));
  AA_LAUNCH(AA_K_BWD_DQ, stream, launch_bwd_dq(a, plan_bufs(L.pq, ws, a.origin), stream));
  if (a.anchor) AA_LAUNCH(AA_K_BWD_ANCHOR, stream, launch_bwd_anchor(a, stream));
  return AA_OK;
}

aa_status anchor_attn_chunk_layout(const int32_t* cu_chunks, const int32_t* chunk_doc, int n_chunks,
                                   int B, int S, int causal, int flags, int32_t* src, int32_t* pos,
                                   void* workspace, size_t ws_bytes, hipStream_t stream) {
  if (!src || !pos || !workspace) return AA_EINVAL;
  const aa_status e = chunk_args_ok(cu_chunks, chunk_doc, n_chunks, flags, B, S, 1, 1, 64, 1.0);
  if (e != AA_OK) return e;
  if (!aligned(src, 4) || !aligned(pos, 4) || !aligned(workspace, kAlign)) return AA_EINVAL;
  const size_t need = anchor_attn_chunks_workspace_size(B, S, 1, 1, 64, n_chunks, 0);
  if (ws_bytes < need) return AA_EWORKSPACE;
  char* ws = (char*)workspace;
  const Layout L = layout(B, S, 1, 1, 64, false);
  const ChunkLayout C = chunk_layout(L.total, B, S, 1, 1, 64, n_chunks, false);
  int32_t* status = (int32_t*)(ws + L.status);
  TokenTables tt{pos, (int32_t*)(ws + L.lo), (int32_t*)(ws + L.hi)};
  ChunkBufs cb = chunk_bufs(C, ws);
  cb.src = src;
  hipLaunchKernelGGL(k_zero_status, dim3(1), dim3(64), 0, stream, status);
  AA_HIP(hipGetLastError());
  AA_HIP(launch_chunk_layout(cu_chunks, chunk_doc, n_chunks, B, S, causal,
                             (flags & AA_FLAG_CONTINUOUS_POS) ? 1 : 0,
                             (flags & AA_FLAG_NO_ANCHOR) ? 0 : 1, cb, tt, status, stream));
  return AA_OK;
}

aa_status anchor_attn_position_ids(const int32_t* cu_doc_lens, int n_seg, int B, int S, int flags,
                                   int32_t* pos, void* workspace, size_t ws_bytes,
                                   hipStream_t stream) {
  if (!cu_doc_lens || !pos || !workspace) return AA_EINVAL;
  if (B < 1 || S < 1 || (long long)B * S > 0x7fffffffLL || n_seg < B) return AA_EINVAL;
  if (!flags_ok(flags)) return AA_EINVAL;
  const int mode = (flags & AA_FLAG_CONTINUOUS_POS) ? 1 : 0;
  const int anchor = (flags & AA_FLAG_NO_ANCHOR) ? 0 : 1;
  if (!aligned(workspace, kAlign) || !aligned(pos, 4) || !aligned(cu_doc_lens, 4)) return AA_EINVAL;
  const size_t T = (size_t)B * S;
  const size_t need = up(4) + 2 * up(T * 4);
  if (ws_bytes < need) return AA_EWORKSPACE;
  char* ws = (char*)workspace;
  int32_t* status = (int32_t*)ws;
  TokenTables tt{pos, (int32_t*)(ws + up(4)), (int32_t*)(ws + up(4) + up(T * 4))};
  hipLaunchKernelGGL(k_zero_status, dim3(1), dim3(64), 0, stream, status);
  AA_HIP(hipGetLastError());
  AA_HIP(launch_positions(cu_doc_lens, n_seg, B, S, 1, mode, anchor, tt, status, stream));
  return AA_OK;
}

static bool tile_ok(int t) { return t >= 16 && t <= 256 && (t & (t - 1)) == 0; }

size_t anchor_attn_plan_capacity(int B, int S, int BM, int BN) {
  if (B < 1 || S < 1 || !tile_ok(BM) || !tile_ok(BN)) return 0;
  return (size_t)B * ((S + BM - 1) / BM) * ((S + BN - 1) / BN);
}

size_t anchor_attn_plan_workspace_size(int B, int S, int BM, int BN) {
  if (B < 1 || S < 1 || !tile_ok(BM) || !tile_ok(BN) || (long long)B * S > 0x7fffffffLL) return 0;
  const size_t T = (size_t)B * S;
  const size_t base = up(4) + 3 * up(T * 4);
  return plan_layout(B, S, BM, BN, base).end;
}

aa_status anchor_attn_tile_plan(const int32_t* cu_doc_lens, int n_seg, int B, int S, int BM, int BN,
                                int causal, int flags, int32_t* qptr, int32_t* kidx, uint8_t* kkind,
                                int32_t* kptr, int32_t* qidx, uint8_t* qkind, int32_t* n_live,
                                void* workspace, size_t ws_bytes, hipStream_t stream) {
  if (!cu_doc_lens || !qptr || !kidx || !kkind || !kptr || !qidx || !qkind || !n_live || !workspace)
    return AA_EINVAL;
  if (B < 1 || S < 1 || (long long)B * S > 0x7fffffffLL || n_seg < B) return AA_EINVAL;
  if (!tile_ok(BM) || !tile_ok(BN)) return AA_EUNSUPPORTED;
  if (!flags_ok(flags, AA_FLAG_GRID_AFTER_ANCHOR)) return AA_EINVAL;
  if (!aligned(workspace, kAlign)) return AA_EINVAL;
  const size_t need = anchor_attn_plan_workspace_size(B, S, BM, BN);
  if (ws_bytes < need) return AA_EWORKSPACE;
  char* ws = (char*)workspace;
  const size_t T = (size_t)B * S;
  int32_t* status = (int32_t*)ws;
  TokenTables tt{(int32_t*)(ws + up(4)), (int32_t*)(ws + up(4) + up(T * 4)),
                 (int32_t*)(ws + up(4) + 2 * up(T * 4))};
  const PlanLayout pl = plan_layout(B, S, BM, BN, up(4) + 3 * up(T * 4));
  PlanBufs pb = plan_bufs(pl, ws, (flags & AA_FLAG_GRID_AFTER_ANCHOR) ? 1 : 0);
  // the caller's output arrays replace the workspace copies
  pb.qptr = qptr; pb.kidx = kidx; pb.kkind = kkind;
  pb.kptr = kptr; pb.qidx = qidx; pb.qkind = qkind; pb.n_live = n_live;
  pb.kpack = nullptr; pb.qpack = nullptr; pb.order = nullptr;
  const int anchor = (flags & AA_FLAG_NO_ANCHOR) ? 0 : 1;
  // the same one-pass build as the attention calls, both layouts of one plan
  AA_HIP(launch_clear(status, pb.cntk, B * pb.nk, stream));
  const PlanSrc src{cu_doc_lens, n_seg, causal, 0, tt, status};
  AA_HIP(launch_plans(src, B, S, anchor, &pb, &pb, stream));
  return AA_OK;
}

static_assert(kOrderLpt == AA_ORDER_LPT && kOrderInterleave == AA_ORDER_INTERLEAVE,
              "work-order flags of the header and the kernels");

aa_status anchor_attn_tile_order(const int32_t* cnt, int n, int32_t* order, hipStream_t stream) {
  if (!cnt || !order || n < 1 || n == 0x7fffffff) return AA_EINVAL;
  if (!aligned(cnt, 4) || !aligned(order, 4)) return AA_EINVAL;
  AA_HIP(launch_tile_order(cnt, n, order, stream));
  return AA_OK;
}

aa_status anchor_attn_rope(const void* x, const int32_t* pos, int B, int S, int H, int D,
                           double rope_base, void* x_rot, float* table, hipStream_t stream) {
  if (!x || !pos || !x_rot || !table) return AA_EINVAL;
  if (B < 1 || S < 1 || H < 1) return AA_EINVAL;
  if (D != 64 && D != 128) return AA_EUNSUPPORTED;
  if (!(rope_base > 0.0) || !isfinite(rope_base)) return AA_EINVAL;
  if (!aligned(x, 16) || !aligned(x_rot, 16) || !aligned(table, 16) || !aligned(pos, 4))
    return AA_EINVAL;
  AA_HIP(launch_rope_table(S, D, make_theta(D, rope_base), table, nullptr, nullptr, 0, stream));
  AA_HIP(launch_rope_apply((const bf16*)x, nullptr, pos, table, S, B, S, H, D, (bf16*)x_rot, stream));
  return AA_OK;
}

aa_status anchor_attn_profile_begin(int max_launches) {
  if (max_launches < 1 || max_launches > (1 << 20)) return AA_EINVAL;
  if (g_prof.ev) return AA_EINVAL;   // already profiling
  g_prof.ev = new hipEvent_t[2 * (size_t)max_launches];
  g_prof.id = new int[max_launches];
  for (int i = 0; i < 2 * max_launches; ++i) {
    if (hipEventCreate(&g_prof.ev[i]) != hipSuccess) {
      for (int j = 0; j < i; ++j) (void)hipEventDestroy(g_prof.ev[j]);
      delete[] g_prof.ev;
      delete[] g_prof.id;
      g_prof = Profiler();
      return AA_EHIP;
    }
  }
  g_prof.cap = max_launches;
  g_prof.used = 0;
  g_prof.on = true;
  return AA_OK;
}

aa_status anchor_attn_profile_end(double* ms, int32_t* count, int n) {
  if (!g_prof.ev) return AA_EINVAL;
  aa_status rc = AA_OK;
  for (int i = 0; i < n; ++i) {
    if (ms) ms[i] = 0.0;
    if (count) count[i] = 0;
  }
  for (int r = 0; r < g_prof.used; ++r) {
    float t = 0.f;
    if (hipEventSynchronize(g_prof.ev[2 * r + 1]) != hipSuccess ||
        hipEventElapsedTime(&t, g_prof.ev[2 * r], g_prof.ev[2 * r + 1]) != hipSuccess) {
      rc = AA_EHIP;
      continue;
    }
    const int k = g_prof.id[r];
    if (k < n) {
      if (ms) ms[k] += t;
      if (count) count[k] += 1;
    }
  }
  for (int i = 0; i < 2 * g_prof.cap; ++i) (void)hipEventDestroy(g_prof.ev[i]);
  delete[] g_prof.ev;
  delete[] g_prof.id;
  g_prof = Profiler();
  return rc;
}

// ---------------------------------------------------------------------------
// Allocation-free backward.  Its workspace is `scratch`, a fixed device array
// of the library's code object: every GPU the library runs on holds its own
// copy from the module's load until the process ends, and every call on that
// GPU shares it (the last call's contents stay; the backward clears the one
// word that must start at zero itself, the device status word).  In host code
// `scratch` names a host-side stand-in, never the device memory: its device
// address is looked up once per device, with that device current, and only
// that address is handed to the kernels.
static __device__ __align__(256) unsigned char scratch[AA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// Device address of this device's scratch array (looked up on the first call
// on the device).
aa_status scratch_of_current_device(hipStream_t stream, void** out) {
  int dev = -1;
  AA_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return AA_EUNSUPPORTED;
  if (stream) {
    hipDevice_t sdev = -1;
    AA_HIP(hipStreamGetDevice(stream, &sdev));
    if (sdev != dev) return AA_EINVAL;   // the stream must belong to the current device
  }
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = p;
  });
  if (g_scratch_err[dev] != hipSuccess || g_scratch_ptr[dev] == nullptr) return AA_EHIP;
  *out = g_scratch_ptr[dev];
  return AA_OK;
}
}  // namespace

aa_status anchor_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                                  const float* lse, const void* dout, const int32_t* cu_doc_lens,
                                  int n_seg, double rope_base, int causal, int flags, int B, int S,
                                  int Hq, int Hkv, int D, float softmax_scale, void* dq, void* dk,
                                  void* dv, hipStream_t stream) {
  if (flags & AA_FLAG_FWD_WORKSPACE) return AA_EINVAL;   // the scratch holds no forward state
  if (!shape_ok(B, S, Hq, Hkv, D) || (D != 64 && D != 128)) return AA_EINVAL;
  if (layout(B, S, Hq, Hkv, D, true).total > (size_t)AA_NOALLOC_SCRATCH_BYTES) return AA_EWORKSPACE;
  void* ws = nullptr;
  const aa_status s = scratch_of_current_device(stream, &ws);
  if (s != AA_OK) return s;
  return bwd_impl(q, k, v, o, lse, dout, cu_doc_lens, n_seg, rope_base, causal, flags, B, S, Hq,
                  Hkv, D, softmax_scale, dq, dk, dv, ws, (size_t)AA_NOALLOC_SCRATCH_BYTES, stream);
}

aa_status anchor_attn_device_status(const void* workspace, hipStream_t stream, int32_t* out) {
  if (!workspace || !out) return AA_EINVAL;
  int32_t v = 0;
  AA_HIP(hipMemcpyAsync(&v, workspace, 4, hipMemcpyDeviceToHost, stream));
  AA_HIP(hipStreamSynchronize(stream));
  *out = v;
  return AA_OK;
}

}  // extern "C"
