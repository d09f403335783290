/*
 * anchor_attn.h -- C ABI of the AnchorAttention library for AMD MI355X (gfx950).
 *
 * The operation is the attention pattern of "When Precision Meets Position:
 * BFloat16 Breaks Down RoPE in Long-Context Training" (arXiv 2411.13476), as
 * summarised on the paper-graph architecture page of that paper ("arch page"
 * below), section 3.4:
 *   - "Intra-document attention with position ID reset (Figure 2, middle)":
 *     position IDs restart at every document; the first token of a document
 *     has ID 1.
 *   - "Rotary Positional Embedding (RoPE)", Eq. 6: adjacent pairs (2p, 2p+1) of
 *     q and k are rotated by pos * theta_p, theta_p = base^(-2p/D).
 *   - "Implementation detail: where precision matters": the rotation is done
 *     in float32 outside the attention kernel and the rotated vectors are
 *     rounded to bfloat16 before the inner products.
 *   - "AnchorAttention: The Shared Anchor Design", "Mask construction": every
 *     query sees the shared anchor (the row's first token, position ID 0);
 *     inside a document attention is causal; documents never see each other;
 *     the anchor sees only itself.
 *   - "Standard attention": O = softmax(scale * Q K^T + M) V; the page leaves
 *     the 1/sqrt(D) scale out of its notation, the library applies it.
 *
 * Conventions shared by every entry point
 *   - Every pointer is a device pointer unless its comment says "host".
 *   - q, o, dout, dq: [B, S, Hq, D] bfloat16, contiguous.
 *     k, v, dk, dv:   [B, S, Hkv, D] bfloat16, contiguous.
 *     lse:            [B, Hq, S] float32 (natural log of the softmax sum,
 *                     logits already scaled).
 *   - D is 64 or 128; Hq is a multiple of Hkv; query head h reads kv head
 *     h / (Hq / Hkv) (contiguous grouped-query groups).
 *   - cu_doc_lens: int32 [n_seg + 1] segment offsets over the flattened B*S
 *     token stream: cu[0] = 0, cu[n_seg] = B*S, strictly increasing; every
 *     row b starts with the one-token anchor segment [b*S, b*S + 1); no
 *     segment crosses a row.  Example for one row of 256 tokens holding
 *     documents of 80, 100 and 75 tokens: {0, 1, 81, 181, 256}.
 *   - causal = 1 is the method.  causal = 0 drops only the "key not after
 *     query" rule inside a document (anchor rules unchanged).
 *   - softmax_scale <= 0 selects 1/sqrt(D).
 *   - All work is enqueued on `stream`; no call synchronises the device
 *     (except anchor_attn_device_status) and no call allocates memory.  The
 *     caller owns every buffer, including the workspace, which must be at
 *     least the size reported by the matching *_workspace_size call and
 *     256-byte aligned; tensors must be 16-byte aligned.
 *   - Argument errors are reported synchronously through the return value
 *     before anything is launched.  The content of the device-resident
 *     cu_doc_lens is validated on the device: a violation sets the status
 *     word in the workspace (read it with anchor_attn_device_status), every
 *     kernel then stays in bounds and the attention outputs are filled with
 *     NaN so that misuse is visible.
 *   - Calls sharing one workspace on different streams race.
 */
#ifndef ANCHOR_ATTN_H
#define ANCHOR_ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  AA_OK = 0,
  AA_EINVAL = 1,        /* null pointer, bad size, bad alignment, Hq % Hkv != 0 */
  AA_EDOCS = 2,         /* cu_doc_lens violates the layout above (device status word) */
  AA_EUNSUPPORTED = 3,  /* D or tile size not supported */
  AA_EWORKSPACE = 4,    /* workspace smaller than required */
  AA_EHIP = 5           /* a HIP runtime call or kernel launch failed */
} aa_status;

/* Tile kinds in a tile plan (uint8 values). */
enum {
  AA_TILE_FULL = 1,     /* every element of the tile exists and is allowed */
  AA_TILE_PARTIAL = 2,  /* live, some elements masked, not anchor-only */
  AA_TILE_ANCHOR = 3    /* key tile 0 whose only allowed key is the anchor column */
};

/* Options of the *_ex entry points, anchor_attn_position_ids and
 * anchor_attn_tile_plan (OR of these; 0 is the method as graded):
 *   AA_FLAG_CONTINUOUS_POS  position IDs are the row-local index t - b*S
 *       instead of restarting at every document: the arch page's "Core
 *       design (Figure 2, right)" description of AnchorAttention (anchor 0,
 *       document tokens counting on from 1 across documents) and, without an
 *       anchor, standard intra-document attention (Figure 2, left).
 *   AA_FLAG_NO_ANCHOR  no shared anchor: cu_doc_lens need not start a row
 *       with a one-token segment, the row's first token is an ordinary
 *       document token, and a query sees only the keys of its own document
 *       (arch page §3.4, "Intra-document attention", Figure 2 left and
 *       middle; with reset IDs every document's first token gets ID 1).
 *       These are the pages' baselines, computed by the same kernels.
 * Unknown bits are rejected with AA_EINVAL. */
#define AA_FLAG_CONTINUOUS_POS 1
#define AA_FLAG_NO_ANCHOR 2
/*   AA_FLAG_FWD_WORKSPACE  (anchor_attn_bwd_ex) the workspace still holds what
 *       anchor_attn_fwd_ex left in it for the same q, k, cu_doc_lens,
 *       rope_base, causal, other flags and shape: it was sized for the
 *       backward (anchor_attn_workspace_size(..., for_bwd = 1)) and given to
 *       the forward, and nothing wrote to it in between.  (A forward given a
 *       workspace of that size also builds the backward's key-major tile plan,
 *       in the same pass as its own.)  The backward then reuses the forward's
 *       position IDs, both tile plans, RoPE table and rotated q, k instead of
 *       rebuilding them (the forward's workspace layout is a prefix of the
 *       backward's).  anchor_attn_fwd_ex ignores it; the other entry points
 *       reject it.  If the promise does not hold the results are wrong;
 *       nothing detects it. */
#define AA_FLAG_FWD_WORKSPACE 4
/*   AA_FLAG_O_FP32  (anchor_attn_fwd_ex, anchor_attn_bwd_ex,
 *       anchor_attn_fwd_chunks, anchor_attn_bwd_chunks) O is float32
 *       [B,S,Hq,D] instead of bf16: the forward writes the normalised output
 *       without the bf16 rounding, and the backward reads O in that dtype
 *       (16-byte aligned in both cases).  The other entry points reject it. */
#define AA_FLAG_O_FP32 8
/*   AA_FLAG_GRID_AFTER_ANCHOR  (the *_ex, chunk and no-alloc attention entry
 *       points, and anchor_attn_tile_plan) place the tile grid after each
 *       row's anchor: query tile qt holds rows 1 + qt*BM .. and key tile kt
 *       keys 1 + kt*BN .. (row-local, cut at S; nq and nk stay ceil(S/BM),
 *       ceil(S/BN)), so no tile holds the anchor's row or column and there is
 *       no AA_TILE_ANCHOR kind; the anchor row's outputs and gradient are
 *       formed outside the tiles.  Results are the same either way (up to
 *       float32 summation order); the choice is about speed: documents whose
 *       lengths are multiples of the tiles then start on tile edges and touch
 *       fewer tiles (many short documents), while long documents gain
 *       nothing.  The attention entry points reject it with
 *       AA_FLAG_NO_ANCHOR; a forward and a backward that share a workspace
 *       (AA_FLAG_FWD_WORKSPACE) must agree on it. */
#define AA_FLAG_GRID_AFTER_ANCHOR 16

/* Human-readable text for a status code (static storage). */
const char* anchor_attn_strerror(aa_status s);

/* Library version string, e.g. "anchor_attn 0.1 gfx950" (static storage). */
const char* anchor_attn_version(void);

/* Workspace bytes needed by anchor_attn_fwd / anchor_attn_bwd for this shape.
 * for_bwd = 0 sizes the forward, 1 the backward.  Returns 0 on bad shape. */
size_t anchor_attn_workspace_size(int B, int S, int Hq, int Hkv, int D, int for_bwd);

/* Forward pass (arch page §3.4: reset position IDs, Eq. 6 RoPE in float32
 * rounded to bf16, Mask construction, flash-style softmax attention).
 * Writes o [B,S,Hq,D] bf16 and lse [B,Hq,S] float32. */
aa_status anchor_attn_fwd(const void* q, const void* k, const void* v,
                          const int32_t* cu_doc_lens, int n_seg, double rope_base, int causal,
                          int B, int S, int Hq, int Hkv, int D, float softmax_scale,
                          void* o, float* lse, void* workspace, size_t ws_bytes,
                          hipStream_t stream);

/* Backward pass of the same operation: given q, k, v, the forward's o and lse,
 * and dout = dL/dO, writes dq [B,S,Hq,D], dk and dv [B,S,Hkv,D] (bf16).  Key
 * gradients sum over the query heads of a group.  Self-contained: it rebuilds
 * the position IDs, tile plan and rotated q/k itself. */
aa_status anchor_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                          const float* lse, const void* dout,
                          const int32_t* cu_doc_lens, int n_seg, double rope_base, int causal,
                          int B, int S, int Hq, int Hkv, int D, float softmax_scale,
                          void* dq, void* dk, void* dv, void* workspace, size_t ws_bytes,
                          hipStream_t stream);

/* anchor_attn_fwd / anchor_attn_bwd with options (AA_FLAG_*, see above):
 * the same arguments, layouts, workspace sizes, ownership and errors, plus
 * `flags` after `causal`.  flags = 0 is exactly anchor_attn_fwd / _bwd. */
aa_status anchor_attn_fwd_ex(const void* q, const void* k, const void* v,
                             const int32_t* cu_doc_lens, int n_seg, double rope_base, int causal,
                             int flags, int B, int S, int Hq, int Hkv, int D, float softmax_scale,
                             void* o, float* lse, void* workspace, size_t ws_bytes,
                             hipStream_t stream);
aa_status anchor_attn_bwd_ex(const void* q, const void* k, const void* v, const void* o,
                             const float* lse, const void* dout,
                             const int32_t* cu_doc_lens, int n_seg, double rope_base, int causal,
                             int flags, int B, int S, int Hq, int Hkv, int D, float softmax_scale,
                             void* dq, void* dk, void* dv, void* workspace, size_t ws_bytes,
                             hipStream_t stream);

/* ---- allocation-free backward --------------------------------------------
 * For callers that cannot allocate device memory at all (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation):
 * anchor_attn_bwd_ex with the same arguments, layouts and results, minus the
 * workspace.  Its workspace is a fixed array of AA_NOALLOC_SCRATCH_BYTES in
 * the library's code object, one per device, held from the library's load
 * until the process ends; the call allocates nothing.
 *   - Shapes whose backward workspace (anchor_attn_workspace_size(..., 1))
 *     exceeds AA_NOALLOC_SCRATCH_BYTES are rejected with AA_EWORKSPACE before
 *     anything is launched (160 MiB holds the backward of 8192 tokens x 32
 *     heads x 128 features).
 *   - AA_FLAG_FWD_WORKSPACE is rejected (AA_EINVAL): the scratch never holds
 *     a forward's state.
 *   - `stream` must belong to the current device (AA_EINVAL otherwise); the
 *     first call on a device looks up its array's address.
 *   - Every call on one device shares that device's array: calls that overlap
 *     on one GPU (other streams, other threads) race and give wrong results.
 *   - The device status word lives in the scratch, out of the caller's
 *     reach: an invalid device cu_doc_lens shows as NaN gradients. */
#define AA_NOALLOC_SCRATCH_BYTES (160u << 20)
aa_status anchor_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                                  const float* lse, const void* dout,
                                  const int32_t* cu_doc_lens, int n_seg, double rope_base,
                                  int causal, int flags, int B, int S, int Hq, int Hkv, int D,
                                  float softmax_scale, void* dq, void* dk, void* dv,
                                  hipStream_t stream);

/* ---- interleaved document chunks -----------------------------------------
 * Arch page §5, "AnchorAttention with Interleaved Chunks" (Figure 5 middle
 * and right): documents are cut into chunks shuffled across a row, every
 * document keeping its own token order.  A query sees its row's anchor (unless
 * AA_FLAG_NO_ANCHOR) and the keys of its own document, in any chunk, that are
 * not after it (or all of them, causal = 0).  Reset position IDs count the
 * document's tokens before the query across its chunks (+1); continuous IDs
 * are the row-local index t - b*S.
 *   cu_chunks  int32 [n_chunks + 1] (device): chunk boundaries over the
 *              flattened B*S stream, cu_chunks[0] = 0, strictly increasing,
 *              cu_chunks[n_chunks] = B*S; no chunk crosses a row.
 *   chunk_doc  int32 [n_chunks] (device): document id of every chunk; chunks
 *              of one row with the same id form one document.  With an anchor
 *              the first chunk of every row is the one-token anchor with id -1
 *              (and no other chunk has -1); otherwise every id is >= 0.
 * At most 4096 chunks per row.  A row that breaks these rules is reported
 * through the device status word (AA_EDOCS) and its outputs are NaN.
 * Layouts, scale, flags and errors as for anchor_attn_fwd_ex / _bwd_ex; the
 * workspace size comes from anchor_attn_chunks_workspace_size (for_bwd 0/1).
 * The library runs the block-sparse kernels on every row permuted so that
 * each document is contiguous (the order inside a document is kept, so the
 * mask is unchanged); the kernels write O, LSE, dq, dk, dv straight to the
 * caller's token order. */
size_t anchor_attn_chunks_workspace_size(int B, int S, int Hq, int Hkv, int D, int n_chunks,
                                         int for_bwd);
aa_status anchor_attn_fwd_chunks(const void* q, const void* k, const void* v,
                                 const int32_t* cu_chunks, const int32_t* chunk_doc, int n_chunks,
                                 double rope_base, int causal, int flags, int B, int S, int Hq,
                                 int Hkv, int D, float softmax_scale, void* o, float* lse,
                                 void* workspace, size_t ws_bytes, hipStream_t stream);
aa_status anchor_attn_bwd_chunks(const void* q, const void* k, const void* v, const void* o,
                                 const float* lse, const void* dout, const int32_t* cu_chunks,
                                 const int32_t* chunk_doc, int n_chunks, double rope_base,
                                 int causal, int flags, int B, int S, int Hq, int Hkv, int D,
                                 float softmax_scale, void* dq, void* dk, void* dv,
                                 void* workspace, size_t ws_bytes, hipStream_t stream);
/* Stage entry point of the chunk layout, for bit-exact tests: src int32 [B*S]
 * receives, for every token p of the permuted rows, the original token it
 * came from; pos int32 [B*S] the position ID of permuted token p.  workspace:
 * anchor_attn_chunks_workspace_size(B, S, 1, 1, 64, n_chunks, 0) bytes. */
aa_status anchor_attn_chunk_layout(const int32_t* cu_chunks, const int32_t* chunk_doc, int n_chunks,
                                   int B, int S, int causal, int flags, int32_t* src, int32_t* pos,
                                   void* workspace, size_t ws_bytes, hipStream_t stream);

/* Position IDs (arch page §3.4, Figure 2 middle: reset per document; the
 * anchor has ID 0, a document's first token ID 1).  pos: int32 [B*S].
 * flags: AA_FLAG_CONTINUOUS_POS gives the row-local index instead (document
 * tokens count on across documents, Figure 2 right as the arch page
 * describes it); AA_FLAG_NO_ANCHOR drops the anchor segment.  workspace
 * needs anchor_attn_plan_workspace_size(B, S, 64, 64) bytes (for the status
 * word). */
aa_status anchor_attn_position_ids(const int32_t* cu_doc_lens, int n_seg, int B, int S, int flags,
                                   int32_t* pos, void* workspace, size_t ws_bytes,
                                   hipStream_t stream);

/* Workspace bytes needed by anchor_attn_tile_plan. */
size_t anchor_attn_plan_workspace_size(int B, int S, int BM, int BN);

/* Upper bound on the number of live tiles of a plan: B * ceil(S/BM) * ceil(S/BN). */
size_t anchor_attn_plan_capacity(int B, int S, int BM, int BN);

/* Block-sparse tile plan (arch page §3.4, "Reduction in attention
 * computations": only in-document pairs plus the anchor column are computed).
 * A (query tile, key tile) pair of BM x BN elements is live when the mask
 * allows at least one of its elements; key tile 0 is live for every query
 * tile because every query sees the anchor.  Kinds as AA_TILE_*.
 *   query-major: qptr int32 [B*nq + 1]; entries qptr[b*nq+qt] .. qptr[b*nq+qt+1]
 *                of kidx int32 / kkind uint8 list the live key tiles ascending.
 *   key-major:   kptr int32 [B*nk + 1]; qidx int32 / qkind uint8 likewise.
 * nq = ceil(S/BM), nk = ceil(S/BN); kidx/kkind/qidx/qkind must hold
 * anchor_attn_plan_capacity() entries; n_live (device int32) receives the
 * number of live tiles.  BM and BN are powers of two in [16, 256].  flags:
 * AA_FLAG_NO_ANCHOR plans rows without an anchor (no anchor column, no
 * AA_TILE_ANCHOR kinds); AA_FLAG_GRID_AFTER_ANCHOR places the grid after the
 * anchor (the attention kernels' grid for rows with an anchor);
 * AA_FLAG_CONTINUOUS_POS does not change a plan. */
aa_status anchor_attn_tile_plan(const int32_t* cu_doc_lens, int n_seg, int B, int S, int BM, int BN,
                                int causal, int flags,
                                int32_t* qptr, int32_t* kidx, uint8_t* kkind,
                                int32_t* kptr, int32_t* qidx, uint8_t* qkind,
                                int32_t* n_live, void* workspace, size_t ws_bytes,
                                hipStream_t stream);

/* Work order of the query tiles of a query-major plan: the order the
 * attention kernels take them in (scheduling only; no result depends on
 * it).  cnt: int32 [n], live key tiles per query tile (qptr differences);
 * order: int32 [n + 1] receives the tiles in launch order, then the flags:
 *   AA_ORDER_LPT        the largest count exceeds 1.5x the mean: tiles by
 *                       descending count, ties by index (longest
 *                       processing time first); otherwise order[i] = i;
 *   AA_ORDER_INTERLEAVE n <= 128, or the natural order: the tiles of the
 *                       heads of an XCD's slice are taken rank by rank.
 * Plans of more than 16384 tiles keep the natural order with flags 0. */
#define AA_ORDER_LPT 1
#define AA_ORDER_INTERLEAVE 2
aa_status anchor_attn_tile_order(const int32_t* cnt, int n, int32_t* order, hipStream_t stream);

/* RoPE stage alone (Eq. 6; angle pos*theta_p formed and reduced in float64,
 * cos/sin rounded to float32, pair rotated in float32, result rounded to
 * bf16 to nearest even).  x, x_rot: [B,S,H,D] bf16; pos: int32 [B*S] with
 * 0 <= pos < S.  table: float32 scratch of S * D floats. */
aa_status anchor_attn_rope(const void* x, const int32_t* pos, int B, int S, int H, int D,
                           double rope_base, void* x_rot, float* table, hipStream_t stream);

/* Reads the device status word of a workspace used by the calls above (this
 * call synchronises `stream`).  *out (host) receives AA_OK or AA_EDOCS. */
aa_status anchor_attn_device_status(const void* workspace, hipStream_t stream, int32_t* out);

/* ---- optional per-kernel timing (diagnostics) -----------------------------
 * Between anchor_attn_profile_begin() and anchor_attn_profile_end(), every
 * kernel that the calls above enqueue from the same host thread is bracketed
 * by HIP events recorded on the call's stream.  The session belongs to the
 * calling thread (thread-local state): calls from other threads are not
 * timed and are unaffected.  begin() creates the events (it allocates; call it outside
 * any graph capture); end() waits for them and writes, for each kernel id
 * below, the summed milliseconds (ms[id], host) and launch count (count[id],
 * host) for ids < n, then releases the events.  At most `max_launches`
 * launches are recorded; later ones run untimed. */
enum {
  AA_K_STATUS = 0, AA_K_POSITIONS = 1, AA_K_PLAN = 2, AA_K_ROPE_TABLE = 3, AA_K_ROPE = 4,
  AA_K_FWD = 5, AA_K_BWD_PRE = 6, AA_K_BWD_DKDV = 7, AA_K_BWD_DQ = 8, AA_K_BWD_ANCHOR = 9,
  AA_K_CHUNKS = 10, AA_K_GATHER = 11,
  AA_K_COUNT = 12
};
aa_status anchor_attn_profile_begin(int max_launches);
aa_status anchor_attn_profile_end(double* ms, int32_t* count, int n);

#ifdef __cplusplus
}
#endif

#endif /* ANCHOR_ATTN_H */
