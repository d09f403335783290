"""Plain, slow CPU oracle for AnchorAttention (float64, NumPy).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this module:
only the tests, the smoke check and the benchmark's CPU-baseline leg call it.
It shares no code with the HIP library and imports nothing from it.

Sources (cited by page title and section; "arch page" below is the
paper-graph "architecture" summary of arXiv 2411.13476, "When Precision Meets
Position: BFloat16 Breaks Down RoPE in Long-Context Training"):

* arch page §3.4, "Rotary Positional Embedding (RoPE): The Theoretical
  Promise" and Eq. 6 (Appendix A): R_{i,theta} is block diagonal; block p
  rotates the adjacent pair (2p, 2p+1) by the angle i*theta_p with
  theta_p = base^(-2p/d), p = 0 .. d/2-1.
* arch page §3.4, "Standard attention": A = softmax(Q K^T + M) with the
  causal mask; the 1/sqrt(d) factor is left out of the page's notation
  only for brevity, so it is applied here (reading (c) of the design notes).
* arch page §3.4, "Implementation detail: where precision matters": the
  rotation is applied to q and k before the attention kernel.  The oracle
  keeps every step in float64 (no bfloat16 rounding of the rotated vectors).
* arch page §3.4, "Intra-document attention with position ID reset
  (Figure 2, middle)": position IDs restart at every document, the first
  token of every document gets ID 1.
* arch page §3.4, "AnchorAttention: The Shared Anchor Design", "Mask
  construction": M_{i,0} = 0 for every i; same document and j <= i -> 0;
  different documents -> -inf; j > i -> -inf.  The anchor (<bos>, position
  ID 0) attends only to itself; its key is rotated by R_0 = I.
* arch page §3.4, "Reduction in attention computations": each token attends
  only within its own document plus the anchor.
* arch page §3.4, "Intra-document attention (Figure 2, left)" and Figure 2,
  middle: the baselines without an anchor, where a query sees only the causal
  keys of its own document; position IDs continue across documents (left) or
  restart at 1 for every document (middle).  ``anchor=False`` computes them.
* The paper's own reading of AnchorAttention (arch page, "Core design
  (Figure 2, right)"): continuous document position IDs counting on from 1
  after the anchor; ``mode="continuous"``.
* arch page §5 "AnchorAttention with Interleaved Chunks" and Figure 5
  (middle, right): documents cut into chunks that are shuffled across the row,
  each document keeping its own token order.  ``seg_doc`` gives the document
  of every segment (chunk); chunks of one row with the same id form one
  document, and a query sees the keys of its document (in every chunk) that
  are not after it.

Readings where the pages are silent (listed with reasons in the design notes):
position IDs are reset per document (first document token = 1, anchor = 0);
scale = 1/sqrt(D); every batch row carries its own anchor at its first token;
grouped-query heads use contiguous groups (kv head = h * Hkv // Hq);
causal=False drops only the "j <= i" rule.

Layouts: q [B,S,Hq,D], k and v [B,S,Hkv,D]; cu_doc_lens int32 [n_seg+1] over
the flattened B*S token stream, every row starting with its one-token anchor
segment.
"""
from __future__ import annotations

import math

import numpy as np

# Tile kinds of the block-sparse plan (values of the plan's kind bytes).
KIND_NONE = 0
KIND_FULL = 1      # every element of the tile exists and is allowed
KIND_PARTIAL = 2   # some but not all elements allowed, not anchor-only
KIND_ANCHOR = 3    # key tile 0 where the only allowed key is the anchor column


# ----------------------------------------------------------------------------
# Segments and position IDs
# ----------------------------------------------------------------------------
def validate_cu(cu, B: int, S: int, anchor: bool = True) -> np.ndarray:
    """Check the packed-segment offsets; raise ValueError on misuse.  Every
    row starts a segment (segments never cross rows); with an anchor that
    first segment is the one-token anchor."""
    cu = np.asarray(cu, dtype=np.int64)
    if cu.ndim != 1 or len(cu) < 2:
        raise ValueError("cu_doc_lens must be a 1-D array with at least two entries")
    if cu[0] != 0 or cu[-1] != B * S:
        raise ValueError("cu_doc_lens must start at 0 and end at B*S")
    if np.any(np.diff(cu) <= 0):
        raise ValueError("cu_doc_lens must be strictly increasing (no empty segments)")
    cs = set(int(x) for x in cu)
    for b in range(B):
        if b * S not in cs:
            raise ValueError(f"a segment crosses into row {b}")
        if anchor and b * S + 1 not in cs:
            raise ValueError(f"row {b} must start with a one-token anchor segment")
    return cu


def segment_ids(cu, B: int, S: int, anchor: bool = True) -> np.ndarray:
    """Index of the segment holding every token of the flattened stream."""
    cu = validate_cu(cu, B, S, anchor)
    t = np.arange(B * S, dtype=np.int64)
    return np.searchsorted(cu, t, side="right") - 1


def document_ids(cu, B: int, S: int, anchor: bool = True, seg_doc=None) -> np.ndarray:
    """A label per token, equal for two tokens exactly when they belong to the
    same document.  Without ``seg_doc`` every segment is a document.  With it,
    segment s belongs to document seg_doc[s] of its row (interleaved chunks);
    the anchor segment carries id -1 and no other segment may."""
    seg = segment_ids(cu, B, S, anchor)
    if seg_doc is None:
        return seg
    seg_doc = np.asarray(seg_doc, dtype=np.int64)
    cu = np.asarray(cu, dtype=np.int64)
    if len(seg_doc) != len(cu) - 1:
        raise ValueError("seg_doc needs one document id per segment")
    starts = cu[:-1]
    is_anchor_seg = (starts % S == 0) & (np.diff(cu) == 1) if anchor else np.zeros(len(starts), bool)
    if anchor and np.any(seg_doc[is_anchor_seg] != -1):
        raise ValueError("the anchor segment of every row must have document id -1")
    if np.any(seg_doc[~is_anchor_seg] < 0):
        raise ValueError("document ids must be >= 0 (-1 marks the anchor)")
    row = np.asarray(starts // S, dtype=np.int64)
    span = int(seg_doc.max()) + 2
    label_of_seg = row * span + seg_doc + 1
    return label_of_seg[seg]


def position_ids(cu, B: int, S: int, mode: str = "reset", anchor: bool = True,
                 seg_doc=None) -> np.ndarray:
    """Position ID of every token (arch page §3.4, Figure 2).

    reset:      anchor -> 0; document token t in segment [s, e) -> t - s + 1.
    continuous: anchor -> 0; document tokens count on from 1 across documents,
                i.e. t - (row start).
    Without an anchor the row's first token is an ordinary document token:
    reset gives it 1, continuous gives it 0 (t - row start).  With interleaved
    chunks (``seg_doc``) reset counts the tokens of the same document before t,
    across its chunks: t's rank in its document + 1.
    """
    cu = validate_cu(cu, B, S, anchor)
    seg = segment_ids(cu, B, S, anchor)
    t = np.arange(B * S, dtype=np.int64)
    row_start = (t // S) * S
    is_anchor = t == row_start
    if mode == "reset" and seg_doc is not None:
        doc = document_ids(cu, B, S, anchor, seg_doc)
        order = np.argsort(doc, kind="stable")            # tokens grouped by document, in order
        first = np.searchsorted(doc[order], doc[order], side="left")
        rank = np.empty_like(t)
        rank[order] = np.arange(len(t)) - first
        pos = rank + 1
    elif mode == "reset":
        pos = t - cu[seg] + 1
    elif mode == "continuous":
        pos = t - row_start
    else:
        raise ValueError(f"unknown position mode {mode!r}")
    if anchor:
        pos = np.where(is_anchor, 0, pos)
    return pos.astype(np.int64)


# ----------------------------------------------------------------------------
# RoPE (Eq. 6)
# ----------------------------------------------------------------------------
def rope_theta(D: int, base: float) -> np.ndarray:
    """theta_p = base^(-2p/D), p = 0 .. D/2-1, in float64."""
    p = np.arange(D // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * p / D)


def rope(x: np.ndarray, pos: np.ndarray, base: float, inverse: bool = False) -> np.ndarray:
    """Apply R_{pos,theta} (or its transpose) to the last axis of x.

    x: [..., T, D] float64 with the token axis second to last, or [T, H, D]
    when ``pos`` has length T and x.shape[-3] == T.  Pairs (2p, 2p+1) are
    rotated by pos*theta_p, as in the block-diagonal matrix of Eq. 6.
    """
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    theta = rope_theta(D, base)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * theta[None, :]   # [T, D/2]
    c, s = np.cos(ang), np.sin(ang)
    if inverse:
        s = -s
    # broadcast over a head axis between tokens and D when present
    if x.ndim >= 3 and x.shape[-3] == len(pos) and x.shape[-2] != len(pos):
        c = c[:, None, :]
        s = s[:, None, :]
    x0 = x[..., 0::2]
    x1 = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


# ----------------------------------------------------------------------------
# The explicit mask
# ----------------------------------------------------------------------------
def allowed(cu, B: int, S: int, rows, cols, causal: bool = True,
            anchor: bool = True, seg_doc=None) -> np.ndarray:
    """Dense boolean mask block allowed[len(rows), len(cols)] (Mask construction).

    rows and cols are flattened token indices.  A query may see a key only in
    its own batch row; there it sees the row's anchor (unless anchor=False),
    and keys of its own document that are not in its future.
    """
    seg = document_ids(cu, B, S, anchor, seg_doc)
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    anchor_of_row = (rows // S) * S
    same_batch_row = (rows[:, None] // S) == (cols[None, :] // S)
    sees_anchor = cols[None, :] == anchor_of_row[:, None]
    same_doc = seg[rows][:, None] == seg[cols][None, :]
    if causal:
        same_doc &= cols[None, :] <= rows[:, None]
    if not anchor:
        return same_batch_row & same_doc
    return same_batch_row & (sees_anchor | same_doc)


def unmasked_pairs(cu, B: int, S: int, causal: bool = True, block: int = 1024,
                   anchor: bool = True, seg_doc=None) -> int:
    """Number of allowed (query, key) pairs, counted on the explicit mask."""
    total = 0
    for b in range(B):
        cols = np.arange(b * S, (b + 1) * S)
        for r0 in range(0, S, block):
            rows = np.arange(b * S + r0, b * S + min(S, r0 + block))
            total += int(allowed(cu, B, S, rows, cols, causal, anchor, seg_doc).sum())
    return total


# ----------------------------------------------------------------------------
# Forward and backward
# ----------------------------------------------------------------------------
def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):          # a torch tensor (any dtype) -> exact float64
        import torch
        return x.detach().to(torch.float64).cpu().numpy()
    return np.asarray(x, dtype=np.float64)


def _blocks_of(rows: np.ndarray, S: int, block: int):
    """Group sorted flattened row indices by batch row and chunk them."""
    rows = np.unique(np.asarray(rows, dtype=np.int64))
    for b in np.unique(rows // S):
        rb = rows[rows // S == b]
        for i in range(0, len(rb), block):
            yield int(b), rb[i:i + block]


def _row_block_forward(qh, kr, vv, cu, B, S, rows_b, b, pos, base, scale, causal, anchor=True,
                       seg_doc=None):
    """Logits, probabilities, output and log-sum-exp for a block of query rows."""
    qr = rope(qh[rows_b - b * S], pos[rows_b], base)               # [R, D]
    # Under the causal rule every key after the block's last query is masked
    # (exp(-inf) contributes exactly 0), so those columns are not formed.
    ncols = int(rows_b.max() - b * S + 1) if causal else S
    cols = np.arange(b * S, b * S + ncols)
    s = scale * (qr @ kr[:ncols].T)                                 # [R, ncols]
    m_allowed = allowed(cu, B, S, rows_b, cols, causal, anchor, seg_doc)
    s = np.where(m_allowed, s, -np.inf)
    m = s.max(axis=1)
    p = np.exp(s - m[:, None])
    l = p.sum(axis=1)
    p = p / l[:, None]
    o = p @ vv[:ncols]
    lse = m + np.log(l)
    return qr, cols, m_allowed, p, o, lse


def forward(q, k, v, cu, rope_base: float, causal: bool = True, scale: float | None = None,
            heads=None, rows=None, block: int = 512, pos_mode: str = "reset", pos=None,
            anchor: bool = True, seg_doc=None):
    """O and LSE (float64) for the chosen q heads and flattened query rows.

    ``pos`` optionally overrides the position IDs (one per flattened token);
    ``anchor=False`` computes the intra-document baselines without an anchor;
    ``seg_doc`` (a document id per segment) describes interleaved chunks.
    Returns (o [len(rows), len(heads), D], lse [len(heads), len(rows)], rows, heads).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    scale = 1.0 / math.sqrt(D) if scale is None or scale <= 0 else float(scale)
    pos = (position_ids(cu, B, S, pos_mode, anchor, seg_doc) if pos is None
           else np.asarray(pos, dtype=np.int64))
    heads = list(range(Hq)) if heads is None else list(heads)
    rows = np.arange(B * S) if rows is None else np.unique(np.asarray(rows, dtype=np.int64))
    where = {int(r): n for n, r in enumerate(rows)}
    o = np.zeros((len(rows), len(heads), D))
    lse = np.zeros((len(heads), len(rows)))
    for hi, h in enumerate(heads):
        g = h * Hkv // Hq
        kr_of = {}
        for b, rb in _blocks_of(rows, S, block):
            if b not in kr_of:      # rotated keys of this row, once per (head, row)
                kr_of = {b: rope(k[b, :, g, :], pos[b * S:(b + 1) * S], rope_base)}
            kr = kr_of[b]
            vv = v[b, :, g, :]
            _, _, _, _, ob, lb = _row_block_forward(q[b, :, h, :], kr, vv, cu, B, S, rb, b, pos,
                                                     rope_base, scale, causal, anchor, seg_doc)
            idx = [where[int(r)] for r in rb]
            o[idx, hi, :] = ob
            lse[hi, idx] = lb
    return o, lse, rows, heads


def backward(q, k, v, do, cu, rope_base: float, causal: bool = True, scale: float | None = None,
             heads=None, q_rows=None, k_cols=None, block: int = 512, pos_mode: str = "reset",
             pos=None, anchor: bool = True, seg_doc=None):
    """Analytic gradients (float64) of sum(O * dO) with respect to q, k, v.

    dV_j = sum_i P_ij dO_i;  dP_ij = dO_i . v_j;  Dv_i = dO_i . O_i;
    dS_ij = P_ij (dP_ij - Dv_i);  dq'_i = scale sum_j dS_ij k'_j;
    dk'_j = scale sum_i dS_ij q'_i;  dq = R(pos)^T dq';  dk = R(pos)^T dk'.
    Key gradients sum over every q head of the chosen set that maps to the
    key's kv head.  dq is returned for ``q_rows`` (default: all) and dk, dv for
    ``k_cols`` (default: all), as [len(rows), len(heads), D] and
    [len(cols), Hkv, D] arrays, with the row/col index arrays.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    scale = 1.0 / math.sqrt(D) if scale is None or scale <= 0 else float(scale)
    pos = (position_ids(cu, B, S, pos_mode, anchor, seg_doc) if pos is None
           else np.asarray(pos, dtype=np.int64))
    heads = list(range(Hq)) if heads is None else list(heads)
    q_rows = np.arange(B * S) if q_rows is None else np.unique(np.asarray(q_rows, dtype=np.int64))
    k_cols = np.arange(B * S) if k_cols is None else np.unique(np.asarray(k_cols, dtype=np.int64))
    qwhere = {int(r): n for n, r in enumerate(q_rows)}
    kwhere = {int(c): n for n, c in enumerate(k_cols)}
    dq = np.zeros((len(q_rows), len(heads), D))
    dk_rot = np.zeros((len(k_cols), Hkv, D))
    dv = np.zeros((len(k_cols), Hkv, D))

    # rows whose contribution is needed: the requested dq rows, and every row
    # that is allowed to see one of the requested keys
    need = set(int(r) for r in q_rows)
    for b in np.unique(k_cols // S):
        kc = k_cols[k_cols // S == b]
        for r0 in range(0, S, 2048):
            rr = np.arange(b * S + r0, b * S + min(S, r0 + 2048))
            hit = allowed(cu, B, S, rr, kc, causal, anchor, seg_doc).any(axis=1)
            need.update(int(x) for x in rr[hit])
    need_rows = np.array(sorted(need), dtype=np.int64)

    for hi, h in enumerate(heads):
        g = h * Hkv // Hq
        kr_of = {}
        for b, rb in _blocks_of(need_rows, S, block):
            if b not in kr_of:
                kr_of = {b: rope(k[b, :, g, :], pos[b * S:(b + 1) * S], rope_base)}
            kr = kr_of[b]
            vv = v[b, :, g, :]
            qr, cols, m_allowed, p, o, _ = _row_block_forward(q[b, :, h, :], kr, vv, cu, B, S, rb, b,
                                                               pos, rope_base, scale, causal, anchor,
                                                               seg_doc)
            dob = do[b, rb - b * S, h, :]                                # [R, D]
            dv_i = np.sum(dob * o, axis=1)                              # Dv
            dp = dob @ vv[:len(cols)].T
            ds = p * (dp - dv_i[:, None])                               # zero where masked
            # dq rows that were asked for
            sel = [n for n, r in enumerate(rb) if int(r) in qwhere]
            if sel:
                dqr = scale * (ds[sel] @ kr[:len(cols)])
                dqb = rope(dqr, pos[rb[sel]], rope_base, inverse=True)
                dq[[qwhere[int(rb[n])] for n in sel], hi, :] = dqb
            # dk, dv columns that were asked for
            csel = [n for n, c in enumerate(cols) if int(c) in kwhere]
            if csel:
                dk_rot[[kwhere[int(cols[n])] for n in csel], g, :] += scale * (ds[:, csel].T @ qr)
                dv[[kwhere[int(cols[n])] for n in csel], g, :] += p[:, csel].T @ dob
    dk = np.empty_like(dk_rot)
    for gi in range(Hkv):
        dk[:, gi, :] = rope(dk_rot[:, gi, :], pos[k_cols], rope_base, inverse=True)
    return dq, dk, dv, q_rows, k_cols


# ----------------------------------------------------------------------------
# Block-sparse tile plan, by brute force over the explicit mask
# ----------------------------------------------------------------------------
def _classify(m: np.ndarray, e: np.ndarray, anchor_col: bool) -> int:
    """Kind of one tile from its allowed / exists element masks [BM, BN];
    anchor_col: the tile's first column is the row's anchor key."""
    if not m.any():
        return KIND_NONE
    if e.all() and m.all():
        return KIND_FULL
    if anchor_col and not m[:, 1:].any():
        return KIND_ANCHOR
    return KIND_PARTIAL


def _grid(S: int, B_: int, origin: int) -> int:
    """Tiles of size B_ along a row of S tokens: ceil(S / B_), whatever the
    origin (with origin 1 the last tile may be short or empty)."""
    return -(-S // B_)


def tile_kinds_row(cu, B: int, S: int, BM: int, BN: int, b: int, qt: int,
                   causal: bool = True, anchor: bool = True, origin: int = 0) -> np.ndarray:
    """Kinds of every key tile for query tile qt of row b, from the dense mask.
    Query tile qt holds rows origin + qt*BM .. origin + (qt+1)*BM - 1 and key
    tile kt keys origin + kt*BN .. (row-local, cut at S); with origin 1 the
    row's anchor (query and key 0) lies outside every tile."""
    nk = _grid(S, BN, origin)
    r0 = origin + qt * BM
    rows = np.arange(b * S + r0, b * S + min(S, r0 + BM))
    cols = np.arange(b * S, (b + 1) * S)
    width = origin + nk * BN
    m = np.zeros((BM, width), dtype=bool)
    e = np.zeros((BM, width), dtype=bool)
    if len(rows):
        m[:len(rows), :S] = allowed(cu, B, S, rows, cols, causal, anchor)
        e[:len(rows), :S] = True
    out = []
    for kt in range(nk):
        c0 = origin + kt * BN
        out.append(_classify(m[:, c0:c0 + BN], e[:, c0:c0 + BN], anchor and c0 == 0))
    return np.array(out, dtype=np.uint8)


def tile_kinds_col(cu, B: int, S: int, BM: int, BN: int, b: int, kt: int,
                   causal: bool = True, anchor: bool = True, origin: int = 0) -> np.ndarray:
    """Kinds of every query tile for key tile kt of row b, from the dense mask
    (tiles placed as in tile_kinds_row)."""
    nq = _grid(S, BM, origin)
    c0 = origin + kt * BN
    cols = np.arange(b * S + c0, b * S + min(S, c0 + BN))
    rows = np.arange(b * S, (b + 1) * S)
    height = origin + nq * BM
    m = np.zeros((height, BN), dtype=bool)
    e = np.zeros((height, BN), dtype=bool)
    if len(cols):
        m[:S, :len(cols)] = allowed(cu, B, S, rows, cols, causal, anchor)
        e[:S, :len(cols)] = True
    out = []
    for qt in range(nq):
        r0 = origin + qt * BM
        out.append(_classify(m[r0:r0 + BM], e[r0:r0 + BM], anchor and c0 == 0))
    return np.array(out, dtype=np.uint8)


def tile_plan(cu, B: int, S: int, BM: int, BN: int, causal: bool = True, anchor: bool = True,
              origin: int = 0):
    """Live (query-tile, key-tile) pairs and their kinds, from the dense mask.

    A tile is live when it holds at least one allowed element.  FULL: all
    BM*BN elements exist (no ragged edge) and are allowed.  ANCHOR: the key
    tile that starts at the anchor column (key tile 0 at origin 0) whose only
    allowed elements lie in that column.  PARTIAL: any other live tile.  With
    origin 1 the grid starts after the anchor (query tile qt holds rows
    1 + qt*BM ..), so no tile holds the anchor's row or column.  Returns a dict
    of int32/uint8 arrays: qptr [B*nq+1], kidx, kkind (query-major, key tiles
    ascending) and kptr [B*nk+1], qidx, qkind (key-major, query tiles
    ascending).
    """
    nq = _grid(S, BM, origin)
    nk = _grid(S, BN, origin)
    kinds = np.zeros((B, nq, nk), dtype=np.uint8)
    for b in range(B):
        for qt in range(nq):
            kinds[b, qt] = tile_kinds_row(cu, B, S, BM, BN, b, qt, causal, anchor, origin)
    qptr = [0]
    kidx, kkind = [], []
    for b in range(B):
        for qt in range(nq):
            for kt in range(nk):
                if kinds[b, qt, kt]:
                    kidx.append(kt)
                    kkind.append(kinds[b, qt, kt])
            qptr.append(len(kidx))
    kptr = [0]
    qidx, qkind = [], []
    for b in range(B):
        for kt in range(nk):
            for qt in range(nq):
                if kinds[b, qt, kt]:
                    qidx.append(qt)
                    qkind.append(kinds[b, qt, kt])
            kptr.append(len(qidx))
    return {
        "qptr": np.asarray(qptr, dtype=np.int32), "kidx": np.asarray(kidx, dtype=np.int32),
        "kkind": np.asarray(kkind, dtype=np.uint8),
        "kptr": np.asarray(kptr, dtype=np.int32), "qidx": np.asarray(qidx, dtype=np.int32),
        "qkind": np.asarray(qkind, dtype=np.uint8),
        "nq": nq, "nk": nk,
    }
