"""Pins of the oracle's interleaved-chunk mode (arch page §5, "AnchorAttention
with Interleaved Chunks", Figure 5 middle and right): documents cut into
chunks shuffled across the row, each document keeping its own order; a query
sees the anchor (if any) and the keys of its own document, in every chunk,
that are not after it.  Routes: positions written out by walking the chunks,
textbook causal attention on each document's gathered tokens (torch), torch
autograd, scalar brute force, and the contiguous case."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W


def _rand(shape, rng):
    return rng.standard_normal(shape)


def _docs_of(cu, chunk_doc, B, S):
    """Token lists of every document, per row, in stream order (walking the chunks)."""
    out = []
    for b in range(B):
        docs = {}
        for c in range(len(chunk_doc)):
            s_, e_ = int(cu[c]), int(cu[c + 1])
            if s_ // S != b:
                continue
            docs.setdefault(int(chunk_doc[c]), []).extend(range(s_ - b * S, e_ - b * S))
        out.append(docs)
    return out


def _positions(cu, chunk_doc, B, S, mode):
    pos = np.zeros(B * S, dtype=np.int64)
    for b, docs in enumerate(_docs_of(cu, chunk_doc, B, S)):
        for d, toks in docs.items():
            for n, t in enumerate(toks):
                if d == -1:
                    pos[b * S + t] = 0
                else:
                    pos[b * S + t] = n + 1 if mode == "reset" else t
    return pos


def _layout(rng, B, S, anchor, max_chunks=4):
    rows = [W.random_partition(rng, S if anchor else S + 1) for _ in range(B)]
    return W.interleaved_chunks(rows, S, rng, max_chunks, anchor)


@pytest.mark.parametrize("anchor", [True, False])
@pytest.mark.parametrize("mode", ["reset", "continuous"])
def test_positions_by_walking_the_chunks(anchor, mode):
    rng = np.random.default_rng(40)
    B, S = 2, 150
    cu, cd = _layout(rng, B, S, anchor)
    got = oracle.position_ids(cu, B, S, mode, anchor, seg_doc=cd)
    assert np.array_equal(got, _positions(cu, cd, B, S, mode))


def test_chunk_ids_are_validated():
    S = 10
    cu = np.array([0, 1, 4, 7, 10])
    oracle.document_ids(cu, 1, S, True, [-1, 0, 1, 0])
    with pytest.raises(ValueError):
        oracle.document_ids(cu, 1, S, True, [0, 0, 1, 0])      # anchor chunk must be -1
    with pytest.raises(ValueError):
        oracle.document_ids(cu, 1, S, True, [-1, 0, -1, 0])    # -1 only for the anchor
    with pytest.raises(ValueError):
        oracle.document_ids(cu, 1, S, True, [-1, 0, 1])        # one id per segment


def _torch_docs(q, k, v, cu, cd, B, S, base, anchor, mode):
    """Textbook causal attention on every document's gathered tokens."""
    Hq, D = q.shape[2], q.shape[3]
    r = Hq // k.shape[2]
    pos = _positions(cu, cd, B, S, mode)
    o = torch.zeros_like(q)
    for b, docs in enumerate(_docs_of(cu, cd, B, S)):
        if anchor:
            o[b, 0] = v[b, 0].repeat_interleave(r, dim=0)
        for d, toks in docs.items():
            if d == -1:
                continue
            idx = ([0] if anchor else []) + toks
            p = pos[[b * S + i for i in idx]]
            th = torch.tensor([base ** (-2.0 * i / D) for i in range(D // 2)], dtype=torch.float64)
            ang = torch.as_tensor(p.astype(np.float64))[:, None] * th[None, :]
            ph = torch.polar(torch.ones_like(ang), ang)[:, None, :]

            def rot(x):
                z = torch.view_as_complex(x.reshape(x.shape[0], x.shape[1], D // 2, 2).contiguous())
                return torch.view_as_real(z * ph).reshape(x.shape)
            qd = rot(q[b, idx])
            kd = rot(k[b, idx]).repeat_interleave(r, dim=1)
            vd = v[b, idx].repeat_interleave(r, dim=1)
            od = torch.nn.functional.scaled_dot_product_attention(
                qd.transpose(0, 1), kd.transpose(0, 1), vd.transpose(0, 1), is_causal=True).transpose(0, 1)
            o[b, toks] = od[1:] if anchor else od
    return o


@pytest.mark.parametrize("anchor,mode", [(True, "reset"), (True, "continuous"), (False, "reset"),
                                         (False, "continuous")])
def test_interleaved_equals_textbook_per_document_with_autograd(anchor, mode):
    rng = np.random.default_rng(41)
    B, S, Hq, Hkv, D, base = 2, 60, 4, 2, 8, 1e4
    cu, cd = _layout(rng, B, S, anchor)
    qn, kn, vn, don = (_rand((B, S, h, D), rng) for h in (Hq, Hkv, Hkv, Hq))
    o, _, _, _ = oracle.forward(qn, kn, vn, cu, base, pos_mode=mode, anchor=anchor, seg_doc=cd)
    q, k, v = (torch.tensor(x, requires_grad=True) for x in (qn, kn, vn))
    ref = _torch_docs(q, k, v, cu, cd, B, S, base, anchor, mode)
    assert np.abs(o - ref.detach().reshape(B * S, Hq, D).numpy()).max() < 1e-12
    (ref * torch.from_numpy(don)).sum().backward()
    dq, dk, dv, _, _ = oracle.backward(qn, kn, vn, don, cu, base, pos_mode=mode, anchor=anchor,
                                       seg_doc=cd)
    assert np.abs(dq - q.grad.reshape(B * S, Hq, D).numpy()).max() < 1e-10
    assert np.abs(dk - k.grad.reshape(B * S, Hkv, D).numpy()).max() < 1e-10
    assert np.abs(dv - v.grad.reshape(B * S, Hkv, D).numpy()).max() < 1e-10


@pytest.mark.parametrize("case", range(4))
def test_brute_force_interleaved(case):
    rng = np.random.default_rng(500 + case)
    anchor = case % 2 == 0
    mode = "reset" if case < 2 else "continuous"
    B, S, D, base = 1, int(rng.integers(4, 25)), 4, 1e4
    cu, cd = _layout(rng, B, S, anchor, 3)
    q, k, v = (_rand((B, S, 1, D), rng) for _ in range(3))
    o, _, _, _ = oracle.forward(q, k, v, cu, base, pos_mode=mode, anchor=anchor, seg_doc=cd)
    pos = _positions(cu, cd, B, S, mode)
    doc = np.zeros(S, dtype=np.int64)
    for c in range(len(cd)):
        doc[cu[c]:cu[c + 1]] = cd[c]

    def rot(vec, p):
        out = [0.0] * D
        for j in range(D // 2):
            a = p * base ** (-2.0 * j / D)
            out[2 * j] = vec[2 * j] * math.cos(a) - vec[2 * j + 1] * math.sin(a)
            out[2 * j + 1] = vec[2 * j] * math.sin(a) + vec[2 * j + 1] * math.cos(a)
        return out
    for i in range(S):
        if anchor and i == 0:
            vis = [0]
        else:
            vis = ([0] if anchor else []) + [j for j in range(i + 1) if doc[j] == doc[i] and not (anchor and j == 0)]
        qi = rot(q[0, i, 0], pos[i])
        lg = [sum(a * b for a, b in zip(qi, rot(k[0, j, 0], pos[j]))) / math.sqrt(D) for j in vis]
        mx = max(lg)
        w = [math.exp(x - mx) for x in lg]
        ref = sum(w[n] / sum(w) * v[0, j, 0] for n, j in enumerate(vis))
        assert np.abs(o[i, 0] - ref).max() < 1e-12


def test_adjacent_chunks_equal_the_contiguous_layout():
    """Chunks that are not interleaved are the ordinary packing."""
    rng = np.random.default_rng(42)
    S = 80
    rows = [[30, 20, 29]]
    cu_docs = W.cu_doc_lens_from_lengths(rows, S)
    cu = np.array([0, 1, 11, 31, 51, 60, 80])          # doc 0 in two chunks, doc 2 in two chunks
    cd = np.array([-1, 0, 0, 1, 2, 2])
    q, k, v, do = (_rand((1, S, 2, 8), rng) for _ in range(4))
    for mode in ("reset", "continuous"):
        assert np.array_equal(oracle.position_ids(cu, 1, S, mode, seg_doc=cd),
                              oracle.position_ids(cu_docs, 1, S, mode))
        a, _, _, _ = oracle.forward(q, k, v, cu, 1e4, pos_mode=mode, seg_doc=cd)
        b, _, _, _ = oracle.forward(q, k, v, cu_docs, 1e4, pos_mode=mode)
        assert np.abs(a - b).max() < 1e-15
