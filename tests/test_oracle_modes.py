"""Pins of the oracle's other modes, by routes other than its own formula.

* Without an anchor (the pages' intra-document baselines, Figure 2 left and
  middle): a query sees only the causal keys of its own document.
* Continuous position IDs with the anchor (Figure 2 right, the paper's own
  reading of AnchorAttention): document tokens count on from 1 after the
  anchor across the whole row.

Routes: complex-number rotation and torch's textbook causal attention on
each document alone, torch autograd, scalar brute force, RoPE's relative
property (Eq. 3) and closed-form tile plans.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W


def _rand(shape, rng):
    return rng.standard_normal(shape)


def _cu(rows, S, anchor):
    return W.cu_doc_lens_from_lengths(rows, S) if anchor else W.cu_doc_lens_no_anchor(rows, S)


def _positions(rows, S, anchor, mode):
    """Position IDs written out from the pages' wording, per row."""
    out = []
    for lens in rows:
        p = [0] if anchor else []
        t = 1 if anchor else 0
        for L in lens:
            for n in range(L):
                p.append(n + 1 if mode == "reset" else t + n)
            t += L
        out.extend(p)
    return np.asarray(out)


def _rot(x, pos, base):
    """RoPE as complex multiplication (x_2p + i x_2p+1) e^{i pos theta_p}, torch."""
    D = x.shape[-1]
    th = torch.tensor([base ** (-2.0 * p / D) for p in range(D // 2)], dtype=torch.float64)
    ang = torch.as_tensor(np.asarray(pos, dtype=np.float64))[:, None] * th[None, :]
    ph = torch.polar(torch.ones_like(ang), ang)[:, None, :]
    z = torch.view_as_complex(x.reshape(x.shape[0], x.shape[1], D // 2, 2).contiguous())
    return torch.view_as_real(z * ph).reshape(x.shape)


def _torch_docs(q, k, v, rows, S, base, anchor, mode):
    """Textbook causal attention over each document alone ([anchor; document]
    when there is an anchor), with the positions the mode assigns."""
    B, _, Hq, D = q.shape
    Hkv = k.shape[2]
    r = Hq // Hkv
    pos = _positions(rows, S, anchor, mode)
    outs = []
    for b in range(B):
        pieces = []
        start = 0
        if anchor:
            pieces.append(v[b, 0:1].repeat_interleave(r, dim=1))   # anchor row: O = v_anchor
            start = 1
        for L in rows[b]:
            idx = ([0] if anchor else []) + list(range(start, start + L))
            p = pos[[b * S + i for i in idx]]
            qd = _rot(q[b, idx], p, base)
            kd = _rot(k[b, idx], p, base).repeat_interleave(r, dim=1)
            vd = v[b, idx].repeat_interleave(r, dim=1)
            od = torch.nn.functional.scaled_dot_product_attention(
                qd.transpose(0, 1), kd.transpose(0, 1), vd.transpose(0, 1), is_causal=True).transpose(0, 1)
            pieces.append(od[1:] if anchor else od)
            start += L
        outs.append(torch.cat(pieces, 0))
    return torch.stack(outs, 0)


@pytest.mark.parametrize("mode", ["reset", "continuous"])
def test_positions_written_out(mode):
    rng = np.random.default_rng(21)
    S = 90
    for anchor in (True, False):
        rows = [W.random_partition(rng, S if anchor else S + 1) for _ in range(2)]
        cu = _cu(rows, S, anchor)
        assert np.array_equal(oracle.position_ids(cu, 2, S, mode, anchor), _positions(rows, S, anchor, mode))


def test_no_anchor_needs_no_anchor_segment():
    S = 10
    cu = W.cu_doc_lens_no_anchor([[4, 6]], S)
    with pytest.raises(ValueError):
        oracle.validate_cu(cu, 1, S)                  # the anchor reading insists on [0, 1)
    oracle.validate_cu(cu, 1, S, anchor=False)
    with pytest.raises(ValueError):                   # a segment may not cross rows
        oracle.validate_cu(np.array([0, 4, 12, 20]), 2, S, anchor=False)


@pytest.mark.parametrize("mode", ["reset", "continuous"])
def test_no_anchor_single_document_is_textbook(mode):
    rng = np.random.default_rng(22)
    S, H, D, base = 77, 2, 16, 1e4
    q, k, v = (_rand((1, S, H, D), rng) for _ in range(3))
    cu = _cu([[S]], S, False)
    o, lse, _, _ = oracle.forward(q, k, v, cu, base, pos_mode=mode, anchor=False)
    pos = np.arange(S) + (1 if mode == "reset" else 0)
    qr = _rot(torch.from_numpy(q[0]), pos, base).permute(1, 0, 2)
    kr = _rot(torch.from_numpy(k[0]), pos, base).permute(1, 0, 2)
    vv = torch.from_numpy(v[0]).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(qr, kr, vv, is_causal=True)
    assert np.abs(o - ref.permute(1, 0, 2).numpy()).max() < 1e-12
    s = (qr @ kr.transpose(1, 2)) / math.sqrt(D)
    s = s.masked_fill(torch.triu(torch.ones(S, S, dtype=torch.bool), 1), float("-inf"))
    assert np.abs(lse - torch.logsumexp(s, -1).numpy()).max() < 1e-12


@pytest.mark.parametrize("anchor,mode", [(False, "reset"), (False, "continuous"), (True, "continuous")])
def test_modes_decompose_into_documents_with_autograd(anchor, mode):
    rng = np.random.default_rng(23)
    B, S, Hq, Hkv, D, base = 2, 40, 4, 2, 8, 1e4
    rows = [[7, 1, 20, 11], [39]] if anchor else [[8, 1, 20, 11], [40]]
    cu = _cu(rows, S, anchor)
    qn, kn, vn, don = (_rand((B, S, h, D), rng) for h in (Hq, Hkv, Hkv, Hq))
    o, _, _, _ = oracle.forward(qn, kn, vn, cu, base, pos_mode=mode, anchor=anchor)
    q, k, v = (torch.tensor(x, requires_grad=True) for x in (qn, kn, vn))
    ref = _torch_docs(q, k, v, rows, S, base, anchor, mode)
    assert np.abs(o - ref.detach().reshape(B * S, Hq, D).numpy()).max() < 1e-12
    (ref * torch.from_numpy(don)).sum().backward()
    dq, dk, dv, _, _ = oracle.backward(qn, kn, vn, don, cu, base, pos_mode=mode, anchor=anchor)
    assert np.abs(dq - q.grad.reshape(B * S, Hq, D).numpy()).max() < 1e-10
    assert np.abs(dk - k.grad.reshape(B * S, Hkv, D).numpy()).max() < 1e-10
    assert np.abs(dv - v.grad.reshape(B * S, Hkv, D).numpy()).max() < 1e-10


def _brute(q, k, v, rows, S, base, anchor, mode, causal):
    """Scalar loops over every (query, key) pair of every document."""
    B, _, Hq, D = q.shape
    Hkv = k.shape[2]
    pos = _positions(rows, S, anchor, mode)
    O = np.zeros((B * S, Hq, D))

    def rot(vec, p):
        out = [0.0] * D
        for j in range(D // 2):
            a = p * base ** (-2.0 * j / D)
            c, s = math.cos(a), math.sin(a)
            out[2 * j] = vec[2 * j] * c - vec[2 * j + 1] * s
            out[2 * j + 1] = vec[2 * j] * s + vec[2 * j + 1] * c
        return out
    for b in range(B):
        vis = {}
        start = 0
        if anchor:
            vis[0] = [0]
            start = 1
        for L in rows[b]:
            for t in range(start, start + L):
                last = t if causal else start + L - 1
                vis[t] = ([0] if anchor else []) + list(range(start, last + 1))
            start += L
        for h in range(Hq):
            g = h * Hkv // Hq
            for t, keys in vis.items():
                qi = rot(q[b, t, h], pos[b * S + t])
                lg = [sum(x * y for x, y in zip(qi, rot(k[b, j, g], pos[b * S + j]))) / math.sqrt(D)
                      for j in keys]
                mx = max(lg)
                w = [math.exp(x - mx) for x in lg]
                for n, j in enumerate(keys):
                    O[b * S + t, h] += w[n] / sum(w) * v[b, j, g]
    return O


@pytest.mark.parametrize("case", range(6))
def test_brute_force_modes(case):
    rng = np.random.default_rng(300 + case)
    anchor = case % 2 == 0
    mode = "continuous" if case in (0, 1, 3) else "reset"
    causal = case != 5
    S = int(rng.integers(3, 30))
    B = int(rng.integers(1, 3))
    D = [2, 4, 8][case % 3]
    Hkv = int(rng.integers(1, 3))
    Hq = Hkv * int(rng.integers(1, 3))
    rows = [W.random_partition(rng, S if anchor else S + 1) for _ in range(B)]
    cu = _cu(rows, S, anchor)
    q, k, v = (_rand((B, S, h, D), rng) for h in (Hq, Hkv, Hkv))
    o, _, _, _ = oracle.forward(q, k, v, cu, 1e4, causal=causal, pos_mode=mode, anchor=anchor)
    assert np.abs(o - _brute(q, k, v, rows, S, 1e4, anchor, mode, causal)).max() < 1e-12


def test_no_anchor_positions_do_not_matter_in_exact_arithmetic():
    # Eq. 3: with every logit inside one document, shifting a document's
    # positions (reset vs continuous) leaves the exact result unchanged.
    rng = np.random.default_rng(24)
    S, D = 300, 16
    rows = [[50, 120, 1, 129]]
    cu = _cu(rows, S, False)
    q, k, v = (_rand((1, S, 2, D), rng) for _ in range(3))
    o1, l1, _, _ = oracle.forward(q, k, v, cu, 5e5, pos_mode="reset", anchor=False)
    o2, l2, _, _ = oracle.forward(q, k, v, cu, 5e5, pos_mode="continuous", anchor=False)
    assert np.abs(o1 - o2).max() < 1e-11 and np.abs(l1 - l2).max() < 1e-11
    # with the anchor the anchor column's logits move, so the results differ
    rows_a = [[49, 120, 1, 129]]
    cu_a = _cu(rows_a, S, True)
    o3, _, _, _ = oracle.forward(q, k, v, cu_a, 5e5, pos_mode="reset")
    o4, _, _, _ = oracle.forward(q, k, v, cu_a, 5e5, pos_mode="continuous")
    assert np.abs(o3[1:50] - o4[1:50]).max() < 1e-12        # first document: same positions
    assert np.abs(o3[50:] - o4[50:]).max() > 1e-6


def test_no_anchor_pair_count():
    rng = np.random.default_rng(25)
    for _ in range(10):
        S = int(rng.integers(2, 200))
        rows = [W.random_partition(rng, S + 1) for _ in range(2)]
        cu = _cu(rows, S, False)
        assert oracle.unmasked_pairs(cu, 2, S, anchor=False) == sum(L * (L + 1) // 2 for r in rows for L in r)
        assert oracle.unmasked_pairs(cu, 2, S, causal=False, anchor=False) == sum(L * L for r in rows for L in r)


@pytest.mark.parametrize("S", [300, 257])
@pytest.mark.parametrize("BM,BN", [(64, 64), (128, 64), (64, 128)])
def test_no_anchor_plan_single_document(BM, BN, S):
    """One document without an anchor: the plan is the causal block triangle."""
    plan = oracle.tile_plan(_cu([[S]], S, False), 1, S, BM, BN, anchor=False)
    nq, nk = -(-S // BM), -(-S // BN)
    kidx, kkind = [], []
    for qt in range(nq):
        last_row = min(S, (qt + 1) * BM) - 1
        for kt in range(nk):
            if kt * BN > last_row:
                continue
            full = (kt + 1) * BN - 1 <= qt * BM and (qt + 1) * BM <= S and (kt + 1) * BN <= S
            kidx.append(kt)
            kkind.append(oracle.KIND_FULL if full else oracle.KIND_PARTIAL)
    assert plan["kidx"].tolist() == kidx and plan["kkind"].tolist() == kkind


def test_no_anchor_plan_has_no_anchor_tiles():
    rng = np.random.default_rng(26)
    S = 200
    rows = [W.random_partition(rng, S + 1) for _ in range(2)]
    for BM, BN in ((32, 32), (1, 4), (2, 8)):
        plan = oracle.tile_plan(_cu(rows, S, False), 2, S, BM, BN, anchor=False)
        assert oracle.KIND_ANCHOR not in set(plan["kkind"].tolist())
    # token 0 alone in its query tile sees only column 0: an ordinary partial tile
    plan = oracle.tile_plan(_cu([[3, 7]], 10, False), 1, 10, 1, 4, anchor=False)
    assert plan["kidx"][0] == 0 and plan["kkind"][0] == oracle.KIND_PARTIAL
