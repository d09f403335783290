"""Pins of the CPU oracle against what the pages and the mathematics fix.

Every check here uses a route other than the oracle's own formula: closed
forms, hand-derived worked values, textbook attention (torch's
scaled_dot_product_attention on independently rotated inputs), complex-number
rotation, scalar brute force, finite differences and invariants.
"""
import cmath
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, rng):
    return rng.standard_normal(shape)


def _cu(rows, S):
    return W.cu_doc_lens_from_lengths(rows, S)


def _rope_complex(x, pos, base):
    """Rotation as complex multiplication: (x_2p + i x_2p+1) * exp(i pos theta_p)."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    z = x[..., 0::2] + 1j * x[..., 1::2]
    theta = np.array([base ** (-2.0 * p / D) for p in range(D // 2)])
    ph = np.exp(1j * np.outer(np.asarray(pos, dtype=np.float64), theta))
    if x.ndim == 3:
        ph = ph[:, None, :]
    w = z * ph
    out = np.empty_like(x)
    out[..., 0::2] = w.real
    out[..., 1::2] = w.imag
    return out


# ---------------------------------------------------------------- worked example
def test_tiny_positions_and_pairs_golden():
    g = json.load(open(os.path.join(GOLDEN, "tiny_worked.json")))
    cu = np.array(g["cu_doc_lens"])
    pos = oracle.position_ids(cu, 1, g["S"])
    assert list(pos[g["position_ids_at"]["t"]]) == g["position_ids_at"]["pos"]
    assert oracle.unmasked_pairs(cu, 1, g["S"]) == g["unmasked_pairs"]
    assert np.array_equal(W.get("tiny").cu_doc_lens, cu)


@pytest.mark.parametrize("tile", ["64x64", "128x128"])
def test_tiny_plan_golden(tile):
    g = json.load(open(os.path.join(GOLDEN, "tiny_worked.json")))
    BM, BN = map(int, tile.split("x"))
    p = oracle.tile_plan(np.array(g["cu_doc_lens"]), 1, g["S"], BM, BN)
    code = {"F": oracle.KIND_FULL, "P": oracle.KIND_PARTIAL, "A": oracle.KIND_ANCHOR}
    for qt, lst in enumerate(g["plan"][tile]["q_major"]):
        a, b = p["qptr"][qt], p["qptr"][qt + 1]
        assert list(p["kidx"][a:b]) == [e[0] for e in lst]
        assert list(p["kkind"][a:b]) == [code[e[1]] for e in lst]


# ---------------------------------------------------------------- positions
def test_positions_closed_form_random():
    rng = np.random.default_rng(5)
    for _ in range(20):
        S = int(rng.integers(2, 200))
        B = int(rng.integers(1, 3))
        rows = [W.random_partition(rng, S) for _ in range(B)]
        cu = _cu(rows, S)
        pos = oracle.position_ids(cu, B, S)
        cont = oracle.position_ids(cu, B, S, "continuous")
        for b, lens in enumerate(rows):
            expect = [0] + [i + 1 for L in lens for i in range(L)]
            assert list(pos[b * S:(b + 1) * S]) == expect
            assert list(cont[b * S:(b + 1) * S]) == list(range(S))


def test_cu_validation_rejects_misuse():
    with pytest.raises(ValueError):
        oracle.validate_cu([0, 5, 8], 1, 8)          # no anchor segment
    with pytest.raises(ValueError):
        oracle.validate_cu([0, 1, 1, 8], 1, 8)       # empty document
    with pytest.raises(ValueError):
        oracle.validate_cu([0, 1, 7], 1, 8)          # wrong total
    with pytest.raises(ValueError):
        oracle.validate_cu([0, 1, 10, 16], 2, 8)     # document crosses rows / no anchor in row 1


# ---------------------------------------------------------------- RoPE (Eq. 6, Eq. 7)
def test_rope_relative_property_and_norm():
    rng = np.random.default_rng(1)
    D, base = 16, 1e4
    eye = np.eye(D)
    def R(i):
        # column c of R_i is R_i applied to e_c
        return oracle.rope(eye, np.full(D, i), base).T
    for i, j in [(0, 0), (3, 10), (1000, 17), (65535, 2)]:
        lhs = R(i).T @ R(j)
        rhs = R(j - i)
        assert np.allclose(lhs, rhs, atol=1e-10)
    x = _rand((50, D), rng)
    pos = rng.integers(0, 1 << 17, 50)
    y = oracle.rope(x, pos, base)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    assert np.allclose(oracle.rope(y, pos, base, inverse=True), x, atol=1e-11)
    assert np.array_equal(oracle.rope(x, np.zeros(50, int), base), x)   # R_0 = I


def test_rope_is_complex_multiplication():
    rng = np.random.default_rng(2)
    # D = 2: theta_0 = 1, so the pair is multiplied by exp(i*pos)
    x = _rand((7, 2), rng)
    pos = np.array([0, 1, 2, 5, 100, 4096, 65535])
    y = oracle.rope(x, pos, 5e6)
    for n in range(7):
        w = complex(x[n, 0], x[n, 1]) * cmath.exp(1j * pos[n])
        assert abs(y[n, 0] - w.real) < 1e-9 and abs(y[n, 1] - w.imag) < 1e-9
    x = _rand((9, 3, 64), rng)
    pos = rng.integers(0, 70000, 9)
    assert np.allclose(oracle.rope(x, pos, 5e6), _rope_complex(x, pos, 5e6), atol=1e-9)


# ---------------------------------------------------------------- one document = textbook
def test_single_document_is_plain_causal_rope_attention():
    rng = np.random.default_rng(3)
    S, H, D, base = 97, 3, 32, 1e4
    q, k, v = (_rand((1, S, H, D), rng) for _ in range(3))
    cu = _cu([[S - 1]], S)
    o, lse, _, _ = oracle.forward(q, k, v, cu, base)
    pos = np.arange(S)                       # one document: positions 0..S-1
    qr = torch.from_numpy(_rope_complex(q[0], pos, base)).permute(1, 0, 2)
    kr = torch.from_numpy(_rope_complex(k[0], pos, base)).permute(1, 0, 2)
    vv = torch.from_numpy(v[0]).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(qr, kr, vv, is_causal=True)
    assert np.abs(o - ref.permute(1, 0, 2).numpy()).max() < 1e-12
    # log-sum-exp from the textbook logits
    s = (qr @ kr.transpose(1, 2)) / math.sqrt(D)
    s = s.masked_fill(torch.triu(torch.ones(S, S, dtype=torch.bool), 1), float("-inf"))
    assert np.abs(lse - torch.logsumexp(s, -1).numpy()).max() < 1e-12


# ---------------------------------------------------------------- shift invariance (Eq. 3)
@pytest.mark.parametrize("delta", [1, 16, 2000, 100000])
def test_shift_invariance(delta):
    rng = np.random.default_rng(4)
    S, D, base = 64, 32, 5e6
    lens = [20, 1, 30, 12]
    cu = _cu([lens], S)
    q, k = _rand((S, D), rng), _rand((S, D), rng)
    pos = oracle.position_ids(cu, 1, S)
    seg = oracle.segment_ids(cu, 1, S)
    def logits(p):
        return oracle.rope(q, p, base) @ oracle.rope(k, p, base).T
    base_l = logits(pos)
    m = oracle.allowed(cu, 1, S, np.arange(S), np.arange(S))
    # (i) every position shifted (anchor too): every logit unchanged
    assert np.abs(logits(pos + delta) - base_l)[m].max() < 1e-9
    # (ii) only document positions shifted: in-document logits unchanged,
    #      logits against the anchor column change
    p2 = np.where(np.arange(S) == 0, 0, pos + delta)
    l2 = logits(p2)
    same_doc = m & (seg[:, None] == seg[None, :]) & (np.arange(S)[None, :] > 0)
    assert np.abs(l2 - base_l)[same_doc].max() < 1e-9
    assert np.abs(l2[1:, 0] - base_l[1:, 0]).max() > 1e-3
    # the full forward is unchanged under (i)
    qb, kb, vb = q[None, :, None, :], k[None, :, None, :], _rand((1, S, 1, D), rng)
    o1, l1, _, _ = oracle.forward(qb, kb, vb, cu, base)
    o2, l2b, _, _ = oracle.forward(qb, kb, vb, cu, base, pos=pos + delta)
    assert np.abs(o1 - o2).max() < 1e-9 and np.abs(l1 - l2b).max() < 1e-9


# ---------------------------------------------------------------- the anchor
def test_every_query_weights_its_anchor():
    rng = np.random.default_rng(6)
    B, S, H, D = 2, 80, 2, 16
    rows = [[30, 1, 48], [79]]
    cu = _cu(rows, S)
    q, k, v = (_rand((B, S, H, D), rng) * 3 for _ in range(3))
    pos = oracle.position_ids(cu, B, S)
    o, lse, r, heads = oracle.forward(q, k, v, cu, 1e4)
    t = np.arange(B * S)
    anchors = (t // S) * S
    assert oracle.allowed(cu, B, S, t, t)[...].shape == (B * S, B * S)
    for i in t:
        assert oracle.allowed(cu, B, S, [i], [anchors[i]])[0, 0]
    for h in range(H):
        for i in t:
            b = i // S
            qi = oracle.rope(q[b, i - b * S, h][None], [pos[i]], 1e4)[0]
            s0 = qi @ k[b, 0, h] / math.sqrt(D)          # anchor key: R_0 = I
            p0 = math.exp(s0 - lse[h, i])
            assert p0 > 0.0
    # the anchor row attends only to itself: O = v_anchor, LSE = s_00
    for b in range(B):
        for h in range(H):
            assert np.allclose(o[b * S, h], v[b, 0, h], atol=1e-12)
            assert abs(lse[h, b * S] - q[b, 0, h] @ k[b, 0, h] / math.sqrt(D)) < 1e-12


# ---------------------------------------------------------------- brute force
def _brute_forward(q, k, v, rows, S, base, causal=True):
    """Scalar loops: walk the documents, rotate with math.cos/sin, softmax."""
    B, _, Hq, D = q.shape
    Hkv = k.shape[2]
    O = np.zeros((B * S, Hq, D))
    L = np.zeros((Hq, B * S))
    def rot(vec, p):
        out = [0.0] * D
        for j in range(D // 2):
            a = p * base ** (-2.0 * j / D)
            c, s = math.cos(a), math.sin(a)
            out[2 * j] = vec[2 * j] * c - vec[2 * j + 1] * s
            out[2 * j + 1] = vec[2 * j] * s + vec[2 * j + 1] * c
        return out
    for b in range(B):
        # (token, position, visible keys) from the document lengths
        toks = [(0, 0, [0])]
        start = 1
        for Ld in rows[b]:
            for n in range(Ld):
                t = start + n
                last = t if causal else start + Ld - 1
                toks.append((t, n + 1, [0] + list(range(start, last + 1))))
            start += Ld
        posl = [p for _, p, _ in toks]
        for h in range(Hq):
            g = h * Hkv // Hq
            for t, p, vis in toks:
                qi = rot(q[b, t, h], p)
                logits = []
                for j in vis:
                    kj = rot(k[b, j, g], posl[j])
                    logits.append(sum(a * c for a, c in zip(qi, kj)) / math.sqrt(D))
                mx = max(logits)
                w = [math.exp(x - mx) for x in logits]
                tot = sum(w)
                for n, j in enumerate(vis):
                    O[b * S + t, h] += w[n] / tot * v[b, j, g]
                L[h, b * S + t] = mx + math.log(tot)
    return O, L


@pytest.mark.parametrize("case", range(8))
def test_brute_force_tiny(case):
    rng = np.random.default_rng(100 + case)
    S = int(rng.integers(2, 40))
    B = int(rng.integers(1, 3))
    D = [2, 4, 8][case % 3]
    Hkv = int(rng.integers(1, 3))
    Hq = Hkv * int(rng.integers(1, 3))
    if case == 0:
        rows = [[S - 1]] * B                    # a single document
    elif case == 1:
        rows = [[1] * (S - 1)] * B              # all documents of length 1
    else:
        rows = [W.random_partition(rng, S) for _ in range(B)]
    cu = _cu(rows, S)
    q, k, v = (_rand((B, S, h, D), rng) for h in (Hq, Hkv, Hkv))
    causal = case != 7
    o, lse, _, _ = oracle.forward(q, k, v, cu, 1e4, causal=causal)
    ob, lb = _brute_forward(q, k, v, rows, S, 1e4, causal)
    assert np.abs(o - ob).max() < 1e-12
    assert np.abs(lse - lb).max() < 1e-12


def test_pair_count_closed_form():
    rng = np.random.default_rng(7)
    for _ in range(20):
        S = int(rng.integers(2, 300))
        B = int(rng.integers(1, 3))
        rows = [W.random_partition(rng, S) for _ in range(B)]
        cu = _cu(rows, S)
        expect = sum(1 + sum(L * (L + 1) // 2 + L for L in r) for r in rows)
        assert oracle.unmasked_pairs(cu, B, S) == expect
        expect_nc = sum(1 + sum(L * L + L for L in r) for r in rows)
        assert oracle.unmasked_pairs(cu, B, S, causal=False) == expect_nc


# ---------------------------------------------------------------- per-document decomposition
def _torch_decomposed(q, k, v, rows, S, base):
    """Textbook causal attention over [anchor; document] alone, per document."""
    B, _, Hq, D = q.shape
    Hkv = k.shape[2]
    outs = []
    for b in range(B):
        pieces = [v[b, 0:1].repeat_interleave(Hq // Hkv, dim=1)]   # anchor row: O = v_anchor
        start = 1
        for Ld in rows[b]:
            idx = [0] + list(range(start, start + Ld))
            pos = np.arange(Ld + 1)
            th = torch.tensor([base ** (-2.0 * p / D) for p in range(D // 2)], dtype=torch.float64)
            ang = torch.from_numpy(pos.astype(np.float64))[:, None] * th[None, :]
            ph = torch.polar(torch.ones_like(ang), ang)[:, None, :]
            def rot(x):
                z = torch.view_as_complex(x.reshape(x.shape[0], x.shape[1], D // 2, 2).contiguous())
                return torch.view_as_real(z * ph).reshape(x.shape)
            qd = rot(q[b, idx])
            kd = rot(k[b, idx]).repeat_interleave(Hq // Hkv, dim=1)
            vd = v[b, idx].repeat_interleave(Hq // Hkv, dim=1)
            od = torch.nn.functional.scaled_dot_product_attention(
                qd.transpose(0, 1), kd.transpose(0, 1), vd.transpose(0, 1), is_causal=True).transpose(0, 1)
            pieces.append(od[1:])
            start += Ld
        outs.append(torch.cat(pieces, 0))
    return torch.stack(outs, 0)


def test_document_decomposition_and_autograd():
    rng = np.random.default_rng(8)
    B, S, Hq, Hkv, D, base = 2, 40, 4, 2, 8, 1e4
    rows = [[7, 1, 20, 11], [39]]
    cu = _cu(rows, S)
    qn, kn, vn, don = (_rand((B, S, h, D), rng) for h in (Hq, Hkv, Hkv, Hq))
    o, _, _, _ = oracle.forward(qn, kn, vn, cu, base)
    q, k, v = (torch.tensor(x, requires_grad=True) for x in (qn, kn, vn))
    ref = _torch_decomposed(q, k, v, rows, S, base)
    assert np.abs(o - ref.detach().reshape(B * S, Hq, D).numpy()).max() < 1e-12
    (ref * torch.from_numpy(don)).sum().backward()
    dq, dk, dv, _, _ = oracle.backward(qn, kn, vn, don, cu, base)
    assert np.abs(dq - q.grad.reshape(B * S, Hq, D).numpy()).max() < 1e-10
    assert np.abs(dk - k.grad.reshape(B * S, Hkv, D).numpy()).max() < 1e-10
    assert np.abs(dv - v.grad.reshape(B * S, Hkv, D).numpy()).max() < 1e-10


def test_documents_do_not_interact():
    rng = np.random.default_rng(9)
    S, D = 50, 8
    rows = [[10, 25, 14]]
    cu = _cu(rows, S)
    q, k, v = (_rand((1, S, 1, D), rng) for _ in range(3))
    o1, _, _, _ = oracle.forward(q, k, v, cu, 1e4)
    # change everything in documents 1 and 3; document 2 (tokens 11..35) is untouched
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    for a in (q2, k2, v2):
        a[0, 1:11] = _rand((10, 1, D), rng)
        a[0, 36:] = _rand((14, 1, D), rng)
    o2, _, _, _ = oracle.forward(q2, k2, v2, cu, 1e4)
    assert np.abs(o1[11:36] - o2[11:36]).max() < 1e-15


# ---------------------------------------------------------------- gradients
def test_finite_differences():
    rng = np.random.default_rng(10)
    B, S, Hq, Hkv, D, base = 1, 12, 2, 1, 4, 100.0
    rows = [[4, 1, 6]]
    cu = _cu(rows, S)
    q, k, v, do = (_rand((B, S, h, D), rng) for h in (Hq, Hkv, Hkv, Hq))
    dq, dk, dv, _, _ = oracle.backward(q, k, v, do, cu, base)
    def loss(q_, k_, v_):
        o, _, _, _ = oracle.forward(q_, k_, v_, cu, base)
        return float((o * do.reshape(B * S, Hq, D)).sum())
    h = 1e-6
    for name, arr, grad, shape in (("q", q, dq, (B * S, Hq, D)), ("k", k, dk, (B * S, Hkv, D)),
                                   ("v", v, dv, (B * S, Hkv, D))):
        for _ in range(12):
            idx = tuple(int(rng.integers(0, n)) for n in arr.shape)
            ap, am = arr.copy(), arr.copy()
            ap[idx] += h
            am[idx] -= h
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = ap, am
            fd = (loss(**{n + "_": a for n, a in args_p.items()}) - loss(**{n + "_": a for n, a in args_m.items()})) / (2 * h)
            g = grad.reshape(shape)[idx[0] * S + idx[1], idx[2], idx[3]]
            assert abs(fd - g) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, g)


def test_value_translation_identity():
    """Softmax rows sum to 1 and the row term Dv is subtracted: adding a constant
    vector c to every value shifts O by c and leaves dq, dk unchanged."""
    rng = np.random.default_rng(11)
    B, S, H, D = 1, 30, 2, 8
    cu = _cu([[9, 12, 8]], S)
    q, k, v, do = (_rand((B, S, H, D), rng) for _ in range(4))
    c = _rand((D,), rng)
    o1, _, _, _ = oracle.forward(q, k, v, cu, 1e4)
    o2, _, _, _ = oracle.forward(q, k, v + c, cu, 1e4)
    assert np.abs(o2 - o1 - c).max() < 1e-12
    g1 = oracle.backward(q, k, v, do, cu, 1e4)
    g2 = oracle.backward(q, k, v + c, do, cu, 1e4)
    assert np.abs(g1[0] - g2[0]).max() < 1e-11 and np.abs(g1[1] - g2[1]).max() < 1e-11


def test_sampled_backward_matches_full():
    rng = np.random.default_rng(12)
    B, S, Hq, Hkv, D = 2, 64, 4, 2, 16
    rows = [[20, 3, 40], [63]]
    cu = _cu(rows, S)
    q, k, v, do = (_rand((B, S, h, D), rng) for h in (Hq, Hkv, Hkv, Hq))
    full = oracle.backward(q, k, v, do, cu, 1e4, block=16)
    qr = np.array([0, 5, 21, 70, 127])
    kc = np.array([0, 1, 23, 24, 64, 100])
    part = oracle.backward(q, k, v, do, cu, 1e4, q_rows=qr, k_cols=kc, block=16)
    assert np.abs(part[0] - full[0][qr]).max() < 1e-12
    assert np.abs(part[1] - full[1][kc]).max() < 1e-12
    assert np.abs(part[2] - full[2][kc]).max() < 1e-12
    o, l, _, _ = oracle.forward(q, k, v, cu, 1e4, rows=qr)
    of, lf, _, _ = oracle.forward(q, k, v, cu, 1e4)
    assert np.abs(o - of[qr]).max() < 1e-12 and np.abs(l - lf[:, qr]).max() < 1e-12


# ---------------------------------------------------------------- tile plan closed forms
@pytest.mark.parametrize("S", [300, 257])
@pytest.mark.parametrize("BM,BN", [(64, 64), (128, 64), (32, 32)])
def test_plan_single_document_is_causal_block_triangle(BM, BN, S):
    p = oracle.tile_plan(_cu([[S - 1]], S), 1, S, BM, BN)
    nq = -(-S // BM)
    for qt in range(nq):
        a, b = p["qptr"][qt], p["qptr"][qt + 1]
        last_row = min(S, (qt + 1) * BM) - 1
        expect_k = list(range(0, last_row // BN + 1))
        assert list(p["kidx"][a:b]) == expect_k
        for kt, kind in zip(p["kidx"][a:b], p["kkind"][a:b]):
            full = (qt + 1) * BM <= S and (kt + 1) * BN - 1 <= qt * BM and not (qt == 0)
            assert kind == (oracle.KIND_FULL if full else oracle.KIND_PARTIAL), (qt, kt, kind)


def test_plan_all_length_one_documents():
    S, BM = 256, 64
    p = oracle.tile_plan(_cu([[1] * (S - 1)], S), 1, S, BM, BM)
    for qt in range(S // BM):
        a, b = p["qptr"][qt], p["qptr"][qt + 1]
        if qt == 0:
            assert list(p["kidx"][a:b]) == [0] and list(p["kkind"][a:b]) == [oracle.KIND_PARTIAL]
        else:
            assert list(p["kidx"][a:b]) == [0, qt]
            assert list(p["kkind"][a:b]) == [oracle.KIND_ANCHOR, oracle.KIND_PARTIAL]


def test_plan_key_major_is_transpose():
    rng = np.random.default_rng(13)
    S, B = 333, 2
    cu = _cu([W.random_partition(rng, S, 9) for _ in range(B)], S)
    p = oracle.tile_plan(cu, B, S, 64, 32)
    nq, nk = p["nq"], p["nk"]
    qm = {}
    for bq in range(B * nq):
        for e in range(p["qptr"][bq], p["qptr"][bq + 1]):
            qm[(bq // nq, bq % nq, int(p["kidx"][e]))] = int(p["kkind"][e])
    km = {}
    for bk in range(B * nk):
        for e in range(p["kptr"][bk], p["kptr"][bk + 1]):
            km[(bk // nk, int(p["qidx"][e]), bk % nk)] = int(p["qkind"][e])
    assert qm == km
    # every query tile keeps key tile 0 (the anchor column)
    for b in range(B):
        for qt in range(nq):
            assert (b, qt, 0) in qm


# ---------------------------------------------------------------- key-major checker
def _brute_kinds(rows, S, BM, BN, causal=True, anchor=True, origin=0):
    """Tile kinds [B, nq, nk] by scalar loops over every element, from the
    document lengths alone (no oracle mask): a query sees its row's anchor
    (with ``anchor``) and the keys of its own document not after it (any of
    them when not ``causal``).  Tile (qt, kt) holds rows origin + qt*BM ..
    and keys origin + kt*BN .. below S.  Kinds: FULL when all BM*BN elements
    exist and are seen, ANCHOR for the tile starting at key 0 when only column
    0 is seen, PARTIAL for any other tile with a seen element."""
    B = len(rows)
    nq, nk = -(-S // BM), -(-S // BN)
    doc = []
    for lens in rows:
        d = []
        if anchor:
            d.append(-1)
        for n, L in enumerate(lens):
            d.extend([n] * L)
        doc.append(d)
    out = np.zeros((B, nq, nk), dtype=np.uint8)
    for b in range(B):
        for qt in range(nq):
            for kt in range(nk):
                seen = exist = 0
                only_anchor = True
                for i in range(origin + qt * BM, origin + (qt + 1) * BM):
                    for j in range(origin + kt * BN, origin + (kt + 1) * BN):
                        if i >= S or j >= S:
                            continue
                        exist += 1
                        if anchor and (i == 0 or doc[b][i] == -1):
                            ok = j == 0
                        elif anchor and j == 0:
                            ok = True
                        else:
                            ok = doc[b][i] == doc[b][j] and (j <= i or not causal)
                        if ok:
                            seen += 1
                            if j != 0:
                                only_anchor = False
                if seen == 0:
                    continue
                if seen == exist == BM * BN:
                    out[b, qt, kt] = oracle.KIND_FULL
                elif anchor and origin + kt * BN == 0 and only_anchor:
                    out[b, qt, kt] = oracle.KIND_ANCHOR
                else:
                    out[b, qt, kt] = oracle.KIND_PARTIAL
    return out


@pytest.mark.parametrize("origin", [0, 1])
@pytest.mark.parametrize("case", range(6))
def test_plan_rows_and_columns_scalar_brute_force(case, origin):
    """tile_kinds_row, tile_kinds_col and tile_plan against element loops,
    with the tile grid at the row's first token or right after the anchor."""
    rng = np.random.default_rng(300 + case)
    anchor = case % 2 == 0
    causal = case != 5
    B = 2
    S = int(rng.integers(20, 90))
    BM, BN = [(16, 16), (32, 16), (16, 32)][case % 3]
    if anchor:
        rows = [W.random_partition(rng, S, 6) for _ in range(B)]
        if case == 0:
            rows[1] = [S - 1]
        cu = _cu(rows, S)
    else:
        rows = [W.random_partition(rng, S + 1, 6) for _ in range(B)]   # partitions of S tokens
        cu = W.cu_doc_lens_no_anchor(rows, S)
    ref = _brute_kinds(rows, S, BM, BN, causal, anchor, origin)
    nq, nk = ref.shape[1:]
    for b in range(B):
        for qt in range(nq):
            got = oracle.tile_kinds_row(cu, B, S, BM, BN, b, qt, causal, anchor, origin)
            assert np.array_equal(got, ref[b, qt]), (b, qt)
        for kt in range(nk):
            got = oracle.tile_kinds_col(cu, B, S, BM, BN, b, kt, causal, anchor, origin)
            assert np.array_equal(got, ref[b, :, kt]), (b, kt)
    p = oracle.tile_plan(cu, B, S, BM, BN, causal, anchor, origin)
    for b in range(B):
        for kt in range(nk):
            a, z = p["kptr"][b * nk + kt], p["kptr"][b * nk + kt + 1]
            live = np.nonzero(ref[b, :, kt])[0]
            assert list(p["qidx"][a:z]) == list(live)
            assert list(p["qkind"][a:z]) == list(ref[b, live, kt])


def test_tile_kinds_col_is_the_key_major_plan():
    """tile_kinds_col(b, kt) is column kt of the plan's key-major CSR, for
    ragged S, two rows, with and without the anchor, causal or not."""
    rng = np.random.default_rng(17)
    for S, BM, BN in [(333, 64, 32), (300, 32, 64), (129, 64, 64)]:
        for anchor in (True, False):
            for causal in (True, False):
                if anchor:
                    cu = _cu([W.random_partition(rng, S, 7) for _ in range(2)], S)
                else:
                    cu = W.cu_doc_lens_no_anchor([W.random_partition(rng, S + 1, 7)
                                                  for _ in range(2)], S)
                p = oracle.tile_plan(cu, 2, S, BM, BN, causal, anchor)
                nq, nk = p["nq"], p["nk"]
                for b in range(2):
                    for kt in range(nk):
                        col = oracle.tile_kinds_col(cu, 2, S, BM, BN, b, kt, causal, anchor)
                        a, z = p["kptr"][b * nk + kt], p["kptr"][b * nk + kt + 1]
                        assert list(np.nonzero(col)[0]) == list(p["qidx"][a:z])
                        assert list(col[np.nonzero(col)[0]]) == list(p["qkind"][a:z])
                        assert len(col) == nq


# ---------------------------------------------------------------- seeded workloads
APPENDIX = os.path.join(GOLDEN, "workload_partitions_and_tiles.json")


def test_workload_partitions_reproduce_the_recorded_ones():
    g = json.load(open(APPENDIX))
    for name, lens in g["partitions"].items():
        w = W.get(name)
        for r in w.doc_rows:
            assert list(r) == lens, name


def _tile_totals(name, BM, BN):
    w = W.get(name)
    p = oracle.tile_plan(w.cu_doc_lens, w.B, w.S, BM, BN)
    kk = p["kkind"]
    tot = [int((kk == oracle.KIND_FULL).sum()), int((kk == oracle.KIND_PARTIAL).sum()),
           int((kk == oracle.KIND_ANCHOR).sum())]
    # the key-major CSR holds the same tiles
    assert len(p["qidx"]) == len(kk) == p["qptr"][-1] == p["kptr"][-1]
    return w, tot


def _check_totals(name):
    g = json.load(open(APPENDIX))
    rec = g["tile_totals"][name]
    for shape, (F, P, A, eff) in rec.items():
        BM, BN = map(int, shape.split("x"))
        w, tot = _tile_totals(name, BM, BN)
        assert tot == [F, P, A], (name, shape, tot)
        pairs = sum(1 + sum(n * (n + 1) // 2 + n for n in r) for r in w.doc_rows)
        assert round(pairs / ((F + P) * BM * BN), 3) == eff, (name, shape)


@pytest.mark.parametrize("name", ["tiny", "8k"])
def test_plan_tile_totals_of_the_workloads(name):
    _check_totals(name)


@pytest.mark.slow
@pytest.mark.parametrize("name", ["short_docs", "64k"])
def test_plan_tile_totals_of_the_large_workloads(name):
    _check_totals(name)


@pytest.mark.parametrize("BM,BN", [(128, 64), (64, 128), (64, 64)])
def test_plan_after_the_anchor_aligned_documents_closed_form(BM, BN):
    """With the grid after the anchor, documents whose lengths are multiples
    of both tile sides start on tile edges: each one is its own causal block
    triangle (query tile i of a document sees its key tiles j with
    j*BN <= (i+1)*BM - 1, FULL when every key of j precedes every row of i),
    no tile is shared by two documents, and no tile holds the anchor."""
    L = max(BM, BN) * 2
    n_docs = 3
    S = 1 + n_docs * L
    cu = _cu([[L] * n_docs], S)
    p = oracle.tile_plan(cu, 1, S, BM, BN, origin=1)
    got = {}
    for qt in range(p["nq"]):
        for e in range(p["qptr"][qt], p["qptr"][qt + 1]):
            got[(qt, int(p["kidx"][e]))] = int(p["kkind"][e])
    want = {}
    for d in range(n_docs):
        q0, k0 = d * L // BM, d * L // BN
        for i in range(L // BM):
            for j in range((i + 1) * BM // BN + (1 if ((i + 1) * BM) % BN else 0)):
                if j * BN > (i + 1) * BM - 1:
                    continue
                full = (j + 1) * BN - 1 <= i * BM
                want[(q0 + i, k0 + j)] = oracle.KIND_FULL if full else oracle.KIND_PARTIAL
    assert got == want
    assert oracle.KIND_ANCHOR not in got.values()
