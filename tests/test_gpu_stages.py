"""GPU stages against the oracle: position IDs and tile plans bit-exact, the
RoPE stage within one bf16 ulp of round-to-nearest-even of the float64 rotation."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from _helpers import bf16_rne, bf16_ulp, f64, say

pytestmark = pytest.mark.gpu


def _partitions():
    rng = np.random.default_rng(77)
    cases = [
        ("tiny", 1, 256, [[80, 100, 75]]),
        ("one_doc_ragged", 1, 1000, [[999]]),
        ("len1_docs", 1, 300, [[1] * 299]),
        ("b2_random", 2, 777, [W.random_partition(rng, 777, 40) for _ in range(2)]),
        ("b2_mixed", 2, 513, [[1, 200, 1, 310], [512]]),
        ("s2", 3, 2, [[1], [1], [1]]),
        ("s1", 2, 1, [[], []]),
    ]
    w8 = W.get("8k")
    cases.append(("8k", 1, w8.S, [list(r) for r in w8.doc_rows]))
    return cases


@pytest.mark.parametrize("case", _partitions(), ids=lambda c: c[0])
def test_position_ids_bit_exact(gpu_lib, case):
    name, B, S, rows = case
    say(f"[positions] {name} B={B} S={S}")
    cu = W.cu_doc_lens_from_lengths(rows, S)
    for mode, label in ((0, "reset"), (1, "continuous")):
        pos, ws = gpu_lib.anchor_attn_position_ids(cu, B, S, mode)
        ref = oracle.position_ids(cu, B, S, label)
        assert np.array_equal(pos.cpu().numpy().astype(np.int64), ref)
        assert gpu_lib.anchor_attn_device_status(ws) == 0


@pytest.mark.parametrize("case", _partitions(), ids=lambda c: c[0])
def test_position_ids_bit_exact_without_anchor(gpu_lib, case):
    name, B, S, rows = case
    say(f"[positions] {name} without anchor B={B} S={S}")
    cu = W.cu_doc_lens_no_anchor(W.rows_without_anchor(rows), S)
    for flags, label in ((2, "reset"), (3, "continuous")):
        pos, ws = gpu_lib.anchor_attn_position_ids(cu, B, S, flags)
        ref = oracle.position_ids(cu, B, S, label, anchor=False)
        assert np.array_equal(pos.cpu().numpy().astype(np.int64), ref)
        assert gpu_lib.anchor_attn_device_status(ws) == 0


def test_segment_crossing_rows_is_reported_without_anchor(gpu_lib):
    S = 100
    bad = np.array([0, 60, 130, 200], dtype=np.int32)        # [60, 130) crosses into row 1
    pos, ws = gpu_lib.anchor_attn_position_ids(bad, 2, S, 2)
    assert gpu_lib.anchor_attn_device_status(ws) == gpu_lib.AA_EDOCS
    assert int(pos.min()) >= 0 and int(pos.max()) < S + 1    # clamped into the row


def _cmp_plan(gp, ref, B):
    qptr = gp["qptr"].cpu().numpy()
    n = int(gp["n_live"].cpu().item())
    assert n == len(ref["kidx"]) == qptr[-1]
    assert np.array_equal(qptr, ref["qptr"])
    assert np.array_equal(gp["kidx"][:n].cpu().numpy(), ref["kidx"])
    assert np.array_equal(gp["kkind"][:n].cpu().numpy(), ref["kkind"])
    assert np.array_equal(gp["kptr"].cpu().numpy(), ref["kptr"])
    assert np.array_equal(gp["qidx"][:n].cpu().numpy(), ref["qidx"])
    assert np.array_equal(gp["qkind"][:n].cpu().numpy(), ref["qkind"])


GRID = 16   # FLAG_GRID_AFTER_ANCHOR: the grid the attention kernels use for rows with an anchor


@pytest.mark.parametrize("tile", [(64, 64), (128, 64), (64, 128), (128, 128), (32, 16)])
@pytest.mark.parametrize("case", _partitions()[:-1], ids=lambda c: c[0])
def test_tile_plan_bit_exact_small(gpu_lib, case, tile):
    name, B, S, rows = case
    BM, BN = tile
    say(f"[plan] {name} B={B} S={S} tile={BM}x{BN}")
    cu = W.cu_doc_lens_from_lengths(rows, S)
    for causal in (True, False):
        for origin in (0, 1):
            gp = gpu_lib.anchor_attn_tile_plan(cu, B, S, BM, BN, causal, flags=GRID if origin else 0)
            ref = oracle.tile_plan(cu, B, S, BM, BN, causal, origin=origin)
            _cmp_plan(gp, ref, B)
    cu_na = W.cu_doc_lens_no_anchor(W.rows_without_anchor(rows), S)
    for causal in (True, False):
        gp = gpu_lib.anchor_attn_tile_plan(cu_na, B, S, BM, BN, causal, flags=gpu_lib.FLAG_NO_ANCHOR)
        ref = oracle.tile_plan(cu_na, B, S, BM, BN, causal, anchor=False)
        _cmp_plan(gp, ref, B)


def test_tile_plan_bit_exact_8k_all_tiles(gpu_lib):
    w = W.get("8k")
    for BM, BN in ((128, 64), (64, 128), (128, 128)):
        for origin in (0, 1):
            say(f"[plan] 8k tile={BM}x{BN} origin={origin}")
            gp = gpu_lib.anchor_attn_tile_plan(w.cu_doc_lens, w.B, w.S, BM, BN,
                                               flags=GRID if origin else 0)
            ref = oracle.tile_plan(w.cu_doc_lens, w.B, w.S, BM, BN, origin=origin)
            _cmp_plan(gp, ref, w.B)


def _rows_of(gp, bq, key="q"):
    if key == "q":
        a, b = gp["qptr"][bq:bq + 2].tolist()
        return gp["kidx"][a:b].cpu().numpy(), gp["kkind"][a:b].cpu().numpy()
    a, b = gp["kptr"][bq:bq + 2].tolist()
    return gp["qidx"][a:b].cpu().numpy(), gp["qkind"][a:b].cpu().numpy()


def _kind_totals(gp):
    n = int(gp["n_live"].cpu().item())
    kk = gp["kkind"][:n].cpu().numpy()
    return [int((kk == 1).sum()), int((kk == 2).sum()), int((kk == 3).sum())]


# F/P/A totals of the 128 x 64 plans of the workloads, recorded independently
# of this repository when the workloads were specified
# (tests/golden/workload_partitions_and_tiles.json)
def _recorded_totals(wname):
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                    "workload_partitions_and_tiles.json")))
    return g["tile_totals"].get(wname, {})


@pytest.mark.parametrize("origin", [0, 1], ids=["grid_first_token", "grid_after_anchor"])
@pytest.mark.parametrize("wname", ["64k", "short_docs"])
def test_tile_plan_bit_exact_full_size_whole(gpu_lib, wname, origin):
    """Whole full-size plans in the kernels' tile shapes (forward and dQ:
    128 x 64 query-major; dK/dV: 64 x 128 key-major), both grids, every entry
    against the brute force; the kind totals of the 128 x 64 plan from the
    row's first token also against the recorded ones."""
    w = W.get(wname)
    cu = w.cu_doc_lens
    for BM, BN in ((128, 64), (64, 128)):
        say(f"[plan] {wname} tile={BM}x{BN} origin={origin}: GPU plan")
        gp = gpu_lib.anchor_attn_tile_plan(cu, w.B, w.S, BM, BN, flags=GRID if origin else 0)
        say(f"[plan] {wname} tile={BM}x{BN} origin={origin}: oracle plan")
        ref = oracle.tile_plan(cu, w.B, w.S, BM, BN, origin=origin)
        _cmp_plan(gp, ref, w.B)
        rec = _recorded_totals(wname).get(f"{BM}x{BN}") if origin == 0 else None
        say(f"[plan] {wname} tile={BM}x{BN} origin={origin}: F/P/A {_kind_totals(gp)} (recorded {rec})")
        if rec:
            assert _kind_totals(gp) == rec[:3]


def test_tile_plan_full_size_128k_sampled(gpu_lib):
    """128K GQA: sampled query tiles (query major) and key tiles (key major)
    of the kernels' plans against the brute force, and the kind totals of the
    128 x 64 plan from the row's first token."""
    w = W.get("128k_gqa")
    cu = w.cu_doc_lens
    rng = np.random.default_rng(5)
    gp0 = gpu_lib.anchor_attn_tile_plan(cu, w.B, w.S, 128, 64)
    assert _kind_totals(gp0) == [391396, 3733, 653]
    for BM, BN in ((128, 64), (64, 128)):
        say(f"[plan] 128k_gqa tile={BM}x{BN}")
        gp = gpu_lib.anchor_attn_tile_plan(cu, w.B, w.S, BM, BN, flags=GRID)
        nq, nk = gp["nq"], gp["nk"]
        for b in range(w.B):
            for qt in sorted(set([0, 1, nq - 1] + list(rng.integers(0, nq, 6)))):
                ref = oracle.tile_kinds_row(cu, w.B, w.S, BM, BN, b, int(qt), origin=1)
                idx, kind = _rows_of(gp, b * nq + int(qt), "q")
                assert np.array_equal(idx, np.nonzero(ref)[0])
                assert np.array_equal(kind, ref[ref != 0])
            for kt in sorted(set([0, 1, nk - 1] + list(rng.integers(0, nk, 4)))):
                ref = oracle.tile_kinds_col(cu, w.B, w.S, BM, BN, b, int(kt), origin=1)
                idx, kind = _rows_of(gp, b * nk + int(kt), "k")
                assert np.array_equal(idx, np.nonzero(ref)[0])
                assert np.array_equal(kind, ref[ref != 0])


@pytest.mark.parametrize("wname", ["tiny", "8k", "64k", "128k_gqa"])
def test_rope_stage_within_one_ulp(gpu_lib, wname):
    w = W.get(wname)
    S = w.S
    say(f"[rope] {wname}")
    g = torch.Generator("cpu").manual_seed(55)
    ntok = min(S, 4096)
    x = torch.randn((1, S, 4, w.D), generator=g).to(torch.bfloat16)
    pos = oracle.position_ids(w.cu_doc_lens[: 2 + len(w.doc_rows[0])], 1, S)
    y = gpu_lib.anchor_attn_rope(x.cuda(), torch.from_numpy(pos.astype(np.int32)), w.rope_base).cpu()
    toks = np.unique(np.concatenate([np.arange(min(S, 64)), np.random.default_rng(1).integers(0, S, ntok)]))
    ref = oracle.rope(f64(x[0, toks]), pos[toks], w.rope_base)          # float64 [n, 4, D]
    want = bf16_rne(ref)
    got = f64(y[0, toks])
    diff = np.abs(got - want)
    ulp = bf16_ulp(want)
    # The rotation runs in float32: besides the final bf16 rounding (one ulp
    # at a near tie), x0*c - x1*s carries float32 rounding of the products,
    # which near cancellation is large next to the result itself.
    xin = f64(x[0, toks])
    pair_mag = np.repeat(np.abs(xin[..., 0::2]) + np.abs(xin[..., 1::2]), 2, axis=-1)
    bound = ulp + 2.0 ** -22 * pair_mag
    assert np.all(diff <= bound), float((diff / bound).max())
    # A result differs from RNE(float64) only when the float32 value and the
    # exact one straddle a bf16 rounding midpoint.  With the float32 error at
    # most delta = 2^-23 (|x0| + |x1|) (cos/sin, the products and the sum each
    # rounded once), that happens with probability at most delta / ulp for a
    # result placed uniformly in its ulp; the mean over the elements is the
    # expected mismatch rate, an upper bound on the measured one.
    pred = float(np.minimum(1.0, 2.0 ** -23 * pair_mag / ulp).mean())
    rate = float((diff > 0).mean())
    say(f"[rope] {wname} mismatch rate {rate:.2e} (bound-derived expectation {pred:.2e})")
    assert rate <= pred
    # the anchor (position 0) is unchanged: R_0 = I
    assert torch.equal(y[0, 0], x[0, 0])


def test_device_status_flags_bad_documents(gpu_lib):
    S = 64
    bad = np.array([0, 10, 64], dtype=np.int32)            # no one-token anchor segment
    pos, ws = gpu_lib.anchor_attn_position_ids(bad, 1, S)
    assert gpu_lib.anchor_attn_device_status(ws) == gpu_lib.AA_EDOCS
    q = torch.randn((1, S, 2, 64)).to(torch.bfloat16).cuda()
    # a host copy is refused by the binding before any launch ...
    with pytest.raises(ValueError, match="anchor"):
        gpu_lib.anchor_attn_fwd(q, q, q, bad, 1e4)
    # ... a device copy reaches the kernels, which flag it and NaN-fill the outputs
    o, lse = gpu_lib.anchor_attn_fwd(q, q, q, torch.from_numpy(bad).cuda(), 1e4)
    assert torch.isnan(o.float()).all() and torch.isnan(lse).all()


def _expected_order(cnt):
    """The work-order rule written out: longest processing time first (stable,
    by descending count) when the largest count exceeds 1.5x the mean, else
    the natural order; heads interleaved for at most 128 tiles or even work;
    more than 16384 tiles keep the natural order with no flags."""
    n = len(cnt)
    if n > 16384:
        return np.arange(n), 0
    lpt = 2 * int(cnt.max()) * n > 3 * int(cnt.sum())
    order = np.argsort(-cnt, kind="stable") if lpt else np.arange(n)
    inter = n <= 128 or not lpt
    return order, (1 if lpt else 0) | (2 if inter else 0)


@pytest.mark.parametrize("case", ["skewed", "even", "ties", "one", "small_skewed", "beyond_limit"])
def test_tile_order(gpu_lib, case):
    """The work order is unique given the counts: bit-exact against the rule."""
    rng = np.random.default_rng(sum(map(ord, case)))
    cnt = {
        "skewed": lambda: rng.integers(1, 400, 3000) ** 2 // 400 + 1,
        "even": lambda: rng.integers(5, 7, 2048),
        "ties": lambda: rng.integers(0, 4, 5000) * 50 + 1,
        "one": lambda: np.array([7]),
        "small_skewed": lambda: np.concatenate([np.full(60, 1), np.array([90, 3, 2])]),
        "beyond_limit": lambda: rng.integers(1, 50, 16385),
    }[case]().astype(np.int32)
    got = gpu_lib.anchor_attn_tile_order(torch.from_numpy(cnt).cuda()).cpu().numpy()
    order, flags = _expected_order(cnt)
    say(f"[order] {case}: n={len(cnt)} flags={got[-1]}")
    assert np.array_equal(got[:-1], order) and got[-1] == flags


@pytest.mark.parametrize("wname", ["8k", "64k", "short_docs"])
def test_tile_order_of_workload_plans(gpu_lib, wname):
    """The order the kernels use for the benchmark workloads: from the live-tile
    counts of the forward's query-major plan (128 x 64 tiles)."""
    w = W.get(wname)
    plan = gpu_lib.anchor_attn_tile_plan(w.cu_doc_lens, w.B, w.S, 128, 64, flags=GRID)
    qptr = plan["qptr"].cpu().numpy().astype(np.int64)
    cnt = np.diff(qptr).astype(np.int32)
    got = gpu_lib.anchor_attn_tile_order(torch.from_numpy(cnt).cuda()).cpu().numpy()
    order, flags = _expected_order(cnt)
    say(f"[order] {wname}: flags={got[-1]} (LPT {bool(got[-1] & 1)}, interleave {bool(got[-1] & 2)})")
    assert np.array_equal(got[:-1], order) and got[-1] == flags
