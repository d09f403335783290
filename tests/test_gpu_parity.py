"""Forward and backward through the C ABI against the float64 oracle.

Bars: max|O - O_ref| <= 4e-3 max|O_ref|; dq, dk, dv within 1e-2 relative
Frobenius error; LSE within 5e-2 absolute (bf16 rounding of the rotated q, k
moves a logit by ~4e-3 per standard deviation, see the design notes).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from _helpers import f64, o_err, rel_frob, say

pytestmark = pytest.mark.gpu

O_TOL, G_TOL, LSE_TOL = 4e-3, 1e-2, 5e-2


def _small_cases():
    rng = np.random.default_rng(2024)
    return [
        # name, B, S, Hq, Hkv, D, rows, base, causal
        ("tiny", 1, 256, 2, 2, 64, [[80, 100, 75]], 1e4, True),
        ("ragged_gqa_d128", 2, 1000, 4, 2, 128, [W.random_partition(rng, 1000, 30) for _ in range(2)], 5e6, True),
        ("one_doc_d64", 1, 777, 2, 2, 64, [[776]], 1e4, True),
        ("len1_docs", 1, 513, 2, 1, 128, [[1] * 512], 5e6, True),
        ("mixed_b2", 2, 640, 2, 2, 128, [[1, 300, 1, 337], [639]], 5e5, True),
        ("noncausal", 1, 600, 2, 2, 128, [[100, 1, 250, 248]], 1e4, False),
        ("s2", 2, 2, 2, 2, 64, [[1], [1]], 1e4, True),
        ("gqa8", 1, 300, 8, 1, 64, [[150, 149]], 1e4, True),
        ("b4_mqa_d128", 4, 333, 4, 1, 128, [[332], [1] * 332, [100, 232], [64, 64, 64, 64, 76]], 5e6, True),
    ]


def _inputs(B, S, Hq, Hkv, D, seed):
    q, k, v, do = W.make_tensors(B, S, Hq, Hkv, D, seed)
    return q, k, v, do


@pytest.mark.parametrize("grid", [0, 16], ids=["grid_first_token", "grid_after_anchor"])
@pytest.mark.parametrize("case", _small_cases(), ids=lambda c: c[0])
def test_fwd_bwd_small_full_compare(gpu_lib, case, grid):
    """Both tile grids (from the row's first token; after the anchor,
    FLAG_GRID_AFTER_ANCHOR) against the oracle in full."""
    name, B, S, Hq, Hkv, D, rows, base, causal = case
    say(f"[parity] {name} B={B} S={S} Hq={Hq} Hkv={Hkv} D={D} causal={causal} grid={grid}")
    cu = W.cu_doc_lens_from_lengths(rows, S)
    q, k, v, do = _inputs(B, S, Hq, Hkv, D, 1234)
    o, lse = gpu_lib.anchor_attn_fwd(q.cuda(), k.cuda(), v.cuda(), cu, base, causal, flags=grid)
    o_ref, lse_ref, _, _ = oracle.forward(q, k, v, cu, base, causal)
    o_g = f64(o).reshape(B * S, Hq, D)
    say(f"[parity] {name} O err {o_err(o_g, o_ref):.2e}")
    assert o_err(o_g, o_ref) <= O_TOL, o_err(o_g, o_ref)
    lse_g = f64(lse).transpose(1, 0, 2).reshape(Hq, B * S)
    assert np.abs(lse_g - lse_ref).max() <= LSE_TOL
    dq, dk, dv = gpu_lib.anchor_attn_bwd(q.cuda(), k.cuda(), v.cuda(), o, lse, do.cuda(), cu, base, causal,
                                         flags=grid)
    dq_r, dk_r, dv_r, _, _ = oracle.backward(q, k, v, do, cu, base, causal)
    e = (rel_frob(f64(dq).reshape(B * S, Hq, D), dq_r), rel_frob(f64(dk).reshape(B * S, Hkv, D), dk_r),
         rel_frob(f64(dv).reshape(B * S, Hkv, D), dv_r))
    say(f"[parity] {name} O {o_err(o_g, o_ref):.2e} dq {e[0]:.2e} dk {e[1]:.2e} dv {e[2]:.2e}")
    assert max(e) <= G_TOL, e


def _mode_cases():
    rng = np.random.default_rng(2025)
    NA, CP, GR = 2, 1, 16     # FLAG_NO_ANCHOR, FLAG_CONTINUOUS_POS, FLAG_GRID_AFTER_ANCHOR
    return [
        # name, B, S, Hq, Hkv, D, rows, base, causal, flags (rows cover S without an anchor)
        ("noanchor_reset_gqa", 2, 1000, 4, 2, 128, [W.random_partition(rng, 1001, 30) for _ in range(2)], 5e6, True, NA),
        ("noanchor_continuous", 1, 777, 2, 2, 64, [[100, 1, 676]], 1e4, True, NA | CP),
        ("noanchor_one_doc", 1, 513, 2, 1, 128, [[513]], 5e6, True, NA),      # plain causal attention
        ("noanchor_len1", 1, 300, 2, 2, 64, [[1] * 300], 1e4, True, NA),
        ("noanchor_noncausal", 1, 600, 2, 2, 128, [[101, 1, 250, 248]], 1e4, False, NA),
        ("noanchor_s1", 2, 1, 2, 2, 64, [[1], [1]], 1e4, True, NA),
        ("anchor_continuous", 2, 1000, 4, 2, 128, [W.random_partition(rng, 1000, 30) for _ in range(2)], 5e6, True, CP),
        ("anchor_continuous_mixed", 2, 640, 2, 2, 128, [[1, 300, 1, 337], [639]], 5e5, True, CP),
        ("anchor_continuous_grid_after", 2, 700, 4, 2, 64, [[128] * 5 + [59], [699]], 1e4, True, CP | GR),
        ("noncausal_grid_after", 1, 600, 2, 2, 128, [[100, 1, 250, 248]], 1e4, False, GR),
        ("anchor_only_s1", 2, 1, 2, 2, 64, [[], []], 1e4, True, 0),           # rows of the anchor alone
        ("anchor_only_s1_grid_after", 2, 1, 2, 2, 128, [[], []], 1e4, True, GR),
    ]


@pytest.mark.parametrize("case", _mode_cases(), ids=lambda c: c[0])
def test_fwd_bwd_modes_full_compare(gpu_lib, case):
    """The pages' other paradigms through the same kernels (options of the
    *_ex entry points) against the oracle's matching modes."""
    name, B, S, Hq, Hkv, D, rows, base, causal, flags = case
    anchor = not flags & 2
    mode = "continuous" if flags & 1 else "reset"
    say(f"[modes] {name} B={B} S={S} Hq={Hq} Hkv={Hkv} D={D} causal={causal} flags={flags}")
    cu = W.cu_doc_lens_from_lengths(rows, S) if anchor else W.cu_doc_lens_no_anchor(rows, S)
    q, k, v, do = _inputs(B, S, Hq, Hkv, D, 4321)
    o, lse = gpu_lib.anchor_attn_fwd(q.cuda(), k.cuda(), v.cuda(), cu, base, causal, flags=flags)
    o_ref, lse_ref, _, _ = oracle.forward(q, k, v, cu, base, causal, pos_mode=mode, anchor=anchor)
    o_g = f64(o).reshape(B * S, Hq, D)
    assert o_err(o_g, o_ref) <= O_TOL, o_err(o_g, o_ref)
    lse_g = f64(lse).transpose(1, 0, 2).reshape(Hq, B * S)
    assert np.abs(lse_g - lse_ref).max() <= LSE_TOL
    dq, dk, dv = gpu_lib.anchor_attn_bwd(q.cuda(), k.cuda(), v.cuda(), o, lse, do.cuda(), cu, base,
                                         causal, flags=flags)
    dq_r, dk_r, dv_r, _, _ = oracle.backward(q, k, v, do, cu, base, causal, pos_mode=mode, anchor=anchor)
    g = (f64(dq).reshape(B * S, Hq, D), f64(dk).reshape(B * S, Hkv, D), f64(dv).reshape(B * S, Hkv, D))
    if all(len(r) == r.count(1) for r in rows):
        # Every query sees only itself: P = 1, so dS = dP - Dv = 0 and the
        # exact dq, dk vanish.  A relative error is undefined there; the GPU's
        # result must be rounding noise next to the O(1) entries of dv = dO.
        assert np.abs(dq_r).max() < 1e-12 and np.abs(dk_r).max() < 1e-12
        noise = max(np.abs(g[0]).max(), np.abs(g[1]).max())
        say(f"[modes] {name} O {o_err(o_g, o_ref):.2e} |dq|,|dk| max {noise:.2e} dv {rel_frob(g[2], dv_r):.2e}")
        assert noise <= 1e-3 and rel_frob(g[2], dv_r) <= G_TOL
        return
    e = (rel_frob(g[0], dq_r), rel_frob(g[1], dk_r), rel_frob(g[2], dv_r))
    say(f"[modes] {name} O {o_err(o_g, o_ref):.2e} dq {e[0]:.2e} dk {e[1]:.2e} dv {e[2]:.2e}")
    assert max(e) <= G_TOL, e


@pytest.mark.parametrize("case", [
    ("ragged_gqa_d128", 2, 1000, 4, 2, 128, None, 5e6, True),
    ("heads16_d64", 1, 1500, 16, 4, 64, [[900, 20, 579]], 1e4, True),
    ("noncausal", 1, 600, 2, 2, 128, [[100, 1, 250, 248]], 1e4, False),
], ids=lambda c: c[0])
def test_fp32_output(gpu_lib, case):
    """FLAG_O_FP32: the forward writes O in float32 (the bf16 output is exactly
    its round-to-nearest-even), the LSE is unchanged, and the backward takes
    the float32 O; both against the oracle."""
    name, B, S, Hq, Hkv, D, rows, base, causal = case
    if rows is None:
        rng = np.random.default_rng(2024)
        rows = [W.random_partition(rng, S, 30) for _ in range(B)]
    cu = W.cu_doc_lens_from_lengths(rows, S)
    q, k, v, do = _inputs(B, S, Hq, Hkv, D, 1234)
    qc, kc, vc, doc = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    f32 = gpu_lib.FLAG_O_FP32
    o32, lse32 = gpu_lib.anchor_attn_fwd(qc, kc, vc, cu, base, causal, flags=f32)
    o16, lse16 = gpu_lib.anchor_attn_fwd(qc, kc, vc, cu, base, causal)
    assert o32.dtype == torch.float32 and o16.dtype == torch.bfloat16
    assert torch.equal(o32.to(torch.bfloat16), o16) and torch.equal(lse32, lse16)
    o_ref, lse_ref, _, _ = oracle.forward(q, k, v, cu, base, causal)
    e32 = o_err(f64(o32).reshape(B * S, Hq, D), o_ref)
    e16 = o_err(f64(o16).reshape(B * S, Hq, D), o_ref)
    dq, dk, dv = gpu_lib.anchor_attn_bwd(qc, kc, vc, o32, lse32, doc, cu, base, causal, flags=f32)
    dq_r, dk_r, dv_r, _, _ = oracle.backward(q, k, v, do, cu, base, causal)
    e = (rel_frob(f64(dq).reshape(B * S, Hq, D), dq_r), rel_frob(f64(dk).reshape(B * S, Hkv, D), dk_r),
         rel_frob(f64(dv).reshape(B * S, Hkv, D), dv_r))
    say(f"[fp32-o] {name} O err fp32 {e32:.2e} (bf16 output {e16:.2e}) dq {e[0]:.2e} dk {e[1]:.2e} "
        f"dv {e[2]:.2e}")
    assert e32 <= O_TOL and max(e) <= G_TOL
    # The bf16 output is the float32 one rounded to nearest even: the rounding
    # moves an entry by at most 2^-9 of its size, so its error is bounded by
    # the float32 error plus 2^-9 max|O| (max|O| within e32 of max|O_ref|).
    assert e16 <= e32 + 2.0 ** -9 * (1.0 + e32), (e16, e32)


def test_interleaved_heads_bit_identical(gpu_lib):
    """16 query heads over few tiles: the work order walks an XCD's slice rank-
    major across its two heads.  Each (head, tile) item is computed the same
    way whatever the order, so the 16-head call must equal, bit for bit, two
    8-head calls on the head halves (one head per slice), forward and backward."""
    B, S, Hq, Hkv, D, base = 1, 1500, 16, 4, 64, 1e4
    cu = W.cu_doc_lens_from_lengths([[900, 20, 579]], S)
    q, k, v, do = (t.cuda() for t in W.make_tensors(B, S, Hq, Hkv, D, 1234))
    o, lse = gpu_lib.anchor_attn_fwd(q, k, v, cu, base)
    dq, dk, dv = gpu_lib.anchor_attn_bwd(q, k, v, o, lse, do, cu, base)
    g = Hq // Hkv
    for half in range(2):
        hs, ks = slice(8 * half, 8 * half + 8), slice(8 * half // g, (8 * half + 8) // g)
        qh, kh, vh, doh = (t[:, :, sl].contiguous() for t, sl in ((q, hs), (k, ks), (v, ks), (do, hs)))
        oh, lseh = gpu_lib.anchor_attn_fwd(qh, kh, vh, cu, base)
        dqh, dkh, dvh = gpu_lib.anchor_attn_bwd(qh, kh, vh, oh, lseh, doh, cu, base)
        say(f"[interleave] heads {hs.start}-{hs.stop - 1} vs the 16-head call")
        assert torch.equal(oh, o[:, :, hs]) and torch.equal(lseh, lse[:, hs])
        assert torch.equal(dqh, dq[:, :, hs])
        assert torch.equal(dkh, dk[:, :, ks]) and torch.equal(dvh, dv[:, :, ks])


def test_determinism(gpu_lib):
    B, S, Hq, Hkv, D = 2, 1000, 4, 2, 128
    rng = np.random.default_rng(3)
    cu = W.cu_doc_lens_from_lengths([W.random_partition(rng, S, 20) for _ in range(B)], S)
    q, k, v, do = (t.cuda() for t in _inputs(B, S, Hq, Hkv, D, 99))
    o1, l1 = gpu_lib.anchor_attn_fwd(q, k, v, cu, 5e6)
    o2, l2 = gpu_lib.anchor_attn_fwd(q, k, v, cu, 5e6)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    g1 = gpu_lib.anchor_attn_bwd(q, k, v, o1, l1, do, cu, 5e6)
    g2 = gpu_lib.anchor_attn_bwd(q, k, v, o1, l1, do, cu, 5e6)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


@pytest.mark.parametrize("flags", [0, 2, 16], ids=["anchor", "no_anchor", "anchor_grid_after"])
def test_backward_reusing_the_forward_workspace(gpu_lib, flags):
    """AA_FLAG_FWD_WORKSPACE: the backward on the forward's workspace gives
    bit-identical gradients to a self-contained backward."""
    B, S, Hq, Hkv, D = 2, 1000, 4, 2, 128
    rng = np.random.default_rng(31)
    anchor = not flags & 2
    rows = [W.random_partition(rng, S if anchor else S + 1, 20) for _ in range(B)]
    cu = W.cu_doc_lens_from_lengths(rows, S) if anchor else W.cu_doc_lens_no_anchor(rows, S)
    q, k, v, do = (t.cuda() for t in _inputs(B, S, Hq, Hkv, D, 55))
    ws = torch.empty(gpu_lib.workspace_size(B, S, Hq, Hkv, D, True), dtype=torch.uint8, device="cuda")
    o, lse = gpu_lib.anchor_attn_fwd(q, k, v, cu, 5e6, workspace=ws, flags=flags)
    g_reuse = gpu_lib.anchor_attn_bwd(q, k, v, o, lse, do, cu, 5e6, workspace=ws,
                                      flags=flags | gpu_lib.FLAG_FWD_WORKSPACE)
    g_self = gpu_lib.anchor_attn_bwd(q, k, v, o, lse, do, cu, 5e6, flags=flags)
    for a, b in zip(g_reuse, g_self):
        assert torch.equal(a, b)


def test_autograd_backward_twice_with_retained_graph(gpu_lib):
    """A second backward through a retained graph reuses the forward's
    workspace kept by the autograd context: both give the same gradients, and
    they match the direct backward."""
    B, S, Hq, Hkv, D = 1, 600, 4, 2, 128
    cu = W.cu_doc_lens_from_lengths([[250, 1, 348]], S)
    q, k, v, do = _inputs(B, S, Hq, Hkv, D, 21)
    qc, kc, vc = (t.cuda().requires_grad_(True) for t in (q, k, v))
    o = gpu_lib.anchor_attention(qc, kc, vc, cu, 5e6)
    o.backward(do.cuda(), retain_graph=True)
    g1 = [t.grad.clone() for t in (qc, kc, vc)]
    for t in (qc, kc, vc):
        t.grad = None
    o.backward(do.cuda())
    g2 = [t.grad for t in (qc, kc, vc)]
    grid = gpu_lib.grid_flag(cu, B, S)      # the autograd path's choice of tile grid
    o2, lse2 = gpu_lib.anchor_attn_fwd(q.cuda(), k.cuda(), v.cuda(), cu, 5e6, flags=grid)
    g3 = gpu_lib.anchor_attn_bwd(q.cuda(), k.cuda(), v.cuda(), o2, lse2, do.cuda(), cu, 5e6,
                                 flags=grid)
    for a, b, c in zip(g1, g2, g3):
        assert torch.equal(a, b) and torch.equal(a, c)


def test_autograd_function(gpu_lib):
    B, S, Hq, Hkv, D = 1, 400, 2, 2, 64
    cu = W.cu_doc_lens_from_lengths([[199, 200]], S)
    q, k, v, do = _inputs(B, S, Hq, Hkv, D, 7)
    qc, kc, vc = (t.cuda().requires_grad_(True) for t in (q, k, v))
    o = gpu_lib.anchor_attention(qc, kc, vc, cu, 1e4)
    o.backward(do.cuda())
    dq_r, dk_r, dv_r, _, _ = oracle.backward(q, k, v, do, cu, 1e4)
    assert rel_frob(f64(qc.grad).reshape(B * S, Hq, D), dq_r) <= G_TOL
    assert rel_frob(f64(kc.grad).reshape(B * S, Hkv, D), dk_r) <= G_TOL
    assert rel_frob(f64(vc.grad).reshape(B * S, Hkv, D), dv_r) <= G_TOL


def _sample_rows(w, rng, n):
    """Query rows to check: anchors, document starts and ends, random rows."""
    S = w.S
    rows = set()
    for b in range(w.B):
        rows.add(b * S)
        rows.update(int(b * S + x) for x in rng.integers(0, S, n))
        cu = w.cu_doc_lens
        for c in cu[1:]:
            if b * S < c < (b + 1) * S:
                rows.add(int(c)); rows.add(int(c) - 1)
    return np.array(sorted(rows))[: 3 * n]


def _sample_keys(w, rng, n, max_doc=2500):
    """Keys in documents short enough for the oracle to sum over (the anchor
    key, which every query of the row sees, is checked at 8K on its own)."""
    cu = w.cu_doc_lens
    keys = set()
    for s, e in zip(cu[:-1], cu[1:]):
        if e - s <= max_doc and e - s > 1:
            keys.update(int(x) for x in rng.integers(s, e, 3))
            keys.add(int(s)); keys.add(int(e) - 1)
    keys = sorted(keys)
    pick = rng.choice(len(keys), size=min(n, len(keys)), replace=False)
    return np.array(sorted(keys[i] for i in pick))


@pytest.mark.parametrize("wname", ["8k", "64k", "128k_gqa", "short_docs", "64k_ulysses8"])
def test_full_size_sampled(gpu_lib, wname):
    """The benchmark's shapes and launch configuration; sampled outputs."""
    w = W.get(wname)
    B, S, Hq, Hkv, D = w.B, w.S, w.Hq, w.Hkv, w.D
    say(f"[full] {wname} generating inputs")
    q, k, v, do = W.make_tensors(B, S, Hq, Hkv, D, w.tensor_seed)
    cu = w.cu_doc_lens
    qc, kc, vc, doc = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    grid = gpu_lib.grid_flag(cu, B, S)          # the benchmark's choice of tile grid
    say(f"[full] {wname} fwd+bwd on GPU (grid flag {grid})")
    o, lse = gpu_lib.anchor_attn_fwd(qc, kc, vc, cu, w.rope_base, flags=grid)
    dq, dk, dv = gpu_lib.anchor_attn_bwd(qc, kc, vc, o, lse, doc, cu, w.rope_base, flags=grid)
    torch.cuda.synchronize()
    assert not torch.isnan(o.float()).any()
    rng = np.random.default_rng(11)
    heads = [0, Hq - 1] if Hq == Hkv else list(range(Hq // Hkv))     # GQA: all of kv group 0
    rows = _sample_rows(w, rng, 48)
    say(f"[full] {wname} oracle forward on {len(rows)} rows x {len(heads)} heads")
    o_ref, lse_ref, _, _ = oracle.forward(q, k, v, cu, w.rope_base, heads=heads, rows=rows)
    o_g = f64(o).reshape(B * S, Hq, D)[rows][:, heads]
    lse_g = f64(lse).transpose(1, 0, 2).reshape(Hq, B * S)[heads][:, rows]
    say(f"[full] {wname} O err {o_err(o_g, o_ref):.2e} lse err {np.abs(lse_g - lse_ref).max():.2e}")
    assert o_err(o_g, o_ref) <= O_TOL
    assert np.abs(lse_g - lse_ref).max() <= LSE_TOL
    keys = _sample_keys(w, rng, 24)
    say(f"[full] {wname} oracle backward on {len(rows)} rows, {len(keys)} keys")
    dq_r, dk_r, dv_r, _, _ = oracle.backward(q, k, v, do, cu, w.rope_base, heads=heads,
                                             q_rows=rows, k_cols=keys)
    dq_g = f64(dq).reshape(B * S, Hq, D)[rows][:, heads]
    g = heads[0] * Hkv // Hq
    dk_g = f64(dk).reshape(B * S, Hkv, D)[keys][:, [g]]
    dv_g = f64(dv).reshape(B * S, Hkv, D)[keys][:, [g]]
    if Hq == Hkv:
        # key gradients from a subset of heads only cover those heads: compare per head
        e_dk = max(rel_frob(f64(dk).reshape(B * S, Hkv, D)[keys][:, [h]], dk_r[:, [h]]) for h in heads)
        e_dv = max(rel_frob(f64(dv).reshape(B * S, Hkv, D)[keys][:, [h]], dv_r[:, [h]]) for h in heads)
    else:
        e_dk = rel_frob(dk_g, dk_r[:, [g]])
        e_dv = rel_frob(dv_g, dv_r[:, [g]])
    e_dq = rel_frob(dq_g, dq_r)
    say(f"[full] {wname} dq {e_dq:.2e} dk {e_dk:.2e} dv {e_dv:.2e}")
    assert max(e_dq, e_dk, e_dv) <= G_TOL


@pytest.mark.parametrize("seed,median,sigma,D", [(31, 256, 1.3, 128), (32, 1024, 1.2, 128),
                                                 (33, 3000, 1.0, 128), (34, 700, 1.2, 64)],
                         ids=["median256", "median1024", "median3000", "median700_d64"])
def test_random_partitions_sampled(gpu_lib, seed, median, sigma, D):
    """Seeded lognormal partitions other than the benchmark's (two rows with
    different documents, GQA 8:2, 16K tokens, head_dim 128 and 64), both tile
    grids against one oracle evaluation; sampled rows and keys, as at full
    size."""
    B, S, Hq, Hkv, base = 2, 16384, 8, 2, 5e6
    rows_len = tuple(tuple(W.sample_doc_lengths(S, median, sigma, 1, S - 1, seed * 10 + b)) for b in range(B))
    w = W.Workload("random", B, S, Hq, Hkv, D, base, True, rows_len, 1100 + seed)
    cu = w.cu_doc_lens
    say(f"[random] seed {seed} median {median}: {[len(r) for r in rows_len]} documents")
    q, k, v, do = W.make_tensors(B, S, Hq, Hkv, D, w.tensor_seed)
    rng = np.random.default_rng(seed)
    heads = list(range(Hq // Hkv))          # all query heads of kv group 0
    rows = _sample_rows(w, rng, 24)
    keys = _sample_keys(w, rng, 16)
    say(f"[random] seed {seed} oracle on {len(rows)} rows, {len(keys)} keys")
    o_ref, lse_ref, _, _ = oracle.forward(q, k, v, cu, base, heads=heads, rows=rows)
    dq_r, dk_r, dv_r, _, _ = oracle.backward(q, k, v, do, cu, base, heads=heads, q_rows=rows, k_cols=keys)
    qc, kc, vc, doc = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    for grid in (0, 16):                    # from the first token; after the anchor
        o, lse = gpu_lib.anchor_attn_fwd(qc, kc, vc, cu, base, flags=grid)
        dq, dk, dv = gpu_lib.anchor_attn_bwd(qc, kc, vc, o, lse, doc, cu, base, flags=grid)
        torch.cuda.synchronize()
        o_g = f64(o).reshape(B * S, Hq, D)[rows][:, heads]
        lse_g = f64(lse).transpose(1, 0, 2).reshape(Hq, B * S)[heads][:, rows]
        e_o = o_err(o_g, o_ref)
        e_dq = rel_frob(f64(dq).reshape(B * S, Hq, D)[rows][:, heads], dq_r)
        e_dk = rel_frob(f64(dk).reshape(B * S, Hkv, D)[keys][:, [0]], dk_r[:, [0]])
        e_dv = rel_frob(f64(dv).reshape(B * S, Hkv, D)[keys][:, [0]], dv_r[:, [0]])
        say(f"[random] seed {seed} grid {grid} O {e_o:.2e} dq {e_dq:.2e} dk {e_dk:.2e} dv {e_dv:.2e}")
        assert e_o <= O_TOL
        assert np.abs(lse_g - lse_ref).max() <= LSE_TOL
        assert max(e_dq, e_dk, e_dv) <= G_TOL


def _long_doc_keys(w):
    """Keys of the row's longest document: its first tokens, the start of
    its second and third 128-key tiles, its middle and its last token."""
    cu = w.cu_doc_lens
    n = int(np.argmax(np.diff(cu)))
    s, e = int(cu[n]), int(cu[n + 1])
    mid = (s + e) // 2
    return s, e, np.array(sorted({s, s + 1, s + 63, s + 64, s + 128, s + 257, mid, mid + 1, e - 1}))


@pytest.mark.parametrize("wname", ["8k", "64k"])
def test_long_document_key_gradients(gpu_lib, wname):
    """dK/dV of keys inside the workload's longest document (8K: 2,532
    tokens, 64K: 17,752 tokens) at full size, so that the key-major kernel's
    walk over every query tile of a long document is compared with the
    oracle; the oracle sums over exactly the rows that see those keys."""
    w = W.get(wname)
    B, S, Hq, Hkv, D = w.B, w.S, w.Hq, w.Hkv, w.D
    s, e, keys = _long_doc_keys(w)
    say(f"[long-doc] {wname} document [{s}, {e}) ({e - s} tokens), keys {keys.tolist()}")
    q, k, v, do = W.make_tensors(B, S, Hq, Hkv, D, w.tensor_seed)
    cu = w.cu_doc_lens
    qc, kc, vc, doc = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    say(f"[long-doc] {wname} fwd+bwd on GPU")
    o, lse = gpu_lib.anchor_attn_fwd(qc, kc, vc, cu, w.rope_base)
    dq, dk, dv = gpu_lib.anchor_attn_bwd(qc, kc, vc, o, lse, doc, cu, w.rope_base)
    torch.cuda.synchronize()
    for h in (0, Hq - 1):
        say(f"[long-doc] {wname} oracle backward, head {h}")
        _, dk_r, dv_r, _, _ = oracle.backward(q, k, v, do, cu, w.rope_base, heads=[h], q_rows=[s],
                                              k_cols=keys)
        e_dk = rel_frob(f64(dk).reshape(B * S, Hkv, D)[keys][:, [h]], dk_r[:, [h]])
        e_dv = rel_frob(f64(dv).reshape(B * S, Hkv, D)[keys][:, [h]], dv_r[:, [h]])
        say(f"[long-doc] {wname} head {h}: dk {e_dk:.2e} dv {e_dv:.2e}")
        assert max(e_dk, e_dv) <= G_TOL


def test_anchor_key_gradients_8k(gpu_lib):
    """dk and dv of the anchor key at the 8K shape: every one of the 8,192
    queries contributes, through the per-64-row partial sums and their
    reduction; against the oracle summing over all rows, per head."""
    w = W.get("8k")
    B, S, Hq, Hkv, D = w.B, w.S, w.Hq, w.Hkv, w.D
    say("[anchor-8k] generating inputs")
    q, k, v, do = W.make_tensors(B, S, Hq, Hkv, D, w.tensor_seed)
    cu = w.cu_doc_lens
    qc, kc, vc, doc = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    say("[anchor-8k] fwd+bwd on GPU")
    o, lse = gpu_lib.anchor_attn_fwd(qc, kc, vc, cu, w.rope_base)
    dq, dk, dv = gpu_lib.anchor_attn_bwd(qc, kc, vc, o, lse, doc, cu, w.rope_base)
    torch.cuda.synchronize()
    heads = [0, Hq - 1]
    say("[anchor-8k] oracle backward for the anchor key over every row")
    _, dk_r, dv_r, _, _ = oracle.backward(q, k, v, do, cu, w.rope_base, heads=heads, q_rows=[0],
                                          k_cols=[0])
    for h in heads:
        e_dk = rel_frob(f64(dk).reshape(B * S, Hkv, D)[[0]][:, [h]], dk_r[:, [h]])
        e_dv = rel_frob(f64(dv).reshape(B * S, Hkv, D)[[0]][:, [h]], dv_r[:, [h]])
        say(f"[anchor-8k] head {h}: dk0 {e_dk:.2e} dv0 {e_dv:.2e}")
        assert max(e_dk, e_dv) <= G_TOL


@pytest.mark.parametrize("mode", ["intra_doc_reset", "full_causal", "anchor_continuous"])
def test_full_size_sampled_modes(gpu_lib, mode):
    """The 64K shape in the benchmark's baseline modes; sampled outputs.
    intra_doc_reset: the 64K documents without an anchor; full_causal: the
    whole row as one document without an anchor (plain causal attention)."""
    w = W.get("64k")
    B, S, Hq, Hkv, D = w.B, w.S, w.Hq, w.Hkv, w.D
    if mode == "anchor_continuous":
        flags, anchor, pos_mode = 1, True, "continuous"
        cu = w.cu_doc_lens
    elif mode == "intra_doc_reset":
        flags, anchor, pos_mode = 2, False, "reset"
        cu = W.cu_doc_lens_no_anchor(W.rows_without_anchor([list(r) for r in w.doc_rows]), S)
    else:
        flags, anchor, pos_mode = 2, False, "reset"
        cu = W.cu_doc_lens_no_anchor([[S]] * B, S)
    say(f"[full-modes] {mode} generating inputs")
    q, k, v, do = W.make_tensors(B, S, Hq, Hkv, D, w.tensor_seed)
    qc, kc, vc, doc = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    say(f"[full-modes] {mode} fwd+bwd on GPU")
    o, lse = gpu_lib.anchor_attn_fwd(qc, kc, vc, cu, w.rope_base, flags=flags)
    dq, dk, dv = gpu_lib.anchor_attn_bwd(qc, kc, vc, o, lse, doc, cu, w.rope_base, flags=flags)
    torch.cuda.synchronize()
    rng = np.random.default_rng(12)
    heads = [0, Hq - 1]
    # uniformly drawn rows estimate the whole tensor's relative Frobenius
    # error without bias; rows at document starts (few keys, cancelling dS
    # terms) join the per-element forward check only
    urows = np.sort(rng.choice(S, 48, replace=False))
    rows = np.unique(np.concatenate([[0, 1, S - 1], cu[1:-1], cu[1:-1] - 1, urows]))[:160]
    rows = rows[(rows >= 0) & (rows < S)]
    say(f"[full-modes] {mode} oracle forward on {len(rows)} rows")
    o_ref, lse_ref, _, _ = oracle.forward(q, k, v, cu, w.rope_base, heads=heads, rows=rows,
                                          pos_mode=pos_mode, anchor=anchor)
    o_g = f64(o).reshape(B * S, Hq, D)[rows][:, heads]
    lse_g = f64(lse).transpose(1, 0, 2).reshape(Hq, B * S)[heads][:, rows]
    say(f"[full-modes] {mode} O err {o_err(o_g, o_ref):.2e} lse err {np.abs(lse_g - lse_ref).max():.2e}")
    assert o_err(o_g, o_ref) <= O_TOL
    assert np.abs(lse_g - lse_ref).max() <= LSE_TOL
    # key gradients need every query that sees the key: take keys near the end
    # of the row (full causal) or in short documents
    if mode == "full_causal":
        keys = np.array(sorted(set([S - 1, S - 2] + list(rng.integers(S - 1500, S, 10)))))
    else:
        keys = _sample_keys(w, rng, 16) if anchor else np.array(
            [int(x) for s_, e_ in zip(cu[:-1], cu[1:]) if e_ - s_ <= 2500 for x in (s_, e_ - 1)])[:16]
    qrows = urows[:32]
    say(f"[full-modes] {mode} oracle backward on {len(qrows)} rows, {len(keys)} keys")
    dq_r, dk_r, dv_r, _, _ = oracle.backward(q, k, v, do, cu, w.rope_base, heads=heads, q_rows=qrows,
                                             k_cols=keys, pos_mode=pos_mode, anchor=anchor)
    e_dq = rel_frob(f64(dq).reshape(B * S, Hq, D)[qrows][:, heads], dq_r)
    # key gradients are exact sums over the chosen heads only when those are all
    # of the group's heads; with MHA (Hq == Hkv) each head is its own group
    e_dk = rel_frob(f64(dk).reshape(B * S, Hkv, D)[keys][:, heads], dk_r[:, heads])
    e_dv = rel_frob(f64(dv).reshape(B * S, Hkv, D)[keys][:, heads], dv_r[:, heads])
    say(f"[full-modes] {mode} dq {e_dq:.2e} dk {e_dk:.2e} dv {e_dv:.2e}")
    assert max(e_dq, e_dk, e_dv) <= G_TOL


def test_many_query_tiles_natural_order(gpu_lib):
    """More query tiles than the work-order kernel ranks (130 rows x 128
    tiles = 16,640 > 16,384): the launches fall back to the natural order,
    head after head; sampled outputs against the oracle."""
    B, S, Hq, Hkv, D, base = 130, 16384, 2, 1, 64, 5e5
    rows_docs = [W.sample_doc_lengths(S, 1024, 1.0, 64, S - 1, 300 + b) for b in range(B)]
    cu = W.cu_doc_lens_from_lengths(rows_docs, S)
    say(f"[many-tiles] B={B} S={S} Hq={Hq} Hkv={Hkv} D={D}: generating inputs")
    q, k, v, do = W.make_tensors(B, S, Hq, Hkv, D, 4321)
    qc, kc, vc, doc = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    say("[many-tiles] fwd+bwd on GPU")
    o, lse = gpu_lib.anchor_attn_fwd(qc, kc, vc, cu, base)
    dq, dk, dv = gpu_lib.anchor_attn_bwd(qc, kc, vc, o, lse, doc, cu, base)
    torch.cuda.synchronize()
    rng = np.random.default_rng(13)
    heads = [0, 1]          # the whole kv group
    rows = np.unique(np.concatenate([[0, S, (B - 1) * S, B * S - 1],
                                     rng.integers(0, B * S, 40), cu[1:-1][rng.integers(0, len(cu) - 2, 16)]]))
    say(f"[many-tiles] oracle forward on {len(rows)} rows")
    o_ref, lse_ref, _, _ = oracle.forward(q, k, v, cu, base, heads=heads, rows=rows)
    ridx = torch.as_tensor(rows, device=o.device)
    o_g = f64(o.reshape(B * S, Hq, D)[ridx][:, heads])
    lse_g = f64(lse).transpose(1, 0, 2).reshape(Hq, B * S)[heads][:, rows]
    say(f"[many-tiles] O err {o_err(o_g, o_ref):.2e} lse err {np.abs(lse_g - lse_ref).max():.2e}")
    assert o_err(o_g, o_ref) <= O_TOL
    assert np.abs(lse_g - lse_ref).max() <= LSE_TOL
    # keys of short documents (every query that sees them is cheap to sum),
    # and the anchors of the first and last rows
    short = [(int(s_), int(e_)) for s_, e_ in zip(cu[:-1], cu[1:]) if 1 < e_ - s_ <= 400]
    keys = np.unique(np.array([0, (B - 1) * S] + [x for s_, e_ in short[:12] for x in (s_, e_ - 1)]))
    qrows = rows[:32]
    say(f"[many-tiles] oracle backward on {len(qrows)} rows, {len(keys)} keys")
    dq_r, dk_r, dv_r, _, _ = oracle.backward(q, k, v, do, cu, base, heads=heads, q_rows=qrows, k_cols=keys)
    qidx = torch.as_tensor(qrows, device=o.device)
    kidx = torch.as_tensor(keys, device=o.device)
    e_dq = rel_frob(f64(dq.reshape(B * S, Hq, D)[qidx][:, heads]), dq_r)
    e_dk = rel_frob(f64(dk.reshape(B * S, Hkv, D)[kidx][:, [0]]), dk_r[:, [0]])
    e_dv = rel_frob(f64(dv.reshape(B * S, Hkv, D)[kidx][:, [0]]), dv_r[:, [0]])
    say(f"[many-tiles] dq {e_dq:.2e} dk {e_dk:.2e} dv {e_dv:.2e}")
    assert max(e_dq, e_dk, e_dv) <= G_TOL
