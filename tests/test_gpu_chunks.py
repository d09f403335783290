"""Interleaved document chunks through the C ABI (arch page §5, "AnchorAttention
with Interleaved Chunks", Figure 5): the chunk layout against the oracle
(positions bit-exact; the permutation, of which several are valid, checked
for what makes it valid), invalid layouts reported, forward and backward
against the oracle's interleaved mode."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from _helpers import f64, o_err, rel_frob, say

pytestmark = pytest.mark.gpu
O_TOL, G_TOL, LSE_TOL = 4e-3, 1e-2, 5e-2


def _layout(seed, B, S, anchor, max_docs=None, max_chunks=4):
    rng = np.random.default_rng(seed)
    rows = [W.random_partition(rng, S if anchor else S + 1, max_docs) for _ in range(B)]
    return W.interleaved_chunks(rows, S, rng, max_chunks, anchor)


@pytest.mark.parametrize("anchor", [True, False])
@pytest.mark.parametrize("flags_pos", [0, 1], ids=["reset", "continuous"])
@pytest.mark.parametrize("shape", [(2, 700, 12), (1, 4096, 40), (3, 5, None)], ids=["b2", "4k", "tiny"])
def test_chunk_layout(gpu_lib, anchor, flags_pos, shape):
    B, S, max_docs = shape
    cu, cd = _layout(11 + S, B, S, anchor, max_docs)
    flags = flags_pos | (0 if anchor else gpu_lib.FLAG_NO_ANCHOR)
    say(f"[chunks] layout B={B} S={S} chunks={len(cd)} flags={flags}")
    src, pos, ws = gpu_lib.anchor_attn_chunk_layout(cu, cd, B, S, True, flags)
    assert gpu_lib.anchor_attn_device_status(ws) == 0
    src = src.cpu().numpy().astype(np.int64)
    pos = pos.cpu().numpy().astype(np.int64)
    # a permutation inside every row
    assert np.array_equal(np.sort(src), np.arange(B * S))
    assert np.all(src // S == np.arange(B * S) // S)
    # position IDs, in the caller's order, exactly the oracle's
    got = np.empty_like(pos)
    got[src] = pos
    ref = oracle.position_ids(cu, B, S, "continuous" if flags_pos else "reset", anchor, seg_doc=cd)
    assert np.array_equal(got, ref)
    # every document contiguous in the permuted row, its own order kept, anchor first
    doc = oracle.document_ids(cu, B, S, anchor, cd)
    dp = doc[src]
    for b in range(B):
        r = slice(b * S, (b + 1) * S)
        if anchor:
            assert src[b * S] == b * S
        change = np.nonzero(np.diff(dp[r]))[0]
        assert len(set(dp[r])) == len(change) + 1          # each label in one run
        for lab in set(dp[r]):
            toks = src[r][dp[r] == lab]
            assert np.all(np.diff(toks) > 0)                # original order kept


def test_invalid_chunk_layouts_are_reported(gpu_lib):
    S = 10
    cases = [
        (np.array([0, 1, 4, 10]), np.array([0, 1, 0])),          # anchor chunk without id -1
        (np.array([0, 1, 4, 10]), np.array([-1, -1, 0])),        # -1 on a document chunk
        (np.array([0, 2, 4, 10]), np.array([-1, 0, 1])),         # anchor chunk of length 2
    ]
    for cu, cd in cases:
        src, pos, ws = gpu_lib.anchor_attn_chunk_layout(cu, cd, 1, S, True, 0)
        assert gpu_lib.anchor_attn_device_status(ws) == gpu_lib.AA_EDOCS
        s = src.cpu().numpy()
        assert s.min() >= 0 and s.max() < S                      # identity fallback stays in the row
    # a chunk crossing into the next row
    src, pos, ws = gpu_lib.anchor_attn_chunk_layout(np.array([0, 1, 12, 20]), np.array([-1, 0, 1]),
                                                     2, S, True, 0)
    assert gpu_lib.anchor_attn_device_status(ws) == gpu_lib.AA_EDOCS
    # more than 4096 chunks in one row
    S2 = 4200
    cu = np.arange(S2 + 1)
    cd = np.concatenate([[-1], np.arange(S2 - 1)])
    src, pos, ws = gpu_lib.anchor_attn_chunk_layout(cu, cd, 1, S2, True, 0)
    assert gpu_lib.anchor_attn_device_status(ws) == gpu_lib.AA_EDOCS


def _cases():
    return [
        # name, seed, B, S, Hq, Hkv, D, anchor, flags_pos, causal, max_docs, max_chunks
        ("b2_gqa_d128", 1, 2, 700, 4, 2, 128, True, 0, True, 12, 4),
        ("one_row_d64_many_chunks", 2, 1, 900, 2, 2, 64, True, 0, True, 6, 12),
        ("no_anchor", 3, 2, 640, 2, 1, 128, False, 0, True, 10, 4),
        ("continuous", 4, 1, 777, 2, 2, 128, True, 1, True, 8, 5),
        ("noncausal", 5, 1, 500, 2, 2, 64, True, 0, False, 6, 3),
        ("grid_after_anchor", 6, 2, 700, 4, 2, 128, True, 16, True, 12, 4),
    ]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c[0])
def test_fwd_bwd_interleaved(gpu_lib, case):
    name, seed, B, S, Hq, Hkv, D, anchor, fpos, causal, max_docs, max_chunks = case
    cu, cd = _layout(100 + seed, B, S, anchor, max_docs, max_chunks)
    flags = fpos | (0 if anchor else gpu_lib.FLAG_NO_ANCHOR)
    mode = "continuous" if fpos & 1 else "reset"
    say(f"[chunks] {name} B={B} S={S} chunks={len(cd)} flags={flags} causal={causal}")
    q, k, v, do = W.make_tensors(B, S, Hq, Hkv, D, 900 + seed)
    o, lse = gpu_lib.anchor_attn_fwd_chunks(q.cuda(), k.cuda(), v.cuda(), cu, cd, 1e4, causal, flags=flags)
    o_ref, lse_ref, _, _ = oracle.forward(q, k, v, cu, 1e4, causal, pos_mode=mode, anchor=anchor, seg_doc=cd)
    o_g = f64(o).reshape(B * S, Hq, D)
    assert o_err(o_g, o_ref) <= O_TOL, o_err(o_g, o_ref)
    lse_g = f64(lse).transpose(1, 0, 2).reshape(Hq, B * S)
    assert np.abs(lse_g - lse_ref).max() <= LSE_TOL
    dq, dk, dv = gpu_lib.anchor_attn_bwd_chunks(q.cuda(), k.cuda(), v.cuda(), o, lse, do.cuda(), cu, cd,
                                                1e4, causal, flags=flags)
    dq_r, dk_r, dv_r, _, _ = oracle.backward(q, k, v, do, cu, 1e4, causal, pos_mode=mode, anchor=anchor,
                                             seg_doc=cd)
    e = (rel_frob(f64(dq).reshape(B * S, Hq, D), dq_r), rel_frob(f64(dk).reshape(B * S, Hkv, D), dk_r),
         rel_frob(f64(dv).reshape(B * S, Hkv, D), dv_r))
    say(f"[chunks] {name} O {o_err(o_g, o_ref):.2e} dq {e[0]:.2e} dk {e[1]:.2e} dv {e[2]:.2e}")
    assert max(e) <= G_TOL, e


def test_interleaved_fp32_output(gpu_lib):
    """FLAG_O_FP32 through the chunk entry points: the float32 O goes through
    the permutation to the caller's order (the bf16 O is exactly its rounding)
    and the backward reads it through the permutation; against the oracle."""
    name, seed, B, S, Hq, Hkv, D, anchor, fpos, causal, max_docs, max_chunks = _cases()[0]
    cu, cd = _layout(100 + seed, B, S, anchor, max_docs, max_chunks)
    q, k, v, do = W.make_tensors(B, S, Hq, Hkv, D, 900 + seed)
    qc, kc, vc, doc = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    f32 = gpu_lib.FLAG_O_FP32
    o16, lse16 = gpu_lib.anchor_attn_fwd_chunks(qc, kc, vc, cu, cd, 1e4, causal)
    o32, lse32 = gpu_lib.anchor_attn_fwd_chunks(qc, kc, vc, cu, cd, 1e4, causal, flags=f32)
    assert o32.dtype == torch.float32
    assert torch.equal(o32.to(torch.bfloat16), o16) and torch.equal(lse32, lse16)
    o_ref, _, _, _ = oracle.forward(q, k, v, cu, 1e4, causal, anchor=anchor, seg_doc=cd)
    e_o = o_err(f64(o32).reshape(B * S, Hq, D), o_ref)
    dq, dk, dv = gpu_lib.anchor_attn_bwd_chunks(qc, kc, vc, o32, lse32, doc, cu, cd, 1e4, causal, flags=f32)
    dq_r, dk_r, dv_r, _, _ = oracle.backward(q, k, v, do, cu, 1e4, causal, anchor=anchor, seg_doc=cd)
    e = (rel_frob(f64(dq).reshape(B * S, Hq, D), dq_r), rel_frob(f64(dk).reshape(B * S, Hkv, D), dk_r),
         rel_frob(f64(dv).reshape(B * S, Hkv, D), dv_r))
    say(f"[chunks] fp32 O {e_o:.2e} dq {e[0]:.2e} dk {e[1]:.2e} dv {e[2]:.2e}")
    assert e_o <= O_TOL and max(e) <= G_TOL, (e_o, e)


def test_interleaved_64k_sampled(gpu_lib):
    """The 64K documents cut into up to 4 chunks each and interleaved; the
    benchmark's shapes; uniformly sampled rows, keys in short documents."""
    w = W.get("64k")
    B, S, Hq, Hkv, D = w.B, w.S, w.Hq, w.Hkv, w.D
    rng = np.random.default_rng(64)
    cu, cd = W.interleaved_chunks([list(r) for r in w.doc_rows], S, rng, 4, True)
    say(f"[chunks] 64k interleaved: {len(cd)} chunks")
    q, k, v, do = W.make_tensors(B, S, Hq, Hkv, D, w.tensor_seed)
    qc, kc, vc, doc = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = gpu_lib.anchor_attn_fwd_chunks(qc, kc, vc, cu, cd, w.rope_base)
    dq, dk, dv = gpu_lib.anchor_attn_bwd_chunks(qc, kc, vc, o, lse, doc, cu, cd, w.rope_base)
    torch.cuda.synchronize()
    heads = [0, Hq - 1]
    rows = np.sort(rng.choice(S, 48, replace=False))
    o_ref, lse_ref, _, _ = oracle.forward(q, k, v, cu, w.rope_base, heads=heads, rows=rows, seg_doc=cd)
    o_g = f64(o).reshape(B * S, Hq, D)[rows][:, heads]
    lse_g = f64(lse).transpose(1, 0, 2).reshape(Hq, B * S)[heads][:, rows]
    say(f"[chunks] 64k O err {o_err(o_g, o_ref):.2e} lse err {np.abs(lse_g - lse_ref).max():.2e}")
    assert o_err(o_g, o_ref) <= O_TOL
    assert np.abs(lse_g - lse_ref).max() <= LSE_TOL
    # keys of documents no longer than 2500 tokens (all their queries are cheap)
    lens = {}
    for c in range(len(cd)):
        lens[int(cd[c])] = lens.get(int(cd[c]), 0) + int(cu[c + 1] - cu[c])
    short = [d for d, L in lens.items() if d >= 0 and L <= 2500]
    keys = np.array(sorted(int(rng.integers(cu[c], cu[c + 1])) for c in range(len(cd)) if cd[c] in short))[:16]
    qrows = rows[:24]
    dq_r, dk_r, dv_r, _, _ = oracle.backward(q, k, v, do, cu, w.rope_base, heads=heads, q_rows=qrows,
                                             k_cols=keys, seg_doc=cd)
    e_dq = rel_frob(f64(dq).reshape(B * S, Hq, D)[qrows][:, heads], dq_r)
    e_dk = rel_frob(f64(dk).reshape(B * S, Hkv, D)[keys][:, heads], dk_r[:, heads])
    e_dv = rel_frob(f64(dv).reshape(B * S, Hkv, D)[keys][:, heads], dv_r[:, heads])
    say(f"[chunks] 64k dq {e_dq:.2e} dk {e_dk:.2e} dv {e_dv:.2e}")
    assert max(e_dq, e_dk, e_dv) <= G_TOL
