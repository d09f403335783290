"""Shift-invariance diagnostic on the GPU bf16 path (arch page §2.2, Eq. 3, Eq. 5).

In exact arithmetic RoPE logits depend only on relative position: shifting
every position by the same amount leaves q'_i . k'_j unchanged (Eq. 3).  The
library's RoPE stage forms the rotation angle in float64, rotates in float32
and rounds the rotated vectors to bfloat16; the attention kernels multiply
those bf16 vectors exactly and accumulate in float32.  The logits below are
formed the same way (bf16 products, float32 sums), so they are the logits the
attention kernels see.  Synthetic N(0,1) q and k stand in for a randomly
initialised model; no trained weights are used.

D_logit(d1, d2) = (1/T) sum_i |A_{i,first}(d1) - A_{i,first}(d2)| (Eq. 5 for
one layer and head), A the pre-softmax logit of token i against the first
token, d1, d2 two shifts of every position.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from _helpers import f64, say

BASE = 5e6


def _qk(T, D, seed):
    g = torch.Generator("cpu").manual_seed(seed)
    q = torch.randn((1, T, 1, D), generator=g).to(torch.bfloat16)
    k = torch.randn((1, T, 1, D), generator=g).to(torch.bfloat16)
    return q, k


def _first_token_logits_fp64(q, k, shift):
    T = q.shape[1]
    pos = np.arange(T) + shift
    qr = oracle.rope(f64(q[0, :, 0]), pos, BASE)
    kr = oracle.rope(f64(k[0, :1, 0]), pos[:1], BASE)
    return qr @ kr[0]


def _rope_gpu(lib, x, shift):
    """x [1,T,1,D] at positions shift .. shift+T-1 through the library's RoPE
    stage (its table covers positions below its sequence length)."""
    T, D = x.shape[1], x.shape[3]
    S = T + shift
    big = torch.zeros((1, S, 1, D), dtype=torch.bfloat16)
    big[:, :T] = x
    pos = torch.zeros(S, dtype=torch.int32)
    pos[:T] = torch.arange(T, dtype=torch.int32) + shift
    return lib.anchor_attn_rope(big.cuda(), pos, BASE)[:, :T]


def _first_token_logits_gpu(lib, q, k, shift):
    qr = _rope_gpu(lib, q, shift)[0, :, 0].float()
    kr = _rope_gpu(lib, k, shift)[0, 0, 0].float()
    return f64((qr * kr).sum(-1))        # bf16 products are exact in float32


def _d_logit(a, b):
    return float(np.abs(a - b).mean())


def test_fp64_first_token_logits_are_shift_invariant():
    q, k = _qk(512, 64, 3)
    a = _first_token_logits_fp64(q, k, 16)
    for d in (0, 1000, 60000):
        assert _d_logit(_first_token_logits_fp64(q, k, d), a) < 1e-10


@pytest.mark.gpu
def test_bf16_path_first_token_logits_move_with_the_shift(gpu_lib):
    D = 128
    rows = []
    for T in (64, 1024, 8192):
        q, k = _qk(T, D, 10 + T)
        ref16 = _first_token_logits_gpu(gpu_lib, q, k, 16)
        exact = _first_token_logits_fp64(q, k, 16)
        # rounding bound of one logit: both factors carry at most 2^-9
        # relative rounding per element, after an accurate rotation
        qr = oracle.rope(f64(q[0, :, 0]), np.arange(T) + 16, BASE)
        kr = oracle.rope(f64(k[0, :1, 0]), [16], BASE)[0]
        bound = float((np.abs(qr) @ np.abs(kr)).mean()) * 2.0 ** -7
        for d1 in (0, 256, 4096, 32768):
            dl = _d_logit(_first_token_logits_gpu(gpu_lib, q, k, d1), ref16)
            dl64 = _d_logit(_first_token_logits_fp64(q, k, d1), exact)
            rows.append((T, d1, dl, dl64))
            say(f"[shift] T={T:5d} d1={d1:5d} d2=16: D_logit bf16 path {dl:.3e}   float64 {dl64:.1e}")
            assert dl64 < 1e-9
            assert dl <= bound
            if d1 != 16:
                assert dl > 0.0          # bf16 breaks the exact invariance
    # the shift-free comparison of the same positions is exactly zero
    q, k = _qk(256, D, 5)
    assert _d_logit(_first_token_logits_gpu(gpu_lib, q, k, 16),
                    _first_token_logits_gpu(gpu_lib, q, k, 16)) == 0.0


@pytest.mark.gpu
@pytest.mark.parametrize("flags", [0, 2, 3], ids=["anchor_reset", "intra_doc_reset", "intra_doc_continuous"])
def test_document_outputs_and_its_place_in_the_pack(gpu_lib, flags):
    """The same document packed at two places of a row, 512 tokens apart (a
    multiple of the kernels' 128-query and 64-key tiles, so both copies get the
    same tile work).  With reset position IDs both copies carry the same
    positions and their outputs are bit-identical, with or without the anchor.
    Without an anchor, continuous IDs put the copies at other absolute
    positions: in exact arithmetic that changes nothing (Eq. 3, every logit is
    inside the document), but the bf16 rotation does, so the copies differ by
    rounding.  (With the anchor, continuous IDs also change each copy's
    distance to the anchor, an exact difference, so that case is not shown.)"""
    D, L, S = 128, 383, 1024
    g = torch.Generator("cpu").manual_seed(77)
    doc_q, doc_k, doc_v = (torch.randn((L, 2, D), generator=g).to(torch.bfloat16) for _ in range(3))
    q, k, v, _ = W.make_tensors(1, S, 2, 2, D, 78)
    # token 0 (anchor, or a one-token document), doc (1..383), filler
    # (384..512), doc again (513..895), filler (896..1023)
    if flags & 2:
        cu = W.cu_doc_lens_no_anchor([[1, L, 129, L, 128]], S)
    else:
        cu = W.cu_doc_lens_from_lengths([[L, 129, L, 128]], S)
    for x, d in ((q, doc_q), (k, doc_k), (v, doc_v)):
        x[0, 1:1 + L] = d
        x[0, 513:513 + L] = d
    o, lse = gpu_lib.anchor_attn_fwd(q.cuda(), k.cuda(), v.cuda(), cu, BASE, flags=flags)
    o = o.cpu()
    a, b = o[0, 1:1 + L], o[0, 513:513 + L]
    diff = float((a.float() - b.float()).abs().max())
    say(f"[shift] packed document twice, flags={flags}: max |O_copy1 - O_copy2| = {diff:.3e}")
    if flags & 1:
        assert 0.0 < diff <= 4e-3 * float(a.float().abs().max())
    else:
        assert diff == 0.0
