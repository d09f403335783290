"""The allocation-free backward (anchor_attn_bwd_noalloc) through the C ABI
against the workspace backward (anchor_attn_bwd) on the same inputs: two
calls in a row, the second on a smaller problem, each bit-identical to the
workspace entry point (the same kernels on the same workspace layout)."""
import numpy as np
import pytest
import torch

import workloads as W
from _helpers import say

pytestmark = pytest.mark.gpu


def _case(B, S, Hq, Hkv, D, rows, seed):
    cu = W.cu_doc_lens_from_lengths(rows, S)
    q, k, v, do = (t.cuda() for t in W.make_tensors(B, S, Hq, Hkv, D, seed))
    return cu, q, k, v, do


def test_noalloc_backward_matches_the_workspace_backward(gpu_lib):
    rng = np.random.default_rng(808)
    cases = [
        ("large", 2, 1500, 8, 2, 128, [W.random_partition(rng, 1500, 12) for _ in range(2)], 5e6),
        ("smaller", 1, 700, 4, 4, 64, [[300, 1, 398]], 1e4),
    ]
    for name, B, S, Hq, Hkv, D, rows, base in cases:
        say(f"[noalloc] {name}: B={B} S={S} Hq={Hq} Hkv={Hkv} D={D}")
        cu, q, k, v, do = _case(B, S, Hq, Hkv, D, rows, 77)
        o, lse = gpu_lib.anchor_attn_fwd(q, k, v, cu, base)
        ref = gpu_lib.anchor_attn_bwd(q, k, v, o, lse, do, cu, base)
        got = gpu_lib.anchor_attn_bwd_noalloc(q, k, v, o, lse, do, cu, base)
        torch.cuda.synchronize()
        for a, b in zip(got, ref):
            assert not torch.isnan(a.float()).any()
            assert torch.equal(a, b), name
