"""A forward + backward step captured in a HIP graph (torch.cuda.CUDAGraph)
and replayed: every replay equals the eager step bit for bit, with eager work
on the same GPU and synchronisations between the replays."""
import numpy as np
import pytest
import torch

import workloads as W
from _helpers import say

pytestmark = pytest.mark.gpu


def test_graph_replay_matches_eager(gpu_lib):
    B, S, Hq, Hkv, D, base = 2, 1000, 4, 2, 128, 5e6
    rng = np.random.default_rng(77)
    cu = torch.from_numpy(W.cu_doc_lens_from_lengths([W.random_partition(rng, S, 12) for _ in range(B)],
                                                     S)).cuda()
    q, k, v, do = (t.cuda() for t in W.make_tensors(B, S, Hq, Hkv, D, 99))
    ws = torch.empty(gpu_lib.workspace_size(B, S, Hq, Hkv, D, True), dtype=torch.uint8, device="cuda")
    bflags = gpu_lib.FLAG_FWD_WORKSPACE

    def step():
        o, lse = gpu_lib.anchor_attn_fwd(q, k, v, cu, base, True, None, ws)
        dq, dk, dv = gpu_lib.anchor_attn_bwd(q, k, v, o, lse, do, cu, base, True, None, ws, flags=bflags)
        return o, lse, dq, dk, dv

    ref = step()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = step()
    # other inputs for the eager work between replays (same shapes, other values)
    q2, k2, v2, do2 = (t.cuda() for t in W.make_tensors(B, S, Hq, Hkv, D, 100))
    ws2 = torch.empty_like(ws)
    for r in range(4):
        for t in out:
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("o", "lse", "dq", "dk", "dv"), out, ref):
            assert torch.equal(a, b), f"replay {r}: {name} differs from the eager step"
        o2, lse2 = gpu_lib.anchor_attn_fwd(q2, k2, v2, cu, base, True, None, ws2)
        gpu_lib.anchor_attn_bwd(q2, k2, v2, o2, lse2, do2, cu, base, True, None, ws2, flags=bflags)
        torch.cuda.synchronize()
        say(f"[graph] replay {r} matches the eager step")
