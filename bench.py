#!/usr/bin/env python3
"""Benchmark: AnchorAttention forward + backward on one MI355X.

One step = one full pass of the hot path over one packed batch: position IDs,
tile plans, RoPE, forward attention, dQ (with the backward's per-row
preprocessing), dK/dV and the anchor-key reduction (the library's anchor_attn_fwd + anchor_attn_bwd).

Prints ONE JSON line.  `value` is fwd+bwd TFLOP/s counting only unmasked
(query, key) pairs (14*D flops per pair and query head); inputs are resident
in HBM before the timed region starts, and the timed steps run without any
per-kernel instrumentation.  A second pass of as many steps, with HIP events
recorded by the library around each of its launches on the call's stream,
gives the per-kernel times: `roofline` reports the dominant kernel's achieved
rate from them, against the nominal peak and against the peak at the engine
clock sampled while the same steps run on for a few seconds afterwards.  `cpu_baseline` times the float64 CPU
oracle on a bounded sample of the same workload."""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA (vendor figure, no sparsity)
PEAK_HBM_GBS = 8000.0

# Algorithmic flops per unmasked (query, key) pair and query head, per kernel:
# forward: S = QK^T, O = PV (2 products); dK/dV kernel: S, dP, dV, dK (4);
# dQ kernel: S, dP, dQ (3).  The headline counts 4 + 10 = 14 per pair.
KERNEL_FLOPS_PER_PAIR_D = {"fwd": 4.0, "bwd_dkdv": 8.0, "bwd_dq": 6.0}
KERNEL_SOURCE = {"fwd": "fwd.hip", "bwd_dkdv": "bwd.hip", "bwd_dq": "bwd.hip"}


def _code_text(path: str) -> bytes:
    """A source file's code without its comments, whitespace runs collapsed:
    editing a comment leaves it (and so the hash below) unchanged."""
    t = open(path, encoding="utf-8").read()
    t = re.sub(r"/\*.*?\*/", " ", t, flags=re.S)
    t = re.sub(r"//[^\n]*", " ", t)
    return " ".join(t.split()).encode()


def _src_hash(kernel: str) -> str:
    """Hash of the code of the kernel's source file and of the header its
    kernels inline (aa_internal.h), followed by the file's extra build flags
    (none for most sources), so a counter summary goes stale when any of them
    changes."""
    from long_context_attention_doc_amd.build import SOURCE_FLAGS
    name = KERNEL_SOURCE[kernel]
    csrc = os.path.join(ROOT, "long_context_attention_doc_amd", "csrc")
    h = hashlib.sha256(_code_text(os.path.join(csrc, name)))
    h.update(b"\0" + _code_text(os.path.join(csrc, "aa_internal.h")))
    h.update(" ".join(SOURCE_FLAGS.get(name, [])).encode())
    return h.hexdigest()[:16]


def _traffic(kernel: str, workload: str):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it
    was taken on the current kernel source; otherwise None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_hbm_counters.txt")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_hash = re.search(r"source_sha256_16:\s*(\w+)", txt)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not m_hash or not m_bytes or m_hash.group(1) != _src_hash(kernel):
        return None
    return float(m_bytes.group(1))


def cpu_baseline(w, q, k, v, do, budget_s: float) -> dict:
    """The float64 oracle on whole documents at the start of row 0, one query
    head at a time until about `budget_s` seconds of CPU work.  Key gradients
    are taken for the documents' keys; the anchor key is left out because its
    gradient sums over every query of the row."""
    import numpy as np
    import oracle
    from long_context_attention_doc_amd.accounting import unmasked_pairs_closed_form
    lens = list(w.doc_rows[0])
    take, tot = [], 0
    for L in lens:
        if tot + L > 6144 and take:
            break
        take.append(L)
        tot += L
    rows = np.arange(0, 1 + tot)
    pairs = unmasked_pairs_closed_form([take])
    t0 = time.perf_counter()
    heads = 0
    for h in range(w.Hq):
        oracle.forward(q, k, v, w.cu_doc_lens, w.rope_base, heads=[h], rows=rows)
        oracle.backward(q, k, v, do, w.cu_doc_lens, w.rope_base, heads=[h], q_rows=rows,
                        k_cols=rows[1:])
        heads += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    flops = 14.0 * w.D * pairs * heads
    try:
        from threadpoolctl import threadpool_info
        blas = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:   # threadpoolctl missing: report the affinity count only
        blas = None
    cores = len(os.sched_getaffinity(0))
    return {
        "value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": blas or cores, "kind": "oracle",
        "sample": (f"row 0, anchor + first {len(take)} documents ({tot} tokens), {heads} of {w.Hq} "
                   f"query heads, forward + backward, {dt:.1f} s; {cores} host cores visible, "
                   f"BLAS threads {blas}"),
        "seconds": dt,
    }


# Attention paradigms (the pages' Figure 2 and the full-attention baseline):
# library flags, whether rows carry the shared anchor, and whether the
# documents are replaced by one document per row.
MODES = {
    "anchor": (0, True, False),
    "anchor_continuous": (1, True, False),
    "intra_doc_reset": (2, False, False),
    "intra_doc_continuous": (3, False, False),
    "full_causal": (2, False, True),
    # AnchorAttention on the same documents cut into up to 4 chunks each and
    # interleaved across the row (the pages' Figure 5, right)
    "interleaved": (0, True, False),
}


def device_peak() -> dict | None:
    """Dense bf16 MFMA peak re-derived on this machine: compute units x max
    engine clock (rocminfo) x 4096 flop/clk/CU (gfx950, 32x32x16 bf16)."""
    import subprocess
    try:
        txt = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60).stdout
    except Exception:   # rocminfo missing or hung: report nothing
        return None
    for agent in txt.split("Agent ")[1:]:
        if "gfx950" not in agent:
            continue
        cu = re.search(r"Compute Unit:\s*(\d+)", agent)
        mhz = re.search(r"Max Clock Freq\. \(MHz\):\s*(\d+)", agent)
        if cu and mhz:
            cus, clk = int(cu.group(1)), int(mhz.group(1))
            return {"compute_units": cus, "max_sclk_mhz": clk,
                    "bf16_dense_peak_tflops": cus * clk * 1e6 * 4096 / 1e12}
    return None


class ClockSampler:
    """Engine clock and socket power of GPU 0 from the firmware's metrics
    table (amdsmi Python API), read by a background thread.  The firmware
    refreshes the table about once a second, so only refreshes stamped after
    the sampler started count (each one once).  It only reads; without amdsmi
    or a device it records nothing."""

    def __init__(self, period_s: float = 0.02):
        import threading
        self.period = period_s
        self.samples = []          # (firmware timestamp, mean MHz over the XCDs, socket W)
        self._stop = threading.Event()
        self._thread = None
        self._t0 = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self._smi = amdsmi
            self._h = amdsmi.amdsmi_get_processor_handles()[0]
            self._t0 = self._smi.amdsmi_get_gpu_metrics_info(self._h).get("firmware_timestamp")
        except Exception:   # no amdsmi or no device: no samples
            self._smi = None

    def _sample(self):
        m = self._smi.amdsmi_get_gpu_metrics_info(self._h)
        ts = m.get("firmware_timestamp")
        if ts == self._t0 or (self.samples and ts == self.samples[-1][0]):
            return
        clks = [c for c in (m.get("current_gfxclks") or []) if isinstance(c, int) and 0 < c < 0xFFFF]
        pw = m.get("current_socket_power")
        if clks:
            self.samples.append((ts, sum(clks) / len(clks),
                                 float(pw) if isinstance(pw, (int, float)) and 0 < pw < 0xFFFF else None))

    def _run(self):
        while not self._stop.is_set():
            try:
                self._sample()
            except Exception:   # a failed read ends the sampling
                return
            self._stop.wait(self.period)

    def __enter__(self):
        import threading
        if self._smi is not None:
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread is not None:
            self._thread.join()
        return False

    def summary(self, skip: int = 1):
        """Mean over the refreshes after the first `skip` (the first one after
        the start may still describe the ramp)."""
        use = self.samples[skip:] if len(self.samples) > skip else []
        if not use:
            return None
        mhz = [u[1] for u in use]
        w = [u[2] for u in use if u[2] is not None]
        return {"gfx_mhz_mean": sum(mhz) / len(mhz), "gfx_mhz_min": min(mhz), "gfx_mhz_max": max(mhz),
                "refreshes": len(use), "socket_power_w_mean": (sum(w) / len(w)) if w else None,
                "source": "amdsmi gpu_metrics current_gfxclks (mean over the XCDs) and "
                          "current_socket_power, firmware refreshes (about 1 s apart) during a pass "
                          "of the same steps run right after the timed and profiled steps"}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="64k",
                    help="tiny | 8k | 64k | 128k_gqa | short_docs | 64k_ulysses8 (one GPU's head share of 64K "
                         "over 8 GPUs) (default: 64k, the headline)")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle time (0: skip)")
    ap.add_argument("--no-fwd-workspace", action="store_true",
                    help="self-contained backward: rebuild positions, plan and rotated q, k "
                         "instead of reusing the forward's workspace")
    ap.add_argument("--clock-s", type=float, default=4.0,
                    help="seconds of extra steps during which the engine clock is sampled (0: skip)")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step captured in a HIP graph and replayed")
    ap.add_argument("--no-graph", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--mode", default="anchor", choices=sorted(MODES),
                    help="anchor (default, the method) | anchor_continuous | intra_doc_reset | "
                         "intra_doc_continuous | full_causal | interleaved: the pages' other "
                         "attention paradigms through the same kernels, on the same documents")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported (this build has no "
              "multi-GPU path; see the sharding notes in DESIGN.md)", file=sys.stderr)
        return 2

    import torch
    import workloads
    from long_context_attention_doc_amd import api
    from long_context_attention_doc_amd.accounting import (algorithmic_bytes, flops_fwd_bwd,
                                                           kernel_algorithmic_bytes, roofline_point)

    w = workloads.get(args.workload)
    flags, anchor, one_doc = MODES[args.mode]
    dev = torch.device("cuda:0")
    q, k, v, do = workloads.make_tensors(w.B, w.S, w.Hq, w.Hkv, w.D, w.tensor_seed)
    qc, kc, vc, doc = (t.to(dev) for t in (q, k, v, do))
    doc_rows = [list(r) for r in w.doc_rows]
    if one_doc:
        doc_rows = [[w.S]] * w.B
    elif not anchor:
        doc_rows = workloads.rows_without_anchor(doc_rows)
    cu_np = (w.cu_doc_lens if anchor else workloads.cu_doc_lens_no_anchor(doc_rows, w.S))
    cu = torch.from_numpy(cu_np).to(dev)
    # the binding's choice of tile grid (after the anchor for short documents)
    flags |= api.grid_flag(cu_np, w.B, w.S, flags)
    ws_f = torch.empty(api.workspace_size(w.B, w.S, w.Hq, w.Hkv, w.D, False), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(api.workspace_size(w.B, w.S, w.Hq, w.Hkv, w.D, True), dtype=torch.uint8, device=dev)
    chunk_doc = None
    if args.mode == "interleaved":
        import numpy as np
        cu_np, cd_np = workloads.interleaved_chunks(doc_rows, w.S, np.random.default_rng(64), 4, True)
        cu = torch.from_numpy(cu_np).to(dev)
        chunk_doc = torch.from_numpy(cd_np).to(dev)
        ws_f = torch.empty(api.chunks_workspace_size(w.B, w.S, w.Hq, w.Hkv, w.D, len(cd_np), False),
                           dtype=torch.uint8, device=dev)
        ws_b = torch.empty(api.chunks_workspace_size(w.B, w.S, w.Hq, w.Hkv, w.D, len(cd_np), True),
                           dtype=torch.uint8, device=dev)

    # Events between the forward and the backward call of every step split
    # the step time; they are on the same stream as the calls.
    marks = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(args.steps)]

    # By default the step runs as the autograd function does: one workspace
    # sized for the backward, which reuses the forward's positions, plan and
    # rotated q, k (AA_FLAG_FWD_WORKSPACE).  Every step still computes them once.
    reuse = chunk_doc is None and not args.no_fwd_workspace
    if reuse:
        ws_f = ws_b
    bflags = flags | (api.FLAG_FWD_WORKSPACE if reuse else 0)

    def step(mark=None):
        if mark is not None:
            mark[2].record()
        if chunk_doc is not None:
            o, lse = api.anchor_attn_fwd_chunks(qc, kc, vc, cu, chunk_doc, w.rope_base, True, None,
                                                ws_f, flags=flags)
        else:
            o, lse = api.anchor_attn_fwd(qc, kc, vc, cu, w.rope_base, True, None, ws_f, flags=flags)
        if mark is not None:
            mark[0].record()
        if w.backward and chunk_doc is not None:
            api.anchor_attn_bwd_chunks(qc, kc, vc, o, lse, doc, cu, chunk_doc, w.rope_base, True,
                                       None, ws_b, flags=flags)
        elif w.backward:
            api.anchor_attn_bwd(qc, kc, vc, o, lse, doc, cu, w.rope_base, True, None, ws_b,
                                flags=bflags)
        if mark is not None:
            mark[1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # The timed steps: no per-kernel events (the library's profiling is off),
    # only the events around the whole region and between fwd and bwd.
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        step(marks[i])
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    bwd_ms = sum(a.elapsed_time(b) for a, b, _ in marks) / args.steps
    fwd_ms = ms - bwd_ms
    per_step = sorted(c.elapsed_time(b) for a, b, c in marks)     # start of step -> end of backward
    median_ms = per_step[len(per_step) // 2]
    # A second pass of as many steps with the library's per-kernel HIP events
    # (recorded on the call's stream around every launch) gives the kernel
    # times of the roofline.
    api.profile_begin(64 * max(1, args.steps))
    p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    p0.record()
    for i in range(args.steps):
        step()
    p1.record()
    torch.cuda.synchronize()
    prof = api.profile_end()
    profiled_ms = p0.elapsed_time(p1) / args.steps
    # The engine clock under this load: the firmware's metrics refresh about
    # once a second, so the same steps run on for a few refreshes.
    clk = ClockSampler()
    if args.clock_s > 0 and clk._smi is not None:
        t_end = time.perf_counter() + args.clock_s
        with clk:
            while time.perf_counter() < t_end:
                for _ in range(5):
                    step()
                torch.cuda.synchronize()

    # The same step captured once in a HIP graph and replayed: the kernels and
    # their work are identical, the host launch gaps between them are gone.
    graph_ms = None
    if args.graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        for _ in range(2):
            graph.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        for _ in range(args.steps):
            graph.replay()
        g1.record()
        torch.cuda.synchronize()
        graph_ms = g0.elapsed_time(g1) / args.steps
        del graph

    fl = flops_fwd_bwd(doc_rows, w.Hq, w.D, anchor=anchor)
    total_flops = fl["total"] if w.backward else fl["fwd"]
    tflops = total_flops / (ms * 1e-3) / 1e12
    tokens = w.B * w.S
    per_kernel_ms = {k_: v_[0] / max(1, args.steps) for k_, v_ in prof.items()}
    nbytes = algorithmic_bytes(w.B, w.S, w.Hq, w.Hkv, w.D, w.backward)

    # dominant kernel and its roofline
    cand = [k_ for k_ in KERNEL_FLOPS_PER_PAIR_D if prof[k_][1] > 0]
    dom = max(cand, key=lambda k_: prof[k_][0])
    launches = prof[dom][1]
    avg_ms = prof[dom][0] / launches
    algo = KERNEL_FLOPS_PER_PAIR_D[dom] * w.D * w.Hq * fl["pairs_per_head"]
    algo_bytes = kernel_algorithmic_bytes(dom, w.B, w.S, w.Hq, w.Hkv, w.D)
    # bound by its flops per byte against the ridge point of the two peaks
    # (2.5 PFLOP/s / 8 TB/s = 312.5 flop/B): the short-documents workload's
    # kernels fall below it
    rp = roofline_point(algo, algo_bytes, avg_ms * 1e-3, PEAK_BF16_TFLOPS, PEAK_HBM_GBS)
    clock = clk.summary()
    dpk = device_peak()
    clock_peak = None
    if clock and dpk:
        # dense bf16 MFMA rate at the engine clock measured during the steps
        clock_peak = dpk["compute_units"] * clock["gfx_mhz_mean"] * 1e6 * 4096 / 1e12
        clock["bf16_dense_peak_tflops_at_clock"] = clock_peak
    roofline = {"bound": rp["bound"], "kernel": f"k_{dom}", "achieved": rp["achieved"],
                "peak": rp["peak"], "unit": rp["unit"], "frac": rp["frac"],
                "frac_at_measured_clock": (rp["achieved"] / clock_peak
                                           if clock_peak and rp["unit"] == "TFLOP/s" else None),
                "traffic": _traffic(dom, w.name) if args.mode == "anchor" else None,
                "avg_launch_ms": avg_ms,
                "algorithmic_flops_per_launch": algo,
                "algorithmic_bytes_per_launch": algo_bytes,
                "flop_per_byte": rp["flop_per_byte"]}

    out = {
        "metric": ("AnchorAttention fwd+bwd unmasked TFLOP/s at 64K (also tokens/s, % of dense bf16 MFMA peak)"
                   if args.mode == "anchor" else
                   f"{args.mode} baseline fwd+bwd unmasked TFLOP/s (same kernels; also tokens/s)"),
        "value": tflops, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "ms_per_step_median": median_ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name if args.mode == "anchor" else f"{w.name}_{args.mode}",
                   "mode": args.mode, "batch": w.B, "seq_len": w.S, "q_heads": w.Hq, "kv_heads": w.Hkv,
                   "head_dim": w.D, "rope_base": w.rope_base, "documents_per_row": len(doc_rows[0]),
                   "backward": w.backward, "unmasked_pairs_per_head": fl["pairs_per_head"],
                   "bwd_reuses_forward_workspace": reuse,
                   "tile_grid": "after the anchor" if flags & api.FLAG_GRID_AFTER_ANCHOR else "from the first token"},
        "graph_ms_per_step": graph_ms,
        "graph_tflops": (total_flops / (graph_ms * 1e-3) / 1e12) if graph_ms else None,
        "tokens_per_s": tokens / (ms * 1e-3),
        "pct_of_bf16_peak": 100.0 * tflops / PEAK_BF16_TFLOPS,
        "pct_of_bf16_peak_at_measured_clock": (100.0 * tflops / clock_peak) if clock_peak else None,
        "clock": clock,
        "profiled_ms_per_step": profiled_ms,
        "fwd_ms": fwd_ms, "bwd_ms": bwd_ms if w.backward else None,
        "tflops_no_recompute": ((fl["total_no_recompute"] if w.backward else fl["fwd"])
                                / (ms * 1e-3) / 1e12),
        "algorithmic_hbm_bytes": nbytes["total"],
        "algorithmic_hbm_gbs": nbytes["total"] / (ms * 1e-3) / 1e9,
        "pct_of_hbm_peak": 100.0 * nbytes["total"] / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "device": dpk,
        "kernel_ms_per_step": {k_: round(v_, 4) for k_, v_ in per_kernel_ms.items()},
        "roofline": roofline,
    }
    if args.cpu_budget > 0 and args.mode == "anchor":
        cb = cpu_baseline(w, q, k, v, do, args.cpu_budget)
        # the whole workload at the oracle's measured rate
        cb["full_workload_estimate_s"] = total_flops / (cb["value"] * 1e12)
        out["cpu_baseline"] = cb
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
