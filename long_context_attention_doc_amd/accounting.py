"""Work accounting for the benchmark (host arithmetic on document lengths).

Counting rule (paper-graph architecture page of arXiv 2411.13476, section
3.4, "Reduction in attention computations": each token attends within its own
document plus the anchor): in one packed row the anchor sees itself, and a
document of N tokens contributes N(N+1)/2 causal in-document pairs plus N
pairs with the anchor.  FLOPs count only these unmasked pairs: 4*D per pair
and query head for the forward (two products), 10*D for the backward (five
products, the usual flash-attention convention that includes recomputing the
scores), 14*D in total.
"""
from __future__ import annotations


def unmasked_pairs_closed_form(doc_rows, causal: bool = True, anchor: bool = True) -> int:
    """Without an anchor (the intra-document baselines) a document of N tokens
    contributes only its N(N+1)/2 causal pairs."""
    total = 0
    for lens in doc_rows:
        total += 1 if anchor else 0
        for n in lens:
            total += (n * (n + 1) // 2 if causal else n * n) + (n if anchor else 0)
    return total


def flops_fwd_bwd(doc_rows, Hq: int, D: int, causal: bool = True, anchor: bool = True) -> dict:
    pairs = unmasked_pairs_closed_form(doc_rows, causal, anchor)
    return {
        "pairs_per_head": pairs,
        "fwd": 4.0 * D * Hq * pairs,
        "bwd": 10.0 * D * Hq * pairs,
        "total": 14.0 * D * Hq * pairs,
        # without recomputing the scores in the backward: 4*D + 8*D
        "total_no_recompute": 12.0 * D * Hq * pairs,
    }


def algorithmic_bytes(B: int, S: int, Hq: int, Hkv: int, D: int, backward: bool = True) -> dict:
    """Minimum HBM traffic of one forward (+ backward) call: every operand
    read once and every result written once, in the library's dtypes (bf16
    tensors, float32 LSE).  Each call also rotates Q and K once (read the
    inputs, write the rotated copies)."""
    xq = 2 * B * S * Hq * D          # one [B,S,Hq,D] bf16 tensor
    xk = 2 * B * S * Hkv * D
    lse = 4 * B * Hq * S
    rope = 2 * (xq + xk)
    fwd = (xq + 2 * xk) + xq + lse + rope                       # Q K V in, O LSE out
    bwd = (xq + 2 * xk + xq + xq + lse) + (xq + 2 * xk) + rope  # Q K V O dO LSE in, dQ dK dV out
    return {"fwd": fwd, "bwd": bwd if backward else 0, "total": fwd + (bwd if backward else 0)}


def kernel_algorithmic_bytes(kernel: str, B: int, S: int, Hq: int, Hkv: int, D: int) -> int:
    """Minimum HBM traffic of one launch of a kernel of the path: each operand
    it needs read once, each result written once (bf16 tensors, float32 per-row
    values [B,Hq,S]).
      fwd       reads q (unrotated), k', v; writes q' (for the backward), O, LSE
      bwd_pre   reads q', O, dO, LSE; writes Dv and the anchor column's dS
      bwd_dkdv  reads q', k', v, dO; writes dK, dV
      bwd_dq    reads q', k', v, dO, LSE, Dv, the anchor column's dS; writes dQ
    The per-tile query records and the anchor partial sums (a few bytes per
    row) are left out."""
    xq = 2 * B * S * Hq * D
    xk = 2 * B * S * Hkv * D
    row = 4 * B * Hq * S          # one float32 value per row and query head
    table = {
        "fwd": 3 * xq + 2 * xk + row,
        "bwd_pre": 3 * xq + 3 * row,
        "bwd_dkdv": 2 * xq + 4 * xk,
        "bwd_dq": 3 * xq + 2 * xk + 3 * row,
    }
    return table[kernel]


def roofline_point(flops: float, nbytes: float, seconds: float, peak_tflops: float,
                   peak_gbs: float) -> dict:
    """Where one launch sits on the roofline: bound by the matrix cores when
    its flops per byte reach the ridge point peak_flops / peak_bandwidth,
    else by HBM.  `achieved` and `peak` are in TFLOP/s or GB/s accordingly."""
    intensity = flops / nbytes
    ridge = peak_tflops * 1e12 / (peak_gbs * 1e9)
    if intensity >= ridge:
        achieved, peak, bound, unit = flops / seconds / 1e12, peak_tflops, "mfma", "TFLOP/s"
    else:
        achieved, peak, bound, unit = nbytes / seconds / 1e9, peak_gbs, "hbm", "GB/s"
    return {"bound": bound, "achieved": achieved, "peak": peak, "unit": unit, "frac": achieved / peak,
            "flop_per_byte": intensity}
