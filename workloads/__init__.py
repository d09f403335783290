"""Seeded synthetic inputs for AnchorAttention workloads.

This module is shared by the CPU oracle's tests, the GPU tests and the
benchmark.  It only draws random numbers and lays documents out in a packed
sequence; it holds none of the attention method's arithmetic (no position
IDs, no rotation, no mask, no softmax).

Workloads follow the packed long-context training setting of "When Precision
Meets Position: BFloat16 Breaks Down RoPE in Long-Context Training"
(arXiv 2411.13476): one shared anchor token at the start of every packed row,
followed by whole documents.  The pages give no document-length distribution,
so lengths are drawn from a clipped lognormal that stands in for SlimPajama
packs; no dataset item is used.

Recipe:
* document lengths: ``numpy.random.default_rng(seed)``; repeatedly draw
  z ~ N(0,1) with ``standard_normal()``, take L = round(exp(ln(median) + sigma*z)),
  clip to [lo, hi], cap at the tokens still free, until the S-1 tokens after
  the anchor are filled (the last document is the remainder, no padding);
* Q, K, V, dO: ``torch.Generator('cpu').manual_seed(seed)``, ``torch.randn``
  in float32 drawn in the order Q, K, V, dO, then rounded to bfloat16 (RNE).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "sample_doc_lengths", "cu_doc_lens_from_lengths", "cu_doc_lens_no_anchor", "rows_without_anchor", "interleaved_chunks",
    "make_tensors", "random_partition", "get",
]


def sample_doc_lengths(S: int, median: float, sigma: float, lo: int, hi: int, seed: int) -> list[int]:
    """Clipped-lognormal document lengths that fill the S-1 slots after the anchor."""
    rng = np.random.default_rng(seed)
    remaining = S - 1
    out: list[int] = []
    while remaining > 0:
        z = rng.standard_normal()
        L = int(round(math.exp(math.log(median) + sigma * z)))
        L = min(max(L, lo), hi)
        L = min(L, remaining)
        out.append(L)
        remaining -= L
    return out


def cu_doc_lens_from_lengths(rows: list[list[int]], S: int) -> np.ndarray:
    """Cumulative segment offsets over the flattened B*S token stream.

    Every row b starts with a one-token anchor segment [b*S, b*S+1), followed by
    that row's documents; the lengths of each row must add up to S-1.
    """
    cu = [0]
    for b, lens in enumerate(rows):
        if sum(lens) != S - 1:
            raise ValueError(f"row {b}: document lengths sum to {sum(lens)}, expected {S - 1}")
        cu.append(cu[-1] + 1)
        for L in lens:
            cu.append(cu[-1] + L)
    return np.asarray(cu, dtype=np.int32)


def cu_doc_lens_no_anchor(rows: list[list[int]], S: int) -> np.ndarray:
    """Segment offsets for rows without an anchor: the documents of each row
    cover it from its first token on, so their lengths add up to S."""
    cu = [0]
    for b, lens in enumerate(rows):
        if sum(lens) != S:
            raise ValueError(f"row {b}: document lengths sum to {sum(lens)}, expected {S}")
        for L in lens:
            cu.append(cu[-1] + L)
    return np.asarray(cu, dtype=np.int32)


def rows_without_anchor(rows: list[list[int]]) -> list[list[int]]:
    """The same documents laid out without an anchor: the first document of
    each row also takes the anchor's slot, so every row still holds S tokens."""
    return [[lens[0] + 1] + list(lens[1:]) if len(lens) else [1] for lens in rows]


def interleaved_chunks(rows: list[list[int]], S: int, rng: np.random.Generator,
                       max_chunks_per_doc: int = 4, anchor: bool = True):
    """Interleaved-chunk packing (documents cut at random points, the chunks of
    a row shuffled with every document keeping its own order): each document of
    length L is cut into min(L, 1 + integers(max_chunks_per_doc)) chunks, then
    the rows are assembled by repeatedly taking the next chunk of a randomly
    chosen document that still has chunks.  Returns (cu, chunk_doc): segment
    offsets over the flattened B*S stream and a document id per segment, the
    anchor segment (when ``anchor``) getting id -1."""
    cu = [0]
    doc_ids = []
    for b, lens in enumerate(rows):
        if sum(lens) != (S - 1 if anchor else S):
            raise ValueError(f"row {b}: document lengths do not fill the row")
        pending = []
        for d, L in enumerate(lens):
            n = int(min(L, 1 + rng.integers(max_chunks_per_doc)))
            cuts = np.sort(rng.choice(np.arange(1, L), size=n - 1, replace=False)) if n > 1 else []
            edges = [0, *[int(c) for c in cuts], L]
            pending.append([d, [edges[i + 1] - edges[i] for i in range(n)]])
        if anchor:
            cu.append(cu[-1] + 1)
            doc_ids.append(-1)
        while pending:
            i = int(rng.integers(len(pending)))
            d, chunks = pending[i]
            cu.append(cu[-1] + chunks.pop(0))
            doc_ids.append(d)
            if not chunks:
                pending.pop(i)
    return np.asarray(cu, dtype=np.int32), np.asarray(doc_ids, dtype=np.int32)


def random_partition(rng: np.random.Generator, S: int, max_docs: int | None = None) -> list[int]:
    """A random split of S-1 tokens into documents (for small property tests)."""
    n = S - 1
    if n == 0:
        return []
    k = int(rng.integers(1, (max_docs or n) + 1))
    k = min(k, n)
    cuts = np.sort(rng.choice(np.arange(1, n), size=k - 1, replace=False)) if k > 1 else np.array([], dtype=int)
    edges = np.concatenate([[0], cuts, [n]])
    return [int(x) for x in np.diff(edges)]


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    S: int
    Hq: int
    Hkv: int
    D: int
    rope_base: float
    backward: bool
    doc_rows: tuple = field(repr=False)   # tuple of tuples of document lengths, one per row
    tensor_seed: int = 1000
    description: str = ""

    @property
    def cu_doc_lens(self) -> np.ndarray:
        return cu_doc_lens_from_lengths([list(r) for r in self.doc_rows], self.S)

    @property
    def n_seg(self) -> int:
        return len(self.cu_doc_lens) - 1


def _mk_workloads() -> dict[str, Workload]:
    w = {}
    w["tiny"] = Workload(
        "tiny", 1, 256, 2, 2, 64, 1e4, False, ((80, 100, 75),), 1000,
        "batch 1, seq 256 = anchor + documents 80/100/75, 2 heads, head_dim 64, base 1e4, forward only")
    w["8k"] = Workload(
        "8k", 1, 8192, 32, 32, 128, 5e6, True,
        (tuple(sample_doc_lengths(8192, 1024, 1.0, 64, 8191, 1)),), 1001,
        "LLaMA-2-7B attention shape: batch 1, seq 8192, 32 heads, head_dim 128, lognormal docs (median 1024, sigma 1.0)")
    w["64k"] = Workload(
        "64k", 1, 65536, 32, 32, 128, 5e6, True,
        (tuple(sample_doc_lengths(65536, 2048, 1.2, 64, 65535, 2)),), 1002,
        "long context: batch 1, seq 65536, 32 heads, head_dim 128, lognormal docs (median 2048, sigma 1.2)")
    w["128k_gqa"] = Workload(
        "128k_gqa", 1, 131072, 32, 8, 128, 5e5, True,
        (tuple(sample_doc_lengths(131072, 4096, 1.2, 64, 131071, 3)),), 1003,
        "GQA: batch 1, seq 131072, 32 query heads / 8 KV heads, head_dim 128, lognormal docs (median 4096, sigma 1.2)")
    w["64k_ulysses8"] = Workload(
        "64k_ulysses8", 1, 65536, 4, 4, 128, 5e6, True, w["64k"].doc_rows, 1005,
        "one GPU's share of the 64K workload under head sharding over 8 GPUs (Ulysses): the same "
        "documents, 4 of the 32 heads")
    short_row = tuple([256] * 127 + [32768 - 1 - 127 * 256])
    w["short_docs"] = Workload(
        "short_docs", 2, 32768, 32, 32, 128, 5e6, True, (short_row, short_row), 1004,
        "sparsity stress: batch 2, seq 32768, 32 heads, head_dim 128, 127 documents of 256 tokens + remainder per row")
    return w


WORKLOADS: dict[str, Workload] = _mk_workloads()


def get(name: str) -> Workload:
    return WORKLOADS[name]


def make_tensors(B: int, S: int, Hq: int, Hkv: int, D: int, seed: int, with_grad_out: bool = True):
    """Seeded bf16 Q [B,S,Hq,D], K/V [B,S,Hkv,D] and dO [B,S,Hq,D] on the CPU."""
    import torch
    g = torch.Generator("cpu").manual_seed(seed)
    q = torch.randn((B, S, Hq, D), generator=g, dtype=torch.float32).to(torch.bfloat16)
    k = torch.randn((B, S, Hkv, D), generator=g, dtype=torch.float32).to(torch.bfloat16)
    v = torch.randn((B, S, Hkv, D), generator=g, dtype=torch.float32).to(torch.bfloat16)
    do = None
    if with_grad_out:
        do = torch.randn((B, S, Hq, D), generator=g, dtype=torch.float32).to(torch.bfloat16)
    return q, k, v, do
