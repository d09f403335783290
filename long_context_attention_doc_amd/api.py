"""Python binding of the AnchorAttention C ABI (include/anchor_attn.h).

Argument marshalling only: every step of the computation runs in the HIP
library.  PyTorch supplies device memory and the current stream.  The
library must be built (``python -m long_context_attention_doc_amd.build``);
if it is missing, every call raises instead of falling back to anything.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libanchor_attn.so")

AA_OK, AA_EINVAL, AA_EDOCS, AA_EUNSUPPORTED, AA_EWORKSPACE, AA_EHIP = range(6)
# Options (anchor_attn.h): continuous position IDs; rows without a shared anchor.
FLAG_CONTINUOUS_POS, FLAG_NO_ANCHOR = 1, 2
# anchor_attn_bwd: the workspace still holds the forward's state (see anchor_attn.h)
FLAG_FWD_WORKSPACE = 4
# O in float32 instead of bf16 (forward output and backward input)
FLAG_O_FP32 = 8
# anchor_attn_tile_plan: the tile grid after each row's anchor (the attention
# kernels' grid for rows with an anchor)
FLAG_GRID_AFTER_ANCHOR = 16
TILE_FULL, TILE_PARTIAL, TILE_ANCHOR = 1, 2, 3

# Tile shapes the attention kernels run with (query tile x key tile).
FWD_TILE = (128, 64)
DKV_TILE = (64, 128)

EXPORTS = (
    "anchor_attn_strerror", "anchor_attn_version", "anchor_attn_workspace_size",
    "anchor_attn_fwd", "anchor_attn_bwd", "anchor_attn_fwd_ex", "anchor_attn_bwd_ex",
    "anchor_attn_bwd_noalloc",
    "anchor_attn_chunks_workspace_size", "anchor_attn_fwd_chunks", "anchor_attn_bwd_chunks",
    "anchor_attn_chunk_layout",
    "anchor_attn_position_ids",
    "anchor_attn_plan_workspace_size", "anchor_attn_plan_capacity", "anchor_attn_tile_plan",
    "anchor_attn_tile_order", "anchor_attn_rope", "anchor_attn_device_status", "anchor_attn_profile_begin",
    "anchor_attn_profile_end",
)
KERNEL_IDS = ("status", "positions", "plan", "rope_table", "rope", "fwd", "bwd_pre", "bwd_dkdv",
              "bwd_dq", "bwd_anchor", "chunks", "gather")

_lib = None


class AnchorAttnError(RuntimeError):
    def __init__(self, code: int, where: str):
        msg = _lib.anchor_attn_strerror(code).decode() if _lib is not None else str(code)
        super().__init__(f"{where}: {msg} (status {code})")
        self.code = code


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"AnchorAttention HIP library not built: {path} is missing "
                          "(run `python -m long_context_attention_doc_amd.build`)")
    lib = ctypes.CDLL(path)
    P, I, D, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_double, ctypes.c_float, ctypes.c_size_t
    sig = {
        "anchor_attn_strerror": (ctypes.c_char_p, [I]),
        "anchor_attn_version": (ctypes.c_char_p, []),
        "anchor_attn_workspace_size": (Z, [I, I, I, I, I, I]),
        "anchor_attn_fwd": (I, [P, P, P, P, I, D, I, I, I, I, I, I, F, P, P, P, Z, P]),
        "anchor_attn_bwd": (I, [P, P, P, P, P, P, P, I, D, I, I, I, I, I, I, F, P, P, P, P, Z, P]),
        "anchor_attn_fwd_ex": (I, [P, P, P, P, I, D, I, I, I, I, I, I, I, F, P, P, P, Z, P]),
        "anchor_attn_bwd_ex": (I, [P, P, P, P, P, P, P, I, D, I, I, I, I, I, I, I, F, P, P, P, P, Z,
                                   P]),
        "anchor_attn_bwd_noalloc": (I, [P, P, P, P, P, P, P, I, D, I, I, I, I, I, I, I, F, P, P, P,
                                        P]),
        "anchor_attn_chunks_workspace_size": (Z, [I, I, I, I, I, I, I]),
        "anchor_attn_fwd_chunks": (I, [P, P, P, P, P, I, D, I, I, I, I, I, I, I, F, P, P, P, Z, P]),
        "anchor_attn_bwd_chunks": (I, [P, P, P, P, P, P, P, P, I, D, I, I, I, I, I, I, I, F, P, P, P, P,
                                       Z, P]),
        "anchor_attn_chunk_layout": (I, [P, P, I, I, I, I, I, P, P, P, Z, P]),
        "anchor_attn_position_ids": (I, [P, I, I, I, I, P, P, Z, P]),
        "anchor_attn_plan_workspace_size": (Z, [I, I, I, I]),
        "anchor_attn_plan_capacity": (Z, [I, I, I, I]),
        "anchor_attn_tile_plan": (I, [P, I, I, I, I, I, I, I, P, P, P, P, P, P, P, P, Z, P]),
        "anchor_attn_tile_order": (I, [P, I, P, P]),
        "anchor_attn_rope": (I, [P, P, I, I, I, I, D, P, P, P]),
        "anchor_attn_device_status": (I, [P, P, P]),
        "anchor_attn_profile_begin": (I, [I]),
        "anchor_attn_profile_end": (I, [P, P, I]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(code: int, where: str) -> None:
    if code != AA_OK:
        raise AnchorAttnError(code, where)


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dev_cu(cu, device) -> torch.Tensor:
    if not isinstance(cu, torch.Tensor):
        cu = torch.as_tensor(cu, dtype=torch.int32)
    return cu.to(device=device, dtype=torch.int32).contiguous()


def _check_host_cu(cu, B: int, S: int, anchor: bool) -> None:
    """The segment layout rules, checked on a host copy of cu_doc_lens before
    anything is launched (the device checks them again): cu[0] = 0, strictly
    increasing, cu[-1] = B*S, no segment crosses a row start, and with the
    anchor every row starts with a one-token anchor segment."""
    import numpy as np
    a = np.asarray(cu.cpu() if isinstance(cu, torch.Tensor) else cu, dtype=np.int64).reshape(-1)
    if a.size < 2 or a[0] != 0 or a[-1] != B * S:
        raise ValueError(f"cu_doc_lens must run from 0 to B*S = {B * S}")
    if np.any(np.diff(a) <= 0):
        raise ValueError("cu_doc_lens must be strictly increasing (no empty segment)")
    starts = np.arange(B, dtype=np.int64) * S
    if not np.all(np.isin(starts, a)):
        raise ValueError("a segment of cu_doc_lens crosses the start of a row")
    if anchor and S > 1 and not np.all(np.isin(starts + 1, a)):
        raise ValueError("every row must start with a one-token anchor segment")


def _check_cu(cu, B: int, S: int, flags: int) -> None:
    if not (isinstance(cu, torch.Tensor) and cu.is_cuda):
        _check_host_cu(cu, B, S, not flags & FLAG_NO_ANCHOR)


# Mean document length up to which the tile grid goes after the anchor.
GRID_AFTER_ANCHOR_MAX_MEAN_DOC = 512


def grid_flag(cu_doc_lens, B: int, S: int, flags: int = 0) -> int:
    """FLAG_GRID_AFTER_ANCHOR when rows carry an anchor and their documents
    are short on average (at most GRID_AFTER_ANCHOR_MAX_MEAN_DOC tokens; the
    grid after the anchor then saves whole tiles per document), else 0.  Read
    from a host copy of cu_doc_lens; a device copy gives 0."""
    import numpy as np
    if flags & FLAG_NO_ANCHOR or (isinstance(cu_doc_lens, torch.Tensor) and cu_doc_lens.is_cuda):
        return 0
    n_seg = np.asarray(cu_doc_lens.cpu() if isinstance(cu_doc_lens, torch.Tensor) else cu_doc_lens).size - 1
    n_docs = max(1, n_seg - B)
    return FLAG_GRID_AFTER_ANCHOR if B * (S - 1) <= GRID_AFTER_ANCHOR_MAX_MEAN_DOC * n_docs else 0


def _need_o(o: torch.Tensor, flags: int) -> None:
    want = torch.float32 if flags & FLAG_O_FP32 else torch.bfloat16
    if o.dtype != want or o.dim() != 4 or not o.is_cuda or not o.is_contiguous():
        raise ValueError(f"o must be a contiguous {want} CUDA tensor with 4 dims "
                         "(float32 exactly when FLAG_O_FP32 is set)")


def _need_bf16(name: str, t: torch.Tensor, ndim: int = 4) -> None:
    if t.dtype != torch.bfloat16 or t.dim() != ndim or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous bfloat16 CUDA tensor with {ndim} dims")


def version() -> str:
    return load().anchor_attn_version().decode()


def workspace_size(B: int, S: int, Hq: int, Hkv: int, D: int, for_bwd: bool) -> int:
    n = load().anchor_attn_workspace_size(B, S, Hq, Hkv, D, int(for_bwd))
    if n == 0:
        raise ValueError("unsupported shape")
    return int(n)


def _workspace(nbytes: int, device) -> torch.Tensor:
    # torch's caching allocator returns 512-byte aligned blocks
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def anchor_attn_fwd(q, k, v, cu_doc_lens, rope_base: float, causal: bool = True,
                    softmax_scale: float | None = None, workspace: torch.Tensor | None = None,
                    flags: int = 0):
    """Forward pass; returns (o [B,S,Hq,D] bf16, or float32 with FLAG_O_FP32; lse [B,Hq,S]
    fp32).  flags: OR of FLAG_CONTINUOUS_POS / FLAG_NO_ANCHOR / FLAG_O_FP32 (0 = the
    method with a bf16 output, anchor_attn_fwd).  A host cu_doc_lens is validated here
    before anything is launched."""
    lib = load()
    _check_cu(cu_doc_lens, q.shape[0], q.shape[1], flags)
    for n, t in (("q", q), ("k", k), ("v", v)):
        _need_bf16(n, t)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    if k.shape != (B, S, Hkv, D) or v.shape != k.shape:
        raise ValueError("k and v must be [B,S,Hkv,D] matching q")
    cu = _dev_cu(cu_doc_lens, q.device)
    ws_n = workspace_size(B, S, Hq, Hkv, D, False)
    if workspace is None or workspace.numel() < ws_n:
        workspace = _workspace(ws_n, q.device)
    o = torch.empty_like(q, dtype=torch.float32 if flags & FLAG_O_FP32 else torch.bfloat16)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
    if flags:
        _check(lib.anchor_attn_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(cu), cu.numel() - 1,
                                      float(rope_base), int(bool(causal)), int(flags), B, S, Hq,
                                      Hkv, D, float(softmax_scale or 0.0), _ptr(o), _ptr(lse),
                                      _ptr(workspace), workspace.numel(), _stream(q.device)),
               "anchor_attn_fwd_ex")
    else:
        _check(lib.anchor_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(cu), cu.numel() - 1,
                                   float(rope_base), int(bool(causal)), B, S, Hq, Hkv, D,
                                   float(softmax_scale or 0.0), _ptr(o), _ptr(lse), _ptr(workspace),
                                   workspace.numel(), _stream(q.device)), "anchor_attn_fwd")
    return o, lse


def anchor_attn_bwd(q, k, v, o, lse, dout, cu_doc_lens, rope_base: float, causal: bool = True,
                    softmax_scale: float | None = None, workspace: torch.Tensor | None = None,
                    flags: int = 0):
    """Backward pass; returns (dq, dk, dv) bf16.  flags as for anchor_attn_fwd."""
    lib = load()
    _check_cu(cu_doc_lens, q.shape[0], q.shape[1], flags)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    ws_n = workspace_size(B, S, Hq, Hkv, D, True)
    if (flags & FLAG_FWD_WORKSPACE) and (workspace is None or workspace.numel() < ws_n):
        # a fresh workspace does not hold the forward's positions, plan and
        # rotated q, k that the flag promises
        raise ValueError("FLAG_FWD_WORKSPACE needs the forward's workspace, sized for the "
                         f"backward ({ws_n} bytes)")
    for n, t in (("q", q), ("k", k), ("v", v), ("dout", dout)):
        _need_bf16(n, t)
    _need_o(o, flags)
    if lse.dtype != torch.float32 or lse.shape != (B, Hq, S) or not lse.is_contiguous():
        raise ValueError("lse must be contiguous float32 [B,Hq,S]")
    cu = _dev_cu(cu_doc_lens, q.device)
    if workspace is None or workspace.numel() < ws_n:
        workspace = _workspace(ws_n, q.device)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    if flags:
        _check(lib.anchor_attn_bwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout),
                                      _ptr(cu), cu.numel() - 1, float(rope_base), int(bool(causal)),
                                      int(flags), B, S, Hq, Hkv, D, float(softmax_scale or 0.0),
                                      _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                                      workspace.numel(), _stream(q.device)), "anchor_attn_bwd_ex")
    else:
        _check(lib.anchor_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout),
                                   _ptr(cu), cu.numel() - 1, float(rope_base), int(bool(causal)), B,
                                   S, Hq, Hkv, D, float(softmax_scale or 0.0), _ptr(dq), _ptr(dk),
                                   _ptr(dv), _ptr(workspace), workspace.numel(), _stream(q.device)),
               "anchor_attn_bwd")
    return dq, dk, dv


# Size of the device array behind anchor_attn_bwd_noalloc (AA_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 160 << 20


def anchor_attn_bwd_noalloc(q, k, v, o, lse, dout, cu_doc_lens, rope_base: float,
                            causal: bool = True, softmax_scale: float | None = None,
                            flags: int = 0, out=None):
    """The allocation-free backward: as anchor_attn_bwd, with the library's
    fixed per-device scratch as its workspace.  Shapes whose backward
    workspace exceeds NOALLOC_SCRATCH_BYTES are refused.  ``out`` may give
    (dq, dk, dv) to write into; otherwise they are allocated here (the library
    call itself allocates nothing)."""
    lib = load()
    _check_cu(cu_doc_lens, q.shape[0], q.shape[1], flags)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    need = workspace_size(B, S, Hq, Hkv, D, True)
    if need > NOALLOC_SCRATCH_BYTES:
        raise ValueError(f"anchor_attn_bwd_noalloc: this shape needs {need} bytes of scratch, more "
                         f"than the fixed {NOALLOC_SCRATCH_BYTES}")
    for n, t in (("q", q), ("k", k), ("v", v), ("dout", dout)):
        _need_bf16(n, t)
    _need_o(o, flags)
    if lse.dtype != torch.float32 or lse.shape != (B, Hq, S) or not lse.is_contiguous():
        raise ValueError("lse must be contiguous float32 [B,Hq,S]")
    cu = _dev_cu(cu_doc_lens, q.device)
    if out is None:
        out = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    dq, dk, dv = out
    for n, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _need_bf16(n, t)
        if t.shape != ref.shape:
            raise ValueError(f"{n} must have the shape of its input")
    _check(lib.anchor_attn_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout),
                                       _ptr(cu), cu.numel() - 1, float(rope_base), int(bool(causal)),
                                       int(flags), B, S, Hq, Hkv, D, float(softmax_scale or 0.0),
                                       _ptr(dq), _ptr(dk), _ptr(dv), _stream(q.device)),
           "anchor_attn_bwd_noalloc")
    return dq, dk, dv


def chunks_workspace_size(B: int, S: int, Hq: int, Hkv: int, D: int, n_chunks: int,
                          for_bwd: bool) -> int:
    n = load().anchor_attn_chunks_workspace_size(B, S, Hq, Hkv, D, n_chunks, int(for_bwd))
    if n == 0:
        raise ValueError("unsupported shape")
    return int(n)


def anchor_attn_fwd_chunks(q, k, v, cu_chunks, chunk_doc, rope_base: float, causal: bool = True,
                           softmax_scale: float | None = None, workspace: torch.Tensor | None = None,
                           flags: int = 0):
    """Forward pass over interleaved document chunks (cu_chunks [n+1], chunk_doc [n]
    int32); returns (o, lse) in the caller's token order."""
    lib = load()
    for n, t in (("q", q), ("k", k), ("v", v)):
        _need_bf16(n, t)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    cu = _dev_cu(cu_chunks, q.device)
    cd = _dev_cu(chunk_doc, q.device)
    if cd.numel() != cu.numel() - 1:
        raise ValueError("chunk_doc needs one id per chunk")
    ws_n = chunks_workspace_size(B, S, Hq, Hkv, D, cd.numel(), False)
    if workspace is None or workspace.numel() < ws_n:
        workspace = _workspace(ws_n, q.device)
    o = torch.empty_like(q, dtype=torch.float32 if flags & FLAG_O_FP32 else torch.bfloat16)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
    _check(lib.anchor_attn_fwd_chunks(_ptr(q), _ptr(k), _ptr(v), _ptr(cu), _ptr(cd), cd.numel(),
                                      float(rope_base), int(bool(causal)), int(flags), B, S, Hq, Hkv,
                                      D, float(softmax_scale or 0.0), _ptr(o), _ptr(lse),
                                      _ptr(workspace), workspace.numel(), _stream(q.device)),
           "anchor_attn_fwd_chunks")
    return o, lse


def anchor_attn_bwd_chunks(q, k, v, o, lse, dout, cu_chunks, chunk_doc, rope_base: float,
                           causal: bool = True, softmax_scale: float | None = None,
                           workspace: torch.Tensor | None = None, flags: int = 0):
    """Backward pass over interleaved document chunks; returns (dq, dk, dv)."""
    lib = load()
    for n, t in (("q", q), ("k", k), ("v", v), ("dout", dout)):
        _need_bf16(n, t)
    _need_o(o, flags)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    if lse.dtype != torch.float32 or lse.shape != (B, Hq, S) or not lse.is_contiguous():
        raise ValueError("lse must be contiguous float32 [B,Hq,S]")
    cu = _dev_cu(cu_chunks, q.device)
    cd = _dev_cu(chunk_doc, q.device)
    ws_n = chunks_workspace_size(B, S, Hq, Hkv, D, cd.numel(), True)
    if workspace is None or workspace.numel() < ws_n:
        workspace = _workspace(ws_n, q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    _check(lib.anchor_attn_bwd_chunks(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout),
                                      _ptr(cu), _ptr(cd), cd.numel(), float(rope_base),
                                      int(bool(causal)), int(flags), B, S, Hq, Hkv, D,
                                      float(softmax_scale or 0.0), _ptr(dq), _ptr(dk), _ptr(dv),
                                      _ptr(workspace), workspace.numel(), _stream(q.device)),
           "anchor_attn_bwd_chunks")
    return dq, dk, dv


def anchor_attn_chunk_layout(cu_chunks, chunk_doc, B: int, S: int, causal: bool = True,
                             flags: int = 0, device="cuda"):
    """(src, pos, workspace): for every token of the permuted rows its original
    token and its position ID."""
    lib = load()
    cu = _dev_cu(cu_chunks, device)
    cd = _dev_cu(chunk_doc, device)
    src = torch.empty(B * S, dtype=torch.int32, device=device)
    pos = torch.empty(B * S, dtype=torch.int32, device=device)
    ws = _workspace(chunks_workspace_size(B, S, 1, 1, 64, cd.numel(), False), device)
    _check(lib.anchor_attn_chunk_layout(_ptr(cu), _ptr(cd), cd.numel(), B, S, int(bool(causal)),
                                        int(flags), _ptr(src), _ptr(pos), _ptr(ws), ws.numel(),
                                        _stream(src.device)), "anchor_attn_chunk_layout")
    return src, pos, ws


def anchor_attn_position_ids(cu_doc_lens, B: int, S: int, flags: int = 0, device="cuda"):
    """Position IDs int32 [B*S]; flags as for anchor_attn_fwd (0: reset, with anchor)."""
    lib = load()
    cu = _dev_cu(cu_doc_lens, device)
    pos = torch.empty(B * S, dtype=torch.int32, device=device)
    ws = _workspace(lib.anchor_attn_plan_workspace_size(B, S, 64, 64), device)
    _check(lib.anchor_attn_position_ids(_ptr(cu), cu.numel() - 1, B, S, flags, _ptr(pos), _ptr(ws),
                                        ws.numel(), _stream(pos.device)),
           "anchor_attn_position_ids")
    return pos, ws


def anchor_attn_tile_plan(cu_doc_lens, B: int, S: int, BM: int, BN: int, causal: bool = True,
                          device="cuda", flags: int = 0):
    """Tile plan as a dict of device tensors (query-major and key-major CSR)."""
    lib = load()
    cu = _dev_cu(cu_doc_lens, device)
    cap = lib.anchor_attn_plan_capacity(B, S, BM, BN)
    if cap == 0:
        raise ValueError("unsupported tile size")
    nq, nk = -(-S // BM), -(-S // BN)
    i32 = dict(dtype=torch.int32, device=device)
    u8 = dict(dtype=torch.uint8, device=device)
    out = {
        "qptr": torch.empty(B * nq + 1, **i32), "kidx": torch.empty(cap, **i32),
        "kkind": torch.empty(cap, **u8), "kptr": torch.empty(B * nk + 1, **i32),
        "qidx": torch.empty(cap, **i32), "qkind": torch.empty(cap, **u8),
        "n_live": torch.empty(1, **i32),
    }
    ws = _workspace(lib.anchor_attn_plan_workspace_size(B, S, BM, BN), device)
    _check(lib.anchor_attn_tile_plan(_ptr(cu), cu.numel() - 1, B, S, BM, BN, int(bool(causal)),
                                     int(flags),
                                     _ptr(out["qptr"]), _ptr(out["kidx"]), _ptr(out["kkind"]),
                                     _ptr(out["kptr"]), _ptr(out["qidx"]), _ptr(out["qkind"]),
                                     _ptr(out["n_live"]), _ptr(ws), ws.numel(),
                                     _stream(ws.device)), "anchor_attn_tile_plan")
    out["workspace"] = ws
    out["nq"], out["nk"] = nq, nk
    return out


ORDER_LPT, ORDER_INTERLEAVE = 1, 2


def anchor_attn_tile_order(cnt: torch.Tensor) -> torch.Tensor:
    """Work order of a query-major plan: cnt int32 [n] (live key tiles per query
    tile) -> int32 [n + 1], the tiles in launch order and then the flags
    (ORDER_LPT, ORDER_INTERLEAVE)."""
    lib = load()
    if cnt.dtype != torch.int32 or cnt.dim() != 1 or not cnt.is_cuda or not cnt.is_contiguous():
        raise ValueError("cnt must be a contiguous int32 CUDA vector")
    out = torch.empty(cnt.numel() + 1, dtype=torch.int32, device=cnt.device)
    _check(lib.anchor_attn_tile_order(_ptr(cnt), cnt.numel(), _ptr(out), _stream(cnt.device)),
           "anchor_attn_tile_order")
    return out


def anchor_attn_rope(x, pos, rope_base: float):
    """RoPE stage alone: x [B,S,H,D] bf16, pos int32 [B*S] -> rotated bf16."""
    lib = load()
    _need_bf16("x", x)
    B, S, H, D = x.shape
    pos = pos.to(device=x.device, dtype=torch.int32).contiguous()
    y = torch.empty_like(x)
    table = torch.empty(S * D, dtype=torch.float32, device=x.device)
    _check(lib.anchor_attn_rope(_ptr(x), _ptr(pos), B, S, H, D, float(rope_base), _ptr(y),
                                _ptr(table), _stream(x.device)), "anchor_attn_rope")
    return y


def anchor_attn_device_status(workspace: torch.Tensor) -> int:
    lib = load()
    out = ctypes.c_int32(0)
    _check(lib.anchor_attn_device_status(_ptr(workspace), _stream(workspace.device),
                                         ctypes.byref(out)), "anchor_attn_device_status")
    return int(out.value)


def profile_begin(max_launches: int = 65536) -> None:
    _check(load().anchor_attn_profile_begin(max_launches), "anchor_attn_profile_begin")


def profile_end() -> dict:
    """{kernel name: (total ms, launches)} since profile_begin()."""
    n = len(KERNEL_IDS)
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int32 * n)()
    _check(load().anchor_attn_profile_end(ms, cnt, n), "anchor_attn_profile_end")
    return {KERNEL_IDS[i]: (float(ms[i]), int(cnt[i])) for i in range(n)}


class _AnchorAttnFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, cu, rope_base, causal, softmax_scale, flags):
        # one workspace sized for the backward: the backward reuses the
        # forward's positions, plan and rotated q, k left in it
        B, S, Hq, D = q.shape
        ws = _workspace(workspace_size(B, S, Hq, k.shape[2], D, True), q.device)
        o, lse = anchor_attn_fwd(q, k, v, cu, rope_base, causal, softmax_scale, ws, flags=flags)
        ctx.save_for_backward(q, k, v, o, lse, cu)
        ctx.ws = ws
        ctx.cfg = (rope_base, causal, softmax_scale, flags)
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse, cu = ctx.saved_tensors
        rope_base, causal, scale, flags = ctx.cfg
        # dO is taken in bf16 (an fp32 O's gradient arrives in fp32)
        # The workspace stays with ctx: the backward writes only past the
        # forward's part of it, so a second backward (retain_graph) finds the
        # forward's state again.
        dq, dk, dv = anchor_attn_bwd(q, k, v, o, lse, do.to(torch.bfloat16).contiguous(), cu,
                                     rope_base, causal, scale, ctx.ws, flags=flags | FLAG_FWD_WORKSPACE)
        return dq, dk, dv, None, None, None, None, None


def anchor_attention(q, k, v, cu_doc_lens, rope_base: float, causal: bool = True,
                     softmax_scale: float | None = None, flags: int = 0):
    """AnchorAttention with autograd: q [B,S,Hq,D], k/v [B,S,Hkv,D] bf16 on the GPU.
    A host cu_doc_lens is validated here, before it is copied to the device."""
    _check_cu(cu_doc_lens, q.shape[0], q.shape[1], flags)
    # the forward and its backward share the grid choice (and the workspace)
    flags |= grid_flag(cu_doc_lens, q.shape[0], q.shape[1], flags)
    cu = _dev_cu(cu_doc_lens, q.device)
    return _AnchorAttnFn.apply(q, k, v, cu, float(rope_base), bool(causal), softmax_scale, int(flags))
