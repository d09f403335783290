"""CPU checks of the C ABI: the library loads, exports every declared entry
point, and rejects bad arguments before launching anything (these calls
return before any HIP runtime call, so no GPU is needed)."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "anchor_attn.h")


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(anchor_attn_\w+)\s*\(", txt)))


@pytest.fixture(scope="module")
def lib():
    from long_context_attention_doc_amd import api
    return api.load()


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("anchor_attn_fwd", "anchor_attn_bwd", "anchor_attn_position_ids",
              "anchor_attn_tile_plan", "anchor_attn_rope", "anchor_attn_workspace_size"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    from long_context_attention_doc_amd import api
    names = _declared()
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(api.EXPORTS) == names


def test_version_and_strerror(lib):
    assert b"gfx950" in lib.anchor_attn_version()
    for code in range(6):
        assert lib.anchor_attn_strerror(code)


def test_workspace_sizes(lib):
    f = lib.anchor_attn_workspace_size
    assert f(1, 65536, 32, 32, 128, 0) > 0
    assert f(1, 65536, 32, 32, 128, 1) > f(1, 65536, 32, 32, 128, 0)
    assert f(1, 256, 32, 8, 96, 0) == 0        # unsupported D
    assert f(1, 256, 30, 8, 128, 0) == 0       # Hq % Hkv != 0
    assert lib.anchor_attn_plan_capacity(1, 300, 64, 128) == 5 * 3
    assert lib.anchor_attn_plan_capacity(1, 300, 48, 128) == 0
    # empty and degenerate shapes: no rows, no tokens, no heads, heads that do
    # not group, more than 2^31 - 1 tokens in all
    for shape in [(0, 256, 4, 2, 128), (1, 0, 4, 2, 128), (1, 256, 0, 1, 128), (1, 256, 4, 0, 128),
                  (1, 256, 3, 2, 128), (2, 1 << 30, 4, 2, 128)]:
        for for_bwd in (0, 1):
            assert f(*shape, for_bwd) == 0, shape
    # the smallest shape (one row of one token: the anchor alone) is valid
    assert f(1, 1, 1, 1, 64, 1) > 0


def test_argument_errors_before_launch(lib):
    from long_context_attention_doc_amd import api
    P = ctypes.c_void_p
    fake = P(0x1000)          # never dereferenced: every call below fails validation first
    def fwd(q=fake, Hq=4, Hkv=2, D=128, ws=fake, wsn=1 << 40, base=1e4, n_seg=4):
        return lib.anchor_attn_fwd(q, fake, fake, fake, n_seg, base, 1, 1, 256, Hq, Hkv, D, 0.0,
                                   fake, fake, ws, wsn, None)
    assert fwd(q=None) == api.AA_EINVAL
    assert fwd(Hq=3) == api.AA_EINVAL
    assert fwd(D=96) == api.AA_EUNSUPPORTED
    assert fwd(wsn=16) == api.AA_EWORKSPACE
    assert fwd(base=-1.0) == api.AA_EINVAL
    assert fwd(ws=P(0x1010)) == api.AA_EINVAL          # workspace not 256-byte aligned
    assert fwd(q=P(0x1002)) == api.AA_EINVAL           # tensor not 16-byte aligned
    assert fwd(n_seg=0) == api.AA_EINVAL
    rc = lib.anchor_attn_bwd(fake, fake, fake, fake, fake, None, fake, 4, 1e4, 1, 1, 256, 4, 2, 128,
                             0.0, fake, fake, fake, fake, 1 << 40, None)
    assert rc == api.AA_EINVAL
    rc = lib.anchor_attn_tile_plan(fake, 4, 1, 256, 48, 64, 1, 0, fake, fake, fake, fake, fake, fake,
                                   fake, fake, 1 << 40, None)
    assert rc == api.AA_EUNSUPPORTED
    # unknown option bits are rejected before anything is launched (a bit no
    # option will take: a call that passed validation would launch kernels)
    UNKNOWN = 1 << 20
    rc = lib.anchor_attn_tile_plan(fake, 4, 1, 256, 64, 64, 1, 4, fake, fake, fake, fake, fake, fake,
                                   fake, fake, 1 << 40, None)
    assert rc == api.AA_EINVAL
    rc = lib.anchor_attn_fwd_ex(fake, fake, fake, fake, 4, 1e4, 1, UNKNOWN, 1, 256, 4, 2, 128, 0.0,
                                fake, fake, fake, 1 << 40, None)
    assert rc == api.AA_EINVAL
    # the forward-workspace promise is only for the forward/backward pair
    rc = lib.anchor_attn_position_ids(fake, 4, 1, 256, 4, fake, fake, 1 << 40, None)
    assert rc == api.AA_EINVAL
    rc = lib.anchor_attn_fwd_chunks(fake, fake, fake, fake, fake, 4, 1e4, 1, 4, 1, 256, 4, 2, 128,
                                    0.0, fake, fake, fake, 1 << 40, None)
    assert rc == api.AA_EINVAL
    rc = lib.anchor_attn_bwd_ex(fake, fake, fake, fake, fake, fake, fake, 4, 1e4, 1, UNKNOWN, 1, 256, 4, 2,
                                128, 0.0, fake, fake, fake, fake, 1 << 40, None)
    assert rc == api.AA_EINVAL
    rc = lib.anchor_attn_position_ids(fake, 4, 1, 256, 4, fake, fake, 1 << 40, None)
    assert rc == api.AA_EINVAL
    # work order: null arrays or no tiles are rejected before any launch
    assert lib.anchor_attn_tile_order(None, 4, fake, None) == api.AA_EINVAL
    assert lib.anchor_attn_tile_order(fake, 0, fake, None) == api.AA_EINVAL
    assert lib.anchor_attn_tile_order(fake, 4, None, None) == api.AA_EINVAL
    # the float32-output option is for the attention entry points only
    assert api.FLAG_O_FP32 == 8
    rc = lib.anchor_attn_position_ids(fake, 4, 1, 256, api.FLAG_O_FP32, fake, fake, 1 << 40, None)
    assert rc == api.AA_EINVAL
    rc = lib.anchor_attn_tile_plan(fake, 4, 1, 256, 64, 64, 1, api.FLAG_O_FP32, fake, fake, fake, fake,
                                   fake, fake, fake, fake, 1 << 40, None)
    assert rc == api.AA_EINVAL
    rc = lib.anchor_attn_chunk_layout(fake, fake, 4, 1, 256, 1, api.FLAG_O_FP32, fake, fake, fake,
                                      1 << 40, None)
    assert rc == api.AA_EINVAL
    # interleaved-chunk entry points: null chunk arrays, unknown flags, too few chunks
    rc = lib.anchor_attn_fwd_chunks(fake, fake, fake, None, fake, 4, 1e4, 1, 0, 1, 256, 4, 2, 128,
                                    0.0, fake, fake, fake, 1 << 40, None)
    assert rc == api.AA_EINVAL
    rc = lib.anchor_attn_fwd_chunks(fake, fake, fake, fake, fake, 4, 1e4, 1, UNKNOWN, 1, 256, 4, 2, 128,
                                    0.0, fake, fake, fake, 1 << 40, None)
    assert rc == api.AA_EINVAL
    rc = lib.anchor_attn_bwd_chunks(fake, fake, fake, fake, fake, fake, fake, fake, 1, 1e4, 1, 0, 2,
                                    256, 4, 2, 128, 0.0, fake, fake, fake, fake, 1 << 40, None)
    assert rc == api.AA_EINVAL
    assert lib.anchor_attn_chunks_workspace_size(1, 256, 4, 2, 96, 4, 0) == 0
    assert lib.anchor_attn_chunks_workspace_size(1, 256, 4, 2, 128, 4, 1) > \
        lib.anchor_attn_workspace_size(1, 256, 4, 2, 128, 1)
    rc = lib.anchor_attn_chunk_layout(fake, fake, 4, 1, 256, 1, 0, fake, fake, fake, 16, None)
    assert rc == api.AA_EWORKSPACE
    rc = lib.anchor_attn_rope(fake, fake, 1, 256, 2, 80, 1e4, fake, fake, None)
    assert rc == api.AA_EUNSUPPORTED


def test_python_binding_checks_host_cu():
    """The binding validates a host cu_doc_lens before any launch: layout
    errors raise ValueError naming cu_doc_lens; a valid layout gets past the
    check (and stops at the CPU tensors)."""
    import torch
    from long_context_attention_doc_amd import api
    q = torch.zeros((2, 8, 2, 64), dtype=torch.bfloat16)
    kv = torch.zeros((2, 8, 1, 64), dtype=torch.bfloat16)
    bad = {
        "not ending at B*S": [0, 1, 8, 9, 15],
        "empty segment": [0, 1, 1, 8, 9, 16],
        "crossing a row": [0, 1, 10, 16],
        "no anchor segment": [0, 8, 9, 16],
    }
    for why, cu in bad.items():
        with pytest.raises(ValueError, match="cu_doc_lens|anchor|row"):
            api.anchor_attn_fwd(q, kv, kv, np.asarray(cu, dtype=np.int32), 1e4)
    # without the anchor option a row may start with a document
    with pytest.raises(ValueError, match="CUDA"):
        api.anchor_attn_fwd(q, kv, kv, np.asarray([0, 8, 9, 16], dtype=np.int32), 1e4,
                            flags=api.FLAG_NO_ANCHOR)
    with pytest.raises(ValueError, match="CUDA"):
        api.anchor_attn_fwd(q, kv, kv, np.asarray([0, 1, 5, 8, 9, 16], dtype=np.int32), 1e4)
    with pytest.raises(ValueError, match="cu_doc_lens"):
        api.anchor_attn_bwd(q, kv, kv, q, torch.zeros((2, 2, 8)), q, [0, 1, 8, 9, 15], 1e4)


def test_python_binding_guards_the_forward_workspace_and_autograd_cu():
    """FLAG_FWD_WORKSPACE without the forward's (backward-sized) workspace is
    rejected before anything is launched, and the autograd entry point checks
    a host cu_doc_lens before copying it to the device."""
    import torch
    from long_context_attention_doc_amd import api
    q = torch.zeros((1, 8, 2, 64), dtype=torch.bfloat16)
    kv = torch.zeros((1, 8, 1, 64), dtype=torch.bfloat16)
    lse = torch.zeros((1, 2, 8))
    cu = np.asarray([0, 1, 8], dtype=np.int32)
    small = torch.zeros(16, dtype=torch.uint8)
    for ws in (None, small):
        with pytest.raises(ValueError, match="FLAG_FWD_WORKSPACE"):
            api.anchor_attn_bwd(q, kv, kv, q, lse, q, cu, 1e4, workspace=ws,
                                flags=api.FLAG_FWD_WORKSPACE)
    with pytest.raises(ValueError, match="cu_doc_lens"):
        api.anchor_attention(q, kv, kv, np.asarray([0, 1, 7], dtype=np.int32), 1e4)
    with pytest.raises(ValueError, match="anchor"):
        api.anchor_attention(q, kv, kv, np.asarray([0, 8], dtype=np.int32), 1e4)


def test_noalloc_backward_refuses_what_does_not_fit(lib):
    """The allocation-free backward refuses, before any HIP call, shapes whose
    workspace exceeds its fixed scratch and the forward-workspace option."""
    from long_context_attention_doc_amd import api
    fake = ctypes.c_void_p(256)
    assert lib.anchor_attn_workspace_size(1, 32768, 32, 32, 128, 1) > api.NOALLOC_SCRATCH_BYTES
    assert lib.anchor_attn_workspace_size(1, 8192, 32, 32, 128, 1) <= api.NOALLOC_SCRATCH_BYTES
    rc = lib.anchor_attn_bwd_noalloc(fake, fake, fake, fake, fake, fake, fake, 2, 1e4, 1, 0, 1,
                                     32768, 32, 32, 128, 0.0, fake, fake, fake, None)
    assert rc == api.AA_EWORKSPACE
    rc = lib.anchor_attn_bwd_noalloc(fake, fake, fake, fake, fake, fake, fake, 2, 1e4, 1,
                                     api.FLAG_FWD_WORKSPACE, 1, 256, 2, 2, 64, 0.0, fake, fake,
                                     fake, None)
    assert rc == api.AA_EINVAL
    rc = lib.anchor_attn_bwd_noalloc(fake, fake, fake, fake, fake, fake, fake, 2, 1e4, 1, 0, 1,
                                     256, 3, 2, 64, 0.0, fake, fake, fake, None)
    assert rc == api.AA_EINVAL


def test_flag_constants_match_the_header(lib):
    """The binding's FLAG_* values are the header's AA_FLAG_* bits, and the
    stage entry points reject the attention-only options."""
    from long_context_attention_doc_amd import api
    text = open(HEADER).read()
    defs = dict(re.findall(r"#define AA_FLAG_(\w+) (\d+)", text))
    assert defs, "no AA_FLAG_ defines found"
    for name, val in defs.items():
        assert getattr(api, "FLAG_" + name) == int(val), name
    assert len(set(defs.values())) == len(defs)
    fake = ctypes.c_void_p(1 << 20)
    for f in (api.FLAG_O_FP32, api.FLAG_FWD_WORKSPACE):
        assert lib.anchor_attn_position_ids(fake, 4, 1, 256, f, fake, fake, 1 << 40, None) == api.AA_EINVAL
        assert lib.anchor_attn_chunk_layout(fake, fake, 4, 1, 256, 1, f, fake, fake, fake, 1 << 40,
                                            None) == api.AA_EINVAL
