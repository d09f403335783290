"""Host-side work accounting of the benchmark: per-kernel algorithmic bytes
and the roofline bound chosen from flops per byte (no GPU)."""
import pytest

import workloads as W
from long_context_attention_doc_amd.accounting import (flops_fwd_bwd, kernel_algorithmic_bytes,
                                                        roofline_point)

PEAK_TF, PEAK_GBS = 2500.0, 8000.0
FLOPS_PER_PAIR_D = {"fwd": 4.0, "bwd_dkdv": 8.0, "bwd_dq": 6.0}


def test_kernel_bytes_mha_and_gqa():
    B, S, H, D = 2, 1024, 4, 128
    x = 2 * B * S * H * D            # one [B,S,H,D] bf16 tensor
    lse = 4 * B * H * S
    assert kernel_algorithmic_bytes("fwd", B, S, H, H, D) == 5 * x + lse
    assert kernel_algorithmic_bytes("bwd_pre", B, S, H, H, D) == 3 * x + 3 * lse
    assert kernel_algorithmic_bytes("bwd_dkdv", B, S, H, H, D) == 6 * x
    assert kernel_algorithmic_bytes("bwd_dq", B, S, H, H, D) == 5 * x + 3 * lse
    # GQA: key-side tensors are Hkv wide
    xk = 2 * B * S * 1 * D
    assert kernel_algorithmic_bytes("bwd_dkdv", B, S, H, 1, D) == 2 * x + 4 * xk
    with pytest.raises(KeyError):
        kernel_algorithmic_bytes("rope", B, S, H, H, D)


def test_roofline_point_sides_of_the_ridge():
    ridge = PEAK_TF * 1e12 / (PEAK_GBS * 1e9)          # 312.5 flop/B
    assert ridge == pytest.approx(312.5)
    hi = roofline_point(1e12, 1e12 / 1000.0, 1e-3, PEAK_TF, PEAK_GBS)
    assert hi["bound"] == "mfma" and hi["unit"] == "TFLOP/s"
    assert hi["achieved"] == pytest.approx(1000.0) and hi["frac"] == pytest.approx(0.4)
    lo = roofline_point(1e9, 1e9, 1e-3, PEAK_TF, PEAK_GBS)
    assert lo["bound"] == "hbm" and lo["unit"] == "GB/s"
    assert lo["achieved"] == pytest.approx(1000.0) and lo["frac"] == pytest.approx(0.125)
    edge = roofline_point(312.5e6, 1e6, 1.0, PEAK_TF, PEAK_GBS)
    assert edge["bound"] == "mfma"


@pytest.mark.parametrize("name,bound", [("8k", "mfma"), ("64k", "mfma"), ("128k_gqa", "mfma"),
                                        ("64k_ulysses8", "mfma"), ("short_docs", "hbm")])
def test_bench_workloads_bound(name, bound):
    """The sparsity-stress workload's attention kernels sit below the ridge
    point (too few pairs per byte moved); the long-context ones far above."""
    w = W.get(name)
    fl = flops_fwd_bwd([list(r) for r in w.doc_rows], w.Hq, w.D)
    for kern, f in FLOPS_PER_PAIR_D.items():
        flops = f * w.D * w.Hq * fl["pairs_per_head"]
        nbytes = kernel_algorithmic_bytes(kern, w.B, w.S, w.Hq, w.Hkv, w.D)
        assert roofline_point(flops, nbytes, 1.0, PEAK_TF, PEAK_GBS)["bound"] == bound


def test_counter_summary_goes_stale_with_source_or_build_flags(monkeypatch, tmp_path):
    """bench.py reports a kernel's HBM traffic from a committed counter summary
    only while the summary's recorded hash matches the code of the kernel's
    source file and of the shared kernel header, and its extra build flags; a
    change of any of them makes it null, an edited comment does not."""
    import bench
    from long_context_attention_doc_amd import build as B
    csrc = tmp_path / "long_context_attention_doc_amd" / "csrc"
    csrc.mkdir(parents=True)
    (tmp_path / "profiles").mkdir()
    (csrc / "bwd.hip").write_text("// kernel source\nint x = 1;\n")
    (csrc / "aa_internal.h").write_text("/* shared header */ int y = 1;\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(B, "SOURCE_FLAGS", {"bwd.hip": ["-mllvm", "-some-option"]})
    h = bench._src_hash("bwd_dkdv")
    (tmp_path / "profiles" / "bwd_dkdv_64k_hbm_counters.txt").write_text(
        f"hbm_bytes_per_launch: 1.5e+09\nsource_sha256_16: {h}   (source + flags)\n")
    assert bench._traffic("bwd_dkdv", "64k") == 1.5e9
    assert bench._traffic("bwd_dkdv", "8k") is None                # no summary for that workload
    monkeypatch.setattr(B, "SOURCE_FLAGS", {})                     # flags changed
    assert bench._src_hash("bwd_dkdv") != h
    assert bench._traffic("bwd_dkdv", "64k") is None
    monkeypatch.setattr(B, "SOURCE_FLAGS", {"bwd.hip": ["-mllvm", "-some-option"]})
    (csrc / "bwd.hip").write_text("// kernel source, comment edited\nint  x = 1;\n")
    assert bench._traffic("bwd_dkdv", "64k") == 1.5e9              # comments and spacing only
    (csrc / "aa_internal.h").write_text("/* shared header */ int y = 2;\n")
    assert bench._traffic("bwd_dkdv", "64k") is None                # header code changed
    (csrc / "aa_internal.h").write_text("/* shared header */ int y = 1;\n")
    (csrc / "bwd.hip").write_text("// kernel source\nint x = 2;\n")  # source code changed
    assert bench._traffic("bwd_dkdv", "64k") is None

