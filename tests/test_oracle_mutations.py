"""Planted mistakes in a copy of the oracle must each fail some pin.

Each case rewrites one line of a private copy of the oracle (on the CPU, in a
temporary directory) and runs the pin tests against that copy in a
subprocess; the pins pass only for the unmodified oracle.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = [
    ("sin sign in the rotation", "out[..., 0::2] = x0 * c - x1 * s", "out[..., 0::2] = x0 * c + x1 * s"),
    ("theta exponent", "return np.power(float(base), -2.0 * p / D)", "return np.power(float(base), -1.0 * p / D)"),
    ("dropped Dv term", "ds = p * (dp - dv_i[:, None])", "ds = p * dp"),
    ("reset starts at 0", "pos = t - cu[seg] + 1", "pos = t - cu[seg]"),
    ("strict causality", "same_doc &= cols[None, :] <= rows[:, None]", "same_doc &= cols[None, :] < rows[:, None]"),
    ("GQA head mapping", "g = h * Hkv // Hq", "g = h % Hkv"),
    ("dK not un-rotated", "dk[:, gi, :] = rope(dk_rot[:, gi, :], pos[k_cols], rope_base, inverse=True)",
     "dk[:, gi, :] = rope(dk_rot[:, gi, :], pos[k_cols], rope_base)"),
    ("anchor column dropped", "return same_batch_row & (sees_anchor | same_doc)", "return same_batch_row & same_doc"),
    ("anchor kind on any key tile", "anchor and c0 == 0))\n    return np.array(out, dtype=np.uint8)\n\n\ndef tile_kinds_col",
     "anchor))\n    return np.array(out, dtype=np.uint8)\n\n\ndef tile_kinds_col"),
    ("anchor kind without an anchor", "        out.append(_classify(m[:, c0:c0 + BN], e[:, c0:c0 + BN], anchor and c0 == 0))",
     "        out.append(_classify(m[:, c0:c0 + BN], e[:, c0:c0 + BN], c0 == 0))"),
    ("grid origin ignored for query tiles", "    r0 = origin + qt * BM\n    rows = np.arange(",
     "    r0 = qt * BM\n    rows = np.arange("),
    ("no-anchor mask keeps the anchor column", "    if not anchor:\n        return same_batch_row & same_doc",
     "    if False:\n        return same_batch_row & same_doc"),
    ("no-anchor first token at position 0", "    if anchor:\n        pos = np.where(is_anchor, 0, pos)",
     "    if True:\n        pos = np.where(is_anchor, 0, pos)"),
    ("continuous positions off by one", "        pos = t - row_start\n", "        pos = t - row_start + 1\n"),
    ("interleaved reset rank off by one", "        pos = rank + 1\n", "        pos = rank\n"),
    ("interleaved chunks ignored", "    if seg_doc is None:\n        return seg", "    if True:\n        return seg"),
    ("document label without its row", "    label_of_seg = row * span + seg_doc + 1",
     "    label_of_seg = seg_doc + 1"),
    ("key-major column with the anchor flag on every tile",
     "        out.append(_classify(m[r0:r0 + BM], e[r0:r0 + BM], anchor and c0 == 0))",
     "        out.append(_classify(m[r0:r0 + BM], e[r0:r0 + BM], anchor))"),
    ("key-major column shifted by one key",
     "    c0 = origin + kt * BN\n    cols = np.arange(b * S + c0, b * S + min(S, c0 + BN))",
     "    c0 = origin + kt * BN\n    cols = np.arange(b * S + c0 + 1, b * S + min(S, c0 + BN + 1))"),
]
PIN_FILES = ("test_oracle_pins.py", "test_oracle_modes.py", "test_oracle_interleaved.py")


@pytest.mark.slow
@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    src = os.path.join(ROOT, "oracle")
    dst = tmp_path / "oracle"
    shutil.copytree(src, dst, ignore=shutil.ignore_patterns("__pycache__"))
    f = dst / "anchor_oracle.py"
    text = f.read_text()
    assert text.count(old) >= 1, f"mutation site not found: {old}"
    f.write_text(text.replace(old, new))
    env = dict(os.environ)
    env["PYTHONPATH"] = str(tmp_path) + os.pathsep + ROOT
    res = subprocess.run(
        [sys.executable, "-m", "pytest", *[os.path.join(ROOT, "tests", f) for f in PIN_FILES], "-x", "-q",
         "-p", "no:cacheprovider", "-m", "not gpu and not slow"],
        cwd=str(tmp_path), env=env, capture_output=True, text=True, timeout=600)
    assert res.returncode != 0, f"mutant '{name}' survived the pins:\n{res.stdout[-2000:]}"
