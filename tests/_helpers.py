"""Shared test helpers: comparisons and bf16 rounding (no method arithmetic)."""
import numpy as np
import torch


def f64(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu", torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def bf16_rne(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value, ties to even."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)


def bf16_ulp(x) -> np.ndarray:
    _, e = np.frexp(np.asarray(x, dtype=np.float64))
    return np.ldexp(1.0, e - 8)


def rel_frob(a, b) -> float:
    a, b = f64(a), f64(b)
    den = np.linalg.norm(b.ravel())
    return float(np.linalg.norm((a - b).ravel()) / max(den, 1e-300))


def o_err(o_gpu, o_ref) -> float:
    """max |O - O_ref| / max |O_ref| (the output bar is 4e-3)."""
    a, b = f64(o_gpu), f64(o_ref)
    return float(np.abs(a - b).max() / np.abs(b).max())


def say(msg: str) -> None:
    print(msg, flush=True)
