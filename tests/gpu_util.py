"""Helpers shared by the GPU parity tests (not collected by pytest)."""
import sys

import numpy as np

U32 = 2.0 ** -24   # FP32 unit roundoff


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def announce(msg: str) -> None:
    """Name the case before a GPU step, flushed, so a crash still says what ran."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def gemv_bound(abs_prod_sum: np.ndarray, k: int, factor: float = 2.0) -> np.ndarray:
    """Rigorous summation bound gamma_n * sum|w x| for an n-term FP32 dot product (any order)."""
    n = factor * (k + 2)
    gamma = n * U32 / (1 - n * U32)
    return gamma * abs_prod_sum + 1e-30


def close_rel(got, ref, rtol, atol):
    """Elementwise |got - ref| <= atol + rtol |ref|; returns (ok, max_abs_err, worst_index)."""
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    err = np.abs(g - r)
    lim = atol + rtol * np.abs(r)
    bad = err > lim
    worst = int(np.argmax(err - lim)) if err.size else -1
    return (not bad.any()), float(err.max() if err.size else 0.0), worst
