"""Shared helpers for GPU parity tests (no GPU work at import time)."""
import numpy as np

RTOL_F32_PATH = 1e-3    # relative L2 bound for the fp32-accumulated decode path
RTOL_GROUPED = 1e-2     # relative L2 bound for the bf16 matrix-core path


def rel_l2(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def same_sets(a, b) -> bool:
    """Selected expert sets per row (order within a row not compared)."""
    return np.array_equal(np.sort(np.asarray(a), axis=-1), np.sort(np.asarray(b), axis=-1))


def weights_by_expert(idx, w):
    """Dict-free comparison helper: weights sorted by expert id per row."""
    idx = np.asarray(idx)
    order = np.argsort(idx, axis=-1, kind="stable")
    return np.take_along_axis(np.asarray(w, np.float64), order, axis=-1)


def log(msg: str):
    print(msg, flush=True)
