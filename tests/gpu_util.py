"""Helpers shared by the GPU parity tests."""
import sys

import numpy as np
import torch

DEV = "cuda"


def announce(msg: str) -> None:
    """Name the case before it touches the GPU (flushed, so it survives a crash)."""
    sys.stdout.write(f"\n[case] {msg}\n")
    sys.stdout.flush()


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def scalerel(ref: np.ndarray, got: np.ndarray) -> float:
    """max|ref - got| / max|ref|: the scale-relative error of the f32 outputs."""
    ref = np.asarray(ref, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64)
    scale = max(np.abs(ref).max(), 1e-30)
    return float(np.abs(ref - got).max() / scale)


# tolerance on f32 outputs against the f64 oracle
TOL = 1e-4
