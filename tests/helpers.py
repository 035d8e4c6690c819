"""Shared helpers for the GPU parity tests (no method arithmetic here)."""
import sys

import numpy as np
import torch


def dev():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return torch.device("cuda:0")


def u16(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 bit patterns (host copy)."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def np_(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def rowinf_rel(got: np.ndarray, ref: np.ndarray) -> float:
    """max over rows of ||got_r - ref_r||_inf / ||ref_r||_inf (rows with a zero
    reference are compared absolutely)."""
    got = np.asarray(got, np.float64).reshape(ref.shape[0], -1)
    ref = np.asarray(ref, np.float64).reshape(ref.shape[0], -1)
    if ref.size == 0:
        return 0.0
    num = np.abs(got - ref).max(axis=1)
    den = np.abs(ref).max(axis=1)
    den = np.where(den == 0, 1.0, den)
    return float((num / den).max())


def say(msg: str):
    """Progress line printed and flushed before a GPU step (names the case)."""
    print(msg, flush=True)
    sys.stdout.flush()


TOL = 2e-3   # per-row infinity-norm relative error bound for FP outputs
