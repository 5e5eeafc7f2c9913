"""Helpers for the GPU tests: device copies that keep a matrix's leading
dimension and alignment, with NaN-filled gaps and canaries around it."""
from __future__ import annotations

import numpy as np
import torch

import dense_fp32_gemm_sgemm_amd as sg

CANARY = 64  # floats of NaN before and after every device matrix


class DevMatrix:
    """A (rows x cols) float32 view with leading dimension ``ld`` placed
    ``offset`` floats into a NaN-filled device buffer (offset counts from the
    end of the leading canary; an offset that is not a multiple of 4 makes the
    view misaligned for 16-byte accesses)."""

    def __init__(self, X: np.ndarray, ld: int | None = None, offset: int = 0,
                 device: str = "cuda"):
        rows, cols = X.shape
        self.rows, self.cols = rows, cols
        self.ld = max(1, cols) if ld is None else ld
        span = (rows - 1) * self.ld + cols if rows and cols else 0
        self.start = CANARY + offset
        self.buf = torch.full((self.start + span + CANARY,), float("nan"), dtype=torch.float32,
                              device=device)
        self.view = torch.as_strided(self.buf, (rows, cols), (self.ld, 1), self.start)
        if rows and cols:
            self.view.copy_(torch.from_numpy(np.ascontiguousarray(X)).to(device))

    def numpy(self) -> np.ndarray:
        return self.view.cpu().numpy()

    def outside_untouched(self) -> bool:
        """Every buffer element outside the view is still NaN."""
        mask = torch.ones_like(self.buf, dtype=torch.bool)
        if self.rows and self.cols:
            idx = (self.start + torch.arange(self.rows, device=self.buf.device)[:, None] * self.ld
                   + torch.arange(self.cols, device=self.buf.device)[None, :])
            mask[idx.reshape(-1)] = False
        return bool(torch.isnan(self.buf[mask]).all().item())


def run(A, B, C=None, alpha=1.0, beta=0.0, *, variant=-1, lds=(None, None, None),
        offsets=(0, 0, 0), check_outside=False, trans_a=False, trans_b=False, workspace=None):
    """Runs the HIP SGEMM on device copies; returns C as numpy (float32).

    A and B are the matrices as stored: with trans_a, A is K x M and op(A) is
    its transpose (likewise B with trans_b).  C=None means a NaN-filled output
    buffer (only valid with beta == 0)."""
    M = A.shape[1] if trans_a else A.shape[0]
    N = B.shape[0] if trans_b else B.shape[1]
    if C is None:
        C = np.full((M, N), np.nan, np.float32)
    dA = DevMatrix(A, lds[0], offsets[0])
    dB = DevMatrix(B, lds[1], offsets[1])
    dC = DevMatrix(C, lds[2], offsets[2])
    sg.gemm(dA.view, dB.view, dC.view, alpha, beta, variant=variant, trans_a=trans_a,
            trans_b=trans_b, workspace=workspace)
    torch.cuda.synchronize()
    out = dC.numpy()
    if check_outside:
        for name, d in (("A", dA), ("B", dB), ("C", dC)):
            assert d.outside_untouched(), "memory outside %s was written" % name
    return out


def describe(**kw) -> str:
    return " ".join("%s=%s" % (k, v) for k, v in kw.items())
