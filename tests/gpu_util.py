"""Helpers shared by the GPU tests: move seeded inputs to the device, run the
library, compare with the oracle."""
from __future__ import annotations

import numpy as np
import torch

import gemm_q4_amd as q4
import oracle

DEV = "cuda:0"
TOL_SMALL_N = 1e-3     # float32-accumulate small-n kernels
TOL_GEMM = 1e-2        # binary16-operand prefill kernel


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def packed_from_blocks(blocks: np.ndarray, out: int, in_: int) -> torch.Tensor:
    b = to_dev(blocks.reshape(-1))
    p = q4.repacked(b, out, in_)
    torch.cuda.synchronize()
    return p


def run(packed, x_np: np.ndarray, out: int, kernel: int = q4.KERNEL_AUTO,
        stream=None) -> np.ndarray:
    x = to_dev(x_np)
    y = q4.matmul(packed, x, out, kernel=kernel, stream=stream)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def ratio(y: np.ndarray, blocks: np.ndarray, x_np: np.ndarray, out: int, in_: int,
          rows=None) -> float:
    y_ref, den = oracle.matmul(blocks, x_np, out, in_, rows=rows)
    yy = y if rows is None else y[:, rows]
    return oracle.max_ratio(yy, y_ref, den)
