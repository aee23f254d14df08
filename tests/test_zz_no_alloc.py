"""q4_0_matmul_static, the entry point that allocates nothing (its scratch is
a static device buffer the library holds per GPU): through the C ABI it gives
q4_0_matmul's result, on two calls in a row whose second input is smaller,
and it refuses a call that needs more scratch than the buffer holds."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import gemm_q4_amd as q4
import oracle
import synth
from gpu_util import DEV, TOL_GEMM, TOL_SMALL_N, packed_from_blocks, to_dev

pytestmark = pytest.mark.gpu


def _both(blk, x_np, out, in_):
    """y of q4_0_matmul_static and of q4_0_matmul (own workspace) on one input."""
    p = packed_from_blocks(blk, out, in_)
    x = to_dev(x_np)
    n = x.shape[0]
    code = q4.dtype_code(x)
    y_static = torch.full((n, out), float("nan"), device=DEV)
    q4.q4_0_matmul_static(p, x, code, y_static, n, out, in_)
    need = q4.q4_0_matmul_workspace_size(n, out, in_, code)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=DEV)
    y_ref = torch.full((n, out), float("nan"), device=DEV)
    q4.q4_0_matmul(p, x, code, y_ref, n, out, in_, ws, need)
    torch.cuda.synchronize()
    return y_static.cpu().numpy(), y_ref.cpu().numpy(), need


@pytest.mark.parametrize("first,second", [
    # decode: a split K range (scratch used), then a smaller call that needs
    # less scratch
    ((8, 2560, 9728, np.float32), (4, 2560, 9728, np.float32)),
    # the activation pre-pass (from 17 rows), then a smaller call
    ((24, 9728, 2560, np.float32), (20, 1024, 2560, np.float32)),
    # prefill: the split tiles' partial sums (15 MiB), then a smaller prefill
    ((512, 9728, 2560, np.float16), (100, 300, 4096, np.float16)),
])
def test_static_scratch_matches_matmul_two_calls(first, second):
    needs = []
    for k, (n, out, in_, dt) in enumerate((first, second)):
        blk = synth.make_blocks(out, in_, seed=90 + k)
        x = synth.make_x(n, in_, seed=91 + k, dtype=dt)
        ys, yr, need = _both(blk, x, out, in_)
        needs.append(need)
        assert np.array_equal(ys, yr), (n, out, in_)
        y_ref, den = oracle.matmul(blk, x, out, in_)
        tol = TOL_GEMM if n > 8 else TOL_SMALL_N
        assert oracle.max_ratio(ys, y_ref, den) <= tol
    assert needs[0] > needs[1] > 0
    assert needs[0] <= q4.STATIC_SCRATCH_BYTES


def test_static_scratch_refuses_calls_that_need_more():
    """The 151936-row head at 64 rows needs more scratch than the static
    buffer: a clear error, nothing enqueued (the pointers are never used)."""
    n, out, in_ = 64, 151936, 2560
    assert q4.q4_0_matmul_workspace_size(n, out, in_) > q4.STATIC_SCRATCH_BYTES
    with pytest.raises(q4.Q4Error) as e:
        q4.q4_0_matmul_static(1 << 20, 1 << 30, q4.F32, 1 << 34, n, out, in_)
    assert e.value.status == q4.EWORKSPACE


def test_static_scratch_needs_no_allocation():
    """Free device memory is unchanged by calls of the static entry point
    (after a first call that loads the code and takes the buffer's
    address)."""
    out, in_, n = 2560, 9728, 8
    p = packed_from_blocks(synth.make_blocks(out, in_, seed=95), out, in_)
    x = to_dev(synth.make_x(n, in_, seed=96))
    y = torch.empty((n, out), device=DEV)
    q4.q4_0_matmul_static(p, x, q4.F32, y, n, out, in_)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    for _ in range(10):
        q4.q4_0_matmul_static(p, x, q4.F32, y, n, out, in_)
    torch.cuda.synchronize()
    assert torch.cuda.mem_get_info()[0] == free0
