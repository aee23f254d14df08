"""The C-ABI library loads on a machine without a GPU, exports every function
include/q4_0.h declares, and rejects every invalid call before touching HIP.
No compute call is made here."""
import ctypes
import os
import re

import pytest

import gemm_q4_amd as q4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q4_0.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(q4_0_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_expected_entry_points():
    names = declared_functions()
    for must in ("q4_0_repack", "q4_0_unpack", "q4_0_matmul", "q4_0_packed_bytes"):
        assert must in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(q4.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing
    assert sorted(q4.EXPORTED) == declared_functions()


def test_header_constants_match_binding():
    text = open(HEADER).read()
    consts = dict((k, int(v)) for k, v in re.findall(r"#define Q4_0_([A-Z_0-9]+) \(?(-?\d+)\)?", text))
    assert consts["OK"] == q4.OK and consts["EINVAL"] == q4.EINVAL
    assert consts["ESHAPE"] == q4.ESHAPE and consts["ENULL"] == q4.ENULL
    assert consts["EALIGN"] == q4.EALIGN and consts["EALIAS"] == q4.EALIAS
    assert consts["EUNSUPPORTED"] == q4.EUNSUPPORTED and consts["EHIP"] == q4.EHIP
    assert consts["EWORKSPACE"] == q4.EWORKSPACE
    assert consts["WORKSPACE_MAX"] == q4.WORKSPACE_MAX
    assert consts["WORKSPACE_ALIGN"] == q4.WORKSPACE_ALIGN
    assert consts["F32"] == q4.F32 and consts["F16"] == q4.F16
    assert consts["KERNEL_AUTO"] == q4.KERNEL_AUTO
    assert consts["KERNEL_GEMV_DPP"] == q4.KERNEL_GEMV_DPP
    assert consts["KERNEL_GEMV_MFMA"] == q4.KERNEL_GEMV_MFMA
    assert consts["KERNEL_GEMM"] == q4.KERNEL_GEMM
    assert consts["MAX_IN"] == q4.MAX_IN and consts["MAX_OUT"] == q4.MAX_OUT
    assert consts["MAX_N"] == q4.MAX_N
    assert consts["MAX_EXPERTS"] == q4.MAX_EXPERTS and consts["MAX_ROUTED"] == q4.MAX_ROUTED
    assert consts["ROUTE_AUTO"] == q4.ROUTE_AUTO
    assert consts["ROUTE_BY_COLUMN"] == q4.ROUTE_BY_COLUMN
    assert consts["ROUTE_BY_EXPERT"] == q4.ROUTE_BY_EXPERT


@pytest.mark.parametrize("out,in_", [(1024, 1024), (9728, 2560), (151936, 2560),
                                     (2560, 9728), (1, 32), (17, 96), (100, 4128)])
def test_sizes(out, in_):
    nb = in_ // 32
    assert q4.q4_0_blocks_bytes(out, in_) == out * nb * 18
    tiles = (out + 15) // 16
    groups = (nb + 3) // 4
    assert q4.q4_0_packed_bytes(out, in_) == tiles * 16 * groups * 4 * 18
    if out % 16 == 0 and in_ % 128 == 0:
        assert q4.q4_0_packed_bytes(out, in_) == q4.q4_0_blocks_bytes(out, in_)


def test_head_block_bytes_match_the_quoted_size():
    # a 151936 x 2560 Q4_0 head is 218,787,840 bytes (18 bytes per 32 weights)
    assert q4.q4_0_blocks_bytes(151936, 2560) == 218_787_840


@pytest.mark.parametrize("out,in_", [(0, 32), (-1, 32), (10, 0), (10, 31), (10, 33),
                                     (10, 16), (q4.MAX_OUT + 1, 32), (1, q4.MAX_IN + 32)])
def test_invalid_shapes_have_no_size(out, in_):
    assert q4.q4_0_blocks_bytes(out, in_) == 0
    assert q4.q4_0_packed_bytes(out, in_) == 0


A16 = 1 << 20      # fake, 16-byte aligned "device" addresses: never dereferenced
B16 = 1 << 30
C16 = 1 << 34


def status_of(fn, *args):
    try:
        fn(*args)
    except q4.Q4Error as e:
        return e.status
    return q4.OK


@pytest.mark.parametrize("args,expect", [
    ((A16, B16, q4.F32, C16, 0, 10, 64), q4.ESHAPE),
    ((A16, B16, q4.F32, C16, 1, 0, 64), q4.ESHAPE),
    ((A16, B16, q4.F32, C16, 1, 10, 48), q4.ESHAPE),
    ((A16, B16, q4.F32, C16, q4.MAX_N + 1, 10, 64), q4.ESHAPE),
    ((A16, B16, 7, C16, 1, 10, 64), q4.EINVAL),
    ((0, B16, q4.F32, C16, 1, 10, 64), q4.ENULL),
    ((A16, 0, q4.F32, C16, 1, 10, 64), q4.ENULL),
    ((A16, B16, q4.F32, 0, 1, 10, 64), q4.ENULL),
    ((A16 + 8, B16, q4.F32, C16, 1, 10, 64), q4.EALIGN),
    ((A16, B16 + 4, q4.F32, C16, 1, 10, 64), q4.EALIGN),
    ((A16, B16, q4.F32, C16 + 2, 1, 10, 64), q4.EALIGN),
    ((A16, B16, q4.F32, B16 + 64, 1, 10, 64), q4.EALIAS),    # y inside x
    ((A16, B16, q4.F32, A16 + 16, 1, 10, 64), q4.EALIAS),    # y inside W
])
def test_matmul_validation(args, expect):
    assert status_of(q4.q4_0_matmul, *args) == expect


def test_matmul_ex_rejects_bad_kernel_and_unsupported_shapes():
    assert status_of(q4.q4_0_matmul_ex, A16, B16, q4.F32, C16, 1, 10, 64, 9) == q4.EINVAL
    assert status_of(q4.q4_0_matmul_ex, A16, B16, q4.F32, C16, 1, 10, 64, -1) == q4.EINVAL
    # the VALU kernel takes n <= 8, the small-n MFMA kernel n <= 64
    assert status_of(q4.q4_0_matmul_ex, A16, B16, q4.F32, C16, 9, 10, 64,
                     q4.KERNEL_GEMV_DPP) == q4.EUNSUPPORTED
    assert status_of(q4.q4_0_matmul_ex, A16, B16, q4.F32, C16, 65, 10, 64,
                     q4.KERNEL_GEMV_MFMA) == q4.EUNSUPPORTED
    # the LDS-staged kernel cannot hold 8 rows of a 16384-wide x
    assert status_of(q4.q4_0_matmul_ex, A16, B16, q4.F32, C16, 8, 10, 16384,
                     q4.KERNEL_GEMV_DPP) == q4.EUNSUPPORTED


@pytest.mark.parametrize("fn", [q4.q4_0_repack, q4.q4_0_unpack])
def test_repack_validation(fn):
    assert status_of(fn, A16, B16, 10, 48, 0) == q4.ESHAPE
    assert status_of(fn, 0, B16, 10, 64, 0) == q4.ENULL
    assert status_of(fn, A16, 0, 10, 64, 0) == q4.ENULL
    src, dst = (A16, B16 + 8) if fn is q4.q4_0_repack else (A16 + 8, B16)
    assert status_of(fn, src, dst, 10, 64, 0) == q4.EALIGN
    assert status_of(fn, A16, A16 + 32, 10, 64, 0) == q4.EALIAS


def test_kernel_choice_table():
    """What the automatic choice runs for the workloads' shapes."""
    sel = q4.q4_0_select_kernel
    assert sel(1, 9728, 2560) in (q4.KERNEL_GEMV_DPP, q4.KERNEL_GEMV_MFMA)
    for n in (2, 4, 8):
        for out, in_ in [(4096, 2560), (1024, 2560), (2560, 4096), (9728, 2560),
                         (2560, 9728), (151936, 2560)]:
            assert sel(n, out, in_) in (q4.KERNEL_GEMV_DPP, q4.KERNEL_GEMV_MFMA)
    assert sel(512, 9728, 2560, q4.F16) == q4.KERNEL_GEMM
    assert sel(512, 2560, 9728, q4.F16) == q4.KERNEL_GEMM
    # the band between decode and prefill: small-n MFMA kernel up to 64 rows
    # (one launch up to 32, two above), the tiled product from 65
    assert sel(9, 100, 64) == q4.KERNEL_GEMV_MFMA
    assert sel(32, 9728, 2560) == q4.KERNEL_GEMV_MFMA
    assert sel(33, 9728, 2560) == q4.KERNEL_GEMV_MFMA
    assert sel(64, 9728, 2560) == q4.KERNEL_GEMV_MFMA
    assert sel(65, 9728, 2560) == q4.KERNEL_GEMM
    with pytest.raises(q4.Q4Error):
        sel(0, 10, 64)
    with pytest.raises(q4.Q4Error):
        sel(1, 10, 64, 5)


def test_kernel_supports():
    assert q4.q4_0_kernel_supports(q4.KERNEL_GEMM, 512, 9728, 2560, q4.F16)
    assert q4.q4_0_kernel_supports(q4.KERNEL_GEMV_MFMA, 8, 2560, 9728)
    assert q4.q4_0_kernel_supports(q4.KERNEL_GEMV_MFMA, 16, 2560, 9728)
    assert q4.q4_0_kernel_supports(q4.KERNEL_GEMV_MFMA, 64, 151936, 2560)
    assert not q4.q4_0_kernel_supports(q4.KERNEL_GEMV_MFMA, 65, 2560, 9728)
    with pytest.raises(q4.Q4Error):
        q4.q4_0_kernel_supports(17, 1, 10, 64)


def test_strerror_covers_every_status():
    for st in (q4.OK, q4.EINVAL, q4.ESHAPE, q4.ENULL, q4.EALIGN, q4.EALIAS,
               q4.EUNSUPPORTED, q4.EHIP, q4.EWORKSPACE):
        assert q4.q4_0_strerror(st) != "unknown status"
    assert q4.q4_0_strerror(-99) == "unknown status"
    assert q4.q4_0_version() >= 100


def test_grouped_validation():
    grp = q4.q4_0_matmul_grouped
    lin = (A16, B16, C16, 10, 64)
    assert status_of(grp, [], q4.F32, 1) == q4.EINVAL                 # count 0
    assert status_of(grp, [lin] * (q4.MAX_GROUP + 1), q4.F32, 1) == q4.EINVAL
    assert status_of(grp, [lin], 7, 1) == q4.EINVAL                   # dtype
    assert status_of(grp, [(A16, B16, C16, 10, 48)], q4.F32, 1) == q4.ESHAPE
    assert status_of(grp, [lin], q4.F32, 0) == q4.ESHAPE
    assert status_of(grp, [(0, B16, C16, 10, 64)], q4.F32, 1) == q4.ENULL
    assert status_of(grp, [(A16, B16, 0, 10, 64)], q4.F32, 1) == q4.ENULL
    assert status_of(grp, [(A16 + 8, B16, C16, 10, 64)], q4.F32, 1) == q4.EALIGN
    # the second linear's x lies inside the first linear's y
    other = (A16 + (1 << 16), C16 + 16, C16 + (1 << 20), 10, 64)
    assert status_of(grp, [lin, other], q4.F32, 1) == q4.EALIAS
    # two outputs overlap
    other = (A16 + (1 << 16), B16, C16 + 8, 10, 64)
    assert status_of(grp, [lin, other], q4.F32, 1) == q4.EALIAS
    # one y inside another linear's packed weights
    other = (C16 - 16, B16, C16 + (1 << 20), 10, 64)
    assert status_of(grp, [lin, other], q4.F32, 1) == q4.EALIAS


def test_argmax_validation():
    am = q4.q4_0_matmul_argmax
    D16 = 1 << 38
    E16 = 1 << 39
    assert status_of(am, A16, B16, q4.F32, C16, 1, 10, 48, D16, E16) == q4.ESHAPE
    assert status_of(am, A16, B16, 5, C16, 1, 10, 64, D16, E16) == q4.EINVAL
    assert status_of(am, A16, B16, q4.F32, C16, 1, 10, 64, 0, E16) == q4.ENULL
    assert status_of(am, A16, B16, q4.F32, C16, 1, 10, 64, D16, 0) == q4.ENULL
    assert status_of(am, 0, B16, q4.F32, C16, 1, 10, 64, D16, E16) == q4.ENULL
    assert status_of(am, A16, B16, q4.F32, C16, 1, 10, 64, D16 + 2, E16) == q4.EALIGN
    assert status_of(am, A16, B16, q4.F32, C16, 1, 10, 64, B16 + 4, E16) == q4.EALIAS
    assert status_of(am, A16, B16, q4.F32, C16, 2, 10, 64, D16, D16 + 4) == q4.EALIAS
    assert status_of(am, A16, B16, q4.F32, C16, 1, 10, 64, C16 + 8, E16) == q4.EALIAS
    assert status_of(am, A16, B16, q4.F32, C16, 65, 10, 64, D16, E16) == q4.EUNSUPPORTED


def test_w4a8_validation():
    qx, mm = q4.q4_0_quantize_x8, q4.q4_0_matmul_w4a8
    D16 = 1 << 38
    assert status_of(qx, A16, q4.F32, B16, C16, 1, 48, 0) == q4.ESHAPE
    assert status_of(qx, A16, 9, B16, C16, 1, 64, 0) == q4.EINVAL
    assert status_of(qx, 0, q4.F32, B16, C16, 1, 64, 0) == q4.ENULL
    assert status_of(qx, A16, q4.F32, B16 + 4, C16, 1, 64, 0) == q4.EALIGN
    assert status_of(qx, A16, q4.F32, A16 + 16, C16, 1, 64, 0) == q4.EALIAS
    assert status_of(qx, A16, q4.F32, B16, B16 + 16, 1, 64, 0) == q4.EALIAS
    assert status_of(mm, A16, B16, C16, D16, 1, 10, 48) == q4.ESHAPE
    assert status_of(mm, A16, 0, C16, D16, 1, 10, 64) == q4.ENULL
    assert status_of(mm, A16, B16 + 8, C16, D16, 1, 10, 64) == q4.EALIGN
    assert status_of(mm, A16, B16, C16, B16 + 32, 1, 10, 64) == q4.EALIAS
    assert status_of(mm, A16, B16, C16, A16 + 64, 1, 10, 64) == q4.EALIAS
    assert status_of(mm, A16, B16, C16, D16, 65, 10, 64) == q4.EUNSUPPORTED


def test_mfma_loop_validation():
    f = q4.q4_0_mfma_loop
    assert status_of(f, 0, 1, 1, 0) == q4.ENULL
    assert status_of(f, A16, 0, 1) == q4.EINVAL
    assert status_of(f, A16, 65537, 1) == q4.EINVAL
    assert status_of(f, A16, 1, 0) == q4.EINVAL
    assert status_of(f, A16, 1, 1000001) == q4.EINVAL


def test_bench_refuses_more_than_one_gpu():
    """The benchmark measures one GPU; --gpus above 1 exits with a message
    (status 2) before touching a device."""
    import json
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert msg["n_gpus_requested"] == 2 and "one GPU" in msg["error"]


def test_routed_validation():
    f = q4.q4_0_matmul_routed
    D16 = 1 << 38
    E16 = 1 << 39
    # experts, n_experts, x, x_dtype, route, k, y, n, out, in
    assert status_of(f, A16, 4, B16, q4.F32, C16, 2, D16, 1, 10, 48) == q4.ESHAPE
    assert status_of(f, A16, 0, B16, q4.F32, C16, 2, D16, 1, 10, 64) == q4.EINVAL
    assert status_of(f, A16, 4, B16, q4.F32, C16, 0, D16, 1, 10, 64) == q4.EINVAL
    assert status_of(f, A16, 4, B16, q4.F32, C16, q4.MAX_ROUTED + 1, D16, 1, 10, 64) == q4.EINVAL
    assert status_of(f, A16, q4.MAX_EXPERTS + 1, B16, q4.F32, C16, 2, D16, 1, 10, 64) == q4.EINVAL
    assert status_of(f, A16, 4, B16, 7, C16, 2, D16, 1, 10, 64) == q4.EINVAL
    assert status_of(f, A16, 4, B16, q4.F32, 0, 2, D16, 1, 10, 64) == q4.ENULL
    assert status_of(f, A16 + 8, 4, B16, q4.F32, C16, 2, D16, 1, 10, 64) == q4.EALIGN
    assert status_of(f, A16, 4, B16, q4.F32, C16 + 2, 2, D16, 1, 10, 64) == q4.EALIGN
    assert status_of(f, A16, 4, B16, q4.F32, C16, 2, B16 + 16, 1, 10, 64) == q4.EALIAS
    assert status_of(f, A16, 4, B16, q4.F32, C16, 2, A16 + 64, 1, 10, 64) == q4.EALIAS
    assert status_of(f, A16, 4, B16, q4.F32, E16, 2, E16 - 64, 1, 10, 64) == q4.EALIAS


def test_routed_ex_and_route_choice():
    D16 = 1 << 38
    f = q4.q4_0_matmul_routed_ex
    assert status_of(f, A16, 4, B16, q4.F32, C16, 2, D16, 1, 10, 64, 3) == q4.EINVAL
    # by expert takes at most 4096 pairs
    assert status_of(f, A16, 4, B16, q4.F32, C16, 64, D16, 65, 10, 64,
                     q4.ROUTE_BY_EXPERT) == q4.EUNSUPPORTED
    sel = q4._lib.q4_0_select_route
    assert sel(1, 8, 128, 768, 2048) == q4.ROUTE_BY_COLUMN
    assert sel(16, 8, 128, 768, 2048) == q4.ROUTE_BY_COLUMN
    assert sel(24, 8, 128, 768, 2048) == q4.ROUTE_BY_EXPERT
    assert sel(65, 64, 128, 768, 2048) == q4.ROUTE_BY_COLUMN    # too many pairs by expert
    assert sel(1, 0, 128, 768, 2048) == q4.EINVAL
    assert sel(1, 8, 128, 768, 48) == q4.ESHAPE


# ---- workspaces: sizes, and calls without enough of one -------------------
W16 = 1 << 42      # a fake, 256-byte aligned workspace address


def test_workspace_sizes_of_the_workloads():
    """The headline decode call needs no workspace, nor does FFN-up up to 16
    rows (one K slice, x converted per workgroup); the activation pre-pass
    (from 17 rows), a split K range (the 9728-wide down projection), the
    split tiles of the prefill product and the greedy pick do."""
    mws = q4.q4_0_matmul_workspace_size
    assert mws(1, 9728, 2560) == 0
    assert mws(1, 151936, 2560) == 0
    assert mws(8, 9728, 2560) == 0
    assert mws(16, 9728, 2560) == 0
    assert 0 < mws(17, 9728, 2560) <= q4.WORKSPACE_MAX
    assert 0 < mws(8, 2560, 9728) <= q4.WORKSPACE_MAX
    assert 0 < mws(512, 9728, 2560, q4.F16) <= q4.WORKSPACE_MAX
    assert mws(1, 9728, 2560, q4.F32, q4.KERNEL_GEMV_DPP) == 0
    assert 0 < q4.q4_0_argmax_workspace_size(1, 151936, 2560) <= q4.WORKSPACE_MAX
    assert q4.q4_0_routed_workspace_size(64, 8, 128, 768, 2048, q4.ROUTE_BY_EXPERT) > 0
    assert q4.q4_0_w4a8_workspace_size(1, 9728, 2560) >= 0
    lin = [(A16, B16, C16, 4096, 2560), (A16 + (1 << 24), B16, C16 + (1 << 24), 1024, 2560)]
    g = q4.q4_0_grouped_workspace_size(lin, q4.F32, 20)
    assert g >= max(mws(20, 4096, 2560), mws(20, 1024, 2560)) > 0
    # an invalid shape or selector is reported as the call would report it
    for bad, st in (((0, 10, 64), q4.ESHAPE), ((1, 10, 48), q4.ESHAPE)):
        with pytest.raises(q4.Q4Error) as e:
            mws(*bad)
        assert e.value.status == st
    with pytest.raises(q4.Q4Error) as e:
        mws(65, 10, 64, q4.F32, q4.KERNEL_GEMV_MFMA)
    assert e.value.status == q4.EUNSUPPORTED


def test_calls_without_enough_workspace_are_refused():
    need = q4.q4_0_matmul_workspace_size(8, 2560, 9728)
    mm = q4.q4_0_matmul
    args = (A16, B16, q4.F32, C16, 8, 2560, 9728)
    assert status_of(mm, *args, None, 0) == q4.EWORKSPACE
    assert status_of(mm, *args, W16, need - 1) == q4.EWORKSPACE
    assert status_of(mm, *args, W16 + 128, need) == q4.EALIGN
    assert status_of(mm, *args, B16 + 256, need) == q4.EALIAS     # inside x
    assert status_of(mm, *args, C16 - 256, need) == q4.EALIAS     # runs into y
    # prefill
    need = q4.q4_0_matmul_workspace_size(512, 9728, 2560, q4.F16)
    assert status_of(mm, A16, B16, q4.F16, C16, 512, 9728, 2560, None, 0) == q4.EWORKSPACE
    assert status_of(mm, A16, B16, q4.F16, C16, 512, 9728, 2560, W16, need // 2) == \
        q4.EWORKSPACE
    # the greedy pick always needs one
    D16, E16 = 1 << 38, 1 << 39
    need = q4.q4_0_argmax_workspace_size(1, 1024, 1024)
    am = q4.q4_0_matmul_argmax
    assert status_of(am, A16, B16, q4.F32, C16, 1, 1024, 1024, D16, E16) == q4.EWORKSPACE
    assert status_of(am, A16, B16, q4.F32, C16, 1, 1024, 1024, D16, E16, D16,
                     need) in (q4.EALIAS,)
    # routed and grouped
    need = q4.q4_0_routed_workspace_size(64, 8, 128, 768, 2048, q4.ROUTE_BY_EXPERT)
    f = q4.q4_0_matmul_routed_ex
    assert status_of(f, A16, 128, B16, q4.F32, C16, 8, D16, 64, 768, 2048,
                     q4.ROUTE_BY_EXPERT, W16, need - 256) == q4.EWORKSPACE
    lin = [(A16, B16, C16, 2560, 9728)]
    assert status_of(q4.q4_0_matmul_grouped, lin, q4.F32, 8) == q4.EWORKSPACE


def test_grouped_call_checks_every_linear_before_enqueuing():
    """A group whose second linear no kernel can take fails with
    EUNSUPPORTED before the first linear is enqueued (on this host, with no
    GPU, any launch would fail with EHIP instead)."""
    n = q4.MAX_N
    ok = (A16, B16, C16, 64, 64)                                   # tiled product
    big = (A16 + (1 << 24), B16, 1 << 45, 40000, 64)               # n * out > 2^31
    ws = q4.WORKSPACE_MAX
    assert status_of(q4.q4_0_matmul_grouped, [ok, big], q4.F32, n, W16, ws) == \
        q4.EUNSUPPORTED
    # a null pointer in the last linear: ENULL, nothing enqueued
    assert status_of(q4.q4_0_matmul_grouped, [ok, (0, B16, 1 << 45, 64, 64)], q4.F32, 1,
                     W16, ws) == q4.ENULL


def test_stream_read_validation():
    f = q4.q4_0_stream_read
    assert status_of(f, A16, 16, 0, 1) == q4.ENULL                # no sink
    assert status_of(f, 0, 16, B16, 1) == q4.ENULL                # bytes but no source
    assert status_of(f, A16, 15, B16, 1) == q4.EINVAL             # not whole 16 bytes
    assert status_of(f, A16, -16, B16, 1) == q4.EINVAL
    assert status_of(f, A16, 16, B16, 0) == q4.EINVAL
    assert status_of(f, A16, 16, B16, 65537) == q4.EINVAL
    assert status_of(f, A16 + 4, 16, B16, 1) == q4.EALIGN
    assert status_of(f, A16, 1 << 20, A16 + 64, 4) == q4.EALIAS
