"""Python binding of libq4_0, the MI355X Q4_0 matmul library (include/q4_0.h).

Argument marshalling only: every q4_0_* function calls the C entry point of
the same name in ``libq4_0.so`` (built in this directory by
``gemm_q4_amd.build``), with the same arguments in the same order.  Pointer
arguments accept torch tensors (their ``data_ptr()``) or integers;
``stream`` accepts a ``torch.cuda.Stream``, an integer hipStream_t, or None
(torch's current stream on the tensors' device, else the null stream).
A negative status raises ``Q4Error``; the *_workspace_size queries return
the byte count.  There is no CPU fallback: importing this package fails if
the HIP library has not been built.

The library allocates nothing: calls that need scratch memory take a
caller-owned workspace.  The torch conveniences at the end of this file
(``matmul``, ``matmul_argmax``, ``matmul_routed``, ...) query the size and
allocate the workspace through torch's allocator, as they do their outputs.

torch is imported before the library is loaded: torch ships its own HIP
runtime under the same soname, and loading ours first would put two HIP
runtimes in one process, whose streams and contexts do not mix.  With torch
loaded first, libq4_0.so binds to torch's runtime; the import checks that
only one copy of the HIP runtime is mapped.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (must precede the CDLL below)

_HERE = os.path.dirname(os.path.abspath(__file__))
# Q4_0_LIBRARY names another build of the same library (a tuning variant)
LIB_PATH = os.environ.get("Q4_0_LIBRARY") or os.path.join(_HERE, "libq4_0.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build the HIP library first "
        "(python -c 'import __graft_entry__ as g; g.build()')")

_lib = ctypes.CDLL(LIB_PATH)


def _mapped_runtimes():
    paths = {}
    try:
        with open("/proc/self/maps") as fh:
            for line in fh:
                parts = line.split()
                if len(parts) >= 6:
                    base = os.path.basename(parts[5])
                    for lib in ("libamdhip64.so",):
                        if base.startswith(lib):
                            paths.setdefault(lib, set()).add(os.path.realpath(parts[5]))
    except OSError:
        pass
    return paths


for _libname, _paths in _mapped_runtimes().items():
    if len(_paths) > 1:
        raise ImportError(f"two copies of {_libname} are loaded ({sorted(_paths)}); "
                          "import torch before anything that loads a HIP runtime")

# constants of include/q4_0.h
OK, EINVAL, ESHAPE, ENULL, EALIGN, EALIAS, EUNSUPPORTED, EHIP, EWORKSPACE = \
    0, -1, -2, -3, -4, -5, -6, -7, -8
F32, F16 = 0, 1
KERNEL_AUTO, KERNEL_GEMV_DPP, KERNEL_GEMV_MFMA, KERNEL_GEMM = 0, 1, 2, 3
KERNEL_NAMES = {KERNEL_AUTO: "auto", KERNEL_GEMV_DPP: "gemv_dpp",
                KERNEL_GEMV_MFMA: "gemv_mfma", KERNEL_GEMM: "gemm"}
MAX_IN, MAX_OUT, MAX_N = 1048576, 16777216, 65536
MAX_EXPERTS, MAX_ROUTED = 4096, 64
WORKSPACE_MAX, WORKSPACE_ALIGN = 134217728, 256
STATIC_SCRATCH_BYTES = 16777216
ROUTE_AUTO, ROUTE_BY_COLUMN, ROUTE_BY_EXPERT = 0, 1, 2

_i64, _vp, _int, _sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
_szp = ctypes.POINTER(_sz)
_SIGS = {
    "q4_0_blocks_bytes": (_sz, [_i64, _i64]),
    "q4_0_packed_bytes": (_sz, [_i64, _i64]),
    "q4_0_repack": (_int, [_vp, _vp, _i64, _i64, _vp]),
    "q4_0_unpack": (_int, [_vp, _vp, _i64, _i64, _vp]),
    "q4_0_matmul": (_int, [_vp, _vp, _int, _vp, _i64, _i64, _i64, _vp, _sz, _vp]),
    "q4_0_matmul_ex": (_int, [_vp, _vp, _int, _vp, _i64, _i64, _i64, _int, _vp, _sz, _vp]),
    "q4_0_matmul_workspace_size": (_int, [_i64, _i64, _i64, _int, _int, _szp]),
    "q4_0_matmul_static": (_int, [_vp, _vp, _int, _vp, _i64, _i64, _i64, _vp]),
    "q4_0_select_kernel": (_int, [_i64, _i64, _i64, _int]),
    "q4_0_kernel_supports": (_int, [_int, _i64, _i64, _i64, _int]),
    "q4_0_strerror": (ctypes.c_char_p, [_int]),
    "q4_0_version": (_int, []),
    "q4_0_matmul_grouped": (_int, [_vp, _int, _int, _i64, _vp, _sz, _vp]),
    "q4_0_grouped_workspace_size": (_int, [_vp, _int, _int, _i64, _szp]),
    "q4_0_matmul_argmax": (_int, [_vp, _vp, _int, _vp, _i64, _i64, _i64, _vp, _vp,
                                  _vp, _sz, _vp]),
    "q4_0_argmax_workspace_size": (_int, [_i64, _i64, _i64, _int, _szp]),
    "q4_0_quantize_x8": (_int, [_vp, _int, _vp, _vp, _i64, _i64, _vp]),
    "q4_0_matmul_w4a8": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _sz, _vp]),
    "q4_0_w4a8_workspace_size": (_int, [_i64, _i64, _i64, _szp]),
    "q4_0_mfma_loop": (_int, [_vp, _i64, _i64, ctypes.POINTER(_i64), _vp]),
    "q4_0_stream_read": (_int, [_vp, _i64, _vp, _i64, _vp]),
    "q4_0_matmul_routed": (_int, [_vp, _i64, _vp, _int, _vp, _i64, _vp, _i64, _i64, _i64,
                                  _vp, _sz, _vp]),
    "q4_0_matmul_routed_ex": (_int, [_vp, _i64, _vp, _int, _vp, _i64, _vp, _i64, _i64, _i64,
                                     _int, _vp, _sz, _vp]),
    "q4_0_select_route": (_int, [_i64, _i64, _i64, _i64, _i64]),
    "q4_0_routed_workspace_size": (_int, [_i64, _i64, _i64, _i64, _i64, _int, _szp]),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args

EXPORTED = tuple(_SIGS)


class Q4Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {q4_0_strerror(status)} (status {status})")


def _ptr(a):
    if a is None:
        return None
    if isinstance(a, int):
        return a
    return a.data_ptr()


def _nbytes(ws, workspace_bytes):
    """Workspace size argument: as given, else the tensor's size, else 0."""
    if workspace_bytes is not None:
        return workspace_bytes
    if ws is None or isinstance(ws, int):
        return 0
    return ws.numel() * ws.element_size()


def _stream(stream, *tensors):
    if stream is None:
        for t in tensors:
            if hasattr(t, "is_cuda") and t.is_cuda:
                import torch
                return torch.cuda.current_stream(t.device).cuda_stream
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, where: str) -> int:
    if status < 0:
        raise Q4Error(status, where)
    return status


def _size(fn, where, *args) -> int:
    out = _sz(0)
    _check(fn(*args, ctypes.byref(out)), where)
    return out.value


def q4_0_strerror(status: int) -> str:
    return _lib.q4_0_strerror(status).decode()


def q4_0_version() -> int:
    return _lib.q4_0_version()


def q4_0_blocks_bytes(out: int, in_: int) -> int:
    return _lib.q4_0_blocks_bytes(out, in_)


def q4_0_packed_bytes(out: int, in_: int) -> int:
    return _lib.q4_0_packed_bytes(out, in_)


def q4_0_repack(blocks, packed, out: int, in_: int, stream=None) -> None:
    _check(_lib.q4_0_repack(_ptr(blocks), _ptr(packed), out, in_,
                            _stream(stream, blocks, packed)), "q4_0_repack")


def q4_0_unpack(packed, blocks, out: int, in_: int, stream=None) -> None:
    _check(_lib.q4_0_unpack(_ptr(packed), _ptr(blocks), out, in_,
                            _stream(stream, packed, blocks)), "q4_0_unpack")


def q4_0_matmul(packed, x, x_dtype: int, y, n: int, out: int, in_: int,
                workspace=None, workspace_bytes=None, stream=None) -> None:
    _check(_lib.q4_0_matmul(_ptr(packed), _ptr(x), x_dtype, _ptr(y), n, out, in_,
                            _ptr(workspace), _nbytes(workspace, workspace_bytes),
                            _stream(stream, packed, x, y)), "q4_0_matmul")


def q4_0_matmul_ex(packed, x, x_dtype: int, y, n: int, out: int, in_: int,
                   kernel: int, workspace=None, workspace_bytes=None, stream=None) -> None:
    _check(_lib.q4_0_matmul_ex(_ptr(packed), _ptr(x), x_dtype, _ptr(y), n, out,
                               in_, kernel, _ptr(workspace),
                               _nbytes(workspace, workspace_bytes),
                               _stream(stream, packed, x, y)), "q4_0_matmul_ex")


def q4_0_matmul_static(packed, x, x_dtype: int, y, n: int, out: int, in_: int,
                       stream=None) -> None:
    _check(_lib.q4_0_matmul_static(_ptr(packed), _ptr(x), x_dtype, _ptr(y), n, out, in_,
                                   _stream(stream, packed, x, y)), "q4_0_matmul_static")


def q4_0_matmul_workspace_size(n: int, out: int, in_: int, x_dtype: int = F32,
                               kernel: int = KERNEL_AUTO) -> int:
    return _size(_lib.q4_0_matmul_workspace_size, "q4_0_matmul_workspace_size",
                 n, out, in_, x_dtype, kernel)


class q4_0_linear(ctypes.Structure):
    """One linear of q4_0_matmul_grouped (struct q4_0_linear of include/q4_0.h)."""
    _fields_ = [("packed", _vp), ("x", _vp), ("y", _vp), ("out", _i64), ("in_", _i64)]


MAX_GROUP = 8


def _linears(linears):
    arr = (q4_0_linear * max(1, len(linears)))()
    tensors = []
    for i, (packed, x, y, out, in_) in enumerate(linears):
        arr[i] = q4_0_linear(_ptr(packed), _ptr(x), _ptr(y), out, in_)
        tensors += [packed, x, y]
    return arr, tensors


def q4_0_matmul_grouped(linears, x_dtype: int, n: int, workspace=None, workspace_bytes=None,
                        stream=None) -> None:
    """linears: sequence of (packed, x, y, out, in) with tensors or pointers."""
    arr, tensors = _linears(linears)
    _check(_lib.q4_0_matmul_grouped(ctypes.cast(arr, _vp), len(linears), x_dtype, n,
                                    _ptr(workspace), _nbytes(workspace, workspace_bytes),
                                    _stream(stream, *tensors)), "q4_0_matmul_grouped")


def q4_0_grouped_workspace_size(linears, x_dtype: int, n: int) -> int:
    arr, _ = _linears(linears)
    return _size(_lib.q4_0_grouped_workspace_size, "q4_0_grouped_workspace_size",
                 ctypes.cast(arr, _vp), len(linears), x_dtype, n)


def q4_0_matmul_argmax(packed, x, x_dtype: int, y, n: int, out: int, in_: int,
                       max_val, max_idx, workspace=None, workspace_bytes=None,
                       stream=None) -> None:
    _check(_lib.q4_0_matmul_argmax(_ptr(packed), _ptr(x), x_dtype, _ptr(y), n, out, in_,
                                   _ptr(max_val), _ptr(max_idx), _ptr(workspace),
                                   _nbytes(workspace, workspace_bytes),
                                   _stream(stream, packed, x, max_val)), "q4_0_matmul_argmax")


def q4_0_argmax_workspace_size(n: int, out: int, in_: int, x_dtype: int = F32) -> int:
    return _size(_lib.q4_0_argmax_workspace_size, "q4_0_argmax_workspace_size",
                 n, out, in_, x_dtype)


def q4_0_quantize_x8(x, x_dtype: int, q, d, n: int, in_: int, stream=None) -> None:
    _check(_lib.q4_0_quantize_x8(_ptr(x), x_dtype, _ptr(q), _ptr(d), n, in_,
                                 _stream(stream, x, q, d)), "q4_0_quantize_x8")


def q4_0_matmul_w4a8(packed, q, d, y, n: int, out: int, in_: int, workspace=None,
                     workspace_bytes=None, stream=None) -> None:
    _check(_lib.q4_0_matmul_w4a8(_ptr(packed), _ptr(q), _ptr(d), _ptr(y), n, out, in_,
                                 _ptr(workspace), _nbytes(workspace, workspace_bytes),
                                 _stream(stream, packed, q, y)), "q4_0_matmul_w4a8")


def q4_0_w4a8_workspace_size(n: int, out: int, in_: int) -> int:
    return _size(_lib.q4_0_w4a8_workspace_size, "q4_0_w4a8_workspace_size", n, out, in_)


def q4_0_select_kernel(n: int, out: int, in_: int, x_dtype: int = F32) -> int:
    return _check(_lib.q4_0_select_kernel(n, out, in_, x_dtype), "q4_0_select_kernel")


def q4_0_kernel_supports(kernel: int, n: int, out: int, in_: int,
                         x_dtype: int = F32) -> bool:
    st = _lib.q4_0_kernel_supports(kernel, n, out, in_, x_dtype)
    if st == EUNSUPPORTED:
        return False
    _check(st, "q4_0_kernel_supports")
    return True


def q4_0_matmul_routed(experts, n_experts: int, x, x_dtype: int, route, k: int, y, n: int,
                       out: int, in_: int, workspace=None, workspace_bytes=None,
                       stream=None) -> None:
    _check(_lib.q4_0_matmul_routed(_ptr(experts), n_experts, _ptr(x), x_dtype, _ptr(route), k,
                                   _ptr(y), n, out, in_, _ptr(workspace),
                                   _nbytes(workspace, workspace_bytes),
                                   _stream(stream, y, x)), "q4_0_matmul_routed")


def q4_0_matmul_routed_ex(experts, n_experts: int, x, x_dtype: int, route, k: int, y, n: int,
                          out: int, in_: int, route_kernel: int, workspace=None,
                          workspace_bytes=None, stream=None) -> None:
    _check(_lib.q4_0_matmul_routed_ex(_ptr(experts), n_experts, _ptr(x), x_dtype, _ptr(route),
                                      k, _ptr(y), n, out, in_, route_kernel, _ptr(workspace),
                                      _nbytes(workspace, workspace_bytes),
                                      _stream(stream, y, x)), "q4_0_matmul_routed_ex")


def q4_0_select_route(n: int, k: int, n_experts: int, out: int, in_: int) -> int:
    return _check(_lib.q4_0_select_route(n, k, n_experts, out, in_), "q4_0_select_route")


def q4_0_routed_workspace_size(n: int, k: int, n_experts: int, out: int, in_: int,
                               route_kernel: int = ROUTE_AUTO) -> int:
    return _size(_lib.q4_0_routed_workspace_size, "q4_0_routed_workspace_size",
                 n, k, n_experts, out, in_, route_kernel)


def q4_0_mfma_loop(sink, workgroups: int, iters: int, stream=None) -> int:
    """Enqueue the MFMA loop measurement aid; returns the launch's flops."""
    flops = _i64(0)
    _check(_lib.q4_0_mfma_loop(_ptr(sink), workgroups, iters, ctypes.byref(flops),
                               _stream(stream, sink)), "q4_0_mfma_loop")
    return flops.value


def q4_0_stream_read(src, nbytes: int, sink, workgroups: int, stream=None) -> None:
    """Enqueue the streaming-read measurement aid (nbytes == 0: an empty launch)."""
    _check(_lib.q4_0_stream_read(_ptr(src), nbytes, _ptr(sink), workgroups,
                                 _stream(stream, sink)), "q4_0_stream_read")


# ---- torch conveniences (allocation through torch, then the C calls above) --
def dtype_code(x) -> int:
    """Q4_0_F32 or Q4_0_F16 for a torch tensor's dtype."""
    import torch
    if x.dtype == torch.float32:
        return F32
    if x.dtype == torch.float16:
        return F16
    raise TypeError(f"x must be float32 or float16, not {x.dtype}")


def workspace(nbytes: int, device):
    """A workspace of nbytes on `device` (torch's allocator aligns to at least
    512 bytes), or None when nothing is needed."""
    import torch
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def repacked(blocks, out: int, in_: int, stream=None):
    """Repack a uint8 CUDA tensor of GGUF blocks into a new packed tensor."""
    import torch
    packed = torch.empty(q4_0_packed_bytes(out, in_), dtype=torch.uint8,
                         device=blocks.device)
    q4_0_repack(blocks, packed, out, in_, stream)
    return packed


def matmul(packed, x, out: int, y=None, kernel: int = KERNEL_AUTO, stream=None, ws=None):
    """y[n x out] = x . W^T for a 2-D CUDA tensor x (float32 or float16)."""
    import torch
    n, in_ = x.shape
    if y is None:
        y = torch.empty((n, out), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = workspace(q4_0_matmul_workspace_size(n, out, in_, dtype_code(x), kernel), x.device)
    q4_0_matmul_ex(packed, x, dtype_code(x), y, n, out, in_, kernel, ws, None, stream)
    return y


def matmul_grouped(linears, x_dtype: int, n: int, stream=None, ws=None):
    """q4_0_matmul_grouped with its workspace allocated through torch."""
    if ws is None and linears:
        dev = next(t.device for t in linears[0][:3] if hasattr(t, "device"))
        ws = workspace(q4_0_grouped_workspace_size(linears, x_dtype, n), dev)
    q4_0_matmul_grouped(linears, x_dtype, n, ws, None, stream)


def matmul_argmax(packed, x, out: int, y=None, stream=None, ws=None):
    """(max value [n] float32, max index [n] int32) of y = x . W^T per row;
    y is written when given."""
    import torch
    n, in_ = x.shape
    mv = torch.empty(n, dtype=torch.float32, device=x.device)
    mi = torch.empty(n, dtype=torch.int32, device=x.device)
    if ws is None:
        ws = workspace(q4_0_argmax_workspace_size(n, out, in_, dtype_code(x)), x.device)
    q4_0_matmul_argmax(packed, x, dtype_code(x), y, n, out, in_, mv, mi, ws, None, stream)
    return mv, mi


def quantize_x8(x, stream=None):
    """(q int8 [n x in], d float32 [n x in/32]) of a 2-D CUDA tensor x."""
    import torch
    n, in_ = x.shape
    q = torch.empty((n, in_), dtype=torch.int8, device=x.device)
    d = torch.empty((n, in_ // 32), dtype=torch.float32, device=x.device)
    q4_0_quantize_x8(x, dtype_code(x), q, d, n, in_, stream)
    return q, d


def matmul_w4a8(packed, q, d, out: int, y=None, stream=None, ws=None):
    """y [n x out] of the W4A8 product on quantized activations (q, d)."""
    import torch
    n, in_ = q.shape
    if y is None:
        y = torch.empty((n, out), dtype=torch.float32, device=q.device)
    if ws is None:
        ws = workspace(q4_0_w4a8_workspace_size(n, out, in_), q.device)
    q4_0_matmul_w4a8(packed, q, d, y, n, out, in_, ws, None, stream)
    return y


def matmul_routed(experts, n_experts: int, x, route, out: int, y=None, stream=None,
                  route_kernel: int = ROUTE_AUTO, ws=None):
    """y[t*k + j] = x[t] . W_{route[t, j]}^T for a stack of repacked experts
    (one flat uint8 tensor, n_experts matrices of q4_0_packed_bytes apart) and
    route an int32 [n x k] device tensor.  Returns y [n*k x out]."""
    import torch
    n, in_ = x.shape
    k = route.shape[1]
    if y is None:
        y = torch.empty((n * k, out), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = workspace(q4_0_routed_workspace_size(n, k, n_experts, out, in_, route_kernel),
                       x.device)
    q4_0_matmul_routed_ex(experts, n_experts, x, dtype_code(x), route, k, y, n, out, in_,
                          route_kernel, ws, None, stream)
    return y
