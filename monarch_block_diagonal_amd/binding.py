"""ctypes binding of the C ABI in include/monarch.h.

Argument marshalling only: every step of the computation runs in the HIP
kernels of libmonarch.so. Functions named like the C entry points take torch
tensors (or raw integer device pointers / None) and a stream, pass pointers
and sizes through, and raise MonarchError on a non-zero status. If the
library has not been built, every call raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

# the in-tree build; MONARCH_LIBRARY may name another build of the same
# sources (the host-sanitizer build of build_lib --sanitize)
LIB_PATH = os.environ.get("MONARCH_LIBRARY") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libmonarch.so")

MONARCH_OK = 0
MONARCH_ERR_NULL = -1
MONARCH_ERR_SHAPE = -2
MONARCH_ERR_DTYPE = -3
MONARCH_ERR_ALIGN = -4
MONARCH_ERR_WORKSPACE = -5
MONARCH_ERR_HIP = -6
MONARCH_ERR_SCRATCH = -7
# static scratch of monarch_bwd_noalloc per GPU (MONARCH_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 256 << 20

F32 = 0
BF16 = 1
ACT_NONE = 0
ACT_RELU = 1

EXPORTED = (
    "monarch_fwd", "monarch_bwd", "monarch_bwd_workspace_bytes", "monarch_fwd_traced",
    "monarch_bwd_traced", "monarch_describe", "monarch_status_string", "monarch_abi_version",
    "monarch_project", "monarch_linear_mid", "monarch_fwd_ex", "monarch_bwd_ex",
    "monarch_bwd_ex_workspace_bytes", "monarch_describe_ex", "monarch_hyper_saved_elems",
    "monarch_hyper_fwd", "monarch_hyper_bwd_workspace_bytes", "monarch_hyper_bwd",
    "monarch_hyper_describe", "monarch_dyad_fwd_workspace_bytes", "monarch_dyad_fwd",
    "monarch_dyad_bwd_workspace_bytes",
    "monarch_dyad_bwd", "monarch_dyad_describe", "monarch_bwd_noalloc", "monarch_stream_copy",
)

_lib = None


class MonarchError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"monarch status {status}: {message}")
        self.status = status


def load_library():
    """Loads libmonarch.so (once). Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built; run `python -m monarch_block_diagonal_amd.build_lib` "
            "(the Monarch path has no CPU fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, c_int, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    shape = [i64] * 5
    lib.monarch_fwd.argtypes = [vp] * 5 + shape + [c_int, c_int, vp]
    lib.monarch_fwd.restype = c_int
    lib.monarch_fwd_traced.argtypes = [vp] * 5 + shape + [c_int, c_int, vp, ctypes.POINTER(vp), c_int]
    lib.monarch_fwd_traced.restype = c_int
    lib.monarch_bwd_workspace_bytes.argtypes = shape + [c_int]
    lib.monarch_bwd_workspace_bytes.restype = sz
    lib.monarch_bwd.argtypes = [vp] * 10 + [sz] + shape + [c_int, c_int, vp]
    lib.monarch_bwd.restype = c_int
    lib.monarch_bwd_traced.argtypes = [vp] * 10 + [sz] + shape + [c_int, c_int, vp,
                                                                   ctypes.POINTER(vp), c_int]
    lib.monarch_bwd_traced.restype = c_int
    lib.monarch_bwd_noalloc.argtypes = [vp] * 9 + shape + [c_int, c_int, vp]
    lib.monarch_bwd_noalloc.restype = c_int
    lib.monarch_stream_copy.argtypes = [vp, vp, sz, vp]
    lib.monarch_stream_copy.restype = c_int
    lib.monarch_describe.argtypes = [c_int] + shape + [c_int, c_int, ctypes.c_char_p, sz]
    lib.monarch_describe.restype = c_int
    lib.monarch_status_string.argtypes = [c_int]
    lib.monarch_status_string.restype = ctypes.c_char_p
    lib.monarch_abi_version.argtypes = []
    lib.monarch_abi_version.restype = c_int
    lib.monarch_project.argtypes = [vp] * 3 + [i64] * 4 + [c_int, c_int, vp, vp]
    lib.monarch_project.restype = c_int
    ev = [ctypes.POINTER(vp), c_int]
    lib.monarch_linear_mid.argtypes = [i64] * 3
    lib.monarch_linear_mid.restype = i64
    lib.monarch_fwd_ex.argtypes = [vp] * 6 + [i64] * 6 + [c_int, c_int, vp] + ev
    lib.monarch_fwd_ex.restype = c_int
    lib.monarch_bwd_ex_workspace_bytes.argtypes = [i64] * 6 + [c_int, c_int]
    lib.monarch_bwd_ex_workspace_bytes.restype = sz
    lib.monarch_bwd_ex.argtypes = [vp] * 11 + [sz] + [i64] * 6 + [c_int, c_int, vp] + ev
    lib.monarch_bwd_ex.restype = c_int
    lib.monarch_describe_ex.argtypes = [c_int] + [i64] * 6 + [c_int, c_int, c_int,
                                                             ctypes.c_char_p, sz]
    lib.monarch_describe_ex.restype = c_int
    pp, pi64 = ctypes.POINTER(vp), ctypes.POINTER(i64)
    lib.monarch_hyper_saved_elems.argtypes = [c_int, pi64, i64]
    lib.monarch_hyper_saved_elems.restype = sz
    lib.monarch_hyper_fwd.argtypes = [vp, pp, vp, vp, c_int, pi64, i64, c_int, vp] + ev
    lib.monarch_hyper_fwd.restype = c_int
    lib.monarch_hyper_bwd_workspace_bytes.argtypes = [c_int, pi64, i64, c_int]
    lib.monarch_hyper_bwd_workspace_bytes.restype = sz
    lib.monarch_hyper_bwd.argtypes = [vp, vp, pp, vp, vp, pp, vp, sz, c_int, pi64, i64, c_int,
                                      vp] + ev
    lib.monarch_hyper_bwd.restype = c_int
    lib.monarch_hyper_describe.argtypes = [c_int, c_int, pi64, i64, c_int, ctypes.c_char_p, sz]
    lib.monarch_hyper_describe.restype = c_int
    lib.monarch_dyad_fwd_workspace_bytes.argtypes = [i64] * 4 + [c_int]
    lib.monarch_dyad_fwd_workspace_bytes.restype = sz
    lib.monarch_dyad_fwd.argtypes = [vp] * 5 + [sz] + [i64] * 4 + [c_int, vp] + ev
    lib.monarch_dyad_fwd.restype = c_int
    lib.monarch_dyad_bwd_workspace_bytes.argtypes = [i64] * 4 + [c_int]
    lib.monarch_dyad_bwd_workspace_bytes.restype = sz
    lib.monarch_dyad_bwd.argtypes = [vp] * 8 + [sz] + [i64] * 4 + [c_int, vp] + ev
    lib.monarch_dyad_bwd.restype = c_int
    lib.monarch_dyad_describe.argtypes = [c_int] + [i64] * 4 + [c_int, ctypes.c_char_p, sz]
    lib.monarch_dyad_describe.restype = c_int
    _lib = lib
    return lib


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _events(events: Optional[Sequence]):
    """Raw hipEvent_t handles. torch creates its events lazily, on first
    record, so an uninitialised torch event is recorded once here first."""
    if events is None:
        return None, 0
    handles = []
    for e in events:
        if hasattr(e, "cuda_event"):
            if not e.cuda_event:
                e.record()
            handles.append(e.cuda_event)
        else:
            handles.append(e)
    arr = (ctypes.c_void_p * len(handles))(*handles)
    return arr, len(handles)


def _check(status: int) -> None:
    if status != MONARCH_OK:
        raise MonarchError(status, load_library().monarch_status_string(status).decode())


def monarch_status_string(status: int) -> str:
    return load_library().monarch_status_string(status).decode()


def monarch_abi_version() -> int:
    return load_library().monarch_abi_version()


def monarch_fwd(x, w1, w2, y, z, in_features, out_features, nblocks1, nblocks2, batch, dtype,
                act=ACT_NONE, stream=None, events=None) -> None:
    lib = load_library()
    args = [_ptr(x), _ptr(w1), _ptr(w2), _ptr(y), _ptr(z), in_features, out_features, nblocks1,
            nblocks2, batch, dtype, act, _stream(stream)]
    if events is None:
        _check(lib.monarch_fwd(*args))
    else:
        arr, n = _events(events)
        _check(lib.monarch_fwd_traced(*args, arr, n))


def monarch_bwd_workspace_bytes(in_features, out_features, nblocks1, nblocks2, batch, dtype) -> int:
    return load_library().monarch_bwd_workspace_bytes(in_features, out_features, nblocks1,
                                                      nblocks2, batch, dtype)


def monarch_bwd(dy, x, w1, w2, z, y, dx, dw1, dw2, workspace, workspace_bytes, in_features,
                out_features, nblocks1, nblocks2, batch, dtype, act=ACT_NONE, stream=None,
                events=None) -> None:
    lib = load_library()
    args = [_ptr(dy), _ptr(x), _ptr(w1), _ptr(w2), _ptr(z), _ptr(y), _ptr(dx), _ptr(dw1),
            _ptr(dw2), _ptr(workspace), workspace_bytes, in_features, out_features, nblocks1,
            nblocks2, batch, dtype, act, _stream(stream)]
    if events is None:
        _check(lib.monarch_bwd(*args))
    else:
        arr, n = _events(events)
        _check(lib.monarch_bwd_traced(*args, arr, n))


def monarch_bwd_noalloc(dy, x, w1, w2, z, y, dx, dw1, dw2, in_features, out_features, nblocks1,
                        nblocks2, batch, dtype, act=ACT_NONE, stream=None) -> None:
    lib = load_library()
    _check(lib.monarch_bwd_noalloc(_ptr(dy), _ptr(x), _ptr(w1), _ptr(w2), _ptr(z), _ptr(y),
                                   _ptr(dx), _ptr(dw1), _ptr(dw2), in_features, out_features,
                                   nblocks1, nblocks2, batch, dtype, act, _stream(stream)))


def monarch_stream_copy(src, dst, nbytes, stream=None) -> None:
    """Device copy of nbytes from src to dst (the HBM roofline reference)."""
    _check(load_library().monarch_stream_copy(_ptr(src), _ptr(dst), nbytes, _stream(stream)))


def monarch_project(m, w1, w2, in_features, out_features, nblocks1, nblocks2, dtype,
                    max_steps=256, converged=None, stream=None) -> None:
    lib = load_library()
    _check(lib.monarch_project(_ptr(m), _ptr(w1), _ptr(w2), in_features, out_features, nblocks1,
                               nblocks2, dtype, max_steps, _ptr(converged), _stream(stream)))


def monarch_describe(direction, in_features, out_features, nblocks1, nblocks2, batch, dtype,
                     act=ACT_NONE):
    """Returns the list of kernel names monarch_fwd (0) / monarch_bwd (1) launches."""
    lib = load_library()
    buf = ctypes.create_string_buffer(1024)
    n = lib.monarch_describe(direction, in_features, out_features, nblocks1, nblocks2, batch,
                             dtype, act, buf, len(buf))
    if n < 0:
        raise MonarchError(n, monarch_status_string(n))
    names = buf.value.decode().split(";") if n else []
    return names


def monarch_linear_mid(in_features, out_features, nblocks) -> int:
    """The MonarchLinear intermediate width for one block count."""
    v = load_library().monarch_linear_mid(in_features, out_features, nblocks)
    if v < 0:
        raise MonarchError(int(v), monarch_status_string(int(v)))
    return int(v)


def monarch_fwd_ex(x, w1, w2, bias, y, z, in_features, out_features, mid_features, nblocks1,
                   nblocks2, batch, dtype, act=ACT_NONE, stream=None, events=None) -> None:
    lib = load_library()
    arr, n = _events(events)
    _check(lib.monarch_fwd_ex(_ptr(x), _ptr(w1), _ptr(w2), _ptr(bias), _ptr(y), _ptr(z),
                              in_features, out_features, mid_features, nblocks1, nblocks2, batch,
                              dtype, act, _stream(stream), arr, n))


def monarch_bwd_ex_workspace_bytes(in_features, out_features, mid_features, nblocks1, nblocks2,
                                   batch, dtype, with_bias=False) -> int:
    return load_library().monarch_bwd_ex_workspace_bytes(in_features, out_features, mid_features,
                                                         nblocks1, nblocks2, batch, dtype,
                                                         1 if with_bias else 0)


def monarch_bwd_ex(dy, x, w1, w2, z, y, dx, dw1, dw2, dbias, workspace, workspace_bytes,
                   in_features, out_features, mid_features, nblocks1, nblocks2, batch, dtype,
                   act=ACT_NONE, stream=None, events=None) -> None:
    lib = load_library()
    arr, n = _events(events)
    _check(lib.monarch_bwd_ex(_ptr(dy), _ptr(x), _ptr(w1), _ptr(w2), _ptr(z), _ptr(y), _ptr(dx),
                              _ptr(dw1), _ptr(dw2), _ptr(dbias), _ptr(workspace), workspace_bytes,
                              in_features, out_features, mid_features, nblocks1, nblocks2, batch,
                              dtype, act, _stream(stream), arr, n))


def monarch_describe_ex(direction, in_features, out_features, mid_features, nblocks1, nblocks2,
                        batch, dtype, act=ACT_NONE, with_bias=False):
    """Kernel names monarch_fwd_ex (0) / monarch_bwd_ex (1) launches."""
    lib = load_library()
    buf = ctypes.create_string_buffer(1024)
    n = lib.monarch_describe_ex(direction, in_features, out_features, mid_features, nblocks1,
                                nblocks2, batch, dtype, act, 1 if with_bias else 0, buf, len(buf))
    if n < 0:
        raise MonarchError(n, monarch_status_string(n))
    return buf.value.decode().split(";") if n else []


def _dims(dims):
    return (ctypes.c_int64 * len(dims))(*[int(d) for d in dims]), len(dims)


def _ptrs(ts):
    return (ctypes.c_void_p * len(ts))(*[_ptr(t) for t in ts])


def monarch_hyper_saved_elems(dims, batch) -> int:
    d, k = _dims(dims)
    return load_library().monarch_hyper_saved_elems(k, d, batch)


def monarch_hyper_fwd(x, ws, y, saved, dims, batch, dtype, stream=None, events=None) -> None:
    lib = load_library()
    d, k = _dims(dims)
    arr, n = _events(events)
    _check(lib.monarch_hyper_fwd(_ptr(x), _ptrs(ws), _ptr(y), _ptr(saved), k, d, batch, dtype,
                                 _stream(stream), arr, n))


def monarch_hyper_bwd_workspace_bytes(dims, batch, dtype) -> int:
    d, k = _dims(dims)
    return load_library().monarch_hyper_bwd_workspace_bytes(k, d, batch, dtype)


def monarch_hyper_bwd(dy, x, ws, saved, dx, dws, workspace, workspace_bytes, dims, batch, dtype,
                      stream=None, events=None) -> None:
    lib = load_library()
    d, k = _dims(dims)
    arr, n = _events(events)
    _check(lib.monarch_hyper_bwd(_ptr(dy), _ptr(x), _ptrs(ws), _ptr(saved), _ptr(dx), _ptrs(dws),
                                 _ptr(workspace), workspace_bytes, k, d, batch, dtype,
                                 _stream(stream), arr, n))


def monarch_hyper_describe(direction, dims, batch, dtype):
    lib = load_library()
    d, k = _dims(dims)
    buf = ctypes.create_string_buffer(1024)
    n = lib.monarch_hyper_describe(direction, k, d, batch, dtype, buf, len(buf))
    if n < 0:
        raise MonarchError(n, monarch_status_string(n))
    return buf.value.decode().split(";") if n else []


def monarch_dyad_fwd_workspace_bytes(in_features, out_features, nblocks, batch, dtype) -> int:
    return load_library().monarch_dyad_fwd_workspace_bytes(in_features, out_features, nblocks,
                                                           batch, dtype)


def monarch_dyad_fwd(x, wa, wb, y, workspace, workspace_bytes, in_features, out_features, nblocks,
                     batch, dtype, stream=None, events=None) -> None:
    lib = load_library()
    arr, n = _events(events)
    _check(lib.monarch_dyad_fwd(_ptr(x), _ptr(wa), _ptr(wb), _ptr(y), _ptr(workspace),
                                workspace_bytes, in_features, out_features, nblocks, batch, dtype,
                                _stream(stream), arr, n))


def monarch_dyad_bwd_workspace_bytes(in_features, out_features, nblocks, batch, dtype) -> int:
    return load_library().monarch_dyad_bwd_workspace_bytes(in_features, out_features, nblocks,
                                                           batch, dtype)


def monarch_dyad_bwd(dy, x, wa, wb, dx, dwa, dwb, workspace, workspace_bytes, in_features,
                     out_features, nblocks, batch, dtype, stream=None, events=None) -> None:
    lib = load_library()
    arr, n = _events(events)
    _check(lib.monarch_dyad_bwd(_ptr(dy), _ptr(x), _ptr(wa), _ptr(wb), _ptr(dx), _ptr(dwa),
                                _ptr(dwb), _ptr(workspace), workspace_bytes, in_features,
                                out_features, nblocks, batch, dtype, _stream(stream), arr, n))


def monarch_dyad_describe(direction, in_features, out_features, nblocks, batch, dtype):
    lib = load_library()
    buf = ctypes.create_string_buffer(1024)
    n = lib.monarch_dyad_describe(direction, in_features, out_features, nblocks, batch, dtype, buf,
                                  len(buf))
    if n < 0:
        raise MonarchError(n, monarch_status_string(n))
    return buf.value.decode().split(";") if n else []
