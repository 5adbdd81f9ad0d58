"""ctypes binding of libdquant (include/dquant.h).

The functions named ``dq_*`` mirror the C entry points one for one and only
marshal arguments: torch tensors become ``dq_tensor`` descriptors (data
pointer, dtype code, dims), executors travel as opaque handles, the stream
is the current HIP stream unless one is given.  The convenience wrappers
``dynamic_quant``, ``ada_layernorm_quant`` and ``antiquantize`` allocate the
outputs with torch (device memory only) and run both phases.

Every computation happens in the HIP kernels of ``libdquant.so``; there is
no fallback of any kind.  If the library has not been built, every call
raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# DQ_LIBRARY selects another build of the library (the CPU sanitizer test
# loads a host-only AddressSanitizer / UBSan build of the validation layer).
library_path = os.environ.get("DQ_LIBRARY") or os.path.join(_HERE, "libdquant.so")

# dq_status
SUCCESS, ERR_NULLPTR, ERR_DTYPE, ERR_SHAPE, ERR_ALIGN, ERR_PARAM, ERR_OVERLAP, ERR_WORKSPACE, \
    ERR_RUNTIME = range(9)
STATUS_NAMES = ["DQ_SUCCESS", "DQ_ERR_NULLPTR", "DQ_ERR_DTYPE", "DQ_ERR_SHAPE", "DQ_ERR_ALIGN",
                "DQ_ERR_PARAM", "DQ_ERR_OVERLAP", "DQ_ERR_WORKSPACE", "DQ_ERR_RUNTIME"]
# dq_dtype
F32, F16, BF16, I8, I4, I32, F8E4M3, F8E5M2, F4E2M1, E8M0 = range(10)
# dq_antiquant_policy
POLICIES = {"per_tensor": 0, "per_channel": 1, "per_token": 2, "per_group": 3}

MAX_DIMS = 8

EXPORTS = [
    "dq_dynamic_quant_get_workspace_size", "dq_dynamic_quant",
    "dq_ada_layernorm_quant_get_workspace_size", "dq_ada_layernorm_quant",
    "dq_antiquantize_get_workspace_size", "dq_antiquantize",
    "dq_mx_quantize_get_workspace_size", "dq_mx_quantize",
    "dq_weight_quant_matmul_get_workspace_size", "dq_weight_quant_matmul",
    "dq_executor_destroy", "dq_get_last_error", "dq_copy_probe",
    "dq_weight_quant_matmul_noalloc",
]


class DquantError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        name = STATUS_NAMES[status] if 0 <= status < len(STATUS_NAMES) else str(status)
        super().__init__(f"{name}: {message}")


class DqTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int), ("ndim", ctypes.c_int32),
                ("dims", ctypes.c_int64 * MAX_DIMS)]


_P = ctypes.POINTER
_vp = ctypes.c_void_p
_lib: Optional[ctypes.CDLL] = None


def library() -> ctypes.CDLL:
    """Load libdquant.so (built in-tree).  Raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise RuntimeError(f"{library_path} is not built; run __graft_entry__.build() "
                               "(hipcc, gfx950) first -- there is no fallback path")
        lib = ctypes.CDLL(library_path)
        st = ctypes.c_int
        lib.dq_dynamic_quant_get_workspace_size.argtypes = [
            _P(DqTensor), _P(DqTensor), _P(DqTensor), ctypes.c_int, _P(DqTensor), _P(DqTensor),
            _P(DqTensor), _P(ctypes.c_size_t), _P(_vp)]
        lib.dq_dynamic_quant_get_workspace_size.restype = st
        lib.dq_ada_layernorm_quant_get_workspace_size.argtypes = [
            _P(DqTensor), _P(DqTensor), _P(DqTensor), _P(DqTensor), _P(DqTensor), _P(DqTensor),
            ctypes.c_double, _P(DqTensor), _P(DqTensor), _P(ctypes.c_size_t), _P(_vp)]
        lib.dq_ada_layernorm_quant_get_workspace_size.restype = st
        lib.dq_antiquantize_get_workspace_size.argtypes = [
            _P(DqTensor), _P(DqTensor), _P(DqTensor), ctypes.c_int, ctypes.c_int32, ctypes.c_uint32,
            _P(DqTensor), _P(ctypes.c_size_t), _P(_vp)]
        lib.dq_antiquantize_get_workspace_size.restype = st
        lib.dq_mx_quantize_get_workspace_size.argtypes = [
            _P(DqTensor), ctypes.c_int32, _P(DqTensor), _P(DqTensor), _P(ctypes.c_size_t), _P(_vp)]
        lib.dq_mx_quantize_get_workspace_size.restype = st
        lib.dq_weight_quant_matmul_get_workspace_size.argtypes = [
            _P(DqTensor), _P(DqTensor), ctypes.c_int32, _P(DqTensor), _P(DqTensor), ctypes.c_int64,
            _P(DqTensor), _P(DqTensor), _P(DqTensor), _P(ctypes.c_size_t), _P(_vp)]
        lib.dq_weight_quant_matmul_get_workspace_size.restype = st
        lib.dq_weight_quant_matmul_noalloc.argtypes = [
            _P(DqTensor), _P(DqTensor), ctypes.c_int32, _P(DqTensor), _P(DqTensor), ctypes.c_int64,
            _P(DqTensor), _P(DqTensor), _P(DqTensor), _vp]
        lib.dq_weight_quant_matmul_noalloc.restype = st
        for name in ("dq_dynamic_quant", "dq_ada_layernorm_quant", "dq_antiquantize",
                     "dq_mx_quantize", "dq_weight_quant_matmul"):
            fn = getattr(lib, name)
            fn.argtypes = [_vp, ctypes.c_size_t, _vp, _vp]
            fn.restype = st
        lib.dq_executor_destroy.argtypes = [_vp]
        lib.dq_executor_destroy.restype = None
        lib.dq_get_last_error.argtypes = []
        lib.dq_get_last_error.restype = ctypes.c_char_p
        lib.dq_copy_probe.argtypes = [_vp, _vp, ctypes.c_size_t, _vp]
        lib.dq_copy_probe.restype = st
        _lib = lib
    return _lib


def dq_get_last_error() -> str:
    return library().dq_get_last_error().decode()


def _check(status: int) -> None:
    if status != SUCCESS:
        raise DquantError(status, dq_get_last_error())


_TORCH_CODES = {
    torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16, torch.int8: I8,
    torch.int32: I32, torch.float8_e4m3fn: F8E4M3, torch.float8_e5m2: F8E5M2,
    torch.float4_e2m1fn_x2: F4E2M1, torch.float8_e8m0fnu: E8M0,
}


def tensor_desc(t: Optional[torch.Tensor], dtype: Optional[int] = None,
                dims: Optional[Sequence[int]] = None) -> Optional[DqTensor]:
    """Descriptor of a dense row-major tensor (None stays None).

    ``dtype`` / ``dims`` override the tensor's own; an INT4 output travels as
    a uint8 tensor of packed bytes with dtype=I4 and its logical dims, and a
    torch.float4_e2m1fn_x2 tensor [..., k] describes k * 2 codes.
    """
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("libdquant takes dense row-major tensors")
    if t.numel() > 0 and not t.is_cuda:
        raise ValueError(f"libdquant takes tensors in GPU memory, got one on {t.device}")
    d = DqTensor()
    d.data = t.data_ptr() if t.numel() > 0 else None
    d.dtype = _TORCH_CODES[t.dtype] if dtype is None else dtype
    shape = list(t.shape) if dims is None else list(dims)
    if dims is None and t.dtype == torch.float4_e2m1fn_x2 and shape:
        shape[-1] *= 2  # each element holds two 4-bit codes
    if len(shape) > MAX_DIMS:
        raise ValueError("at most 8 dimensions")
    d.ndim = len(shape)
    for i, s in enumerate(shape):
        d.dims[i] = int(s)
    return d


def _one_device(*tensors) -> Optional[torch.device]:
    """The device all non-empty tensors of one call share; raises if they
    are spread over several (a kernel runs on one device and reads its own
    memory)."""
    devs = {t.device for t in tensors if t is not None and t.numel() > 0}
    if len(devs) > 1:
        raise ValueError(f"the tensors of one call must be on one device, got {sorted(map(str, devs))}")
    return devs.pop() if devs else None


def _ref(d: Optional[DqTensor]):
    return None if d is None else ctypes.byref(d)


def _stream_handle(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _stream_on(stream, device):
    """The caller's stream, else the current stream of the device the
    tensors live on (not of whichever device is current)."""
    if stream is not None or device is None or device.type != "cuda":
        return stream
    return torch.cuda.current_stream(device)


def _y_desc(y: torch.Tensor, x_shape, out_dtype: Optional[str]):
    if out_dtype is None:
        out_dtype = {torch.int8: "int8", torch.int32: "int32", torch.uint8: "int4"}[y.dtype]
    if out_dtype == "int4":
        return tensor_desc(y, I4, list(x_shape))
    if out_dtype == "int32":
        return tensor_desc(y, I32)
    return tensor_desc(y, I8)


# -- phase 1 / phase 2 entry points, named as in dquant.h ---------------------

def dq_dynamic_quant_get_workspace_size(x, smooth_scales, group_index, symmetric, y, scale, offset,
                                        out_dtype: Optional[str] = None) -> Tuple[int, int]:
    """Returns (workspace_size, executor handle).  ``y`` is int8 (INT8),
    uint8 [..., N/2] (INT4) or int32 [..., N/8] (INT32)."""
    lib = library()
    _one_device(x, smooth_scales, group_index, y, scale, offset)
    descs = [tensor_desc(x), tensor_desc(smooth_scales), tensor_desc(group_index),
             _y_desc(y, x.shape, out_dtype), tensor_desc(scale), tensor_desc(offset)]
    ws = ctypes.c_size_t(0)
    ex = _vp(None)
    _check(lib.dq_dynamic_quant_get_workspace_size(
        _ref(descs[0]), _ref(descs[1]), _ref(descs[2]), 1 if symmetric else 0, _ref(descs[3]),
        _ref(descs[4]), _ref(descs[5]), ctypes.byref(ws), ctypes.byref(ex)))
    return ws.value, ex.value


def dq_dynamic_quant(workspace, workspace_size: int, executor: int, stream=None) -> None:
    _check(library().dq_dynamic_quant(_ws_ptr(workspace), workspace_size, executor,
                                      _stream_handle(stream)))


def dq_ada_layernorm_quant_get_workspace_size(x, scale, shift, weight, bias, smooth_scales,
                                              epsilon: float, out, quant_scale) -> Tuple[int, int]:
    lib = library()
    _one_device(x, scale, shift, weight, bias, smooth_scales, out, quant_scale)
    d = [tensor_desc(t) for t in (x, scale, shift, weight, bias, smooth_scales, out, quant_scale)]
    ws = ctypes.c_size_t(0)
    ex = _vp(None)
    _check(lib.dq_ada_layernorm_quant_get_workspace_size(
        _ref(d[0]), _ref(d[1]), _ref(d[2]), _ref(d[3]), _ref(d[4]), _ref(d[5]), float(epsilon),
        _ref(d[6]), _ref(d[7]), ctypes.byref(ws), ctypes.byref(ex)))
    return ws.value, ex.value


def dq_ada_layernorm_quant(workspace, workspace_size: int, executor: int, stream=None) -> None:
    _check(library().dq_ada_layernorm_quant(_ws_ptr(workspace), workspace_size, executor,
                                            _stream_handle(stream)))


def dq_antiquantize_get_workspace_size(src, scale, offset, policy, k_dim: int, group_size: int,
                                       dst) -> Tuple[int, int]:
    lib = library()
    pol = POLICIES[policy] if isinstance(policy, str) else int(policy)
    _one_device(src, scale, offset, dst)
    d = [tensor_desc(t) for t in (src, scale, offset, dst)]
    ws = ctypes.c_size_t(0)
    ex = _vp(None)
    _check(lib.dq_antiquantize_get_workspace_size(
        _ref(d[0]), _ref(d[1]), _ref(d[2]), pol, int(k_dim), int(group_size), _ref(d[3]),
        ctypes.byref(ws), ctypes.byref(ex)))
    return ws.value, ex.value


def dq_antiquantize(workspace, workspace_size: int, executor: int, stream=None) -> None:
    _check(library().dq_antiquantize(_ws_ptr(workspace), workspace_size, executor,
                                     _stream_handle(stream)))


def dq_mx_quantize_get_workspace_size(x, axis: int, y, scale) -> Tuple[int, int]:
    lib = library()
    _one_device(x, y, scale)
    d = [tensor_desc(t) for t in (x, y, scale)]
    ws = ctypes.c_size_t(0)
    ex = _vp(None)
    _check(lib.dq_mx_quantize_get_workspace_size(_ref(d[0]), int(axis), _ref(d[1]), _ref(d[2]),
                                                 ctypes.byref(ws), ctypes.byref(ex)))
    return ws.value, ex.value


def dq_mx_quantize(workspace, workspace_size: int, executor: int, stream=None) -> None:
    _check(library().dq_mx_quantize(_ws_ptr(workspace), workspace_size, executor,
                                    _stream_handle(stream)))


def _w_desc(x2, weight: Optional[str]):
    """int8 weights as they are; int4 weights travel as uint8 bytes holding two
    codes each along the stored last dimension."""
    if weight is None:
        weight = "int8" if x2.dtype == torch.int8 else "int4"
    if weight == "int4":
        r, c = x2.shape
        return tensor_desc(x2, I4, [r, 2 * c])
    return tensor_desc(x2, I8)


def _wq_descs(x1, x2, antiquant_scale, antiquant_offset, bias, x3, out, weight):
    _one_device(x1, x2, antiquant_scale, antiquant_offset, bias, x3, out)
    return [tensor_desc(x1), _w_desc(x2, weight), tensor_desc(antiquant_scale),
            tensor_desc(antiquant_offset), tensor_desc(bias), tensor_desc(x3), tensor_desc(out)]


def dq_weight_quant_matmul_get_workspace_size(x1, x2, transpose_x2, antiquant_scale,
                                              antiquant_offset, group_size, bias, x3, out,
                                              weight: Optional[str] = None) -> Tuple[int, int]:
    lib = library()
    d = _wq_descs(x1, x2, antiquant_scale, antiquant_offset, bias, x3, out, weight)
    ws = ctypes.c_size_t(0)
    ex = _vp(None)
    _check(lib.dq_weight_quant_matmul_get_workspace_size(
        _ref(d[0]), _ref(d[1]), 1 if transpose_x2 else 0, _ref(d[2]), _ref(d[3]), int(group_size),
        _ref(d[4]), _ref(d[5]), _ref(d[6]), ctypes.byref(ws), ctypes.byref(ex)))
    return ws.value, ex.value


def dq_weight_quant_matmul(workspace, workspace_size: int, executor: int, stream=None) -> None:
    _check(library().dq_weight_quant_matmul(_ws_ptr(workspace), workspace_size, executor,
                                            _stream_handle(stream)))


def dq_weight_quant_matmul_noalloc(x1, x2, transpose_x2, antiquant_scale, antiquant_offset, group_size,
                                   bias, x3, out, stream=None, weight: Optional[str] = None) -> None:
    """The allocation-free call: split-k partial sums go to the library's
    per-GPU scratch array (at most WQ_SCRATCH_BYTES); out is written in place."""
    lib = library()
    d = _wq_descs(x1, x2, antiquant_scale, antiquant_offset, bias, x3, out, weight)
    _check(lib.dq_weight_quant_matmul_noalloc(
        _ref(d[0]), _ref(d[1]), 1 if transpose_x2 else 0, _ref(d[2]), _ref(d[3]), int(group_size),
        _ref(d[4]), _ref(d[5]), _ref(d[6]), _stream_handle(stream)))


WQ_SCRATCH_BYTES = 32 << 20  # DQ_WQ_SCRATCH_BYTES in include/dquant.h


def dq_executor_destroy(executor: int) -> None:
    library().dq_executor_destroy(executor)


def dq_copy_probe(dst: torch.Tensor, src: torch.Tensor, nbytes: Optional[int] = None,
                  stream=None) -> None:
    n = src.numel() * src.element_size() if nbytes is None else nbytes
    if not (src.is_cuda and dst.is_cuda) or _one_device(dst, src) is None:
        raise ValueError("the copy probe takes two non-empty tensors on one GPU")
    _check(library().dq_copy_probe(dst.data_ptr(), src.data_ptr(), n, _stream_handle(stream)))


def _ws_ptr(workspace) -> Optional[int]:
    if workspace is None:
        return None
    if isinstance(workspace, int):
        return workspace
    return workspace.data_ptr()


def _workspace(size: int, device) -> Optional[torch.Tensor]:
    return torch.empty(size, dtype=torch.uint8, device=device) if size > 0 else None


def _release_after(workspace: Optional[torch.Tensor], stream) -> None:
    """A workspace dropped on return goes back to torch's caching allocator,
    which may hand it out again on the stream it was allocated on while the
    kernel that uses it still runs on `stream`: record that stream on it so
    the memory is reused only after the work queued there so far."""
    if workspace is None or stream is None:
        return
    if isinstance(stream, int):
        stream = torch.cuda.ExternalStream(stream, device=workspace.device)
    workspace.record_stream(stream)


# -- prepared calls: descriptors built once, both phases per call ---------------

class PreparedCall:
    """Both phases of one op with fixed tensors: the dq_tensor descriptors are
    built once, so each call is the get-workspace-size call plus the execute
    call (two C calls, no per-call Python marshalling of tensors).  A
    workspace, when the op asks for one, is allocated on the first call and
    reused while it is large enough, so calls of one PreparedCall on
    different streams must be ordered by the caller."""

    def __init__(self, phase1, execute, args, keep, device=None):
        self._phase1 = phase1
        self._execute = execute
        self._ws = ctypes.c_size_t(0)
        self._ex = _vp(None)
        self._args = tuple(args) + (ctypes.byref(self._ws), ctypes.byref(self._ex))
        self._keep = keep  # descriptors and tensors referenced by the args
        self._device = device
        self._workspace: Optional[torch.Tensor] = None

    def __call__(self, stream=None) -> None:
        st = self._phase1(*self._args)
        if st != SUCCESS:
            raise DquantError(st, dq_get_last_error())
        size = self._ws.value
        ptr = None
        if size:
            if self._device is None:
                library().dq_executor_destroy(self._ex)
                raise DquantError(ERR_WORKSPACE, "this prepared call has no device for a workspace")
            if self._workspace is None or self._workspace.numel() < size:
                self._workspace = torch.empty(size, dtype=torch.uint8, device=self._device)
            ptr = self._workspace.data_ptr()
        st = self._execute(ptr, size, self._ex, _stream_handle(stream))
        if st != SUCCESS:
            raise DquantError(st, dq_get_last_error())


def prepare_dynamic_quant(x, smooth_scales, group_index, symmetric, y, scale, offset,
                          out_dtype: Optional[str] = None) -> PreparedCall:
    lib = library()
    _one_device(x, smooth_scales, group_index, y, scale, offset)
    d = [tensor_desc(x), tensor_desc(smooth_scales), tensor_desc(group_index),
         _y_desc(y, x.shape, out_dtype), tensor_desc(scale), tensor_desc(offset)]
    args = [_ref(d[0]), _ref(d[1]), _ref(d[2]), 1 if symmetric else 0, _ref(d[3]), _ref(d[4]),
            _ref(d[5])]
    return PreparedCall(lib.dq_dynamic_quant_get_workspace_size, lib.dq_dynamic_quant, args,
                        (d, x, smooth_scales, group_index, y, scale, offset))


def prepare_ada_layernorm_quant(x, scale, shift, weight, bias, smooth_scales, epsilon, out,
                                quant_scale) -> PreparedCall:
    lib = library()
    _one_device(x, scale, shift, weight, bias, smooth_scales, out, quant_scale)
    d = [tensor_desc(t) for t in (x, scale, shift, weight, bias, smooth_scales, out, quant_scale)]
    args = [_ref(d[0]), _ref(d[1]), _ref(d[2]), _ref(d[3]), _ref(d[4]), _ref(d[5]),
            ctypes.c_double(float(epsilon)), _ref(d[6]), _ref(d[7])]
    return PreparedCall(lib.dq_ada_layernorm_quant_get_workspace_size, lib.dq_ada_layernorm_quant,
                        args, (d, x, scale, shift, weight, bias, smooth_scales, out, quant_scale))


def prepare_antiquantize(src, scale, offset, policy, k_dim: int, group_size: int,
                         dst) -> PreparedCall:
    lib = library()
    pol = POLICIES[policy] if isinstance(policy, str) else int(policy)
    _one_device(src, scale, offset, dst)
    d = [tensor_desc(t) for t in (src, scale, offset, dst)]
    args = [_ref(d[0]), _ref(d[1]), _ref(d[2]), pol, int(k_dim), int(group_size), _ref(d[3])]
    return PreparedCall(lib.dq_antiquantize_get_workspace_size, lib.dq_antiquantize, args,
                        (d, src, scale, offset, dst))


def prepare_mx_quantize(x, axis: int, y, scale) -> PreparedCall:
    lib = library()
    _one_device(x, y, scale)
    d = [tensor_desc(t) for t in (x, y, scale)]
    args = [_ref(d[0]), int(axis), _ref(d[1]), _ref(d[2])]
    return PreparedCall(lib.dq_mx_quantize_get_workspace_size, lib.dq_mx_quantize, args,
                        (d, x, y, scale))


def prepare_weight_quant_matmul(x1, x2, transpose_x2, antiquant_scale, antiquant_offset, group_size,
                                bias, x3, out, weight: Optional[str] = None) -> PreparedCall:
    lib = library()
    d = _wq_descs(x1, x2, antiquant_scale, antiquant_offset, bias, x3, out, weight)
    args = [_ref(d[0]), _ref(d[1]), 1 if transpose_x2 else 0, _ref(d[2]), _ref(d[3]),
            ctypes.c_int64(int(group_size)), _ref(d[4]), _ref(d[5]), _ref(d[6])]
    return PreparedCall(lib.dq_weight_quant_matmul_get_workspace_size, lib.dq_weight_quant_matmul,
                        args, (d, x1, x2, antiquant_scale, antiquant_offset, bias, x3, out),
                        device=out.device)


# -- convenience wrappers ------------------------------------------------------

def dynamic_quant(x: torch.Tensor, smooth_scales: Optional[torch.Tensor] = None,
                  group_index: Optional[torch.Tensor] = None, symmetric: bool = True,
                  out_dtype: str = "int8", stream=None):
    """Per-token dynamic quantization.  Returns (y, scale, offset); offset is
    None when symmetric.  y: int8 [..., N] ('int8'), uint8 [..., N/2] packed
    ('int4'), int32 [..., N/8] ('int32')."""
    lead = tuple(x.shape[:-1])
    n = x.shape[-1]
    dev = x.device
    if out_dtype == "int8":
        y = torch.empty(x.shape, dtype=torch.int8, device=dev)
    elif out_dtype == "int4":
        y = torch.empty(lead + (n // 2,), dtype=torch.uint8, device=dev)
    elif out_dtype == "int32":
        y = torch.empty(lead + (n // 8,), dtype=torch.int32, device=dev)
    else:
        raise ValueError(f"unknown out_dtype {out_dtype}")
    scale = torch.empty(lead, dtype=torch.float32, device=dev)
    offset = None if symmetric else torch.empty(lead, dtype=torch.float32, device=dev)
    ws, ex = dq_dynamic_quant_get_workspace_size(x, smooth_scales, group_index, symmetric, y, scale,
                                                 offset, out_dtype)
    s = _stream_on(stream, dev)
    w = _workspace(ws, dev)
    dq_dynamic_quant(w, ws, ex, s)
    _release_after(w, s)
    return y, scale, offset


def ada_layernorm_quant(x: torch.Tensor, scale: torch.Tensor, shift: torch.Tensor,
                        weight: Optional[torch.Tensor] = None, bias: Optional[torch.Tensor] = None,
                        smooth_scales: Optional[torch.Tensor] = None, epsilon: float = 1e-5,
                        stream=None):
    """AdaLayerNorm + symmetric INT8 quantization.  Returns (out int8
    [B, S, H], quant_scale fp32 [B, S])."""
    B, S, _ = x.shape
    out = torch.empty(x.shape, dtype=torch.int8, device=x.device)
    qs = torch.empty((B, S), dtype=torch.float32, device=x.device)
    ws, ex = dq_ada_layernorm_quant_get_workspace_size(x, scale, shift, weight, bias, smooth_scales,
                                                       epsilon, out, qs)
    s = _stream_on(stream, x.device)
    w = _workspace(ws, x.device)
    dq_ada_layernorm_quant(w, ws, ex, s)
    _release_after(w, s)
    return out, qs


def antiquantize(src: torch.Tensor, scale: torch.Tensor, offset: Optional[torch.Tensor] = None,
                 policy="per_tensor", k_dim: int = 1, group_size: int = 0,
                 dst_dtype: torch.dtype = torch.bfloat16, stream=None) -> torch.Tensor:
    """Dequantize src [m, n] into dst_dtype.  src: int8, float8_e4m3fn,
    float8_e5m2, or float4_e2m1fn_x2 [m, n/2] (two codes per byte, with a
    float8_e8m0fnu PER_GROUP scale and no offset); scale / offset float32,
    float16 or bfloat16 for the 8-bit sources."""
    shape = list(src.shape)
    if src.dtype == torch.float4_e2m1fn_x2:
        shape[-1] *= 2
    dst = torch.empty(shape, dtype=dst_dtype, device=src.device)
    ws, ex = dq_antiquantize_get_workspace_size(src, scale, offset, policy, k_dim, group_size, dst)
    s = _stream_on(stream, src.device)
    w = _workspace(ws, src.device)
    dq_antiquantize(w, ws, ex, s)
    _release_after(w, s)
    return dst


def mx_scale_shape(rows: int, n: int, axis: int = 1) -> Tuple[int, int]:
    """Shape of the e8m0 scale of an mx-quantized [rows, n] tensor."""
    return (rows, (n + 31) // 32) if axis == 1 else ((rows + 31) // 32, n)


def mx_quantize(x: torch.Tensor, elem: torch.dtype = torch.float8_e4m3fn, axis: int = 1,
                stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """mx block quantization of x [rows, n] (float16 / bfloat16): returns
    (codes, scale).  elem: torch.float8_e4m3fn or torch.float8_e5m2 (codes
    [rows, n]) or torch.float4_e2m1fn_x2 (codes [rows, n/2], two per byte,
    the even element in the low nibble).  scale: float8_e8m0fnu, one per
    block of 32 along n (axis 1) or down the rows (axis 0)."""
    rows, n = x.shape
    if elem == torch.float4_e2m1fn_x2:
        y = torch.empty((rows, n // 2), dtype=torch.uint8, device=x.device).view(elem)
    else:
        y = torch.empty((rows, n), dtype=elem, device=x.device)
    scale = torch.empty(mx_scale_shape(rows, n, axis), dtype=torch.uint8,
                        device=x.device).view(torch.float8_e8m0fnu)
    ws, ex = dq_mx_quantize_get_workspace_size(x, axis, y, scale)
    s = _stream_on(stream, x.device)
    w = _workspace(ws, x.device)
    dq_mx_quantize(w, ws, ex, s)
    _release_after(w, s)
    return y, scale


def weight_quant_matmul(x1: torch.Tensor, x2: torch.Tensor, antiquant_scale: torch.Tensor,
                        antiquant_offset: Optional[torch.Tensor] = None, group_size: int = 0,
                        bias: Optional[torch.Tensor] = None, x3: Optional[torch.Tensor] = None,
                        transpose_x2: bool = True, weight: Optional[str] = None,
                        stream=None) -> torch.Tensor:
    """x1 @ dequant(x2) + bias + x3 in x1's dtype.  x2: int8 [n, k]
    (transpose_x2) or [k, n]; int4 weights as uint8 bytes [n, k/2] or
    [k, n/2] (weight='int4' or any uint8 tensor)."""
    n = x2.shape[0] if transpose_x2 else x2.shape[1] * (2 if x2.dtype == torch.uint8 else 1)
    out = torch.empty(tuple(x1.shape[:-1]) + (n,), dtype=x1.dtype, device=x1.device)
    ws, ex = dq_weight_quant_matmul_get_workspace_size(x1, x2, transpose_x2, antiquant_scale,
                                                       antiquant_offset, group_size, bias, x3, out,
                                                       weight)
    s = _stream_on(stream, x1.device)
    w = _workspace(ws, x1.device)
    dq_weight_quant_matmul(w, ws, ex, s)
    _release_after(w, s)
    return out
