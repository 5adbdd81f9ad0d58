"""CPU oracle for per-token dynamic quantization, AdaLayerNorm-quant,
AntiQuantize, mx block quantization and the weight-quantized matmul -- TEST
INFRASTRUCTURE ONLY.

Only ``tests/``, the smoke check in ``__graft_entry__`` and the CPU-baseline
leg of ``bench.py`` may import this package.  The product path (the HIP
library and its binding) never calls it, and shares no code with it.

The arithmetic lives in ``dquant_oracle.c`` (plain, single-threaded C with
one IEEE binary32 rounding per step); this module only marshals numpy / CPU
torch arrays into it through ctypes.  Each function cites, in the C file,
the passage of the pages it follows:

* ``dynamic_quant``           -- aclnnDynamicQuantV2, Formula.
* ``ada_layernorm_modulate``  -- aclnnAdaLayerNormQuant, Formula steps 1-3.
* ``ada_layernorm_quant``     -- aclnnAdaLayerNormQuant, Formula steps 1-5.
* ``antiquantize``            -- AntiQuantize, 功能说明 / 表1-表3.
* ``mx_quantize``             -- aclnnQuantBatchMatmulInplaceAdd, 计算公式
  (mx量化), read as the OCP Microscaling v1.0 conversion.
* ``weight_dequant`` / ``weight_quant_matmul`` -- aclnnWeightQuantMatmulAllReduce
  on one rank (API function, constraints).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "dquant_oracle.c")
# DQ_ORACLE_LIBRARY points at another build of the same source (the sanitizer
# test loads an AddressSanitizer / UBSan build this way).
LIBRARY = os.environ.get("DQ_ORACLE_LIBRARY") or os.path.join(HERE, "liboracle.so")

# The oracle's own type codes (see the enum in dquant_oracle.c).
F32, F16, BF16, I8, I4, I32, F8E4M3 = 0, 1, 2, 3, 4, 5, 6
F8E5M2, F4E2M1, E8M0 = 8, 9, 10
# Raw byte codes passed as (name, uint8 ndarray) pairs.
_BYTE_CODES = {"float8_e4m3fn": F8E4M3, "float8_e5m2": F8E5M2, "float4_e2m1x2": F4E2M1,
               "float8_e8m0": E8M0}
_OUT_CODES = {"int8": I8, "int4": I4, "int32": I32}
_FLOAT_CODES = {"float32": F32, "float16": F16, "bfloat16": BF16}
POLICIES = {"per_tensor": 0, "per_channel": 1, "per_token": 2, "per_group": 3}

CFLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
          "-Wall", "-Wextra"]


def build(source: str = SOURCE, output: str = LIBRARY) -> str:
    """Compile the oracle with the host C compiler (no GPU code involved)."""
    cmd = ["gcc", *CFLAGS, "-o", output, source, "-lm"]
    subprocess.run(cmd, check=True)
    return output


_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int
_dbl = ctypes.c_double


def _bind(lib: ctypes.CDLL) -> ctypes.CDLL:
    lib.oracle_dynamic_quant.argtypes = [_vp, _int, _i64, _i64, _vp, _vp, _i64, _int, _int,
                                         _vp, _vp, _vp]
    lib.oracle_dynamic_quant.restype = None
    lib.oracle_ada_layernorm_modulate.argtypes = [_vp, _int, _i64, _i64, _i64,
                                                  _vp, _int, _vp, _int, _vp, _int, _vp, _int,
                                                  _vp, _int, _dbl, _vp]
    lib.oracle_ada_layernorm_modulate.restype = None
    lib.oracle_ada_layernorm_quant.argtypes = [_vp, _int, _i64, _i64, _i64,
                                               _vp, _int, _vp, _int, _vp, _int, _vp, _int,
                                               _vp, _int, _dbl, _vp, _vp, _vp]
    lib.oracle_ada_layernorm_quant.restype = None
    lib.oracle_antiquantize.argtypes = [_vp, _int, _i64, _i64, _vp, _int, _vp, _int,
                                        _int, _int, _i64, _int, _vp]
    lib.oracle_antiquantize.restype = None
    lib.oracle_mx_quantize.argtypes = [_vp, _int, _i64, _i64, _int, _int, _vp, _vp]
    lib.oracle_mx_quantize.restype = None
    lib.oracle_weight_dequant.argtypes = [_vp, _int, _i64, _i64, _int, _vp, _vp, _int, _int,
                                          _i64, _vp]
    lib.oracle_weight_dequant.restype = None
    lib.oracle_weight_quant_matmul.argtypes = [_vp, _int, _i64, _i64, _i64, _vp, _vp, _vp, _vp,
                                               _vp]
    lib.oracle_weight_quant_matmul.restype = None
    lib.orc_convert_f64_to_half.argtypes = [_vp, _i64, _int, _vp]
    lib.orc_convert_f64_to_half.restype = None
    lib.orc_convert_to_f32.argtypes = [_vp, _int, _i64, _vp]
    lib.orc_convert_to_f32.restype = None
    lib.orc_convert_from_f32.argtypes = [_vp, _i64, _int, _vp]
    lib.orc_convert_from_f32.restype = None
    return lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _buffer(t) -> Tuple[Optional[np.ndarray], int]:
    """Contiguous host buffer and the oracle type code of an array.

    Accepts numpy arrays and CPU torch tensors; 16-bit floats travel as raw
    bit patterns, since numpy has no bfloat16.
    """
    if t is None:
        return None, F32
    if isinstance(t, tuple):
        return np.ascontiguousarray(t[1], dtype=np.uint8), _BYTE_CODES[t[0]]
    try:
        import torch
    except ImportError:  # pragma: no cover - torch is always present here
        torch = None
    if torch is not None and isinstance(t, torch.Tensor):
        t = t.detach().contiguous().cpu()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy().view(np.uint16), BF16
        if t.dtype == torch.float16:
            return t.view(torch.int16).numpy().view(np.uint16), F16
        if t.dtype == torch.float8_e4m3fn:
            return t.view(torch.uint8).numpy(), F8E4M3
        if t.dtype == torch.float8_e5m2:
            return t.view(torch.uint8).numpy(), F8E5M2
        if t.dtype == torch.float4_e2m1fn_x2:
            return t.view(torch.uint8).numpy(), F4E2M1
        if t.dtype == torch.float8_e8m0fnu:
            return t.view(torch.uint8).numpy(), E8M0
        t = t.numpy()
    a = np.ascontiguousarray(t)
    if a.dtype == np.float32:
        return a, F32
    if a.dtype == np.float16:
        return a.view(np.uint16), F16
    if a.dtype == np.int8:
        return a, I8
    if a.dtype == np.int32:
        return a, I32
    raise TypeError(f"oracle: unsupported array dtype {a.dtype}")


class Oracle:
    """ctypes front end of one compiled oracle library."""

    def __init__(self, path: str = LIBRARY):
        self.path = path
        self.lib = _bind(ctypes.CDLL(path))

    # -- element conversions (pinned against library routines in the tests) --
    def to_f32(self, t) -> np.ndarray:
        a, code = _buffer(t)
        out = np.empty(a.size, dtype=np.float32)
        self.lib.orc_convert_to_f32(_ptr(a), code, a.size, _ptr(out))
        return out.reshape(a.shape)

    def from_f32(self, a: np.ndarray, dtype: str) -> np.ndarray:
        """Round fp32 values to 'bfloat16' or 'float16'; returns raw uint16 bits."""
        a = np.ascontiguousarray(a, dtype=np.float32)
        out = np.empty(a.size, dtype=np.uint16)
        self.lib.orc_convert_from_f32(_ptr(a), a.size, _FLOAT_CODES[dtype], _ptr(out))
        return out.reshape(a.shape)

    def e4m3_to_f32(self, codes: np.ndarray) -> np.ndarray:
        return self.bytes_to_f32(codes, "float8_e4m3fn")

    def bytes_to_f32(self, codes: np.ndarray, kind: str) -> np.ndarray:
        """Decode byte codes of kind 'float8_e4m3fn', 'float8_e5m2',
        'float8_e8m0' (one value per byte) or 'float4_e2m1x2' (two values per
        byte, low nibble first: the result has twice the bytes' count)."""
        a = np.ascontiguousarray(codes, dtype=np.uint8)
        code = _BYTE_CODES[kind]
        count = a.size * (2 if code == F4E2M1 else 1)
        out = np.empty(count, dtype=np.float32)
        self.lib.orc_convert_to_f32(_ptr(a), code, count, _ptr(out))
        return out

    # -- aclnnDynamicQuantV2 --------------------------------------------------
    def dynamic_quant(self, x, smooth=None, group_index=None, symmetric=True, out="int8"):
        """Return (y, scale, offset); offset is None when symmetric.

        x: [..., N] fp16/bf16 (torch CPU tensor or float16 numpy array).
        y: int8 [..., N] for 'int8'; uint8 [..., N/2] for 'int4' (two codes
        per byte); uint32 [..., N/8] for 'int32'.
        """
        xa, xcode = _buffer(x)
        shape = xa.shape
        n = int(shape[-1])
        rows = int(np.prod(shape[:-1], dtype=np.int64)) if len(shape) > 1 else 1
        s = None if smooth is None else np.ascontiguousarray(smooth, dtype=np.float32)
        gi = None if group_index is None else np.ascontiguousarray(group_index, dtype=np.int32)
        n_exp = 0 if gi is None else gi.size
        code = _OUT_CODES[out]
        if out == "int8":
            y = np.empty(shape, dtype=np.int8)
        elif out == "int4":
            y = np.empty(shape[:-1] + (n // 2,), dtype=np.uint8)
        else:
            y = np.empty(shape[:-1] + (n // 8,), dtype=np.uint32)
        scale = np.empty(shape[:-1], dtype=np.float32)
        offset = None if symmetric else np.empty(shape[:-1], dtype=np.float32)
        self.lib.oracle_dynamic_quant(_ptr(xa), xcode, rows, n, _ptr(s), _ptr(gi), n_exp,
                                      1 if symmetric else 0, code, _ptr(y), _ptr(scale),
                                      _ptr(offset))
        return y, scale, offset

    # -- aclnnAdaLayerNormQuant -----------------------------------------------
    def _ada_args(self, x, scale, shift, weight, bias, smooth):
        xa, xc = _buffer(x)
        if xa.ndim != 3:
            raise ValueError("oracle: AdaLayerNorm x must be [B, S, H]")
        B, S, H = (int(d) for d in xa.shape)
        sc, scc = _buffer(scale)
        sh, shc = _buffer(shift)
        w, wc = _buffer(weight)
        b, bc = _buffer(bias)
        sm, smc = _buffer(smooth)
        keep = (xa, sc, sh, w, b, sm)
        args = [_ptr(xa), xc, B, S, H, _ptr(sc), scc, _ptr(sh), shc, _ptr(w), wc, _ptr(b), bc,
                _ptr(sm), smc]
        return (B, S, H), args, keep

    def ada_layernorm_modulate(self, x, scale, shift, weight=None, bias=None, smooth=None,
                               eps=1e-5) -> np.ndarray:
        (B, S, H), args, keep = self._ada_args(x, scale, shift, weight, bias, smooth)
        y = np.empty((B, S, H), dtype=np.float64)
        self.lib.oracle_ada_layernorm_modulate(*args, float(eps), _ptr(y))
        del keep
        return y

    def ada_layernorm_quant(self, x, scale, shift, weight=None, bias=None, smooth=None,
                            eps=1e-5, want_y=False):
        """Return (out int8 [B,S,H], quant_scale fp32 [B,S]) (+ y fp64 if want_y)."""
        (B, S, H), args, keep = self._ada_args(x, scale, shift, weight, bias, smooth)
        out = np.empty((B, S, H), dtype=np.int8)
        qs = np.empty((B, S), dtype=np.float32)
        y = np.empty((B, S, H), dtype=np.float64) if want_y else None
        self.lib.oracle_ada_layernorm_quant(*args, float(eps), _ptr(out), _ptr(qs), _ptr(y))
        del keep
        return (out, qs, y) if want_y else (out, qs)

    # -- AntiQuantize ---------------------------------------------------------
    def antiquantize(self, src, scale, offset=None, policy="per_tensor", kdim=1,
                     group_size=0, dst="bfloat16") -> np.ndarray:
        """Return dst [m, n]: raw uint16 bits for bf16/fp16, float32 for 'float32'.

        src: int8 [m, n] numpy/torch, torch float8_e4m3fn / float8_e5m2, or a
        (kind, uint8 codes) pair with kind 'float8_e4m3fn', 'float8_e5m2' or
        'float4_e2m1x2' (codes [m, n/2], two per byte, low nibble first).
        scale / offset: float32, float16 or bfloat16 arrays, or
        ('float8_e8m0', uint8 codes) for the float4 case.
        """
        sa, scode = _buffer(src)
        if sa.ndim != 2:
            raise ValueError("oracle: AntiQuantize src must be 2-D")
        m, n = (int(d) for d in sa.shape)
        if scode == F4E2M1:
            n *= 2
        sc, scc = _buffer(scale)
        of, ofc = _buffer(offset)
        dcode = {"bfloat16": BF16, "float16": F16, "float32": F32}[dst]
        out = np.empty((m, n), dtype=np.float32 if dcode == F32 else np.uint16)
        self.lib.oracle_antiquantize(_ptr(sa), scode, m, n, _ptr(sc), scc, _ptr(of), ofc,
                                     POLICIES[policy], int(kdim), int(group_size), dcode,
                                     _ptr(out))
        return out

    # -- mx block quantization ------------------------------------------------
    def mx_quantize(self, x, elem="float8_e4m3fn", axis=1):
        """Return (codes, scale), both uint8.

        x: [rows, n] fp16/bf16.  elem: 'float8_e4m3fn', 'float8_e5m2' or
        'float4_e2m1x2' (codes [rows, n/2], two per byte, low nibble first).
        axis 1: blocks of 32 along n, scale [rows, ceil(n/32)]; axis 0:
        blocks of 32 along rows, scale [ceil(rows/32), n].
        """
        xa, xcode = _buffer(x)
        if xa.ndim != 2:
            raise ValueError("oracle: mx quantize x must be 2-D")
        rows, n = (int(d) for d in xa.shape)
        ecode = _BYTE_CODES[elem]
        if ecode == F4E2M1 and n % 2:
            raise ValueError("oracle: float4 codes need an even last dimension")
        y = np.zeros((rows, n // 2 if ecode == F4E2M1 else n), np.uint8)
        if axis == 1:
            scale = np.empty((rows, (n + 31) // 32), np.uint8)
        else:
            scale = np.empty(((rows + 31) // 32, n), np.uint8)
        self.lib.oracle_mx_quantize(_ptr(xa), xcode, rows, n, ecode, int(axis), _ptr(y),
                                    _ptr(scale))
        return y, scale

    # -- weight-quantized matmul ------------------------------------------------
    def _weight(self, x2, transpose_x2):
        """(buffer, code, k, n) of an int8 array or an ('int4', uint8 bytes) pair."""
        if isinstance(x2, tuple):
            assert x2[0] == "int4"
            wa = np.ascontiguousarray(x2[1], dtype=np.uint8)
            r, c = wa.shape
            code, shape = I4, (r, 2 * c)
        else:
            wa, code = _buffer(x2)
            if code != I8:
                raise TypeError("oracle: weights are int8 or ('int4', bytes)")
            shape = wa.shape
        k, n = (shape[1], shape[0]) if transpose_x2 else shape
        return wa, code, int(k), int(n)

    def weight_dequant(self, x2, scale, offset=None, policy="per_channel", group_size=0,
                       transpose_x2=False) -> np.ndarray:
        """W [k, n] as raw bf16 / fp16 bits (the parameters' dtype)."""
        wa, wcode, k, n = self._weight(x2, transpose_x2)
        sc, scode = _buffer(scale)
        of, _ = _buffer(offset)
        W = np.empty((k, n), np.uint16)
        self.lib.oracle_weight_dequant(_ptr(wa), wcode, k, n, 1 if transpose_x2 else 0, _ptr(sc),
                                       _ptr(of), scode, POLICIES[policy], int(group_size), _ptr(W))
        return W

    def weight_quant_matmul(self, x1, x2, scale, offset=None, policy="per_channel", group_size=0,
                            transpose_x2=False, bias=None, x3=None):
        """Return (out, mag, W): out = x1 @ W + bias + x3 and sum |x1 * W|, both
        float64 [m, n] and unrounded; W as in weight_dequant."""
        xa, xcode = _buffer(x1)
        m, k = (int(d) for d in xa.shape)
        W = self.weight_dequant(x2, scale, offset, policy, group_size, transpose_x2)
        n = W.shape[1]
        if W.shape[0] != k:
            raise ValueError("oracle: x1 and x2 disagree on k")
        ba, _ = _buffer(bias)
        x3a, _ = _buffer(x3)
        out = np.empty((m, n), np.float64)
        mag = np.empty((m, n), np.float64)
        self.lib.oracle_weight_quant_matmul(_ptr(xa), xcode, m, k, n, _ptr(W), _ptr(ba), _ptr(x3a),
                                            _ptr(out), _ptr(mag))
        return out, mag, W

    def f64_to_half(self, a: np.ndarray, dtype: str) -> np.ndarray:
        """Round binary64 values once to 'bfloat16' or 'float16'; raw uint16 bits."""
        a = np.ascontiguousarray(a, dtype=np.float64)
        out = np.empty(a.size, np.uint16)
        self.lib.orc_convert_f64_to_half(_ptr(a), a.size, _FLOAT_CODES[dtype], _ptr(out))
        return out.reshape(a.shape)


_default: Optional[Oracle] = None


def load() -> Oracle:
    """The oracle built in-tree; compiled on first use if it is not there."""
    global _default
    if _default is None:
        if not os.path.exists(LIBRARY):
            build()
        _default = Oracle(LIBRARY)
    return _default
