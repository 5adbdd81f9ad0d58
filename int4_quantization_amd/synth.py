"""Seeded synthetic inputs shared by the tests, the smoke check and bench.py.

This module holds random draws and dtype narrowing only -- none of the
quantization arithmetic.  Every generator uses numpy's PCG64
``default_rng(seed)``, draws in the order written, produces values in
float32 and narrows them to bf16 / fp16 / fp8 with torch's
round-to-nearest-even casts (fp4 and e8m0 inputs are drawn as codes).
Tensors are returned on the CPU.

The full-size workloads are the ones the benchmark and the large parity
tests use (rows x columns):

* ``dq_sym_f16_64x256``             symmetric INT8, fp16 x, no smooth
* ``dq_sym_smooth_bf16_8192x7168``  symmetric INT8, bf16 x with 0.1 % outliers
                                    +-U(20, 60), fp32 smooth U(0.5, 2)
* ``dq_moe_asym_{int8,int4}_bf16_32768x4096``  asymmetric, 64 experts, fp32
                                    smooth [64, 4096], multinomial row counts
* ``ada_ln_quant_bf16_4x4096x3072`` AdaLayerNorm + smooth + INT8
* ``aq_{per_tensor,per_channel,per_token,per_group}_int8_16384x8192`` and
  ``aq_per_group_fp8e4m3_16384x8192``  AntiQuantize to bf16
* ``aq_per_channel_fp8e5m2_bf16param_16384x8192``  fp8-e5m2 source, bf16
                                    scale / offset (a 表3 combination)
* ``aq_per_group_fp4e2m1_e8m0_16384x8192``  the float4 case: fp4 e2m1 codes,
                                    e8m0 scales per 32 columns, no offset
* ``mx_{e4m3,e2m1}_bf16_8192x7168``  mx block quantization of an activation
                                    [M, K] (x as in the 8192x7168 DynamicQuant
                                    workload), blocks of 32 along K
* ``mx_e4m3_axis0_bf16_7168x8192``  mx block quantization of a weight [K, N],
                                    blocks of 32 down K
* ``wq_int4_g128_bf16_16x8192x28672``  weight-quantized matmul, decode-shaped:
                                    16 tokens, int4 weights [n, k] with
                                    per-group (128) scale and offset, bias
* ``wq_int8_channel_bf16_4096x8192x8192``  prefill-shaped: 4096 tokens, int8
                                    weights [n, k], per-channel scale, bias
* ``wq_int4_g128_bf16_512x8192x28672``  prefill-shaped with int4 weights and
                                    per-group (128) scale and offset, bias
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np
import torch

_TORCH = {"bfloat16": torch.bfloat16, "float16": torch.float16}


def _narrow(a: np.ndarray, dtype: str) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(_TORCH[dtype])


def dq_inputs(rows: int, n: int, seed: int, *, dtype: str = "bfloat16",
              smooth: Optional[str] = None, experts: int = 0,
              outlier_frac: float = 0.0) -> Dict[str, object]:
    """Inputs of one DynamicQuant call.

    Draw order: x ~ N(0, 1) [rows, n]; if outlier_frac > 0: positions
    (without replacement), signs (+-1 equiprobable), magnitudes U(20, 60);
    smooth ~ U(0.5, 2.0) of shape [n] ('vector') or [experts, n]
    ('experts'); then the per-expert row counts ~ multinomial(rows, uniform
    over experts), whose running sum is the int32 group index.
    """
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, n), dtype=np.float32)
    if outlier_frac > 0.0 and rows * n > 0:
        k = int(round(rows * n * outlier_frac))
        pos = rng.choice(rows * n, size=k, replace=False)
        sign = rng.integers(0, 2, size=k).astype(np.float32) * 2.0 - 1.0
        mag = rng.uniform(20.0, 60.0, size=k).astype(np.float32)
        x.reshape(-1)[pos] = sign * mag
    out: Dict[str, object] = {"x": _narrow(x, dtype), "smooth": None, "group_index": None}
    if smooth == "vector":
        out["smooth"] = torch.from_numpy(rng.uniform(0.5, 2.0, n).astype(np.float32))
    elif smooth == "experts":
        out["smooth"] = torch.from_numpy(rng.uniform(0.5, 2.0, (experts, n)).astype(np.float32))
        counts = rng.multinomial(rows, [1.0 / experts] * experts)
        out["group_index"] = torch.from_numpy(np.cumsum(counts).astype(np.int32))
    return out


def ada_inputs(B: int, S: int, H: int, seed: int, *, dtype: str = "bfloat16",
               affine: bool = True, smooth: bool = True) -> Dict[str, object]:
    """Inputs of one AdaLayerNormQuant call.

    Draw order: x ~ N(0, 1) [B, S, H]; scale, shift ~ N(0, 0.1) [B, 1, H];
    weight ~ N(1, 0.05) [H]; bias ~ N(0, 0.05) [H]; smooth ~ U(0.5, 2.0) [H]
    (fp32).  eps = 1e-5.
    """
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, S, H), dtype=np.float32)
    sc = rng.normal(0.0, 0.1, (B, 1, H)).astype(np.float32)
    sh = rng.normal(0.0, 0.1, (B, 1, H)).astype(np.float32)
    w = rng.normal(1.0, 0.05, H).astype(np.float32)
    b = rng.normal(0.0, 0.05, H).astype(np.float32)
    sm = rng.uniform(0.5, 2.0, H).astype(np.float32)
    return {
        "x": _narrow(x, dtype), "scale": _narrow(sc, dtype), "shift": _narrow(sh, dtype),
        "weight": _narrow(w, dtype) if affine else None,
        "bias": _narrow(b, dtype) if affine else None,
        "smooth": torch.from_numpy(sm) if smooth else None,
        "eps": 1e-5,
    }


def aq_param_shape(policy: str, m: int, n: int, kdim: int = 1, group_size: int = 128):
    if policy == "per_tensor":
        return (1,)
    if policy == "per_channel":
        return (1, n)
    if policy == "per_token":
        return (m, 1)
    if kdim == 1:
        return (m, -(-n // group_size))
    return (-(-m // group_size), n)


def aq_inputs(m: int, n: int, policy: str, seed: int, *, src: str = "int8", kdim: int = 1,
              group_size: int = 128, offset: bool = True,
              param_dtype: str = "float32") -> Dict[str, object]:
    """Inputs of one AntiQuantize call.

    Draw order: src, then scale, then offset.
      src 'int8': uniform over [-128, 127].
      src 'float8_e4m3fn' / 'float8_e5m2': N(0, 4) clipped to the format's
        largest finite value (448 / 57344), then rounded to nearest even.
      src 'float4_e2m1': bytes uniform over [0, 255] (two codes each),
        [m, n/2], as torch.float4_e2m1fn_x2.
    b8 sources: scale ~ U(0.001, 0.05) and offset ~ U(-8, 8) in fp32, in the
    policy's shape, then rounded to param_dtype ('float32', 'float16',
    'bfloat16').  float4: scale = e8m0 codes uniform over [117, 137]
    (2^-10 .. 2^10) as torch.float8_e8m0fnu; no offset.
    """
    rng = np.random.default_rng(seed)
    shape = aq_param_shape(policy, m, n, kdim, group_size)
    gs = group_size if policy == "per_group" else 0
    if src == "float4_e2m1":
        codes = rng.integers(0, 256, (m, n // 2)).astype(np.uint8)
        sc = rng.integers(117, 138, shape).astype(np.uint8)
        return {"src": torch.from_numpy(codes).view(torch.float4_e2m1fn_x2),
                "scale": torch.from_numpy(sc).view(torch.float8_e8m0fnu), "offset": None,
                "policy": policy, "kdim": kdim, "group_size": gs}
    if src == "int8":
        s = torch.from_numpy(rng.integers(-128, 128, (m, n)).astype(np.int8))
    else:
        fmt = getattr(torch, src)
        top = float(torch.finfo(fmt).max)
        v = np.clip(rng.normal(0.0, 4.0, (m, n)).astype(np.float32), -top, top)
        s = torch.from_numpy(v).to(fmt)
    pdt = getattr(torch, param_dtype)
    scale = torch.from_numpy(rng.uniform(0.001, 0.05, shape).astype(np.float32)).to(pdt)
    off = torch.from_numpy(rng.uniform(-8.0, 8.0, shape).astype(np.float32)).to(pdt) if offset else None
    return {"src": s, "scale": scale, "offset": off, "policy": policy, "kdim": kdim,
            "group_size": gs}


MX_ELEMS = ("float8_e4m3fn", "float8_e5m2", "float4_e2m1x2")


def mx_inputs(rows: int, n: int, seed: int, *, dtype: str = "bfloat16",
              elem: str = "float8_e4m3fn", axis: int = 1, outlier_frac: float = 0.001,
              spread: int = 0) -> Dict[str, object]:
    """Inputs of one mx block quantization call.

    Draw order: x ~ N(0, 1) [rows, n]; if outlier_frac > 0: positions
    (without replacement), signs, magnitudes U(20, 60) as in dq_inputs; if
    spread > 0: one exponent per row ~ U{-spread, .., spread} multiplying
    the row by 2^e (blocks of very different magnitudes).
    """
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, n), dtype=np.float32)
    if outlier_frac > 0.0 and rows * n > 0:
        k = int(round(rows * n * outlier_frac))
        pos = rng.choice(rows * n, size=k, replace=False)
        sign = rng.integers(0, 2, size=k).astype(np.float32) * 2.0 - 1.0
        mag = rng.uniform(20.0, 60.0, size=k).astype(np.float32)
        x.reshape(-1)[pos] = sign * mag
    if spread > 0:
        e = rng.integers(-spread, spread + 1, size=(rows, 1))
        x = x * np.exp2(e).astype(np.float32)
    return {"x": _narrow(x, dtype), "elem": elem, "axis": axis}


def _pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """Signed 4-bit codes [r, 2c] -> bytes [r, c], the even element in the low
    nibble (storage only, no arithmetic of the method)."""
    u = (codes.astype(np.int16) & 0xF).astype(np.uint8)
    return np.ascontiguousarray(u[:, 0::2] | (u[:, 1::2] << 4))


def wq_inputs(m: int, k: int, n: int, seed: int, *, dtype: str = "bfloat16", weight: str = "int8",
              group_size: int = 0, per_tensor: bool = False, offset: bool = True, bias: bool = True,
              x3: bool = False, transpose_x2: bool = True) -> Dict[str, object]:
    """Inputs of one weight-quantized matmul.

    Draw order: x1 ~ N(0, 1) [m, k]; weight codes ~ U{-128..127} (int8) or
    U{-8..7} (int4) [k, n]; scale ~ U(0.002, 0.02) and offset ~ U(-2, 2) in
    the policy's shape ([1]; [n]; or [ceil(k/gs), n]); bias ~ N(0, 1) [n];
    x3 ~ N(0, 1) [m, n].  With transpose_x2 the codes are stored [n, k] and
    per-group parameters [n, ceil(k/gs)].  int4 codes travel packed two per
    byte along the stored last dimension.
    """
    rng = np.random.default_rng(seed)
    x1 = rng.standard_normal((m, k), dtype=np.float32)
    lo, hi = (-128, 128) if weight == "int8" else (-8, 8)
    codes = rng.integers(lo, hi, (k, n)).astype(np.int8)
    if per_tensor:
        pshape = (1,)
    elif group_size == 0:
        pshape = (n,)
    else:
        pshape = (-(-k // group_size), n)
    sc = rng.uniform(0.002, 0.02, pshape).astype(np.float32)
    of = rng.uniform(-2.0, 2.0, pshape).astype(np.float32) if offset else None
    b = rng.standard_normal(n).astype(np.float32) if bias else None
    x3v = rng.standard_normal((m, n)).astype(np.float32) if x3 else None
    stored = np.ascontiguousarray(codes.T) if transpose_x2 else codes
    if weight == "int4":
        x2 = torch.from_numpy(_pack_nibbles(stored))
    else:
        x2 = torch.from_numpy(stored)
    if transpose_x2 and group_size > 0 and not per_tensor:
        sc, of = np.ascontiguousarray(sc.T), (None if of is None else np.ascontiguousarray(of.T))
    return {"x1": _narrow(x1, dtype), "x2": x2, "weight": weight, "transpose_x2": transpose_x2,
            "scale": _narrow(sc, dtype), "offset": None if of is None else _narrow(of, dtype),
            "group_size": group_size, "bias": None if b is None else _narrow(b, dtype),
            "x3": None if x3v is None else _narrow(x3v, dtype)}


# Full-size workloads: name -> (op, builder).
WORKLOADS = {
    "dq_sym_f16_64x256": (
        "dynamic_quant",
        lambda: dict(dq_inputs(64, 256, 1, dtype="float16"), symmetric=True, out="int8")),
    "dq_sym_smooth_bf16_8192x7168": (
        "dynamic_quant",
        lambda: dict(dq_inputs(8192, 7168, 2, smooth="vector", outlier_frac=0.001),
                     symmetric=True, out="int8")),
    "dq_moe_asym_int8_bf16_32768x4096": (
        "dynamic_quant",
        lambda: dict(dq_inputs(32768, 4096, 3, smooth="experts", experts=64),
                     symmetric=False, out="int8")),
    "dq_moe_asym_int4_bf16_32768x4096": (
        "dynamic_quant",
        lambda: dict(dq_inputs(32768, 4096, 3, smooth="experts", experts=64),
                     symmetric=False, out="int4")),
    "ada_ln_quant_bf16_4x4096x3072": (
        "ada_layernorm_quant", lambda: ada_inputs(4, 4096, 3072, 4)),
    "aq_per_tensor_int8_16384x8192": (
        "antiquantize", lambda: aq_inputs(16384, 8192, "per_tensor", 5)),
    "aq_per_channel_int8_16384x8192": (
        "antiquantize", lambda: aq_inputs(16384, 8192, "per_channel", 5)),
    "aq_per_token_int8_16384x8192": (
        "antiquantize", lambda: aq_inputs(16384, 8192, "per_token", 5)),
    "aq_per_group_int8_16384x8192": (
        "antiquantize", lambda: aq_inputs(16384, 8192, "per_group", 5, group_size=128)),
    "aq_per_group_fp8e4m3_16384x8192": (
        "antiquantize",
        lambda: aq_inputs(16384, 8192, "per_group", 6, src="float8_e4m3fn", group_size=128)),
    "aq_per_channel_fp8e5m2_bf16param_16384x8192": (
        "antiquantize",
        lambda: aq_inputs(16384, 8192, "per_channel", 7, src="float8_e5m2", param_dtype="bfloat16")),
    "aq_per_group_fp4e2m1_e8m0_16384x8192": (
        "antiquantize",
        lambda: aq_inputs(16384, 8192, "per_group", 8, src="float4_e2m1", group_size=32)),
    "mx_e4m3_bf16_8192x7168": (
        "mx_quantize", lambda: mx_inputs(8192, 7168, 9, elem="float8_e4m3fn")),
    "mx_e2m1_bf16_8192x7168": (
        "mx_quantize", lambda: mx_inputs(8192, 7168, 9, elem="float4_e2m1x2")),
    "mx_e4m3_axis0_bf16_7168x8192": (
        "mx_quantize", lambda: mx_inputs(7168, 8192, 10, elem="float8_e4m3fn", axis=0)),
    "wq_int4_g128_bf16_16x8192x28672": (
        "weight_quant_matmul",
        lambda: wq_inputs(16, 8192, 28672, 11, weight="int4", group_size=128)),
    "wq_int8_channel_bf16_4096x8192x8192": (
        "weight_quant_matmul",
        lambda: wq_inputs(4096, 8192, 8192, 12, weight="int8", offset=False)),
    "wq_int4_g128_bf16_512x8192x28672": (
        "weight_quant_matmul",
        lambda: wq_inputs(512, 8192, 28672, 14, weight="int4", group_size=128)),
}
