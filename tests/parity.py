"""Helpers for the GPU parity tests: run a libdquant op through the C ABI
(via the binding) and the CPU oracle on the same seeded inputs, compare.

Bars:
* DynamicQuant, AntiQuantize: bit-exact -- codes / packed bytes identical,
  scale / offset / dst bits identical (two NaNs compare equal: x86 and the
  GPU produce different default-NaN payloads).
* mx block quantization: bit-exact codes and scale bytes.
* AdaLayerNormQuant: |quantScale - ref| <= 1e-5 * ref, codes within +-1
  everywhere and different on at most 0.01 % of the elements (rounded up to
  a whole element for small cases).
"""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import int4_quantization_amd as dq

DEV = torch.device("cuda:0")


def announce(*parts) -> None:
    print("case:", *parts, flush=True)
    sys.stdout.flush()


def f32_bits_equal(gpu: np.ndarray, ref: np.ndarray) -> bool:
    g = np.ascontiguousarray(gpu, dtype=np.float32)
    r = np.ascontiguousarray(ref, dtype=np.float32)
    if g.shape != r.shape:
        return False
    gn, rn = np.isnan(g), np.isnan(r)
    if not np.array_equal(gn, rn):
        return False
    return np.array_equal(g[~gn].view(np.uint32), r[~rn].view(np.uint32))


def first_mismatch(a: np.ndarray, b: np.ndarray) -> str:
    idx = np.argwhere(a != b)
    if idx.size == 0:
        return "none"
    i = tuple(idx[0])
    return f"{len(idx)} mismatches, first at {i}: gpu={a[i]} ref={b[i]}"


_BYTE_VIEWS = (torch.float4_e2m1fn_x2, torch.float8_e8m0fnu)


def to_dev(t):
    """Copy to the GPU; 1-byte formats torch cannot copy travel as bytes."""
    if t is None:
        return None
    if t.dtype in _BYTE_VIEWS:
        return t.view(torch.uint8).to(DEV).view(t.dtype)
    return t.to(DEV)


def check_dynamic_quant(orc, x, smooth=None, group_index=None, symmetric=True, out="int8",
                        x_dev=None):
    """Run both and assert bit-exact parity; returns the GPU outputs."""
    xd = to_dev(x) if x_dev is None else x_dev
    y, s, o = dq.dynamic_quant(xd, to_dev(smooth), to_dev(group_index), symmetric, out)
    sm = None if smooth is None else smooth.numpy()
    gi = None if group_index is None else group_index.numpy()
    ry, rs, ro = orc.dynamic_quant(x, sm, gi, symmetric, out)
    torch.cuda.synchronize()
    gy = y.cpu().numpy()
    if out == "int32":
        gy = gy.view(np.uint32)
    assert gy.shape == ry.shape
    assert np.array_equal(gy, ry), "codes: " + first_mismatch(gy, ry)
    assert f32_bits_equal(s.cpu().numpy(), rs), "scale: " + first_mismatch(s.cpu().numpy(), rs)
    if not symmetric:
        assert f32_bits_equal(o.cpu().numpy(), ro), "offset: " + first_mismatch(o.cpu().numpy(), ro)
    return y, s, o


def aq_bits(t: torch.Tensor) -> np.ndarray:
    t = t.cpu()
    if t.dtype == torch.float32:
        return t.numpy()
    return t.view(torch.int16).numpy().view(np.uint16)


_DST_NAMES = {torch.bfloat16: "bfloat16", torch.float16: "float16", torch.float32: "float32"}


def check_antiquantize(orc, src, scale, offset=None, policy="per_tensor", k_dim=1, group_size=0,
                       dst_dtype=torch.bfloat16):
    d = dq.antiquantize(to_dev(src), to_dev(scale), to_dev(offset), policy, k_dim, group_size,
                        dst_dtype)
    ref = orc.antiquantize(src, scale, offset, policy, k_dim, group_size, _DST_NAMES[dst_dtype])
    torch.cuda.synchronize()
    g = aq_bits(d)
    if dst_dtype == torch.float32:
        assert f32_bits_equal(g, ref), "dst: " + first_mismatch(g, ref)
    else:
        gf = d.cpu().float().numpy()
        rf = torch.from_numpy(ref.view(np.int16).copy()).view(dst_dtype).float().numpy()
        gn, rn = np.isnan(gf), np.isnan(rf)
        assert np.array_equal(gn, rn), "NaN positions differ"
        assert np.array_equal(g[~gn], ref[~rn]), "dst: " + first_mismatch(g, ref)
    return d


def ada_tolerance_ok(out: np.ndarray, qs: np.ndarray, rout: np.ndarray, rqs: np.ndarray):
    qs_ok = np.all(np.abs(qs.astype(np.float64) - rqs) <= 1e-5 * np.abs(rqs.astype(np.float64)))
    diff = np.abs(out.astype(np.int32) - rout.astype(np.int32))
    allowed = max(1, math.ceil(1e-4 * diff.size))
    return bool(qs_ok), int(diff.max(initial=0)), int(np.count_nonzero(diff)), allowed


def check_ada_layernorm_quant(orc, inp, dev_override=None):
    """dev_override: device tensors to pass instead of copies of inp's (same
    values, e.g. an unaligned view)."""
    names = ("x", "scale", "shift", "weight", "bias", "smooth")
    dev = {k: to_dev(inp[k]) for k in names}
    dev.update(dev_override or {})
    out, qs = dq.ada_layernorm_quant(*[dev[k] for k in names], epsilon=inp["eps"])
    sm = None if inp["smooth"] is None else inp["smooth"].numpy()
    rout, rqs = orc.ada_layernorm_quant(inp["x"], inp["scale"], inp["shift"], inp["weight"],
                                        inp["bias"], sm, inp["eps"])
    torch.cuda.synchronize()
    qs_ok, dmax, nflip, allowed = ada_tolerance_ok(out.cpu().numpy(), qs.cpu().numpy(), rout, rqs)
    assert qs_ok, "quantScale outside 1e-5 relative"
    assert dmax <= 1, f"code difference {dmax} > 1"
    assert nflip <= allowed, f"{nflip} codes differ by 1 (allowed {allowed})"
    return out, qs, nflip


MX_TORCH = {"float8_e4m3fn": torch.float8_e4m3fn, "float8_e5m2": torch.float8_e5m2,
            "float4_e2m1x2": torch.float4_e2m1fn_x2}


def check_mx_quantize(orc, x, kind, axis=1, x_dev=None):
    """GPU codes and e8m0 scale bytes equal the oracle's, byte for byte.
    x_dev: the device input to use instead of a fresh copy of x (for
    unaligned views)."""
    xd = to_dev(x) if x_dev is None else x_dev
    y, s = dq.mx_quantize(xd, MX_TORCH[kind], axis)
    torch.cuda.synchronize()
    ry, rs = orc.mx_quantize(x, kind, axis)
    gy = y.view(torch.uint8).cpu().numpy()
    gs = s.view(torch.uint8).cpu().numpy()
    assert gs.shape == rs.shape and gy.shape == ry.shape
    assert np.array_equal(gs, rs), "scale: " + first_mismatch(gs, rs)
    assert np.array_equal(gy, ry), "codes: " + first_mismatch(gy, ry)
