"""Helpers for the GPU parity tests: run a libdquant op through the C ABI
(via the binding) and the CPU oracle on the same seeded inputs, compare.

Bars:
* DynamicQuant, AntiQuantize: bit-exact -- codes / packed bytes identical,
  scale / offset / dst bits identical (two NaNs compare equal: x86 and the
  GPU produce different default-NaN payloads).
* mx block quantization: bit-exact codes and scale bytes.
* Weight-quantized matmul: every element within the binary32 summation
  bound gamma_{k+2} * (sum |x1 W| + |bias| + |x3|) plus half an ulp of the
  output type of the oracle's binary64 result, and at least 90% of the
  elements equal to that result rounded once to the output type.
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


def half_ulp(x: np.ndarray, dtype: str) -> np.ndarray:
    """Half the spacing of bf16 / fp16 values at magnitude |x| (subnormal
    spacing below the smallest normal)."""
    mbits, emin = (7, -126) if dtype == "bfloat16" else (10, -14)
    a = np.maximum(np.abs(x), 2.0 ** emin)
    e = np.floor(np.log2(a))
    return np.exp2(e - mbits - 1)


def wq_oracle_args(q):
    """The oracle's view of a wq_inputs dict (int4 bytes as a tagged pair)."""
    x2 = ("int4", q["x2"].numpy()) if q["weight"] == "int4" else q["x2"]
    if q["group_size"] > 0:
        policy = "per_group"
    elif q["scale"].numel() == 1 and q["scale"].dim() == 1:
        policy = "per_tensor"
    else:
        policy = "per_channel"
    return x2, policy


def check_weight_quant_matmul(orc, q, rows=None, dev=None):
    """GPU out against the oracle; rows: indices of x1 rows to check (all by
    default), the oracle computing only those.  dev: device inputs to use."""
    d = dev or {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in q.items()}
    out = dq.weight_quant_matmul(d["x1"], d["x2"], d["scale"], d["offset"], q["group_size"], d["bias"],
                                 d["x3"], q["transpose_x2"], q["weight"])
    torch.cuda.synchronize()
    m_all = int(np.prod(q["x1"].shape[:-1]))
    k, n = q["x1"].shape[-1], out.shape[-1]
    x1 = q["x1"].reshape(m_all, k)
    x3 = None if q["x3"] is None else q["x3"].reshape(m_all, n)
    if rows is not None:
        x1 = x1[rows].contiguous()
        x3 = None if x3 is None else x3[rows].contiguous()
    x2, policy = wq_oracle_args(q)
    ref, mag, _ = orc.weight_quant_matmul(x1, x2, q["scale"], q["offset"], policy, q["group_size"],
                                          q["transpose_x2"], q["bias"], x3)
    sel = out.reshape(m_all, n)
    if rows is not None:  # select on the device: the whole output may be many GB
        sel = sel[torch.as_tensor(np.asarray(rows), device=out.device)]
    g = sel.float().cpu().numpy().astype(np.float64)
    tname = "bfloat16" if q["x1"].dtype == torch.bfloat16 else "float16"
    gamma = (k + 2) * 2.0 ** -24 / (1 - (k + 2) * 2.0 ** -24)
    extra = np.zeros_like(ref)
    if q["bias"] is not None:
        extra += np.abs(q["bias"].double().numpy())[None, :]
    if x3 is not None:
        extra += np.abs(x3.double().numpy())
    bound = gamma * (mag + extra) + half_ulp(np.maximum(np.abs(g), np.abs(ref)), tname)
    err = np.abs(g - ref)
    assert np.all(np.isfinite(g)), "non-finite output"
    bad = err > bound
    assert not bad.any(), f"{bad.sum()} elements beyond the bound; worst err {err.max():.3g}, bound there " \
                          f"{bound.reshape(-1)[np.argmax(err)]:.3g}"
    rounded = orc.f64_to_half(ref, tname)
    gb = sel.view(torch.int16).cpu().numpy().view(np.uint16)
    frac = float(np.mean(gb == rounded)) if gb.size else 1.0
    assert frac >= 0.9, f"only {frac:.3f} of the elements equal the once-rounded exact result"
    return frac
