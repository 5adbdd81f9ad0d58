"""Parity at shapes and parameter combinations nobody picked by hand.

Cases are drawn once, at import, from a fixed seed (so every run sees the
same ones): row counts and widths across the register-resident, vector,
generic and split-k paths, with every dtype, policy and option the entry
points accept, kept small enough for the oracle.  Each is checked against
the oracle to the same bar as the hand-picked parity tests: bit-exact for
DynamicQuant, AntiQuantize and mx quantize, the stated tolerance for
AdaLayerNorm, the binary32 bound for the matmul."""
import numpy as np
import pytest
import torch

from int4_quantization_amd import synth
from parity import (announce, check_ada_layernorm_quant, check_antiquantize, check_dynamic_quant,
                    check_mx_quantize, check_weight_quant_matmul)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

_rng = np.random.default_rng(20261203)


def _width(lo, hi, multiple=1):
    """A width in [lo, hi], log-uniform, rounded up to `multiple`."""
    v = int(np.exp(_rng.uniform(np.log(lo), np.log(hi))))
    return max(multiple, -(-v // multiple) * multiple)


def _dq_cases(count):
    out = []
    for i in range(count):
        kind = _rng.choice(["int8", "int4", "int32"])
        n = _width(1, 20000, {"int8": 1, "int4": 2, "int32": 8}[kind])
        rows = int(_rng.integers(1, 70))
        out.append((i, rows, n, str(_rng.choice(["bfloat16", "float16"])), bool(_rng.integers(2)), str(kind),
                    str(_rng.choice(["none", "vector", "experts"])), int(_rng.integers(1, 80))))
    return out


def _aq_cases(count):
    out = []
    for i in range(count):
        src = str(_rng.choice(["int8", "float8_e4m3fn", "float8_e5m2", "float4_e2m1"]))
        policy = "per_group" if src == "float4_e2m1" else str(
            _rng.choice(["per_tensor", "per_channel", "per_token", "per_group"]))
        n = _width(32, 6000, 64 if src == "float4_e2m1" else 32)
        m = int(_rng.integers(1, 300))
        kdim = 1 if src == "float4_e2m1" else int(_rng.integers(2))
        gs = 32 if src == "float4_e2m1" else int(_rng.choice([32, 64, 128, 256]))
        dst = str(_rng.choice(["bfloat16", "float16"] + ([] if src == "float4_e2m1" else ["float32"])))
        pdt = str(_rng.choice(["float32", "float16", "bfloat16"]))
        out.append((i, m, n, src, policy, kdim, gs, dst, pdt, bool(_rng.integers(2))))
    return out


def _mx_cases(count):
    out = []
    for i in range(count):
        elem = str(_rng.choice(list(synth.MX_ELEMS)))
        n = _width(1, 5000, 2 if elem == "float4_e2m1x2" else 1)
        out.append((i, int(_rng.integers(1, 200)), n, elem, int(_rng.integers(2)),
                    str(_rng.choice(["bfloat16", "float16"]))))
    return out


def _wq_cases(count):
    out = []
    for i in range(count):
        weight = str(_rng.choice(["int8", "int4"]))
        trans = bool(_rng.random() < 0.8)
        gs = int(_rng.choice([0, 0, 32, 64, 128, 256]))
        k = _width(32, 4096, 64 if weight == "int4" else 32) if _rng.random() < 0.8 else _width(2, 700, 2)
        n = _width(1, 900, 2 if (weight == "int4" and not trans) else 1)
        m = int(_rng.choice([int(_rng.integers(1, 17)), int(_rng.integers(17, 160))]))
        out.append((i, m, k, n, weight, trans, gs, bool(_rng.integers(2)), bool(_rng.integers(2)),
                    bool(_rng.integers(2)), str(_rng.choice(["bfloat16", "float16"]))))
    return out


def _ada_cases(count):
    return [(i, int(_rng.integers(1, 4)), int(_rng.integers(1, 40)), _width(8, 8192),
             str(_rng.choice(["bfloat16", "float16"])), bool(_rng.integers(2)), bool(_rng.integers(2)))
            for i in range(count)]


DQ = _dq_cases(100)
AQ = _aq_cases(100)
MX = _mx_cases(80)
WQ = _wq_cases(70)
ADA = _ada_cases(30)


def _moe_index(rows, experts, seed):
    rng = np.random.default_rng(seed)
    counts = rng.multinomial(rows, [1.0 / experts] * experts)
    return torch.from_numpy(np.cumsum(counts).astype(np.int32))


@pytest.mark.parametrize("case", DQ, ids=[f"dq{c[0]}" for c in DQ])
def test_random_dynamic_quant(orc, case):
    i, rows, n, dtype, sym, out, smooth, experts = case
    announce("random dq", case)
    seed = 1000 + i
    if smooth == "experts":
        inp = synth.dq_inputs(rows, n, seed, dtype=dtype, smooth="experts", experts=experts)
        gi = _moe_index(rows, experts, seed)
    else:
        inp = synth.dq_inputs(rows, n, seed, dtype=dtype, smooth=None if smooth == "none" else "vector",
                              outlier_frac=0.001)
        gi = None
    check_dynamic_quant(orc, inp["x"], inp["smooth"], gi, sym, out)


@pytest.mark.parametrize("case", AQ, ids=[f"aq{c[0]}" for c in AQ])
def test_random_antiquantize(orc, case):
    i, m, n, src, policy, kdim, gs, dst, pdt, offset = case
    announce("random aq", case)
    q = synth.aq_inputs(m, n, policy, 2000 + i, src=src, kdim=kdim, group_size=gs, offset=offset,
                        param_dtype=pdt)
    check_antiquantize(orc, q["src"], q["scale"], q["offset"], q["policy"], q["kdim"], q["group_size"],
                       getattr(torch, dst))


@pytest.mark.parametrize("case", MX, ids=[f"mx{c[0]}" for c in MX])
def test_random_mx_quantize(orc, case):
    i, rows, n, elem, axis, dtype = case
    announce("random mx", case)
    q = synth.mx_inputs(rows, n, 3000 + i, dtype=dtype, elem=elem, axis=axis)
    check_mx_quantize(orc, q["x"], elem, axis)


@pytest.mark.parametrize("case", WQ, ids=[f"wq{c[0]}" for c in WQ])
def test_random_weight_quant_matmul(orc, case):
    i, m, k, n, weight, trans, gs, offset, bias, x3, dtype = case
    announce("random wq", case)
    q = synth.wq_inputs(m, k, n, 4000 + i, dtype=dtype, weight=weight, group_size=gs, offset=offset, bias=bias,
                        x3=x3, transpose_x2=trans)
    check_weight_quant_matmul(orc, q)


@pytest.mark.parametrize("case", ADA, ids=[f"ada{c[0]}" for c in ADA])
def test_random_ada_layernorm_quant(orc, case):
    i, B, S, H, dtype, affine, smooth = case
    announce("random ada", case)
    inp = synth.ada_inputs(B, S, H, 5000 + i, dtype=dtype, affine=affine, smooth=smooth)
    check_ada_layernorm_quant(orc, inp)
