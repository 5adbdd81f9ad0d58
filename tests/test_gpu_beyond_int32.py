"""Tensors of more than 2^31 elements and 4 GiB.

Phase 1 accepts up to 2^31 - 1 rows, so every element, byte and row offset
in the kernels must be formed in 64 bits.  Each op runs once on a tensor
past both limits (inputs drawn on the device from a seeded torch
generator); the rows around the 2^31-byte, 2^31-element and 2^32-byte
crossings, and the first and last rows, are copied back and checked
against the oracle on exactly those rows (rows are independent in every
case chosen here: no MoE index, per-channel parameters, blocks along the
row or whole 32-row blocks)."""
import numpy as np
import pytest
import torch

import int4_quantization_amd as dq
from int4_quantization_amd import synth
from parity import (DEV, ada_tolerance_ok, announce, aq_bits, check_weight_quant_matmul, f32_bits_equal,
                    first_mismatch)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

E31 = 1 << 31


def _crossing_rows(rows, n, elem_bytes):
    """First/last rows and the rows on either side of each 2^31 / 2^32
    crossing of the element index and of the byte offset."""
    picks = {0, 1, rows - 2, rows - 1}
    for limit in (E31, 2 * E31):
        for per_row in (n, n * elem_bytes):
            r = limit // per_row
            picks.update({r - 1, r, r + 1})
    return np.array(sorted(p for p in picks if 0 <= p < rows))


def _gen(seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return g


@pytest.fixture(autouse=True)
def _free_between():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("sym,out", [(True, "int8"), (False, "int4")])
def test_dynamic_quant_beyond_int32(orc, sym, out):
    rows, n = 270000, 8192                        # 2.2e9 elements, 4.4 GB of bf16
    announce("dq beyond int32", rows, n, sym, out)
    x = torch.randn((rows, n), generator=_gen(71), device=DEV, dtype=torch.bfloat16)
    smooth = torch.rand(n, generator=_gen(72), device=DEV) + 0.5
    y, s, o = dq.dynamic_quant(x, smooth, None, sym, out)
    torch.cuda.synchronize()
    pick = _crossing_rows(rows, n, 2)
    idx = torch.as_tensor(pick, device=DEV)
    ry, rs, ro = orc.dynamic_quant(x[idx].cpu(), smooth.cpu().numpy(), None, sym, out)
    gy = y[idx].cpu().numpy()
    assert np.array_equal(gy, ry), "codes: " + first_mismatch(gy, ry)
    assert f32_bits_equal(s[idx].cpu().numpy(), rs)
    if not sym:
        assert f32_bits_equal(o[idx].cpu().numpy(), ro)


def test_antiquantize_beyond_int32(orc):
    m, n = 70000, 32768                           # 2.3e9 int8 elements; 4.6 GB of bf16 out
    announce("aq beyond int32", m, n)
    src = torch.randint(-128, 128, (m, n), generator=_gen(73), device=DEV, dtype=torch.int8)
    scale = torch.rand((1, n), generator=_gen(74), device=DEV) * 0.05 + 0.001
    offset = torch.rand((1, n), generator=_gen(75), device=DEV) * 16 - 8
    dst = dq.antiquantize(src, scale, offset, "per_channel", 1, 0, torch.bfloat16)
    torch.cuda.synchronize()
    pick = _crossing_rows(m, n, 2)
    idx = torch.as_tensor(pick, device=DEV)
    ref = orc.antiquantize(src[idx].cpu(), scale.cpu(), offset.cpu(), "per_channel", 1, 0, "bfloat16")
    g = aq_bits(dst[idx])
    assert np.array_equal(g, ref.view(np.uint16)), "dst: " + first_mismatch(g, ref.view(np.uint16))


@pytest.mark.parametrize("kind,axis", [("float8_e4m3fn", 1), ("float4_e2m1x2", 1), ("float8_e5m2", 0)])
def test_mx_quantize_beyond_int32(orc, kind, axis):
    rows, n = 70000, 32768                        # 2.3e9 elements, 4.6 GB of bf16
    announce("mx beyond int32", rows, n, kind, axis)
    x = torch.randn((rows, n), generator=_gen(76), device=DEV, dtype=torch.bfloat16)
    elem = {"float8_e4m3fn": torch.float8_e4m3fn, "float8_e5m2": torch.float8_e5m2,
            "float4_e2m1x2": torch.float4_e2m1fn_x2}[kind]
    y, s = dq.mx_quantize(x, elem, axis)
    torch.cuda.synchronize()
    yb, sb = y.view(torch.uint8), s.view(torch.uint8)
    if axis == 1:
        pick = _crossing_rows(rows, n, 2)
        idx = torch.as_tensor(pick, device=DEV)
        ry, rs = orc.mx_quantize(x[idx].cpu(), kind, 1)
        gy, gs = yb[idx].cpu().numpy(), sb[idx].cpu().numpy()
        assert np.array_equal(gs, rs) and np.array_equal(gy, ry)
        return
    # blocks of 32 rows: the blocks holding the crossing rows, and the ragged last one
    blocks = sorted({int(r) // 32 for r in _crossing_rows(rows, n, 2)})
    for b in blocks:
        r0, r1 = 32 * b, min(32 * b + 32, rows)
        ry, rs = orc.mx_quantize(x[r0:r1].cpu(), kind, 0)
        assert np.array_equal(sb[b:b + 1].cpu().numpy(), rs), f"scale block {b}"
        assert np.array_equal(yb[r0:r1].cpu().numpy(), ry), f"codes block {b}"


def test_ada_layernorm_quant_beyond_int32(orc):
    S, H = 270000, 8192                           # one batch of 2.2e9 elements
    announce("ada beyond int32", S, H)
    small = synth.ada_inputs(1, 1, H, 77)
    x = torch.randn((1, S, H), generator=_gen(78), device=DEV, dtype=torch.bfloat16)
    dev = {k: small[k].to(DEV) for k in ("scale", "shift", "weight", "bias", "smooth")}
    out, qs = dq.ada_layernorm_quant(x, dev["scale"], dev["shift"], dev["weight"], dev["bias"], dev["smooth"],
                                     small["eps"])
    torch.cuda.synchronize()
    pick = _crossing_rows(S, H, 2)
    idx = torch.as_tensor(pick, device=DEV)
    rout, rqs = orc.ada_layernorm_quant(x[:, idx].cpu(), small["scale"], small["shift"], small["weight"],
                                        small["bias"], small["smooth"].numpy(), small["eps"])
    qs_ok, dmax, nflip, allowed = ada_tolerance_ok(out[:, idx].cpu().numpy(), qs[:, idx].cpu().numpy(), rout, rqs)
    assert qs_ok and dmax <= 1 and nflip <= allowed, (qs_ok, dmax, nflip, allowed)


@pytest.mark.parametrize("weight,gs", [("int8", 0), ("int4", 32)])
def test_weight_quant_matmul_beyond_int32(orc, weight, gs):
    m, k, n = 33000, 64, 65535                    # out: 2.16e9 elements, 4.3 GB
    announce("wq beyond int32", m, k, n, weight, gs)
    q = synth.wq_inputs(m, k, n, 79, weight=weight, group_size=gs, bias=True)
    check_weight_quant_matmul(orc, q, rows=_crossing_rows(m, n, 2))
