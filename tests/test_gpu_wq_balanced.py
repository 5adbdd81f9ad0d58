"""The balanced decode kernel of the weight-quantized matmul on the GPU
(through the C ABI) against the CPU oracle.

It takes at most 16 rows of x1 with int4 weights stored [n, k] in groups of
128 along k, k a multiple of 8192 and n a multiple of 4096 up to 7 * 4096:
one workgroup of eight waves per compute unit, each wave an eighth of k
over the workgroup's n / 256 columns, partial sums added in LDS.  Covered:
every column count per workgroup (1 to 7 blocks of 16), m from 1 to 16,
k of one and two parameter chunks per wave, with and without offset, bf16
and fp16, bias and x3; W bit-exact through identity rows, with parameters
spread over the type's range (the one-FMA, the two-step and the
overflow-guarded dequantization paths); bit-identical repeats."""
import numpy as np
import pytest
import torch

from int4_quantization_amd import synth
from parity import DEV, announce, check_weight_quant_matmul, wq_oracle_args

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

# (m, k, n, dtype, offset, bias, x3): n / 4096 blocks of 16 columns per workgroup.
CASES = [
    (1, 8192, 4096, "bfloat16", True, True, False),
    (7, 8192, 8192, "float16", False, False, True),
    (16, 8192, 12288, "bfloat16", True, True, True),
    (4, 16384, 16384, "float16", True, False, False),
    (3, 8192, 20480, "bfloat16", False, True, False),
    (5, 8192, 24576, "bfloat16", True, False, True),
    (2, 16384, 28672, "bfloat16", True, True, False),
    (12, 8192, 28672, "float16", True, True, True),
]


@pytest.mark.parametrize("m,k,n,dtype,offset,bias,x3", CASES,
                         ids=[f"{m}x{k}x{n}-{d[:4]}-o{int(o)}b{int(b)}x{int(x)}" for m, k, n, d, o, b, x in CASES])
def test_wq_balanced_parity(orc, m, k, n, dtype, offset, bias, x3):
    announce("wq balanced", m, k, n, dtype, offset, bias, x3)
    q = synth.wq_inputs(m, k, n, 6100 + m + n // 4096 + k // 8192, dtype=dtype, weight="int4", group_size=128,
                        offset=offset, bias=bias, x3=x3)
    check_weight_quant_matmul(orc, q)


def _wide_params(q, dtype, seed):
    """Scales and offsets spread over the type's range, every weight finite
    (as in the decode kernel's weight-exposure test)."""
    g = torch.Generator().manual_seed(seed)
    shape = q["scale"].shape
    fp16 = dtype == "float16"
    e_o = torch.empty(shape).uniform_(-16.0 if fp16 else -20.0, 15.0 if fp16 else 126.0, generator=g).floor()
    if q["offset"] is None:
        e_o = torch.zeros(shape)
    e_s = torch.empty(shape).uniform_(-20.0 if fp16 else -60.0, 7.0 if fp16 else 60.0, generator=g).floor()
    e_s = (e_s - e_o.clamp(min=0.0)).clamp(-24.0 if fp16 else -126.0, 14.0 if fp16 else 120.0)
    mant = 1.0 + torch.rand(shape, generator=g)
    sgn = torch.where(torch.rand(shape, generator=g) < 0.5, -1.0, 1.0)
    q["scale"] = (sgn * mant * torch.exp2(e_s)).to(q["scale"].dtype)
    if q["offset"] is not None:
        mo = 1.0 + torch.rand(shape, generator=g)
        so = torch.where(torch.rand(shape, generator=g) < 0.5, -1.0, 1.0)
        q["offset"] = (so * mo * torch.exp2(e_o)).to(q["offset"].dtype)


@pytest.mark.parametrize("dtype", ["bfloat16", "float16"])
@pytest.mark.parametrize("offset", [True, False])
@pytest.mark.parametrize("wide", [False, True])
def test_wq_balanced_exposes_weight(orc, dtype, offset, wide):
    """Row i of x1 is the unit vector e_(16 b + i): each call returns 16 rows
    of W exactly (one wave's partial sum is the weight, the other seven add
    +0), and k / 16 calls return all of it, bit for bit against the oracle's
    dequantized W (zeros compared without their sign)."""
    announce("wq balanced exposes weight", dtype, offset, wide)
    k, n = 8192, 4096
    q = synth.wq_inputs(16, k, n, 6200 + int(offset) + 2 * int(wide), dtype=dtype, weight="int4",
                        group_size=128, offset=offset, bias=False)
    if wide:
        _wide_params(q, dtype, 6211 + int(offset))
    d = {key: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for key, v in q.items()}
    import int4_quantization_amd as dq
    x2, policy = wq_oracle_args(q)
    W = orc.weight_dequant(x2, q["scale"], q["offset"], policy, 128, True)
    eye = torch.eye(k, dtype=q["x1"].dtype, device=DEV)
    got = np.empty_like(W)
    outs = []
    for b in range(k // 16):
        outs.append(dq.weight_quant_matmul(eye[16 * b:16 * b + 16].contiguous(), d["x2"], d["scale"], d["offset"],
                                           128, None, None, True, "int4"))
    for b, out in enumerate(outs):
        got[16 * b:16 * b + 16] = out.view(torch.int16).cpu().numpy().view(np.uint16)
    zero = lambda a: np.where((a & 0x7FFF) == 0, 0, a)
    assert np.array_equal(zero(got), zero(W)), f"{int((zero(got) != zero(W)).sum())} of {W.size} weights differ"


def test_wq_balanced_deterministic():
    """Two calls give identical bits (the eight partial sums are added in
    wave order)."""
    announce("wq balanced determinism")
    q = synth.wq_inputs(16, 8192, 28672, 6300, weight="int4", group_size=128, bias=True)
    d = {key: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for key, v in q.items()}
    import int4_quantization_amd as dq
    args = (d["x1"], d["x2"], d["scale"], d["offset"], 128, d["bias"], None, True, "int4")
    a, b = dq.weight_quant_matmul(*args), dq.weight_quant_matmul(*args)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
