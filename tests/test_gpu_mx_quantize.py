"""mx block quantization on the GPU (through the C ABI) against the CPU
oracle, bit-exact in codes and e8m0 scale bytes.

Covered: fp8 e4m3fn / e5m2 and fp4 e2m1 codes; bf16 and fp16 inputs; blocks
along the last dimension (full blocks, a short last block, n not a multiple
of 8) and down the rows (a short last row block); several workgroups with a
ragged last one; unaligned inputs (the generic kernel); zero, NaN and
infinity blocks, subnormal-only blocks, grid ties and values above the
largest code; every 16-bit input pattern.  The full-size workloads are in
test_gpu_full_size.py."""
import numpy as np
import pytest
import torch

from int4_quantization_amd import synth
from parity import DEV, MX_TORCH, announce, check_mx_quantize

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

KINDS = list(synth.MX_ELEMS)
DTYPES = ["bfloat16", "float16"]

# (rows, n): flat rows (n % 32 == 0), ragged rows (n % 8 == 0, short last
# block), tiny rows, and n % 8 != 0 (generic kernel).  37 x 2088 has 2442
# blocks: ten workgroups, the last one partly idle.
AXIS1 = [(1, 32), (7, 256), (37, 2080), (37, 2088), (5, 40), (3, 8), (9, 100), (4, 6)]
# Axis 0: row blocks of 32 with a short last one; n % 8 != 0 takes the
# generic kernel.
AXIS0 = [(32, 64), (40, 24), (70, 1032), (33, 30), (96, 2056)]


@pytest.mark.parametrize("rows,n", AXIS1, ids=[f"{r}x{n}" for r, n in AXIS1])
@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("dtype", DTYPES)
def test_mx_axis1(orc, rows, n, kind, dtype):
    announce("mx axis1", rows, n, kind, dtype)
    q = synth.mx_inputs(rows, n, 500 + rows + n, dtype=dtype, elem=kind, spread=30)
    check_mx_quantize(orc, q["x"], kind, 1)


@pytest.mark.parametrize("rows,n", AXIS0, ids=[f"{r}x{n}" for r, n in AXIS0])
@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("dtype", DTYPES)
def test_mx_axis0(orc, rows, n, kind, dtype):
    announce("mx axis0", rows, n, kind, dtype)
    q = synth.mx_inputs(rows, n, 600 + rows + n, dtype=dtype, elem=kind, axis=0, spread=30)
    check_mx_quantize(orc, q["x"], kind, 0)


@pytest.mark.parametrize("kind", ["float8_e4m3fn", "float8_e5m2"])
@pytest.mark.parametrize("shape,axis", [((5, 33), 1), ((65, 7), 0)])
def test_mx_odd_n(orc, kind, shape, axis):
    """Odd n (fp8 only): the generic kernel, one thread per block or per
    column pair with a lone last column."""
    announce("mx odd n", shape, axis, kind)
    q = synth.mx_inputs(*shape, 700, elem=kind, axis=axis, spread=10)
    check_mx_quantize(orc, q["x"], kind, axis)


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("axis", [1, 0])
def test_mx_unaligned_input(orc, kind, axis):
    """An input starting 2 bytes into its buffer (not 16-byte aligned) runs
    the generic kernel and gives the same bytes."""
    announce("mx unaligned", kind, axis)
    rows, n = (19, 96) if axis == 1 else (70, 48)
    x = synth.mx_inputs(rows, n, 800 + axis, elem=kind, axis=axis, spread=12)["x"]
    buf = torch.empty(rows * n + 8, dtype=torch.bfloat16, device=DEV)
    xd = buf[1:1 + rows * n].view(rows, n)
    xd.copy_(x.to(DEV))
    assert xd.data_ptr() % 16 != 0
    check_mx_quantize(orc, x, kind, axis, x_dev=xd)


def _table(kind):
    if kind == "float4_e2m1x2":
        return np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    dt = torch.float8_e4m3fn if kind == "float8_e4m3fn" else torch.float8_e5m2
    v = torch.arange(128, dtype=torch.int32).to(torch.uint8).view(dt).float().numpy().astype(np.float64)
    return v[np.isfinite(v)]


def _special_rows(kind, dtype):
    """Rows of 64 (two blocks each): all zeros with signed zeros; a NaN, +inf
    or -inf beside ordinary values; subnormal-only blocks; the largest code
    times 2^k followed by ties between adjacent codes and values above the
    largest code (which saturate), at several k."""
    tdt = torch.bfloat16 if dtype == "bfloat16" else torch.float16
    rng = np.random.default_rng(900)
    rows = []
    rows.append(np.array([0.0] * 20 + [-0.0] * 44))
    for bad in (np.nan, np.inf, -np.inf):
        r = rng.standard_normal(64)
        r[37] = bad
        rows.append(r)
    if dtype == "bfloat16":
        rows.append(rng.choice([1, 2, 3, 5, 7, -1, -6], 64) * 2.0 ** -133)
        rows.append(np.concatenate([rng.standard_normal(32) * 2.0 ** -128, rng.standard_normal(32) * 2.0 ** 120]))
    else:
        rows.append(rng.choice([1, 2, 3, 5, 7, -1, -6], 64) * 2.0 ** -24)
        rows.append(np.concatenate([rng.standard_normal(32) * 2.0 ** -20, rng.standard_normal(32) * 2.0 ** 14]))
    pos = _table(kind)
    top = pos[-1]
    emax = int(np.frexp(top)[1]) - 1
    ks = (-40, -3, 0, 5) if dtype == "bfloat16" else (-8, -3, 0)
    for k in ks:
        if dtype == "float16" and (top * 2.0 ** k > 60000 or 2.0 ** (k - 16) < 2.0 ** -24):
            continue
        mids = (pos[:-1] + pos[1:]) / 2
        blk = np.concatenate([[top], rng.choice(mids, 23),
                              top + (2.0 ** (emax + 1) - top) * (0.02 + 0.9 * rng.random(8))])
        blk = blk * rng.choice([-1.0, 1.0], 32) * 2.0 ** k
        rows.append(np.concatenate([blk, blk[::-1]]))
    x = torch.from_numpy(np.stack(rows).astype(np.float32)).to(tdt)
    return x


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("axis", [1, 0])
def test_mx_special_blocks(orc, kind, dtype, axis):
    announce("mx special", kind, dtype, axis)
    x = _special_rows(kind, dtype)
    if axis == 0:
        x = x.t().contiguous()  # [64, rows]: the same blocks down the rows
        if x.shape[1] % 2 and kind == "float4_e2m1x2":
            x = torch.cat([x, x[:, :1]], dim=1)
    check_mx_quantize(orc, x, kind, axis)


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("order", ["sorted", "shuffled"])
def test_mx_every_input_pattern(orc, kind, dtype, order):
    """All 65536 16-bit patterns, in blocks of similar magnitude (sorted by
    magnitude) or at random, along rows and down columns."""
    announce("mx all patterns", kind, dtype, order)
    tdt = torch.bfloat16 if dtype == "bfloat16" else torch.float16
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    if order == "sorted":
        bits = bits[np.argsort(bits & 0x7FFF, kind="stable")]
    else:
        bits = np.random.default_rng(77).permutation(bits)
    x = torch.from_numpy(bits.view(np.int16).copy()).view(tdt).reshape(256, 256)
    check_mx_quantize(orc, x, kind, 1)
    check_mx_quantize(orc, x.t().contiguous(), kind, 0)
