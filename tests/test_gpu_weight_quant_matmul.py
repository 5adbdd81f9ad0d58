"""Weight-quantized matmul on the GPU (through the C ABI) against the CPU
oracle: every element within the binary32 summation bound of the oracle's
binary64 result, and at least 90% equal to it rounded once.

Covered: int8 and int4 weights stored [n, k] (the matrix-core kernel) and
[k, n] (the generic kernel); per-tensor, per-channel and per-group (32, 64,
128, a short last group) parameters, with and without offset; bias and x3;
bf16 and fp16; m from 1 to several tiles with ragged edges, n ragged, k not
a multiple of the 128-wide superstep; 3-D x1; the page's empty-k case;
unaligned x1; the full-size workloads on sampled rows."""
import numpy as np
import pytest
import torch

from int4_quantization_amd import synth
from parity import DEV, announce, check_weight_quant_matmul

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

SHAPES = [(1, 128, 64), (5, 160, 100), (16, 256, 48), (37, 384, 300), (200, 192, 130), (300, 640, 200)]
PARAMS = [("tensor", 0), ("channel", 0), ("group", 32), ("group", 64), ("group", 128)]


@pytest.mark.parametrize("m,k,n", SHAPES, ids=[f"{m}x{k}x{n}" for m, k, n in SHAPES])
@pytest.mark.parametrize("kind,gs", PARAMS, ids=[f"{p}{g}" for p, g in PARAMS])
@pytest.mark.parametrize("weight", ["int8", "int4"])
def test_wq_mfma(orc, m, k, n, kind, gs, weight):
    if weight == "int4" and k % 64:
        k += 32  # int4 rows are whole 64-code runs on the matrix-core path
    announce("wq mfma", m, k, n, kind, gs, weight)
    q = synth.wq_inputs(m, k, n, 1000 + m + k + n + gs, weight=weight, group_size=gs,
                        per_tensor=kind == "tensor", offset=(m + gs) % 2 == 0, bias=True, x3=m % 2 == 1)
    check_weight_quant_matmul(orc, q)


@pytest.mark.parametrize("dtype", ["bfloat16", "float16"])
@pytest.mark.parametrize("weight", ["int8", "int4"])
@pytest.mark.parametrize("kind,gs", [("tensor", 0), ("channel", 0), ("group", 64)])
@pytest.mark.parametrize("offset", [True, False])
@pytest.mark.parametrize("k", [128, 384])
def test_wq_identity_exposes_weight(orc, dtype, weight, kind, gs, offset, k):
    """x1 = identity [k, k]: each output is one exact product W[k, n] * 1 plus
    zeros, so out must equal the oracle's dequantized W bit for bit (the
    dequantization itself is exact, whatever the summation order).  k = 384
    gives more than 128 rows, the LDS-tiled kernel, where a k slot of x1
    paired with the wrong slot of W would move a weight."""
    announce("wq identity", dtype, weight, kind, gs, offset, k)
    n = 96
    q = synth.wq_inputs(k, k, n, 4000 + gs, dtype=dtype, weight=weight, group_size=gs,
                        per_tensor=kind == "tensor", offset=offset, bias=False)
    q["x1"] = torch.eye(k, dtype=q["x1"].dtype)
    d = {key: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for key, v in q.items()}
    import int4_quantization_amd as dq
    out = dq.weight_quant_matmul(d["x1"], d["x2"], d["scale"], d["offset"], gs, None, None, True, weight)
    from parity import wq_oracle_args
    x2, policy = wq_oracle_args(q)
    W = orc.weight_dequant(x2, q["scale"], q["offset"], policy, gs, True)
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, W), f"{int((got != W).sum())} of {W.size} weights differ"


@pytest.mark.parametrize("dtype", ["float16", "bfloat16"])
@pytest.mark.parametrize("offset,bias,x3", [(True, False, False), (False, True, True), (True, True, True)])
def test_wq_dtypes_and_epilogue(orc, dtype, offset, bias, x3):
    announce("wq dtype/epilogue", dtype, offset, bias, x3)
    q = synth.wq_inputs(48, 512, 96, 2000, dtype=dtype, weight="int8", group_size=128, offset=offset,
                        bias=bias, x3=x3)
    check_weight_quant_matmul(orc, q)


@pytest.mark.parametrize("weight", ["int8", "int4"])
@pytest.mark.parametrize("kind,gs", [("channel", 0), ("group", 32), ("group", 96)])
def test_wq_generic_layout(orc, weight, kind, gs):
    """Weights stored [k, n]: the generic kernel.  gs = 96 leaves a short last
    group (k = 160)."""
    announce("wq generic", weight, kind, gs)
    q = synth.wq_inputs(7, 160, 72, 3000 + gs, weight=weight, group_size=gs, offset=True, bias=True, x3=True,
                        transpose_x2=False)
    check_weight_quant_matmul(orc, q)


def test_wq_ragged_k_generic(orc):
    """k not a multiple of 32 with weights [n, k]: the generic kernel."""
    announce("wq ragged k")
    q = synth.wq_inputs(9, 100, 40, 3100, weight="int8", group_size=32, offset=True)
    check_weight_quant_matmul(orc, q)


def test_wq_three_d_x1(orc):
    announce("wq 3-D")
    q = synth.wq_inputs(2 * 24, 256, 80, 3200, weight="int4", group_size=64, x3=True)
    q["x1"] = q["x1"].reshape(2, 24, 256)
    q["x3"] = q["x3"].reshape(2, 24, 80)
    check_weight_quant_matmul(orc, q)


def test_wq_unaligned_x1(orc):
    announce("wq unaligned x1")
    q = synth.wq_inputs(6, 128, 64, 3300, weight="int8", group_size=0)
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in q.items()}
    buf = torch.empty(q["x1"].numel() + 8, dtype=q["x1"].dtype, device=DEV)
    x1 = buf[1:1 + q["x1"].numel()].view(q["x1"].shape)
    x1.copy_(d["x1"])
    assert x1.data_ptr() % 16 != 0
    d["x1"] = x1
    check_weight_quant_matmul(orc, q, dev=d)


@pytest.mark.parametrize("m,k,n,weight", [(1, 4096, 256, "int4"), (16, 8192, 192, "int4"), (24, 2048, 64, "int4"),
                                          (130, 1024, 96, "int4"), (17, 608, 72, "int8"), (260, 2048, 136, "int8")])
def test_wq_split_k(orc, m, k, n, weight):
    """Few output tiles: k is split across workgroups (binary32 partial sums
    in the workspace, added in split order by a second kernel), for the
    decode kernel and for the LDS-tiled one with one, two and three
    128-row tiles (ragged), ragged columns and k not a multiple of the
    split."""
    announce("wq split k", m, k, n, weight)
    q = synth.wq_inputs(m, k, n, 5000 + m, weight=weight, group_size=128 if weight == "int4" else 64,
                        bias=True, x3=True)
    check_weight_quant_matmul(orc, q)


@pytest.mark.parametrize("m,k,n,weight,offset,dtype", [(130, 1024, 96, "int4", True, "bfloat16"),
                                                       (300, 1024, 1100, "int4", True, "bfloat16"),
                                                       (260, 4096, 136, "int4", True, "bfloat16"),
                                                       (140, 2048, 256, "int8", False, "bfloat16"),
                                                       (150, 2048, 200, "int4", True, "float16")])
def test_wq_group128_windows(orc, m, k, n, weight, offset, dtype):
    """Groups of 128 with a multiple of 8 groups: the LDS-tiled kernel takes
    the per-group parameters in windows of 8 groups per column (k splits,
    if any, planned in whole windows); unsplit and split, ragged m and n,
    bf16 and fp16."""
    announce("wq g128 windows", m, k, n, weight, offset, dtype)
    q = synth.wq_inputs(m, k, n, 5200 + m, dtype=dtype, weight=weight, group_size=128, offset=offset, bias=True,
                        x3=m % 2 == 0)
    check_weight_quant_matmul(orc, q)


@pytest.mark.parametrize("m,k,n,weight,offset,dtype", [(16, 4096, 96, "int4", True, "float16"),
                                                       (3, 2048, 200, "int4", False, "bfloat16"),
                                                       (9, 8192, 72, "int8", True, "float16")])
def test_wq_decode_paired_groups(orc, m, k, n, weight, offset, dtype):
    """At most 16 rows with groups of 128 and a group count that is a
    multiple of the batch (4 supersteps for int4, 2 for int8): the decode
    kernel loads all parameter groups of a batch with one load.  The small
    n splits k, so each split starts on a batch boundary."""
    announce("wq decode paired groups", m, k, n, weight, offset, dtype)
    q = synth.wq_inputs(m, k, n, 5300 + m, dtype=dtype, weight=weight, group_size=128, offset=offset, bias=True,
                        x3=True)
    check_weight_quant_matmul(orc, q)


@pytest.mark.parametrize("weight", ["int8", "int4"])
@pytest.mark.parametrize("offset", [True, False])
def test_wq_identity_group128_windows(orc, weight, offset):
    """x1 = identity [1024, 1024] with groups of 128: out must be the
    oracle's dequantized W bit for bit, so a parameter taken from the wrong
    slot of a window would show."""
    announce("wq identity g128", weight, offset)
    k, n = 1024, 80
    q = synth.wq_inputs(k, k, n, 4300, weight=weight, group_size=128, offset=offset, bias=False)
    q["x1"] = torch.eye(k, dtype=q["x1"].dtype)
    d = {key: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for key, v in q.items()}
    import int4_quantization_amd as dq
    out = dq.weight_quant_matmul(d["x1"], d["x2"], d["scale"], d["offset"], 128, None, None, True, weight)
    from parity import wq_oracle_args
    x2, policy = wq_oracle_args(q)
    W = orc.weight_dequant(x2, q["scale"], q["offset"], policy, 128, True)
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, W), f"{int((got != W).sum())} of {W.size} weights differ"


@pytest.mark.parametrize("dtype", ["bfloat16", "float16"])
@pytest.mark.parametrize("weight", ["int8", "int4"])
@pytest.mark.parametrize("kind,gs", [("tensor", 0), ("channel", 0), ("group", 64), ("group", 128)])
@pytest.mark.parametrize("offset", [True, False])
@pytest.mark.parametrize("wide", [False, True])
@pytest.mark.parametrize("k", [512, 576])
def test_wq_decode_exposes_weight(orc, dtype, weight, kind, gs, offset, wide, k):
    """At most 16 rows (the decode kernel): row i of x1 is the unit vector
    e_(16 b + i), so one call returns rows 16 b .. 16 b + 15 of W exactly and
    k / 16 calls return all of it, bit for bit against the oracle's
    dequantized W.  k = 576 ends in a partial batch, whose lanes past k
    take clamped weights and parameters.  wide = True spreads the parameters over the type's
    range (bf16: offsets from 2^-20 to 2^126, where 16 o overflows
    binary32, and scales down to 2^-126; fp16: offsets from the subnormals
    to 2^15, scales down to the subnormals), on both sides of the bounds
    where the kernel takes offset and scale in one FMA, keeping every
    weight finite: a zero of x1 times an infinite weight would be NaN."""
    announce("wq decode exposes weight", dtype, weight, kind, gs, offset, wide, k)
    n = 80
    q = synth.wq_inputs(16, k, n, 4700 + gs, dtype=dtype, weight=weight, group_size=gs,
                        per_tensor=kind == "tensor", offset=offset, bias=False)
    if wide:
        g = torch.Generator().manual_seed(4711 + gs)
        shape = q["scale"].shape
        fp16 = dtype == "float16"
        # Exponents: |W| stays below 2^15 (fp16) or 2^70 (bf16) for |code| <= 128.
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
    d = {key: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for key, v in q.items()}
    import int4_quantization_amd as dq
    from parity import wq_oracle_args
    x2, policy = wq_oracle_args(q)
    W = orc.weight_dequant(x2, q["scale"], q["offset"], policy, gs, True)
    eye = torch.eye(k, dtype=q["x1"].dtype)
    got = np.empty_like(W)
    for b in range(k // 16):
        x1 = eye[16 * b:16 * b + 16].contiguous().to(DEV)
        out = dq.weight_quant_matmul(x1, d["x2"], d["scale"], d["offset"], gs, None, None, True, weight)
        got[16 * b:16 * b + 16] = out.view(torch.int16).cpu().numpy().view(np.uint16)
    # A weight of -0 (code 0 under a negative scale) sums to +0 with the
    # zero products of the other k, so zeros compare without their sign.
    zero = lambda a: np.where((a & 0x7FFF) == 0, 0, a)
    assert np.array_equal(zero(got), zero(W)), f"{int((zero(got) != zero(W)).sum())} of {W.size} weights differ"


def test_wq_split_k_deterministic():
    """Two calls give identical bits (the split sums are added in order)."""
    announce("wq split k determinism")
    q = synth.wq_inputs(16, 8192, 512, 5100, weight="int8", group_size=0, bias=True)
    d = {key: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for key, v in q.items()}
    import int4_quantization_amd as dq
    args = (d["x1"], d["x2"], d["scale"], d["offset"], 0, d["bias"], None, True, "int8")
    a, b = dq.weight_quant_matmul(*args), dq.weight_quant_matmul(*args)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_wq_empty_k(orc):
    """The page's empty case: k = 0 gives bias + x3."""
    announce("wq k=0")
    q = synth.wq_inputs(5, 0, 32, 3400, weight="int8", group_size=0, bias=True, x3=True)
    check_weight_quant_matmul(orc, q)


@pytest.mark.parametrize("weight,gs", [("int4", 128), ("int8", 0)])
def test_wq_empty_batch(orc, weight, gs):
    """m = 0 (an empty batch) on the matrix-core layout: an empty output and
    no launch."""
    announce("wq m=0", weight)
    q = synth.wq_inputs(0, 256, 64, 3500, weight=weight, group_size=gs, bias=True, x3=True)
    check_weight_quant_matmul(orc, q)


@pytest.mark.parametrize("name", ["wq_int4_g128_bf16_16x8192x28672", "wq_int8_channel_bf16_4096x8192x8192",
                                  "wq_int4_g128_bf16_512x8192x28672"])
def test_wq_full_size_sampled(orc, name):
    """The benchmark workloads: every column of a sample of rows (4 of the 16
    decode rows; 24 rows spread over the 4096-row prefill shape and 12 over
    the 512-row one, including the first and last), the oracle computing only
    those rows."""
    announce("wq full size", name)
    q = synth.WORKLOADS[name][1]()
    m = q["x1"].shape[0]
    count = 4 if m <= 16 else 12 if m <= 512 else 24
    rows = np.unique(np.linspace(0, m - 1, count).astype(int))
    frac = check_weight_quant_matmul(orc, q, rows=rows)
    print(f"{name}: {frac:.4f} of sampled outputs equal the once-rounded exact result", flush=True)


# The wide kernel (256 x 256 workgroup tiles, weights loaded straight into
# the matrix-core operands, x1 through LDS) takes at least 256 rows when its
# tiles alone give 128 workgroups, k is a multiple of 128 and groups a
# multiple of 64: ragged rows and columns, every policy, offsets, bias, x3,
# bf16 and fp16, checked on sampled rows (the first and last rows of every
# row tile among them).
WIDE = [(300, 256, 64 * 256 - 37, "int8", "channel", 0, False, "bfloat16", True),
        (257, 384, 16384, "int4", "group", 64, True, "float16", False),
        (512, 512, 16384, "int4", "group", 128, True, "bfloat16", True),
        (260, 640, 16400, "int8", "group", 128, True, "float16", True),
        (256, 256, 32768, "int4", "tensor", 0, False, "bfloat16", False),
        (256, 1024, 32768 - 5, "int8", "channel", 0, True, "bfloat16", True)]


@pytest.mark.parametrize("m,k,n,weight,kind,gs,offset,dtype,x3", WIDE,
                         ids=[f"{w[0]}x{w[1]}x{w[2]}-{w[3]}-{w[4]}{w[5]}" for w in WIDE])
def test_wq_wide_tiles(orc, m, k, n, weight, kind, gs, offset, dtype, x3):
    announce("wq wide", m, k, n, weight, kind, gs, offset, dtype, x3)
    q = synth.wq_inputs(m, k, n, 6100 + m + k, dtype=dtype, weight=weight, group_size=gs,
                        per_tensor=kind == "tensor", offset=offset, bias=True, x3=x3)
    edges = [min(r, m - 1) for t in range(0, m, 256) for r in (t, t + 1, t + 255)]
    rows = np.unique(np.r_[edges, np.linspace(0, m - 1, 12).astype(int), m - 1])
    check_weight_quant_matmul(orc, q, rows=rows)


@pytest.mark.parametrize("weight", ["int8", "int4"])
@pytest.mark.parametrize("kind,gs", [("tensor", 0), ("channel", 0), ("group", 64), ("group", 128)])
@pytest.mark.parametrize("offset", [True, False])
def test_wq_wide_identity_exposes_weight(orc, weight, kind, gs, offset):
    """x1 = identity [256, 256] against 32768 columns (128 wide tiles): out
    must be the oracle's dequantized W bit for bit, so a weight paired with
    the wrong k slot of x1, or dequantized with another step's parameters,
    would show."""
    announce("wq wide identity", weight, kind, gs, offset)
    k, n = 256, 32768
    q = synth.wq_inputs(k, k, n, 6400 + gs, weight=weight, group_size=gs, per_tensor=kind == "tensor",
                        offset=offset, bias=False)
    q["x1"] = torch.eye(k, dtype=q["x1"].dtype)
    d = {key: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for key, v in q.items()}
    import int4_quantization_amd as dq
    out = dq.weight_quant_matmul(d["x1"], d["x2"], d["scale"], d["offset"], gs, None, None, True, weight)
    from parity import wq_oracle_args
    x2, policy = wq_oracle_args(q)
    W = orc.weight_dequant(x2, q["scale"], q["offset"], policy, gs, True)
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, W), f"{int((got != W).sum())} of {W.size} weights differ"
