"""AntiQuantize on the GPU (through the C ABI) against the CPU oracle,
bit-exact: every policy (PER_GROUP along n and along m, with a short last
group), int8, fp8-e4m3fn and fp8-e5m2 sources, fp32 / fp16 / bf16
parameters, bf16 / fp16 / fp32 destinations, with and without offset, on a
ragged grid; the page's worked example; every fp8 code of both formats; the
float4 case (fp4 e2m1 source, e8m0 scales, PER_GROUP along n and along m)
on every byte value and every e8m0 code."""
import numpy as np
import pytest
import torch

from int4_quantization_amd import synth
from parity import DEV, announce, check_antiquantize

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

# m = 37 leaves a partial 16-row tile; n = 2080 leaves a partial 1024-column
# strip (32 columns); group sizes 96 (n) and 32 (m) leave short last groups.
POLICIES = [("per_tensor", 1, 0), ("per_channel", 1, 0), ("per_token", 1, 0),
            ("per_group", 1, 128), ("per_group", 1, 96), ("per_group", 0, 32)]
DSTS = [torch.bfloat16, torch.float16, torch.float32]


@pytest.mark.parametrize("policy,kdim,gs", POLICIES, ids=[f"{p}-k{k}-g{g}" for p, k, g in POLICIES])
@pytest.mark.parametrize("src", ["int8", "float8_e4m3fn", "float8_e5m2"])
@pytest.mark.parametrize("dst", DSTS, ids=["bf16", "f16", "f32"])
@pytest.mark.parametrize("with_offset", [True, False], ids=["offset", "no_offset"])
def test_antiquantize_parity(orc, policy, kdim, gs, src, dst, with_offset):
    announce("antiquantize", policy, kdim, gs, src, dst, with_offset)
    q = synth.aq_inputs(37, 2080, policy, 100 + gs + kdim, src=src, kdim=kdim,
                        group_size=gs or 128, offset=with_offset)
    check_antiquantize(orc, q["src"], q["scale"], q["offset"], policy, kdim, q["group_size"], dst)


@pytest.mark.parametrize("policy,kdim,gs", POLICIES, ids=[f"{p}-k{k}-g{g}" for p, k, g in POLICIES])
@pytest.mark.parametrize("pdt", ["float16", "bfloat16"])
@pytest.mark.parametrize("src", ["int8", "float8_e5m2"])
def test_antiquantize_half_params(orc, policy, kdim, gs, pdt, src):
    """fp16 / bf16 scale and offset (表3's half and bfloat16_t ScaleT /
    OffsetT), widened exactly, into the same dtype and into fp32."""
    announce("antiquantize half params", policy, kdim, gs, pdt, src)
    q = synth.aq_inputs(37, 2080, policy, 300 + gs + kdim, src=src, kdim=kdim,
                        group_size=gs or 128, param_dtype=pdt)
    for dst in (getattr(torch, pdt), torch.float32):
        check_antiquantize(orc, q["src"], q["scale"], q["offset"], policy, kdim, q["group_size"], dst)


# Rows of whole waves (n a multiple of 512, or of 256 for fp32 output) with
# fp32 parameters: PER_TOKEN takes scalar parameter loads; PER_GROUP along n
# on the same shapes (groups of 128 / 384, a short last group) for contrast.
SCALAR_PATH = [("per_token", 0, 2048), ("per_token", 0, 1536), ("per_group", 128, 2048),
               ("per_group", 384, 2560)]


@pytest.mark.parametrize("policy,gs,n", SCALAR_PATH, ids=[f"{p}-g{g}-n{n}" for p, g, n in SCALAR_PATH])
@pytest.mark.parametrize("dst", DSTS, ids=["bf16", "f16", "f32"])
@pytest.mark.parametrize("with_offset", [True, False], ids=["offset", "no_offset"])
def test_antiquantize_scalar_parameter_path(orc, policy, gs, n, dst, with_offset):
    announce("antiquantize scalar params", policy, gs, n, dst, with_offset)
    q = synth.aq_inputs(37, n, policy, 500 + gs + n, kdim=1, group_size=gs or 128, offset=with_offset)
    check_antiquantize(orc, q["src"], q["scale"], q["offset"], policy, 1, q["group_size"], dst)


# PER_CHANNEL in 2-D tiles (64 chunks x 32 rows per workgroup): n a multiple
# of 512 (256 for fp32 output); 37 and 100 rows leave a partial last row tile,
# 4608 columns an odd number of column tiles.
TILE_SHAPES = [(37, 2048), (100, 1536), (37, 4608)]


TILE_TYPES = [("float32", torch.bfloat16), ("float32", torch.float16), ("float32", torch.float32),
              ("bfloat16", torch.bfloat16), ("bfloat16", torch.float32)]


@pytest.mark.parametrize("m,n", TILE_SHAPES, ids=[f"{m}x{n}" for m, n in TILE_SHAPES])
@pytest.mark.parametrize("pdt,dst", TILE_TYPES, ids=["f32-bf16", "f32-f16", "f32-f32", "bf16-bf16", "bf16-f32"])
@pytest.mark.parametrize("with_offset", [True, False], ids=["offset", "no_offset"])
def test_antiquantize_per_channel_tiles(orc, m, n, pdt, dst, with_offset):
    announce("antiquantize per-channel tiles", m, n, dst, pdt, with_offset)
    q = synth.aq_inputs(m, n, "per_channel", 700 + m + n, kdim=1, offset=with_offset, param_dtype=pdt)
    check_antiquantize(orc, q["src"], q["scale"], q["offset"], "per_channel", 1, q["group_size"], dst)


FP4_CASES = [(1, 32), (1, 96), (0, 32), (0, 64)]


@pytest.mark.parametrize("kdim,gs", FP4_CASES, ids=[f"k{k}-g{g}" for k, g in FP4_CASES])
@pytest.mark.parametrize("dst", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
def test_antiquantize_float4(orc, kdim, gs, dst):
    """The float4 case on a ragged grid (37 rows: a partial block of 8 rows
    for kDim = 0; n = 2112 with groups of 96 leaves a short last group)."""
    announce("antiquantize float4", kdim, gs, dst)
    q = synth.aq_inputs(37, 2112, "per_group", 400 + gs + kdim, src="float4_e2m1", kdim=kdim,
                        group_size=gs)
    check_antiquantize(orc, q["src"], q["scale"], None, "per_group", kdim, gs, dst)


def test_antiquantize_float4_all_codes(orc):
    """Every fp4 byte in every position, against every e8m0 code (0 gives
    2^-127, 254 overflows to infinity, 255 is NaN): row r takes e8m0 code r
    for its groups of 32."""
    announce("antiquantize float4 codes")
    codes = np.tile(np.arange(256, dtype=np.uint8), (256, 1))          # [256 rows, 512 codes]
    sc = np.repeat(np.arange(256, dtype=np.uint8)[:, None], 16, axis=1)  # [256, 512 / 32]
    src = torch.from_numpy(codes).view(torch.float4_e2m1fn_x2)
    scale = torch.from_numpy(sc).view(torch.float8_e8m0fnu)
    for dst in (torch.bfloat16, torch.float16):
        check_antiquantize(orc, src, scale, None, "per_group", 1, 32, dst)
    sc0 = np.tile(np.arange(256, dtype=np.uint8), 2)[None, :].repeat(8, axis=0)  # [256 / 32, 512]
    check_antiquantize(orc, src, torch.from_numpy(np.ascontiguousarray(sc0)).view(torch.float8_e8m0fnu),
                       None, "per_group", 0, 32, torch.bfloat16)


def test_antiquantize_page_example(orc):
    """scale 1, offset 0 leave dst = src (the page's own example, in fp16)."""
    announce("antiquantize page example")
    row = np.array([-4, 2, -2, -3, -1, -4, 1, 3, 4, 1, -2, 0] + [1] * 20, dtype=np.int8)
    src = torch.from_numpy(np.stack([row, -row]))
    for pol, shape in (("per_tensor", (1,)), ("per_channel", (1, 32)), ("per_token", (2, 1))):
        d = check_antiquantize(orc, src, torch.ones(shape), torch.zeros(shape), pol, 1, 0,
                               torch.float16)
        assert torch.equal(d.cpu().float(), src.float())


@pytest.mark.parametrize("fmt", ["float8_e4m3fn", "float8_e5m2"])
def test_antiquantize_all_fp8_codes(orc, fmt):
    announce("antiquantize fp8 codes", fmt)
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).reshape(8, 32).view(getattr(torch, fmt))
    for dst in DSTS:
        check_antiquantize(orc, codes, torch.ones(1), torch.zeros(1), "per_tensor", 1, 0, dst)
        check_antiquantize(orc, codes, torch.full((1,), 0.75), None, "per_tensor", 1, 0, dst)


def test_antiquantize_empty_and_wide(orc):
    announce("antiquantize empty / wide")
    empty = torch.empty(0, 64, dtype=torch.int8)
    d = check_antiquantize(orc, empty, torch.ones(1), torch.zeros(1), "per_tensor")
    assert d.numel() == 0
    q = synth.aq_inputs(16, 32768, "per_group", 12, group_size=4096)
    check_antiquantize(orc, q["src"], q["scale"], q["offset"], "per_group", 1, 4096)


def test_antiquantize_overflow_and_tiny(orc):
    """Large scales overflow bf16/fp16 to inf; tiny ones reach subnormals."""
    announce("antiquantize overflow / tiny")
    src = torch.arange(-128, 128, dtype=torch.int32).to(torch.int8).reshape(8, 32)
    for s in (1e36, 3e-41, 1e3, 2.0 ** -20):
        for dst in DSTS:
            check_antiquantize(orc, src, torch.full((1,), s), torch.full((1,), 0.5), "per_tensor", 1,
                               0, dst)
