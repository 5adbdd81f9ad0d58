"""AntiQuantize on the GPU (through the C ABI) against the CPU oracle,
bit-exact: every policy (PER_GROUP along n and along m, with a short last
group), int8 and fp8-e4m3fn sources, bf16 / fp16 / fp32 destinations, with
and without offset, on a ragged tile grid; the page's worked example; every
fp8 code."""
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
@pytest.mark.parametrize("src", ["int8", "float8_e4m3fn"])
@pytest.mark.parametrize("dst", DSTS, ids=["bf16", "f16", "f32"])
@pytest.mark.parametrize("with_offset", [True, False], ids=["offset", "no_offset"])
def test_antiquantize_parity(orc, policy, kdim, gs, src, dst, with_offset):
    announce("antiquantize", policy, kdim, gs, src, dst, with_offset)
    q = synth.aq_inputs(37, 2080, policy, 100 + gs + kdim, src=src, kdim=kdim,
                        group_size=gs or 128, offset=with_offset)
    check_antiquantize(orc, q["src"], q["scale"], q["offset"], policy, kdim, q["group_size"], dst)


def test_antiquantize_page_example(orc):
    """scale 1, offset 0 leave dst = src (the page's own example, in fp16)."""
    announce("antiquantize page example")
    row = np.array([-4, 2, -2, -3, -1, -4, 1, 3, 4, 1, -2, 0] + [1] * 20, dtype=np.int8)
    src = torch.from_numpy(np.stack([row, -row]))
    for pol, shape in (("per_tensor", (1,)), ("per_channel", (1, 32)), ("per_token", (2, 1))):
        d = check_antiquantize(orc, src, torch.ones(shape), torch.zeros(shape), pol, 1, 0,
                               torch.float16)
        assert torch.equal(d.cpu().float(), src.float())


def test_antiquantize_all_fp8_codes(orc):
    announce("antiquantize fp8 codes")
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).reshape(8, 32).view(torch.float8_e4m3fn)
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
