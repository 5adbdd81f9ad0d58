"""DynamicQuant on the GPU (through the C ABI) against the CPU oracle,
bit-exact: every kernel variant (rows of 1..16 vectors per lane, four-wave
rows, the generic path for ragged / unaligned / very long rows), symmetric
and asymmetric, INT8 / INT4 / INT32, no smooth / smooth / MoE smooth, fp16
and bf16, and the degenerate rows the formulas allow."""
import numpy as np
import pytest
import torch

from int4_quantization_amd import synth
from parity import DEV, announce, check_dynamic_quant

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

# (rows, n): widths chosen to hit each register-resident size (1, 2, 4, 8,
# 12, 14, 16 vectors per lane), the four-wave variant (8192, 32768), the team
# variant whose waves cover the row exactly (3072: 6 waves x 1 vector per
# lane, 2560: 5 x 1, 3584: 7 x 1, 5632: 11 x 1, 5120: 5 x 2, 7168: 7 x 2,
# 12288: 12 x 2, 14336: 14 x 2), and the generic variant (40000 > 32768, 250
# and 7 not multiples of 8).  Row counts leave partial row groups.
SHAPES = [(37, 64), (37, 256), (19, 1000), (29, 3072), (33, 4096), (6, 5632), (21, 7168),
          (9, 8192), (5, 12288), (3, 32768), (3, 40000), (13, 250), (7, 7), (37, 2560), (33, 3584),
          (11, 5120), (7, 14336)]


def _moe_index(rows: int, experts: int, seed: int) -> torch.Tensor:
    """Cumulative row ends with an empty expert and two rows past the end."""
    rng = np.random.default_rng(seed)
    counts = rng.multinomial(max(rows - 2, 0), [1.0 / experts] * experts)
    counts[1] = 0
    return torch.from_numpy(np.cumsum(counts).astype(np.int32))


def _cases():
    for rows, n in SHAPES:
        for sym in (True, False):
            for out in ("int8", "int4", "int32"):
                if out == "int4" and n % 2:
                    continue
                if out == "int32" and n % 8:
                    continue
                for smooth in ("none", "vector", "experts"):
                    yield rows, n, "bfloat16", sym, out, smooth
    for rows, n in [(37, 256), (21, 7168), (13, 250), (3, 40000)]:
        yield rows, n, "float16", True, "int8", "none"
        yield rows, n, "float16", False, "int4", "experts"


CASES = list(_cases())


@pytest.mark.parametrize("rows,n,dtype,sym,out,smooth", CASES,
                         ids=[f"{r}x{n}-{d[:4]}-{'sym' if s else 'asym'}-{o}-{sm}"
                              for r, n, d, s, o, sm in CASES])
def test_dynamic_quant_parity(orc, rows, n, dtype, sym, out, smooth):
    announce("dynamic_quant", rows, n, dtype, sym, out, smooth)
    seed = rows * 7919 + n
    if smooth == "experts":
        inp = synth.dq_inputs(rows, n, seed, dtype=dtype, smooth="experts", experts=5)
        inp["group_index"] = _moe_index(rows, 5, seed)
    else:
        inp = synth.dq_inputs(rows, n, seed, dtype=dtype,
                              smooth=None if smooth == "none" else "vector", outlier_frac=0.001)
    check_dynamic_quant(orc, inp["x"], inp["smooth"], inp["group_index"], sym, out)


def test_dynamic_quant_many_experts(orc):
    """More than 64 experts: the expert search walks several ballots."""
    announce("dynamic_quant many experts")
    rows, n, E = 300, 512, 70
    inp = synth.dq_inputs(rows, n, 77, smooth="experts", experts=E)
    for sym, out in ((True, "int8"), (False, "int4")):
        check_dynamic_quant(orc, inp["x"], inp["smooth"], inp["group_index"], sym, out)
    gi = _moe_index(rows, E, 78)
    check_dynamic_quant(orc, inp["x"], inp["smooth"], gi, False, "int8")


def _arbitrary_index(kind: str, rows: int, experts: int, seed: int) -> torch.Tensor:
    """group_index contents the header allows but a sorted MoE batch never
    has: the kernel must still pick the first e with row < gi[e] (the last
    expert when there is none), as the oracle's linear scan does."""
    rng = np.random.default_rng(seed)
    if kind == "unsorted":
        gi = rng.integers(-5, rows + 6, size=experts)
    elif kind == "extremes":
        gi = rng.choice([np.iinfo(np.int32).min, -1, 0, rows // 3, rows, np.iinfo(np.int32).max], size=experts)
    elif kind == "all_negative":   # no row below any end: every row to the last expert
        gi = -rng.integers(1, 1000, size=experts)
    else:                          # "all_huge": every row to expert 0
        gi = np.full(experts, np.iinfo(np.int32).max)
    return torch.from_numpy(gi.astype(np.int32))


@pytest.mark.parametrize("rows,n", [(300, 512), (37, 7168), (5, 12288), (9, 40000)])
@pytest.mark.parametrize("experts", [5, 70])
@pytest.mark.parametrize("kind", ["unsorted", "extremes", "all_negative", "all_huge"])
def test_dynamic_quant_arbitrary_group_index(orc, rows, n, experts, kind):
    announce("dynamic_quant arbitrary group_index", rows, n, experts, kind)
    seed = rows * 31 + n + experts
    inp = synth.dq_inputs(rows, n, seed, smooth="experts", experts=experts)
    gi = _arbitrary_index(kind, rows, experts, seed)
    check_dynamic_quant(orc, inp["x"], inp["smooth"], gi, experts % 2 == 1, "int8" if n % 2 else "int4")


# Inputs of at least 8192 rows without a group index take the team variant's
# long schedule (16 rows per team, two rows in flight ahead of the one being
# converted): ragged row counts, teams of 5, 6, 7 and 14 waves.
LONG_SHAPES = [(8192 + 37, 7168), (8192 + 5, 5120), (8200, 3072), (8192 + 15, 14336)]
LONG_MODES = [(True, "int8", "vector"), (False, "int4", "none"), (False, "int8", "vector"),
              (True, "int32", "none")]


@pytest.mark.parametrize("rows,n", LONG_SHAPES)
@pytest.mark.parametrize("sym,out,smooth", LONG_MODES)
def test_dynamic_quant_long_team_schedule(orc, rows, n, sym, out, smooth):
    announce("dynamic_quant long team schedule", rows, n, sym, out, smooth)
    inp = synth.dq_inputs(rows, n, rows + n, smooth=None if smooth == "none" else "vector",
                          outlier_frac=0.001)
    check_dynamic_quant(orc, inp["x"], inp["smooth"], None, sym, out)


def test_dynamic_quant_long_team_schedule_degenerate_rows(orc):
    """Rows whose divisor leaves the fast range (zero, tiny, huge, overflowing)
    spread over the long schedule's teams and steps."""
    announce("dynamic_quant long team schedule degenerate")
    rows, n = 8192 + 3, 7168
    inp = synth.dq_inputs(rows, n, 4242, smooth="vector")
    x = inp["x"].clone()
    special = _special_rows(n)
    for i, r in enumerate(range(1, rows, rows // (3 * special.shape[0]))):
        x[r] = special[i % special.shape[0]]
    x[rows - 1] = special[0]
    for sym, out in ((True, "int8"), (False, "int8"), (False, "int4")):
        check_dynamic_quant(orc, x, inp["smooth"], None, sym, out)
        check_dynamic_quant(orc, x, None, None, sym, out)


def test_dynamic_quant_long_moe_keeps_short_schedule(orc):
    """MoE inputs of many rows keep 4 consecutive rows per team (they share
    an expert's smooth row); parity across expert boundaries."""
    announce("dynamic_quant long moe")
    rows, n = 8192 + 21, 7168
    inp = synth.dq_inputs(rows, n, 99, smooth="experts", experts=7)
    check_dynamic_quant(orc, inp["x"], inp["smooth"], inp["group_index"], True, "int8")
    check_dynamic_quant(orc, inp["x"], inp["smooth"], inp["group_index"], False, "int4")


def _special_rows(n: int) -> torch.Tensor:
    rng = np.random.default_rng(5)
    rows = [
        np.zeros(n),                                   # all zero
        np.full(n, 3.0), np.full(n, -2.5),             # constant rows
        rng.standard_normal(n) * 1e-30,                # scale below 2^-60: exact-division path
        rng.standard_normal(n) * 1e25,                 # scale above 2^60
        rng.standard_normal(n) * 1e-39,                # bf16 subnormals
        np.where(np.arange(n) % 2 == 0, 3.0e38, -3.0e38),  # max - min overflows to inf
        np.full(n, 1.0) + np.arange(n) * 2 ** -7,      # all positive, narrow range
        -np.abs(rng.standard_normal(n)) - 100.0,       # all negative: offset far above 127
        np.r_[rng.standard_normal(n - 1), 0.0] * 1e-45,  # mostly zero after rounding
    ]
    return torch.from_numpy(np.stack(rows).astype(np.float32)).to(torch.bfloat16)


@pytest.mark.parametrize("n", [256, 4096, 250])
@pytest.mark.parametrize("sym,out", [(True, "int8"), (False, "int8"), (True, "int4"),
                                     (False, "int4")])
def test_dynamic_quant_degenerate_rows(orc, n, sym, out):
    announce("dynamic_quant degenerate", n, sym, out)
    x = _special_rows(n)
    check_dynamic_quant(orc, x, None, None, sym, out)
    sm = torch.full((n,), 2.0, dtype=torch.float32)
    check_dynamic_quant(orc, x, sm, None, sym, out)


def test_dynamic_quant_unaligned_input_uses_generic_path(orc):
    announce("dynamic_quant unaligned")
    inp = synth.dq_inputs(11, 4096, 9, smooth="vector")
    x = inp["x"]
    big = torch.empty(x.numel() + 1, dtype=x.dtype, device=DEV)
    xd = big[1:].view(x.shape)
    xd.copy_(x.to(DEV))
    assert xd.data_ptr() % 16 != 0
    check_dynamic_quant(orc, x, inp["smooth"], None, True, "int8", x_dev=xd)
    check_dynamic_quant(orc, x, inp["smooth"], None, False, "int4", x_dev=xd)


def test_dynamic_quant_rank3_and_empty(orc):
    announce("dynamic_quant rank3 / empty")
    inp = synth.dq_inputs(24, 512, 10)
    x3 = inp["x"].reshape(2, 12, 512)
    check_dynamic_quant(orc, x3, None, None, False, "int8")
    empty = torch.empty(0, 64, dtype=torch.bfloat16)
    y, s, _ = check_dynamic_quant(orc, empty, None, None, True, "int8")
    assert y.numel() == 0 and s.numel() == 0


def test_dynamic_quant_deterministic():
    announce("dynamic_quant determinism")
    import int4_quantization_amd as dq
    inp = synth.dq_inputs(64, 7168, 11, smooth="vector", outlier_frac=0.001)
    x, sm = inp["x"].to(DEV), inp["smooth"].to(DEV)
    a = dq.dynamic_quant(x, sm, None, False, "int8")
    b = dq.dynamic_quant(x, sm, None, False, "int8")
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u.view(torch.int8) if u.dtype != torch.float32 else u.view(torch.int32),
                           v.view(torch.int8) if v.dtype != torch.float32 else v.view(torch.int32))
