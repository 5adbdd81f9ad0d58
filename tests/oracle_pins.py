"""Pins of the CPU oracle against things other than itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError
when the oracle disagrees with a value fixed by the pages, by hand-worked
arithmetic, by a closed form, by an invariant the formulas imply, or by a
library routine that a special case reduces to.  ``test_oracle_pins.py``
runs them on the real oracle; ``test_oracle_mutants.py`` runs them on copies
of the oracle with planted mistakes and expects each copy to fail one.

No expected value here is computed by the oracle itself or by the HIP
library.
"""
from __future__ import annotations

import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
f32 = np.float32


def _bf16(values):
    return torch.tensor(values, dtype=torch.float32).to(torch.bfloat16)


def _f16(values):
    return torch.tensor(values, dtype=torch.float32).to(torch.float16)


def _bits_to_bf16_f32(bits: np.ndarray) -> np.ndarray:
    return torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).float().numpy()


def _bits_to_f16_f32(bits: np.ndarray) -> np.ndarray:
    return bits.view(np.float16).astype(np.float32)


# ---------------------------------------------------------------------------
# aclnnDynamicQuantV2 -- hand-worked rows (Formula)
# ---------------------------------------------------------------------------

def pin_dq_sym_unit_scale_ties(orc):
    """Symmetric INT8, scale exactly 1: row max |x| = 127, so 127/127 = 1 and
    every quotient is x itself; round-half-to-even decides the ties
    (0.5 -> 0, 1.5 -> 2, 2.5 -> 2, -63.5 -> -64, -2.5 -> -2)."""
    for mk in (_bf16, _f16):
        x = mk([[127, -63.5, 0.5, 1.5, 2.5, -0.5, -2.5, 3.25]])
        y, s, o = orc.dynamic_quant(x)
        assert o is None
        assert s.tolist() == [1.0]
        assert y.tolist() == [[127, -64, 0, 2, 2, 0, -2, 3]]


def pin_dq_sym_true_division(orc):
    """x = [1, -2, 0.5, 4]: scale = RN(4/127) = 0x3D010204.  Dividing by that
    binary32 value gives the quotients 31.75, -63.5, 15.875, 127 exactly
    (checked by hand: 4/127 rounds down by less than half an ulp of the
    quotient), so the codes are 32, -64, 16, 127."""
    y, s, _ = orc.dynamic_quant(_f16([[1, -2, 0.5, 4]]))
    assert s.view(np.uint32).tolist() == [0x3D010204]
    assert y.tolist() == [[32, -64, 16, 127]]


def pin_dq_sym_smooth_multiplies(orc):
    """smoothScalesOptional multiplies x element-wise: x = [1, -2, 0.5, 4],
    smooth = [2, 0.5, 4, 0.25] gives input = [2, -1, 2, 1] (exact), scale =
    RN(2/127) (the pin above halved), quotients 127, -63.5, 127, 63.5 and
    codes 127, -64, 127, 64."""
    y, s, _ = orc.dynamic_quant(_bf16([[1, -2, 0.5, 4]]), smooth=np.array([2, 0.5, 4, 0.25], f32))
    assert s.view(np.uint32).tolist() == [0x3C810204]
    assert y.tolist() == [[127, -64, 127, 64]]


def pin_dq_asym_int8_rne(orc):
    """Asymmetric INT8 (scale_opt 255, offset_opt 127): x = [127.5, -127.5, 0,
    1, 2, -1, 3] has max - min = 255, so scale = 1, offset = 127 - 127.5 =
    -0.5 and the codes are round(x - 0.5) = [127, -128, -0.5->0, 0.5->0,
    1.5->2, -1.5->-2, 2.5->2].  Half-away-from-zero would give -1, 1, 3."""
    y, s, o = orc.dynamic_quant(_bf16([[127.5, -127.5, 0, 1, 2, -1, 3]]), symmetric=False)
    assert s.tolist() == [1.0] and o.tolist() == [-0.5]
    assert y.tolist() == [[127, -128, 0, 0, 2, -2, 2]]


def pin_dq_asym_int4_nibbles(orc):
    """Asymmetric INT4 (15, 7): x = [7.5, -7.5, 0, 1, 2, -1.5] -> scale 1,
    offset -0.5, codes [7, -8, 0, 0, 2, -2]; two codes per byte, the first
    in the low nibble: 0x87, 0x00, 0xE2."""
    y, s, o = orc.dynamic_quant(_bf16([[7.5, -7.5, 0, 1, 2, -1.5]]), symmetric=False, out="int4")
    assert s.tolist() == [1.0] and o.tolist() == [-0.5]
    assert y.tolist() == [[0x87, 0x00, 0xE2]]


def pin_dq_asym_int32_word(orc):
    """INT32 packs eight codes per word, code i in bits [4i, 4i+3]: codes
    [7, -8, 0, 0, 2, -2, 1, -1] give 0xF1E20087, whose little-endian bytes
    equal the INT4 bytes of the same row."""
    x = _bf16([[7.5, -7.5, 0, 1, 2, -1.5, 1.5, -0.5]])
    y32, _, _ = orc.dynamic_quant(x, symmetric=False, out="int32")
    y4, _, _ = orc.dynamic_quant(x, symmetric=False, out="int4")
    assert y32.tolist() == [[0xF1E20087]]
    assert y32.view(np.uint8).tolist() == y4.tolist() == [[0x87, 0x00, 0xE2, 0xF1]]


def pin_dq_sym_int4_divisor(orc):
    """Symmetric INT4: the divisor is 7 (the top of the INT4 code range).
    x = [7, -3.5, 1, 0.5] -> scale 1, codes [7, -4, 1, 0] -> bytes 0xC7 0x01."""
    y, s, _ = orc.dynamic_quant(_bf16([[7, -3.5, 1, 0.5]]), out="int4")
    assert s.tolist() == [1.0]
    assert y.tolist() == [[0xC7, 0x01]]


def pin_dq_degenerate_rows(orc):
    """IEEE propagation plus saturation: an all-zero row (symmetric) has
    scale 0 and 0/0 = NaN quotients, which map to code 0.  A constant row
    (asymmetric) has scale 0, offset -inf / +inf / NaN and codes 0."""
    y, s, _ = orc.dynamic_quant(_bf16([[0, 0, 0, 0]]))
    assert s.tolist() == [0.0] and y.tolist() == [[0, 0, 0, 0]]
    x = _bf16([[3, 3, 3, 3], [-2, -2, -2, -2], [0, 0, 0, 0]])
    y, s, o = orc.dynamic_quant(x, symmetric=False)
    assert s.tolist() == [0.0, 0.0, 0.0]
    assert o[0] == -np.inf and o[1] == np.inf and np.isnan(o[2])
    assert not y.any()


# ---------------------------------------------------------------------------
# aclnnDynamicQuantV2 -- invariants on random rows
# ---------------------------------------------------------------------------

def _rand_bf16(rng, shape, scale=1.0):
    return torch.from_numpy((rng.standard_normal(shape) * scale).astype(np.float32)).to(torch.bfloat16)


def pin_dq_sym_absmax_and_error(orc):
    """Symmetric INT8 on random rows: the absmax element maps to +-127 and
    every element satisfies |in - code * scale| <= scale * (1/2 + 2^-16)
    (half a step plus the binary32 roundings)."""
    rng = np.random.default_rng(11)
    x = _rand_bf16(rng, (64, 200))
    sm = rng.uniform(0.5, 2.0, 200).astype(f32)
    y, s, _ = orc.dynamic_quant(x, smooth=sm)
    v = (x.float().numpy() * sm).astype(np.float64)
    assert np.all(np.abs(y).max(axis=1) == 127)
    am = np.abs(v).argmax(axis=1)
    assert np.all(np.abs(y[np.arange(64), am]) == 127)
    err = np.abs(v - y.astype(np.float64) * s[:, None].astype(np.float64))
    assert np.all(err <= s[:, None] * (0.5 + 2.0 ** -16))


def pin_dq_asym_extremes(orc):
    """Asymmetric on random rows: row_max maps to offset_opt and row_min to
    offset_opt - scale_opt (127 / -128 for INT8, 7 / -8 for INT4), and
    |in - (code - offset) * scale| <= scale * (1/2 + 2^-14)."""
    rng = np.random.default_rng(12)
    x = _rand_bf16(rng, (64, 96), scale=3.0)
    v = x.float().numpy().astype(np.float64)
    for out, top, bot in (("int8", 127, -128), ("int4", 7, -8)):
        y, s, o = orc.dynamic_quant(x, symmetric=False, out=out)
        c = y.astype(np.int64) if out == "int8" else _unpack_int4(y)
        r = np.arange(64)
        assert np.all(c[r, v.argmax(axis=1)] == top)
        assert np.all(c[r, v.argmin(axis=1)] == bot)
        rec = (c - o[:, None].astype(np.float64)) * s[:, None].astype(np.float64)
        assert np.all(np.abs(v - rec) <= s[:, None] * (0.5 + 2.0 ** -14))


def _unpack_int4(y: np.ndarray) -> np.ndarray:
    lo = (y & 0xF).astype(np.int64)
    hi = (y >> 4).astype(np.int64)
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(y.shape[:-1] + (2 * y.shape[-1],), dtype=np.int64)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def pin_dq_power_of_two_scaling(orc):
    """Multiplying x (or the smooth scales) by 2^k leaves every code and the
    offset unchanged and multiplies scale by exactly 2^k (no rounding is
    introduced by a power of two away from under/overflow)."""
    rng = np.random.default_rng(13)
    x = _rand_bf16(rng, (16, 64))
    sm = rng.uniform(0.5, 2.0, 64).astype(f32)
    for sym in (True, False):
        for out in ("int8", "int4"):
            y0, s0, o0 = orc.dynamic_quant(x, smooth=sm, symmetric=sym, out=out)
            y1, s1, o1 = orc.dynamic_quant((x.float() * 8).to(torch.bfloat16), smooth=sm,
                                           symmetric=sym, out=out)
            y2, s2, o2 = orc.dynamic_quant(x, smooth=sm / 4, symmetric=sym, out=out)
            assert np.array_equal(y0, y1) and np.array_equal(y0, y2)
            assert np.array_equal(s1, s0 * 8) and np.array_equal(s2, s0 / 4)
            if not sym:
                assert np.array_equal(o0, o1) and np.array_equal(o0, o2)


def pin_dq_smooth_one_and_permutation(orc):
    """smooth = 1 is the same as no smooth; permuting the columns of x and
    of smooth together permutes the codes and keeps scale and offset."""
    rng = np.random.default_rng(14)
    x = _rand_bf16(rng, (8, 48))
    sm = rng.uniform(0.5, 2.0, 48).astype(f32)
    perm = rng.permutation(48)
    for sym in (True, False):
        a = orc.dynamic_quant(x, symmetric=sym)
        b = orc.dynamic_quant(x, smooth=np.ones(48, f32), symmetric=sym)
        assert all(np.array_equal(u, w) for u, w in zip(a, b) if u is not None)
        c = orc.dynamic_quant(x, smooth=sm, symmetric=sym)
        d = orc.dynamic_quant(x[:, perm].contiguous(), smooth=sm[perm], symmetric=sym)
        assert np.array_equal(c[0][:, perm], d[0])
        assert np.array_equal(c[1], d[1])
        if not sym:
            assert np.array_equal(c[2], d[2])


def pin_dq_moe_reductions(orc):
    """MoE: groupIndex holds cumulative per-expert row ends.  Every row must
    equal the non-MoE result of that row with its own expert's smooth row,
    with expert e owning rows [gi[e-1], gi[e]), empty experts skipped and
    rows past gi[E-1] taken by the last expert; E = 1 with gi = [R] equals
    the non-MoE smooth call."""
    rng = np.random.default_rng(15)
    R, N = 12, 32
    x = _rand_bf16(rng, (R, N))
    sm = rng.uniform(0.5, 2.0, (4, N)).astype(f32)
    gi = np.array([3, 3, 7, 10], np.int32)  # expert 1 is empty; rows 10, 11 past the end
    owner = [0, 0, 0, 2, 2, 2, 2, 3, 3, 3, 3, 3]
    for sym in (True, False):
        for out in ("int8", "int4"):
            y, s, o = orc.dynamic_quant(x, smooth=sm, group_index=gi, symmetric=sym, out=out)
            for r in range(R):
                yr, sr, orr = orc.dynamic_quant(x[r:r + 1], smooth=sm[owner[r]],
                                                symmetric=sym, out=out)
                assert np.array_equal(y[r:r + 1], yr) and s[r] == sr[0]
                if not sym:
                    assert o[r] == orr[0]
            one = orc.dynamic_quant(x, smooth=sm[2:3], group_index=np.array([R], np.int32),
                                    symmetric=sym, out=out)
            ref = orc.dynamic_quant(x, smooth=sm[2], symmetric=sym, out=out)
            assert all(np.array_equal(u, w) for u, w in zip(one, ref) if u is not None)


def pin_dq_leading_dims(orc):
    """x of rank 3 is quantized per row of its last dimension: the result
    equals the rank-2 call on the flattened rows."""
    rng = np.random.default_rng(16)
    x = _rand_bf16(rng, (3, 5, 16))
    a = orc.dynamic_quant(x, symmetric=False)
    b = orc.dynamic_quant(x.reshape(15, 16), symmetric=False)
    assert np.array_equal(a[0].reshape(15, 16), b[0])
    assert np.array_equal(a[1].reshape(15), b[1]) and np.array_equal(a[2].reshape(15), b[2])



# ---------------------------------------------------------------------------
# aclnnDynamicQuantV2 -- the whole formula against numpy float32 (Formula)
#
# numpy evaluates every step as one IEEE binary32 operation (np.float32
# `*`, `/`, `+`, `-` round to nearest even) and np.rint rounds half to
# even, so it is an independent, vectorized statement of the Formula.  The
# rows are built so that division and reciprocal multiplication disagree:
# x is +-1 and the smooth scales carry arbitrary binary32 magnitudes, placed
# within a few ulps of the points where a quotient crosses k + 1/2.  Each
# pin first checks, in numpy, that its inputs tell RN(v / scale) apart from
# RN(v * RN(1 / scale)), and only then compares the oracle.
# ---------------------------------------------------------------------------

_DQ_CONST = {"int8": (255.0, 127.0, -128, 127), "int4": (15.0, 7.0, -8, 7)}


def _ulp_walk(center: np.ndarray, steps) -> np.ndarray:
    """Positive binary32 values `d` ulps from each center, for d in steps."""
    bits = np.abs(center.astype(f32)).view(np.int32).astype(np.int64)
    out = [(bits + d).astype(np.int32).view(f32) for d in steps]
    return np.concatenate(out)


def _np_dq(x, smooth, owner, symmetric, out, recip=False):
    """numpy float32 statement of the Formula for rows x (torch bf16/fp16),
    smooth rows `smooth[owner[r]]` (or none).  `recip` swaps every division
    by the row scale for a multiplication by RN(1 / scale) -- used only to
    show that an input discriminates."""
    opt_s, opt_o, lo, hi = (f32(v) for v in _DQ_CONST[out])
    with np.errstate(all="ignore"):
        v = x.float().numpy().astype(f32)
        if smooth is not None:
            v = (v * smooth[owner]).astype(f32)
        div = (lambda a, b: a * (f32(1) / b)) if recip else (lambda a, b: a / b)
        if symmetric:
            sc = np.abs(v).max(axis=1) / opt_o
            t = div(v, sc[:, None])
            off = None
        else:
            vmax, vmin = v.max(axis=1), v.min(axis=1)
            sc = (vmax - vmin) / opt_s
            off = opt_o - div(vmax, sc)
            t = div(v, sc[:, None]) + off[:, None]
        t = np.where(np.isnan(t), f32(0), t)
        c = np.clip(np.rint(t), lo, hi).astype(np.int64)
    return c, sc.astype(f32), None if off is None else off.astype(f32)


def _codes_of(y, out):
    return y.astype(np.int64) if out == "int8" else _unpack_int4(y)


def _sym_row_magnitudes(rng, n, out):
    """|v| of one symmetric row: an absmax A and values around (k + 1/2) *
    RN(A / D) for every code step k."""
    _, D, _, top = _DQ_CONST[out]
    A = f32(rng.uniform(1.0, 2.0) * 2.0 ** rng.integers(-20, 20))
    sc = A / f32(D)
    k = np.arange(top, dtype=np.float64)
    near = _ulp_walk((k + 0.5) * np.float64(sc), range(-3, 4))
    near = near[near < A]
    row = np.concatenate([[A], near, rng.uniform(0, 1, n).astype(f32) * A])[:n]
    return rng.permutation(row).astype(f32)


def _asym_row_magnitudes(rng, n, out):
    """Signed v of one asymmetric row: max hi, min lo and values around
    the points where RN(v / scale) + offset crosses k + 1/2."""
    opt_s, opt_o, lo_c, hi_c = _DQ_CONST[out]
    hi = f32(rng.uniform(1.0, 2.0) * 2.0 ** rng.integers(-12, 12))
    lo = f32(-hi * rng.uniform(0.3, 3.0))
    sc = (hi - lo) / f32(opt_s)
    off = f32(opt_o) - hi / sc
    k = np.arange(lo_c, hi_c, dtype=np.float64)
    centers = (k + 0.5 - np.float64(off)) * np.float64(sc)
    near = np.concatenate([np.sign(c) * _ulp_walk(np.array([c]), range(-3, 4)) for c in centers])
    near = near[(near > lo) & (near < hi)].astype(f32)
    row = np.concatenate([[hi, lo], near, rng.uniform(lo, hi, n).astype(f32)])[:n]
    return rng.permutation(row).astype(f32)


def _signed_inputs(v: np.ndarray):
    """x = sign(v) as bf16 and smooth = |v| (x * smooth = v exactly)."""
    x = torch.from_numpy(np.where(v < 0, -1.0, 1.0).astype(np.float32)).to(torch.bfloat16)
    return x, np.abs(v).astype(f32)


def pin_dq_matches_numpy_float32(orc):
    """Symmetric and asymmetric, INT8 and INT4, with a smooth vector: codes,
    scale and offset equal numpy's binary32 evaluation bit for bit, on rows
    where true division and reciprocal multiplication disagree."""
    rng = np.random.default_rng(17)
    R, N = 24, 1024
    for out in ("int8", "int4"):
        for sym in (True, False):
            build = _sym_row_magnitudes if sym else _asym_row_magnitudes
            v = np.stack([build(rng, N, out) for _ in range(R)])
            if sym:
                v = v * np.where(rng.random(v.shape) < 0.5, f32(-1), f32(1))
            # Each row has its own smooth row: R experts, one row each.
            x, sm = _signed_inputs(v)
            gi = np.arange(1, R + 1, dtype=np.int32)
            owner = np.arange(R)
            want = _np_dq(x, sm, owner, sym, out)
            alt = _np_dq(x, sm, owner, sym, out, recip=True)
            assert not np.array_equal(want[0], alt[0]), "inputs must tell division from reciprocal"
            y, s, o = orc.dynamic_quant(x, smooth=sm, group_index=gi, symmetric=sym, out=out)
            assert np.array_equal(_codes_of(y, out), want[0]), (out, sym)
            assert np.array_equal(s.view(np.uint32), want[1].view(np.uint32)), (out, sym)
            if not sym:
                assert np.array_equal(o.view(np.uint32), want[2].view(np.uint32)), (out, sym)


def pin_dq_scale_is_true_quotient(orc):
    """scale = RN(row_max|in| / 127) and RN(RN(max - min) / 255) (7 and 15
    for INT4) are true binary32 quotients: on rows where the quotient and
    the reciprocal product RN(a * RN(1 / D)) differ, the oracle's scale
    equals the quotient."""
    rng = np.random.default_rng(18)
    K = 64
    gi = np.arange(1, K + 1, dtype=np.int32)
    for out in ("int8", "int4"):
        opt_s, opt_o, _, _ = _DQ_CONST[out]
        A = (rng.uniform(1.0, 2.0, 200000) * 2.0 ** rng.integers(-30, 30, 200000)).astype(f32)
        A = A[(A / f32(opt_o)) != A * (f32(1) / f32(opt_o))][:K]
        assert A.size == K
        row = np.repeat(A[:, None] * f32(0.25), 8, axis=1)
        row[:, 0] = A
        x, sm = _signed_inputs(row)
        _, s, _ = orc.dynamic_quant(x, smooth=sm, group_index=gi, out=out)
        assert np.array_equal(s.view(np.uint32), (A / f32(opt_o)).view(np.uint32)), out
        # Asymmetric: max hi and min lo, with RN(hi - lo) / scale_opt discriminating.
        hi = (rng.uniform(1.0, 2.0, 200000) * 2.0 ** rng.integers(-30, 30, 200000)).astype(f32)
        lo = (-hi * rng.uniform(0.1, 2.0, 200000)).astype(f32)
        rg = (hi - lo).astype(f32)
        keep = (rg / f32(opt_s)) != rg * (f32(1) / f32(opt_s))
        hi, lo, rg = hi[keep][:K], lo[keep][:K], rg[keep][:K]
        assert hi.size == K
        row = np.repeat(((hi + lo) * f32(0.5))[:, None], 8, axis=1).astype(f32)
        row[:, 0], row[:, 1] = hi, lo
        x, sm = _signed_inputs(row)
        _, s, o = orc.dynamic_quant(x, smooth=sm, group_index=gi, symmetric=False, out=out)
        assert np.array_equal(s.view(np.uint32), (rg / f32(opt_s)).view(np.uint32)), out
        want = _np_dq(x, sm, np.arange(K), False, out)
        assert np.array_equal(o.view(np.uint32), want[2].view(np.uint32)), out


def pin_dq_natural_rows_match_numpy(orc):
    """Random bf16 and fp16 rows with 0.1 % outliers, without smooth, with a
    smooth vector and with MoE expert rows (an empty expert, rows past the
    last bound): every output equals numpy's binary32 evaluation, with the
    owner of row r taken as numpy's searchsorted over the row ends."""
    rng = np.random.default_rng(19)
    R, N, E = 40, 320, 6
    for dtype in (torch.bfloat16, torch.float16):
        xf = rng.standard_normal((R, N)).astype(f32)
        pos = rng.choice(R * N, 13, replace=False)
        xf.reshape(-1)[pos] = rng.uniform(20, 60, 13).astype(f32) * np.where(rng.random(13) < 0.5, -1, 1)
        x = torch.from_numpy(xf).to(dtype)
        sm_e = rng.uniform(0.5, 2.0, (E, N)).astype(f32)
        gi = np.array([5, 5, 12, 20, 31, 36], np.int32)  # expert 1 empty; rows 36..39 past the end
        owner = np.minimum(np.searchsorted(gi, np.arange(R), side="right"), E - 1)
        for out in ("int8", "int4"):
            for sym in (True, False):
                for smooth, g, own in ((None, None, None), (sm_e[3], None, np.zeros(R, np.int64)),
                                       (sm_e, gi, owner)):
                    sm_rows = None if smooth is None else (smooth if smooth.ndim == 2 else smooth[None])
                    want = _np_dq(x, sm_rows, own, sym, out)
                    y, s, o = orc.dynamic_quant(x, smooth=smooth, group_index=g, symmetric=sym, out=out)
                    assert np.array_equal(_codes_of(y, out), want[0]), (dtype, out, sym)
                    assert np.array_equal(s.view(np.uint32), want[1].view(np.uint32))
                    if not sym:
                        assert np.array_equal(o.view(np.uint32), want[2].view(np.uint32))

# ---------------------------------------------------------------------------
# aclnnAdaLayerNormQuant
# ---------------------------------------------------------------------------

def _ada_params(rng, B, H, dtype=torch.bfloat16):
    mk = lambda a: torch.from_numpy(a.astype(np.float32)).to(dtype)
    return (mk(rng.normal(0, 0.1, (B, 1, H))), mk(rng.normal(0, 0.1, (B, 1, H))),
            mk(rng.normal(1, 0.05, H)), mk(rng.normal(0, 0.05, H)))


def pin_ada_layernorm_matches_torch(orc):
    """With scale = shift = 0 and no smooth, y is LayerNorm(x) with weight and
    bias, which torch.nn.functional.layer_norm computes in float64
    (biased variance) to 1e-12."""
    rng = np.random.default_rng(21)
    B, S, H = 2, 3, 64
    x = _rand_bf16(rng, (B, S, H))
    _, _, w, b = _ada_params(rng, B, H)
    zero = torch.zeros(B, 1, H, dtype=torch.bfloat16)
    for eps in (1e-5, 0.5):
        y = orc.ada_layernorm_modulate(x, zero, zero, w, b, None, eps)
        ref = torch.nn.functional.layer_norm(x.double(), (H,), w.double(), b.double(), eps)
        assert np.allclose(y, ref.numpy(), rtol=0, atol=1e-12)
        y0 = orc.ada_layernorm_modulate(x, zero, zero, None, None, None, eps)
        ref0 = torch.nn.functional.layer_norm(x.double(), (H,), None, None, eps)
        assert np.allclose(y0, ref0.numpy(), rtol=0, atol=1e-12)


def pin_ada_modulation_special_cases(orc):
    """y = LN(x) * (1 + scale) + shift, then * smooth, with scale and shift
    taken from the row's batch.  scale = 1 doubles LN; scale = -1 leaves
    exactly shift * smooth; scale = 2^k - 1 per column (or per batch)
    multiplies LN by 2^k; shift enters additively."""
    rng = np.random.default_rng(22)
    B, S, H = 2, 2, 32
    x = _rand_bf16(rng, (B, S, H))
    sc, sh, w, b = _ada_params(rng, B, H)
    sm = rng.uniform(0.5, 2.0, H).astype(f32)
    zero = torch.zeros(B, 1, H, dtype=torch.bfloat16)
    ln = orc.ada_layernorm_modulate(x, zero, zero, w, b, None)
    one = torch.ones(B, 1, H, dtype=torch.bfloat16)
    assert np.array_equal(orc.ada_layernorm_modulate(x, one, zero, w, b, None), 2 * ln)
    y = orc.ada_layernorm_modulate(x, -one, sh, w, b, sm)
    exact = sh.double().numpy() * sm.astype(np.float64)
    assert np.array_equal(y, np.broadcast_to(exact, y.shape))
    k = rng.integers(-2, 3, H)
    pw = torch.from_numpy((2.0 ** k - 1).astype(np.float32)).to(torch.bfloat16).expand(B, 1, H)
    y = orc.ada_layernorm_modulate(x, pw.contiguous(), zero, w, b, None)
    assert np.allclose(y, ln * 2.0 ** k, rtol=1e-15, atol=0)
    per_batch = torch.tensor([0.0, 3.0], dtype=torch.bfloat16).reshape(B, 1, 1).expand(B, 1, H)
    y = orc.ada_layernorm_modulate(x, per_batch.contiguous(), zero, w, b, None)
    assert np.allclose(y, ln * np.array([1.0, 4.0]).reshape(B, 1, 1), rtol=1e-15, atol=0)
    y = orc.ada_layernorm_modulate(x, zero, sh, w, b, None)
    assert np.allclose(y - ln, np.broadcast_to(sh.double().numpy(), y.shape), rtol=0, atol=1e-15)
    y = orc.ada_layernorm_modulate(x, zero, zero, w, b, sm)
    assert np.allclose(y, ln * sm.astype(np.float64), rtol=1e-15, atol=0)


def pin_ada_worked_row(orc):
    """Row [1, 2, 3, 4], eps 1e-5, no affine or modulation: LN is
    [-1.5, -0.5, 0.5, 1.5] / sqrt(1.25 + eps), so the codes are
    round(127 * [-1, -1/3, 1/3, 1]) = [-127, -42, 42, 127]; a constant row
    normalizes to 0, leaving y = bias * (1 + scale) + shift."""
    x = _bf16([[[1, 2, 3, 4]]])
    z = torch.zeros(1, 1, 4, dtype=torch.bfloat16)
    out, qs = orc.ada_layernorm_quant(x, z, z, None, None, None, 1e-5)
    assert out.tolist() == [[[-127, -42, 42, 127]]]
    assert np.isclose(qs[0, 0], 1.5 / np.sqrt(1.25 + 1e-5) / 127, rtol=1e-6)
    xc = _bf16([[[0.75] * 4]])
    bias = _bf16([0.5, -1, 2, 0.25])
    sc = _bf16([[[1, 0, -0.5, 3]]])
    sh = _bf16([[[0.25, 0.5, -1, 0]]])
    y = orc.ada_layernorm_modulate(xc, sc, sh, None, bias, None)
    assert y.tolist() == [[[1.25, -0.5, 0.0, 1.0]]]


def pin_ada_quant_matches_dq_sym(orc):
    """Steps 4-5 are symmetric INT8 dynamic quantization of y.  With
    scale = -1, y = shift * smooth exactly (a bf16 times an fp32 is exact in
    float64), so codes and quantScale must equal DynamicQuant's symmetric
    INT8 result for x = shift and the same smooth scales (hand-pinned
    above), row by row."""
    rng = np.random.default_rng(23)
    B, S, H = 2, 3, 40
    x = _rand_bf16(rng, (B, S, H))
    _, sh, w, b = _ada_params(rng, B, H)
    sm = rng.uniform(0.5, 2.0, H).astype(f32)
    minus = -torch.ones(B, 1, H, dtype=torch.bfloat16)
    out, qs = orc.ada_layernorm_quant(x, minus, sh, w, b, sm)
    yd, sd, _ = orc.dynamic_quant(sh.reshape(B, H), smooth=sm)
    for s in range(S):
        assert np.array_equal(out[:, s, :], yd)
        assert np.array_equal(qs[:, s], sd)


def pin_ada_absmax_code(orc):
    """Every row's absmax element quantizes to +-127 and all codes reproduce
    y within half a step (plus binary32 rounding)."""
    rng = np.random.default_rng(24)
    B, S, H = 2, 8, 96
    x = _rand_bf16(rng, (B, S, H))
    sc, sh, w, b = _ada_params(rng, B, H)
    sm = rng.uniform(0.5, 2.0, H).astype(f32)
    out, qs, y = orc.ada_layernorm_quant(x, sc, sh, w, b, sm, want_y=True)
    assert np.all(np.abs(out).max(axis=2) == 127)
    err = np.abs(y - out.astype(np.float64) * qs[..., None].astype(np.float64))
    assert np.all(err <= qs[..., None] * (0.5 + 2.0 ** -16))



def _discriminating_absmax(rng, D):
    """A binary32 A with RN(A / D) != RN(A * RN(1 / D))."""
    while True:
        A = (rng.uniform(1.0, 2.0, 4096) * 2.0 ** rng.integers(-20, 20, 4096)).astype(f32)
        A = A[(A / f32(D)) != A * (f32(1) / f32(D))]
        if A.size:
            return A[0]


def pin_ada_quant_steps_match_numpy_float32(orc):
    """Steps 4-5 in binary32 (R14: y rounded once to binary32, then
    quantScale = RN(max|y| / 127) and out = rne(RN(y / quantScale))) against
    numpy float32.  With scale = -1 the LayerNorm term vanishes and
    y = shift * smooth exactly in binary64, so y can be placed at will:
      - shift = +-1: y is the binary32 smooth value; the row maximum makes
        RN(A / 127) differ from A * RN(1 / 127), and the other values sit
        within a few ulps of the points where y / quantScale crosses k + 1/2,
        where division and reciprocal multiplication disagree;
      - shift = +-1.5: y = 1.5 * smooth needs 25 bits, and the values are
        chosen where rounding y to binary32 first moves the quotient across
        k + 1/2, so deciding the code from the binary64 y would differ.
    Then random rows through the whole formula, steps 4-5 applied by numpy
    to the oracle's binary64 y (steps 1-3 are pinned against torch)."""
    rng = np.random.default_rng(25)
    B, S, H = 3, 2, 1024
    A = _discriminating_absmax(rng, 127.0)
    sc32 = A / f32(127)
    k = np.arange(127, dtype=np.float64)
    near = _ulp_walk((k + 0.5) * np.float64(sc32), range(-3, 4))
    near = near[near < A]
    mags = rng.permutation(np.concatenate([[A], near, rng.uniform(0, 1, H).astype(f32) * A])[:H]).astype(f32)
    signs = np.where(rng.random((B, 1, H)) < 0.5, -1.0, 1.0).astype(np.float32)
    sh = torch.from_numpy(signs).to(torch.bfloat16)
    minus = -torch.ones(B, 1, H, dtype=torch.bfloat16)
    x = _rand_bf16(rng, (B, S, H))
    out, qs = orc.ada_layernorm_quant(x, minus, sh, None, None, mags)
    y32 = (signs * mags).astype(f32)  # exact: +-1 times a binary32
    want_qs = np.abs(y32).max(axis=2) / f32(127)
    assert not np.array_equal(want_qs, (np.abs(y32).max(axis=2) * (f32(1) / f32(127))).astype(f32))
    with np.errstate(all="ignore"):
        want = np.clip(np.rint(y32 / want_qs[..., None]), -128, 127)
        alt = np.clip(np.rint(y32 * (f32(1) / want_qs[..., None])), -128, 127)
    assert not np.array_equal(want, alt), "inputs must tell division from reciprocal"
    for s in range(S):
        assert np.array_equal(out[:, s, :].astype(np.int64), want[:, 0, :].astype(np.int64))
        assert np.array_equal(qs[:, s].view(np.uint32), want_qs[:, 0].view(np.uint32))
    # shift = +-1.5: the binary32 rounding of y decides codes.
    A = f32(rng.uniform(1.0, 2.0) * 2.0 ** 3)
    q32 = (f32(1.5) * A).astype(f32) / f32(127)  # RN(RN(1.5 A) / 127), the quantScale
    cand = []
    for kk in range(127):
        c = (kk + 0.5) * np.float64(q32) / 1.5
        for d in range(-40, 41):
            sm = _ulp_walk(np.array([c]), [d])[0]
            y64 = 1.5 * np.float64(sm)
            y32 = np.float32(y64)
            if y64 < 1.5 * np.float64(A) and np.rint(np.float64(y32 / q32)) != np.rint(y64 / np.float64(q32)):
                cand.append(sm)
    assert len(cand) > 0
    mags = np.concatenate([[A], np.array(cand, f32), rng.uniform(0, 1, H).astype(f32) * A])[:H].astype(f32)
    mags = rng.permutation(mags)
    signs = np.where(rng.random((1, 1, H)) < 0.5, -1.5, 1.5).astype(np.float32)
    sh = torch.from_numpy(signs).to(torch.bfloat16)
    out, qs = orc.ada_layernorm_quant(x[:1], -torch.ones(1, 1, H, dtype=torch.bfloat16), sh, None, None, mags)
    y64 = signs.astype(np.float64) * mags.astype(np.float64)
    y32 = y64.astype(f32)
    want_qs = np.abs(y32).max(axis=2) / f32(127)
    want = np.clip(np.rint(y32 / want_qs[..., None]), -128, 127).astype(np.int64)
    wide = np.clip(np.rint(y64 / want_qs[..., None].astype(np.float64)), -128, 127).astype(np.int64)
    assert not np.array_equal(want, wide), "inputs must tell a binary32 decision from a binary64 one"
    for s in range(S):
        assert np.array_equal(out[:, s, :].astype(np.int64), want[:, 0, :])
        assert np.array_equal(qs[:, s].view(np.uint32), want_qs[:, 0].view(np.uint32))
    # Random rows, every optional tensor present.
    B, S, H = 2, 6, 320
    x = _rand_bf16(rng, (B, S, H))
    sc, sh, w, b = _ada_params(rng, B, H)
    sm = rng.uniform(0.5, 2.0, H).astype(f32)
    out, qs, y = orc.ada_layernorm_quant(x, sc, sh, w, b, sm, want_y=True)
    y32 = y.astype(f32)
    want_qs = np.abs(y32).max(axis=2) / f32(127)
    want = np.clip(np.rint(y32 / want_qs[..., None]), -128, 127).astype(np.int64)
    assert np.array_equal(out.astype(np.int64), want)
    assert np.array_equal(qs.view(np.uint32), want_qs.view(np.uint32))

# ---------------------------------------------------------------------------
# AntiQuantize
# ---------------------------------------------------------------------------

def _golden_identity_row():
    with open(os.path.join(GOLDEN, "antiquantize_identity_example.txt")) as f:
        rows = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    return np.array([int(v) for v in rows[0]], dtype=np.int8)


def pin_aq_page_identity_example(orc):
    """The page's worked example: scale 1 and offset 0 (scalar for
    PER_TENSOR, vectors otherwise) leave dst equal to src."""
    row = _golden_identity_row()
    m, n = 3, row.size
    src = np.stack([row, row[::-1], -row]).astype(np.int8)
    cases = {
        "per_tensor": (np.ones(1, f32), np.zeros(1, f32), {}),
        "per_channel": (np.ones((1, n), f32), np.zeros((1, n), f32), {}),
        "per_token": (np.ones((m, 1), f32), np.zeros((m, 1), f32), {}),
        "per_group": (np.ones((m, 1), f32), np.zeros((m, 1), f32), {"kdim": 1, "group_size": n}),
    }
    for pol, (s, o, kw) in cases.items():
        for dst, widen in (("float16", _bits_to_f16_f32), ("bfloat16", _bits_to_bf16_f32)):
            d = orc.antiquantize(src, s, o, policy=pol, dst=dst, **kw)
            assert np.array_equal(widen(d), src.astype(np.float32)), (pol, dst)
            d_half_params = orc.antiquantize(src, s.astype(np.float16), o.astype(np.float16),
                                             policy=pol, dst=dst, **kw)
            assert np.array_equal(d_half_params, d)


def pin_aq_policy_reductions(orc):
    """PER_GROUP with kDim=1 and groupSize >= n is PER_TOKEN; kDim=0 and
    groupSize >= m is PER_CHANNEL; PER_CHANNEL / PER_TOKEN with constant
    vectors are PER_TENSOR; a PER_GROUP column block (kDim=1) is PER_TOKEN on
    that block with that group's column, including a short last group."""
    rng = np.random.default_rng(31)
    m, n, gs = 6, 80, 32  # three groups along n, the last one 16 wide
    src = rng.integers(-128, 128, (m, n)).astype(np.int8)
    s_tok = rng.uniform(0.001, 0.05, (m, 1)).astype(f32)
    o_tok = rng.uniform(-8, 8, (m, 1)).astype(f32)
    s_ch = rng.uniform(0.001, 0.05, (1, n)).astype(f32)
    o_ch = rng.uniform(-8, 8, (1, n)).astype(f32)
    tok = orc.antiquantize(src, s_tok, o_tok, "per_token")
    assert np.array_equal(orc.antiquantize(src, s_tok, o_tok, "per_group", 1, n), tok)
    assert np.array_equal(orc.antiquantize(src, s_tok, o_tok, "per_group", 1, 4 * n), tok)
    ch = orc.antiquantize(src, s_ch, o_ch, "per_channel")
    assert np.array_equal(orc.antiquantize(src, s_ch, o_ch, "per_group", 0, m), ch)
    assert np.array_equal(orc.antiquantize(src, s_ch, o_ch, "per_group", 0, 64), ch)
    t = orc.antiquantize(src, s_tok[:1, 0], o_tok[:1, 0], "per_tensor")
    assert np.array_equal(orc.antiquantize(src, np.repeat(s_tok[:1], n, 1),
                                           np.repeat(o_tok[:1], n, 1), "per_channel"), t)
    assert np.array_equal(orc.antiquantize(src, np.repeat(s_tok[:1], m, 0),
                                           np.repeat(o_tok[:1], m, 0), "per_token"), t)
    G = -(-n // gs)
    s_g = rng.uniform(0.001, 0.05, (m, G)).astype(f32)
    o_g = rng.uniform(-8, 8, (m, G)).astype(f32)
    g = orc.antiquantize(src, s_g, o_g, "per_group", 1, gs)
    for k in range(G):
        blk = slice(k * gs, min(n, (k + 1) * gs))
        ref = orc.antiquantize(np.ascontiguousarray(src[:, blk]), s_g[:, k:k + 1].copy(),
                               o_g[:, k:k + 1].copy(), "per_token")
        assert np.array_equal(g[:, blk], ref), k
    mg = 70  # kDim = 0: groups along m, the last one short
    src0 = rng.integers(-128, 128, (mg, 16)).astype(np.int8)
    G0 = -(-mg // gs)
    s0 = rng.uniform(0.001, 0.05, (G0, 16)).astype(f32)
    o0 = rng.uniform(-8, 8, (G0, 16)).astype(f32)
    g0 = orc.antiquantize(src0, s0, o0, "per_group", 0, gs)
    for k in range(G0):
        blk = slice(k * gs, min(mg, (k + 1) * gs))
        ref = orc.antiquantize(np.ascontiguousarray(src0[blk]), s0[k:k + 1].copy(),
                               o0[k:k + 1].copy(), "per_channel")
        assert np.array_equal(g0[blk], ref), k


def pin_aq_power_of_two_closed_form(orc):
    """With scale 2^k and an integer offset, (src + offset) * scale is exact
    in binary32 and, for |src + offset| < 256, in bf16 and fp16 too; so dst
    equals (src + offset) * 2^k, checked for every int8 code.  Without an
    offset dst = src * 2^k."""
    src = np.arange(-128, 128, dtype=np.int8).reshape(4, 64)
    for k, off in ((0, 0), (-3, 5), (2, -7), (-10, 100)):
        s = np.full(1, 2.0 ** k, f32)
        o = np.full(1, off, f32)
        want = (src.astype(np.float64) + off) * 2.0 ** k
        if np.abs(src.astype(np.int64) + off).max() < 256:
            for dst, widen in (("bfloat16", _bits_to_bf16_f32), ("float16", _bits_to_f16_f32)):
                d = widen(orc.antiquantize(src, s, o, "per_tensor", dst=dst))
                assert np.array_equal(d.astype(np.float64), want), (k, off, dst)
        d32 = orc.antiquantize(src, s, o, "per_tensor", dst="float32")
        assert np.array_equal(d32.astype(np.float64), want)
        d32 = orc.antiquantize(src, s, None, "per_tensor", dst="float32")
        assert np.array_equal(d32.astype(np.float64), src * 2.0 ** k)


def pin_aq_fp8_source(orc):
    """An fp8-e4m3fn source is decoded exactly: with scale 1 and offset 0
    the fp32 result equals torch's float8_e4m3fn -> float32 decode for all
    256 codes (NaN codes stay NaN)."""
    codes = np.arange(256, dtype=np.uint8).reshape(8, 32)
    d = orc.antiquantize(("float8_e4m3fn", codes), np.ones(1, f32), np.zeros(1, f32),
                         "per_tensor", dst="float32")
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(d), nan)
    assert np.array_equal(d[~nan], ref[~nan])


def _np_aq_params(policy, m, n, kdim, gs, s, o):
    """Broadcast a parameter tensor of the policy's shape to [m, n]."""
    if policy == "per_tensor":
        return np.full((m, n), s.reshape(-1)[0]), None if o is None else np.full((m, n), o.reshape(-1)[0])
    if policy == "per_channel":
        idx = (np.zeros((m, n), np.int64), np.broadcast_to(np.arange(n), (m, n)))
    elif policy == "per_token":
        idx = (np.broadcast_to(np.arange(m)[:, None], (m, n)), np.zeros((m, n), np.int64))
    elif kdim == 1:
        idx = (np.broadcast_to(np.arange(m)[:, None], (m, n)), np.broadcast_to(np.arange(n) // gs, (m, n)))
    else:
        idx = (np.broadcast_to((np.arange(m) // gs)[:, None], (m, n)), np.broadcast_to(np.arange(n), (m, n)))
    return s[idx], None if o is None else o[idx]


def pin_aq_matches_numpy_float32(orc):
    """Every policy (per-tensor, per-channel, per-token, per-group along n
    and along m with a short last group), int8 / e4m3fn / e5m2 sources,
    fp32 / fp16 / bf16 parameters, with and without offset: dst equals
    numpy's binary32 (v + o) * s (or v * s), rounded once by torch's bf16
    cast or numpy's fp16 cast, or kept in fp32.  The scales are not powers
    of two, and the inputs are checked to tell (v + o) * s apart from
    v * s + o * s and from a fused multiply-add."""
    rng = np.random.default_rng(33)
    m, n, gs = 70, 96, 32
    srcs = {
        "int8": rng.integers(-128, 128, (m, n)).astype(np.int8),
        "float8_e4m3fn": torch.from_numpy(np.clip(rng.normal(0, 4, (m, n)), -448, 448).astype(np.float32))
                             .to(torch.float8_e4m3fn),
        "float8_e5m2": torch.from_numpy(np.clip(rng.normal(0, 4, (m, n)), -57344, 57344).astype(np.float32))
                           .to(torch.float8_e5m2),
    }
    shapes = {"per_tensor": ((1,), 1, 0), "per_channel": ((1, n), 1, 0), "per_token": ((m, 1), 1, 0),
              "per_group1": ((m, -(-n // gs)), 1, gs), "per_group0": ((-(-m // gs), n), 0, gs)}
    told_apart = [False, False]
    for sname, src in srcs.items():
        v = src.astype(np.float32) if isinstance(src, np.ndarray) else src.float().numpy()
        for pname, (shape, kdim, g) in shapes.items():
            policy = pname[:-1] if pname.startswith("per_group") else pname
            s32 = rng.uniform(0.001, 0.05, shape).astype(f32)
            o32 = rng.uniform(-8, 8, shape).astype(f32)
            for pdt in ("float32", "float16", "bfloat16"):
                if pdt == "float32":
                    s, o = s32, o32
                    sw, ow = s32, o32
                elif pdt == "float16":
                    s, o = s32.astype(np.float16), o32.astype(np.float16)
                    sw, ow = s.astype(f32), o.astype(f32)
                else:
                    s, o = _bf16(s32), _bf16(o32)
                    sw, ow = s.float().numpy(), o.float().numpy()
                S_, O_ = _np_aq_params(policy, m, n, kdim, g, sw, ow)
                for with_off in (True, False):
                    t = ((v + O_).astype(f32) * S_).astype(f32) if with_off else (v * S_).astype(f32)
                    if with_off:
                        dist = ((v * S_).astype(f32) + (O_ * S_).astype(f32)).astype(f32)
                        fma = (v.astype(np.float64) * S_ + (O_ * S_).astype(f32)).astype(f32)
                        told_apart[0] |= not np.array_equal(t, dist)
                        told_apart[1] |= not np.array_equal(t, fma)
                    kw = {"kdim": kdim, "group_size": g} if policy == "per_group" else {}
                    oo = o if with_off else None
                    d32 = orc.antiquantize(src, s, oo, policy, dst="float32", **kw)
                    assert np.array_equal(d32.view(np.uint32), t.view(np.uint32)), (sname, pname, pdt)
                    dbf = orc.antiquantize(src, s, oo, policy, dst="bfloat16", **kw)
                    want_bf = torch.from_numpy(t).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
                    assert np.array_equal(dbf, want_bf), (sname, pname, pdt)
                    dh = orc.antiquantize(src, s, oo, policy, dst="float16", **kw)
                    assert np.array_equal(dh, t.astype(np.float16).view(np.uint16)), (sname, pname, pdt)
    assert all(told_apart), "inputs must tell the two-step form from the distributed and fused forms"


def pin_aq_e5m2_source(orc):
    """An fp8-e5m2 source is decoded exactly: e5m2 is the upper byte of a
    binary16, so with scale 1 and offset 0 the fp32 result equals numpy's
    float16 of bits (code << 8) for all 256 codes (infinities included, NaN
    codes stay NaN); the fp16 destination then holds exactly those bits."""
    codes = np.arange(256, dtype=np.uint8).reshape(8, 32)
    ref = (codes.astype(np.uint16) << 8).view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    d = orc.antiquantize(("float8_e5m2", codes), np.ones(1, f32), np.zeros(1, f32),
                         "per_tensor", dst="float32")
    assert np.array_equal(np.isnan(d), nan)
    assert np.array_equal(d[~nan], ref[~nan])
    h = orc.antiquantize(("float8_e5m2", codes), np.ones(1, f32), None, "per_tensor", dst="float16")
    assert np.array_equal(h[~nan], (codes.astype(np.uint16) << 8)[~nan])


# The OCP Microscaling (MX) v1.0 table of FP4 E2M1 values, codes 0..15.
OCP_E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
            -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]


def pin_aq_float4_per_group_worked(orc):
    """The float4 case of 表3 (PER_GROUP, fp4x2 e2m1 source, e8m0 scale, no
    offset), worked by hand.  Row 0: group 0 has e8m0 127 (x1), group 1 has
    130 (x8); row 1: 126 (x0.5) and 255 (NaN).  Codes, two per byte with the
    first element in the low nibble: row 0 starts 0x71 -> [0.5, 6], its
    second group 0xB3 -> [1.5, -1.5] x 8 = [12, -12]; row 1 starts 0x6E ->
    [-4, 4] x 0.5 = [-2, 2]; its second group is NaN.  kDim = 0 with groups
    of 32 rows: rows 0..31 take scale row 0."""
    m, n, gs = 2, 64, 32
    src = np.zeros((m, n // 2), np.uint8)
    src[0, 0], src[0, 16], src[1, 0], src[1, 16] = 0x71, 0xB3, 0x6E, 0x22
    sc = np.array([[127, 130], [126, 255]], np.uint8)
    d = orc.antiquantize(("float4_e2m1x2", src), ("float8_e8m0", sc), None, "per_group", kdim=1,
                         group_size=gs, dst="float32")
    assert d.shape == (m, n)
    assert d[0, :2].tolist() == [0.5, 6.0] and d[0, 32:34].tolist() == [12.0, -12.0]
    assert d[1, :2].tolist() == [-2.0, 2.0] and np.all(np.isnan(d[1, 32:]))
    assert np.all(d[0, 2:32] == 0) and np.all(d[0, 34:] == 0) and np.all(d[1, 2:32] == 0)
    sc0 = np.full((1, n), 127, np.uint8)
    sc0[0, 33] = 131  # x16 on column 33 for both rows
    d0 = orc.antiquantize(("float4_e2m1x2", src), ("float8_e8m0", sc0), None, "per_group", kdim=0,
                          group_size=gs, dst="float32")
    assert d0[0, :2].tolist() == [0.5, 6.0] and d0[0, 32:34].tolist() == [1.5, -24.0]
    assert d0[1, :2].tolist() == [-4.0, 4.0] and d0[1, 32:34].tolist() == [1.0, 16.0]


def pin_aq_float4_table_and_scaling(orc):
    """With e8m0 127 (x1) every code decodes to the OCP E2M1 table, for both
    nibble positions, and the bf16 / fp16 destinations hold those values
    exactly; e8m0 k multiplies by 2^(k - 127) exactly down to 2^-127 (a
    binary32 subnormal), and products of 2^128 or more overflow to infinity
    (2 x 2^127 does, 1.5 x 2^127 does not)."""
    codes = np.arange(256, dtype=np.uint8).reshape(8, 32)
    lo, hi = codes & 0xF, codes >> 4
    want = np.empty((8, 64), np.float64)
    want[:, 0::2] = np.array(OCP_E2M1)[lo]
    want[:, 1::2] = np.array(OCP_E2M1)[hi]
    one = ("float8_e8m0", np.full((8, 2), 127, np.uint8))
    d = orc.antiquantize(("float4_e2m1x2", codes), one, None, "per_group", kdim=1, group_size=32,
                         dst="float32")
    assert np.array_equal(d.astype(np.float64), want)
    assert np.array_equal(np.signbit(d), np.signbit(want))
    for dst, cast in (("bfloat16", _bits_to_bf16_f32), ("float16", _bits_to_f16_f32)):
        b = orc.antiquantize(("float4_e2m1x2", codes), one, None, "per_group", kdim=1,
                             group_size=32, dst=dst)
        assert np.array_equal(cast(b).astype(np.float64), want)
    for k in (0, 1, 100, 127, 200, 253, 254):
        sc = ("float8_e8m0", np.full((8, 2), k, np.uint8))
        d = orc.antiquantize(("float4_e2m1x2", codes), sc, None, "per_group", kdim=1, group_size=32,
                             dst="float32")
        with np.errstate(over="ignore"):
            exact = (want * 2.0 ** (k - 127)).astype(np.float32)  # exact product, one rounding
        assert np.array_equal(d, exact)
    assert np.isinf(exact[np.abs(want) >= 2.0]).all() and np.isfinite(exact[np.abs(want) < 2.0]).all()


def pin_roundtrip_dq_asym_aq_token(orc):
    """Round trip: AntiQuantize PER_TOKEN of DynamicQuant's asymmetric INT8
    output, with scale = scaleOut and offset = -offsetOut, reproduces x to
    within half a quantization step plus the binary32 roundings of both ops
    and the final bf16 rounding.  This ties the reading dst = (src +
    offset) * scale to DynamicQuant's y = x / scale + offset."""
    rng = np.random.default_rng(41)
    x = _rand_bf16(rng, (32, 128), scale=2.0)
    y, s, o = orc.dynamic_quant(x, symmetric=False)
    d = orc.antiquantize(y, s[:, None].copy(), -o[:, None], "per_token", dst="bfloat16")
    xr = _bits_to_bf16_f32(d).astype(np.float64)
    xv = x.float().numpy().astype(np.float64)
    ulp = np.abs(xr) * 2.0 ** -8
    assert np.all(np.abs(xr - xv) <= s[:, None] * (0.5 + 2.0 ** -14) + ulp)


# ---------------------------------------------------------------------------
# mx block quantization (aclnnQuantBatchMatmulInplaceAdd, 计算公式 mx量化,
# read as the OCP Microscaling v1.0 conversion)
# ---------------------------------------------------------------------------

MX_KINDS = ("float8_e4m3fn", "float8_e5m2", "float4_e2m1x2")


def _mx_table(kind):
    """Values of every code of an element format, from torch's fp8 decoders
    and the OCP E2M1 table (not from the oracle), NaN / inf marked
    non-finite."""
    if kind == "float4_e2m1x2":
        return np.array(OCP_E2M1, np.float64)
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    dt = torch.float8_e4m3fn if kind == "float8_e4m3fn" else torch.float8_e5m2
    return codes.view(dt).float().numpy().astype(np.float64)


def _mx_brute(block, kind):
    """Reference quantization of one block by search: the scale exponent is
    the smallest k in [-127, 127] with max|v| < 2^(emax + 1 + k), emax being
    the binade of the largest finite code; each code is the finite code of
    v's sign nearest to v / 2^k (ties to the code with an even last bit).
    Returns (scale byte, codes)."""
    vals = _mx_table(kind)
    fin = np.isfinite(vals)
    emax = int(np.frexp(vals[fin].max())[1]) - 1
    block = np.asarray(block, np.float64)
    if not np.all(np.isfinite(block)):
        return 0xFF, np.zeros(block.size, np.int64)
    amax = np.abs(block).max()
    k = next(k for k in range(-127, 128) if amax < 2.0 ** (emax + 1 + k))
    t = block * 2.0 ** -k
    codes = np.arange(vals.size)
    out = []
    for ti in t:
        ok = fin & (np.signbit(vals) == np.signbit(ti))
        d = np.where(ok, np.abs(vals - ti), np.inf)
        best = codes[d == d.min()]
        if best.size > 1:
            best = best[best % 2 == 0]
        assert best.size == 1
        out.append(int(best[0]))
    return k + 127, np.array(out)


def _unpack_fp4(y):
    y = np.asarray(y, np.uint8)
    out = np.empty(y.shape[:-1] + (2 * y.shape[-1],), np.int64)
    out[..., 0::2] = y & 0xF
    out[..., 1::2] = y >> 4
    return out


def _mx_codes(y, kind):
    return _unpack_fp4(y) if kind == "float4_e2m1x2" else np.asarray(y, np.int64)


def pin_mx_worked_blocks(orc):
    """Worked by hand.  Block [12, 3, -5, 0.5, 1.5, 0.75, -0, 9, 11, 7, 0...]:
    max 12 has binade 3.  fp4 (emax 2): shared 1, scale byte 128, quotients
    6, 1.5, -2.5, 0.25, 0.75, 0.375, -0, 4.5, 5.5, 3.5 -> codes 7, 3, 0xC
    (2.5 ties to 2), 0 (0.25 ties to 0), 2 (0.75 ties to 1.0), 1, 8 (-0), 6
    (4.5 -> 4), 7 (5.5 -> 6), 6 (3.5 ties to 4).  fp8 e4m3 (emax 8): shared
    -5, byte 122, 12 x 32 = 384 = 1.5 x 2^8 -> 0x7C.  fp8 e5m2 (emax 15):
    shared -12, byte 115, 12 x 4096 = 1.5 x 2^15 -> 0x7A."""
    row = [12, 3, -5, 0.5, 1.5, 0.75, -0.0, 9, 11, 7] + [0.0] * 22
    for mk in (_bf16, _f16):
        x = mk([row])
        y, s = orc.mx_quantize(x, "float4_e2m1x2")
        assert s.tolist() == [[128]]
        assert y[0, :5].tolist() == [0x37, 0x0C, 0x12, 0x68, 0x67] and not y[0, 5:].any()
        y, s = orc.mx_quantize(x, "float8_e4m3fn")
        assert s.tolist() == [[122]] and y[0, 0] == 0x7C and y[0, 6] == 0x80
        y, s = orc.mx_quantize(x, "float8_e5m2")
        assert s.tolist() == [[115]] and y[0, 0] == 0x7A and y[0, 6] == 0x80


def _mx_random_blocks(rng, nblk, dtype):
    """Blocks whose magnitudes span the input format: each block draws a
    binade, normal values around it and a few zeros and sign flips."""
    lo, hi = (-140, 120) if dtype == torch.bfloat16 else (-24, 15)
    e = rng.integers(lo, hi, nblk)
    v = rng.standard_normal((nblk, 32)) * np.exp2(e)[:, None]
    v[rng.random((nblk, 32)) < 0.05] = 0.0
    return torch.from_numpy(v.astype(np.float32)).to(dtype)


def pin_mx_brute_force_nearest(orc):
    """Random blocks over the whole input range, both input types, all three
    element formats: scale bytes and codes equal the search in _mx_brute."""
    rng = np.random.default_rng(61)
    for dtype in (torch.bfloat16, torch.float16):
        x = _mx_random_blocks(rng, 96, dtype).reshape(12, 256)
        xv = x.float().numpy().astype(np.float64)
        for kind in MX_KINDS:
            y, s = orc.mx_quantize(x, kind)
            c = _mx_codes(y, kind)
            for r in range(12):
                for j in range(8):
                    ws, wc = _mx_brute(xv[r, 32 * j:32 * j + 32], kind)
                    assert s[r, j] == ws, (kind, r, j)
                    assert np.array_equal(c[r, 32 * j:32 * j + 32], wc), (kind, r, j)


def pin_mx_ties_and_saturation(orc):
    """Blocks built on the element grid: the first element is the largest
    finite code times 2^k (so the scale byte is k + 127 for the format's
    emax), the rest are midpoints between adjacent codes (ties, which go to
    the even code) and values between the largest code and the next binade
    (which saturate)."""
    rng = np.random.default_rng(62)
    for kind in MX_KINDS:
        vals = _mx_table(kind)
        fin = np.isfinite(vals) & ~np.signbit(vals)
        pos = np.sort(vals[fin])
        top = pos[-1]
        emax = int(np.frexp(top)[1]) - 1
        for k in (-20, 0, 7):
            mids = (pos[:-1] + pos[1:]) / 2
            pick = rng.choice(mids, 24)
            over = top + (2.0 ** (emax + 1) - top) * (0.01 + 0.98 * rng.random(7))
            blk = np.concatenate([[top], pick, over]) * rng.choice([-1.0, 1.0], 32)
            x = torch.from_numpy((blk * 2.0 ** k)[None].astype(np.float32)).to(torch.bfloat16)
            blk = x.float().numpy()[0].astype(np.float64) * 2.0 ** -k  # bf16-rounded
            assert np.all(np.abs(blk[25:]) > top) and np.all(np.abs(blk) < 2.0 ** (emax + 1))
            y, s = orc.mx_quantize(x, kind)
            ws, wc = _mx_brute(blk * 2.0 ** k, kind)
            assert s[0, 0] == ws == k + 127
            assert np.array_equal(_mx_codes(y, kind)[0], wc)
            got = vals[_mx_codes(y, kind)[0]]
            assert np.all(np.abs(got[25:]) == top)  # saturated


def pin_mx_fp8_matches_torch_cast(orc):
    """For fp8 elements the code of v equals torch's float32 -> float8 cast of
    v / 2^shared (a library rounding, nearest-even), wherever that quotient
    is within the format's finite range."""
    rng = np.random.default_rng(63)
    x = _mx_random_blocks(rng, 256, torch.bfloat16).reshape(32, 256)
    xv = x.float().numpy().astype(np.float64)
    for kind, dt in (("float8_e4m3fn", torch.float8_e4m3fn), ("float8_e5m2", torch.float8_e5m2)):
        y, s = orc.mx_quantize(x, kind)
        q = xv.reshape(32, 8, 32) * np.exp2(127.0 - s.astype(np.float64))[:, :, None]
        q = q.reshape(32, 256).astype(np.float32)
        ref = torch.from_numpy(q).to(dt).view(torch.uint8).numpy()
        ok = np.abs(q) <= torch.finfo(dt).max
        assert ok.mean() > 0.9
        assert np.array_equal(y[ok], ref[ok])


def pin_mx_power_of_two_shift(orc):
    """Scaling the input by 2^m adds m to every scale byte and leaves every
    code unchanged, as long as no block's exponent leaves [-127, 127]."""
    rng = np.random.default_rng(64)
    v = rng.standard_normal((8, 96)) * np.exp2(rng.integers(-8, 8, (8, 1)))
    x = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16)
    for kind in MX_KINDS:
        y0, s0 = orc.mx_quantize(x, kind)
        for m in (-60, -1, 1, 60):
            y1, s1 = orc.mx_quantize(x * 2.0 ** m, kind)
            assert np.array_equal(y1, y0)
            assert np.array_equal(s1.astype(int), s0.astype(int) + m)


def pin_mx_roundtrip_through_antiquantize(orc):
    """Producer against consumer: grid values (a code times 2^(e - 127), each
    block holding one code of the top binade) decoded by the AntiQuantize
    float4 path (PER_GROUP, groups of 32, e8m0 scale), or for fp8 by torch's
    decoder, quantize back to the same codes and scale bytes."""
    rng = np.random.default_rng(65)
    rows, n = 6, 128
    codes = rng.integers(0, 16, (rows, n)).astype(np.uint8)
    codes[:, ::32] = rng.choice([6, 7, 14, 15], (rows, n // 32))  # top binade [4, 8)
    sc = rng.integers(100, 150, (rows, n // 32)).astype(np.uint8)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    d = orc.antiquantize(("float4_e2m1x2", packed), ("float8_e8m0", sc), None, "per_group",
                         kdim=1, group_size=32, dst="bfloat16")
    x = torch.from_numpy(d.view(np.int16).copy()).view(torch.bfloat16)
    y, s = orc.mx_quantize(x, "float4_e2m1x2")
    assert np.array_equal(s, sc)
    # zero codes may come back as the other zero; compare values and signs
    want = np.where(codes & 7, codes, codes & 8)
    assert np.array_equal(_unpack_fp4(y), want)
    for kind in ("float8_e4m3fn", "float8_e5m2"):
        vals = _mx_table(kind)
        fin = np.flatnonzero(np.isfinite(vals))
        top = fin[np.frexp(np.abs(vals[fin]))[1] - 1 == np.frexp(np.nanmax(vals[fin]))[1] - 1]
        c = rng.choice(fin, (rows, n))
        c[:, ::32] = rng.choice(top, (rows, n // 32))
        e = rng.integers(100, 150, (rows, n // 32))
        v = vals[c] * np.exp2(np.repeat(e, 32, axis=1) - 127.0)
        x = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16)
        assert np.array_equal(x.float().numpy(), v.astype(np.float32))
        y, s = orc.mx_quantize(x, kind)
        assert np.array_equal(s.astype(np.int64), e)
        back = vals[y.astype(np.int64)]
        assert np.array_equal(back, vals[c])
        assert np.array_equal(np.signbit(back), np.signbit(vals[c]))


def pin_mx_special_blocks(orc):
    """An all-zero block: scale byte 0 (the exponent clamps to -127), codes
    are zeros of each element's sign.  A block with a NaN or an infinity:
    scale byte 0xFF, all codes 0.  Tiny blocks: bf16 2^-130 has binade -130,
    so e4m3's exponent -138 clamps to -127 and the quotient 2^-3 encodes as
    0x20; fp16 2^-24 has exponent -32 and quotient 2^8 -> 0x78."""
    z = _bf16([[0.0] * 16 + [-0.0] * 16])
    for kind in MX_KINDS:
        y, s = orc.mx_quantize(z, kind)
        assert s.tolist() == [[0]]
        c = _mx_codes(y, kind)[0]
        sign = 0x8 if kind == "float4_e2m1x2" else 0x80
        assert np.all(c[:16] == 0) and np.all(c[16:] == sign)
    for bad in (float("nan"), float("inf"), float("-inf")):
        x = _bf16([[1.0] * 32 + [bad] + [2.0] * 31])
        for kind in MX_KINDS:
            y, s = orc.mx_quantize(x, kind)
            assert s[0, 1] == 0xFF and s[0, 0] != 0xFF
            assert not _mx_codes(y, kind)[0, 32:].any()
    y, s = orc.mx_quantize(_bf16([[2.0 ** -130] * 32]), "float8_e4m3fn")
    assert s.tolist() == [[0]] and np.all(y == 0x20)
    y, s = orc.mx_quantize(_f16([[2.0 ** -24] + [0.0] * 31]), "float8_e4m3fn")
    assert s.tolist() == [[127 - 32]] and y[0, 0] == 0x78


def pin_mx_short_block_and_axis(orc):
    """n = 72: blocks [0, 32), [32, 64), [64, 72); the short block's scale
    follows its own 8 elements.  Axis 0 (blocks down the rows) on x equals
    axis 1 on x transposed, codes and scales transposed back."""
    rng = np.random.default_rng(66)
    v = rng.standard_normal((5, 72))
    v[:, :64] *= 1000.0
    x = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16)
    xv = x.float().numpy().astype(np.float64)
    for kind in MX_KINDS:
        y, s = orc.mx_quantize(x, kind)
        assert s.shape == (5, 3)
        c = _mx_codes(y, kind)
        for r in range(5):
            ws, wc = _mx_brute(xv[r, 64:], kind)
            assert s[r, 2] == ws and np.array_equal(c[r, 64:], wc)
        xt = x.t().contiguous()  # [72, 5]; axis 0 -> blocks along 72
        if kind != "float4_e2m1x2":
            y0, s0 = orc.mx_quantize(xt, kind, axis=0)
            assert s0.shape == (3, 5)
            assert np.array_equal(s0, s.T) and np.array_equal(y0, y.T)
    x2 = torch.from_numpy(rng.standard_normal((72, 6)).astype(np.float32)).to(torch.bfloat16)
    y0, s0 = orc.mx_quantize(x2, "float4_e2m1x2", axis=0)
    y1, s1 = orc.mx_quantize(x2.t().contiguous(), "float8_e4m3fn")
    assert s0.shape == (3, 6) and np.array_equal(s0.astype(int), s1.T.astype(int) + 6)
    xv2 = x2.float().numpy().astype(np.float64)
    c0 = _unpack_fp4(y0)
    for col in range(6):
        for j in range(3):
            ws, wc = _mx_brute(xv2[32 * j:32 * j + 32, col], "float4_e2m1x2")
            assert s0[j, col] == ws and np.array_equal(c0[32 * j:32 * j + 32, col], wc)


# ---------------------------------------------------------------------------
# Weight-quantized matmul (aclnnWeightQuantMatmulAllReduce on one rank)
# ---------------------------------------------------------------------------

def _pack_int4(codes: np.ndarray) -> np.ndarray:
    """Signed 4-bit codes [r, 2c] -> bytes [r, c], the even element low."""
    u = (codes.astype(np.int16) & 0xF).astype(np.uint8)
    return (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)


def _wq_case(rng, k, n, policy, gs, dtype, w="int8", offset=True, transpose=False):
    """Random weights and parameters; returns the oracle arguments and, for
    the reference, the signed codes [k, n] and parameters as float32."""
    lo, hi = (-128, 128) if w == "int8" else (-8, 8)
    codes = rng.integers(lo, hi, (k, n)).astype(np.int8)
    if policy == "per_tensor":
        pshape = (1,)
    elif policy == "per_channel":
        pshape = (n,)
    else:
        pshape = (-(-k // gs), n)
    sc = torch.from_numpy(rng.uniform(0.01, 0.1, pshape).astype(np.float32)).to(dtype)
    of = torch.from_numpy(rng.uniform(-4, 4, pshape).astype(np.float32)).to(dtype) if offset else None
    stored = codes.T.copy() if transpose else codes
    x2 = stored if w == "int8" else ("int4", _pack_int4(stored))
    if transpose and policy == "per_group":
        sc_arg = sc.t().contiguous()
        of_arg = None if of is None else of.t().contiguous()
    else:
        sc_arg, of_arg = sc, of
    return x2, sc_arg, of_arg, codes, sc.float().numpy(), None if of is None else of.float().numpy()


def _numpy_dequant(codes, s, o, policy, gs, dtype):
    """W from numpy float32 arithmetic and torch's float32 -> T cast."""
    k, n = codes.shape
    if policy == "per_tensor":
        S = np.full((k, n), s[0], np.float32)
        O = None if o is None else np.full((k, n), o[0], np.float32)
    elif policy == "per_channel":
        S = np.broadcast_to(s, (k, n))
        O = None if o is None else np.broadcast_to(o, (k, n))
    else:
        S = np.repeat(s, gs, axis=0)[:k]
        O = None if o is None else np.repeat(o, gs, axis=0)[:k]
    v = codes.astype(np.float32)
    t = (v + O) * S if O is not None else v * S
    return torch.from_numpy(t.astype(np.float32)).to(dtype)


def pin_wq_empty_k_is_bias_plus_x3(orc):
    """The page's empty-tensor case: with k = 0 the output is bias + x3."""
    rng = np.random.default_rng(71)
    x1 = torch.zeros((3, 0), dtype=torch.bfloat16)
    x2 = np.zeros((0, 8), np.int8)
    bias = _bf16(rng.standard_normal(8).tolist())
    x3 = _bf16(rng.standard_normal((3, 8)).tolist())
    sc = _bf16([0.5] * 8)
    out, mag, W = orc.weight_quant_matmul(x1, x2, sc, bias=bias, x3=x3)
    assert W.shape == (0, 8) and np.all(mag == 0)
    want = bias.double().numpy()[None, :] + x3.double().numpy()
    assert np.array_equal(out, want)


def pin_wq_identity_weight(orc):
    """x2 = identity, scale 1 per tensor, no offset: the output is x1 exactly
    (plus bias and x3)."""
    rng = np.random.default_rng(72)
    for mk in (_bf16, _f16):
        x1 = mk(rng.standard_normal((5, 64)).tolist())
        eye = np.eye(64, dtype=np.int8)
        out, _, _ = orc.weight_quant_matmul(x1, eye, mk([1.0]), policy="per_tensor")
        assert np.array_equal(out, x1.double().numpy())
        out, _, _ = orc.weight_quant_matmul(x1, ("int4", _pack_int4(eye)), mk([1.0]), policy="per_tensor")
        assert np.array_equal(out, x1.double().numpy())


def pin_wq_int4_nibbles_worked(orc):
    """int4 weights [1, 6] from bytes 0x7F 0x80 0x19: low nibble first,
    sign-extended: 0xF -> -1, 7, 0, 0x8 -> -8, 0x9 -> -7, 1.  Scale 1."""
    W = orc.weight_dequant(("int4", np.array([[0x7F, 0x80, 0x19]], np.uint8)), _bf16([1.0]),
                           policy="per_tensor")
    assert _bits_to_bf16_f32(W).tolist() == [[-1.0, 7.0, 0.0, -8.0, -7.0, 1.0]]
    Wt = orc.weight_dequant(("int4", np.array([[0x7F], [0x80], [0x19]], np.uint8)), _bf16([1.0]),
                            policy="per_tensor", transpose_x2=True)
    assert _bits_to_bf16_f32(Wt).tolist() == [[-1.0, 0.0, -7.0], [7.0, -8.0, 1.0]]


def pin_wq_dequant_matches_numpy(orc):
    """W equals numpy's float32 (x2 + offset) * scale cast to T by torch, for
    every policy, int8 and int4, with and without offset, both layouts and
    both dtypes (a short last group included)."""
    rng = np.random.default_rng(73)
    k, n = 96, 40
    for dtype in (torch.bfloat16, torch.float16):
        for policy, gs in (("per_tensor", 0), ("per_channel", 0), ("per_group", 64), ("per_group", 32)):
            for w in ("int8", "int4"):
                for off in (True, False):
                    for tr in (False, True):
                        x2, sc, of, codes, s, o = _wq_case(rng, k, n, policy, gs, dtype, w, off, tr)
                        W = orc.weight_dequant(x2, sc, of, policy, gs, tr)
                        ref = _numpy_dequant(codes, s, o, policy, gs, dtype)
                        assert np.array_equal(W, ref.view(torch.int16).numpy().view(np.uint16)), \
                            (dtype, policy, gs, w, off, tr)


def pin_wq_matmul_matches_numpy(orc):
    """out equals numpy's float64 x1 @ W + bias + x3 on the decoded values
    (to 1e-12 relative: the summation orders differ), and mag is
    |x1| @ |W|."""
    rng = np.random.default_rng(74)
    m, k, n = 7, 160, 24
    x2, sc, of, codes, s, o = _wq_case(rng, k, n, "per_group", 32, torch.bfloat16, "int4", True, False)
    x1 = _bf16(rng.standard_normal((m, k)).tolist())
    bias = _bf16(rng.standard_normal(n).tolist())
    x3 = _bf16(rng.standard_normal((m, n)).tolist())
    out, mag, W = orc.weight_quant_matmul(x1, x2, sc, of, "per_group", 32, bias=bias, x3=x3)
    Wd = _bits_to_bf16_f32(W).astype(np.float64)
    xd = x1.double().numpy()
    ref = xd @ Wd + bias.double().numpy()[None, :] + x3.double().numpy()
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12 * np.abs(xd) @ np.abs(Wd))
    assert np.allclose(mag, np.abs(xd) @ np.abs(Wd), rtol=1e-12)


def pin_wq_policy_reductions(orc):
    """Per group with gs >= k is per channel with the group row; per channel
    with a constant vector is per tensor; the transposed layout (weights and
    group parameters transposed together) gives the same W."""
    rng = np.random.default_rng(75)
    k, n = 64, 48
    codes = rng.integers(-128, 128, (k, n)).astype(np.int8)
    s = _bf16(rng.uniform(0.01, 0.1, (1, n)).tolist())
    o = _bf16(rng.uniform(-4, 4, (1, n)).tolist())
    a = orc.weight_dequant(codes, s, o, "per_group", 64)
    b = orc.weight_dequant(codes, s[0], o[0], "per_channel")
    assert np.array_equal(a, b)
    c = orc.weight_dequant(codes, _bf16([0.03] * n), _bf16([1.5] * n), "per_channel")
    d = orc.weight_dequant(codes, _bf16([0.03]), _bf16([1.5]), "per_tensor")
    assert np.array_equal(c, d)
    s4 = _bf16(rng.uniform(0.01, 0.1, (2, n)).tolist())
    e = orc.weight_dequant(codes, s4, None, "per_group", 32)
    f = orc.weight_dequant(codes.T.copy(), s4.t().contiguous(), None, "per_group", 32, transpose_x2=True)
    assert np.array_equal(e, f)


def pin_f64_to_half_rounding(orc):
    """binary64 -> bf16 / fp16 rounds once: it equals torch's cast for values
    that are binary32 already; 1 + 2^-8 + 2^-30 rounds up to 1 + 2^-7 in
    bf16 (a detour through binary32 would land on the tie and round to 1);
    numpy's float64 -> float16 cast agrees on random doubles."""
    rng = np.random.default_rng(76)
    a = (rng.standard_normal(4000) * np.exp2(rng.integers(-30, 30, 4000))).astype(np.float32).astype(np.float64)
    ref = torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(orc.f64_to_half(a, "bfloat16"), ref)
    x = np.array([1 + 2.0 ** -8 + 2.0 ** -30, 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8])
    got = _bits_to_bf16_f32(orc.f64_to_half(x, "bfloat16")).tolist()
    assert got == [1 + 2.0 ** -7, 1.0, 1 + 2.0 ** -6]
    d = rng.standard_normal(4000) * np.exp2(rng.integers(-26, 16, 4000))
    with np.errstate(over="ignore"):
        assert np.array_equal(orc.f64_to_half(d, "float16"), d.astype(np.float16).view(np.uint16))


# ---------------------------------------------------------------------------
# Element conversions against library routines
# ---------------------------------------------------------------------------

def _interesting_f32(rng, n):
    with np.errstate(over="ignore"):
        a = rng.standard_normal(n).astype(f32) * np.exp2(rng.integers(-140, 128, n)).astype(f32)
    bits = rng.integers(0, 2 ** 32, n, dtype=np.uint64).astype(np.uint32)
    ties = (bits & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    specials = np.array([0.0, -0.0, np.inf, -np.inf, 65504, 65519.99, 65520, 65536, 6.1e-5,
                         5.96e-8, 2.98e-8, 2.99e-8, 3.4e38, 1e-45, 448, 0.5, 1.5, 2.5], f32)
    return np.concatenate([a, bits.view(f32), ties.view(f32), specials])


def pin_conversions_against_libraries(orc):
    """bf16 rounding equals torch's float32 -> bfloat16 cast; fp16 rounding
    equals numpy's float32 -> float16 cast; widening of both equals torch's;
    the e4m3fn decode equals torch's float8_e4m3fn -> float32 for all 256
    codes (0x7E = 448, 0x01 = 2^-9, 0x08 = 2^-6, 0x7F / 0xFF NaN); the e5m2
    decode equals torch's float8_e5m2 and binary16's upper byte; e8m0 is
    2^(k - 127); e2m1 is the OCP table."""
    rng = np.random.default_rng(51)
    a = _interesting_f32(rng, 20000)
    fin = ~np.isnan(a)
    bf = orc.from_f32(a, "bfloat16")
    ref_bf = torch.from_numpy(a.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf[fin], ref_bf[fin])
    assert np.all(np.isnan(_bits_to_bf16_f32(bf[~fin])))
    h = orc.from_f32(a, "float16")
    with np.errstate(over="ignore"):
        ref_h = a.astype(np.float16).view(np.uint16)
    assert np.array_equal(h[fin], ref_h[fin])
    bits16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    w_bf = orc.to_f32(torch.from_numpy(bits16.view(np.int16).copy()).view(torch.bfloat16))
    ref = torch.from_numpy(bits16.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(w_bf), nan) and np.array_equal(w_bf[~nan], ref[~nan])
    w_h = orc.to_f32(bits16.view(np.float16))
    ref = bits16.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(w_h), nan) and np.array_equal(w_h[~nan], ref[~nan])
    codes = np.arange(256, dtype=np.uint8)
    e = orc.e4m3_to_f32(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(e), nan) and np.array_equal(e[~nan], ref[~nan])
    assert e[0x7E] == 448 and e[0x01] == 2.0 ** -9 and e[0x08] == 2.0 ** -6
    assert np.isnan(e[0x7F]) and np.isnan(e[0xFF])
    # e5m2 equals torch's float8_e5m2 decode and binary16's top byte.
    e5 = orc.bytes_to_f32(codes, "float8_e5m2")
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e5m2).float().numpy()
    ref16 = (codes.astype(np.uint16) << 8).view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(e5), nan) and np.array_equal(np.isnan(ref16), nan)
    assert np.array_equal(e5[~nan], ref[~nan]) and np.array_equal(e5[~nan], ref16[~nan])
    assert e5[0x7B] == 57344 and e5[0x01] == 2.0 ** -16 and e5[0x7C] == np.inf
    # e8m0: 2^(k - 127), 0xFF NaN (closed form).
    e8 = orc.bytes_to_f32(codes, "float8_e8m0")
    assert np.isnan(e8[255])
    assert np.array_equal(e8[:255].astype(np.float64), np.ldexp(1.0, np.arange(255) - 127))
    # e2m1: the OCP table, low nibble first.
    e2 = orc.bytes_to_f32(np.array([0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE], np.uint8),
                          "float4_e2m1x2")
    assert np.array_equal(e2, np.array(OCP_E2M1, np.float32))
    assert np.array_equal(np.signbit(e2), np.signbit(np.array(OCP_E2M1)))


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_") and callable(v)]
