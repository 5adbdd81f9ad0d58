"""The C ABI without a GPU: the library loads, exports every entry point the
header declares, and phase 1 (validation, no HIP calls) returns the right
status for every rule it enforces.  No kernel is launched here."""
import ctypes
import os
import re

import pytest
import torch

from int4_quantization_amd import dquant as D

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(D.library_path):
        from int4_quantization_amd import build
        build.build(verbose=False)
    return D.library()


def desc(dtype, dims, ptr=0x10000):
    d = D.DqTensor()
    d.data = ptr
    d.dtype = dtype
    d.ndim = len(dims)
    for i, s in enumerate(dims):
        d.dims[i] = s
    return d


def ref(d):
    return None if d is None else ctypes.byref(d)


def dq_ws(lib, x, sm, gi, sym, y, sc, off):
    ws = ctypes.c_size_t(99)
    ex = ctypes.c_void_p(None)
    st = lib.dq_dynamic_quant_get_workspace_size(ref(x), ref(sm), ref(gi), sym, ref(y), ref(sc),
                                                 ref(off), ctypes.byref(ws), ctypes.byref(ex))
    if st == D.SUCCESS:
        assert ex.value and ws.value == 0
        lib.dq_executor_destroy(ex)
    else:
        assert ex.value is None
        assert lib.dq_get_last_error().decode() != ""
    return st


def test_exports_match_header(lib):
    header = open(os.path.join(ROOT, "include", "dquant.h")).read()
    declared = set(re.findall(r"^\s*(?:dq_status|void|const char\*)\s+(dq_\w+)\s*\(", header, re.M))
    assert declared == set(D.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_struct_layout_matches_header():
    assert ctypes.sizeof(D.DqTensor) == 80
    assert D.DqTensor.dims.offset == 16


# ---- DynamicQuant ------------------------------------------------------------

R, N = 6, 64


def good_dq():
    return dict(x=desc(D.BF16, [R, N]), sm=None, gi=None, sym=1, y=desc(D.I8, [R, N]),
                sc=desc(D.F32, [R]), off=None)


@pytest.mark.parametrize("change,status", [
    ({}, D.SUCCESS),
    ({"x": None}, D.ERR_NULLPTR),
    ({"y": None}, D.ERR_NULLPTR),
    ({"sc": None}, D.ERR_NULLPTR),
    ({"x": desc(D.BF16, [R, N], ptr=0)}, D.ERR_NULLPTR),
    ({"x": desc(D.F32, [R, N])}, D.ERR_DTYPE),
    ({"y": desc(D.F16, [R, N])}, D.ERR_DTYPE),
    ({"sc": desc(D.F16, [R])}, D.ERR_DTYPE),
    ({"x": desc(D.BF16, [R, 0]), "y": desc(D.I8, [R, 0])}, D.ERR_SHAPE),
    ({"y": desc(D.I8, [R, N + 1])}, D.ERR_SHAPE),
    ({"sc": desc(D.F32, [R + 1])}, D.ERR_SHAPE),
    ({"sc": desc(D.F32, [R, 1])}, D.ERR_SHAPE),
    ({"x": desc(D.BF16, [R, 7]), "y": desc(D.I4, [R, 7])}, D.ERR_SHAPE),       # INT4: even N
    ({"x": desc(D.BF16, [R, 12]), "y": desc(D.I32, [R, 1])}, D.ERR_SHAPE),     # INT32: N % 8
    ({"y": desc(D.I32, [R, N])}, D.ERR_SHAPE),                                 # INT32: [.., N/8]
    ({"y": desc(D.I32, [R, N // 8])}, D.SUCCESS),
    ({"y": desc(D.I4, [R, N])}, D.SUCCESS),
    ({"off": desc(D.F32, [R])}, D.ERR_PARAM),                                  # sym with offset
    ({"sym": 0}, D.ERR_NULLPTR),                                               # asym needs offset
    ({"sym": 0, "off": desc(D.F16, [R])}, D.ERR_DTYPE),
    ({"sym": 0, "off": desc(D.F32, [R + 2])}, D.ERR_SHAPE),
    ({"sym": 0, "off": desc(D.F32, [R])}, D.SUCCESS),
    ({"sm": desc(D.F32, [N])}, D.SUCCESS),
    ({"sm": desc(D.F16, [N])}, D.ERR_DTYPE),
    ({"sm": desc(D.F32, [N + 8])}, D.ERR_SHAPE),
    ({"gi": desc(D.I32, [4])}, D.ERR_SHAPE),                                   # gi needs smooth
    ({"gi": desc(D.I32, [4]), "sm": desc(D.F32, [4, N])}, D.SUCCESS),
    ({"gi": desc(D.I8, [4]), "sm": desc(D.F32, [4, N])}, D.ERR_DTYPE),
    ({"gi": desc(D.I32, [4]), "sm": desc(D.F32, [3, N])}, D.ERR_SHAPE),
    ({"gi": desc(D.I32, [0]), "sm": desc(D.F32, [0, N])}, D.ERR_SHAPE),
    ({"gi": desc(D.I32, [4]), "sm": desc(D.F32, [N])}, D.ERR_SHAPE),
    ({"x": desc(D.BF16, [0, N]), "y": desc(D.I8, [0, N]), "sc": desc(D.F32, [0])}, D.SUCCESS),
    ({"x": desc(D.F16, [2, 3, N]), "y": desc(D.I8, [2, 3, N]), "sc": desc(D.F32, [2, 3])}, D.SUCCESS),
    ({"x": desc(D.F16, [2, 3, N]), "y": desc(D.I8, [2, 3, N]), "sc": desc(D.F32, [6])}, D.ERR_SHAPE),
    ({"x": desc(D.BF16, [2**31, 8]), "y": desc(D.I8, [2**31, 8]), "sc": desc(D.F32, [2**31])}, D.ERR_SHAPE),
    ({"x": desc(D.BF16, [2**31 - 1, 8]), "y": desc(D.I8, [2**31 - 1, 8]), "sc": desc(D.F32, [2**31 - 1])},
     D.SUCCESS),
])
def test_dynamic_quant_validation(lib, change, status):
    a = good_dq()
    a.update(change)
    assert dq_ws(lib, a["x"], a["sm"], a["gi"], a["sym"], a["y"], a["sc"], a["off"]) == status


# ---- AdaLayerNorm-quant ------------------------------------------------------

B, S, H = 2, 3, 64


def good_ada():
    return dict(x=desc(D.BF16, [B, S, H]), sc=desc(D.BF16, [B, 1, H]), sh=desc(D.BF16, [B, 1, H]),
                w=desc(D.BF16, [H]), b=desc(D.BF16, [H]), sm=desc(D.F32, [H]), eps=1e-5,
                out=desc(D.I8, [B, S, H]), qs=desc(D.F32, [B, S]))


def ada_ws(lib, a):
    ws = ctypes.c_size_t(99)
    ex = ctypes.c_void_p(None)
    st = lib.dq_ada_layernorm_quant_get_workspace_size(
        ref(a["x"]), ref(a["sc"]), ref(a["sh"]), ref(a["w"]), ref(a["b"]), ref(a["sm"]), a["eps"],
        ref(a["out"]), ref(a["qs"]), ctypes.byref(ws), ctypes.byref(ex))
    if st == D.SUCCESS:
        assert ex.value and ws.value == 0
        lib.dq_executor_destroy(ex)
    return st


@pytest.mark.parametrize("change,status", [
    ({}, D.SUCCESS),
    ({"w": None, "b": None, "sm": None}, D.SUCCESS),
    ({"sc": desc(D.BF16, [B, H]), "sh": desc(D.BF16, [B, H])}, D.SUCCESS),
    ({"x": None}, D.ERR_NULLPTR),
    ({"sc": None}, D.ERR_NULLPTR),
    ({"out": None}, D.ERR_NULLPTR),
    ({"x": desc(D.F32, [B, S, H])}, D.ERR_DTYPE),
    ({"sc": desc(D.F16, [B, 1, H])}, D.ERR_DTYPE),
    ({"w": desc(D.F32, [H])}, D.ERR_DTYPE),
    ({"sm": desc(D.BF16, [H])}, D.ERR_DTYPE),
    ({"out": desc(D.I4, [B, S, H])}, D.ERR_DTYPE),
    ({"qs": desc(D.F16, [B, S])}, D.ERR_DTYPE),
    ({"x": desc(D.BF16, [B * S, H])}, D.ERR_SHAPE),
    ({"sc": desc(D.BF16, [B, 2, H])}, D.ERR_SHAPE),
    ({"sh": desc(D.BF16, [B + 1, 1, H])}, D.ERR_SHAPE),
    ({"w": desc(D.BF16, [H + 1])}, D.ERR_SHAPE),
    ({"sm": desc(D.F32, [2 * H])}, D.ERR_SHAPE),
    ({"out": desc(D.I8, [B, S, H + 8])}, D.ERR_SHAPE),
    ({"qs": desc(D.F32, [B * S])}, D.ERR_SHAPE),
    ({"x": desc(D.BF16, [B, S, 0]), "sc": desc(D.BF16, [B, 1, 0]), "sh": desc(D.BF16, [B, 1, 0]),
      "w": None, "b": None, "sm": None, "out": desc(D.I8, [B, S, 0])}, D.ERR_SHAPE),
    ({"eps": 0.0}, D.ERR_PARAM),
    ({"eps": -1.0}, D.ERR_PARAM),
    ({"eps": float("inf")}, D.ERR_PARAM),
    ({"eps": float("nan")}, D.ERR_PARAM),
    ({"x": desc(D.BF16, [2**16, 2**15, H]), "sc": desc(D.BF16, [2**16, 1, H]), "sh": desc(D.BF16, [2**16, 1, H]),
      "out": desc(D.I8, [2**16, 2**15, H]), "qs": desc(D.F32, [2**16, 2**15])}, D.ERR_SHAPE),   # B*S = 2^31
])
def test_ada_validation(lib, change, status):
    a = good_ada()
    a.update(change)
    assert ada_ws(lib, a) == status


# ---- AntiQuantize ------------------------------------------------------------

M, NN = 40, 256


def aq_ws(lib, src, sc, off, pol, kdim, gs, dst):
    ws = ctypes.c_size_t(99)
    ex = ctypes.c_void_p(None)
    st = lib.dq_antiquantize_get_workspace_size(ref(src), ref(sc), ref(off), pol, kdim, gs, ref(dst),
                                                ctypes.byref(ws), ctypes.byref(ex))
    if st == D.SUCCESS:
        assert ex.value and ws.value == 0
        lib.dq_executor_destroy(ex)
    return st


SRC_PTR, DST_PTR = 0x100000, 0x800000


@pytest.mark.parametrize("pol,kdim,gs,sshape,status", [
    (0, -1, 0, [1], D.SUCCESS),
    (0, 1, 0, [M], D.ERR_SHAPE),
    (1, 1, 0, [1, NN], D.SUCCESS),
    (1, 1, 0, [NN], D.SUCCESS),
    (1, 1, 0, [M, 1], D.ERR_SHAPE),
    (2, 1, 0, [M, 1], D.SUCCESS),
    (2, 1, 0, [1, NN], D.ERR_SHAPE),
    (3, 1, 128, [M, 2], D.SUCCESS),
    (3, 1, 96, [M, 3], D.SUCCESS),          # ceil(256 / 96) = 3, short last group
    (3, 1, 96, [M, 2], D.ERR_SHAPE),
    (3, 0, 32, [2, NN], D.SUCCESS),         # ceil(40 / 32) = 2
    (3, 0, 32, [M, 8], D.ERR_SHAPE),
    (3, 1, 0, [M, 2], D.ERR_PARAM),         # groupSize must be > 0
    (3, 1, 48, [M, 6], D.ERR_PARAM),        # and a multiple of 32
    (3, 2, 32, [M, 8], D.ERR_PARAM),        # kDim is 0 or 1
    (4, 1, 0, [1], D.ERR_PARAM),            # unknown policy
])
def test_antiquantize_policy_shapes(lib, pol, kdim, gs, sshape, status):
    src = desc(D.I8, [M, NN], SRC_PTR)
    dst = desc(D.BF16, [M, NN], DST_PTR)
    sc = desc(D.F32, sshape, 0x20000)
    off = desc(D.F32, sshape, 0x40000)
    assert aq_ws(lib, src, sc, off, pol, kdim, gs, dst) == status
    if status == D.SUCCESS:
        assert aq_ws(lib, src, sc, None, pol, kdim, gs, dst) == D.SUCCESS


@pytest.mark.parametrize("src,dst,off,status", [
    (desc(D.I8, [M, NN], SRC_PTR), desc(D.F16, [M, NN], DST_PTR), None, D.SUCCESS),
    (desc(D.F8E4M3, [M, NN], SRC_PTR), desc(D.BF16, [M, NN], DST_PTR), None, D.SUCCESS),
    (desc(D.I8, [M, NN], SRC_PTR), desc(D.F32, [M, NN], DST_PTR), None, D.SUCCESS),
    (desc(D.F16, [M, NN], SRC_PTR), desc(D.BF16, [M, NN], DST_PTR), None, D.ERR_DTYPE),
    (desc(D.I8, [M, NN], SRC_PTR), desc(D.I8, [M, NN], DST_PTR), None, D.ERR_DTYPE),
    (desc(D.I8, [M, NN], SRC_PTR), desc(D.BF16, [M, NN], DST_PTR), desc(D.F16, [1], 0x40000), D.ERR_DTYPE),
    (desc(D.I8, [M, NN], SRC_PTR), desc(D.BF16, [M, NN], DST_PTR), desc(D.F32, [2], 0x40000), D.ERR_SHAPE),
    (desc(D.I8, [2, M, NN], SRC_PTR), desc(D.BF16, [2, M, NN], DST_PTR), None, D.ERR_SHAPE),
    (desc(D.I8, [M, NN], SRC_PTR), desc(D.BF16, [M, NN + 32], DST_PTR), None, D.ERR_SHAPE),
    (desc(D.I8, [M, 48], SRC_PTR), desc(D.BF16, [M, 48], DST_PTR), None, D.ERR_ALIGN),   # 48 B rows
    (desc(D.I8, [M, NN], SRC_PTR + 8), desc(D.BF16, [M, NN], DST_PTR), None, D.ERR_ALIGN),
    (desc(D.I8, [M, NN], SRC_PTR), desc(D.BF16, [M, NN], SRC_PTR + 64), None, D.ERR_OVERLAP),
    (desc(D.I8, [M, NN], SRC_PTR), desc(D.BF16, [M, NN], SRC_PTR - 2 * M * NN + 16), None, D.ERR_OVERLAP),
    (desc(D.I8, [0, NN], SRC_PTR), desc(D.BF16, [0, NN], DST_PTR), None, D.SUCCESS),
    (desc(D.I8, [2**31, 32], SRC_PTR), desc(D.BF16, [2**31, 32], DST_PTR), None, D.ERR_SHAPE),  # rows
])
def test_antiquantize_types_alignment_overlap(lib, src, dst, off, status):
    sc = desc(D.F32, [1], 0x20000)
    assert aq_ws(lib, src, sc, off, 0, -1, 0, dst) == status


@pytest.mark.parametrize("src,sc,off,pol,kdim,gs,dst,status", [
    # b8 sources with fp16 / bf16 parameters (表3), and e5m2
    (D.F8E5M2, (D.F32, [1]), None, 0, -1, 0, D.BF16, D.SUCCESS),
    (D.F8E5M2, (D.F16, [1, NN]), (D.F16, [1, NN]), 1, 1, 0, D.F16, D.SUCCESS),
    (D.I8, (D.BF16, [M, 1]), (D.BF16, [M, 1]), 2, 1, 0, D.F32, D.SUCCESS),
    (D.I8, (D.F16, [1]), (D.F32, [1]), 0, -1, 0, D.BF16, D.ERR_DTYPE),      # offset dtype != scale
    (D.I8, (D.E8M0, [M, NN // 32]), None, 3, 1, 32, D.BF16, D.ERR_DTYPE),   # e8m0 is for fp4 only
    # the float4 case: PER_GROUP, e8m0 scale, no offset, bf16 / fp16 dst
    (D.F4E2M1, (D.E8M0, [M, NN // 32]), None, 3, 1, 32, D.BF16, D.SUCCESS),
    (D.F4E2M1, (D.E8M0, [2, NN]), None, 3, 0, 32, D.F16, D.SUCCESS),
    (D.F4E2M1, (D.E8M0, [M, NN // 32]), (D.E8M0, [M, NN // 32]), 3, 1, 32, D.BF16, D.ERR_DTYPE),
    (D.F4E2M1, (D.F32, [M, NN // 32]), None, 3, 1, 32, D.BF16, D.ERR_DTYPE),
    (D.F4E2M1, (D.E8M0, [M, NN // 32]), None, 3, 1, 32, D.F32, D.ERR_DTYPE),
    (D.F4E2M1, (D.E8M0, [M, 1]), None, 2, 1, 0, D.BF16, D.ERR_PARAM),       # PER_TOKEN
    (D.F4E2M1, (D.E8M0, [1]), None, 0, -1, 0, D.BF16, D.ERR_PARAM),         # PER_TENSOR
])
def test_antiquantize_new_types(lib, src, sc, off, pol, kdim, gs, dst, status):
    s = desc(src, [M, NN], SRC_PTR)
    d = desc(dst, [M, NN], DST_PTR)
    scd = desc(sc[0], sc[1], 0x20000)
    ofd = None if off is None else desc(off[0], off[1], 0x40000)
    assert aq_ws(lib, s, scd, ofd, pol, kdim, gs, d) == status


def test_antiquantize_float4_shape_and_alignment(lib):
    """fp4: n even (SHAPE) and n/2 bytes per row a multiple of 32 (ALIGN);
    kDim = 0 e8m0 scales need 8-byte alignment."""
    e8 = lambda shape, ptr=0x20000: desc(D.E8M0, shape, ptr)
    assert aq_ws(lib, desc(D.F4E2M1, [M, 65], SRC_PTR), e8([M, 3]), None, 3, 1, 32,
                 desc(D.BF16, [M, 65], DST_PTR)) == D.ERR_SHAPE
    assert aq_ws(lib, desc(D.F4E2M1, [M, 32], SRC_PTR), e8([M, 1]), None, 3, 1, 32,
                 desc(D.BF16, [M, 32], DST_PTR)) == D.ERR_ALIGN
    assert aq_ws(lib, desc(D.F4E2M1, [M, 64], SRC_PTR), e8([M, 2]), None, 3, 1, 32,
                 desc(D.BF16, [M, 64], DST_PTR)) == D.SUCCESS
    assert aq_ws(lib, desc(D.F4E2M1, [M, NN], SRC_PTR), e8([2, NN], 0x20008), None, 3, 0, 32,
                 desc(D.BF16, [M, NN], DST_PTR)) == D.SUCCESS
    assert aq_ws(lib, desc(D.F4E2M1, [M, NN], SRC_PTR), e8([2, NN], 0x20004), None, 3, 0, 32,
                 desc(D.BF16, [M, NN], DST_PTR)) == D.ERR_ALIGN


def test_antiquantize_channel_params_alignment(lib):
    src = desc(D.I8, [M, NN], SRC_PTR)
    dst = desc(D.BF16, [M, NN], DST_PTR)
    assert aq_ws(lib, src, desc(D.F32, [1, NN], 0x20004), None, 1, 1, 0, dst) == D.ERR_ALIGN
    assert aq_ws(lib, src, desc(D.F32, [M, 1], 0x20004), None, 2, 1, 0, dst) == D.SUCCESS


# ---- mx block quantization ----------------------------------------------------

def mx_ws(lib, x, axis, y, sc):
    ws = ctypes.c_size_t(99)
    ex = ctypes.c_void_p(None)
    st = lib.dq_mx_quantize_get_workspace_size(ref(x), axis, ref(y), ref(sc), ctypes.byref(ws),
                                               ctypes.byref(ex))
    if st == D.SUCCESS:
        assert ex.value and ws.value == 0
        lib.dq_executor_destroy(ex)
    else:
        assert ex.value is None
        assert lib.dq_get_last_error().decode() != ""
    return st


X_PTR, Y_PTR, S_PTR = 0x100000, 0x900000, 0xF00000


@pytest.mark.parametrize("xdt,ydt,sdt,shape,axis,sshape,status", [
    (D.BF16, D.F8E4M3, D.E8M0, [4, 64], 1, [4, 2], D.SUCCESS),
    (D.F16, D.F8E5M2, D.E8M0, [4, 64], 1, [4, 2], D.SUCCESS),
    (D.BF16, D.F4E2M1, D.E8M0, [4, 64], 1, [4, 2], D.SUCCESS),
    (D.BF16, D.F8E4M3, D.E8M0, [4, 70], 1, [4, 3], D.SUCCESS),      # short last block
    (D.BF16, D.F8E4M3, D.E8M0, [40, 6], 0, [2, 6], D.SUCCESS),      # axis 0
    (D.BF16, D.F8E4M3, D.E8M0, [0, 64], 1, [0, 2], D.SUCCESS),      # no rows
    (D.BF16, D.F4E2M1, D.E8M0, [4, 65], 1, [4, 3], D.ERR_SHAPE),    # fp4 needs even n
    (D.BF16, D.F8E4M3, D.E8M0, [4, 64], 1, [4, 3], D.ERR_SHAPE),
    (D.BF16, D.F8E4M3, D.E8M0, [40, 6], 0, [1, 6], D.ERR_SHAPE),
    (D.BF16, D.F8E4M3, D.E8M0, [4, 0], 1, [4, 0], D.ERR_SHAPE),
    (D.BF16, D.F8E4M3, D.E8M0, [4, 64], 2, [4, 2], D.ERR_PARAM),
    (D.F32, D.F8E4M3, D.E8M0, [4, 64], 1, [4, 2], D.ERR_DTYPE),
    (D.BF16, D.I8, D.E8M0, [4, 64], 1, [4, 2], D.ERR_DTYPE),
    (D.BF16, D.F8E4M3, D.F32, [4, 64], 1, [4, 2], D.ERR_DTYPE),
])
def test_mx_quantize_validation(lib, xdt, ydt, sdt, shape, axis, sshape, status):
    assert mx_ws(lib, desc(xdt, shape, X_PTR), axis, desc(ydt, shape, Y_PTR),
                 desc(sdt, sshape, S_PTR)) == status


def test_mx_quantize_rank_overlap_and_nulls(lib):
    x = desc(D.BF16, [4, 64], X_PTR)
    y = desc(D.F8E4M3, [4, 64], Y_PTR)
    s = desc(D.E8M0, [4, 2], S_PTR)
    assert mx_ws(lib, desc(D.BF16, [256], X_PTR), 1, desc(D.F8E4M3, [256], Y_PTR),
                 desc(D.E8M0, [8], S_PTR)) == D.ERR_SHAPE
    assert mx_ws(lib, x, 1, desc(D.F8E4M3, [4, 64], X_PTR + 100), s) == D.ERR_OVERLAP
    assert mx_ws(lib, x, 1, y, desc(D.E8M0, [4, 2], Y_PTR + 255)) == D.ERR_OVERLAP
    assert mx_ws(lib, x, 1, y, desc(D.E8M0, [4, 2], Y_PTR + 256)) == D.SUCCESS
    assert mx_ws(lib, x, 1, desc(D.F8E4M3, [4, 64], 0), s) == D.ERR_NULLPTR
    assert mx_ws(lib, None, 1, y, s) == D.ERR_NULLPTR
    assert lib.dq_mx_quantize(None, 0, None, None) == D.ERR_NULLPTR


def test_mx_binding_shapes():
    assert D.mx_scale_shape(5, 70, 1) == (5, 3)
    assert D.mx_scale_shape(70, 5, 0) == (3, 5)


# ---- weight-quantized matmul ----------------------------------------------------

def wq_ws(lib, x1, x2, trans, sc, of, gs, bias, x3, out, keep=False):
    ws = ctypes.c_size_t(99)
    ex = ctypes.c_void_p(None)
    st = lib.dq_weight_quant_matmul_get_workspace_size(ref(x1), ref(x2), trans, ref(sc), ref(of), gs, ref(bias),
                                                       ref(x3), ref(out), ctypes.byref(ws), ctypes.byref(ex))
    if st == D.SUCCESS:
        assert ex.value
        if keep:
            return st, ws.value, ex
        lib.dq_executor_destroy(ex)
    else:
        assert ex.value is None
        assert lib.dq_get_last_error().decode() != ""
    return st


A1, A2, A3, A4 = 0x1000000, 0x3000000, 0x5000000, 0x7000000


@pytest.mark.parametrize("xdt,wdt,trans,sshape,gs,status", [
    (D.BF16, D.I8, 1, [64], 0, D.SUCCESS),                 # per channel, [n, k] weights
    (D.BF16, D.I8, 1, [1], 0, D.SUCCESS),                  # per tensor
    (D.F16, D.I4, 1, [64, 2], 128, D.SUCCESS),             # per group, transposed params
    (D.BF16, D.I4, 0, [2, 64], 128, D.SUCCESS),            # per group, [k, n] weights
    (D.BF16, D.I8, 1, [2, 64], 128, D.ERR_SHAPE),          # group params not transposed with x2
    (D.BF16, D.I8, 1, [64, 2], 100, D.ERR_PARAM),          # group size not a multiple of 32
    (D.BF16, D.I8, 1, [64, 8], -32, D.ERR_PARAM),
    (D.BF16, D.I8, 1, [7], 0, D.ERR_SHAPE),
    (D.BF16, D.F32, 1, [64], 0, D.ERR_DTYPE),
    (D.F32, D.I8, 1, [64], 0, D.ERR_DTYPE),
])
def test_wq_validation(lib, xdt, wdt, trans, sshape, gs, status):
    m, k, n = 16, 256, 64
    x1 = desc(xdt, [m, k], A1)
    x2 = desc(wdt, [n, k] if trans else [k, n], A2)
    sc = desc(xdt if xdt in (D.BF16, D.F16) else D.BF16, sshape, A3)
    out = desc(xdt, [m, n], A4)
    assert wq_ws(lib, x1, x2, trans, sc, None, gs, None, None, out) == status


def test_wq_shapes_dtypes_overlap(lib):
    m, k, n = 16, 256, 64
    x1 = desc(D.BF16, [m, k], A1)
    x2 = desc(D.I8, [n, k], A2)
    sc = desc(D.BF16, [n], A3)
    out = desc(D.BF16, [m, n], A4)
    assert wq_ws(lib, x1, desc(D.I8, [n, k + 32], A2), 1, sc, None, 0, None, None, out) == D.ERR_SHAPE
    assert wq_ws(lib, x1, x2, 1, desc(D.F16, [n], A3), None, 0, None, None, out) == D.ERR_DTYPE
    assert wq_ws(lib, x1, x2, 1, sc, desc(D.BF16, [1], A3 + 0x1000), 0, None, None, out) == D.ERR_SHAPE
    assert wq_ws(lib, x1, x2, 1, sc, None, 0, desc(D.BF16, [n + 1], A3 + 0x2000), None, out) == D.ERR_SHAPE
    assert wq_ws(lib, x1, x2, 1, sc, None, 0, None, desc(D.BF16, [m, n + 1], A3 + 0x4000), out) == D.ERR_SHAPE
    assert wq_ws(lib, x1, x2, 1, sc, None, 0, None, None, desc(D.BF16, [m, n], A1 + 64)) == D.ERR_OVERLAP
    assert wq_ws(lib, x1, desc(D.I4, [n, 63], A2), 1, sc, None, 0, None, None, out) == D.ERR_SHAPE
    big = desc(D.I8, [70000, k], A2)
    assert wq_ws(lib, x1, big, 1, desc(D.BF16, [70000], A3), None, 0, None, None,
                 desc(D.BF16, [m, 70000], A4)) == D.ERR_SHAPE
    # 3-D x1 and the empty-k case
    assert wq_ws(lib, desc(D.BF16, [2, 8, k], A1), x2, 1, sc, None, 0, None, None,
                 desc(D.BF16, [2, 8, n], A4)) == D.SUCCESS
    assert wq_ws(lib, desc(D.BF16, [m, 0], A1), desc(D.I8, [n, 0], A2), 1, sc, None, 0, None, None,
                 out) == D.SUCCESS


def test_wq_split_k_workspace(lib):
    """Few output tiles ask for a workspace of binary32 partial sums; executing
    without it fails before any launch."""
    m, k, n = 16, 8192, 256
    st, ws, ex = wq_ws(lib, desc(D.BF16, [m, k], A1), desc(D.I8, [n, k], A2), 1, desc(D.BF16, [n], A3), None, 0,
                       None, None, desc(D.BF16, [m, n], A4), keep=True)
    assert st == D.SUCCESS and ws > 0 and ws % (m * n * 4) == 0
    assert lib.dq_weight_quant_matmul(None, 0, ex, None) == D.ERR_WORKSPACE
    n2 = 8192  # enough output tiles: no split, no workspace
    st, ws2, ex = wq_ws(lib, desc(D.BF16, [4096, k], A1), desc(D.I8, [n2, k], A2), 1, desc(D.BF16, [n2], 0x9000000),
                        None, 0, None, None, desc(D.BF16, [4096, n2], 0x10000000), keep=True)
    assert st == D.SUCCESS and ws2 == 0
    lib.dq_executor_destroy(ex)


def test_wq_balanced_plan(lib):
    """int4 in groups of 128 with at most 16 rows, k a multiple of 8192 and n
    a multiple of 4096 (up to 7 * 4096) plan the balanced decode kernel: one
    workgroup per compute unit and no k split, so no workspace, where the
    per-wave decode kernel would split k over its few output tiles."""
    def plan_ws(m, k, n, wdt=D.I4, gs=128):
        sshape = [n, -(-k // gs)] if gs else [n]
        # addresses 256 MB apart: the weights reach 117 MB
        st, ws, ex = wq_ws(lib, desc(D.BF16, [m, k], 0x1000000), desc(wdt, [n, k], 0x10000000), 1,
                           desc(D.BF16, sshape, 0x20000000), desc(D.BF16, sshape, 0x30000000), gs, None, None,
                           desc(D.BF16, [m, n], 0x40000000), keep=True)
        assert st == D.SUCCESS
        lib.dq_executor_destroy(ex)
        return ws
    assert plan_ws(16, 8192, 4096) == 0
    assert plan_ws(1, 16384, 8192) == 0
    assert plan_ws(16, 8192, 7 * 4096) == 0
    assert plan_ws(16, 4096, 4096) > 0         # k not whole runs of 8192: the decode kernel, split
    assert plan_ws(16, 8192, 4096 + 64) > 0    # n not a multiple of 4096
    assert plan_ws(16, 8192, 4096, gs=64) > 0  # groups of 64
    assert plan_ws(16, 8192, 4096, wdt=D.I8) > 0


# ---- execute-phase errors that never reach the device -------------------------

def test_execute_null_executor(lib):
    for fn in (lib.dq_dynamic_quant, lib.dq_ada_layernorm_quant, lib.dq_antiquantize, lib.dq_mx_quantize,
               lib.dq_weight_quant_matmul):
        assert fn(None, 0, None, None) == D.ERR_NULLPTR


def test_execute_wrong_executor_kind(lib):
    a = good_dq()
    ws = ctypes.c_size_t(0)
    ex = ctypes.c_void_p(None)
    st = lib.dq_dynamic_quant_get_workspace_size(ref(a["x"]), None, None, 1, ref(a["y"]), ref(a["sc"]),
                                                 None, ctypes.byref(ws), ctypes.byref(ex))
    assert st == D.SUCCESS
    # consumed (freed) even though it fails
    assert lib.dq_antiquantize(None, 0, ex, None) == D.ERR_PARAM
    assert "dq_antiquantize_get_workspace_size" in lib.dq_get_last_error().decode()


def test_copy_probe_validation(lib):
    assert lib.dq_copy_probe(0x1000, 0x2001, 64, None) == D.ERR_ALIGN
    assert lib.dq_copy_probe(0x1000, 0x2000, 60, None) == D.ERR_ALIGN
    assert lib.dq_copy_probe(0x1000, 0x1010, 64, None) == D.ERR_OVERLAP
    assert lib.dq_copy_probe(None, 0x2000, 64, None) == D.ERR_NULLPTR
    assert lib.dq_copy_probe(0x1000, 0x2000, 0, None) == D.SUCCESS


def test_python_binding_raises_without_gpu_launch(lib):
    # empty tensors: no pointer, so the binding passes them on from the host
    x = torch.zeros(0, 7, dtype=torch.bfloat16)
    with pytest.raises(D.DquantError) as e:
        D.dq_dynamic_quant_get_workspace_size(x, None, None, True, torch.zeros(0, 3, dtype=torch.uint8),
                                              torch.zeros(0), None, "int4")
    assert e.value.status == D.ERR_SHAPE
    assert "even" in str(e.value)


def test_binding_rejects_host_tensors(lib):
    """Host memory never reaches a kernel: the binding refuses CPU tensors
    (empty ones carry no pointer and pass) before any C call."""
    import int4_quantization_amd as dq
    x = torch.randn(4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU memory"):
        dq.dynamic_quant(x)
    with pytest.raises(ValueError, match="GPU memory"):
        dq.mx_quantize(x)
    with pytest.raises(ValueError, match="GPU memory"):
        dq.antiquantize(torch.zeros(4, 64, dtype=torch.int8), torch.ones(1))
    with pytest.raises(ValueError, match="GPU memory"):
        dq.weight_quant_matmul(x, torch.zeros(32, 64, dtype=torch.int8), torch.ones(32, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="on one GPU"):
        D.dq_copy_probe(torch.empty(16, dtype=torch.uint8), torch.empty(16, dtype=torch.uint8))
    assert D.tensor_desc(torch.empty(0, 64)).data is None


def test_binding_rejects_mixed_devices():
    with pytest.raises(ValueError, match="one device"):
        D._one_device(torch.empty(2, device="meta"), torch.empty(2))
    assert D._one_device(torch.empty(0), None, torch.empty(3)) == torch.device("cpu")


def test_binding_rejects_strided_tensors():
    """Descriptors describe dense row-major memory only: a transposed or
    sliced view raises before any C call instead of being read as if
    dense."""
    base = torch.zeros(8, 64, dtype=torch.bfloat16)
    for view in (base.t(), base[:, ::2], base[:, 1:]):
        with pytest.raises(ValueError, match="dense row-major"):
            D.tensor_desc(view)
    with pytest.raises(ValueError, match="GPU memory"):  # a row slice is dense: only its memory is refused
        D.tensor_desc(base[2:5])


# ---- allocation-free matmul ----------------------------------------------------

def _wq_noalloc(lib, m, k, n, x3=False, gs=0, w_dtype=None):
    x1 = desc(D.BF16, [m, k], 0x100000)
    x2 = desc(w_dtype or D.I8, [n, k], 0x40000000)
    sc = desc(D.BF16, [n, -(-k // gs)] if gs else [n], 0x80000000)
    out = desc(D.BF16, [m, n], 0xC0000000)
    x3d = desc(D.BF16, [m, n], 0xE0000000) if x3 else None
    return lib.dq_weight_quant_matmul_noalloc(ref(x1), ref(x2), 1, ref(sc), None, gs, None,
                                              ref(x3d) if x3d else None, ref(out), None)


def test_noalloc_validation_without_gpu(lib):
    """Validation and the scratch-size limit are host-side: they answer
    without touching a GPU (the scratch address is looked up only for a
    call that launches)."""
    assert lib.dq_weight_quant_matmul_noalloc(None, None, 1, None, None, 0, None, None, None, None) == D.ERR_NULLPTR
    x1 = desc(D.F32, [4, 128], 0x100000)
    x2 = desc(D.I8, [64, 128], 0x40000000)
    sc = desc(D.BF16, [64], 0x80000000)
    out = desc(D.BF16, [4, 64], 0xC0000000)
    assert lib.dq_weight_quant_matmul_noalloc(ref(x1), ref(x2), 1, ref(sc), None, 0, None, None, ref(out),
                                              None) == D.ERR_DTYPE
    # 384 x 4096 output, k 4096: 96 tiles of 128 x 128, split 6 ways -> 6 * 384 * 4096 * 4 bytes > 32 MiB.
    assert _wq_noalloc(lib, 384, 4096, 4096) == D.ERR_WORKSPACE
    assert "scratch" in lib.dq_get_last_error().decode()
    # m == 0 launches nothing.
    assert _wq_noalloc(lib, 0, 4096, 4096) == D.SUCCESS
