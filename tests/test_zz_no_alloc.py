"""The allocation-free matmul entry point against the two-phase pair, on
the GPU through the C ABI.

dq_weight_quant_matmul_noalloc runs the same plan and kernels as
dq_weight_quant_matmul_get_workspace_size + dq_weight_quant_matmul, with the
split-k partial sums in the library's own per-GPU scratch array instead of
a caller workspace, so the outputs must be identical bit for bit.  Calls come
in a row on one stream, each later one smaller than the one before, so a
later call reads scratch that an earlier, larger call left behind.
"""
import ctypes

import numpy as np
import pytest
import torch

from int4_quantization_amd import dquant as D
from int4_quantization_amd import synth

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = torch.device("cuda:0")

# (m, k, n, weight, group size, seed): decode and prefill tiles that split k,
# largest first; the last two do not split.
CASES = [
    (200, 2048, 1024, "int4", 128, 71),  # LDS-tiled kernel, k split, parameter windows
    (8, 4096, 1024, "int4", 128, 72),    # decode kernel, k split
    (3, 2048, 512, "int8", 0, 73),       # smaller decode, k split
    (2, 1024, 4096, "int8", 64, 74),     # enough output tiles: no split
    (4, 8192, 4096, "int4", 128, 75),    # balanced decode kernel: one workgroup per compute unit, no split
]


def _device(q):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in q.items()}


def _two_phase(d, out):
    ws, ex = D.dq_weight_quant_matmul_get_workspace_size(d["x1"], d["x2"], d["transpose_x2"], d["scale"],
                                                         d["offset"], d["group_size"], d["bias"], d["x3"],
                                                         out, d["weight"])
    w = torch.empty(max(ws, 16), dtype=torch.uint8, device=DEV)
    D.dq_weight_quant_matmul(w if ws else None, ws, ex, torch.cuda.current_stream())
    return ws, w


def test_noalloc_matches_two_phase_calls_in_a_row():
    seen_split = 0
    keep = []
    for m, k, n, weight, gs, seed in CASES:
        print(f"noalloc case m={m} k={k} n={n} {weight} gs={gs}", flush=True)
        q = _device(synth.wq_inputs(m, k, n, seed, weight=weight, group_size=gs, x3=True))
        ref = torch.empty((m, n), dtype=q["x1"].dtype, device=DEV)
        ws, w = _two_phase(q, ref)
        keep.append(w)
        assert ws <= D.WQ_SCRATCH_BYTES
        seen_split += ws > 0
        out = torch.full((m, n), float("nan"), dtype=q["x1"].dtype, device=DEV)
        D.dq_weight_quant_matmul_noalloc(q["x1"], q["x2"], q["transpose_x2"], q["scale"], q["offset"],
                                         q["group_size"], q["bias"], q["x3"], out,
                                         torch.cuda.current_stream(), q["weight"])
        torch.cuda.synchronize()
        a = out.view(torch.int16).cpu().numpy()
        b = ref.view(torch.int16).cpu().numpy()
        assert np.array_equal(a, b), f"{int((a != b).sum())} of {a.size} outputs differ (m={m} n={n})"
    assert seen_split >= 3, "the cases must exercise the split-k scratch"


def test_noalloc_repeated_calls_reuse_scratch():
    """The same smaller call twice after a larger one gives the same bits."""
    outs = []
    for m, k, n, weight, gs, seed in (CASES[0], CASES[2], CASES[2]):
        q = _device(synth.wq_inputs(m, k, n, seed, weight=weight, group_size=gs, x3=True))
        out = torch.empty((m, n), dtype=q["x1"].dtype, device=DEV)
        D.dq_weight_quant_matmul_noalloc(q["x1"], q["x2"], q["transpose_x2"], q["scale"], q["offset"],
                                         q["group_size"], q["bias"], q["x3"], out, None, q["weight"])
        outs.append(out)
    torch.cuda.synchronize()
    assert torch.equal(outs[1].view(torch.int16), outs[2].view(torch.int16))
