"""Every benchmark workload at its full size, element by element, through the
same C-ABI calls and launch configuration the benchmark times, against the
CPU oracle: DynamicQuant, AntiQuantize and mx block quantization bit-exact,
AdaLayerNorm-quant at the stated tolerance.  Also: two launches give identical bits.
The weight-quantized matmul workloads are checked on sampled rows in
test_gpu_weight_quant_matmul.py (the oracle's binary64 matmul is too slow for
every row)."""
import numpy as np
import pytest
import torch

import int4_quantization_amd as dq
from int4_quantization_amd import synth
from parity import (DEV, announce, check_ada_layernorm_quant, check_antiquantize, check_dynamic_quant,
                    check_mx_quantize)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.mark.parametrize("name", [w for w, (op, _) in synth.WORKLOADS.items() if op != "weight_quant_matmul"])
def test_full_size_parity(orc, name):
    announce("full size", name)
    op, build = synth.WORKLOADS[name]
    h = build()
    if op == "dynamic_quant":
        check_dynamic_quant(orc, h["x"], h["smooth"], h["group_index"], h["symmetric"], h["out"])
    elif op == "ada_layernorm_quant":
        _, _, nflip = check_ada_layernorm_quant(orc, h)
        print(f"{name}: {nflip} of {h['x'].numel()} codes differ by 1", flush=True)
    elif op == "mx_quantize":
        check_mx_quantize(orc, h["x"], h["elem"], h["axis"])
    else:
        check_antiquantize(orc, h["src"], h["scale"], h["offset"], h["policy"], h["kdim"],
                           h["group_size"], torch.bfloat16)


@pytest.mark.parametrize("name", ["dq_moe_asym_int4_bf16_32768x4096", "ada_ln_quant_bf16_4x4096x3072",
                                  "aq_per_group_fp8e4m3_16384x8192"])
def test_full_size_deterministic(name):
    announce("full size determinism", name)
    op, build = synth.WORKLOADS[name]
    h = build()
    if op == "dynamic_quant":
        args = [h["x"].to(DEV), h["smooth"].to(DEV), h["group_index"].to(DEV), h["symmetric"], h["out"]]
        a, b = dq.dynamic_quant(*args), dq.dynamic_quant(*args)
    elif op == "ada_layernorm_quant":
        args = [h[k].to(DEV) for k in ("x", "scale", "shift", "weight", "bias", "smooth")]
        a = dq.ada_layernorm_quant(*args, epsilon=h["eps"])
        b = dq.ada_layernorm_quant(*args, epsilon=h["eps"])
    else:
        args = [h["src"].to(DEV), h["scale"].to(DEV), h["offset"].to(DEV), h["policy"], h["kdim"],
                h["group_size"]]
        a, b = (dq.antiquantize(*args),), (dq.antiquantize(*args),)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        if u is None:
            continue
        assert torch.equal(u.view(torch.uint8), v.view(torch.uint8))
