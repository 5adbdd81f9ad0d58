"""Stream and graph semantics on the GPU.

* Every op runs on the stream it is given: on a side stream (ordered after
  the producer of its inputs) it gives bit-identical results to the same
  call on the default stream, whether the side stream is the current one or
  is passed explicitly.
* The execute calls enqueue kernels only (no allocation, no memset, no
  synchronization), so prepared calls can be captured in a HIP graph: each
  replay, with new inputs copied in eagerly and the program's own eager
  work and synchronizations between replays, equals an eager call on the
  same inputs, bit for bit.  The split-k matmul is included (its partial
  sums live in the prepared call's workspace), and so is the balanced
  decode matmul (direct-to-LDS staging, no workspace).
"""
import pytest
import torch

import int4_quantization_amd as dq
from int4_quantization_amd import dquant as D
from int4_quantization_amd import synth
from parity import DEV, announce

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _bits(t: torch.Tensor) -> torch.Tensor:
    t = t.contiguous()
    return t.view(torch.uint8) if t.numel() else t


def _same(a, b):
    for u, v in zip(a, b):
        if u is None:
            assert v is None
            continue
        assert u.shape == v.shape and u.dtype == v.dtype
        assert torch.equal(_bits(u), _bits(v))


def _to_dev(d):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def _op(name):
    """(inputs on the device, run(inputs, stream) -> outputs)."""
    if name == "dynamic_quant":
        inp = _to_dev(synth.dq_inputs(300, 7168, 901, smooth="vector"))
        return inp, lambda i, s: dq.dynamic_quant(i["x"], i["smooth"], None, False, "int4", stream=s)
    if name == "ada_layernorm_quant":
        inp = _to_dev(synth.ada_inputs(2, 40, 3072, 902))
        return inp, lambda i, s: dq.ada_layernorm_quant(i["x"], i["scale"], i["shift"], i["weight"], i["bias"],
                                                         i["smooth"], i["eps"], stream=s)
    if name == "antiquantize":
        inp = _to_dev(synth.aq_inputs(512, 1024, "per_group", 903))
        return inp, lambda i, s: (dq.antiquantize(i["src"], i["scale"], i["offset"], i["policy"], i["kdim"],
                                                  i["group_size"], stream=s),)
    if name == "mx_quantize":
        inp = _to_dev(synth.mx_inputs(256, 2048, 904))
        return inp, lambda i, s: dq.mx_quantize(i["x"], torch.float8_e4m3fn, 1, stream=s)
    if name in ("weight_quant_matmul_split_k", "weight_quant_matmul_balanced"):
        n = 512 if name.endswith("split_k") else 4096  # 4096: the balanced decode kernel
        inp = _to_dev(synth.wq_inputs(16, 8192, n, 905, weight="int4", group_size=128))
        return inp, lambda i, s: (dq.weight_quant_matmul(i["x1"], i["x2"], i["scale"], i["offset"],
                                                         i["group_size"], i["bias"], i["x3"],
                                                         i["transpose_x2"], i["weight"], stream=s),)
    raise KeyError(name)


OPS = ["dynamic_quant", "ada_layernorm_quant", "antiquantize", "mx_quantize", "weight_quant_matmul_split_k",
       "weight_quant_matmul_balanced"]


@pytest.mark.parametrize("name", OPS)
def test_side_stream_matches_default_stream(name):
    announce("side stream", name)
    inp, run = _op(name)
    ref = run(inp, None)
    torch.cuda.synchronize()
    side = torch.cuda.Stream(device=DEV)             # default priority
    side.wait_stream(torch.cuda.current_stream())    # inputs were produced on the default stream
    with torch.cuda.stream(side):
        current = run(inp, None)                     # the side stream is the current one
    explicit = run(inp, side)                        # passed explicitly from the default context
    raw = run(inp, side.cuda_stream)                 # as a raw handle
    torch.cuda.synchronize()
    _same(ref, current)
    _same(ref, explicit)
    _same(ref, raw)


def _prepared(name):
    """(static inputs, refresh(seed) writing new inputs in place, prepared
    call, static outputs)."""
    if name == "dynamic_quant":
        rows, n = 300, 7168
        inp = _to_dev(synth.dq_inputs(rows, n, 911, smooth="vector"))
        y = torch.empty(rows, n, dtype=torch.int8, device=DEV)
        scale = torch.empty(rows, dtype=torch.float32, device=DEV)
        call = D.prepare_dynamic_quant(inp["x"], inp["smooth"], None, True, y, scale, None, "int8")

        def refresh(seed):
            inp["x"].copy_(synth.dq_inputs(rows, n, seed, smooth="vector")["x"])
        return inp, refresh, call, (y, scale)
    m, k, n = 16, 8192, 512 if name.endswith("split_k") else 4096
    inp = _to_dev(synth.wq_inputs(m, k, n, 912, weight="int4", group_size=128))
    out = torch.empty(m, n, dtype=inp["x1"].dtype, device=DEV)
    call = D.prepare_weight_quant_matmul(inp["x1"], inp["x2"], inp["transpose_x2"], inp["scale"], inp["offset"],
                                         inp["group_size"], inp["bias"], inp["x3"], out, inp["weight"])

    def refresh(seed):
        inp["x1"].copy_(synth.wq_inputs(m, k, n, seed, weight="int4", group_size=128)["x1"])
    return inp, refresh, call, (out,)


@pytest.mark.parametrize("name", ["dynamic_quant", "weight_quant_matmul_split_k", "weight_quant_matmul_balanced"])
def test_graph_replay_matches_eager(name):
    announce("graph replay", name)
    inp, refresh, call, outs = _prepared(name)
    side = torch.cuda.Stream(device=DEV)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()   # warm-up: allocates the workspace (split-k) outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        call()
    torch.cuda.synchronize()
    for rep, seed in enumerate([921, 922, 923, 922]):
        refresh(seed)                         # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in outs]
        for o in outs:
            o.fill_(0)                        # eager work: the next eager call must write everything
        call()                                # eager call on the same inputs, default stream
        torch.cuda.synchronize()
        for g, e in zip(got, outs):
            assert torch.equal(_bits(g), _bits(e)), f"replay {rep} (seed {seed}) differs from eager"
