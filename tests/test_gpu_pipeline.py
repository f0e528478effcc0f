"""Decode-on-use pipeline: ECF8Linear and DecodePipeline against resident FP8 weights.

Every decoded weight must equal the original E4M3 bytes exactly, so every
layer output must equal the output of the same FP8 GEMM on the original
weight bit for bit, whatever the pool size, look-ahead or decode grid.
"""
import numpy as np
import pytest
import torch

import synth
import lossless_entropy_coded_ecf8_amd as E
from lossless_entropy_coded_ecf8_amd import pipeline as P

pytestmark = pytest.mark.gpu

SHAPES = [(1024, 1024), (256, 1024), (256, 1024), (1024, 1024), (2816, 1024), (2816, 1024), (1024, 2816)]


def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def make_layers(d, shapes=SHAPES, seed=0):
    ws, layers = [], []
    for i, (o, k) in enumerate(shapes):
        w = torch.from_numpy(synth.small_stable(o * k, 1.8, seed * 100 + i)).view(o, k)
        ws.append(w.to(d))
        layers.append(E.ECF8Linear(w, scale=0.5 + 0.01 * i, device=d))
    return ws, layers


def make_inputs(d, layers, tokens, seed=1):
    g = torch.Generator(device="cpu").manual_seed(seed)
    xs, scs = [], []
    for l in layers:
        x = (torch.randn(tokens, l.in_features, generator=g) * 4).clamp(-448, 448).to(torch.float8_e4m3fn)
        xs.append(x.to(d))
        scs.append(torch.tensor(0.25, dtype=torch.float32, device=d))
    return xs, scs


def reference(ws, layers, xs, scs):
    return [P.linear_fp8(x, s, w, l.w_scale, l.bias) for w, l, x, s in zip(ws, layers, xs, scs)]


def test_ecf8_linear_decodes_exact_weight_and_output():
    d = dev()
    ws, layers = make_layers(d, SHAPES[:3])
    xs, scs = make_inputs(d, layers, 64)
    for w, l, x, s in zip(ws, layers, xs, scs):
        assert torch.equal(l.decoded_weight(), w)
        assert l.compressed_bytes() < w.numel()
        y = l(x, s)
        torch.cuda.synchronize()
        assert torch.equal(y, P.linear_fp8(x, s, w, l.w_scale))


def test_from_linear_round_trip():
    d = dev()
    torch.manual_seed(3)
    lin = torch.nn.Linear(512, 384, bias=True)
    l = E.ECF8Linear.from_linear(lin, device=d)
    q, scale = E.fp8_e4m3_bytes(lin.weight.detach())
    assert torch.equal(l.decoded_weight().cpu(), q)
    assert float(l.w_scale) == float(np.float32(scale))          # the scale is kept as float32
    assert torch.equal(l.bias.cpu(), lin.bias.detach())


@pytest.mark.parametrize("slots,ahead,workgroups", [(3, 2, None), (2, 1, None), (1, 0, None), (4, 3, 64),
                                                    (3, 1, 7)])
def test_pipeline_matches_resident_weights(slots, ahead, workgroups):
    d = dev()
    ws, layers = make_layers(d)
    xs, scs = make_inputs(d, layers, 96)
    ref = reference(ws, layers, xs, scs)
    pipe = E.DecodePipeline(layers, slots=slots, ahead=ahead, workgroups=workgroups)
    assert pipe.pool_bytes() == slots * ((max(l.numel for l in layers) + 255) // 256 * 256)
    torch.cuda.synchronize()
    for rep in range(3):                                     # the pool is reused across runs
        before = torch.cuda.memory_allocated(d)
        outs = pipe.run(xs, scs)
        torch.cuda.synchronize()
        grown = torch.cuda.memory_allocated(d) - before
        out_bytes = sum(o.numel() * o.element_size() for o in outs)
        assert grown <= out_bytes + (1 << 20), (rep, grown, out_bytes)   # no weight-sized allocation
        for i, (o, r) in enumerate(zip(outs, ref)):
            assert torch.equal(o, r), (rep, i)
        del outs


def test_pipeline_more_layers_than_slots_with_repeats():
    """14 layers over 3 slots: every slot is overwritten several times per run."""
    d = dev()
    ws, layers = make_layers(d)
    ws2, layers2 = ws + ws, layers + layers
    xs, scs = make_inputs(d, layers2, 32, seed=5)
    ref = reference(ws2, layers2, xs, scs)
    pipe = E.DecodePipeline(layers2, slots=3, ahead=2, workgroups=128)
    outs = pipe.run(xs, scs)
    torch.cuda.synchronize()
    for i, (o, r) in enumerate(zip(outs, ref)):
        assert torch.equal(o, r), i
