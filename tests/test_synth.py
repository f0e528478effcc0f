"""Pins for the seeded input generator (not part of the method's arithmetic)."""
import numpy as np
import pytest
import torch

import synth


def test_e4m3_rne_and_saturation_spot_values():
    """RNE ties to even and clamp-then-cast saturation at +-448."""
    x = torch.tensor([17.0, 19.0, 448.0, 1000.0, -1000.0, 2.0 ** -10, 0.0, -0.0, 1.0])
    b = synth.to_e4m3_bytes(x).tolist()
    # 17 -> 16 (0x58), 19 -> 20 (0x5A), 448 -> 0x7E, saturate +-1000 -> +-448,
    # 2^-10 rounds to 0 (smallest subnormal is 2^-9), -0 keeps its sign, 1.0 = 0x38
    assert b == [0x58, 0x5A, 0x7E, 0x7E, 0xFE, 0x00, 0x00, 0x80, 0x38]


def test_e4m3_cast_matches_float_decode():
    """Every finite E4M3 byte decodes to a float that casts back to itself."""
    allb = torch.arange(256, dtype=torch.uint8)
    vals = allb.view(torch.float8_e4m3fn).to(torch.float32)
    finite = torch.isfinite(vals)
    back = synth.to_e4m3_bytes(vals[finite])
    a = allb[finite]
    # -0 and +0 both map to themselves
    assert torch.equal(back, a)


def test_cms_alpha2_is_gaussian_with_variance_2gamma2():
    """Chambers-Mallows-Stuck at alpha = 2 gives N(0, 2 gamma^2) (closed form)."""
    g = torch.Generator().manual_seed(7)
    x = synth.alpha_stable(2.0, 400_000, g, "cpu", gamma=0.5).numpy()
    var = 2 * 0.5 ** 2
    assert abs(x.mean()) < 0.01
    assert abs(x.var() / var - 1) < 0.01
    k = ((x - x.mean()) ** 4).mean() / x.var() ** 2
    assert abs(k - 3.0) < 0.05


def test_cms_matches_scipy_levy_stable():
    """KS test of the sampler against scipy.stats.levy_stable (S1 parameterisation, beta = 0)."""
    from scipy import stats
    g = torch.Generator().manual_seed(11)
    x = synth.alpha_stable(1.7, 3000, g, "cpu", gamma=1.0).numpy()
    d, p = stats.kstest(x, stats.levy_stable(1.7, 0.0).cdf)
    assert p > 1e-3, (d, p)


def test_seeds_are_stable():
    assert synth.seed_of("llama70b", "q_proj", 0) == synth.seed_of("llama70b", "q_proj", 0)
    assert synth.seed_of("llama70b", "q_proj", 0) != synth.seed_of("llama70b", "k_proj", 0)
    a = synth.small_stable(1000, 1.8, 3)
    b = synth.small_stable(1000, 1.8, 3)
    assert np.array_equal(a, b)


def test_workload_shapes():
    assert sum(int(np.prod(s)) for _, s in synth.WORKLOADS["llama70b"]) == 855_638_016
    assert sum(int(np.prod(s)) for _, s in synth.WORKLOADS["llama8b"]) == 218_103_808
    assert sum(int(np.prod(s)) for _, s in synth.WORKLOADS["dit14b"]) == 351_272_960
    specs = synth.tensor_specs("moe256")
    assert len(specs) == 768
    assert sum(int(np.prod(s)) for _, s, _, _ in specs) == 11_274_289_152
    r = synth.moe_routing()
    assert len(set(r)) == 8 and all(0 <= e < 256 for e in r)
    assert all(1.5 <= synth.moe_alpha(e) <= 2.0 for e in range(256))


def test_dit_tile_scaling_hits_448_per_tile():
    x = synth.dit_tensor((256, 384), synth.seed_of("t", 1)).to(torch.int64)
    mags = (x & 0x7F)
    t = mags.reshape(2, 128, 3, 128).amax(dim=(1, 3))
    assert bool((t == 0x7E).all())


def test_fp8_weight_quantizer_scale_and_saturation():
    """Per-tensor max-abs scaling puts max|w| at 448 exactly; the cast is round-to-nearest-even."""
    import torch
    from lossless_entropy_coded_ecf8_amd.pipeline import fp8_e4m3_bytes
    w = torch.tensor([[0.0, -3.5, 7.0, 1.0], [2.0, -7.0, 0.125, 6.9]])
    q, scale = fp8_e4m3_bytes(w)
    assert q.dtype == torch.uint8 and q.shape == w.shape
    assert scale == 7.0 / 448.0
    f = q.view(torch.float8_e4m3fn).float()
    assert f.abs().max().item() == 448.0
    assert q[0, 2].item() == 0x7E and q[1, 1].item() == 0xFE          # +-448
    assert q[0, 0].item() == 0x00
    # 1.0 / scale = 64 exactly representable
    assert f[0, 3].item() == 64.0
    z, s0 = fp8_e4m3_bytes(torch.zeros(3, 3))
    assert s0 == 1.0 and int(z.sum()) == 0


def test_pipeline_argument_checks():
    import pytest as _pt
    from lossless_entropy_coded_ecf8_amd.pipeline import DecodePipeline
    with _pt.raises(ValueError):
        DecodePipeline([])
    with _pt.raises(ValueError):
        DecodePipeline([object()], slots=2, ahead=2)
    with _pt.raises(ValueError):
        DecodePipeline([object()], slots=0, ahead=0)


def test_float_weights_are_the_e4m3_tensors_before_rounding():
    for wl in ("gauss1m", "llama8b"):
        name, shape, kind, params = synth.tensor_specs(wl)[0]
        if wl == "llama8b":
            shape = (64, 128)                     # a small tensor of the same kind and seed
        x = synth.float_weights(wl, name, shape, kind, params)
        ref = synth.make_tensor(wl, name, shape, kind, params)
        assert torch.equal(synth.to_e4m3_bytes(synth.maxabs_scale(x.reshape(-1))).reshape(shape), ref)


def test_workload_as_bf16_and_e5m2():
    (n1, b), = list(synth.workload_tensors_as("gauss1m", "bf16"))
    (n2, e), = list(synth.workload_tensors_as("gauss1m", "e5m2"))
    assert b.dtype == torch.bfloat16 and e.dtype == torch.uint8 and b.shape == e.shape == (1024, 1024)
    assert float(e.view(torch.float8_e5m2).float().abs().max()) == 57344.0
