"""Seeded synthetic FP8 E4M3 weight tensors.

This module only makes inputs: it holds none of the ECF8 coding arithmetic and
is shared by the oracle-side tests and the GPU-side tests / benchmark.

Weight model (ECF8 blog, codearts.csdn.net, §2.1): trained weights follow a
symmetric alpha-stable law S_alpha(beta=0, gamma, delta=0) with alpha in
[1.5, 2.0].  Samples come from the Chambers-Mallows-Stuck (1976) method; the
values are scaled so that max|w| maps to 448 (the E4M3 maximum) and cast to
FP8 E4M3 with round-to-nearest-even after clamping to +-448 (saturation).
The pages measure trained checkpoints (Llama3-70B, DeepSeek-R1, Wan2.2, ...);
these seeded tensors with the same shapes and alpha range stand in for them.

Workloads (shapes follow the public model configurations):
  gauss1m   one 1024x1024 tensor, w ~ N(0, 0.02)
  llama8b   Llama-3-8B attention + MLP projections, alpha = 1.8, gamma = 0.01
  llama70b  Llama-3-70B transformer block, alpha = 1.9
  dit14b    14B-DiT block (hidden 5120), alpha = 1.5 plus 2% N(0, 0.2)
            outliers, per-128x128-tile scaling
  moe256    256 experts x (gate, up 7168x2048; down 2048x7168),
            alpha ~ U[1.5, 2.0] per expert; 8 experts chosen by a seeded
            uniform draw without replacement
"""
from __future__ import annotations

import hashlib
import math

import numpy as np
import torch

E4M3_MAX = 448.0

WORKLOADS = {
    "gauss1m": [("w", (1024, 1024))],
    "llama8b": [("q_proj", (4096, 4096)), ("k_proj", (4096, 1024)), ("v_proj", (4096, 1024)),
                ("o_proj", (4096, 4096)), ("gate_proj", (4096, 14336)), ("up_proj", (4096, 14336)),
                ("down_proj", (14336, 4096))],
    "llama70b": [("q_proj", (8192, 8192)), ("k_proj", (8192, 1024)), ("v_proj", (8192, 1024)),
                 ("o_proj", (8192, 8192)), ("gate_proj", (8192, 28672)), ("up_proj", (8192, 28672)),
                 ("down_proj", (28672, 8192))],
    "dit14b": [("self_q", (5120, 5120)), ("self_k", (5120, 5120)), ("self_v", (5120, 5120)),
               ("self_o", (5120, 5120)), ("cross_q", (5120, 5120)), ("cross_k", (5120, 5120)),
               ("cross_v", (5120, 5120)), ("cross_o", (5120, 5120)), ("ffn_up", (5120, 13824)),
               ("ffn_down", (13824, 5120))],
}
MOE_EXPERTS = 256
MOE_TENSORS = [("gate_proj", (7168, 2048)), ("up_proj", (7168, 2048)), ("down_proj", (2048, 7168))]
MOE_TOPK = 8

ALPHA = {"llama8b": 1.8, "llama70b": 1.9, "dit14b": 1.5}
GAMMA = 0.01  # scale of the alpha-stable law (cancels under max-abs scaling)


def seed_of(*parts) -> int:
    """Stable 63-bit seed from a tuple of names / numbers (independent of PYTHONHASHSEED)."""
    h = hashlib.sha256("/".join(str(p) for p in parts).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def alpha_stable(alpha: float, numel: int, gen: torch.Generator, device, gamma: float = 1.0) -> torch.Tensor:
    """Chambers-Mallows-Stuck sampler for S_alpha(beta=0, gamma, 0), computed in fp64."""
    eps = 1e-12
    u = torch.rand(numel, generator=gen, device=device, dtype=torch.float64)
    u = (u * (1 - 2 * eps) + eps - 0.5) * math.pi            # U ~ Uniform(-pi/2, pi/2), open
    r = torch.rand(numel, generator=gen, device=device, dtype=torch.float64)
    w = -torch.log1p(-r * (1 - eps))                           # W ~ Exp(1)
    if abs(alpha - 1.0) < 1e-12:
        x = torch.tan(u)
    else:
        x = (torch.sin(alpha * u) / torch.cos(u) ** (1.0 / alpha)
             * (torch.cos((1.0 - alpha) * u) / w) ** ((1.0 - alpha) / alpha))
    return x * gamma


def to_e4m3_bytes(x: torch.Tensor) -> torch.Tensor:
    """Clamp to +-448 (saturation) and cast with round-to-nearest-even; return uint8 bytes."""
    x = x.to(torch.float32).clamp_(-E4M3_MAX, E4M3_MAX)
    return x.to(torch.float8_e4m3fn).view(torch.uint8)


def maxabs_scale(x: torch.Tensor) -> torch.Tensor:
    m = x.abs().max()
    return x * (E4M3_MAX / m) if float(m) > 0 else x


def tile_scale(x: torch.Tensor, tile: int = 128) -> torch.Tensor:
    """Per-(tile x tile) max-abs scaling of a 2-D tensor to 448."""
    r, c = x.shape
    assert r % tile == 0 and c % tile == 0
    v = x.reshape(r // tile, tile, c // tile, tile)
    m = v.abs().amax(dim=(1, 3), keepdim=True).clamp_min(1e-30)
    return (v * (E4M3_MAX / m)).reshape(r, c)


def gauss_tensor(shape, std: float, seed: int, device="cpu") -> torch.Tensor:
    g = _gen(seed, device)
    n = int(np.prod(shape))
    x = torch.randn(n, generator=g, device=device, dtype=torch.float64) * std
    return to_e4m3_bytes(maxabs_scale(x)).reshape(shape)


def stable_tensor(shape, alpha: float, seed: int, device="cpu", gamma: float = GAMMA) -> torch.Tensor:
    g = _gen(seed, device)
    n = int(np.prod(shape))
    x = alpha_stable(alpha, n, g, device, gamma)
    return to_e4m3_bytes(maxabs_scale(x)).reshape(shape)


def dit_tensor(shape, seed: int, device="cpu", alpha: float = 1.5, outlier_frac: float = 0.02,
               outlier_std: float = 0.2) -> torch.Tensor:
    g = _gen(seed, device)
    n = int(np.prod(shape))
    x = alpha_stable(alpha, n, g, device, GAMMA)
    mask = torch.rand(n, generator=g, device=device, dtype=torch.float64) < outlier_frac
    out = torch.randn(n, generator=g, device=device, dtype=torch.float64) * outlier_std
    x = torch.where(mask, out, x)
    return to_e4m3_bytes(tile_scale(x.reshape(shape)))


def moe_alpha(expert: int, base_seed: int = 0) -> float:
    rng = np.random.default_rng(seed_of("moe256", "alpha", expert, base_seed))
    return float(rng.uniform(1.5, 2.0))


def moe_routing(base_seed: int = 0, topk: int = MOE_TOPK):
    rng = np.random.default_rng(seed_of("moe256", "routing", base_seed))
    return sorted(int(e) for e in rng.choice(MOE_EXPERTS, topk, replace=False))


def tensor_specs(workload: str, experts=None):
    """List of (name, shape, kind, params) describing a workload's tensors."""
    if workload == "gauss1m":
        return [("w", (1024, 1024), "gauss", {"std": 0.02})]
    if workload in ("llama8b", "llama70b"):
        return [(nm, sh, "stable", {"alpha": ALPHA[workload]}) for nm, sh in WORKLOADS[workload]]
    if workload == "dit14b":
        return [(nm, sh, "dit", {}) for nm, sh in WORKLOADS[workload]]
    if workload == "moe256":
        ex = range(MOE_EXPERTS) if experts is None else experts
        return [("expert%03d.%s" % (e, nm), sh, "stable", {"alpha": moe_alpha(e)})
                for e in ex for nm, sh in MOE_TENSORS]
    raise KeyError(workload)


def make_tensor(workload: str, name: str, shape, kind: str, params: dict, device="cpu",
                base_seed: int = 0) -> torch.Tensor:
    """FP8 E4M3 bytes (uint8 tensor of `shape`) for one named tensor of a workload."""
    seed = seed_of(workload, name, base_seed)
    if kind == "gauss":
        return gauss_tensor(shape, params["std"], seed, device)
    if kind == "stable":
        return stable_tensor(shape, params["alpha"], seed, device)
    if kind == "dit":
        return dit_tensor(shape, seed, device)
    raise KeyError(kind)


def float_weights(workload: str, name: str, shape, kind: str, params: dict, device="cpu",
                  base_seed: int = 0) -> torch.Tensor:
    """The same tensor as make_tensor before any scaling or rounding (float64, `shape`)."""
    seed = seed_of(workload, name, base_seed)
    g = _gen(seed, device)
    n = int(np.prod(shape))
    if kind == "gauss":
        x = torch.randn(n, generator=g, device=device, dtype=torch.float64) * params["std"]
    elif kind == "stable":
        x = alpha_stable(params["alpha"], n, g, device, GAMMA)
    elif kind == "dit":
        x = alpha_stable(1.5, n, g, device, GAMMA)
        mask = torch.rand(n, generator=g, device=device, dtype=torch.float64) < 0.02
        out = torch.randn(n, generator=g, device=device, dtype=torch.float64) * 0.2
        x = torch.where(mask, out, x)
    else:
        raise KeyError(kind)
    return x.reshape(shape)


E5M2_MAX = 57344.0


def workload_tensors_as(workload: str, fmt: str, device="cpu", experts=None, base_seed: int = 0):
    """Yield (name, tensor) for every tensor of a workload in another float format:
    "bf16" -> torch.bfloat16 (round to nearest even, no scaling), "e5m2" -> uint8 bytes of
    torch.float8_e5m2 after per-tensor max-abs scaling to 57344."""
    for name, shape, kind, params in tensor_specs(workload, experts):
        x = float_weights(workload, name, shape, kind, params, device, base_seed)
        if fmt == "bf16":
            yield name, x.to(torch.bfloat16)
        elif fmt == "e5m2":
            amax = x.abs().max()
            s = torch.where(amax > 0, E5M2_MAX / amax, torch.ones_like(amax))
            yield name, (x * s).clamp(-E5M2_MAX, E5M2_MAX).to(torch.float8_e5m2).view(torch.uint8)
        else:
            raise KeyError(fmt)
        del x


def workload_tensors(workload: str, device="cpu", experts=None, base_seed: int = 0):
    """Yield (name, uint8 tensor) for every tensor of a workload, one at a time."""
    for name, shape, kind, params in tensor_specs(workload, experts):
        yield name, make_tensor(workload, name, shape, kind, params, device, base_seed)


def small_stable(n: int, alpha: float, seed: int) -> np.ndarray:
    """Small alpha-stable FP8 sample on the CPU (tests)."""
    return stable_tensor((n,), alpha, seed, "cpu").numpy()


def random_bytes(n: int, seed: int) -> np.ndarray:
    """Uniformly random bytes: every exponent value, NaN (0x7F/0xFF) and +-0 included."""
    return np.random.default_rng(seed).integers(0, 256, n, dtype=np.uint8)
