"""Decode-on-use of ECF8-compressed linear layers.

ECF8 technical blog (codearts.csdn.net):
  * §3.2.2 memory management: a pool sized for the largest layer is
    allocated once, a layer's weights are decoded into it when the layer is
    about to run, and the pool is reused with no further allocation;
  * §3.3: layer-wise pipelining (and, on large GPUs, resident compressed
    weights with batched decode);
  * deployment notes: while layer N computes, the weights of layer N + 2 are
    decoded in the background;
  * integration notes: an ``ECF8Linear`` wrapper replaces a linear layer and
    decodes its weight when it is used.

Every decode is the library's HIP kernel (``DecodePlan``) and every product is
a library GEMM (``torch._scaled_mm`` on FP8 operands, i.e. hipBLASLt); this
module only allocates the pool once and orders launches on two HIP streams
with events.
"""
from __future__ import annotations

from typing import List, Optional, Sequence

import torch

from . import binding

E4M3_MAX = 448.0


def fp8_e4m3_bytes(w: torch.Tensor) -> "tuple[torch.Tensor, float]":
    """Per-tensor max-abs scaling of a float weight to FP8 E4M3 bytes.

    Returns (uint8 bytes, scale) with w ~= e4m3(bytes) * scale; values are
    clamped to +-448 before the round-to-nearest-even cast.
    """
    amax = float(w.detach().abs().max())
    scale = amax / E4M3_MAX if amax > 0 else 1.0
    q = (w.detach().float() / scale).clamp_(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
    return q.view(torch.uint8), scale


def _scaled_mm_ok(device) -> bool:
    """Whether torch._scaled_mm runs FP8 E4M3 here (probed once per device)."""
    key = str(device)
    if key not in _SCALED_MM_OK:
        try:
            a = torch.zeros(16, 32, dtype=torch.float8_e4m3fn, device=device)
            b = torch.zeros(16, 32, dtype=torch.float8_e4m3fn, device=device)
            one = torch.ones((), dtype=torch.float32, device=device)
            torch._scaled_mm(a, b.t(), scale_a=one, scale_b=one, out_dtype=torch.bfloat16)
            _SCALED_MM_OK[key] = True
        except (RuntimeError, TypeError, AttributeError):
            _SCALED_MM_OK[key] = False
    return _SCALED_MM_OK[key]


_SCALED_MM_OK: dict = {}


def linear_fp8(x_fp8: torch.Tensor, x_scale: torch.Tensor, w_u8: torch.Tensor, w_scale: torch.Tensor,
               bias: Optional[torch.Tensor] = None, out_dtype=torch.bfloat16) -> torch.Tensor:
    """y = (x * x_scale) @ (w * w_scale)^T + bias for FP8 E4M3 x (T x K) and w (N x K).

    The FP8 GEMM is hipBLASLt's, through torch._scaled_mm.  There is no other
    GEMM path: where torch._scaled_mm does not run FP8 E4M3 this raises.
    """
    w = w_u8.view(torch.float8_e4m3fn)
    if not _scaled_mm_ok(x_fp8.device):
        raise RuntimeError("torch._scaled_mm does not run FP8 E4M3 GEMMs on %s" % x_fp8.device)
    y = torch._scaled_mm(x_fp8, w.t(), scale_a=x_scale, scale_b=w_scale, out_dtype=out_dtype)
    if bias is not None:
        y = y + bias.to(out_dtype)
    return y


def check_decode(plan: binding.DecodePlan, stream=None):
    """Checked mode: synchronize `stream` and raise if a run of `plan` since the
    previous check flagged any block (its decoded symbol count disagreed with
    blk_off); each check restarts the count."""
    bad = plan.status(stream)
    if bad:
        raise binding.Ecf8Error(-5, "ECF8 decode (%d corrupt blocks)" % bad)


class ECF8Linear(torch.nn.Module):
    """A linear layer whose FP8 E4M3 weight is kept ECF8-compressed on the GPU.

    ``weight_u8`` is the (out_features x in_features) weight as E4M3 bytes and
    ``scale`` its per-tensor scale.  The compressed form (stream, nibble plane,
    gaps, block offsets) is device resident; ``forward`` decodes it (into a
    buffer the caller passes, or one the layer allocates on first use) and runs
    the FP8 GEMM.
    """

    def __init__(self, weight_u8: torch.Tensor, scale: float, bias: Optional[torch.Tensor] = None,
                 device="cuda", checked: bool = False, max_code_len: int = 11):
        """checked: after each decode into the layer's own buffer, synchronize
        and raise if the decode's block check flagged a block (a corrupt
        stream, gap or block offset) instead of feeding the GEMM.
        max_code_len: the code length limit of the weight's encoding; at 11
        every codeword fits the decode table's 11-bit index, so the decode
        takes its one-shift form (the limit costs a few hundredths of a
        percent of the stream on typical weights); 16 is plain Huffman."""
        super().__init__()
        self.checked = checked
        if weight_u8.dim() != 2 or weight_u8.dtype != torch.uint8:
            raise ValueError("weight_u8 must be a 2-D uint8 tensor of FP8 E4M3 bytes")
        self.out_features, self.in_features = (int(s) for s in weight_u8.shape)
        self.device = torch.device(device)
        self.enc = binding.encode(weight_u8.contiguous().cpu(), max_len=max_code_len).to(self.device)
        self.register_buffer("w_scale", torch.tensor(float(scale), dtype=torch.float32, device=self.device))
        self.bias = None if bias is None else bias.detach().to(self.device)
        self._own: Optional[torch.Tensor] = None
        self._own_plan: Optional[binding.DecodePlan] = None

    @classmethod
    def from_linear(cls, linear: torch.nn.Linear, device="cuda") -> "ECF8Linear":
        """Quantize an nn.Linear weight to FP8 E4M3 (per-tensor max-abs scale) and compress it."""
        q, scale = fp8_e4m3_bytes(linear.weight.detach().cpu())
        return cls(q, scale, linear.bias, device)

    @property
    def numel(self) -> int:
        return self.out_features * self.in_features

    def compressed_bytes(self) -> int:
        return self.enc.compressed_bytes()

    def plan_into(self, out_u8: torch.Tensor, workspace=None, stream=None,
                  workgroups: Optional[int] = None) -> binding.DecodePlan:
        """A decode plan writing this layer's weight bytes into out_u8[:numel]."""
        return binding.DecodePlan([self.enc], out=out_u8, offsets=[0], workspace=workspace, stream=stream,
                                  workgroups=workgroups)

    def decoded_weight(self, stream=None) -> torch.Tensor:
        """Decode into the layer's own buffer (allocated on first use) and return it (uint8, out x in)."""
        if self._own is None:
            self._own = torch.empty(self.numel, dtype=torch.uint8, device=self.device)
            self._own_plan = self.plan_into(self._own, stream=stream)
        self._own_plan.run(stream)
        if self.checked:
            check_decode(self._own_plan, stream)
        return self._own.view(self.out_features, self.in_features)

    def forward(self, x_fp8: torch.Tensor, x_scale: torch.Tensor,
                weight_u8: Optional[torch.Tensor] = None) -> torch.Tensor:
        w = self.decoded_weight() if weight_u8 is None else weight_u8.view(self.out_features, self.in_features)
        return linear_fp8(x_fp8, x_scale, w, self.w_scale, self.bias)


class DecodePipeline:
    """Runs ECF8Linear layers in order, decoding each layer's weight ahead of use.

    One pool of ``slots`` weight buffers (each the size of the largest layer)
    is allocated at construction; layer i decodes into slot i % slots on a side
    stream, ``ahead`` layers before it runs on the caller's stream.  Events
    order the two streams: layer i's GEMM waits for its decode, and the decode
    that reuses a slot waits for the GEMM that last read it.  ``ahead`` = 0
    decodes each layer on the caller's stream right before its GEMM (no
    overlap).  ``workgroups`` caps the decode grid so that GEMMs keep compute
    units while a decode runs beside them.
    """

    def __init__(self, layers: Sequence[ECF8Linear], slots: int = 3, ahead: int = 2,
                 workgroups: Optional[int] = None, checked: bool = False):
        """checked: at the end of each run, synchronize and raise if any layer's
        decode flagged a block (every plan has its own workspace, so each
        layer's block check is read separately)."""
        self.checked = checked
        if not layers:
            raise ValueError("no layers")
        if ahead < 0 or (ahead > 0 and ahead > slots - 1) or slots < 1:
            raise ValueError("need 0 <= ahead <= slots - 1")
        self.layers = list(layers)
        self.slots, self.ahead = slots, ahead
        dev = self.layers[0].device
        self.slot_bytes = (max(l.numel for l in self.layers) + 255) // 256 * 256
        self.pool = torch.empty(slots * self.slot_bytes, dtype=torch.uint8, device=dev)
        self.side = torch.cuda.Stream(device=dev) if ahead > 0 else None
        self.plans: List[binding.DecodePlan] = []
        for i, layer in enumerate(self.layers):
            self.plans.append(layer.plan_into(self.slot(i), stream=self.side, workgroups=workgroups))
        if self.side is not None:
            self.side.synchronize()
        self.decoded = [torch.cuda.Event() for _ in self.layers]
        self.used = [torch.cuda.Event() for _ in self.layers]

    def slot(self, i: int) -> torch.Tensor:
        k = i % self.slots
        return self.pool[k * self.slot_bytes: k * self.slot_bytes + self.layers[i].numel]

    def pool_bytes(self) -> int:
        return self.pool.numel()

    def run(self, xs: Sequence[torch.Tensor], x_scales: Sequence[torch.Tensor]) -> List[torch.Tensor]:
        """Layer i computes on xs[i]; returns the outputs (caller's stream order)."""
        L = len(self.layers)
        main = torch.cuda.current_stream(self.layers[0].device)
        outs = []
        if self.ahead == 0:
            for i in range(L):
                self.plans[i].run(main)
                outs.append(self.layers[i](xs[i], x_scales[i], weight_u8=self.slot(i)))
            self._check(main)
            return outs
        side = self.side
        side.wait_stream(main)          # inputs and the pool are ready on the caller's stream
        for j in range(min(self.ahead, L)):
            self.plans[j].run(side)
            self.decoded[j].record(side)
        for i in range(L):
            j = i + self.ahead
            if j < L:
                if j - self.slots >= 0:
                    side.wait_event(self.used[j - self.slots])
                self.plans[j].run(side)
                self.decoded[j].record(side)
            main.wait_event(self.decoded[i])
            outs.append(self.layers[i](xs[i], x_scales[i], weight_u8=self.slot(i)))
            self.used[i].record(main)
        main.wait_stream(side)
        self._check(main)
        return outs

    def _check(self, stream):
        if self.checked:
            for p in self.plans:
                check_decode(p, stream)
