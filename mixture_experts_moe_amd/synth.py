"""Seeded synthetic inputs for the fused MoE layer.

This module only draws random numbers and packs them into the storage formats
the layer reads; it holds none of the layer's arithmetic.  Tests feed the same
tensors to the HIP path and to the CPU oracle, and bench.py uses them as its
workload.  Every tensor has its own generator, seeded from (seed, tensor tag),
so x can be redrawn for another T without changing the weights.

The pages measure on trained models ("a representative MoE model", "large MoE
models", FP8-quantised models); no trained weights or routing traces are
available, so these seeded Gaussian tensors of the same shapes stand in.

Workloads (hidden d, experts E, top-k, intermediate I):
  tiny_fp32    T=16, d=256, E=8, k=2, I=512; fp32 x ~ N(0,1), weights ~ N(0,0.02)
  decode_bf16  T in {1,8,32,64}, d=4096, E=8, k=2, I=14336; bf16 x and weights
               ~ N(0,0.02)
  prefill_bf16 T=4096, same shapes; x ~ N(0,1), weights ~ N(0,0.02)
  fp8          T in {64,2048}, d=7168, E=256, k=8, I=2048; bf16 x ~ N(0,1);
               weights ~ N(0,0.02) quantised to e4m3fn with one fp32 scale per
               output channel (scale = row amax / 448, 1 for an all-zero row)
  prefill_w8a8 the prefill_bf16 shapes with e4m3fn weights (per-channel
               scales, as fp8) and the W8A8 mode: x and h block-scaled
               e4m3fn (act_quant "mx_e4m3")
  skew         T=512, d=2880, E=32, k=4, I=2880; bf16 x ~ N(0,1) with
               x[:,0] = 1 (a constant feature) and W_gate[e,0] = b_e so that
               expert popularity follows a Zipf(1.2)-like tail; experts 3, 11,
               19 and 27 get b_e = -50 and receive no tokens.
The router W_gate is fp32 ~ N(0,0.02) in every workload.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence, Union

import torch

E4M3FN_MAX = 448.0

WORKLOADS = {
    "tiny_fp32": dict(T=(16,), d=256, E=8, k=2, I=512, act="f32", w="f32",
                      x_std=1.0, w_std=0.02, skew=False),
    "decode_bf16": dict(T=(1, 8, 32, 64), d=4096, E=8, k=2, I=14336, act="bf16", w="bf16",
                        x_std=0.02, w_std=0.02, skew=False),
    "prefill_bf16": dict(T=(4096,), d=4096, E=8, k=2, I=14336, act="bf16", w="bf16",
                         x_std=1.0, w_std=0.02, skew=False),
    "fp8": dict(T=(64, 2048), d=7168, E=256, k=8, I=2048, act="bf16", w="e4m3fn",
                x_std=1.0, w_std=0.02, skew=False),
    "prefill_w8a8": dict(T=(4096,), d=4096, E=8, k=2, I=14336, act="bf16", w="e4m3fn",
                         x_std=1.0, w_std=0.02, skew=False, act_quant="mx_e4m3"),
    "skew": dict(T=(512,), d=2880, E=32, k=4, I=2880, act="bf16", w="bf16",
                 x_std=1.0, w_std=0.02, skew=True),
}

SKEW_IDLE_EXPERTS = (3, 11, 19, 27)
SKEW_ZIPF_S = 1.2
SKEW_ALPHA = 0.75
SKEW_IDLE_BIAS = -50.0

_TAGS = {"x": 1, "w_gate": 2, "w13": 3, "w2": 4}


@dataclasses.dataclass
class MoEInputs:
    """One layer's inputs in storage format (torch tensors on one device).

    x      [T, d]  float32 or bfloat16
    w_gate [E, d]  float32
    w13    [E, 2I, d] float32 / bfloat16 / uint8 (e4m3fn bytes)
    w2     [E, d, I]  same dtype as w13
    s13    [E, 2I] float32 per-channel scales (e4m3fn only, else None)
    s2     [E, d]  float32 (e4m3fn only, else None)
    act_quant  None, or "mx_e4m3" for the W8A8 mode
    """
    x: torch.Tensor
    w_gate: torch.Tensor
    w13: torch.Tensor
    w2: torch.Tensor
    s13: Optional[torch.Tensor]
    s2: Optional[torch.Tensor]
    top_k: int
    act: str
    w: str
    name: str
    act_quant: Optional[str] = None

    @property
    def T(self) -> int:
        return self.x.shape[0]

    @property
    def d(self) -> int:
        return self.x.shape[1]

    @property
    def E(self) -> int:
        return self.w_gate.shape[0]

    @property
    def I(self) -> int:
        return self.w2.shape[2]


def _gen(seed: int, tag: str, device, extra: int = 0) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1_000_003 + _TAGS[tag] * 7919 + extra)
    return g


def _randn(shape, std: float, gen: torch.Generator, device) -> torch.Tensor:
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32) * std


def quantize_e4m3fn_rows(w: torch.Tensor):
    """fp32 [rows, K] -> (e4m3fn bytes as uint8 [rows, K], fp32 scale [rows]).

    Input preparation, not part of the layer: one scale per row (output
    channel), scale = amax(|row|) / 448 (1 for an all-zero row), codes =
    round-to-nearest-even of w / scale via torch's float8_e4m3fn cast, after
    clamping to the finite range.
    """
    amax = w.abs().amax(dim=1)
    scale = torch.where(amax > 0, amax / E4M3FN_MAX, torch.ones_like(amax))
    q = (w / scale[:, None]).clamp_(-E4M3FN_MAX, E4M3FN_MAX).to(torch.float8_e4m3fn)
    return q.view(torch.uint8), scale.to(torch.float32)


def skew_biases(E: int = 32) -> torch.Tensor:
    """Router bias b_e for the skewed workload (fp32 [E])."""
    b = torch.empty(E, dtype=torch.float32)
    rank = 0
    for e in range(E):
        if e in SKEW_IDLE_EXPERTS:
            b[e] = SKEW_IDLE_BIAS
        else:
            rank += 1
            b[e] = -SKEW_ALPHA * SKEW_ZIPF_S * math.log(rank)
    return b


def make_x(T: int, d: int, act: str, std: float, seed: int, device, skew: bool = False) -> torch.Tensor:
    g = _gen(seed, "x", device, extra=T)
    x = _randn((T, d), std, g, device)
    if skew and T > 0:
        x[:, 0] = 1.0
    return x.to(torch.bfloat16) if act == "bf16" else x


def make_inputs(workload: Union[str, dict] = "tiny_fp32", T: Optional[int] = None, *,
                device="cpu", seed: int = 0, d: Optional[int] = None, E: Optional[int] = None,
                k: Optional[int] = None, I: Optional[int] = None, act: Optional[str] = None,
                w: Optional[str] = None, x_std: Optional[float] = None,
                w_std: Optional[float] = None, skew: Optional[bool] = None,
                scale_mode: str = "channel", act_quant: Optional[str] = None) -> MoEInputs:
    """Draw one layer's inputs.  Keyword overrides change single dimensions
    (tests use them for edge shapes); ``scale_mode`` is "channel" or "tensor"
    for e4m3fn weights."""
    if isinstance(workload, str):
        cfg = dict(WORKLOADS[workload])
        name = workload
    else:
        cfg = dict(workload)
        name = cfg.pop("name", "custom")
    over = dict(d=d, E=E, k=k, I=I, act=act, w=w, x_std=x_std, w_std=w_std, skew=skew,
                act_quant=act_quant)
    for key, val in over.items():
        if val is not None:
            cfg[key] = val
    if T is None:
        T = cfg["T"][0] if isinstance(cfg["T"], Sequence) else cfg["T"]
    d_, E_, k_, I_ = cfg["d"], cfg["E"], cfg["k"], cfg["I"]
    dev = torch.device(device)

    x = make_x(T, d_, cfg["act"], cfg["x_std"], seed, dev, skew=cfg["skew"])
    w_gate = _randn((E_, d_), 0.02, _gen(seed, "w_gate", dev), dev)
    if cfg["skew"]:
        w_gate[:, 0] = skew_biases(E_).to(dev)

    wdt = {"f32": torch.float32, "bf16": torch.bfloat16, "e4m3fn": torch.uint8}[cfg["w"]]
    w13 = torch.empty((E_, 2 * I_, d_), dtype=wdt, device=dev)
    w2 = torch.empty((E_, d_, I_), dtype=wdt, device=dev)
    s13 = s2 = None
    if cfg["w"] == "e4m3fn":
        s13 = torch.empty((E_, 2 * I_), dtype=torch.float32, device=dev)
        s2 = torch.empty((E_, d_), dtype=torch.float32, device=dev)
    g13 = _gen(seed, "w13", dev)
    g2 = _gen(seed, "w2", dev)
    for e in range(E_):          # one expert at a time keeps fp32 temporaries small
        a = _randn((2 * I_, d_), cfg["w_std"], g13, dev)
        b = _randn((d_, I_), cfg["w_std"], g2, dev)
        if cfg["w"] == "e4m3fn":
            quant = _quantize_tensor if scale_mode == "tensor" else quantize_e4m3fn_rows
            qa, sa = quant(a)
            qb, sb = quant(b)
            s13[e] = sa          # a 0-d scale broadcasts over the row
            s2[e] = sb
            w13[e] = qa
            w2[e] = qb
        else:
            w13[e] = a.to(wdt)
            w2[e] = b.to(wdt)
    if cfg["w"] == "e4m3fn" and scale_mode == "tensor":
        s13 = s13[:, 0].contiguous()
        s2 = s2[:, 0].contiguous()
    return MoEInputs(x=x, w_gate=w_gate, w13=w13, w2=w2, s13=s13, s2=s2, top_k=k_,
                     act=cfg["act"], w=cfg["w"], name=name, act_quant=cfg.get("act_quant"))


def _quantize_tensor(w: torch.Tensor):
    amax = w.abs().amax()
    scale = amax / E4M3FN_MAX if float(amax) > 0 else torch.ones((), device=w.device)
    q = (w / scale).clamp_(-E4M3FN_MAX, E4M3FN_MAX).to(torch.float8_e4m3fn)
    return q.view(torch.uint8), scale.to(torch.float32)


def to_oracle(inp: MoEInputs, experts: Optional[Sequence[int]] = None) -> dict:
    """Host copies in the raw formats the oracle reads (bf16 -> uint16 bit
    patterns, e4m3fn -> uint8, fp32 -> float32), as keyword arguments for the
    oracle's layer function.  Weights are fetched lazily per expert."""
    def raw(t: torch.Tensor):
        t = t.detach()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).cpu().numpy().view("uint16")
        return t.cpu().numpy()

    class _Lazy:
        def __init__(self, t):
            self.t = t
            self.cache = {}

        def __getitem__(self, e):
            e = int(e)
            if e not in self.cache:
                self.cache[e] = raw(self.t[e])
            return self.cache[e]

    kw = dict(x=raw(inp.x), w_gate=inp.w_gate.detach().cpu().numpy(),
              w13=_Lazy(inp.w13), w2=_Lazy(inp.w2), top_k=inp.top_k,
              act_fmt=inp.act, w_fmt=inp.w)
    if inp.w == "e4m3fn":
        kw.update(s13=raw(inp.s13), s2=raw(inp.s2),
                  scale_mode="tensor" if inp.s13.dim() == 1 else "channel")
    if inp.act_quant is not None:
        kw["act_quant"] = inp.act_quant
    return kw
