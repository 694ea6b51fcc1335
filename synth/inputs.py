"""Seeded synthetic inputs for the MoE layer forward, and nothing else.

Recipe (the same on every machine):

* generators: PCG64 streams ``default_rng(SeedSequence([seed, tensor, expert]))``,
  one per tensor and, for expert weights, one per expert (so experts can be drawn
  in parallel); seed 0 unless stated; tensor ids: x 0, router weights 1, router
  bias 2, first expert matrix 3, third (SwiGLU) matrix 4, last matrix 5; expert
  is 0 for the non-expert tensors;
* every tensor is drawn with ``standard_normal(n, dtype=float32)`` and scaled by
  its standard deviation in float32; for bfloat16 layers the values are then
  rounded to bfloat16 (round to nearest, ties to even) and the rounded values are
  what both the GPU and the oracle receive;
* shapes: x (T, D); router weights (D, E); router bias (E); first matrix
  (E, D, DH) (or (E, D, D_out) for a linear expert), third matrix (E, D, DH) for
  SwiGLU, last matrix (E, DH, D_out);
* a Zipf-skewed bias is not drawn: expert e gets ``-ln(e + 1)``, so that
  ``softmax(bias)`` is proportional to ``1 / rank`` with rank = e + 1.

Weights are laid out (in, out) row-major, as in ``x @ W`` on every page that
defines the layer.
"""

from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Optional, Union

import numpy as np

_THREADS = max(1, min(16, len(os.sched_getaffinity(0))))

Std = Union[float, str]  # a number, or "fanin" for 1/sqrt(fan_in)


@dataclass(frozen=True)
class LayerSpec:
    name: str
    T: int
    D: int
    DH: int  # expert hidden width; 0 for a linear expert
    D_out: int
    E: int
    top_k: int
    kind: str  # "linear" | "relu2" | "swiglu"
    dtype: str  # "f32" | "bf16"
    capacity_factor: float  # <= 0 means no capacity limit
    x_std: Std = 1.0
    router_std: Std = 1.0
    bias: str = "none"  # "none" | "normal" | "zipf"
    w_std: Std = 1.0  # first (and third) expert matrix
    w2_std: Std = 1.0  # last expert matrix
    description: str = ""

    def with_(self, **kw) -> "LayerSpec":
        out = dataclasses.replace(self, **kw)
        if out.kind == "linear":
            out = dataclasses.replace(out, DH=0)
        elif "D_out" not in kw:
            out = dataclasses.replace(out, D_out=out.D)
        return out

    @property
    def slots(self) -> int:
        return self.T * self.top_k


CONFIGS = {
    "tiny_linear_f32": LayerSpec(
        "tiny_linear_f32", T=6, D=4, DH=0, D_out=3, E=4, top_k=2, kind="linear", dtype="f32",
        capacity_factor=0.0, x_std=1.0, router_std=1.0, w_std=1.0, w2_std=1.0,
        description="tiny linear-expert MoE, fp32, T=6 d=4 E=4 k=2, W_e (4,3)"),
    "small_relu_f32": LayerSpec(
        "small_relu_f32", T=16, D=32, DH=64, D_out=32, E=8, top_k=2, kind="relu2", dtype="f32",
        capacity_factor=0.0, x_std=1.0, router_std="fanin", w_std="fanin", w2_std="fanin",
        description="small ReLU-MLP-expert MoE, fp32, T=16 D=32 DH=64 E=8 k=2"),
    "switch_top1_cap_bf16": LayerSpec(
        "switch_top1_cap_bf16", T=8192, D=1024, DH=4096, D_out=1024, E=64, top_k=1, kind="relu2",
        dtype="bf16", capacity_factor=1.25, x_std=1.0, router_std="fanin", bias="normal",
        w_std="fanin", w2_std="fanin",
        description="Switch-style top-1, capacity factor 1.25, bf16, T=8192 D=1024 DH=4096 E=64"),
    "mixtral_swiglu_bf16": LayerSpec(
        "mixtral_swiglu_bf16", T=4096, D=4096, DH=14336, D_out=4096, E=8, top_k=2, kind="swiglu",
        dtype="bf16", capacity_factor=0.0, x_std=1.0, router_std=0.02, w_std=0.02, w2_std=0.02,
        description="Mixtral-shaped SwiGLU MoE layer, bf16, T=4096 D=4096 DH=14336 E=8 k=2"),
    "fine_grained_zipf_bf16": LayerSpec(
        "fine_grained_zipf_bf16", T=16384, D=2048, DH=1408, D_out=2048, E=64, top_k=6,
        kind="swiglu", dtype="bf16", capacity_factor=2.0, x_std=1.0, router_std=0.02,
        bias="zipf", w_std=0.02, w2_std=0.02,
        description="fine-grained 64-expert SwiGLU MoE, Zipf-skewed router, capacity factor 2.0, "
                    "bf16, T=16384 D=2048 DH=1408 E=64 k=6"),
}


def spec(name: str, **overrides) -> LayerSpec:
    """A named configuration, optionally with some fields replaced."""
    base = CONFIGS[name]
    return base.with_(**overrides) if overrides else base


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest, ties to even."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    bias = (u >> np.uint32(16)) & np.uint32(1)
    bias += np.uint32(0x7FFF)
    bias += u
    bias >>= np.uint32(16)
    return bias.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> the exactly equal float32 values."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _std(s: Std, fan_in: int) -> float:
    if isinstance(s, str):
        if s != "fanin":
            raise ValueError(f"unknown std rule {s!r}")
        return 1.0 / math.sqrt(fan_in)
    return float(s)


@dataclass
class LayerInputs:
    """Drawn tensors. bf16 tensors are held as uint16 bit patterns, f32 as float32."""

    spec: LayerSpec
    x: np.ndarray
    w_router: np.ndarray
    bias: Optional[np.ndarray]  # float32 (E,) or None
    w1: np.ndarray  # (E, D, DH) or (E, D, D_out) for linear
    w3: Optional[np.ndarray]  # (E, D, DH) for SwiGLU
    w2: Optional[np.ndarray]  # (E, DH, D_out), None for linear

    def values(self, name: str) -> Optional[np.ndarray]:
        """float32 array holding exactly the stored values of tensor ``name``."""
        a = getattr(self, name)
        if a is None:
            return None
        if a.dtype == np.uint16:
            return bf16_bits_to_f32(a)
        return a


X_ID, ROUTER_ID, BIAS_ID, W1_ID, W3_ID, W2_ID, NOISE_W_ID, NOISE_ID = range(8)


def _rng(seed: int, tensor: int, expert: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, tensor, expert]))


def _draw(rng: np.random.Generator, shape, std: float, dtype: str) -> np.ndarray:
    n = int(np.prod(shape))
    a = rng.standard_normal(n, dtype=np.float32)
    a *= np.float32(std)
    a = a.reshape(shape)
    if dtype == "bf16":
        return f32_to_bf16_bits(a)
    return a


def _draw_experts(seed, tensor, E, shape, std, dtype) -> np.ndarray:
    out = np.empty((E,) + tuple(shape), dtype=np.uint16 if dtype == "bf16" else np.float32)

    def one(e):
        out[e] = _draw(_rng(seed, tensor, e), shape, std, dtype)

    n = int(np.prod(shape))
    if E > 1 and n >= (1 << 20):
        with ThreadPoolExecutor(min(E, _THREADS)) as ex:
            list(ex.map(one, range(E)))
    else:
        for e in range(E):
            one(e)
    return out


def make_inputs(sp: LayerSpec, seed: int = 0, router_zero: bool = False) -> LayerInputs:
    """Draw the inputs of layer ``sp`` from the seeded streams described above.

    ``router_zero`` sets the router weights to zero (the uniform-router case) and
    leaves every other tensor as drawn.
    """
    x = _draw(_rng(seed, X_ID), (sp.T, sp.D), _std(sp.x_std, sp.D), sp.dtype)
    w_router = _draw(_rng(seed, ROUTER_ID), (sp.D, sp.E), _std(sp.router_std, sp.D), sp.dtype)
    if router_zero:
        w_router = np.zeros_like(w_router)
    bias = None
    if sp.bias == "normal":
        bias = _rng(seed, BIAS_ID).standard_normal(sp.E, dtype=np.float32)
    elif sp.bias == "zipf":
        bias = (-np.log(np.arange(1, sp.E + 1, dtype=np.float64))).astype(np.float32)
    elif sp.bias != "none":
        raise ValueError(f"unknown bias rule {sp.bias!r}")
    wstd = _std(sp.w_std, sp.D)
    if sp.kind == "linear":
        w1 = _draw_experts(seed, W1_ID, sp.E, (sp.D, sp.D_out), wstd, sp.dtype)
        return LayerInputs(sp, x, w_router, bias, w1, None, None)
    w1 = _draw_experts(seed, W1_ID, sp.E, (sp.D, sp.DH), wstd, sp.dtype)
    w3 = None
    if sp.kind == "swiglu":
        w3 = _draw_experts(seed, W3_ID, sp.E, (sp.D, sp.DH), wstd, sp.dtype)
    elif sp.kind != "relu2":
        raise ValueError(f"unknown expert kind {sp.kind!r}")
    w2 = _draw_experts(seed, W2_ID, sp.E, (sp.DH, sp.D_out), _std(sp.w2_std, sp.DH), sp.dtype)
    return LayerInputs(sp, x, w_router, bias, w1, w3, w2)


@dataclass
class RouterNoise:
    """Router-noise inputs: ``w_noise`` (D, E) stored like the layer's tensors (uint16 bf16 bit
    patterns or float32) and ``noise`` (T, E) float32 standard-normal draws."""

    w_noise: np.ndarray
    noise: np.ndarray

    def w_values(self) -> np.ndarray:
        """float32 array holding exactly the stored values of ``w_noise``."""
        if self.w_noise.dtype == np.uint16:
            return bf16_bits_to_f32(self.w_noise)
        return self.w_noise


def make_router_noise(sp: LayerSpec, seed: int = 0, w_std: Std = "fanin",
                      noise_scale: float = 1.0) -> RouterNoise:
    """The noise weights (N(0, w_std), fan-in by default, so x . W_noise is about unit scale)
    and the (T, E) standard-normal draw, times ``noise_scale`` (0 gives an all-zero draw), from
    their own seeded streams."""
    w_noise = _draw(_rng(seed, NOISE_W_ID), (sp.D, sp.E), _std(w_std, sp.D), sp.dtype)
    noise = _rng(seed, NOISE_ID).standard_normal((sp.T, sp.E), dtype=np.float32)
    noise *= np.float32(noise_scale)
    return RouterNoise(w_noise, noise)
