"""Helpers shared by the GPU tests: device transfer, running the C ABI, comparisons."""

from __future__ import annotations

import numpy as np

import oracle
from synth import LayerInputs

# Tolerances: routing and dispatch bit-exact; outputs max-abs-rel 2e-2 (bf16) / 1e-5 (fp32);
# gates and the loss 1e-6 relative.
OUT_TOL = {"bf16": 2e-2, "f32": 1e-5}
GATE_TOL = 1e-6
AUX_TOL = 1e-6


def to_dev(a, name=""):
    import torch
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_host(t) -> np.ndarray:
    import torch
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()


def device_inputs(I: LayerInputs) -> dict:
    return {n: to_dev(getattr(I, n)) for n in ("x", "w_router", "bias", "w1", "w3", "w2")}


def run_forward(I: LayerInputs, T=None):
    import torch
    from expert_ffn_layer_router_amd import binding as B
    p = B.Problem.from_spec(I.spec)
    d = device_inputs(I)
    outs = B.forward(p, d["x"], d["w_router"], d["bias"], d["w1"], d["w3"], d["w2"])
    torch.cuda.synchronize()
    return {k: to_host(v) for k, v in outs.items()}


def run_oracle(I: LayerInputs, tokens=None) -> dict:
    sp = I.spec
    return oracle.moe_forward(I.values("x"), I.values("w_router"), sp.top_k, sp.kind,
                              I.values("w1"), I.values("w2"), I.values("w3"),
                              bias=I.bias, capacity_factor=sp.capacity_factor, tokens=tokens)


def max_abs_rel(got: np.ndarray, ref: np.ndarray) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    scale = np.abs(ref).max() if ref.size else 0.0
    err = np.abs(got - ref).max() if ref.size else 0.0
    if scale == 0.0:
        return float(err)
    return float(err / scale)


def rel_err(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if got.size == 0:
        return 0.0
    return float((np.abs(got - ref) / np.maximum(np.abs(ref), 1e-300)).max())


def check_routing(g: dict, r: dict):
    """Bit-exact routing and dispatch; gates and aux within 1e-6 relative."""
    assert np.array_equal(g["expert_indices"], r["expert_indices"]), "expert_indices differ"
    assert np.array_equal(g["expert_counts"], r["counts"]), "expert_counts differ"
    assert np.array_equal(g["expert_offsets"], r["offsets"]), "expert_offsets differ"
    assert np.array_equal(g["slot_row"], r["slot_row"]), "slot_row (drop set) differs"
    assert rel_err(g["gates"], r["gates"]) <= GATE_TOL, rel_err(g["gates"], r["gates"])
    assert rel_err(g["aux_loss"][0], r["aux_loss"]) <= AUX_TOL, (g["aux_loss"], r["aux_loss"])
