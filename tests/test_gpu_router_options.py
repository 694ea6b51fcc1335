"""GPU parity of the router options and the capacity-padded layout (moe_options), through
the C ABI, against the CPU oracle.

Bars as for the plain layer: routing, counts, offsets, perm and slot_row bit-exact; gates
and aux_loss within 1e-6 relative; outputs max-abs-rel 2e-2 (bf16) / 1e-5 (fp32). The
importance loss is CV^2 of per-expert gate sums whose relative error is at most rho = 1e-6
(sums of gates that are each within 1e-6); to first order that moves CV^2 by at most
rho * (4 sqrt(CV^2) + 2 CV^2), plus the float32 rounding of the result.
"""

from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
from gpu_util import (AUX_TOL, GATE_TOL, OUT_TOL, device_inputs, max_abs_rel, rel_err, to_dev,
                      to_host)
from synth import make_inputs, make_router_noise, spec

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def importance_tol(c: float) -> float:
    return 1e-6 * (4.0 * math.sqrt(max(c, 0.0)) + 2.0 * c) + 2.0 ** -24 * c + 1e-12


def _options(B, N, renormalise, padded, imp):
    return B.Options(w_noise=None if N is None else to_dev(N.w_noise),
                     noise=None if N is None else to_dev(N.noise),
                     renormalise=renormalise, padded=padded, importance_loss=imp)


def run_forward_ex(I, N=None, renormalise=True, padded=False):
    import torch
    from expert_ffn_layer_router_amd import binding as B
    p = B.Problem.from_spec(I.spec)
    d = device_inputs(I)
    imp = torch.full((1,), float("nan"), dtype=torch.float32, device="cuda")
    o = _options(B, N, renormalise, padded, imp)
    ws = B.alloc_workspace(p, o=o)
    outs = B.alloc_outputs(p)
    B.moe_forward_ex(p, o, d["x"], d["w_router"], d["bias"], d["w1"], d["w3"], d["w2"],
                     outs["out"], outs["expert_indices"], outs["gates"], outs["aux_loss"],
                     outs["expert_counts"], outs["expert_offsets"], outs["slot_row"], ws)
    torch.cuda.synchronize()
    res = {k: to_host(v) for k, v in outs.items()}
    res["importance_loss"] = float(to_host(imp)[0])
    return res


def run_oracle_ex(I, N=None, renormalise=True):
    sp = I.spec
    return oracle.moe_forward(I.values("x"), I.values("w_router"), sp.top_k, sp.kind,
                              I.values("w1"), I.values("w2"), I.values("w3"), bias=I.bias,
                              capacity_factor=sp.capacity_factor,
                              w_noise=None if N is None else N.w_values(),
                              noise=None if N is None else N.noise, renormalise=renormalise)


def check_route(g, r):
    assert np.array_equal(g["expert_indices"], r["expert_indices"]), "expert_indices differ"
    assert np.array_equal(g["expert_counts"], r["counts"]), "expert_counts differ"
    assert rel_err(g["gates"], r["gates"]) <= GATE_TOL, rel_err(g["gates"], r["gates"])
    assert rel_err(g["aux_loss"][0], r["aux_loss"]) <= AUX_TOL, (g["aux_loss"], r["aux_loss"])
    c = r["importance_loss"]
    assert abs(g["importance_loss"] - c) <= importance_tol(c), (g["importance_loss"], c)


NOISY_CASES = {
    "swiglu_e8_k2": spec("mixtral_swiglu_bf16", T=700, D=256, DH=384, E=8),
    "swiglu_zipf_cap": spec("fine_grained_zipf_bf16", T=1000, D=512, DH=320),
    "relu_top1_cap": spec("switch_top1_cap_bf16", T=1500, D=256, DH=512),
    "relu_256_experts": spec("switch_top1_cap_bf16", T=600, D=64, DH=64, E=256, top_k=8,
                             capacity_factor=0.0),
    "relu_f32_ragged": spec("small_relu_f32", T=333, D=40, DH=70, E=5, top_k=3,
                            capacity_factor=1.3),
    "swiglu_f32": spec("small_relu_f32", T=50, D=12, DH=20, E=6, top_k=2, kind="swiglu"),
    # 2 E router columns (logits, then the noise router's) in 2, 3 and 4 tiles of 16 on the
    # exact float64 route, ragged token counts
    "swiglu_e16_k4": spec("mixtral_swiglu_bf16", T=909, D=320, DH=256, E=16, top_k=4),
    "swiglu_e24_k3_cap": spec("fine_grained_zipf_bf16", T=611, D=128, DH=192, E=24, top_k=3,
                              capacity_factor=1.5),
    "relu_e32_top1_cap": spec("switch_top1_cap_bf16", T=517, D=192, DH=128, E=32),
    # edges of the exact noisy route: one token, k = E (every expert chosen), the smallest D
    "swiglu_e8_k8_one_token": spec("mixtral_swiglu_bf16", T=1, D=64, DH=64, E=8, top_k=8),
    "relu_e32_k32": spec("switch_top1_cap_bf16", T=17, D=64, DH=64, E=32, top_k=32,
                         capacity_factor=0.0),
}


def _exact_noisy_route(sp) -> bool:
    """bf16 layers whose 2 E router columns (the logits' and the noise router's) fit the exact
    float64 route's 64 (E a multiple of 8): every noisy logit exact to float64 rounding, no
    token recomputed."""
    return sp.dtype == "bf16" and 8 <= sp.E <= 32 and sp.E % 8 == 0 and sp.D % 64 == 0


@pytest.mark.parametrize("renormalise", [True, False], ids=["renorm", "probs"])
@pytest.mark.parametrize("name", sorted(NOISY_CASES))
def test_noisy_router_forward(name, renormalise):
    sp = NOISY_CASES[name]
    _say(f"[gpu] noisy forward {name} renormalise={renormalise} {sp}")
    I = make_inputs(sp, seed=11)
    N = make_router_noise(sp, seed=11)
    g, r = run_forward_ex(I, N, renormalise=renormalise), run_oracle_ex(I, N, renormalise)
    check_route(g, r)
    assert np.array_equal(g["expert_offsets"], r["offsets"])
    assert np.array_equal(g["slot_row"], r["slot_row"])
    err = max_abs_rel(g["out"], r["output"])
    _say(f"  out max-abs-rel {err:.3e}, importance {g['importance_loss']:.6g}")
    assert err <= OUT_TOL[sp.dtype]
    if not renormalise:
        assert (g["gates"].sum(axis=1) <= 1.0 + 1e-6).all()


@pytest.mark.parametrize("name", sorted(n for n, c in NOISY_CASES.items()
                                         if c.dtype == "f32" or _exact_noisy_route(c)))
def test_noisy_route_exports_noisy_logits(name):
    """moe_route_ex's logits_out holds the noisy logits (the ones the top-k, probabilities and
    gates use), as the float32 rounding of the oracle's float64 values: on the exact float64
    route and on the float32 layers every noisy logit is exact to float64 rounding."""
    import torch
    from expert_ffn_layer_router_amd import binding as B
    sp = NOISY_CASES[name]
    _say(f"[gpu] noisy logits {name} {sp}")
    I = make_inputs(sp, seed=13)
    N = make_router_noise(sp, seed=13)
    p = B.Problem.from_spec(sp)
    o = _options(B, N, True, False, None)
    ws = B.alloc_workspace(p, o=o)
    T, k, E = sp.T, sp.top_k, sp.E
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    gates = torch.empty((T, k), dtype=torch.float32, device="cuda")
    aux = torch.empty(1, dtype=torch.float32, device="cuda")
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    logits = torch.full((T, E), float("nan"), dtype=torch.float32, device="cuda")
    unc = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    B.moe_route_ex(p, o, to_dev(I.x), to_dev(I.w_router), to_dev(I.bias), idx, gates, aux,
                   counts, logits, unc, ws)
    torch.cuda.synchronize()
    ref = oracle.noisy_router_logits(I.values("x"), I.values("w_router"), I.bias,
                                     N.w_values(), N.noise)
    assert max_abs_rel(to_host(logits), ref) <= 1e-6
    assert np.array_equal(to_host(idx), oracle.top_k_sorted(ref, k))
    assert int(unc.cpu()[0]) == 0


def test_noise_changes_decisions_and_zero_noise_does_not():
    """Noise of the size of the logit gaps moves some choices; a zero draw moves none, and
    then the layer is the plain one bit for bit."""
    sp = spec("mixtral_swiglu_bf16", T=512, D=256, DH=256, E=8)
    I = make_inputs(sp, seed=12)
    plain = run_forward_ex(I)
    zero = run_forward_ex(I, make_router_noise(sp, seed=12, noise_scale=0.0))
    for k in ("out", "expert_indices", "gates", "aux_loss", "slot_row"):
        assert np.array_equal(plain[k], zero[k]), k
    N = make_router_noise(sp, seed=12, w_std=1.0, noise_scale=1.0)
    noisy = run_forward_ex(I, N)
    r = run_oracle_ex(I, N)
    check_route(noisy, r)
    moved = (noisy["expert_indices"] != plain["expert_indices"]).any(axis=1).sum()
    _say(f"  tokens that changed an expert under noise: {moved} of {sp.T}")
    assert moved > 0


def test_importance_loss_page_table_on_gpu():
    """The page's 64-token, 8-expert, top-1 tables: importance 0.301 and 7.000."""
    import torch
    from expert_ffn_layer_router_amd import binding as B
    from golden_io import load
    g = load("sparsely_gated_importance.txt")
    E = g["E"]
    for name in ("random", "collapsed"):
        tok = np.repeat(np.arange(E), g[f"{name}_counts"])
        np.random.default_rng(5).shuffle(tok)
        x = np.eye(E, dtype=np.float32)[tok]
        w = (10.0 * np.eye(E)).astype(np.float32)
        w1 = np.ones((E, E, 8), dtype=np.float32)
        p = B.Problem(T=g["T"], D=E, DH=0, D_out=8, E=E, top_k=1, dtype="f32", kind="linear")
        imp = torch.zeros(1, dtype=torch.float32, device="cuda")
        o = B.Options(importance_loss=imp)
        ws = B.alloc_workspace(p, o=o)
        outs = B.alloc_outputs(p)
        B.moe_forward_ex(p, o, to_dev(x), to_dev(w), None, to_dev(w1), None, None, outs["out"],
                         outs["expert_indices"], outs["gates"], outs["aux_loss"],
                         outs["expert_counts"], outs["expert_offsets"], outs["slot_row"], ws)
        torch.cuda.synchronize()
        v = float(imp.cpu()[0])
        _say(f"  {name}: importance {v}")
        assert round(v, g["decimals"]) == g[f"{name}_importance"]
        want = oracle.importance_loss(to_host(outs["expert_indices"]), to_host(outs["gates"]), E)
        assert abs(v - want) <= importance_tol(want)


PADDED_CASES = {
    "relu_top1_cap": spec("switch_top1_cap_bf16", T=1500, D=256, DH=512),
    "swiglu_zipf_cap2": spec("fine_grained_zipf_bf16", T=1000, D=512, DH=320),
    "swiglu_e8_cap1": spec("mixtral_swiglu_bf16", T=700, D=256, DH=384, E=8,
                           capacity_factor=1.0),
    "relu_f32_cap": spec("small_relu_f32", T=333, D=40, DH=70, E=5, top_k=3,
                         capacity_factor=1.3),
}


@pytest.mark.parametrize("name", sorted(PADDED_CASES))
def test_padded_forward(name):
    """The capacity-padded layout computes the same layer: padded rows and batch starts as
    the oracle lays them out, and outputs within the bar (and equal to the compact run's
    within it)."""
    sp = PADDED_CASES[name]
    _say(f"[gpu] padded forward {name} {sp}")
    I = make_inputs(sp, seed=13)
    g, r = run_forward_ex(I, padded=True), run_oracle_ex(I)
    cap = r["capacity"]
    pad = oracle.padded_layout(r, sp.E, cap)
    check_route(g, r)
    assert np.array_equal(g["expert_offsets"], np.arange(sp.E + 1) * cap)
    assert np.array_equal(g["slot_row"], pad["slot_row_padded"])
    err = max_abs_rel(g["out"], r["output"])
    _say(f"  cap {cap}, padded rows {sp.E * cap}, kept {r['offsets'][-1]}, out {err:.3e}")
    assert err <= OUT_TOL[sp.dtype]
    compact = run_forward_ex(I)
    check_route(compact, r)
    assert max_abs_rel(g["out"], compact["out"]) <= OUT_TOL[sp.dtype]


IMPORTANCE_CASES = {
    "swiglu_e8_k2": spec("mixtral_swiglu_bf16", T=700, D=256, DH=384, E=8),
    "swiglu_zipf_cap": spec("fine_grained_zipf_bf16", T=1000, D=512, DH=320),
    "relu_top1_cap": spec("switch_top1_cap_bf16", T=1500, D=256, DH=512),
    "relu_e24_k3": spec("switch_top1_cap_bf16", T=901, D=192, DH=256, E=24, top_k=3,
                        capacity_factor=0.0),
}


@pytest.mark.parametrize("renormalise", [True, False], ids=["renorm", "probs"])
@pytest.mark.parametrize("name", sorted(IMPORTANCE_CASES))
def test_importance_loss_without_noise(name, renormalise):
    """The importance loss (Sparsely-Gated Layer page, the importance loss: CV^2 of the
    per-expert gate sums) on the plain router, compact layout, with and without renormalised
    gates, at shapes the single-launch exact route takes (bf16, 8 to 64 experts): routing,
    placement and outputs as for the plain layer, the loss within its bar."""
    sp = IMPORTANCE_CASES[name]
    _say(f"[gpu] importance without noise {name} renormalise={renormalise} {sp}")
    I = make_inputs(sp, seed=21)
    g, r = run_forward_ex(I, renormalise=renormalise), run_oracle_ex(I, renormalise=renormalise)
    check_route(g, r)
    assert np.array_equal(g["expert_offsets"], r["offsets"])
    assert np.array_equal(g["slot_row"], r["slot_row"])
    assert max_abs_rel(g["out"], r["output"]) <= OUT_TOL[sp.dtype]


@pytest.mark.parametrize("name", ["relu_top1_cap", "swiglu_zipf_cap2", "relu_f32_cap"])
def test_dispatch_padded_stage(name):
    """moe_dispatch_padded alone: perm (with -1 for empty rows), slot_row and batch starts
    bit-exact; x_pad holds each kept slot's token row exactly and zero rows elsewhere."""
    import torch
    from expert_ffn_layer_router_amd import binding as B
    sp = PADDED_CASES[name]
    I = make_inputs(sp, seed=14)
    r = run_oracle_ex(I)
    cap = r["capacity"]
    pad = oracle.padded_layout(r, sp.E, cap)
    p = B.Problem.from_spec(sp)
    o = B.Options(padded=True)
    ws = B.alloc_workspace(p, o=o)
    i32 = torch.int32
    idx = torch.from_numpy(r["expert_indices"].astype(np.int32)).cuda()
    x = to_dev(I.x)
    counts = torch.empty(sp.E, dtype=i32, device="cuda")
    offs = torch.empty(sp.E + 1, dtype=i32, device="cuda")
    perm = torch.full((max(sp.E * cap, 1),), -7, dtype=i32, device="cuda")
    slot_row = torch.empty(sp.T * sp.top_k, dtype=i32, device="cuda")
    x_pad = torch.full((max(sp.E * cap, 1), sp.D), 3.0, dtype=x.dtype, device="cuda")
    B.moe_dispatch_padded(p, idx, x, counts, offs, perm, slot_row, x_pad, ws)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(counts), r["counts"])
    assert np.array_equal(to_host(offs), np.arange(sp.E + 1) * cap)
    assert np.array_equal(to_host(perm)[:sp.E * cap], pad["perm_padded"])
    assert np.array_equal(to_host(slot_row), pad["slot_row_padded"])
    xp = to_host(x_pad)[:sp.E * cap]
    xv = I.values("x")
    kept = pad["perm_padded"] >= 0
    assert np.array_equal(xp[kept], xv[pad["perm_padded"][kept] // sp.top_k])
    assert (xp[~kept] == 0).all()


FULL_ROUTE = {
    "mixtral_noisy": ("mixtral_swiglu_bf16", True),
    "mixtral_noisy_probs": ("mixtral_swiglu_bf16", False),
    "zipf_noisy": ("fine_grained_zipf_bf16", True),
}


@pytest.mark.parametrize("case", sorted(FULL_ROUTE))
def test_noisy_route_full_size(case):
    """moe_route_ex at the full layer sizes: every token's choices bit-exact, every gate,
    the Switch loss and the importance loss within their bars (routing only: the oracle's
    float64 router covers all tokens in seconds)."""
    import torch
    from expert_ffn_layer_router_amd import binding as B
    name, renorm = FULL_ROUTE[case]
    sp = spec(name)
    _say(f"[gpu] full-size noisy route {case} {sp}")
    I = make_inputs(sp, seed=0)
    N = make_router_noise(sp, seed=0)
    p = B.Problem.from_spec(sp)
    imp = torch.zeros(1, dtype=torch.float32, device="cuda")
    o = _options(B, N, renorm, False, imp)
    ws = B.alloc_workspace(p, o=o)
    i32 = torch.int32
    idx = torch.empty((sp.T, sp.top_k), dtype=i32, device="cuda")
    gates = torch.empty((sp.T, sp.top_k), dtype=torch.float32, device="cuda")
    aux = torch.empty(1, dtype=torch.float32, device="cuda")
    counts = torch.empty(sp.E, dtype=i32, device="cuda")
    unc = torch.zeros(1, dtype=i32, device="cuda")
    B.moe_route_ex(p, o, to_dev(I.x), to_dev(I.w_router), to_dev(I.bias), idx, gates, aux,
                   counts, None, unc, ws)
    torch.cuda.synchronize()
    logits = oracle.noisy_router_logits(I.values("x"), I.values("w_router"), I.bias,
                                        N.w_values(), N.noise)
    probs = oracle.softmax_rows(logits)
    ridx = oracle.top_k_sorted(logits, sp.top_k)
    rg = (oracle.gates_from_logits(logits, ridx) if renorm
          else oracle.gates_from_probs(probs, ridx))
    _say(f"  recomputed exactly: {int(unc.cpu()[0])} of {sp.T} tokens")
    assert np.array_equal(to_host(idx), ridx)
    assert np.array_equal(to_host(counts), np.bincount(ridx.ravel(), minlength=sp.E))
    assert rel_err(to_host(gates), rg) <= GATE_TOL
    assert rel_err(to_host(aux)[0], oracle.switch_aux_loss(ridx, probs, sp.E)) <= AUX_TOL
    c = oracle.importance_loss(ridx, rg, sp.E)
    assert abs(float(imp.cpu()[0]) - c) <= importance_tol(c)
    if _exact_noisy_route(sp):
        assert int(unc.cpu()[0]) == 0
    elif not renorm:
        assert int(unc.cpu()[0]) == sp.T


def test_options_with_no_tokens():
    import torch
    from expert_ffn_layer_router_amd import binding as B
    sp = spec("mixtral_swiglu_bf16", T=0, D=64, DH=64)
    p = B.Problem.from_spec(sp)
    imp = torch.full((1,), 5.0, dtype=torch.float32, device="cuda")
    w_noise = torch.zeros((sp.D, sp.E), dtype=torch.bfloat16, device="cuda")
    noise = torch.zeros((1, sp.E), dtype=torch.float32, device="cuda")
    o = B.Options(w_noise=w_noise, noise=noise, importance_loss=imp)
    ws = B.alloc_workspace(p, o=o)
    I = make_inputs(spec("mixtral_swiglu_bf16", T=1, D=64, DH=64))
    d = device_inputs(I)
    outs = B.alloc_outputs(p)
    B.moe_forward_ex(p, o, d["x"], d["w_router"], d["bias"], d["w1"], d["w3"], d["w2"],
                     outs["out"], outs["expert_indices"], outs["gates"], outs["aux_loss"],
                     outs["expert_counts"], outs["expert_offsets"], outs["slot_row"], ws)
    torch.cuda.synchronize()
    assert float(imp.cpu()[0]) == 0.0 and float(outs["aux_loss"].cpu()[0]) == 0.0
    assert (to_host(outs["expert_counts"]) == 0).all()
