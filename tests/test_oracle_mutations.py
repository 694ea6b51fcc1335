"""Plant plausible mistakes in the CPU oracle and check that some pin fails.

Each mutation replaces one step of ``oracle.moe`` (on the CPU, inside this test
only) with a plausible wrong version: a flipped tie-break, a missing term, a
wrong normaliser, a transposed operand, a wrong drop order. The pins must not
all pass against any of them.
"""

import math

import numpy as np
import pytest

import oracle_pins
from oracle import moe as O


def _ties_to_higher_index(logits, k):
    z = np.asarray(logits, dtype=np.float64)[:, ::-1]
    order = np.argsort(-z, axis=-1, kind="stable")
    return (z.shape[1] - 1 - order)[:, :k]


def _ascending(logits, k):
    return np.argsort(np.asarray(logits, dtype=np.float64), axis=-1, kind="stable")[:, :k]


def _gates_not_renormalised(logits, idx):
    return np.take_along_axis(O.softmax_rows(logits), idx, axis=-1)


def _f_over_T(idx, probs, E):
    T, k = idx.shape
    counts = np.bincount(idx.ravel(), minlength=E)
    return float(E * np.sum(counts / T * np.asarray(probs).mean(axis=0)))


def _P_from_max_prob(idx, probs, E):
    T, k = idx.shape
    counts = np.bincount(idx.ravel(), minlength=E)
    P = np.asarray(probs).max(axis=0)
    return float(E * np.sum(counts / (T * k) * P))


def _capacity_ceil(cf, T, k, E):
    if cf is None or cf <= 0:
        return None
    return int(math.ceil(cf * T * k / E))


def _no_bias(x, w, bias=None):
    return np.asarray(x, dtype=np.float64) @ np.asarray(w, dtype=np.float64)


_orig_dispatch = O.dispatch_from_indices


def _keep_last(idx, E, capacity):
    """Drops the first tokens of an overflowing expert instead of the last ones."""
    idx = np.asarray(idx)
    T, k = idx.shape
    rev = _orig_dispatch(idx[::-1], E, capacity)
    slot_row_rev = rev["slot_row"].reshape(T, k)[::-1].reshape(-1)
    kept = slot_row_rev >= 0
    out = _orig_dispatch(idx, E, None)
    perm = [s for s in out["perm"] if kept[s]]
    perm = np.array(perm, dtype=np.int64)
    slot_row = np.full(T * k, -1, dtype=np.int64)
    slot_row[perm] = np.arange(perm.size)
    return dict(out, kept=rev["kept"], offsets=rev["offsets"], perm=perm, slot_row=slot_row,
                dropped=int(T * k - perm.size))


def _slot_major_perm(idx, E, capacity):
    """Orders an expert's rows by (rank j, token) instead of by token."""
    out = _orig_dispatch(idx, E, capacity)
    k = np.asarray(idx).shape[1]
    perm = out["perm"].copy()
    for e in range(E):
        seg = perm[out["offsets"][e]:out["offsets"][e + 1]]
        perm[out["offsets"][e]:out["offsets"][e + 1]] = seg[np.lexsort((seg // k, seg % k))]
    slot_row = np.full_like(out["slot_row"], -1)
    slot_row[perm] = np.arange(perm.size)
    return dict(out, perm=perm, slot_row=slot_row)


_orig_expert = O.expert_forward


def _swiglu_swapped(kind, xr, w1, w2=None, w3=None):
    if kind == "swiglu":
        return _orig_expert(kind, xr, w3, w2, w1)
    return _orig_expert(kind, xr, w1, w2, w3)


def _transposed_second(kind, xr, w1, w2=None, w3=None):
    """Applies the second matrix transposed (only expressible when it is square)."""
    if kind != "linear" and np.asarray(w2).shape[0] == np.asarray(w2).shape[1]:
        return _orig_expert(kind, xr, w1, np.asarray(w2).T, w3)
    return _orig_expert(kind, xr, w1, w2, w3)


def _silu_wrong_sign(z):
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(z))


def _relu_as_abs(kind, xr, w1, w2=None, w3=None):
    if kind == "relu2":
        return np.abs(np.asarray(xr, float) @ np.asarray(w1, float)) @ np.asarray(w2, float)
    return _orig_expert(kind, xr, w1, w2, w3)


_orig_forward = O.moe_forward


def _drops_ignored_in_output(*a, **kw):
    cf = kw.pop("capacity_factor", 0.0)
    r = _orig_forward(*a, **kw)
    if cf and cf > 0:
        r2 = _orig_forward(*a, capacity_factor=cf, **kw)
        r = dict(r2, output=r["output"])
    return r


def _renormalise_after_drop(*a, **kw):
    r = _orig_forward(*a, **kw)
    T, k = r["gates"].shape
    kept = (r["slot_row"].reshape(T, k) >= 0)
    if kept.all():
        return r
    # rescale each token's output by 1 / (sum of its kept gates)
    s = (r["gates"] * kept).sum(axis=1)
    scale = np.where(s > 0, 1.0 / np.where(s > 0, s, 1.0), 0.0)
    return dict(r, output=r["output"] * scale[:, None])


def _softplus_is_exp(z):
    return np.exp(np.asarray(z, dtype=np.float64))


_orig_noisy = O.noisy_router_logits


def _noise_unscaled(x, w_router, bias=None, w_noise=None, noise=None):
    base = O.router_logits(x, w_router, bias)
    return base if w_noise is None else base + np.asarray(noise, dtype=np.float64)


def _noise_scale_transposed(x, w_router, bias=None, w_noise=None, noise=None):
    """Reads W_noise's transpose where it is square (x @ W_noise^T)."""
    if w_noise is not None and np.asarray(w_noise).shape[0] == np.asarray(w_noise).shape[1]:
        return _orig_noisy(x, w_router, bias, np.asarray(w_noise).T, noise)
    return _orig_noisy(x, w_router, bias, w_noise, noise)


def _importance_sample_std(idx, gates, E):
    imp = np.bincount(np.asarray(idx).ravel(), weights=np.asarray(gates, float).ravel(),
                      minlength=E)
    return 0.0 if imp.mean() == 0 else float(imp.std(ddof=1) ** 2 / imp.mean() ** 2)


def _importance_cv_not_squared(idx, gates, E):
    imp = np.bincount(np.asarray(idx).ravel(), weights=np.asarray(gates, float).ravel(),
                      minlength=E)
    return 0.0 if imp.mean() == 0 else float(imp.std() / imp.mean())


def _importance_from_counts(idx, gates, E):
    imp = np.bincount(np.asarray(idx).ravel(), minlength=E).astype(float)
    return 0.0 if imp.mean() == 0 else float(imp.std() ** 2 / imp.mean() ** 2)


def _probs_renormalised_anyway(probs, idx):
    p = np.take_along_axis(np.asarray(probs, dtype=np.float64), idx, axis=-1)
    return p / p.sum(axis=-1, keepdims=True)


def _silu_grad_sigma_only(z):
    z = np.asarray(z, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-z))


_orig_backward = O.moe_backward


def _backward_without_loss_term(*a, **kw):
    kw["d_aux"] = 0.0
    return _orig_backward(*a, **kw)


_orig_expert_backward = O.expert_backward


def _expert_backward_w2_untransposed(kind, xr, dy, w1, w2=None, w3=None):
    """Uses dy @ W2 instead of dy @ W2^T for dL/dh where the shapes allow it."""
    if w2 is not None and np.asarray(w2).shape[0] == np.asarray(w2).shape[1]:
        return _orig_expert_backward(kind, xr, dy, w1, np.asarray(w2).T, w3)
    g = _orig_expert_backward(kind, xr, dy, w1, w2, w3)
    g["dx"] = -g["dx"]
    return g


MUTATIONS = {
    "ties_to_higher_index": ("top_k_sorted", _ties_to_higher_index),
    "ascending_top_k": ("top_k_sorted", _ascending),
    "gates_not_renormalised": ("gates_from_logits", _gates_not_renormalised),
    "f_normalised_by_T": ("switch_aux_loss", _f_over_T),
    "P_from_max_prob": ("switch_aux_loss", _P_from_max_prob),
    "capacity_rounds_up": ("capacity_slots", _capacity_ceil),
    "bias_dropped": ("router_logits", _no_bias),
    "drops_first_tokens": ("dispatch_from_indices", _keep_last),
    "slot_major_order": ("dispatch_from_indices", _slot_major_perm),
    "swiglu_w1_w3_swapped": ("expert_forward", _swiglu_swapped),
    "second_matrix_transposed": ("expert_forward", _transposed_second),
    "silu_sign_flipped": ("silu", _silu_wrong_sign),
    "relu_is_abs": ("expert_forward", _relu_as_abs),
    "drops_still_contribute": ("moe_forward", _drops_ignored_in_output),
    "gates_renormalised_after_drop": ("moe_forward", _renormalise_after_drop),
    "softplus_is_exp": ("softplus", _softplus_is_exp),
    "noise_without_softplus_scale": ("noisy_router_logits", _noise_unscaled),
    "noise_scale_transposed": ("noisy_router_logits", _noise_scale_transposed),
    "importance_sample_std": ("importance_loss", _importance_sample_std),
    "importance_cv_not_squared": ("importance_loss", _importance_cv_not_squared),
    "importance_from_counts": ("importance_loss", _importance_from_counts),
    "unrenormalised_gates_renormalised": ("gates_from_probs", _probs_renormalised_anyway),
    "silu_grad_sigma_only": ("silu_grad", _silu_grad_sigma_only),
    "backward_without_loss_term": ("moe_backward", _backward_without_loss_term),
    "expert_backward_wrong_dh": ("expert_backward", _expert_backward_w2_untransposed),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_some_pin_catches(name, monkeypatch):
    attr, fake = MUTATIONS[name]
    monkeypatch.setattr(O, attr, fake)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin()
        except Exception:  # an assertion, or a crash on the wrong arithmetic
            failed.append(pin.__name__)
    assert failed, f"mutation {name} passed every pin"
