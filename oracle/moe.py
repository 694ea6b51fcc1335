"""Plain NumPy float64 reference of the top-k MoE layer forward.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing on the product
path imports this module.

Every input is widened exactly to float64 (float32 and bfloat16 values are all
exactly representable), and every step below is computed in float64 in the
order the pages give it. The top-k decision is therefore taken on float64
logits, the precision of the pages' own NumPy code.

Steps, with the passage each follows:

1. router logits ``x @ W_router`` (+ optional per-expert bias) --
   ML Grind "Mixture-of-Experts (MoE) Routing", Algorithm step 1; the bias is
   the ``bias`` argument of ``router()`` in "Mixture of Experts: the
   Sparsely-Gated Layer", section "The code", stage (1) SCORE.
2. ``probs = softmax(logits)`` per row, max-subtracted -- ML Grind, Algorithm
   step 1; the max subtraction as in Bendersky's ``softmax_lastdim``.
3. top-k experts by descending logit, ties to the lower expert index (a
   stable sort of the negated logits) -- ML Grind, Algorithm step 2 and "Edge
   cases and conventions".
4. gates = softmax over the k chosen logits -- ML Grind, Algorithm step 2.
   (Equal to renormalised probabilities: Sparsely-Gated Layer, "The one
   formula", KeepTopK/softmax row.)
5. Switch loss ``aux = E * sum_e f_e * P_e`` with ``f_e`` the share of the T*k
   routing slots that chose e and ``P_e`` the mean router probability --
   ML Grind, Algorithm, load-balancing step.
6. capacity ``floor(capacity_factor * T * k / E)``; per expert, the routed
   tokens in ascending token order, the first ``capacity`` kept and the rest
   dropped ("first come, first served") -- ML Grind, Follow-up; Sparsely-Gated
   Layer, "Switch: top-1, one loss, and a rate limit" and ``moe_forward`` in
   "The code".
7. each expert runs only on its kept tokens; outputs added back weighted by
   their gate, dropped slots add nothing and gates are not renormalised after
   a drop -- ML Grind, Algorithm step 3 and "Constraints"; Sparsely-Gated
   Layer, ``moe_forward``.

Backward (``moe_backward``): the gradients of ``sum(out * dout) + d_aux * aux``
with respect to x, the router and the experts, by the chain rule through the steps
above in reverse; the decisions are piecewise constant, so the gradient flows through
the gates and through P in the Switch loss, and f (a count) has none (Sparsely-Gated
Layer, "Hot shards"). Pinned by central finite differences of ``moe_forward``.

Router options (Sparsely-Gated Layer, "The one formula" and "The code",
``router()`` stages (2) and (5); "Hot shards: the load-balancing loss"):

* noise: ``logits + noise * softplus(x @ W_noise)``, with the standard-normal
  draw ``noise`` (T, E) given as an input so that both sides use the same one;
  probabilities, top-k and gates are then taken from the noisy logits.
* ``renormalise=False``: the gates are the chosen experts' probabilities
  over all E experts, without the division by their sum.
* importance loss: ``importance_e`` = the sum over tokens of expert e's gate
  (zero where e was not chosen); the loss is its squared coefficient of
  variation, (population standard deviation / mean)^2; 0 when T = 0.
* padded layout (Switch capacity, "Switch: top-1, one loss, and a rate
  limit": experts run as fixed-size batches): expert e's kept slots at rows
  ``e * capacity + rank``, the other rows of its batch empty.

Experts: linear ``x @ W`` (ML Grind, Background), two-layer ReLU
``relu(x @ Wh) @ Wo`` without biases (Sparsely-Gated Layer ``expert_forward``;
Bendersky ``FFParams``), and SwiGLU ``(silu(x @ W1) * (x @ W3)) @ W2`` with
``silu(z) = z / (1 + exp(-z))`` (ML Grind, Background names SwiGLU experts; the
form is the textbook one).

Pins (the ``-m "not gpu"`` tests): the three worked examples of ML Grind, the
top_k = 1 convention, the token-0 gates printed on the Sparsely-Gated Layer
page (renormalised and not), its capacity/drop table and its importance-loss
values, softplus and noise closed forms, the k = E and uniform-router closed forms,
identity-weight closed forms of each expert, permutation equivariance, and a
second, per-token implementation (``moe_forward_per_token``) on tiny random
inputs. There is no printed worked example of the absolute output values at
the large configurations; those are covered by the structural pins only.
"""

from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


# --- routing -----------------------------------------------------------------

def router_logits(x, w_router, bias=None) -> np.ndarray:
    """Step 1: ``x @ W_router`` (+ bias), float64, (T, E)."""
    logits = _f64(x) @ _f64(w_router)
    if bias is not None:
        logits = logits + _f64(bias)[None, :]
    return logits


def softmax_rows(z: np.ndarray) -> np.ndarray:
    """Step 2: row softmax with the row maximum subtracted first."""
    z = _f64(z)
    m = z.max(axis=-1, keepdims=True)
    ez = np.exp(z - m)
    return ez / ez.sum(axis=-1, keepdims=True)


def top_k_sorted(logits: np.ndarray, k: int) -> np.ndarray:
    """Step 3: the k largest logits per row, best first, ties -> lower index."""
    order = np.argsort(-_f64(logits), axis=-1, kind="stable")
    return order[:, :k].astype(np.int64)


def gates_from_logits(logits: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Step 4: softmax over the k chosen logits, aligned with ``idx``."""
    chosen = np.take_along_axis(_f64(logits), idx, axis=-1)
    return softmax_rows(chosen)


def switch_aux_loss(idx: np.ndarray, probs: np.ndarray, E: int) -> float:
    """Step 5: ``E * sum_e f_e * P_e``; f counts routed slots before capacity."""
    T, k = idx.shape
    counts = np.bincount(idx.ravel(), minlength=E).astype(np.float64)
    f = counts / (T * k)
    P = _f64(probs).mean(axis=0)
    return float(E * np.sum(f * P))


# --- router options: noise, renormalisation, importance loss ----------------------------

def softplus(z):
    """``log(1 + e^z)``, without overflow (``logaddexp(0, z)``)."""
    return np.logaddexp(0.0, _f64(z))


def noisy_router_logits(x, w_router, bias=None, w_noise=None, noise=None) -> np.ndarray:
    """Router logits plus ``noise * softplus(x @ W_noise)`` (Sparsely-Gated Layer, "The
    one formula", the + noise row; ``router()`` stage (2)). ``noise`` is the (T, E)
    standard-normal draw. Without ``w_noise`` these are the plain logits."""
    logits = router_logits(x, w_router, bias)
    if w_noise is None:
        return logits
    return logits + _f64(noise) * softplus(_f64(x) @ _f64(w_noise))


def gates_from_probs(probs: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """``renormalise=False``: the chosen experts' probabilities over all experts, aligned
    with ``idx`` (``router()`` without stage (5))."""
    return np.take_along_axis(_f64(probs), idx, axis=-1)


def importance_loss(idx: np.ndarray, gates: np.ndarray, E: int) -> float:
    """Shazeer's importance loss: CV^2 of the per-expert sums of the gate values
    (Sparsely-Gated Layer, "Hot shards"; ``importance_loss()``). The dense gate matrix
    is zero off the chosen experts, so expert e's sum runs over the slots that chose e.
    Population standard deviation; 0 when no slot was routed."""
    imp = np.bincount(np.asarray(idx).ravel(), weights=_f64(gates).ravel(), minlength=E)
    mean = imp.mean()
    if mean == 0.0:
        return 0.0
    return float(imp.std() ** 2 / mean ** 2)


# --- dispatch ----------------------------------------------------------------

def capacity_slots(capacity_factor: float, T: int, k: int, E: int) -> Optional[int]:
    """Step 6: ``floor(capacity_factor * T * k / E)``; None when there is no limit."""
    if capacity_factor is None or capacity_factor <= 0:
        return None
    return int(math.floor(capacity_factor * T * k / E))


def dispatch_from_indices(idx: np.ndarray, E: int, capacity: Optional[int]) -> dict:
    """Step 6: per-expert counts, kept slots, expert-contiguous order.

    Returns ``counts`` (E,) routed slots before capacity, ``kept`` (E,),
    ``offsets`` (E+1,) exclusive prefix sum of ``kept``, ``perm`` (R,) the kept
    slot ids ``t*k + j`` in (expert, token) order, ``slot_row`` (T*k,) the row
    of each slot in that order or -1 when dropped, and ``dropped``.
    """
    idx = np.asarray(idx)
    T, k = idx.shape
    flat = idx.reshape(-1).astype(np.int64)  # slot s = t*k + j chose expert flat[s]
    # Group the slots by expert with a stable sort: within one expert the slot ids, and so
    # the token indices (a token picks an expert at most once), stay ascending.
    order = np.argsort(flat, kind="stable")
    counts = np.bincount(flat, minlength=E).astype(np.int64)
    start = np.concatenate([[0], np.cumsum(counts)])
    # rank of each slot among the slots of its expert, in token order
    rank = np.empty(T * k, dtype=np.int64)
    rank[order] = np.arange(T * k) - start[flat[order]]
    # capacity keeps the `capacity` earliest tokens of each expert and drops the rest
    keep = np.ones(T * k, dtype=bool) if capacity is None else rank < capacity
    kept = np.bincount(flat[keep], minlength=E).astype(np.int64)
    perm = order[keep[order]]  # kept slots in (expert, token) order
    offsets = np.concatenate([[0], np.cumsum(kept)]).astype(np.int64)
    slot_row = np.full(T * k, -1, dtype=np.int64)
    slot_row[perm] = np.arange(perm.size)
    return dict(counts=counts, kept=kept, offsets=offsets, perm=perm, slot_row=slot_row,
                dropped=int(T * k - perm.size))


def padded_layout(disp: dict, E: int, capacity: int) -> dict:
    """Capacity-padded rows: expert e's batch is rows ``e*capacity .. (e+1)*capacity-1``,
    its kept slots first in token order, the rest of the batch empty. Returns
    ``slot_row_padded`` (T*k,) the padded row of each slot or -1 when dropped, and
    ``perm_padded`` (E*capacity,) the slot of each row or -1 for an empty row."""
    slot_row = np.asarray(disp["slot_row"])
    perm_padded = np.full(E * capacity, -1, dtype=np.int64)
    for e in range(E):
        seg = disp["perm"][disp["offsets"][e]:disp["offsets"][e + 1]]
        perm_padded[e * capacity:e * capacity + seg.size] = seg
    slot_row_padded = np.full(slot_row.size, -1, dtype=np.int64)
    rows = np.flatnonzero(perm_padded >= 0)
    slot_row_padded[perm_padded[rows]] = rows
    return dict(slot_row_padded=slot_row_padded, perm_padded=perm_padded)


# --- experts -----------------------------------------------------------------

def silu(z):
    """``z * sigmoid(z) = z / (1 + exp(-z))``."""
    z = _f64(z)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def expert_forward(kind: str, xr: np.ndarray, w1, w2=None, w3=None) -> np.ndarray:
    """One expert on the rows ``xr``; the weights are that expert's matrices."""
    xr = _f64(xr)
    if kind == "linear":
        return xr @ _f64(w1)
    if kind == "relu2":
        return np.maximum(xr @ _f64(w1), 0.0) @ _f64(w2)
    if kind == "swiglu":
        return (silu(xr @ _f64(w1)) * (xr @ _f64(w3))) @ _f64(w2)
    raise ValueError(f"unknown expert kind {kind!r}")


def _expert_weights(e, w1, w2, w3):
    return w1[e], (None if w2 is None else w2[e]), (None if w3 is None else w3[e])


# --- the layer ----------------------------------------------------------------

def moe_forward(x, w_router, top_k: int, kind: str, w1, w2=None, w3=None, bias=None,
                capacity_factor: float = 0.0, tokens: Optional[Sequence[int]] = None,
                w_noise=None, noise=None, renormalise: bool = True) -> dict:
    """The layer forward, steps 1-7, with the router options above.

    ``w1``/``w3`` are (E, D, DH) (``w1`` is (E, D, D_out) for a linear expert),
    ``w2`` is (E, DH, D_out). Expert weights are widened to float64 one expert
    at a time. ``tokens`` restricts the expert evaluation (step 7) to those
    token rows; routing, dispatch and the loss always cover every token, since
    which slots an expert keeps depends on all earlier tokens. Rows not in
    ``tokens`` are left zero.
    """
    x = np.asarray(x)
    T = x.shape[0]
    E = np.asarray(w_router).shape[1]
    if not 1 <= top_k <= E:
        raise ValueError("top_k must satisfy 1 <= top_k <= E")
    logits = noisy_router_logits(x, w_router, bias, w_noise, noise)
    probs = softmax_rows(logits)
    idx = top_k_sorted(logits, top_k)
    gates = gates_from_logits(logits, idx) if renormalise else gates_from_probs(probs, idx)
    aux = switch_aux_loss(idx, probs, E)
    imp = importance_loss(idx, gates, E)
    cap = capacity_slots(capacity_factor, T, top_k, E)
    disp = dispatch_from_indices(idx, E, cap)

    d_out = np.asarray(w1).shape[2] if kind == "linear" else np.asarray(w2).shape[2]
    out = np.zeros((T, d_out), dtype=np.float64)
    want = None
    if tokens is not None:
        want = np.zeros(T, dtype=bool)
        want[np.asarray(tokens, dtype=np.int64)] = True
    flat_gates = gates.reshape(-1)
    for e in range(E):
        rows = disp["perm"][disp["offsets"][e]:disp["offsets"][e + 1]]  # slot ids
        if want is not None:
            rows = rows[want[rows // top_k]]
        if rows.size == 0:
            continue
        t = rows // top_k
        y = expert_forward(kind, x[t], *_expert_weights(e, w1, w2, w3))
        # one slot per (token, expert), so no two rows of t repeat here
        out[t] += flat_gates[rows][:, None] * y
    return dict(output=out, expert_indices=idx, gates=gates, aux_loss=aux, logits=logits,
                probs=probs, capacity=cap, importance_loss=imp, **disp)


# --- backward -------------------------------------------------------------------------

def silu_grad(z):
    """d silu / dz = sigma(z) * (1 + z * (1 - sigma(z)))."""
    z = _f64(z)
    with np.errstate(over="ignore"):
        sig = 1.0 / (1.0 + np.exp(-z))
    return sig * (1.0 + z * (1.0 - sig))


def expert_backward(kind: str, xr: np.ndarray, dy: np.ndarray, w1, w2=None, w3=None) -> dict:
    """Gradients of one expert on its rows: given dL/dy for y = expert(x), returns dL/dx
    and dL/dW for each of its matrices (chain rule through the forms of expert_forward;
    relu'(0) is taken as 0)."""
    xr, dy = _f64(xr), _f64(dy)
    if kind == "linear":
        W = _f64(w1)
        return dict(dx=dy @ W.T, dw1=xr.T @ dy)
    W1, W2 = _f64(w1), _f64(w2)
    a = xr @ W1
    if kind == "relu2":
        h = np.maximum(a, 0.0)
        dh = dy @ W2.T
        da = dh * (a > 0.0)
        return dict(dx=da @ W1.T, dw1=xr.T @ da, dw2=h.T @ dy)
    if kind == "swiglu":
        W3 = _f64(w3)
        b = xr @ W3
        h = silu(a) * b
        dh = dy @ W2.T
        da = dh * b * silu_grad(a)
        db = dh * silu(a)
        return dict(dx=da @ W1.T + db @ W3.T, dw1=xr.T @ da, dw3=xr.T @ db, dw2=h.T @ dy)
    raise ValueError(f"unknown expert kind {kind!r}")


def moe_backward(x, w_router, top_k: int, kind: str, w1, w2=None, w3=None, bias=None,
                 capacity_factor: float = 0.0, dout=None, d_aux: float = 0.0,
                 tokens: Optional[Sequence[int]] = None) -> dict:
    """Gradients of L = sum(out * dout) + d_aux * aux_loss with respect to x, the router
    (weights and bias) and every expert matrix, for the layer of moe_forward (no router
    noise, renormalised gates).

    The routing decisions (top-k and the drop set) are piecewise constant, so the gradient
    flows through the gates and through P in the Switch loss; f (a count) has none
    (f_e is a step function of the logits, so only P_e carries gradient: ML Grind, the
    load-balancing step; Sparsely-Gated Layer, Hot shards).
    In reverse order: the combine gives dL/dgate = <dout_t, y_e(x_t)> for a kept slot (0 for
    a dropped one) and dL/dy = gate * dout_t; each expert's backward on its kept rows; the
    gates' softmax over the k chosen logits; the loss through P_e = mean_t probs[t, e] and
    the full softmax; the router product logits = x @ W_router + bias.

    ``tokens`` restricts the work to those tokens' rows: their dx, dgates and dlogits rows
    are exact (routing, drops and f still cover every token) and every other row is zero;
    the weight gradients then hold only those tokens' share."""
    r = moe_forward(x, w_router, top_k, kind, w1, w2, w3, bias=bias,
                    capacity_factor=capacity_factor, tokens=tokens)
    x = _f64(x)
    T, D = x.shape
    E = np.asarray(w_router).shape[1]
    dout = _f64(dout)
    idx, gates, probs = r["expert_indices"], r["gates"], r["probs"]
    dgates = np.zeros_like(gates)
    dx = np.zeros_like(x)
    dw1 = np.zeros(np.asarray(w1).shape)
    dw2 = None if w2 is None else np.zeros(np.asarray(w2).shape)
    dw3 = None if w3 is None else np.zeros(np.asarray(w3).shape)
    flat_gates = gates.reshape(-1)
    want = np.ones(T, dtype=bool)
    if tokens is not None:
        want = np.zeros(T, dtype=bool)
        want[np.asarray(tokens, dtype=np.int64)] = True
    for e in range(E):
        rows = r["perm"][r["offsets"][e]:r["offsets"][e + 1]]  # kept slot ids of e
        rows = rows[want[rows // top_k]]
        if rows.size == 0:
            continue
        t = rows // top_k
        we = _expert_weights(e, w1, w2, w3)
        y = expert_forward(kind, x[t], *we)
        dgates.reshape(-1)[rows] = np.einsum("rd,rd->r", dout[t], y)
        g = expert_backward(kind, x[t], flat_gates[rows][:, None] * dout[t], *we)
        np.add.at(dx, t, g["dx"])
        dw1[e] += g["dw1"]
        if dw2 is not None:
            dw2[e] += g["dw2"]
        if dw3 is not None:
            dw3[e] += g["dw3"]
    # gates = softmax(chosen logits): dl_c = g_c * (dg_c - sum_c' g_c' dg_c')
    dl = np.zeros((T, E))
    dl_chosen = gates * (dgates - (gates * dgates).sum(axis=1, keepdims=True))
    np.add.at(dl, (np.arange(T)[:, None].repeat(top_k, 1), idx), dl_chosen)
    # aux = E * sum_e f_e * P_e with P_e = mean_t probs[t, e]: dL/dprobs[t, e] = d_aux E f_e / T
    if T > 0:
        f = np.bincount(idx.ravel(), minlength=E) / (T * top_k)
        a = d_aux * E * f / T
        dl += probs * (a[None, :] - (probs * a[None, :]).sum(axis=1, keepdims=True))
    dl[~want] = 0.0
    dw_router = x.T @ dl
    dbias = dl.sum(axis=0)
    dx += dl @ _f64(w_router).T
    return dict(dx=dx, dw_router=dw_router, dbias=dbias, dw1=dw1, dw2=dw2, dw3=dw3,
                dgates=dgates, dlogits=dl, forward=r)


def _expert_one_token(kind: str, xt: np.ndarray, w1, w2=None, w3=None) -> np.ndarray:
    """One expert on one token, column by column (vector dot products only)."""
    def vecmat(v, W):
        W = _f64(W)
        return np.array([float(np.dot(v, W[:, c])) for c in range(W.shape[1])])

    if kind == "linear":
        return vecmat(xt, w1)
    if kind == "relu2":
        h = np.array([max(v, 0.0) for v in vecmat(xt, w1)])
        return vecmat(h, w2)
    if kind == "swiglu":
        a = vecmat(xt, w1)
        g = vecmat(xt, w3)
        h = np.array([(ai / (1.0 + math.exp(-ai)) if ai > -700 else 0.0) * gi
                      for ai, gi in zip(a, g)])
        return vecmat(h, w2)
    raise ValueError(f"unknown expert kind {kind!r}")


def _softplus_scalar(z: float) -> float:
    return z + math.log1p(math.exp(-z)) if z > 0 else math.log1p(math.exp(z))


def moe_forward_per_token(x, w_router, top_k: int, kind: str, w1, w2=None, w3=None, bias=None,
                          capacity_factor: float = 0.0, w_noise=None, noise=None,
                          renormalise: bool = True) -> dict:
    """A second, independent implementation: token by token, plain Python.

    The shape of Bendersky's ``moe`` loop ("A Minimal Numpy Implementation")
    and of ML Grind's ``y_t = sum_j gates[t, j] * expert(x_t)``. The top-k uses
    Python's ``sorted`` with an explicit (-logit, index) key, the softmaxes use
    ``math.exp``, and a slot is kept when fewer than ``capacity`` earlier
    tokens chose the same expert. For tiny inputs only.
    """
    x = _f64(x)
    W = _f64(w_router)
    T, _ = x.shape
    E = W.shape[1]
    b = np.zeros(E) if bias is None else _f64(bias)
    rows_idx, rows_gate, rows_prob = [], [], []
    for t in range(T):
        logit = [float(np.dot(x[t], W[:, e])) + float(b[e]) for e in range(E)]
        if w_noise is not None:
            Wn, eps = _f64(w_noise), _f64(noise)
            logit = [logit[e] + float(eps[t, e]) * _softplus_scalar(float(np.dot(x[t], Wn[:, e])))
                     for e in range(E)]
        order = sorted(range(E), key=lambda e: (-logit[e], e))[:top_k]
        m = max(logit)
        ez = [math.exp(v - m) for v in logit]
        s = sum(ez)
        rows_prob.append([v / s for v in ez])
        rows_idx.append(order)
        if renormalise:
            mk = max(logit[e] for e in order)
            gz = [math.exp(logit[e] - mk) for e in order]
            gs = sum(gz)
            rows_gate.append([v / gs for v in gz])
        else:
            rows_gate.append([rows_prob[t][e] for e in order])
    counts = [0] * E
    for order in rows_idx:
        for e in order:
            counts[e] += 1
    P = [sum(rows_prob[t][e] for t in range(T)) / T for e in range(E)]
    aux = E * sum((counts[e] / (T * top_k)) * P[e] for e in range(E))
    imp = [0.0] * E
    for t in range(T):
        for j, e in enumerate(rows_idx[t]):
            imp[e] += rows_gate[t][j]
    mean_imp = sum(imp) / E
    var_imp = sum((v - mean_imp) ** 2 for v in imp) / E
    importance = var_imp / mean_imp ** 2 if mean_imp > 0 else 0.0

    cap = None
    if capacity_factor and capacity_factor > 0:
        cap = int(math.floor(capacity_factor * T * top_k / E))
    seen = [0] * E
    kept = [[False] * top_k for _ in range(T)]
    for t in range(T):
        for j, e in enumerate(rows_idx[t]):
            kept[t][j] = cap is None or seen[e] < cap
            seen[e] += 1

    d_out = np.asarray(w1).shape[2] if kind == "linear" else np.asarray(w2).shape[2]
    out = np.zeros((T, d_out))
    for t in range(T):
        for j, e in enumerate(rows_idx[t]):
            if kept[t][j]:
                y = _expert_one_token(kind, x[t], *_expert_weights(e, w1, w2, w3))
                out[t] += rows_gate[t][j] * y
    return dict(output=out, expert_indices=np.array(rows_idx, dtype=np.int64),
                gates=np.array(rows_gate), aux_loss=float(aux), importance_loss=float(importance),
                counts=np.array(counts, dtype=np.int64),
                kept_mask=np.array(kept, dtype=bool))
