"""Pins of the CPU oracle: facts fixed by the pages and by mathematics.

Each ``pin_*`` function raises ``AssertionError`` when the oracle disagrees with
the fact it checks. The functions look the oracle's steps up on the
``oracle.moe`` module at call time, so ``test_oracle_mutations.py`` can plant a
mistake there and show that some pin catches it. None of the expected values
comes from the GPU path: each is printed on a page (``tests/golden/``), a closed
form, or an invariant.
"""

from __future__ import annotations

import math

import numpy as np

from oracle import moe as O
from golden_io import load

RNG_SEED = 1234


def _rng(salt=0):
    return np.random.default_rng(RNG_SEED + salt)


def _linear_case(T, d, E, d_out, salt=0):
    r = _rng(salt)
    return (r.standard_normal((T, d)), r.standard_normal((d, E)),
            r.standard_normal((E, d, d_out)))


# --- ML Grind "Mixture-of-Experts (MoE) Routing", section "Examples" -------------------

def pin_mlgrind_example1_shapes():
    g = load("mlgrind_examples.txt")
    x, w, we = _linear_case(g["ex1_T"], g["ex1_d"], g["ex1_E"], g["ex1_d_out"])
    r = O.moe_forward(x, w, g["ex1_top_k"], "linear", we)
    assert list(r["output"].shape) == g["ex1_output_shape"]
    assert list(r["expert_indices"].shape) == g["ex1_indices_shape"]
    assert list(r["gates"].shape) == g["ex1_gates_shape"]
    assert isinstance(r["aux_loss"], float)


def pin_mlgrind_example2_uniform_router():
    """W_router = 0: every P_e = 1/4 exactly and the f_e sum to 1, so aux = 1.0."""
    g = load("mlgrind_examples.txt")
    x, w, we = _linear_case(6, 4, 4, 3, salt=1)
    r = O.moe_forward(x, np.zeros_like(w), g["ex2_top_k"], "linear", we)
    assert r["aux_loss"] == g["ex2_aux_loss"]
    # all logits tie at 0.0: the stable order picks experts 0, 1 with equal gates
    assert (r["expert_indices"] == np.array([0, 1])).all()
    assert (r["gates"] == 0.5).all()
    # the same holds for any top_k and E: aux = E * sum_{e<k} (1/k)(1/E) = 1
    for E in (2, 3, 5, 8):
        for k in range(1, E + 1):
            x, w, we = _linear_case(7, 5, E, 2, salt=10 * E + k)
            r = O.moe_forward(x, np.zeros_like(w), k, "linear", we)
            assert abs(r["aux_loss"] - 1.0) < 1e-14
            assert (r["expert_indices"] == np.arange(k)).all()
            assert np.allclose(r["gates"], 1.0 / k, rtol=0, atol=1e-15)


def pin_mlgrind_example3_collapse():
    """x = ones, the router strongly prefers expert 0, top_k = 1, E = 4: aux = 4.0."""
    g = load("mlgrind_examples.txt")
    T, d, E = g["ex3_T"], g["ex3_d"], g["ex3_E"]
    w = np.zeros((d, E))
    w[:, 0] = 10.0  # logits [40, 0, 0, 0] on every token
    we = _rng(3).standard_normal((E, d, 3))
    r = O.moe_forward(np.ones((T, d)), w, g["ex3_top_k"], "linear", we)
    assert abs(r["aux_loss"] - g["ex3_aux_loss"]) < 1e-6
    assert (r["expert_indices"] == 0).all()
    assert (r["gates"] == 1.0).all()


# --- ML Grind, "Edge cases and conventions" and "Expected Return Format" ----------------

def pin_top1_gate_is_one_and_output_is_the_expert():
    for kind in ("linear", "relu2", "swiglu"):
        r_ = _rng(4)
        T, D, DH, E = 9, 6, 5, 4
        x = r_.standard_normal((T, D))
        w = r_.standard_normal((D, E))
        w1 = r_.standard_normal((E, D, DH if kind != "linear" else 3))
        w3 = r_.standard_normal((E, D, DH)) if kind == "swiglu" else None
        w2 = r_.standard_normal((E, DH, D)) if kind != "linear" else None
        r = O.moe_forward(x, w, 1, kind, w1, w2, w3)
        assert (r["gates"] == 1.0).all()
        logits = x @ w
        assert (r["expert_indices"][:, 0] == logits.argmax(axis=1)).all()
        for t in range(T):
            e = r["expert_indices"][t, 0]
            single = O.expert_forward(kind, x[t:t + 1], w1[e], None if w2 is None else w2[e],
                                      None if w3 is None else w3[e])[0]
            # same math; BLAS may round a one-row product differently from a batch
            assert np.allclose(r["output"][t], single, rtol=1e-13, atol=1e-13)


def pin_gate_rows_and_topk_property():
    """Rows of gates sum to 1; k distinct indices, best first; no unchosen logit beats a chosen one."""
    for (T, D, E, k, salt) in [(40, 7, 8, 3, 5), (33, 16, 16, 5, 6), (20, 4, 3, 3, 7)]:
        r_ = _rng(salt)
        x = r_.standard_normal((T, D))
        w = r_.standard_normal((D, E))
        bias = r_.standard_normal(E)
        we = r_.standard_normal((E, D, 2))
        r = O.moe_forward(x, w, k, "linear", we, bias=bias)
        idx, gates = r["expert_indices"], r["gates"]
        logits = np.einsum("td,de->te", x, w) + bias
        assert np.allclose(gates.sum(axis=1), 1.0, rtol=0, atol=1e-14)
        assert (gates > 0).all()
        for t in range(T):
            assert len(set(idx[t].tolist())) == k
            chosen = logits[t, idx[t]]
            assert (np.diff(chosen) <= 0).all()
            rest = np.delete(logits[t], idx[t])
            if rest.size:
                assert rest.max() <= chosen.min()
            assert (np.diff(gates[t]) <= 1e-15).all()  # aligned with descending logits


# --- "Mixture of Experts: the Sparsely-Gated Layer" ------------------------------------

def pin_token0_renormalised_gates():
    """Token 0 of the page's routing table: experts [6, 3], gates [0.627, 0.373]."""
    g = load("sparsely_gated_token0_gates.txt")
    probs = np.array(g["probs"], dtype=np.float64)
    logits = np.log(probs)[None, :]  # any logits with these softmax ratios
    idx = O.top_k_sorted(logits, g["top_k"])
    gates = O.gates_from_logits(logits, idx)
    assert idx[0].tolist() == g["expert_indices"]
    assert np.round(gates[0], g["decimals"]).tolist() == g["gates"]
    # renormalised top probabilities give the same gates ("softmax first and
    # renormalise after ... gives the same numbers")
    p = O.softmax_rows(logits)[0, idx[0]]
    assert np.allclose(p / p.sum(), gates[0], rtol=1e-14, atol=0)
    assert np.round(O.softmax_rows(logits)[0, idx[0]], 3).tolist() == g["top_probs"]


def _tokens_with_counts(counts, salt):
    """A top-1 routing of sum(counts) tokens with exactly these per-expert counts, shuffled."""
    idx = np.repeat(np.arange(len(counts)), counts)
    _rng(salt).shuffle(idx)
    return idx[:, None]


def pin_capacity_and_drops_table():
    """The page's capacity table: dropped 15/7/0 (random) and 56/54/48 (collapsed)."""
    g = load("sparsely_gated_capacity.txt")
    T, E, k = g["T"], g["E"], g["top_k"]
    for f, cap in zip(g["factors"], g["capacities"]):
        assert O.capacity_slots(f, T, k, E) == cap
    for name in ("random", "collapsed"):
        idx = _tokens_with_counts(g[f"{name}_counts"], salt=11)
        assert sum(g[f"{name}_counts"]) == T
        for f, want in zip(g["factors"], g[f"{name}_dropped"]):
            cap = O.capacity_slots(f, T, k, E)
            d = O.dispatch_from_indices(idx, E, cap)
            assert d["counts"].tolist() == g[f"{name}_counts"]
            assert d["dropped"] == want
            # the dropped tokens of expert e are its last (count - cap) tokens in token order
            seen = np.zeros(E, dtype=int)
            for t in range(T):
                e = idx[t, 0]
                assert (d["slot_row"][t] < 0) == (seen[e] >= cap)
                seen[e] += 1
    # the same table end to end: tokens one-hot on their expert, router = 10 * I
    idx = _tokens_with_counts(g["random_counts"], salt=12)[:, 0]
    x = np.eye(E)[idx]
    we = _rng(13).standard_normal((E, E, 4))
    for f, want in zip(g["factors"], g["random_dropped"]):
        r = O.moe_forward(x, 10.0 * np.eye(E), 1, "linear", we, capacity_factor=f)
        assert r["dropped"] == want
        dropped_tokens = np.flatnonzero(r["slot_row"] < 0)
        assert np.array_equal(r["output"][dropped_tokens], np.zeros((len(dropped_tokens), 4)))


def pin_capacity_rounds_down():
    """capacity = floor(factor * T * k / E): the page's formula with a fractional product."""
    assert O.capacity_slots(1.1, 64, 1, 8) == 8  # 8.8
    assert O.capacity_slots(1.25, 10, 2, 3) == 8  # 8.33
    assert O.capacity_slots(0.05, 16, 1, 8) == 0  # 0.1: every slot dropped
    assert O.capacity_slots(0.0, 16, 1, 8) is None
    idx = _tokens_with_counts([3, 2, 4], salt=14)
    d = O.dispatch_from_indices(idx, 3, 0)
    assert d["dropped"] == 9 and (d["slot_row"] == -1).all() and d["offsets"].tolist() == [0] * 4


def pin_bias_collapses_router():
    """A +8 logit bias on expert 3 sends all 64 top-1 tokens there (the page's collapsed router)."""
    g = load("sparsely_gated_capacity.txt")
    T, E = g["T"], g["E"]
    r_ = _rng(15)
    D = 16
    x = r_.standard_normal((T, D))
    w = r_.standard_normal((D, E)) / math.sqrt(D)
    bias = np.zeros(E)
    bias[3] = 8.0
    r = O.moe_forward(x, w, 1, "linear", r_.standard_normal((E, D, 2)), bias=bias)
    assert r["counts"].tolist() == g["collapsed_counts"]
    base = O.moe_forward(x, w, 1, "linear", r_.standard_normal((E, D, 2)))
    assert base["counts"].tolist() != g["collapsed_counts"]


def pin_counts_sum_to_slots():
    """Every token got exactly k experts: sum of counts = T * k."""
    for (T, E, k, salt) in [(16, 8, 2, 16), (50, 6, 4, 17), (31, 5, 1, 18)]:
        x, w, we = _linear_case(T, 5, E, 2, salt)
        r = O.moe_forward(x, w, k, "linear", we)
        assert int(r["counts"].sum()) == T * k


# --- closed forms ------------------------------------------------------------------------

def pin_k_equals_E_is_dense():
    """k = E: f_e = 1/E so aux = sum_e P_e = 1; gates are the sorted probs; linear experts
    give x_t @ sum_e p_te W_e."""
    for (T, D, E, salt) in [(12, 5, 4, 19), (9, 3, 7, 20)]:
        x, w, we = _linear_case(T, D, E, 3, salt)
        r = O.moe_forward(x, w, E, "linear", we)
        assert abs(r["aux_loss"] - 1.0) < 1e-14
        logits = np.einsum("td,de->te", x, w)
        p = np.exp(logits - logits.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        assert np.allclose(r["gates"], -np.sort(-p, axis=1), rtol=1e-13, atol=0)
        dense = np.einsum("td,te,edo->to", x, p, we)
        assert np.allclose(r["output"], dense, rtol=1e-12, atol=1e-12)


def pin_huge_capacity_equals_no_capacity():
    x, w, we = _linear_case(30, 6, 5, 4, salt=21)
    a = O.moe_forward(x, w, 2, "linear", we)
    b = O.moe_forward(x, w, 2, "linear", we, capacity_factor=5.0 / 2)  # cap = 30 = T
    assert b["capacity"] == 30 and b["dropped"] == 0
    for key in ("output", "expert_indices", "gates", "perm", "slot_row", "offsets"):
        assert np.array_equal(a[key], b[key]), key


def pin_token_permutation_equivariance():
    """Without capacity, tokens are independent: permuting them permutes every per-token output."""
    r_ = _rng(22)
    T, D, DH, E, k = 24, 6, 5, 6, 3
    x = r_.standard_normal((T, D))
    w = r_.standard_normal((D, E))
    w1, w3 = r_.standard_normal((E, D, DH)), r_.standard_normal((E, D, DH))
    w2 = r_.standard_normal((E, DH, D))
    a = O.moe_forward(x, w, k, "swiglu", w1, w2, w3)
    pi = r_.permutation(T)
    b = O.moe_forward(x[pi], w, k, "swiglu", w1, w2, w3)
    assert np.allclose(b["output"], a["output"][pi], rtol=1e-13, atol=1e-13)
    assert np.array_equal(b["expert_indices"], a["expert_indices"][pi])
    assert np.array_equal(b["counts"], a["counts"])
    assert abs(a["aux_loss"] - b["aux_loss"]) < 1e-13


def _silu_scalar(z):
    return z / (1.0 + math.exp(-z)) if z > -700 else -0.0


def pin_expert_closed_forms():
    """Each expert with diagonal/permutation weights has an elementwise closed form."""
    r_ = _rng(23)
    n = 6
    x = r_.standard_normal((5, n)) * 3
    a = r_.uniform(0.5, 2.0, n)
    b = r_.uniform(-2.0, -0.5, n)
    P = np.eye(n)[r_.permutation(n)]  # y = h @ P permutes the columns of h
    cols = P.argmax(axis=0)  # y[:, c] = h[:, cols[c]]
    # linear: x @ (diag(a) P)
    y = O.expert_forward("linear", x, np.diag(a) @ P)
    assert np.allclose(y, (x * a)[:, cols], rtol=1e-15, atol=0)
    # ReLU two-layer: relu(x @ diag(a)) @ P
    y = O.expert_forward("relu2", x, np.diag(a), P)
    assert np.array_equal(y, np.maximum(x * a, 0)[:, cols])
    # SwiGLU: (silu(x @ diag(a)) * (x @ diag(b))) @ P
    y = O.expert_forward("swiglu", x, np.diag(a), P, np.diag(b))
    want = np.array([[_silu_scalar(x[i, j] * a[j]) * (x[i, j] * b[j]) for j in range(n)]
                     for i in range(x.shape[0])])[:, cols]
    assert np.allclose(y, want, rtol=1e-14, atol=1e-15)
    # a non-square, non-diagonal case against a hand loop
    w1 = r_.standard_normal((4, 3))
    w2 = r_.standard_normal((3, 2))
    xx = r_.standard_normal((2, 4))
    h = [[max(sum(xx[i, p] * w1[p, q] for p in range(4)), 0.0) for q in range(3)] for i in range(2)]
    want = [[sum(h[i][q] * w2[q, c] for q in range(3)) for c in range(2)] for i in range(2)]
    assert np.allclose(O.expert_forward("relu2", xx, w1, w2), want, rtol=1e-13, atol=1e-14)


def pin_silu_identities():
    z = np.linspace(-30, 30, 121)
    s = O.silu(z)
    assert O.silu(np.array([0.0]))[0] == 0.0
    assert np.allclose(O.silu(-z), s - z, rtol=0, atol=1e-12)  # silu(-z) = silu(z) - z
    assert abs(O.silu(np.array([40.0]))[0] - 40.0) < 1e-12
    assert abs(O.silu(np.array([-40.0]))[0]) < 1e-15
    assert abs(O.silu(np.array([1.0]))[0] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16
    assert O.silu(np.array([-800.0]))[0] == 0.0


def pin_dispatch_structure():
    """Dispatch invariants: counts, offsets, per-expert token order, inverse map."""
    r_ = _rng(24)
    for (T, E, k, cap) in [(60, 8, 3, None), (60, 8, 3, 13), (45, 5, 1, 4), (10, 4, 4, 2)]:
        idx = np.array([r_.permutation(E)[:k] for _ in range(T)])
        d = O.dispatch_from_indices(idx, E, cap)
        assert d["counts"].tolist() == np.bincount(idx.ravel(), minlength=E).tolist()
        kept = np.minimum(d["counts"], cap if cap is not None else T)
        assert d["offsets"].tolist() == [0] + np.cumsum(kept).tolist()
        for e in range(E):
            seg = d["perm"][d["offsets"][e]:d["offsets"][e + 1]]
            tok, j = seg // k, seg % k
            assert (idx[tok, j] == e).all()
            assert (np.diff(tok) > 0).all()
        R = d["offsets"][-1]
        assert np.array_equal(d["slot_row"][d["perm"]], np.arange(R))
        assert (d["slot_row"] >= 0).sum() == R == T * k - d["dropped"]


def pin_matches_per_token_implementation():
    """The vectorised oracle equals the token-by-token one on tiny random layers."""
    r_ = _rng(25)
    cases = 0
    for kind in ("linear", "relu2", "swiglu"):
        for E in (1, 2, 3, 5, 8):
            for k in sorted({1, 2, E}):
                if k > E:
                    continue
                T = int(r_.integers(1, 40))
                D, DH = int(r_.integers(1, 7)), int(r_.integers(1, 6))
                x = r_.standard_normal((T, D))
                w = r_.standard_normal((D, E))
                bias = r_.standard_normal(E) if r_.random() < 0.5 else None
                cf = float(r_.choice([0.0, 0.5, 1.0, 1.5]))
                w1 = r_.standard_normal((E, D, DH if kind != "linear" else 3))
                w3 = r_.standard_normal((E, D, DH)) if kind == "swiglu" else None
                w2 = r_.standard_normal((E, DH, 3)) if kind != "linear" else None
                opts = {}
                if r_.random() < 0.5:
                    opts = dict(w_noise=r_.standard_normal((D, E)),
                                noise=r_.standard_normal((T, E)))
                opts["renormalise"] = bool(r_.random() < 0.6)
                a = O.moe_forward(x, w, k, kind, w1, w2, w3, bias=bias, capacity_factor=cf,
                                  **opts)
                b = O.moe_forward_per_token(x, w, k, kind, w1, w2, w3, bias=bias,
                                            capacity_factor=cf, **opts)
                assert np.array_equal(a["expert_indices"], b["expert_indices"])
                assert np.allclose(a["gates"], b["gates"], rtol=1e-13, atol=0)
                assert abs(a["aux_loss"] - b["aux_loss"]) <= 1e-13 * max(1.0, b["aux_loss"])
                assert abs(a["importance_loss"] - b["importance_loss"]) <= 1e-12 * max(
                    1.0, b["importance_loss"])
                assert np.array_equal(a["counts"], b["counts"])
                assert np.array_equal(a["slot_row"].reshape(T, k) >= 0, b["kept_mask"])
                scale = max(1.0, np.abs(b["output"]).max())
                assert np.abs(a["output"] - b["output"]).max() <= 1e-12 * scale
                cases += 1
    assert cases >= 30


# --- router options on the Sparsely-Gated Layer page: noise, renormalise, importance ----

def pin_importance_loss_page_values():
    """The page's importance losses: 0.301 for the untouched router, 7.000 collapsed."""
    g = load("sparsely_gated_importance.txt")
    T, E, k = g["T"], g["E"], g["top_k"]
    for name in ("random", "collapsed"):
        idx = _tokens_with_counts(g[f"{name}_counts"], salt=31)
        v = O.importance_loss(idx, np.ones((T, k)), E)  # top-1 gates are exactly 1
        assert round(v, g["decimals"]) == g[f"{name}_importance"]
    # one expert takes every token: exactly E - 1
    idx = _tokens_with_counts(g["collapsed_counts"], salt=31)
    assert abs(O.importance_loss(idx, np.ones((T, k)), E) - (E - 1)) <= 1e-12
    # the same through the layer: tokens one-hot on their expert, router 10 * I, top-1
    tok = _tokens_with_counts(g["random_counts"], salt=32)[:, 0]
    r = O.moe_forward(np.eye(E)[tok], 10.0 * np.eye(E), 1, "linear",
                      _rng(33).standard_normal((E, E, 2)))
    assert round(r["importance_loss"], g["decimals"]) == g["random_importance"]


def pin_importance_closed_forms():
    """CV^2 of the per-expert gate sums: 0 for equal sums, E - 1 when one expert has all,
    invariant to scaling every gate, and built from gate values, not counts."""
    E = 5
    idx = np.array([[e, (e + 1) % E] for e in range(E)] * 3)
    assert abs(O.importance_loss(idx, np.tile([0.7, 0.3], (idx.shape[0], 1)), E)) <= 1e-15
    # two experts, each chosen twice: sums 0.9 + 0.4 and 0.1 + 0.6 -> mean 1, variance 0.09
    idx = np.array([[0, 1], [1, 0]])
    gates = np.array([[0.9, 0.1], [0.6, 0.4]])
    assert abs(O.importance_loss(idx, gates, 2) - 0.09) <= 1e-14
    r_ = _rng(34)
    idx = np.array([r_.permutation(7)[:3] for _ in range(50)])
    g = r_.random((50, 3)) + 0.05
    a, b = O.importance_loss(idx, g, 7), O.importance_loss(idx, 3.0 * g, 7)
    assert abs(a - b) <= 1e-13 * max(a, 1.0)
    assert abs(O.importance_loss(np.zeros((10, 1), int), r_.random((10, 1)) + 0.1, 6) - 5) <= 1e-12
    assert O.importance_loss(np.zeros((0, 2), int), np.zeros((0, 2)), 4) == 0.0


def pin_token0_unrenormalised_gates():
    """renormalise=False: token 0's gates are its top-2 probabilities 0.39 and 0.232, summing
    to 0.622 as printed; with k = E they are all the probabilities, best first."""
    g = load("sparsely_gated_token0_gates.txt")
    logits = np.log(np.array(g["probs"], dtype=np.float64))[None, :]
    probs = O.softmax_rows(logits)
    idx = O.top_k_sorted(logits, g["top_k"])
    gates = O.gates_from_probs(probs, idx)
    assert idx[0].tolist() == g["expert_indices"]
    assert np.round(gates[0], g["decimals"]).tolist() == g["top_probs"]
    # the printed probabilities are rounded (they sum to 0.999), so the printed sum holds to
    # the rounding of two probabilities and of the sum itself
    half = 0.5 * 10.0 ** -g["decimals"]
    assert abs(float(gates[0].sum()) - g["top_probs_sum"]) <= 3 * half
    idx8 = O.top_k_sorted(logits, 8)
    g8 = O.gates_from_probs(probs, idx8)
    assert np.allclose(np.sort(g8[0])[::-1], np.sort(probs[0])[::-1], rtol=1e-15, atol=0)
    # through the layer, top-1: the gate is the winner's probability, not 1
    x = np.eye(3)
    r = O.moe_forward(x, np.diag([2.0, 1.0, 0.5]), 1, "linear", np.ones((3, 3, 1)),
                      renormalise=False)
    p = O.softmax_rows(np.diag([2.0, 1.0, 0.5]))
    assert np.allclose(r["gates"][:, 0], p.max(axis=1), rtol=1e-15, atol=0)
    assert np.allclose(r["output"][:, 0], p.max(axis=1), rtol=1e-15, atol=0)


def pin_softplus_identities():
    """softplus(0) = ln 2, softplus(z) - softplus(-z) = z, softplus(z) -> z and -> e^z."""
    z = np.array([-30.0, -1.5, -1e-9, 0.0, 1e-9, 2.5, 30.0, 700.0])
    sp = O.softplus(z)
    assert sp[3] == math.log(2.0)
    assert np.allclose(sp - O.softplus(-z), z, rtol=1e-13, atol=1e-15)
    assert abs(sp[-1] - 700.0) <= 1e-13 * 700.0
    assert abs(sp[0] - math.exp(-30.0)) <= 1e-12 * math.exp(-30.0)
    assert (np.diff(sp) > 0).all() and (sp > 0).all()


def pin_noise_closed_forms():
    """Noisy logits = logits + noise * softplus(x @ W_noise): zero noise leaves the logits
    exactly; W_noise = 0 scales the noise by ln 2; one-hot tokens read one row of W_noise;
    noise larger than the margin flips the choice (the page's noise-on runs differ)."""
    r_ = _rng(35)
    T, D, E = 9, 6, 6  # square W_noise: a transposed read would go unnoticed otherwise
    x, w, b = r_.standard_normal((T, D)), r_.standard_normal((D, E)), r_.standard_normal(E)
    wn, eps = r_.standard_normal((D, E)), r_.standard_normal((T, E))
    base = O.router_logits(x, w, b)
    assert np.array_equal(O.noisy_router_logits(x, w, b, wn, np.zeros((T, E))), base)
    assert np.allclose(O.noisy_router_logits(x, w, b, np.zeros((D, E)), eps),
                       base + eps * math.log(2.0), rtol=0, atol=1e-14)
    x1 = np.eye(D)[[0, 3, 1, 2]]
    e1 = r_.standard_normal((4, E))
    want = np.array([[x1[t] @ w[:, e] + e1[t, e] * math.log1p(math.exp(wn[np.argmax(x1[t]), e]))
                      for e in range(E)] for t in range(4)])
    assert np.allclose(O.noisy_router_logits(x1, w, None, wn, e1), want, rtol=1e-14, atol=1e-14)
    common = dict(w_noise=np.zeros((1, 2)))
    lay = (np.array([[1.0]]), np.array([[1.0, 0.0]]), 1, "linear", np.ones((2, 1, 1)))
    assert O.moe_forward(*lay, noise=np.zeros((1, 2)), **common)["expert_indices"].tolist() == [[0]]
    # 1 - 2 ln 2 < 0: the noise moves expert 0 below expert 1
    assert O.moe_forward(*lay, noise=np.array([[-2.0, 0.0]]), **common)["expert_indices"].tolist() == [[1]]


def pin_padded_layout():
    """Capacity-padded rows: each kept slot at e * capacity + its rank in the compact
    layout, the kept rows first in every batch and the rest empty."""
    r_ = _rng(36)
    for (T, E, k, cap) in [(60, 8, 3, 13), (45, 5, 1, 4), (10, 4, 4, 2), (12, 3, 2, 0)]:
        idx = np.array([r_.permutation(E)[:k] for _ in range(T)])
        d = O.dispatch_from_indices(idx, E, cap)
        p = O.padded_layout(d, E, cap)
        assert p["perm_padded"].shape == (E * cap,)
        flat = idx.reshape(-1)
        for s_ in range(T * k):
            if d["slot_row"][s_] < 0:
                assert p["slot_row_padded"][s_] == -1
            else:
                e = flat[s_]
                assert p["slot_row_padded"][s_] == e * cap + d["slot_row"][s_] - d["offsets"][e]
        for e in range(E):
            seg = p["perm_padded"][e * cap:(e + 1) * cap]
            n = d["kept"][e]
            assert (seg[:n] >= 0).all() and (seg[n:] == -1).all()
        rows = np.flatnonzero(p["perm_padded"] >= 0)
        assert np.array_equal(p["slot_row_padded"][p["perm_padded"][rows]], rows)


# --- backward: the analytic gradients against finite differences of the forward ---------

def _loss(args, kw, dout, d_aux):
    r = O.moe_forward(*args, **kw)
    return float(np.sum(r["output"] * dout) + d_aux * r["aux_loss"])


def _fd_case(kind, T, D, DH, E, k, cf, with_bias, salt):
    r_ = _rng(salt)
    x = r_.standard_normal((T, D))
    w = r_.standard_normal((D, E)) * 1.5
    bias = r_.standard_normal(E) if with_bias else None
    if kind == "linear":
        w1, w2, w3 = r_.standard_normal((E, D, 3)), None, None
    else:
        w1 = r_.standard_normal((E, D, DH))
        w3 = r_.standard_normal((E, D, DH)) if kind == "swiglu" else None
        w2 = r_.standard_normal((E, DH, 3))
    return x, w, bias, w1, w2, w3


def pin_backward_matches_finite_differences():
    """moe_backward against central differences of L = sum(out * dout) + d_aux * aux, for
    every expert kind, k in {1, 2, E}, with and without capacity and bias. Each case first
    checks that its routing margins (and ReLU pre-activations) are far from a kink, so the
    perturbation cannot change a decision."""
    h = 1e-5
    cases = 0
    for kind in ("linear", "relu2", "swiglu"):
        for (k, cf, with_bias) in [(1, 0.0, True), (2, 0.0, False), (2, 0.8, True), (4, 0.0, True)]:
            for salt in range(40, 60):
                T, D, DH, E = 6, 4, 3, 4
                x, w, bias, w1, w2, w3 = _fd_case(kind, T, D, DH, E, k, cf, with_bias, salt)
                lg = O.router_logits(x, w, bias)
                srt = np.sort(lg, axis=1)[:, ::-1]
                if k < E and np.min(srt[:, k - 1] - srt[:, k]) < 1e-2:
                    continue  # a near tie: pick another draw
                if kind == "relu2" and np.min(np.abs(np.einsum("td,edh->teh", x, w1))) < 1e-3:
                    continue
                break
            else:
                raise AssertionError("no draw with clear margins")
            r_ = _rng(salt + 100)
            dout = r_.standard_normal((T, 3))
            d_aux = 0.7
            g = O.moe_backward(x, w, k, kind, w1, w2, w3, bias=bias, capacity_factor=cf,
                               dout=dout, d_aux=d_aux)
            params = dict(x=x, w=w, w1=w1)
            if bias is not None:
                params["bias"] = bias
            if w2 is not None:
                params["w2"] = w2
            if w3 is not None:
                params["w3"] = w3
            grads = dict(x=g["dx"], w=g["dw_router"], bias=g["dbias"], w1=g["dw1"],
                         w2=g["dw2"], w3=g["dw3"])

            def call(pp):
                return _loss((pp["x"], pp["w"], k, kind, pp["w1"], pp.get("w2"), pp.get("w3")),
                             dict(bias=pp.get("bias"), capacity_factor=cf), dout, d_aux)

            scale = max(1.0, max(np.abs(v).max() for v in grads.values() if v is not None))
            for name, val in params.items():
                num = np.zeros_like(val)
                for i in np.ndindex(val.shape):
                    pp = {n: v.copy() for n, v in params.items()}
                    pp[name][i] += h
                    up = call(pp)
                    pp[name][i] -= 2 * h
                    dn = call(pp)
                    num[i] = (up - dn) / (2 * h)
                assert np.abs(num - grads[name]).max() <= 1e-6 * scale, (kind, k, cf, name)
            cases += 1
    assert cases == 12


def pin_backward_closed_forms():
    """Gradient closed forms: with k = E the Switch loss is 1 for any router, so its
    gradient is zero; top-1 gates are identically 1, so without the loss the router gets no
    gradient; linear experts with k = E and no capacity give dW_e = sum_t p_te x_t^T dout_t
    and dx_t = sum_e p_te dout_t W_e^T plus the router term."""
    r_ = _rng(60)
    T, D, E = 7, 5, 4
    x, w = r_.standard_normal((T, D)), r_.standard_normal((D, E))
    we = r_.standard_normal((E, D, 3))
    g = O.moe_backward(x, w, E, "linear", we, dout=np.zeros((T, 3)), d_aux=1.3)
    assert np.abs(g["dlogits"]).max() <= 1e-14 and np.abs(g["dw_router"]).max() <= 1e-13
    g = O.moe_backward(x, w, 1, "linear", we, dout=r_.standard_normal((T, 3)), d_aux=0.0)
    assert np.abs(g["dw_router"]).max() == 0.0 and np.abs(g["dbias"]).max() == 0.0
    dout = r_.standard_normal((T, 3))
    g = O.moe_backward(x, w, E, "linear", we, dout=dout, d_aux=0.0)
    p = O.softmax_rows(O.router_logits(x, w))
    for e in range(E):
        want = (x * p[:, e:e + 1]).T @ dout
        assert np.allclose(g["dw1"][e], want, rtol=1e-12, atol=1e-12)


def pin_backward_token_subset():
    """Restricted to a token subset, the backward gives those tokens' dx, dgates and dlogits
    rows exactly as the full one (the routing, drops and loss counts still cover all)."""
    r_ = _rng(61)
    T, D, DH, E, k = 12, 5, 4, 4, 2
    x, w = r_.standard_normal((T, D)), r_.standard_normal((D, E))
    w1, w3, w2 = (r_.standard_normal((E, D, DH)), r_.standard_normal((E, D, DH)),
                  r_.standard_normal((E, DH, 3)))
    dout = r_.standard_normal((T, 3))
    full = O.moe_backward(x, w, k, "swiglu", w1, w2, w3, capacity_factor=0.7, dout=dout,
                          d_aux=0.4)
    sub = [0, 3, 4, 10]
    part = O.moe_backward(x, w, k, "swiglu", w1, w2, w3, capacity_factor=0.7, dout=dout,
                          d_aux=0.4, tokens=sub)
    for name in ("dx", "dgates", "dlogits"):
        assert np.allclose(part[name][sub], full[name][sub], rtol=1e-13, atol=1e-13), name
        rest = np.setdiff1d(np.arange(T), sub)
        assert (part[name][rest] == 0).all(), name


def pin_silu_grad():
    """silu'(0) = 1/2, the asymptotes 1 and 0, and central differences of silu."""
    assert O.silu_grad(0.0) == 0.5
    assert abs(O.silu_grad(40.0) - 1.0) <= 1e-12 and abs(O.silu_grad(-40.0)) <= 1e-12
    z = np.linspace(-6, 6, 49)
    h = 1e-6
    num = (O.silu(z + h) - O.silu(z - h)) / (2 * h)
    assert np.abs(num - O.silu_grad(z)).max() <= 1e-8


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_") and callable(v)]
