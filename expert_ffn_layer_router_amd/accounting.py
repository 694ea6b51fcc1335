"""Work accounting for the MoE layer forward: FLOPs and algorithmic HBM bytes.

Host arithmetic only (no layer math). The FLOP count follows the accounting of
"Mixture of Experts: the Sparsely-Gated Layer", section "Eight times the
parameters, twice the compute": the router costs ``2*d*N`` per token and each of
the k visited experts costs two flops per weight it applies (``4*d*h`` for the
two-layer ReLU expert, ``6*d*h`` for the three-matrix SwiGLU expert).
"""

from __future__ import annotations


def expert_flops_per_slot(kind: str, D: int, DH: int, D_out: int) -> int:
    """Multiply-add flops one expert spends on one routed token."""
    if kind == "linear":
        return 2 * D * D_out
    if kind == "relu2":
        return 2 * D * DH + 2 * DH * D_out
    if kind == "swiglu":
        return 4 * D * DH + 2 * DH * D_out
    raise ValueError(kind)


def router_flops_per_token(D: int, E: int) -> int:
    return 2 * D * E


def flops_per_token(kind: str, D: int, DH: int, D_out: int, E: int, k: int) -> int:
    """Router plus k expert evaluations, as the page counts them."""
    return router_flops_per_token(D, E) + k * expert_flops_per_slot(kind, D, DH, D_out)


def expert_params(kind: str, D: int, DH: int, D_out: int) -> int:
    if kind == "linear":
        return D * D_out
    if kind == "relu2":
        return D * DH + DH * D_out
    if kind == "swiglu":
        return 2 * D * DH + DH * D_out
    raise ValueError(kind)


def layer_params(kind: str, D: int, DH: int, D_out: int, E: int) -> int:
    """All experts plus the (D, E) router."""
    return E * expert_params(kind, D, DH, D_out) + D * E


# --- algorithmic HBM bytes per kernel (each input read once, each output written once)

def route_bytes(T: int, D: int, E: int, k: int, act_bytes: int) -> int:
    """Read x (T, D) and the router (D, E); write indices and gates (T, k) int32 + fp32."""
    return T * D * act_bytes + D * E * act_bytes + T * k * 8


def route_noise_bytes(T: int, D: int, E: int, act_bytes: int) -> int:
    """Router noise adds a read of W_noise (D, E) and of the (T, E) float32 draw."""
    return D * E * act_bytes + T * E * 4


def padded_permute_bytes(used_tokens: int, rows: int, D: int, act_bytes: int) -> int:
    """The padded copy: each used x row read once, all E * capacity rows written (kept rows
    and zero rows)."""
    return used_tokens * D * act_bytes + rows * D * act_bytes


def permute_bytes(used_tokens: int, R: int, D: int, act_bytes: int) -> int:
    """Read each used x row once, write R expert-ordered rows."""
    return used_tokens * D * act_bytes + R * D * act_bytes


def combine_bytes(T: int, k: int, R: int, D_out: int, act_bytes: int) -> int:
    """Read R expert-output rows, gates and slot rows; write T output rows."""
    return R * D_out * act_bytes + T * k * 8 + T * D_out * act_bytes
