"""FLOP and parameter accounting against the numbers printed on
"Mixture of Experts: the Sparsely-Gated Layer", section "Eight times the parameters,
twice the compute" (tests/golden/sparsely_gated_flops.txt)."""

from expert_ffn_layer_router_amd import accounting as A
from golden_io import load


def test_flops_per_token_table():
    g = load("sparsely_gated_flops.txt")
    d, h, N = g["d_model"], g["ffn_hidden"], g["experts"]
    for k, want in zip(g["ks"], g["flops_per_token"]):
        assert A.flops_per_token("relu2", d, h, d, N, k) == want


def test_parameter_counts():
    g = load("sparsely_gated_flops.txt")
    d, h, N = g["d_model"], g["ffn_hidden"], g["experts"]
    assert A.expert_params("relu2", d, h, d) == g["dense_params"]
    assert A.layer_params("relu2", d, h, d, N) == g["moe_params"]
    md, mh = g["mixtral_d"], g["mixtral_h"]
    one = A.expert_params("swiglu", md, mh, md)
    assert one == g["mixtral_one_expert"]
    assert one * g["mixtral_experts"] * g["mixtral_layers"] == g["mixtral_all_experts"]
    assert one * g["mixtral_top_k"] * g["mixtral_layers"] == g["mixtral_active"]


def test_swiglu_flops_are_three_matrices():
    # three (D x DH)-sized products per slot, two flops per multiply-add
    assert A.expert_flops_per_slot("swiglu", 4096, 14336, 4096) == 6 * 4096 * 14336
