"""CPU oracle for the top-k Mixture-of-Experts layer forward (NumPy, float64).

TEST INFRASTRUCTURE ONLY. This package is the slow, plain reference that the
GPU path is checked against. Only the tests, the smoke check of the package
entry file and the CPU-baseline leg of the benchmark may import it. The product
path (the HIP kernels behind the C ABI and their Python binding) never imports,
links or calls anything here, and this package imports nothing from it.

Sources (web pages; cited by title and section):

* "Mixture-of-Experts (MoE) Routing" (ML Grind, LLM Internals): the algorithm,
  the inputs, the return format, the edge cases and the worked examples. It is
  the primary definition.
* "Mixture of Experts: the Sparsely-Gated Layer" (paperfordummies, Shazeer 2017
  with Switch 2021): capacity and first-come-first-served dropping, the optional
  router bias, the two-layer ReLU expert, the FLOP accounting, and the router
  options: noise, gates without renormalisation, Shazeer's importance loss and
  the capacity-padded expert batches.
* "Sparsely-gated Mixture of Experts (MoE)" (Eli Bendersky): the per-token
  formulation (section "A Minimal Numpy Implementation"), the D, DH, NEXP,
  TOPK naming.

Every function is pinned by the ``-m "not gpu"`` tests, with one exception
stated in ``moe.py``'s header ("parity unpinned").
"""

from .moe import (  # noqa: F401
    capacity_slots,
    dispatch_from_indices,
    expert_backward,
    expert_forward,
    gates_from_logits,
    gates_from_probs,
    importance_loss,
    moe_backward,
    moe_forward,
    moe_forward_per_token,
    noisy_router_logits,
    padded_layout,
    router_logits,
    silu,
    silu_grad,
    softmax_rows,
    softplus,
    switch_aux_loss,
    top_k_sorted,
)
