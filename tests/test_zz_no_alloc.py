"""The allocation-free routing entry point (moe_route_noalloc) against moe_route.

moe_route_noalloc runs moe_route's kernels with their scratch in a fixed device array inside
the library instead of a caller workspace, so its results must equal moe_route's bit for bit:
indices, counts and the uncertified count (integers) and gates, aux_loss and the logits
(identical arithmetic). Two calls in a row share the array, the second on a smaller problem,
and each must match moe_route on its own inputs.
"""

from __future__ import annotations

import numpy as np
import pytest

from gpu_util import device_inputs, run_oracle, to_host
from synth import make_inputs, spec

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _route_outputs(sp):
    import torch
    T, k, E = sp.T, sp.top_k, sp.E
    return dict(idx=torch.full((T, k), -5, dtype=torch.int32, device="cuda"),
                gates=torch.full((T, k), 9.0, dtype=torch.float32, device="cuda"),
                aux=torch.full((1,), 9.0, dtype=torch.float32, device="cuda"),
                counts=torch.full((E,), -5, dtype=torch.int32, device="cuda"),
                logits=torch.full((T, E), 9.0, dtype=torch.float32, device="cuda"),
                unc=torch.full((1,), -5, dtype=torch.int32, device="cuda"))


def _with_workspace(sp, d):
    import torch
    from expert_ffn_layer_router_amd import binding as B
    p = B.Problem.from_spec(sp)
    o = _route_outputs(sp)
    ws = B.alloc_workspace(p)
    B.moe_route(p, d["x"], d["w_router"], d["bias"], o["idx"], o["gates"], o["aux"],
                o["counts"], o["logits"], o["unc"], ws)
    torch.cuda.synchronize()
    return {n: to_host(v) for n, v in o.items()}


def _no_alloc(sp, d):
    import torch
    from expert_ffn_layer_router_amd import binding as B
    p = B.Problem.from_spec(sp)
    o = _route_outputs(sp)
    B.moe_route_noalloc(p, d["x"], d["w_router"], d["bias"], o["idx"], o["gates"], o["aux"],
                        o["counts"], o["logits"], o["unc"])
    torch.cuda.synchronize()
    return {n: to_host(v) for n, v in o.items()}


def _same(a, b, what):
    for n in a:
        assert np.array_equal(a[n], b[n]), f"{what}: {n} differs"


# pairs (first call, second call on a smaller problem)
PAIRS = {
    # 64 and 8 experts: exact float64 logits, one slot per routing block in the scratch
    "bf16_zipf_e64": (spec("fine_grained_zipf_bf16", T=3000, D=512, DH=64),
                      spec("fine_grained_zipf_bf16", T=700, D=512, DH=64)),
    "bf16_mixtral_e8": (spec("mixtral_swiglu_bf16", T=1500, D=4096, DH=64),
                        spec("mixtral_swiglu_bf16", T=129, D=4096, DH=64)),
    # 128 experts, top 6: the certified path, its partial logits and fallback list in the scratch
    "bf16_e128_k6": (spec("fine_grained_zipf_bf16", T=2000, D=512, DH=64, E=128),
                     spec("fine_grained_zipf_bf16", T=333, D=512, DH=64, E=128)),
    # 96 experts, top 2: the certified single-pass path, its group slots in the scratch
    "bf16_e96_k2": (spec("mixtral_swiglu_bf16", T=1500, D=1024, DH=64, E=96),
                    spec("mixtral_swiglu_bf16", T=200, D=1024, DH=64, E=96)),
    "f32_relu": (spec("small_relu_f32", T=500, D=96, DH=32, E=12, top_k=3),
                 spec("small_relu_f32", T=37, D=96, DH=32, E=12, top_k=3)),
}


@pytest.mark.parametrize("name", sorted(PAIRS))
def test_no_alloc_route_matches_route_twice(name):
    big, small = PAIRS[name]
    _say(f"[gpu] moe_route_noalloc {name}: T={big.T} then T={small.T}")
    Ib, Is = make_inputs(big, seed=31), make_inputs(small, seed=32)
    db, ds = device_inputs(Ib), device_inputs(Is)
    ref_b, ref_s = _with_workspace(big, db), _with_workspace(small, ds)
    got_b = _no_alloc(big, db)
    got_s = _no_alloc(small, ds)  # the array still holds the first call's contents
    _same(got_b, ref_b, f"{name} first call")
    _same(got_s, ref_s, f"{name} second (smaller) call")
    # and the decisions are the oracle's
    r = run_oracle(Is, tokens=[])
    assert np.array_equal(got_s["idx"], r["expert_indices"])
    assert np.array_equal(got_s["counts"], r["counts"])


def test_no_alloc_route_zero_router_and_full_size():
    """The all-tie router (every token recomputed in float64) and then the Zipf-shaped layer at
    full size, the largest routing scratch of the five workloads."""
    sp0 = spec("fine_grained_zipf_bf16", T=300, D=256, DH=64, bias="none")
    I0 = make_inputs(sp0, seed=4, router_zero=True)
    d0 = device_inputs(I0)
    _same(_no_alloc(sp0, d0), _with_workspace(sp0, d0), "zero router")
    sp = spec("fine_grained_zipf_bf16")
    _say(f"[gpu] moe_route_noalloc full size {sp.name}")
    I = make_inputs(sp)
    d = device_inputs(I)
    _same(_no_alloc(sp, d), _with_workspace(sp, d), "full-size Zipf")


def test_no_alloc_route_empty_and_rejected():
    import torch
    from expert_ffn_layer_router_amd import binding as B
    sp = spec("mixtral_swiglu_bf16", T=0, D=64, DH=64)
    d = device_inputs(make_inputs(sp))
    o = _route_outputs(sp)
    B.moe_route_noalloc(B.Problem.from_spec(sp), d["x"], d["w_router"], None, o["idx"],
                        o["gates"], o["aux"], o["counts"], None, o["unc"])
    torch.cuda.synchronize()
    assert o["aux"].item() == 0.0 and (o["counts"] == 0).all() and o["unc"].item() == 0
    # a problem whose routing scratch does not fit: rejected before anything is launched
    big = B.Problem.from_spec(spec("fine_grained_zipf_bf16", T=1 << 20, D=2048, DH=64, E=256))
    fake = 1 << 20
    st = B.lib().moe_route_noalloc(big.c(), fake, fake, None, fake, fake, fake, None, None,
                                   None, None)
    assert st == B.MOE_ERR_SCRATCH_LIMIT
