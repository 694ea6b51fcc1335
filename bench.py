#!/usr/bin/env python3
"""Throughput of the MoE layer forward on one MI355X.

A step is one moe_forward (route -> dispatch -> expert up GEMM -> expert down GEMM ->
combine, plus the Switch loss) over one batch of seeded synthetic input that is already
resident in HBM. Default workload: the Mixtral-shaped SwiGLU layer (T=4096 tokens, D=4096,
DH=14336, E=8 experts, top-2, bf16 storage with fp32 accumulation, no capacity limit).

Prints ONE JSON line on stdout. Besides the required fields it carries:
  roofline      the dominant kernel (the expert up-projection GEMM) against bf16 MFMA peak,
                timed with HIP events recorded around it inside every timed step;
  stages        per-stage device time and its roofline figure;
  cpu_baseline  the CPU oracle timed on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3  # MI355X fp32 vector


# HBM traffic of the expert up-projection GEMM, per launch, from two rocprofv3 --pmc passes
# (FETCH_SIZE, then WRITE_SIZE, KiB summed over the launch) over this same command. Each
# counter is divided by what it reads per byte for a plain device copy of known size
# (--copy-calibration-mib): FETCH_SIZE reads 0.500 KiB per KiB copied, WRITE_SIZE 1.000.
# The figures hold only for the kernel sources whose hash is given; once those change
# the field is reported as null until the counters are taken again.
GEMM_SOURCES = ("expert_ffn_layer_router_amd/csrc/expert_gemm_bf16.hip",
                "expert_ffn_layer_router_amd/csrc/tile_schedule.hpp",
                "expert_ffn_layer_router_amd/csrc/common.hpp")
FETCH_PER_BYTE = 0.500
WRITE_PER_BYTE = 1.000
MEASURED_TRAFFIC = {
    # config: (sha256 of GEMM_SOURCES, FETCH_SIZE KiB per launch, WRITE_SIZE KiB per launch)
    "mixtral_swiglu_bf16": ("24d43825e0129a9bca595627fdc1e58621428b9200f9e57bb1a0e837ee2aa0dd",
                            3467390.5803571427, 229562.7142857143),
    "switch_top1_cap_bf16": ("24d43825e0129a9bca595627fdc1e58621428b9200f9e57bb1a0e837ee2aa0dd",
                             224213.6517857143, 26562.758928571428),
    "fine_grained_zipf_bf16": ("24d43825e0129a9bca595627fdc1e58621428b9200f9e57bb1a0e837ee2aa0dd",
                               1007214.1339285715, 143432.9107142857),
}


def gemm_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        h.update((ROOT / f).read_bytes())
    return h.hexdigest()


def measured_traffic(config: str):
    rec = MEASURED_TRAFFIC.get(config)
    if rec is None or rec[0] != gemm_source_hash():
        return None
    _, fetch_kib, write_kib = rec
    return (fetch_kib / FETCH_PER_BYTE + write_kib / WRITE_PER_BYTE) * 1024.0


def copy_calibration(mib: int) -> int:
    """A plain device-to-device copy of `mib` MiB, three times: the known-size kernel that
    calibrates the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "copies": 3}), flush=True)
    return 0


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def device_tensor(a):
    import numpy as np
    import torch
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def cpu_baseline(I, tokens: int, min_seconds: float = 10.0, max_passes: int = 4, N=None,
                 renormalise: bool = True, dout=None, d_aux: float = 0.0) -> dict:
    """The oracle as it stands, on the first `tokens` tokens of the same inputs (and router
    options), repeated until at least `min_seconds` of wall time (at most `max_passes`
    passes). With `dout` (host values, (T, D_out)), each pass is the oracle's backward (its
    forward and every gradient), the work of a forward+backward step."""
    from threadpoolctl import threadpool_info

    import oracle
    sp = I.spec
    x = I.values("x")[:tokens]
    wr, w1, w2, w3 = I.values("w_router"), I.values("w1"), I.values("w2"), I.values("w3")
    passes, t0 = 0, time.perf_counter()
    while passes < max_passes and (passes == 0 or time.perf_counter() - t0 < min_seconds):
        if dout is not None:
            oracle.moe_backward(x, wr, sp.top_k, sp.kind, w1, w2, w3, bias=I.bias,
                                capacity_factor=sp.capacity_factor, dout=dout[:tokens],
                                d_aux=d_aux)
            passes += 1
            continue
        oracle.moe_forward(x, wr, sp.top_k, sp.kind, w1, w2, w3, bias=I.bias,
                           capacity_factor=sp.capacity_factor,
                           w_noise=None if N is None else N.w_values(),
                           noise=None if N is None else N.noise[:tokens],
                           renormalise=renormalise)
        passes += 1
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    threads = min(threads, len(os.sched_getaffinity(0)))
    return {"value": passes * tokens / dt, "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"oracle.{'moe_backward (forward and all gradients)' if dout is not None else 'moe_forward'}"
                      f" (NumPy float64, BLAS on {threads} threads) over the "
                      f"first {tokens} of {sp.T} tokens of the same seeded inputs, {passes} "
                      f"pass(es), {dt:.1f} s wall"
                      + ("" if dout is not None else "; each pass widens every expert's "
                                                     "weights to float64 one expert at a time")}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="mixtral_swiglu_bf16")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-baseline-tokens", type=int, default=0,
                    help="tokens in the CPU oracle sample (0: the whole batch)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--router-noise", action="store_true",
                    help="noisy router: + noise * softplus(x @ W_noise), seeded draw")
    ap.add_argument("--no-renormalise", action="store_true",
                    help="gates = the chosen experts' probabilities")
    ap.add_argument("--padded", action="store_true",
                    help="capacity-padded expert batches (needs a capacity factor)")
    ap.add_argument("--backward", action="store_true",
                    help="time forward + moe_backward per step (a training step of the layer)")
    ap.add_argument("--train", action="store_true",
                    help="time moe_forward_train + moe_backward_saved per step (the training "
                         "step that keeps the forward's state instead of recomputing it)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one MI355X: the layer runs on a single GPU (no sharding, no "
              "collectives), so --gpus must be 1", file=sys.stderr)
        return 2

    if args.copy_calibration_mib > 0:
        return copy_calibration(args.copy_calibration_mib)

    import numpy as np
    import torch

    from expert_ffn_layer_router_amd import accounting as A
    from expert_ffn_layer_router_amd import binding as B
    from synth import make_inputs, make_router_noise, spec

    sp = spec(args.config)
    log(f"[bench] generating {sp.name} inputs (seed {args.seed})")
    I = make_inputs(sp, seed=args.seed)
    p = B.Problem.from_spec(sp)
    dev = {n: device_tensor(getattr(I, n)) for n in ("x", "w_router", "bias", "w1", "w3", "w2")}
    outs = B.alloc_outputs(p)
    options = args.router_noise or args.no_renormalise or args.padded
    N, opts, importance = None, None, None
    if options:
        if args.padded and not sp.capacity_factor > 0:
            print("--padded needs a layer with a capacity factor", file=sys.stderr)
            return 2
        if args.router_noise:
            N = make_router_noise(sp, seed=args.seed)
        importance = torch.zeros(1, dtype=torch.float32, device="cuda")
        opts = B.Options(w_noise=None if N is None else device_tensor(N.w_noise),
                         noise=None if N is None else device_tensor(N.noise),
                         renormalise=not args.no_renormalise, padded=args.padded,
                         importance_loss=importance)
    ws = B.alloc_workspace(p, o=opts)
    bwd = None
    train = args.train
    if train:
        args.backward = True
    if args.backward:
        if options:
            print("--backward runs the plain layer (no router options)", file=sys.stderr)
            return 2
        dt = torch.bfloat16 if sp.dtype == "bf16" else torch.float32
        gen = torch.Generator(device="cuda").manual_seed(args.seed + 1)
        bwd = dict(
            dout=torch.randn((sp.T, sp.D_out), generator=gen, device="cuda").to(dt),
            dx=torch.empty((sp.T, sp.D), dtype=dt, device="cuda"),
            dwr=torch.empty((sp.D, sp.E), dtype=torch.float32, device="cuda"),
            db=torch.empty((sp.E,), dtype=torch.float32, device="cuda"),
            dw1=torch.empty_like(dev["w1"]),
            dw3=None if dev["w3"] is None else torch.empty_like(dev["w3"]),
            dw2=None if dev["w2"] is None else torch.empty_like(dev["w2"]),
            ws=torch.empty(max(B.backward_workspace_size(p), 1), dtype=torch.uint8,
                           device="cuda"),
            ev=[], fev=[],
            saved=torch.empty(max(B.saved_size(p), 1), dtype=torch.uint8, device="cuda")
            if train else None)
    torch.cuda.synchronize()

    def forward_train(timed=False):
        if timed:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
        B.moe_forward_train(p, dev["x"], dev["w_router"], dev["bias"], dev["w1"], dev["w3"],
                            dev["w2"], outs["out"], outs["expert_indices"], outs["gates"],
                            outs["aux_loss"], outs["expert_counts"], outs["expert_offsets"],
                            outs["slot_row"], bwd["saved"], ws)
        if timed:
            e1.record()
            bwd["fev"].append((e0, e1))

    def backward_step(timed=False):
        if timed:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
        if train:
            B.moe_backward_saved(p, dev["x"], dev["w_router"], dev["w1"], dev["w3"], dev["w2"],
                                 outs["expert_indices"], outs["gates"], outs["expert_counts"],
                                 outs["expert_offsets"], outs["slot_row"], bwd["saved"],
                                 bwd["dout"], 0.01, bwd["dx"], bwd["dwr"], bwd["db"],
                                 bwd["dw1"], bwd["dw3"], bwd["dw2"], bwd["ws"])
        else:
            B.moe_backward(p, dev["x"], dev["w_router"], dev["bias"], dev["w1"], dev["w3"],
                           dev["w2"], bwd["dout"], 0.01, bwd["dx"], bwd["dwr"], bwd["db"],
                           bwd["dw1"], bwd["dw3"], bwd["dw2"], bwd["ws"])
        if timed:
            e1.record()
            bwd["ev"].append((e0, e1))

    def step(ev=None):
        if opts is None:
            B.moe_forward_timed(p, dev["x"], dev["w_router"], dev["bias"], dev["w1"], dev["w3"],
                                dev["w2"], outs["out"], outs["expert_indices"], outs["gates"],
                                outs["aux_loss"], outs["expert_counts"], outs["expert_offsets"],
                                outs["slot_row"], ws, None if ev is None else ev.events)
        else:
            B.moe_forward_ex(p, opts, dev["x"], dev["w_router"], dev["bias"], dev["w1"],
                             dev["w3"], dev["w2"], outs["out"], outs["expert_indices"],
                             outs["gates"], outs["aux_loss"], outs["expert_counts"],
                             outs["expert_offsets"], outs["slot_row"], ws,
                             None if ev is None else ev.events)

    log(f"[bench] warmup {args.warmup} steps")
    for _ in range(args.warmup):
        forward_train() if train else step()
        if bwd is not None:
            backward_step()
    torch.cuda.synchronize()
    # Timed steps: the up-projection GEMM (the roofline kernel) carries events recorded by its
    # own kernel dispatch, so it is timed live in these steps at the least cost to the stream.
    gemm_stages = ("expert_up",)
    events = [B.StageEvents(gemm_stages) for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        # (the training forward records no stage events: its GEMM figures come from the
        # stage-timing steps below, which run the plain forward)
        forward_train() if train else step(events[i])
        if bwd is not None:
            backward_step()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    stage_ms = {} if train else {k: float(np.mean([e.elapsed_ms()[k] for e in events]))
                                 for k in gemm_stages}
    for e in events:
        e.close()
    # The other stages' times come from a few further steps with an event pair around every
    # stage (those records can leave the device idle briefly, so they stay out of the timing).
    extra = [B.StageEvents() for _ in range(min(args.steps, 5))]
    for e in extra:
        step(e)
        if train:
            forward_train(timed=True)
        if bwd is not None:
            backward_step(timed=True)
    torch.cuda.synchronize()
    for k in (("expert_up",) if train else ()) + ("route", "dispatch", "expert_down", "combine"):
        stage_ms[k] = float(np.mean([e.elapsed_ms()[k] for e in extra]))
    for e in extra:
        e.close()

    T, D, DH, Do, E, k = sp.T, sp.D, sp.DH, sp.D_out, sp.E, sp.top_k
    R = int((outs["slot_row"] >= 0).sum().cpu())  # kept slots (either layout)
    rows = E * B.capacity(p) if args.padded else R  # rows the expert GEMMs run over
    es = 2 if sp.dtype == "bf16" else 4
    peak_tf = BF16_PEAK_TFLOPS if sp.dtype == "bf16" else FP32_PEAK_TFLOPS
    used_tokens = int(np.count_nonzero((outs["slot_row"].view(T, k) >= 0).any(dim=1).cpu()))

    # algorithmic work per launch: flops, and the bytes a launch must move at least (the
    # weights of the experts that have rows, the rows read, the rows written)
    kept = np.diff(outs["expert_offsets"].cpu().numpy().astype(np.int64))
    if args.padded:
        kept = np.full(E, B.capacity(p), dtype=np.int64)
    active = int(np.count_nonzero(kept))
    if sp.kind == "linear":
        up_flops, down_flops = 2 * D * Do * R, 0
        up_w = E * D * Do * es
        up_bytes = active * D * Do * es + rows * (D + Do) * es
        down_bytes = 0
    else:
        up_mult = 4 if sp.kind == "swiglu" else 2
        up_flops, down_flops = up_mult * D * DH * R, 2 * DH * Do * R
        wmats = 2 if sp.kind == "swiglu" else 1
        up_w = wmats * E * D * DH * es
        up_bytes = wmats * active * D * DH * es + rows * (D + DH) * es
        down_bytes = active * DH * Do * es + rows * (DH + Do) * es
    # a GEMM whose flops per algorithmic byte fall below the machine balance is bound by HBM
    balance = peak_tf * 1e12 / (HBM_PEAK_GBS * 1e9)
    route_b = A.route_bytes(T, D, E, k, es)
    if N is not None:
        route_b += A.route_noise_bytes(T, D, E, es)
    combine_b = A.combine_bytes(T, k, R, Do, es)

    def tf(fl, ms_):
        return fl / (ms_ * 1e-3) / 1e12 if ms_ > 0 else 0.0

    def gbs(b, ms_):
        return b / (ms_ * 1e-3) / 1e9 if ms_ > 0 else 0.0

    up_tf = tf(up_flops, stage_ms["expert_up"])
    up_hbm = up_flops < balance * up_bytes
    stages = {
        "route": {"us": stage_ms["route"] * 1e3, "GB/s": gbs(route_b, stage_ms["route"]),
                  "hbm_frac": gbs(route_b, stage_ms["route"]) / HBM_PEAK_GBS,
                  "algorithmic_bytes": route_b},
        "dispatch": {"us": stage_ms["dispatch"] * 1e3} if not args.padded else {
            "us": stage_ms["dispatch"] * 1e3,
            "GB/s": gbs(A.padded_permute_bytes(used_tokens, rows, D, es), stage_ms["dispatch"]),
            "algorithmic_bytes": A.padded_permute_bytes(used_tokens, rows, D, es)},
        "expert_up": {"us": stage_ms["expert_up"] * 1e3, "TFLOP/s": up_tf,
                      "mfma_frac": up_tf / peak_tf, "algorithmic_flops": up_flops,
                      "GB/s": gbs(up_bytes, stage_ms["expert_up"]),
                      "hbm_frac": gbs(up_bytes, stage_ms["expert_up"]) / HBM_PEAK_GBS,
                      "algorithmic_bytes": up_bytes,
                      "bound": "hbm" if up_hbm else "mfma"},
        "expert_down": {"us": stage_ms["expert_down"] * 1e3,
                        "TFLOP/s": tf(down_flops, stage_ms["expert_down"]),
                        "mfma_frac": tf(down_flops, stage_ms["expert_down"]) / peak_tf,
                        "algorithmic_flops": down_flops,
                        "GB/s": gbs(down_bytes, stage_ms["expert_down"]),
                        "hbm_frac": gbs(down_bytes, stage_ms["expert_down"]) / HBM_PEAK_GBS,
                        "algorithmic_bytes": down_bytes,
                        "bound": "hbm" if down_flops < balance * down_bytes else "mfma"},
        "combine": {"us": stage_ms["combine"] * 1e3, "GB/s": gbs(combine_b, stage_ms["combine"]),
                    "hbm_frac": gbs(combine_b, stage_ms["combine"]) / HBM_PEAK_GBS,
                    "algorithmic_bytes": combine_b},
    }
    result = {
        "metric": "MoE layer forward tokens/s at 1 MI355X",
        "value": T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if sp.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0, sigma) inputs and random-init weights)",
        "config": {"workload": sp.description + "".join(
                       s_ for s_, on in ((", router noise", N is not None),
                                         (", gates not renormalised", args.no_renormalise),
                                         (", capacity-padded expert batches", args.padded))
                       if on),
                   "T": T, "D": D, "DH": DH, "E": E, "top_k": k,
                   "expert": sp.kind, "capacity_factor": sp.capacity_factor,
                   "kept_slots": R, "dropped_slots": T * k - R, "used_tokens": used_tokens,
                   "expert_rows": rows},
        "roofline": ({"kernel": "expert up-projection grouped GEMM (stage expert_up)",
                      "bound": "hbm", "achieved": gbs(up_bytes, stage_ms["expert_up"]),
                      "peak": HBM_PEAK_GBS, "unit": "GB/s",
                      "frac": gbs(up_bytes, stage_ms["expert_up"]) / HBM_PEAK_GBS,
                      "algorithmic_bytes_per_launch": up_bytes} if up_hbm else
                     {"kernel": "expert up-projection grouped GEMM (stage expert_up)",
                      "bound": "mfma", "achieved": up_tf, "peak": peak_tf, "unit": "TFLOP/s",
                      "frac": up_tf / peak_tf}) | {
                     "traffic": None if options else measured_traffic(sp.name),
                     "algorithmic_flops_per_launch": up_flops,
                     "launch_us": stage_ms["expert_up"] * 1e3,
                     "weight_bytes": up_w},
        "stages": stages,
    }
    if importance is not None:
        result["importance_loss"] = float(importance.cpu()[0])
    if bwd is not None:
        bwd_ms = float(np.mean([a.elapsed_time(b) for a, b in bwd["ev"]]))
        bwd_flops = 2 * (up_flops + down_flops)  # dgrad + wgrad of every expert GEMM
        result["metric"] = "MoE layer forward+backward tokens/s at 1 MI355X"
        result["config"]["workload"] += (", training forward and backward from its saved state"
                                         if train else ", forward and backward")
        stages["backward"] = {"us": bwd_ms * 1e3, "TFLOP/s": tf(bwd_flops, bwd_ms),
                              "mfma_frac": tf(bwd_flops, bwd_ms) / peak_tf,
                              "algorithmic_flops": bwd_flops,
                              "note": ("dgrad + wgrad of the expert GEMMs, from the training "
                                       "forward's saved state (moe_backward_saved)") if train else
                                      ("dgrad + wgrad of the expert GEMMs; the recomputed "
                                       "forward inside the call is not counted")}
        if train:
            fwd_ms = float(np.mean([a.elapsed_time(b) for a, b in bwd["fev"]]))
            stages["forward_train"] = {"us": fwd_ms * 1e3,
                                       "note": "moe_forward_train: the forward that also keeps "
                                               "the pre-activations, h, y, logits and perm"}
            result["roofline"]["kernel"] += ", timed in plain forward steps beside the timed ones"
    if not args.no_cpu_baseline:
        # the whole batch for the forward; the backward oracle (about ten times the work a
        # token) on a 1024-token sample unless asked otherwise
        n = (min(args.cpu_baseline_tokens, T) if args.cpu_baseline_tokens > 0
             else (min(T, 1024) if bwd is not None else T))
        log(f"[bench] CPU oracle baseline on {n} tokens")
        dout_host = None
        if bwd is not None:
            dout_host = bwd["dout"].float().cpu().numpy().astype(np.float64)
        result["cpu_baseline"] = cpu_baseline(I, n, N=N, renormalise=not args.no_renormalise,
                                              dout=dout_host, d_aux=0.01)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
