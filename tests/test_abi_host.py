"""The C ABI on the host: the library loads, exports every declared symbol, and its
host-side checks behave as include/moe.h states. No GPU and no kernel launch."""

import ctypes
import re
from pathlib import Path

import pytest

from expert_ffn_layer_router_amd import binding as B
from golden_io import load

HEADER = Path(__file__).resolve().parent.parent / "include" / "moe.h"


def declared_functions():
    text = re.sub(r"/\*.*?\*/", "", HEADER.read_text(), flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_header_declares_the_five_stages():
    names = declared_functions()
    for n in ("moe_route", "moe_dispatch", "moe_expert_ffn", "moe_combine", "moe_forward"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = B.lib()
    names = declared_functions()
    assert set(names) == set(B.EXPORTED)
    for n in names:
        assert getattr(lib, n) is not None


def P(**kw):
    base = dict(T=64, D=32, DH=48, D_out=32, E=8, top_k=2, capacity_factor=0.0, dtype="bf16",
                kind="swiglu")
    base.update(kw)
    return B.Problem(**base)


@pytest.mark.parametrize("kw,want", [
    ({}, B.MOE_OK),
    (dict(top_k=0), B.MOE_ERR_INVALID_ARG),
    (dict(top_k=9), B.MOE_ERR_INVALID_ARG),
    (dict(T=-1), B.MOE_ERR_INVALID_ARG),
    (dict(D=0), B.MOE_ERR_INVALID_ARG),
    (dict(DH=0), B.MOE_ERR_INVALID_ARG),
    (dict(DH=0, kind="linear"), B.MOE_OK),
    (dict(E=0, top_k=0), B.MOE_ERR_INVALID_ARG),
    (dict(E=257, top_k=2), B.MOE_ERR_UNSUPPORTED),
    (dict(E=256, top_k=256), B.MOE_OK),
    (dict(D=36), B.MOE_ERR_UNSUPPORTED),
    (dict(D=36, dtype="f32"), B.MOE_OK),
    (dict(DH=44), B.MOE_ERR_UNSUPPORTED),
    (dict(D_out=12), B.MOE_ERR_UNSUPPORTED),
    (dict(T=0), B.MOE_OK),
    (dict(T=2**30, top_k=2), B.MOE_ERR_UNSUPPORTED),
    (dict(capacity_factor=float("nan")), B.MOE_ERR_INVALID_ARG),
])
def test_problem_checks(kw, want):
    assert B.check_problem(P(**kw)) == want


def test_capacity_matches_the_pages_table():
    """capacity = floor(factor * T * k / E): the Sparsely-Gated Layer page's table."""
    g = load("sparsely_gated_capacity.txt")
    for f, cap in zip(g["factors"], g["capacities"]):
        assert B.capacity(P(T=g["T"], E=g["E"], top_k=1, capacity_factor=f)) == cap
    assert B.capacity(P(capacity_factor=0.0)) == -1
    assert B.capacity(P(capacity_factor=-1.0)) == -1
    assert B.capacity(P(T=64, E=8, top_k=1, capacity_factor=1.1)) == 8
    assert B.capacity(P(T=16, E=8, top_k=1, capacity_factor=0.05)) == 0
    # the two capacity configurations: 1.25 * 8192 * 1 / 64 and 2.0 * 16384 * 6 / 64
    assert B.capacity(P(T=8192, D=1024, DH=4096, D_out=1024, E=64, top_k=1,
                        capacity_factor=1.25)) == 160
    assert B.capacity(P(T=16384, D=2048, DH=1408, D_out=2048, E=64, top_k=6,
                        capacity_factor=2.0)) == 3072
    assert B.capacity(P(top_k=0)) == -2


def test_workspace_size():
    assert B.workspace_size(P(top_k=0)) == 0
    a = B.workspace_size(P(T=100))
    b = B.workspace_size(P(T=1000))
    assert 0 < a < b
    # forward keeps the hidden activations and the expert outputs of every slot
    p = P(T=1000)
    assert b >= p.T * p.top_k * (p.DH + p.D_out) * 2
    assert B.workspace_size(P(T=0)) >= 0


def test_workspace_split_slots_follow_k():
    """The bf16 GEMMs' split-K partial tiles (64 MiB at most) are reserved only where a K can
    be split (K >= 4096, at least two parts of 2048), and only as many as the launch's tile
    bound allows: a 16-token layer with short K needs none of them."""
    mib, tile = 1 << 20, 256 * 256 * 4
    small = B.workspace_size(P(T=16, D=512, DH=1024, D_out=512, E=8, top_k=2))
    assert small < mib
    # the same layer with DH = 4096: the down product's K can be split, into at most as many
    # parts as its launch has blocks: (1 M-tile + 8 experts' last tiles) x 2 column tiles,
    # rounded up to 8 = 24 tiles of 256 KiB
    deep = B.workspace_size(P(T=16, D=512, DH=4096, D_out=512, E=8, top_k=2))
    extra_h = 32 * (4096 - 1024) * 2  # the larger hidden activations
    assert deep - small - extra_h == 24 * tile
    # fp32 layers never split
    f32 = B.workspace_size(P(T=16, D=512, DH=4096, D_out=512, E=8, top_k=2, dtype="f32"))
    assert f32 < deep
    # the Mixtral-shaped layer reserves all 256 slots (64 MiB)
    big = B.workspace_size(P(T=4096, D=4096, DH=14336, D_out=4096, E=8, top_k=2))
    assert big >= 8192 * (14336 + 4096) * 2 + 256 * tile


def _call(fn, p, *ptrs, ws_bytes=0):
    lib = B.lib()
    return getattr(lib, fn)(ctypes.byref(p.c()), *ptrs)


def test_error_paths_return_before_any_launch():
    """Invalid arguments are reported from host checks alone (no device is touched)."""
    lib = B.lib()
    fake = 1 << 20  # never dereferenced: every call below fails its host checks first
    p_bad = P(top_k=0)
    assert lib.moe_route(ctypes.byref(p_bad.c()), fake, fake, None, fake, fake, fake, None,
                         None, None, fake, 1 << 30, None) == B.MOE_ERR_INVALID_ARG
    p = P()
    # missing aux_loss
    assert lib.moe_route(ctypes.byref(p.c()), fake, fake, None, fake, fake, None, None, None,
                         None, fake, 1 << 30, None) == B.MOE_ERR_INVALID_ARG
    # workspace too small / misaligned / missing
    assert lib.moe_route(ctypes.byref(p.c()), fake, fake, None, fake, fake, fake, None, None,
                         None, fake, 16, None) == B.MOE_ERR_WORKSPACE
    assert lib.moe_route(ctypes.byref(p.c()), fake, fake, None, fake, fake, fake, None, None,
                         None, fake + 8, 1 << 30, None) == B.MOE_ERR_WORKSPACE
    assert lib.moe_route(ctypes.byref(p.c()), fake, fake, None, fake, fake, fake, None, None,
                         None, None, 0, None) == B.MOE_ERR_WORKSPACE
    # SwiGLU without its third matrix; ReLU without its second
    assert lib.moe_expert_ffn(ctypes.byref(p.c()), fake, fake, fake, None, fake, fake, fake,
                              1 << 30, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_expert_ffn(ctypes.byref(P(kind="relu2").c()), fake, fake, fake, None, None,
                              fake, fake, 1 << 30, None) == B.MOE_ERR_INVALID_ARG
    # dispatch without offsets; combine without gates
    assert lib.moe_dispatch(ctypes.byref(p.c()), fake, fake, fake, None, fake, fake, None, fake,
                            1 << 30, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_combine(ctypes.byref(p.c()), fake, fake, None, fake, None) == \
        B.MOE_ERR_INVALID_ARG
    # forward: unsupported expert count, null problem
    assert lib.moe_forward(ctypes.byref(P(E=300, top_k=2).c()), *([fake] * 14), 1 << 30,
                           None) == B.MOE_ERR_UNSUPPORTED
    assert lib.moe_forward(None, *([fake] * 14), 1 << 30, None) == B.MOE_ERR_INVALID_ARG


def test_no_alloc_route_host_checks():
    """moe_route_noalloc: invalid arguments, and a problem whose routing scratch exceeds the
    fixed device array, are refused by host checks before the device is touched."""
    lib = B.lib()
    fake = 1 << 20
    assert lib.moe_route_noalloc(ctypes.byref(P(top_k=0).c()), fake, fake, None, fake, fake,
                                 fake, None, None, None, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_route_noalloc(ctypes.byref(P().c()), fake, fake, None, fake, fake, None,
                                 None, None, None, None) == B.MOE_ERR_INVALID_ARG
    big = P(T=1 << 20, D=2048, E=256, top_k=8)
    assert lib.moe_route_noalloc(ctypes.byref(big.c()), fake, fake, None, fake, fake, fake,
                                 None, None, None, None) == B.MOE_ERR_SCRATCH_LIMIT
    assert "MOE_NOALLOC_SCRATCH_BYTES" in B.status_string(B.MOE_ERR_SCRATCH_LIMIT)


def test_status_strings():
    for s in range(6):
        assert B.status_string(s).startswith("MOE_")
    assert "unknown" in B.status_string(99)


def test_binding_refuses_host_tensors():
    import torch
    with pytest.raises(ValueError):
        B._ptr(torch.zeros(4))


def test_product_path_never_touches_the_oracle():
    """The package and its binding import nothing from oracle/ (the oracle is test
    infrastructure only), checked both on the sources and in a fresh interpreter."""
    import subprocess
    import sys
    pkg = Path(B.__file__).resolve().parent
    for f in list(pkg.rglob("*.py")) + list(pkg.rglob("*.hip")) + list(pkg.rglob("*.hpp")):
        text = f.read_text()
        assert not re.search(r"^\s*(import|from)\s+oracle\b", text, flags=re.M), f
        assert "oracle/" not in text, f
    code = ("import sys, expert_ffn_layer_router_amd as m; "
            "from expert_ffn_layer_router_amd import binding, accounting; binding.lib(); "
            "assert not any(k == 'oracle' or k.startswith('oracle.') for k in sys.modules)")
    subprocess.run([sys.executable, "-c", code], check=True, cwd=str(pkg.parent))


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "LIB_PATH", tmp_path / "libmoe.so")
    with pytest.raises(RuntimeError, match="not built"):
        B.lib()


# --- moe_options (host checks only; every call below returns before any launch) ---------

def test_workspace_size_ex():
    p = P(capacity_factor=2.0)
    assert B.workspace_size_ex(p, None) == B.workspace_size(p)
    L = B.lib()
    opts = B.MoeOptions(None, None, 1, 0, None)
    assert L.moe_workspace_size_ex(ctypes.byref(p.c()), ctypes.byref(opts)) == B.workspace_size(p)
    # the padded layout needs room for E * capacity rows (> T * k at capacity factor 2)
    padded = B.MoeOptions(None, None, 0, 1, None)
    assert L.moe_workspace_size_ex(ctypes.byref(p.c()), ctypes.byref(padded)) > B.workspace_size(p)
    # ... and a capacity
    assert L.moe_workspace_size_ex(ctypes.byref(P().c()), ctypes.byref(padded)) == 0
    # noise weights without the draw (or the reverse) are not options
    half = B.MoeOptions(0x1000, None, 0, 0, None)
    assert L.moe_workspace_size_ex(ctypes.byref(p.c()), ctypes.byref(half)) == 0


def test_option_entry_points_reject_bad_options_before_launching():
    L = B.lib()
    p = P()
    pc = ctypes.byref(p.c())
    fake = 0x1000  # never dereferenced: the checks fail first
    half = ctypes.byref(B.MoeOptions(fake, None, 0, 0, None))
    st = L.moe_route_ex(pc, half, fake, fake, None, fake, fake, fake, None, None, None, fake,
                        1 << 30, None)
    assert st == B.MOE_ERR_INVALID_ARG
    padded_nocap = ctypes.byref(B.MoeOptions(None, None, 0, 1, None))
    st = L.moe_forward_ex(pc, padded_nocap, fake, fake, None, fake, fake, fake, fake, fake, fake,
                          fake, fake, fake, fake, fake, 1 << 30, None, None)
    assert st == B.MOE_ERR_INVALID_ARG
    # padded dispatch without a capacity
    st = L.moe_dispatch_padded(pc, fake, fake, fake, fake, fake, fake, None, fake, 1 << 30, None)
    assert st == B.MOE_ERR_INVALID_ARG
    # a workspace too small for the padded layout
    pcap = P(capacity_factor=2.0)
    need = B.workspace_size_ex(pcap, None)
    padded = ctypes.byref(B.MoeOptions(None, None, 0, 1, None))
    st = L.moe_forward_ex(ctypes.byref(pcap.c()), padded, fake, fake, None, fake, fake, fake, fake,
                          fake, fake, fake, fake, fake, fake, 1 << 20, need, None, None)
    assert st == B.MOE_ERR_WORKSPACE



def test_backward_and_training_entry_points_check_before_launching():
    """moe_backward, moe_forward_train and moe_backward_saved report bad arguments from host
    checks alone (no device is touched)."""
    lib = B.lib()
    fake = 1 << 20  # never dereferenced
    big = 1 << 40
    p = P()
    pp = ctypes.byref(p.c())
    # moe_backward: a NaN loss weight; SwiGLU without dw2; a short workspace
    assert lib.moe_backward(pp, fake, fake, None, fake, fake, fake, fake, float("nan"), fake,
                            fake, None, fake, fake, fake, fake, big, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_backward(pp, fake, fake, None, fake, fake, fake, fake, 0.5, fake, fake, None,
                            fake, fake, None, fake, big, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_backward(pp, fake, fake, None, fake, fake, fake, fake, 0.5, fake, fake, None,
                            fake, fake, fake, fake, 16, None) == B.MOE_ERR_WORKSPACE
    # moe_forward_train: no aux_loss; a short, a misaligned and a missing saved buffer
    assert lib.moe_forward_train(pp, fake, fake, None, fake, fake, fake, fake, fake, fake, None,
                                 fake, fake, fake, fake, big, fake, big,
                                 None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_forward_train(pp, fake, fake, None, fake, fake, fake, fake, fake, fake, fake,
                                 fake, fake, fake, fake, 16, fake, big,
                                 None) == B.MOE_ERR_WORKSPACE
    assert lib.moe_forward_train(pp, fake, fake, None, fake, fake, fake, fake, fake, fake, fake,
                                 fake, fake, fake, fake + 8, big, fake, big,
                                 None) == B.MOE_ERR_WORKSPACE
    assert lib.moe_forward_train(pp, fake, fake, None, fake, fake, fake, fake, fake, fake, fake,
                                 fake, fake, fake, None, 0, fake, big,
                                 None) == B.MOE_ERR_WORKSPACE
    # moe_backward_saved: no expert_counts; a short saved buffer
    assert lib.moe_backward_saved(pp, fake, fake, fake, fake, fake, fake, fake, None, fake, fake,
                                  fake, big, fake, 0.5, fake, fake, None, fake, fake, fake, fake,
                                  big, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_backward_saved(pp, fake, fake, fake, fake, fake, fake, fake, fake, fake, fake,
                                  fake, 16, fake, 0.5, fake, fake, None, fake, fake, fake, fake,
                                  big, None) == B.MOE_ERR_WORKSPACE


def test_saved_size():
    """The saved state holds the logits, the permutation and a, b, h, y per slot row."""
    p = P(T=64, D=32, DH=48, D_out=32, E=8, top_k=2)
    R = 64 * 2
    need = 64 * 8 * 4 + R * 4 + 3 * R * 48 * 2 + R * 32 * 2
    got = B.saved_size(p)
    assert need <= got <= need + 6 * 256
    assert B.saved_size(P(kind="relu2")) < got  # no b
    assert B.saved_size(P(top_k=0)) == 0
