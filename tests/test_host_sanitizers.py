"""The host code of the library (argument checks, workspace layout arithmetic, status strings)
built with AddressSanitizer and UndefinedBehaviorSanitizer, with the host-only ABI tests run
against that build. CPU only: nothing is launched."""

import shutil

import pytest

from expert_ffn_layer_router_amd import sanitize_host as S


@pytest.mark.timeout(900)
def test_host_abi_tests_pass_under_asan_and_ubsan():
    if shutil.which("hipcc") is None and not S.Path("/opt/rocm/bin/hipcc").exists():
        pytest.skip("hipcc is not installed")
    try:
        rt = S.runtime()
    except Exception as e:  # no sanitizer runtime in this toolchain
        pytest.skip(f"no ASan runtime: {e}")
    assert rt.is_file()
    lib = S.build()
    r = S.run_host_tests(lib)
    report = (r.stdout[-4000:] + "\n" + r.stderr[-4000:])
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, report
    assert r.returncode == 0, report
    assert " passed" in r.stdout, report
