"""The host runtime under AddressSanitizer: the library built with
`python -m transformer_lm_gpt_amd.build --asan` (runtime.cpp instrumented for the
host, the same gfx950 kernels) runs the C-ABI tests, which need no GPU, in a child
process with the sanitizer runtime preloaded. Any invalid host memory access in
the configuration checks, layout planning or error paths aborts that process."""
import os
import subprocess
import sys

import pytest

from transformer_lm_gpt_amd import build as Bl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_abi_tests_pass_under_host_asan():
    try:
        Bl.asan_runtime()
    except RuntimeError:
        pytest.skip("no AddressSanitizer runtime in this toolchain")
    Bl.build_asan(jobs=min(8, os.cpu_count() or 1))
    syms = subprocess.run(["nm", "-D", Bl.ASAN_LIB], capture_output=True, text=True).stdout
    assert "__asan_report_load" in syms            # the runtime is instrumented
    env = dict(os.environ, **Bl.asan_env())
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr
