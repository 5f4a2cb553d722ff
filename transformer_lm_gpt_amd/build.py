"""Builds libgpt.so (the gfx950 kernels and the C ABI) in-tree with hipcc.

    python -m transformer_lm_gpt_amd.build [--jobs N]
    python -m transformer_lm_gpt_amd.build --asan

Every HIP source is compiled for gfx950 only. Packed fp32 instructions are
disabled for device code (-packed-fp32-ops); hipcc's host pass warns that it
does not know that feature, which is harmless.

--asan builds a second library, _build/asan/libgpt.so, whose host runtime
(runtime.cpp: configuration checks, layout planning, the launch sequences and
the error paths) is compiled with AddressSanitizer for the host only; the
kernels are the same gfx950 objects. Load it into a process with the sanitizer
runtime preloaded (asan_env() gives the environment), e.g. for the ABI tests,
which need no GPU:

    env $(python -m transformer_lm_gpt_amd.build --asan --print-env) python -m pytest tests/test_abi.py
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libgpt.so")

SOURCES = ["gemm.hip", "attention.hip", "rowops.hip", "embed_bwd.hip", "optim.hip", "decode.hip", "lora.hip", "runtime.cpp"]
ARCH = "gfx950"
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# per-source device flags: attention keeps its MFMA accumulators in ordinary VGPRs,
# so the softmax arithmetic on them needs no copies out of the accumulation registers
SOURCE_FLAGS = {"attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
COMMON_FLAGS = ["-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function"]


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found")
    return p


SNAP = os.path.join(BUILD, "src")
SNAP_CSRC = os.path.join(SNAP, os.path.relpath(CSRC, ROOT))
SNAP_INC = ["-I", os.path.join(SNAP, "include"), "-I", SNAP_CSRC]


def _snapshot() -> None:
    """Copies csrc/ and include/ into _build/src, in the repository's layout (the
    sources include the public header by a relative path). hipcc reads a source once for the
    device pass and again for the host pass; compiling from a frozen copy keeps an
    edit made during a build from giving host stubs and device code of different
    versions (a launch of such a kernel fails with a missing-symbol error)."""
    for d in (CSRC, INCLUDE):
        dst = os.path.join(SNAP, os.path.relpath(d, ROOT))
        if os.path.isdir(dst):
            shutil.rmtree(dst)
        shutil.copytree(d, dst, ignore=shutil.ignore_patterns("*.o", "__pycache__"))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON_FLAGS, *SNAP_INC, "-c", os.path.join(SNAP_CSRC, src), "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = [f"--offload-arch={ARCH}", *DEVICE_FLAGS, *SOURCE_FLAGS.get(src, [])]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


ASAN_DIR = os.path.join(BUILD, "asan")
ASAN_LIB = os.path.join(ASAN_DIR, "libgpt.so")
# host-only sanitizer flags: each -fsanitize= right after -Xarch_host
ASAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-fno-omit-frame-pointer", "-g"]


def asan_runtime() -> str:
    """Path of the compiler's shared AddressSanitizer runtime."""
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm", "bin", "clang++")
    if not os.path.exists(clang):
        clang = shutil.which("clang++") or clang
    r = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.exists(path):
        raise RuntimeError("AddressSanitizer runtime not found")
    return path


def asan_env() -> dict:
    """Environment that loads the sanitized library into an unsanitized Python:
    the runtime preloaded, leak checks off (the interpreter's own allocations are
    not ours), the binding pointed at the sanitized build."""
    return {"LD_PRELOAD": asan_runtime(), "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
            "GPT_MI355X_LIB": ASAN_LIB}


def build_asan(jobs: int = 8, verbose: bool = False) -> str:
    """The kernels as usual, runtime.cpp with host AddressSanitizer, linked into ASAN_LIB."""
    os.makedirs(ASAN_DIR, exist_ok=True)
    _snapshot()
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(_compile, [x for x in SOURCES if x != "runtime.cpp"]))
    obj = os.path.join(ASAN_DIR, "runtime.o")
    cmd = [hipcc(), *COMMON_FLAGS, *SNAP_INC, *ASAN_FLAGS, "-c", os.path.join(SNAP_CSRC, "runtime.cpp"), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
           "-shared-libasan", "-o", ASAN_LIB, *objs, obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(f"built {ASAN_LIB}")
    return ASAN_LIB


def build(jobs: int = 8, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    _snapshot()
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=min(8, os.cpu_count() or 1))
    ap.add_argument("--asan", action="store_true", help="build the host-sanitized runtime into _build/asan")
    ap.add_argument("--print-env", action="store_true", help="with --asan: only print the environment to load it")
    a = ap.parse_args(argv)
    if a.asan and a.print_env:
        print(" ".join(f"{k}={v}" for k, v in asan_env().items()))
        return 0
    if a.asan:
        build_asan(a.jobs, verbose=True)
    else:
        build(a.jobs, verbose=True)


if __name__ == "__main__":
    sys.exit(main())
