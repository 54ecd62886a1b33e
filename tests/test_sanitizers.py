"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU
only; no kernel is launched):

* the oracle (oracle/lora_oracle.c) built with gcc and both sanitizers, every
  exported function run on small seeded inputs with ragged sizes;
* the library's host code (api.cpp: argument checks, workspace planning, the
  segment-table checker, status strings; packer.cpp: the batching helpers)
  built with the sanitizers on its host pass only, linked with the library's
  own (uninstrumented) kernel objects, and driven through every rejection path
  and seeded random batches.

Any sanitizer report aborts the driver (-fno-sanitize-recover=all)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "lora_fine_tuning_amd", "csrc")
BUILD = os.path.join(ROOT, "lora_fine_tuning_amd", "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANGXX = "/opt/rocm/llvm/bin/clang++"
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=300, **kw)
    assert res.returncode == 0, f"{' '.join(cmd)}\n{res.stdout}\n{res.stderr}"
    return res


def test_oracle_under_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("no gcc")
    exe = str(tmp_path / "oracle_san")
    run(["gcc", "-O1", "-g", "-fopenmp", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-fno-omit-frame-pointer", os.path.join(ROOT, "oracle", "lora_oracle.c"),
         os.path.join(HERE, "oracle_driver.c"), "-o", exe, "-lm"])
    res = run([exe], env=dict(os.environ, OMP_NUM_THREADS="2"))
    assert "all calls completed" in res.stdout


def test_library_host_code_under_sanitizers(tmp_path):
    kernels = [os.path.join(BUILD, f) for f in ("lowrank_kernels.hip.o", "gemm_kernels.hip.o", "dora_kernels.hip.o")]
    if not (os.path.exists(HIPCC) and os.path.exists(CLANGXX) and all(map(os.path.exists, kernels))):
        pytest.skip("hipcc / clang++ or the built kernel objects are missing")
    flags = ["-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-I", os.path.join(ROOT, "include"),
             "-I", CSRC, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    objs = []
    for src in ("api.cpp", "packer.cpp"):
        obj = str(tmp_path / (src + ".o"))
        run([HIPCC] + flags + SAN_HOST + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    drv = str(tmp_path / "abi_driver.o")
    run([CLANGXX, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
         "-c", os.path.join(HERE, "abi_driver.cpp"), "-o", drv])
    exe = str(tmp_path / "abi_san")
    run([CLANGXX, "-fsanitize=address,undefined", drv] + objs + kernels +
        ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    res = run([exe])
    assert "all checks passed" in res.stdout
