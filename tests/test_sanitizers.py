"""AddressSanitizer and UndefinedBehaviorSanitizer builds of the CPU-side code, run on the CPU.

- The oracle (oracle/moe_oracle.c), built with gcc under both sanitizers, runs every function on small seeded
  layers (tests/sanitize/oracle_driver.c); any report aborts it.
- The library's host code (argument checks, workspace sizing, path choice, the static entry point's checks),
  built host-only under both sanitizers, is driven over 20000 random shapes by tests/sanitize/abi_driver.cpp,
  which never reaches the GPU.
"""
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
SAN_ENV = dict(os.environ, UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd[:3])} ... failed:\n{r.stderr[-3000:]}"



def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    subprocess.run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off", "-fopenmp",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-o", exe,
                    os.path.join(ROOT, "oracle", "moe_oracle.c"), os.path.join(SAN, "oracle_driver.c"), "-lm"],
                   check=True)
    env = dict(SAN_ENV, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1")
    r = subprocess.run([exe], env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "oracle driver ok" in r.stdout


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not found")
def test_abi_host_code_under_sanitizers(tmp_path):
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all"]
    srcs = sorted(glob.glob(os.path.join(ROOT, "routed_expert_ffn_sigmoid_amd", "csrc", "*.hip")))
    objs = [str(tmp_path / (os.path.basename(src) + ".o")) for src in srcs]
    with cf.ThreadPoolExecutor(min(len(srcs), os.cpu_count() or 4)) as ex:
        list(ex.map(lambda so: _run(["hipcc", "-std=c++17", "-O1", "-g", "-fPIC", "--offload-arch=gfx950", *san,
                                     "-c", "-o", so[1], so[0]]), zip(srcs, objs)))
    drv = str(tmp_path / "abi_driver.o")
    _run(["hipcc", "-std=c++17", "-O1", "-g", "-fPIC", "--offload-arch=gfx950", "--cuda-host-only", *san, "-c", "-o",
          drv, os.path.join(SAN, "abi_driver.cpp")])
    exe = str(tmp_path / "abi_driver")
    _run(["hipcc", "--offload-arch=gfx950", *san, "-o", exe, drv, *objs])
    # the HIP runtime keeps allocations until exit: leak reports would be its, so leak checking is off here
    env = dict(SAN_ENV, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    r = subprocess.run([exe], env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi driver ok" in r.stdout
