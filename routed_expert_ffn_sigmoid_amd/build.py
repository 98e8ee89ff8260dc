"""Builds the HIP library libmoe_hip.so for gfx950 with hipcc (in-tree).

Each source is compiled to an object of its own, in parallel, then the objects are linked into the
shared library.  Every call compiles everything again.
"""
import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmoe_hip.so")
ARCH = "gfx950"

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed-fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden", "-Wall", "-Wno-unused-result",
]
# hipcc's host pass warns that it does not know the packed-fp32 feature; that line is dropped
_NOISE = ("'-packed-fp32-ops' is not a recognized feature", "(ignoring feature)")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if not any(n in l for n in _NOISE))
    return r.returncode, err


def build(verbose: bool = False, extra=()) -> str:
    os.makedirs(OBJ, exist_ok=True)
    jobs = []
    for src in sources():
        obj = os.path.join(OBJ, os.path.basename(src)[:-4] + ".o")
        jobs.append((["hipcc", *FLAGS, *extra, "-c", "-o", obj, src], obj))
    if verbose:
        for cmd, _ in jobs:
            print(" ".join(cmd), flush=True)
    workers = min(len(jobs), max(1, (os.cpu_count() or 4)))
    with cf.ThreadPoolExecutor(workers) as ex:
        results = list(ex.map(lambda j: _run(j[0]), jobs))
    failed = False
    for (cmd, _), (rc, err) in zip(jobs, results):
        if err.strip():
            print(err, file=sys.stderr)
        failed = failed or rc != 0
    if failed:
        raise RuntimeError("hipcc failed")
    link = ["hipcc", "-shared", f"--offload-arch={ARCH}", "-fPIC", "-o", LIB + ".tmp", *[o for _, o in jobs]]
    if verbose:
        print(" ".join(link), flush=True)
    rc, err = _run(link)
    if err.strip():
        print(err, file=sys.stderr)
    if rc != 0:
        raise RuntimeError(f"hipcc link failed ({rc})")
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
