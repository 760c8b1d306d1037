"""Build libzcmoe.so (the HIP kernels and the C ABI) for gfx950, in-tree.

Each .hip file is compiled to an object with hipcc, then linked into
moe_layer_zero_amd/libzcmoe.so.  Flags:
  --offload-arch=gfx950                  MI355X only, no other targets
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                         keep packed fp32 ops out of the ISA
  -ffp-contract=off (router, pid)        the routing keys and the bias update
                                         follow a fixed IEEE operation order
  -mllvm -amdgpu-atomic-optimizer-strategy=None (packed GEMMs)
                                         tile claims stay single-lane atomics
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
OUT = os.path.join(HERE, "libzcmoe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
SOURCES = ["api.hip", "router.hip", "dispatch.hip", "gemm.hip", "gemm_fwd.hip", "gemm_fwdp.hip",
           "gemm_fwdq.hip", "gemm_dw.hip", "gemm_rmw.hip", "combine.hip", "pid.hip"]
STRICT_FP = {"router.hip", "pid.hip"}
# The persistent GEMMs claim tiles with one lane's atomic whose result is used
# a whole tile later; the atomic optimizer would broadcast it to the wave at
# once, making every claim wait for all memory operations in flight.
NO_ATOMIC_OPT = {"gemm_fwdp.hip", "gemm_fwdq.hip", "gemm_dw.hip", "gemm_rmw.hip"}

COMMON = ["-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
          "-Wno-unused-function", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          f"-I{CSRC}"]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, src.replace(".hip", ".o"))
    cmd = [HIPCC, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
    if src in STRICT_FP:
        cmd.insert(1, "-ffp-contract=off")
    if src in NO_ATOMIC_OPT:
        cmd[1:1] = ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in (r.stderr or "").splitlines()
                    if "packed-fp32-ops" not in l and "is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip() and verbose:
        print(err, flush=True)
    return obj


def build(verbose: bool = False, jobs: int = 6) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", OUT + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(OUT + ".tmp", OUT)
    return OUT


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print("built", OUT)
