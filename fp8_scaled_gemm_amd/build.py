"""Build libfp8sg.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Flags that matter for the numerics:
  -ffp-contract=off     no FMA contraction: the fp32 multiplies of the scale,
                        quantize, epilogue and unscale steps stay single-rounded
  -fhip-fp32-correctly-rounded-divide-sqrt   IEEE fp32 division (1/scale)
  -Xclang -target-feature -Xclang -packed-fp32-ops   no packed fp32 VALU ops
No fast-math: the fp64 scale divisions must stay IEEE.

The compiler's per-kernel resource report is read on every build: a kernel
that spills more than MAX_SPILL_VGPRS registers to scratch fails the build (a
change to the GEMM's loop shape once spilled its accumulators and ran 30x
slower with correct results).
"""
import concurrent.futures as cf
import glob
import os
import re
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfp8sg.so")
OBJDIR = os.path.join(HERE, "_build")
ARCH = os.environ.get("FP8SG_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
         "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-command-line-argument"]
MAX_SPILL_VGPRS = 64


def spills(stderr: str) -> dict:
    """{kernel: VGPRs spilled} from -Rpass-analysis=kernel-resource-usage remarks."""
    out, name = {}, None
    for line in stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
        m = re.search(r"VGPRs Spill: (\d+)", line)
        if m and name:
            out[name] = int(m.group(1))
    return out


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _compile(src, verbose):
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-Rpass-analysis=kernel-resource-usage", "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    bad = {k: v for k, v in spills(r.stderr or "").items() if v > MAX_SPILL_VGPRS}
    if bad:
        raise RuntimeError(f"{src}: kernels spill registers to scratch: {bad}")
    # the host pass does not know the packed-fp32 feature and says so; drop that
    # noise, and the resource remarks
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stderr or "").splitlines()
                    if noise not in l and "remark" not in l and "-Rpass" not in l).strip()
    if msg and verbose:
        print(msg, flush=True)
    return obj


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(jobs, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
