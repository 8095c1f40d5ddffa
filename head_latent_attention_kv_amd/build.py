"""Build libmla_laga.so (HIP, gfx950) in-tree.

    python -m head_latent_attention_kv_amd.build

Every source under csrc/ is compiled with hipcc for gfx950 into _build/ at
the repository root and linked into head_latent_attention_kv_amd/
libmla_laga.so. Packed fp32 VALU instructions are turned off for device code
(-packed-fp32-ops); the host pass warns that it does not know the feature,
which is harmless.
"""

from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmla_laga.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
    "-Wno-unused-function", "-Wno-unused-command-line-argument",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


# Per-source device flags. The backward kernels keep their large gradient
# accumulators next to score tiles that the softmax reads on the VALU; the
# backend otherwise picks the AGPR form for every MFMA of such a kernel and
# then copies each score tile back to VGPRs, so ask for the VGPR form there.
DEVICE_FLAGS = {
    "fast_bwd.hip": ["-Xarch_device", "-mllvm=-amdgpu-mfma-vgpr-form"],
    # decode attention: the score tile and the output accumulators both in
    # VGPRs; the AGPR form put the score chain in AGPRs next to the
    # accumulators and spilled to scratch
    "decode.hip": ["-Xarch_device", "-mllvm=-amdgpu-mfma-vgpr-form"],
    # forward attention: the backend's ILP-first scheduling strategy orders
    # the two score chains' fragment reads and the softmax work better
    # around the products (about 1.5% on the attention kernel)
    "fast_fwd.hip": ["-Xarch_device", "-mllvm=-amdgpu-sched-strategy=max-ilp"],
}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMMON, *DEVICE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the device-only feature flag: harmless
    noise = ("packed-fp32-ops' is not a recognized feature",)
    err = "\n".join(ln for ln in r.stderr.splitlines()
                    if ln.strip() and not any(n in ln for n in noise))
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip():
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    workers = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


if __name__ == "__main__":
    build()
