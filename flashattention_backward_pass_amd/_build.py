"""Builds libfabwd.so (gfx950) in-tree with hipcc.

Every source under csrc/ is compiled to an object in _build/ (in parallel),
then linked into flashattention_backward_pass_amd/libfabwd.so.  Run as
``python -m flashattention_backward_pass_amd._build`` or through
``__graft_entry__.build()``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfabwd.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # hardware fp32 atomics for dQaccum (no compare-and-swap loops)
    "-munsafe-fp-atomics",
    "-Wno-unused-result",
    "-I", os.path.join(ROOT, "include"),
]


# Per-file flags.  The dK/dV kernel keeps every matrix accumulator in VGPRs
# (the softmax-gradient VALU work reads S and dP straight from them; the
# K/V operand slices are pinned to AGPRs in the source).
FILE_FLAGS = {
    "bwd_dkdv.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "bwd_fused.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],  # runs the dK/dV work units too
}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMMON_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass warns that it does not know the packed-fp32 feature; keep other messages
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compilation of {os.path.basename(src)} failed:\n{msg}")
    if verbose and msg.strip():
        print(msg, flush=True)
    return obj


def build(verbose: bool = False, jobs: int | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(8, len(srcs), os.cpu_count() or 1)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link of libfabwd.so failed:\n{r.stdout}{r.stderr}")
    _check_kernel_stubs(tmp)
    os.replace(tmp, LIB)
    return LIB


def _check_kernel_stubs(lib: str) -> None:
    """Fails if a kernel launch stub is missing from the library: the host
    compilation can drop a kernel without a diagnostic (seen with array
    elements passed straight into buffer-load builtins), which would only
    surface as an unresolved symbol when the library is loaded."""
    nm = shutil.which("nm") or "/opt/rocm/llvm/bin/llvm-nm"
    r = subprocess.run([nm, "-D", "--undefined-only", lib], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"nm failed on {lib}:\n{r.stderr}")
    missing = [l.split()[-1] for l in r.stdout.splitlines() if "__device_stub__" in l]
    if missing:
        raise RuntimeError("kernel launch stubs missing from libfabwd.so: " + ", ".join(missing))


PROBES = {
    "dq_update_probe": os.path.join(PKG, "probes", "dq_update_probe.cpp"),
    "issue_mix_probe": os.path.join(PKG, "probes", "issue_mix_probe.hip"),
}


def build_probe() -> list:
    """Builds the standalone measurement probes (probes/: the dQ-update traffic
    probe and the issue-mix probe) into _build/<name>; run them directly (or
    under rocprofv3).  Returns the binaries' paths."""
    os.makedirs(BUILD, exist_ok=True)
    out = []
    for name, src in PROBES.items():
        exe = os.path.join(BUILD, name)
        cmd = [hipcc(), "-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", src, "-o", exe]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"build of {name} failed:\n{r.stdout}{r.stderr}")
        out.append(exe)
    return out


if __name__ == "__main__":
    if "--probe" in sys.argv:
        print(build_probe())
    else:
        print(build(verbose="-v" in sys.argv))
