"""Build the halo-attention HIP library for gfx950 (MI355X).

Compiles ``csrc/*.hip`` with hipcc into ``libhaloattn.so`` next to this file.
hipcc cross-compiles for gfx950 without a GPU present.  Packed fp32 VALU
instructions are disabled for all device code.
"""
from __future__ import annotations

import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB_PATH = os.path.join(HERE, "libhaloattn.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    raise RuntimeError("hipcc not found")


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def source_id() -> str:
    """First 16 hex digits of SHA-256 over csrc/'s file names and contents
    (name order): the identifier compiled into the library."""
    import hashlib
    h = hashlib.sha256()
    for path in sorted(glob.glob(os.path.join(CSRC, "*"))):
        if os.path.isfile(path):
            h.update(os.path.basename(path).encode())
            with open(path, "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()[:16]


# Extra flags per source.  The matrix-core kernel keeps MFMA results in
# ordinary VGPRs (no accumulator-register copies) and, having no NaN
# semantics to preserve in its max reductions, skips NaN canonicalisation.
PER_FILE_FLAGS = {
    "kernel_mfma.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form"],
    "kernel_ring.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form"],
    "kernel_tile.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form"],
    "kernel_bwd_mfma.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form"],
    "kernel_bwd_tile.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form"],
    "kernel_wide.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form"],
    "kernel_layer.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-command-line-argument"]


def build(verbose: bool = False, defines: tuple = (), out: str | None = None) -> str:
    """Compile every csrc/*.hip for gfx950 and link libhaloattn.so.

    ``defines``: extra -D flags (tuning builds); ``out``: output path.
    """
    out = out or LIB_PATH
    bdir = os.path.join(HERE, "_build", f"{os.getpid()}")
    os.makedirs(bdir, exist_ok=True)
    objs, logs = [], []
    procs = []
    build_id = source_id()
    for src in sources():
        obj = os.path.join(bdir, os.path.basename(src) + ".o")
        cmd = [hipcc(), f"--offload-arch={ARCH}", *COMMON, "-I", INCLUDE, *[f"-D{d}" for d in defines],
               f'-DHALO_BUILD_ID="{build_id}"', *PER_FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        objs.append(obj)
    for cmd, pr in procs:
        text, _ = pr.communicate()
        if pr.returncode != 0:
            raise RuntimeError(f"hipcc failed ({pr.returncode}):\n{' '.join(cmd)}\n{text}")
        logs.append(text)
    tmp = out + f".tmp{os.getpid()}"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,--no-undefined", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed ({res.returncode}):\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    if verbose:
        noise = "is not a recognized feature for this target"
        for line in "".join(logs).splitlines():
            if noise not in line:
                print(line)
    os.replace(tmp, out)
    for o in objs:
        os.remove(o)
    os.rmdir(bdir)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
