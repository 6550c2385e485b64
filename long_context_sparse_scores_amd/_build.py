"""Compile the HIP sources under csrc/ into long_context_sparse_scores_amd/libdsa.so (gfx950)."""
import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libdsa.so")
ARCH = "gfx950"

# Packed-fp32 VALU forms are disabled for every HIP translation unit.  MFMA
# results go to VGPRs rather than AGPRs (no v_accvgpr_read copies before the
# indexers' epilogues; the other kernels compile the same either way).
HIP_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-mllvm", "-amdgpu-mfma-vgpr-form"]


# Per-file additions.  indexer.hip: its ReLU (fmaxf) is one v_max_f32 only
# when NaNs need not be quieted; the scores are defined for finite inputs.
FILE_FLAGS = {"indexer.hip": ["-fno-honor-nans"]}


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile each .hip to an object (in parallel), then link libdsa.so."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    procs, objs = [], []
    for src in sources():
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        objs.append(obj)
        cmd = ["hipcc"] + HIP_FLAGS + FILE_FLAGS.get(os.path.basename(src), []) + ["-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        if len([p for _, p in procs if p.poll() is None]) >= jobs:
            procs[0][1].wait()
    for cmd, p in procs:
        out, _ = p.communicate()
        text = "\n".join(l for l in out.decode(errors="replace").splitlines() if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            raise RuntimeError("hip compile failed: %s\n%s" % (" ".join(cmd), text))
        if verbose and text.strip():
            print(text)
    tmp = LIB + ".tmp"
    link = ["hipcc", "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
