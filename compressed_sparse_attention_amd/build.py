"""Builds libcsa2.so in-tree with hipcc for gfx950 (MI355X)."""
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SO = os.path.join(HERE, "libcsa2.so")
SOURCES = sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))
HEADERS = sorted(glob.glob(os.path.join(HERE, "csrc", "*.h"))) + [os.path.join(ROOT, "include", "csa2.h")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-shared",
    "-fPIC",
    "-fvisibility=hidden",
    "-DCSA2_BUILDING_LIBRARY",
    "-I" + os.path.join(ROOT, "include"),
    # packed FP32 VALU forms are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in VGPRs: the epilogues read them without v_accvgpr_read copies
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def up_to_date():
    if not os.path.exists(SO):
        return False
    t = os.path.getmtime(SO)
    return all(os.path.getmtime(f) <= t for f in SOURCES + HEADERS + [__file__])


def build(force=True, verbose=False):
    if not force and up_to_date():
        return SO
    tmp = SO + ".tmp"
    cmd = [HIPCC, *FLAGS, *SOURCES, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops"
    msgs = [l for l in (r.stdout + r.stderr).splitlines() if noise not in l and l.strip()]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), file=sys.stderr)
    os.replace(tmp, SO)
    return SO


if __name__ == "__main__":
    print(build(force=True, verbose=True))
