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
    "-fPIC",
    "-fvisibility=hidden",
    "-DCSA2_BUILDING_LIBRARY",
    "-I" + os.path.join(ROOT, "include"),
    # packed FP32 VALU forms are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# MFMA results in VGPRs: the epilogues read them without v_accvgpr_read copies.
# A source listed in AGPR_SOURCES is compiled without it (none is at present).
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
AGPR_SOURCES = set()


def up_to_date():
    if not os.path.exists(SO):
        return False
    t = os.path.getmtime(SO)
    return all(os.path.getmtime(f) <= t for f in SOURCES + HEADERS + [__file__])


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops"
    msgs = [l for l in (r.stdout + r.stderr).splitlines() if noise not in l and l.strip()]
    return r.returncode, msgs


def build(force=True, verbose=False):
    """Compile every .hip source to an object (in parallel), then link them
    into libcsa2.so."""
    if not force and up_to_date():
        return SO
    from concurrent.futures import ThreadPoolExecutor

    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src):
        name = os.path.basename(src)
        obj = os.path.join(objdir, name + ".o")
        extra = [] if name in AGPR_SOURCES else VGPR_FORM
        rc, msgs = _run([HIPCC, *FLAGS, *extra, "-c", src, "-o", obj])
        return src, obj, rc, msgs

    workers = max(1, min(len(SOURCES), os.cpu_count() or 4, 8))
    with ThreadPoolExecutor(workers) as ex:
        results = list(ex.map(compile_one, SOURCES))
    all_msgs = []
    for src, _, rc, msgs in results:
        if rc != 0:
            raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n" + "\n".join(msgs))
        all_msgs += msgs
    tmp = SO + ".tmp"
    rc, msgs = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *[o for _, o, _, _ in results], "-o", tmp])
    if rc != 0:
        raise RuntimeError("link failed:\n" + "\n".join(msgs))
    all_msgs += msgs
    if verbose and all_msgs:
        print("\n".join(all_msgs), file=sys.stderr)
    os.replace(tmp, SO)
    return SO


if __name__ == "__main__":
    print(build(force=True, verbose=True))
