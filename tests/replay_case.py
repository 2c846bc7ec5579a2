"""Run a saved case again: python tests/replay_case.py DIR [--cpu-only]

DIR holds a workload written by synth.replay (the GPU parity tests write one
per failing case when CSA2_SAVE_FAILED names a directory).  The oracle's layer
chain runs on it; with a GPU (and without --cpu-only) the library's chain runs
too, and every layer's indices and attention output are compared under the
parity tests' bars.  Exit status 0 when they agree, 1 when they do not."""
import argparse
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, HERE)

import oracle  # noqa: E402
from synth.replay import load_workload  # noqa: E402


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("dir")
    ap.add_argument("--cpu-only", action="store_true")
    args = ap.parse_args()
    wl = load_workload(args.dir)
    print(f"{wl.name}: seed {wl.seed:#x}, {wl.n_seq} sequences, {wl.total_q} query rows, "
          f"{len(wl.layers)} layers", flush=True)
    ref = oracle.layer_chain(wl)
    print("oracle: done", flush=True)
    if args.cpu_only:
        return 0
    import torch
    if not torch.cuda.is_available():
        print("no GPU: oracle only")
        return 0
    from gpu_util import DevWorkload, run_chain
    outs, _, _ = run_chain(DevWorkload(wl))
    torch.cuda.synchronize()
    bad = 0
    for o, r in zip(outs, ref):
        idx_ok = np.array_equal(o["idx"].cpu().numpy(), r["idx"])
        got = o["out"].cpu().numpy().astype(np.float64)
        err = np.abs(got - r["out"])
        n_out = int((err > 2e-3 + 1e-2 * np.abs(r["out"])).sum())
        print(f"layer {r['layer']}: indices {'equal' if idx_ok else 'DIFFER'}, attention max abs err "
              f"{err.max():.3e}, {n_out} elements out of tolerance", flush=True)
        bad += (not idx_ok) + (n_out > 0)
    return 1 if bad else 0


if __name__ == "__main__":
    sys.exit(main())
