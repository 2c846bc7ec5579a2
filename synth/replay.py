"""Save a generated workload to disk and load it back, so that a failing case
can be replayed exactly: every array as raw little-endian bytes in its own
``.bin`` file, and a ``manifest.json`` with the workload's scalar fields, each
array's file, dtype, shape and SHA-256, and the layer schedule.  A layer cache
that is the workload's own array is stored once and referenced.  Loading checks
every file's size and digest and raises ``ValueError`` on any mismatch.

This is input plumbing only; it holds no step of the method.
"""
from __future__ import annotations

import hashlib
import json
import os

import numpy as np

from . import Layer, Workload

FORMAT = "csa2-workload-v1"

_WL_SCALARS = ("name", "seed", "ratio", "H", "Hm", "K", "W", "block", "max_blocks", "kv_fmt", "swa_fmt")
_WL_ARRAYS = ("n_entries", "entry_off", "q_off", "q_pos", "row_seq", "swa_row_off", "swa_pos0", "swa_len", "k_idx",
              "k_sc", "kv", "kv_sc", "replay_s")
_LAYER_SCALARS = ("index", "mode", "q_fmt", "build_pool")
_LAYER_ARRAYS = ("q_idx", "q_sc", "w", "q_main", "swa", "k_idx", "k_sc", "kv", "kv_sc")
_SHARED = ("k_idx", "k_sc", "kv", "kv_sc")  # a layer's caches may be the workload's own


def _put(directory, key, a, arrays):
    a = np.ascontiguousarray(a)
    raw = a.astype(a.dtype.newbyteorder("<"), copy=False).tobytes()
    fname = key + ".bin"
    with open(os.path.join(directory, fname), "wb") as f:
        f.write(raw)
    arrays[key] = {"file": fname, "dtype": a.dtype.newbyteorder("<").str, "shape": list(a.shape),
                   "sha256": hashlib.sha256(raw).hexdigest()}


def _get(directory, meta):
    path = os.path.join(directory, meta["file"])
    with open(path, "rb") as f:
        raw = f.read()
    dt = np.dtype(meta["dtype"])
    n = int(np.prod(meta["shape"], dtype=np.int64))
    if len(raw) != n * dt.itemsize:
        raise ValueError(f"{meta['file']}: {len(raw)} bytes, expected {n * dt.itemsize}")
    if hashlib.sha256(raw).hexdigest() != meta["sha256"]:
        raise ValueError(f"{meta['file']}: SHA-256 does not match the manifest")
    return np.frombuffer(raw, dtype=dt).astype(dt.newbyteorder("="), copy=True).reshape(meta["shape"])


def save_workload(wl: Workload, directory: str, note: str = "") -> str:
    """Write wl under `directory` (created if missing); returns the manifest path."""
    os.makedirs(directory, exist_ok=True)
    arrays = {}
    scalars = {k: (str(wl.name) if k == "name" else int(getattr(wl, k))) for k in _WL_SCALARS}
    man = {"format": FORMAT, "note": note, "scalars": scalars, "arrays": arrays, "layers": []}
    for k in _WL_ARRAYS:
        a = getattr(wl, k, None)
        if a is not None:
            _put(directory, k, a, arrays)
    for i, L in enumerate(wl.layers):
        ent = {k: (bool(getattr(L, k)) if k == "build_pool" else int(getattr(L, k))) for k in _LAYER_SCALARS}
        refs = {}
        for k in _LAYER_ARRAYS:
            a = getattr(L, k, None)
            if a is None:
                continue
            if k in _SHARED and getattr(wl, k) is a:
                refs[k] = "workload"
                continue
            key = f"layer{i}_{k}"
            _put(directory, key, a, arrays)
            refs[k] = key
        ent["arrays"] = refs
        man["layers"].append(ent)
    path = os.path.join(directory, "manifest.json")
    with open(path, "w") as f:
        json.dump(man, f, indent=1, sort_keys=True)
    return path


def load_workload(directory: str) -> Workload:
    """Read a workload written by save_workload, checking every array."""
    with open(os.path.join(directory, "manifest.json")) as f:
        man = json.load(f)
    if man.get("format") != FORMAT:
        raise ValueError(f"{directory}: not a {FORMAT} manifest")
    arrays = {k: _get(directory, m) for k, m in man["arrays"].items()}
    sc = man["scalars"]
    wl = Workload(sc["name"], int(sc["seed"]), int(sc["ratio"]), int(sc["H"]), int(sc["Hm"]), int(sc["K"]),
                  int(sc["W"]), int(sc["block"]), int(sc["max_blocks"]), arrays["n_entries"], arrays["entry_off"],
                  arrays["q_off"], arrays["q_pos"], arrays["row_seq"], arrays["swa_row_off"], arrays["swa_pos0"],
                  arrays["swa_len"])
    for k in ("k_idx", "k_sc", "kv", "kv_sc", "replay_s"):
        if k in arrays:
            setattr(wl, k, arrays[k])
    wl.kv_fmt = int(sc["kv_fmt"])
    wl.swa_fmt = int(sc["swa_fmt"])
    for ent in man["layers"]:
        L = Layer(index=int(ent["index"]), mode=int(ent["mode"]), q_fmt=int(ent["q_fmt"]),
                  build_pool=bool(ent["build_pool"]))
        for k, ref in ent["arrays"].items():
            setattr(L, k, getattr(wl, k) if ref == "workload" else arrays[ref])
        wl.layers.append(L)
    return wl
