"""Helpers for the GPU tests: upload a synthetic workload and run the layer
chain through the C ABI.  (Not a test module.)"""
import contextlib
import math
import os
import re

import numpy as np
import torch

from compressed_sparse_attention_amd import csa2 as C

SCALE = 1.0 / math.sqrt(512.0)


def dev(a, device="cuda"):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(device)


class DevWorkload:
    def __init__(self, wl, device="cuda"):
        self.wl = wl
        self.device = torch.device(device)
        self.batch = C.Batch.from_workload(wl, device)
        self.swa = C.SwaLayout.from_workload(wl, replay_s=getattr(wl, "replay_s", None), device=device)
        self.k_idx = dev(wl.k_idx, device)
        self.k_sc = dev(wl.k_sc, device)
        self.kv = dev(wl.kv, device)
        self.kv_sc = dev(wl.kv_sc, device)
        self.layers = []
        for L in wl.layers:
            d = {"index": L.index, "mode": L.mode, "q_fmt": L.q_fmt, "build_pool": L.build_pool}
            for f in ("q_idx", "q_sc", "w", "q_main", "swa"):
                a = getattr(L, f)
                d[f] = None if a is None else dev(a, device)
            # a Full layer's own caches; the first Full layer's are the workload's
            for f in ("k_idx", "k_sc", "kv", "kv_sc"):
                a = getattr(L, f, None)
                d[f] = None if a is None else (getattr(self, f) if a is getattr(wl, f) else dev(a, device))
            self.layers.append(d)


def prepare_chain(dw, want_idx=True, want_lse=True, ws=None, pool=True):
    """Allocate the outputs and build the csa2_layer array once; returns
    (call, outs, pools) where call() enqueues one csa2_layer_chain."""
    wl = dw.wl
    nq = wl.total_q
    device = dw.device
    specs, outs = [], []
    for d in dw.layers:
        out = torch.empty((nq, wl.Hm, 512), dtype=torch.float32, device=device)
        lse = torch.empty((nq, wl.Hm), dtype=torch.float32, device=device) if want_lse else None
        idx = torch.empty((nq, wl.K), dtype=torch.int32, device=device) if want_idx else None
        sp = {"mode": d["mode"], "flags": C.CSA2_LAYER_BUILD_POOL if d["build_pool"] else 0, "q_fmt": d["q_fmt"],
              "q_idx": d["q_idx"], "q_sc": d["q_sc"], "w": d["w"], "q_main": d["q_main"], "swa": d["swa"],
              "out": out, "lse": lse, "idx_out": idx}
        if d["mode"] == C.CSA2_MODE_FULL:
            own = d.get("kv") is not None
            sp.update(kv_fp4=d["kv"] if own else dw.kv, kv_sc=d["kv_sc"] if own else dw.kv_sc,
                      k_fp4=d["k_idx"] if own else dw.k_idx, k_sc=d["k_sc"] if own else dw.k_sc,
                      kv_fmt=getattr(wl, "kv_fmt", 0))
        specs.append(sp)
        outs.append({"layer": d["index"], "out": out, "lse": lse, "idx": idx})
    layers = C.make_layers(specs)
    params = C.csa2_chain_params(wl.H, wl.Hm, wl.K, wl.block, wl.max_blocks, SCALE)
    pb = torch.empty((nq, wl.max_blocks), dtype=torch.int32, device=device) if pool else None
    pp = torch.empty((nq, wl.max_blocks * wl.block), dtype=torch.int32, device=device) if pool else None
    pc = torch.empty((nq,), dtype=torch.int32, device=device) if pool else None
    if ws is None:
        ws = C.workspace(C.csa2_workspace_size(C.CSA2_WS_LAYER_CHAIN, dw.batch, wl.K, wl.max_blocks, len(specs)),
                         device)

    def call():
        C.csa2_layer_chain(dw.batch, params, layers, dw.swa, pb, pp, pc, ws)

    call.keep = (specs, layers, params, ws)
    return call, outs, (pb, pp, pc)


def run_chain(dw, want_idx=True, want_lse=True, ws=None, pool=True):
    call, outs, pools = prepare_chain(dw, want_idx, want_lse, ws, pool)
    call()
    return outs, pools, call.keep


def assert_close_attn(got, ref, what=""):
    """Attention tolerance: |gpu - ref| <= 2e-3 + 1e-2 |ref| elementwise."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(got - ref)
    bad = err > 2e-3 + 1e-2 * np.abs(ref)
    assert not bad.any(), f"{what}: {bad.sum()} elements out of tolerance; max abs {err.max():.3e}"
    return float(err.max())


@contextlib.contextmanager
def saved_on_failure(wl, tag):
    """With CSA2_SAVE_FAILED set to a directory, a failure inside the block
    writes wl's inputs there (synth.replay format, one folder per tag) before
    the failure propagates; tests/replay_case.py runs them again."""
    try:
        yield
    except BaseException:
        root = os.environ.get("CSA2_SAVE_FAILED")
        if root:
            from synth.replay import save_workload
            save_workload(wl, os.path.join(root, re.sub(r"[^A-Za-z0-9_.-]+", "_", tag)), note=f"failed: {tag}")
        raise
