"""Host-only checks of the C ABI: the library loads without a GPU, exports every
function include/csa2.h declares, and rejects bad arguments with the documented
status codes before any device work (device pointers here are dummies that the
library never dereferences on the host)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

from compressed_sparse_attention_amd import csa2 as C

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa2.h")

FAKE = 0x7F0000000000  # a device address the host never touches


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"CSA2_API\s+[\w\s\*]+?\b(csa2_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = C.lib()
    names = declared_functions()
    assert set(names) == set(C.EXPORTS)
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", C.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (csa2_\w+)", out))
    assert exported == set(names)  # nothing else leaks out of the library


def test_status_strings_and_version():
    L = C.lib()
    assert L.csa2_version() >= 1
    for s in range(6):
        assert L.csa2_status_string(s) != b"unknown status"
    assert L.csa2_status_string(99) == b"unknown status"


class HostBatch:
    """A csa2_batch whose device arrays are dummy addresses."""

    def __init__(self, n_entries, q_pos, ratio=1):
        n_entries = np.asarray(n_entries, np.int64)
        self.entry_off = np.zeros(len(n_entries) + 1, np.int64)
        self.entry_off[1:] = np.cumsum(n_entries)
        self.q_pos = np.ascontiguousarray(np.concatenate([np.asarray(p, np.int32) for p in q_pos]), np.int32)
        self.q_off = np.zeros(len(n_entries) + 1, np.int32)
        self.q_off[1:] = np.cumsum([len(p) for p in q_pos])
        self.c = C.csa2_batch(len(n_entries), len(self.q_pos), ratio, 0, self.entry_off.ctypes.data,
                              self.q_off.ctypes.data, self.q_pos.ctypes.data, FAKE, FAKE, FAKE, FAKE)


def _score(b, **kw):
    args = dict(H=64, q_fmt=0, q=FAKE, q_sc=FAKE, w=FAKE, k=FAKE, k_sc=FAKE, cand=None, cstride=0, scores=FAKE,
                stride=1000, hist=None, stream=None)
    args.update(kw)
    return C.lib().csa2_index_score(ctypes.byref(b.c), args["H"], args["q_fmt"], args["q"], args["q_sc"], args["w"],
                                    args["k"], args["k_sc"], args["cand"], args["cstride"], args["scores"],
                                    args["stride"], args["hist"], args["stream"])


def test_index_score_validation():
    b = HostBatch([1000, 500], [[999], [499]])
    assert _score(b, H=48) == C.CSA2_ERR_UNSUPPORTED
    assert _score(b, q_fmt=7) == C.CSA2_ERR_INVALID_ARG
    assert _score(b, q=None) == C.CSA2_ERR_INVALID_ARG
    assert _score(b, stride=999) == C.CSA2_ERR_INVALID_ARG            # score_stride < max N_b
    assert _score(b, cand=FAKE, cstride=0) == C.CSA2_ERR_INVALID_ARG
    assert _score(b, cand=FAKE, cstride=64, stride=32) == C.CSA2_ERR_INVALID_ARG
    assert _score(b, cand=FAKE, cstride=64, stride=64, q_fmt=1) == C.CSA2_ERR_UNSUPPORTED
    assert _score(b, q_fmt=1, hist=FAKE) == C.CSA2_ERR_UNSUPPORTED   # no fused histogram for E4M3 queries
    assert _score(b, q_fmt=3) == C.CSA2_ERR_INVALID_ARG
    many = HostBatch([1000], [list(range(990, 1000))])
    assert _score(many, hist=FAKE) == C.CSA2_ERR_UNSUPPORTED         # nor for the many-query scan


def test_batch_validation():
    b = HostBatch([10], [[5]])
    b.c.total_q = 2  # q_off[n_seq] != total_q
    assert _score(b) == C.CSA2_ERR_INVALID_ARG
    b = HostBatch([10], [[-1]])
    assert _score(b) == C.CSA2_ERR_INVALID_ARG
    b = HostBatch([10], [[5]])
    b.entry_off[0] = 1
    assert _score(b) == C.CSA2_ERR_INVALID_ARG
    b = HostBatch([10], [[5]], ratio=0)
    assert _score(b) == C.CSA2_ERR_INVALID_ARG
    b = HostBatch([10], [[5]])
    b.c.d_row_seq = None
    assert _score(b) == C.CSA2_ERR_INVALID_ARG
    b = HostBatch([1 << 31], [[5]])
    assert _score(b, stride=1 << 31) == C.CSA2_ERR_UNSUPPORTED


def test_topk_validation():
    L = C.lib()
    b = HostBatch([1000], [[999]])
    need = L.csa2_workspace_size(C.CSA2_WS_TOPK, ctypes.byref(b.c), 512, 2048, 1)
    assert need > 0
    topk = lambda K, ws, n, stride=1000, cand=None, cnt=None, cs=0: L.csa2_topk(
        ctypes.byref(b.c), FAKE, stride, cand, cs, cnt, K, None, FAKE, ws, n, None)
    assert topk(0, FAKE, need) == C.CSA2_ERR_INVALID_ARG
    assert topk(4096, FAKE, need) == C.CSA2_ERR_UNSUPPORTED
    assert topk(512, None, 0) == C.CSA2_ERR_WORKSPACE
    assert topk(512, FAKE, need - 1) == C.CSA2_ERR_WORKSPACE
    assert topk(512, FAKE + 8, need) == C.CSA2_ERR_WORKSPACE        # misaligned
    assert topk(512, FAKE, need, stride=10) == C.CSA2_ERR_INVALID_ARG
    assert topk(512, FAKE, need, cand=FAKE, cs=64, stride=64) == C.CSA2_ERR_INVALID_ARG  # no cand_count


def test_block_pool_validation():
    L = C.lib()
    b = HostBatch([1000], [[999]])
    need = L.csa2_workspace_size(C.CSA2_WS_BLOCK_POOL, ctypes.byref(b.c), 512, 2048, 1)
    pool = lambda block, mb, ws=FAKE, n=need: L.csa2_block_pool(ctypes.byref(b.c), FAKE, 1000, block, mb, FAKE, FAKE,
                                                                 FAKE, ws, n, None)
    assert pool(16, 2048) == C.CSA2_ERR_UNSUPPORTED
    assert pool(0, 2048) == C.CSA2_ERR_INVALID_ARG
    assert pool(8, 0) == C.CSA2_ERR_INVALID_ARG
    assert pool(8, 4096) == C.CSA2_ERR_UNSUPPORTED
    assert pool(8, 2048, None, 0) == C.CSA2_ERR_WORKSPACE


def _swa(window, row_off, pos0, length, replay=None):
    arrs = [np.ascontiguousarray(row_off, np.int64), np.ascontiguousarray(pos0, np.int32),
            np.ascontiguousarray(length, np.int32)]
    rep = None if replay is None else np.ascontiguousarray(replay, np.int32)
    s = C.csa2_swa_layout(window, 0, arrs[0].ctypes.data, arrs[1].ctypes.data, arrs[2].ctypes.data,
                          None if rep is None else rep.ctypes.data, FAKE, FAKE, None if rep is None else FAKE)
    s._keep = (arrs, rep)
    return s


def test_sparse_attn_validation():
    L = C.lib()
    b = HostBatch([1000], [[999]])
    attn = lambda Hm=64, K=512, sw=None, scale=0.04, kv_fmt=0: L.csa2_sparse_attn(
        ctypes.byref(b.c), Hm, FAKE, kv_fmt, FAKE, FAKE, FAKE, K, FAKE, ctypes.byref(sw), scale, FAKE, None, None, 0,
        None)
    ok = _swa(128, [0], [872], [128])
    assert attn(kv_fmt=2, sw=ok) == C.CSA2_ERR_UNSUPPORTED  # main-KV scales: E8M0/32 or E4M3/16 only
    bad_fmt = _swa(128, [0], [872], [128])
    bad_fmt.fmt = 2
    assert attn(sw=bad_fmt) == C.CSA2_ERR_UNSUPPORTED  # SWA rows: bf16 or MXFP8 only
    assert attn(Hm=40, sw=ok) == C.CSA2_ERR_UNSUPPORTED
    assert attn(K=0, sw=ok) == C.CSA2_ERR_INVALID_ARG
    assert attn(scale=0.0, sw=ok) == C.CSA2_ERR_INVALID_ARG
    assert attn(scale=float("nan"), sw=ok) == C.CSA2_ERR_INVALID_ARG
    assert attn(sw=_swa(128, [0], [873], [127])) == C.CSA2_ERR_INVALID_ARG   # window starts before the rows
    assert attn(sw=_swa(128, [0], [872], [127])) == C.CSA2_ERR_INVALID_ARG   # row of t missing
    assert attn(sw=_swa(2048, [0], [0], [1000])) == C.CSA2_ERR_UNSUPPORTED
    # a replay start inside the window shortens it: rows from 950 suffice
    assert attn(sw=_swa(128, [0], [951], [49], replay=[950])) == C.CSA2_ERR_INVALID_ARG
    assert attn(sw=_swa(128, [0], [950], [50], replay=None)) == C.CSA2_ERR_INVALID_ARG


def test_layer_chain_schedule_validation():
    L = C.lib()
    b = HostBatch([1000], [[999]])
    sw = _swa(128, [0], [872], [128])
    need = L.csa2_workspace_size(C.CSA2_WS_LAYER_CHAIN, ctypes.byref(b.c), 512, 2048, 2)
    p = C.csa2_chain_params(64, 64, 512, 8, 2048, 0.044)
    base = dict(q_main=FAKE, swa=FAKE, out=FAKE)
    full = dict(mode=C.CSA2_MODE_FULL, q_idx=FAKE, q_sc=FAKE, w=FAKE, kv_fp4=FAKE, kv_sc=FAKE, k_fp4=FAKE, k_sc=FAKE,
                **base)

    def run(specs, ws=FAKE, n=need, params=p):
        arr = (C.csa2_layer * len(specs))()
        for i, sp in enumerate(specs):
            for k, v in sp.items():
                setattr(arr[i], k, v)
        return L.csa2_layer_chain(ctypes.byref(b.c), ctypes.byref(params), len(specs), arr, ctypes.byref(sw), None,
                                  None, None, ws, n, None)

    assert run([dict(mode=C.CSA2_MODE_REUSE, **base)]) == C.CSA2_ERR_INVALID_ARG        # Reuse before any indices
    assert run([dict(mode=C.CSA2_MODE_REINDEX, q_idx=FAKE, q_sc=FAKE, w=FAKE, **base)]) == C.CSA2_ERR_INVALID_ARG
    assert run([dict(full, flags=1), dict(full, flags=1)]) == C.CSA2_ERR_INVALID_ARG     # two pool builders
    assert run([dict(mode=9, **base)]) == C.CSA2_ERR_INVALID_ARG
    assert run([full], ws=None, n=0) == C.CSA2_ERR_WORKSPACE
    assert run([dict(full, q_main=None)]) == C.CSA2_ERR_INVALID_ARG
    assert run([full], params=C.csa2_chain_params(64, 64, 512, 16, 2048, 0.044)) == C.CSA2_ERR_UNSUPPORTED
    # a Reindex layer reads its source's indexer K, whose scale layout follows
    # the source's format: MXFP4 queries exactly when the source has them
    rx = dict(mode=C.CSA2_MODE_REINDEX, q_idx=FAKE, q_sc=FAKE, w=FAKE, **base)
    mx = C.CSA2_Q_MXFP4
    assert run([dict(full, q_fmt=mx), dict(rx, q_fmt=C.CSA2_Q_FP4)]) == C.CSA2_ERR_INVALID_ARG
    assert run([full, dict(rx, q_fmt=mx)]) == C.CSA2_ERR_INVALID_ARG
    assert run([full, dict(rx, q_fmt=C.CSA2_Q_FP8)]) == C.CSA2_ERR_UNSUPPORTED
    assert run([dict(full, q_fmt=3)]) == C.CSA2_ERR_INVALID_ARG


def test_kv_append_validation():
    L = C.lib()

    def app(n=4, x=FAKE, cs=FAKE, dst=FAKE, rows=8, fmt=1, kv=FAKE, sc=FAKE):
        return L.csa2_kv_append(n, x, cs, dst, rows, fmt, kv, sc, None)

    assert app(n=-1) == C.CSA2_ERR_INVALID_ARG
    assert app(fmt=2) == C.CSA2_ERR_UNSUPPORTED
    assert app(n=0, x=None) == C.CSA2_OK          # nothing to do, nothing launched
    assert app(x=None) == C.CSA2_ERR_INVALID_ARG
    assert app(dst=None) == C.CSA2_ERR_INVALID_ARG
    assert app(rows=0) == C.CSA2_ERR_INVALID_ARG
    assert app(x=FAKE + 4) == C.CSA2_ERR_INVALID_ARG   # x must be 16-byte aligned


def test_compress_validation():
    L = C.lib()

    def comp(n=4, m=2, c=FAKE, z=FAKE, out=FAKE):
        return L.csa2_compress(n, m, c, z, out, None)

    assert comp(n=-1) == C.CSA2_ERR_INVALID_ARG
    assert comp(m=0) == C.CSA2_ERR_UNSUPPORTED
    assert comp(m=17) == C.CSA2_ERR_UNSUPPORTED
    assert comp(n=0, c=None) == C.CSA2_OK
    assert comp(z=None) == C.CSA2_ERR_INVALID_ARG
    assert comp(out=FAKE + 8) == C.CSA2_ERR_INVALID_ARG


def test_index_k_project_validation():
    L = C.lib()

    def proj(n=4, x=FAKE, cs=None, W=FAKE, dst=FAKE, rows=8, fmt=C.CSA2_Q_MXFP4, kf=FAKE, ks=FAKE):
        return L.csa2_index_k_project(n, x, cs, W, dst, rows, fmt, kf, ks, None)

    assert proj(n=-1) == C.CSA2_ERR_INVALID_ARG
    assert proj(fmt=5) == C.CSA2_ERR_INVALID_ARG
    assert proj(n=0, x=None) == C.CSA2_OK
    assert proj(W=None) == C.CSA2_ERR_INVALID_ARG
    assert proj(rows=0) == C.CSA2_ERR_INVALID_ARG
    assert proj(W=FAKE + 4) == C.CSA2_ERR_INVALID_ARG
    assert proj(cs=FAKE + 8) == C.CSA2_ERR_INVALID_ARG


def test_rope_cast_validation():
    L = C.lib()

    def rc(n=4, h=64, x=FAKE, cs=FAKE, out=FAKE):
        return L.csa2_rope_cast(n, h, x, cs, 0, out, None)

    assert rc(n=-1) == C.CSA2_ERR_INVALID_ARG
    assert rc(h=0) == C.CSA2_ERR_INVALID_ARG
    assert rc(n=0, x=None) == C.CSA2_OK
    assert rc(cs=None) == C.CSA2_ERR_INVALID_ARG
    assert rc(out=FAKE + 2) == C.CSA2_ERR_INVALID_ARG


def test_topk_noalloc_validation():
    """The allocation-free Top-K validates like csa2_topk and refuses a batch
    whose workspace exceeds its static scratch (more than 256 query rows)
    before any device work."""
    L = C.lib()

    def call(b, scores=FAKE, stride=1000, K=512, idx=FAKE, cand=None, cstride=0, cnt=None):
        return L.csa2_topk_noalloc(ctypes.byref(b.c), scores, stride, cand, cstride, cnt, K, None, idx, None)

    b = HostBatch([1000, 500], [[999], [499]])
    assert call(b, scores=None) == C.CSA2_ERR_INVALID_ARG
    assert call(b, idx=None) == C.CSA2_ERR_INVALID_ARG
    assert call(b, K=0) == C.CSA2_ERR_INVALID_ARG
    assert call(b, K=4096) == C.CSA2_ERR_UNSUPPORTED
    assert call(b, stride=999) == C.CSA2_ERR_INVALID_ARG
    assert call(b, cand=FAKE, cstride=64, cnt=None) == C.CSA2_ERR_INVALID_ARG
    big = HostBatch([100000] * 257, [[99999]] * 257)
    assert call(big, stride=100000) == C.CSA2_ERR_SCRATCH
    assert L.csa2_status_string(C.CSA2_ERR_SCRATCH).startswith(b"the problem exceeds")


def test_sparse_attn_rope_validation():
    b = HostBatch([1000], [[999]])
    L = C.lib()
    row_off, pos0, ln = np.zeros(1, np.int64), np.array([872], np.int32), np.array([128], np.int32)
    sw = C.csa2_swa_layout(128, 0, row_off.ctypes.data, pos0.ctypes.data, ln.ctypes.data, None, FAKE, FAKE, None)

    def call(Hm=64, q=FAKE, cs=FAKE, kv_fmt=0, K=512, out=FAKE, scale=0.044):
        return L.csa2_sparse_attn_rope(ctypes.byref(b.c), Hm, q, cs, kv_fmt, FAKE, FAKE, FAKE, K, FAKE,
                                       ctypes.byref(sw), scale, out, None, None, 0, None)

    assert call(q=None) == C.CSA2_ERR_INVALID_ARG
    assert call(cs=None) == C.CSA2_ERR_INVALID_ARG
    assert call(out=None) == C.CSA2_ERR_INVALID_ARG
    assert call(q=FAKE + 4) == C.CSA2_ERR_INVALID_ARG      # query rows are read 16 bytes at a time
    assert call(out=FAKE + 2) == C.CSA2_ERR_INVALID_ARG    # bf16 pairs are stored 4 bytes at a time
    assert call(kv_fmt=5) == C.CSA2_ERR_UNSUPPORTED
    assert call(Hm=24) == C.CSA2_ERR_UNSUPPORTED
    assert call(K=0) == C.CSA2_ERR_INVALID_ARG
    assert call(scale=0.0) == C.CSA2_ERR_INVALID_ARG
