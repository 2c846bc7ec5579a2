"""CPU oracle for the CSA2 hot path (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline leg
may import this package.  The product path (``compressed_sparse_attention_amd``)
never does, and the two share no code.  The arithmetic lives in csa2_oracle.c;
this file marshals numpy arrays and composes the per-layer steps into the
layer chain.

Sources: the report "DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache
Compression" (sections 2.3, 2.3.1, 2.3.2, 4.2.1) and the reading note "DeepSeek
V4.1 Flash: Pushing the Limits of KV Cache Compression" (mode table, decoder
schedule table, decoder search-range / read-range table).
"""
from __future__ import annotations

import copy
import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# CSA2_ORACLE_SO: a library built from a modified copy of the source (the
# mutation test of the pins loads planted mistakes through it)
_SO = os.environ.get("CSA2_ORACLE_SO") or os.path.join(_HERE, "libcsa2_oracle.so")
_SRC = os.path.join(_HERE, "csa2_oracle.c")

MODE_SWA_ONLY, MODE_FULL, MODE_REINDEX, MODE_REUSE = 0, 1, 2, 3
Q_FP4, Q_FP8 = 0, 1

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-pthread", "-shared", "-fPIC"]


def build(force: bool = False) -> str:
    if os.environ.get("CSA2_ORACLE_SO"):
        return _SO
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", _SO, "-lm"])
    return _SO


_lib = None
NTHREADS = int(os.environ.get("CSA2_ORACLE_THREADS", "0")) or (os.cpu_count() or 8)


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_SO)
        vp, i64, i32, d = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
        L.orc_e2m1.argtypes = [ctypes.c_uint8]
        L.orc_e2m1.restype = d
        L.orc_e8m0.argtypes = [ctypes.c_uint8]
        L.orc_e8m0.restype = d
        L.orc_e4m3.argtypes = [ctypes.c_uint8]
        L.orc_e4m3.restype = d
        L.orc_bf16.argtypes = [ctypes.c_uint16]
        L.orc_bf16.restype = ctypes.c_float
        L.orc_visible.argtypes = [i64, i64, i32]
        L.orc_visible.restype = i64
        L.orc_index_score.argtypes = [i64, vp, vp, vp, i32, i32, i32, vp, vp, vp, vp, vp, vp, i64, i64, vp, i64, i32]
        L.orc_index_score.restype = i32
        L.orc_kv_append.argtypes = [i64, vp, vp, vp, i32, i64, vp, vp]
        L.orc_kv_append.restype = i32
        L.orc_compress.argtypes = [i64, i32, vp, vp, vp]
        L.orc_compress.restype = i32
        L.orc_rope_cast.argtypes = [i64, i32, vp, vp, i32, vp]
        L.orc_rope_cast.restype = i32
        L.orc_index_k_project.argtypes = [i64, vp, vp, vp, vp, i32, i64, vp, vp, vp]
        L.orc_index_k_project.restype = i32
        L.orc_topk.argtypes = [i64, vp, i64, vp, vp, i64, i32, vp, i32]
        L.orc_block_pool.argtypes = [i64, vp, i64, vp, i32, i32, vp, vp, vp, i32]
        L.orc_gather_dequant.argtypes = [i64, vp, vp, vp, vp, i32, vp, i32, vp]
        L.orc_sparse_attn.argtypes = [i64, vp, vp, vp, vp, i32, vp, vp, i32, vp, i32, vp, i32, vp, vp, i32, vp, d, vp,
                                      vp, i32]
        _lib = L
    return _lib


def _p(a):
    if a is None:
        return None
    assert isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous numpy arrays"
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


# --- formats ----------------------------------------------------------------

def e2m1(code):
    return lib().orc_e2m1(code)


def e8m0(code):
    return lib().orc_e8m0(code)


def e4m3(code):
    return lib().orc_e4m3(code)


def bf16(bits):
    return lib().orc_bf16(bits)


def visible(n_entries, t, ratio):
    return lib().orc_visible(int(n_entries), int(t), int(ratio))


def row_visible(wl):
    """vis(t) for every query row of a workload."""
    return np.array([visible(wl.n_entries[b], t, wl.ratio) for b, t in zip(wl.row_seq, wl.q_pos)], np.int64)


# --- steps ------------------------------------------------------------------

def index_k_project(x, W, dst, k_fmt, rows, want_y=False, cs=None):
    """Indexer K from main-KV entries: y = x W (fp32 multiply-add chain over
    the 512 channels, ascending), then E2M1 with one E8M0 per row (k_fmt 0)
    or per 32 channels (k_fmt 1), into rows dst of a [rows][64] cache.  x is
    the entry after RoPE, or before it when its angles cs [n][32][2] are
    given (then turned first, as kv_append turns it)."""
    x, W, dst = _c(x, np.float32), _c(W, np.float32), _c(dst, np.int64)
    cs = None if cs is None else _c(cs, np.float32)
    k_fp4 = np.zeros((rows, 64), np.uint8)
    k_sc = np.zeros((rows, 4) if k_fmt == 1 else (rows,), np.uint8)
    y = np.zeros((len(dst), 128), np.float32) if want_y else None
    if lib().orc_index_k_project(len(dst), _p(x), _p(cs), _p(W), _p(dst), k_fmt, rows, _p(k_fp4), _p(k_sc), _p(y)):
        raise ValueError("index_k_project: bad format or destination row")
    return (k_fp4, k_sc, y) if want_y else (k_fp4, k_sc)


def rope_cast(x, cs, inverse):
    """Rotate channels 448..511 of every head row of x [n][heads][512] f32 by
    the row's angles cs [n][32][2] (negated with `inverse`), then cast all to
    bf16 (nearest even); returns the bf16 bits [n][heads][512] u16."""
    x, cs = _c(x, np.float32), _c(cs, np.float32)
    out = np.empty(x.shape, np.uint16)
    if lib().orc_rope_cast(x.shape[0], x.shape[1], _p(x), _p(cs), int(inverse), _p(out)):
        raise ValueError("rope_cast: bad arguments")
    return out


def compress(c_tok, z_tok, m):
    """Compressor: entry j = per-channel softmax over its m tokens of Z,
    weighting C (tokens jm .. jm + m - 1).  c_tok, z_tok [n m][512] f32."""
    c_tok = _c(c_tok, np.float32)
    z_tok = _c(z_tok, np.float32)
    n = c_tok.shape[0] // m
    out = np.empty((n, 512), np.float32)
    if lib().orc_compress(n, m, _p(c_tok), _p(z_tok), _p(out)):
        raise ValueError("compress: bad arguments")
    return out


def kv_append(x, cs, dst, kv_fmt, rows, kv_fp4=None, kv_sc=None):
    """Cache append: RoPE on the last 64 latent channels, then quantise all 512
    (report 2.4.4) into rows dst of a main-KV cache of `rows` rows.  x [n][512]
    f32, cs [n][32][2] f32 (cos, sin per pair), dst [n] i64.  Returns the
    cache arrays (fresh zeroed ones unless given)."""
    x = _c(x, np.float32)
    cs = _c(cs, np.float32)
    dst = _c(dst, np.int64)
    if kv_fp4 is None:
        kv_fp4 = np.zeros((rows, 256), np.uint8)
    if kv_sc is None:
        kv_sc = np.zeros((rows, 32 if kv_fmt == 1 else 16), np.uint8)
    rc = lib().orc_kv_append(len(dst), _p(x), _p(cs), _p(dst), kv_fmt, rows, _p(kv_fp4), _p(kv_sc))
    if rc:
        raise ValueError("kv_append: bad format or destination row")
    return kv_fp4, kv_sc


def index_score(wl, q_idx, q_sc, w, q_fmt, cand=None, n_slots=None, rows=None):
    """Scores [rows][slots] f32.  Full mode (cand None): slots = max N_b;
    Reindex mode: slot s of row r is position cand[r][s]."""
    row_seq, q_pos = wl.row_seq, wl.q_pos
    if rows is not None:  # a subset of query rows (large workloads)
        rows = np.asarray(rows, np.int64)
        row_seq, q_pos = row_seq[rows], q_pos[rows]
        q_idx, q_sc, w = q_idx[rows], q_sc[rows], w[rows]
        if cand is not None:
            cand = cand[rows]
    nr = len(q_pos)
    if cand is None:
        stride = int(wl.n_entries.max())
        ns = stride
        cstride = 0
    else:
        cand = _c(cand, np.int32)
        stride = cand.shape[1]
        ns = stride if n_slots is None else n_slots
        cstride = cand.shape[1]
    out = np.full((nr, stride), -np.inf, np.float32)
    rc = lib().orc_index_score(nr, _p(_c(row_seq, np.int32)), _p(_c(q_pos, np.int32)), _p(_c(wl.entry_off, np.int64)),
                               wl.ratio, q_sc.shape[1], q_fmt, _p(_c(q_idx, np.uint8)), _p(_c(q_sc, np.uint8)),
                               _p(_c(w, np.float32)), _p(wl.k_idx), _p(wl.k_sc), _p(cand), cstride, ns, _p(out),
                               stride, NTHREADS)
    if rc != 0:
        raise ValueError("index score: a dot product left the exactly representable range")
    return out


def topk(scores, n_valid, K, cand=None):
    scores = _c(scores, np.float32)
    nr = scores.shape[0]
    idx = np.empty((nr, K), np.int32)
    cand_c = None if cand is None else _c(cand, np.int32)
    lib().orc_topk(nr, _p(scores), scores.shape[1], _p(_c(n_valid, np.int64)), _p(cand_c),
                   0 if cand is None else cand_c.shape[1], K, _p(idx), NTHREADS)
    return idx


def block_pool(scores, vis, block=8, max_blocks=2048):
    scores = _c(scores, np.float32)
    nr = scores.shape[0]
    blocks = np.empty((nr, max_blocks), np.int32)
    pool = np.empty((nr, max_blocks * block), np.int32)
    cnt = np.empty(nr, np.int32)
    lib().orc_block_pool(nr, _p(scores), scores.shape[1], _p(_c(vis, np.int64)), block, max_blocks, _p(blocks),
                         _p(pool), _p(cnt), NTHREADS)
    return blocks, pool, cnt


def gather_dequant(wl, idx):
    idx = _c(idx, np.int32)
    nr, K = idx.shape
    out = np.empty((nr, K, 512), np.uint16)
    lib().orc_gather_dequant(nr, _p(_c(wl.row_seq, np.int32)), _p(wl.entry_off), _p(wl.kv), _p(wl.kv_sc),
                             getattr(wl, "kv_fmt", 0), _p(idx), K, _p(out))
    return out


def sparse_attn(wl, q_main, idx, swa, replay_s=None, rows=None, scale=None, with_lse=True, idx_of_rows=False):
    """rows: a subset of query rows; idx then holds either every row's indices
    (selected here) or, with idx_of_rows, only the subset's."""
    row_seq, q_pos = wl.row_seq, wl.q_pos
    if rows is not None:
        rows = np.asarray(rows, np.int64)
        row_seq, q_pos, q_main = row_seq[rows], q_pos[rows], q_main[rows]
        if not idx_of_rows:
            idx = idx[rows]
    q_main = _c(q_main, np.uint16)
    idx = _c(idx, np.int32)
    nr, Hm, _ = q_main.shape
    out = np.empty((nr, Hm, 512), np.float32)
    lse = np.empty((nr, Hm), np.float32) if with_lse else None
    sc = 1.0 / math.sqrt(512.0) if scale is None else scale
    lib().orc_sparse_attn(nr, _p(_c(row_seq, np.int32)), _p(_c(q_pos, np.int32)), _p(wl.entry_off), _p(q_main), Hm,
                          _p(wl.kv), _p(wl.kv_sc), getattr(wl, "kv_fmt", 0), _p(idx), idx.shape[1],
                          _p(_c(swa, np.uint8 if getattr(wl, "swa_fmt", 0) == 1 else np.uint16)), getattr(wl, "swa_fmt", 0),
                          _p(_c(wl.swa_row_off, np.int64)), _p(_c(wl.swa_pos0, np.int32)), wl.W,
                          _p(None if replay_s is None else _c(replay_s, np.int32)), sc, _p(out), _p(lse), NTHREADS)
    return out, lse


# --- layer chain --------------------------------------------------------------

def _with_source(wl, L):
    """The workload as the layers after Full layer L read it: main KV and
    indexer K are L's own when it carries them ([R] 2.3.1: a Full layer
    generates global KV; Reindex and Reuse layers read the preceding Full
    layer's)."""
    if L.kv is None:
        return wl
    v = copy.copy(wl)
    v.k_idx, v.k_sc, v.kv, v.kv_sc = L.k_idx, L.k_sc, L.kv, L.kv_sc
    return v


def layer_chain(wl, rows=None, attn=True):
    """Run the layers in index order ([R] 2.3.1 modes; [N4] schedule table).

    FULL    scores every visible entry with its own indexer q, takes Top-K and,
            when it is the layer flagged to build the pool (the first decoder Full
            layer, [R] 2.3.2), the block pool from the same scores.
    REINDEX scores only the pool positions (all visible positions when no pool
            exists) against the shared indexer K with its own q, takes Top-K.
    REUSE   attends with the latest indices.
    SWA_ONLY attends to its window only.
    Main KV and indexer K come from the latest Full layer (its own caches when
    it carries them, else the workload's).
    Returns per-layer dicts with idx (and pool fields for the pool layer) and
    the attention output."""
    nr_all = wl.total_q
    sel_rows = np.arange(nr_all) if rows is None else np.asarray(rows, np.int64)
    vis = row_visible(wl)[sel_rows]
    idx_cur = None
    pool = None
    results = []
    src = wl  # the workload as seen through the latest Full layer's caches
    for L in wl.layers:
        res = {"layer": L.index, "mode": L.mode}
        if L.mode == MODE_FULL:
            src = _with_source(wl, L)
            pool = None
            sc = index_score(src, L.q_idx, L.q_sc, L.w, L.q_fmt, rows=sel_rows)
            idx_cur = topk(sc, vis, wl.K)
            if L.build_pool:
                blocks, pool_pos, cnt = block_pool(sc, vis, wl.block, wl.max_blocks)
                pool = (blocks, pool_pos, cnt)
                res["blocks"], res["pool_pos"], res["pool_count"] = blocks, pool_pos, cnt
            res["scores"] = sc
        elif L.mode == MODE_REINDEX:
            if pool is not None:
                pool_pos, cnt = pool[1], pool[2]
                sc = _reindex_scores(src, L, sel_rows, pool_pos)
                idx_cur = topk(sc, cnt.astype(np.int64), wl.K, cand=pool_pos)
            else:
                sc = index_score(src, L.q_idx, L.q_sc, L.w, L.q_fmt, rows=sel_rows)
                idx_cur = topk(sc, vis, wl.K)
            res["scores"] = sc
        elif L.mode == MODE_SWA_ONLY:
            idx_cur_layer = np.full((len(sel_rows), wl.K), -1, np.int32)
        if L.mode == MODE_SWA_ONLY:
            use_idx = idx_cur_layer
        else:
            if idx_cur is None:
                raise ValueError("a Reuse layer needs an earlier Full or Reindex layer")
            use_idx = idx_cur
        res["idx"] = use_idx
        if attn:
            res["out"], res["lse"] = sparse_attn(src, L.q_main, use_idx, L.swa, replay_s=getattr(wl, "replay_s", None),
                                                 rows=sel_rows, idx_of_rows=True)
        results.append(res)
    return results


def _reindex_scores(wl, L, sel_rows, pool_pos):
    """Reindex scoring over the pool: a subset of rows is handled by building
    a row-restricted view of the workload's query-side arrays."""
    row_seq = wl.row_seq[sel_rows]
    q_pos = wl.q_pos[sel_rows]
    nr = len(sel_rows)
    stride = pool_pos.shape[1]
    out = np.full((nr, stride), -np.inf, np.float32)
    rc = lib().orc_index_score(nr, _p(_c(row_seq, np.int32)), _p(_c(q_pos, np.int32)), _p(wl.entry_off), wl.ratio,
                               L.q_sc.shape[1], L.q_fmt, _p(_c(L.q_idx[sel_rows], np.uint8)),
                               _p(_c(L.q_sc[sel_rows], np.uint8)), _p(_c(L.w[sel_rows], np.float32)), _p(wl.k_idx),
                               _p(wl.k_sc), _p(_c(pool_pos, np.int32)), stride, stride, _p(out), stride, NTHREADS)
    if rc != 0:
        raise ValueError("index score: a dot product left the exactly representable range")
    return out
