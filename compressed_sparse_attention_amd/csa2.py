"""Python binding of libcsa2.so (ctypes).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  Functions carry the C names; tensors are torch CUDA (HIP) tensors
owned by the caller, host descriptor arrays are numpy arrays.  A missing or
unloadable library raises ``RuntimeError`` on first use -- there is no other
implementation to fall back to.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcsa2.so")

CSA2_OK, CSA2_ERR_INVALID_ARG, CSA2_ERR_UNSUPPORTED, CSA2_ERR_WORKSPACE, CSA2_ERR_HIP = 0, 1, 2, 3, 4
CSA2_ERR_SCRATCH = 5
CSA2_Q_FP4, CSA2_Q_FP8, CSA2_Q_MXFP4 = 0, 1, 2
CSA2_KV_MXFP4, CSA2_KV_E4M3_16 = 0, 1
CSA2_MODE_SWA_ONLY, CSA2_MODE_FULL, CSA2_MODE_REINDEX, CSA2_MODE_REUSE = 0, 1, 2, 3
CSA2_LAYER_BUILD_POOL = 1
CSA2_WS_TOPK, CSA2_WS_BLOCK_POOL, CSA2_WS_SPARSE_ATTN, CSA2_WS_LAYER_CHAIN = 1, 2, 3, 4

EXPORTS = ("csa2_index_score", "csa2_topk", "csa2_topk_noalloc", "csa2_block_pool", "csa2_sparse_attn_rope", "csa2_gather_dequant", "csa2_sparse_attn",
           "csa2_layer_chain", "csa2_rope_cast", "csa2_index_k_project", "csa2_compress", "csa2_kv_append", "csa2_workspace_size", "csa2_status_string", "csa2_last_hip_error",
           "csa2_version")

_vp = ctypes.c_void_p


class csa2_batch(ctypes.Structure):
    _fields_ = [("n_seq", ctypes.c_int32), ("total_q", ctypes.c_int32), ("ratio", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("h_entry_off", _vp), ("h_q_off", _vp), ("h_q_pos", _vp),
                ("d_entry_off", _vp), ("d_q_off", _vp), ("d_q_pos", _vp), ("d_row_seq", _vp)]


class csa2_swa_layout(ctypes.Structure):
    _fields_ = [("window", ctypes.c_int32), ("fmt", ctypes.c_int32), ("h_row_off", _vp), ("h_pos0", _vp),
                ("h_len", _vp), ("h_replay_s", _vp), ("d_row_off", _vp), ("d_pos0", _vp), ("d_replay_s", _vp)]


class csa2_layer(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("flags", ctypes.c_int32), ("q_fmt", ctypes.c_int32),
                ("kv_fmt", ctypes.c_int32), ("q_idx", _vp), ("q_sc", _vp), ("w", _vp), ("kv_fp4", _vp),
                ("kv_sc", _vp), ("k_fp4", _vp), ("k_sc", _vp), ("q_main", _vp), ("swa", _vp), ("out", _vp),
                ("lse", _vp), ("idx_out", _vp)]


class csa2_chain_params(ctypes.Structure):
    _fields_ = [("H", ctypes.c_int32), ("Hm", ctypes.c_int32), ("K", ctypes.c_int32), ("block", ctypes.c_int32),
                ("max_blocks", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
                ("scan_begin", ctypes.c_void_p), ("scan_end", ctypes.c_void_p)]


class CSA2Error(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = _lib_handle.csa2_status_string(status).decode() if _lib_handle else str(status)
        extra = f" (hipError {_lib_handle.csa2_last_hip_error()})" if status == CSA2_ERR_HIP and _lib_handle else ""
        super().__init__(f"{where}: {msg}{extra}")


_lib_handle = None


def lib():
    """Load libcsa2.so (raises RuntimeError when it is missing)."""
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libcsa2.so not built ({LIB_PATH}); run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        i32, i64, f32, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
        B, S = ctypes.POINTER(csa2_batch), ctypes.POINTER(csa2_swa_layout)
        L.csa2_index_score.argtypes = [B, i32, i32, _vp, _vp, _vp, _vp, _vp, _vp, i32, _vp, i64, _vp, _vp]
        L.csa2_topk.argtypes = [B, _vp, i64, _vp, i32, _vp, i32, _vp, _vp, _vp, sz, _vp]
        L.csa2_topk_noalloc.argtypes = [B, _vp, i64, _vp, i32, _vp, i32, _vp, _vp, _vp]
        L.csa2_block_pool.argtypes = [B, _vp, i64, i32, i32, _vp, _vp, _vp, _vp, sz, _vp]
        L.csa2_gather_dequant.argtypes = [B, i32, _vp, _vp, _vp, i32, _vp, _vp]
        L.csa2_rope_cast.argtypes = [ctypes.c_int64, i32, _vp, _vp, i32, _vp, _vp]
        L.csa2_index_k_project.argtypes = [ctypes.c_int64, _vp, _vp, _vp, _vp, ctypes.c_int64, i32, _vp, _vp, _vp]
        L.csa2_compress.argtypes = [ctypes.c_int64, i32, _vp, _vp, _vp, _vp]
        L.csa2_kv_append.argtypes = [ctypes.c_int64, _vp, _vp, _vp, ctypes.c_int64, i32, _vp, _vp, _vp]
        L.csa2_sparse_attn.argtypes = [B, i32, _vp, i32, _vp, _vp, _vp, i32, _vp, S, f32, _vp, _vp, _vp, sz, _vp]
        L.csa2_sparse_attn_rope.argtypes = [B, i32, _vp, _vp, i32, _vp, _vp, _vp, i32, _vp, S, f32, _vp, _vp, _vp, sz,
                                            _vp]
        L.csa2_layer_chain.argtypes = [B, ctypes.POINTER(csa2_chain_params), i32, ctypes.POINTER(csa2_layer), S, _vp,
                                       _vp, _vp, _vp, sz, _vp]
        L.csa2_workspace_size.argtypes = [i32, B, i32, i32, i32]
        L.csa2_workspace_size.restype = sz
        L.csa2_status_string.argtypes = [i32]
        L.csa2_status_string.restype = ctypes.c_char_p
        L.csa2_last_hip_error.restype = i32
        L.csa2_version.restype = i32
        for name in ("csa2_index_score", "csa2_topk", "csa2_topk_noalloc", "csa2_block_pool", "csa2_gather_dequant",
                     "csa2_sparse_attn", "csa2_sparse_attn_rope", "csa2_layer_chain", "csa2_rope_cast", "csa2_index_k_project", "csa2_compress",
                     "csa2_kv_append"):
            getattr(L, name).restype = i32
        _lib_handle = L
    return _lib_handle


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        assert t.flags["C_CONTIGUOUS"]
        return t.ctypes.data
    assert t.is_contiguous(), "tensors passed to libcsa2 must be contiguous"
    return t.data_ptr()


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check(status, where):
    if status != CSA2_OK:
        raise CSA2Error(status, where)


class Batch:
    """A ragged batch: host arrays (numpy) plus device copies (torch)."""

    def __init__(self, n_entries, q_pos_per_seq, ratio=1, device="cuda"):
        n_entries = np.asarray(n_entries, np.int64)
        self.n_entries = n_entries
        self.entry_off = np.zeros(len(n_entries) + 1, np.int64)
        self.entry_off[1:] = np.cumsum(n_entries)
        self.q_pos = np.ascontiguousarray(np.concatenate([np.asarray(p, np.int64) for p in q_pos_per_seq]), np.int32)
        self.q_off = np.zeros(len(n_entries) + 1, np.int32)
        self.q_off[1:] = np.cumsum([len(p) for p in q_pos_per_seq])
        self.row_seq = np.repeat(np.arange(len(n_entries), dtype=np.int32), [len(p) for p in q_pos_per_seq])
        self.ratio = int(ratio)
        dev = torch.device(device)
        self.d_entry_off = torch.from_numpy(self.entry_off).to(dev)
        self.d_q_off = torch.from_numpy(self.q_off).to(dev)
        self.d_q_pos = torch.from_numpy(self.q_pos).to(dev)
        self.d_row_seq = torch.from_numpy(self.row_seq).to(dev)
        self.c = csa2_batch(len(n_entries), len(self.q_pos), self.ratio, 0, _ptr(self.entry_off), _ptr(self.q_off),
                            _ptr(self.q_pos), _ptr(self.d_entry_off), _ptr(self.d_q_off), _ptr(self.d_q_pos),
                            _ptr(self.d_row_seq))

    @classmethod
    def from_workload(cls, wl, device="cuda"):
        qp = [wl.q_pos[wl.q_off[b]:wl.q_off[b + 1]] for b in range(wl.n_seq)]
        return cls(wl.n_entries, qp, wl.ratio, device)

    @property
    def total_q(self):
        return len(self.q_pos)

    @property
    def max_entries(self):
        return int(self.n_entries.max())


class SwaLayout:
    def __init__(self, window, row_off, pos0, length, replay_s=None, device="cuda", fmt=0):
        dev = torch.device(device)
        self.h_row_off = np.ascontiguousarray(row_off, np.int64)
        self.h_pos0 = np.ascontiguousarray(pos0, np.int32)
        self.h_len = np.ascontiguousarray(length, np.int32)
        self.h_replay = None if replay_s is None else np.ascontiguousarray(replay_s, np.int32)
        self.d_row_off = torch.from_numpy(self.h_row_off).to(dev)
        self.d_pos0 = torch.from_numpy(self.h_pos0).to(dev)
        self.d_replay = None if replay_s is None else torch.from_numpy(self.h_replay).to(dev)
        self.c = csa2_swa_layout(int(window), int(fmt), _ptr(self.h_row_off), _ptr(self.h_pos0), _ptr(self.h_len),
                                 _ptr(self.h_replay), _ptr(self.d_row_off), _ptr(self.d_pos0), _ptr(self.d_replay))

    @classmethod
    def from_workload(cls, wl, replay_s=None, device="cuda"):
        return cls(wl.W, wl.swa_row_off, wl.swa_pos0, wl.swa_len, replay_s, device, getattr(wl, "swa_fmt", 0))


HIST_BINS = 4096


def hist_buffer(batch, device="cuda"):
    """A zeroed [total_q][4096] histogram buffer for csa2_index_score / csa2_topk."""
    return torch.zeros((batch.total_q, HIST_BINS), dtype=torch.int32, device=device)


def workspace(nbytes, device="cuda"):
    """A 256-byte aligned workspace tensor (torch's allocator aligns to 512 B)."""
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def csa2_workspace_size(which, batch, K=512, max_blocks=2048, n_layers=1):
    return int(lib().csa2_workspace_size(which, ctypes.byref(batch.c), K, max_blocks, n_layers))


def csa2_index_score(batch, H, q_fmt, q, q_sc, w, k_fp4, k_sc, cand=None, scores=None, hist=None, stream=None):
    if cand is None:
        stride = batch.max_entries
        cstride = 0
    else:
        stride = cand.shape[1]
        cstride = cand.shape[1]
    if scores is None:
        scores = torch.empty((batch.total_q, max(stride, 1)), dtype=torch.float32, device=q.device)
    st = lib().csa2_index_score(ctypes.byref(batch.c), H, q_fmt, _ptr(q), _ptr(q_sc), _ptr(w), _ptr(k_fp4),
                                _ptr(k_sc), _ptr(cand), cstride, _ptr(scores), scores.shape[1], _ptr(hist),
                                _stream(stream))
    _check(st, "csa2_index_score")
    return scores


def csa2_topk(batch, scores, K, cand=None, cand_count=None, hist=None, idx=None, ws=None, stream=None):
    if idx is None:
        idx = torch.empty((batch.total_q, K), dtype=torch.int32, device=scores.device)
    if ws is None:
        ws = workspace(csa2_workspace_size(CSA2_WS_TOPK, batch, K), scores.device)
    st = lib().csa2_topk(ctypes.byref(batch.c), _ptr(scores), scores.shape[1], _ptr(cand),
                         0 if cand is None else cand.shape[1], _ptr(cand_count), K, _ptr(hist), _ptr(idx), _ptr(ws),
                         ws.numel(), _stream(stream))
    _check(st, "csa2_topk")
    return idx


def csa2_topk_noalloc(batch, scores, K, idx, cand=None, cand_count=None, hist=None, stream=None):
    """csa2_topk with its workspace in the library's static scratch (no
    allocation by the library; the caller passes the output idx)."""
    st = lib().csa2_topk_noalloc(ctypes.byref(batch.c), _ptr(scores), scores.shape[1], _ptr(cand),
                                 0 if cand is None else cand.shape[1], _ptr(cand_count), K, _ptr(hist), _ptr(idx),
                                 _stream(stream))
    _check(st, "csa2_topk_noalloc")
    return idx


def csa2_block_pool(batch, scores, block=8, max_blocks=2048, ws=None, stream=None):
    dev = scores.device
    blocks = torch.empty((batch.total_q, max_blocks), dtype=torch.int32, device=dev)
    pool = torch.empty((batch.total_q, max_blocks * block), dtype=torch.int32, device=dev)
    cnt = torch.empty((batch.total_q,), dtype=torch.int32, device=dev)
    if ws is None:
        ws = workspace(csa2_workspace_size(CSA2_WS_BLOCK_POOL, batch, 512, max_blocks), dev)
    st = lib().csa2_block_pool(ctypes.byref(batch.c), _ptr(scores), scores.shape[1], block, max_blocks, _ptr(blocks),
                               _ptr(pool), _ptr(cnt), _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "csa2_block_pool")
    return blocks, pool, cnt


def csa2_rope_cast(x, rope_cs, inverse=False, out=None, stream=None):
    """Rotate channels 448..511 of every head row of x [n][heads][512] f32 by
    the row's angles (negated with inverse) and cast to bf16 (u16 bits)."""
    n, heads = int(x.shape[0]), int(x.shape[1])
    if out is None:
        out = torch.empty(x.shape, dtype=torch.uint16, device=x.device)
    st = lib().csa2_rope_cast(n, heads, _ptr(x), _ptr(rope_cs), int(bool(inverse)), _ptr(out), _stream(stream))
    _check(st, "csa2_rope_cast")
    return out


def csa2_index_k_project(x, W, dst_row, k_fp4, k_sc, q_fmt=CSA2_Q_FP4, rope_cs=None, stream=None):
    """Indexer K of n entries: y = x W (fp32 chain), E2M1 with one E8M0 per row
    or per 32 channels (CSA2_Q_MXFP4), into rows dst_row of k_fp4 [rows][64].
    x is after RoPE, or before it when its angles rope_cs [n][32][2] are given."""
    n = int(dst_row.shape[0])
    st = lib().csa2_index_k_project(n, _ptr(x), _ptr(rope_cs), _ptr(W), _ptr(dst_row), int(k_fp4.shape[0]),
                                    int(q_fmt), _ptr(k_fp4), _ptr(k_sc), _stream(stream))
    _check(st, "csa2_index_k_project")


def csa2_compress(c_tok, z_tok, m, out=None, stream=None):
    """Entries from m tokens each: the per-channel softmax over an entry's
    tokens of z_tok weights c_tok ([n m][512] f32 each, on the device)."""
    n = int(c_tok.shape[0]) // int(m)
    if out is None:
        out = torch.empty((n, 512), dtype=torch.float32, device=c_tok.device)
    st = lib().csa2_compress(n, int(m), _ptr(c_tok), _ptr(z_tok), _ptr(out), _stream(stream))
    _check(st, "csa2_compress")
    return out


def csa2_kv_append(x, rope_cs, dst_row, kv_fp4, kv_sc, kv_fmt=CSA2_KV_MXFP4, stream=None):
    """Rotate and quantise n new main-KV entries into rows dst_row of the cache
    (kv_fp4 [rows][256], kv_sc [rows][16] or [rows][32]); x [n][512] f32,
    rope_cs [n][32][2] f32, dst_row [n] i64, all on the device."""
    n = int(dst_row.shape[0])
    st = lib().csa2_kv_append(n, _ptr(x), _ptr(rope_cs), _ptr(dst_row), int(kv_fp4.shape[0]), int(kv_fmt),
                              _ptr(kv_fp4), _ptr(kv_sc), _stream(stream))
    _check(st, "csa2_kv_append")


def csa2_gather_dequant(batch, kv_fp4, kv_sc, idx, stream=None, kv_fmt=CSA2_KV_MXFP4):
    K = idx.shape[1]
    out = torch.empty((batch.total_q, K, 512), dtype=torch.uint16, device=idx.device)
    st = lib().csa2_gather_dequant(ctypes.byref(batch.c), int(kv_fmt), _ptr(kv_fp4), _ptr(kv_sc), _ptr(idx), K,
                                   _ptr(out), _stream(stream))
    _check(st, "csa2_gather_dequant")
    return out


def csa2_sparse_attn(batch, q_bf16, kv_fp4, kv_sc, idx, swa_rows, swa_layout, softmax_scale, out=None, lse=None,
                     want_lse=True, ws=None, split=True, stream=None, kv_fmt=CSA2_KV_MXFP4):
    Hm = q_bf16.shape[1]
    dev = q_bf16.device
    if out is None:
        out = torch.empty((batch.total_q, Hm, 512), dtype=torch.float32, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((batch.total_q, Hm), dtype=torch.float32, device=dev)
    if ws is None and split:
        ws = workspace(csa2_workspace_size(CSA2_WS_SPARSE_ATTN, batch, idx.shape[1]), dev)
    st = lib().csa2_sparse_attn(ctypes.byref(batch.c), Hm, _ptr(q_bf16), int(kv_fmt), _ptr(kv_fp4), _ptr(kv_sc), _ptr(idx),
                                idx.shape[1], _ptr(swa_rows), ctypes.byref(swa_layout.c), float(softmax_scale),
                                _ptr(out), _ptr(lse), _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream))
    _check(st, "csa2_sparse_attn")
    return out, lse


def csa2_sparse_attn_rope(batch, q_bf16, rope_cs, kv_fp4, kv_sc, idx, swa_rows, swa_layout, softmax_scale, out=None,
                          lse=None, want_lse=True, ws=None, split=True, stream=None, kv_fmt=CSA2_KV_MXFP4):
    """Sparse attention with the RoPE steps fused: bf16 query before RoPE in
    (u16 bits), bf16 output (u16 bits) with its rotated channels turned back."""
    Hm = q_bf16.shape[1]
    dev = q_bf16.device
    if out is None:
        out = torch.empty((batch.total_q, Hm, 512), dtype=torch.uint16, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((batch.total_q, Hm), dtype=torch.float32, device=dev)
    if ws is None and split:
        ws = workspace(csa2_workspace_size(CSA2_WS_SPARSE_ATTN, batch, idx.shape[1]), dev)
    st = lib().csa2_sparse_attn_rope(ctypes.byref(batch.c), Hm, _ptr(q_bf16), _ptr(rope_cs), int(kv_fmt), _ptr(kv_fp4),
                                     _ptr(kv_sc), _ptr(idx), idx.shape[1], _ptr(swa_rows), ctypes.byref(swa_layout.c),
                                     float(softmax_scale), _ptr(out), _ptr(lse), _ptr(ws),
                                     0 if ws is None else ws.numel(), _stream(stream))
    _check(st, "csa2_sparse_attn_rope")
    return out, lse


def make_layers(specs):
    """specs: list of dicts with the csa2_layer fields (tensors or None)."""
    arr = (csa2_layer * len(specs))()
    for i, sp in enumerate(specs):
        L = arr[i]
        L.mode = sp["mode"]
        L.flags = sp.get("flags", 0)
        L.q_fmt = sp.get("q_fmt", CSA2_Q_FP4)
        L.kv_fmt = sp.get("kv_fmt", CSA2_KV_MXFP4)
        for f in ("q_idx", "q_sc", "w", "kv_fp4", "kv_sc", "k_fp4", "k_sc", "q_main", "swa", "out", "lse", "idx_out"):
            setattr(L, f, _ptr(sp.get(f)))
    return arr


def csa2_layer_chain(batch, params, layers, swa_layout, pool_blocks=None, pool_pos=None, pool_count=None, ws=None,
                     stream=None):
    st = lib().csa2_layer_chain(ctypes.byref(batch.c), ctypes.byref(params), len(layers), layers,
                                ctypes.byref(swa_layout.c), _ptr(pool_blocks), _ptr(pool_pos), _ptr(pool_count),
                                _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream))
    _check(st, "csa2_layer_chain")
