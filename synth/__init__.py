"""Seeded synthetic inputs for the CSA2 hot path.

This module is shared by the GPU tests, the benchmark and the oracle's tests.
It only draws random numbers (a counter-based generator, see csa2_synth.c) and
encodes them into the cache formats; it computes no step of the method.

Workloads (shapes follow the report's configuration, section 4.2.1, and the
reading note's decoder schedule table):
  decode_c0   1 sequence, 4,096 entries, 1 query at t = 4,095, one Full layer
  decode_c1   64 sequences x 131,072 entries, 1 query each at t = N-1, one Full layer
  chain_c2    16 sequences x 1,048,576 entries, decoder layers 20..39
              (20 Full + pool, 24/28/32/36 Reindex, the rest Reuse)
  prefill_c3  1 sequence of 262,144 tokens at ratio 2 (131,072 entries),
              8,192 query tokens t = 253,952..262,143, Full + 5 Reuse, FP8 indexer q
  ragged_c4   48 sequences, N_b log-uniform in [4,096, 1,048,576], 4 queries at
              t = N_b-4..N_b-1, decoder layers 20..39
  replay_c5   decoder SWA bounded replay: 16 x 131,072 entries, the last 128
              prompt tokens through decoder layers 20..39, windows cut at the
              replay start
  encoder_replay  encoder SWA bounded replay: 262,144 tokens at ratio 2, the
              last 128 tokens of a cached prefix replayed with a 1,024-token
              uncached suffix (1,152 E4M3 query rows), Full + 5 Reuse
  decode_step_40  one decode token through all 40 layers (encoder chain 0..19
              at ratio 2 with three Full caches, decoder chain 20..39)
Every raw value is N(0,1) before encoding; head weights are U(0,1).
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# CSA2_SYNTH_SO: a library built elsewhere from the same source (the
# sanitizer run of the CPU tests loads an instrumented build through it)
_SO = os.environ.get("CSA2_SYNTH_SO") or os.path.join(_HERE, "libcsa2_synth.so")
_SRC = os.path.join(_HERE, "csa2_synth.c")

MODE_SWA_ONLY, MODE_FULL, MODE_REINDEX, MODE_REUSE = 0, 1, 2, 3
Q_FP4, Q_FP8, Q_MXFP4 = 0, 1, 2

TID_K, TID_KV, TID_LEN = 1, 2, 3


def _tid(layer: int, what: int) -> int:
    return 100 + 10 * layer + what


def build(force: bool = False) -> str:
    """Compile the generator with gcc (host code only)."""
    if os.environ.get("CSA2_SYNTH_SO"):
        return _SO
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-pthread", "-shared", "-fPIC", _SRC, "-o", _SO, "-lm"])
    return _SO


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_SO)
        u64, i64, i32, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        L.csa2synth_normal_f32.argtypes = [u64, u64, i64, i64, vp]
        L.csa2synth_uniform_f32.argtypes = [u64, u64, i64, i64, vp]
        L.csa2synth_normal_f64.argtypes = [u64, u64, i64, i64, vp]
        L.csa2synth_normal_bf16.argtypes = [u64, u64, i64, i64, vp]
        L.csa2synth_mxfp4_rows.argtypes = [u64, u64, i64, i64, i32, i32, vp, vp]
        L.csa2synth_e4m3_rows.argtypes = [u64, u64, i64, i64, i32, vp, vp]
        L.csa2synth_e2m1_e4m3_rows.argtypes = [u64, u64, i64, i64, i32, vp, vp]
        L.csa2synth_mxfp8_rows.argtypes = [u64, u64, i64, i64, i32, vp]
        L.csa2synth_encode_e2m1.argtypes = [ctypes.c_double]
        L.csa2synth_encode_e2m1.restype = ctypes.c_uint8
        L.csa2synth_encode_e4m3.argtypes = [ctypes.c_double]
        L.csa2synth_encode_e4m3.restype = ctypes.c_uint8
        L.csa2synth_encode_bf16.argtypes = [ctypes.c_float]
        L.csa2synth_encode_bf16.restype = ctypes.c_uint16
        L.csa2synth_hash.argtypes = [u64, u64, u64]
        L.csa2synth_hash.restype = u64
        L.csa2synth_set_threads.argtypes = [i32]
        L.csa2synth_set_threads(min(16, os.cpu_count() or 8))
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def normal_f32(seed, tid, n, off=0):
    out = np.empty(n, np.float32)
    lib().csa2synth_normal_f32(seed, tid, off, n, _ptr(out))
    return out


def normal_f64(seed, tid, n, off=0):
    out = np.empty(n, np.float64)
    lib().csa2synth_normal_f64(seed, tid, off, n, _ptr(out))
    return out


def uniform_f32(seed, tid, n, off=0):
    out = np.empty(n, np.float32)
    lib().csa2synth_uniform_f32(seed, tid, off, n, _ptr(out))
    return out


def normal_bf16(seed, tid, n, off=0):
    out = np.empty(n, np.uint16)
    lib().csa2synth_normal_bf16(seed, tid, off, n, _ptr(out))
    return out


def mxfp4_rows(seed, tid, nrows, row_len, block, row0=0):
    codes = np.empty((nrows, row_len // 2), np.uint8)
    scales = np.empty((nrows, row_len // block), np.uint8)
    rc = lib().csa2synth_mxfp4_rows(seed, tid, row0, nrows, row_len, block, _ptr(codes), _ptr(scales))
    assert rc == 0
    return codes, scales


def e4m3_rows(seed, tid, nrows, row_len, row0=0):
    codes = np.empty((nrows, row_len), np.uint8)
    scales = np.empty((nrows,), np.uint8)
    rc = lib().csa2synth_e4m3_rows(seed, tid, row0, nrows, row_len, _ptr(codes), _ptr(scales))
    assert rc == 0
    return codes, scales


def e2m1_e4m3_rows(seed, tid, nrows, row_len, row0=0):
    """E2M1 rows with one E4M3 scale per 16 values (the report's main-KV format)."""
    codes = np.empty((nrows, row_len // 2), np.uint8)
    scales = np.empty((nrows, row_len // 16), np.uint8)
    rc = lib().csa2synth_e2m1_e4m3_rows(seed, tid, row0, nrows, row_len, _ptr(codes), _ptr(scales))
    assert rc == 0
    return codes, scales


def mxfp8_rows(seed, tid, nrows, row_len, row0=0):
    """OCP MXFP8 rows (E4M3 elements, one E8M0 per 32), codes then scales per row."""
    out = np.empty((nrows, row_len + row_len // 32), np.uint8)
    rc = lib().csa2synth_mxfp8_rows(seed, tid, row0, nrows, row_len, _ptr(out))
    assert rc == 0
    return out


def uniform_u64(seed, tid, i):
    return lib().csa2synth_hash(seed, tid, i)


# ---------------------------------------------------------------------------
# Workload description
# ---------------------------------------------------------------------------

@dataclass
class Layer:
    index: int
    mode: int
    q_fmt: int = Q_FP4
    q_idx: Optional[np.ndarray] = None    # FP4 [T][H][64] or FP8 [T][H][128], u8
    q_sc: Optional[np.ndarray] = None     # [T][H] u8 (E8M0), or [T][H][4] for Q_MXFP4
    w: Optional[np.ndarray] = None        # [T][H] f32
    q_main: Optional[np.ndarray] = None   # [T][Hm][512] bf16 bits (u16)
    swa: Optional[np.ndarray] = None      # [rows][512] bf16 bits (u16)
    build_pool: bool = False
    # a Full layer's own caches (None: the workload's); the layers up to the
    # next Full layer read them (report 2.3.1: Reindex and Reuse share the
    # global KV and indexer K of the preceding Full layer)
    k_idx: Optional[np.ndarray] = None
    k_sc: Optional[np.ndarray] = None
    kv: Optional[np.ndarray] = None
    kv_sc: Optional[np.ndarray] = None


@dataclass
class Workload:
    name: str
    seed: int
    ratio: int
    H: int            # indexer heads
    Hm: int           # main query heads
    K: int            # Top-K
    W: int            # SWA window
    block: int
    max_blocks: int
    n_entries: np.ndarray      # [n_seq] i64
    entry_off: np.ndarray      # [n_seq+1] i64
    q_off: np.ndarray          # [n_seq+1] i32
    q_pos: np.ndarray          # [total_q] i32 token positions
    row_seq: np.ndarray        # [total_q] i32
    swa_row_off: np.ndarray    # [n_seq] i64
    swa_pos0: np.ndarray       # [n_seq] i32
    swa_len: np.ndarray        # [n_seq] i32
    k_idx: np.ndarray = None   # [sumN][64] u8
    k_sc: np.ndarray = None    # [sumN] u8, or [sumN][4] when the layers use Q_MXFP4
    kv: np.ndarray = None      # [sumN][256] u8
    kv_sc: np.ndarray = None   # [sumN][16] u8
    layers: List[Layer] = field(default_factory=list)
    replay_s: Optional[np.ndarray] = None  # [n_seq] i32 SWA replay start per sequence (None: 0)
    kv_fmt: int = 0                        # main-KV scales: 0 E8M0 per 32 channels, 1 E4M3 per 16 channels
    swa_fmt: int = 0                       # SWA rows: 0 bf16 [rows][512], 1 MXFP8 [rows][528] (codes, then scales)

    @property
    def n_seq(self):
        return len(self.n_entries)

    @property
    def total_q(self):
        return len(self.q_pos)

    @property
    def total_entries(self):
        return int(self.entry_off[-1])


def decoder_schedule(first=20, last=39):
    """Decoder layers 20..39: 20 Full (builds the pool), 24/28/32/36 Reindex,
    the rest Reuse (report 4.2.1; reading note schedule table)."""
    out = []
    for l in range(first, last + 1):
        if l == 20:
            out.append((l, MODE_FULL, True))
        elif l in (24, 28, 32, 36):
            out.append((l, MODE_REINDEX, False))
        else:
            out.append((l, MODE_REUSE, False))
    return out


def encoder_schedule():
    """Encoder layers 0..19 (report 4.2.1): layers 0 and 1 pure sliding window,
    then three groups of six at ratio 2, each a Full layer and five Reuse."""
    out = [(0, MODE_SWA_ONLY, False), (1, MODE_SWA_ONLY, False)]
    for g0 in (2, 8, 14):
        out.append((g0, MODE_FULL, False))
        out += [(l, MODE_REUSE, False) for l in range(g0 + 1, g0 + 6)]
    return out


def decode_step_40(n_seq=64, tokens=131072, **kw):
    """One decode token of every sequence through all 40 layers (report 4.2.1),
    as the two chains the layers form: the encoder layers 0..19 at ratio 2 over
    tokens / 2 entries (two sliding-window layers, then three groups of a Full
    layer and five Reuse layers, each Full layer with its own caches) and the
    decoder layers 20..39 at ratio 1 over `tokens` entries with the pool.
    Returns the workloads in layer order."""
    t = [np.array([tokens - 1], np.int64)] * n_seq
    seed = 0xC5A20000 + CONFIG_IDS["decode_step_40"]
    enc = make_workload("step40_enc", seed, [tokens // 2] * n_seq, 1, encoder_schedule(), ratio=2, q_pos=t,
                        own_caches=True, **kw)
    dec = make_workload("step40_dec", seed + 64, [tokens] * n_seq, 1, decoder_schedule(), q_pos=t, **kw)
    return [enc, dec]


def ragged_lengths(seed, n_seq, lo=4096, hi=1048576):
    """N_b = round(exp(U(ln lo, ln hi))), U from the counter generator."""
    out = np.empty(n_seq, np.int64)
    for b in range(n_seq):
        u = (uniform_u64(seed, TID_LEN, b) >> 40) * 2.0 ** -24
        out[b] = int(round(math.exp(math.log(lo) + u * (math.log(hi) - math.log(lo)))))
    return out


def make_workload(name, seed, n_entries, queries_per_seq, schedule, ratio=1, H=64, Hm=64, K=512, W=128,
                  block=8, max_blocks=2048, q_fmt=Q_FP4, q_pos=None, gen_kv=True, gen_layers=True, replay_s=None,
                  kv_fmt=0, swa_fmt=0, own_caches=False):
    """Build a workload.  n_entries: per-sequence entry counts.  queries_per_seq:
    T (same for all sequences).  q_pos: explicit token positions per sequence
    (list of arrays) or None for the decode shape t = N*ratio - T + i.
    schedule: list of (layer index, mode, build_pool).  replay_s: per-sequence
    SWA replay start s (a query at t sees window rows max(s, t - W + 1) .. t).
    kv_fmt: main-KV scales, 0 = OCP MXFP4 (E8M0 per 32 channels), 1 = the
    report's E4M3 per 16 channels.  swa_fmt: SWA rows, 0 = bf16, 1 = OCP
    MXFP8 (E4M3 with one E8M0 per 32 channels, codes then scales per row).
    q_fmt: indexer queries, Q_FP4 / Q_FP8 (one E8M0 per head row, indexer K
    with one E8M0 per row), or Q_MXFP4 (the report's indexer format: queries
    and indexer K both OCP MXFP4 with one E8M0 per 32 channels).
    own_caches: every Full layer draws its own main KV and indexer K (the
    first Full layer's are also the workload's), as the encoder's Full layers
    2, 8 and 14 each generate theirs."""
    n_entries = np.asarray(n_entries, np.int64)
    n_seq = len(n_entries)
    entry_off = np.zeros(n_seq + 1, np.int64)
    entry_off[1:] = np.cumsum(n_entries)
    T = int(queries_per_seq)
    if q_pos is None:
        q_pos = [np.arange(int(n) * ratio - T, int(n) * ratio, dtype=np.int64) for n in n_entries]
    q_pos_all = np.concatenate([np.asarray(p, np.int64) for p in q_pos]).astype(np.int32)
    q_off = np.zeros(n_seq + 1, np.int32)
    q_off[1:] = np.cumsum([len(p) for p in q_pos])
    row_seq = np.repeat(np.arange(n_seq, dtype=np.int32), [len(p) for p in q_pos])
    # SWA rows: token positions [min(t) - W + 1, max(t)] clipped at 0, per
    # sequence (none for a sequence without query rows)
    swa_pos0 = np.array([max(0, int(np.min(p)) - W + 1) if len(p) else 0 for p in q_pos], np.int32)
    swa_len = np.array([int(np.max(p)) - s + 1 if len(p) else 0 for p, s in zip(q_pos, swa_pos0)], np.int32)
    swa_row_off = np.zeros(n_seq, np.int64)
    swa_row_off[1:] = np.cumsum(swa_len)[:-1]
    wl = Workload(name, seed, ratio, H, Hm, K, W, block, max_blocks, n_entries, entry_off, q_off, q_pos_all,
                  row_seq, swa_row_off, swa_pos0, swa_len)
    if replay_s is not None:
        wl.replay_s = np.ascontiguousarray(replay_s, np.int32)
    wl.kv_fmt = int(kv_fmt)
    wl.swa_fmt = int(swa_fmt)
    total = int(entry_off[-1])

    def caches(tid_k, tid_kv):
        if q_fmt == Q_MXFP4:  # the report's indexer format: one E8M0 per 32 channels
            k_idx, k_sc = mxfp4_rows(seed, tid_k, total, 128, 32)
        else:
            k_idx, ksc = mxfp4_rows(seed, tid_k, total, 128, 128)
            k_sc = np.ascontiguousarray(ksc.reshape(total))
        if kv_fmt == 1:
            kv, kv_sc = e2m1_e4m3_rows(seed, tid_kv, total, 512)
        else:
            kv, kv_sc = mxfp4_rows(seed, tid_kv, total, 512, 32)
        return k_idx, k_sc, kv, kv_sc

    if gen_kv:
        wl.k_idx, wl.k_sc, wl.kv, wl.kv_sc = caches(TID_K, TID_KV)
    nq = len(q_pos_all)
    swa_rows = int(swa_len.sum())
    first_full = True
    for (li, mode, pool) in schedule:
        L = Layer(index=li, mode=mode, q_fmt=q_fmt, build_pool=pool)
        if own_caches and gen_kv and mode == MODE_FULL:
            if first_full:
                L.k_idx, L.k_sc, L.kv, L.kv_sc = wl.k_idx, wl.k_sc, wl.kv, wl.kv_sc
            else:
                L.k_idx, L.k_sc, L.kv, L.kv_sc = caches(_tid(li, 4), _tid(li, 5))
            first_full = False
        if gen_layers:
            if mode in (MODE_FULL, MODE_REINDEX):
                if q_fmt == Q_FP4:
                    c, s = mxfp4_rows(seed, _tid(li, 0), nq * H, 128, 128)
                    L.q_idx = c.reshape(nq, H, 64)
                    L.q_sc = s.reshape(nq, H)
                elif q_fmt == Q_MXFP4:
                    c, s = mxfp4_rows(seed, _tid(li, 0), nq * H, 128, 32)
                    L.q_idx = c.reshape(nq, H, 64)
                    L.q_sc = s.reshape(nq, H, 4)
                else:
                    c, s = e4m3_rows(seed, _tid(li, 0), nq * H, 128)
                    L.q_idx = c.reshape(nq, H, 128)
                    L.q_sc = s.reshape(nq, H)
                L.w = uniform_f32(seed, _tid(li, 1), nq * H).reshape(nq, H)
            L.q_main = normal_bf16(seed, _tid(li, 2), nq * Hm * 512).reshape(nq, Hm, 512)
            if swa_fmt == 1:
                L.swa = mxfp8_rows(seed, _tid(li, 3), swa_rows, 512)
            else:
                L.swa = normal_bf16(seed, _tid(li, 3), swa_rows * 512).reshape(swa_rows, 512)
        wl.layers.append(L)
    return wl


CONFIG_IDS = {"decode_c0": 0, "decode_c1": 1, "chain_c2": 2, "prefill_c3": 3, "ragged_c4": 4, "replay_c5": 5,
              "decode_step_40": 6, "encoder_replay": 7}


def config(name, **kw):
    """The five workloads at full size (keyword overrides shrink them for tests)."""
    cid = CONFIG_IDS[name]
    seed = kw.pop("seed", 0xC5A20000 + cid)
    if name == "decode_c0":
        return make_workload(name, seed, kw.pop("n_entries", [4096]), 1, [(20, MODE_FULL, False)], **kw)
    if name == "decode_c1":
        n_seq = kw.pop("n_seq", 64)
        n = kw.pop("n", 131072)
        return make_workload(name, seed, [n] * n_seq, 1, [(20, MODE_FULL, False)], **kw)
    if name == "chain_c2":
        n_seq = kw.pop("n_seq", 16)
        n = kw.pop("n", 1048576)
        sched = kw.pop("schedule", decoder_schedule())
        return make_workload(name, seed, [n] * n_seq, 1, sched, **kw)
    if name == "prefill_c3":
        tokens = kw.pop("tokens", 262144)
        T = kw.pop("T", 8192)
        n_layers = kw.pop("n_layers", 6)
        sched = [(2, MODE_FULL, False)] + [(2 + i, MODE_REUSE, False) for i in range(1, n_layers)]
        qp = [np.arange(tokens - T, tokens, dtype=np.int64)]
        return make_workload(name, seed, [tokens // 2], T, sched, ratio=2, q_fmt=Q_FP8, q_pos=qp, **kw)
    if name == "replay_c5":
        # decoder SWA bounded replay: the last T = W prompt tokens of each
        # sequence run the decoder layers again as T query rows against the
        # decoder's global cache, every window cut at the first replayed token
        n_seq = kw.pop("n_seq", 16)
        n = kw.pop("n", 131072)
        T = kw.pop("T", 128)
        sched = kw.pop("schedule", decoder_schedule())
        return make_workload(name, seed, [n] * n_seq, T, sched, replay_s=[n - T] * n_seq, **kw)
    if name == "encoder_replay":
        # encoder SWA bounded replay: a cached prefix of `prefix` tokens whose
        # encoder SWA KV is missing; its last W tokens are replayed together
        # with an uncached suffix through one encoder group (Full + 5 Reuse at
        # ratio 2, E4M3 indexer queries).  The replayed rows reuse the cached
        # global KV, the suffix's entries are in the cache too (the suffix
        # writes global KV), and every window is cut at the replay start
        tokens = kw.pop("tokens", 262144)
        suffix = kw.pop("suffix", 1024)
        W = kw.get("W", 128)
        n_layers = kw.pop("n_layers", 6)
        s0 = tokens - suffix - W
        sched = [(2, MODE_FULL, False)] + [(2 + i, MODE_REUSE, False) for i in range(1, n_layers)]
        qp = [np.arange(s0, tokens, dtype=np.int64)]
        return make_workload(name, seed, [tokens // 2], len(qp[0]), sched, ratio=2, q_fmt=Q_FP8, q_pos=qp,
                             replay_s=[s0], **kw)
    if name == "ragged_c4":
        n_seq = kw.pop("n_seq", 48)
        lens = kw.pop("lengths", None)
        if lens is None:
            lens = ragged_lengths(seed, n_seq)
        sched = kw.pop("schedule", decoder_schedule())
        return make_workload(name, seed, lens, 4, sched, **kw)
    raise KeyError(name)
