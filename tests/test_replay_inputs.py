"""Saved inputs (synth.replay): a workload written as .bin files plus a JSON
manifest loads back array for array, keeps the layers' shared caches shared,
gives the oracle the same results, and is refused when a file was altered."""
import json
import os

import numpy as np
import pytest

import oracle
import synth
from synth.replay import load_workload, save_workload


def _small():
    # an encoder group at ratio 2 with per-Full-layer caches, a replay start and
    # MXFP8 SWA rows: every optional field of a workload is present
    return synth.make_workload("replay_io", 0xC5A2F001, [700, 2500], 3,
                               [(0, synth.MODE_SWA_ONLY, False), (2, synth.MODE_FULL, False),
                                (3, synth.MODE_REUSE, False), (4, synth.MODE_REINDEX, False),
                                (8, synth.MODE_FULL, False), (9, synth.MODE_REUSE, False)],
                               ratio=2, Hm=16, own_caches=True, swa_fmt=1, kv_fmt=1,
                               q_pos=[np.array([1390, 1395, 1399]), np.array([4000, 4990, 4999])],
                               replay_s=np.array([1300, 0], np.int32))


def _same(a, b):
    return a is None and b is None or (a is not None and b is not None and a.dtype == b.dtype and a.shape == b.shape
                                       and np.array_equal(a, b))


def test_round_trip_and_oracle(tmp_path):
    wl = _small()
    save_workload(wl, str(tmp_path), note="round trip")
    got = load_workload(str(tmp_path))
    for k in ("name", "seed", "ratio", "H", "Hm", "K", "W", "block", "max_blocks", "kv_fmt", "swa_fmt"):
        assert getattr(got, k) == getattr(wl, k), k
    for k in ("n_entries", "entry_off", "q_off", "q_pos", "row_seq", "swa_row_off", "swa_pos0", "swa_len", "k_idx",
              "k_sc", "kv", "kv_sc", "replay_s"):
        assert _same(getattr(got, k), getattr(wl, k)), k
    assert len(got.layers) == len(wl.layers)
    for a, b in zip(got.layers, wl.layers):
        assert (a.index, a.mode, a.q_fmt, a.build_pool) == (b.index, b.mode, b.q_fmt, b.build_pool)
        for k in ("q_idx", "q_sc", "w", "q_main", "swa", "k_idx", "k_sc", "kv", "kv_sc"):
            assert _same(getattr(a, k), getattr(b, k)), (a.index, k)
            # a cache that was the workload's own is the loaded workload's own again
            if k in ("k_idx", "k_sc", "kv", "kv_sc") and getattr(b, k) is getattr(wl, k):
                assert getattr(a, k) is getattr(got, k)
    # shared caches are written once
    assert not any(f.startswith("layer1_k") for f in os.listdir(tmp_path))
    ref, rep = oracle.layer_chain(wl), oracle.layer_chain(got)
    for r, q in zip(ref, rep):
        assert np.array_equal(r["idx"], q["idx"])
        assert np.array_equal(r["out"].view(np.uint64), q["out"].view(np.uint64))


def test_altered_files_are_refused(tmp_path):
    wl = _small()
    save_workload(wl, str(tmp_path))
    path = tmp_path / "q_pos.bin"
    raw = bytearray(path.read_bytes())
    raw[0] ^= 1
    path.write_bytes(bytes(raw))
    with pytest.raises(ValueError, match="SHA-256"):
        load_workload(str(tmp_path))
    path.write_bytes(bytes(raw[:-4]))
    with pytest.raises(ValueError, match="bytes"):
        load_workload(str(tmp_path))
    man = json.loads((tmp_path / "manifest.json").read_text())
    man["format"] = "something else"
    (tmp_path / "manifest.json").write_text(json.dumps(man))
    with pytest.raises(ValueError, match="manifest"):
        load_workload(str(tmp_path))
