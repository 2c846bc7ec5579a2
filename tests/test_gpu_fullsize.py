"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (one csa2_layer_chain call over the whole batch).  The oracle
recomputes a sample of query rows: their indices and block pools must match bit
for bit, their attention outputs within |gpu - ref| <= 2e-3 + 1e-2 |ref|.

  decode_c0   1 x 4,096 entries, one Full layer (every row checked)
  decode_c1   64 x 131,072 entries, one Full layer (16 rows sampled; index scores
              of 4 rows compared over all 131,072 slots)
  chain_c2    16 x 1,048,576 entries, decoder layers 20..39 with pool (2 rows)
  prefill_c3  8,192 E4M3 query rows over 131,072 entries (ratio 2), Full + 5 Reuse
              (first, last and every 512th row); the index scores of every 16th
              row and the first and last 64 rows, over all 131,072 slots
  encoder_replay  1,152 E4M3 query rows (the last 128 prefix tokens replayed with
              a 1,024-token suffix) over 131,072 entries, Full + 5 Reuse
  decode_step_40  one decode token of 64 sequences through all 40 layers, in the
              pages' exact configuration (32 indexer heads, E4M3/16 main KV,
              MXFP4 indexer, FP8 SWA): 4 sequences checked
  ragged_c4   48 sequences of 4K..1M entries, 4 rows each, layers 20..39 with pool
              (the shortest and the longest sequence plus two more: 16 rows)
  replay_c5   decoder SWA bounded replay: 16 x 131,072 entries, the last 128
              prompt tokens of each sequence as FP4 query rows through layers
              20..39 with pool, windows cut at the replay start (the first,
              two middle and the last row of 4 sequences: 16 rows)
  decode_step_40 in the library's default formats as well (4 sequences)
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from compressed_sparse_attention_amd import csa2 as C
from gpu_util import DevWorkload, assert_close_attn, run_chain

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


def _check_chain(wl, rows, what):
    _say(f"[{what}] uploading {wl.total_entries} entries, {wl.total_q} rows, {len(wl.layers)} layers")
    dw = DevWorkload(wl)
    outs, (pb, pp, pc), _ = run_chain(dw)
    torch.cuda.synchronize()
    _say(f"[{what}] GPU chain done; oracle on {len(rows)} rows")
    ref = oracle.layer_chain(wl, rows=rows)
    worst = 0.0
    for o, r in zip(outs, ref):
        got_idx = o["idx"].cpu().numpy()[rows]
        assert np.array_equal(got_idx, r["idx"]), f"{what} layer {r['layer']}: indices differ"
        worst = max(worst, assert_close_attn(o["out"].cpu().numpy()[rows], r["out"], f"{what} layer {r['layer']}"))
        if "pool_pos" in r:
            assert np.array_equal(pb.cpu().numpy()[rows], r["blocks"]), f"{what}: pool blocks differ"
            assert np.array_equal(pp.cpu().numpy()[rows], r["pool_pos"]), f"{what}: pool positions differ"
            assert np.array_equal(pc.cpu().numpy()[rows], r["pool_count"]), f"{what}: pool counts differ"
    _say(f"[{what}] indices equal on every layer, attention max abs err {worst:.2e}")
    return dw


def test_fullsize_decode_c0():
    wl = synth.config("decode_c0")
    _check_chain(wl, np.arange(wl.total_q), "decode_c0")


def test_fullsize_decode_c1():
    wl = synth.config("decode_c1")
    rows = np.arange(0, 64, 4)
    dw = _check_chain(wl, rows, "decode_c1")
    # index scores of four rows over every slot, bit for bit
    L, dL = wl.layers[0], dw.layers[0]
    got = C.csa2_index_score(dw.batch, wl.H, C.CSA2_Q_FP4, dL["q_idx"], dL["q_sc"], dL["w"], dw.k_idx, dw.k_sc)
    sample = np.array([0, 21, 42, 63])
    ref = oracle.index_score(wl, L.q_idx, L.q_sc, L.w, synth.Q_FP4, rows=sample)
    assert np.array_equal(got.cpu().numpy()[sample].view(np.uint32), ref.view(np.uint32))


def test_fullsize_chain_c2():
    wl = synth.config("chain_c2")
    _check_chain(wl, np.array([0, 15]), "chain_c2")


def test_fullsize_prefill_c3():
    wl = synth.config("prefill_c3")
    rows = np.unique(np.concatenate([np.arange(0, 8192, 512), [1, 8190, 8191]]))
    _check_chain(wl, rows, "prefill_c3")


@pytest.mark.timeout(600)
def test_fullsize_prefill_c3_scores():
    """The prefill scorer's scores at full size, bit for bit, on every 16th row
    plus the first and last 64 (its segments, double buffer and causal cut-offs
    at the real shape)."""
    wl = synth.config("prefill_c3", n_layers=1, Hm=16)
    dw = DevWorkload(wl)
    L, dL = wl.layers[0], dw.layers[0]
    rows = np.unique(np.concatenate([np.arange(0, 8192, 16), np.arange(64), np.arange(8192 - 64, 8192)]))
    got = C.csa2_index_score(dw.batch, wl.H, C.CSA2_Q_FP8, dL["q_idx"], dL["q_sc"], dL["w"], dw.k_idx, dw.k_sc)
    got = got[torch.from_numpy(rows).to(got.device)].cpu().numpy()
    _say(f"[prefill_c3 scores] GPU done; oracle on {len(rows)} rows x {wl.total_entries} slots")
    ref = oracle.index_score(wl, L.q_idx, L.q_sc, L.w, synth.Q_FP8, rows=rows)
    bad = np.nonzero((got.view(np.uint32) != ref.view(np.uint32)).any(axis=1))[0]
    assert len(bad) == 0, f"{len(bad)} rows differ, first row {rows[bad[0]]}"
    _say(f"[prefill_c3 scores] {len(rows)} rows equal bit for bit")


def test_fullsize_encoder_replay():
    wl = synth.config("encoder_replay")
    rows = np.unique(np.concatenate([np.arange(0, wl.total_q, 64), [1, 127, 128, 129, wl.total_q - 1]]))
    _check_chain(wl, rows, "encoder_replay")


def test_fullsize_decode_step_40_pages():
    for wl in synth.decode_step_40(kv_fmt=1, swa_fmt=1, q_fmt=synth.Q_MXFP4, H=32):
        _check_chain(wl, np.array([0, 21, 42, 63]), wl.name)


def test_fullsize_ragged_c4():
    wl = synth.config("ragged_c4")
    n = wl.n_entries
    seqs = np.unique([int(np.argmin(n)), int(np.argmax(n)), 7, 30])
    rows = np.concatenate([np.arange(wl.q_off[b], wl.q_off[b + 1]) for b in seqs])
    _say(f"[ragged_c4] sum N = {int(n.sum())}, min {int(n.min())}, max {int(n.max())}; sampled sequences {seqs.tolist()}")
    _check_chain(wl, rows, "ragged_c4")


def test_fullsize_replay_c5():
    wl = synth.config("replay_c5")
    rows = np.concatenate([wl.q_off[b] + np.array([0, 63, 64, 127]) for b in (0, 5, 10, 15)])
    _check_chain(wl, rows, "replay_c5")


def test_fullsize_decode_step_40_default():
    for wl in synth.decode_step_40():
        _check_chain(wl, np.array([0, 21, 42, 63]), wl.name)
