"""GPU parity: every call of the C ABI against the CPU oracle on the same seeded
inputs.  Scores, indices, pools and dequantised rows must match bit for bit;
attention outputs within |gpu - ref| <= 2e-3 + 1e-2 |ref|.

Sizes are small enough for the oracle to finish in seconds while spanning
several tiles, ragged tails and the degenerate cases (1-entry sequences, fewer
visible entries than K, contexts shorter than the SWA window, ties)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from compressed_sparse_attention_amd import csa2 as C
from gpu_util import SCALE, DevWorkload, assert_close_attn, dev, run_chain, saved_on_failure

pytestmark = pytest.mark.gpu


def _full_rows_equal(got, ref, wl):
    """Compare score rows over slots 0..N_b-1 of each row's sequence, bitwise."""
    got = got.cpu().numpy()
    for r in range(wl.total_q):
        n = int(wl.n_entries[wl.row_seq[r]])
        g, o = got[r, :n], ref[r, :n]
        if not np.array_equal(g.view(np.uint32), o.view(np.uint32)):
            bad = np.nonzero(g.view(np.uint32) != o.view(np.uint32))[0]
            raise AssertionError(f"row {r}: {len(bad)} scores differ, first at slot {bad[0]}: {g[bad[0]]!r} vs {o[bad[0]]!r}")


DECODE_CASES = {
    "c0_4096": dict(name="decode_c0"),
    "ragged_t1": dict(name="decode_c1", lens=[1, 7, 63, 64, 65, 255, 4097, 9000]),
    "ragged_t4": dict(name="ragged_c4", lens=[5, 64, 300, 5000, 70000], T=4),
    "h32": dict(name="decode_c1", lens=[100, 3000], H=32),
    # the report's indexer format: FP4 queries and keys with an E8M0 per 32
    # channels (one query row and four rows per sequence, 64 and 32 heads)
    "c0_mx": dict(name="decode_c0", q_fmt=synth.Q_MXFP4),
    "ragged_t4_mx": dict(name="ragged_c4", lens=[5, 64, 300, 5000, 70000], T=4, q_fmt=synth.Q_MXFP4),
    "h32_mx": dict(name="decode_c1", lens=[100, 3000], H=32, q_fmt=synth.Q_MXFP4),
}


def _decode_wl(case):
    c = DECODE_CASES[case]
    q_fmt = c.get("q_fmt", synth.Q_FP4)
    if "lens" not in c:
        return synth.config(c["name"], q_fmt=q_fmt)
    T = c.get("T", 1)
    return synth.make_workload(case, 0xC5A2F000 + len(case), c["lens"], T, [(20, synth.MODE_FULL, False)],
                               H=c.get("H", 64), Hm=16, q_fmt=q_fmt)


@pytest.mark.parametrize("case", list(DECODE_CASES))
def test_index_score_full_bitwise(case):
    wl = _decode_wl(case)
    dw = DevWorkload(wl)
    L, dL = wl.layers[0], dw.layers[0]
    got = C.csa2_index_score(dw.batch, wl.H, L.q_fmt, dL["q_idx"], dL["q_sc"], dL["w"], dw.k_idx, dw.k_sc)
    torch.cuda.synchronize()
    ref = oracle.index_score(wl, L.q_idx, L.q_sc, L.w, L.q_fmt)
    _full_rows_equal(got, ref, wl)
    # deterministic across runs; the variant that also builds the Top-K histogram
    # writes the same scores, and its histogram equals one counted on the host
    hist = C.hist_buffer(dw.batch)
    again = C.csa2_index_score(dw.batch, wl.H, L.q_fmt, dL["q_idx"], dL["q_sc"], dL["w"], dw.k_idx, dw.k_sc,
                               hist=hist)
    _full_rows_equal(again, ref, wl)  # slots past N_b are not written; compare the written ones
    vis = oracle.row_visible(wl)
    h = hist.cpu().numpy()
    for r in range(wl.total_q):
        bins = ref[r, :vis[r]].view(np.uint32) >> 19
        assert np.array_equal(h[r], np.bincount(bins, minlength=4096)), r
    # Top-K from the fused histogram equals Top-K without it
    assert torch.equal(C.csa2_topk(dw.batch, got, 512, hist=hist), C.csa2_topk(dw.batch, got, 512))


@pytest.mark.parametrize("q_fmt", [synth.Q_FP4, synth.Q_MXFP4])
def test_index_score_cand_bitwise(q_fmt):
    wl = synth.config("chain_c2", n_seq=2, n=30000, Hm=16, q_fmt=q_fmt)
    dw = DevWorkload(wl)
    full = wl.layers[0]
    sc = oracle.index_score(wl, full.q_idx, full.q_sc, full.w, q_fmt)
    vis = oracle.row_visible(wl)
    _, pool, cnt = oracle.block_pool(sc, vis)
    pool[0, 100:140] = -1  # holes are allowed in a candidate list
    L = [x for x in wl.layers if x.mode == synth.MODE_REINDEX][0]
    dL = [x for x in dw.layers if x["index"] == L.index][0]
    hist = C.hist_buffer(dw.batch)
    got = C.csa2_index_score(dw.batch, wl.H, q_fmt, dL["q_idx"], dL["q_sc"], dL["w"], dw.k_idx, dw.k_sc,
                             cand=dev(pool), hist=hist)
    torch.cuda.synchronize()
    ref = oracle.index_score(wl, L.q_idx, L.q_sc, L.w, q_fmt, cand=pool)
    assert np.array_equal(got.cpu().numpy().view(np.uint32), ref.view(np.uint32))
    h = hist.cpu().numpy()
    for r in range(wl.total_q):
        fin = ref[r][np.isfinite(ref[r])]
        assert np.array_equal(h[r], np.bincount(fin.view(np.uint32) >> 19, minlength=4096)), r


# E4M3 query rows over 60,000 entries at ratio 2: four 16,384-position
# segments of the prefill scorer, rows of one 8-row group with causal cutoffs
# early, mid-segment, mid-chunk (not a multiple of 512) and at the end
_PF8_SEG_T = np.array([9999, 32770, 33000, 40033, 65535, 66001, 99999, 100001, 110003, 119999, 20, 1], np.int64)


@pytest.mark.parametrize("fmt", ["fp8", "fp8_h32", "fp8_segments", "fp4", "mxfp4", "mxfp4_h32"])
def test_index_score_prefill_bitwise(fmt):
    if fmt == "fp8":
        wl = synth.config("prefill_c3", tokens=6002, T=150, n_layers=1, Hm=16)
    elif fmt == "fp8_segments":
        wl = synth.make_workload("pf8seg", 92, [60000], len(_PF8_SEG_T), [(2, synth.MODE_FULL, False)], ratio=2,
                                 Hm=16, q_fmt=synth.Q_FP8, q_pos=[_PF8_SEG_T])
    elif fmt == "fp8_h32":  # 32 indexer heads, two sequences, 61 rows each (a ragged row group)
        wl = synth.make_workload("pf8h32", 91, [2500, 3100], 61, [(2, synth.MODE_FULL, False)], ratio=2, H=32,
                                 Hm=16, q_fmt=synth.Q_FP8)
    elif fmt == "fp4":  # FP4 queries, 9 rows per sequence, ratio 2: the many-query kernel
        wl = synth.make_workload("pf4", 77, [1500, 2100], 9, [(2, synth.MODE_FULL, False)], ratio=2, Hm=16)
    else:  # the same kernel with the report's MXFP4 indexer format
        wl = synth.make_workload("pf4mx", 78, [1500, 2100], 9, [(2, synth.MODE_FULL, False)], ratio=2, Hm=16,
                                 H=32 if fmt.endswith("h32") else 64, q_fmt=synth.Q_MXFP4)
    dw = DevWorkload(wl)
    L, dL = wl.layers[0], dw.layers[0]
    got = C.csa2_index_score(dw.batch, wl.H, L.q_fmt, dL["q_idx"], dL["q_sc"], dL["w"], dw.k_idx, dw.k_sc)
    torch.cuda.synchronize()
    ref = oracle.index_score(wl, L.q_idx, L.q_sc, L.w, L.q_fmt)
    _full_rows_equal(got, ref, wl)


def _topk_batch(lens, T):
    qp = [np.arange(n - T, n) for n in lens]
    return C.Batch(lens, qp), qp


def _signed_scores(rng, nq, stride):
    """Scores of both signs: normal values, some rows all negative, exact
    zeros of both signs, ties and -inf slots."""
    s = rng.standard_normal((nq, stride)).astype(np.float32)
    s[::3] = -np.abs(s[::3])                        # rows with no non-negative score
    s[:, 5::97] = 0.0
    s[:, 7::89] = -0.0
    s[:, 11::53] = np.round(s[:, 11::53] * 4) / 4   # ties
    s[1::2, 13::61] = -np.inf
    return s


@pytest.mark.parametrize("distinct", [4, 1000, 0, -1])
def test_topk_full_bitwise(distinct):
    rng = np.random.default_rng(11 + distinct)
    lens = [3, 511, 512, 513, 20000, 70000]
    b, qp = _topk_batch(lens, 2)
    nq = b.total_q
    stride = max(lens)
    if distinct > 0:
        s = (rng.integers(0, distinct, size=(nq, stride)) * 0.5).astype(np.float32)
    elif distinct == 0:  # continuous
        s = rng.random((nq, stride)).astype(np.float32) * 100
    else:  # both signs, -inf slots
        s = _signed_scores(rng, nq, stride)
    vis = np.array([min(n, t + 1) for n, p in zip(lens, qp) for t in p], np.int64)
    for K in (512, 2048, 17):
        got = C.csa2_topk(b, dev(s), K)
        torch.cuda.synchronize()
        ref = oracle.topk(s, vis, K)
        assert np.array_equal(got.cpu().numpy(), ref), K


@pytest.mark.parametrize("distinct", [4, 1000, 0, 1, -1])
def test_topk_rows_bitwise(distinct):
    """Rows of at most 16,384 slots: one workgroup per row selects from the
    scores held in registers (few distinct values, continuous, all equal,
    both signs with -inf slots)."""
    rng = np.random.default_rng(23 + distinct)
    lens = [2, 3, 511, 512, 513, 9000, 16384]
    b, qp = _topk_batch(lens, 2)
    nq = b.total_q
    stride = max(lens)
    if distinct > 0:
        s = (rng.integers(0, distinct, size=(nq, stride)) * 0.5).astype(np.float32)
    elif distinct == 0:
        s = rng.random((nq, stride)).astype(np.float32) * 100
    else:
        s = _signed_scores(rng, nq, stride)
    vis = np.array([min(n, t + 1) for n, p in zip(lens, qp) for t in p], np.int64)
    for K in (512, 2048, 17):
        got = C.csa2_topk(b, dev(s), K)
        torch.cuda.synchronize()
        ref = oracle.topk(s, vis, K)
        assert np.array_equal(got.cpu().numpy(), ref), K


def test_topk_all_equal_uses_fallback():
    # every score equal: the candidate list overflows and the fallback picks the lowest positions
    lens = [50000, 9000]
    b, qp = _topk_batch(lens, 1)
    s = np.full((2, 50000), 3.25, np.float32)
    got = C.csa2_topk(b, dev(s), 512).cpu().numpy()
    assert np.array_equal(got[0], np.arange(512)) and np.array_equal(got[1], np.arange(512))
    vis = np.array([50000, 9000])
    assert np.array_equal(got, oracle.topk(s, vis, 512))


def test_topk_cand_bitwise():
    rng = np.random.default_rng(5)
    lens = [100000, 40000]
    b, qp = _topk_batch(lens, 1)
    stride = 16384
    cand = np.full((2, stride), -1, np.int32)
    cnt = np.array([16384, 7001], np.int32)
    for r in range(2):
        cand[r, :cnt[r]] = np.sort(rng.choice(lens[r], cnt[r], replace=False))
    s = (rng.integers(0, 300, size=(2, stride)) * 0.25).astype(np.float32)
    got = C.csa2_topk(b, dev(s), 512, cand=dev(cand), cand_count=dev(cnt))
    ref = oracle.topk(s, cnt.astype(np.int64), 512, cand=cand)
    assert np.array_equal(got.cpu().numpy(), ref)


def test_block_pool_bitwise():
    rng = np.random.default_rng(8)
    lens = [7, 16384, 16385, 30001, 90000]
    b, qp = _topk_batch(lens, 1)
    s = (rng.integers(0, 5000, size=(len(lens), max(lens))) * 0.125).astype(np.float32)
    vis = np.array(lens, np.int64)
    blocks, pool, cnt = C.csa2_block_pool(b, dev(s))
    rb, rp, rc = oracle.block_pool(s, vis)
    assert np.array_equal(blocks.cpu().numpy(), rb)
    assert np.array_equal(pool.cpu().numpy(), rp)
    assert np.array_equal(cnt.cpu().numpy(), rc)


@pytest.mark.parametrize("kv_fmt", [0, 1])
def test_gather_dequant_bitwise(kv_fmt):
    """kv_fmt 0: E8M0 per 32 channels; 1: the report's E4M3 per 16 channels."""
    wl = synth.config("decode_c1", n_seq=3, n=5000, Hm=16, kv_fmt=kv_fmt)
    dw = DevWorkload(wl)
    rng = np.random.default_rng(2)
    idx = np.stack([np.sort(rng.choice(5000, 512, replace=False)) for _ in range(3)]).astype(np.int32)
    idx[1, 400:] = -1
    got = C.csa2_gather_dequant(dw.batch, dw.kv, dw.kv_sc, dev(idx), kv_fmt=kv_fmt)
    assert np.array_equal(got.cpu().numpy(), oracle.gather_dequant(wl, idx))


ATTN_CASES = ["decode", "short_ctx", "ragged_t4", "swa_only", "replay", "sparse_idx", "swa_only_h64", "replay_h64",
              "decode_e4m3kv", "small_e4m3kv", "decode_swa8", "small_swa8", "replay_swa8",
              # at least 512 (row, 64-head) workgroups: one workgroup per row and 64 heads
              "rows_h64", "rows_h64_e4m3kv_swa8", "rows_h128_replay", "rows_h64_holes", "rows_h64_swa_only"]


@pytest.mark.parametrize("case", ATTN_CASES)
def test_sparse_attn_tolerance(case):
    rng = np.random.default_rng(3)
    replay = None
    if case in ("rows_h64", "rows_h64_holes"):  # 8 sequences x 65 rows, 300 entries each
        wl = synth.make_workload(case, 21, [300] * 8, 65, [(20, synth.MODE_FULL, False)], Hm=64)
    elif case == "rows_h64_e4m3kv_swa8":
        wl = synth.make_workload(case, 22, [300, 2000, 140, 700], 130, [(20, synth.MODE_FULL, False)], Hm=64,
                                 kv_fmt=1, swa_fmt=1)
    elif case == "rows_h128_replay":  # two 64-head groups per row; windows cut at the replay start
        wl = synth.make_workload(case, 23, [1500, 400], 130, [(20, synth.MODE_FULL, False)], Hm=128)
        replay = np.array([1400, 0], np.int32)
    elif case == "rows_h64_swa_only":
        wl = synth.make_workload(case, 24, [200] * 4, 130, [(0, synth.MODE_SWA_ONLY, False)], Hm=64)
    elif case == "decode":
        wl = synth.config("decode_c1", n_seq=3, n=6000, Hm=64)
    elif case == "decode_e4m3kv":  # the report's main-KV scales (E4M3 per 16 channels), big grid
        wl = synth.config("decode_c1", n_seq=3, n=6000, Hm=64, kv_fmt=1)
    elif case == "small_e4m3kv":  # the same with two pipes and split keys (a small grid)
        wl = synth.make_workload(case, 10, [3000], 1, [(20, synth.MODE_FULL, False)], Hm=16, kv_fmt=1)
    elif case == "decode_swa8":  # SWA rows in MXFP8 (E4M3, one E8M0 per 32 channels), big grid
        wl = synth.config("decode_c1", n_seq=3, n=6000, Hm=64, swa_fmt=1)
    elif case == "small_swa8":  # the same with two pipes and split keys, and the report's main-KV scales
        wl = synth.make_workload(case, 11, [3000, 90], 1, [(20, synth.MODE_FULL, False)], Hm=16, swa_fmt=1, kv_fmt=1)
    elif case == "replay_swa8":
        wl = synth.make_workload(case, 12, [2000, 300], 1, [(20, synth.MODE_FULL, False)], Hm=16, swa_fmt=1)
        replay = np.array([1950, 0], np.int32)
    elif case == "short_ctx":
        wl = synth.make_workload(case, 5, [40, 100, 1], 1, [(20, synth.MODE_FULL, False)], Hm=32)
    elif case == "ragged_t4":
        wl = synth.make_workload(case, 6, [130, 900, 3000], 4, [(20, synth.MODE_FULL, False)], Hm=16)
    elif case in ("swa_only", "swa_only_h64"):
        wl = synth.make_workload(case, 7, [2000, 300], 2, [(0, synth.MODE_SWA_ONLY, False)],
                                 Hm=64 if case.endswith("h64") else 16)
    elif case in ("replay", "replay_h64"):
        wl = synth.make_workload(case, 8, [2000, 300], 1, [(20, synth.MODE_FULL, False)],
                                 Hm=64 if case.endswith("h64") else 16)
        replay = np.array([1950, 0], np.int32)
    else:
        wl = synth.make_workload(case, 9, [5000], 1, [(20, synth.MODE_FULL, False)], Hm=16)
    dw = DevWorkload(wl)
    nq = wl.total_q
    vis = oracle.row_visible(wl)
    idx = np.full((nq, 512), -1, np.int32)
    if "swa_only" not in case:
        for r in range(nq):
            v = int(vis[r])
            m = min(v, 512)
            idx[r, :m] = np.sort(rng.choice(v, m, replace=False)) if v > 0 else []
    if case == "sparse_idx":
        idx[0, 10:300:3] = -1  # holes inside the list
    if case == "rows_h64_holes":  # holes inside the lists, some rows with no selected entry
        idx[::3, 5:250:2] = -1
        idx[1::7, :] = -1
    L, dL = wl.layers[0], dw.layers[0]
    sw = C.SwaLayout.from_workload(wl, replay_s=replay)
    assert sw.c.fmt == wl.swa_fmt
    out, lse = C.csa2_sparse_attn(dw.batch, dL["q_main"], dw.kv, dw.kv_sc, dev(idx), dL["swa"], sw, SCALE,
                                  kv_fmt=wl.kv_fmt)
    torch.cuda.synchronize()
    ro, rl = oracle.sparse_attn(wl, L.q_main, idx, L.swa, replay_s=replay)
    assert_close_attn(out.cpu().numpy(), ro, case)
    np.testing.assert_allclose(lse.cpu().numpy(), rl, rtol=1e-4, atol=1e-4)


CHAIN_CASES = {
    "c2_small": lambda: synth.config("chain_c2", n_seq=2, n=24000, Hm=16),
    "c2_small_h64": lambda: synth.config("chain_c2", n_seq=2, n=24000, Hm=64),
    # the report's main-KV scales (E4M3 per 16 channels) through Full + pool, Reindex and Reuse
    "c2_small_e4m3kv": lambda: synth.config("chain_c2", n_seq=2, n=24000, Hm=16, kv_fmt=1),
    # the pages' cache formats for main KV (E4M3 per 16 channels) and SWA (FP8, as OCP MXFP8)
    "c2_small_pages_fmt": lambda: synth.config("chain_c2", n_seq=2, n=24000, Hm=16, kv_fmt=1, swa_fmt=1),
    # the report's indexer format (MXFP4 queries and keys) through Full + pool, Reindex and Reuse
    "c2_small_mx_idx": lambda: synth.config("chain_c2", n_seq=2, n=24000, Hm=16, q_fmt=synth.Q_MXFP4),
    # every cache in the pages' format: main KV E2M1 + E4M3/16, indexer MXFP4, SWA FP8 (MXFP8)
    "c2_small_pages_all": lambda: synth.config("chain_c2", n_seq=2, n=24000, Hm=16, kv_fmt=1, swa_fmt=1,
                                               q_fmt=synth.Q_MXFP4),
    "c4_small": lambda: synth.config("ragged_c4", lengths=[4096, 5000, 17000, 33001], Hm=16),
    "c4_small_mx_idx": lambda: synth.config("ragged_c4", lengths=[4096, 5000, 17000, 33001], Hm=16,
                                            q_fmt=synth.Q_MXFP4),
    "c3_small": lambda: synth.config("prefill_c3", tokens=4000, T=96, Hm=16),
    # 520 prefill rows of 64 heads: attention with one workgroup per row and 64 heads
    "c3_rows_h64": lambda: synth.config("prefill_c3", tokens=4000, T=520, Hm=64),
    # degenerate rows: a sequence with no entries (its row attends to its
    # window alone), one with entries but no query row, and one with a
    # single entry; Full with pool, Reindex and Reuse
    "degenerate": lambda: synth.make_workload("degenerate", 0xC5A2D000, [0, 3000, 5000, 1], 1,
                                              [(20, synth.MODE_FULL, True), (24, synth.MODE_REINDEX, False),
                                               (25, synth.MODE_REUSE, False)], Hm=16,
                                              q_pos=[np.array([5]), np.array([], np.int64),
                                                     np.array([4990, 4999]), np.array([0])]),
    # decoder SWA bounded replay: the last 128 prompt tokens as FP4 query rows
    # through Full + pool, Reindex and Reuse, windows cut at the replay start
    "decoder_replay": lambda: synth.config("replay_c5", n_seq=2, n=6000, T=128, Hm=16,
                                           schedule=[(20, synth.MODE_FULL, True), (24, synth.MODE_REINDEX, False),
                                                     (25, synth.MODE_REUSE, False)]),
    # rows longer than 16,384 slots from the prefill scorers: rows of at least
    # K = 512 tiles of 64 slots take the bound from their tiles' maxima, the
    # others the chunk bounds; E4M3 queries at ratio 2 with visible counts
    # from 1 to 60,000 (32,768 is exactly 512 tiles), and FP4 replay rows over
    # 40,000 entries, whose pool selects from the 8-slot block maxima the
    # scorer writes
    "prefill_tiles_fp8": lambda: synth.make_workload("pf8tiles", 0xC5A2D002, [60000], len(_PF8_SEG_T),
                                                     [(2, synth.MODE_FULL, False), (3, synth.MODE_REUSE, False)],
                                                     ratio=2, Hm=16, q_fmt=synth.Q_FP8, q_pos=[_PF8_SEG_T]),
    "replay_tiles_fp4": lambda: synth.config("replay_c5", n_seq=1, n=40000, T=64, Hm=16,
                                             schedule=[(20, synth.MODE_FULL, True), (24, synth.MODE_REINDEX, False),
                                                       (25, synth.MODE_REUSE, False)]),
    # encoder layers 0..19 as one chain at ratio 2: layers 0-1 sliding window
    # only, then Full layers 2, 8 and 14, each with its own main KV and indexer
    # K, read by the Reuse layers after it (report 2.3.1; reading note schedule
    # table); FP4 query rows (decode) and E4M3 query rows (prefill)
    "encoder_20": lambda: synth.make_workload("enc20", 13, [3000, 9000], 2, synth.encoder_schedule(), ratio=2, Hm=16,
                                              q_pos=[np.array([5990, 5999]), np.array([17000, 17999])],
                                              own_caches=True),
    "encoder_20_fp8": lambda: synth.make_workload("enc20f8", 14, [4000], 40, synth.encoder_schedule(), ratio=2,
                                                  Hm=16, q_fmt=synth.Q_FP8, own_caches=True,
                                                  q_pos=[np.arange(7960, 8000)]),
    # the report's 32 indexer heads through the chain: the one-row and the
    # four-row scan with their fused lists, Reindex on the pool
    "c2_small_h32": lambda: synth.config("chain_c2", n_seq=2, n=24000, Hm=16, H=32),
    "c4_small_h32": lambda: synth.config("ragged_c4", lengths=[4096, 5000, 17000, 33001], Hm=16, H=32),
    # the pages' exact configuration: 32 indexer heads, E4M3/16 main KV, MXFP4
    # indexer q and K, FP8 SWA (as OCP MXFP8)
    "c2_small_pages_h32": lambda: synth.config("chain_c2", n_seq=2, n=24000, Hm=16, H=32, kv_fmt=1, swa_fmt=1,
                                               q_fmt=synth.Q_MXFP4),
    "c4_small_pages_h32": lambda: synth.config("ragged_c4", lengths=[4096, 5000, 17000, 33001], Hm=16, H=32,
                                               kv_fmt=1, swa_fmt=1, q_fmt=synth.Q_MXFP4),
    # encoder SWA bounded replay (course notes "3. 通用基础设施" §3.2.2,
    # encoder paragraph): the last 128 tokens of the cached prefix replayed
    # with a 200-token uncached suffix as E4M3 query rows through one encoder
    # group at ratio 2, every window cut at the replay start
    "encoder_replay": lambda: synth.config("encoder_replay", tokens=6000, suffix=200, Hm=16),
    # Top-K at the library's largest K (2048 entries plus the window: 34 key
    # blocks) and at small odd K, through the one-row scan with its fused
    # selection, the pool and Reindex, and the four-row scan
    "c1_k2048": lambda: synth.config("decode_c1", n_seq=3, n=40000, Hm=16, K=2048),
    "c2_k2048": lambda: synth.config("chain_c2", n_seq=2, n=24000, Hm=16, K=2048),
    "c4_k100": lambda: synth.config("ragged_c4", lengths=[4096, 5000, 17000, 33001], Hm=16, K=100),
    "c1_k17": lambda: synth.config("decode_c1", n_seq=3, n=9000, Hm=16, K=17),
    "encoder_group": lambda: synth.make_workload("enc", 12, [700, 2500], 3, [(0, synth.MODE_SWA_ONLY, False),
                                                                             (2, synth.MODE_FULL, False),
                                                                             (3, synth.MODE_REUSE, False),
                                                                             (4, synth.MODE_REINDEX, False)],
                                                 ratio=2, Hm=16,
                                                 q_pos=[np.array([1390, 1395, 1399]), np.array([4000, 4990, 4999])]),
}


@pytest.mark.parametrize("case", list(CHAIN_CASES))
def test_layer_chain_matches_oracle(case):
    wl = CHAIN_CASES[case]()
    with saved_on_failure(wl, f"chain_{case}"):
        dw = DevWorkload(wl)
        outs, (pb, pp, pc), _ = run_chain(dw)
        torch.cuda.synchronize()
        ref = oracle.layer_chain(wl)
        for o, r in zip(outs, ref):
            assert np.array_equal(o["idx"].cpu().numpy(), r["idx"]), f"layer {r['layer']} indices"
            assert_close_attn(o["out"].cpu().numpy(), r["out"], f"layer {r['layer']}")
            np.testing.assert_allclose(o["lse"].cpu().numpy(), r["lse"], rtol=1e-4, atol=1e-4)
            if "pool_pos" in r:
                assert np.array_equal(pb.cpu().numpy(), r["blocks"])
                assert np.array_equal(pp.cpu().numpy(), r["pool_pos"])
                assert np.array_equal(pc.cpu().numpy(), r["pool_count"])


@pytest.mark.parametrize("case", ["c2_small", "c4_small_pages_h32", "c3_small", "encoder_20"])
def test_reruns_are_bitwise_identical(case):
    """Two runs on the same inputs agree bit for bit: the Full layer's scores,
    every layer's indices, attention outputs and log-sum-exps, and the pool
    (no floating-point sum depends on the order in which workgroups finish)."""
    wl = CHAIN_CASES[case]()
    dw = DevWorkload(wl)
    full = next(i for i, L in enumerate(wl.layers) if L.mode == synth.MODE_FULL)
    L, dL = wl.layers[full], dw.layers[full]
    k_idx = dw.k_idx if dL["k_idx"] is None else dL["k_idx"]
    k_sc = dw.k_sc if dL["k_sc"] is None else dL["k_sc"]
    s1 = C.csa2_index_score(dw.batch, wl.H, L.q_fmt, dL["q_idx"], dL["q_sc"], dL["w"], k_idx, k_sc)
    s2 = C.csa2_index_score(dw.batch, wl.H, L.q_fmt, dL["q_idx"], dL["q_sc"], dL["w"], k_idx, k_sc)
    a, pa, _ = run_chain(dw)
    b, pb, _ = run_chain(dw)
    torch.cuda.synchronize()
    g1, g2 = s1.cpu().numpy().view(np.uint32), s2.cpu().numpy().view(np.uint32)
    for r in range(wl.total_q):  # the slots of the row's sequence (the rest of a row is not written)
        n = int(wl.n_entries[wl.row_seq[r]])
        assert np.array_equal(g1[r, :n], g2[r, :n]), f"row {r} scores"
    for x, y in zip(a, b):
        assert torch.equal(x["idx"], y["idx"]), f"layer {x['layer']} indices"
        assert torch.equal(x["out"].view(torch.int32), y["out"].view(torch.int32)), f"layer {x['layer']} output"
        assert torch.equal(x["lse"].view(torch.int32), y["lse"].view(torch.int32)), f"layer {x['layer']} lse"
    if any(L.build_pool for L in wl.layers):  # otherwise the pool outputs are never written
        for u, v in zip(pa, pb):
            assert torch.equal(u, v), "pool"


@pytest.mark.gpu
@pytest.mark.parametrize("fmt", ["default", "pages"])
def test_decode_step_40_matches_oracle(fmt):
    """One decode token through all 40 layers, as the two chains the layers
    form (the encoder layers 0..19 at ratio 2 with three Full caches, the
    decoder at ratio 1), each against the oracle; in this library's default
    formats and in the pages' exact configuration (32 indexer heads, E4M3/16
    main KV, MXFP4 indexer, FP8 SWA; report 4.2.1 and 2.4.4)."""
    kw = dict(kv_fmt=1, swa_fmt=1, q_fmt=synth.Q_MXFP4, H=32) if fmt == "pages" else {}
    for wl in synth.decode_step_40(n_seq=2, tokens=6000, Hm=16, **kw):
        with saved_on_failure(wl, f"step40_{fmt}_{wl.name}"):
            dw = DevWorkload(wl)
            outs, (pb, pp, pc), _ = run_chain(dw)
            torch.cuda.synchronize()
            ref = oracle.layer_chain(wl)
            assert [o["layer"] for o in outs] == [r["layer"] for r in ref]
            for o, r in zip(outs, ref):
                assert np.array_equal(o["idx"].cpu().numpy(), r["idx"]), f"{wl.name} layer {r['layer']} indices"
                assert_close_attn(o["out"].cpu().numpy(), r["out"], f"{wl.name} layer {r['layer']}")
                np.testing.assert_allclose(o["lse"].cpu().numpy(), r["lse"], rtol=1e-4, atol=1e-4)
                if "pool_pos" in r:
                    assert np.array_equal(pp.cpu().numpy(), r["pool_pos"])


TIE_CASES = {
    # every score 0 (all head weights 0): each chunk keeps all its positions,
    # the rows overflow the candidate list and take the exact fallback
    "all_equal_t1": dict(lens=[3, 700, 9000, 20000], T=1, heads=0),
    "all_equal_t4": dict(lens=[5, 3000, 20000], T=4, heads=0),
    # one head: few distinct scores, long runs of ties at the thresholds
    "one_head_t1": dict(lens=[3, 700, 9000, 20000], T=1, heads=1),
    "one_head_t4": dict(lens=[5, 3000, 20000], T=4, heads=1),
    # rows of at most 262,144 entries take the one-kernel selection over the
    # scan's lists: lists held in registers (up to 22,528 entries) with every
    # score tied, few distinct scores with four rows per sequence, distinct
    # scores; lists streamed from memory (more than 22,528 entries) with their
    # candidates in LDS, and with every score tied (candidates overflow LDS)
    "all_equal_fused_t1": dict(lens=[3, 700, 9000, 16384], T=1, heads=0),
    "one_head_fused_t4": dict(lens=[5, 3000, 8192], T=4, heads=1),
    "fused_h64": dict(lens=[16384, 1000], T=1, heads=64),
    "fused_stream": dict(lens=[262144, 3000], T=1, heads=64),
    "all_equal_long": dict(lens=[40000, 100], T=1, heads=0),
    # longer rows: the lists are filtered by many workgroups first, from the
    # scan's histograms (a row of 74 chunks, and heavy ties)
    "split_topk": dict(lens=[300000, 5000], T=1, heads=64),
    "all_equal_split": dict(lens=[270000, 100], T=1, heads=0),
}


@pytest.mark.parametrize("case", list(TIE_CASES))
def test_layer_chain_ties(case):
    c = TIE_CASES[case]
    wl = synth.make_workload(case, 0xC5A2E000 + len(case), c["lens"], c["T"],
                             [(20, synth.MODE_FULL, True), (24, synth.MODE_REINDEX, False), (25, synth.MODE_REUSE, False)],
                             Hm=16)
    for L in wl.layers:
        if L.w is not None:
            L.w[:, c["heads"]:] = 0.0
    dw = DevWorkload(wl)
    outs, (pb, pp, pc), _ = run_chain(dw)
    torch.cuda.synchronize()
    ref = oracle.layer_chain(wl)
    for o, r in zip(outs, ref):
        assert np.array_equal(o["idx"].cpu().numpy(), r["idx"]), f"layer {r['layer']} indices"
        assert_close_attn(o["out"].cpu().numpy(), r["out"], f"layer {r['layer']}")
        if "pool_pos" in r:
            assert np.array_equal(pb.cpu().numpy(), r["blocks"])
            assert np.array_equal(pp.cpu().numpy(), r["pool_pos"])
            assert np.array_equal(pc.cpu().numpy(), r["pool_count"])


PREFILL_TIE_CASES = {
    # the prefill scorers' tile bound under ties: one head (few distinct
    # scores, long runs of ties at the bound) and none (every score 0: the
    # bound falls in bin 0 and is not used), E4M3 rows at ratio 2 on both
    # sides of the K-tile boundary and FP4 replay rows over 40,000 entries
    "fp8_one_head": dict(fp8=True, heads=1),
    "fp8_all_equal": dict(fp8=True, heads=0),
    "fp4_one_head": dict(fp8=False, heads=1),
    # head weights of both signs, every third row all negative (its tile
    # maxima lie in bin 0, so its bound is the chunk bounds'), and K = 1,024
    # (a row needs 1,024 tiles, 65,536 slots, for the tile bound)
    "fp8_negative_weights": dict(fp8=True, heads=64, negw=True),
    "fp8_k1024": dict(fp8=True, heads=64, K=1024, n=80000),
}


@pytest.mark.parametrize("case", list(PREFILL_TIE_CASES))
def test_layer_chain_prefill_tile_ties(case):
    c = PREFILL_TIE_CASES[case]
    if c["fp8"]:
        n = c.get("n", 60000)  # visible counts (t + 1) / 2 up to 60,000 of the n entries
        wl = synth.make_workload("pf8ties_" + case, 0xC5A2D010 + len(case), [n], len(_PF8_SEG_T),
                                 [(2, synth.MODE_FULL, False), (3, synth.MODE_REUSE, False)], ratio=2, Hm=16,
                                 K=c.get("K", 512), q_fmt=synth.Q_FP8,
                                 q_pos=[_PF8_SEG_T + 2 * (n - 60000)])
    else:
        wl = synth.config("replay_c5", n_seq=1, n=40000, T=64, Hm=16, seed=0xC5A2D020,
                          schedule=[(20, synth.MODE_FULL, True), (24, synth.MODE_REINDEX, False),
                                    (25, synth.MODE_REUSE, False)])
    for L in wl.layers:
        if L.w is not None:
            L.w[:, c["heads"]:] = 0.0
            if c.get("negw"):
                L.w[:] = L.w * 2.0 - 1.0
                L.w[::3] = -np.abs(L.w[::3])
    with saved_on_failure(wl, "prefill_ties_" + case):
        dw = DevWorkload(wl)
        outs, (pb, pp, pc), _ = run_chain(dw)
        torch.cuda.synchronize()
        ref = oracle.layer_chain(wl)
        for o, r in zip(outs, ref):
            assert np.array_equal(o["idx"].cpu().numpy(), r["idx"]), f"layer {r['layer']} indices"
            assert_close_attn(o["out"].cpu().numpy(), r["out"], f"layer {r['layer']}")
            if "pool_pos" in r:
                assert np.array_equal(pb.cpu().numpy(), r["blocks"])
                assert np.array_equal(pp.cpu().numpy(), r["pool_pos"])
                assert np.array_equal(pc.cpu().numpy(), r["pool_count"])


NEGW_CASES = {
    # head weights of both signs (U(-1, 1)); every third row all negative, so
    # all of its scores are <= 0 and its threshold lies in bin 0
    "fused_t1": dict(lens=[3, 700, 9000, 20000, 70000], T=1),
    "t4": dict(lens=[5, 3000, 20000, 40000], T=4),
    "split": dict(lens=[300000, 5000], T=1),
}


@pytest.mark.parametrize("case", list(NEGW_CASES))
def test_layer_chain_negative_weights(case):
    """Negative head weights give negative scores; the Top-K, the block pool
    and Reindex order them by value (scan lists, the one-kernel and the split
    selection from lists, pool and Reindex rows)."""
    c = NEGW_CASES[case]
    wl = synth.make_workload("negw_" + case, 0xC5A2B000 + len(case), c["lens"], c["T"],
                             [(20, synth.MODE_FULL, True), (24, synth.MODE_REINDEX, False), (25, synth.MODE_REUSE, False)],
                             Hm=16)
    for L in wl.layers:
        if L.w is not None:
            L.w[:] = L.w * 2.0 - 1.0
            L.w[::3] = -np.abs(L.w[::3])
    dw = DevWorkload(wl)
    outs, (pb, pp, pc), _ = run_chain(dw)
    torch.cuda.synchronize()
    ref = oracle.layer_chain(wl)
    assert (ref[0]["scores"][np.isfinite(ref[0]["scores"])] < 0).any()
    for o, r in zip(outs, ref):
        assert np.array_equal(o["idx"].cpu().numpy(), r["idx"]), f"layer {r['layer']} indices"
        assert_close_attn(o["out"].cpu().numpy(), r["out"], f"layer {r['layer']}")
        if "pool_pos" in r:
            assert np.array_equal(pb.cpu().numpy(), r["blocks"])
            assert np.array_equal(pp.cpu().numpy(), r["pool_pos"])
            assert np.array_equal(pc.cpu().numpy(), r["pool_count"])


def test_layer_chain_hot_region():
    """A row whose Top-K lies in two adjacent chunks: the keys of positions
    [40960, 49152) of the first sequence get their E8M0 scale raised by 2 (their
    scores times 4), so each of those chunks' lists holds at least K entries
    above every other chunk's bound, more than the gathered candidates of one
    filter workgroup may hold: that row is selected from the lists, the other
    sequence's rows from the gathered candidates, in the same launch."""
    wl = synth.make_workload("hot_region", 0xC5A2D001, [131072, 131072], 1,
                             [(20, synth.MODE_FULL, True), (24, synth.MODE_REINDEX, False), (25, synth.MODE_REUSE, False)],
                             Hm=16)
    seen = set()
    for ks in [wl.k_sc] + [L.k_sc for L in wl.layers]:
        if ks is not None and id(ks) not in seen:
            seen.add(id(ks))
            ks[40960:49152] += 2
    dw = DevWorkload(wl)
    outs, (pb, pp, pc), _ = run_chain(dw)
    torch.cuda.synchronize()
    ref = oracle.layer_chain(wl)
    hot = ref[0]["idx"][0]
    assert ((hot >= 40960) & (hot < 49152)).all(), "the first row's Top-K lies in the raised region"
    for o, r in zip(outs, ref):
        assert np.array_equal(o["idx"].cpu().numpy(), r["idx"]), f"layer {r['layer']} indices"
        assert_close_attn(o["out"].cpu().numpy(), r["out"], f"layer {r['layer']}")
        if "pool_pos" in r:
            assert np.array_equal(pb.cpu().numpy(), r["blocks"])
            assert np.array_equal(pp.cpu().numpy(), r["pool_pos"])
            assert np.array_equal(pc.cpu().numpy(), r["pool_count"])


def test_layer_chain_equals_composition():
    """The chain's indices and outputs equal those of the individual calls."""
    wl = synth.config("chain_c2", n_seq=2, n=20000, Hm=16,
                      schedule=[(20, synth.MODE_FULL, True), (21, synth.MODE_REUSE, False),
                                (24, synth.MODE_REINDEX, False)])
    dw = DevWorkload(wl)
    outs, (pb, pp, pc), _ = run_chain(dw)
    b = dw.batch
    f, r = dw.layers[0], dw.layers[2]
    sc = C.csa2_index_score(b, 64, 0, f["q_idx"], f["q_sc"], f["w"], dw.k_idx, dw.k_sc)
    idx20 = C.csa2_topk(b, sc, 512)
    blocks, pool, cnt = C.csa2_block_pool(b, sc)
    psc = C.csa2_index_score(b, 64, 0, r["q_idx"], r["q_sc"], r["w"], dw.k_idx, dw.k_sc, cand=pool)
    idx24 = C.csa2_topk(b, psc, 512, cand=pool, cand_count=cnt)
    o20, _ = C.csa2_sparse_attn(b, f["q_main"], dw.kv, dw.kv_sc, idx20, f["swa"], dw.swa, SCALE)
    o21, _ = C.csa2_sparse_attn(b, dw.layers[1]["q_main"], dw.kv, dw.kv_sc, idx20, dw.layers[1]["swa"], dw.swa, SCALE)
    o24, _ = C.csa2_sparse_attn(b, r["q_main"], dw.kv, dw.kv_sc, idx24, r["swa"], dw.swa, SCALE)
    torch.cuda.synchronize()
    assert torch.equal(outs[0]["idx"], idx20) and torch.equal(outs[2]["idx"], idx24)
    assert torch.equal(pp, pool) and torch.equal(pc, cnt) and torch.equal(pb, blocks)
    assert torch.equal(outs[0]["out"], o20) and torch.equal(outs[1]["out"], o21) and torch.equal(outs[2]["out"], o24)


@pytest.mark.gpu
@pytest.mark.parametrize("kv_fmt", [0, 1])
@pytest.mark.parametrize("n", [1, 5, 3000, 131072])
def test_kv_append_bitwise(kv_fmt, n):
    """The cache append (RoPE on the last 64 channels, then quantisation)
    equals the oracle bit for bit: latents of three magnitudes, an all-zero
    block and a saturating one, random angles, rows written out of order into
    a larger cache whose other rows keep their contents.  131,072 entries is
    one source layer's cache of the prefill context at ratio 2."""
    rng = np.random.default_rng(1000 + n + kv_fmt)
    x = (rng.standard_normal((n, 512), dtype=np.float32) * rng.choice([1e-3, 1.0, 40.0], size=(n, 1))).astype(np.float32)
    if n >= 5:
        x[2, :64] = 0.0
        x[3, 100:140] = 7000.0
    th = rng.uniform(-np.pi, np.pi, size=(n, 32))
    cs = np.stack([np.cos(th), np.sin(th)], -1).astype(np.float32)
    rows = n + 7
    dst = rng.permutation(rows)[:n].astype(np.int64)
    ref_kv, ref_sc = oracle.kv_append(x, cs, dst, kv_fmt, rows)
    nsc = 32 if kv_fmt == 1 else 16
    kv = torch.full((rows, 256), 0xAB, dtype=torch.uint8, device="cuda")
    sc = torch.full((rows, nsc), 0xCD, dtype=torch.uint8, device="cuda")
    C.csa2_kv_append(dev(x), dev(cs), dev(dst), kv, sc, kv_fmt=kv_fmt)
    torch.cuda.synchronize()
    got_kv, got_sc = kv.cpu().numpy(), sc.cpu().numpy()
    assert np.array_equal(got_kv[dst], ref_kv[dst])
    assert np.array_equal(got_sc[dst], ref_sc[dst])
    untouched = np.setdiff1d(np.arange(rows), dst)
    assert np.all(got_kv[untouched] == 0xAB) and np.all(got_sc[untouched] == 0xCD)
    # a destination outside the cache is skipped; the rest are written as before
    if n >= 5:
        bad = dst.copy()
        bad[1] = rows + 3
        kv2 = torch.zeros_like(kv)
        sc2 = torch.zeros_like(sc)
        C.csa2_kv_append(dev(x), dev(cs), dev(bad), kv2, sc2, kv_fmt=kv_fmt)
        torch.cuda.synchronize()
        keep = np.delete(np.arange(n), 1)
        assert np.array_equal(kv2.cpu().numpy()[dst[keep]], ref_kv[dst[keep]])
        assert not kv2.cpu().numpy()[dst[1]].any()


COMPOSE_CASES = {
    "default": dict(),
    # the report's formats: E4M3/16 main KV, MXFP4 indexer K and queries, 32 heads
    "pages": dict(kv_fmt=1, q_fmt=synth.Q_MXFP4, H=32),
}


@pytest.mark.gpu
@pytest.mark.parametrize("case", list(COMPOSE_CASES))
def test_write_path_feeds_the_chain(case):
    """The write path composed and read back: tokens -> csa2_compress (m = 2)
    -> csa2_kv_append and csa2_index_k_project, both from the entries before
    RoPE with the same angles -> the caches one encoder group (Full, Reuse,
    Reindex) scores, selects and attends over.  Each channel's compression
    weights are equal over its two tokens or leave one token's weight below
    float32's range, so the compressor is exact on both sides; the caches then
    equal the oracle's bit for bit, and the chain run on the GPU-written caches
    equals the oracle's chain on its own (indices exact, attention within the
    attention tolerance)."""
    kw = COMPOSE_CASES[case]
    wl = synth.make_workload("compose", 13, [700, 2500], 3, [(2, synth.MODE_FULL, False),
                                                             (3, synth.MODE_REUSE, False),
                                                             (4, synth.MODE_REINDEX, False)],
                             ratio=2, Hm=16, q_pos=[np.array([1390, 1395, 1399]), np.array([4000, 4990, 4999])],
                             **kw)
    n, m = int(wl.entry_off[-1]), 2
    rng = np.random.default_rng(77 + len(case))
    c_tok = (rng.standard_normal((n * m, 512)) * rng.choice([0.05, 1.0, 8.0], size=(n * m, 1))).astype(np.float32)
    z_tok = np.zeros((n, m, 512), np.float32)
    pick = rng.integers(0, 3, size=(n, 512))  # 0: equal weights, 1 or 2: that token alone
    z_tok[:, 0][pick == 1] = 200.0
    z_tok[:, 1][pick == 2] = 200.0
    z_tok = z_tok.reshape(n * m, 512)
    th = rng.uniform(-np.pi, np.pi, size=(n, 32))
    cs = np.stack([np.cos(th), np.sin(th)], -1).astype(np.float32)
    W = (rng.standard_normal((512, 128)) * 0.05).astype(np.float32)
    dst = np.arange(n, dtype=np.int64)
    kv_fmt = getattr(wl, "kv_fmt", 0)
    k_fmt = 1 if kw.get("q_fmt") == synth.Q_MXFP4 else 0

    x = C.csa2_compress(dev(c_tok), dev(z_tok), m)
    kv = torch.zeros(wl.kv.shape, dtype=torch.uint8, device="cuda")
    kv_sc = torch.zeros(wl.kv_sc.shape, dtype=torch.uint8, device="cuda")
    k_idx = torch.zeros(wl.k_idx.shape, dtype=torch.uint8, device="cuda")
    k_sc = torch.zeros(wl.k_sc.shape, dtype=torch.uint8, device="cuda")
    C.csa2_kv_append(x, dev(cs), dev(dst), kv, kv_sc, kv_fmt=kv_fmt)
    C.csa2_index_k_project(x, dev(W), dev(dst), k_idx, k_sc, q_fmt=kw.get("q_fmt", synth.Q_FP4), rope_cs=dev(cs))

    xr = oracle.compress(c_tok, z_tok, m)
    assert np.array_equal(x.cpu().numpy(), xr)
    ref_kv, ref_kv_sc = oracle.kv_append(xr, cs, dst, kv_fmt, n)
    ref_k, ref_k_sc = oracle.index_k_project(xr, W, dst, k_fmt, n, cs=cs)
    for got, want, what in ((kv, ref_kv, "kv"), (kv_sc, ref_kv_sc, "kv_sc"), (k_idx, ref_k, "k_idx"),
                            (k_sc, ref_k_sc, "k_sc")):
        assert np.array_equal(got.cpu().numpy(), want.reshape(got.shape)), what

    wl.kv, wl.kv_sc, wl.k_idx, wl.k_sc = ref_kv, ref_kv_sc, ref_k, ref_k_sc.reshape(wl.k_sc.shape)
    dw = DevWorkload(wl)
    dw.kv, dw.kv_sc, dw.k_idx, dw.k_sc = kv, kv_sc, k_idx, k_sc  # the chain reads what the GPU wrote
    outs, _, _ = run_chain(dw)
    torch.cuda.synchronize()
    ref = oracle.layer_chain(wl)
    for o, r in zip(outs, ref):
        assert np.array_equal(o["idx"].cpu().numpy(), r["idx"]), f"layer {r['layer']} indices"
        assert_close_attn(o["out"].cpu().numpy(), r["out"], f"layer {r['layer']}")
        np.testing.assert_allclose(o["lse"].cpu().numpy(), r["lse"], rtol=1e-4, atol=1e-4)


@pytest.mark.parametrize("m,n", [(1, 7), (2, 1), (2, 4099), (4, 300), (2, 131072)])
def test_compress_tolerance(m, n):
    """The compressor against the oracle (float64), within a bound derived
    from its float32 arithmetic: an exp of at most a few units in the last
    place, m products and sums, one division; 2e-6 of the weighted magnitude.
    131,072 entries at m = 2 is the 262,144-token prefill context."""
    rng = np.random.default_rng(3000 + 7 * m + n)
    c = rng.standard_normal((n * m, 512), dtype=np.float32) * np.float32(3.0)
    z = rng.standard_normal((n * m, 512), dtype=np.float32) * np.float32(4.0)
    if n > 2:
        z[:m, :8] = 80.0  # equal, large weights in one entry's first channels
    ref = oracle.compress(c, z, m)
    got = C.csa2_compress(dev(c), dev(z), m).cpu().numpy()
    zz = z.reshape(n, m, 512).astype(np.float64)
    w = np.exp(zz - zz.max(1, keepdims=True))
    mag = (w * np.abs(c.reshape(n, m, 512))).sum(1) / w.sum(1)
    assert np.all(np.abs(got.astype(np.float64) - ref) <= 2e-6 * mag + 1e-30)


@pytest.mark.parametrize("rope", [False, True])
@pytest.mark.parametrize("q_fmt", [synth.Q_FP4, synth.Q_MXFP4])
@pytest.mark.parametrize("n", [1, 17, 5000, 131072])
def test_index_k_project_bitwise(q_fmt, n, rope):
    """The indexer-K projection equals the oracle bit for bit (same float32
    multiply-add chain, same quantiser), rows written out of order, from the
    entry after RoPE or, given its angles, before it.  At 131,072 entries (one
    source layer of the prefill context) the GPU writes every row and the
    oracle checks 3,000 sampled ones."""
    rng = np.random.default_rng(4000 + n + q_fmt + 7 * rope)
    x = rng.standard_normal((n, 512), dtype=np.float32) * np.float32(3.0)
    if n >= 17:
        x[5] = 0.0  # an all-zero row: scale 2^0, codes 0
    W = rng.standard_normal((512, 128), dtype=np.float32) * np.float32(0.05)
    rows = n + 3
    dst = rng.permutation(rows)[:n].astype(np.int64)
    kf = torch.full((rows, 64), 0xAB, dtype=torch.uint8, device="cuda")
    ks = torch.full((rows, 4) if q_fmt == synth.Q_MXFP4 else (rows,), 0xCD, dtype=torch.uint8, device="cuda")
    cs = None
    if rope:
        th = rng.uniform(-np.pi, np.pi, size=(n, 32))
        cs = np.stack([np.cos(th), np.sin(th)], -1).astype(np.float32)
    C.csa2_index_k_project(dev(x), dev(W), dev(dst), kf, ks, q_fmt=q_fmt, rope_cs=dev(cs))
    torch.cuda.synchronize()
    k_fmt = 1 if q_fmt == synth.Q_MXFP4 else 0
    sel = np.arange(n) if n <= 5000 else np.sort(rng.choice(n, 3000, replace=False))
    ref_f, ref_s = oracle.index_k_project(x[sel], W, dst[sel], k_fmt, rows, cs=None if cs is None else cs[sel])
    got_f, got_s = kf.cpu().numpy(), ks.cpu().numpy()
    assert np.array_equal(got_f[dst[sel]], ref_f[dst[sel]])
    assert np.array_equal(got_s[dst[sel]], ref_s[dst[sel]])
    untouched = np.setdiff1d(np.arange(rows), dst)
    assert np.all(got_f[untouched] == 0xAB)


@pytest.mark.parametrize("inverse", [False, True])
@pytest.mark.parametrize("n,heads", [(1, 1), (7, 64), (2048, 64)])
def test_rope_cast_bitwise(n, heads, inverse):
    """RoPE and cast around attention equal the oracle bit for bit: random
    rows of three magnitudes, random angles, both directions.  2,048 rows of
    64 heads is the query block of the 128-token replay over 16 sequences."""
    rng = np.random.default_rng(5000 + n + heads + inverse)
    x = rng.standard_normal((n, heads, 512), dtype=np.float32) * rng.choice([1e-3, 1.0, 50.0], size=(n, 1, 1)).astype(np.float32)
    th = rng.uniform(-np.pi, np.pi, size=(n, 32))
    cs = np.stack([np.cos(th), np.sin(th)], -1).astype(np.float32)
    got = C.csa2_rope_cast(dev(x), dev(cs), inverse=inverse).cpu().numpy()
    assert np.array_equal(got, oracle.rope_cast(x, cs, inverse))


def test_rope_cast_specials_bitwise():
    """NaNs (quiet and signalling), infinities, the largest float32 and ties
    around the largest bf16, in the channels that are only cast: equal to the
    oracle bit for bit (NaNs stay NaNs, overflow gives infinity)."""
    from test_oracle_pins import BF16_SPECIAL
    x = np.random.default_rng(77).standard_normal((3, 4, 512), dtype=np.float32)
    bits = np.array([b for b, _ in BF16_SPECIAL], np.uint32)
    x[:, :, : len(bits)] = bits.view(np.float32)
    th = np.random.default_rng(78).uniform(-np.pi, np.pi, size=(3, 32))
    cs = np.stack([np.cos(th), np.sin(th)], -1).astype(np.float32)
    got = C.csa2_rope_cast(dev(x), dev(cs)).cpu().numpy()
    assert np.array_equal(got, oracle.rope_cast(x, cs, False))
    assert [int(v) for v in got[0, 0, : len(bits)]] == [w for _, w in BF16_SPECIAL]


ROPE_CASES = {
    # 3 rows of 64 heads: the 16-head kernel with its keys split and merged
    "decode_split": lambda: synth.config("decode_c1", n_seq=3, n=6000, Hm=64),
    # the same without a workspace: no split, the kernel stores the output itself
    "decode_nosplit": lambda: synth.config("decode_c1", n_seq=3, n=6000, Hm=64),
    # one row of 16 heads: two pipes per workgroup
    "two_pipes_e4m3kv_swa8": lambda: synth.make_workload("rp2", 31, [3000], 1, [(20, synth.MODE_FULL, False)], Hm=16,
                                                        kv_fmt=1, swa_fmt=1),
    # 520 rows of 64 heads: one workgroup per row and 64 heads
    "rows": lambda: synth.make_workload("rprows", 32, [300] * 8, 65, [(20, synth.MODE_FULL, False)], Hm=64),
    "rows_e4m3kv_swa8": lambda: synth.make_workload("rprows8", 33, [300] * 4, 130, [(20, synth.MODE_FULL, False)],
                                                    Hm=64, kv_fmt=1, swa_fmt=1),
}


@pytest.mark.parametrize("case", list(ROPE_CASES))
def test_sparse_attn_rope_equals_composition(case):
    """csa2_sparse_attn_rope on a bf16 query before RoPE equals csa2_rope_cast
    (of the query widened to f32) -> csa2_sparse_attn -> csa2_rope_cast
    (inverse) bit for bit (output and log-sum-exp), and the oracle's
    composition within the attention tolerance plus the bf16 cast."""
    wl = ROPE_CASES[case]()
    dw = DevWorkload(wl)
    nq, Hm = wl.total_q, wl.Hm
    rng = np.random.default_rng(600 + len(case))
    vis = oracle.row_visible(wl)
    idx = np.full((nq, 512), -1, np.int32)
    for r in range(nq):
        m = min(int(vis[r]), 512)
        idx[r, :m] = np.sort(rng.choice(int(vis[r]), m, replace=False))
    # the query before RoPE in bf16
    q16 = (rng.standard_normal((nq, Hm, 512), dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
    q32 = (q16.astype(np.uint32) << 16).view(np.float32)
    th = rng.uniform(-np.pi, np.pi, size=(nq, 32))
    cs = np.stack([np.cos(th), np.sin(th)], -1).astype(np.float32)
    dq, dq32, dcs, didx = dev(q16), dev(q32), dev(cs), dev(idx)
    L, dL = wl.layers[0], dw.layers[0]
    split = case != "decode_nosplit"
    qb = C.csa2_rope_cast(dq32, dcs)
    o32, l1 = C.csa2_sparse_attn(dw.batch, qb, dw.kv, dw.kv_sc, didx, dL["swa"], dw.swa, SCALE, kv_fmt=wl.kv_fmt,
                                 split=split)
    want = C.csa2_rope_cast(o32, dcs, inverse=True)
    got, l2 = C.csa2_sparse_attn_rope(dw.batch, dq, dcs, dw.kv, dw.kv_sc, didx, dL["swa"], dw.swa, SCALE,
                                      kv_fmt=wl.kv_fmt, split=split)
    torch.cuda.synchronize()
    assert torch.equal(got, want), f"{case}: {(got != want).sum().item()} output values differ"
    assert torch.equal(l1, l2)
    # against the oracle: its query cast, attention and cast back
    qref = oracle.rope_cast(q32, cs, False)
    ro, _ = oracle.sparse_attn(wl, qref, idx, L.swa)
    ref = (oracle.rope_cast(ro, cs, True).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    g = (got.cpu().numpy().astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.all(np.abs(g - ref) <= 2e-3 + 1.2e-2 * np.abs(ref)), f"{case}: max abs err {np.abs(g - ref).max():.3e}"
