"""Pins against values the pages print: the fixtures under tests/golden/ hold
them as data, each file naming the passage it copies.  The path's sizes and the
layer schedule come from the report "DeepSeek-V4.1-Flash: Pushing the Limits of
KV Cache Compression" (sections 4.2.1 and 2.3.2) and the reading note "DeepSeek
V4.1 Flash: Pushing the Limits of KV Cache Compression" (mode and search
tables); the byte ledger comes from that reading note's section on the 890
bytes and from the report's section 2.4.4."""
import inspect
import json
import math
import os

import numpy as np

import oracle
import synth
from synth import MODE_FULL, MODE_REINDEX, MODE_REUSE

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
MODES = {"full": MODE_FULL, "reindex": MODE_REINDEX, "reuse": MODE_REUSE}


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_decoder_schedule_matches_pages():
    cfg = golden("pages_config.json")["decoder"]
    first, last = cfg["layers"]
    sched = synth.decoder_schedule(first, last)
    assert [l for l, _, _ in sched] == list(range(first, last + 1))
    for i, (l, mode, pool) in enumerate(sched):
        group, pos = divmod(i, cfg["group_size"])
        want = (cfg["first_group"] if group == 0 else cfg["other_groups"])[pos]
        assert mode == MODES[want], l
        assert pool == (i == 0), l  # the pool comes from the first decoder Full layer
    # the decode chains run exactly this schedule at the decoder's ratio
    for name in ("chain_c2", "ragged_c4"):
        kw = {"n_seq": 1, "n": 256} if name == "chain_c2" else {"n_seq": 1, "lengths": [256]}
        wl = synth.config(name, **kw)
        assert [(L.index, L.mode, L.build_pool) for L in wl.layers] == sched
        assert wl.ratio == cfg["ratio"]


def test_encoder_group_matches_pages():
    cfg = golden("pages_config.json")["encoder"]
    lo, hi = cfg["csa2_layers"]
    assert (hi - lo + 1) % cfg["group_size"] == 0
    wl = synth.config("prefill_c3", tokens=512, T=8)
    assert [L.mode for L in wl.layers] == [MODES[m] for m in cfg["group"]]
    assert wl.layers[0].index == lo  # the first group starts at the first CSA2 encoder layer
    assert wl.ratio == cfg["ratio"]
    assert not any(L.build_pool for L in wl.layers)  # encoder Full layers build no pool


def test_forty_layer_step_matches_pages():
    """The encoder schedule and the 40-layer decode step: layers 0..39 once each,
    the pure sliding-window layers first, the encoder groups at ratio 2 over
    half the tokens, the decoder at ratio 1 over all of them."""
    cfg = golden("pages_config.json")
    enc = cfg["encoder"]
    sched = synth.encoder_schedule()
    assert [l for l, _, _ in sched] == list(range(0, enc["csa2_layers"][1] + 1))
    assert [l for l, m, _ in sched if m == synth.MODE_SWA_ONLY] == enc["pure_swa_layers"]
    csa2 = [(l, m) for l, m, _ in sched if m != synth.MODE_SWA_ONLY]
    for i, (l, m) in enumerate(csa2):
        assert m == MODES[enc["group"][i % enc["group_size"]]], l
    assert not any(p for _, _, p in sched)
    tokens = 1000
    wls = synth.decode_step_40(n_seq=2, tokens=tokens, Hm=16)
    layers = [L.index for wl in wls for L in wl.layers]
    assert layers == list(range(40))
    for wl in wls:
        dec = wl.layers[0].index >= cfg["decoder"]["layers"][0]
        assert wl.ratio == (cfg["decoder"]["ratio"] if dec else enc["ratio"])
        assert list(wl.n_entries) == [tokens if dec else tokens // 2] * 2
        assert list(wl.q_pos) == [tokens - 1] * 2
    # the encoder layers form one chain in which every group's Full layer
    # carries its own source cache
    assert len(wls) == 2
    fulls = [L for L in wls[0].layers if L.mode == synth.MODE_FULL]
    assert [L.index for L in fulls] == [2, 8, 14]
    assert len({L.k_idx.tobytes() for L in fulls}) == 3 and len({L.kv.tobytes() for L in fulls}) == 3


def test_path_sizes_match_pages():
    cfg = golden("pages_config.json")
    wl = synth.config("decode_c0", n_entries=[64])
    assert wl.K == cfg["attention_topk"]
    assert wl.W == cfg["swa_window"]
    assert wl.block == cfg["block_positions"] and wl.max_blocks == cfg["max_blocks"]
    assert cfg["block_positions"] * cfg["max_blocks"] == cfg["max_pool_positions"]
    assert wl.Hm == cfg["main_query_heads"]
    # packed E2M1 rows: two channels per byte
    assert wl.k_idx.shape[1] * 2 == cfg["indexer_head_dim"]
    assert wl.kv.shape[1] * 2 == cfg["main_head_dim"]
    assert wl.layers[0].q_main.shape[-1] == cfg["main_head_dim"]
    # the oracle's block pool defaults to the pages' blocks
    sig = inspect.signature(oracle.block_pool).parameters
    assert sig["block"].default == cfg["block_positions"] and sig["max_blocks"].default == cfg["max_blocks"]
    # the pages' 32 indexer heads (the workloads default to 64): the oracle scores them
    wl32 = synth.config("decode_c0", n_entries=[64], H=cfg["indexer_query_heads"])
    L = wl32.layers[0]
    assert L.q_idx.shape[1] == cfg["indexer_query_heads"]
    s = oracle.index_score(wl32, L.q_idx, L.q_sc, L.w, L.q_fmt)
    assert s.shape == (1, 64) and np.all(np.isfinite(s)) and np.all(s >= 0)


def test_cache_ledger_matches_pages():
    g = golden("cache_ledger.json")
    bp = g["bytes_per_position"]
    parts = [bp["main_latent_fp4_values"], bp["main_latent_scales_one_per_16_channels"], bp["indexer_k_fp4_values"],
             bp["indexer_k_scales_one_per_32_channels"]]
    # each entry from its channel count, as the ledger derives it
    assert parts == [512 // 2, 512 // 16, 128 // 2, 128 // 32]
    assert sum(parts) == bp["total"]
    from compressed_sparse_attention_amd import ledger
    assert ledger.bytes_per_position("pages") == bp["total"]
    src = g["source_layers"]
    per_token = bp["total"] * (src["encoder_half_length"] / 2 + src["decoder_full_length"])
    assert per_token == g["bytes_per_token"] == ledger.bytes_per_token("pages")
    assert round(g["bytes_per_token"] * g["one_sequence_tokens"] / 2 ** 30, 2) == g["one_sequence_gib_approx"]
    fm = g["main_kv_format_max_magnitude"]
    # the oracle's decoders reach exactly the format maxima the report multiplies
    assert max(abs(oracle.e2m1(c)) for c in range(16)) == fm["e2m1_max"]
    e4 = [oracle.e4m3(c) for c in range(256)]
    assert max(abs(v) for v in e4 if math.isfinite(v)) == fm["e4m3_scale_max"]
    assert fm["e4m3_scale_max"] * fm["e2m1_max"] == fm["product"]
    assert round(math.sqrt(512), 1) == g["latent_l2_bound_sqrt_512_approx"]
