"""Pins for the CPU oracle: every check compares the oracle with something other
than itself -- the format tables of the OCP MX v1.0 spec, closed forms, exact
rational arithmetic, brute force through a different library (numpy / torch),
and the invariants the pages fix (Top-K inside the block pool, Reindex with the
Full layer's own query, Reuse = re-gather, sparse = dense when Top-K covers the
visible range, SWA-only layers, compression ratio 2 visibility).

Pages: the report "DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache
Compression" (sections 2.3, 2.3.1, 2.3.2, 2.4.4, 4.2.1), the reading note
"DeepSeek V4.1 Flash: Pushing the Limits of KV Cache Compression" (mode,
schedule and search/read tables; the 890-byte ledger) and the course notes
"3. 通用基础设施" (section 3.2.2, SWA window equation).
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from synth import MODE_FULL, MODE_REINDEX, MODE_REUSE, MODE_SWA_ONLY, Q_FP4, Q_FP8, Q_MXFP4, Layer, Workload

# ---------------------------------------------------------------------------
# helpers (encoders written from the spec; independent of the oracle)
# ---------------------------------------------------------------------------

# OCP MX v1.0, E2M1 element encodings: magnitude codes 0..7 -> these values.
E2M1_SPEC = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
E2M1_CODE = {v: i for i, v in enumerate(E2M1_SPEC)}


def fp4_code(v):
    return E2M1_CODE[abs(v)] | (8 if v < 0 else 0)


def pack_fp4(vals):
    """Values on the E2M1 grid -> packed bytes, element 2i in the low nibble."""
    codes = [fp4_code(v) for v in vals]
    return np.array([codes[2 * i] | (codes[2 * i + 1] << 4) for i in range(len(codes) // 2)], np.uint8)


def rne_f32(x: Fraction) -> float:
    """Round an exact rational to the nearest binary32 (ties to even)."""
    if x == 0:
        return 0.0
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    q = Fraction(2) ** (e - 23)
    m = a / q
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return float(sign * fl * q)


def tiny_workload(n_entries, q_pos, ratio=1, H=1, Hm=1, K=512, W=128, block=8, max_blocks=2048):
    """A workload skeleton with hand-filled caches (one sequence per n_entries item)."""
    n_entries = np.asarray(n_entries, np.int64)
    entry_off = np.zeros(len(n_entries) + 1, np.int64)
    entry_off[1:] = np.cumsum(n_entries)
    q_pos_all = np.concatenate([np.asarray(p, np.int64) for p in q_pos]).astype(np.int32)
    q_off = np.zeros(len(n_entries) + 1, np.int32)
    q_off[1:] = np.cumsum([len(p) for p in q_pos])
    row_seq = np.repeat(np.arange(len(n_entries), dtype=np.int32), [len(p) for p in q_pos])
    swa_pos0 = np.array([max(0, int(min(p)) - W + 1) for p in q_pos], np.int32)
    swa_len = np.array([int(max(p)) - s + 1 for p, s in zip(q_pos, swa_pos0)], np.int32)
    swa_row_off = np.zeros(len(n_entries), np.int64)
    swa_row_off[1:] = np.cumsum(swa_len)[:-1]
    tot = int(entry_off[-1])
    wl = Workload("tiny", 0, ratio, H, Hm, K, W, block, max_blocks, n_entries, entry_off, q_off, q_pos_all,
                  row_seq, swa_row_off, swa_pos0, swa_len)
    wl.k_idx = np.zeros((tot, 64), np.uint8)
    wl.k_sc = np.full(tot, 127, np.uint8)
    wl.kv = np.zeros((tot, 256), np.uint8)
    wl.kv_sc = np.full((tot, 16), 127, np.uint8)
    return wl


def decode_kv(wl):
    """Main KV as float64 from the spec table (independent of the oracle)."""
    lo = wl.kv & 15
    hi = wl.kv >> 4
    codes = np.stack([lo, hi], -1).reshape(wl.kv.shape[0], 512)
    mag = np.array(E2M1_SPEC)[codes & 7]
    val = np.where(codes & 8, -mag, mag)
    scale = np.exp2(wl.kv_sc.astype(np.float64) - 127.0)
    return val * np.repeat(scale, 32, axis=1)


def decode_fp4_rows(codes_u8, n):
    lo = codes_u8 & 15
    hi = codes_u8 >> 4
    c = np.stack([lo, hi], -1).reshape(*codes_u8.shape[:-1], n)
    mag = np.array(E2M1_SPEC)[c & 7]
    return np.where(c & 8, -mag, mag)


def bf16_to_f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# formats
# ---------------------------------------------------------------------------

def test_e2m1_table_matches_spec():
    for code in range(16):
        v = oracle.e2m1(code)
        mag = E2M1_SPEC[code & 7]
        assert v == (-mag if code & 8 else mag)
        assert math.copysign(1.0, v) == (-1.0 if code & 8 else 1.0)


def test_e8m0_values():
    assert oracle.e8m0(127) == 1.0
    assert oracle.e8m0(0) == 2.0 ** -127
    assert oracle.e8m0(254) == 2.0 ** 127
    assert oracle.e8m0(130) == 8.0
    assert math.isnan(oracle.e8m0(255))


def test_e4m3fn_spec_points():
    # OCP MX v1.0 / OFP8 E4M3: bias 7, max normal 448, min normal 2^-6, min subnormal 2^-9, NaN S.1111.111
    assert oracle.e4m3(0x00) == 0.0
    assert oracle.e4m3(0x01) == 2.0 ** -9
    assert oracle.e4m3(0x07) == 7 * 2.0 ** -9
    assert oracle.e4m3(0x08) == 2.0 ** -6
    assert oracle.e4m3(0x38) == 1.0
    assert oracle.e4m3(0x7E) == 448.0
    assert oracle.e4m3(0xB8) == -1.0
    assert math.isnan(oracle.e4m3(0x7F)) and math.isnan(oracle.e4m3(0xFF))
    vals = [oracle.e4m3(c) for c in range(0x7F)]
    assert all(a < b for a, b in zip(vals, vals[1:]))  # monotone over the positive codes
    finite = {oracle.e4m3(c) for c in range(256) if not math.isnan(oracle.e4m3(c))}
    assert len(finite) == 253  # 254 non-NaN codes, +0 and -0 equal


def test_bf16_points():
    assert oracle.bf16(0x3F80) == 1.0
    assert oracle.bf16(0xC000) == -2.0
    assert math.isinf(oracle.bf16(0x7F80))
    assert oracle.bf16(0x3F00) == 0.5


def test_generator_encoders_agree_with_spec():
    L = synth.lib()
    for i, v in enumerate(E2M1_SPEC):
        assert L.csa2synth_encode_e2m1(v) == i
        if v:
            assert L.csa2synth_encode_e2m1(-v) == i | 8
    assert L.csa2synth_encode_e2m1(0.25) == 0  # tie to even (0)
    assert L.csa2synth_encode_e2m1(0.75) == 2  # tie to even (1.0)
    assert L.csa2synth_encode_e2m1(2.5) == 4   # tie to even (2.0)
    assert L.csa2synth_encode_e2m1(5.0) == 6   # tie to even (4.0)
    assert L.csa2synth_encode_e2m1(100.0) == 7
    for c in range(0x7F):
        assert L.csa2synth_encode_e4m3(oracle.e4m3(c)) == c


# ---------------------------------------------------------------------------
# visibility and compression ratio (report 2.3: entry j covers tokens jm..jm+m-1)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("m", [1, 2])
def test_visibility_brute_force(m):
    rng = np.random.default_rng(1)
    for _ in range(300):
        n = int(rng.integers(0, 50))
        t = int(rng.integers(-1, 120))
        brute = sum(1 for j in range(n) if (j + 1) * m - 1 <= t)
        assert oracle.visible(n, t, m) == brute


def test_prefill_chunk_visibility_closed_form():
    # 8,192 query tokens at the end of 262,144 tokens, ratio 2 -> 131,072 entries
    ts = np.arange(253952, 262144)
    vis = np.array([oracle.visible(131072, int(t), 2) for t in ts])
    assert vis.min() == 126976 and vis.max() == 131072
    assert int(vis.sum()) == 1056964608
    assert all(v == (t + 1) // 2 for v, t in zip(vis[:100], ts[:100]))


# ---------------------------------------------------------------------------
# index score
# ---------------------------------------------------------------------------

def _score_wl(q_vals_per_head, k_vals, w, q_sc=None, k_sc=127, t=0, n=1):
    H = len(q_vals_per_head)
    wl = tiny_workload([n], [[t]], H=H)
    for j in range(n):
        wl.k_idx[j] = pack_fp4(k_vals)
        wl.k_sc[j] = k_sc
    q = np.stack([pack_fp4(v) for v in q_vals_per_head])[None]
    qs = np.full((1, H), 127, np.uint8) if q_sc is None else np.asarray(q_sc, np.uint8)[None]
    return wl, q, qs, np.asarray(w, np.float32)[None]


def test_score_hand_values():
    wl, q, qs, w = _score_wl([[1.0] * 128], [0.5] * 128, [1.0], t=0)
    s = oracle.index_score(wl, q, qs, w, Q_FP4)
    assert s[0, 0] == 64.0  # 128 * 1.0 * 0.5
    wl, q, qs, w = _score_wl([[1.0] * 128], [0.5] * 128, [1.0], q_sc=[128], k_sc=126)
    assert oracle.index_score(wl, q, qs, w, Q_FP4)[0, 0] == 64.0  # x2 then x0.5
    wl, q, qs, w = _score_wl([[1.0] * 128], [0.5] * 128, [0.25], q_sc=[129])
    assert oracle.index_score(wl, q, qs, w, Q_FP4)[0, 0] == 64.0  # 0.25 * 4 * 64


def test_score_relu_and_sign():
    # a negative dot product contributes nothing; a positive one counts once
    wl, q, qs, w = _score_wl([[1.0] * 128, [-1.0] * 128], [0.5] * 128, [1.0, 1.0])
    s = oracle.index_score(wl, q, qs, w, Q_FP4)[0, 0]
    assert s == 64.0 and math.copysign(1, s) == 1
    wl, q, qs, w = _score_wl([[-1.0] * 128], [0.5] * 128, [1.0])
    s = oracle.index_score(wl, q, qs, w, Q_FP4)[0, 0]
    assert s == 0.0 and math.copysign(1, s) == 1.0  # +0, never -0


def test_score_invisible_is_neg_inf():
    # query at t = 2 over 5 entries (ratio 1): entries 3, 4 are not visible
    wl, q, qs, w = _score_wl([[1.0] * 128], [0.5] * 128, [1.0], t=2, n=5)
    s = oracle.index_score(wl, q, qs, w, Q_FP4)[0]
    assert list(s[:3]) == [64.0] * 3 and np.all(np.isneginf(s[3:]))


def test_score_head_sum_order_exact_rational():
    """The canonical fp32 head sum (one fused multiply-add per head, h ascending)
    against an exact rational evaluation with round-to-nearest-even per step."""
    rng = np.random.default_rng(7)
    H = 64
    for trial in range(6):
        dots = rng.integers(-40, 60, size=H)
        qv = []
        for d in dots:  # q_h = d ones (or minus ones), k = all ones -> dot = d
            row = [0.0] * 128
            for i in range(abs(int(d))):
                row[i] = 1.0 if d > 0 else -1.0
            qv.append(row)
        w = rng.random(H, dtype=np.float32)
        eq = rng.integers(120, 135, size=H)
        ek = int(rng.integers(120, 135))
        wl, q, qs, ww = _score_wl(qv, [1.0] * 128, w, q_sc=eq, k_sc=ek)
        got = oracle.index_score(wl, q, qs, ww, Q_FP4)[0, 0]
        acc = Fraction(0)
        for h in range(H):
            r = Fraction(max(int(dots[h]), 0)) * Fraction(2) ** (int(eq[h]) - 127)
            acc = Fraction(rne_f32(Fraction(float(w[h])) * r + acc))
        want = rne_f32(acc * Fraction(2) ** (ek - 127))
        assert got == want, (trial, got, want)


def test_score_exact_against_float64_dot():
    """Random quantised data, w = 1 for every head: the head sum is then exact,
    so the score equals the float64 value of the definition."""
    wl = synth.config("decode_c0", n_entries=[300])
    L = wl.layers[0]
    w1 = np.ones_like(L.w)
    s = oracle.index_score(wl, L.q_idx, L.q_sc, w1, Q_FP4)[0]
    k = decode_fp4_rows(wl.k_idx, 128)                      # [N][128]
    q = decode_fp4_rows(L.q_idx[0], 128)                    # [H][128]
    d = q @ k.T                                             # exact in float64
    r = np.maximum(d, 0) * np.exp2(L.q_sc[0].astype(np.float64) - 127)[:, None]
    want = r.sum(0) * np.exp2(wl.k_sc.astype(np.float64) - 127)
    assert np.array_equal(s[:300].astype(np.float64), want)


def test_score_mxfp4_block_scales_hand_value():
    """The report's indexer format (OCP MXFP4 on both sides, one E8M0 per 32
    channels): every block's scales enter the dot product, and no per-entry
    factor follows the head sum.  q = k = 1 everywhere, so block b contributes
    32 * 2^(eq_b + ek_b - 254)."""
    wl, q, _, w = _score_wl([[1.0] * 128], [1.0] * 128, [1.0])
    wl.k_sc = np.array([[127, 127, 127, 129]], np.uint8)
    qs = np.array([[[127, 128, 126, 127]]], np.uint8)
    assert oracle.index_score(wl, q, qs, w, Q_MXFP4)[0, 0] == 32 * (1 + 2 + 0.5 + 4)
    # a negative dot product is cut by the ReLU after the block scales apply:
    # block 0 -> -32 * 2^3, blocks 1..3 -> +32 each: the sum is negative
    q2 = np.stack([pack_fp4([-1.0] * 32 + [1.0] * 96)])[None]
    wl.k_sc = np.array([[130, 127, 127, 127]], np.uint8)
    qs = np.full((1, 1, 4), 127, np.uint8)
    s = oracle.index_score(wl, q2, qs, w, Q_MXFP4)[0, 0]
    assert s == 0.0 and math.copysign(1, s) == 1.0


def test_score_mxfp4_flags_wide_block_spread_even_when_blocks_cancel():
    """The exactness bound of the MXFP4 score is on the sum of the products'
    magnitudes in units of the finest block grid, not on the final dot
    product.  q = +6 on block 0 and -6 on block 1, k = 6, and the key's scales
    of blocks 0 and 1 sit 2^sh above those of blocks 2 and 3: the two big blocks
    cancel, so d_h is small, while a binary32 accumulation passes through
    32 * 36 * 2^sh.  In quarter-units the magnitudes sum to 2 * 4,608 * 2^sh
    plus the small blocks: above 2^24 at sh = 11, which must be refused, and
    below it at sh = 10, where d_h = 64 * 0.5 * 6 = 192 exactly."""
    vals = [6.0] * 32 + [-6.0] * 32 + [0.5] * 64
    wl, q, _, w = _score_wl([vals], [6.0] * 128, [1.0])
    for sh, flagged in ((11, True), (10, False)):
        wl.k_sc = np.array([[127 + sh, 127 + sh, 127, 127]], np.uint8)
        qs = np.full((1, 1, 4), 127, np.uint8)
        if flagged:
            with pytest.raises(ValueError):
                oracle.index_score(wl, q, qs, w, Q_MXFP4)
        else:
            # blocks 0, 1 cancel exactly; blocks 2, 3: 64 * 0.5 * 6 = 192
            assert oracle.index_score(wl, q, qs, w, Q_MXFP4)[0, 0] == 192.0


def test_score_mxfp4_exact_rational_on_generated_rows():
    """Generated MXFP4 rows (OCP scale rule per 32-channel block): the block
    dot products summed in float64 are exact, fit binary32 exactly (the block
    scales of a q/K pair span a few powers of two), and the head sum with one
    correctly rounded fused multiply-add per head, evaluated in rationals,
    equals the oracle's score bit for bit."""
    wl = synth.config("decode_c0", n_entries=[160], q_fmt=Q_MXFP4)
    L = wl.layers[0]
    assert L.q_sc.shape == (1, 64, 4) and wl.k_sc.shape == (160, 4)
    got = oracle.index_score(wl, L.q_idx, L.q_sc, L.w, Q_MXFP4)[0]
    q = decode_fp4_rows(L.q_idx[0], 128) * np.repeat(np.exp2(L.q_sc[0].astype(np.float64) - 127), 32, axis=1)
    k = decode_fp4_rows(wl.k_idx, 128) * np.repeat(np.exp2(wl.k_sc.astype(np.float64) - 127), 32, axis=1)
    d = q @ k.T                                             # [H][N], exact in float64
    assert np.array_equal(d.astype(np.float32).astype(np.float64), d)
    spread = np.ptp(L.q_sc[0][:, None, :].astype(int) + wl.k_sc[None].astype(int), axis=-1)
    assert spread.max() <= 6
    for j in range(160):
        acc = Fraction(0)
        for h in range(64):
            acc = Fraction(rne_f32(Fraction(float(L.w[0, h])) * Fraction(max(d[h, j], 0.0)) + acc))
        assert got[j] == float(acc), (j, got[j], float(acc))


def test_score_fp8_query_hand_and_random():
    # E4M3 query code 0x38 = 1.0, 0x30 = 0.5 ; k = 0.5
    wl = tiny_workload([1], [[1]], ratio=2, H=1)
    wl.k_idx[0] = pack_fp4([0.5] * 128)
    q = np.full((1, 1, 128), 0x38, np.uint8)
    q[0, 0, 64:] = 0x30
    s = oracle.index_score(wl, q, np.full((1, 1), 127, np.uint8), np.ones((1, 1), np.float32), Q_FP8)
    assert s[0, 0] == 64 * 0.5 + 64 * 0.25
    # random FP8 rows from the generator, w = 1: exact float64 comparison
    wl = synth.config("prefill_c3", tokens=600, T=8, n_layers=1)
    L = wl.layers[0]
    w1 = np.ones_like(L.w)
    s = oracle.index_score(wl, L.q_idx, L.q_sc, w1, Q_FP8)
    e4 = np.array([oracle.e4m3(c) if (c & 0x7F) != 0x7F else 0.0 for c in range(256)])
    k = decode_fp4_rows(wl.k_idx, 128)
    for r in range(8):
        q = e4[L.q_idx[r]]
        d = q @ k.T
        rr = np.maximum(d, 0) * np.exp2(L.q_sc[r].astype(np.float64) - 127)[:, None]
        want = rr.sum(0) * np.exp2(wl.k_sc.astype(np.float64) - 127)
        vis = oracle.visible(300, int(wl.q_pos[r]), 2)
        assert np.array_equal(s[r, :vis].astype(np.float64), want[:vis])
        assert np.all(np.isneginf(s[r, vis:300]))


# ---------------------------------------------------------------------------
# Top-K (report 2.3; K = 512 in 4.2.1)
# ---------------------------------------------------------------------------

def test_topk_hand_ties():
    s = np.array([[3, 5, 5, 1, 5]], np.float32)
    assert list(oracle.topk(s, [5], 2)[0]) == [1, 2]
    assert list(oracle.topk(s, [5], 4)[0]) == [0, 1, 2, 4]
    assert list(oracle.topk(s, [5], 7)[0]) == [0, 1, 2, 3, 4, -1, -1]
    assert list(oracle.topk(s, [3], 2)[0]) == [1, 2]   # only slots 0..2 take part
    cand = np.array([[10, 20, 30, -1, -1]], np.int32)
    s2 = np.array([[1, 2, 2, 0, 0]], np.float32)
    assert list(oracle.topk(s2, [3], 1, cand=cand)[0]) == [20]


@pytest.mark.parametrize("distinct", [3, 50, 100000])
def test_topk_against_lexsort(distinct):
    rng = np.random.default_rng(distinct)
    rows, n, K = 6, 3000, 512
    s = (rng.integers(0, distinct, size=(rows, n)) * 0.125).astype(np.float32)
    nv = rng.integers(100, n, size=rows)
    got = oracle.topk(s, nv, K)
    for r in range(rows):
        m = int(nv[r])
        order = np.lexsort((np.arange(m), -s[r, :m].astype(np.float64)))
        want = np.sort(order[:K])
        want = np.concatenate([want, -np.ones(K - len(want), np.int64)])
        assert np.array_equal(got[r], want)


# ---------------------------------------------------------------------------
# block pool (report 2.3.2; reading note decoder indexer paragraph)
# ---------------------------------------------------------------------------

def test_block_pool_hand_case():
    s = np.array([[1, 9, 3, 3, 9, 0, 2, 2, 5]], np.float32)
    blocks, pool, cnt = oracle.block_pool(s, [9], block=2, max_blocks=2)
    assert list(blocks[0]) == [0, 2]
    assert list(pool[0][:4]) == [0, 1, 4, 5] and cnt[0] == 4
    # partial last block counts its visible positions only; a tie goes to the lower block
    s = np.array([[1, 1, 0, 0, 1]], np.float32)
    blocks, pool, cnt = oracle.block_pool(s, [5], block=2, max_blocks=2)
    assert list(blocks[0]) == [0, 2] and list(pool[0]) == [0, 1, 4, -1] and cnt[0] == 3


def test_block_pool_brute_force_and_invariants():
    rng = np.random.default_rng(3)
    rows, n = 3, 40000
    s = (rng.integers(0, 2000, size=(rows, n)) * 0.5).astype(np.float32)
    vis = np.array([40000, 39999, 17000])
    blocks, pool, cnt = oracle.block_pool(s, vis, 8, 2048)
    topk = oracle.topk(s, vis, 512)
    for r in range(rows):
        v = int(vis[r])
        nb = (v + 7) // 8
        padded = np.full(nb * 8, -np.inf)
        padded[:v] = s[r, :v]
        bmax = padded.reshape(nb, 8).max(1)
        order = np.lexsort((np.arange(nb), -bmax))
        want = np.sort(order[:2048])
        assert np.array_equal(blocks[r][: len(want)], want) and np.all(blocks[r][len(want):] == -1)
        pp = pool[r][: cnt[r]]
        assert cnt[r] <= 16384 and np.all(np.diff(pp) > 0) and np.all(pool[r][cnt[r]:] == -1)
        assert set(pp.tolist()) == {j for b in want for j in range(8 * b, min(8 * b + 8, v))}
        # Top-512 is inside the pool: every block ranked ahead of a selected
        # position's block holds a distinct position ranked ahead of it.
        sel = topk[r][topk[r] >= 0]
        assert set(sel.tolist()) <= set(pp.tolist())


def test_block_pool_is_everything_when_small():
    rng = np.random.default_rng(4)
    s = rng.random((1, 16384)).astype(np.float32)
    blocks, pool, cnt = oracle.block_pool(s, [16384], 8, 2048)
    assert cnt[0] == 16384 and np.array_equal(pool[0], np.arange(16384))
    blocks, pool, cnt = oracle.block_pool(s, [1001], 8, 2048)
    assert cnt[0] == 1001 and np.array_equal(pool[0][:1001], np.arange(1001))


# ---------------------------------------------------------------------------
# gather + dequant (report 2.4.4)
# ---------------------------------------------------------------------------

def test_gather_dequant_against_spec_decode():
    wl = synth.config("decode_c0", n_entries=[700])
    rng = np.random.default_rng(5)
    idx = np.sort(rng.choice(700, 512, replace=False)).astype(np.int32)[None]
    idx[0, -5:] = -1
    out = oracle.gather_dequant(wl, idx)
    ref = decode_kv(wl)
    got = bf16_to_f64(out[0])
    for s in range(512):
        if idx[0, s] < 0:
            assert np.all(out[0, s] == 0)
        else:
            assert np.array_equal(got[s], ref[idx[0, s]])


# ---------------------------------------------------------------------------
# attention (report 2.3; reading note Figure 4: selected main KV concatenated
# with the SWA KV; course notes 3.2.2: window [max(s, i-W+1), i])
# ---------------------------------------------------------------------------

def _dense_ref(q, keys, scale):
    """torch's scaled_dot_product_attention in float64 on the CPU with K = V =
    keys; the heads are the batch dimension."""
    qt = torch.from_numpy(np.ascontiguousarray(q))[:, None, :]          # [H, 1, 512]
    kt = torch.from_numpy(np.ascontiguousarray(keys))[None].expand(q.shape[0], *keys.shape).contiguous()
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, kt, scale=scale)
    return out[:, 0, :].numpy()


def _attn_setup(n, Hm=4, t=None, W=128):
    wl = synth.config("decode_c0", n_entries=[n], Hm=Hm, W=W)
    return wl, wl.layers[0]


def test_sparse_equals_dense_when_topk_covers_all():
    wl, L = _attn_setup(300)
    idx = np.full((1, 512), -1, np.int32)
    idx[0, :300] = np.arange(300)
    out, lse = oracle.sparse_attn(wl, L.q_main, idx, L.swa)
    keys = np.concatenate([decode_kv(wl)[:300], bf16_to_f64(L.swa)])  # window rows 172..299
    assert L.swa.shape[0] == 128
    q = bf16_to_f64(L.q_main[0])
    ref = _dense_ref(q, keys, 1 / math.sqrt(512))
    np.testing.assert_allclose(out[0], ref, rtol=1e-6, atol=1e-6)
    logits = (q @ keys.T) / math.sqrt(512)
    np.testing.assert_allclose(lse[0], np.log(np.exp(logits).sum(1)), rtol=1e-6)


def test_swa_only_equals_dense_window():
    wl, L = _attn_setup(300)
    idx = np.full((1, 512), -1, np.int32)
    out, _ = oracle.sparse_attn(wl, L.q_main, idx, L.swa)
    ref = _dense_ref(bf16_to_f64(L.q_main[0]), bf16_to_f64(L.swa), 1 / math.sqrt(512))
    np.testing.assert_allclose(out[0], ref, rtol=1e-6, atol=1e-6)


def test_short_context_window_and_replay_start():
    # t = 40 < W - 1: the window is [0, 40]; with a replay start s = 25 it is [25, 40]
    wl = synth.config("decode_c0", n_entries=[41], Hm=2)
    L = wl.layers[0]
    assert L.swa.shape[0] == 41
    idx = np.full((1, 512), -1, np.int32)
    out, _ = oracle.sparse_attn(wl, L.q_main, idx, L.swa)
    q = bf16_to_f64(L.q_main[0])
    np.testing.assert_allclose(out[0], _dense_ref(q, bf16_to_f64(L.swa), 1 / math.sqrt(512)), rtol=1e-6, atol=1e-6)
    out, _ = oracle.sparse_attn(wl, L.q_main, idx, L.swa, replay_s=np.array([25], np.int32))
    np.testing.assert_allclose(out[0], _dense_ref(q, bf16_to_f64(L.swa[25:]), 1 / math.sqrt(512)), rtol=1e-6,
                               atol=1e-6)


def test_identical_keys_closed_form():
    # every key equal -> softmax is uniform: output = the key, lse = logit + log(n)
    wl = tiny_workload([600], [[599]], Hm=2)
    row = pack_fp4(([1.0, -0.5, 2.0, 0.0] * 128)[:512])
    wl.kv[:] = row
    wl.kv_sc[:] = 126
    key = decode_kv(wl)[0]
    swa = np.tile(((key.astype(np.float32).view(np.uint32)) >> 16).astype(np.uint16), (128, 1))
    q = np.tile(((np.linspace(-1, 1, 512).astype(np.float32).view(np.uint32)) >> 16).astype(np.uint16), (1, 2, 1))
    idx = np.arange(512, dtype=np.int32)[None]
    out, lse = oracle.sparse_attn(wl, q, idx, swa)
    np.testing.assert_allclose(out[0, 0], key, rtol=1e-12, atol=1e-12)
    logit = bf16_to_f64(q[0, 0]) @ key / math.sqrt(512)
    assert abs(lse[0, 0] - (logit + math.log(640))) < 1e-5


def test_attention_order_invariant():
    wl, L = _attn_setup(2000)
    rng = np.random.default_rng(9)
    idx = np.sort(rng.choice(2000, 512, replace=False)).astype(np.int32)[None]
    out1, lse1 = oracle.sparse_attn(wl, L.q_main, idx, L.swa)
    out2, lse2 = oracle.sparse_attn(wl, L.q_main, idx[:, ::-1].copy(), L.swa)
    np.testing.assert_allclose(out1, out2, rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(lse1, lse2, rtol=1e-7)


# ---------------------------------------------------------------------------
# modes and the layer chain (report 2.3.1; reading note mode + schedule tables)
# ---------------------------------------------------------------------------

def _small_chain(n=24000, n_seq=2):
    return synth.config("chain_c2", n_seq=n_seq, n=n, Hm=4)


def test_reuse_equals_regather_with_source_indices():
    wl = _small_chain()
    res = oracle.layer_chain(wl)
    by = {r["layer"]: r for r in res}
    # layers 21..23 reuse 20's indices; 25..27 reuse 24's
    for reuse, src in [(21, 20), (23, 20), (25, 24), (39, 36)]:
        assert np.array_equal(by[reuse]["idx"], by[src]["idx"])
        L = [x for x in wl.layers if x.index == reuse][0]
        out, _ = oracle.sparse_attn(wl, L.q_main, by[src]["idx"], L.swa)
        assert np.array_equal(out, by[reuse]["out"])


def test_reindex_with_full_layer_query_reproduces_full_topk():
    wl = _small_chain()
    full = [x for x in wl.layers if x.index == 20][0]
    for L in wl.layers:
        if L.mode == MODE_REINDEX:
            L.q_idx, L.q_sc, L.w = full.q_idx, full.q_sc, full.w
    by = {r["layer"]: r for r in oracle.layer_chain(wl, attn=False)}
    for l in (24, 28, 32, 36):
        assert np.array_equal(by[l]["idx"], by[20]["idx"])


def test_reindex_equals_full_scores_masked_to_pool():
    """Reading note implementation table: the released reference scores the
    whole range and then masks to the candidates; the pool-only path must agree."""
    wl = _small_chain()
    by = {r["layer"]: r for r in oracle.layer_chain(wl, attn=False)}
    vis = oracle.row_visible(wl)
    L = [x for x in wl.layers if x.index == 28][0]
    full = oracle.index_score(wl, L.q_idx, L.q_sc, L.w, Q_FP4)
    for r in range(wl.total_q):
        pp = by[20]["pool_pos"][r][: by[20]["pool_count"][r]]
        masked = np.full(full.shape[1], -np.inf, np.float32)
        masked[pp] = full[r, pp]
        nv = int(vis[r])
        order = np.lexsort((np.arange(nv), -masked[:nv].astype(np.float64)))
        want = np.sort(order[:512])
        assert np.array_equal(by[28]["idx"][r], want)
    assert not np.array_equal(by[28]["idx"], by[20]["idx"])  # a different selection in general


def test_pool_contains_full_topk_and_is_bounded():
    wl = _small_chain()
    by = {r["layer"]: r for r in oracle.layer_chain(wl, attn=False)}
    for r in range(wl.total_q):
        cnt = by[20]["pool_count"][r]
        assert cnt == 16384  # 24,000 entries -> 3,000 blocks > 2,048
        assert set(by[20]["idx"][r].tolist()) <= set(by[20]["pool_pos"][r][:cnt].tolist())
        for l in (24, 28, 32, 36):
            assert set(by[l]["idx"][r].tolist()) <= set(by[20]["pool_pos"][r][:cnt].tolist())


def test_swa_only_layers_and_encoder_ratio():
    # layers 0-1 are SWA only; an encoder group at ratio 2 is Full + 5 Reuse
    wl = synth.make_workload("enc", 11, [500], 3, [(0, MODE_SWA_ONLY, False), (1, MODE_SWA_ONLY, False),
                                                  (2, MODE_FULL, False), (3, MODE_REUSE, False)],
                             ratio=2, Hm=2, q_pos=[np.array([900, 950, 999])])
    res = oracle.layer_chain(wl)
    assert np.all(res[0]["idx"] == -1) and np.all(res[1]["idx"] == -1)
    vis = [oracle.visible(500, t, 2) for t in (900, 950, 999)]
    assert vis == [450, 475, 500]
    for r in range(3):
        sel = res[2]["idx"][r]
        assert np.all(sel[sel >= 0] < vis[r])
    L0 = wl.layers[0]
    for r, t in enumerate((900, 950, 999)):
        lo = t - 127 - int(wl.swa_pos0[0])
        keys = bf16_to_f64(L0.swa[lo: lo + 128])
        ref = _dense_ref(bf16_to_f64(L0.q_main[r]), keys, 1 / math.sqrt(512))
        np.testing.assert_allclose(res[0]["out"][r], ref, rtol=1e-6, atol=1e-6)


def test_encoder_chain_reads_each_full_layers_caches():
    """Report 2.3.1 (Reindex and Reuse read the global KV of the preceding Full
    layer) with the reading note's encoder schedule (Full layers 2, 8 and 14,
    each generating its own KV): layers 0..19 as one chain at ratio 2.  With at
    most 512 visible entries the Top-K covers them all, so every layer equals
    dense attention over [all visible entries of its group's Full cache ++ its
    window], decoded here from the spec table.  A chain that kept the first
    Full layer's cache would fail from layer 8 on."""
    n, t = 400, 799  # ratio 2: all 400 entries visible to t = 799
    wl = synth.make_workload("enc20", 31, [n], 1, synth.encoder_schedule(), ratio=2, Hm=2,
                             q_pos=[np.array([t])], own_caches=True)
    fulls = {L.index: L for L in wl.layers if L.mode == MODE_FULL}
    assert sorted(fulls) == [2, 8, 14]
    assert not np.array_equal(fulls[2].kv, fulls[8].kv) and not np.array_equal(fulls[8].k_idx, fulls[14].k_idx)
    res = oracle.layer_chain(wl)
    for L, r in zip(wl.layers, res):
        q = bf16_to_f64(L.q_main[0])
        win = bf16_to_f64(L.swa[t - 127 - int(wl.swa_pos0[0]): t + 1 - int(wl.swa_pos0[0])])
        if L.mode == MODE_SWA_ONLY:
            assert np.all(r["idx"] == -1)
            keys = win
        else:
            g = max(i for i in fulls if i <= L.index)
            assert np.array_equal(r["idx"][0, :n], np.arange(n)) and np.all(r["idx"][0, n:] == -1)
            view = synth.Workload(**{f: getattr(wl, f) for f in wl.__dataclass_fields__})
            view.kv, view.kv_sc = fulls[g].kv, fulls[g].kv_sc
            keys = np.concatenate([decode_kv(view)[:n], win])
        ref = _dense_ref(q, keys, 1 / math.sqrt(512))
        np.testing.assert_allclose(r["out"][0], ref, rtol=1e-6, atol=1e-6, err_msg=f"layer {L.index}")


def test_cache_ledger_of_this_layout():
    # the pages' ledger is pinned against tests/golden/cache_ledger.json; this
    # library's layout: MXFP4 main KV (256 + 16 B) and E2M1 indexer K with one
    # E8M0 per row (64 + 1 B), under the same source layers
    from compressed_sparse_attention_amd import ledger
    assert ledger.bytes_per_position("mxfp4_e8m0") == 337
    assert ledger.bytes_per_token("mxfp4_e8m0") == 842.5


def test_decoder_replay_chain():
    """Decoder SWA bounded replay (course notes "3. 通用基础设施" §3.2.2: a query
    at t sees window rows max(s, t - W + 1) .. t): the last T = W prompt tokens
    rerun the decoder layers with s at the first of them.  A start at 0 changes
    nothing; the last token's window is not cut, so its row equals the chain
    without replay; every earlier row loses window keys, so its log-sum-exp is
    strictly lower (a softmax over a subset of the keys) and its output moves.
    The selections do not depend on the window."""
    n, T = 1500, 128
    sched = [(20, MODE_FULL, True), (24, MODE_REINDEX, False), (25, MODE_REUSE, False)]
    base = synth.config("replay_c5", n_seq=1, n=n, T=T, Hm=16, schedule=sched)
    assert list(base.replay_s) == [n - T] and base.q_pos[0] == n - T and base.q_pos[-1] == n - 1
    plain = synth.config("replay_c5", n_seq=1, n=n, T=T, Hm=16, schedule=sched)
    plain.replay_s = None
    zero = synth.config("replay_c5", n_seq=1, n=n, T=T, Hm=16, schedule=sched)
    zero.replay_s = np.zeros(1, np.int32)
    rp, rn, rz = oracle.layer_chain(base), oracle.layer_chain(plain), oracle.layer_chain(zero)
    for a, b, c in zip(rp, rn, rz):
        assert np.array_equal(a["idx"], b["idx"])
        np.testing.assert_array_equal(c["out"], b["out"])
        np.testing.assert_array_equal(c["lse"], b["lse"])
        np.testing.assert_array_equal(a["out"][-1], b["out"][-1])
        np.testing.assert_array_equal(a["lse"][-1], b["lse"][-1])
        assert np.all(a["lse"][:-1] < b["lse"][:-1])
        assert np.all(np.abs(a["out"][:-1] - b["out"][:-1]).max(axis=(1, 2)) > 0)


def test_e2m1_e4m3_block_encoder():
    """The report's main-KV cache format (section 2.4.4: E2M1 with one E4M3
    scale per 16 channels, NVFP4 without its second-level global scale) as the
    generator writes it, checked by brute force over the spec grids: the scale
    is the E4M3 value nearest to amax / 6 (ties to the even code; a block whose
    scale would be 0 takes the smallest step), every element the E2M1 value
    nearest to x / X (ties to the even code, saturating at 6)."""
    rows, seed, tid = 24, 321, 17
    codes, scales = synth.e2m1_e4m3_rows(seed, tid, rows, 512)
    x = synth.normal_f64(seed, tid, rows * 512).reshape(rows, 32, 16)
    pos = [c for c in range(1, 127)]  # finite positive E4M3 codes (0x7F is NaN)
    vals = np.array([oracle.e4m3(c) for c in pos])
    e2 = np.array(E2M1_SPEC)
    for r in range(rows):
        for b in range(32):
            blk = x[r, b]
            t = np.abs(blk).max() / 6.0
            d = np.abs(vals - t)
            best = [pos[i] for i in np.flatnonzero(d == d.min())]
            want = min(best, key=lambda c: (c & 1, c)) if len(best) > 1 else best[0]
            assert scales[r, b] == want, (r, b)
            X = oracle.e4m3(int(scales[r, b]))
            for c in range(16):
                a = abs(blk[c]) / X
                if a >= 6.0:
                    m = 7
                else:
                    dd = np.abs(e2 - a)
                    cand = np.flatnonzero(dd == dd.min())
                    m = int(cand[0]) if len(cand) == 1 else int(cand[0] if cand[0] % 2 == 0 else cand[1])
                byte = codes[r, (16 * b + c) // 2]
                nib = (byte >> 4) if c & 1 else (byte & 15)
                assert nib & 7 == m, (r, b, c)
                assert (nib >> 3) == (1 if blk[c] < 0 and m != 0 else 0)


def test_gather_dequant_e4m3_scales_against_spec_decode():
    """fmt 1 main KV: value = E2M1 * E4M3(scale of its 16-channel block), exact
    in bf16, decoded here from the spec tables."""
    wl = synth.config("decode_c0", n_entries=[300], kv_fmt=1)
    idx = np.array([[0, 5, -1, 299, 17]], np.int32)
    got = oracle.gather_dequant(wl, idx)
    for s, j in enumerate(idx[0]):
        if j < 0:
            assert not got[0, s].any()
            continue
        for ch in range(0, 512, 7):
            byte = wl.kv[j, ch // 2]
            nib = (byte >> 4) if ch & 1 else (byte & 15)
            v = (-1 if nib & 8 else 1) * E2M1_SPEC[nib & 7] * oracle.e4m3(int(wl.kv_sc[j, ch // 16]))
            f = np.float32(v)
            assert abs(float(f) - v) == 0.0
            assert got[0, s, ch] == (f.view(np.uint32) >> 16), (s, ch)


def test_mxfp8_swa_encoder_and_decode():
    """SWA rows in OCP MXFP8 (the report's section 2.4.4 keeps SWA KV in FP8;
    the OCP MX family the pages name gives its block form): per 32 channels
    X = 2^(floor(log2 amax) - 8) (emax of E4M3 is 8), elements the E4M3 values
    nearest to x / X (ties to the even code), checked by brute force over the
    spec grid; the oracle's attention reads them as E4M3 * E8M0, which for a
    lone key in the window (no selected entries) is its output exactly."""
    rows, seed, tid = 6, 77, 5
    enc = synth.mxfp8_rows(seed, tid, rows, 512)
    x = synth.normal_f64(seed, tid, rows * 512).reshape(rows, 16, 32)
    codes = [c for c in range(256) if (c & 0x7F) != 0x7F]
    vals = np.array([oracle.e4m3(c) for c in codes])
    for r in range(rows):
        for b in range(16):
            blk = x[r, b]
            se = math.floor(math.log2(np.abs(blk).max())) - 8
            assert enc[r, 512 + b] == se + 127
            for c in range(32):
                t = blk[c] / 2.0 ** se
                d = np.abs(vals - t)
                best = [codes[i] for i in np.flatnonzero(d == d.min())]
                want = best[0] if len(best) == 1 else min(best, key=lambda k: (k & 1, k))
                assert oracle.e4m3(int(enc[r, 32 * b + c])) == oracle.e4m3(int(want)), (r, b, c)
    # one query at t = 0 sees exactly one SWA row and no entry: out = that row
    wl = synth.make_workload("swa8", 3, [1], 1, [(0, MODE_SWA_ONLY, False)], Hm=16, swa_fmt=1, q_pos=[np.array([0])])
    L = wl.layers[0]
    out, lse = oracle.sparse_attn(wl, L.q_main, np.full((1, 512), -1, np.int32), L.swa)
    row = L.swa[0]
    want = np.array([oracle.e4m3(int(row[c])) * oracle.e8m0(int(row[512 + c // 32])) for c in range(512)], np.float32)
    for h in range(16):
        np.testing.assert_array_equal(out[0, h], want)


# ---------------------------------------------------------------------------
# cache append: RoPE on the last 64 latent channels, then quantise all 512
# (report 2.4.4); the encoder below is written from the format definitions
# ---------------------------------------------------------------------------

def _e4m3_spec(code):
    """OCP OFP8 E4M3 (FN) value of a non-negative code 0..126, from its fields."""
    e, m = code >> 3, code & 7
    return Fraction(m, 8) * Fraction(2) ** -6 if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)


E4M3_SPEC = [_e4m3_spec(c) for c in range(127)]


def _nearest_even(a: Fraction, grid):
    """Index of the grid value nearest to a >= 0; ties go to the even index."""
    best = min(range(len(grid)), key=lambda i: (abs(a - grid[i]), i & 1))
    return best


def _spec_append(x, cs, kv_fmt):
    """One entry: rotation in float32 (products, then difference / sum), then
    the quantiser with its decisions on float32 quotients."""
    v = np.asarray(x, np.float32).copy()
    for i in range(32):
        a, b = v[448 + 2 * i], v[449 + 2 * i]
        co, si = np.float32(cs[i, 0]), np.float32(cs[i, 1])
        v[448 + 2 * i] = np.float32(a * co) - np.float32(b * si)
        v[449 + 2 * i] = np.float32(a * si) + np.float32(b * co)
    bl = 16 if kv_fmt == 1 else 32
    codes, scales = [], []
    e2m1 = [Fraction(z).limit_denominator(2) for z in E2M1_SPEC]
    for b0 in range(0, 512, bl):
        blk = v[b0:b0 + bl]
        amax = np.float32(np.max(np.abs(blk)))
        if kv_fmt == 1:
            sc = _nearest_even(Fraction(float(np.float32(amax / np.float32(6.0)))), E4M3_SPEC) or 1
            X = np.float32(float(E4M3_SPEC[sc]))
        else:
            se = max(math.frexp(float(amax))[1] - 3, -127) if amax > 0 else 0
            sc, X = se + 127, np.float32(2.0 ** se)
        scales.append(sc)
        for z in blk:
            q = np.float32(z / X)
            c = _nearest_even(abs(Fraction(float(q))), e2m1)
            codes.append(c | (8 if q < 0 else 0))
    packed = np.array([codes[2 * i] | (codes[2 * i + 1] << 4) for i in range(256)], np.uint8)
    return packed, np.array(scales, np.uint8)


def _angles(rng, n):
    th = rng.uniform(-np.pi, np.pi, size=(n, 32))
    return np.stack([np.cos(th), np.sin(th)], -1).astype(np.float32)


@pytest.mark.parametrize("kv_fmt", [0, 1])
def test_kv_append_matches_spec_encoder(kv_fmt):
    """Random latents (three magnitudes of block, an all-zero block, a block
    past the saturation point), random angles, rows written out of order:
    every row equals the encoder written here from the format definitions,
    and rows not written stay untouched."""
    rng = np.random.default_rng(11 + kv_fmt)
    n = 6
    x = (rng.standard_normal((n, 512)) * np.array([1, 30, 1e-3, 1, 1, 1])[:, None]).astype(np.float32)
    x[3, 0:32] = 0.0                       # an all-zero block
    x[4, 64:96] = 5000.0                   # beyond 6 x 448: the E4M3 scale saturates
    cs = _angles(rng, n)
    dst = np.array([7, 2, 0, 5, 3, 9])
    kv, sc = oracle.kv_append(x, cs, dst, kv_fmt, 10)
    for e in range(n):
        want_c, want_s = _spec_append(x[e], cs[e], kv_fmt)
        assert np.array_equal(kv[dst[e]], want_c), e
        assert np.array_equal(sc[dst[e]], want_s), e
    for r in set(range(10)) - set(dst.tolist()):
        assert not kv[r].any() and not sc[r].any()
    with pytest.raises(ValueError):
        oracle.kv_append(x[:1], cs[:1], np.array([10]), kv_fmt, 10)


@pytest.mark.parametrize("kv_fmt", [0, 1])
def test_kv_append_quarter_turn_and_error_bound(kv_fmt):
    """A quarter turn maps (a, b) to (-b, a) exactly, so appending x with it
    equals appending the pre-turned x unrotated.  For any angle the decoded
    row is within the quantiser's half step of the float64 rotation."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((4, 512)).astype(np.float32)
    quarter = np.zeros((4, 32, 2), np.float32)
    quarter[..., 1] = 1.0
    ident = np.zeros((4, 32, 2), np.float32)
    ident[..., 0] = 1.0
    xt = x.copy()
    xt[:, 448::2], xt[:, 449::2] = -x[:, 449::2], x[:, 448::2]
    dst = np.arange(4)
    a = oracle.kv_append(x, quarter, dst, kv_fmt, 4)
    b = oracle.kv_append(xt, ident, dst, kv_fmt, 4)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    cs = _angles(rng, 4)
    kv, sc = oracle.kv_append(x, cs, dst, kv_fmt, 4)
    rot = x.astype(np.float64).copy()
    co, si = cs[..., 0].astype(np.float64), cs[..., 1].astype(np.float64)
    p, q = x[:, 448::2].astype(np.float64), x[:, 449::2].astype(np.float64)
    rot[:, 448::2], rot[:, 449::2] = p * co - q * si, p * si + q * co
    if kv_fmt == 1:
        scale = np.repeat(np.array([[oracle.e4m3(int(c)) for c in r] for r in sc]), 16, axis=1)
    else:
        scale = np.repeat(np.exp2(sc.astype(np.float64) - 127), 32, axis=1)
    deq = decode_fp4_rows(kv, 512) * scale
    # the E2M1 grid steps by at most 2 below 6, so a half step is at most one
    # scale unit.  The E4M3 scale follows amax / 6, so nothing saturates by
    # more than that; the MX scale 2^(floor(log2 amax) - 2) leaves values up to
    # 8 units that clamp to 6: two units.  1e-6 covers the rotation's rounding.
    units = 1.0 if kv_fmt == 1 else 2.0
    assert np.all(np.abs(deq - rot) <= units * scale * (1 + 1e-6))


# ---------------------------------------------------------------------------
# compressor: entry = per-channel softmax over its m tokens of Z, weighting C
# ---------------------------------------------------------------------------

def test_compress_special_cases():
    rng = np.random.default_rng(21)
    c = rng.standard_normal((12, 512)).astype(np.float32)
    z = (rng.standard_normal((12, 512)) * 3).astype(np.float32)
    # m = 1: every entry is its token
    assert np.array_equal(oracle.compress(c, z, 1), c)
    # equal weights: the mean of the m tokens
    e = oracle.compress(c, np.zeros_like(z), 3)
    assert np.allclose(e, c.reshape(4, 3, 512).mean(1), rtol=1e-6, atol=1e-7)
    # one token's weight far above the others': that token
    zz = np.zeros_like(z)
    zz[1::2] = 200.0
    assert np.array_equal(oracle.compress(c, zz, 2), c[1::2])
    # a constant added to a channel's Z over an entry's tokens changes nothing
    # (up to the float32 rounding of Z + shift, about 1e-5 here); a channel
    # or token mix-up would move the result by order 1
    shift = np.repeat(rng.standard_normal((6, 512)).astype(np.float32) * 50, 2, axis=0)
    a, b = oracle.compress(c, z, 2), oracle.compress(c, (z + shift).astype(np.float32), 2)
    assert np.allclose(a, b, rtol=0, atol=1e-4)


def test_compress_two_tokens_closed_form():
    """m = 2: the softmax of two weights is the logistic function of their
    difference, so e = C1 + sigma(z0 - z1) (C0 - C1)."""
    rng = np.random.default_rng(22)
    c = rng.standard_normal((40, 512)).astype(np.float32)
    z = rng.standard_normal((40, 512)).astype(np.float32)
    c0, c1, z0, z1 = (a.astype(np.float64) for a in (c[0::2], c[1::2], z[0::2], z[1::2]))
    want = c1 + (c0 - c1) / (1.0 + np.exp(z1 - z0))
    assert np.allclose(oracle.compress(c, z, 2), want, rtol=1e-6, atol=1e-7)


# ---------------------------------------------------------------------------
# indexer-K projection: y = x W (fp32 multiply-add chain), then MXFP4 codes
# ---------------------------------------------------------------------------

def _spec_mx_codes(y, bl):
    """E2M1 codes and E8M0 scales of one row y (float32) with blocks of bl,
    from the OCP MX scale rule and exact nearest-even rounding."""
    e2m1 = [Fraction(z).limit_denominator(2) for z in E2M1_SPEC]
    codes, scales = [], []
    for b0 in range(0, len(y), bl):
        amax = float(np.max(np.abs(y[b0:b0 + bl])))
        se = max(math.frexp(amax)[1] - 3, -127) if amax > 0 else 0
        scales.append(se + 127)
        for z in y[b0:b0 + bl]:
            q = Fraction(float(z)) / Fraction(2) ** se
            codes.append(_nearest_even(abs(q), e2m1) | (8 if q < 0 else 0))
    return np.array([codes[2 * i] | (codes[2 * i + 1] << 4) for i in range(len(y) // 2)], np.uint8), scales


@pytest.mark.parametrize("k_fmt", [0, 1])
def test_index_k_project_selection_matrix(k_fmt):
    """W picks and scales single channels (one nonzero per column, a power of
    two), so every multiply-add chain is exact: y[o] = 2^s x[p(o)].  The codes
    and scales equal the spec encoder's on that y."""
    rng = np.random.default_rng(31)
    x = rng.standard_normal((5, 512)).astype(np.float32) * np.float32(3.0)
    W = np.zeros((512, 128), np.float32)
    perm = rng.permutation(512)[:128]
    sh = rng.integers(-3, 4, size=128)
    W[perm, np.arange(128)] = np.exp2(sh).astype(np.float32)
    dst = np.array([4, 0, 2, 6, 1])
    kf, ks = oracle.index_k_project(x, W, dst, k_fmt, 8)
    for e in range(5):
        y = (x[e, perm] * np.exp2(sh)).astype(np.float32)
        codes, scales = _spec_mx_codes(y, 32 if k_fmt == 1 else 128)
        assert np.array_equal(kf[dst[e]], codes), e
        assert list(np.atleast_1d(ks[dst[e]])) == scales, e
    assert not kf[[3, 5, 7]].any()


def test_index_k_project_chain_order():
    """The projection is the fp32 multiply-add chain in ascending channel
    order: y equals that chain evaluated in exact rationals with one rounding
    per step, bit for bit, on values whose products are not exact (a tree or
    a reversed order would differ in the last bits of most outputs)."""
    rng = np.random.default_rng(32)
    x = rng.standard_normal((1, 512)).astype(np.float32)
    W = (rng.standard_normal((512, 128)) * 0.05).astype(np.float32)
    _, _, y = oracle.index_k_project(x, W, np.array([0]), 0, 1, want_y=True)
    for o in (0, 77, 127):
        acc = Fraction(0)
        for k in range(512):
            acc = Fraction(rne_f32(Fraction(float(x[0, k])) * Fraction(float(W[k, o])) + acc))
        assert y[0, o] == float(acc), o


@pytest.mark.parametrize("k_fmt", [0, 1])
def test_index_k_project_rotates_like_the_append(k_fmt):
    """With the entry's angles the projection takes the entry before RoPE.
    The identity angle changes nothing; a quarter turn maps (a, b) to (-b, a)
    exactly, so it equals the projection of the pre-turned x; for any angle,
    a selection matrix that reads rotated channels gives 2^s times each
    rotated value, within the rounding of two products and a sum of the
    float64 rotation (a swapped cos and sin, a wrong sign or a wrong pair
    would miss by order 1)."""
    rng = np.random.default_rng(33)
    n = 6
    x = rng.standard_normal((n, 512)).astype(np.float32)
    W = (rng.standard_normal((512, 128)) * 0.05).astype(np.float32)
    dst = np.array([3, 0, 5, 1, 4, 2])
    ident = np.zeros((n, 32, 2), np.float32)
    ident[..., 0] = 1.0
    quarter = np.zeros((n, 32, 2), np.float32)
    quarter[..., 1] = 1.0
    xt = x.copy()
    xt[:, 448::2], xt[:, 449::2] = -x[:, 449::2], x[:, 448::2]
    plain = oracle.index_k_project(x, W, dst, k_fmt, n, want_y=True)
    for got, want in zip(oracle.index_k_project(x, W, dst, k_fmt, n, want_y=True, cs=ident), plain):
        assert np.array_equal(got, want)
    turned = oracle.index_k_project(xt, W, dst, k_fmt, n, want_y=True)
    for got, want in zip(oracle.index_k_project(x, W, dst, k_fmt, n, want_y=True, cs=quarter), turned):
        assert np.array_equal(got, want)
    assert not np.array_equal(turned[2], plain[2])
    cs = _angles(rng, n)
    Ws = np.zeros((512, 128), np.float32)
    pick = 448 + rng.permutation(64)
    sh = rng.integers(-2, 3, size=64)
    Ws[pick, np.arange(64)] = np.exp2(sh).astype(np.float32)
    Ws[np.arange(64), 64 + np.arange(64)] = 1.0  # unrotated channels pass through
    _, _, y = oracle.index_k_project(x, Ws, dst, k_fmt, n, want_y=True, cs=cs)
    rot = x.astype(np.float64).copy()
    co, si = cs[..., 0].astype(np.float64), cs[..., 1].astype(np.float64)
    p, q = x[:, 448::2].astype(np.float64), x[:, 449::2].astype(np.float64)
    rot[:, 448::2], rot[:, 449::2] = p * co - q * si, p * si + q * co
    mag = np.empty_like(rot)
    mag[:, 448::2], mag[:, 449::2] = np.abs(p * co) + np.abs(q * si), np.abs(p * si) + np.abs(q * co)
    want = rot[:, pick] * np.exp2(sh)
    # two rounded products and their rounded sum: at most 2^-24 of each
    # product's magnitude plus half an ulp of the result, here doubled
    bound = (mag[:, pick] * 2.0 ** -23 + np.abs(rot[:, pick]) * 2.0 ** -23) * np.exp2(sh)
    assert np.all(np.abs(y[:, :64] - want) <= bound)
    assert np.array_equal(y[:, 64:], x[:, :64])


# ---------------------------------------------------------------------------
# RoPE and cast around attention
# ---------------------------------------------------------------------------

def _bf16_rne_spec(v):
    """Nearest bf16 (ties to an even last mantissa bit) of a finite float32,
    by exact comparison with the two neighbouring bf16 values."""
    f = Fraction(float(v))
    u = int(np.float32(v).view(np.uint32))
    lo = u & 0xFFFF0000
    hi = lo + 0x10000
    flo = Fraction(float(np.uint32(lo).view(np.float32)))
    fhi = Fraction(float(np.uint32(hi).view(np.float32)))
    dl, dh = abs(f - flo), abs(fhi - f)
    pick = lo if dl < dh or (dl == dh and ((lo >> 16) & 1) == 0) else hi
    return pick >> 16


def test_rope_cast_zero_angle_is_the_bf16_cast_and_ties_go_even():
    rng = np.random.default_rng(41)
    x = rng.standard_normal((2, 3, 512)).astype(np.float32)
    x[0, 0, :4] = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 1 + 2 ** -9], np.float32)  # two ties, one not
    cs = np.zeros((2, 32, 2), np.float32)
    cs[..., 0] = 1.0
    got = oracle.rope_cast(x, cs, False)
    want = np.vectorize(_bf16_rne_spec, otypes=[np.uint16])(x)
    assert np.array_equal(got, want)
    assert list(got[0, 0, :2]) == [0x3F80, 0x3F82]  # 1 + 2^-8 -> 1 (even); 1 + 3 2^-8 -> 1 + 2^-6 (even)


# float32 bit patterns and their bf16 to nearest even, from the format's
# definition (sign, 8-bit exponent, 7 stored fraction bits; NaNs stay NaNs
# with the quiet bit set and the sign and leading payload kept)
BF16_SPECIAL = [
    (0x7FC00001, 0x7FC0), (0xFFC00001, 0xFFC0),   # quiet NaNs
    (0x7F800001, 0x7FC0), (0xFF800001, 0xFFC0),   # signalling NaNs: not infinities
    (0x7FBFFFFF, 0x7FFF),                          # a full payload does not carry into the sign
    (0x7F800000, 0x7F80), (0xFF800000, 0xFF80),   # infinities
    (0x7F7FFFFF, 0x7F80), (0xFF7FFFFF, 0xFF80),   # the largest float32 rounds to infinity
    (0x7F7F8000, 0x7F80),                          # halfway above the largest bf16 (odd): infinity
    (0x7F7F7FFF, 0x7F7F),                          # just below halfway: the largest bf16
    (0x7F7E8000, 0x7F7E),                          # halfway, even below: stays
    (0x00000001, 0x0000), (0x00008000, 0x0000),   # the smallest subnormal; a tie to the even zero
    (0x00018000, 0x0002),                          # a subnormal tie to even upwards
    (0x80000000, 0x8000), (0x00000000, 0x0000),   # signed zeros
    (0x3F808000, 0x3F80), (0x3F818000, 0x3F82),   # ties in the normal range
]


def test_rope_cast_bf16_specials():
    x = np.zeros((1, 1, 512), np.float32)
    bits = np.array([b for b, _ in BF16_SPECIAL], np.uint32)
    x[0, 0, : len(bits)] = bits.view(np.float32)
    cs = np.zeros((1, 32, 2), np.float32)
    cs[..., 0] = 1.0
    got = oracle.rope_cast(x, cs, False)[0, 0, : len(bits)]
    assert [int(v) for v in got] == [w for _, w in BF16_SPECIAL]


def test_rope_cast_quarter_turns_and_inverse():
    """A quarter turn maps (a, b) to (-b, a) exactly, its inverse (-sin) maps
    (a, b) to (b, -a); for any angle the inverse undoes the rotation to within
    the casts' rounding."""
    rng = np.random.default_rng(42)
    x = rng.standard_normal((3, 2, 512)).astype(np.float32)
    q = np.zeros((3, 32, 2), np.float32)
    q[..., 1] = 1.0
    fwd = oracle.rope_cast(x, q, False)
    inv = oracle.rope_cast(x, q, True)
    ident = np.zeros_like(q)
    ident[..., 0] = 1.0
    xt = x.copy()
    xt[..., 448::2], xt[..., 449::2] = -x[..., 449::2], x[..., 448::2]
    assert np.array_equal(fwd, oracle.rope_cast(xt, ident, False))
    xi = x.copy()
    xi[..., 448::2], xi[..., 449::2] = x[..., 449::2], -x[..., 448::2]
    assert np.array_equal(inv, oracle.rope_cast(xi, ident, False))
    th = rng.uniform(-np.pi, np.pi, size=(3, 32))
    cs = np.stack([np.cos(th), np.sin(th)], -1).astype(np.float32)
    rot = (oracle.rope_cast(x, cs, False).astype(np.uint32) << 16).view(np.float32)
    back = (oracle.rope_cast(rot, cs, True).astype(np.uint32) << 16).view(np.float32)
    # two bf16 casts (2^-9 relative each) around a rotation: the error of a
    # rotated channel scales with its pair's magnitude, the rest with itself
    mag = np.abs(x).astype(np.float64)
    pair = np.maximum(np.abs(x[..., 448::2]), np.abs(x[..., 449::2]))
    mag[..., 448::2] = pair
    mag[..., 449::2] = pair
    assert np.all(np.abs(back.astype(np.float64) - x) <= 2 ** -6 * mag + 1e-30)
