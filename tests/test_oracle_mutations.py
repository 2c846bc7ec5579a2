"""The pins catch planted mistakes: each case copies the oracle's C source,
plants one plausible mistake (a dropped term, a swapped nibble, a reversed tie,
an off-by-one, an unfused sum, ...), builds it, and runs the pins that cover
that step against it in a separate process.  Every mutant must fail a pin; the
unmodified copy must pass the same pins."""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "csa2_oracle.c")

# (name, text in the source, replacement, pins to run (pytest -k))
MUTATIONS = [
    ("relu_dropped", "float rh = fmaxf(d, 0.0f) * sq;", "float rh = d * sq;", "score"),
    ("relu_dropped_mx", "acc = fmaf(c->w[r * c->H + h], fmaxf(d, 0.0f), acc);",
     "acc = fmaf(c->w[r * c->H + h], d, acc);", "mxfp4"),
    ("key_nibbles_swapped", "uint8_t byte = c->k[e * 64 + ch / 2];\n    uint8_t nib = (ch & 1) ? (byte >> 4) : (byte & 15);",
     "uint8_t byte = c->k[e * 64 + ch / 2];\n    uint8_t nib = (ch & 1) ? (byte & 15) : (byte >> 4);", "score"),
    ("tie_to_higher_position", "return (x->pos < y->pos) ? -1 : (x->pos > y->pos);",
     "return (x->pos > y->pos) ? -1 : (x->pos < y->pos);", "topk"),
    ("block_sum_for_max", "if (s > m) m = s;", "m = (m == -INFINITY ? 0.0f : m) + s;", "block_pool"),
    ("visibility_off_by_one", "int64_t v = (t + 1) / m;", "int64_t v = (t + 2) / m;", "visib"),
    ("head_sum_unfused", "acc = fmaf(c->w[r * c->H + h], rh, acc);", "acc = acc + c->w[r * c->H + h] * rh;",
     "head_sum_order"),
    ("key_scale_dropped", "return acc * (float)orc_e8m0(c->k_sc[e]);", "return acc;", "score"),
    ("wrong_scale_block", "return orc_e2m1(nib) * orc_e8m0(kv_sc[e * 16 + ch / 32]);",
     "return orc_e2m1(nib) * orc_e8m0(kv_sc[e * 16 + ch / 64]);", "gather"),
    ("window_off_by_one", "int64_t u_lo = t - c->W + 1;", "int64_t u_lo = t - c->W;", "dense or window or replay"),
    ("e2m1_subnormal", "double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);",
     "double mag = (e == 0) ? 1.0 * m : ldexp(1.0 + 0.5 * m, e - 1);", "e2m1"),
    ("bf16_ties_up", "if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) == 1.0)) r += 1.0;", "if (frac >= 0.5) r += 1.0;",
     "rope"),
    ("mx_flag_dropped", "        if (total >= (1LL << 24)) ((score_ctx*)c)->status = 2;\n        float d = (float)ldexp((double)dot, emin - 2);",
     "        float d = (float)ldexp((double)dot, emin - 2);", "cancel"),
    ("rope_sin_sign", "v[448 + 2 * i] = ac - bs;", "v[448 + 2 * i] = ac + bs;", "kv_append"),
    ("projection_rope_dropped", "if (cs) rope_latent(v, cs + e * 64);", "", "index_k_project"),
]


def _build_and_run(tmp, name, text, k):
    src = open(SRC).read()
    if text is not None:
        old, new = text
        assert src.count(old) == 1, f"{name}: the planted text must occur once"
        src = src.replace(old, new)
    csrc = os.path.join(tmp, name + ".c")
    so = os.path.join(tmp, name + ".so")
    open(csrc, "w").write(src)
    subprocess.check_call(["gcc", *oracle.CFLAGS, csrc, "-o", so, "-lm"])
    env = dict(os.environ, CSA2_ORACLE_SO=so, CSA2_ORACLE_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_oracle_pins.py"), "-x", "-q",
                        "-p", "no:cacheprovider", "-k", k], cwd=ROOT, env=env, capture_output=True, text=True)
    return r.returncode, r.stdout[-600:]


def test_pins_catch_planted_mistakes():
    with tempfile.TemporaryDirectory() as tmp:
        jobs = [(name, (old, new), k) for name, old, new, k in MUTATIONS]
        jobs += [("unmodified_" + k.replace(" ", "_"), None, k) for k in sorted({m[3] for m in MUTATIONS})]
        with ThreadPoolExecutor(4) as ex:
            res = list(ex.map(lambda j: (j[0], j[1] is None) + _build_and_run(tmp, *j), jobs))
    for name, clean, rc, out in res:
        if clean:
            assert rc == 0, f"the unmodified oracle fails pins '{name}':\n{out}"
        else:
            assert rc == 1, f"mutant {name} passed its pins (rc {rc}):\n{out}"
