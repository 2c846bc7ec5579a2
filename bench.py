#!/usr/bin/env python3
"""Benchmark of the CSA2 hot path on one MI355X.

Default workload (decode_c1): 64 sequences x 131,072 global entries (ratio 1),
one query each at t = N-1, one Full-mode layer: lightning-indexer scan over the
FP4 indexer K of every visible entry, Top-512, gather + dequant of the MXFP4
main-KV latents, SWA-128, latent attention with 64 heads of 512.  A step is
one csa2_layer_chain call over the whole batch, i.e. one decode layer-step.

Prints ONE JSON line with the contract fields plus:
  roofline      the dominant kernel (the indexer scan), its algorithmic bytes per
                launch / its mean launch time, timed here with HIP events on the
                stream it runs on, against the 8 TB/s HBM peak
  cpu_baseline  the CPU oracle on a bounded sample of the same workload
  prefill_index the prefill indexer (8,192 E4M3 queries x 131,072 entries at
                ratio 2, causal) in TFLOP/s of algorithmic FLOPs
  workloads     the layer chain of the other four workloads (decode_c0; the
                decoder chain of chain_c2 and ragged_c4 with block pool, Reindex
                and Reuse layers; the prefill_c3 chunk): time per chain and its
                algorithmic HBM bytes (decode) or FLOPs (prefill)
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "CSA2 decode layer-steps/s at 128K ctx + achieved HBM GB/s; prefill index TFLOP/s"
HBM_PEAK_GBS = 8000.0
# the pages' exact cache configuration (report 2.4.4 and 4.2.1): 32 indexer
# heads, E2M1 main KV with an E4M3 scale per 16 channels, MXFP4 indexer q and
# K, FP8 SWA (as OCP MXFP8); Q_MXFP4 = 2 in the generator
PAGES_FMT = dict(kv_fmt=1, swa_fmt=1, q_fmt=2, H=32)
FP8_PEAK_TFLOPS = 5000.0
BF16_PEAK_TFLOPS = 2500.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--n-seq", type=int, default=64)
    ap.add_argument("--n", type=int, default=131072)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--cpu-sample-seqs", type=int, default=64)
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the layer-chain timings of the other four workloads")
    ap.add_argument("--workload", default="decode_c1",
                    choices=["decode_c1", "decode_c0", "chain_c2", "prefill_c3", "ragged_c4", "replay_c5",
                             "encoder_replay", "decode_step_40", "decode_step_40_pages_fmt"],
                    help="decode_c1 (default) prints the full line; the others time their layer chain only")
    ap.add_argument("--profile-pass", action="store_true",
                    help="short run for hardware-counter collection: a few steps, a few scan launches and one "
                         "512 MiB device copy that calibrates the byte counters")
    a = ap.parse_args()
    if a.profile_pass:
        a.steps, a.warmup, a.no_cpu_baseline, a.no_prefill, a.no_workloads = 3, 1, True, True, True
    return a


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "scan_traffic_decode_c1.json")
SCAN_SOURCES = [os.path.join(ROOT, "compressed_sparse_attention_amd", "csrc", f)
                for f in ("k_index_score.hip", "csa2_internal.h")]


def scan_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in SCAN_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per scan launch from the committed counter runs, if they were
    taken on the kernel source as it is now; otherwise None."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    return rec.get("bytes_per_launch") if rec.get("source_sha") == scan_source_hash() else None


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def hip_events(n):
    """n pairs of HIP events from the HIP runtime torch has loaded (same soname)."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so.7")
    pairs = []
    for _ in range(2 * n):
        e = ctypes.c_void_p()
        if hip.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        pairs.append(e)
    return hip, pairs[:n], pairs[n:]


def hip_elapsed_ms(hip, a, b):
    import ctypes
    ms = ctypes.c_float()
    if hip.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
        raise RuntimeError("hipEventElapsedTime failed")
    return ms.value


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path (--gpus 1).", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import synth
    from compressed_sparse_attention_amd import csa2 as C

    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from gpu_util import DevWorkload, prepare_chain, run_chain

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    C.lib()
    dev = torch.device("cuda:0")
    if args.workload.startswith("decode_step_40"):
        res = {"metric": METRIC, "workload": args.workload}
        fmt = PAGES_FMT if args.workload.endswith("pages_fmt") else {}
        res.update(bench_step_40(synth, torch, dev, reps=args.steps, **fmt))
        print(json.dumps(res), flush=True)
        return
    if args.workload != "decode_c1":
        return chain_only(args, synth, C, torch, dev)

    t0 = time.time()
    wl = synth.config("decode_c1", n_seq=args.n_seq, n=args.n)
    log(f"[bench] generated decode_c1 inputs in {time.time() - t0:.1f}s")
    dw = DevWorkload(wl, dev)
    # a second copy of every cache so that consecutive steps do not hit in the 256 MB MALL
    dw2 = DevWorkload.__new__(DevWorkload)
    dw2.__dict__.update(dw.__dict__)
    dw2.k_idx, dw2.k_sc, dw2.kv, dw2.kv_sc = dw.k_idx.clone(), dw.k_sc.clone(), dw.kv.clone(), dw.kv_sc.clone()
    nq, n_layers = wl.total_q, len(wl.layers)
    ws = C.workspace(C.csa2_workspace_size(C.CSA2_WS_LAYER_CHAIN, dw.batch, wl.K, wl.max_blocks, n_layers), dev)
    copies = [dw, dw2]
    calls = [prepare_chain(d, want_idx=False, want_lse=False, ws=ws, pool=False)[0] for d in copies]

    # the chain stamps a pair of HIP events with its index-scan kernel's
    # dispatch (on the stream that kernel runs on) in every SCAN_EVERY-th timed
    # step: each stamped dispatch leaves the queue idle for a few us around
    # it, which would otherwise count in every step
    SCAN_EVERY = 4
    timed_scans = [i for i in range(args.steps) if i % SCAN_EVERY == SCAN_EVERY - 1] or [args.steps - 1]
    hip, ev_b, ev_e = hip_events(len(timed_scans))
    ev_of = {i: k for k, i in enumerate(timed_scans)}

    def step(i, timed=False):
        c = calls[i % 2]
        prm = c.keep[2]
        k = ev_of.get(i) if timed else None
        prm.scan_begin, prm.scan_end = (ev_b[k].value, ev_e[k].value) if k is not None else (None, None)
        c()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        step(i, timed=True)
    end.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / args.steps
    scan_each = [hip_elapsed_ms(hip, ev_b[k], ev_e[k]) for k in range(len(timed_scans))]
    scan_ms = sum(scan_each) / len(scan_each)
    log(f"[bench] layer chain: {ms_step * 1000:.1f} us per decode layer-step; its index scan "
        f"{scan_ms * 1000:.1f} us (min {min(scan_each) * 1000:.1f})")

    # algorithmic bytes of one layer-step: scan 65 B per visible entry per sequence,
    # per query: q/w (64 x (64 + 1 + 4) B), gathered 512 x 272 B, SWA 128 x 1024 B,
    # main q 64 x 512 x 2 B, output 64 x 512 x 4 B, indices 512 x 4 B
    vis_total = int(sum(min(int(wl.n_entries[b]), int(t) + 1) for b, t in zip(wl.row_seq, wl.q_pos)))
    per_q = wl.H * (64 + 1 + 4) + wl.K * 272 + wl.W * 1024 + wl.Hm * 512 * 2 + wl.Hm * 512 * 4 + wl.K * 4
    step_bytes = vis_total * 65 + nq * per_q
    step_gbs = step_bytes / (ms_step * 1e-3) / 1e9

    # dominant kernel: the chain's index scan (timed above)
    scan_bytes = vis_total * 65 + nq * wl.H * (64 + 1 + 4)
    scan_gbs = scan_bytes / (scan_ms * 1e-3) / 1e9
    log(f"[bench] scan kernel: {scan_ms * 1000:.1f} us, {scan_gbs:.0f} GB/s algorithmic")

    ceiling = measured_ceiling(torch, dev, scan_bytes)
    log(f"[bench] plain device copy {ceiling['copy_gbs']:.0f} GB/s (read + write), plain read "
        f"{ceiling['read_gbs']:.0f} GB/s over {scan_bytes / 1e6:.0f} MB")
    result = {
        "metric": METRIC,
        "value": round(1000.0 / ms_step, 2),
        "unit": "layer-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4+bf16",
        "data": "synthetic",
        "config": {"workload": "decode_c1", "batch": wl.n_seq, "entries_per_seq": int(wl.n_entries[0]),
                   "ratio": wl.ratio, "layers": 1, "mode": "full", "topk": wl.K, "swa_window": wl.W,
                   "index_heads": wl.H, "main_heads": wl.Hm, "latent_dim": 512,
                   "step_algorithmic_bytes": step_bytes, "step_hbm_gbs": round(step_gbs, 1),
                   "sequence_layer_steps_per_s": round(wl.n_seq * 1000.0 / ms_step, 1)},
        "roofline": {"kernel": "k_score_decode<64,1,2> (indexer scan writing per-chunk candidate lists)",
                     "bound": "hbm", "achieved": round(scan_gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(scan_gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(), "mean_launch_us": round(scan_ms * 1000, 2),
                     "algorithmic_bytes_per_launch": scan_bytes,
                     "measured_ceiling": dict(ceiling, frac_of_read=round(scan_gbs / ceiling["read_gbs"], 4))},
    }
    if args.profile_pass:  # calibration copy for the byte counters
        a = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        result["calibration_copy_bytes"] = 512 << 20
        result["scan_source_sha"] = scan_source_hash()

    if not args.no_prefill:
        result["prefill_index"] = bench_prefill(args, C, synth, torch, dev)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args, wl, dw, C, run_chain)

    if not args.no_workloads:
        del dw, dw2, copies, calls, ws
        torch.cuda.empty_cache()
        result["workloads"] = bench_workloads(synth, C, torch, dev)

    print(json.dumps(result), flush=True)


def measured_ceiling(torch, dev, nbytes, reps=10):
    """Secondary denominators for the scan: what plain torch kernels reach on
    this device over the same byte count.  A device-to-device copy (bytes read
    + bytes written per second) and a plain read (an int64 sum of the buffer:
    bytes read per second).  Buffers are rotated so that the 256 MB MALL does
    not serve repeats."""
    n = (nbytes // 8) * 8
    bufs = [torch.ones(n // 8, dtype=torch.int64, device=dev) for _ in range(2)]
    dst = torch.empty_like(bufs[0])
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn):
        for i in range(3):
            fn(bufs[i & 1])
        torch.cuda.synchronize()
        best = None
        for i in range(reps):
            s.record()
            fn(bufs[i & 1])
            e.record()
            torch.cuda.synchronize()
            ms = s.elapsed_time(e)
            best = ms if best is None else min(best, ms)
        return best

    t_copy = timed(lambda a: dst.copy_(a))
    t_read = timed(lambda a: a.sum())
    del bufs, dst
    torch.cuda.empty_cache()
    return {"copy_gbs": round(2 * n / (t_copy * 1e-3) / 1e9, 1), "read_gbs": round(n / (t_read * 1e-3) / 1e9, 1),
            "bytes": n, "how": "best of 10: torch copy_ (read + write) and int64 sum (read) of the scan's byte count"}


def chain_only(args, synth, C, torch, dev):
    """Time the layer chain of another workload (one call = all its layers)."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from gpu_util import DevWorkload, prepare_chain

    t0 = time.time()
    wl = synth.config(args.workload)
    log(f"[bench] generated {args.workload} in {time.time() - t0:.1f}s")
    dw = DevWorkload(wl, dev)
    call = prepare_chain(dw, want_idx=False, want_lse=False)[0]
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(args.steps):
        call()
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / args.steps
    n_layers = len(wl.layers)
    res = {"metric": METRIC, "workload": args.workload, "ms_per_chain": round(ms, 4), "layers": n_layers,
           "value": round(n_layers * 1000.0 / ms, 2), "unit": "layer-steps/s", "rows": wl.total_q,
           "entries": wl.total_entries}
    print(json.dumps(res), flush=True)


def chain_bytes(wl, outs, pool_pos, pool_count):
    """Algorithmic HBM bytes of one decode step of a layer chain, from the
    realised selections: the Full layer's scan (65 B per visible entry, read
    once per sequence; 68 B in the MXFP4 indexer format) and query/weights;
    each Reindex layer's gathered indexer-K rows (the union of a sequence's
    pools, 65 or 68 B each); per layer and
    row the gathered main-KV rows (272 B per selected entry; 288 B with E4M3
    scales per 16 channels), the SWA rows (1,024 B; 528 B in MXFP8), the main
    query, the output and the indices."""
    import numpy as np

    H, Hm, K, W = wl.H, wl.Hm, wl.K, wl.W
    vis = np.minimum(wl.n_entries[wl.row_seq], (wl.q_pos.astype(np.int64) + 1) // wl.ratio)
    seq_vis = np.zeros(wl.n_seq, np.int64)
    np.maximum.at(seq_vis, wl.row_seq, vis)
    n_swa = np.minimum(W, wl.q_pos.astype(np.int64) + 1)
    mx = wl.layers and any(L.q_fmt == synth_mode_q("MXFP4") for L in wl.layers)
    k_row = 68 if mx else 65
    qw = wl.total_q * H * (64 + (4 if mx else 1) + 4)
    total = 0
    for L, o in zip(wl.layers, outs):
        if L.mode == synth_mode("FULL"):
            total += int(seq_vis.sum()) * k_row + qw
        elif L.mode == synth_mode("REINDEX"):
            pp, pc = pool_pos.cpu().numpy(), pool_count.cpu().numpy()
            for b in range(wl.n_seq):
                rows = np.nonzero(wl.row_seq == b)[0]
                u = np.unique(np.concatenate([pp[r, :pc[r]] for r in rows])) if len(rows) else []
                total += len(u) * k_row
            total += qw
        n_sel = (o["idx"].cpu().numpy() >= 0).sum(axis=1) if L.mode != synth_mode("SWA_ONLY") else 0
        kv_row = 288 if getattr(wl, "kv_fmt", 0) == 1 else 272
        swa_row = 528 if getattr(wl, "swa_fmt", 0) == 1 else 1024
        total += int(np.sum(n_sel) * kv_row + n_swa.sum() * swa_row) + wl.total_q * (Hm * 512 * 6 + K * 4)
    return total


def synth_mode(name):
    import synth

    return getattr(synth, "MODE_" + name)


def synth_mode_q(name):
    import synth

    return getattr(synth, "Q_" + name)


def bench_workloads(synth, C, torch, dev):
    """The layer chain of the other workloads: one call = every layer of one
    decode step (or of the prefill chunk, or of the 128-token decoder replay)
    for the whole batch."""
    import numpy as np

    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from gpu_util import DevWorkload, prepare_chain

    res = {}
    # decode_c1_pages_fmt: decode_c1 in the pages' exact configuration: 32
    # indexer heads, main KV with E4M3 scales per 16 channels, indexer q and K
    # in OCP MXFP4 (the 356-byte position) and SWA in FP8 (as OCP MXFP8)
    for name, reps in (("decode_c0", 20), ("decode_c1_pages_fmt", 10), ("chain_c2", 5), ("ragged_c4", 5),
                       ("prefill_c3", 3), ("replay_c5", 3), ("encoder_replay", 5)):
        t0 = time.time()
        if name == "decode_c1_pages_fmt":
            wl = synth.config("decode_c1", **PAGES_FMT)
        else:
            wl = synth.config(name)
        dw = DevWorkload(wl, dev)
        call, outs, (pb, pp, pc) = prepare_chain(dw, want_idx=True, want_lse=False)
        call()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            call()
        e.record()
        torch.cuda.synchronize()
        ms = s.elapsed_time(e) / reps
        n_layers = len(wl.layers)
        r = {"ms_per_chain": round(ms, 4), "layers": n_layers, "rows": wl.total_q,
             "entries": wl.total_entries, "layer_steps_per_s": round(n_layers * 1000.0 / ms, 1)}
        if name in ("prefill_c3", "replay_c5", "encoder_replay"):
            # many query rows share each scan: FLOP/s.  Full layers score every
            # visible entry, Reindex layers their pool; attention reads the
            # selected entries and the (replay-cut) window
            t = wl.q_pos.astype(np.int64)
            vis = np.minimum(wl.n_entries[wl.row_seq], (t + 1) // wl.ratio)
            n_full = sum(1 for L in wl.layers if L.mode == synth.MODE_FULL)
            n_reindex = sum(1 for L in wl.layers if L.mode == synth.MODE_REINDEX)
            pooled = float(pc.cpu().numpy().sum()) if n_reindex and pc is not None else 0.0
            idx_flops = 2.0 * wl.H * 128 * (n_full * float(vis.sum()) + n_reindex * pooled)
            lo = np.maximum(t - wl.W + 1, 0)
            if wl.replay_s is not None:
                lo = np.maximum(lo, wl.replay_s[wl.row_seq].astype(np.int64))
            n_swa = t - lo + 1
            keys = sum(float((o["idx"].cpu().numpy() >= 0).sum()) + float(n_swa.sum()) for o in outs)
            attn_flops = keys * wl.Hm * 512 * 4  # Q K^T and P V
            r.update({"index_flops": idx_flops, "attn_flops": attn_flops,
                      "tflops": round((idx_flops + attn_flops) / (ms * 1e-3) / 1e12, 1)})
        else:
            nb = chain_bytes(wl, outs, pp, pc)
            gbs = nb / (ms * 1e-3) / 1e9
            r.update({"algorithmic_bytes": nb, "hbm_gbs": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)})
        log(f"[bench] {name}: {ms:.3f} ms per chain of {n_layers} layers ({time.time() - t0:.0f} s incl. inputs)")
        res[name] = r
        del dw, outs, call, pb, pp, pc, wl
        torch.cuda.empty_cache()
    res["decode_step_40"] = bench_step_40(synth, torch, dev)
    # the same step in the pages' exact configuration (32 indexer heads,
    # E4M3/16 main KV, MXFP4 indexer, FP8 SWA as MXFP8)
    res["decode_step_40_pages_fmt"] = bench_step_40(synth, torch, dev, **PAGES_FMT)
    for kv_fmt in (1, 0):
        res["kv_append_e4m3" if kv_fmt == 1 else "kv_append_mxfp4"] = bench_append(C, torch, dev, kv_fmt)
    res["attn_rope"] = bench_attn_rope(synth, C, torch, dev)
    res["compress"] = bench_compress(C, torch, dev)
    res["index_k_project"] = bench_project(C, torch, dev)
    res["index_k_project_rope"] = bench_project(C, torch, dev, rope=True)
    return res


def bench_attn_rope(synth, C, torch, dev, reps=20):
    """The RoPE steps around attention (the report's RoPE-attention-RoPE-cast
    flow) fused into the attention call (bf16 query before RoPE in, bf16 out),
    against plain attention (bf16 query in, f32 out) and against the three
    separate calls (query rotation and cast, attention, output rotation and
    cast), at a decode shape (64
    rows) and a replay shape (2,048 rows), 64 heads, Top-512 of 32,768
    entries plus a 128-token window."""
    import numpy as np

    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from gpu_util import SCALE, DevWorkload

    out = {}
    for name, n_seq, T in (("decode_64_rows", 64, 1), ("replay_2048_rows", 16, 128)):
        wl = synth.make_workload("attn_rope", 77, [32768] * n_seq, T, [(20, synth.MODE_FULL, False)])
        dw = DevWorkload(wl, dev)
        nq, Hm = wl.total_q, wl.Hm
        g = torch.Generator(device=dev).manual_seed(11)
        idx = torch.sort(torch.randint(0, 32768 - T, (nq, 512), generator=g, device=dev), dim=1).values.to(torch.int32)
        q32 = torch.randn((nq, Hm, 512), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16).float()
        q16 = q32.to(torch.bfloat16).view(torch.uint16)  # the query before RoPE
        th = torch.rand((nq, 32), generator=g, device=dev) * 6.2831853
        cs = torch.stack([torch.cos(th), torch.sin(th)], -1).contiguous()
        L = dw.layers[0]
        ws = C.workspace(C.csa2_workspace_size(C.CSA2_WS_SPARSE_ATTN, dw.batch, 512), dev)
        qb = C.csa2_rope_cast(q32, cs)
        o32 = torch.empty((nq, Hm, 512), dtype=torch.float32, device=dev)
        o16 = torch.empty((nq, Hm, 512), dtype=torch.uint16, device=dev)

        def plain():
            C.csa2_sparse_attn(dw.batch, qb, dw.kv, dw.kv_sc, idx, L["swa"], dw.swa, SCALE, out=o32, want_lse=False,
                               ws=ws)

        def three():
            C.csa2_rope_cast(q32, cs, out=qb)
            plain()
            C.csa2_rope_cast(o32, cs, inverse=True, out=o16)

        def fused():
            C.csa2_sparse_attn_rope(dw.batch, q16, cs, dw.kv, dw.kv_sc, idx, L["swa"], dw.swa, SCALE, out=o16,
                                    want_lse=False, ws=ws)

        r = {}
        for label, fn in (("plain_attention_us", plain), ("three_calls_us", three), ("fused_us", fused)):
            fn()
            torch.cuda.synchronize()
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            for _ in range(reps):
                fn()
            e.record()
            torch.cuda.synchronize()
            r[label] = round(s.elapsed_time(e) * 1000.0 / reps, 2)
        log(f"[bench] attention with RoPE, {name}: plain {r['plain_attention_us']} us, three calls "
            f"{r['three_calls_us']} us, fused {r['fused_us']} us")
        r["rows"] = nq
        out[name] = r
        del dw, q32, q16, qb, o32, o16, ws, idx
        torch.cuda.empty_cache()
    return out


def bench_project(C, torch, dev, n=131072, reps=10, rope=False):
    """The indexer-K projection of 131,072 entries (one source layer of the
    prefill context): 2 x 512 x 128 flops an entry as float32 multiply-add
    chains (against the vector fp32 peak), then MXFP4 codes.  With `rope` the
    entries come before RoPE with their angles (the rotation is not counted)."""
    g = torch.Generator(device=dev).manual_seed(9)
    x = torch.randn((n, 512), generator=g, device=dev, dtype=torch.float32)
    W = torch.randn((512, 128), generator=g, device=dev, dtype=torch.float32) * 0.05
    th = torch.rand((n, 32), generator=g, device=dev, dtype=torch.float32) * 6.283
    cs = torch.stack([th.cos(), th.sin()], -1).contiguous() if rope else None
    dst = torch.arange(n, device=dev, dtype=torch.int64)
    kf = torch.empty((n, 64), dtype=torch.uint8, device=dev)
    ks = torch.empty((n, 4), dtype=torch.uint8, device=dev)
    C.csa2_index_k_project(x, W, dst, kf, ks, q_fmt=C.CSA2_Q_MXFP4, rope_cs=cs)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        C.csa2_index_k_project(x, W, dst, kf, ks, q_fmt=C.CSA2_Q_MXFP4, rope_cs=cs)
    e.record()
    torch.cuda.synchronize()
    us = s.elapsed_time(e) * 1000.0 / reps
    flops = 2.0 * n * 512 * 128
    tf = flops / (us * 1e-6) / 1e12
    log(f"[bench] index_k_project{' from entries before RoPE' if rope else ''}: {us:.1f} us for {n} entries, "
        f"{tf:.1f} TFLOP/s fp32")
    r = {"us": round(us, 2), "entries": n, "flops": flops, "tflops": round(tf, 2), "frac_fp32_vector_peak": round(tf / 157.3, 4)}
    del x, W, th, cs, dst, kf, ks
    torch.cuda.empty_cache()
    return r


def bench_compress(C, torch, dev, n=131072, m=2, reps=20):
    """The compressor over the 262,144-token prefill context at ratio 2:
    131,072 entries.  Algorithmic bytes per entry: m rows of C and of Z read
    (f32), one f32 row written."""
    g = torch.Generator(device=dev).manual_seed(8)
    c = torch.randn((n * m, 512), generator=g, device=dev, dtype=torch.float32)
    z = torch.randn((n * m, 512), generator=g, device=dev, dtype=torch.float32)
    out = torch.empty((n, 512), dtype=torch.float32, device=dev)
    C.csa2_compress(c, z, m, out=out)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        C.csa2_compress(c, z, m, out=out)
    e.record()
    torch.cuda.synchronize()
    us = s.elapsed_time(e) * 1000.0 / reps
    nb = n * (2 * m + 1) * 2048
    gbs = nb / (us * 1e-6) / 1e9
    log(f"[bench] compress (m {m}): {us:.1f} us for {n} entries, {gbs:.0f} GB/s")
    r = {"us": round(us, 2), "entries": n, "m": m, "algorithmic_bytes": nb, "hbm_gbs": round(gbs, 1),
         "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
    del c, z, out
    torch.cuda.empty_cache()
    return r


def bench_append(C, torch, dev, kv_fmt, n=131072, reps=20):
    """The cache append (RoPE on 64 channels, then FP4 quantisation) of
    131,072 entries, one source layer's cache of the 262,144-token prefill
    context at ratio 2.  Algorithmic bytes per entry: the f32 latent (2,048),
    its angles (256) and row index (8) read; the code row (256) and its scales
    (32 or 16) written."""
    g = torch.Generator(device=dev).manual_seed(7)
    x = torch.randn((n, 512), generator=g, device=dev, dtype=torch.float32)
    th = torch.rand((n, 32), generator=g, device=dev) * 6.2831853
    cs = torch.stack([torch.cos(th), torch.sin(th)], -1).contiguous()
    dst = torch.randperm(n, generator=g, device=dev).to(torch.int64)
    kv = torch.empty((n, 256), dtype=torch.uint8, device=dev)
    sc = torch.empty((n, 32 if kv_fmt == 1 else 16), dtype=torch.uint8, device=dev)
    C.csa2_kv_append(x, cs, dst, kv, sc, kv_fmt=kv_fmt)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        C.csa2_kv_append(x, cs, dst, kv, sc, kv_fmt=kv_fmt)
    e.record()
    torch.cuda.synchronize()
    us = s.elapsed_time(e) * 1000.0 / reps
    nb = n * (2048 + 256 + 8 + 256 + sc.shape[1])
    gbs = nb / (us * 1e-6) / 1e9
    log(f"[bench] kv_append (kv_fmt {kv_fmt}): {us:.1f} us for {n} entries, {gbs:.0f} GB/s")
    r = {"us": round(us, 2), "entries": n, "algorithmic_bytes": nb, "hbm_gbs": round(gbs, 1),
         "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
    del x, th, cs, dst, kv, sc
    torch.cuda.empty_cache()
    return r


def bench_step_40(synth, torch, dev, reps=5, **fmt):
    """One decode token of each of 64 sequences at 131,072 tokens through all 40
    layers: the two chains the layers form (the encoder layers 0..19 at ratio
    2 over 65,536 entries, with three Full layers each reading its own caches;
    the decoder at ratio 1 over 131,072 entries with the pool), run back to
    back on one stream and timed together."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from gpu_util import DevWorkload, prepare_chain

    t0 = time.time()
    wls = synth.decode_step_40(**fmt)
    dws = [DevWorkload(wl, dev) for wl in wls]
    calls = [prepare_chain(dw, want_idx=False, want_lse=False)[0] for dw in dws]

    def step():
        for c in calls:
            c()

    step()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        step()
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / reps
    n_layers = sum(len(wl.layers) for wl in wls)
    n_seq = wls[0].n_seq
    log(f"[bench] decode_step_40{' (pages formats)' if fmt else ''}: {ms:.3f} ms per 40-layer step of {n_seq} sequences ({time.time() - t0:.0f} s incl. inputs)")
    r = {"ms_per_step": round(ms, 4), "layers": n_layers, "sequences": n_seq, "tokens": int(wls[-1].n_entries[0]),
         "tokens_per_s": round(n_seq * 1000.0 / ms, 1), "layer_steps_per_s": round(n_layers * 1000.0 / ms, 1),
         "chains": [wl.name for wl in wls]}
    del calls, dws, wls
    torch.cuda.empty_cache()
    return r


def bench_prefill(args, C, synth, torch, dev):
    """Prefill indexer: 8,192 E4M3 query rows (t = 253,952..262,143) against
    131,072 entries (262,144 tokens at ratio 2), causal."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from gpu_util import DevWorkload

    wl = synth.config("prefill_c3", n_layers=1, Hm=16)
    dw = DevWorkload(wl, dev)
    L = dw.layers[0]
    nq = wl.total_q
    sc = torch.empty((nq, dw.batch.max_entries), dtype=torch.float32, device=dev)

    def run():
        C.csa2_index_score(dw.batch, wl.H, C.CSA2_Q_FP8, L["q_idx"], L["q_sc"], L["w"], dw.k_idx, dw.k_sc, scores=sc)

    run()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = max(3, args.steps // 4)
    s.record()
    for _ in range(reps):
        run()
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / reps
    pairs = int(sum(min(int(wl.n_entries[0]), (int(t) + 1) // 2) for t in wl.q_pos))
    flops = 2.0 * pairs * wl.H * 128
    tflops = flops / (ms * 1e-3) / 1e12
    log(f"[bench] prefill index: {ms:.2f} ms, {tflops:.0f} TFLOP/s")
    del sc
    return {"workload": "prefill_c3 index score", "ms": round(ms, 3), "pairs": pairs, "flops": flops,
            "tflops": round(tflops, 1), "frac_fp8_peak": round(tflops / FP8_PEAK_TFLOPS, 4),
            "frac_bf16_peak": round(tflops / BF16_PEAK_TFLOPS, 4),
            "mfma": "bf16 32x32x16 (E4M3 x E2M1 operands converted exactly)"}


def host_cpu():
    """The host's logical CPU count (`nproc`: the ones this process may use),
    os.cpu_count() and the CPU model name from /proc/cpuinfo."""
    import subprocess

    try:
        nproc = int(subprocess.run(["nproc"], capture_output=True, text=True, check=True).stdout.strip())
    except (OSError, ValueError, subprocess.CalledProcessError):
        nproc = len(os.sched_getaffinity(0))
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"nproc": nproc, "os_cpu_count": os.cpu_count(), "model": model}


def cpu_baseline(args, wl, dw, C, run_chain):
    """The CPU oracle on the first cpu_sample_seqs sequences of the same
    workload (their full layer chain), on every core this process may use,
    scaled to layer-steps/s of the whole batch.  Its indices are also
    compared with the GPU's for those rows."""
    import numpy as np

    import oracle

    host = host_cpu()
    threads = max(1, host["nproc"])
    oracle.NTHREADS = threads
    rows = np.arange(min(args.cpu_sample_seqs, wl.total_q))
    t0 = time.time()
    ref = oracle.layer_chain(wl, rows=rows)
    dt = time.time() - t0
    outs, _, _ = run_chain(dw, want_idx=True, want_lse=False, pool=False)
    got_idx = outs[0]["idx"].cpu().numpy()[rows]
    got_out = outs[0]["out"].cpu().numpy()[rows]
    idx_equal = bool(np.array_equal(got_idx, ref[0]["idx"]))
    err = float(np.abs(got_out.astype(np.float64) - ref[0]["out"]).max())
    frac = len(rows) / wl.total_q
    value = 1.0 / (dt / frac)
    log(f"[bench] oracle: {dt:.1f}s for {len(rows)} sequences on {threads} threads ({host['model']})")
    return {"value": round(value, 5), "unit": "layer-steps/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(rows)} of {wl.total_q} sequences of decode_c1 (full 131,072-entry scan, Top-512, "
                      f"attention), {dt:.1f} s wall, scaled by {wl.total_q}/{len(rows)}",
            "host": host, "work_units": "score rows split into 65,536-slot pieces, attention rows",
            "sample_indices_equal_gpu": idx_equal, "sample_attn_max_abs_err": err}


if __name__ == "__main__":
    main()
