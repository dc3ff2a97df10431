#!/usr/bin/env python3
"""Decode benchmark of the MI355X block-quantized Llama hot path.

Default workload: Llama-70B-shaped decode with Q4_K weights fully resident in HBM (hidden 8192,
64/8 heads, FFN 28672, 80 layers, vocab 128256, fp16 KV cache of 2048 positions), seeded
synthetic weights.  One step = one greedy token through every layer (embedding row, 80 x
[RMSNorm + fused QKV GEMV + RoPE/KV append, GQA attention, Wo GEMV + residual, RMSNorm +
gate|up GEMV + SwiGLU, down GEMV + residual], final RMSNorm, head GEMV, argmax).

Prints one JSON line: decode tok/s (value); the roofline of the fused dequant-GEMV over a whole step
(sum of the algorithmic bytes of all 321 GEMV launches over the sum of their kernel durations, HIP
events at each kernel's own start and end on the compute stream, against 8 TB/s), per class; the
plain-read HBM ceiling (best of a sweep); the single Q8_0 4096 x 4096 GEMV on cold copies with the
oracle beside it at one thread and at all threads; and the CPU oracle's rate on a bounded sample of
the decode workload.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused dequant-GEMV HBM GB/s (% of 8 TB/s); decode tok/s, 70B-shape Q4_K/Q6_K"
HBM_PEAK_GBPS = 8000.0

# HBM traffic of the GEMV launches of one decode step from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE
# passes over the default workload (KiB per dispatch, averaged per class), each scaled by what the
# counter reads for a device copy of 256 MiB (FETCH_SIZE reads half of the copy's 256 MiB: scale
# 1.99975; WRITE_SIZE all of it: scale 1.0).  Valid only for the kernel sources it was taken on (their
# sha256 below): after any change to them `roofline.traffic` is reported as null until the passes are
# taken again, or until the decode kernels' device assembly is shown to be unchanged (label numbers
# aside) and the sha is moved to the new sources.
GEMV_TRAFFIC = {
    "workload": "llama70b-q4_k-resident",
    "sources_sha256": "9194cdf48ad4306f4c39fca075009f893957c666c49a9df4a6680050005a2a8e",
    "fetch_scale": 1.99975, "write_scale": 1.00000,
    "classes": {  # label -> (fetch KiB, write KiB) per launch
        "qkv": (24028.3, 44.8),
        "wo": (19190.3, 80.0),
        "gate_up": (132506.8, 112.1),
        "down": (65731.6, 80.0),
        "head": (290369.3, 539.4),
    },
}
GEMV_SOURCES = ("qwg_gemv.hip", "qwg_formats.h", "qwg_kernels.h")


def gemv_sources_sha256() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in GEMV_SOURCES:
        with open(os.path.join(ROOT, "quantized_weight_streaming_gemv_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def gemv_traffic(wl, launches):
    """Counter-derived HBM bytes of the step's GEMV launches per launch (launches: label -> count per
    step), or None if the counters were not taken on the current sources."""
    t = GEMV_TRAFFIC
    if t["sources_sha256"] is None or t["workload"] != wl.name or t["sources_sha256"] != gemv_sources_sha256():
        return None
    if set(t["classes"]) != set(launches):
        return None
    tot = sum(n * (t["classes"][c][0] * t["fetch_scale"] + t["classes"][c][1] * t["write_scale"]) * 1024
              for c, n in launches.items())
    return int(round(tot / sum(launches.values())))


def log(msg: str) -> None:
    print("[bench] " + msg, file=sys.stderr, flush=True)


def workloads():
    import synth
    return {
        "llama70b-q4_k": synth.LLAMA70B_Q4_K,
        "llama8b-q8_0": synth.LLAMA8B_Q8_0,
        "llama70b-q4_k_m": synth.LLAMA70B_Q4_K_M,
        "llama70b-q6_k": synth.replace(synth.LLAMA70B_Q6_K_STREAM, n_resident=-1, skip_tau=0.0),
        "llama70b-q6_k-slep": synth.LLAMA70B_Q6_K_STREAM,
        "llama70b-q6_k-q5_k": synth.LLAMA70B_Q6_K_Q5_K_SPEC,
        # self-speculative decoding in streaming mode: drafts from the 20 resident layers, one
        # 4-column verify pass streams the other (non-skipped) layers per round
        "llama70b-q6_k-slep-selfspec": synth.replace(synth.LLAMA70B_Q6_K_STREAM, draft_layers=20, draft_k=3),
    }


def gemv_classes(wl):
    """(timing class id, label, weight tensor ids) of the five GEMV launches of a step."""
    import synth
    from quantized_weight_streaming_gemv_amd import _lib
    return [(_lib.T_WQ, "qkv", (synth.WQ, synth.WK, synth.WV)), (_lib.T_WO, "wo", (synth.WO,)),
            (_lib.T_WGATE, "gate_up", (synth.WGATE, synth.WUP)), (_lib.T_WDOWN, "down", (synth.WDOWN,)),
            (_lib.T_HEAD, "head", (synth.HEAD,))]


def token_bytes(wl, n_pos: int) -> int:
    """Algorithmic bytes of one decode token: canonical weight bytes of every layer, the head and one
    embedding row, plus the K and V rows read by attention (n_pos positions)."""
    import synth
    head = synth.row_bytes(wl.qtype_head, wl.hidden) * wl.vocab
    emb = synth.row_bytes(wl.qtype_embed, wl.hidden)
    kv = 2 * n_pos * wl.n_kv * wl.head_dim * 2
    return wl.layers_bytes() + wl.n_layers * kv + head + emb


def round_bytes(wl, n_pos: int) -> int:
    """Algorithmic bytes of one self-speculative round: k draft steps over the first draft_layers
    layers (+ head, embedding row, their K/V reads) and one (k+1)-column verify over every layer
    (weights and the K/V rows read once for all columns)."""
    import synth
    head = synth.row_bytes(wl.qtype_head, wl.hidden) * wl.vocab
    emb = synth.row_bytes(wl.qtype_embed, wl.hidden)
    kv_row = 2 * wl.n_kv * wl.head_dim * 2
    k = wl.draft_k
    draft_w = sum(wl.layer_bytes(l) for l in range(wl.draft_layers))
    draft = sum(draft_w + wl.draft_layers * (n_pos + j) * kv_row + head + emb for j in range(k))
    verify = wl.layers_bytes() + wl.n_layers * (n_pos + k) * kv_row + head + (k + 1) * emb
    return draft + verify


def measure_read_ceiling(wl):
    """A plain streaming read (the GEMV's 16-byte non-temporal load pattern, no arithmetic) of the
    gate|up matrix's bytes, rotating over enough copies that each read is cold with respect to the 256 MB
    last-level cache, for a sweep of grid sizes and loads in flight; kernel time from events at the
    kernel's own start and end.  The best configuration is the achievable-bandwidth ceiling."""
    import synth
    import torch
    from quantized_weight_streaming_gemv_amd import ops
    nbytes = (synth.row_bytes(wl.qtype_ffn, wl.hidden) * 2 * wl.ffn + 255) // 256 * 256
    ncopy = max(4, -(-1200000000 // nbytes))
    bufs = [torch.empty(nbytes // 4, dtype=torch.int32, device="cuda") for _ in range(ncopy)]
    for b in bufs:
        b.fill_(1)
    sink = ops.read_bytes(bufs[0])
    sweep = []
    for grid in (1024, 2048, 4096, 8192):
        for unroll in (4, 8, 16):
            for i in range(ncopy):  # warm-up
                ops.read_bytes(bufs[i], sink=sink, grid=grid, unroll=unroll)
            ms = [ops.read_bytes(bufs[i % ncopy], sink=sink, grid=grid, unroll=unroll, timed=True)
                  for i in range(2 * ncopy)]
            us = 1e3 * sum(ms) / len(ms)
            sweep.append({"grid": grid, "unroll": unroll, "us": round(us, 3),
                          "gbps": round(nbytes / (us * 1e-6) / 1e9, 1)})
    best = max(sweep, key=lambda r: r["gbps"])
    log("plain streaming read of %.1f MB: best %.1f GB/s (grid %d, %d loads in flight per lane, %.2f us)"
        % (nbytes / 1e6, best["gbps"], best["grid"], best["unroll"], best["us"]))
    del bufs
    torch.cuda.empty_cache()
    return {"bytes": nbytes, "best": best, "sweep": sweep,
            "note": "kernel time per launch (events at the kernel's start and end), cold copies"}


def measure_h2d_ceiling():
    """hipMemcpyAsync from pinned host memory into HBM, swept over chunk sizes 64 MiB .. 1 GiB on one
    stream and split over two streams; 2 GiB per configuration, best of 3.  The best is the ceiling."""
    import torch
    total = 2 << 30
    src = torch.empty(total, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(total, dtype=torch.uint8, device="cuda")
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    sweep = []
    for chunk in (64 << 20, 256 << 20, 1 << 30):
        for ns in (1, 2):
            best = 0.0
            for _ in range(3):
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                for i, off in enumerate(range(0, total, chunk)):
                    with torch.cuda.stream(streams[i % ns]):
                        dst[off:off + chunk].copy_(src[off:off + chunk], non_blocking=True)
                torch.cuda.synchronize()
                best = max(best, total / (time.perf_counter() - t0) / 1e9)
            sweep.append({"chunk_mib": chunk >> 20, "streams": ns, "gbps": round(best, 2)})
    top = max(sweep, key=lambda r: r["gbps"])
    log("H2D ceiling (pinned): %.1f GB/s (%d MiB chunks, %d stream(s))" % (top["gbps"], top["chunk_mib"],
                                                                            top["streams"]))
    del src, dst
    return {"gbps": top["gbps"], "best": top, "sweep": sweep}


def measure_q8_0_gemv():
    """The single-GEMV workload: Q8_0 W 4096 x 4096 (q ~ U[-127,127], d = |N|*0.02), x ~ N(0,1), rotated
    over 16 independent copies (286 MB, beyond the 256 MB last-level cache) so every launch reads cold
    weights; kernel time from events at the kernel's start and end.  Beside it the oracle on the same
    GEMV at one thread and at all host threads."""
    import numpy as np
    import oracle
    import synth
    import torch
    from quantized_weight_streaming_gemv_amd import ops
    qt, rows, k, ncopy = synth.Q8_0, 4096, 4096, 16
    x = synth.normal_f32(synth.key(0, synth.stream_id(0, -1, synth.XVEC)), k)
    dx = torch.from_numpy(x).cuda()
    packs = []
    for c in range(ncopy):
        W = synth.matrix(synth.DEFAULT_DIST[qt], k, rows, tkey=synth.key(c, synth.stream_id(0, -1, synth.WQ)))
        packs.append(ops.repack(qt, torch.from_numpy(W).cuda(), rows, k))
        if c == 0:
            W0 = W
    y = torch.empty(rows, dtype=torch.float32, device="cuda")
    work = torch.empty(ops.gemv_work_bytes(qt, rows, k, 1), dtype=torch.uint8, device="cuda")
    for p in packs:
        ops.gemv(qt, p, rows, k, dx, out=y, work=work)
    ms = [ops.gemv_timed(qt, packs[i % ncopy], rows, k, dx, y, work) for i in range(4 * ncopy)]
    us = 1e3 * sum(ms) / len(ms)
    alg = synth.row_bytes(qt, k) * rows + k * 4 + rows * 4
    gbps = alg / (us * 1e-6) / 1e9
    cores = oracle.threads()
    t = {}
    for n in (1, cores):
        prev = oracle.set_threads(n)
        reps = 3 if n == 1 else 10
        t0 = time.perf_counter()
        for _ in range(reps):
            oracle.gemv(qt, W0, rows, k, x)
        t[n] = (time.perf_counter() - t0) / reps
        oracle.set_threads(prev)
    log("Q8_0 4096 x 4096 GEMV (16 cold copies): %.2f us, %.1f GB/s; oracle %.1f ms at 1 thread, %.1f ms at %d"
        % (us, gbps, t[1] * 1e3, t[cores] * 1e3, cores))
    return {"rows": rows, "k": k, "copies": ncopy, "bytes_per_launch": alg, "us_per_launch": round(us, 3),
            "gbps": round(gbps, 1), "frac": round(gbps / HBM_PEAK_GBPS, 4),
            "cpu_oracle": {"ms_1_thread": round(t[1] * 1e3, 3), "ms_all_threads": round(t[cores] * 1e3, 3),
                           "cores": cores, "gbps_1_thread": round(alg / t[1] / 1e9, 3),
                           "gbps_all_threads": round(alg / t[cores] / 1e9, 3)}}


def cpu_baseline(wl, n_sample_layers: int):
    """The CPU oracle (fp64, OpenMP over rows) on a bounded sample of the same workload: layers
    0..n-1 and the output head for one token at the first decode position."""
    import numpy as np
    import oracle
    import synth
    pos = wl.n_prior
    ctx = pos + 1
    h = oracle.dequant(wl.qtype_embed, wl.weight(-1, synth.EMBED, wl.first_token(), 1), 1, wl.hidden)[0]
    t_layers = []
    for l in range(n_sample_layers):
        ws = {t: wl.weight(l, t) for t in oracle.OracleModel.TENSORS}
        kc = np.zeros((ctx, wl.n_kv, wl.head_dim), np.uint16)
        vc = np.zeros_like(kc)
        kc[:pos] = wl.kv_prior(l, synth.KCACHE)
        vc[:pos] = wl.kv_prior(l, synth.VCACHE)
        t0 = time.perf_counter()
        h = oracle.layer_forward(wl, l, ws, h, kc, vc, pos)
        t_layers.append(time.perf_counter() - t0)
        del ws
    head = wl.weight(-1, synth.HEAD)
    t0 = time.perf_counter()
    oracle.head_logits(wl, head, h)
    t_head = time.perf_counter() - t0
    per_token = wl.n_layers * (sum(t_layers) / len(t_layers)) + t_head
    return {
        "value": 1.0 / per_token,
        "unit": "tok/s",
        "cores": oracle.threads(),
        "kind": "oracle",
        "sample": ("layers 0..%d of %d and the output head for one token at position %d (%.1f s of CPU work); "
                   "the rate is extrapolated to a whole step: tok/s = 1 / (%d x mean layer time + head time)"
                   % (n_sample_layers - 1, wl.n_layers, pos, sum(t_layers) + t_head, wl.n_layers)),
        "extrapolated_from_layers": n_sample_layers,
        "layer_s": sum(t_layers) / len(t_layers),
        "head_s": t_head,
    }


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=32)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama70b-q4_k", choices=sorted(workloads()))
    ap.add_argument("--class-steps", type=int, default=4, help="steps per GEMV class for the per-class table")
    ap.add_argument("--cpu-layers", type=int, default=24, help="oracle layers in the CPU-baseline sample (about 11 s of CPU work at the 70B shapes)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-read-ceiling", action="store_true", help="skip the plain streaming-read reference")
    ap.add_argument("--no-q8-gemv", action="store_true", help="skip the single Q8_0 4096 x 4096 GEMV measurement")
    ap.add_argument("--hbm-budget-gb", type=float, default=0.0,
                    help="place layers automatically for this device-memory budget (GB): the resident tier "
                         "gets what fits, the rest streams from pinned host memory (0: the workload's placement)")
    ap.add_argument("--file-layers", type=int, default=0,
                    help="move the first N streamed layers to files (the file-backed tier; files in $TMPDIR)")
    ap.add_argument("--prefill", type=int, default=64,
                    help="after the decode measurements, time a prefill of this many prompt tokens (0: none); "
                         "reported under 'prefill', the metric stays decode tok/s")
    ap.add_argument("--prefill-cols", type=int, default=64, help="columns per prefill pass (the model's max_cols)")
    ap.add_argument("--prefill-reps", type=int, default=5, help="timed prefill passes (the median is reported)")
    ap.add_argument("--verify-form", choices=["mfma", "dot"], default="mfma",
                    help="2..4-column Q5_K/Q6_K GEMVs of the verify pass: matrix cores or integer dot products")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run one device-to-device copy of this many MiB first (scale for PMC byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        return 2

    import torch
    import synth
    from quantized_weight_streaming_gemv_amd import _lib, ops, synthetic

    if not os.path.exists(_lib.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    ops.set_gemv_mfma(args.verify_form == "mfma")
    wl = workloads()[args.workload]
    spec = wl.draft_layers > 0
    total_steps = args.warmup + args.steps * 2 + args.class_steps * 5 + 1
    max_ctx = wl.n_prior + total_steps * (wl.draft_k + 1 if spec else 1) + 8 + 2 * max(0, args.prefill)
    max_cols = max(wl.draft_k + 1 if spec else 1, args.prefill_cols if args.prefill > 0 else 1)
    if args.copy_probe_mib > 0:
        src = torch.ones(args.copy_probe_mib << 18, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log("copy probe: %d MiB device-to-device" % args.copy_probe_mib)
        del src, dst
    read_ceiling = None if args.no_read_ceiling else measure_read_ceiling(wl)
    q8 = None if args.no_q8_gemv else measure_q8_0_gemv()
    log("workload %s: %d layers, %.2f GB of weights, KV %d positions" %
        (wl.name, wl.n_layers, wl.model_bytes() / 1e9, wl.n_prior))
    if args.hbm_budget_gb > 0:
        n_res, a_b, p_b = synthetic.plan_residency_of(wl, max_ctx=max_ctx, max_cols=max_cols,
                                                      device_budget=int(args.hbm_budget_gb * 1e9))
        wl = synth.replace(wl, n_resident=n_res)
        log("automatic placement for %.1f GB of HBM: %d of %d layers resident (arena %.2f GB, pinned %.2f GB)"
            % (args.hbm_budget_gb, n_res, wl.n_layers, a_b / 1e9, p_b / 1e9))
    m = synthetic.make_model(wl, max_ctx=max_ctx, max_cols=max_cols)
    log("arena %.2f GB" % (m.arena_bytes / 1e9))
    load_s = synthetic.load(m, wl, log=log)
    log("loaded in %.1f s" % load_s)
    spill_dir = None
    if args.file_layers > 0:
        import shutil
        import tempfile
        streamed = [l for l in range(wl.n_layers) if l >= wl.resident_layers]
        spill = streamed[: args.file_layers]
        spill_dir = tempfile.mkdtemp(prefix="qwg-tier-c-")
        for l in spill:
            m.spill_layer(l, os.path.join(spill_dir, "layer%03d.img" % l))
        log("file-backed tier: layers %d..%d in %s" % (spill[0], spill[-1], spill_dir))

    tok = wl.first_token()
    if wl.skip_tau > 0:
        tok, cos, mask = m.calibrate_skip(wl.skip_tau, tok)
        log("skip calibration: %d of %d layers skipped" % (int(mask.sum()), wl.n_layers))
    for _ in range(args.warmup):
        tok, _ = m.decode_step(tok)

    # timed region: K greedy tokens (self-speculative workload: K rounds of k drafts + one verify)
    n_tok = n_acc = 0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        if spec:
            out, acc = m.spec_step(tok, wl.draft_layers, wl.draft_k)
            tok = out[-1]
            n_tok += len(out)
            n_acc += acc
        else:
            tok, _ = m.decode_step(tok)
            n_tok += 1
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms_per_step = dt * 1e3 / args.steps
    tok_s = n_tok / dt
    n_pos_mid = wl.n_prior + args.warmup + args.steps // 2
    log("%s: %.3f ms/step, %.1f tok/s (%d tokens)" % ("spec rounds" if spec else "decode", ms_per_step, tok_s, n_tok))

    # the same K decode steps again with HIP events at the start and end of every GEMV kernel of the
    # step (recorded by the dispatch itself, on the compute stream)
    m.set_timing(_lib.TIME_ALL_GEMV)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        tok, _ = m.decode_step(tok)
    torch.cuda.synchronize()
    dt_ev = time.perf_counter() - t0
    classes = {}
    launches = {}
    tot_b = tot_ms = 0.0
    tot_n = 0
    for cid, label, _ in gemv_classes(wl):
        ms, n, b = m.get_timing_class(cid)
        if n == 0:
            continue
        classes[label] = {"launches_per_step": n // args.steps, "us_per_launch": round(ms / n * 1e3, 3),
                          "bytes_per_launch": b // n, "gbps": round(b / (ms * 1e-3) / 1e9, 1),
                          "frac": round(b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
        launches[label] = n // args.steps
        tot_b += b
        tot_ms += ms
        tot_n += n
    gemv_gbps = tot_b / (tot_ms * 1e-3) / 1e9
    log("all GEMVs of a step: %d launches, %.1f GB/s (%.1f%% of 8 TB/s), %.3f ms of %.3f ms per step (with events %.3f)"
        % (tot_n // args.steps, gemv_gbps, 100 * gemv_gbps / HBM_PEAK_GBPS, tot_ms / args.steps, ms_per_step,
           dt_ev * 1e3 / args.steps))
    for label, c in classes.items():
        log("  %-8s %6.2f us  %7.1f GB/s (%4.1f%%)" % (label, c["us_per_launch"], c["gbps"], 100 * c["frac"]))
    verify_classes = None
    if spec:
        # the verify pass alone (k+1 columns through every layer; it leaves the model state as it was)
        vtoks = [tok] * (wl.draft_k + 1)
        verify_classes = {}
        m.set_timing(_lib.TIME_ALL_GEMV)
        for _ in range(args.class_steps):
            m.verify(vtoks, want_logits=False)
        for cid, label, _ in gemv_classes(wl):
            ms, n, b = m.get_timing_class(cid)
            if n:
                verify_classes[label] = {"us_per_launch": round(ms / n * 1e3, 3), "bytes_per_launch": b // n,
                                         "gbps": round(b / (ms * 1e-3) / 1e9, 1)}
        log("verify GEMVs (%d columns, %s): %s" % (wl.draft_k + 1, args.verify_form, json.dumps(verify_classes)))
    m.set_timing(-1)
    prefill = None
    if args.prefill > 0:
        # a deterministic synthetic prompt, after everything else, each pass after the workload's
        # cached positions: the context is cut back to them before the warm-up pass and after every
        # timed pass (the decode steps' KV rows are overwritten; nothing after this reads them)
        prompt = [(wl.first_token() + 7919 * i) % wl.vocab for i in range(args.prefill)]
        base = wl.n_prior
        m.truncate(base)
        m.prefill(prompt[: max_cols])  # warm-up pass
        m.truncate(base)
        reps = []
        for _ in range(max(1, args.prefill_reps)):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            m.prefill(prompt)
            torch.cuda.synchronize()
            reps.append(time.perf_counter() - t0)
            m.truncate(base)
        dt_p = statistics.median(reps)
        # passes wider than 8 columns need the prompt GEMM: K-quant layer matrices with K % 512 == 0
        kq = all(wl.qtype_of(t, l) in (synth.Q4_K, synth.Q5_K, synth.Q6_K)
                 for l in range(wl.n_layers) for t in (synth.WQ, synth.WO, synth.WGATE, synth.WDOWN))
        kq = kq and wl.hidden % 512 == 0 and wl.ffn % 512 == 0 and (wl.n_q * wl.head_dim) % 512 == 0
        width = max_cols if kq else min(max_cols, 8)
        prefill = {"tokens": args.prefill, "columns_per_pass": width, "ms": round(dt_p * 1e3, 3),
                   "tok_s": round(args.prefill / dt_p, 1), "timing": "median of %d passes" % len(reps),
                   "ms_each": [round(x * 1e3, 3) for x in reps], "context_before": base,
                   "arithmetic": ("passes of 9-64 columns: Q4_K/Q5_K GEMMs and the attention on "
                                  "v_mfma_f32_16x16x32_f16 with exact fp16 weights (K/V) and two-piece "
                                  "fp16 activations (queries, softmax weights), fp32 accumulation; "
                                  "Q6_K GEMMs exact int8 products")}
        log("prefill of %d tokens in passes of %d columns: %.2f ms, %.1f tok/s"
            % (args.prefill, width, dt_p * 1e3, args.prefill / dt_p))
    h2d_b, h2d_ms = m.stream_stats()
    file_b, file_ms = m.file_stats()
    step_bytes = round_bytes(wl, n_pos_mid) if spec else token_bytes(wl, n_pos_mid)
    h2d_ceiling = measure_h2d_ceiling() if h2d_b else None
    m.close()
    del m
    torch.cuda.empty_cache()
    if spill_dir:
        shutil.rmtree(spill_dir, ignore_errors=True)

    cpu = None
    if not args.no_cpu_baseline:
        log("CPU oracle baseline (%d layers + head) ..." % args.cpu_layers)
        cpu = cpu_baseline(wl, args.cpu_layers)
        log("oracle: %.3g tok/s on %d threads" % (cpu["value"], cpu["cores"]))

    gate = classes.get("gate_up", {})
    out = {
        "metric": METRIC,
        "value": round(tok_s, 3),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4" if wl.qtype_ffn in (synth.Q4_K, synth.Q4_0) else "int8",
        "dtype_note": ("exact integer dot products (v_dot8_i32_i4 on 4-bit quants / v_dot4_i32_i8 on byte quants) "
                       "against 32-bit block fixed-point activation digits (one power-of-two scale per 32 "
                       "elements), int32 chunk sums recombined and scaled in fp32; fp16 KV cache, fp32 "
                       "attention and norms"),
        "data": "synthetic (seeded random weights of the stated shapes and distributions)",
        "config": {"workload": wl.name, "layers": wl.n_layers, "hidden": wl.hidden, "n_q": wl.n_q, "n_kv": wl.n_kv,
                   "head_dim": wl.head_dim, "ffn": wl.ffn, "vocab": wl.vocab, "kv_positions": wl.n_prior,
                   "weights": synth.QTYPE_NAMES[wl.qtype_attn] + "/" + synth.QTYPE_NAMES[wl.qtype_ffn]
                   + ("" if not wl.wide_down_every else " (W_down of every %d. layer %s, head %s)" % (
                       wl.wide_down_every, synth.QTYPE_NAMES[wl.wide_qtype], synth.QTYPE_NAMES[wl.qtype_head])),
                   "batch": 1, "greedy": True,
                   "resident_layers": wl.n_layers if wl.n_resident < 0 else wl.n_resident,
                   "hbm_budget_gb": args.hbm_budget_gb or None},
        "roofline": {"bound": "hbm",
                     "kernel": "fused dequant-GEMV, every launch of a decode step (QKV, Wo, gate|up, down, head)",
                     "achieved": round(gemv_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gemv_gbps / HBM_PEAK_GBPS, 4), "traffic": gemv_traffic(wl, launches),
                     "bytes_per_launch": int(round(tot_b / tot_n)), "us_per_launch": round(tot_ms / tot_n * 1e3, 3),
                     "launches_per_step": tot_n // args.steps, "ms_per_step": round(tot_ms / args.steps, 4),
                     "classes": classes,
                     "gate_up": {"achieved": gate.get("gbps"), "frac": gate.get("frac"),
                                 "us_per_launch": gate.get("us_per_launch")}},
        "step_effective_gbps": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "step_bytes": step_bytes,
        "cpu_baseline": cpu,
        "pages_context": "NTransformer pages: ~49 tok/s 8B Q8_0 resident, 0.2-0.5 tok/s 70B Q6_K/Q4_K_M streamed, "
                         "RTX 3090 (other hardware and mode; not comparable)",
    }
    if q8:
        out["gemv_q8_0_4096"] = q8
    if h2d_b:
        out["h2d"] = {"bytes": h2d_b, "ms": round(h2d_ms, 3), "gbps": round(h2d_b / (h2d_ms * 1e-3) / 1e9, 2),
                      "ceiling_gbps": h2d_ceiling["gbps"], "ceiling": h2d_ceiling}
    if read_ceiling:
        out["hbm_read_ceiling"] = read_ceiling
    if prefill:
        out["prefill"] = prefill
    if spill_dir:
        out["file_tier"] = {"layers": args.file_layers, "bytes": file_b, "host_ms": round(file_ms, 3),
                            "gbps": round(file_b / (file_ms * 1e-3) / 1e9, 2) if file_ms > 0 else None,
                            "note": "host reads of freshly written files (page cache) into pinned staging"}
    if spec:
        out["spec"] = {"rounds": args.steps, "tokens": n_tok, "ms_per_round": round(ms_per_step, 3),
                       "accepted_drafts": n_acc, "acceptance_rate": round(n_acc / (args.steps * wl.draft_k), 4),
                       "draft_layers": wl.draft_layers, "k": wl.draft_k, "verify_form": args.verify_form,
                       "verify_gemv": verify_classes,
                       "note": ("tok/s depends on the acceptance rate: with these synthetic weights the greedy "
                                "sequence collapses to a repeated token, which the drafts predict, so acceptance "
                                "is near 1; at acceptance 0 a round emits one token (1000 / ms_per_round tok/s)")}
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
