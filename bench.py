#!/usr/bin/env python3
"""PBD window-step benchmark on one MI355X.

Times K consecutive calls of la_pbd_step on the full 36-layer, 152,681-token
decoder at batch 1, prefix 1280 (synthetic, random-init weights, inputs resident
in HBM before the timed region), and prints one JSON line with the window steps
per second, the roofline figures of the dominant kernel and the CPU oracle timed
on the host as a reference.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
CAL_COPY_BYTES = 256 << 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gate_up_traffic_step_b1_p1280.json")
METRIC = "PBD window steps/sec (≈boxes/sec) at batch 1 and 32; achieved HBM GB/s vs peak"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def weight_bytes(w):
    """Bytes of the matrix itself (tile padding rows excluded)."""
    n, k = int(w["n"]), int(w["k"])
    if w["fmt"] == "bf16":
        return n * k * 2
    return n * k // 2 + n * (k // int(w["group"])) * 2


def gate_up_bytes(w, T, H, F):
    """Algorithmic bytes of one gate/up launch: the weights once, the packed
    operand (bf16 hi + lo of T rows) once, the fp32 output once."""
    return weight_bytes(w) + T * H * 4 + T * F * 4


def kernel_source_digest():
    """Digest of the small-batch GEMM kernel's sources: counter-based traffic
    is only reported for the kernel it was measured on."""
    h = hashlib.sha256()
    for name in ("la_gemm.hip", "la_gemm_common.hpp", "la_common.hpp"):
        with open(os.path.join(ROOT, "box_decoding_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per gate/up launch from the committed counter summary, or None
    when it was taken on another version of the kernel."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != kernel_source_digest():
        return None
    return rec.get("traffic_bytes_per_launch")


def pmc_summary(fetch_db, write_db, out_path):
    """Turn two rocprofv3 --pmc runs of this script (FETCH_SIZE, then
    WRITE_SIZE) into HBM bytes per gate/up launch, each counter scaled by what
    it reads for the calibration copy of CAL_COPY_BYTES."""
    import sqlite3

    def per_kernel(db, counter):
        con = sqlite3.connect(db)
        rows = con.execute(
            "select kernel_name, dispatch_id, sum(value) from counters_collection "
            "where counter_name = ? group by dispatch_id", (counter,)).fetchall()
        con.close()
        return rows

    def summarize(db, counter):
        rows = per_kernel(db, counter)
        gu = [v for name, _, v in rows if "k_gemm<1, false, 1, 2>" in name]
        # the calibration copy is the runtime's copy kernel moving CAL_COPY_BYTES,
        # the largest such dispatch of the run
        copies = [v for name, _, v in rows if name.startswith("__amd_rocclr_copyBuffer")]
        cal = max(copies)
        factor = CAL_COPY_BYTES / (cal * 1024.0)
        return sum(gu) / len(gu) * 1024.0 * factor, factor, len(gu), cal

    f_bytes, f_factor, n_f, f_cal = summarize(fetch_db, "FETCH_SIZE")
    w_bytes, w_factor, n_w, w_cal = summarize(write_db, "WRITE_SIZE")
    rec = {
        "kernel": "k_gemm<1, false, 1, 2> (gate/up + SiLU, LDS-staged ring)",
        "kernel_source_sha256_16": kernel_source_digest(),
        "fetch_bytes_per_launch": round(f_bytes), "write_bytes_per_launch": round(w_bytes),
        "traffic_bytes_per_launch": round(f_bytes + w_bytes),
        "fetch_scale": f_factor, "write_scale": w_factor,
        "calibration_copy_bytes": CAL_COPY_BYTES,
        "calibration_fetch_kib": f_cal, "calibration_write_kib": w_cal,
        "dispatches": [n_f, n_w],
    }
    with open(out_path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def step_bytes(model, dims, prefix_len, W):
    """Algorithmic HBM bytes of one step: every weight once, the KV read once,
    the window's K/V written once, the gathered embedding rows."""
    total = 0
    for lay in model["layers"]:
        for k in ("qkv", "o", "gate_up", "down"):
            total += weight_bytes(lay[k])
        total += (lay["in_norm"].numel() + lay["post_norm"].numel()) * 2
        if lay.get("qkv_bias") is not None:
            total += lay["qkv_bias"].numel() * 2
    lm = model["lm_head"] if model.get("lm_head") is not None else model["embed"]
    total += weight_bytes(lm) + model["final_norm"].numel() * 2
    per_tok = dims.n_layers * 2 * dims.n_kv_heads * dims.head_dim * 2
    keys = int(sum(int(p) + W for p in prefix_len.tolist()))
    total += keys * per_tok + len(prefix_len) * W * per_tok
    total += len(prefix_len) * W * dims.hidden * 2
    return total


def cpu_baseline(workload_name, sample_layers, min_seconds=10.0):
    """The oracle as it stands, on a bounded sample of the same workload."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_info

    import oracle as O
    from box_decoding_amd import synth

    w = synth.WORKLOADS[workload_name]
    d = w.dims
    import dataclasses
    ds = dataclasses.replace(d, n_layers=sample_layers)
    log(f"cpu_baseline: generating a {sample_layers}-layer sample on the host")
    model = synth.to_numpy_tree(synth.make_model(ds, w.wfmt, w.model_seed, "cpu"))
    model["dims"] = ds
    P = synth.draw_prefix_lens(w)
    cache = synth.to_numpy_tree(synth.make_cache(ds, P, w.window, seed=w.input_seed, device="cpu"))
    ids = synth.draw_window_ids(w.batch, w.window, d.vocab, w.input_seed).numpy()
    h0 = O.embed_rows(ids.reshape(-1), model["embed"])
    lm = model["lm_head"] if model.get("lm_head") is not None else model["embed"]
    # whole passes over the sample (its layers, then the final norm and the
    # full lm_head argmax) until at least min_seconds of work are measured
    t_layers = t_lm = 0.0
    passes = 0
    while passes == 0 or t_layers + t_lm < min_seconds:
        h = h0
        t0 = time.perf_counter()
        for l in range(sample_layers):
            h, _, _ = O.decoder_layer(h, model["layers"][l], ds, cache, l, P.numpy(), w.window)
        t_layers += time.perf_counter() - t0
        f = O.rmsnorm(h, O.bf16_to_float(model["final_norm"]), d.rms_eps)
        t0 = time.perf_counter()
        O.lm_head_argmax(f, lm)
        t_lm += time.perf_counter() - t0
        passes += 1
    t_layers /= passes
    t_lm /= passes
    t_step = t_layers / sample_layers * d.n_layers + t_lm
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": 1.0 / t_step, "unit": "steps/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{workload_name}: {passes} pass(es) over {sample_layers} of {d.n_layers} "
                      f"decoder layers ({t_layers:.2f} s per pass) + the full lm_head argmax "
                      f"({t_lm:.2f} s per pass), float64 numpy, extrapolated to one "
                      f"{d.n_layers}-layer step ({t_step:.2f} s)",
            "host_cpus": len(os.sched_getaffinity(0))}


def batch32_leg(B, synth, torch, dm, model, dev, stream, timed, args):
    """Steps/s of the batched step (32 ragged sequences, same model) and the
    useful matrix-core rate of its gate/up GEMM (192 rows), against the dense
    bf16 peak.  The kernel splits activations into bf16 hi + lo halves, so the
    matrix cores do twice the useful work."""
    w = synth.WORKLOADS["step_b32_ragged"]
    d = w.dims
    log("bench: batch-32 leg")
    P = synth.draw_prefix_lens(w)
    cache = synth.make_cache(d, P, w.window, seed=w.input_seed, device=dev)
    ids = synth.draw_window_ids(w.batch, w.window, d.vocab, w.input_seed, device=dev)
    dc = B.DeviceCache(cache, d.n_layers)
    Pd = P.to(dev)
    max_len = int(P.max()) + w.window
    ws = B.Workspace(dev)
    out_ids = torch.empty((w.batch, w.window), dtype=torch.int32, device=dev)
    out_gap = torch.empty((w.batch, w.window), dtype=torch.float32, device=dev)
    graph = B.StepGraph(dm, dc, ids, Pd, max_len, out_ids, out_gap, ws=ws)
    for _ in range(max(2, args.warmup)):
        graph.replay()
    steps = max(5, args.steps // 3)
    ms_step, _ = timed(graph.replay, steps)
    sbytes = step_bytes(model, d, P, w.window)
    T = w.batch * w.window
    F, H = d.inter, d.hidden
    xin = torch.randn((T, H), device=dev, generator=torch.Generator(device=dev).manual_seed(1))
    packed = B.pack_rows(xin, w.wfmt, norm_gain=model["layers"][0]["post_norm"])
    yout = torch.empty((T, F), dtype=torch.float32, device=dev)
    for l in range(3):
        B.wgemm_packed(packed, T, model["layers"][l]["gate_up"], silu_gate=True, out=yout)
    reps = max(8, args.kernel_reps // 4)

    def gemm():
        for r in range(reps):
            B.wgemm_packed(packed, T, model["layers"][r % d.n_layers]["gate_up"], silu_gate=True, out=yout)

    k_ms = timed(gemm, 1)[0] / reps
    flops = 2.0 * T * H * 2 * F
    tflops = flops / (k_ms * 1e-3) / 1e12
    log(f"bench: batch 32: {ms_step:.3f} ms/step, {1000.0 / ms_step:.1f} steps/s; "
        f"gate_up GEMM {k_ms * 1e3:.1f} us, {tflops:.0f} TFLOP/s useful")
    del graph, cache, dc, ws
    torch.cuda.synchronize()
    return {"workload": w.name, "batch": w.batch, "window": w.window, "steps": steps,
            "ms_per_step": round(ms_step, 4), "steps_per_s": round(1000.0 / ms_step, 3),
            "windows_per_s": round(1000.0 / ms_step * w.batch, 2),
            "step_hbm_gbps": round(sbytes / ms_step / 1e6, 1),
            "step_hbm_frac": round(sbytes / ms_step / 1e6 / HBM_PEAK_GBPS, 4),
            "gate_up_gemm": {"rows": T, "launch_us": round(k_ms * 1e3, 2),
                             "useful_tflops": round(tflops, 1), "peak_tflops": MFMA_BF16_PEAK_TFLOPS,
                             "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                             "matrix_core_frac_with_hi_lo": round(2 * tflops / MFMA_BF16_PEAK_TFLOPS, 4)}}


def emission_leg(B, synth, torch, dm, model, dev, stream, args):
    """The dense-scene emission loop: 16 sequences from prefix 2048 run 40
    consecutive window steps, each committed on the device (prefix += 6, next
    window = [last output id, mask x 5]) -- one captured graph of step + commit,
    replayed 40 times per loop."""
    w = synth.WORKLOADS["emit_b16_p2048_x40"]
    d = w.dims
    log("bench: emission-loop leg")
    P = synth.draw_prefix_lens(w)
    cache = synth.make_cache(d, P, w.window, extra_tokens=w.steps * w.window, seed=w.input_seed,
                             device=dev)
    ids = synth.draw_window_ids(w.batch, w.window, d.vocab, w.input_seed, device=dev)
    mask_id = int(ids[0, 1].item())
    ids0, P0 = ids.clone(), P.to(dev)
    dc = B.DeviceCache(cache, d.n_layers)
    Pd = P0.clone()
    max_len = int(P.max()) + (w.steps + 1) * w.window
    ws = B.Workspace(dev)
    out_ids = torch.empty((w.batch, w.window), dtype=torch.int32, device=dev)
    out_gap = torch.empty((w.batch, w.window), dtype=torch.float32, device=dev)
    graph = B.StepGraph(dm, dc, ids, Pd, max_len, out_ids, out_gap, ws=ws, commit_mask_id=mask_id)

    def run_loop():
        ids.copy_(ids0)
        Pd.copy_(P0)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(w.steps):
            graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    run_loop()  # warm-up loop
    loop_ms = run_loop()
    assert int((Pd - P0).min().item()) == w.steps * w.window
    ms_step = loop_ms / w.steps
    mid = P + w.window * (w.steps - 1) // 2
    sbytes = step_bytes(model, d, mid, w.window)
    log(f"bench: emission loop: {loop_ms:.2f} ms for {w.steps} steps, {ms_step:.3f} ms/step, "
        f"{w.batch * 1000.0 / ms_step:.0f} windows/s")
    del graph, cache, dc, ws
    torch.cuda.synchronize()
    return {"workload": w.name, "batch": w.batch, "window": w.window, "steps_per_loop": w.steps,
            "prefix_start": int(P.max()), "loop_ms": round(loop_ms, 3), "ms_per_step": round(ms_step, 4),
            "steps_per_s": round(1000.0 / ms_step, 3),
            "windows_per_s": round(1000.0 / ms_step * w.batch, 2),
            "step_hbm_gbps": round(sbytes / ms_step / 1e6, 1),
            "step_hbm_frac": round(sbytes / ms_step / 1e6 / HBM_PEAK_GBPS, 4)}


def probe_leg(B, synth, torch, dm, model, dev, stream, timed, args):
    """The long-context probe: one sequence at prefix 32768, window 6."""
    w = synth.WORKLOADS["probe_b1_p32768"]
    d = w.dims
    log("bench: long-context leg")
    P = synth.draw_prefix_lens(w)
    cache = synth.make_cache(d, P, w.window, seed=w.input_seed, device=dev)
    ids = synth.draw_window_ids(w.batch, w.window, d.vocab, w.input_seed, device=dev)
    dc = B.DeviceCache(cache, d.n_layers)
    Pd = P.to(dev)
    max_len = int(P.max()) + w.window
    ws = B.Workspace(dev)
    out_ids = torch.empty((w.batch, w.window), dtype=torch.int32, device=dev)
    out_gap = torch.empty((w.batch, w.window), dtype=torch.float32, device=dev)
    graph = B.StepGraph(dm, dc, ids, Pd, max_len, out_ids, out_gap, ws=ws)
    for _ in range(max(2, args.warmup)):
        graph.replay()
    steps = max(5, args.steps // 3)
    ms_step, _ = timed(graph.replay, steps)
    sbytes = step_bytes(model, d, P, w.window)
    log(f"bench: prefix 32768: {ms_step:.3f} ms/step, {1000.0 / ms_step:.1f} steps/s")
    del graph, cache, dc, ws
    torch.cuda.synchronize()
    return {"workload": w.name, "batch": w.batch, "window": w.window, "prefix": int(P.max()),
            "steps": steps, "ms_per_step": round(ms_step, 4), "steps_per_s": round(1000.0 / ms_step, 3),
            "step_hbm_gbps": round(sbytes / ms_step / 1e6, 1),
            "step_hbm_frac": round(sbytes / ms_step / 1e6 / HBM_PEAK_GBPS, 4)}


def refeed_leg(B, synth, torch, dm, model, dev, stream, args):
    """The emission loop of the dense-scene workload with re-feeding: every
    step re-sends the 6 tokens it accepted last time causally before a new
    block of 6 (window W = 11: 5 re-fed rows, the block; the first step has
    the block only), and a device-side commit accepts the whole block -- one
    captured graph of la_pbd_step_refeed + la_pbd_commit_refeed, 40 replays."""
    w = synth.WORKLOADS["emit_b16_p2048_x40"]
    d = w.dims
    block, W = w.window, 2 * w.window - 1
    log("bench: re-fed emission-loop leg")
    P = synth.draw_prefix_lens(w)
    cache = synth.make_cache(d, P, W, extra_tokens=w.steps * block, seed=w.input_seed, device=dev)
    first = synth.draw_window_ids(w.batch, block, d.vocab, w.input_seed, device=dev)
    mask_id = int(first[0, 1].item())
    ids0 = torch.full((w.batch, W), mask_id, dtype=torch.int32, device=dev)
    ids0[:, 0] = first[:, 0]
    ids, P0 = ids0.clone(), P.to(dev)
    cr0 = torch.zeros(w.batch, dtype=torch.int32, device=dev)
    wl0 = torch.full((w.batch,), block, dtype=torch.int32, device=dev)
    cr, wl = cr0.clone(), wl0.clone()
    dc = B.DeviceCache(cache, d.n_layers)
    Pd = P0.clone()
    max_len = int(P.max()) + W + w.steps * block
    ws = B.Workspace(dev)
    out_ids = torch.empty((w.batch, W), dtype=torch.int32, device=dev)
    graph = B.StepGraph(dm, dc, ids, Pd, max_len, out_ids, None, ws=ws, commit_mask_id=mask_id,
                        refeed=(cr, wl, block, None))

    def run_loop():
        for t, t0 in ((ids, ids0), (Pd, P0), (cr, cr0), (wl, wl0)):
            t.copy_(t0)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(w.steps):
            graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    run_loop()  # warm-up loop
    loop_ms = run_loop()
    # the first step commits its block's first row, every later one 6 rows
    assert int((Pd - P0).min().item()) == 1 + (w.steps - 1) * block
    ms_step = loop_ms / w.steps
    log(f"bench: re-fed emission loop: {loop_ms:.2f} ms for {w.steps} steps, {ms_step:.3f} ms/step, "
        f"{w.batch * 1000.0 / ms_step:.0f} windows/s")
    del graph, cache, dc, ws
    torch.cuda.synchronize()
    return {"workload": w.name + "_refeed", "batch": w.batch, "window": W, "block": block,
            "steps_per_loop": w.steps, "prefix_start": int(P.max()), "loop_ms": round(loop_ms, 3),
            "ms_per_step": round(ms_step, 4), "steps_per_s": round(1000.0 / ms_step, 3),
            "windows_per_s": round(1000.0 / ms_step * w.batch, 2)}


def prefill_leg(B, synth, torch, dm, model, dev, timed, args):
    """Prefill of the batch-1 workload's prompt: 256 image-token rows (N(0,1)
    features spliced in) and 64 prompt tokens, all causal, as one captured
    graph replayed; K/V of the 320 rows written, the first generated id out."""
    w = synth.WORKLOADS["step_b1_p1280"]
    d = w.dims
    n_img, n_txt = 256, 64
    L = n_img + n_txt
    log("bench: prefill leg")
    P = torch.zeros(1, dtype=torch.int32)
    cache = synth.make_cache(d, P, L, seed=w.input_seed, device=dev)
    ids = synth.draw_window_ids(1, L, d.vocab, w.input_seed, mask_id=-1, device=dev)
    ids[:, :n_img] = -1
    emb = torch.randn((1, L, d.hidden), device=dev, generator=torch.Generator(device=dev).manual_seed(5))
    dc = B.DeviceCache(cache, d.n_layers)
    Pd = P.to(dev)
    ws = B.Workspace(dev)
    B.pbd_prefill(dm, dc, ids, Pd, L, embeds=emb, ws=ws)  # sizes the workspace
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        B.pbd_prefill(dm, dc, ids, Pd, L, embeds=emb, ws=ws)
    for _ in range(max(2, args.warmup)):
        graph.replay()
    reps = max(3, args.steps // 6)
    ms, _ = timed(graph.replay, reps)
    log(f"bench: prefill of {L} rows ({n_img} spliced + {n_txt} tokens): {ms:.3f} ms, "
        f"{L * 1000.0 / ms:.0f} rows/s")
    del graph, cache, dc, ws
    torch.cuda.synchronize()
    return {"workload": "prefill_b1_l320", "batch": 1, "rows": L, "spliced_rows": n_img, "reps": reps,
            "ms": round(ms, 4), "rows_per_s": round(L * 1000.0 / ms, 1)}


def causal_leg(B, synth, torch, model, dev, timed, args):
    """The batch-1 step with the RK3588 conversion's causal window (window row j
    sees the prefix and window rows 0..j) instead of the bidirectional one."""
    w = synth.WORKLOADS["step_b1_p1280"]
    d = w.dims
    log("bench: causal-window leg")
    P = synth.draw_prefix_lens(w)
    cache = synth.make_cache(d, P, w.window, seed=w.input_seed, device=dev)
    ids = synth.draw_window_ids(w.batch, w.window, d.vocab, w.input_seed, device=dev)
    dmc = B.DeviceModel(model, causal_window=True)
    dc = B.DeviceCache(cache, d.n_layers)
    Pd = P.to(dev)
    ws = B.Workspace(dev)
    out_ids = torch.empty((w.batch, w.window), dtype=torch.int32, device=dev)
    out_gap = torch.empty((w.batch, w.window), dtype=torch.float32, device=dev)
    graph = B.StepGraph(dmc, dc, ids, Pd, int(P.max()) + w.window, out_ids, out_gap, ws=ws)
    for _ in range(max(2, args.warmup)):
        graph.replay()
    steps = max(5, args.steps // 3)
    ms_step, _ = timed(graph.replay, steps)
    log(f"bench: causal window, batch 1: {ms_step:.3f} ms/step, {1000.0 / ms_step:.1f} steps/s")
    del graph, cache, dc, ws
    torch.cuda.synchronize()
    return {"workload": w.name, "window_mask": "causal", "steps": steps,
            "ms_per_step": round(ms_step, 4), "steps_per_s": round(1000.0 / ms_step, 3)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="step_b1_p1280")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-layers", type=int, default=4)
    ap.add_argument("--kernel-reps", type=int, default=72)
    ap.add_argument("--row-major", action="store_true", help="keep the row-major weight layout")
    ap.add_argument("--no-extra-legs", action="store_true",
                    help="skip the emission-loop, prefix-32768, causal-window, re-fed loop and prefill legs")
    ap.add_argument("--no-batch32", action="store_true",
                    help="skip the batch-32 leg reported beside the batch-1 step")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DB", "WRITE_DB"),
                    help="summarise two rocprofv3 --pmc runs of this script into the traffic file")
    args = ap.parse_args()
    if args.pmc_summary:
        pmc_summary(args.pmc_summary[0], args.pmc_summary[1], TRAFFIC_FILE)
        return
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: the PBD step here is a single-GPU path "
              "(data-parallel serving would run one independent copy per GPU).", file=sys.stderr)
        sys.exit(2)

    import torch

    from box_decoding_amd import binding as B
    from box_decoding_amd import synth

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    B.load()
    dev = "cuda:0"
    torch.cuda.set_device(0)
    w = synth.WORKLOADS[args.workload]
    d = w.dims
    log(f"bench: building {args.workload} on the GPU")
    model = synth.make_model(d, w.wfmt, w.model_seed, dev)
    if not args.row_major:
        # the serving layout: weights regrouped once into 16-row tiles
        model = B.pack_model(model)
        torch.cuda.synchronize()
    P = synth.draw_prefix_lens(w)
    cache = synth.make_cache(d, P, w.window, seed=w.input_seed, device=dev)
    ids = synth.draw_window_ids(w.batch, w.window, d.vocab, w.input_seed, device=dev)
    dm, dc = B.DeviceModel(model), B.DeviceCache(cache, d.n_layers)
    Pd = P.to(dev)
    max_len = int(P.max()) + w.window
    ws = B.Workspace(dev)
    out_ids = torch.empty((w.batch, w.window), dtype=torch.int32, device=dev)
    out_gap = torch.empty((w.batch, w.window), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()

    def timed(fn, n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n, (time.perf_counter() - t0) / n * 1e3

    def eager():
        B.pbd_step(dm, dc, ids, Pd, max_len, ws=ws, out_ids=out_ids, out_gap=out_gap)

    for _ in range(args.warmup):
        eager()
    torch.cuda.synchronize()
    eager_ms, _ = timed(eager, max(3, args.steps // 5))
    # the serving loop replays the step as one captured graph
    graph = B.StepGraph(dm, dc, ids, Pd, max_len, out_ids, out_gap, ws=ws)
    for _ in range(args.warmup):
        graph.replay()
    log(f"bench: warmup done (eager {eager_ms:.3f} ms/step), timing {args.steps} graph replays")
    ms_step, wall_ms = timed(graph.replay, args.steps)
    steps_per_s = 1000.0 / ms_step
    sbytes = step_bytes(model, d, P, w.window)
    log(f"bench: {ms_step:.3f} ms/step (wall {wall_ms:.3f} ms), "
        f"{steps_per_s:.1f} steps/s, {sbytes / ms_step / 1e6:.0f} GB/s algorithmic")

    # Dominant kernel: the gate/up projection with the SiLU epilogue (58% of a
    # layer's weight bytes), the GEMM alone on a pre-packed operand.  Timed with
    # HIP events on the stream the library launches on (torch's current
    # stream), cycling through the 36 layers' weights so that they stream from
    # HBM.
    F, H = d.inter, d.hidden
    T = w.batch * w.window
    xin = torch.randn((T, H), device=dev, generator=torch.Generator(device=dev).manual_seed(1))
    gain = model["layers"][0]["post_norm"]
    packed = B.pack_rows(xin, w.wfmt, norm_gain=gain)
    yout = torch.empty((T, F), dtype=torch.float32, device=dev)
    for l in range(4):
        B.wgemm_packed(packed, T, model["layers"][l]["gate_up"], silu_gate=True, out=yout)
    torch.cuda.synchronize()
    k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    k0.record(stream)
    for r in range(args.kernel_reps):
        B.wgemm_packed(packed, T, model["layers"][r % d.n_layers]["gate_up"], silu_gate=True,
                       out=yout)
    k1.record(stream)
    torch.cuda.synchronize()
    k_ms = k0.elapsed_time(k1) / args.kernel_reps
    gu_bytes = gate_up_bytes(model["layers"][0]["gate_up"], T, H, F)
    k_gbps = gu_bytes / (k_ms * 1e-3) / 1e9
    log(f"bench: gate_up GEMM {k_ms * 1e3:.1f} us, {k_gbps:.0f} GB/s")

    # a plain copy of known size: the scale for the HBM byte counters
    cal_src = torch.empty(CAL_COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
    cal_dst = torch.empty_like(cal_src)
    cal_dst.copy_(cal_src)
    torch.cuda.synchronize()
    del cal_src, cal_dst
    # the counters were taken on the batch-1 tiled workload's gate/up launch
    traffic = measured_traffic() if args.workload == "step_b1_p1280" and not args.row_major else None

    result = {
        "metric": METRIC,
        "value": round(steps_per_s, 3),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "eager_ms_per_step": round(eager_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded random-init weights and KV cache, uniform token ids)",
        "config": {"workload": args.workload, "batch": w.batch, "window": w.window,
                   "prefix": int(P.max()), "layers": d.n_layers, "vocab": d.vocab,
                   "weights": w.wfmt, "layout": "row-major" if args.row_major else "tiled16"},
        "tokens_per_s": round(steps_per_s * T, 2),
        "windows_per_s": round(steps_per_s * w.batch, 3),
        "step_hbm_gbps": round(sbytes / ms_step / 1e6, 1),
        "step_hbm_frac": round(sbytes / ms_step / 1e6 / HBM_PEAK_GBPS, 4),
        "step_bytes": sbytes,
        "roofline": {"bound": "hbm", "kernel": "gate_up GEMM + SiLU (la_wgemm_packed)",
                     "achieved": round(k_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(k_gbps / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "launch_us": round(k_ms * 1e3, 2), "bytes_per_launch": gu_bytes},
    }
    if args.workload == "step_b1_p1280" and not args.no_batch32 and not args.row_major:
        # the metric's second batch size: the same model, 32 ragged sequences
        del cache, dc
        torch.cuda.synchronize()
        result["batch32"] = batch32_leg(B, synth, torch, dm, model, dev, stream, timed, args)
    if args.workload == "step_b1_p1280" and not args.no_extra_legs and not args.row_major:
        # the other bf16 workloads on the same model
        result["emission_loop"] = emission_leg(B, synth, torch, dm, model, dev, stream, args)
        result["prefix_32768"] = probe_leg(B, synth, torch, dm, model, dev, stream, timed, args)
        result["causal_window"] = causal_leg(B, synth, torch, model, dev, timed, args)
        result["refeed_loop"] = refeed_leg(B, synth, torch, dm, model, dev, stream, args)
        result["prefill"] = prefill_leg(B, synth, torch, dm, model, dev, timed, args)
    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(args.workload, args.cpu_sample_layers)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
