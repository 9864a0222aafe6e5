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
FRONT_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "front_traffic_step_b1_p1280.json")
FRONT_DOWN_SLICES = 4  # K slices of the down projection when the front-half launch runs it
METRIC = "PBD window steps/sec (≈boxes/sec) at batch 1 and 32; achieved HBM GB/s vs peak"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def weight_bytes(w):
    """Bytes of the matrix itself (tile padding rows excluded)."""
    n, k = int(w["n"]), int(w["k"])
    if w["fmt"] == "bf16":
        return n * k * 2
    if w["fmt"] == "w8a8":
        return n * k + n * 4
    return n * k // 2 + n * (k // int(w["group"])) * 2


def gate_up_bytes(w, T, H, F):
    """Algorithmic bytes of one gate/up launch: the weights once, the packed
    operand (bf16 hi + lo of T rows; w8a8: int8 rows and their scales) once,
    the fp32 output once."""
    op = T * H + T * 4 if w["fmt"] == "w8a8" else T * H * 4
    return weight_bytes(w) + op + T * F * 4


# The kernels with counter-based traffic: (name in the profile, sources it is
# built from, summary file).
BIG_SOURCES = ("la_gemm_big.hip", "la_gemm_common.hpp", "la_common.hpp")
TRAFFIC_KERNELS = {
    "gate_up": ("k_gemm<1, false, 1, 2>", ("la_gemm.hip", "la_gemm_common.hpp", "la_common.hpp"),
                TRAFFIC_FILE, "k_gemm<1, false, 1, 2> (gate/up + SiLU, LDS-staged ring)"),
    "gate_up_b32": ("k_gemm_big<3, false, 1, 1>", BIG_SOURCES,
                    os.path.join(ROOT, "profiles", "gate_up_traffic_step_b32_ragged.json"),
                    "k_gemm_big<3, false, 1, 1> (gate/up + SiLU, 192 rows, 96-column items)"),
    "gate_up_int4": ("k_gemm_big<3, true, 1, 4>", BIG_SOURCES,
                     os.path.join(ROOT, "profiles", "gate_up_traffic_step_int4_b8_p1280.json"),
                     "k_gemm_big<3, true, 1, 4> (INT4 gate/up + SiLU, 48 rows, exact-fit grid)"),
    "front": ("la::k_front(", ("la_front.hip", "la_attn_common.hpp", "la_internal.hpp", "la_common.hpp"),
              FRONT_TRAFFIC_FILE, "k_front (a layer in one launch: RMSNorm, QKV, attention, O, gate/up + SiLU, down)"),
}


def front_bytes(lay, dims, prefix_len, W):
    """Algorithmic bytes of one front-half launch (a layer's attention block):
    the QKV and O weights, the QKV bias and the two norm gains once; the K/V of
    every key read once and the window's K/V written once; the rows h read
    once; h1, its per-tile sums of squares and the packed gate/up operand (bf16
    hi + lo) written once.  What the launch hands on between its own steps (q,
    the packed QKV operand, the attention partials and output) is not counted."""
    T = len(prefix_len) * W
    H = dims.hidden
    total = weight_bytes(lay["qkv"]) + weight_bytes(lay["o"])
    total += (lay["in_norm"].numel() + lay["post_norm"].numel()) * 2
    if lay.get("qkv_bias") is not None:
        total += lay["qkv_bias"].numel() * 2
    kv_tok = 2 * dims.n_kv_heads * dims.head_dim * 2
    keys = int(sum(int(p) + W for p in prefix_len.tolist()))
    total += keys * kv_tok + T * kv_tok
    total += T * H * 4
    total += T * H * 4 + T * (H // 16) * 4 + 2 * T * H * 2
    return total


def fused_front_bytes(lay, dims, prefix_len, W):
    """Algorithmic bytes of the front-half launch when it also runs the gate/up
    projection: the front half's bytes and the gate/up weights once, the
    packed SiLU output (bf16 hi + lo of T rows) written once; the packed
    post-norm operand and its sums of squares stay inside the launch."""
    T = len(prefix_len) * W
    H, F = dims.hidden, dims.inter
    total = front_bytes(lay, dims, prefix_len, W)
    total -= T * (H // 16) * 4 + 2 * T * H * 2
    return total + weight_bytes(lay["gate_up"]) + T * F * 4


def fused_layer_bytes(lay, dims, prefix_len, W):
    """Algorithmic bytes of the front-half launch when it runs the whole layer
    (the down projection too): fused_front_bytes with the down weights read
    once and its K-slice sums written once instead of the packed SiLU output,
    which stays inside the launch."""
    T = len(prefix_len) * W
    H, F = dims.hidden, dims.inter
    total = fused_front_bytes(lay, dims, prefix_len, W) - T * F * 4
    return total + weight_bytes(lay["down"]) + FRONT_DOWN_SLICES * T * H * 4


def front_fuses_down(w, row_major):
    """Whether the front-half launch also runs the down projection (with
    gate/up; LA_PBD_FRONT_DOWN=0 turns it off)."""
    return front_fuses_gate_up(w, row_major) and os.environ.get("LA_PBD_FRONT_DOWN", "1") != "0"


def front_fuses_gate_up(w, row_major):
    """Whether the library's front-half launch also runs gate/up: bf16 tiled
    weights at up to 8 rows, unless LA_PBD_FRONT_GU=0 turns it off."""
    return (w.batch * w.window <= 8 and w.wfmt == "bf16" and not row_major
            and os.environ.get("LA_PBD_FRONT_GU", "1") != "0"
            and os.environ.get("LA_PBD_FRONT", "1") != "0")


def kernel_source_digest(which="gate_up"):
    """Digest of a kernel's sources: counter-based traffic is only reported for
    the kernel it was measured on."""
    h = hashlib.sha256()
    for name in TRAFFIC_KERNELS[which][1]:
        with open(os.path.join(ROOT, "box_decoding_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(which="gate_up"):
    """HBM bytes per launch from the committed counter summary, or None when it
    was taken on another version of the kernel."""
    try:
        with open(TRAFFIC_KERNELS[which][2]) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != kernel_source_digest(which):
        return None
    return rec.get("traffic_bytes_per_launch")


def pmc_summary(fetch_db, write_db):
    """Turn two rocprofv3 --pmc runs of this script (FETCH_SIZE, then
    WRITE_SIZE) into HBM bytes per launch of the gate/up GEMM and of the
    front-half launch, each counter scaled by what it reads for the
    calibration copy of CAL_COPY_BYTES."""
    for which in TRAFFIC_KERNELS:
        pmc_summary_one(fetch_db, write_db, which)


def pmc_summary_one(fetch_db, write_db, which):
    """One kernel's summary; a kernel the runs did not dispatch is skipped."""
    pattern, _, out_path, label = TRAFFIC_KERNELS[which]
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
        gu = [v for name, _, v in rows if pattern in name]
        if not gu:
            return None
        # the calibration copy is the runtime's copy kernel moving CAL_COPY_BYTES,
        # the largest such dispatch of the run
        copies = [v for name, _, v in rows if name.startswith("__amd_rocclr_copyBuffer")]
        cal = max(copies)
        factor = CAL_COPY_BYTES / (cal * 1024.0)
        return sum(gu) / len(gu) * 1024.0 * factor, factor, len(gu), cal

    fs, ws = summarize(fetch_db, "FETCH_SIZE"), summarize(write_db, "WRITE_SIZE")
    if fs is None or ws is None:
        return
    f_bytes, f_factor, n_f, f_cal = fs
    w_bytes, w_factor, n_w, w_cal = ws
    rec = {
        "kernel": label,
        "kernel_source_sha256_16": kernel_source_digest(which),
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


def hbm_ceiling(torch, dev, nbytes=1 << 30, reps=5):
    """The practical HBM ceiling beside the 8 TB/s spec: a 1 GiB fp32 copy
    (x * 1 into another buffer: read + write), the best of `reps` runs timed
    with HIP events.  A plain torch kernel, so the runtime's copy kernel stays
    the counters' calibration.  (torch's sum reads at about 3.7 TB/s here,
    below this library's own weight streams, so it is no ceiling.)"""
    a = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)

    def best(fn):
        fn()
        torch.cuda.synchronize()
        ms = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        return min(ms)

    copy_ms = best(lambda: torch.mul(a, 1.0, out=b))
    del a, b
    return {"copy_gbps": round(2 * nbytes / (copy_ms * 1e-3) / 1e9, 1),
            "how": "1 GiB fp32, x * 1 into another buffer (read + write bytes), best of 5"}


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


def layer_bytes(lay, dims, prefix_len, W):
    """Algorithmic HBM bytes of one decoder layer: its weights once, the KV
    read once, the window's K/V written once."""
    total = sum(weight_bytes(lay[k]) for k in ("qkv", "o", "gate_up", "down"))
    total += (lay["in_norm"].numel() + lay["post_norm"].numel()) * 2
    if lay.get("qkv_bias") is not None:
        total += lay["qkv_bias"].numel() * 2
    per_tok = 2 * dims.n_kv_heads * dims.head_dim * 2
    keys = int(sum(int(p) + W for p in prefix_len.tolist()))
    return total + keys * per_tok + len(prefix_len) * W * per_tok


def oracle_rate(workload_name, sample_layers, min_seconds):
    """Oracle steps/s of a workload: whole passes over `sample_layers` of its
    decoder layers (then the final norm and the full lm_head argmax, when the
    workload has one) until min_seconds of work are measured, extrapolated to
    every layer."""
    import dataclasses

    import numpy as np  # noqa: F401
    from box_decoding_amd import synth

    import oracle as O

    w = synth.WORKLOADS[workload_name]
    d = w.dims
    ds = dataclasses.replace(d, n_layers=min(sample_layers, d.n_layers))
    model = synth.to_numpy_tree(synth.make_model(ds, w.wfmt, w.model_seed, "cpu"))
    model["dims"] = ds
    P = synth.draw_prefix_lens(w)
    cache = synth.to_numpy_tree(synth.make_cache(ds, P, w.window, seed=w.input_seed, device="cpu"))
    if w.lm_head:
        ids = synth.draw_window_ids(w.batch, w.window, d.vocab, w.input_seed).numpy()
        h0 = O.embed_rows(ids.reshape(-1), model["embed"])
    else:
        h0 = synth.make_hidden(w.batch * w.window, d.hidden, w.input_seed).numpy().astype("float64")
    lm = model["lm_head"] if model.get("lm_head") is not None else model["embed"]
    t_layers = t_lm = 0.0
    passes = 0
    while passes == 0 or t_layers + t_lm < min_seconds:
        h = h0
        t0 = time.perf_counter()
        for l in range(ds.n_layers):
            h, _, _ = O.decoder_layer(h, model["layers"][l], ds, cache, l, P.numpy(), w.window)
        t_layers += time.perf_counter() - t0
        if w.lm_head:
            f = O.rmsnorm(h, O.bf16_to_float(model["final_norm"]), d.rms_eps)
            t0 = time.perf_counter()
            O.lm_head_argmax(f, lm)
            t_lm += time.perf_counter() - t0
        passes += 1
    t_layers /= passes
    t_lm /= passes
    t_step = t_layers / ds.n_layers * d.n_layers + t_lm
    return 1.0 / t_step, {"passes": passes, "sampled_layers": ds.n_layers, "layers": d.n_layers,
                          "s_per_pass_layers": round(t_layers, 3), "s_per_pass_lm_head": round(t_lm, 3),
                          "s_per_step": round(t_step, 3)}


def cpu_baselines():
    """The oracle on the other workloads (BASELINE's CPU plan): the one-layer
    workload with every BLAS thread and with one, and one step of the batch-32,
    INT4 batch-8 and 16-sequence workloads from 2 of their 36 layers."""
    from threadpoolctl import threadpool_limits

    out = {}
    log("cpu_baseline: one layer, all threads / one thread")
    r, info = oracle_rate("layer_b1_p512", 1, 2.0)
    out["layer_b1_p512"] = {"steps_per_s": round(r, 3), **info}
    with threadpool_limits(limits=1):
        r, info = oracle_rate("layer_b1_p512", 1, 2.0)
    out["layer_b1_p512_1thread"] = {"steps_per_s": round(r, 3), "threads": 1, **info}
    for name in ("step_b32_ragged", "step_int4_b8_p1280", "emit_b16_p2048_x40"):
        log(f"cpu_baseline: {name}")
        r, info = oracle_rate(name, 2, 0.0)
        out[name] = {"steps_per_s": round(r, 4), **info}
    return out


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


def step_modes(B, dm, dc, ids, Pd, max_len, ws, out_ids, out_gap, timed, steps, warmup):
    """The step launched kernel by kernel and as a replayed HIP graph, each
    timed over `steps` steps after `warmup` untimed ones: (faster ms/step, its
    mode)."""
    def eager():
        B.pbd_step(dm, dc, ids, Pd, max_len, ws=ws, out_ids=out_ids, out_gap=out_gap)

    for _ in range(warmup):
        eager()
    e_ms, _ = timed(eager, steps)
    graph = B.StepGraph(dm, dc, ids, Pd, max_len, out_ids, out_gap, ws=ws)
    for _ in range(warmup):
        graph.replay()
    g_ms, _ = timed(graph.replay, steps)
    del graph
    return (e_ms, "eager") if e_ms <= g_ms else (g_ms, "graph")


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
    steps = max(5, args.steps // 3)
    ms_step, mode = step_modes(B, dm, dc, ids, Pd, max_len, ws, out_ids, out_gap, timed, steps,
                               max(2, args.warmup))
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
    gu_bytes = gate_up_bytes(model["layers"][0]["gate_up"], T, H, F)
    flops = 2.0 * T * H * 2 * F
    tflops = flops / (k_ms * 1e-3) / 1e12
    log(f"bench: batch 32: {ms_step:.3f} ms/step, {1000.0 / ms_step:.1f} steps/s; "
        f"gate_up GEMM {k_ms * 1e3:.1f} us, {tflops:.0f} TFLOP/s useful")
    del cache, dc, ws
    torch.cuda.synchronize()
    return {"workload": w.name, "batch": w.batch, "window": w.window, "steps": steps,
            "ms_per_step": round(ms_step, 4), "launch": mode, "steps_per_s": round(1000.0 / ms_step, 3),
            "windows_per_s": round(1000.0 / ms_step * w.batch, 2),
            "step_hbm_gbps": round(sbytes / ms_step / 1e6, 1),
            "step_hbm_frac": round(sbytes / ms_step / 1e6 / HBM_PEAK_GBPS, 4),
            "gate_up_gemm": {"rows": T, "launch_us": round(k_ms * 1e3, 2),
                             "useful_tflops": round(tflops, 1), "peak_tflops": MFMA_BF16_PEAK_TFLOPS,
                             "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                             "matrix_core_frac_with_hi_lo": round(2 * tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                             "bytes_per_launch": gu_bytes, "traffic": measured_traffic("gate_up_b32")}}


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
    steps = max(5, args.steps // 3)
    ms_step, mode = step_modes(B, dm, dc, ids, Pd, max_len, ws, out_ids, out_gap, timed, steps,
                               max(2, args.warmup))
    sbytes = step_bytes(model, d, P, w.window)
    log(f"bench: prefix 32768: {ms_step:.3f} ms/step, {1000.0 / ms_step:.1f} steps/s")
    del cache, dc, ws
    torch.cuda.synchronize()
    return {"workload": w.name, "batch": w.batch, "window": w.window, "prefix": int(P.max()),
            "steps": steps, "ms_per_step": round(ms_step, 4), "launch": mode, "steps_per_s": round(1000.0 / ms_step, 3),
            "step_hbm_gbps": round(sbytes / ms_step / 1e6, 1),
            "step_hbm_frac": round(sbytes / ms_step / 1e6 / HBM_PEAK_GBPS, 4)}


def emission_leg(B, synth, torch, dm, model, dev, stream, args):
    """The dense-scene emission loop: 16 sequences from prefix 2048, 40
    consecutive window steps, each appending the K/V of the 6 tokens it
    accepted: every step re-sends the tokens accepted last time causally before
    a new block of 6 (window W = 11: 5 re-fed rows, the block; the first step
    has the block only), and a device-side commit accepts the whole block --
    one captured graph of la_pbd_step_refeed + la_pbd_commit_refeed, 40
    replays."""
    w = synth.WORKLOADS["emit_b16_p2048_x40"]
    d = w.dims
    block, W = w.window, 2 * w.window - 1
    log("bench: emission-loop leg (re-fed windows)")
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
    mid = P + (1 + block * (w.steps - 1)) // 2
    sbytes = step_bytes(model, d, mid, W)
    log(f"bench: emission loop: {loop_ms:.2f} ms for {w.steps} steps, {ms_step:.3f} ms/step, "
        f"{w.batch * 1000.0 / ms_step:.0f} windows/s")
    del graph, cache, dc, ws
    torch.cuda.synchronize()
    return {"workload": w.name, "batch": w.batch, "window": W, "block": block, "refeed": True,
            "steps_per_loop": w.steps, "prefix_start": int(P.max()), "loop_ms": round(loop_ms, 3),
            "ms_per_step": round(ms_step, 4), "steps_per_s": round(1000.0 / ms_step, 3),
            "windows_per_s": round(1000.0 / ms_step * w.batch, 2),
            "step_hbm_gbps": round(sbytes / ms_step / 1e6, 1),
            "step_hbm_frac": round(sbytes / ms_step / 1e6 / HBM_PEAK_GBPS, 4)}


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


def sampling_leg(B, synth, torch, dm, model, dev, timed, args):
    """The batch-1 step with the sampled selection (temperature 0.7, top-p 0.9,
    the RK3588 page's defaults) in place of the argmax: the lm_head stores the
    logits, one workgroup per row samples them; the draw counter lives in device
    memory and advances on every replay."""
    w = synth.WORKLOADS["step_b1_p1280"]
    d = w.dims
    log("bench: sampling leg")
    P = synth.draw_prefix_lens(w)
    cache = synth.make_cache(d, P, w.window, seed=w.input_seed, device=dev)
    ids = synth.draw_window_ids(w.batch, w.window, d.vocab, w.input_seed, device=dev)
    dc = B.DeviceCache(cache, d.n_layers)
    Pd = P.to(dev)
    ws = B.Workspace(dev)
    out_ids = torch.empty((w.batch, w.window), dtype=torch.int32, device=dev)
    off = torch.zeros(1, dtype=torch.int64, device=dev)
    smp = B.Sampling(0.7, 0.9, seed=1, offset_dev=off)
    max_len = int(P.max()) + w.window
    B.pbd_step(dm, dc, ids, Pd, max_len, ws=ws, out_ids=out_ids, sampling=smp)  # sizes buffers
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        B.pbd_step(dm, dc, ids, Pd, max_len, ws=ws, out_ids=out_ids, want_gap=False, sampling=smp)
    for _ in range(max(2, args.warmup)):
        graph.replay()
    steps = max(5, args.steps // 3)
    g_ms, _ = timed(graph.replay, steps)
    e_ms, _ = timed(lambda: B.pbd_step(dm, dc, ids, Pd, max_len, ws=ws, out_ids=out_ids, want_gap=False,
                                       sampling=smp), steps)
    ms_step, mode = (e_ms, "eager") if e_ms <= g_ms else (g_ms, "graph")
    log(f"bench: sampled step, batch 1: {ms_step:.3f} ms/step, {1000.0 / ms_step:.1f} steps/s ({mode})")
    del graph, cache, dc, ws
    torch.cuda.synchronize()
    return {"workload": w.name, "selection": "temperature 0.7, top-p 0.9", "steps": steps, "launch": mode,
            "ms_per_step": round(ms_step, 4), "steps_per_s": round(1000.0 / ms_step, 3)}


def layer_leg(B, synth, torch, dev, timed, args, copies=5):
    """One decoder layer, batch 1, prefix 512 (la_pbd_layer, which also runs its
    per-call prologue), over `copies` weight copies in turn (770 MB > the 256 MB
    MALL, so no call finds its weights there), as one captured graph."""
    w = synth.WORKLOADS["layer_b1_p512"]
    d = w.dims
    log("bench: one-layer leg")
    dms, models = [], []
    for c in range(copies):
        m = B.pack_model(synth.make_model(d, "bf16", w.model_seed + 100 * c, dev))
        models.append(m)
        dms.append(B.DeviceModel(m))
    P = synth.draw_prefix_lens(w)
    cache = synth.make_cache(d, P, w.window, seed=w.input_seed, device=dev)
    dc = B.DeviceCache(cache, d.n_layers)
    x = synth.make_hidden(w.batch * w.window, d.hidden, w.input_seed, dev)
    Pd = P.to(dev)
    ws = B.Workspace(dev)
    max_len = int(P.max()) + w.window
    reps = 4 * copies
    B.pbd_layer(dms[0], 0, dc, x, Pd, w.batch, w.window, max_len, ws=ws)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for r in range(reps):
            B.pbd_layer(dms[r % copies], 0, dc, x, Pd, w.batch, w.window, max_len, ws=ws)
    graph.replay()
    ms, _ = timed(graph.replay, 3)
    us = ms * 1e3 / reps
    lbytes = layer_bytes(models[0]["layers"][0], d, P, w.window)
    log(f"bench: one layer (b1 p512): {us:.1f} us, {lbytes / us / 1e3:.0f} GB/s")
    del graph, cache, dc, ws, dms, models
    torch.cuda.synchronize()
    return {"workload": w.name, "batch": 1, "window": w.window, "prefix": int(P.max()),
            "weight_copies": copies, "us_per_layer": round(us, 2), "layer_bytes": lbytes,
            "hbm_gbps": round(lbytes / us / 1e3, 1), "hbm_frac": round(lbytes / us / 1e3 / HBM_PEAK_GBPS, 4)}


def int4_leg(B, synth, torch, dev, stream, timed, args, name="step_int4_b8_p1280"):
    """A quantised-weight step as graph replays: the INT4 weight-only step at
    batch 8, prefix 1280 (group-128 linears and lm_head, group-32 embedding
    gathered on the device), or (name step_w8a8_b1_p1280) the w8a8 step at
    batch 1 (int8 linears and lm_head, int8 activations per row)."""
    w = synth.WORKLOADS[name]
    d = w.dims
    log(f"bench: {w.wfmt} batch-{w.batch} leg")
    model = B.pack_model(synth.make_model(d, w.wfmt, w.model_seed, dev))
    dm = B.DeviceModel(model)
    P = synth.draw_prefix_lens(w)
    cache = synth.make_cache(d, P, w.window, seed=w.input_seed, device=dev)
    ids = synth.draw_window_ids(w.batch, w.window, d.vocab, w.input_seed, device=dev)
    dc = B.DeviceCache(cache, d.n_layers)
    Pd = P.to(dev)
    ws = B.Workspace(dev)
    out_ids = torch.empty((w.batch, w.window), dtype=torch.int32, device=dev)
    out_gap = torch.empty((w.batch, w.window), dtype=torch.float32, device=dev)
    steps = max(5, args.steps // 3)
    ms_step, mode = step_modes(B, dm, dc, ids, Pd, int(P.max()) + w.window, ws, out_ids, out_gap, timed, steps,
                               max(2, args.warmup))
    sbytes = step_bytes(model, d, P, w.window)
    # its dominant kernel: gate/up with the SiLU epilogue at 48 rows
    T, F, H = w.batch * w.window, d.inter, d.hidden
    xin = torch.randn((T, H), device=dev, generator=torch.Generator(device=dev).manual_seed(1))
    packed = B.pack_rows(xin, w.wfmt, norm_gain=model["layers"][0]["post_norm"])
    yout = torch.empty((T, F), dtype=torch.float32, device=dev)
    for l in range(3):
        B.wgemm_packed(packed, T, model["layers"][l]["gate_up"], silu_gate=True, out=yout)
    reps = 36

    def gemm():
        for r in range(reps):
            B.wgemm_packed(packed, T, model["layers"][r % d.n_layers]["gate_up"], silu_gate=True, out=yout)

    k_ms = timed(gemm, 1)[0] / reps
    gu_bytes = gate_up_bytes(model["layers"][0]["gate_up"], T, H, F)
    log(f"bench: {w.wfmt} batch {w.batch}: {ms_step:.3f} ms/step, {1000.0 / ms_step:.1f} steps/s; gate_up "
        f"{k_ms * 1e3:.1f} us, {gu_bytes / k_ms / 1e6:.0f} GB/s")
    del cache, dc, ws, dm, model
    torch.cuda.synchronize()
    return {"workload": w.name, "batch": w.batch, "window": w.window, "prefix": int(P.max()), "weights": w.wfmt,
            "steps": steps, "ms_per_step": round(ms_step, 4), "launch": mode, "steps_per_s": round(1000.0 / ms_step, 3),
            "windows_per_s": round(1000.0 / ms_step * w.batch, 2),
            "step_hbm_gbps": round(sbytes / ms_step / 1e6, 1),
            "step_hbm_frac": round(sbytes / ms_step / 1e6 / HBM_PEAK_GBPS, 4),
            "gate_up_gemm": {"rows": T, "launch_us": round(k_ms * 1e3, 2), "bytes_per_launch": gu_bytes,
                             "gbps": round(gu_bytes / k_ms / 1e6, 1),
                             "frac": round(gu_bytes / k_ms / 1e6 / HBM_PEAK_GBPS, 4),
                             "traffic": measured_traffic("gate_up_int4") if w.wfmt == "int4" else None}}


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
    steps = max(5, args.steps // 3)
    ms_step, mode = step_modes(B, dmc, dc, ids, Pd, int(P.max()) + w.window, ws, out_ids, out_gap, timed,
                               steps, max(2, args.warmup))
    log(f"bench: causal window, batch 1: {ms_step:.3f} ms/step, {1000.0 / ms_step:.1f} steps/s ({mode})")
    del cache, dc, ws
    torch.cuda.synchronize()
    return {"workload": w.name, "window_mask": "causal", "steps": steps, "launch": mode,
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
        pmc_summary(args.pmc_summary[0], args.pmc_summary[1])
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

    # the step launched kernel by kernel, and the same step captured once as a
    # HIP graph and replayed: each timed over the K steps, the faster one is
    # the value (a graph's per-node launch costs more here than it saves)
    for _ in range(args.warmup):
        eager()
    torch.cuda.synchronize()
    log(f"bench: warmup done, timing {args.steps} eager steps")
    eager_ms, eager_wall = timed(eager, args.steps)
    graph = B.StepGraph(dm, dc, ids, Pd, max_len, out_ids, out_gap, ws=ws)
    for _ in range(args.warmup):
        graph.replay()
    log(f"bench: eager {eager_ms:.3f} ms/step, timing {args.steps} graph replays")
    graph_ms, graph_wall = timed(graph.replay, args.steps)
    launch_mode = "eager" if eager_ms <= graph_ms else "graph"
    ms_step, wall_ms = (eager_ms, eager_wall) if launch_mode == "eager" else (graph_ms, graph_wall)
    steps_per_s = 1000.0 / ms_step
    sbytes = step_bytes(model, d, P, w.window)
    log(f"bench: {ms_step:.3f} ms/step (wall {wall_ms:.3f} ms), "
        f"{steps_per_s:.1f} steps/s, {sbytes / ms_step / 1e6:.0f} GB/s algorithmic")

    # Dominant kernel: the front half of each layer (one persistent launch at
    # up to 8 bf16 rows: RMSNorm, QKV, attention, O; the workloads with more
    # rows run it as separate kernels, and their line reports the gate/up GEMM
    # below), timed live with HIP events
    # the library records around every layer's attention block on its stream
    # (eager steps on the same inputs: the window's K/V land in the same slots).
    bev = B.BlockEvents(d.n_layers)
    block_ms = []
    for r in range(4):
        B.pbd_step(dm, dc, ids, Pd, max_len, ws=ws, out_ids=out_ids, out_gap=out_gap,
                   block_events=bev)
        torch.cuda.synchronize()
        if r:
            block_ms.extend(bev.ms())
    front_us = sum(block_ms) / len(block_ms) * 1e3
    fused = front_fuses_gate_up(w, args.row_major)
    fused_dn = front_fuses_down(w, args.row_major)
    fb = fused_layer_bytes if fused_dn else fused_front_bytes if fused else front_bytes
    fbytes = sum(fb(lay, d, P, w.window) for lay in model["layers"]) / d.n_layers
    front_gbps = fbytes / (front_us * 1e-6) / 1e9
    front_launch = w.batch * w.window <= 8 and w.wfmt == "bf16" and not args.row_major
    log(f"bench: attention block (front-half launch{' + gate/up' if fused else ''}{' + down' if fused_dn else ''}) "
        f"{front_us:.1f} us, {front_gbps:.0f} GB/s")

    # The weight-streaming kernel with the most bytes: the gate/up projection
    # with the SiLU epilogue (58% of a layer's weight bytes), the GEMM alone on
    # a pre-packed operand.  Timed with HIP events on the stream the library
    # launches on (torch's current stream), cycling through the 36 layers'
    # weights so that they stream from HBM.
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

    ceiling = hbm_ceiling(torch, dev)
    log(f"bench: practical HBM ceiling: copy {ceiling['copy_gbps']:.0f} GB/s")

    # a plain copy of known size: the scale for the HBM byte counters
    cal_src = torch.empty(CAL_COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
    cal_dst = torch.empty_like(cal_src)
    cal_dst.copy_(cal_src)
    torch.cuda.synchronize()
    del cal_src, cal_dst
    # the counters were taken on each workload's own tiled launches
    b1 = args.workload == "step_b1_p1280" and not args.row_major
    gu_kernel = {"step_b1_p1280": "gate_up", "step_b32_ragged": "gate_up_b32",
                 "step_int4_b8_p1280": "gate_up_int4"}.get(args.workload)
    traffic = measured_traffic(gu_kernel) if gu_kernel and not args.row_major else None
    front_traffic = measured_traffic("front") if b1 else None

    roof_gu = {"bound": "hbm", "kernel": "gate_up GEMM + SiLU (la_wgemm_packed)",
               "achieved": round(k_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
               "frac": round(k_gbps / HBM_PEAK_GBPS, 4), "traffic": traffic,
               "launch_us": round(k_ms * 1e3, 2), "bytes_per_launch": gu_bytes}
    roof_front = {"bound": "hbm",
                  "kernel": ("a layer in one persistent launch" if fused_dn else "front half of a layer, one persistent launch")
                            + " (k_front: RMSNorm, QKV, attention, O"
                            + (", gate/up + SiLU" if fused else "") + (", down)" if fused_dn else ")"),
                  "achieved": round(front_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                  "frac": round(front_gbps / HBM_PEAK_GBPS, 4), "traffic": front_traffic,
                  "launch_us": round(front_us, 2), "bytes_per_launch": round(fbytes)}
    result = {
        "metric": METRIC,
        "value": round(steps_per_s, 3),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "eager_ms_per_step": round(eager_ms, 5),
        "graph_ms_per_step": round(graph_ms, 5),
        "launch": launch_mode,
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
        "roofline": roof_front if front_launch else roof_gu,
        "hbm_ceiling": ceiling,
    }
    if front_launch:
        result["roofline_gate_up"] = roof_gu
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
        result["sampling"] = sampling_leg(B, synth, torch, dm, model, dev, timed, args)
        result["prefill"] = prefill_leg(B, synth, torch, dm, model, dev, timed, args)
        del dm, model
        torch.cuda.synchronize()
        result["layer_b1_p512"] = layer_leg(B, synth, torch, dev, timed, args)
        result["int4_b8"] = int4_leg(B, synth, torch, dev, stream, timed, args)
        result["w8a8_b1"] = int4_leg(B, synth, torch, dev, stream, timed, args, name="step_w8a8_b1_p1280")
    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(args.workload, args.cpu_sample_layers)
        if args.workload == "step_b1_p1280" and not args.no_extra_legs:
            result["cpu_baseline"]["other_workloads"] = cpu_baselines()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
