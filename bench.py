#!/usr/bin/env python3
"""Benchmark of the int4 weight-only greedy decode step on one MI355X.

The default run prints one JSON line with both halves of the metric:
  - batch 1 (the headline `value`): the 28-layer Qwen3-VL-2B-shaped text decoder
    (hidden 2048, 16/8 heads of 128, SwiGLU 6144, int4 group-128 decoder linears,
    bf16 lm_head of 151936 x 2048) at cache_position 700 of a 1024-slot static
    cache; exactly --steps steps (each one kmr_decode_step: embedding, 28 layers,
    final norm, lm_head, argmax) in one synchronised region split into 5 timed
    parts (median over the region, p10/p90 over the parts), repeating the step at
    the same cache position;
  - batch 4 ("batch4"): 4 continuous-batching rows (one finished) over the
    workload's 64 consecutive greedy steps with the token fed back and positions
    advancing on the device, the whole loop timed 5 times from its initial state;
  - one decoder layer ("layer"): kmr_decode_layer at batch 1, cache position 600,
    rotating over 16 copies of the layer's weights and cache so that the 256 MB
    Infinity Cache cannot serve them;
  - the device's streaming-read rate ("stream_read_peak"), measured with the same
    16-byte non-temporal loads the GEMVs use over a 4 GiB buffer, and each
    workload's GB/s as a fraction of it;
  - the CPU oracle baseline on batch-1 steps.
Weights, cache and inputs are seeded synthetic data made on the device.

Other workloads, one line each: `--workload step` (batch 1 only), `batch4` (its
steps timed as the headline), `long16` (16 rows with caches of 2048..8000 of
8192 positions, on the per-phase kernels with the matrix-core int4 GEMV; its
roofline covers the whole step), `layer`, `kv_copy` (kmr_kv_copy_row of a
1024-position row) and `prefill512` (kmr_prefill of a 512-token prompt; its
roofline is the matrix cores' fp16 dense peak).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

HBM_PEAK_GBPS = 8000.0
ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "int4_weight_only_gemv_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")
METRIC = "decode tok/s + achieved HBM GB/s (% of peak), int4 Qwen3-VL-2B shape, batch 1/4"


def algorithmic_bytes(dims, batch, cache_positions, with_lm=True):
    """Bytes the method must move for one step: int4 codes + (scale, zero) of every
    decoder linear, norm gains, embedding rows, K/V rows 0..c_b read (the new slot
    written), bf16 lm_head.  Activations (< 0.1 %) are not counted."""
    H, D, Hq, Hkv, I, G = dims.hidden, dims.head_dim, dims.n_heads, dims.n_kv_heads, dims.intermediate, dims.group_size
    lin = [((Hq + 2 * Hkv) * D, H), (H, Hq * D), (2 * I, H), (H, I)]
    w_layer = sum(n * k // 2 + n * (k // G) * 4 for n, k in lin) + (2 * H + 2 * D) * 2
    kv_read = sum(2 * Hkv * D * 2 * (int(c) + 1) for c in cache_positions)      # includes the new slot
    total = dims.n_layers * (w_layer + kv_read)
    if with_lm:
        total += dims.vocab * H * 2 + H * 2 + batch * H * 2
    return total


def _strip_comments(src):
    """C/C++ source without its comments and trailing blanks (string literals
    with comment markers inside are not expected in these files)."""
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    return "\n".join(line.rstrip() for line in src.splitlines() if line.strip())


def kernel_source_hash():
    """sha256 over the HIP sources (name + text without comments, sorted):
    identifies the kernel build that a stored counter summary was taken from, and
    stays put when only comments change."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".h", ".hip")):
            h.update(name.encode())
            with open(os.path.join(CSRC, name), encoding="utf-8") as f:
                h.update(_strip_comments(f.read()).encode())
    return h.hexdigest()


PROFILE_TAG = {"step": "qwen3vl2b_b1", "batch4": "qwen3vl2b_b4"}
# The kernel a step of these workloads runs: the persistent XCD-local step kernel
# (batch <= 4, 8 kv heads), one launch per step.
STEP_KERNEL = "k_stepx"


def stored_traffic(workload_name):
    """HBM bytes per launch of the step kernel from the committed rocprofv3 PMC
    summary of this workload (FETCH_SIZE + WRITE_SIZE, each scaled by the copy-kernel
    calibration factor), or None when there is none or the kernel sources changed
    since it was taken."""
    if workload_name not in PROFILE_TAG:
        return None
    path = os.path.join(PROFILES, f"{STEP_KERNEL}_{PROFILE_TAG[workload_name]}_pmc.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            m = re.match(r"^([a-z_0-9]+):\s*(\S+)", line.strip())
            if m:
                fields[m.group(1)] = m.group(2)
    if fields.get("kernel_source_sha256") != kernel_source_hash():
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration(mib):
    """A plain device copy of `mib` MiB (torch's copy kernel), launched three times,
    for scaling the FETCH_SIZE / WRITE_SIZE counters of a PMC run."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()


def build(workload_name):
    import torch
    from int4_weight_only_gemv_amd import kmr, synth
    w = synth.WORKLOADS[workload_name]
    seed = synth.base_seed(w)
    layers = []
    for l in range(w.dims.n_layers):
        layers.append(synth.layer_weights(w.dims, seed, l, where="device", device="cuda"))
    glob = synth.model_globals(w.dims, seed, where="device", device="cuda")
    model = kmr.DeviceModel(w.dims, layers, glob)
    kv = kmr.KVCache(model.cfg, w.batch, w.max_len, zero=False)
    k, v = synth.kv_cache(w.dims, seed, w.batch, w.max_len, where="device", device="cuda")
    kv.k.copy_(k)
    kv.v.copy_(v)
    del k, v
    torch.cuda.synchronize()
    return w, model, kv, layers, glob


def cpu_baseline(w, layers, glob, inp, budget_s=10.0):
    """The oracle as it stands, on this host's cores, over a bounded sample of the
    same workload: whole decode steps, as many as fit in about budget_s (at least 3)."""
    import oracle
    from int4_weight_only_gemv_amd import synth
    t0 = time.time()
    host_layers = [{k: oracle.as_u16(v) for k, v in l.items()} for l in layers]
    ora = oracle.Model(w.dims, host_layers, {k: oracle.as_u16(v) for k, v in glob.items()})
    del host_layers
    kh, vh = synth.kv_cache(w.dims, synth.base_seed(w), w.batch, w.max_len, where="device", device="cuda")
    kh, vh = oracle.as_u16(kh), oracle.as_u16(vh)
    setup = time.time() - t0
    times = []
    while len(times) < 3 or sum(times) < budget_s:
        t = time.time()
        ora.decode_step(kh, vh, inp["ids"], inp["positions"].copy(), inp["cache_position"].copy(),
                        finished=inp["finished"].copy(), want_logits=False)
        times.append(time.time() - t)
    sec = float(np.median(times))
    active = int((inp["finished"] == 0).sum())
    return {"value": active / sec, "unit": "tok/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": f"{len(times)} whole decode step(s) of the same workload (median {sec:.2f} s/step; "
                      f"oracle setup {setup:.1f} s untimed)"}


def bench_kv_copy(args):
    """Slot copy of a continuous-batching cache: row 0 of a batch-1 cache -> row 2 of
    a batch-4 cache, positions [0, 1024), every layer and kv head, K and V, at the
    28-layer model's cache shape (bf16 [28][B][8][1024][128])."""
    import torch
    from int4_weight_only_gemv_amd import kmr, synth
    dims = synth.WORKLOADS["step"].dims
    cfg = kmr.make_config(dims)
    M, n = 1024, 1024
    src = kmr.KVCache(cfg, 1, M, zero=False)
    dst = kmr.KVCache(cfg, 4, M, zero=True)
    g = torch.Generator(device="cuda").manual_seed(7)
    for t_ in (src.k, src.v):
        t_.copy_(torch.randn(t_.shape, generator=g, device="cuda").to(torch.bfloat16))
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        kmr.kv_copy_row(dst, 2, src, 0, n, stream=stream)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        kmr.kv_copy_row(dst, 2, src, 0, n, stream=stream)
    stop.record(stream)
    torch.cuda.synchronize()
    us = start.elapsed_time(stop) * 1000 / args.steps
    assert torch.equal(dst.k[:, 2], src.k[:, 0]) and torch.equal(dst.v[:, 2], src.v[:, 0])
    moved = 2 * 2 * dims.n_layers * dims.n_kv_heads * n * dims.head_dim * 2   # K and V, read + write
    gbps = moved / (us * 1e-6) / 1e9
    out = {"metric": "KV slot copy GB/s (read + write), Qwen3-VL-2B cache shape", "value": round(gbps, 1),
           "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(us / 1000, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "kv-row-copy-28L-8kv-128d-1024pos", "positions": n, "layers": dims.n_layers},
           "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                        "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None, "kernel": "k_kv_copy_row",
                        "launches_per_step": 1, "kernel_us_per_launch": round(us, 2)},
           "cpu_baseline": None}
    if not args.no_cpu_baseline:
        from oracle import slots
        sk, sv = src.k.cpu().view(torch.int16).numpy(), src.v.cpu().view(torch.int16).numpy()
        dk, dv = dst.k.cpu().view(torch.int16).numpy(), dst.v.cpu().view(torch.int16).numpy()
        reps, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < 3.0 or reps < 3:
            slots.kv_copy_row(dk, dv, 2, sk, sv, 0, n)
            reps += 1
        sec = (time.perf_counter() - t0) / reps
        out["cpu_baseline"] = {"value": round(moved / sec / 1e9, 2), "unit": "GB/s", "cores": 1,
                               "kind": "oracle", "sample": f"{reps} whole row copies (numpy, one thread)"}
    print(json.dumps(out), flush=True)


F16_DENSE_PEAK_TFLOPS = 2500.0   # MI355X dense fp16/bf16 matrix peak


def bench_prefill(args):
    """kmr_prefill of a 512-token prompt (token ids U[0, V), text positions t = h = w
    = 0..511) into row 0 of the 28-layer model's 1024-slot cache, start 0."""
    import torch
    from int4_weight_only_gemv_amd import kmr
    w, model, kv, _, _ = build("step")
    d, T = w.dims, 512
    g = torch.Generator(device="cuda").manual_seed(11)
    ids = torch.randint(0, d.vocab, (T,), generator=g, device="cuda", dtype=torch.int32)
    pos = torch.arange(T, dtype=torch.int32, device="cuda").repeat(3, 1).contiguous()
    ws = kmr.Workspace.for_prefill(model.cfg, T, w.max_len)
    nxt = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        model.prefill(kv, 0, ids, pos, 0, nxt, ws, stream=stream)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        model.prefill(kv, 0, ids, pos, 0, nxt, ws, stream=stream)
    stop.record(stream)
    torch.cuda.synchronize()
    assert ws.status() == 0
    ms = start.elapsed_time(stop) / args.steps
    # algorithmic flops: the decoder linears for every token, causal attention
    # (q k^T and p v over positions 0..t of token t), the lm_head for the last token
    lin = ((d.n_heads + 2 * d.n_kv_heads) * d.head_dim * d.hidden + d.hidden * d.n_heads * d.head_dim
           + 3 * d.intermediate * d.hidden)
    attn = 4 * d.n_heads * d.head_dim * T * (T + 1) // 2
    flops = d.n_layers * (2 * lin * T + attn) + 2 * d.vocab * d.hidden
    tflops = flops / (ms * 1e-3) / 1e12
    out = {"metric": "prefill tokens/s, 512-token prompt, Qwen3-VL-2B-shaped int4 decoder", "value": round(T / ms * 1e3, 1),
           "unit": "tok/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int4xf16->f32", "data": "synthetic",
           "config": {"workload": "prefill-512-tokens-28L-int4-g128", "tokens": T, "chunk": kmr.KMR_PREFILL_CHUNK},
           "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": F16_DENSE_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(tflops / F16_DENSE_PEAK_TFLOPS, 5), "traffic": None,
                        "kernel": "whole prefill, one 512-token chunk: per layer 4 stagings, 4 matrix-core "
                                  "int4 GEMMs (128-token x 64-row tiles), q/k norm + RoPE, causal flash attention",
                        "launches_per_step": 10 * d.n_layers + 4, "kernel_us_per_launch": None},
           "cpu_baseline": None}
    print(json.dumps(out), flush=True)


def timed_segments(stream, run, n, segments):
    """Runs run(i) for i < n inside one region bracketed by synchronisations, with
    events between `segments` equal parts; returns (ms per call over the region,
    [ms per call of each part], wall seconds)."""
    import torch
    cuts = [round(k * n / segments) for k in range(segments + 1)]
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(segments + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs[0].record(stream)
    for k in range(segments):
        for i in range(cuts[k], cuts[k + 1]):
            run(i)
        evs[k + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    parts = [evs[k].elapsed_time(evs[k + 1]) / max(cuts[k + 1] - cuts[k], 1) for k in range(segments)]
    return evs[0].elapsed_time(evs[-1]) / n, parts, wall


def per_launch_ms(stream, run, n):
    """Average duration of one call with events right around it (a separate pass)."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    torch.cuda.synchronize()
    for i in range(n):
        evs[i][0].record(stream)
        run(i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in evs]))


def pct(xs, q):
    return float(np.percentile(np.asarray(xs, np.float64), q))


def stream_read_peak(reps=10, gib=4):
    """Achievable streaming-read rate of this device: kmr_read_probe over a buffer of
    `gib` GiB (16x the 256 MB Infinity Cache), best of `reps` timed passes."""
    import torch
    from int4_weight_only_gemv_amd import kmr
    buf = torch.ones(gib * (1 << 30) // 4, dtype=torch.int32, device="cuda")
    sink = torch.empty(kmr.KMR_READ_PROBE_THREADS, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    for _ in range(2):
        kmr.read_probe(buf, sink, stream=stream)
    times = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        kmr.read_probe(buf, sink, stream=stream)
        b.record(stream)
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    nbytes = buf.numel() * 4
    del buf
    torch.cuda.empty_cache()
    return {"gbps": round(nbytes / (min(times) * 1e-3) / 1e9, 1), "bytes": nbytes, "passes": reps,
            "kernel": "k_read_probe (16-byte non-temporal loads)", "frac_of_spec": None}


def bench_batch4(model, kv, w, loops=5):
    """The batch-4 workload as specified: 64 consecutive greedy steps with the token
    fed back and positions advancing on the device, timed as one region per loop,
    each loop from the workload's initial state."""
    import torch
    from int4_weight_only_gemv_amd import kmr, synth
    inp = synth.step_inputs(w)
    B, steps = w.batch, w.steps
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    ws = kmr.Workspace(model.cfg, B, w.max_len)
    ids = [dev(inp["ids"]), torch.zeros(B, dtype=torch.int32, device="cuda")]
    pos, cpos, fin = dev(inp["positions"]), dev(inp["cache_position"]), dev(inp["finished"])
    stream = torch.cuda.current_stream()

    def reset():
        ids[0].copy_(dev(inp["ids"])); pos.copy_(dev(inp["positions"]))
        cpos.copy_(dev(inp["cache_position"])); fin.copy_(dev(inp["finished"]))

    def step(i):
        model.decode_step(kv, ids[i % 2], pos, cpos, ids[(i + 1) % 2], ws, finished=fin, advance=True, stream=stream)

    for i in range(10):
        step(i)
    loop_ms = []
    for _ in range(loops):
        reset()
        ms, _, _ = timed_segments(stream, step, steps, 1)
        loop_ms.append(ms)
    reset()
    kernel_ms = per_launch_ms(stream, step, steps)
    reset()
    # tokens produced by live rows over the loop (rows that finish by length stop counting)
    live_tokens, c, f = 0, inp["cache_position"].astype(np.int64).copy(), inp["finished"].astype(bool).copy()
    mean_c = []
    for _ in range(steps):
        live_tokens += int((~f).sum())
        mean_c.append(c.copy())
        adv = ~f & (c + 1 < w.max_len)
        f |= ~f & (c + 1 >= w.max_len)
        c = c + adv
    status = ws.status()
    if status:
        raise SystemExit(f"batch4: device status bits set: {status}")
    cps = np.mean(np.stack(mean_c), axis=0)
    nbytes = algorithmic_bytes(w.dims, B, cps)
    med = float(np.median(loop_ms))
    kernel_gbps = nbytes / (kernel_ms * 1e-3) / 1e9
    return {
        "workload": f"qwen3vl2b-28L-int4g128-decode-b{B}-{steps}steps", "batch": B,
        "active_rows_at_start": int((inp["finished"] == 0).sum()), "steps_per_loop": steps, "loops": loops,
        "tok_s": round(live_tokens / (med * steps * 1e-3), 1),
        "ms_per_step": round(med, 4), "ms_per_step_p10": round(pct(loop_ms, 10), 4),
        "ms_per_step_p90": round(pct(loop_ms, 90), 4),
        "hbm_gbps": round(nbytes / (med * 1e-3) / 1e9, 1),
        "hbm_frac_of_peak": round(nbytes / (med * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "algorithmic_bytes_per_step": int(nbytes),
        "roofline": {"bound": "hbm", "achieved": round(kernel_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(kernel_gbps / HBM_PEAK_GBPS, 4), "traffic": stored_traffic("batch4"),
                     "kernel": STEP_KERNEL, "launches_per_step": 1,
                     "kernel_us_per_launch": round(kernel_ms * 1000, 1)},
    }


def bench_layer(copies=16, rounds=10):
    """One full-size decoder layer (kmr_decode_layer, batch 1, cache position 600 of
    1024) over `copies` distinct copies of the layer's weights and KV cache used in
    turn, so that the 256 MB Infinity Cache cannot hold them between uses (16 copies
    = 16 x 26.7 MB of weights + 16 x 4.2 MB of cache rows)."""
    import torch
    from int4_weight_only_gemv_amd import kmr, synth
    w = synth.WORKLOADS["layer"]
    d, seed = w.dims, synth.base_seed(w)
    inp = synth.step_inputs(w)
    models, caches = [], []
    for i in range(copies):
        lw = synth.layer_weights(d, seed + 101 * i, 0, where="device", device="cuda")
        models.append(kmr.DeviceModel(d, [lw], None))
        kv = kmr.KVCache(models[-1].cfg, 1, w.max_len, zero=False)
        k, v = synth.kv_cache(d, seed + 101 * i, 1, w.max_len, where="device", device="cuda")
        kv.k.copy_(k); kv.v.copy_(v)
        caches.append(kv)
        del lw, k, v
    ws = kmr.Workspace(models[0].cfg, 1, w.max_len)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    x = synth.hidden_input(d, seed, 1).cuda()
    x0 = x.clone()
    pos, cpos = dev(inp["positions"]), dev(inp["cache_position"])
    stream = torch.cuda.current_stream()

    def run(i):
        models[i % copies].decode_layer(0, caches[i % copies], x, pos, cpos, ws, stream=stream)

    for i in range(2 * copies):
        run(i)
    x.copy_(x0)
    n = copies * rounds
    ms, parts, _ = timed_segments(stream, run, n, 5)
    status = ws.status()
    if status:
        raise SystemExit(f"layer: device status bits set: {status}")
    nbytes = algorithmic_bytes(d, 1, [int(c) for c in inp["cache_position"]], with_lm=False)
    gbps = nbytes / (ms * 1e-3) / 1e9
    out = {"workload": "qwen3vl2b-1layer-int4g128-decode-b1-c600", "copies_rotated": copies, "calls": n,
           "us_per_layer": round(ms * 1000, 2), "us_per_layer_p10": round(pct(parts, 10) * 1000, 2),
           "us_per_layer_p90": round(pct(parts, 90) * 1000, 2), "algorithmic_bytes": int(nbytes),
           "hbm_gbps": round(gbps, 1), "hbm_frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4),
           "path": "kmr_decode_layer (per-phase kernels: prep, QKV GEMV, attention, O GEMV with the split merge, "
                   "gate-up GEMV, down GEMV)"}
    del models, caches
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", choices=["default", "step", "batch4", "long16", "layer", "kv_copy", "prefill512"],
                    default="default",
                    help="default: batch 1 (the headline), the 64-step batch-4 loop, the single layer and the "
                         "streaming-read peak in one line")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="first run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this decode step runs on a single MI355X and "
              "is not sharded across GPUs (--gpus must be 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    from int4_weight_only_gemv_amd import kmr, synth

    if args.calibrate_copy_mib > 0:
        copy_calibration(args.calibrate_copy_mib)
    if args.workload == "kv_copy":
        bench_kv_copy(args)
        return
    if args.workload == "prefill512":
        bench_prefill(args)
        return
    if args.workload == "layer":
        print(json.dumps(bench_layer()), flush=True)
        return
    full = args.workload == "default"
    headline = "step" if full else args.workload
    w, model, kv, layers, glob = build(headline)
    inp = synth.step_inputs(w)
    B = w.batch
    ws = kmr.Workspace(model.cfg, B, w.max_len)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    ids = [dev(inp["ids"]), torch.zeros(B, dtype=torch.int32, device="cuda")]
    pos, cpos, fin = dev(inp["positions"]), dev(inp["cache_position"]), dev(inp["finished"])
    advance = headline == "batch4"
    stream = torch.cuda.current_stream()

    def step(i):
        model.decode_step(kv, ids[i % 2], pos, cpos, ids[(i + 1) % 2], ws, finished=fin,
                          advance=advance, stream=stream)

    def reset():
        ids[0].copy_(dev(inp["ids"])); pos.copy_(dev(inp["positions"]))
        cpos.copy_(dev(inp["cache_position"])); fin.copy_(dev(inp["finished"]))

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    if advance:   # restart the timed run from the workload's own state
        reset()
    # exactly `steps` steps in one synchronised region, with events between 5 equal parts
    segs = min(5, args.steps)
    ms, parts, wall = timed_segments(stream, step, args.steps, segs)
    # the step kernel's own average launch duration: events right around each launch,
    # in a second pass of the same steps
    if advance:
        reset()
    kernel_ms = per_launch_ms(stream, step, args.steps)
    status = ws.status()
    if status:
        print(f"device status bits set: {status}", file=sys.stderr)
        sys.exit(3)

    active = int((inp["finished"] == 0).sum())
    if advance:   # positions advance by one per step for live rows: mean over the run
        cps = [int(c) + args.steps / 2 for c, f in zip(inp["cache_position"], inp["finished"])]
    else:
        cps = [int(c) for c in inp["cache_position"]]
    nbytes = algorithmic_bytes(w.dims, B, cps)
    gbps = nbytes / (ms * 1e-3) / 1e9
    kernel_gbps = nbytes / (kernel_ms * 1e-3) / 1e9
    tok_s = active * 1000.0 / ms
    out = {
        "metric": METRIC, "value": round(tok_s, 2), "unit": "tok/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        # int4 weights times fp16 activations (dequantized in registers) with fp32
        # accumulation; bf16 lm_head with fp32 accumulation; fp32 norms and attention
        "dtype": "int4xf16->f32",
        "data": "synthetic",
        "config": {"workload": f"qwen3vl2b-28L-int4g128-decode-b{B}", "batch": B,
                   "active_rows": active, "cache_position": [int(c) for c in inp["cache_position"]],
                   "max_len": w.max_len, "layers": w.dims.n_layers, "vocab": w.dims.vocab},
        "hbm_gbps": round(gbps, 1), "hbm_frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4),
        "ms_per_step_p10": round(pct(parts, 10), 4), "ms_per_step_p90": round(pct(parts, 90), 4),
        "timing_parts": segs,
        "algorithmic_bytes_per_step": nbytes, "wall_s_timed": round(wall, 4),
        # One launch of the persistent step kernel per step (all layers,
        # final norm, lm_head and argmax), so its algorithmic bytes per launch are
        # the step's; its average launch duration comes from per-launch events.
        # (long16: the per-phase kernels, so the figure covers the whole step.)
        "roofline": {"bound": "hbm", "achieved": round(kernel_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(kernel_gbps / HBM_PEAK_GBPS, 4), "traffic": stored_traffic(headline),
                     "kernel": STEP_KERNEL if B <= 4 else "per-phase step kernels (k_gemv_int4_mfma, k_attn, "
                                                          "k_lmhead, ...)",
                     "launches_per_step": 1 if B <= 4 else None,
                     "kernel_us_per_launch": round(kernel_ms * 1000, 1) if B <= 4 else None,
                     "step_us": round(kernel_ms * 1000, 1)},
        "cpu_baseline": None,
    }
    del ws
    if full:
        del kv
        torch.cuda.empty_cache()
        w4 = synth.WORKLOADS["batch4"]
        kv4 = kmr.KVCache(model.cfg, w4.batch, w4.max_len, zero=False)
        k, v = synth.kv_cache(w4.dims, synth.base_seed(w4), w4.batch, w4.max_len, where="device", device="cuda")
        kv4.k.copy_(k); kv4.v.copy_(v)
        del k, v
        out["batch4"] = bench_batch4(model, kv4, w4)
        del kv4
        torch.cuda.empty_cache()
        out["layer"] = bench_layer()
        peak = stream_read_peak()
        peak["frac_of_spec"] = round(peak["gbps"] / HBM_PEAK_GBPS, 4)
        out["stream_read_peak"] = peak
        out["hbm_frac_of_stream_peak"] = round(gbps / peak["gbps"], 4)
        out["batch4"]["hbm_frac_of_stream_peak"] = round(out["batch4"]["hbm_gbps"] / peak["gbps"], 4)
        out["layer"]["hbm_frac_of_stream_peak"] = round(out["layer"]["hbm_gbps"] / peak["gbps"], 4)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, layers, glob, inp)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
