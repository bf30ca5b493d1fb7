"""Benchmark of one decode step over a low-rank, quantised KV cache on one MI355X.

A step is one pass of the hot path for one decoder layer, one starkv_decode_step call:
compress_append of the step's n_q new tokens per sequence (latent projection +
quantise/round + pack), then decode attention read directly from the latent cache (query
projection, key scores and softmax statistics, P.C_v, split merge and up-projection); the
append and the query projection share the first launch.  Inputs are resident in HBM before
timing starts.  Steps rotate over distinct layers (own factors, own cache) totalling more
than 1 GiB, so every step reads cold HBM rather than the 256 MB Infinity Cache.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 4] [--no-cpu] [--no-sub]
Prints one JSON line on stdout; progress goes to stderr.  The headline is workload 4, the
13B-class high-batch step (64 ragged sequences, 4 queries each); the 7B-class bf16 and int8/int4
layers and the long-context GQA layer are measured in the same run as sub-results.

Two helper modes serve the HBM-traffic figures:
  --copy-probe       copies 1 GiB between two device buffers a few times (a plain copy
                     kernel of known size, run under rocprofv3 --pmc to calibrate counters);
  --pmc-summary F W CF CW  reads four rocprofv3 --pmc output folders (FETCH_SIZE and
                     WRITE_SIZE of a bench run, then of the copy probe), prints a summary and
                     records bytes per launch of each step kernel in profiles/traffic.json.
"""

from __future__ import annotations

import argparse
import csv
import dataclasses
import gc
import glob
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "low-rank KV decode attention queries/s + achieved HBM GB/s vs ~8 TB/s peak"
HBM_PEAK_GBPS = 8000.0
MIN_ROTATION_BYTES = 1 << 30
EAGER_SEG = 32  # eager steps issued between synchronisations


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def to_dev_bf16(x: np.ndarray, dev: str):
    import torch
    from rank_kv_cache_starkv_amd import inputs as I
    return torch.from_numpy(I.to_bf16_bits(x).view(np.int16)).to(dev).view(torch.bfloat16)


# quantised latents: the denominator of the high-precision share (int8 region) of a segment
QUANTIZED = {"mix84": 4, "had43": 5, "had43p": 5}


def algorithmic_bytes(w, ranks, r_v, lens, n_q, hidden=False):
    """Bytes the method must move per step (each latent once, factors once, q, out, X_new, A).
    hidden: the hidden states [B, n_q, d] meet the absorbed factors W_q^h B_g^T (G n_key x d,
    4 bytes per element) in a GEMM that writes the raw projection (fp32), which the query
    projection then reads instead of q and B_k."""
    elem = {"f32": 4, "bf16": 2}[w.dtype]
    if w.latent in QUANTIZED:
        # bytes of the int8 region (leading quarter, or the outlier fifth) + the int4 region;
        # packed (had43p): 4-bit outliers + 3-bit inliers
        den = QUANTIZED[w.latent]
        n8 = [-(-int(r) // den) for r in ranks]
        n8v = -(-r_v // den)
        hi_b, lo_b = (0.5, 3.0 / 8.0) if w.latent == "had43p" else (1.0, 0.5)
        key_tok = hi_b * sum(n8) + lo_b * (sum(int(r) for r in ranks) - sum(n8))
        val_tok = hi_b * n8v + lo_b * (r_v - n8v)
        scale_k, scale_v = 2 * int(sum(ranks)), 2 * r_v
    else:
        le = 4 if w.latent == "f32" else 2
        key_tok, val_tok = le * float(sum(ranks)), le * float(r_v)
        scale_k = scale_v = 0
    n_key = int(sum(ranks))
    tokens = float(np.sum(lens))
    qo = w.B * n_q * w.H_q * w.d_h * elem
    qproj = qo + n_key * w.d_h * elem + scale_k
    raw = w.B * n_q * (w.H_q // w.H_kv) * n_key * 4
    if hidden:
        qproj = raw + scale_k
    b = {
        "decode_qproj": qproj,
        "decode_scores": tokens * key_tok,
        "decode_values": tokens * val_tok,
        "decode_zmerge": scale_v,
        "decode_upproj": r_v * w.H_kv * w.d_h * elem + qo,
        "append": w.B * n_q * w.d * elem + (n_key + r_v) * w.d * elem + w.B * n_q * (key_tok + val_tok)
        + scale_k + scale_v,
    }
    if hidden:
        b["decode_hidden_q"] = w.B * n_q * w.d * elem + (w.H_q // w.H_kv) * n_key * w.d * 4 + raw
    b["decode"] = sum(v for k, v in b.items() if k.startswith("decode_"))
    b["step"] = b["decode"] + b["append"]
    b["step_front"] = b["append"] + b["decode_qproj"]  # fused launch: append + query projection
    return b


# dense MFMA peaks of MI355X (TFLOP/s or TOP/s) by the operand type each decode contraction uses
MFMA_PEAK = {"f32": 157.3, "bf16": 2500.0, "f16": 2500.0, "i8": 5000.0}


def algorithmic_flops(w, ranks, r_v, lens, n_q):
    """Multiply-adds (x2) the decode contractions must do per step, with the MFMA operand type of
    each: key scores (every query row against its KV head's r_g channels of every cached token),
    value aggregation (every query row against the r_v value channels of every token) and the
    up-projection (r_v x d_h per row and head)."""
    tokens = float(np.sum(lens))
    G = w.H_q // w.H_kv
    n_key = int(sum(ranks))
    quant = w.latent in QUANTIZED
    t_sc = "f32" if w.latent == "f32" else ("i8" if quant else "bf16")
    t_v = "f32" if w.latent == "f32" else ("f16" if quant else "bf16")
    return {
        "decode_scores": (2.0 * n_q * G * n_key * tokens, t_sc),
        "decode_values": (2.0 * w.H_q * n_q * r_v * tokens, t_v),
        "decode_upproj": (2.0 * w.B * n_q * w.H_q * r_v * w.d_h, "f32" if w.latent == "f32" else "bf16"),
    }


def roofline_of(kernel, us, byts, flops, traffic):
    """Roofline of one kernel: HBM (algorithmic bytes at 8 TB/s) and MFMA (algorithmic flops at
    the dense peak of its operand type); the bound is the larger of the two ideal times, and both
    fractions are reported."""
    t_hbm = byts / (HBM_PEAK_GBPS * 1e9)
    hbm = {"achieved": byts / (us * 1e-6) / 1e9, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
           "frac": byts / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS}
    r = {"kernel": kernel, "traffic": traffic, "alg_bytes_per_launch": byts, "us_per_launch": us}
    if flops is not None:
        fl, ty = flops
        peak = MFMA_PEAK[ty]
        t_mfma = fl / (peak * 1e12)
        mfma = {"achieved": fl / (us * 1e-6) / 1e12, "peak": peak, "unit": "TFLOP/s" if ty != "i8" else "TOP/s",
                "frac": fl / (us * 1e-6) / 1e12 / peak, "operands": ty}
        r["alg_flops_per_launch"] = fl
        r["hbm"] = hbm
        r["mfma"] = mfma
        if t_mfma > t_hbm:
            return {"bound": "mfma", **{k: mfma[k] for k in ("achieved", "peak", "unit", "frac")}, **r}
    return {"bound": "hbm", **{k: hbm[k] for k in ("achieved", "peak", "unit", "frac")}, **r}


def source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "rank_kv_cache_starkv_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h")):
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def traffic_for(kernel: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counters, if taken on the current kernels."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except Exception:
        return None
    e = d.get(workload, {}).get(kernel)
    if not e or e.get("source_hash") != source_hash():
        return None
    return float(e["bytes_per_launch"])


KERNEL_KEYS = (("k_step_front", "step_front"), ("k_qproj", "decode_qproj"), ("k_scores", "decode_scores"),
               ("k_values", "decode_values"), ("k_zmerge", "decode_zmerge"), ("k_upproj", "decode_upproj"),
               ("k_latent_gemm", "append"))


COPY_PROBE_MIB = 1024


def copy_probe(mib: int = COPY_PROBE_MIB) -> int:
    """A plain device-to-device copy of known size, for calibrating the traffic counters."""
    import torch
    n = mib << 20
    src = torch.ones((n,), dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "launches": 5}))
    return 0


def _pmc_rows(folder: str):
    files = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {folder}")
    rows = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            key = (f, int(r["Dispatch_Id"]))
            e = rows.setdefault(key, {"name": r["Kernel_Name"], "grid": int(r["Grid_Size"]), "v": 0.0})
            e["v"] += float(r["Counter_Value"])  # KiB; summed over the counter's instances
    return [rows[k] for k in sorted(rows)]


def _step_kernels(rows):
    """Per-launch counter values of the step kernels, keyed like the bench's kernel timers:
    only dispatches from the first step's front launch on (prefill launches come before it)."""
    first = next((i for i, r in enumerate(rows) if "k_qproj" in r["name"] or "k_step_front" in r["name"]), None)
    out = {}
    if first is None:
        return out
    # without the fused front launch the step's append precedes its query projection
    start = first if "k_step_front" in rows[first]["name"] else max(0, first - 1)
    for r in rows[start:]:
        for pat, key in KERNEL_KEYS:
            if pat in r["name"]:
                out.setdefault(key, []).append(r["v"])
    return out


def pmc_summary(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, workload: str) -> int:
    def copy_kib(folder):
        vals = [r["v"] for r in _pmc_rows(folder) if "copy" in r["name"].lower()]
        return float(np.median(vals)), len(vals)
    cf, ncf = copy_kib(copy_fetch_dir)
    cw, ncw = copy_kib(copy_write_dir)
    copy_bytes = float(COPY_PROBE_MIB << 20)
    f_fetch = copy_bytes / (cf * 1024.0)
    f_write = copy_bytes / (cw * 1024.0)
    fk = _step_kernels(_pmc_rows(fetch_dir))
    wk = _step_kernels(_pmc_rows(write_dir))
    path = os.path.join(ROOT, "profiles", "traffic.json")
    d = json.load(open(path)) if os.path.exists(path) else {}
    ent = d.setdefault(workload, {})
    h = source_hash()
    print(f"copy probe {copy_bytes / 2**20:.0f} MiB: FETCH_SIZE {cf:.0f} KiB ({ncf} launches) -> factor {f_fetch:.3f}; "
          f"WRITE_SIZE {cw:.0f} KiB ({ncw} launches) -> factor {f_write:.3f}")
    print(f"workload {workload}, kernel sources {h}")
    print("| kernel | launches | FETCH_SIZE KiB/launch | WRITE_SIZE KiB/launch | calibrated HBM MB/launch |")
    print("|---|---|---|---|---|")
    for key in [k for _, k in KERNEL_KEYS]:
        if key not in fk or key not in wk:
            continue
        fv, wv = float(np.mean(fk[key])), float(np.mean(wk[key]))
        tb = f_fetch * fv * 1024.0 + f_write * wv * 1024.0
        print(f"| {key} | {len(fk[key])} | {fv:.1f} | {wv:.1f} | {tb / 1e6:.3f} |")
        ent[key] = {"bytes_per_launch": tb, "fetch_kib": fv, "write_kib": wv, "fetch_factor": f_fetch,
                    "write_factor": f_write, "source_hash": h}
    json.dump(d, open(path, "w"), indent=1, sort_keys=True)
    return 0


def host_info() -> dict:
    """The host the CPU baseline ran on: core counts, CPU model, BLAS library and its threads."""
    info = {"os_cpu_count": os.cpu_count()}
    try:
        info["affinity"] = len(os.sched_getaffinity(0))
    except Exception:
        info["affinity"] = None
    try:
        model = [ln.split(":", 1)[1].strip() for ln in open("/proc/cpuinfo") if ln.startswith("model name")]
        info["cpu_model"] = model[0] if model else None
    except Exception:
        info["cpu_model"] = None
    try:
        from threadpoolctl import threadpool_info
        blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        info["blas"] = [f"{p.get('internal_api')} {p.get('version')} ({p.get('num_threads')} threads)" for p in blas]
        info["blas_threads"] = max((p.get("num_threads", 1) for p in blas), default=1)
    except Exception:
        info["blas"], info["blas_threads"] = None, None
    return info


def cpu_baseline(w, lf, lens, n_q, X0, Xcal, q_step, X_step, budget_s: float):
    """The CPU oracle (NumPy fp64) on one sequence: one decode step = append n_q tokens +
    attention, repeated until ``budget_s`` of CPU time is used; then the same with one BLAS
    thread for a fifth of the budget, and the append alone."""
    from oracle import starkv_oracle as O
    host = host_info()
    OL = O.build_layer(lf.U_k, lf.s_k, lf.V_k, lf.tau_k, lf.U_v, lf.s_v, lf.V_v, lf.tau_v, w.H_q, w.latent, w.dtype)
    scales = O.calibrate_scales(Xcal, OL.A_cat, O.channel_qmax(OL)) if w.latent in QUANTIZED else None
    t_setup = time.perf_counter()
    base = O.compress(X0, OL, scales)
    log(f"[cpu] oracle prefill of sequence 0 ({X0.shape[0]} tokens): {time.perf_counter() - t_setup:.1f} s")

    def run(budget):
        reps, spent = 0, 0.0
        while spent < budget or reps == 0:
            t0 = time.perf_counter()
            new = O.compress(X_step[0], OL, scales)
            cache = O.SequenceCache(np.concatenate([base.key, new.key]), np.concatenate([base.value, new.value]))
            O.decode(q_step[0].astype(np.float64), cache, OL, n_q, scales)
            spent += time.perf_counter() - t0
            reps += 1
        return reps, spent

    reps, spent = run(budget_s)
    qps = reps * n_q / spent
    # the append alone (projection + quantisation of the step's tokens), all BLAS threads
    t0, na = time.perf_counter(), 0
    while time.perf_counter() - t0 < 1.0 or na == 0:
        O.compress(X_step.reshape(-1, X_step.shape[-1]), OL, scales)
        na += 1
    append_tps = na * X_step.shape[0] * X_step.shape[1] / (time.perf_counter() - t0)
    single = None
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            r1, s1 = run(budget_s / 5)
        single = r1 * n_q / s1
    except Exception:
        pass
    return {"value": qps, "unit": "queries/s", "cores": int(host.get("blas_threads") or host["os_cpu_count"] or 1),
            "kind": "oracle",
            "sample": f"sequence 0 of {w.B} (context {int(lens[0])}), {reps} decode steps "
                      f"(append {n_q} token(s) + attention), {spent:.1f} s; GPU value is all {w.B} sequences",
            "single_thread_value": single, "append_tokens_per_s": append_tps, "host": host}


def measure(w, args, dev, with_cpu: bool, steps: int, warmup: int) -> dict:
    """Set up one workload (rotated layers, prefilled caches), time `steps` decode steps (graph
    replay: exactly `steps` steps in one captured graph; eager alongside), time each kernel, and
    return the result fields of the JSON line."""
    import torch
    import rank_kv_cache_starkv_amd as S
    from rank_kv_cache_starkv_amd import inputs as I

    n_q = w.n_q
    lens = I.context_lengths(w) + w.n_append  # lengths at decode (include the n_q step tokens)
    if not w.ragged:
        lens = np.full(w.B, w.T, np.int32)
    lens = lens.astype(np.int32)
    lens_pre = (lens - n_q).astype(np.int32)  # each step appends at lens_pre and attends over lens
    T_max = int(-(-int(lens.max()) // 32) * 32)
    if args.lens_dev:
        # device lengths: the plan and the cache take a capacity, the kernels read the lengths
        T_max = max(T_max, int(-(-args.lens_dev // 32) * 32))
    tdt = torch.float32 if w.dtype == "f32" else torch.bfloat16

    t0 = time.perf_counter()
    lf = I.layer_factors(w, 0)
    log(f"[setup] workload {w.cfg_id} {w.name}: host factors {time.perf_counter() - t0:.1f} s")
    U = [torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev) for a in (lf.U_k, lf.V_k, lf.U_v, lf.V_v)]
    Xcal = I.as_dtype(I.x_calibration(w), w.dtype) if w.latent in QUANTIZED else None
    gen = torch.Generator(device=dev)
    gen.manual_seed(2606_08382)

    def new_layer():
        L = S.Layer(w.H_q, w.H_kv, w.d_h, w.d, w.dtype, w.latent, lf.s_k, lf.tau_k, lf.s_v, lf.tau_v)
        L.build_factors(*U)
        if Xcal is not None:
            L.calibrate(to_dev_bf16(Xcal, dev) if w.dtype == "bf16" else torch.from_numpy(Xcal).to(dev))
        if args.rope:
            L.set_rope(args.rope)
        return L

    probe = new_layer()
    kb, vb = probe.cache_bytes(w.B, T_max)
    inf = probe.info
    per_layer = kb + vb + inf["a_bytes"] + inf["bk_bytes"] + inf["bv_bytes"]
    n_layers = args.layers or max(2, math.ceil(MIN_ROTATION_BYTES / per_layer))
    log(f"[setup] {n_layers} layers x {per_layer / 2**20:.0f} MiB (cache {(kb + vb) / 2**20:.0f} MiB), T_max {T_max}")

    # host-generated prefill of sequence 0 of layer 0 (the CPU baseline attends over the same tokens)
    X0 = I.as_dtype(I.x_prefill(w, 0, 0, int(lens_pre[0])), w.dtype)
    layers, caches = [], []
    t0 = time.perf_counter()
    for li in range(n_layers):
        L = probe if li == 0 else new_layer()
        c = L.new_cache(w.B, T_max)
        for b in range(w.B):
            n = int(lens_pre[b])
            view = c.seq(b)
            for s0 in range(0, n, 4096):
                s1 = min(n, s0 + 4096)
                if li == 0 and b == 0:
                    X = (to_dev_bf16(X0[s0:s1], dev) if w.dtype == "bf16" else torch.from_numpy(X0[s0:s1]).to(dev))
                else:
                    X = torch.randn((s1 - s0, w.d), generator=gen, device=dev, dtype=torch.float32).to(tdt)
                L.append(view, X[None].contiguous(), [s0])
        layers.append(L)
        caches.append(c)
    torch.cuda.synchronize()
    log(f"[setup] prefill {n_layers} layers ({n_layers * int(lens_pre.sum())} tokens): {time.perf_counter() - t0:.1f} s")

    q_np = I.as_dtype(I.queries(w), w.dtype)
    X_np = I.as_dtype(I.x_new(w, n_q), w.dtype)
    q = to_dev_bf16(q_np, dev) if w.dtype == "bf16" else torch.from_numpy(q_np).to(dev)
    X_step = to_dev_bf16(X_np, dev) if w.dtype == "bf16" else torch.from_numpy(X_np).to(dev)
    # with --lens-dev the step is planned at the capacity for every sequence and the kernels take
    # the lengths from a device array
    lens_plan = np.full(w.B, T_max, np.int32) if args.lens_dev else lens
    lens_dev = torch.from_numpy(lens).to(dev) if args.lens_dev else None
    ws_bytes = max(L.workspace_bytes(w.B, n_q, lens_plan) for L in layers)
    ws = torch.empty((ws_bytes,), dtype=torch.uint8, device=dev)
    outs = [torch.empty_like(q) for _ in range(n_layers)]

    def step(i):
        li = i % n_layers
        layers[li].step(caches[li], X_step, q, lens_plan, out=outs[li], ws=ws, lens_dev=lens_dev)

    if args.hidden_query:
        # each layer absorbs its own synthetic W_q [d, H_q d_h]; the step appends, then attends
        # with the queries formed from hidden states inside the query projection
        for L in layers:
            Wq = (torch.randn((w.d, w.H_q * w.d_h), generator=gen, device=dev, dtype=torch.float32)
                  / math.sqrt(w.d)).to(tdt)
            L.absorb_query(Wq)
            del Wq
        xq_np = I.as_dtype(I.query_hidden(w), w.dtype)
        x_q = to_dev_bf16(xq_np, dev) if w.dtype == "bf16" else torch.from_numpy(xq_np).to(dev)

        def step(i):  # noqa: F811
            li = i % n_layers
            layers[li].append(caches[li], X_step, lens_pre)
            layers[li].decode_hidden(caches[li], x_q, lens, out=outs[li], ws=ws)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    # eager: one host call per step (append + attention), issued in segments of EAGER_SEG steps
    # with a synchronisation between segments, so that the host issue time is the calls' own cost
    # (when the GPU is the slower side, a long run fills the HIP queue and further launches wait
    # for free slots).  Python's cyclic collector is paused while timing: a full collection over
    # this process's objects landing inside the loop showed up as 0.2-0.4 ms/step of host issue.
    gc.collect()
    gc.disable()
    t_host, ms_eager = 0.0, 0.0
    for i0 in range(0, steps, EAGER_SEG):
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        ev0.record()
        for i in range(i0, min(steps, i0 + EAGER_SEG)):
            step(warmup + i)
        ev1.record()
        t_host += time.perf_counter() - t0
        torch.cuda.synchronize()
        ms_eager += ev0.elapsed_time(ev1)
    gc.enable()
    ms_step_eager = ms_eager / steps
    host_us = t_host / steps * 1e6
    log(f"[time] eager: {ms_step_eager * 1000:.2f} us/step (host issue {host_us:.1f} us/step)")

    # graph: exactly `steps` steps (rotating over the layers) captured once and replayed once
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        for li in range(n_layers):
            step(li)
        side.synchronize()
        with torch.cuda.graph(graph, stream=side):
            for i in range(steps):
                step(i)
    torch.cuda.synchronize()
    graph.replay()  # untimed: the first replay uploads the graph
    torch.cuda.synchronize()
    ev0.record()
    graph.replay()
    ev1.record()
    torch.cuda.synchronize()
    ms_total = ev0.elapsed_time(ev1)
    ms_step = ms_total / steps
    log(f"[time] graph: {steps} steps: {ms_total:.3f} ms, {ms_step * 1000:.2f} us/step")
    del graph

    # second pass with per-kernel events (same steps, same stream)
    S.profile_enable(True)
    S.profile_read(reset=True)
    for i in range(steps):
        step(warmup + steps + i)
    torch.cuda.synchronize()
    prof = S.profile_read(reset=True)
    S.profile_enable(False)
    kern_us = {k: 1000.0 * ms / n for k, (n, ms) in prof.items()}
    for k, us in sorted(kern_us.items()):
        log(f"[kernel] {k:14s} {us:9.2f} us/launch ({prof[k][0]} launches)")

    ab = algorithmic_bytes(w, probe.ranks, probe.r_v, lens, n_q, hidden=args.hidden_query)
    recon = bool(args.rope) and not any(k.startswith("decode_") for k in kern_us)
    if recon:
        # rotary layers past 32 query rows per KV head: reconstructed keys and values; the
        # dominant kernel against the MFMA peak (up to 32 rows, the latent-space decode rebuilds
        # key tiles in its score kernel, which reads the same latent as the plain one: HBM roofline)
        fl = prefill_flops(w, probe.ranks, probe.r_v, lens, n_q, "prefill_recon_v" in kern_us)
        dom = max((k for k in kern_us if k in fl), key=lambda k: kern_us[k])
        ab.update(fl)
        achieved = fl[dom] / (kern_us[dom] * 1e-6) / 1e12
        traffic = None
    else:
        dom = max((k for k in kern_us if k.startswith("decode_")), key=lambda k: kern_us[k])
        # counters cover the q path of unrotated layers only
        traffic = None if args.hidden_query or args.rope or args.lens_dev else traffic_for(dom, w.name)
        fls = algorithmic_flops(w, probe.ranks, probe.r_v, lens, n_q)
    dec_us = sum(us for k, us in kern_us.items() if k.startswith("decode_"))
    res = {
        "value": w.B * n_q / (ms_step * 1e-3),
        "ms_per_step": ms_step,
        "config": {"workload": w.name, "batch": w.B, "context": int(lens.max()) if not w.ragged else "ragged",
                   "context_tokens": int(lens.sum()), "queries_per_seq": n_q, "H_q": w.H_q, "H_kv": w.H_kv,
                   "d_h": w.d_h, "hidden": w.d, "key_rank_sum": int(np.sum(probe.ranks)), "value_rank": probe.r_v,
                   "latent": w.latent, "layers_rotated": n_layers,
                   "query": "hidden states, absorbed W_q B_g^T" if args.hidden_query else "q",
                   "rope_theta": args.rope or None,
                   "lens_dev_capacity": T_max if args.lens_dev else None},
        "dtype": {"f32": "f32", "bf16": "bf16", "mix84": "int8/int4 codes, f16 MFMA, fp32 accumulate",
                  "had43": "4-bit/3-bit codes in int8/int4 bytes, f16 MFMA, fp32 accumulate",
                  "had43p": "4-bit/3-bit codes packed (3.2 bits), f16 MFMA, fp32 accumulate"}[w.latent],
        "roofline": ({"bound": "mfma", "kernel": dom, "achieved": achieved, "peak": 2500.0, "unit": "TFLOP/s",
                      "frac": achieved / 2500.0, "traffic": None, "alg_flops_per_launch": ab[dom],
                      "us_per_launch": kern_us[dom]} if recon else
                     roofline_of(dom, kern_us[dom], ab[dom], fls.get(dom), traffic)),
        "ms_per_step_eager": ms_step_eager,
        "host_issue_us_per_step": host_us,
        "step_hbm_gbps": ab["step"] / (ms_step * 1e-3) / 1e9,
        "step_frac": ab["step"] / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "decode_kernels_us": dec_us,
        "decode_hbm_gbps": ab["decode"] / (dec_us * 1e-6) / 1e9 if dec_us > 0 else None,
        "kv_tokens_per_s": float(lens.sum()) / (ms_step * 1e-3),
        "kernel_us": kern_us,
        "alg_bytes": ab,
    }
    if with_cpu and not args.hidden_query:
        t0 = time.perf_counter()
        res["cpu_baseline"] = cpu_baseline(w, lf, lens, n_q, X0, Xcal, q_np, X_np, args.cpu_budget)
        log(f"[cpu] {time.perf_counter() - t0:.1f} s")
    else:
        res["cpu_baseline"] = None
    del layers, caches, outs, ws, U, probe
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def prefill_flops(w, ranks, r_v, lens, n_q, split_values: bool):
    """Algorithmic flops of attention over reconstructed keys and values: rebuilding K^ (each
    head's r_g channels) and V^ (r_v channels per KV head) for every cached token, then causal
    attention of the chunk (query j of n_q sees lens - n_q + j + 1 tokens; QK^T and PV).  With
    split_values the values' rebuild is its own kernel (prefill_recon_v)."""
    rk = sum(2.0 * int(T) * w.d_h * float(np.sum(ranks)) for T in lens)
    rv = sum(2.0 * int(T) * w.d_h * w.H_kv * r_v for T in lens)
    attend = 0.0
    for T in lens:
        seen = float(n_q * (int(T) - n_q) + n_q * (n_q + 1) / 2)
        attend += 4.0 * w.H_q * w.d_h * seen
    if split_values:
        return {"prefill_recon": rk, "prefill_recon_v": rv, "prefill_attend": attend}
    return {"prefill_recon": rk + rv, "prefill_attend": attend}


def measure_prefill(w, args, dev, n_q: int, steps: int, warmup: int) -> dict:
    """A query chunk of n_q per sequence (the workload's batch and context) attending over keys and
    values reconstructed from its latent cache: starkv_prefill_attention, timed like the decode
    step (graph of `steps` calls), with the MFMA roofline of the dominant kernel."""
    import torch
    import rank_kv_cache_starkv_amd as S
    from rank_kv_cache_starkv_amd import inputs as I

    lens = I.context_lengths(w) + w.n_append
    if not w.ragged:
        lens = np.full(w.B, w.T, np.int32)
    lens = lens.astype(np.int32)
    T_max = int(-(-int(lens.max()) // 32) * 32)
    tdt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    lf = I.layer_factors(w, 0)
    U = [torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev) for a in (lf.U_k, lf.V_k, lf.U_v, lf.V_v)]
    L = S.Layer(w.H_q, w.H_kv, w.d_h, w.d, w.dtype, w.latent, lf.s_k, lf.tau_k, lf.s_v, lf.tau_v)
    L.build_factors(*U)
    if w.latent in QUANTIZED:
        L.calibrate(to_dev_bf16(I.as_dtype(I.x_calibration(w), w.dtype), dev))
    if args.rope:
        L.set_rope(args.rope)
    gen = torch.Generator(device=dev)
    gen.manual_seed(2606_08382)
    c = L.new_cache(w.B, T_max)
    for b in range(w.B):
        for s0 in range(0, int(lens[b]), 4096):
            s1 = min(int(lens[b]), s0 + 4096)
            X = torch.randn((s1 - s0, w.d), generator=gen, device=dev, dtype=torch.float32).to(tdt)
            L.append(c.seq(b), X[None].contiguous(), [s0])
    wq = dataclasses.replace(w, n_q=n_q)
    q = to_dev_bf16(I.as_dtype(I.queries(wq), w.dtype), dev)
    ws = torch.empty((L.prefill_workspace_bytes(w.B, n_q, lens),), dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    log(f"[prefill] {w.name}: B={w.B} n_q={n_q} lens {int(lens.min())}..{int(lens.max())}, "
        f"workspace {ws.numel() / 2**20:.0f} MiB")
    for _ in range(warmup):
        L.prefill(c, q, lens, out=out, ws=ws)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        L.prefill(c, q, lens, out=out, ws=ws)
        side.synchronize()
        with torch.cuda.graph(graph, stream=side):
            for _ in range(steps):
                L.prefill(c, q, lens, out=out, ws=ws)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    graph.replay()
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps
    log(f"[time] graph: {steps} calls, {ms * 1000:.1f} us/call")
    S.profile_enable(True)
    S.profile_read(reset=True)
    for _ in range(steps):
        L.prefill(c, q, lens, out=out, ws=ws)
    torch.cuda.synchronize()
    prof = S.profile_read(reset=True)
    S.profile_enable(False)
    kern_us = {k: 1000.0 * t / n for k, (n, t) in prof.items()}
    for k, us in sorted(kern_us.items()):
        log(f"[kernel] {k:14s} {us:9.2f} us/launch ({prof[k][0]} launches)")
    fl = prefill_flops(w, L.ranks, L.r_v, lens, n_q, "prefill_recon_v" in kern_us)
    dom = max((k for k in kern_us if k in fl), key=lambda k: kern_us[k])
    tflops = fl[dom] / (kern_us[dom] * 1e-6) / 1e12
    return {
        "metric": "attention over reconstructed keys and values: queries/s (query chunk per sequence)",
        "value": w.B * n_q / (ms * 1e-3), "unit": "queries/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16 MFMA (reconstructed K, V, P), bf16 reconstruction, fp32 accumulate", "data": "synthetic",
        "config": {"workload": f"{w.name}-chunk{n_q}" + (f"-rope{args.rope:g}" if args.rope else ""), "batch": w.B,
                   "context_tokens": int(lens.sum()), "queries_per_seq": n_q, "latent": w.latent},
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": tflops, "peak": 2500.0, "unit": "TFLOP/s",
                     "frac": tflops / 2500.0, "traffic": None, "alg_flops_per_launch": fl[dom],
                     "us_per_launch": kern_us[dom]},
        "kernel_us": kern_us, "tokens_per_s_reconstructed": float(lens.sum()) / (ms * 1e-3),
    }


def measure_append(w, args, dev, n_new: int, steps: int, warmup: int) -> dict:
    """starkv_compress_append of n_new tokens per sequence (B x n_new rows of hidden states
    projected, quantised and packed into the cache), over enough rotated layers that the factors
    come from HBM; graph of `steps` calls, with the append kernel's MFMA and HBM rates."""
    import torch
    import rank_kv_cache_starkv_amd as S
    from rank_kv_cache_starkv_amd import inputs as I

    tdt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    lf = I.layer_factors(w, 0)
    U = [torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev) for a in (lf.U_k, lf.V_k, lf.U_v, lf.V_v)]
    Xcal = I.as_dtype(I.x_calibration(w), w.dtype) if w.latent in QUANTIZED else None
    T_max = -(-n_new // 32) * 32
    lens_pre = np.zeros(w.B, np.int32)  # every call writes positions [0, n_new) again

    def new_layer():
        L = S.Layer(w.H_q, w.H_kv, w.d_h, w.d, w.dtype, w.latent, lf.s_k, lf.tau_k, lf.s_v, lf.tau_v)
        L.build_factors(*U)
        if Xcal is not None:
            L.calibrate(to_dev_bf16(Xcal, dev) if w.dtype == "bf16" else torch.from_numpy(Xcal).to(dev))
        return L

    probe = new_layer()
    kb, vb = probe.cache_bytes(w.B, T_max)
    inf = probe.info
    per_layer = kb + vb + inf["a_bytes"]
    n_layers = args.layers or max(2, math.ceil(MIN_ROTATION_BYTES / per_layer))
    layers = [probe] + [new_layer() for _ in range(n_layers - 1)]
    caches = [L.new_cache(w.B, T_max) for L in layers]
    gen = torch.Generator(device=dev)
    gen.manual_seed(2606_08382)
    X = torch.randn((w.B, n_new, w.d), generator=gen, device=dev, dtype=torch.float32).to(tdt)
    log(f"[append] {w.name}: B={w.B} n_new={n_new} ({w.B * n_new} rows), {n_layers} layers x "
        f"{per_layer / 2**20:.0f} MiB")
    for i in range(warmup):
        layers[i % n_layers].append(caches[i % n_layers], X, lens_pre)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        layers[0].append(caches[0], X, lens_pre)
        side.synchronize()
        with torch.cuda.graph(graph, stream=side):
            for i in range(steps):
                layers[i % n_layers].append(caches[i % n_layers], X, lens_pre)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    graph.replay()
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps
    log(f"[time] graph: {steps} calls, {ms * 1000:.2f} us/call")
    S.profile_enable(True)
    S.profile_read(reset=True)
    for i in range(steps):
        layers[i % n_layers].append(caches[i % n_layers], X, lens_pre)
    torch.cuda.synchronize()
    prof = S.profile_read(reset=True)
    S.profile_enable(False)
    kern_us = {k: 1000.0 * t / n for k, (n, t) in prof.items()}
    for k, us in sorted(kern_us.items()):
        log(f"[kernel] {k:14s} {us:9.2f} us/launch ({prof[k][0]} launches)")
    M = w.B * n_new
    n_lat = int(np.sum(probe.ranks)) + int(probe.r_v)
    flops = 2.0 * M * w.d * n_lat
    elem = 4 if w.dtype == "f32" else 2
    byts = float(inf["a_bytes"]) + M * w.d * elem + M * (inf["k_row_bytes"] + inf["v_tile_rows"] * elem_of(w.latent))
    us = kern_us["append"]
    tf = flops / (us * 1e-6) / 1e12
    gbps = byts / (us * 1e-6) / 1e9
    log(f"[append] {flops / 1e9:.2f} GFLOP, {byts / 1e6:.1f} MB per call: {tf:.1f} TFLOP/s "
        f"({tf / 2500.0:.3f} of MFMA peak), {gbps:.0f} GB/s ({gbps / 8000.0:.3f} of HBM peak)")
    return {
        "metric": "compress_append: tokens/s projected, quantised and packed into the latent cache",
        "value": M / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": f"{w.dtype} MFMA, fp32 accumulate, {w.latent} store", "data": "synthetic",
        "config": {"workload": f"{w.name}-append{n_new}", "batch": w.B, "new_tokens_per_seq": n_new,
                   "rows": M, "hidden": w.d, "latent_channels": n_lat, "latent": w.latent},
        "roofline": {"bound": "mfma", "kernel": "append", "achieved": tf, "peak": 2500.0, "unit": "TFLOP/s",
                     "frac": tf / 2500.0, "traffic": None, "alg_flops_per_launch": flops, "us_per_launch": us},
        "hbm": {"achieved": gbps, "peak": 8000.0, "unit": "GB/s", "frac": gbps / 8000.0, "alg_bytes_per_launch": byts},
        "kernel_us": kern_us,
    }


def elem_of(latent: str) -> float:
    """Bytes per value-tile row element of one token (value tile rows hold one byte, or one
    bf16/fp32 element, per token)."""
    return {"f32": 4, "bf16": 2}.get(latent, 1)


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=4,
                    help="workload id (0-6); 4 (the 13B-class ragged high-batch step) is the headline")
    ap.add_argument("--layers", type=int, default=0, help="layers to rotate (0: enough for 1 GiB)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-sub", action="store_true", help="skip the other workloads' sub-results")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--hidden-query", action="store_true",
                    help="queries from hidden states through the absorbed factors W_q B_g^T (step = append, "
                         "then starkv_decode_attention_hidden); no CPU baseline")
    ap.add_argument("--prefill", type=int, default=0, metavar="N",
                    help="time a chunk of N queries per sequence attending over reconstructed keys and values "
                         "(starkv_prefill_attention) instead of the decode step")
    ap.add_argument("--append", type=int, default=0, metavar="N",
                    help="time starkv_compress_append of N tokens per sequence (the append GEMM's MFMA and "
                         "HBM rates) instead of the decode step")
    ap.add_argument("--rope", type=float, default=0.0, metavar="THETA",
                    help="rotary layers (base THETA): decode and prefill attend over reconstructed keys")
    ap.add_argument("--lens-dev", type=int, default=0, metavar="CAP",
                    help="plan the step at a capacity of CAP tokens per sequence and pass the lengths on "
                         "the device (starkv_decode_step's lens_dev)")
    ap.add_argument("--copy-probe", action="store_true", help=f"copy {COPY_PROBE_MIB} MiB device to device")
    ap.add_argument("--pmc-summary", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"))
    args = ap.parse_args()
    if args.pmc_summary:
        from rank_kv_cache_starkv_amd import inputs as I
        return pmc_summary(*args.pmc_summary, I.WORKLOADS[args.workload].name)
    if args.copy_probe:
        return copy_probe()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the library runs on a single "
              f"MI355X; sharding across GPUs by sequence, KV head or context is not built)", file=sys.stderr)
        return 2

    import torch
    from rank_kv_cache_starkv_amd import inputs as I

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda:0"
    torch.cuda.set_device(0)
    w = I.WORKLOADS[args.workload]
    if args.prefill:
        print(json.dumps(measure_prefill(w, args, dev, args.prefill, args.steps, args.warmup)))
        return 0
    if args.append:
        print(json.dumps(measure_append(w, args, dev, args.append, args.steps, args.warmup)))
        return 0
    r = measure(w, args, dev, with_cpu=not args.no_cpu and not args.rope, steps=args.steps, warmup=args.warmup)
    result = {
        "metric": METRIC,
        "value": r["value"],
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": r["dtype"],
        "data": "synthetic",
        "config": r["config"],
        "roofline": r["roofline"],
        "cpu_baseline": r["cpu_baseline"],
        "timing": "HIP graph of exactly `steps` steps (rotating over the layers), replayed once; events on the "
                  "replay stream",
    }
    result.update({k: r[k] for k in ("ms_per_step_eager", "host_issue_us_per_step", "step_hbm_gbps", "step_frac",
                                     "decode_kernels_us", "decode_hbm_gbps", "kv_tokens_per_s", "kernel_us",
                                     "alg_bytes")})
    if not args.no_sub and args.workload == 4 and not args.hidden_query and not args.rope:
        # the other workloads of the same metric, measured in the same run (no CPU baseline)
        subs = {}
        for wid in (1, 2, 3):
            ws = I.WORKLOADS[wid]
            sr = measure(ws, args, dev, with_cpu=False, steps=min(args.steps, 100), warmup=min(args.warmup, 10))
            subs[ws.name] = {"queries_per_s": sr["value"], "ms_per_step": sr["ms_per_step"],
                             "ms_per_step_eager": sr["ms_per_step_eager"],
                             "host_issue_us_per_step": sr["host_issue_us_per_step"],
                             "kv_tokens_per_s": sr["kv_tokens_per_s"], "step_frac": sr["step_frac"],
                             "roofline": {k: sr["roofline"][k] for k in ("bound", "kernel", "achieved", "unit", "frac",
                                                                          "traffic", "us_per_launch", "hbm", "mfma")
                                          if k in sr["roofline"]},
                             "kernel_us": sr["kernel_us"], "config": sr["config"]}
        result["sub_results"] = subs
    print(json.dumps(result))
    return 0


if __name__ == "__main__":
    sys.exit(main())
