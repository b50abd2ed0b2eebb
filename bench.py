"""Decode-step benchmark on one MI355X.

Default workload: the 135M-shaped Llama (dim 576, 9/3 heads, head_dim 64, 30
layers, SwiGLU 1536, vocab 49152, tied, bf16 weights), batch 1, 5-token
prompt, greedy decode at positions 5..11 (the five-prompt / eight-new-token
generation), cycled: after every 7 steps the cache length is rewound to 5, so
every timed step is one of those 7 positions.  Steps are chained on the GPU
(the token written by step k is the token read by step k+1).

Prints one JSON line with decode tok/s, the whole step's algorithmic HBM
bytes and GB/s, a roofline entry for the dominant kernel (timed with events
on the stream the library launches it on), and the reference decoder's
throughput on the host as the CPU baseline.  At batch 1 the whole step is one
persistent kernel; its roofline entry divides the step's algorithmic bytes by
that kernel's mean launch duration.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

HBM_PEAK_GBPS = 8000.0
KERNELS = ["qkv", "attn", "attn_combine", "wo", "w13", "w2", "logits"]


DTYPE = {
    "bf16": "f32 (fp32 accumulation; bf16 weights times fp32 activations as bf16 hi+lo pairs)",
    "q8": "f32 (fp32 accumulation; int8 weights with an fp32 scale per 32 values, times fp32 activations)",
    "q4": "f32 (fp32 accumulation; int4 weights with an fp32 scale per 32 values, times fp32 activations)",
}


def step_bytes(m: synth.ModelShape, lengths_before: np.ndarray) -> int:
    """Algorithmic HBM bytes of one decode step: every weight matrix once (the
    tied embedding once, as the vocabulary product; an untied embedding only
    through the gathered rows, the separate head as the vocabulary product),
    the embedding rows gathered, the norm gains, the K/V rows read (positions
    0..n_b) and written, and the fp32 logits written."""
    table, _ = synth.tensor_table(m)
    B = len(lengths_before)
    mats = sum(synth.tensor_bytes(s, dt) for name, _, s, dt in table
               if len(s) == 2 and (m.tied_embeddings or name != "token_emb"))
    gains = sum(int(np.prod(s)) * 4 for _, _, s, dt in table if len(s) == 1)
    kv_row = m.n_layers * 2 * m.n_kv_heads * m.head_dim * (2 if m.cache_dtype == synth.BF16 else 4)
    gather = int(B * m.dim * elem_bytes(m))
    kv_read = int(np.sum(lengths_before.astype(np.int64) + 1)) * kv_row
    kv_write = B * kv_row
    logits = B * m.vocab_size * 4
    return mats + gains + gather + kv_read + kv_write + logits


def elem_bytes(m: synth.ModelShape) -> float:
    """Bytes per matrix element, a Q8 element's share of its block scale included."""
    if m.weight_dtype in (synth.Q8, synth.Q4):
        return m.wbytes + 4.0 / synth.Q8_BLOCK
    return float(m.wbytes)


def kernel_bytes(m: synth.ModelShape, which: str, B: int, n_ctx: float) -> float:
    """Algorithmic bytes of one launch of a step kernel (weights + activations
    in and out), n_ctx = mean cached positions read by attention."""
    d, F, V, D = m.dim, m.hidden_dim, m.vocab_size, m.head_dim
    w = elem_bytes(m)
    qr, kvr = m.n_heads * D, m.n_kv_heads * D
    if which == "qkv":
        return (qr + 2 * kvr) * d * w + B * (d * 4 + d * 4 + (qr + 2 * kvr) * 4)
    if which == "attn":
        return B * (2 * kvr * n_ctx * (2 if m.cache_dtype == synth.BF16 else 4) + qr * 4)
    if which == "wo":
        return d * qr * w + B * (qr * 4 + 2 * d * 4)
    if which == "w13":
        return 2 * F * d * w + B * (d * 4 + d * 4 + F * 4)
    if which == "w2":
        return d * F * w + B * (F * 4 + 2 * d * 4)
    if which == "logits":
        return V * d * w + B * (d * 4 + d * 4 + V * 4)
    return 0.0


# the sources each counted kernel is built from
KERNEL_SOURCES = {"k_persist": ("persist.hip", "device.h", "kernels.h"),
                  "k_attn_g": ("kernels.hip", "device.h", "kernels.h")}


def kernel_sources_hash(kernel: str = "k_persist") -> str:
    """First 16 hex digits of the sha256 of the kernel's sources."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "decode_step_02_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kernel: str = "k_persist"):
    """HBM bytes per launch of `kernel` (the single-launch step, or the split-K
    attention) from the committed FETCH_SIZE / WRITE_SIZE summary, if it was
    taken on the current sources."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.md")
    if not os.path.exists(path):
        return None, "no counter summary for this workload"
    fields = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and line.split(":")[0] in ("traffic_bytes_per_launch", "kernel_sources_sha256_16"):
                k, v = line.split(":", 1)
                fields[k] = v.strip()
    if fields.get("kernel_sources_sha256_16") != kernel_sources_hash(kernel):
        return None, "kernel changed since the counters were taken"
    return float(fields["traffic_bytes_per_launch"]), "FETCH_SIZE + WRITE_SIZE, copy-calibrated (" + os.path.relpath(path, ROOT) + ")"


def cpu_baseline(w: synth.Workload, arena: np.ndarray, budget_s: float) -> dict:
    """The reference decoder (single thread) on the host: prefill the prompt,
    then decode steps at positions prompt_len .. prompt_len+decode_calls-1,
    cycled, until `budget_s` seconds of decode work are done."""
    import oracle
    m = oracle.Model(w.model, arena, 1, w.ctx)
    prompt = synth.prompts(w)[0]
    for t, tk in enumerate(prompt):
        tok, _ = m.forward(0, t, int(tk))
    steps, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        pos = len(prompt) + steps % w.decode_calls
        tok, _ = m.forward(0, pos, tok)
        steps += 1
    dt = time.perf_counter() - t0
    return {"value": steps / dt, "unit": "tok/s", "cores": 1, "kind": "oracle",
            "sample": f"{steps} decode steps of {w.name} (positions {len(prompt)}.."
                      f"{len(prompt) + w.decode_calls - 1}, cycled) on one host thread, {dt:.1f} s",
            "host": host_cpu()}


def host_cpu() -> dict:
    """The host the CPU baseline ran on: CPU model, logical CPUs, and the CPUs
    this process may use."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {"cpu_model": model, "nproc": os.cpu_count(), "usable_cpus": usable}


def prefill_bench(dsa, torch, model, w, prompt, stream, reps, per_position=True):
    """Prompt prefill of one sequence into an empty batch-1 cache: the batched
    prefill (median of `reps` runs after one warm-up) and the one-position-
    per-pass prefill (one run after one warm-up), both timed with events on
    `stream` around the call."""
    toks = [int(t) for t in prompt]
    n = len(toks)
    kv = dsa.KVCache(model, 1, w.ctx)
    out = torch.zeros(1, dtype=torch.int32, device="cuda")

    def timed(fn):
        kv.reset(0, stream)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn(0, toks, out, stream)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b)

    timed(kv.prefill_batched)
    ms_b = sorted(timed(kv.prefill_batched) for _ in range(reps))[reps // 2]
    tok_b = int(out.item())
    ms_p, tok_p = float("nan"), tok_b
    if per_position:
        timed(kv.prefill)
        ms_p = timed(kv.prefill)
        tok_p = int(out.item())
    kv.check(stream)
    kv.close()
    return {"metric": f"prefill tok/s ({w.name}, prompt of {n})", "value": n / (ms_b * 1e-3), "unit": "tok/s",
            "n_gpus": 1, "higher_is_better": True, "ms_per_prefill": ms_b, "reps": reps,
            "per_position": {"value": n / (ms_p * 1e-3), "ms_per_prefill": ms_p},
            "speedup": ms_p / ms_b, "same_first_token": tok_b == tok_p,
            "dtype": "f32 (fp32 accumulation; bf16 weights times fp32 activations as bf16 hi+lo pairs)",
            "data": "synthetic (seeded random weights N(0,0.02), uniform prompt ids)",
            "config": {"workload": w.name, "prompt_len": n, "ctx": w.ctx, "batch": 1}}


def replicate_bench(dsa, torch, model, w, prompt, stream, n_rows, reps=10):
    """Copy one prefilled sequence into n_rows sequences of a decode cache:
    the rows [0, len) of every layer's keys and values, per destination."""
    toks = [int(t) for t in prompt]
    src = dsa.KVCache(model, 1, w.ctx)
    out = torch.zeros(1, dtype=torch.int32, device="cuda")
    src.prefill_batched(0, toks, out, stream)
    dst = dsa.KVCache(model, n_rows, w.ctx)
    dst.replicate_from(src, 0, 0, n_rows, stream)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        dst.replicate_from(src, 0, 0, n_rows, stream)
    b.record(stream)
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1000.0 / reps
    m = w.model
    per_row = len(toks) * m.n_layers * 2 * m.n_kv_heads * m.head_dim * 4  # bytes written per row (and read once)
    dst.check(stream)
    src.close()
    dst.close()
    return {"metric": f"cache replication ({w.name}, {len(toks)} positions into {n_rows} rows)",
            "value": us, "unit": "us per call", "higher_is_better": False,
            "bytes_written": per_row * n_rows,
            "algorithmic_GBps": (per_row * n_rows + per_row) / (us * 1e-6) / 1e9,
            "n_gpus": 1, "config": {"workload": w.name, "prompt_len": len(toks), "rows": n_rows, "ctx": w.ctx}}


MFMA_KINDS = {"qkv", "wo", "w13", "w2"}  # the projections that take the MFMA path at B >= 16
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16


def kernel_flops(m: synth.ModelShape, which: str, B: int) -> float:
    """Useful flops of one launch of a projection: 2 per weight per item."""
    d, F, D = m.dim, m.hidden_dim, m.head_dim
    qr, kvr = m.n_heads * D, m.n_kv_heads * D
    rows_cols = {"qkv": (qr + 2 * kvr) * d, "wo": d * qr, "w13": 2 * F * d, "w2": d * F}
    return 2.0 * B * rows_cols.get(which, 0)


def flush_and_copy_peak(torch, stream, mib: int):
    """Two device buffers of `mib` MiB each (the halves of one): copying one
    into the other reads and writes 2 x mib MiB, more than the 256 MB Infinity
    Cache and the L2s hold, so it evicts whatever a step left there.  Returns
    (half a, half b, the whole) and the copy's rate (bytes read + written per
    second, median of 5), a measured streaming peak the fractions are also
    reported against."""
    n = mib * (1 << 20) // 4
    whole = torch.ones(2 * n, dtype=torch.float32, device="cuda")  # the read probe streams all of it
    a, b = whole[:n], whole[n:]
    with torch.cuda.stream(stream):
        b.copy_(a)
        torch.cuda.synchronize()
        ts = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            b.copy_(a)
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
    t = sorted(ts)[2]
    return (a, b, whole), {"bytes_read": 4 * n, "bytes_written": 4 * n, "us_per_copy": t * 1e6,
                           "GBps": 8 * n / t / 1e9}


def read_peak(dsa, torch, stream, buf, reps=5) -> dict:
    """The library's plain streaming read (ds_bench_stream) over `buf`, median
    of `reps` launches: the read bandwidth a kernel doing nothing else gets."""
    out = torch.zeros(4096, dtype=torch.int32, device="cuda")
    with torch.cuda.stream(stream):
        dsa.ds_bench_stream(buf, out, 1, stream)
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            dsa.ds_bench_stream(buf, out, 1, stream)
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
    t = sorted(ts)[reps // 2]
    nbytes = buf.numel() * buf.element_size()
    return {"bytes_read": nbytes, "us_per_read": t * 1e6, "GBps": nbytes / t / 1e9}


def decode_bench(dsa, torch, w, args, stream, steps, warmup, samp=None, flush=None, copy_peak=None,
                 rpeak=None) -> dict:
    """Decode steps of workload `w`: prompts prefilled (untimed), then `steps`
    chained steps after `warmup`, cycled over the workload's positions
    (lengths rewound every decode_calls steps).  Returns the result record
    (without the CPU baseline)."""
    m = w.model
    arena = synth.make_arena(m, w.model_seed)
    prompts = synth.prompts(w)
    B = w.batch
    with torch.cuda.stream(stream):
        model = dsa.Model(m, arena)
        kv = dsa.KVCache(model, B, w.ctx)
        kv.set_dispatch(1 if args.dispatch == "graph" else 0)
        tok = torch.zeros(B, dtype=torch.int32, device="cuda")
        for b, p in enumerate(prompts):  # setup, untimed: every prompt's positions as one batch
            kv.prefill_batched(b, [int(t) for t in p], tok)
        base = np.array([len(p) for p in prompts], np.int32)
        cycle = w.decode_calls
        ubuf = None
        if samp:
            ubuf = torch.from_numpy(np.random.default_rng(5).random((64, B)).astype(np.float32)).cuda()

        def run(n, start):
            for i in range(start, start + n):
                if i % cycle == 0 and i > 0:
                    kv.set_lengths(base)
                kv.decode_step(tok, tok)
                if samp:
                    kv.sample(ubuf[i % 64], *samp, tok, stream)

        run(warmup, 0)
        kv.set_lengths(base)
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        run(steps, 0)
        ev1.record(stream)
        torch.cuda.synchronize()
        ms_total = ev0.elapsed_time(ev1)
        kv.check()
        ms_step = ms_total / steps

        sampler_us = None
        if samp:  # the sampling kernel alone, on the last step's logits
            s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s0.record(stream)
            for i in range(100):
                kv.sample(ubuf[i % 64], *samp, tok, stream)
            s1.record(stream)
            torch.cuda.synchronize()
            sampler_us = s0.elapsed_time(s1) * 10.0

        lengths_seq = [base + (i % cycle) for i in range(cycle)]
        bytes_step = float(np.mean([step_bytes(m, L) for L in lengths_seq]))

        def timed_steps(n, before=None):
            """Each step bracketed by its own events on the library's stream
            (`before` runs ahead of every step, outside the events)."""
            kv.set_lengths(base)
            run(cycle, 0)
            kv.set_lengths(base)
            torch.cuda.synchronize()
            pairs = []
            for i in range(n):
                if i % cycle == 0 and i > 0:
                    kv.set_lengths(base)
                if before:
                    before()
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                kv.decode_step(tok, tok)
                b.record(stream)
                pairs.append((a, b))
            torch.cuda.synchronize()
            kv.check()
            return [1000.0 * a.elapsed_time(b) for a, b in pairs]

        single = B == 1 and kv.single_launch_ctx() >= int(base.max()) + cycle
        kern = {}
        floor_us = None
        if single:
            # The whole step is one persistent kernel.  Time each launch with
            # events around it on the library's stream (eager dispatch, so the
            # events bracket the kernel itself), over the same step sequence.
            kv.set_dispatch(0)
            per = timed_steps(steps)
            us = float(np.mean(per))
            dom = "k_persist (whole step)"
            dk = {"us_per_launch": us, "launches_per_step": 1, "us_per_step": us, "bytes_per_launch": bytes_step}
            kern[dom] = dk
            # the handoff floor: the same launch, phases and handoff words
            # with no weight or cache traffic, at the same position
            kv.bench_kernel(7, 0, 3, stream)
            f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            f0.record(stream)
            kv.bench_kernel(7, 0, args.kernel_reps, stream)
            f1.record(stream)
            torch.cuda.synchronize()
            kv.check()
            floor_us = f0.elapsed_time(f1) * 1000.0 / args.kernel_reps
        else:
            # one launch per operation: each kernel timed alone on the library's
            # stream, consecutive launches cycling through the layers
            mean_ctx = float(np.mean(base)) + (cycle - 1) / 2.0 + 1.0
            for k, name in enumerate(KERNELS):
                layer = m.n_layers // 2
                try:
                    kv.bench_kernel(k, layer, 5, stream)
                except dsa.DSError as e:
                    if e.status != -8:  # DS_ERR_STATE: not part of this step's kernel sequence
                        raise
                    continue
                reps = args.kernel_reps if name != "logits" else max(args.kernel_reps // 4, 5)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                kv.bench_kernel(k, layer, reps, stream)
                e1.record(stream)
                torch.cuda.synchronize()
                us = e0.elapsed_time(e1) * 1000.0 / reps
                per_step = 1 if name == "logits" else m.n_layers
                kern[name] = {"us_per_launch": us, "launches_per_step": per_step,
                              "us_per_step": us * per_step,
                              "bytes_per_launch": kernel_bytes(m, name, B, mean_ctx)}
            dom = max(kern, key=lambda n: kern[n]["us_per_step"])
            dk = kern[dom]
            per = timed_steps(steps)  # each step bracketed by events (graph dispatch)
        achieved = dk["bytes_per_launch"] / (dk["us_per_launch"] * 1e-6) / 1e9

        cold = None
        if flush is not None:
            fa, fb = flush[0], flush[1]
            us_cold = float(np.mean(timed_steps(min(steps, 4 * cycle), before=lambda: fb.copy_(fa))))
            gb_cold = bytes_step / (us_cold * 1e-6) / 1e9
            cold = {"us_per_step": us_cold, "tok_s": B * 1e6 / us_cold, "achieved_GBps": gb_cold,
                    "frac_of_hbm_peak": gb_cold / HBM_PEAK_GBPS,
                    "frac_of_copy_peak": gb_cold / copy_peak["GBps"] if copy_peak else None,
                    "frac_of_read_peak": gb_cold / rpeak["GBps"] if rpeak else None,
                    "flush": f"{2 * fa.numel() * 4 >> 20} MiB copied on the same stream before every step, outside "
                             f"the step's events (evicts the 256 MB Infinity Cache and the L2s)"}
        kv.close()
        model.close()

    gbps = bytes_step / (ms_step * 1e-3) / 1e9
    if single:
        traffic, traffic_note = measured_traffic(w.name, "k_persist")
    elif dom == "attn" and args.cache == "f32" and args.weights == "bf16":
        traffic, traffic_note = measured_traffic(w.name, "k_attn_g")
    else:
        traffic, traffic_note = None, "no counter summary for this kernel"
    out = {
        "metric": ("decode tok/s (135M-shaped Llama, B=1)" if w.name == "llama135m_p5"
                   else "decode tok/s (135M-shaped Llama, B=64)" if w.name == "llama135m_b64"
                   else f"decode tok/s ({w.name})")
                  + {"q8": " int8 weights", "q4": " int4 weights"}.get(args.weights, "")
                  + (" bf16 cache" if args.cache == "bf16" else "")
                  + (" with sampling" if samp else ""),
        "value": B * steps / (ms_total * 1e-3),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE[args.weights],
        "data": "synthetic (seeded random weights N(0,0.02), uniform prompt ids)",
        "config": {"workload": w.name, "description": w.description, "batch": B, "ctx": w.ctx,
                   "weights": args.weights, "cache": args.cache,
                   "decode_positions": [int(base.min()), int(base.max() + cycle - 1)],
                   "dispatch": "direct" if single else args.dispatch, "single_launch_step": bool(single)},
        "step_bytes": bytes_step,
        "achieved_GBps": gbps,
        "frac_of_hbm_peak": gbps / HBM_PEAK_GBPS,
        "frac_of_copy_peak": gbps / copy_peak["GBps"] if copy_peak else None,
        "frac_of_read_peak": gbps / rpeak["GBps"] if rpeak else None,
        "step_us": {"mean": float(np.mean(per)), "median": float(np.median(per)), "min": float(np.min(per)),
                    "n": len(per), "how": "events around each step on the library's stream"},
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
                     "frac_of_read_peak": achieved / rpeak["GBps"] if rpeak else None,
                     "us_per_launch": dk["us_per_launch"], "bytes_per_launch": dk["bytes_per_launch"]},
        "kernels_us_per_step": {n: round(v["us_per_step"], 2) for n, v in kern.items()},
        "traffic_note": traffic_note,
    }
    if single:
        out["roofline"]["frac_of_floor"] = floor_us / dk["us_per_launch"]
        out["floor"] = {"us_per_launch": floor_us, "frac_of_floor": floor_us / dk["us_per_launch"],
                        "what": "k_persist's handoff floor (ds_bench_kernel 7): the single launch's phases and "
                                "handoff words with no weight or cache loads, back-to-back launches at the same "
                                "position; frac_of_floor = floor / step time"}
    mm = {n: v for n, v in kern.items() if n in MFMA_KINDS and B >= 16}
    if mm:
        rows = {}
        for n, v in mm.items():
            tf = kernel_flops(m, n, B) / (v["us_per_launch"] * 1e-6) / 1e12
            rows[n] = {"us_per_launch": v["us_per_launch"], "useful_TFLOPs": tf,
                       "frac_of_bf16_peak": tf / BF16_MFMA_PEAK_TFLOPS}
        out["mfma"] = {"peak_TFLOPs": BF16_MFMA_PEAK_TFLOPS, "kernels": rows,
                       "note": "useful flops (2 per weight per item) over the launch time; the products issue "
                               "twice that, one bf16 MFMA for each of the activation's hi and lo terms"}
    if cold:
        out["cold"] = cold
    if samp:
        out["config"]["sampling"] = {"temperature": samp[0], "top_k": samp[1], "top_p": samp[2]}
        out["sampler_us_per_call"] = sampler_us
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=700)
    ap.add_argument("--warmup", type=int, default=28)
    ap.add_argument("--workload", default="llama135m_p5")
    ap.add_argument("--dispatch", choices=["graph", "eager"], default="graph")
    ap.add_argument("--kernel-reps", type=int, default=200)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-b64", action="store_true",
                    help="with the default workload: skip the nested B=64 record")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold variant (Infinity Cache flushed before every step)")
    ap.add_argument("--flush-mib", type=int, default=512,
                    help="MiB per flush buffer (two of them; a copy between them streams twice this size)")
    ap.add_argument("--prefill", action="store_true",
                    help="measure the prompt prefill of the workload's first prompt instead of decode steps: "
                         "ds_prefill_batched (positions as the items of a pass) against ds_prefill (one "
                         "position per pass); prints a prefill tok/s line")
    ap.add_argument("--prefill-reps", type=int, default=5)
    ap.add_argument("--replicate", type=int, default=0,
                    help="N: prefill the workload's first prompt once (batched) and time copying its cache rows "
                         "into N sequences of a decode cache (ds_kv_cache_replicate); prints a replication line")
    ap.add_argument("--sample", default="",
                    help="T,K,P: after every decode step draw the next tokens with ds_sample (temperature T, "
                         "top-k K, top-p P; seeded uniforms) instead of keeping the greedy ones")
    ap.add_argument("--prefill-batched-only", action="store_true",
                    help="with --prefill: skip the one-position-per-pass prefill (for kernel profiles)")
    ap.add_argument("--weights", choices=["bf16", "q8", "q4"], default="bf16",
                    help="matrix storage: the workload's bf16, or block-quantised int8 / int4 (an fp32 scale "
                         "per 32 values) from the same seeded draws")
    ap.add_argument("--cache", choices=["f32", "bf16"], default="f32",
                    help="key/value cache element type (bf16: rows rounded when stored)")
    ap.add_argument("--calibrate-copy-mb", type=int, default=0,
                    help="first run a plain copy kernel (read N MB, write N MB) three times, as the "
                         "known-size reference for hardware byte counters; its rate is reported")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    import torch
    import decode_step_02_amd as dsa

    def variant(w):
        if args.weights in ("q8", "q4"):
            qdt = synth.Q8 if args.weights == "q8" else synth.Q4
            w = dataclasses.replace(w, model=dataclasses.replace(w.model, weight_dtype=qdt))
        if args.cache == "bf16":
            w = dataclasses.replace(w, model=dataclasses.replace(w.model, cache_dtype=synth.BF16))
        return w

    w = variant(synth.WORKLOADS[args.workload])
    stream = torch.cuda.Stream()
    copy_cal = None
    if args.calibrate_copy_mb > 0:
        with torch.cuda.stream(stream):
            n = args.calibrate_copy_mb * (1 << 20) // 4
            src = torch.ones(n, dtype=torch.float32, device="cuda")
            dst = torch.empty_like(src)
            torch.mul(src, 1.0, out=dst)
            torch.cuda.synchronize()
            c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            c0.record(stream)
            for _ in range(3):
                torch.mul(src, 1.0, out=dst)
            c1.record(stream)
            torch.cuda.synchronize()
            us = c0.elapsed_time(c1) * 1000.0 / 3
            copy_cal = {"bytes_read": 4 * n, "bytes_written": 4 * n, "us_per_launch": us,
                        "GBps": 8 * n / (us * 1e-6) / 1e9}
            del src, dst
    if args.replicate > 0 or args.prefill:
        arena = synth.make_arena(w.model, w.model_seed)
        prompts = synth.prompts(w)
        with torch.cuda.stream(stream):
            model = dsa.Model(w.model, arena)
            if args.replicate > 0:
                print(json.dumps(replicate_bench(dsa, torch, model, w, prompts[0], stream, args.replicate)))
            else:
                print(json.dumps(prefill_bench(dsa, torch, model, w, prompts[0], stream, args.prefill_reps,
                                               not args.prefill_batched_only)))
        return

    samp = None
    if args.sample:
        st_, sk_, sp_ = args.sample.split(",")
        samp = (float(st_), int(sk_), float(sp_))
    flush, copy_peak = (None, None) if args.no_cold else flush_and_copy_peak(torch, stream, args.flush_mib)
    rpeak = read_peak(dsa, torch, stream, flush[2]) if flush else None
    out = decode_bench(dsa, torch, w, args, stream, args.steps, args.warmup, samp, flush, copy_peak, rpeak)
    if copy_peak:
        out["copy_peak"] = copy_peak
    if rpeak:
        out["read_peak"] = rpeak
    if (args.workload == "llama135m_p5" and not args.no_b64 and not samp):
        # BASELINE's metric names both batch sizes of the 135M shape: the
        # batch-64 ragged decode rides along as a nested record
        w64 = variant(synth.WORKLOADS["llama135m_b64"])
        out["b64"] = decode_bench(dsa, torch, w64, args, stream, max(args.steps // 16, 16), max(args.warmup, 16),
                                  None, flush, copy_peak, rpeak)
    if copy_cal:
        out["copy_calibration"] = copy_cal
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, synth.make_arena(w.model, w.model_seed), args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
