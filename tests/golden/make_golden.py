"""Writes the expected values of the large-workload GPU parity tests.

Every number stored here comes from the reference decoder (``oracle/``) run
on the seeded inputs of ``synth``; nothing comes from the HIP library.  The
full-size workloads are too slow for the single-threaded reference inside a
GPU test, so the script stores sampled outputs:

* llama135m_p1000 -- the whole run: 1000-token prompt then 23 greedy steps;
  per step the top-8 logits, 64 fixed sampled logits, max |logit| and the
  top-2 gap, plus sampled cache rows.
* llama135m_b64 -- a few sampled sequences of the 64, each run alone (rows of
  a batched decode are independent), prompt then 16 greedy steps.
* llama8b_p4096 -- (a) the full-size model on the first 5 prompt tokens with
  4 greedy steps; (b) the layer-0 key/value rows of sampled positions of the
  4096-token prompt, which depend only on that position's token.

Usage: python tests/golden/make_golden.py [workload ...]   (about 10 min)
"""
from __future__ import annotations

import hashlib
import json
import os
import sys
import time
from concurrent.futures import ProcessPoolExecutor

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402

N_SAMPLE = 64
N_TOP = 8


def fingerprint(shape, arena) -> str:
    """sha256 over the first 4 KiB of every arena tensor and the arena size."""
    h = hashlib.sha256(str(arena.nbytes).encode())
    for _, off, _, _ in synth.tensor_table(shape)[0]:
        h.update(arena[off:off + 4096].tobytes())
    return h.hexdigest()


def sample_indices(V: int, seed: int) -> list[int]:
    return sorted(np.random.default_rng(seed).choice(V, N_SAMPLE, replace=False).tolist())


def summarize(logits: np.ndarray, idx: list[int]) -> dict:
    top = np.argsort(-logits.astype(np.float64), kind="stable")[:N_TOP]
    s = np.sort(logits.astype(np.float64))
    return {
        "token": int(oracle.argmax(logits)),
        "top_idx": [int(i) for i in top],
        "top_val": [float(logits[i]) for i in top],
        "sample_val": [float(logits[i]) for i in idx],
        "max_abs": float(np.abs(logits).max()),
        "gap": float(s[-1] - s[-2]),
    }


def run_sequence(shape, arena, prompt, n_new, T, cache_probe=None):
    """Reference greedy run of one sequence: logits summary per new token and
    optional cache rows [(layer, kv, group, pos)] read at the end."""
    m = oracle.Model(shape, arena, 1, T)
    idx = sample_indices(shape.vocab_size, 7)
    steps = []
    tok = None
    for t, tk in enumerate(prompt):
        tok, lg = m.forward(0, t, int(tk))
    steps.append(summarize(lg, idx))
    pos = len(prompt)
    for _ in range(n_new - 1):
        tok, lg = m.forward(0, pos, tok)
        steps.append(summarize(lg, idx))
        pos += 1
    rows = []
    if cache_probe:
        cv = m.cache_view()
        for (l, kv, g, p) in cache_probe:
            rows.append({"layer": l, "kv": kv, "group": g, "pos": p,
                         "val": [float(v) for v in cv[l, kv, 0, g, p]]})
    return {"sample_idx": idx, "steps": steps, "cache_rows": rows}


def golden_p1000():
    w = synth.WORKLOADS["llama135m_p1000"]
    arena = synth.make_arena(w.model, w.model_seed)
    prompt = synth.prompts(w)[0]
    probe = [(l, kv, g, p) for l in (0, 14, 29) for kv in (0, 1) for g in (0, 2) for p in (0, 511, 999, 1022)]
    t0 = time.time()
    out = run_sequence(w.model, arena, prompt, w.decode_calls + 1, w.ctx, probe)
    out.update(workload=w.name, fingerprint=fingerprint(w.model, arena), seconds=time.time() - t0)
    return out


def _b64_one(b):
    w = synth.WORKLOADS["llama135m_b64"]
    arena = synth.make_arena(w.model, w.model_seed, threads=1)
    prompt = synth.prompts(w)[b]
    n = len(prompt)
    probe = [(l, kv, 1, p) for l in (0, 29) for kv in (0, 1) for p in sorted({0, n - 1, n + 15})]
    r = run_sequence(w.model, arena, prompt, w.decode_calls + 1, w.ctx, probe)
    r["seq"] = int(b)
    r["prompt_len"] = int(n)
    return r


def golden_b64():
    w = synth.WORKLOADS["llama135m_b64"]
    lens = synth.prompt_lengths(w)
    order = np.argsort(lens, kind="stable")
    picks = sorted({int(order[0]), int(order[1]), int(order[len(order) // 2]), int(order[-1])})
    arena = synth.make_arena(w.model, w.model_seed)
    t0 = time.time()
    with ProcessPoolExecutor(len(picks)) as ex:
        seqs = list(ex.map(_b64_one, picks))
    return {"workload": w.name, "fingerprint": fingerprint(w.model, arena), "lengths": lens.tolist(),
            "sequences": seqs, "seconds": time.time() - t0}


def golden_8b():
    w = synth.WORKLOADS["llama8b_p4096"]
    m = w.model
    t0 = time.time()
    arena = synth.make_arena(m, w.model_seed)
    prompt = synth.prompts(w)[0]
    short = run_sequence(m, arena, prompt[:5], 5, 16)
    # layer-0 key/value rows of sampled prompt positions: embedding row ->
    # attn_norm -> Wk / Wv -> RoPE on k (each needs only that position's token)
    v = synth.views(m, arena)
    rows = []
    for p in (0, 1, 1000, 2047, 4095):
        tok = int(prompt[p])
        emb = np.zeros(m.dim, np.float32)
        oracle.lib().orc_widen_bf16_array(np.ascontiguousarray(v["token_emb"][tok]), emb, m.dim)
        xn = oracle.rmsnorm(emb, v["l0.attn_norm"], m.norm_eps)
        k = oracle.matvec(v["l0.wk"], xn)
        vv = oracle.matvec(v["l0.wv"], xn)
        for g in (0, m.n_kv_heads - 1):
            kg = oracle.rope_apply(k[g * m.head_dim:(g + 1) * m.head_dim], p, m.rope_theta)
            rows.append({"layer": 0, "kv": 0, "group": g, "pos": p, "val": [float(x) for x in kg]})
            rows.append({"layer": 0, "kv": 1, "group": g, "pos": p,
                         "val": [float(x) for x in vv[g * m.head_dim:(g + 1) * m.head_dim]]})
    return {"workload": w.name, "fingerprint": fingerprint(m, arena), "short_prompt": prompt[:5].tolist(),
            "short": short, "prefill_rows": rows, "seconds": time.time() - t0}


JOBS = {"llama135m_p1000": golden_p1000, "llama135m_b64": golden_b64, "llama8b_p4096": golden_8b}


def main(names):
    for name in names or list(JOBS):
        t0 = time.time()
        data = JOBS[name]()
        path = os.path.join(HERE, f"{name}.json")
        with open(path, "w") as f:
            json.dump(data, f, separators=(",", ":"))
        print(f"{name}: {os.path.getsize(path)} bytes in {time.time() - t0:.0f} s", flush=True)


if __name__ == "__main__":
    main(sys.argv[1:])
