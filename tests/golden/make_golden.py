"""Writes the expected values of the full-size GPU parity tests.

Every number stored here comes from the reference decoder (``oracle/``) run
on the seeded inputs of ``synth``; nothing comes from the HIP library.  The
batched evaluation (``Model.prefill_fast`` / ``Model.decode_fast``, bit-
identical to the per-position decoder, pinned in tests/test_oracle_batch.py)
makes the full workloads affordable on the host:

* llama135m_b64.npz -- all 64 sequences of the ragged batch: their prompts
  (lengths uniform in [1, 1008]), then 16 greedy decode steps of the whole
  batch.  Per sequence and new token: the greedy token, the top-2 gap, the
  top-8 logits, 64 fixed sampled logits and max |logit|; sampled cache rows
  of every sequence.
* llama8b_p4096.npz -- the 8B-shaped model, 4096-token prompt, then 32
  greedy decode steps at positions 4096..4127 (T = 4160).  Per new token the
  same summary with 256 sampled logits; cache rows at layers 0, 15 and 31.

The 1000-token 135M workload is checked against the reference decoder live
in its GPU test (a couple of seconds on the host), with full logits.

Usage: python tests/golden/make_golden.py [workload ...]
"""
from __future__ import annotations

import hashlib
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402

N_TOP = 8


def fingerprint(shape, arena) -> str:
    """sha256 over the first 4 KiB of every arena tensor and the arena size."""
    h = hashlib.sha256(str(arena.nbytes).encode())
    for _, off, _, _ in synth.tensor_table(shape)[0]:
        h.update(arena[off:off + 4096].tobytes())
    return h.hexdigest()


def sample_indices(V: int, n: int, seed: int) -> np.ndarray:
    return np.sort(np.random.default_rng(seed).choice(V, n, replace=False)).astype(np.int32)


class Summary:
    """Per new token: greedy token, top-2 gap, top-8 (index, value), the
    logits at fixed sampled indices, and max |logit|."""

    def __init__(self, idx: np.ndarray):
        self.idx = idx
        self.rows = {k: [] for k in ("token", "gap", "top_idx", "top_val", "sample_val", "max_abs")}

    def add(self, logits: np.ndarray):
        lg = logits.astype(np.float64)
        top = np.argsort(-lg, kind="stable")[:N_TOP]
        s = np.sort(lg)
        self.rows["token"].append(int(oracle.argmax(logits)))
        self.rows["gap"].append(float(s[-1] - s[-2]))
        self.rows["top_idx"].append(top.astype(np.int32))
        self.rows["top_val"].append(logits[top].astype(np.float32))
        self.rows["sample_val"].append(logits[self.idx].astype(np.float32))
        self.rows["max_abs"].append(float(np.abs(lg).max()))

    def arrays(self, prefix=""):
        return {prefix + k: np.array(v) for k, v in self.rows.items()}


def cache_rows(m: oracle.Model, probe):
    """probe: (seq, layer, kv, group, pos) tuples -> (meta int32 [R][5], values f32 [R][D])."""
    cv = m.cache_view()
    meta = np.array(probe, np.int32)
    vals = np.stack([cv[l, kv, b, g, p] for (b, l, kv, g, p) in probe]).astype(np.float32)
    return meta, vals


def golden_b64():
    w = synth.WORKLOADS["llama135m_b64"]
    m_shape = w.model
    arena = synth.make_arena(m_shape, w.model_seed)
    prompts = synth.prompts(w)
    lens = np.array([len(p) for p in prompts], np.int32)
    B = len(prompts)
    m = oracle.Model(m_shape, arena, B, w.ctx)
    t0 = time.time()
    # every prompt position of every sequence as the items of one pass
    seq = np.concatenate([np.full(n, b, np.int32) for b, n in enumerate(lens)])
    pos = np.concatenate([np.arange(n, dtype=np.int32) for n in lens])
    tok = np.concatenate([np.asarray(p, np.int32) for p in prompts])
    want = np.concatenate([(np.arange(n) == n - 1).astype(np.int32) for n in lens])
    tok_out, logits = m.forward_items(seq, pos, tok, want)
    print(f"b64: prefill of {len(seq)} positions in {time.time() - t0:.0f} s", flush=True)
    idx = sample_indices(m_shape.vocab_size, 64, 7)
    sums = [Summary(idx) for _ in range(B)]
    for b in range(B):
        sums[b].add(logits[b])
    cur = tok_out[want == 1].copy()
    lengths = lens.copy()
    for k in range(w.decode_calls):
        cur, lg = m.decode_fast(lengths, cur)
        for b in range(B):
            sums[b].add(lg[b])
    print(f"b64: {w.decode_calls} decode steps done at {time.time() - t0:.0f} s", flush=True)
    probe = []
    for b in range(B):
        n = int(lens[b])
        for l in (0, 29):
            for kv in (0, 1):
                for p in sorted({0, n - 1, n + w.decode_calls - 1}):
                    probe.append((b, l, kv, b % m_shape.n_kv_heads, p))
    meta, vals = cache_rows(m, probe)
    out = {"sample_idx": idx, "lengths": lens, "rows_meta": meta, "rows_val": vals}
    per = [s.arrays() for s in sums]
    for k in per[0]:
        out[k] = np.stack([p[k] for p in per])  # [B][steps][...]
    out["fingerprint"] = np.array(fingerprint(m_shape, arena))
    out["seconds"] = np.array(time.time() - t0)
    return out


def golden_8b():
    w = synth.WORKLOADS["llama8b_p4096"]
    ms = w.model
    t0 = time.time()
    arena = synth.make_arena(ms, w.model_seed)
    fp = fingerprint(ms, arena)
    print(f"8b: arena in {time.time() - t0:.0f} s", flush=True)
    prompt = synth.prompts(w)[0]
    m = oracle.Model(ms, arena, 1, w.ctx)
    t1 = time.time()
    tok, lg = m.prefill_fast(0, prompt, chunk=len(prompt))
    print(f"8b: prefill of {len(prompt)} positions in {time.time() - t1:.0f} s", flush=True)
    idx = sample_indices(ms.vocab_size, 256, 8)
    s = Summary(idx)
    s.add(lg)
    lengths = np.array([len(prompt)], np.int32)
    cur = np.array([tok], np.int32)
    for k in range(w.decode_calls):
        cur, lgs = m.decode_fast(lengths, cur)
        s.add(lgs[0])
    print(f"8b: {w.decode_calls} decode steps done at {time.time() - t1:.0f} s", flush=True)
    n = len(prompt)
    probe = [(0, l, kv, g, p) for l in (0, 15, 31) for kv in (0, 1) for g in (0, 3, 7)
             for p in (0, 1, 2047, n - 1, n, n + 15, n + w.decode_calls - 1)]
    meta, vals = cache_rows(m, probe)
    out = {"sample_idx": idx, "rows_meta": meta, "rows_val": vals, "prompt_len": np.array(n)}
    out.update(s.arrays())
    out["fingerprint"] = np.array(fp)
    out["seconds"] = np.array(time.time() - t0)
    return out


JOBS = {"llama135m_b64": golden_b64, "llama8b_p4096": golden_8b}


def main(names):
    for name in names or list(JOBS):
        t0 = time.time()
        data = JOBS[name]()
        path = os.path.join(HERE, f"{name}.npz")
        np.savez_compressed(path, **data)
        print(f"{name}: {os.path.getsize(path)} bytes in {time.time() - t0:.0f} s", flush=True)


if __name__ == "__main__":
    main(sys.argv[1:])
