"""Parity helpers shared by the GPU tests: the logit tolerance, the near-tie
protocol for greedy tokens, and teacher-forced runs of the HIP path and the
reference decoder on the same seeded inputs."""
from __future__ import annotations

import numpy as np

ABS_TOL = 5e-4   # max |logit_gpu - logit_ref|
REL_TOL = 1e-4   # max |logit_gpu - logit_ref| / max |logit_ref|



def logit_errors(got: np.ndarray, ref: np.ndarray):
    d = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    mx = float(d.max()) if d.size else 0.0
    scale = float(np.abs(ref).max()) if ref.size else 1.0
    return mx, mx / max(scale, 1e-30)


def assert_logits_close(got, ref, what="", tol=(ABS_TOL, REL_TOL)):
    assert np.all(np.isfinite(got)), f"{what}: non-finite GPU values"
    mx, rel = logit_errors(got, ref)
    assert mx <= tol[0] and rel <= tol[1], f"{what}: max|d|={mx:.3e} rel={rel:.3e}"
    return mx


def top2_gap(v: np.ndarray) -> float:
    s = np.sort(v.astype(np.float64))
    return float(s[-1] - s[-2])


def check_tokens(gpu_tok, ref_tok, ref_logits, gpu_logits, what=""):
    """Greedy tokens must match, except where the reference's top-2 gap is
    within twice the measured logit error (a near-tie: both picks are correct
    to fp32 rounding).  Returns the number of near-ties."""
    ties = 0
    for b in range(len(ref_tok)):
        if int(gpu_tok[b]) == int(ref_tok[b]):
            continue
        err = float(np.abs(gpu_logits[b].astype(np.float64) - ref_logits[b]).max())
        gap = top2_gap(ref_logits[b])
        assert gap <= 2 * err, (f"{what}: seq {b} token {gpu_tok[b]} != {ref_tok[b]} "
                                f"(gap {gap:.3e} > 2 x err {err:.3e})")
        assert ref_logits[b][int(gpu_tok[b])] >= ref_logits[b].max() - 2 * err
        ties += 1
    return ties


def _bf16_steps_apart(a, b):
    """|a - b| in units in the last place of bf16 at the larger magnitude."""
    m = np.maximum(np.abs(a), np.abs(b)).astype(np.float64)
    ulp = np.where(m > 0, 2.0 ** (np.floor(np.log2(np.where(m > 0, m, 1.0))) - 7), 1.0)
    return np.where(m > 0, np.abs(a.astype(np.float64) - b.astype(np.float64)) / ulp, 0.0)


def bf16_teacher_forced(shape, arena, gpu_cache, gpu_lgs, positions, tokens, T, n_samples=8):
    """Each step of a bf16-cache run recomputed by the oracle from the GPU's
    own cache, so that the two sides start the step from the same state.

    Both sides round keys and values to bf16 from fp32 numbers computed in
    different orders, so a value within fp32 rounding of a bf16 rounding
    boundary lands one bf16 step apart, and later positions attend over it:
    compared from scratch, the runs drift apart by amounts no fp32 tolerance
    covers.  Fed the GPU's cached rows, the oracle's step differs from the
    GPU's only by fp32 rounding and by such flips in the row the step itself
    writes.  So for step k (positions[k][b], tokens[k][b] for every sequence
    b), with the oracle's cache set to the GPU's final cache (rows a step reads
    were final when it ran), the logits must agree within the fp32 tolerance
    plus an allowance of 2 x (the step's new-row differences, in bf16 steps) x
    (the largest logit change per bf16 step of one cached value, measured in
    the oracle on up to n_samples values moved one step).  Returns per step
    (max |d|, max |ref|, allowance, new-row steps)."""
    import oracle
    B = len(positions[0])
    gc = np.ascontiguousarray(gpu_cache, dtype=np.float32)
    assert not np.any(gc[np.isfinite(gc)].view(np.uint32) & 0xFFFF), "a cache value is not a bf16 value"

    def step(cache, k, b_only=None):
        m = oracle.Model(shape, arena, B, T)
        m.cache[:] = cache.reshape(-1)
        bs = list(range(B)) if b_only is None else [b_only]
        _, lg = m.forward_items(bs, [positions[k][b] for b in bs], [int(tokens[k][b]) for b in bs], [1] * len(bs))
        return m, lg.astype(np.float64)

    # sensitivity: the last step, one cached value it reads moved one bf16 step
    rng = np.random.default_rng(97)
    k_last = len(positions) - 1
    per_step = 0.0
    base = {}
    for _ in range(n_samples):
        b = int(rng.integers(0, B))
        p = positions[k_last][b]
        if p < 1:
            continue
        if b not in base:
            base[b] = step(gc, k_last, b)[1][0]
        l, kv = int(rng.integers(0, shape.n_layers)), int(rng.integers(0, 2))
        g, t, e = int(rng.integers(0, shape.n_kv_heads)), int(rng.integers(0, p)), int(rng.integers(0, shape.head_dim))
        c = gc.copy()
        v = c[l, kv, b, g, t, e]
        c[l, kv, b, g, t, e] = (np.float32(v).view(np.uint32) + np.uint32(0x10000)).view(np.float32)
        st = float(_bf16_steps_apart(np.float32(v), c[l, kv, b, g, t, e]))
        if st > 0:
            per_step = max(per_step, float(np.abs(step(c, k_last, b)[1][0] - base[b]).max()) / st)
    out = []
    for k in range(len(positions)):
        m, lg = step(gc, k)
        cv = m.cache_view()
        new_steps = 0.0
        for b in range(B):
            p = positions[k][b]
            new_steps += float(_bf16_steps_apart(cv[:, :, b, :, p], gc[:, :, b, :, p]).sum())
        d = float(np.abs(lg - gpu_lgs[k].astype(np.float64)).max())
        out.append((d, float(np.abs(lg).max()), 2.0 * new_steps * per_step, new_steps))
    return out


def oracle_run(shape, arena, prompts, decode_calls, T, feed=None, fast=False):
    """Reference decoder: ragged prompts, then `decode_calls` batched greedy
    steps.  Returns (first tokens, first logits, [tokens per step], [logits per
    step], oracle model).  feed[k] overrides the tokens fed at step k.  With
    `fast`, the batched evaluation (bit-identical, pinned in
    test_oracle_batch.py) does the work: for long prompts."""
    import oracle
    B = len(prompts)
    m = oracle.Model(shape, arena, B, T)
    V = shape.vocab_size
    first_tok = np.zeros(B, np.int32)
    first_lg = np.zeros((B, V), np.float32)
    for b, p in enumerate(prompts):
        if fast:
            tok, lg = m.prefill_fast(b, p)
        else:
            for t, tk in enumerate(p):
                tok, lg = m.forward(b, t, int(tk))
        first_tok[b], first_lg[b] = tok, lg
    lengths = np.array([len(p) for p in prompts], np.int32)
    toks, lgs = [], []
    cur = first_tok.copy()
    for k in range(decode_calls):
        fed = cur if feed is None else np.asarray(feed[k], np.int32)
        cur, lg = (m.decode_fast if fast else m.decode_step)(lengths, fed)
        toks.append(cur.copy())
        lgs.append(lg.copy())
    return first_tok, first_lg, toks, lgs, m
