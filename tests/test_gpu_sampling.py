"""Parity of the sampling epilogue (ds_sample) with the oracle's sampler
(needs a gfx950 GPU).

The GPU samples from the logits its own step produced; the oracle's sampler
(orc_sample, pinned in test_oracle_sampling.py) runs on the same fp32 logits
read back, with the same uniform draw.  The token must be the oracle's, or,
where the draw sits within 2e-5 of the boundary between two candidates (the
GPU sums its weights in fp32 in another order), the neighbouring candidate.
The same tolerance applies to where top-p cuts the candidate list.
"""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

EPS = 2e-5

CONFIGS = [  # temperature, top_k, top_p
    (0.8, 40, 0.95),   # the defaults of the simple-llm CLI
    (1.0, 0, 1.0),     # every token, index order
    (0.7, 1, 1.0),     # a single candidate: the argmax
    (1.5, 1024, 1.0),  # the largest top-k
    (1.0, 2, 1.0),     # the pages' top-k example size
    (1.0, 50, 0.5),    # a tight nucleus
    (0.3, 300, 0.9),
]


def check_token(got, row, t, k, p, u, what):
    tok, cand, cum = oracle.sample(row, t, k, p, u)
    if got == tok:
        return 0
    # neighbours in draw order, with the draw on their shared boundary
    _, full, _ = oracle.sample(row, t, k, 1.0, 0.0)
    where = {int(c): j for j, c in enumerate(full)}
    assert got in where, f"{what}: token {got} is not a candidate"
    jg, jo = where[got], where[tok]
    assert abs(jg - jo) == 1, f"{what}: token {got} (#{jg}) vs oracle {tok} (#{jo}) at u={u}"
    lo = min(jg, jo)
    if lo < len(cum):
        assert abs(cum[lo] - u) <= EPS or jg >= len(cum), f"{what}: draw {u} far from boundary {cum[lo]}"
    if jg >= len(cum):  # the GPU kept one more candidate: top-p at its boundary
        w = np.cumsum(oracle.sample(row, t, k, 1.0, 0.0)[2])
        assert abs(w[len(cum) - 1] - p) <= EPS, f"{what}: top-p cut differs far from the boundary"
    return 1


def _run(shape, arena, B, prompt_len, steps, seed):
    import torch
    import decode_step_02_amd as dsa
    model = dsa.Model(shape, arena)
    kv = dsa.KVCache(model, B, prompt_len + steps + 1)
    prompts = [synth.random_tokens(seed + b, prompt_len, shape.vocab_size) for b in range(B)]
    tok = torch.zeros(B, dtype=torch.int32, device="cuda")
    kv.prefill_batch([[int(x) for x in p] for p in prompts], tok)
    rng = np.random.default_rng(seed)
    out = torch.zeros(B, dtype=torch.int32, device="cuda")
    near = checked = 0
    for s in range(steps + 1):
        if s > 0:
            kv.decode_step(tok, tok)
        logits = kv.logits().cpu().numpy()
        for (t, k, p) in CONFIGS:
            u = rng.random(B).astype(np.float32)
            kv.sample(torch.from_numpy(u).cuda(), t, k, p, out)
            got = out.cpu().numpy()
            for b in range(B):
                near += check_token(int(got[b]), logits[b], t, k, p, float(u[b]),
                                    f"step {s} seq {b} t={t} k={k} p={p}")
                checked += 1
        # feed a sampled token on to the next step
        tok.copy_(out)
    kv.check()
    kv.close()
    model.close()
    return checked, near


def test_sampling_tiny_matches_oracle():
    shape = synth.TINY
    arena = synth.make_arena(shape, 5, std=0.15)
    checked, near = _run(shape, arena, 3, 6, 4, 900)
    print(f"tiny: {checked} draws, {near} on a boundary", flush=True)
    assert near <= checked // 50


def test_sampling_135m_matches_oracle():
    w = synth.WORKLOADS["llama135m_p5"]
    arena = synth.make_arena(w.model, w.model_seed)
    checked, near = _run(w.model, arena, 2, 5, 3, 901)
    print(f"135m: {checked} draws, {near} on a boundary", flush=True)
    assert near <= checked // 50


def test_sampling_frequencies_follow_the_distribution():
    """A grid of 2048 uniform draws through the GPU sampler, one call each on
    the same logits, gives the oracle's probabilities as frequencies (the
    draw is an inverse distribution function)."""
    import torch
    import decode_step_02_amd as dsa
    shape = synth.TINY
    arena = synth.make_arena(shape, 6, std=0.3)
    model = dsa.Model(shape, arena)
    kv = dsa.KVCache(model, 1, 8)
    tok = torch.zeros(1, dtype=torch.int32, device="cuda")
    kv.prefill(0, [3, 1, 4], tok)
    logits = kv.logits().cpu().numpy()[0]
    n = 2048
    u = torch.from_numpy(((np.arange(n) + 0.5) / n).astype(np.float32)).cuda()
    outs = torch.zeros(n, dtype=torch.int32, device="cuda")
    for (t, k, p) in [(1.0, 0, 1.0), (0.9, 5, 1.0), (1.2, 20, 0.8)]:
        for i in range(n):
            kv.sample(u[i:i + 1], t, k, p, outs[i:i + 1])
        got = np.bincount(outs.cpu().numpy(), minlength=shape.vocab_size) / n
        _, cand, cum = oracle.sample(logits, t, k, p, 0.0)
        want = np.zeros(shape.vocab_size)
        want[cand] = np.diff(np.concatenate([[0.0], cum]))
        assert np.abs(got - want).max() <= 2.0 / n, f"t={t} k={k} p={p}"
    kv.close()
    model.close()


def test_sampling_argument_errors():
    import torch
    import decode_step_02_amd as dsa
    shape = synth.TINY
    model = dsa.Model(shape, synth.make_arena(shape, 1))
    kv = dsa.KVCache(model, 1, 8)
    u = torch.zeros(1, dtype=torch.float32, device="cuda")
    out = torch.zeros(1, dtype=torch.int32, device="cuda")
    for args, status in [((0.0, 10, 1.0), -1), ((1.0, -1, 1.0), -1), ((1.0, 10, 0.0), -1),
                         ((1.0, 10, 1.5), -1), ((1.0, 0, 0.9), -2)]:
        with pytest.raises(dsa.DSError) as e:
            kv.sample(u, *args, out)
        assert e.value.status == status, args
    kv.sample(u, 1.0, 2000, 1.0, out)  # top_k above V is V (256 <= 1024)
    kv.close()
    model.close()
