"""The stored goldens are the reference decoder's own output on the seeded
inputs (CPU only): part of tests/golden/llama135m_b64.npz is recomputed here
and must match bit for bit.

The B = 64 golden was computed for all 64 sequences in one batch; the rows of
a batch are independent (pinned in test_oracle_model.py), so one sequence run
alone gives the same numbers.  The shortest sequence is recomputed with the
oracle's batched evaluation: its prompt, then 16 greedy steps.
"""
import os

import numpy as np

import oracle
import synth
from conftest import GOLDEN


def _golden(name):
    with np.load(os.path.join(GOLDEN, name), allow_pickle=False) as z:
        return {k: z[k] for k in z.files}


def test_b64_golden_shortest_sequence_recomputed():
    g = _golden("llama135m_b64.npz")
    w = synth.WORKLOADS["llama135m_b64"]
    prompts = synth.prompts(w)
    lens = np.array([len(p) for p in prompts])
    assert lens.tolist() == g["lengths"].tolist()
    b = int(np.argmin(lens))
    arena = synth.make_arena(w.model, w.model_seed)
    m = oracle.Model(w.model, arena, 1, w.ctx)
    tok, lg = m.prefill_fast(0, prompts[b])
    steps = [lg.copy()]
    toks = [tok]
    lengths = np.array([len(prompts[b])], np.int32)
    for _ in range(w.decode_calls):
        t, l = m.decode_fast(lengths, np.array([toks[-1]], np.int32))
        toks.append(int(t[0]))
        steps.append(l[0].copy())
    idx = g["sample_idx"]
    assert toks == g["token"][b].tolist()
    for k, lgk in enumerate(steps):
        assert np.array_equal(lgk[idx].view(np.uint32), g["sample_val"][b, k].view(np.uint32)), k
        assert np.array_equal(lgk[g["top_idx"][b, k]].view(np.uint32), g["top_val"][b, k].view(np.uint32)), k
    cv = m.cache_view()
    rows = [(r, v) for r, v in zip(g["rows_meta"], g["rows_val"]) if r[0] == b]
    assert rows
    for (seq, l, kv, grp, p), val in rows:
        assert np.array_equal(cv[l, kv, 0, grp, p].view(np.uint32), val.view(np.uint32))
