"""Pins for the batched evaluation of the reference decoder (oracle/batch.c).

orc_forward_items must give exactly what orc_forward gives, bit for bit, for
every item: the logits, the greedy tokens and every cache value.  It changes
only which independent sums run side by side (vector lanes, host threads), and
the prompt's positions go layer by layer together ([NANO] "Attention
Mechanism Integration").  These tests run the plain per-position decoder and
the batched one on the same seeded inputs and compare the bits, in every
weight and cache format, through both product kernels (items in lanes for 16
or more items, rows in lanes below that), with one and several threads.
"""
import dataclasses

import numpy as np
import pytest

import oracle
import synth


def _plain_and_batched(shape, arena, prompts, steps, T, threads, chunk):
    B = len(prompts)
    a = oracle.Model(shape, arena, B, T)
    b = oracle.Model(shape, arena, B, T)
    first_a, first_b = [], []
    for s, p in enumerate(prompts):
        for t, tk in enumerate(p):
            tok, lg = a.forward(s, t, int(tk))
        first_a.append((tok, lg))
        first_b.append(b.prefill_fast(s, p, chunk=chunk, threads=threads))
    for (ta, la), (tb, lb) in zip(first_a, first_b):
        assert ta == tb and np.array_equal(la.view(np.uint32), lb.view(np.uint32))
    assert np.array_equal(a.cache.view(np.uint32), b.cache.view(np.uint32))
    len_a = np.array([len(p) for p in prompts], np.int32)
    len_b = len_a.copy()
    tok = np.array([t for t, _ in first_a], np.int32)
    for k in range(steps):
        t1, l1 = a.decode_step(len_a, tok)
        t2, l2 = b.decode_fast(len_b, tok, threads=threads)
        assert np.array_equal(t1, t2), f"step {k}"
        assert np.array_equal(l1.view(np.uint32), l2.view(np.uint32)), f"step {k}"
        tok = t1
    assert np.array_equal(len_a, len_b)
    assert np.array_equal(a.cache.view(np.uint32), b.cache.view(np.uint32))


TINY_CASES = {
    "fp32_gains_ragged": dict(shape={}, gain_sigma=0.1, lens=(70, 5, 23, 1), chunk=33),
    "fp32_20_sequences": dict(shape={}, lens=tuple(range(3, 23)), chunk=16),
    "bf16_mqa": dict(shape=dict(weight_dtype=synth.BF16, n_kv_heads=1), lens=(40, 17), chunk=64),
    "bf16_cache_untied": dict(shape=dict(cache_dtype=synth.BF16, tied_embeddings=0), lens=(33, 33, 2), chunk=12),
    "q8": dict(shape=dict(weight_dtype=synth.Q8, hidden_dim=192), lens=(40,) * 17, chunk=40),
    "q4": dict(shape=dict(weight_dtype=synth.Q4, hidden_dim=192), lens=(29, 3), chunk=20),
    "mha_head_dim_32": dict(shape=dict(n_kv_heads=4, head_dim=32, dim=96, rope_theta=5e5), lens=(50,), chunk=50),
}


@pytest.mark.parametrize("name", list(TINY_CASES))
@pytest.mark.parametrize("threads", [1, 4])
def test_batched_equals_plain_tiny(name, threads):
    spec = TINY_CASES[name]
    shape = dataclasses.replace(synth.TINY, **spec["shape"])
    arena = synth.make_arena(shape, 11, std=0.15, gain_sigma=spec.get("gain_sigma", 0.0))
    prompts = [synth.random_tokens(100 + i, n, shape.vocab_size) for i, n in enumerate(spec["lens"])]
    _plain_and_batched(shape, arena, prompts, 3, 96, threads, spec["chunk"])


def test_batched_equals_plain_135m():
    """The 135M shape: a 20-position prompt as one batch (items in lanes),
    then a decode step at batch 1 (rows in lanes)."""
    shape = synth.M135
    arena = synth.make_arena(shape, 2)
    prompt = synth.prompts(synth.WORKLOADS["llama135m_p1000"])[0][:20]
    _plain_and_batched(shape, arena, [prompt], 1, 32, 8, 64)


def test_batched_rejects_bad_items():
    shape = synth.TINY
    m = oracle.Model(shape, synth.make_arena(shape, 1), 2, 8)
    ones = np.ones(2, np.int32)
    with pytest.raises(ValueError):  # one (sequence, position) twice
        m.forward_items([0, 0], [3, 3], [1, 2], ones)
    with pytest.raises(ValueError):  # token out of range
        m.forward_items([0, 1], [0, 0], [1, 256], ones)
    with pytest.raises(ValueError):  # position past T
        m.forward_items([0, 1], [0, 8], [1, 1], ones)
    with pytest.raises(ValueError):  # sequence past B
        m.forward_items([0, 2], [0, 0], [1, 1], ones)
    assert np.all(m.cache == 0)
