"""Pins for the reference decoder as a whole (CPU only)."""
import dataclasses

import numpy as np
import pytest

import oracle
import synth
from conftest import golden
import hf_reference


def _run(shape, seed, prompt, n_new, gain_sigma=0.0, T=64, uncached=False):
    arena = synth.make_arena(shape, seed, gain_sigma=gain_sigma)
    m = oracle.Model(shape, arena, 1, T)
    toks, lg, passes = m.generate(0, prompt, n_new, uncached=uncached)
    return arena, m, toks, lg, passes


def test_layout_agrees_with_generator():
    for w in synth.WORKLOADS.values():
        off, total = oracle.tensor_offsets(w.model)
        table, total2 = synth.tensor_table(w.model)
        assert total == total2 and off == [t[1] for t in table]


def test_135m_shape_matches_page():
    """GOTOken: 134.5M weights, a 270 MB bf16 checkpoint, 576 query outputs."""
    g = golden("smollm2_135m_shape.json")
    m = synth.M135
    table, _ = synth.tensor_table(m)
    n = sum(int(np.prod(s)) for _, _, s, _ in table)
    assert round(n / 1e6, 1) == g["weights_millions"]
    assert abs(n * 2 / 1e6 - g["checkpoint_megabytes_bf16"]) / g["checkpoint_megabytes_bf16"] < 0.01
    assert m.q_rows == g["q_projection_outputs"]
    assert synth.WORKLOADS["llama135m_p5"].ctx == g["context"]


VARIANTS = {
    "tiny": dict(),
    "tiny_gains": dict(gain_sigma=0.1),
    "mha": dict(shape=dict(n_kv_heads=4)),
    "mqa": dict(shape=dict(n_kv_heads=1), gain_sigma=0.1),
    "bf16": dict(shape=dict(weight_dtype=synth.BF16), gain_sigma=0.1),
    "untied_d128": dict(shape=dict(tied_embeddings=0, head_dim=32, dim=96, rope_theta=5e5)),
}


@pytest.mark.parametrize("name", list(VARIANTS))
def test_oracle_against_hf_llama_fp64(name):
    """The library the GOTOken page matches its engine against, run in
    float64 over the full causal sequence, gives the logits of every
    generated token within fp32 rounding error."""
    spec = VARIANTS[name]
    shape = dataclasses.replace(synth.TINY, **spec.get("shape", {}))
    # larger weights than the configs' 0.02 so attention and the MLP move
    # the residual stream visibly and a wrong term cannot hide
    arena = synth.make_arena(shape, 7, std=0.15, gain_sigma=spec.get("gain_sigma", 0.0))
    prompt = synth.random_tokens(77, 6, shape.vocab_size)
    m = oracle.Model(shape, arena, 1, 64)
    toks, lg, _ = m.generate(0, prompt, 6)
    seq = np.concatenate([prompt, toks[:-1]])
    ref = hf_reference.logits(hf_reference.build(shape, arena), seq)[len(prompt) - 1:]
    err = np.abs(lg - ref).max()
    assert err <= 2e-5 * np.abs(ref).max(), err
    assert np.array_equal(toks, ref.argmax(-1))


def test_oracle_against_hf_llama_fp64_at_135m_shape():
    shape = synth.M135
    arena = synth.make_arena(shape, 2)
    prompt = synth.prompts(synth.WORKLOADS["llama135m_p5"])[0][:3]
    m = oracle.Model(shape, arena, 1, 8)
    toks, lg, _ = m.generate(0, prompt, 2)
    seq = np.concatenate([prompt, toks[:-1]])
    ref = hf_reference.logits(hf_reference.build(shape, arena), seq)[len(prompt) - 1:]
    assert np.abs(lg - ref).max() <= 2e-5 * np.abs(ref).max()
    assert np.array_equal(toks, ref.argmax(-1))


def test_cached_equals_uncached_and_pass_counts():
    """GOTOken, 'About one token per second': 5 + 8 tokens take 68 passes
    uncached and 12 cached, with bit-identical output."""
    g = golden("kv_cache_passes.json")
    w = synth.WORKLOADS["tiny_p5"]
    prompt = synth.prompts(w)[0]
    assert len(prompt) == g["prompt_tokens"]
    arena = synth.make_arena(w.model, 5, std=0.15, gain_sigma=0.1)
    a = oracle.Model(w.model, arena, 1, w.ctx)
    b = oracle.Model(w.model, arena, 1, w.ctx)
    ta, la, pa = a.generate(0, prompt, g["new_tokens"])
    tb, lb, pb = b.generate(0, prompt, g["new_tokens"], uncached=True)
    assert (pa, pb) == (g["cached_passes"], g["uncached_passes"])
    assert np.array_equal(ta, tb)
    assert np.array_equal(la.view(np.uint32), lb.view(np.uint32))
    assert np.array_equal(a.cache.view(np.uint32), b.cache.view(np.uint32))


def test_cached_equals_uncached_at_135m_shape():
    shape = synth.M135
    arena = synth.make_arena(shape, 2)
    prompt = synth.prompts(synth.WORKLOADS["llama135m_p5"])[0][:3]
    a = oracle.Model(shape, arena, 1, 8)
    b = oracle.Model(shape, arena, 1, 8)
    ta, la, pa = a.generate(0, prompt, 3)
    tb, lb, pb = b.generate(0, prompt, 3, uncached=True)
    assert (pa, pb) == (5, 3 + 4 + 5)
    assert np.array_equal(ta, tb) and np.array_equal(la, lb)


def test_written_rows_never_change():
    """Rows of earlier positions are never rewritten by later steps."""
    shape = synth.TINY
    arena = synth.make_arena(shape, 3, std=0.15)
    m = oracle.Model(shape, arena, 1, 32)
    lengths = np.zeros(1, np.int32)
    tok = np.array([17], np.int32)
    snaps = []
    for step in range(10):
        tok, _ = m.decode_step(lengths, tok)
        snaps.append(m.cache_view()[:, :, 0, :, :step + 1].copy())
    final = m.cache_view()[:, :, 0]
    for step, s in enumerate(snaps):
        assert np.array_equal(final[:, :, :, :step + 1], s)
    assert np.all(final[:, :, :, 10:] == 0)


def test_batch_rows_are_independent():
    """Row b of a batched decode equals a batch-1 run of sequence b: the
    tokens and logits, and every cached row of slot b, bit for bit."""
    shape = synth.small_shape(n_kv_heads=2)
    arena = synth.make_arena(shape, 4, std=0.15)
    B, T = 3, 40
    prompts = [synth.random_tokens(s, n, shape.vocab_size) for s, n in ((1, 4), (2, 9), (3, 1))]
    mb = oracle.Model(shape, arena, B, T)
    lengths = np.zeros(B, np.int32)
    # ragged prefill: sequence b is fed its prompt one position per step
    longest = max(len(p) for p in prompts)
    singles = [oracle.Model(shape, arena, 1, T) for _ in range(B)]
    for b, p in enumerate(prompts):
        for t, tk in enumerate(p):
            mb.forward(b, t, tk)
            singles[b].forward(0, t, tk)
        lengths[b] = len(p)
    tok = np.array([5, 6, 7], np.int32)
    for step in range(4):
        tok_b, lg_b = mb.decode_step(lengths, tok)
        for b in range(B):
            t1, lg1 = singles[b].forward(0, int(lengths[b]) - 1, tok[b])
            assert t1 == tok_b[b] and np.array_equal(lg1, lg_b[b])
        tok = tok_b
    assert longest == 9
    # the B axis of the (L, 2, B, Hkv, T, D) cache: slot b of the batched
    # cache holds what slot 0 of sequence b's own cache holds, and nothing
    # else was written
    cb = mb.cache_view()
    for b in range(B):
        cs = singles[b].cache_view()[:, :, 0]
        assert np.array_equal(cb[:, :, b].view(np.uint32), cs.view(np.uint32))
        n = int(lengths[b])
        assert np.any(cs[:, :, :, :n] != 0) and np.all(cs[:, :, :, n:] == 0)


def test_cache_index_is_row_major_over_l_2_b_h_t_d(orc):
    """[NANO] "Cache Architecture": one (L, 2, B, H, T, D) tensor; element 0
    of row (l, kv, b, g, t) sits where numpy's row-major order puts it."""
    import ctypes as C
    shape = synth.small_shape(n_kv_heads=2)
    cfg = oracle.config_of(shape)
    rng = np.random.default_rng(3)
    L, B, H, T, D = shape.n_layers, 5, shape.n_kv_heads, 37, shape.head_dim
    dims = (L, 2, B, H, T, D)
    for _ in range(200):
        l, kv, b, g, t = (int(rng.integers(0, n)) for n in dims[:5])
        got = orc.orc_cache_index(C.byref(cfg), B, T, l, kv, b, g, t)
        assert got == np.ravel_multi_index((l, kv, b, g, t, 0), dims)


def test_gqa_equals_mha_with_repeated_kv_rows():
    """Grouped-query attention with Hkv key/value heads is multi-head
    attention whose key/value projections repeat each group's rows for the
    H/Hkv query heads that share it; both give bit-identical results."""
    gqa = synth.TINY  # H=4, Hkv=2
    mha = dataclasses.replace(gqa, n_kv_heads=gqa.n_heads)
    a_g = synth.make_arena(gqa, 9, std=0.15, gain_sigma=0.1)
    a_m = np.zeros(synth.arena_bytes(mha), np.uint8)
    vg, vm = synth.views(gqa, a_g), synth.views(mha, a_m)
    rep = gqa.n_heads // gqa.n_kv_heads
    D = gqa.head_dim
    for name in vm:
        if name.endswith(".wk") or name.endswith(".wv"):
            src = vg[name].reshape(gqa.n_kv_heads, D, gqa.dim)
            vm[name][...] = np.repeat(src, rep, axis=0).reshape(-1, gqa.dim)
        else:
            vm[name][...] = vg[name]
    prompt = synth.random_tokens(12, 5, gqa.vocab_size)
    tg, lg, _ = oracle.Model(gqa, a_g, 1, 32).generate(0, prompt, 6)
    tm, lm, _ = oracle.Model(mha, a_m, 1, 32).generate(0, prompt, 6)
    assert np.array_equal(tg, tm) and np.array_equal(lg.view(np.uint32), lm.view(np.uint32))


def test_bad_arguments_are_rejected():
    shape = synth.TINY
    m = oracle.Model(shape, synth.make_arena(shape, 1), 1, 8)
    for b, pos, tok in ((0, 0, 256), (0, 0, -1), (0, 8, 1), (1, 0, 1)):
        with pytest.raises(ValueError):
            m.forward(b, pos, tok)
