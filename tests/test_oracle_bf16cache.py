"""Pins of the oracle's bf16 key/value cache (cache_dtype = BF16), independent
of the oracle's own code.

"simple-llm / kasahare" (PyPI README 0.4.0, section "Limitations
(intentional)") lists cache compression among what it leaves out; the
reduced-precision variants read a bf16 cache as: every key and value row is
rounded to bfloat16 (nearest, ties to even) when stored, and attention reads
the rounded values.

- the rounding against torch's float32 -> bfloat16 conversion, on random
  values over a wide exponent range and on exact ties (kept part even and
  odd);
- layer 0 at position 0 does not depend on the cache, so its stored rows are
  exactly the rounded rows of the fp32-cache run, and every stored value of
  the bf16 run is a bfloat16;
- cached decoding equals the uncached rerun bit for bit in this mode too;
- the rounding is applied (logits differ from the fp32-cache run) and its
  effect is small.
"""
import dataclasses

import numpy as np
import pytest

import oracle
import synth


def test_round_bf16_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(51)
    x = (rng.standard_normal(200000) * np.exp2(rng.integers(-60, 60, 200000))).astype(np.float32)
    ties = np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x40490000 | 0x8000, 0x00018000], np.uint32).view(np.float32)
    x = np.concatenate([x, ties, np.array([0.0, -0.0, 1.0, -3.5], np.float32)])
    got = np.array([oracle.lib().orc_round_bf16(float(v)) for v in x], np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def _shape(cdt):
    return dataclasses.replace(synth.small_shape(hidden_dim=192), cache_dtype=cdt)


def test_first_position_rows_are_the_rounded_fp32_rows():
    s32, s16 = _shape(synth.F32), _shape(synth.BF16)
    arena = synth.make_arena(s32, 52, std=0.1, gain_sigma=0.1)
    m32 = oracle.Model(s32, arena, 1, 8)
    m16 = oracle.Model(s16, arena, 1, 8)
    m32.forward(0, 0, 17)
    m16.forward(0, 0, 17)
    c32, c16 = m32.cache_view(), m16.cache_view()
    r32 = c32[0, :, 0, :, 0]
    want = np.array([oracle.lib().orc_round_bf16(float(v)) for v in r32.reshape(-1)], np.float32).reshape(r32.shape)
    assert np.array_equal(c16[0, :, 0, :, 0].view(np.uint32), want.view(np.uint32))
    assert not np.array_equal(r32, want)  # the rows were not already bf16
    for p in range(1, 5):
        m16.forward(0, p, 30 + p)
    assert np.all((m16.cache.view(np.uint32) & 0xFFFF) == 0)


def test_cached_equals_uncached_with_a_bf16_cache():
    s16 = _shape(synth.BF16)
    arena = synth.make_arena(s16, 53, std=0.1)
    prompt = synth.random_tokens(54, 4, s16.vocab_size)
    a = oracle.Model(s16, arena, 1, 16).generate(0, prompt, 5)
    b = oracle.Model(s16, arena, 1, 16).generate(0, prompt, 5, uncached=True)
    assert np.array_equal(a[0], b[0])
    assert np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))


def test_bf16_cache_changes_the_logits_a_little():
    s32, s16 = _shape(synth.F32), _shape(synth.BF16)
    arena = synth.make_arena(s32, 55, std=0.1)
    m32, m16 = oracle.Model(s32, arena, 1, 16), oracle.Model(s16, arena, 1, 16)
    for p, t in enumerate(synth.random_tokens(56, 8, s32.vocab_size)):
        _, l32 = m32.forward(0, p, int(t))
        _, l16 = m16.forward(0, p, int(t))
    d = np.abs(l16 - l32).max() / np.abs(l32).max()
    assert 0 < d < 2e-2
