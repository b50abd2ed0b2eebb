"""Parity of the block-quantised int8 and int4 weights (DS_Q8, DS_Q4) on the
GPU (needs a gfx950 GPU).

The reading ("simple-llm / kasahare" PyPI README 0.4.0, section "Where to go
from here": INT8 weight loading, block-quantised): int8 values and one fp32
scale per 32 values of a row, element = scale * value.  The oracle's Q8 path
is pinned in test_oracle_q8.py.  Here:

- small shapes and the 135M shape against the oracle, one launch per
  operation at batch 1, 3 and 20 (Q8 has no single-launch step and no MFMA
  projections), over the fused short attention and the split-K attention;
- the full 8B shape: a Q8 model whose weights equal those of a bf16 model
  (every weight k / 4096, |k| <= 127: q = k, s = 2^-12; for Q4 k / 512,
  |k| <= 7) must give the bf16 model's logits, whose own parity with the
  oracle the 8B golden test pins.
The GPU sums each 16-value chunk of a block before multiplying by the
scale, the oracle multiplies each weight by its scale first: the rounding
order differs, so the logits tolerance of the other parity tests applies.
"""
import dataclasses

import numpy as np
import pytest

import synth
from parity import assert_logits_close, check_tokens
from test_gpu_parity import compare, gpu_run

pytestmark = pytest.mark.gpu

Q8_SMALL = synth.small_shape(dim=128, n_heads=4, n_kv_heads=2, head_dim=32, hidden_dim=256, vocab_size=512,
                             weight_dtype=synth.Q8)
DTYPES = {"q8": synth.Q8, "q4": synth.Q4}


@pytest.mark.parametrize("dt", ["q8", "q4"])
@pytest.mark.parametrize("B", [1, 3, 20])
def test_q8_small_matches_oracle(B, dt):
    shape = dataclasses.replace(Q8_SMALL, weight_dtype=DTYPES[dt])
    arena = synth.make_arena(shape, 41, std=0.1, gain_sigma=0.1)
    rng = np.random.default_rng(40 + B)
    lens = rng.integers(1, 50, size=B)
    prompts = [synth.random_tokens(700 + b, int(n), shape.vocab_size) for b, n in enumerate(lens)]
    compare(shape, arena, prompts, 3, 64, f"{dt} B={B}")


@pytest.mark.parametrize("dt", ["q8", "q4"])
def test_q8_small_batched_prefill_matches_oracle(dt):
    shape = dataclasses.replace(Q8_SMALL, weight_dtype=DTYPES[dt])
    arena = synth.make_arena(shape, 42, std=0.1, gain_sigma=0.1)
    prompts = [synth.random_tokens(710, 45, shape.vocab_size)]
    compare(shape, arena, prompts, 2, 64, f"{dt} batched prefill", batched=True)


@pytest.mark.parametrize("dt", ["q8", "q4"])
def test_q8_135m_matches_oracle(dt):
    w = synth.WORKLOADS["llama135m_p5"]
    shape = dataclasses.replace(w.model, weight_dtype=DTYPES[dt])
    arena = synth.make_arena(shape, w.model_seed)
    prompts = [synth.random_tokens(711, 5, shape.vocab_size)]
    compare(shape, arena, prompts, 3, 64, f"{dt} 135m")


@pytest.mark.parametrize("dt", ["q8", "q4"])
def test_q8_8b_equals_bf16_on_the_exact_grid(dt):
    import torch
    import decode_step_02_amd as dsa
    w = synth.WORKLOADS["llama8b_p4096"]
    bf = w.model
    q8 = dataclasses.replace(bf, weight_dtype=DTYPES[dt])
    grid = True if dt == "q8" else "q4"
    prompt = [int(t) for t in synth.random_tokens(712, 40, bf.vocab_size)]
    feed = [int(t) for t in synth.random_tokens(713, 3, bf.vocab_size)]
    out = {}
    for name, shape in (("bf16", bf), ("q8", q8)):
        arena = synth.make_arena(shape, w.model_seed, exact=grid)
        model = dsa.Model(shape, arena)
        del arena
        kv = dsa.KVCache(model, 1, 64)
        tok = torch.zeros(1, dtype=torch.int32, device="cuda")
        kv.prefill_batched(0, prompt, tok)
        lgs = [kv.logits().cpu().numpy()[0].copy()]
        toks = [tok.item()]
        for t in feed:
            tok.fill_(t)
            kv.decode_step(tok, tok)
            lgs.append(kv.logits().cpu().numpy()[0].copy())
            toks.append(tok.item())
        kv.check()
        out[name] = (toks, lgs)
        kv.close()
        model.close()
        del model
        torch.cuda.empty_cache()
        print(f"8b {name}: tokens {toks}", flush=True)
    for k, (a, b) in enumerate(zip(out["q8"][1], out["bf16"][1])):
        assert_logits_close(a, b, f"8b exact grid step {k}")
        check_tokens([out["q8"][0][k]], [out["bf16"][0][k]], [b], [a], f"8b exact grid step {k}")
