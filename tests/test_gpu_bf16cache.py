"""Parity of the bf16 key/value cache (cache_dtype = DS_BF16) with the oracle's
bf16-cache mode (pinned in test_oracle_bf16cache.py) on the GPU (needs a
gfx950 GPU).

Both sides round every stored key and value to bfloat16, nearest-even, and
attend over the rounded values.  The fp32 values they round differ in their
last bits (the GPU sums in another order), so a value near a rounding
boundary may land one bf16 step apart: cache rows are compared to within
one step, and the logits with the tolerance of every other parity test.
"""
import dataclasses

import numpy as np
import pytest

import synth
from test_gpu_parity import compare, gpu_run

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("D,H,Hkv", [(64, 2, 2), (64, 6, 2), (64, 8, 2), (128, 4, 1), (128, 2, 2)],
                         ids=["d64-rep1", "d64-rep3", "d64-rep4", "d128-rep4", "d128-rep1"])
@pytest.mark.parametrize("B", [1, 3])
def test_bf16_cache_small_matches_oracle(D, H, Hkv, B):
    shape = synth.small_shape(dim=128, n_heads=H, n_kv_heads=Hkv, head_dim=D, hidden_dim=192, vocab_size=256,
                              cache_dtype=synth.BF16)
    arena = synth.make_arena(shape, 61, std=0.1, gain_sigma=0.1)
    rng = np.random.default_rng(62 + B)
    lens = rng.integers(1, 140, size=B)
    prompts = [synth.random_tokens(800 + b, int(n), shape.vocab_size) for b, n in enumerate(lens)]
    compare(shape, arena, prompts, 3, 160, f"bf16 cache D={D} H={H} Hkv={Hkv} B={B}")


@pytest.mark.parametrize("split", ["split", "tiled"])
def test_bf16_cache_mfma_projections_match_oracle(split, monkeypatch):
    """B = 20 with bf16 weights: the MFMA projections' epilogues store the
    rounded keys and values."""
    if split == "tiled":
        monkeypatch.setenv("DS_MM_SPLIT", "0")
    shape = synth.small_shape(dim=128, n_heads=4, n_kv_heads=2, head_dim=64, hidden_dim=256, vocab_size=512,
                              weight_dtype=synth.BF16, cache_dtype=synth.BF16)
    arena = synth.make_arena(shape, 63, std=0.1, gain_sigma=0.1)
    rng = np.random.default_rng(64)
    prompts = [synth.random_tokens(820 + b, int(n), shape.vocab_size) for b, n in enumerate(rng.integers(1, 80, 20))]
    compare(shape, arena, prompts, 3, 96, f"bf16 cache mfma {split}")


def test_bf16_cache_batched_prefill_matches_oracle():
    shape = synth.small_shape(dim=128, n_heads=4, n_kv_heads=2, head_dim=64, hidden_dim=256, vocab_size=512,
                              weight_dtype=synth.BF16, cache_dtype=synth.BF16)
    arena = synth.make_arena(shape, 65, std=0.1, gain_sigma=0.1)
    prompts = [synth.random_tokens(840, 90, shape.vocab_size)]
    compare(shape, arena, prompts, 2, 128, "bf16 cache batched prefill", batched=True)


def test_bf16_cache_135m_matches_oracle():
    w = synth.WORKLOADS["llama135m_p5"]
    shape = dataclasses.replace(w.model, cache_dtype=synth.BF16)
    arena = synth.make_arena(shape, w.model_seed)
    prompts = [synth.random_tokens(841, 70, shape.vocab_size)]
    compare(shape, arena, prompts, 3, 128, "bf16 cache 135m")


def test_bf16_cache_replication_and_limits():
    import torch
    import decode_step_02_amd as dsa
    shape = synth.small_shape(dim=128, n_heads=4, n_kv_heads=2, head_dim=64, hidden_dim=192, vocab_size=256,
                              cache_dtype=synth.BF16)
    model = dsa.Model(shape, synth.make_arena(shape, 66, std=0.1))
    src = dsa.KVCache(model, 1, 64)
    assert src.cache.dtype == torch.bfloat16 and src.single_launch_ctx() == 0
    tok = torch.zeros(1, dtype=torch.int32, device="cuda")
    src.prefill(0, [int(t) for t in synth.random_tokens(842, 20, shape.vocab_size)], tok)
    dst = dsa.KVCache(model, 3, 64)
    dst.cache.fill_(float("nan"))
    dst.replicate_from(src, 0, 1, 2)
    sv, dv = src.cache_view().float().cpu().numpy(), dst.cache_view().float().cpu().numpy()
    for r in (1, 2):
        assert np.array_equal(dv[:, :, r, :, :20].view(np.uint32), sv[:, :, 0, :, :20].view(np.uint32))
        assert np.all(np.isnan(dv[:, :, r, :, 20:]))
    assert np.all(np.isnan(dv[:, :, 0]))
    f32 = dsa.KVCache(dsa.Model(dataclasses.replace(shape, cache_dtype=synth.F32), synth.make_arena(shape, 66, std=0.1)), 2, 64)
    with pytest.raises(dsa.DSError):
        f32.replicate_from(src, 0, 0, 1)  # different element types
    bad = dataclasses.replace(shape, head_dim=32, n_heads=8)
    assert dsa.ds_weights_bytes(dsa.ds_config.of(bad)) == 0 and "bf16 cache" in dsa.ds_last_error()
