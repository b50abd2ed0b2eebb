"""The allocation-free sampling entry point (ds_sample_noalloc) against
ds_sample (needs a gfx950 GPU).

ds_sample_noalloc runs the same sampling kernels as ds_sample, with its
scratch in a static device array of the library instead of the cache's
workspace.  On the same logits and uniforms both must give the same tokens,
bit for bit, on two calls in a row, the second with fewer rows and a smaller
vocabulary, in each sampling mode (the two-kernel path with and without
top-k, and the one-workgroup path for a long top-k list); the array keeps the
last call's contents, so the second call also shows that nothing carries over.
"""
import dataclasses

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

MODES = [  # temperature, top_k, top_p
    (0.8, 40, 0.95),
    (1.0, 0, 1.0),
    (0.5, 1024, 0.9),
]


def _step_logits(shape, B, seed):
    """A model and a B-row cache after a prefill and one decode step."""
    import torch
    import decode_step_02_amd as dsa
    arena = synth.make_arena(shape, seed, std=0.15)
    model = dsa.Model(shape, arena)
    kv = dsa.KVCache(model, B, 32)
    tok = torch.zeros(B, dtype=torch.int32, device="cuda")
    kv.prefill_batch([[int(x) for x in synth.random_tokens(seed + b, 5, shape.vocab_size)] for b in range(B)], tok)
    kv.decode_step(tok, tok)
    return model, kv


def test_noalloc_matches_ds_sample_twice_second_smaller():
    import torch
    import decode_step_02_amd as dsa
    big = dataclasses.replace(synth.TINY, vocab_size=4000)   # 4 slices of 1024 logits
    small = dataclasses.replace(synth.TINY, vocab_size=1500)
    rng = np.random.default_rng(17)
    for shape, B in ((big, 37), (small, 5)):
        print(f"noalloc: B={B} V={shape.vocab_size}", flush=True)
        model, kv = _step_logits(shape, B, 3 + B)
        logits = kv.logits().clone()
        for (t, k, p) in MODES:
            u = torch.from_numpy(rng.random(B).astype(np.float32)).cuda()
            ref = torch.full((B,), -1, dtype=torch.int32, device="cuda")
            got = torch.full((B,), -2, dtype=torch.int32, device="cuda")
            kv.sample(u, t, k, p, ref)
            dsa.ds_sample_noalloc(logits, B, shape.vocab_size, u, t, k, p, got)
            torch.cuda.synchronize()
            r, g = ref.cpu().numpy(), got.cpu().numpy()
            assert np.all((r >= 0) & (r < shape.vocab_size))
            assert np.array_equal(r, g), f"B={B} V={shape.vocab_size} t={t} k={k} p={p}: {r} vs {g}"
        kv.check()
        kv.close()
        model.close()


def test_noalloc_in_a_captured_graph():
    """The caller it is for: ds_sample_noalloc captured into a graph
    (torch.cuda.CUDAGraph) over fixed input and output buffers, replayed with
    new uniforms copied in between replays, gives ds_sample's tokens on every
    replay."""
    import torch
    import decode_step_02_amd as dsa
    shape = dataclasses.replace(synth.TINY, vocab_size=3000)
    B = 9
    model, kv = _step_logits(shape, B, 77)
    logits = kv.logits().clone()
    u = torch.zeros(B, dtype=torch.float32, device="cuda")
    got = torch.zeros(B, dtype=torch.int32, device="cuda")
    st = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            dsa.ds_sample_noalloc(logits, B, shape.vocab_size, u, 0.9, 50, 0.9, got, st)
    rng = np.random.default_rng(5)
    for r in range(3):
        draws = torch.from_numpy(rng.random(B).astype(np.float32)).cuda()
        u.copy_(draws)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = torch.full((B,), -1, dtype=torch.int32, device="cuda")
        kv.sample(draws, 0.9, 50, 0.9, ref)
        torch.cuda.synchronize()
        assert np.array_equal(got.cpu().numpy(), ref.cpu().numpy()), f"replay {r}"
    kv.check()
    kv.close()
    model.close()


def test_noalloc_rejects_rows_above_its_scratch():
    import torch
    import decode_step_02_amd as dsa
    n = dsa.DS_SAMPLE_NOALLOC_MAX_ROWS + 1
    logits = torch.zeros((n, 64), dtype=torch.float32, device="cuda")
    u = torch.zeros(n, dtype=torch.float32, device="cuda")
    out = torch.zeros(n, dtype=torch.int32, device="cuda")
    with pytest.raises(dsa.DSError) as e:
        dsa.ds_sample_noalloc(logits, n, 64, u, 1.0, 0, 1.0, out)
    assert e.value.status == -2
    with pytest.raises(dsa.DSError):
        dsa.ds_sample_noalloc(logits, 2, 64, u, 0.0, 0, 1.0, out)  # temperature 0
    dsa.ds_sample_noalloc(logits, 0, 64, u, 1.0, 0, 1.0, out)     # B == 0 does nothing
