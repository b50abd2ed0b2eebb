"""Cache replication and per-row decode steps (needs a gfx950 GPU).

"Inside nanochat Part 4", section "Batch Prefilling via Cache Replication":
a batch-1 prefill is copied into the rows of a decode cache and the rows
then decode in parallel; section "Early Stopping Implementation": rows that
have finished stop.  ds_kv_cache_replicate copies the rows (bit for bit,
positions past the length untouched); ds_decode_step_rows advances the listed
rows only.  Each row is checked against the reference decoder run on that
row's own token sequence, with the tolerance of the other parity tests.
"""
import numpy as np
import pytest

import synth
from parity import assert_logits_close

pytestmark = pytest.mark.gpu


def _oracle_rows(shape, arena, prompt, feeds, T):
    """Reference logits of one prompt continued by each row's own tokens:
    feeds[r][k] is fed at position len(prompt) + k."""
    import oracle
    out = []
    for f in feeds:
        m = oracle.Model(shape, arena, 1, T)
        for t, tk in enumerate(prompt):
            m.forward(0, t, int(tk))
        lgs = []
        for k, tk in enumerate(f):
            lgs.append(m.forward(0, len(prompt) + k, int(tk))[1])
        out.append(lgs)
    return out


def _feeds(rows, steps, V, seed):
    rng = np.random.default_rng(seed)
    return [[int(x) for x in rng.integers(0, V, steps)] for _ in range(rows)]


@pytest.mark.parametrize("which", ["tiny", "135m"])
def test_replicate_prefill_then_parallel_decode(which):
    import torch
    import decode_step_02_amd as dsa
    if which == "tiny":
        shape = synth.TINY
        arena = synth.make_arena(shape, 21, std=0.15)
        rows, steps, T = 5, 4, 32
    else:
        w = synth.WORKLOADS["llama135m_p5"]
        shape, arena = w.model, synth.make_arena(w.model, w.model_seed)
        rows, steps, T = 3, 2, 32
    prompt = [int(x) for x in synth.random_tokens(500, 7, shape.vocab_size)]
    model = dsa.Model(shape, arena)
    src = dsa.KVCache(model, 1, 16)
    tok = torch.zeros(1, dtype=torch.int32, device="cuda")
    src.prefill(0, prompt, tok)
    dst = dsa.KVCache(model, rows + 1, T)
    dst.cache.fill_(float("nan"))
    dst.replicate_from(src, 0, 1, rows)  # slots 1..rows; slot 0 stays empty
    n = len(prompt)
    assert dst.get_lengths() == [0] + [n] * rows
    assert dst.lengths.cpu().tolist() == [0] + [n] * rows
    sv, dv = src.cache_view().cpu().numpy(), dst.cache_view().cpu().numpy()
    for r in range(1, rows + 1):
        assert np.array_equal(dv[:, :, r, :, :n].view(np.uint32), sv[:, :, 0, :, :n].view(np.uint32))
        assert np.all(np.isnan(dv[:, :, r, :, n:]))
    assert np.all(np.isnan(dv[:, :, 0]))
    feeds = _feeds(rows, steps, shape.vocab_size, 501)
    ref = _oracle_rows(shape, arena, prompt, feeds, T)
    tin = torch.zeros(rows + 1, dtype=torch.int32, device="cuda")
    out = torch.zeros(rows + 1, dtype=torch.int32, device="cuda")
    live = list(range(1, rows + 1))
    for k in range(steps):
        tin.copy_(torch.tensor([0] + [feeds[r][k] for r in range(rows)], dtype=torch.int32))
        dst.decode_step_rows(live, tin, out)
        lg = dst.logits().cpu().numpy()
        for r in range(rows):
            assert_logits_close(lg[r + 1], ref[r][k], f"{which} row {r} step {k}")
    dst.check()
    assert dst.get_lengths() == [0] + [n + steps] * rows
    assert np.all(np.isnan(dst.cache_view().cpu().numpy()[:, :, 0]))  # the empty slot was never written


def test_replicate_within_a_cache_and_stop_rows():
    """Copies within one cache, then rows stop one after the other: a row
    that is not listed keeps its length and its rows past it."""
    import torch
    import decode_step_02_amd as dsa
    shape = synth.small_shape(n_kv_heads=2, head_dim=32, dim=128, n_heads=4)
    arena = synth.make_arena(shape, 22, std=0.15)
    model = dsa.Model(shape, arena)
    B, T = 4, 40
    kv = dsa.KVCache(model, B, T)
    kv.cache.fill_(float("nan"))
    prompt = [int(x) for x in synth.random_tokens(502, 9, shape.vocab_size)]
    tok = torch.zeros(B, dtype=torch.int32, device="cuda")
    kv.prefill(0, prompt, tok)
    kv.replicate_from(kv, 0, 1, 3)
    n = len(prompt)
    steps = 5
    feeds = _feeds(B, steps, shape.vocab_size, 503)
    ref = _oracle_rows(shape, arena, prompt, feeds, T)
    tin = torch.zeros(B, dtype=torch.int32, device="cuda")
    out = torch.zeros(B, dtype=torch.int32, device="cuda")
    done = [0] * B
    for k in range(steps):
        live = [r for r in range(B) if r <= k + 1 or r == 3]  # rows 0..3 join; row 2 stops after step 1
        live = [r for r in live if not (r == 2 and k >= 2)]
        tin.copy_(torch.tensor([feeds[r][done[r]] for r in range(B)], dtype=torch.int32))
        kv.decode_step_rows(live, tin, out)
        lg = kv.logits().cpu().numpy()
        for r in live:
            assert_logits_close(lg[r], ref[r][done[r]], f"row {r} token {done[r]}")
            done[r] += 1
    kv.check()
    assert kv.get_lengths() == [n + d for d in done]
    assert kv.lengths.cpu().tolist() == [n + d for d in done]
    cv = kv.cache_view().cpu().numpy()
    for r in range(B):
        assert np.all(np.isnan(cv[:, :, r, :, n + done[r]:])), f"row {r} written past its length"
    with pytest.raises(dsa.DSError) as e:
        kv.decode_step_rows([1, 1], tin, out)
    assert e.value.status == -1
    with pytest.raises(dsa.DSError) as e:
        kv.replicate_from(kv, 0, 0, 2)  # the source among the destinations
    assert e.value.status == -1
    with pytest.raises(dsa.DSError) as e:
        kv.replicate_from(kv, 0, 3, 2)  # past B
    assert e.value.status == -1
    small = dsa.KVCache(model, 1, 8)
    with pytest.raises(dsa.DSError) as e:
        small.replicate_from(kv, 1, 0, 1)  # 9 + positions into T = 8
    assert e.value.status == -4
    other = dsa.Model(synth.TINY, synth.make_arena(synth.TINY, 1))
    okv = dsa.KVCache(other, 1, 64)
    with pytest.raises(dsa.DSError) as e:
        okv.replicate_from(kv, 0, 0, 1)  # different key/value shapes
    assert e.value.status == -1
