"""Parity of the HIP decode path with the reference decoder (needs a gfx950 GPU).

Every case runs the same seeded synthetic inputs through the library (via its
C ABI) and through the reference decoder, feeds the GPU the reference's greedy
tokens (teacher forcing), and compares logits (max |d| <= 5e-4 and relative
<= 1e-4), greedy tokens (exact, or a near-tie), cache rows (same tolerance),
untouched cache slots (still the NaN sentinel) and lengths (exact).
"""
import dataclasses
import sys

import numpy as np
import pytest

import synth
from parity import ABS_TOL, REL_TOL, assert_logits_close, bf16_teacher_forced, check_tokens, oracle_run

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def gpu_run(shape, arena, prompts, feed, T, dispatch=1, use_batch_prefill=True, stream=None, batched=False):
    """Prefill the prompts (ds_prefill_batch over the sequences, ds_prefill
    per sequence, or with `batched` ds_prefill_batched per sequence), then one
    decode step per entry of `feed` (tokens for every sequence).  Returns
    first tokens/logits, per-step tokens/logits, the cache and lengths as
    numpy arrays."""
    torch = _torch()
    import decode_step_02_amd as dsa
    B = len(prompts)
    model = dsa.Model(shape, arena)
    kv = dsa.KVCache(model, B, T)
    kv.set_dispatch(dispatch)
    kv.cache.fill_(float("nan"))
    tok_out = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    if batched:
        for b, p in enumerate(prompts):
            kv.prefill_batched(b, [int(t) for t in p], tok_out, stream)
    elif use_batch_prefill:
        kv.prefill_batch([list(p) for p in prompts], tok_out, stream)
    else:
        for b, p in enumerate(prompts):
            kv.prefill(b, list(p), tok_out, stream)
    first_tok = tok_out.cpu().numpy().copy()
    first_lg = kv.logits(stream).cpu().numpy().copy()
    toks, lgs = [], []
    tok_in = torch.zeros(B, dtype=torch.int32, device="cuda")
    for f in feed:
        tok_in.copy_(torch.from_numpy(np.asarray(f, np.int32)))
        kv.decode_step(tok_in, tok_out, stream)
        toks.append(tok_out.cpu().numpy().copy())
        lgs.append(kv.logits(stream).cpu().numpy().copy())
    if stream is not None:
        stream.synchronize()
    kv.check(stream)
    out = dict(first_tok=first_tok, first_lg=first_lg, toks=toks, lgs=lgs,
               cache=kv.cache_view().float().cpu().numpy(), lengths=kv.lengths.cpu().numpy(),
               mirror=np.array(kv.get_lengths()), single_launch_ctx=kv.single_launch_ctx())
    kv.close()
    model.close()
    return out


def bf16_rows_close(got, ref, what):
    """Cache rows of a bf16 cache.  Where both sides rounded a value near a
    rounding boundary they land one bf16 step apart, and later rows that
    attend over it inherit the difference; so every value must be within one
    bf16 step of the rows' largest magnitude (2^-7 max|ref|), and at least
    90% of the values must be bit-equal (a different rounding rule, or none,
    misses that by far)."""
    assert np.all(np.isfinite(got)), f"{what}: non-finite GPU values"
    d = np.abs(got.astype(np.float64) - ref)
    bound = 2.0 ** -7 * max(float(np.abs(ref).max()), 1.0)
    assert d.max() <= bound, f"{what}: max|d| {d.max():.3e} above one bf16 step {bound:.3e}"
    eq = float(np.mean(got.view(np.uint32) == np.ascontiguousarray(ref, np.float32).view(np.uint32)))
    assert eq >= 0.9, f"{what}: only {eq:.1%} of the values bit-equal"
    return eq


def compare(shape, arena, prompts, decode_calls, T, what, fast=False, **kw):
    ref_first, ref_first_lg, ref_toks, ref_lgs, om = oracle_run(shape, arena, prompts, decode_calls, T, fast=fast)
    feed = [ref_first] + ref_toks[:-1]
    g = gpu_run(shape, arena, prompts, feed, T, **kw)
    lengths = np.array([len(p) + decode_calls for p in prompts], np.int32)
    bf16 = shape.cache_dtype == synth.BF16
    note = ""
    if bf16:
        # (1) every step from the GPU's own cache: fp32 tolerance plus the
        # allowance for flips in the row the step writes
        positions = [[len(p) - 1 + k for p in prompts] for k in range(decode_calls + 1)]
        tokens = [[p[-1] for p in prompts]] + [list(feed[k]) for k in range(decode_calls)]
        tf = bf16_teacher_forced(shape, arena, g["cache"], [g["first_lg"]] + g["lgs"], positions, tokens, T)
        for k, (d, scale, allow, new_steps) in enumerate(tf):
            assert d <= ABS_TOL + allow and d <= REL_TOL * scale + allow, \
                f"{what} step {k} from the GPU's cache: max|d| {d:.3e} (new-row steps {new_steps:.0f}, allowance {allow:.2e})"
        # (2) from scratch: the GPU's bf16 run stays closer to the oracle's
        # than the bf16 rounding moves the oracle itself (its fp32-cache run
        # on the same tokens)
        f32 = dataclasses.replace(shape, cache_dtype=synth.F32)
        r32_first, r32_first_lg, _, r32_lgs, _ = oracle_run(f32, arena, prompts, decode_calls, T, feed=feed, fast=fast)
        own = [float(np.abs(r32_first_lg.astype(np.float64) - ref_first_lg).max())] + \
              [float(np.abs(r32_lgs[k].astype(np.float64) - ref_lgs[k]).max()) for k in range(decode_calls)]
        note = (f", from the GPU's cache max|d| {max(t[0] for t in tf):.2e} (new-row steps "
                f"{sum(t[3] for t in tf):.0f}); bf16 rounding moves the oracle by {min(own):.2e}..{max(own):.2e}")

    def close(got, ref, w, k):
        assert np.all(np.isfinite(got)), f"{w}: non-finite GPU values"
        d = float(np.abs(got.astype(np.float64) - ref.astype(np.float64)).max())
        if bf16:
            assert d <= own[k], f"{w}: max|d| {d:.3e} above the bf16 rounding's own effect {own[k]:.3e}"
        else:
            assert d <= ABS_TOL and d <= REL_TOL * float(np.abs(ref).max()), f"{w}: max|d|={d:.3e}"
        return d

    ties = check_tokens(g["first_tok"], ref_first, ref_first_lg, g["first_lg"], f"{what} prefill")
    worst = close(g["first_lg"], ref_first_lg, f"{what} prefill", 0)
    for k in range(decode_calls):
        worst = max(worst, close(g["lgs"][k], ref_lgs[k], f"{what} step {k}", k + 1))
        ties += check_tokens(g["toks"][k], ref_toks[k], ref_lgs[k], g["lgs"][k], f"{what} step {k}")
    assert np.array_equal(g["lengths"], lengths) and np.array_equal(g["mirror"], lengths)
    ref_cache = om.cache_view()
    for b, n in enumerate(lengths):
        got = g["cache"][:, :, b, :, :n]
        if shape.cache_dtype == synth.BF16:
            bf16_rows_close(got, ref_cache[:, :, b, :, :n], f"{what} cache seq {b}")
        else:
            assert_logits_close(got, ref_cache[:, :, b, :, :n], f"{what} cache seq {b}")
        assert np.all(np.isnan(g["cache"][:, :, b, :, n:])), f"{what}: slot beyond length written"
    _say(f"{what}: max|dlogit| {worst:.2e}, near-ties {ties}{note}")
    return g


def test_tiny_cached_decode_matches_oracle():
    w = synth.WORKLOADS["tiny_p5"]
    arena = synth.make_arena(w.model, w.model_seed)
    compare(w.model, arena, synth.prompts(w), w.decode_calls, w.ctx, "tiny")


def test_tiny_larger_weights_eager_and_graph_bitwise_equal():
    """std 0.15 weights move the residual stream far from the embedding, so
    greedy tokens vary; eager and graph dispatch give identical bits."""
    shape = synth.TINY
    arena = synth.make_arena(shape, 7, std=0.15, gain_sigma=0.1)
    prompts = [synth.random_tokens(77, 6, shape.vocab_size)]
    torch = _torch()
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        g_graph = compare(shape, arena, prompts, 20, 64, "tiny std0.15 graph", dispatch=1, stream=st)
        g_eager = compare(shape, arena, prompts, 20, 64, "tiny std0.15 eager", dispatch=0, stream=st)
    for a, b in zip(g_graph["lgs"], g_eager["lgs"]):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_tiny_uncached_equals_cached_on_gpu():
    """GOTOken, 'About one token per second': rerunning the whole prefix for
    every new token gives the cached result bit for bit (68 vs 12 passes)."""
    torch = _torch()
    import decode_step_02_amd as dsa
    w = synth.WORKLOADS["tiny_p5"]
    shape = w.model
    arena = synth.make_arena(shape, 3, std=0.15)
    prompt = list(synth.prompts(w)[0])
    model = dsa.Model(shape, arena)
    kv = dsa.KVCache(model, 1, w.ctx)
    out = torch.zeros(1, dtype=torch.int32, device="cuda")
    kv.prefill(0, prompt, out)
    cached_toks, cached_lg = [int(out.item())], [kv.logits().cpu().numpy().copy()]
    for _ in range(7):
        kv.decode_step(out, out)
        cached_toks.append(int(out.item()))
        cached_lg.append(kv.logits().cpu().numpy().copy())
    seq = list(prompt)
    passes = 0
    for k in range(8):
        kv.reset(0)
        kv.prefill(0, seq, out)
        passes += len(seq)
        assert int(out.item()) == cached_toks[k]
        assert np.array_equal(kv.logits().cpu().numpy().view(np.uint32), cached_lg[k].view(np.uint32))
        seq.append(int(out.item()))
    assert passes == 68


def test_prefill_reproduces_decode_steps_bitwise_past_the_short_path():
    """ds_prefill feeds one position per pass through the decode kernels, so
    re-prefilling a sequence together with its decoded tokens gives the decode
    steps' logits bit for bit, also with head_dim 64 and bf16 weights, whose
    multi-position passes take another attention kernel, and past the short
    path (positions 70.., split-K attention)."""
    torch = _torch()
    import decode_step_02_amd as dsa
    shape = synth.small_shape(dim=128, n_heads=4, n_kv_heads=2, head_dim=64, hidden_dim=192, vocab_size=256,
                              weight_dtype=synth.BF16)
    arena = synth.make_arena(shape, 48, std=0.1, gain_sigma=0.1)
    prompt = [int(t) for t in synth.random_tokens(1300, 70, shape.vocab_size)]
    model = dsa.Model(shape, arena)
    kv = dsa.KVCache(model, 2, 128)
    out = torch.zeros(2, dtype=torch.int32, device="cuda")
    kv.prefill(1, prompt, out)
    toks, lgs = [int(out[1].item())], [kv.logits().cpu().numpy()[1].copy()]
    for _ in range(4):
        kv.decode_step_rows([1], out, out)
        toks.append(int(out[1].item()))
        lgs.append(kv.logits().cpu().numpy()[1].copy())
    seq = list(prompt)
    for k in range(5):
        kv.reset(1)
        kv.prefill(1, seq, out)
        assert int(out[1].item()) == toks[k]
        assert np.array_equal(kv.logits().cpu().numpy()[1].view(np.uint32), lgs[k].view(np.uint32)), f"step {k}"
        seq.append(toks[k])
    kv.check()
    kv.close()
    model.close()


def test_ragged_batch_tiny_matches_oracle():
    shape = dataclasses.replace(synth.TINY, n_kv_heads=1)
    arena = synth.make_arena(shape, 4, std=0.15, gain_sigma=0.1)
    lens = [1, 9, 4, 70, 2, 33, 5]
    prompts = [synth.random_tokens(100 + i, n, shape.vocab_size) for i, n in enumerate(lens)]
    compare(shape, arena, prompts, 6, 128, "tiny ragged B=7 batch-prefill")
    compare(shape, arena, prompts, 3, 128, "tiny ragged B=7 per-slot prefill", use_batch_prefill=False)


def test_batched_prefill_tiny_matches_oracle():
    """ds_prefill_batched: prompt positions as the items of one pass (up to 64
    at a time), each attending over the rows up to its own position.  Prompt
    lengths cover 1 (no batched part), 2, one item under and over the
    16-item MFMA threshold, exactly 64 + 1, and two chunks plus a tail."""
    shape = synth.small_shape(n_kv_heads=2, head_dim=32, dim=128, n_heads=4)
    arena = synth.make_arena(shape, 9, std=0.15, gain_sigma=0.1)
    lens = [1, 2, 16, 17, 65, 130]
    prompts = [synth.random_tokens(300 + i, n, shape.vocab_size) for i, n in enumerate(lens)]
    compare(shape, arena, prompts, 3, 192, "tiny batched prefill", batched=True)


@pytest.mark.parametrize("wdt", ["F32", "BF16"])
def test_long_ffn_rows_ragged(wdt):
    """hidden_dim above 8192 takes the 8-wave W2 blocks (16 rows each); dim 40
    leaves the last block half empty."""
    shape = synth.small_shape(dim=40, n_heads=4, n_kv_heads=2, head_dim=16, hidden_dim=8200,
                              weight_dtype=getattr(synth, wdt))
    arena = synth.make_arena(shape, 12, std=0.05, gain_sigma=0.1)
    prompts = [synth.random_tokens(400 + i, n, shape.vocab_size) for i, n in enumerate([3, 7])]
    compare(shape, arena, prompts, 3, 16, f"long ffn rows {wdt}")


def test_attention_chunk_boundaries_tiny():
    """Lengths around multiples of the 64-position attention chunk, up to T."""
    shape = synth.small_shape(n_kv_heads=2, head_dim=32, dim=128, n_heads=4)
    arena = synth.make_arena(shape, 8, std=0.15)
    lens = [63, 64, 65, 127, 128, 129, 190]
    prompts = [synth.random_tokens(200 + i, n, shape.vocab_size) for i, n in enumerate(lens)]
    compare(shape, arena, prompts, 2, 192, "tiny chunk edges")


def test_135m_p5_matches_oracle():
    w = synth.WORKLOADS["llama135m_p5"]
    arena = synth.make_arena(w.model, w.model_seed)
    compare(w.model, arena, synth.prompts(w), w.decode_calls, w.ctx, "135m p5")


def test_errors_are_reported_without_enqueueing():
    torch = _torch()
    import decode_step_02_amd as dsa
    shape = synth.TINY
    model = dsa.Model(shape, synth.make_arena(shape, 1))
    kv = dsa.KVCache(model, 2, 8)
    out = torch.zeros(2, dtype=torch.int32, device="cuda")
    with pytest.raises(dsa.DSError) as e:
        kv.prefill(0, [1, 2, 300])
    assert e.value.status == -5
    with pytest.raises(dsa.DSError) as e:
        kv.prefill(2, [1])
    assert e.value.status == -1
    kv.prefill(0, [1] * 8)
    with pytest.raises(dsa.DSError) as e:
        kv.decode_step(out, out)
    assert e.value.status == -4
    assert kv.get_lengths() == [8, 0]
    kv.set_lengths([3, 0])
    bad = torch.tensor([5, 999], dtype=torch.int32, device="cuda")
    kv.decode_step(bad, out)
    with pytest.raises(dsa.DSError) as e:
        kv.check()
    assert e.value.status == -5
    kv.check()  # the flag was cleared
    assert kv.lengths.cpu().tolist() == [4, 1]


MM_SHAPE = synth.small_shape(dim=128, n_heads=4, n_kv_heads=2, head_dim=32, hidden_dim=256, vocab_size=512,
                             weight_dtype=synth.BF16)


# K = 192 is six 32-wide k-steps (two for waves 0 and 1, one for waves 2 and
# 3 of the split-K kernel); 20 Q/K/V row tiles leave four padding blocks
MM_SHAPE2 = synth.small_shape(dim=192, n_heads=6, n_kv_heads=2, head_dim=32, hidden_dim=320, vocab_size=640,
                              weight_dtype=synth.BF16)


# Rows long enough for the split-K kernel's batch loop: Q/K/V and W2 inputs
# of 1152 and 2304 values (9 and 18 k-steps per wave, ragged last batches),
# Wo's input 36 * 64 = 2304
MM_SHAPE_LONG = synth.small_shape(dim=1152, n_heads=36, n_kv_heads=12, head_dim=64, hidden_dim=2304,
                                  vocab_size=512, weight_dtype=synth.BF16)


@pytest.fixture(params=["split", "tiled"])
def mm_kernel(request, monkeypatch):
    """Both MFMA projection kernels: split-K (the default for narrow
    projections) and tiled (DS_MM_SPLIT=0)."""
    if request.param == "tiled":
        monkeypatch.setenv("DS_MM_SPLIT", "0")
    return request.param


def test_batched_prefill_bf16_mfma_matches_oracle(mm_kernel):
    """bf16 weights: 16 or more positions take the MFMA projections."""
    arena = synth.make_arena(MM_SHAPE, 12, std=0.1, gain_sigma=0.1)
    lens = [40, 3, 100]
    prompts = [synth.random_tokens(400 + i, n, MM_SHAPE.vocab_size) for i, n in enumerate(lens)]
    compare(MM_SHAPE, arena, prompts, 2, 128, "bf16 batched prefill", batched=True)


PF_ATTN = {
    # (head_dim, H, Hkv, cache) with bf16 weights
    "d64-rep3": (64, 9, 3, "F32"),
    "d64-rep1": (64, 2, 2, "F32"),
    "d128-rep4": (128, 8, 2, "F32"),
    "d128-rep2": (128, 4, 2, "F32"),
    "d64-rep2-bf16": (64, 4, 2, "BF16"),
    "d128-rep4-bf16": (128, 8, 2, "BF16"),
}


@pytest.mark.parametrize("name", list(PF_ATTN))
def test_batched_prefill_attention_matches_oracle(name):
    """ds_prefill_batched with head_dim 64 or 128: the positions of a pass
    share one sequence, so its attention (k_attn_pf) stages every 64-position
    chunk once for all of them and multiplies on the matrix cores.  Prompts of
    2, 17, 64, 65, 130 and 200 tokens: passes of one position and of 64,
    chunk edges, up to four chunks; then two decode steps."""
    D, H, Hkv, cdt = PF_ATTN[name]
    shape = synth.small_shape(dim=128, n_heads=H, n_kv_heads=Hkv, head_dim=D, hidden_dim=192, vocab_size=256,
                              weight_dtype=synth.BF16, cache_dtype=getattr(synth, cdt))
    arena = synth.make_arena(shape, 47, std=0.1, gain_sigma=0.1)
    prompts = [synth.random_tokens(1200 + b, n, shape.vocab_size) for b, n in enumerate([2, 17, 64, 65, 130, 200])]
    compare(shape, arena, prompts, 2, 256, f"batched prefill attention {name}", batched=True)


# Q/K/V rows of 1344 values take the long-row loop, whose waves cover 4 row
# tiles each; (4 + 2 * 1) * 16 = 96 rows are 6 tiles, so the second group of
# 4 holds two clamped tiles that are computed and not stored.  Its weights
# are drawn with half the spread of the other shapes': at 0.1 its logits
# reach 14, where fp32 rounding alone (about 5e-5 relative, in the tiled
# kernel too) exceeds the absolute bar.
MM_SHAPE_TILES6 = synth.small_shape(dim=1344, n_heads=4, n_kv_heads=1, head_dim=16, hidden_dim=1344,
                                    vocab_size=512, weight_dtype=synth.BF16)


@pytest.mark.parametrize("B,shape,std", [(20, MM_SHAPE, 0.1), (70, MM_SHAPE, 0.1), (37, MM_SHAPE2, 0.1),
                                         (18, MM_SHAPE_LONG, 0.1), (18, MM_SHAPE_TILES6, 0.05)],
                         ids=["20", "70", "37-k192", "18-long-rows", "18-six-row-tiles"])
def test_batched_mfma_projections_match_oracle(B, shape, std, mm_kernel):
    """Batches of 16+ sequences take the MFMA projections (bf16 weights, fp32
    activations split into two bf16 terms): 20 leaves part of a 16-item MFMA
    column group empty, 70 needs two 64-item launches of the tiled kernel."""
    arena = synth.make_arena(shape, 11, std=std, gain_sigma=0.1)
    rng = np.random.default_rng(B)
    lens = rng.integers(1, 40, size=B)
    prompts = [synth.random_tokens(300 + b, int(n), shape.vocab_size) for b, n in enumerate(lens)]
    compare(shape, arena, prompts, 3, 64, f"mfma B={B}")


def test_batched_mfma_long_rows_six_tiles_per_wave():
    """Q/K/V rows of 1344 values (the long-row loop) over (64 + 2 * 16) heads
    of 64, 384 row tiles: at 64 items the loop takes 6 row tiles per wave
    (256 blocks) where 4 would give 384 blocks, two rounds of a 256-CU
    device; Wo (rows of 4096) and W2 keep 4.  64 ragged sequences against
    the oracle, weights drawn with the six-tile shape's spread of 0.05."""
    shape = synth.small_shape(dim=1344, n_heads=64, n_kv_heads=16, head_dim=64, hidden_dim=1344, vocab_size=512,
                              weight_dtype=synth.BF16)
    arena = synth.make_arena(shape, 12, std=0.05, gain_sigma=0.1)
    rng = np.random.default_rng(64)
    lens = rng.integers(1, 40, size=64)
    prompts = [synth.random_tokens(900 + b, int(n), shape.vocab_size) for b, n in enumerate(lens)]
    _say(f"six row tiles per wave: B=64, Q/K/V tiles {(64 + 32) * 64 // 16}")
    compare(shape, arena, prompts, 3, 64, "mfma long rows, 6 tiles per wave", fast=True)


@pytest.mark.parametrize("D,H,Hkv", [(64, 2, 2), (64, 4, 2), (64, 6, 2), (64, 8, 2), (128, 4, 1)],
                         ids=["d64-rep1", "d64-rep2", "d64-rep3", "d64-rep4", "d128-rep4"])
@pytest.mark.parametrize("kernel", ["dpp", "shfl"])
def test_split_attention_kernels_match_oracle(D, H, Hkv, kernel, monkeypatch):
    """The split-K attention of head_dim 64 and 128 (DPP-reduced kernel, and
    the shuffle-reduced one with DS_ATTN_G=0) over 1..3 64-position chunks,
    the last one ragged, with the short-context path off."""
    monkeypatch.setenv("DS_SHORT_ATTN", "0")
    if kernel == "shfl":
        monkeypatch.setenv("DS_ATTN_G", "0")
    shape = synth.small_shape(dim=128, n_heads=H, n_kv_heads=Hkv, head_dim=D, hidden_dim=192, vocab_size=256)
    arena = synth.make_arena(shape, 14, std=0.1, gain_sigma=0.1)
    prompts = [synth.random_tokens(600 + b, n, shape.vocab_size) for b, n in enumerate([70, 130, 9])]
    compare(shape, arena, prompts, 3, 160, f"attention D={D} H={H} Hkv={Hkv} {kernel}")


LONG_ATTN = {
    # head_dim 256 (k_attn_d<256>), few (sequence, head) pairs: each head's
    # dims over 4 combine blocks; 18 chunks
    "d256-b1": (256, 2, 1, [1100], 1184),
    # head_dim 128 (k_attn_g<128>) with the 8B shape's allocated context: 65
    # chunks, combine over 4 blocks of 32 dims with 16 chunks per thread
    "d128-b1-T4160": (128, 4, 1, [1100], 4160),
    # H * B = 128 pairs: one combine block per head (256 dims, one chunk
    # group), so past 48 chunks (3072 positions) it takes several batches;
    # the short sequences also run the fused short-context path at D = 256
    "d256-b16-multibatch": (256, 8, 2, [3100, 3080] + [5 + 3 * i for i in range(14)], 3136),
    # head_dim 64 (k_attn_g<64, 3>) with 10 chunk slots: the launch grid is
    # 17 chunk indices wide (1 mod 8, so each sequence's chunks start on the
    # next XCD), the 7 past the cache returning at once; lengths reach every
    # chunk from the first to the last, each sequence ragged in its last
    "d64-b6-T640-grid17": (64, 6, 2, [600, 530, 70, 260, 129, 3], 640),
    # head_dim 64 with 32 chunk slots and 8 (sequence, head) pairs: the
    # one-wave merge of up to 80 chunks, a sequence short of half of them
    "d64-b2-T2048-merge32": (64, 4, 2, [1500, 700], 2048),
}


@pytest.mark.parametrize("name", list(LONG_ATTN))
def test_long_context_attention_head_dims(name):
    """Split-K attention and its combine at long contexts for head_dim 128
    and 256, against the reference decoder (its batched evaluation)."""
    D, H, Hkv, lens, T = LONG_ATTN[name]
    shape = synth.small_shape(dim=128, n_heads=H, n_kv_heads=Hkv, head_dim=D, hidden_dim=192, vocab_size=256)
    arena = synth.make_arena(shape, 31, std=0.1, gain_sigma=0.1)
    prompts = [synth.random_tokens(700 + b, n, shape.vocab_size) for b, n in enumerate(lens)]
    _say(f"long attention {name}: B={len(lens)} longest {max(lens)} T={T}")
    compare(shape, arena, prompts, 3, T, f"long attention {name}", fast=True)


def test_single_launch_steps_in_a_captured_graph():
    """Batch-1 single-launch steps captured by the caller into a graph
    (torch.cuda.CUDAGraph around ds_decode_step) and replayed: each replay
    advances the step like an eager call, with the same bits, with eager
    work and synchronisation between the replays."""
    torch = _torch()
    import decode_step_02_amd as dsa
    w = synth.WORKLOADS["llama135m_p5"]
    arena = synth.make_arena(w.model, w.model_seed)
    prompt = [int(t) for t in synth.prompts(w)[0]]
    model = dsa.Model(w.model, arena)
    outs = {}
    for mode in ("eager", "graph"):
        kv = dsa.KVCache(model, 1, w.ctx)
        assert kv.single_launch_ctx() >= len(prompt) + 6
        st = torch.cuda.Stream()
        tok = torch.zeros(1, dtype=torch.int32, device="cuda")
        with torch.cuda.stream(st):
            kv.prefill(0, prompt, tok, st)
            st.synchronize()
            seq, lgs = [], []
            if mode == "graph":
                g = torch.cuda.CUDAGraph()
                kv.set_lengths([len(prompt)], st)
                with torch.cuda.graph(g, stream=st):
                    kv.decode_step(tok, tok, st)  # captured, not run
                kv.set_lengths([len(prompt)], st)
                st.synchronize()
            for k in range(6):
                if mode == "graph":
                    g.replay()
                else:
                    kv.decode_step(tok, tok, st)
                st.synchronize()
                seq.append(int(tok.item()))
                lgs.append(kv.logits(st).cpu().numpy().copy())
                kv.set_lengths([len(prompt) + k + 1], st)  # the graph does not advance the host mirror
        kv.check(st)
        outs[mode] = (seq, lgs, kv.cache_view()[:, :, 0, :, :len(prompt) + 6].cpu().numpy())
        kv.close()
    (sa, la, ca), (sb, lb, cb) = outs["eager"], outs["graph"]
    assert sa == sb
    for a, b in zip(la, lb):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert np.array_equal(ca.view(np.uint32), cb.view(np.uint32))
    model.close()


def test_single_launch_replay_outside_its_context_class_is_reported():
    """A batch-1 single-launch step captured by the caller at a one-chunk
    context (32 positions) replays correctly in that class; replayed once
    more, its context (33) is in the longer class, which another
    instantiation serves: that launch writes nothing and the next check
    raises DS_ERR_DEVICE.  An eager step then takes the longer class's
    kernel and proceeds."""
    torch = _torch()
    import decode_step_02_amd as dsa
    w = synth.WORKLOADS["llama135m_p5"]
    arena = synth.make_arena(w.model, w.model_seed)
    model = dsa.Model(w.model, arena)
    kv = dsa.KVCache(model, 1, w.ctx)
    assert kv.single_launch_ctx() >= 40
    kv.cache.fill_(float("nan"))
    prompt = [int(t) for t in synth.random_tokens(77, 31, w.model.vocab_size)]
    st = torch.cuda.Stream()
    tok = torch.zeros(1, dtype=torch.int32, device="cuda")
    with torch.cuda.stream(st):
        kv.prefill(0, prompt, tok, st)
        st.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=st):
            kv.decode_step(tok, tok, st)  # captured at context 32, not run
        kv.set_lengths([31], st)
        st.synchronize()
        g.replay()  # context 32: the class of the capture
        st.synchronize()
        kv.check(st)
        assert kv.lengths.cpu().tolist() == [32]
        assert torch.isfinite(kv.cache_view()[:, :, 0, :, 31].float()).all()
        g.replay()  # context 33: the longer class
        st.synchronize()
        with pytest.raises(dsa.DSError) as err:
            kv.check(st)
        assert err.value.status == -9  # DS_ERR_DEVICE
        assert kv.lengths.cpu().tolist() == [32]
        assert torch.isnan(kv.cache_view()[:, :, 0, :, 32].float()).all()  # nothing written
        kv.set_lengths([32], st)
        kv.decode_step(tok, tok, st)  # eager: the longer class's kernel
        st.synchronize()
        kv.check(st)
        assert kv.lengths.cpu().tolist() == [33]
        assert torch.isfinite(kv.cache_view()[:, :, 0, :, 32].float()).all()
        assert torch.isfinite(kv.logits(st)).all()
    kv.close()
    model.close()


def test_batched_prefill_past_the_host_lengths_is_reported():
    """ds_prefill_batched sizes each pass's attention launch to the
    64-position chunks up to the pass's last position as the host recorded
    the sequence's length.  Replays of a captured decode step move the
    device's length on without the host: a batched prefill whose positions
    then fall in a chunk the launch does not cover trips the launch-shape
    guard (DS_ERR_DEVICE at the next check).  With the lengths set in step
    again, the same prefill passes the check."""
    torch = _torch()
    import decode_step_02_amd as dsa
    w = synth.WORKLOADS["llama135m_p5"]
    arena = synth.make_arena(w.model, w.model_seed)
    model = dsa.Model(w.model, arena)
    kv = dsa.KVCache(model, 1, w.ctx)
    prompt = [int(t) for t in synth.random_tokens(78, 60, w.model.vocab_size)]
    extra = [int(t) for t in synth.random_tokens(79, 3, w.model.vocab_size)]
    st = torch.cuda.Stream()
    tok = torch.zeros(1, dtype=torch.int32, device="cuda")
    with torch.cuda.stream(st):
        kv.prefill(0, prompt, tok, st)
        st.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=st):
            kv.decode_step(tok, tok, st)  # captured, not run
        kv.set_lengths([60], st)
        st.synchronize()
        for _ in range(4):
            g.replay()  # the device's length 61 .. 64; the host's stays 60
        st.synchronize()
        kv.check(st)
        assert kv.lengths.cpu().tolist() == [64]
        # batched positions 60, 61 for the host (chunk 0), 64, 65 on the device (chunk 1)
        kv.prefill_batched(0, extra, tok, st)
        st.synchronize()
        with pytest.raises(dsa.DSError) as err:
            kv.check(st)
        assert err.value.status == -9  # DS_ERR_DEVICE
        kv.set_lengths([64], st)
        kv.prefill_batched(0, extra, tok, st)
        st.synchronize()
        kv.check(st)
        assert kv.lengths.cpu().tolist() == [67]
        assert torch.isfinite(kv.logits(st)).all()
    kv.close()
    model.close()


FULL_ATTN = {
    # (head_dim, H, Hkv, cache): 64 sequences x Hkv >= 128 (item, group)
    # pairs, so decode steps take the one-block-per-pair attention; the
    # ragged prefill's later passes (fewer sequences) take split-K
    "d64-rep2": (64, 4, 2, "F32"),
    "d64-rep3": (64, 6, 2, "F32"),
    "d64-rep4": (64, 8, 2, "F32"),
    "d128-rep4": (128, 8, 2, "F32"),
    "d128-rep1": (128, 2, 2, "F32"),
    "d64-rep3-bf16": (64, 6, 2, "BF16"),
    "d128-rep2-bf16": (128, 4, 2, "BF16"),
}


@pytest.mark.parametrize("name", list(FULL_ATTN))
def test_one_block_per_pair_attention(name, monkeypatch):
    """k_attn_full (DS_ATTN_FULL=1): each (sequence, key/value group) in one
    block, waves walking 16-position runs with an online softmax, merged once
    in LDS.
    Lengths 1 (one wave, one run), 15..17, 255..257 (one and two runs per
    wave), up to 700, and one sequence of 1100 positions (five runs on some
    waves)."""
    monkeypatch.setenv("DS_ATTN_FULL", "1")  # read when the cache is created
    D, H, Hkv, cdt = FULL_ATTN[name]
    shape = synth.small_shape(dim=128, n_heads=H, n_kv_heads=Hkv, head_dim=D, hidden_dim=192, vocab_size=256,
                              cache_dtype=getattr(synth, cdt))
    arena = synth.make_arena(shape, 41, std=0.1, gain_sigma=0.1)
    rng = np.random.default_rng(42)
    lens = [1, 15, 16, 17, 255, 256, 257, 1100] + [int(n) for n in rng.integers(1, 700, 56)]
    prompts = [synth.random_tokens(900 + b, n, shape.vocab_size) for b, n in enumerate(lens)]
    _say(f"one block per pair {name}: B=64 longest {max(lens)}")
    compare(shape, arena, prompts, 3, 1104, f"one block per pair {name}", fast=True)


def test_batch1_multi_chunk_attention_tiny():
    """Batch-1 steps past 32 positions merge per-chunk attention partials
    (positions 70..99 span three and four 32-position chunks)."""
    shape = synth.TINY
    arena = synth.make_arena(shape, 12, std=0.15, gain_sigma=0.1)
    prompts = [synth.random_tokens(500, 70, shape.vocab_size)]
    compare(shape, arena, prompts, 30, 128, "tiny B=1 multi-chunk")


def test_batch1_multi_chunk_attention_135m():
    w = synth.WORKLOADS["llama135m_p5"]
    arena = synth.make_arena(w.model, w.model_seed)
    prompts = [synth.random_tokens(501, 40, w.model.vocab_size)]
    compare(w.model, arena, prompts, 6, w.ctx, "135m B=1 positions 40..45")


def test_batch1_single_launch_matches_per_operation_launches(monkeypatch):
    """The single-launch batch-1 step and the one-launch-per-operation path
    (DS_PERSIST=0) give the same greedy tokens and logits within tolerance."""
    shape = synth.TINY
    arena = synth.make_arena(shape, 13, std=0.15, gain_sigma=0.1)
    prompts = [synth.random_tokens(502, 30, shape.vocab_size)]
    feed = [[int(t)] for t in synth.random_tokens(503, 12, shape.vocab_size)]
    a = gpu_run(shape, arena, prompts, feed, 128)
    monkeypatch.setenv("DS_PERSIST", "0")
    b = gpu_run(shape, arena, prompts, feed, 128)
    assert np.array_equal(a["first_tok"], b["first_tok"])
    assert_logits_close(a["first_lg"], b["first_lg"], "first")
    for k in range(len(feed)):
        assert_logits_close(a["lgs"][k], b["lgs"][k], f"step {k}")
    n = len(prompts[0]) + len(feed)
    assert_logits_close(a["cache"][:, :, 0, :, :n], b["cache"][:, :, 0, :, :n], "cache")


def test_single_launch_several_partials_135m(monkeypatch):
    """Past 128 positions the single launch's attention blocks each fold four
    32-position chunks into one partial and the Wo blocks merge the partials:
    positions 157..168 span five and six chunks, so the second partial holds
    one or two of them.  Checked against the per-operation launches, which
    the oracle pins at 1000 positions."""
    _torch()
    w = synth.WORKLOADS["llama135m_p5"]
    arena = synth.make_arena(w.model, w.model_seed)
    prompts = [synth.random_tokens(504, 157, w.model.vocab_size)]
    feed = [[int(t)] for t in synth.random_tokens(505, 12, w.model.vocab_size)]
    a = gpu_run(w.model, arena, prompts, feed, w.ctx)
    assert a["single_launch_ctx"] >= 169
    monkeypatch.setenv("DS_PERSIST", "0")
    b = gpu_run(w.model, arena, prompts, feed, w.ctx)
    for k in range(len(feed)):
        assert_logits_close(a["lgs"][k], b["lgs"][k], f"step {k}")
        check_tokens(a["toks"][k], b["toks"][k], b["lgs"][k], a["lgs"][k], f"step {k}")
    n = len(prompts[0]) + len(feed)
    assert_logits_close(a["cache"][:, :, 0, :, :n], b["cache"][:, :, 0, :, :n], "cache")


def test_single_launch_step_is_taken_at_batch_1():
    """Batch-1 caches of the instantiated shape classes run their steps as one
    launch (so the parity cases above exercise it); larger batches do not."""
    _torch()
    import decode_step_02_amd as dsa
    w = synth.WORKLOADS["llama135m_p5"]
    model = dsa.Model(w.model, synth.make_arena(w.model, w.model_seed))
    kv = dsa.KVCache(model, 1, w.ctx)
    assert kv.single_launch_ctx() == 1024  # the whole context (up to 2048 fit)
    kv.close()
    kv = dsa.KVCache(model, 2, 64)
    assert kv.single_launch_ctx() == 0
    kv.close()
    model.close()
    tiny = dsa.Model(synth.TINY, synth.make_arena(synth.TINY, 1))
    kv = dsa.KVCache(tiny, 1, 128)
    assert kv.single_launch_ctx() == 128
    kv.close()
    tiny.close()
