"""Pins of the oracle's block-quantised int8 and int4 weights (ORC_Q8, ORC_Q4),
independent of the oracle's own code.

The pages name INT8 weight loading, block-quantised as in GGUF, as the next
step ("simple-llm / kasahare" PyPI README 0.4.0, section "Where to go from
here") without fixing a format.  The reading used here: a matrix [rows][cols]
is int8 values q, then (from the next 256-byte boundary) one fp32 scale per
32 consecutive values of a row, and element (r, c) is s[r][c/32] * q[r][c].

- hand-built blocks: the element values in closed form, including the sign
  of negative int8 values and the scale of the second block of a row;
- the arena layout: the oracle's tensor offsets equal the input generator's
  (two independent writings of the layout above);
- an exact pair: a bf16 model whose every weight is k / 4096 (|k| <= 127) and
  the Q8 model with q = k and s = 2^-12 hold the same weights, so the Q8
  forward pass must equal the (pinned) bf16 forward pass bit for bit;
- the input quantiser (the generator, not the oracle) keeps every weight
  within half a step of its block's scale.
The same pins hold the 4-bit reading (the section also names INT4): values
packed two per byte, the even index in the low nibble, two's complement in
[-8, 7], the scales as for int8; its exact pair uses the grid k / 512,
|k| <= 7.
"""
import ctypes as C
import dataclasses

import numpy as np
import pytest

import oracle
import synth

Q8_SHAPE = synth.small_shape(weight_dtype=synth.Q8, hidden_dim=192)


def _weight(buf, rows, cols, r, c):
    return oracle.lib().orc_weight(buf.ctypes.data_as(C.c_void_p), oracle.ORC_Q8,
                                   rows, cols, r, c)


def test_hand_built_blocks():
    rows, cols = 2, 64
    q = np.zeros((rows, cols), np.int8)
    q[0, :4] = [1, -1, 127, -127]
    q[0, 32] = 5
    q[1, 63] = -3
    sc = np.array([[0.5, 0.25], [2.0, -1.5]], np.float32)
    buf = np.zeros(256 + sc.nbytes, np.uint8)  # 128 int8 values, padded to 256 bytes, then the scales
    buf[:rows * cols] = q.view(np.uint8).reshape(-1)
    buf[256:] = sc.view(np.uint8).reshape(-1)
    got = [_weight(buf, rows, cols, 0, c) for c in range(4)]
    assert got == [0.5, -0.5, 63.5, -63.5]
    assert _weight(buf, rows, cols, 0, 32) == 1.25  # second block of row 0
    assert _weight(buf, rows, cols, 1, 63) == 4.5   # -3 * -1.5
    assert _weight(buf, rows, cols, 1, 0) == 0.0


def test_layout_matches_the_generator():
    for shape in (Q8_SHAPE, dataclasses.replace(Q8_SHAPE, tied_embeddings=0)):
        off, total = oracle.tensor_offsets(shape)
        table, gtotal = synth.tensor_table(shape)
        assert off == [o for _, o, _, _ in table]
        assert total == gtotal
        q_rows = shape.n_heads * shape.head_dim
        # wq of layer 0: values, pad to 256, then rows * cols / 32 scales
        wq_bytes = (q_rows * shape.dim + 255) // 256 * 256 + 4 * q_rows * shape.dim // 32
        assert off[3] - off[2] == (wq_bytes + 255) // 256 * 256


@pytest.mark.parametrize("tied", [1, 0])
def test_exact_pair_equals_bf16_bit_for_bit(tied):
    q8 = dataclasses.replace(Q8_SHAPE, tied_embeddings=tied)
    bf = dataclasses.replace(q8, weight_dtype=synth.BF16)
    a_q8 = synth.make_arena(q8, 31, exact=True, gain_sigma=0.1)
    a_bf = synth.make_arena(bf, 31, exact=True, gain_sigma=0.1)
    vq, vb = synth.views(q8, a_q8), synth.views(bf, a_bf)
    k = vq["l0.w2"].astype(np.float32) * vq["l0.w2.scale"].repeat(32, axis=1)
    assert np.array_equal(k, (vb["l0.w2"].astype(np.uint32) << 16).view(np.float32))
    prompt = synth.random_tokens(32, 6, q8.vocab_size)
    mq = oracle.Model(q8, a_q8, 1, 16)
    mb = oracle.Model(bf, a_bf, 1, 16)
    for pos, t in enumerate(prompt):
        tq, lq = mq.forward(0, pos, int(t))
        tb, lb = mb.forward(0, pos, int(t))
        assert tq == tb
        assert np.array_equal(lq.view(np.uint32), lb.view(np.uint32)), f"position {pos}"
    assert np.array_equal(mq.cache.view(np.uint32), mb.cache.view(np.uint32))


def test_exact_pair_logits_differ_from_a_plain_quantised_model():
    """The Q8 path reads the scales: the quantised N(0, 0.02) model (its own
    scales per block) gives logits near, not equal to, the exact-grid ones."""
    a = synth.make_arena(Q8_SHAPE, 33)
    m = oracle.Model(Q8_SHAPE, a, 1, 8)
    _, lg = m.forward(0, 0, 5)
    assert np.all(np.isfinite(lg)) and np.abs(lg).max() > 0


def test_input_quantiser_error_bound():
    rng = np.random.default_rng(34)
    w = (rng.standard_normal(32 * 500) * 0.02).astype(np.float32)
    w[:32] = 0.0  # an all-zero block
    q, sc = synth.quantize_q8(w)
    b = w.reshape(-1, 32)
    deq = q.reshape(-1, 32).astype(np.float64) * sc[:, None]
    assert np.all(np.abs(deq - b) <= sc[:, None] * (0.5 + 1e-6))
    assert np.all(np.abs(q.reshape(-1, 32)[1:]).max(axis=1) == 127)
    assert np.all(q[:32] == 0)


# ---- 4-bit values (ORC_Q4): two per byte, even index in the low nibble ----

Q4_SHAPE = synth.small_shape(weight_dtype=synth.Q4, hidden_dim=192)


def _weight4(buf, rows, cols, r, c):
    return oracle.lib().orc_weight(buf.ctypes.data_as(C.c_void_p), oracle.ORC_Q4, rows, cols, r, c)


def test_q4_hand_built_blocks():
    rows, cols = 2, 64
    q = np.zeros((rows, cols), np.int8)
    q[0, :4] = [1, -1, 7, -8]
    q[0, 33] = 5   # odd index (high nibble) in the second block
    q[1, 62] = -3
    sc = np.array([[0.5, 0.25], [2.0, -1.5]], np.float32)
    packed = synth.pack_q4(q.reshape(-1))
    assert packed[0] == 0xF1 and packed[1] == 0x87  # (1, -1) and (7, -8): low nibble first
    buf = np.zeros(256 + sc.nbytes, np.uint8)  # 64 bytes of values, padded to 256, then the scales
    buf[:packed.size] = packed
    buf[256:] = sc.view(np.uint8).reshape(-1)
    assert [_weight4(buf, rows, cols, 0, c) for c in range(4)] == [0.5, -0.5, 3.5, -4.0]
    assert _weight4(buf, rows, cols, 0, 33) == 1.25
    assert _weight4(buf, rows, cols, 1, 62) == 4.5
    assert _weight4(buf, rows, cols, 1, 63) == 0.0


def test_q4_layout_matches_the_generator():
    off, total = oracle.tensor_offsets(Q4_SHAPE)
    table, gtotal = synth.tensor_table(Q4_SHAPE)
    assert off == [o for _, o, _, _ in table] and total == gtotal


@pytest.mark.parametrize("tied", [1, 0])
def test_q4_exact_pair_equals_bf16_bit_for_bit(tied):
    q4 = dataclasses.replace(Q4_SHAPE, tied_embeddings=tied)
    bf = dataclasses.replace(q4, weight_dtype=synth.BF16)
    a_q4 = synth.make_arena(q4, 35, exact="q4", gain_sigma=0.1)
    a_bf = synth.make_arena(bf, 35, exact="q4", gain_sigma=0.1)
    prompt = synth.random_tokens(36, 6, q4.vocab_size)
    mq = oracle.Model(q4, a_q4, 1, 16)
    mb = oracle.Model(bf, a_bf, 1, 16)
    for pos, t in enumerate(prompt):
        tq, lq = mq.forward(0, pos, int(t))
        tb, lb = mb.forward(0, pos, int(t))
        assert tq == tb
        assert np.array_equal(lq.view(np.uint32), lb.view(np.uint32)), f"position {pos}"
    assert np.array_equal(mq.cache.view(np.uint32), mb.cache.view(np.uint32))


def test_q4_input_quantiser_error_bound():
    rng = np.random.default_rng(37)
    w = (rng.standard_normal(32 * 300) * 0.02).astype(np.float32)
    packed, sc = synth.quantize_q4(w)
    lo = (packed & 15).astype(np.int16)
    hi = (packed >> 4).astype(np.int16)
    q = np.empty(w.size, np.int16)
    q[0::2], q[1::2] = lo, hi
    q = np.where(q >= 8, q - 16, q)
    deq = q.reshape(-1, 32).astype(np.float64) * sc[:, None]
    assert np.all(np.abs(deq - w.reshape(-1, 32)) <= sc[:, None] * (0.5 + 1e-6))
    assert np.all(np.abs(q.reshape(-1, 32)).max(axis=1) == 7)
