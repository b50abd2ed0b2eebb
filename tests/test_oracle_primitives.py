"""Pins for the reference decoder's primitives (CPU only).

Each test ties one oracle function to something other than itself: a library
conversion, a float64 evaluation within a proven rounding bound, a closed
form, or a special case that the pages fix.
"""
import math
import os
import subprocess
import tempfile

import numpy as np
import pytest
import torch

import oracle
from conftest import golden

U = 2.0 ** -24  # unit roundoff of binary32


def gamma(n):
    return n * U / (1 - n * U)


def widen_np(u16):
    return (u16.astype(np.uint32) << 16).view(np.float32)


# ---- bf16 widening -----------------------------------------------------------

def test_widen_matches_torch_for_every_bf16_pattern(orc):
    """GOTOken, 'Loading the model and tokenizer': bf16 -> fp32 is a 16-bit
    left shift.  All 65,536 patterns (zeros, subnormals, infinities, NaN
    payloads) against torch's own bfloat16 -> float32 conversion."""
    src = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    out = np.zeros(65536, np.float32)
    orc.orc_widen_bf16_array(src, out, 65536)
    ref = torch.from_numpy(src.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(out.view(np.uint32), ref.view(np.uint32))
    assert orc.orc_widen_bf16(0x3F80) == 1.0
    assert orc.orc_widen_bf16(0xC000) == -2.0


# ---- matvec ------------------------------------------------------------------

@pytest.mark.parametrize("n_out,n_in,bf16", [(576, 576, True), (172, 64, False), (64, 172, False),
                                             (7, 1536, True), (33, 1, False)])
def test_matvec_within_fp64_bound(n_out, n_in, bf16):
    """|y - y64| <= gamma_n * sum|W||x| (Higham's bound for a recursive sum
    of n rounded products), against float64 evaluation of the same product."""
    rng = np.random.default_rng(n_out * 1000 + n_in)
    Wf = (rng.standard_normal((n_out, n_in)) * 0.05).astype(np.float32)
    if bf16:
        W = (Wf.view(np.uint32) >> 16).astype(np.uint16)
        W64 = widen_np(W).astype(np.float64)
    else:
        W, W64 = Wf, Wf.astype(np.float64)
    x = rng.standard_normal(n_in).astype(np.float32)
    y = oracle.matvec(W, x)
    y64 = W64 @ x.astype(np.float64)
    bound = gamma(n_in) * (np.abs(W64) @ np.abs(x.astype(np.float64))) + 1e-300
    assert np.all(np.abs(y.astype(np.float64) - y64) <= bound)


def test_matvec_rounding_order_replay():
    """GOTOken, 'Building it one piece at a time': a replay of the row-major
    loop in fp32 with the same rounding order matches every one of the 576
    query-projection outputs bit for bit.  The replay here sweeps columns in
    numpy, one separately rounded multiply and add per step."""
    g = golden("rounding_order.json")
    n = g["outputs"]
    rng = np.random.default_rng(3)
    W = (rng.standard_normal((n, n)).astype(np.float32) * np.float32(0.02))
    Wb = (W.view(np.uint32) >> 16).astype(np.uint16)
    x = rng.standard_normal(n).astype(np.float32)
    y = oracle.matvec(Wb, x)
    Wf = widen_np(Wb)
    acc = np.zeros(n, np.float32)
    for j in range(n):
        acc = acc + Wf[:, j] * x[j]
    assert int(np.sum(y.view(np.uint32) == acc.view(np.uint32))) == g["sequential_replay_matches"]
    # a replay whose multiply-add is rounded once (float64 product, exact for
    # bf16 x fp32, then one rounding of the sum) must disagree somewhere, as
    # the page's fused replay did
    fma = np.zeros(n, np.float32)
    for j in range(n):
        fma = (fma.astype(np.float64) + Wf[:, j].astype(np.float64) * np.float64(x[j])).astype(np.float32)
    assert int(np.sum(fma.view(np.uint32) == y.view(np.uint32))) < n


def test_contracted_build_differs_from_strict_build():
    """The strict build (-ffp-contract=off) is what makes the replay above
    exact; a copy built with contraction to FMA gives other bits."""
    rng = np.random.default_rng(11)
    W = (rng.standard_normal((576, 576)) * 0.02).astype(np.float32)
    x = rng.standard_normal(576).astype(np.float32)
    strict = oracle.matvec(W, x)
    with tempfile.TemporaryDirectory() as td:
        so = os.path.join(td, "liboracle_fma.so")
        oracle.build(so, ["-ffp-contract=fast", "-mfma", "-O2"])
        lib = oracle.load(so)
        y = np.zeros(576, np.float32)
        lib.orc_matvec(W.ctypes.data, 0, 576, 576, x, y)
    assert not np.array_equal(strict.view(np.uint32), y.view(np.uint32))
    assert np.allclose(strict, y, rtol=1e-4, atol=1e-5)


# ---- RMSNorm ----------------------------------------------------------------

@pytest.mark.parametrize("n,c,gain", [(64, 0.5, 1.5), (576, -0.75, 1.0), (4096, 0.125, 0.5)])
def test_rmsnorm_constant_vector_closed_form(n, c, gain):
    """x = c * ones gives y = g * c / sqrt(c^2 + eps) exactly; the oracle is
    within five roundings of it."""
    eps = 1e-5
    x = np.full(n, c, np.float32)
    g = np.full(n, gain, np.float32)
    y = oracle.rmsnorm(x, g, eps)
    exact = gain * c / np.sqrt(c * c + np.float64(np.float32(eps)))
    assert np.all(np.abs(y.astype(np.float64) - exact) <= 3 * U * abs(exact))


def test_rmsnorm_random_against_fp64():
    rng = np.random.default_rng(5)
    for n in (64, 576, 1536):
        x = rng.standard_normal(n).astype(np.float32)
        g = (1 + 0.1 * rng.standard_normal(n)).astype(np.float32)
        eps = np.float32(1e-5)
        y = oracle.rmsnorm(x, g, eps)
        x64 = x.astype(np.float64)
        ref = g.astype(np.float64) * x64 / np.sqrt(np.mean(x64 * x64) + np.float64(eps))
        assert np.max(np.abs(y - ref) / np.abs(ref).max()) < (n + 8) * U


# ---- RoPE -------------------------------------------------------------------

@pytest.mark.parametrize("D,theta", [(16, 1e4), (64, 1e5), (128, 5e5)])
def test_rope_identity_at_position_zero(D, theta):
    rng = np.random.default_rng(D)
    v = rng.standard_normal(D).astype(np.float32)
    r = oracle.rope_apply(v, 0, theta)
    assert np.array_equal(r.view(np.uint32), v.view(np.uint32))


def test_rope_frequencies_closed_form():
    """Pair i turns by pos * theta^(-2i/D): pair 0 by pos radians exactly, and
    with D=16, theta=1e4 pair 4 by pos/100."""
    for pos in (1, 7, 1000):
        c, s = oracle.rope_angles(pos, 16, 1e4)
        assert c[0] == np.float32(np.cos(float(pos))) and s[0] == np.float32(np.sin(float(pos)))
        ang = pos * 0.01
        assert abs(c[4] - np.cos(ang)) <= 2 * U and abs(s[4] - np.sin(ang)) <= 2 * U
        ang7 = pos * 1e4 ** (-14 / 16)
        assert abs(c[7] - np.cos(ang7)) <= 2 * U and abs(s[7] - np.sin(ang7)) <= 2 * U


def test_rope_pairs_are_rotations():
    """Each pair (v[i], v[i+D/2]) keeps its length, and the score between a
    rotated query at m and key at n depends only on m - n."""
    rng = np.random.default_rng(9)
    D, theta = 64, 1e5
    q = rng.standard_normal(D).astype(np.float32)
    k = rng.standard_normal(D).astype(np.float32)
    r = oracle.rope_apply(q, 37, theta).astype(np.float64)
    h = D // 2
    q64 = q.astype(np.float64)
    assert np.allclose(r[:h] ** 2 + r[h:] ** 2, q64[:h] ** 2 + q64[h:] ** 2, rtol=8 * U, atol=0)
    s1 = oracle.rope_apply(q, 50, theta).astype(np.float64) @ oracle.rope_apply(k, 20, theta)
    s2 = oracle.rope_apply(q, 130, theta).astype(np.float64) @ oracle.rope_apply(k, 100, theta)
    assert abs(s1 - s2) < 1e-4 * np.linalg.norm(q) * np.linalg.norm(k)
    # the rotation direction: for pair 0 at angle a, (1, 0) -> (cos a, sin a)
    e = np.zeros(D, np.float32)
    e[0] = 1
    r = oracle.rope_apply(e, 1, theta)
    assert r[0] == np.float32(np.cos(1.0)) and r[h] == np.float32(np.sin(1.0))


def test_rope_adjacent_pair_convention_with_permuted_rows():
    """GOTOken, 'Loading the model and tokenizer': rotating adjacent pairs
    after reordering the q/k rows gives the same attention scores as rotating
    (j, j+D/2).  Row 2i of the reordered head is row i, row 2i+1 is row
    i+D/2; the adjacent rotation then reproduces the oracle's output in the
    reordered positions bit for bit."""
    rng = np.random.default_rng(21)
    D, theta, pos = 64, 1e5, 29
    q = rng.standard_normal(D).astype(np.float32)
    k = rng.standard_normal(D).astype(np.float32)
    perm = np.empty(D, np.int64)
    perm[0::2] = np.arange(D // 2)
    perm[1::2] = np.arange(D // 2) + D // 2
    c, s = oracle.rope_angles(pos, D, theta)

    def adjacent(v):
        v = v.copy()
        a, b = v[0::2].copy(), v[1::2].copy()
        v[0::2] = a * c - b * s
        v[1::2] = a * s + b * c
        return v

    qa, ka = adjacent(q[perm]), adjacent(k[perm])
    qr, kr = oracle.rope_apply(q, pos, theta), oracle.rope_apply(k, pos, theta)
    assert np.array_equal(qa, qr[perm]) and np.array_equal(ka, kr[perm])
    # fp32 x fp32 products are exact in float64 and fsum is exact, so the
    # scores agree exactly whatever the summation order
    assert math.fsum(qa.astype(np.float64) * ka) == math.fsum(qr.astype(np.float64) * kr)


# ---- attention ----------------------------------------------------------------

def test_attention_single_position_returns_v():
    rng = np.random.default_rng(1)
    for D in (16, 64, 128):
        q = rng.standard_normal(D).astype(np.float32)
        K = rng.standard_normal((1, D)).astype(np.float32)
        V = rng.standard_normal((1, D)).astype(np.float32)
        out, p = oracle.attend(q, K, V)
        assert p[0] == 1.0
        assert np.array_equal(out.view(np.uint32), V[0].view(np.uint32))


def test_attention_zero_query_is_mean():
    rng = np.random.default_rng(2)
    n, D = 37, 64
    K = rng.standard_normal((n, D)).astype(np.float32)
    V = rng.standard_normal((n, D)).astype(np.float32)
    out, p = oracle.attend(np.zeros(D, np.float32), K, V)
    assert np.all(p == np.float32(1.0) / np.float32(n))
    ref = V.astype(np.float64).mean(0)
    assert np.all(np.abs(out - ref) <= gamma(2 * n + 2) * np.abs(V).astype(np.float64).sum(0) / n * 2)


@pytest.mark.parametrize("n,D", [(1, 16), (5, 16), (12, 64), (300, 64), (1025, 128)])
def test_attention_against_fp64(n, D):
    """Softmax weights sum to 1 within 2n roundings, and the output is within
    a rounding bound of the float64 softmax-weighted sum."""
    rng = np.random.default_rng(n + D)
    q = (rng.standard_normal(D) * 2).astype(np.float32)
    K = rng.standard_normal((n, D)).astype(np.float32)
    V = rng.standard_normal((n, D)).astype(np.float32)
    out, p = oracle.attend(q, K, V)
    assert abs(float(np.sum(p.astype(np.float64))) - 1.0) <= 2 * n * U + 1e-7
    s = (K.astype(np.float64) @ q.astype(np.float64)) / np.sqrt(D)
    w = np.exp(s - s.max())
    w /= w.sum()
    ref = w @ V.astype(np.float64)
    assert np.max(np.abs(p - w)) < 1e-6
    assert np.max(np.abs(out - ref)) < 1e-5 * np.abs(V).max()


def test_silu_mul_against_fp64():
    a = np.linspace(-20, 20, 2001).astype(np.float32)
    u = np.float32(1.25)
    lib = oracle.lib()
    got = np.array([lib.orc_silu_mul(float(x), float(u)) for x in a], np.float64)
    a64 = a.astype(np.float64)
    ref = a64 / (1 + np.exp(-a64)) * float(u)
    assert np.all(np.abs(got - ref) <= 6 * U * np.abs(ref) + 1e-30)


# ---- argmax ---------------------------------------------------------------------

def test_argmax_lowest_index_on_ties_and_greedy_example():
    g = golden("greedy_example.json")
    p = np.array(g["probabilities"], np.float32)
    assert g["tokens"][oracle.argmax(p)] == g["greedy_pick"]
    assert oracle.argmax(np.array([1, 3, 3, 2], np.float32)) == 1
    assert oracle.argmax(np.array([-1, -1, -1], np.float32)) == 0
    assert oracle.argmax(np.array([0.0, -0.0, 0.0], np.float32)) == 0
    rng = np.random.default_rng(4)
    for _ in range(50):
        v = rng.integers(-3, 4, size=200).astype(np.float32)
        assert oracle.argmax(v) == int(np.argmax(v)) == int(torch.argmax(torch.from_numpy(v)))
