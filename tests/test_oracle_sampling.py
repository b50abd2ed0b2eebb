"""Pins of the oracle's sampling epilogue (orc_sample) to the pages and to
the mathematics, independent of the oracle's own code:

- "Inside nanochat Part 4", section "Top-K Filtering": the worked example
  with probabilities (0.45, 0.30, 0.15, 0.10) and k = 2 renormalises to
  (0.60, 0.40), and the last two tokens are never drawn;
- the same section, "Greedy Decoding": temperature 0 is the argmax;
- temperature scaling in closed form: softmax(l / t) is p^(1/t) renormalised;
- the draw is an inverse distribution function, so a fine uniform grid of
  draws reproduces the probabilities as frequencies;
- the nucleus reading of --top-p ("simple-llm / kasahare", section "CLI
  flags"): the shortest prefix of the sorted candidates whose mass reaches
  top_p.
"""
import numpy as np
import pytest

import oracle

P4 = np.array([0.45, 0.30, 0.15, 0.10])


def _logits(p):
    return np.log(np.asarray(p, np.float64)).astype(np.float32)


def test_top_k_example_of_the_pages():
    lg = _logits(P4)
    tok, cand, cum = oracle.sample(lg, 1.0, 2, 1.0, 0.0)
    assert cand.tolist() == [0, 1]
    assert np.allclose(cum, [0.60, 1.00], atol=1e-7)
    drawn = {oracle.sample(lg, 1.0, 2, 1.0, u)[0] for u in np.linspace(0, 0.999, 1000)}
    assert drawn == {0, 1}  # "table" and "car" have zero probability
    assert oracle.sample(lg, 1.0, 2, 1.0, 0.599)[0] == 0
    assert oracle.sample(lg, 1.0, 2, 1.0, 0.601)[0] == 1


def test_greedy_is_the_argmax_lowest_index_on_ties():
    lg = np.array([0.1, 2.0, -1.0, 2.0], np.float32)
    for u in (0.0, 0.5, 0.99):
        assert oracle.sample(lg, 0.0, 0, 1.0, u)[0] == 1
        assert oracle.sample(lg, 0.0, 3, 0.5, u)[0] == 1


@pytest.mark.parametrize("t", [0.5, 0.7, 1.0, 1.5])
def test_temperature_closed_form(t):
    p = np.array([0.1, 0.2, 0.3, 0.4])
    q = p ** (1.0 / t)
    q /= q.sum()
    _, cand, cum = oracle.sample(_logits(p), t, 0, 1.0, 0.0)
    assert cand.tolist() == [0, 1, 2, 3]  # top_k 0: index order
    assert np.allclose(cum, np.cumsum(q), atol=1e-6)
    _, cand, cum = oracle.sample(_logits(p), t, 4, 1.0, 0.0)
    assert cand.tolist() == [3, 2, 1, 0]  # top_k: largest first
    assert np.allclose(cum, np.cumsum(q[::-1]), atol=1e-6)


@pytest.mark.parametrize("k", [0, 3, 5])
def test_draws_reproduce_the_distribution(k):
    rng = np.random.default_rng(11)
    lg = rng.standard_normal(5).astype(np.float32)
    t = 0.8
    order = np.argsort(-lg.astype(np.float64), kind="stable") if k else np.arange(5)
    keep = order[:k] if k else order
    w = np.exp((lg[keep].astype(np.float64) - lg.max()) / t)
    want = w / w.sum()
    n = 20000
    counts = np.zeros(5)
    for u in (np.arange(n) + 0.5) / n:
        counts[oracle.sample(lg, t, k, 1.0, u)[0]] += 1
    assert np.allclose(counts[keep] / n, want, atol=2.0 / n)
    assert counts.sum() == counts[keep].sum()


def test_top_p_nucleus_reading():
    lg = _logits(P4)
    # 0.45 + 0.30 = 0.75 reaches 0.70 and 0.75: two candidates, as top-k 2
    for tp in (0.70, 0.75):
        _, cand, cum = oracle.sample(lg, 1.0, 4, tp, 0.0)
        assert cand.tolist() == [0, 1] and np.allclose(cum, [0.6, 1.0], atol=1e-6)
    _, cand, cum = oracle.sample(lg, 1.0, 4, 0.76, 0.0)
    assert cand.tolist() == [0, 1, 2] and np.allclose(cum, [0.5, 0.75 / 0.9, 1.0], atol=1e-6)
    _, cand, _ = oracle.sample(lg, 1.0, 4, 0.40, 0.9)  # the first candidate alone reaches 0.40
    assert cand.tolist() == [0]


def test_equal_logits_sort_by_index_and_k_above_v():
    lg = np.array([1.0, 3.0, 1.0, 3.0, 0.0], np.float32)
    _, cand, cum = oracle.sample(lg, 1.0, 10, 1.0, 0.0)
    assert cand.tolist() == [1, 3, 0, 2, 4]
    assert cum[-1] == 1.0 and np.all(np.diff(cum) > 0)


def test_large_temperature_flattens():
    lg = np.array([5.0, 0.0, -5.0], np.float32)
    _, _, cum = oracle.sample(lg, 1e6, 0, 1.0, 0.0)
    assert np.allclose(cum, [1 / 3, 2 / 3, 1.0], atol=1e-4)


@pytest.mark.parametrize("args", [(-1.0, 0, 1.0, 0.5), (1.0, -1, 1.0, 0.5), (1.0, 0, 0.9, 0.5),
                                  (1.0, 2, 0.0, 0.5), (1.0, 2, 1.0, 1.0), (1.0, 2, 1.5, 0.5)])
def test_bad_arguments(args):
    with pytest.raises(ValueError):
        oracle.sample(np.zeros(4, np.float32), *args)
