"""Pins of the sampling oracle (top-k / temperature draw, Philox4x32-10).

- The generator against the published known-answer vectors (tests/golden).
- The draw against closed forms: on a fine grid of u the share of draws that
  pick each candidate equals its softmax probability restricted to the top k;
  k = 1 and a vanishing temperature give the argmax; candidates are ordered by
  logit with ties to the lower index; nothing outside the top k is drawn.
- Planted mistakes in copies of the oracle are rejected by these pins.
"""
import json
import os

import numpy as np
import pytest

from oracle import sampling as osm

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.json")


def check_philox(fn) -> bool:
    with open(GOLDEN) as f:
        vecs = json.load(f)["vectors"]
    return all(fn([int(x, 16) for x in v["counter"]], [int(x, 16) for x in v["key"]]) ==
               [int(x, 16) for x in v["out"]] for v in vecs)


def test_philox_known_answers():
    assert check_philox(osm.philox4x32_10)


def test_uniform_pinned_to_first_known_answer_vector():
    # seed 0 is key (0, 0) and position 0 is counter (0, 0, 0, 0): the first published
    # known-answer vector, whose first output word is the uniform's numerator
    with open(GOLDEN) as f:
        kat = json.load(f)["vectors"][0]
    assert kat["counter"] == ["00000000"] * 4 and kat["key"] == ["00000000"] * 2
    assert osm.uniform(0, 0) == int(kat["out"][0], 16) / 2.0 ** 32
    assert osm.uniform(0, 0) == 0x6627E8D5 / 2.0 ** 32


def test_uniform_range_and_inputs():
    us = [osm.uniform(1234, p) for p in range(200)]
    assert all(0.0 <= u < 1.0 for u in us)
    assert len(set(us)) == len(us)                         # the position is part of the counter
    assert osm.uniform(1234, 5) != osm.uniform(1234 + (1 << 32), 5)  # both key words matter
    assert abs(np.mean(us) - 0.5) < 0.06


def check_draw(fn_sample) -> bool:
    """Inverse-CDF draw vs closed-form probabilities on a grid of u."""
    z = np.array([0.3, 2.0, -1.0, 2.0, 1.1, 0.9])
    ok = True
    for k, t in ((4, 0.8), (6, 1.7), (2, 0.3)):
        order = np.lexsort((np.arange(z.size), -z))[:k]
        p = np.exp((z[order] - z[order].max()) / t)
        p /= p.sum()
        n = 20000
        counts = {}
        for j in range(n):
            tok = fn_sample(z, k, t, (j + 0.5) / n)[0]
            counts[tok] = counts.get(tok, 0) + 1
        ok &= set(counts) <= set(order.tolist())
        ok &= all(abs(counts.get(int(i), 0) / n - pi) <= 2.0 / n for i, pi in zip(order, p))
    return bool(ok)


def test_draw_matches_softmax_on_the_top_k():
    assert check_draw(osm.sample)


def test_greedy_limits():
    rng = np.random.default_rng(0)
    for _ in range(20):
        z = rng.standard_normal(50)
        u = rng.random()
        assert osm.sample(z, 1, 1.0, u)[0] == int(np.argmax(z))
        assert osm.sample(z, 10, 1e-6, u)[0] == int(np.argmax(z))
    # equal logits: the lower index comes first
    z = np.array([1.0, 3.0, 3.0, 0.0])
    assert osm.top_k_order(z, 3).tolist() == [1, 2, 0]
    assert osm.sample(z, 1, 1.0, 0.9)[0] == 1


def test_ambiguity_measure():
    z = np.array([1.0, 1.0 + 1e-9, -5.0])
    assert osm.draw_ambiguity(z, 1, 1.0, 0.3) < 1e-8       # near-tie at the top-k boundary
    z = np.array([0.0, 0.0, -50.0])                        # two equal weights: boundary at u = 0.5
    assert osm.draw_ambiguity(z, 2, 1.0, 0.5) < 1e-12


# ---------------------------------------------------------------- planted mistakes
def _philox_wrong_multiplier(counter, key):
    c = list(counter)
    k = list(key)
    for r in range(10):
        if r:
            k = [(k[0] + osm.PHILOX_W0) & osm.MASK32, (k[1] + osm.PHILOX_W1) & osm.MASK32]
        p0 = 0xD2511F55 * c[0]
        p1 = osm.PHILOX_M1 * c[2]
        c = [(p1 >> 32) ^ c[1] ^ k[0], p1 & osm.MASK32, (p0 >> 32) ^ c[3] ^ k[1], p0 & osm.MASK32]
    return c


def _philox_no_key_bump(counter, key):
    c = list(counter)
    for _ in range(10):
        p0 = osm.PHILOX_M0 * c[0]
        p1 = osm.PHILOX_M1 * c[2]
        c = [(p1 >> 32) ^ c[1] ^ key[0], p1 & osm.MASK32, (p0 >> 32) ^ c[3] ^ key[1], p0 & osm.MASK32]
    return c


def _sample_no_temperature(z, k, t, u):
    return osm.sample(z, k, 1.0, u)


def _sample_ascending(z, k, t, u):
    return osm.sample(-np.asarray(z), k, t, u)


def _sample_full_vocabulary(z, k, t, u):
    return osm.sample(z, len(z), t, u)


@pytest.mark.parametrize("bad", [_philox_wrong_multiplier, _philox_no_key_bump])
def test_planted_generator_mistakes_are_caught(bad):
    assert not check_philox(bad)


@pytest.mark.parametrize("bad", [_sample_no_temperature, _sample_ascending, _sample_full_vocabulary])
def test_planted_draw_mistakes_are_caught(bad):
    assert not check_draw(bad)
