"""Hand-derived values (tests/golden/derived_values.json) against the oracle, the input
generator and the schedule's byte accounting."""
import json
import math
import os

import numpy as np
import pytest

import decode_megakernel_wave_amd as mk
from decode_megakernel_wave_amd import inputs
from oracle import chain as ochain
from oracle import decoder as od

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "derived_values.json")))
MODELS = {"tiny": inputs.TINY, "0.5b": inputs.M05, "2b": inputs.M2B, "2b-tp8-shard": inputs.M2B_TP8}


@pytest.mark.parametrize("name", list(MODELS))
def test_parameter_counts(name):
    assert MODELS[name].n_params() == GOLD["n_params"][name]


@pytest.mark.parametrize("name", list(MODELS))
def test_weight_bytes_of_the_schedule(name):
    w = inputs.WORKLOADS[name]
    info = mk.mk_plan_check(w.model, w.max_seq, 128)
    assert info["weight_bytes"] == GOLD["weight_bytes_per_token"][name]


@pytest.mark.parametrize("name", list(inputs.WORKLOADS))
def test_mean_bytes_per_token(name):
    w = inputs.WORKLOADS[name]
    g = GOLD["mean_bytes_per_token"][name]
    assert (w.prompt_len, w.decode_steps) == (g["P"], g["n"])
    m = w.model
    kv = 2 * m.n_layers * m.n_kv_heads * m.head_dim * 2
    assert kv == GOLD["kv_bytes_per_position"][m.name]
    info = mk.mk_plan_check(m, w.max_seq, 128)
    # the per-launch figure the library reports, summed the same way: step s attends to P + s positions
    total = sum(info["weight_bytes"] + kv * (w.prompt_len + s) for s in range(1, w.decode_steps + 1))
    assert total == g["bytes"] * w.decode_steps


def test_rmsnorm_of_an_embedding_row():
    g = GOLD["rmsnorm_of_embedding_row"]
    x = np.full(2048, math.sqrt(g["m"]))
    x[::2] *= -1
    h = od.rmsnorm(x, np.ones(2048), g["eps"])
    assert abs(np.mean(h * h) - g["mean_h2"]) < 1e-12


def test_rope_frequency():
    g = GOLD["rope_frequency"]
    hd = g["hd"]
    e = np.zeros((1, hd))
    e[0, g["i"]] = 1.0
    r = od.rope_rotate(e, 1, g["theta"])[0]
    assert abs(math.atan2(r[g["i"] + hd // 2], r[g["i"]]) - g["w"]) < 1e-12


def test_chain_gain_of_the_generated_weights():
    g = GOLD["chain_gain"]
    W = inputs.make_chain_weights(g["n"], 2, seed=0).astype(np.float64)
    x = inputs.make_chain_x0(g["n"], seed=2).astype(np.float64)
    y = W[0] @ x
    ratio = np.sqrt(np.mean(y * y) / np.mean(x * x))
    assert abs(ratio - g["gain"]) < 0.03
    # the first stage of the oracle chain is tanh of that product
    ys = ochain.chain(W, x.astype(np.float32))
    assert np.allclose(ys[0], np.tanh(y), atol=1e-6)
