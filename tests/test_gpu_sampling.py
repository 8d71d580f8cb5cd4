"""GPU top-k / temperature sampling inside the monokernel against the CPU sampling oracle.

The monokernel draws each token itself (every workgroup merges the per-workgroup
top-k lists, computes the same Philox4x32-10 uniform and picks by the inverse-CDF
rule).  Each step's draw is checked against ``oracle.sampling.sample`` applied to
that step's GPU logits (float64) with the oracle's own Philox uniform for the
position the step consumes: the model arithmetic is checked against the decoder
oracle elsewhere, here the choice is.  The GPU weighs candidates in fp32 and
takes u = floor(word / 2^8) / 2^24, so a draw whose running sum lies within
1e-5 (relative) of u * total, or whose k-th and (k+1)-th logits are within
1e-5, could go either way; those draws are skipped (and counted).
"""
import os

import numpy as np
import pytest

import decode_megakernel_wave_amd as mk
from decode_megakernel_wave_amd import inputs
from gpu_util import load
from oracle import sampling as osamp

pytestmark = pytest.mark.gpu

AMBIGUOUS = 1e-5
P, N = 32, 16


def _sampled_run(model, w, ids, n, top_k, temperature, seed, **opts):
    ctx = load(mk, model, w, len(ids) + n + 1, **opts)
    try:
        mk.mk_set_sampling(ctx, top_k, temperature, seed)
        t0 = mk.mk_prefill(ctx, ids)
        toks, logits = mk.mk_decode(ctx, n, vocab=model.vocab)
        sent = mk.mk_count_sentinels(ctx)
        # t0 again: rewind to the last prompt position and decode it once with logits
        mk.mk_rewind(ctx, len(ids) - 1)
        t0b, l0 = mk.mk_decode(ctx, 1, vocab=model.vocab)
    finally:
        mk.mk_destroy(ctx)
    return t0, toks, logits, sent, int(t0b[0]), l0[0]


def _check_draws(tokens, logits, positions, top_k, temperature, seed):
    compared = 0
    for tok, z, p in zip(tokens, logits, positions):
        z = z.astype(np.float64)
        u = osamp.uniform(seed, int(p))
        want, cand, _, _ = osamp.sample(z, top_k, temperature, u)
        assert int(tok) in set(cand.tolist()), f"position {p}: token {tok} not among the top-{top_k}"
        if osamp.draw_ambiguity(z, top_k, temperature, u) <= AMBIGUOUS:
            continue
        assert int(tok) == want, f"position {p}: GPU drew {tok}, oracle {want} (u={u:.6f})"
        compared += 1
    return compared


@pytest.fixture(scope="module")
def tiny():
    w = inputs.make_weights(inputs.TINY, seed=0)
    ids = inputs.make_prompt(inputs.TINY, P, seed=1)
    return w, ids


@pytest.mark.parametrize("top_k,temperature,seed", [(2, 1.0, 7), (8, 0.7, 1234), (16, 1.5, 2**40 + 3)])
def test_tiny_draws_match_the_oracle(tiny, top_k, temperature, seed):
    w, ids = tiny
    t0, toks, logits, sent, t0b, l0 = _sampled_run(inputs.TINY, w, ids, N, top_k, temperature, seed)
    assert sent == 0
    assert t0 == t0b  # the prompt's last step draws the same token with the same logits and counter
    n = _check_draws(toks, logits, P + np.arange(N), top_k, temperature, seed)
    n += _check_draws([t0b], [l0], [P - 1], top_k, temperature, seed)
    assert n >= N - 2, f"only {n} of {N + 1} draws were unambiguous"
    # the draws are not all the greedy choice (the tiny model's logits are close together)
    assert np.any(toks != np.argmax(logits, axis=-1))


def test_top1_is_greedy(tiny):
    w, ids = tiny
    t0, toks, logits, sent, _, _ = _sampled_run(inputs.TINY, w, ids, N, 1, 0.5, 99)
    assert sent == 0
    assert np.array_equal(toks, np.argmax(logits, axis=-1))


def test_seeded_runs_repeat_and_seeds_differ(tiny):
    w, ids = tiny
    a = _sampled_run(inputs.TINY, w, ids, N, 16, 1.0, 5)[1]
    b = _sampled_run(inputs.TINY, w, ids, N, 16, 1.0, 5)[1]
    c = _sampled_run(inputs.TINY, w, ids, N, 16, 1.0, 6)[1]
    assert np.array_equal(a, b)
    assert not np.array_equal(a, c)


def test_counter_mode_draws_the_same_tokens(tiny):
    w, ids = tiny
    s = _sampled_run(inputs.TINY, w, ids, N, 8, 0.9, 42)
    c = _sampled_run(inputs.TINY, w, ids, N, 8, 0.9, 42, sync_mode=mk.MK_SYNC_COUNTER)
    assert s[0] == c[0] and np.array_equal(s[1], c[1])
    assert np.array_equal(s[2].view(np.uint32), c[2].view(np.uint32))


def test_half_billion_model_draws_match(tiny):
    cfg = inputs.M05
    w = inputs.make_weights(cfg, seed=0)
    ids = inputs.make_prompt(cfg, 16, seed=1)
    t0, toks, logits, sent, t0b, l0 = _sampled_run(cfg, w, ids, 8, 16, 1.0, 77)
    assert sent == 0 and t0 == t0b
    n = _check_draws(toks, logits, 16 + np.arange(8), 16, 1.0, 77)
    assert n >= 6


def test_long_context_kernel_draws_match_and_equal_the_general_kernel():
    """Top-16 sampling on the ~2B geometry (2 layers) after a 1100-token prompt: every split is
    longer than 32 positions, so the long-context kernel (DMA-fed K/V rings) draws the tokens;
    the draws match the oracle's choice on its logits, and the general kernel draws the same
    tokens from bitwise the same logits."""
    cfg = inputs.M2B_GEOM_L2
    w = inputs.make_weights(cfg, seed=0)
    ids = inputs.make_prompt(cfg, 1100, seed=2)
    n, top_k, temperature, seed = 6, 16, 1.0, 91
    ctx = load(mk, cfg, w, len(ids) + n + 1)
    try:
        mk.mk_set_sampling(ctx, top_k, temperature, seed)
        mk.mk_prefill(ctx, ids)
        toks, logits = mk.mk_decode(ctx, n, vocab=cfg.vocab)
        assert mk.mk_kernel_name(ctx) == "mk_monokernel_w4h128_long"
        sent = mk.mk_count_sentinels(ctx)
        mk.mk_rewind(ctx, len(ids))
        os.environ["MK_GENERAL_KERNEL"] = "1"
        try:
            g_toks, g_logits = mk.mk_decode(ctx, n, vocab=cfg.vocab)
        finally:
            del os.environ["MK_GENERAL_KERNEL"]
    finally:
        mk.mk_destroy(ctx)
    assert sent == 0
    assert np.array_equal(g_toks, toks)
    assert np.array_equal(g_logits.view(np.uint32), logits.view(np.uint32))
    assert _check_draws(toks, logits, len(ids) + np.arange(n), top_k, temperature, seed) >= n - 1


def test_invalid_sampling_arguments(tiny):
    w, ids = tiny
    ctx = load(mk, inputs.TINY, w, P + 4)
    try:
        for k, t in [(0, 1.0), (17, 1.0), (4, 0.0), (4, -1.0), (4, float("inf")), (4, float("nan"))]:
            with pytest.raises(mk.MkError) as e:
                mk.mk_set_sampling(ctx, k, t, 1)
            assert e.value.code == mk.MK_EINVAL
        mk.mk_set_sampling(ctx, 1, 0.0, 1)  # temperature is ignored for greedy
        assert mk.mk_prefill(ctx, ids) >= 0
    finally:
        mk.mk_destroy(ctx)


def test_generate_and_chunked_decode_draw_the_same_sequence(tiny):
    """mk_generate (prefill + one decode launch) and prefill + two decode launches of half the
    steps draw the same tokens: the Philox counter is the position, not the launch step."""
    w, ids = tiny
    ctx = load(mk, inputs.TINY, w, P + N + 1)
    try:
        mk.mk_set_sampling(ctx, 8, 1.0, 321)
        gen = mk.mk_generate(ctx, ids, N)
        t0 = mk.mk_prefill(ctx, ids)
        a = mk.mk_decode(ctx, N // 2)
        b = mk.mk_decode(ctx, N - N // 2)
    finally:
        mk.mk_destroy(ctx)
    assert gen[0] == t0
    assert np.array_equal(gen[1:], np.concatenate([a, b]))
