"""Long context: the 8192-token prompt of the long-context workload.

- The tiny decoder with an 8192-token prompt against the oracle: the split
  attention (S splits per kv head merged inside the attention stage) over the
  full context length, with the chosen split count and with 16 and 64.
- The ~2B decoder with an 8192-token prompt (the long-context benchmark's own
  shape): the oracle cannot prefill 8192 tokens of the 2B model in float64 in
  test time, so this checks what holds at any size -- every step's logits are
  finite, no sentinel survives, one launch of 8 steps equals two launches of 4
  bit for bit, and the greedy tokens are the argmax of the logits.
"""
import numpy as np
import pytest
import torch

import decode_megakernel_wave_amd as mk
from decode_megakernel_wave_amd import inputs
from gpu_util import MARGIN, check_step_logits, oracle_run

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

P_LONG = 8192


@pytest.fixture(scope="module")
def tiny_long():
    cfg = inputs.TINY
    w = inputs.make_weights(cfg, seed=0)
    ids = inputs.make_prompt(cfg, P_LONG, seed=1)
    t0, toks, logs, _, m0 = oracle_run(cfg, w, ids, 4)
    return cfg, w, ids, t0, toks, logs, m0


@pytest.mark.parametrize("splits", [0, 16, 64])
def test_tiny_long_context_parity(tiny_long, splits):
    cfg, w, ids, t0_ref, toks_ref, logs_ref, m0 = tiny_long
    opts = mk.mk_default_options(attn_splits=splits)
    ctx = mk.mk_create(cfg, max_seq=P_LONG + 5, opts=opts)
    try:
        mk.mk_load_weights(ctx, mk.to_device(w))
        t0 = mk.mk_prefill(ctx, ids)
        feed = np.concatenate([[t0_ref], toks_ref[:-1]])
        toks, logits = mk.mk_decode_forced(ctx, feed, vocab=cfg.vocab)
        sent = mk.mk_count_sentinels(ctx)
    finally:
        mk.mk_destroy(ctx)
    err = check_step_logits(logits, logs_ref, toks, toks_ref)
    print(f"tiny P=8192 splits={splits}: max |dlogit| {err:.2e}")
    if m0 > MARGIN:
        assert t0 == t0_ref
    assert sent == 0


def test_2b_long_context_consistency():
    model = inputs.M2B
    w = inputs.make_weights(model, seed=0)
    ids = inputs.make_prompt(model, P_LONG, seed=1)
    ctx = mk.mk_create(model, max_seq=P_LONG + 9)
    try:
        wd = mk.to_device(w)
        mk.mk_load_weights(ctx, wd)
        del wd
        mk.mk_prefill(ctx, ids)
        toks, logits = mk.mk_decode(ctx, 8, vocab=model.vocab)
        sent = mk.mk_count_sentinels(ctx)
        mk.mk_rewind(ctx, P_LONG)
        a, la = mk.mk_decode(ctx, 4, vocab=model.vocab)
        b, lb = mk.mk_decode(ctx, 4, vocab=model.vocab)
        st = mk.mk_stats(ctx)
    finally:
        mk.mk_destroy(ctx)
        torch.cuda.empty_cache()
    assert np.all(np.isfinite(logits))
    assert sent == 0
    assert st["fault"]["code"] == 0
    assert np.array_equal(toks, np.argmax(logits, axis=-1))
    assert np.array_equal(toks, np.concatenate([a, b]))
    assert np.array_equal(logits.view(np.uint32), np.concatenate([la, lb]).view(np.uint32))
