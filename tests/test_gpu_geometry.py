"""GPU parity on two layers of the ~2B decoder's geometry, at the contexts the
benchmarks run and the full-size parity tests cannot reach.

The float64 oracle cannot prefill the whole ~2B model at long prompts in test
time, so these cases keep every shape that decides which kernel path runs --
d 2048, 16 query / 8 kv heads of 128 (two query heads per kv head), rows of
2048 and 8192 columns -- and cut the depth to 2 layers and the vocabulary to
4096.  Each asserts that the kernel specialised to that geometry
(``mk_monokernel_w4h128``, or at long contexts its variant
``mk_monokernel_w4h128_long``) is the one that runs, in the benchmark's launch
configuration (grid = CUs x occupancy, 32 attention splits per kv head), and
that the general kernel (``mk_monokernel``, register-loaded long splits) gives
bitwise the same logits for the same steps.

- Long context (the 8192-token benchmark's prompt): every split holds about
  257 positions, so attention takes the long-split path for head_dim 128 with
  two query heads per pass.
- The upper half of the 512 + 512-token benchmark's context, T in (768, 1024]:
  32 splits of 25..32 positions, so each wavefront of a short split holds 4
  positions (the full short-split batch).
"""
import os

import numpy as np
import pytest
import torch

import decode_megakernel_wave_amd as mk
from decode_megakernel_wave_amd import inputs
from gpu_util import MARGIN, check_step_logits, oracle_run

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

SPEC = "mk_monokernel_w4h128"
SPEC_LONG = "mk_monokernel_w4h128_long"  # the same, with long splits' K/V streamed through LDS by DMA
SHORT_SPLIT_MAX = 4 * 8   # positions per split that the short path takes: 4 per wavefront x 8 wavefronts


def _parity(model, P, n, expect_long):
    w = inputs.make_weights(model, seed=0)
    ids = inputs.make_prompt(model, P, seed=1)
    print(f"[{model.name} P={P}] oracle prefill + {n} steps", flush=True)
    t0_ref, toks_ref, logs_ref, _, m0 = oracle_run(model, w, ids, n)
    print(f"[{model.name} P={P}] GPU prefill + teacher-forced decode", flush=True)
    ctx = mk.mk_create(model, max_seq=P + n + 1)
    try:
        wd = mk.to_device(w)
        mk.mk_load_weights(ctx, wd)
        del wd
        assert mk.mk_kernel_name(ctx) == SPEC
        t0 = mk.mk_prefill(ctx, ids)
        grid = mk.mk_stats(ctx)["grid"]
        splits = mk.mk_plan_check(model, P + n + 1, grid)["attn_splits"]
        feed = np.concatenate([[t0_ref], toks_ref[:-1]])
        toks, logits = mk.mk_decode_forced(ctx, feed, vocab=model.vocab)
        ran = mk.mk_kernel_name(ctx)
        sent = mk.mk_count_sentinels(ctx)
        fault = mk.mk_stats(ctx)["fault"]["code"]
        # the same steps again on the general kernel (register-loaded long splits): bitwise equal
        mk.mk_rewind(ctx, P)
        os.environ["MK_GENERAL_KERNEL"] = "1"
        try:
            g_toks, g_logits = mk.mk_decode_forced(ctx, feed, vocab=model.vocab)
            assert mk.mk_kernel_name(ctx) == "mk_monokernel"
        finally:
            del os.environ["MK_GENERAL_KERNEL"]
    finally:
        mk.mk_destroy(ctx)
        torch.cuda.empty_cache()
    assert np.array_equal(g_toks, toks)
    assert np.array_equal(g_logits.view(np.uint32), logits.view(np.uint32)), "general and specialised kernels differ"
    # which attention path ran: split length ceil(T / S) for every decoded position T = P + s + 1
    chunks = [-(-(P + s + 1) // splits) for s in range(n)]
    if expect_long:
        assert min(chunks) > SHORT_SPLIT_MAX, chunks
        assert ran == SPEC_LONG, ran
    else:
        assert all(3 * 8 < c <= SHORT_SPLIT_MAX for c in chunks), chunks
        assert ran == SPEC, ran
    err = check_step_logits(logits, logs_ref, toks, toks_ref)
    print(f"[{model.name} P={P}] grid {grid}, {splits} splits, split lengths {chunks}: max |dlogit| {err:.2e}")
    if m0 > MARGIN:
        assert t0 == t0_ref, "token after the prompt"
    assert sent == 0
    assert fault == 0
    return err


def test_2b_geometry_long_context_8192():
    """Prompt of 8192 tokens: the long-split attention path for head_dim 128, two query heads per kv head."""
    _parity(inputs.M2B_GEOM_L2_NARROW, P=8192, n=4, expect_long=True)


@pytest.mark.parametrize("P", [770, 1020])
def test_2b_geometry_upper_half_context(P):
    """T = 771..774 (splits of 25 positions: wavefront 0 holds 4, the others 3) and T = 1021..1024
    (splits of 32: every wavefront holds the full batch of 4 positions)."""
    _parity(inputs.M2B_GEOM_L2, P=P, n=4, expect_long=False)


def test_2b_geometry_long_kernel_just_past_the_short_bound():
    """T = 1031..1034: splits of 33 positions (9 groups of 4), so the long-context kernel runs and
    each wavefront's K/V ring holds one or two groups (the prefetch before the q poll is partial
    for most); the last split holds 8..11 positions and takes the short path inside that kernel."""
    _parity(inputs.M2B_GEOM_L2, P=1030, n=4, expect_long=True)


def test_2b_geometry_prompt_6000_partial_attention_round():
    """Prompt of 6000 tokens: 47 super-blocks of 128 queries x 8 kv heads = 376 prefill attention
    items, so the second round of the static deal (dealt in reverse super-block order) is partial
    (120 items); 47 row tiles of 128 with a ragged last one (112 positions) on the 256-row GEMM
    tiles; then decode on the long-split path."""
    _parity(inputs.M2B_GEOM_L2_NARROW, P=6000, n=4, expect_long=True)
