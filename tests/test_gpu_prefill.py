"""GPU parity of the MFMA prompt prefill against the CPU oracle.

mk_prefill runs positions 0..P-2 of the prompt in one launch of the prefill
kernel (MFMA GEMMs on fp16 hi + lo halves of the fp32 activations, causal
attention tiles) and the last prompt token as one decode step.  Checked here:

- the KV cache it writes, every layer, kv head and position, against the
  oracle's fp16 K and V: in layer 0 within one fp16 unit in the last place
  (the float32 GEMM and the float64 oracle on either side of a rounding
  boundary) plus 2e-5 of the head row's RMS (float32 error of values far
  below the row's scale); in later layers one ulp plus 2e-3 of the row's RMS
  (the one-ulp flips propagate);
- t0 and the teacher-forced decode after it against the oracle, with the
  prefill kernel's position count reported by mk_stats;
- prompts that leave ragged GEMM and attention tiles (1, 2, 33, 129, 200
  positions; 2100, long enough for the 256-row weight tiles), and the
  token-by-token prefill (MK_PREFILL_STEPS) giving the same first token and the
  same decode within the acceptance rule;
- the dynamic work queue (option work_queue) giving bitwise the results of
  the static deal.
"""
import numpy as np
import pytest
import torch

import decode_megakernel_wave_amd as mk
from decode_megakernel_wave_amd import inputs
from gpu_util import MARGIN, check_step_logits, oracle_run

pytestmark = pytest.mark.gpu


def _kv_check(ctx, dec, model, P):
    """Cached K/V of positions 0..P-1 against the oracle's fp16 values.

    Layer 0 sees the same inputs on both sides: each value equals the oracle's, or is one fp16
    ulp away where the float32 GEMM and the float64 oracle fall on either side of a rounding
    boundary, or -- for values far below the row's scale, whose ulp is tiny -- within the float32
    error of the dot product (bound: one ulp plus 2e-5 of the RMS of its head's row).  Those
    one-ulp flips (2^-11 relative) reach the later layers' inputs at about 1e-4 relative, so from
    layer 1 on the bound is one ulp plus 2e-3 of the row's RMS."""
    mism, total, worst = 0, 0, 0.0
    for layer in range(model.n_layers):
        for g in range(model.n_kv_heads):
            k, v = mk.mk_debug_kv(ctx, layer, g, 0, P, model.head_dim)
            for got, ref in ((k, dec.K[layer, :P, g]), (v, dec.V[layer, :P, g])):
                ref16 = ref.astype(np.float16)
                assert np.array_equal(ref16.astype(np.float64), ref)  # the oracle stores fp16 values
                diff = np.abs(got.astype(np.float64) - ref)
                ulp = np.spacing(np.abs(ref16)).astype(np.float64)
                rms = np.sqrt(np.mean(ref * ref, axis=-1, keepdims=True))
                bound = ulp + (2e-5 if layer == 0 else 2e-3) * rms
                worst = max(worst, float(np.max(diff / bound)))
                mism += int(np.count_nonzero(got != ref16))
                total += got.size
    assert worst <= 1.0, f"a cached value is {worst:.2f} x its bound from the oracle's"
    return mism, total


def _run(model, P, n, seed=1, w=None, env_steps=False, monkeypatch=None, **opts):
    w = w if w is not None else inputs.make_weights(model, seed=0)
    ids = inputs.make_prompt(model, P, seed=seed)
    t0_ref, toks_ref, logs_ref, dec, m0 = oracle_run(model, w, ids, n)
    if env_steps:
        monkeypatch.setenv("MK_PREFILL_STEPS", "1")
    ctx = mk.mk_create(model, max_seq=P + n + 1, opts=mk.mk_default_options(**opts) if opts else None)
    try:
        wd = mk.to_device(w)
        mk.mk_load_weights(ctx, wd)
        del wd
        t0 = mk.mk_prefill(ctx, ids)
        st = mk.mk_stats(ctx)
        # the cache after prefill (the oracle's positions 0..P-1 are the prompt's too)
        mism, total = _kv_check(ctx, dec, model, P)
        feed = np.concatenate([[t0_ref], toks_ref[:-1]])
        toks, logits = mk.mk_decode_forced(ctx, feed, vocab=model.vocab)
        sent = mk.mk_count_sentinels(ctx)
    finally:
        mk.mk_destroy(ctx)
        torch.cuda.empty_cache()
    err = check_step_logits(logits, logs_ref, toks, toks_ref)
    if m0 > MARGIN:
        assert t0 == t0_ref, "token after the prompt"
    assert sent == 0
    return st, err, (mism, total), t0, logits, m0


@pytest.mark.parametrize("P", [1, 2, 33, 129, 200, 2100])
def test_tiny_prefill_ragged_prompts(P):
    """P = 2100 has 17 row tiles: the stages take the 256-row weight tiles of long prompts."""
    st, err, (mism, total), _, _, _ = _run(inputs.TINY, P, 4)
    assert st["prefill_positions"] == P - 1
    assert (st["prefill_grid"] > 0) == (P >= 2)
    print(f"tiny P={P}: max |dlogit| {err:.2e}, cached values off by one ulp: {mism}/{total}")


def test_05b_prefill_prompt128():
    st, err, (mism, total), _, _, _ = _run(inputs.M05, 128, 4)
    assert st["prefill_positions"] == 127
    print(f"0.5B P=128: prefill {st['prefill_ms']:.2f} ms, max |dlogit| {err:.2e}, ulp-off values {mism}/{total}")


def test_2b_geometry_prefill_prompt512():
    st, err, (mism, total), _, _, _ = _run(inputs.M2B_GEOM_L2, 512, 4)
    assert st["prefill_positions"] == 511
    print(f"2B geometry P=512: prefill {st['prefill_ms']:.2f} ms, max |dlogit| {err:.2e}, "
          f"ulp-off values {mism}/{total}")


@pytest.mark.parametrize("model,P", [(inputs.TINY, 200), (inputs.M2B_GEOM_L2, 512)])
def test_prefill_work_queue(model, P):
    """Tiles and attention items claimed from a per-stage work queue instead of the static deal:
    the same parity, and the same KV cache bit for bit (each tile is computed the same way
    whichever workgroup claims it)."""
    w = inputs.make_weights(model, seed=0)
    st, err, _, t0, log_q, _ = _run(model, P, 2, w=w, work_queue=1)
    assert st["prefill_positions"] == P - 1
    _, _, _, t0_s, log_s, _ = _run(model, P, 2, w=w)
    assert t0 == t0_s
    assert np.array_equal(log_q.view(np.uint32), log_s.view(np.uint32))
    print(f"{model.name} P={P} work queue: max |dlogit| {err:.2e}")


def test_prefill_token_by_token_agrees(monkeypatch):
    """The MFMA prefill and the token-by-token prefill both meet the acceptance rule and choose the same t0."""
    model, P = inputs.TINY, 40
    w = inputs.make_weights(model, seed=0)
    st_a, err_a, _, t0_a, log_a, m0 = _run(model, P, 4, w=w)
    st_b, err_b, _, t0_b, log_b, _ = _run(model, P, 4, w=w, env_steps=True, monkeypatch=monkeypatch)
    assert st_a["prefill_positions"] == P - 1 and st_b["prefill_positions"] == 0
    if m0 > 1e-3:
        assert t0_a == t0_b
    assert float(np.max(np.abs(log_a - log_b))) <= 1e-2
