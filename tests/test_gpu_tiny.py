"""GPU parity of the monokernel on the tiny decoder against the CPU oracle.

Tiny decoder: 2 layers, d 256, 4 x 64 MHA, SwiGLU 688, vocab 1024, RMSNorm eps
1e-5, RoPE theta 1e4; 32-token prompt, 16 decode steps.  688 = 1.34 chunks of
512, so the MLP rows exercise zero padding and ragged K slices; 768 QKV rows
over 256 workgroups leave most workgroups with one or two rotary pairs.
"""
import numpy as np
import pytest

import decode_megakernel_wave_amd as mk
from decode_megakernel_wave_amd import inputs
from gpu_util import MARGIN, check_free_run, check_step_logits, load, oracle_run

pytestmark = pytest.mark.gpu

CFG = inputs.TINY
P, N = 32, 16


@pytest.fixture(scope="module")
def tiny():
    w = inputs.make_weights(CFG, seed=0)
    ids = inputs.make_prompt(CFG, P, seed=1)
    t0, toks, logs, dec, m0 = oracle_run(CFG, w, ids, N)
    return w, ids, t0, toks, logs, m0


def _forced_run(tiny, **opts):
    w, ids, t0_ref, toks_ref, logs_ref, _ = tiny
    ctx = load(mk, CFG, w, P + N + 1, **opts)
    try:
        t0 = mk.mk_prefill(ctx, ids)
        feed = np.concatenate([[t0_ref], toks_ref[:-1]])
        toks, logits = mk.mk_decode_forced(ctx, feed, vocab=CFG.vocab)
        sent = mk.mk_count_sentinels(ctx)
        stats = mk.mk_stats(ctx)
    finally:
        mk.mk_destroy(ctx)
    return t0, toks, logits, sent, stats


def test_tiny_teacher_forced_parity(tiny):
    w, ids, t0_ref, toks_ref, logs_ref, m0 = tiny
    t0, toks, logits, sent, stats = _forced_run(tiny)
    print("tiny forced: max |dlogit| %.3e" % check_step_logits(logits, logs_ref, toks, toks_ref))
    if m0 > MARGIN:
        assert t0 == t0_ref
    assert sent == 0
    assert stats["fault"]["code"] == 0


def test_tiny_greedy_matches_oracle_until_first_close_call(tiny):
    w, ids, t0_ref, toks_ref, logs_ref, m0 = tiny
    from oracle.decoder import top2_margin
    ctx = load(mk, CFG, w, P + N + 1)
    try:
        out = mk.mk_generate(ctx, ids, N)
    finally:
        mk.mk_destroy(ctx)
    check_free_run(out, np.concatenate([[t0_ref], toks_ref]), np.concatenate([[m0], top2_margin(logs_ref)]))


def test_tiny_counter_mode_is_bitwise_identical(tiny):
    a = _forced_run(tiny)
    b = _forced_run(tiny, sync_mode=mk.MK_SYNC_COUNTER)
    assert a[0] == b[0]
    assert np.array_equal(a[1], b[1])
    assert np.array_equal(a[2].view(np.uint32), b[2].view(np.uint32))


def test_tiny_single_replica_is_bitwise_identical(tiny):
    a = _forced_run(tiny)
    b = _forced_run(tiny, xcd_replicas=1)
    assert np.array_equal(a[2].view(np.uint32), b[2].view(np.uint32))


def test_tiny_run_to_run_determinism(tiny):
    a = _forced_run(tiny)
    b = _forced_run(tiny)
    assert np.array_equal(a[2].view(np.uint32), b[2].view(np.uint32))


def test_tiny_chunked_decode_equals_one_launch(tiny):
    w, ids = tiny[0], tiny[1]
    ctx = load(mk, CFG, w, P + N + 1)
    try:
        mk.mk_prefill(ctx, ids)
        whole, lw = mk.mk_decode(ctx, N, vocab=CFG.vocab)
        mk.mk_rewind(ctx, P)
        a, la = mk.mk_decode(ctx, 5, vocab=CFG.vocab)
        b, lb = mk.mk_decode(ctx, N - 5, vocab=CFG.vocab)
    finally:
        mk.mk_destroy(ctx)
    assert np.array_equal(whole, np.concatenate([a, b]))
    assert np.array_equal(lw.view(np.uint32), np.concatenate([la, lb]).view(np.uint32))


def test_tiny_split_counts_agree(tiny):
    """Split attention merged over 1, 3 or 64 splits matches the oracle."""
    w, ids, t0_ref, toks_ref, logs_ref, _ = tiny
    for s in (1, 3, 64):
        _, toks, logits, sent, _ = _forced_run(tiny, attn_splits=s)
        check_step_logits(logits, logs_ref, toks, toks_ref)
        assert sent == 0


def test_tiny_small_grids(tiny):
    """Fewer workgroups than CUs: units wrap onto fewer workgroups."""
    w, ids, t0_ref, toks_ref, logs_ref, _ = tiny
    for g in (1, 8, 61):
        _, toks, logits, sent, st = _forced_run(tiny, grid=g)
        assert st["grid"] == g
        check_step_logits(logits, logs_ref, toks, toks_ref)
        assert sent == 0


def test_tiny_several_splits_per_workgroup(tiny):
    """More attention units (kv head x split) than workgroups: one workgroup
    holds several splits of the same kv head and merges them only after all
    its partials are published; both synchronisation modes."""
    w, ids, t0_ref, toks_ref, logs_ref, _ = tiny
    for g, s in ((1, 3), (8, 16), (61, 16)):
        for mode in (mk.MK_SYNC_SENTINEL, mk.MK_SYNC_COUNTER):
            _, toks, logits, sent, st = _forced_run(tiny, grid=g, attn_splits=s, sync_mode=mode)
            assert st["grid"] == g and st["fault"]["code"] == 0
            err = check_step_logits(logits, logs_ref, toks, toks_ref)
            print(f"grid {g} splits {s} mode {mode}: max |dlogit| {err:.2e}")
            assert sent == 0


def test_tiny_runs_the_general_kernel():
    """head_dim 64 and one-chunk rows do not fit the specialised kernel."""
    w = inputs.make_weights(CFG, seed=0)
    ctx = load(mk, CFG, w, P + 2)
    try:
        assert mk.mk_kernel_name(ctx) == "mk_monokernel"
    finally:
        mk.mk_destroy(ctx)
