"""Head geometries and boundaries not covered by the workload models.

- Query groups of 4 and 8 and head_dim 256 (the workloads only have G <= 2
  and head_dim 64 / 128), each with the chosen split count (short splits,
  one position per wavefront) and with one split (long splits, 16-byte K/V
  loads), against the oracle; G = 8 at head_dim 128 needs two head passes.
- A one-token prompt decoded until the KV cache is exactly full, against
  the oracle; one more step is refused and leaves the context usable.
- Calls out of order or out of range fail with the documented codes.
- The watchdog: a wait the host arms never to be satisfied ends the launch
  with MK_ETIMEOUT, every workgroup exits, and the context recovers.
"""
import numpy as np
import pytest

import decode_megakernel_wave_amd as mk
from decode_megakernel_wave_amd import inputs
from gpu_util import MARGIN, check_step_logits, load, oracle_run

pytestmark = pytest.mark.gpu

GEOMETRIES = {
    "g4_hd128": inputs.ModelConfig("g4_hd128", n_layers=2, d_model=512, n_heads=4, n_kv_heads=1,
                                   head_dim=128, ffn=1024, vocab=1024),
    "g8_hd128": inputs.ModelConfig("g8_hd128", n_layers=2, d_model=512, n_heads=8, n_kv_heads=1,
                                   head_dim=128, ffn=1024, vocab=1024),
    "g2_hd256": inputs.ModelConfig("g2_hd256", n_layers=2, d_model=512, n_heads=2, n_kv_heads=1,
                                   head_dim=256, ffn=1024, vocab=1024),
    "g8_hd64": inputs.ModelConfig("g8_hd64", n_layers=2, d_model=512, n_heads=8, n_kv_heads=1,
                                  head_dim=64, ffn=1024, vocab=1024),
}
P, N = 40, 8


@pytest.fixture(scope="module", params=list(GEOMETRIES))
def geometry(request):
    model = GEOMETRIES[request.param]
    w = inputs.make_weights(model, seed=0)
    ids = inputs.make_prompt(model, P, seed=1)
    t0, toks, logs, _, m0 = oracle_run(model, w, ids, N)
    return model, w, ids, t0, toks, logs, m0


@pytest.mark.parametrize("splits", [0, 1])
def test_geometry_parity(geometry, splits):
    model, w, ids, t0_ref, toks_ref, logs_ref, m0 = geometry
    ctx = load(mk, model, w, P + N + 1, attn_splits=splits)
    try:
        t0 = mk.mk_prefill(ctx, ids)
        toks, logits = mk.mk_decode_forced(ctx, np.concatenate([[t0_ref], toks_ref[:-1]]), vocab=model.vocab)
        sent = mk.mk_count_sentinels(ctx)
    finally:
        mk.mk_destroy(ctx)
    err = check_step_logits(logits, logs_ref, toks, toks_ref)
    print(f"{model.name} splits={splits}: max |dlogit| {err:.2e}")
    if m0 > MARGIN:
        assert t0 == t0_ref
    assert sent == 0


def test_one_token_prompt_until_the_cache_is_full():
    model, max_seq = inputs.TINY, 8
    w = inputs.make_weights(model, seed=0)
    ids = inputs.make_prompt(model, 1, seed=3)
    t0_ref, toks_ref, logs_ref, _, m0 = oracle_run(model, w, ids, max_seq - 1)
    ctx = load(mk, model, w, max_seq)
    try:
        t0 = mk.mk_prefill(ctx, ids)
        toks, logits = mk.mk_decode_forced(ctx, np.concatenate([[t0_ref], toks_ref[:-1]]), vocab=model.vocab)
        assert mk.mk_position(ctx)[0] == max_seq
        with pytest.raises(mk.MkError) as e:
            mk.mk_decode(ctx, 1)
        assert e.value.code == mk.MK_ERANGE
        # the refused call changed nothing: rewind and decode again
        mk.mk_rewind(ctx, 1)
        again = mk.mk_decode_forced(ctx, np.concatenate([[t0_ref], toks_ref[:-1]]))
        sent = mk.mk_count_sentinels(ctx)
    finally:
        mk.mk_destroy(ctx)
    check_step_logits(logits, logs_ref, toks, toks_ref)
    if m0 > MARGIN:
        assert t0 == t0_ref
    assert np.array_equal(again, toks)
    assert sent == 0


def test_calls_out_of_order_or_range_fail_cleanly():
    model = inputs.TINY
    w = inputs.make_weights(model, seed=0)
    ctx = mk.mk_create(model, max_seq=16)
    try:
        with pytest.raises(mk.MkError) as e:
            mk.mk_prefill(ctx, [1, 2, 3])
        assert e.value.code == mk.MK_ESTATE  # no weights yet
        mk.mk_load_weights(ctx, mk.to_device(w))
        with pytest.raises(mk.MkError) as e:
            mk.mk_decode(ctx, 1)
        assert e.value.code == mk.MK_ESTATE  # no prompt yet
        for ids, code in (([], mk.MK_EINVAL), (list(range(17)), mk.MK_ERANGE), ([0, model.vocab], mk.MK_ERANGE)):
            with pytest.raises(mk.MkError) as e:
                mk.mk_prefill(ctx, ids)
            assert e.value.code == code
        mk.mk_prefill(ctx, [5, 6, 7, 8])
        with pytest.raises(mk.MkError) as e:
            mk.mk_decode(ctx, 0)
        assert e.value.code == mk.MK_EINVAL
        for pos in (0, 5):
            with pytest.raises(mk.MkError) as e:
                mk.mk_rewind(ctx, pos)
            assert e.value.code == mk.MK_ERANGE
        with pytest.raises(mk.MkError) as e:
            mk.mk_decode(ctx, 13)  # 4 + 13 > 16
        assert e.value.code == mk.MK_ERANGE
        assert len(mk.mk_decode(ctx, 12)) == 12  # exactly fills the cache
        assert mk.mk_stats(ctx)["fault"]["code"] == 0
    finally:
        mk.mk_destroy(ctx)


def test_watchdog_reports_a_lost_dependency_and_every_workgroup_exits():
    """The failure path, forced from the host: in one launch workgroup 1 waits (step 0, before its
    argmax) for a sync word the host never writes.  That wait's watchdog fires after watchdog_us,
    the fault record and the error text name the wait, every other workgroup leaves its own waits
    through the abort flag, the launch ends normally with MK_ETIMEOUT, the context asks for a new
    prefill, and the next launch (not armed) decodes normally."""
    model = inputs.TINY
    w = inputs.make_weights(model, seed=0)
    ids = inputs.make_prompt(model, 4, seed=3)
    ctx = load(mk, model, w, 16, watchdog_us=2000)
    try:
        mk.mk_debug_force_stall(ctx, 1)
        with pytest.raises(mk.MkError) as e:
            mk.mk_prefill(ctx, ids)
        assert e.value.code == mk.MK_ETIMEOUT
        assert "device watchdog" in str(e.value)
        st = mk.mk_stats(ctx)
        assert st["fault"]["code"] == mk.MK_ETIMEOUT
        assert st["fault"]["step"] in (0, 1)
        # every workgroup stopped by step 1: none ran on past the lost dependency
        prog = mk.mk_debug_progress(ctx, st["grid"])
        assert int((prog >> 16).max()) <= 1
        with pytest.raises(mk.MkError) as e:
            mk.mk_decode(ctx, 1)
        assert e.value.code == mk.MK_ESTATE
        t0 = mk.mk_prefill(ctx, ids)
        toks = mk.mk_decode(ctx, 4)
        assert mk.mk_count_sentinels(ctx) == 0
        assert mk.mk_stats(ctx)["fault"]["code"] == 0
    finally:
        mk.mk_destroy(ctx)
    ref = mk.mk_create(model, max_seq=16)
    try:
        mk.mk_load_weights(ref, mk.to_device(w))
        assert mk.mk_prefill(ref, ids) == t0
        assert np.array_equal(mk.mk_decode(ref, 4), toks)
    finally:
        mk.mk_destroy(ref)
