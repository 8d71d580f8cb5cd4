"""The allocation-free entry point mk_count_sentinels_noalloc against mk_count_sentinels.

Its counter lives in a static per-GPU device array instead of a per-call
allocation.  Two calls in a row, the second on a smaller input (a context
whose last launch covered a smaller arena and fewer KV positions), each equal
to the allocating entry point's count; the counts are made non-zero by a
host-armed watchdog stall (the launch ends early and leaves sync words at the
sentinel), and a good run counts zero on both.
"""
import numpy as np
import pytest

import decode_megakernel_wave_amd as mk
from decode_megakernel_wave_amd import inputs

pytestmark = pytest.mark.gpu


def _stalled_counts(max_seq, P):
    model = inputs.TINY
    w = inputs.make_weights(model, seed=0)
    ids = inputs.make_prompt(model, P, seed=3)
    ctx = mk.mk_create(model, max_seq=max_seq, opts=mk.mk_default_options(watchdog_us=2000))
    try:
        mk.mk_load_weights(ctx, mk.to_device(w))
        with pytest.raises(mk.MkError) as e:
            mk.mk_count_sentinels_noalloc(ctx)
        assert e.value.code == mk.MK_ESTATE  # no launch yet
        mk.mk_prefill(ctx, ids)
        # two decode steps, workgroup 1 stalled before step 0's argmax: step 1 never runs, so its
        # sync buffers and its KV position keep the sentinel
        mk.mk_debug_force_stall(ctx, 1)
        with pytest.raises(mk.MkError) as e:
            mk.mk_decode(ctx, 2)
        assert e.value.code == mk.MK_ETIMEOUT
        a = mk.mk_count_sentinels(ctx)
        b = mk.mk_count_sentinels_noalloc(ctx)
        # the context recovers; after a good launch both count zero
        mk.mk_prefill(ctx, ids)
        mk.mk_decode(ctx, 2)
        z = (mk.mk_count_sentinels(ctx), mk.mk_count_sentinels_noalloc(ctx))
    finally:
        mk.mk_destroy(ctx)
    return a, b, z


def test_noalloc_count_equals_allocating_count_two_calls():
    a1, b1, z1 = _stalled_counts(max_seq=24, P=8)
    a2, b2, z2 = _stalled_counts(max_seq=8, P=3)
    print(f"counts: first {a1} / {b1}, second {a2} / {b2}")
    assert a1 > 0 and a1 == b1
    assert a2 > 0 and a2 == b2
    assert a2 < a1
    assert z1 == (0, 0) and z2 == (0, 0)
