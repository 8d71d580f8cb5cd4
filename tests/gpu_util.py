"""Helpers shared by the GPU parity tests (no test functions here)."""
import numpy as np

from decode_megakernel_wave_amd import inputs
from oracle import decoder as od

LOGIT_TOL = 1e-2      # |dlogit| bound of the acceptance rule
MARGIN = 2e-2         # tokens must agree where the oracle's top-2 margin exceeds this


def oracle_run(model, w, ids, n):
    """Free-running oracle: (t0, tokens[n], logits[n, V], decoder, top-2 margin of the prompt logits)."""
    dec = od.Decoder(w, model.n_heads, model.n_kv_heads, model.rms_eps, model.rope_theta,
                     max_seq=len(ids) + n + 1)
    l0 = dec.prefill(ids)
    t = int(np.argmax(l0))
    t0, toks, logs = t, [], []
    for s in range(n):
        lg = dec.step(t, len(ids) + s)
        t = int(np.argmax(lg))
        toks.append(t)
        logs.append(lg)
    return t0, np.array(toks, dtype=np.int32), np.array(logs), dec, float(od.top2_margin(l0[None])[0])


def check_free_run(free, ref, margins):
    """Greedy tokens must agree until the first step whose oracle top-2 margin is a close call
    (<= MARGIN): there either token is acceptable and the sequences may part."""
    for s in range(len(ref)):
        if margins[s] <= MARGIN:
            break
        assert free[s] == ref[s], f"free-running token {s}: {free[s]} != {ref[s]}"


def check_step_logits(gpu_logits, ref_logits, gpu_tokens, ref_tokens, tol=LOGIT_TOL):
    """Acceptance rule: |dlogit| <= tol everywhere; equal argmax where the margin is clear."""
    err = np.abs(gpu_logits.astype(np.float64) - ref_logits)
    assert np.all(np.isfinite(gpu_logits)), "non-finite GPU logits"
    worst = float(err.max())
    assert worst <= tol, f"max |dlogit| {worst:.3e} > {tol}"
    clear = od.top2_margin(ref_logits) > MARGIN
    bad = np.nonzero(clear & (gpu_tokens != ref_tokens))[0]
    assert bad.size == 0, f"token mismatch at clear-margin steps {bad.tolist()}"
    # the GPU's token is the argmax of its own logits (lowest index on ties)
    assert np.array_equal(gpu_tokens, np.argmax(gpu_logits, axis=-1))
    return worst


def load(mk, model, w, max_seq, **opts):
    ctx = mk.mk_create(model, max_seq=max_seq, opts=mk.mk_default_options(**opts) if opts else None)
    mk.mk_load_weights(ctx, mk.to_device(w))
    return ctx


__all__ = ["inputs", "oracle_run", "check_step_logits", "check_free_run", "load", "LOGIT_TOL", "MARGIN"]
