"""Inter-stage handoff latency from the monokernel's time journal.

The journal (``mk_read_trace`` / ``mk_chain_read_trace``) holds one record of
8 uint32 per (workgroup, step, instruction): {cta, step, pc,
op | layer << 8 | xcc << 24 | 1 << 31, t_wait (low 32 bits of the 100 MHz
device clock), t_ready - t_wait, t_done - t_wait, t_pub - t_wait}: t_ready =
inputs staged, t_pub = the instruction's output stores issued (thread 0, right
after the op), t_done = after the workgroup's failure vote.  Records without
bit 31 come from builds that journalled {..., op | layer << 8, ..., xcc} and
no publish time; their done time stands in for it.  Every workgroup runs the
same instruction sequence and each instruction consumes what the one before
it produced (the first QKV instruction of a step consumes the token every
workgroup computed itself).

Handoff latency is measured the way "7 - AMD et le monokernel" (section 7.3)
frames the cost of a synchronisation: from the moment the last producer of a
stage has published (its ``t_pub``: the stores are issued then, so this is an
upper bound of the latency) to the moment a consumer that was already waiting
has its inputs staged (``t_ready``).  Per stage the critical-path handoff is
the last consumer's ready time minus the last producer's publish time.
Consumers staged before the last producer published depended only on earlier
producers (an attention split needs the q rows of its own kv head): they are
counted ("early_consumers"), not timed.  Consumers that started waiting after
the data was complete only pay a load round trip; they are reported apart.
"""
from __future__ import annotations

import numpy as np

TICK_US = 0.01  # the device wall clock runs at 100 MHz

OP_NAMES = {1: "qkv", 2: "attention", 4: "o_proj", 5: "up_gate", 6: "down", 7: "lm_head", 8: "argmax",
            9: "chain"}


def _relative_ticks(t: np.ndarray) -> np.ndarray:
    """Unwrap 32-bit clock samples of one launch into signed ticks relative to the first."""
    t = t.astype(np.int64)
    return ((t - t[0] + (1 << 31)) % (1 << 32)) - (1 << 31)


def handoffs(records: np.ndarray) -> dict:
    """Per-op handoff statistics (microseconds) of a time journal.

    Returns {op_name: {"stages" (stages with a waiting consumer), "waiting_consumers",
    "early_consumers", "median_us", "p99_us",
    "critical_median_us", "critical_p99_us", "late_staging_median_us",
    "span_median_us", "span_mean_us"}} plus an "all" entry pooling every op.  The
    span of a stage is its share of the critical path: from the last producer's
    done time to the last consumer's.
    """
    r = np.asarray(records, dtype=np.uint32).reshape(-1, 8)
    r = r[r[:, 6] != 0]
    if len(r) == 0:
        return {}
    tw = _relative_ticks(r[:, 4])
    ready_rel = r[:, 5].astype(np.int64)
    done = tw + r[:, 6].astype(np.int64)
    ready = tw + ready_rel
    has_pub = (r[:, 3] >> 31) == 1
    pub = np.where(has_pub, tw + r[:, 7].astype(np.int64), done)
    step = r[:, 1].astype(np.int64)
    pc = r[:, 2].astype(np.int64)
    op = (r[:, 3] & 0xFF).astype(np.int64)
    key = step * (1 << 20) + pc
    order = np.unique(key)
    groups = {k: np.nonzero(key == k)[0] for k in order}
    per_op: dict[str, dict[str, list]] = {}
    for prev_k, k in zip(order[:-1], order[1:]):
        prod = groups[prev_k]
        cons = groups[k]
        cons = cons[ready_rel[cons] != 0]  # instructions without a staging mark have no handoff
        if len(cons) == 0:
            continue
        last_done = done[prod].max()
        last_pub = pub[prod].max()
        name = OP_NAMES.get(int(op[cons[0]]), str(int(op[cons[0]])))
        d = per_op.setdefault(name, {"lat": [], "crit": [], "late": [], "span": [], "early": 0})
        # the span is every stage's share of the critical path
        d["span"].append(int(done[groups[k]].max() - last_done))
        if int(op[prod[0]]) == 8:
            # after the argmax every workgroup starts the next step from the token it
            # computed itself: no handoff between workgroups
            continue
        # consumers that were waiting when the last producer published and were staged after
        # it; one staged earlier needed only some producers: not a handoff from the last one
        waiting = cons[(tw[cons] <= last_pub) & (ready[cons] >= last_pub)]
        d["early"] += int(np.count_nonzero(ready[cons] < last_pub))
        late = cons[tw[cons] > last_pub]
        d["lat"].extend((ready[waiting] - last_pub).tolist())
        d["late"].extend(ready_rel[late].tolist())
        if len(waiting):
            d["crit"].append(int(ready[cons].max() - last_pub))
    out = {}
    pooled = {"lat": [], "crit": [], "late": [], "span": [], "early": 0}
    for name, d in per_op.items():
        for k in ("lat", "crit", "late", "span"):
            pooled[k].extend(d[k])
        pooled["early"] += d["early"]
        out[name] = _summary(d)
    if per_op:
        out["all"] = _summary(pooled)
    return out


def _summary(d: dict) -> dict:
    def q(v, p):
        return float(np.percentile(np.asarray(v, dtype=np.float64) * TICK_US, p)) if len(v) else None

    return {"stages": len(d["crit"]), "waiting_consumers": len(d["lat"]), "early_consumers": d["early"],
            "median_us": q(d["lat"], 50), "p99_us": q(d["lat"], 99),
            "critical_median_us": q(d["crit"], 50), "critical_p99_us": q(d["crit"], 99),
            "late_staging_median_us": q(d["late"], 50), "span_median_us": q(d["span"], 50),
            "span_mean_us": float(np.mean(d["span"]) * TICK_US) if len(d["span"]) else None}


# Phases between the fine marks that wavefront 0 of every workgroup takes per
# instruction (marks: 0 start, 1 inputs polled, 2 staged after the barrier,
# 5 activations in registers -- short attention split: the wavefront's
# positions done; long split: its first K/V group loaded,
# 7 first weight chunk read -- short split: wavefront partials combined; long
# split: the wavefront's positions done,
# 6 own rows done -- attention: split partials published, 3 op end (the
# workgroup's rows published; attention: split merge done), 4 failure vote done).
FINE_PHASES = (("wait_and_poll", 0, 1), ("barrier", 1, 2), ("activations", 2, 5),
               ("first_chunk", 5, 7), ("own_rows", 7, 6), ("workgroup_and_publish", 6, 3),
               ("vote", 3, 4), ("total", 0, 4))


def fine_marks(ts: np.ndarray, ops: list) -> dict:
    """Median duration in µs of each phase per op over every workgroup and every
    instruction of that op.  ts: [grid][n_ins][8] 100 MHz ticks (0 = not
    recorded); ops: the op name of each instruction index (None to skip one)."""
    t = ts.astype(np.int64)
    out = {}
    for name in dict.fromkeys(o for o in ops if o is not None):
        a = t[:, [i for i, o in enumerate(ops) if o == name], :]
        d = {}
        for ph, i, j in FINE_PHASES:
            ok = (a[..., i] > 0) & (a[..., j] > 0)
            if ok.any():
                d[ph] = round(float(np.median((a[..., j] - a[..., i])[ok])) * 0.01, 3)
        out[name] = d
    return out
