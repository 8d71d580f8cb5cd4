"""Host-side checks of the C ABI (no GPU needed).

- libmk.so loads and exports exactly the functions include/*.h declare;
- the ctypes mirrors of the ABI structs have the C compiler's layout;
- the schedule builder accepts every model at the grids the kernel runs at,
  conserves the weight bytes (every matrix byte streamed once per step), fits
  the 160 KB LDS, balances the per-wavefront streams, and rejects unsupported
  shapes and options with a reason.
"""
import ctypes as C
import glob
import os
import re
import shutil
import subprocess

import pytest

import decode_megakernel_wave_amd as mk
from decode_megakernel_wave_amd import capi, inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mk.h")
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))


def _declared():
    names = set()
    for h in HEADERS:
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(mk_\w+)\s*\(", text, flags=re.M))
    return names


def test_library_exports_every_declared_function():
    lib = capi.lib()
    declared = _declared()
    assert len(declared) >= 20
    missing = sorted(n for n in declared if not hasattr(lib, n))
    assert not missing, f"declared but not exported: {missing}"


@pytest.mark.skipif(shutil.which("nm") is None, reason="nm not available")
def test_library_exports_nothing_undeclared():
    out = subprocess.run(["nm", "-D", "--defined-only", capi._LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if re.search(r" T mk_\w+$", ln)}
    extra = sorted(exported - _declared())
    assert not extra, f"exported but not declared in include/*.h: {extra}"


_STRUCTS = ["mk_config", "mk_options", "mk_weights", "mk_fault", "mk_stats_t", "mk_plan_info"]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_ctypes_struct_layout_matches_header(tmp_path):
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "mk.h"', "int main(void) {"]
    for s in _STRUCTS:
        lines.append(f'  printf("{s} size %zu\\n", sizeof({s}));')
        for f, _ in getattr(capi, s)._fields_:
            lines.append(f'  printf("{s} {f} %zu\\n", offsetof({s}, {f}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)],
                   check=True)
    got = {}
    for ln in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.splitlines():
        s, f, v = ln.split()
        got[(s, f)] = int(v)
    for s in _STRUCTS:
        cls = getattr(capi, s)
        assert got[(s, "size")] == C.sizeof(cls), s
        for f, _ in cls._fields_:
            assert got[(s, f)] == getattr(cls, f).offset, f"{s}.{f}"


def test_default_options():
    o = mk.mk_default_options()
    assert (o.sync_mode, o.xcd_replicas, o.attn_splits, o.grid) == (mk.MK_SYNC_SENTINEL, 8, 0, 0)
    assert o.watchdog_us > 0 and o.trace_steps == 0 and o.work_queue == 0


def _matrix_params(m: inputs.ModelConfig) -> int:
    qd, kvd = m.n_heads * m.head_dim, m.n_kv_heads * m.head_dim
    per_layer = qd * m.d_model + 2 * kvd * m.d_model + m.d_model * qd + 3 * m.ffn * m.d_model
    return m.n_layers * per_layer + m.vocab * m.d_model


def _padded_params(m: inputs.ModelConfig) -> int:
    """Matrix elements once every row is zero-padded to whole 512-column chunks."""
    pad = lambda k: -(-k // 512) * 512
    qd, kvd = m.n_heads * m.head_dim, m.n_kv_heads * m.head_dim
    per_layer = (qd + 2 * kvd + 2 * m.ffn) * pad(m.d_model) + m.d_model * pad(qd) + m.d_model * pad(m.ffn)
    return m.n_layers * per_layer + m.vocab * pad(m.d_model)


@pytest.mark.parametrize("name", list(inputs.WORKLOADS))
@pytest.mark.parametrize("grid", [61, 128, 256])
def test_plan_accepts_workloads(name, grid):
    w = inputs.WORKLOADS[name]
    m = w.model
    info = mk.mk_plan_check(m, w.max_seq, grid)
    assert info["n_cta"] == grid
    assert info["lds_bytes"] <= 160 * 1024
    assert 1 <= info["attn_splits"] <= 64
    # every matrix element is streamed exactly once per step (plus zero padding of ragged rows)
    assert info["stream_bytes"] == 2 * _padded_params(m) == info["stream_chunks"] * 1024
    # algorithmic bytes: the matrices, the 2L+1 norm gains and one embedding row
    assert info["weight_bytes"] == 2 * (_matrix_params(m) + (2 * m.n_layers + 1) * m.d_model + m.d_model)
    # stages with outputs: per layer QKV, attention (with the split merge), O, up/gate, down; then the LM head
    # (its argmax keys are the last stage's output; the argmax produces only the token)
    assert info["n_sync_ids"] == 5 * m.n_layers + 1
    mean = info["stream_chunks"] / (grid * 8)
    assert info["min_wave_chunks"] <= mean <= info["max_wave_chunks"]
    if grid == 256 and m is inputs.M2B:
        # the benchmark's model on a full chip: no wavefront streams more than 1% over the mean
        assert info["max_wave_chunks"] <= 1.01 * mean


def test_plan_wide_query_groups():
    # 8 query heads per kv head: attention combines them in passes of 4 (hd 128) or 8 (hd 64)
    for hd in (64, 128, 256):
        m = _cfg(n_heads=16, n_kv_heads=2, head_dim=hd, d_model=1024)
        mk.mk_plan_check(m, 64, 64)


def test_plan_single_workgroup_tiny():
    w = inputs.WORKLOADS["tiny"]
    info = mk.mk_plan_check(w.model, w.max_seq, 1)
    assert info["min_wave_chunks"] == info["max_wave_chunks"]


@pytest.mark.parametrize("splits", [1, 2, 7, 64])
def test_plan_attention_splits(splits):
    w = inputs.WORKLOADS["0.5b"]
    info = mk.mk_plan_check(w.model, w.max_seq, 256, mk.mk_default_options(attn_splits=splits))
    assert info["attn_splits"] == splits


@pytest.mark.parametrize("replicas", [1, 2, 4, 8])
@pytest.mark.parametrize("sync", [mk.MK_SYNC_SENTINEL, mk.MK_SYNC_COUNTER])
def test_plan_options(replicas, sync):
    w = inputs.WORKLOADS["tiny"]
    mk.mk_plan_check(w.model, w.max_seq, 64, mk.mk_default_options(xcd_replicas=replicas, sync_mode=sync))


def _cfg(**kw):
    d = dict(name="t", n_layers=2, d_model=256, n_heads=4, n_kv_heads=4, head_dim=64, ffn=688, vocab=1024)
    d.update(kw)
    return inputs.ModelConfig(**d)


@pytest.mark.parametrize("model,max_seq,grid,opts,reason", [
    (_cfg(n_kv_heads=3), 64, 64, {}, "multiple of n_kv_heads"),
    (_cfg(head_dim=96, n_heads=4, n_kv_heads=4), 64, 64, {}, "head_dim"),
    (_cfg(d_model=258), 64, 64, {}, "multiples of 4"),
    (_cfg(ffn=20000), 64, 64, {}, "at most 16384"),
    (_cfg(vocab=1), 64, 64, {}, "positive"),
    (_cfg(), 1, 64, {}, "positive"),
    (_cfg(), 64, 0, {}, "at least one workgroup"),
    (_cfg(d_model=2048, ffn=512), 64, 1, {}, "residual rows"),
    (inputs.M2B, 1025, 1, {}, "no K split fits"),
])
def test_plan_rejects(model, max_seq, grid, opts, reason):
    with pytest.raises(mk.MkError) as e:
        mk.mk_plan_check(model, max_seq, grid, mk.mk_default_options(**opts) if opts else None)
    assert e.value.code == mk.MK_EINVAL
    assert reason in str(e.value)


@pytest.mark.parametrize("field,value", [("xcd_replicas", 3), ("attn_splits", 65), ("sync_mode", 2),
                                         ("watchdog_us", 0), ("work_queue", 2), ("grid", -1), ("attn_splits", -1)])
def test_plan_rejects_options(field, value):
    w = inputs.WORKLOADS["tiny"]
    with pytest.raises(mk.MkError) as e:
        mk.mk_plan_check(w.model, w.max_seq, 64, mk.mk_default_options(**{field: value}))
    assert e.value.code == mk.MK_EINVAL


@pytest.mark.parametrize("name,grid,expect", [("2b", 256, 1), ("2b-long", 256, 1), ("2b", 61, 1),
                                              ("0.5b", 256, 0), ("tiny", 256, 0)])
def test_specialised_kernel_choice(name, grid, expect):
    """The ~2B schedule (4-chunk slices, head_dim 128, two query heads per kv head) fits the
    specialised monokernel at any grid; head_dim 64 or narrower rows do not."""
    w = inputs.WORKLOADS[name]
    info = mk.mk_plan_check(w.model, w.max_seq, grid)
    assert info["specialised"] == expect


def test_specialised_kernel_needs_two_query_heads_per_kv_head():
    m = inputs.M2B
    mha = inputs.ModelConfig("2b-mha", n_layers=2, d_model=m.d_model, n_heads=16, n_kv_heads=16, head_dim=128,
                             ffn=m.ffn, vocab=4096, rms_eps=m.rms_eps, rope_theta=m.rope_theta)
    assert mk.mk_plan_check(mha, 64, 256)["specialised"] == 0
