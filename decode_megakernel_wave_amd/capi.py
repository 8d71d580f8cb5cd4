"""Thin ctypes binding of ``include/mk.h`` (argument marshalling only).

Every function here has the name of the C entry point it calls.  Device
memory and streams come from PyTorch: weight tensors must be fp16 CUDA
tensors on the context's device, and the stream defaults to torch's current
stream.  All compute happens in ``libmk.so``; if that library is missing the
first call raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

from . import inputs

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmk.so")
_lib = None

MK_OK, MK_EINVAL, MK_ENOMEM, MK_EHIP, MK_ESTATE, MK_ERANGE, MK_EOCC, MK_ETIMEOUT, MK_ENAN = 0, -1, -2, -3, -4, -5, -6, -7, -8
ERROR_NAMES = {0: "MK_OK", -1: "MK_EINVAL", -2: "MK_ENOMEM", -3: "MK_EHIP", -4: "MK_ESTATE", -5: "MK_ERANGE",
               -6: "MK_EOCC", -7: "MK_ETIMEOUT", -8: "MK_ENAN"}
MK_SYNC_SENTINEL, MK_SYNC_COUNTER = 0, 1


class MkError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{ERROR_NAMES.get(code, code)}: {msg}")
        self.code = code


class mk_config(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("n_layers", "d_model", "n_heads", "n_kv_heads", "head_dim", "ffn",
                                          "vocab", "max_seq")] + [("rms_eps", C.c_float), ("rope_theta", C.c_float)]


class mk_options(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("sync_mode", "xcd_replicas", "attn_splits", "trace_steps",
                                          "watchdog_us", "grid", "work_queue")]


_PP = C.POINTER(C.c_void_p)


class mk_weights(C.Structure):
    _fields_ = [("embed", C.c_void_p), ("final_norm", C.c_void_p), ("lm_head", C.c_void_p)] + \
               [(n, _PP) for n in ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down")]


class mk_fault(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("code", "cta", "pc", "op", "step", "layer", "index", "pad")]


class mk_stats_t(C.Structure):
    _fields_ = [("gpu_ms", C.c_double), ("steps", C.c_int32), ("pos0", C.c_int32), ("grid", C.c_int32),
                ("block", C.c_int32), ("lds_bytes", C.c_int32), ("ring_depth", C.c_int32),
                ("stream_bytes", C.c_int64), ("weight_bytes", C.c_int64), ("kv_bytes_per_pos", C.c_int64),
                ("algo_bytes", C.c_int64), ("n_cu", C.c_int32), ("occupancy", C.c_int32), ("fault", mk_fault),
                ("prefill_ms", C.c_double), ("prefill_positions", C.c_int32), ("prefill_grid", C.c_int32)]


class mk_plan_info(C.Structure):
    _fields_ = [("n_cta", C.c_int32), ("max_ins_per_cta", C.c_int32), ("n_sync_ids", C.c_int32),
                ("lds_bytes", C.c_int32), ("stream_chunks", C.c_int64), ("stream_bytes", C.c_int64),
                ("weight_bytes", C.c_int64), ("min_wave_chunks", C.c_int32), ("max_wave_chunks", C.c_int32),
                ("attn_splits", C.c_int32), ("specialised", C.c_int32)]


# Every symbol of include/mk.h: (name, restype, argtypes)
SIGNATURES = [
    ("mk_default_options", C.c_int, [C.POINTER(mk_options)]),
    ("mk_create", C.c_int, [C.POINTER(mk_config), C.POINTER(mk_options), C.c_int, C.c_void_p, C.POINTER(C.c_void_p)]),
    ("mk_load_weights", C.c_int, [C.c_void_p, C.POINTER(mk_weights)]),
    ("mk_prefill", C.c_int, [C.c_void_p, C.POINTER(C.c_int32), C.c_int32, C.POINTER(C.c_int32)]),
    ("mk_decode", C.c_int, [C.c_void_p, C.c_int32, C.POINTER(C.c_int32), C.POINTER(C.c_float)]),
    ("mk_decode_forced", C.c_int, [C.c_void_p, C.c_int32, C.POINTER(C.c_int32), C.POINTER(C.c_int32),
                                   C.POINTER(C.c_float)]),
    ("mk_generate", C.c_int, [C.c_void_p, C.POINTER(C.c_int32), C.c_int32, C.c_int32, C.POINTER(C.c_int32)]),
    ("mk_rewind", C.c_int, [C.c_void_p, C.c_int32]),
    ("mk_set_sampling", C.c_int, [C.c_void_p, C.c_int32, C.c_float, C.c_uint64]),
    ("mk_kernel_name", C.c_char_p, [C.c_void_p]),
    ("mk_probe_launch", C.c_int, [C.c_int, C.c_void_p, C.c_int32, C.POINTER(C.c_double), C.POINTER(C.c_double)]),
    ("mk_probe_read", C.c_int, [C.c_int, C.c_void_p, C.c_void_p, C.c_int64, C.c_int32, C.POINTER(C.c_double)]),
    ("mk_probe_barrier", C.c_int, [C.c_int, C.c_void_p, C.c_int32, C.POINTER(C.c_double)]),
    ("mk_probe_handoff", C.c_int, [C.c_int, C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.POINTER(C.c_double),
                                   C.POINTER(C.c_double), C.POINTER(C.c_double)]),
    ("mk_position", C.c_int, [C.c_void_p, C.POINTER(C.c_int32), C.POINTER(C.c_int32)]),
    ("mk_stats", C.c_int, [C.c_void_p, C.POINTER(mk_stats_t)]),
    ("mk_count_sentinels", C.c_int, [C.c_void_p, C.POINTER(C.c_int64)]),
    ("mk_count_sentinels_noalloc", C.c_int, [C.c_void_p, C.POINTER(C.c_int64)]),
    ("mk_read_trace", C.c_int, [C.c_void_p, C.POINTER(C.c_uint32), C.c_int64, C.POINTER(C.c_int64)]),
    ("mk_debug_streams", C.c_int, [C.c_void_p, C.POINTER(C.c_void_p), C.POINTER(C.c_void_p), C.POINTER(C.c_void_p)]),
    ("mk_debug_layout", C.c_int, [C.c_void_p, C.POINTER(C.c_int64)]),
    ("mk_debug_arena", C.c_int, [C.c_void_p, C.c_int64, C.c_int64, C.POINTER(C.c_uint32)]),
    ("mk_debug_progress", C.c_int, [C.c_void_p, C.POINTER(C.c_uint32), C.c_int32]),
    ("mk_debug_force_stall", C.c_int, [C.c_void_p, C.c_int32]),
    ("mk_debug_prefill_marks", C.c_int, [C.c_void_p, C.POINTER(C.c_uint64), C.c_int32]),
    ("mk_debug_kv", C.c_int, [C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.POINTER(C.c_uint16),
                              C.POINTER(C.c_uint16)]),
    ("mk_debug_ts", C.c_int, [C.c_void_p, C.POINTER(C.c_uint64), C.c_int64]),
    ("mk_last_error", C.c_char_p, [C.c_void_p]),
    ("mk_destroy", None, [C.c_void_p]),
    ("mk_chain_create", C.c_int, [C.c_int32, C.c_int32, C.c_void_p, C.POINTER(mk_options), C.c_int, C.c_void_p,
                                  C.POINTER(C.c_void_p)]),
    ("mk_chain_run", C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p]),
    ("mk_chain_stats", C.c_int, [C.c_void_p, C.POINTER(mk_stats_t)]),
    ("mk_chain_read_trace", C.c_int, [C.c_void_p, C.POINTER(C.c_uint32), C.c_int64, C.POINTER(C.c_int64)]),
    ("mk_chain_last_error", C.c_char_p, [C.c_void_p]),
    ("mk_chain_destroy", None, [C.c_void_p]),
    ("mk_plan_check", C.c_int, [C.POINTER(mk_config), C.POINTER(mk_options), C.c_int32, C.POINTER(mk_plan_info),
                                C.POINTER(C.c_char_p)]),
]


def lib():
    """Load ``libmk.so`` (raises if it has not been built)."""
    global _lib
    if _lib is None:
        # torch first: libmk.so then binds to the HIP runtime torch ships, so
        # torch's streams and device pointers are valid in the library.
        import torch  # noqa: F401
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with `python -m decode_megakernel_wave_amd.build` "
                               "(there is no fallback path)")
        L = C.CDLL(_LIB_PATH)
        for name, res, args in SIGNATURES:
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(rc: int, ctx=None, chain: bool = False):
    if rc != MK_OK:
        L = lib()
        msg = (L.mk_chain_last_error(ctx) if chain else L.mk_last_error(ctx)) or b""
        raise MkError(rc, msg.decode(errors="replace"))


def make_config(model: inputs.ModelConfig, max_seq: int) -> mk_config:
    return mk_config(model.n_layers, model.d_model, model.n_heads, model.n_kv_heads, model.head_dim, model.ffn,
                     model.vocab, max_seq, model.rms_eps, model.rope_theta)


def mk_default_options(**overrides) -> mk_options:
    o = mk_options()
    _check(lib().mk_default_options(C.byref(o)))
    for k, v in overrides.items():
        setattr(o, k, int(v))
    return o


def _stream_handle(stream):
    if stream is not None:
        return C.c_void_p(int(stream))
    import torch
    return C.c_void_p(int(torch.cuda.current_stream().cuda_stream))


def mk_plan_check(model: inputs.ModelConfig, max_seq: int, n_cta: int, opts: mk_options | None = None) -> dict:
    """Build and check the schedule on the host (no GPU).  Raises MkError."""
    cfg = make_config(model, max_seq)
    info = mk_plan_info()
    msg = C.c_char_p()
    rc = lib().mk_plan_check(C.byref(cfg), C.byref(opts) if opts else None, n_cta, C.byref(info), C.byref(msg))
    if rc != MK_OK:
        raise MkError(rc, (msg.value or b"").decode())
    return {f: getattr(info, f) for f, _ in mk_plan_info._fields_}


def mk_create(model: inputs.ModelConfig, max_seq: int, opts: mk_options | None = None, device: int = 0,
              stream=None) -> C.c_void_p:
    cfg = make_config(model, max_seq)
    ctx = C.c_void_p()
    rc = lib().mk_create(C.byref(cfg), C.byref(opts) if opts else None, device, _stream_handle(stream), C.byref(ctx))
    _check(rc, None)
    return ctx


def _ptr(t) -> int:
    import torch
    if not (t.is_cuda and t.dtype == torch.float16 and t.is_contiguous()):
        raise ValueError("weights must be contiguous fp16 CUDA tensors")
    return t.data_ptr()


def mk_load_weights(ctx, w: dict) -> None:
    """``w``: the canonical layout of ``inputs.make_weights`` as torch fp16 CUDA tensors."""
    layers = w["layers"]
    n = len(layers)
    arrays = {}
    for key in ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down"):
        arrays[key] = (C.c_void_p * n)(*[_ptr(lw[key]) for lw in layers])
    mw = mk_weights(_ptr(w["embed"]), _ptr(w["final_norm"]), _ptr(w["lm_head"]),
                    *[C.cast(arrays[k], _PP) for k in ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm",
                                                       "w_gate", "w_up", "w_down")])
    _check(lib().mk_load_weights(ctx, C.byref(mw)), ctx)


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def mk_prefill(ctx, ids) -> int:
    ids = _i32(ids)
    t0 = C.c_int32()
    _check(lib().mk_prefill(ctx, ids.ctypes.data_as(C.POINTER(C.c_int32)), len(ids), C.byref(t0)), ctx)
    return int(t0.value)


def mk_decode(ctx, n_steps: int, vocab: int | None = None):
    """Returns ``tokens`` (int32 [n]) or ``(tokens, logits[n, vocab])`` when ``vocab`` is given."""
    toks = np.empty(n_steps, dtype=np.int32)
    logits = np.empty((n_steps, vocab), dtype=np.float32) if vocab else None
    lp = logits.ctypes.data_as(C.POINTER(C.c_float)) if logits is not None else None
    _check(lib().mk_decode(ctx, n_steps, toks.ctypes.data_as(C.POINTER(C.c_int32)), lp), ctx)
    return (toks, logits) if vocab else toks


def mk_decode_forced(ctx, tokens_in, vocab: int | None = None):
    tin = _i32(tokens_in)
    n = len(tin)
    toks = np.empty(n, dtype=np.int32)
    logits = np.empty((n, vocab), dtype=np.float32) if vocab else None
    lp = logits.ctypes.data_as(C.POINTER(C.c_float)) if logits is not None else None
    _check(lib().mk_decode_forced(ctx, n, tin.ctypes.data_as(C.POINTER(C.c_int32)),
                                  toks.ctypes.data_as(C.POINTER(C.c_int32)), lp), ctx)
    return (toks, logits) if vocab else toks


def mk_generate(ctx, ids, n_steps: int) -> np.ndarray:
    ids = _i32(ids)
    out = np.empty(n_steps + 1, dtype=np.int32)
    _check(lib().mk_generate(ctx, ids.ctypes.data_as(C.POINTER(C.c_int32)), len(ids), n_steps,
                             out.ctypes.data_as(C.POINTER(C.c_int32))), ctx)
    return out


def mk_kernel_name(ctx) -> str:
    """The monokernel the context launches (specialised or general)."""
    return (lib().mk_kernel_name(ctx) or b"").decode()


def mk_set_sampling(ctx, top_k: int = 1, temperature: float = 1.0, seed: int = 0) -> None:
    """Top-k / temperature sampling for later steps (top_k = 1: greedy)."""
    _check(lib().mk_set_sampling(ctx, int(top_k), float(temperature), int(seed) & 0xFFFFFFFFFFFFFFFF), ctx)


def mk_probe_launch(n_launches: int = 1000, device: int = 0, stream=None) -> dict:
    """Empty-kernel launch cost in host microseconds: back to back, and launch + synchronise."""
    a, b = C.c_double(), C.c_double()
    _check(lib().mk_probe_launch(device, _stream_handle(stream), n_launches, C.byref(a), C.byref(b)))
    return {"us_per_launch_pipelined": a.value, "us_per_launch_round_trip": b.value}


def mk_probe_read(buf, repeats: int = 5, device: int = 0, stream=None) -> float:
    """GB/s of nontemporal 16-byte reads over the CUDA tensor ``buf``."""
    g = C.c_double()
    _check(lib().mk_probe_read(device, _stream_handle(stream), C.c_void_p(buf.data_ptr()),
                               buf.numel() * buf.element_size(), repeats, C.byref(g)))
    return g.value


def mk_probe_handoff(mode: int, same_xcd: bool = False, rounds: int = 2000, device: int = 0, stream=None) -> dict:
    """Cross-workgroup handoff latency under weight streaming (see include/mk_diag.h)."""
    us, gbs, same = C.c_double(), C.c_double(), C.c_double()
    _check(lib().mk_probe_handoff(device, _stream_handle(stream), int(mode), int(bool(same_xcd)), int(rounds),
                                  C.byref(us), C.byref(gbs), C.byref(same)))
    return {"us_per_handoff": us.value, "stream_GB_per_s": gbs.value, "same_xcd_pairs": same.value}


def mk_probe_barrier(rounds: int = 1000, device: int = 0, stream=None) -> float:
    """Microseconds per naive atomic grid barrier (one workgroup per CU)."""
    u = C.c_double()
    _check(lib().mk_probe_barrier(device, _stream_handle(stream), rounds, C.byref(u)))
    return u.value


def mk_rewind(ctx, pos: int) -> None:
    _check(lib().mk_rewind(ctx, pos), ctx)


def mk_position(ctx):
    p, t = C.c_int32(), C.c_int32()
    _check(lib().mk_position(ctx, C.byref(p), C.byref(t)), ctx)
    return int(p.value), int(t.value)


def _stats_dict(s: mk_stats_t) -> dict:
    d = {f: getattr(s, f) for f, _ in mk_stats_t._fields_ if f != "fault"}
    d["fault"] = {f: getattr(s.fault, f) for f, _ in mk_fault._fields_}
    return d


def mk_stats(ctx) -> dict:
    s = mk_stats_t()
    _check(lib().mk_stats(ctx, C.byref(s)), ctx)
    return _stats_dict(s)


def mk_count_sentinels(ctx) -> int:
    n = C.c_int64()
    _check(lib().mk_count_sentinels(ctx, C.byref(n)), ctx)
    return int(n.value)


def mk_count_sentinels_noalloc(ctx) -> int:
    """mk_count_sentinels without any allocation (a static per-GPU counter); see include/mk_diag.h."""
    n = C.c_int64()
    _check(lib().mk_count_sentinels_noalloc(ctx, C.byref(n)), ctx)
    return int(n.value)


def mk_read_trace(ctx) -> np.ndarray:
    n = C.c_int64()
    _check(lib().mk_read_trace(ctx, None, 0, C.byref(n)), ctx)
    buf = np.zeros((n.value, 8), dtype=np.uint32)
    if n.value:
        _check(lib().mk_read_trace(ctx, buf.ctypes.data_as(C.POINTER(C.c_uint32)), n.value, C.byref(n)), ctx)
    return buf


def mk_debug_ts(ctx, grid: int, max_ins: int) -> np.ndarray:
    """Fine marks of step 0 of the last launch (recorded when MK_DEBUG_TS was set at launch):
    uint64 [grid][max_ins][8], 100 MHz device-clock ticks, 0 where not recorded."""
    buf = np.zeros((grid, max_ins, 8), dtype=np.uint64)
    _check(lib().mk_debug_ts(ctx, buf.ctypes.data_as(C.POINTER(C.c_uint64)), buf.size), ctx)
    return buf


def mk_debug_streams(ctx):
    b, o, n = C.c_void_p(), C.c_void_p(), C.c_void_p()
    _check(lib().mk_debug_streams(ctx, C.byref(b), C.byref(o), C.byref(n)), ctx)
    return b.value, o.value, n.value


def mk_debug_layout(ctx) -> list:
    off = (C.c_int64 * 16)()
    _check(lib().mk_debug_layout(ctx, off), ctx)
    return list(off)


def mk_debug_arena(ctx, word_off: int, n_words: int) -> np.ndarray:
    buf = np.zeros(n_words, dtype=np.uint32)
    _check(lib().mk_debug_arena(ctx, word_off, n_words, buf.ctypes.data_as(C.POINTER(C.c_uint32))), ctx)
    return buf


def mk_debug_progress(ctx, grid: int) -> np.ndarray:
    buf = np.zeros(grid, dtype=np.uint32)
    _check(lib().mk_debug_progress(ctx, buf.ctypes.data_as(C.POINTER(C.c_uint32)), grid), ctx)
    return buf


def mk_debug_kv(ctx, layer: int, kv_head: int, pos0: int, n: int, head_dim: int):
    """Cached K and V of positions [pos0, pos0 + n) of one layer and kv head: two float16 [n, head_dim] arrays."""
    k = np.zeros((n, head_dim), dtype=np.uint16)
    v = np.zeros((n, head_dim), dtype=np.uint16)
    _check(lib().mk_debug_kv(ctx, layer, kv_head, pos0, n, k.ctypes.data_as(C.POINTER(C.c_uint16)),
                             v.ctypes.data_as(C.POINTER(C.c_uint16))), ctx)
    return k.view(np.float16), v.view(np.float16)


def mk_debug_prefill_marks(ctx, n_layers: int) -> np.ndarray:
    """Device-clock ticks (100 MHz) when the last prefill launch left each grid barrier: 1 + 5 n_layers."""
    buf = np.zeros(1 + 5 * n_layers, dtype=np.uint64)
    _check(lib().mk_debug_prefill_marks(ctx, buf.ctypes.data_as(C.POINTER(C.c_uint64)), buf.size), ctx)
    return buf


def mk_debug_force_stall(ctx, cta: int) -> None:
    """Arm the failure-path test for the next launch (see include/mk_diag.h)."""
    _check(lib().mk_debug_force_stall(ctx, int(cta)), ctx)


def mk_last_error(ctx=None) -> str:
    return (lib().mk_last_error(ctx) or b"").decode(errors="replace")


def mk_destroy(ctx) -> None:
    if ctx:
        lib().mk_destroy(ctx)


def mk_chain_create(n: int, stages: int, W, opts: mk_options | None = None, device: int = 0, stream=None):
    """``W``: fp16 CUDA tensor [stages, n, n]."""
    ch = C.c_void_p()
    rc = lib().mk_chain_create(n, stages, C.c_void_p(_ptr(W)), C.byref(opts) if opts else None, device,
                               _stream_handle(stream), C.byref(ch))
    _check(rc, None, chain=True)
    return ch


def mk_chain_run(ch, x0, y) -> None:
    """``x0``: fp32 CUDA tensor [n]; ``y``: fp32 CUDA tensor [stages, n] (written)."""
    _check(lib().mk_chain_run(ch, C.c_void_p(x0.data_ptr()), C.c_void_p(y.data_ptr())), ch, chain=True)


def mk_chain_stats(ch) -> dict:
    s = mk_stats_t()
    _check(lib().mk_chain_stats(ch, C.byref(s)), ch, chain=True)
    return _stats_dict(s)


def mk_chain_read_trace(ch) -> np.ndarray:
    n = C.c_int64()
    _check(lib().mk_chain_read_trace(ch, None, 0, C.byref(n)), ch, chain=True)
    buf = np.zeros((n.value, 8), dtype=np.uint32)
    if n.value:
        _check(lib().mk_chain_read_trace(ch, buf.ctypes.data_as(C.POINTER(C.c_uint32)), n.value, C.byref(n)),
               ch, chain=True)
    return buf


def mk_chain_destroy(ch) -> None:
    if ch:
        lib().mk_chain_destroy(ch)
