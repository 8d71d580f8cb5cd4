"""Seeded synthetic inputs for the decoder and the GEMV-tanh chain.

This module only draws random numbers and lays them out; it holds none of the
decoder's arithmetic.  Both the HIP path (through the Python binding) and the
CPU oracle consume exactly the bytes produced here.

Workloads (shapes and distributions) follow the decode monokernel workload of
"7 - AMD et le monokernel" (section 7.1: a 2B-parameter FP16 model decoded at
batch 1): random-init fp16 weights ~ N(0, 0.02^2), RMSNorm gains 1.0, prompt
ids uniform over the vocabulary.  There are no trained weights or datasets.

Determinism: every tensor is split into fixed blocks of ``_BLOCK`` elements and
block ``b`` of tensor ``t`` is drawn from ``PCG64(SeedSequence([seed, t, b]))``,
so the bytes do not depend on the number of worker threads.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_BLOCK = 1 << 22


@dataclasses.dataclass(frozen=True)
class ModelConfig:
    """Dimensions of a Llama-style decoder (pre-norm, RoPE, SwiGLU, untied head)."""

    name: str
    n_layers: int
    d_model: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    rms_eps: float = 1e-5
    rope_theta: float = 10000.0

    @property
    def q_dim(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    def n_params(self) -> int:
        d, f = self.d_model, self.ffn
        per_layer = 2 * d + (self.q_dim + 2 * self.kv_dim) * d + d * self.q_dim + 3 * f * d
        return self.n_layers * per_layer + 2 * self.vocab * d + d


@dataclasses.dataclass(frozen=True)
class Workload:
    """A decode workload: model, prompt length and number of greedy decode steps."""

    model: ModelConfig
    prompt_len: int
    decode_steps: int

    @property
    def max_seq(self) -> int:
        return self.prompt_len + self.decode_steps + 1


TINY = ModelConfig("tiny", n_layers=2, d_model=256, n_heads=4, n_kv_heads=4,
                   head_dim=64, ffn=688, vocab=1024)
M05 = ModelConfig("0.5b", n_layers=24, d_model=1024, n_heads=16, n_kv_heads=8,
                  head_dim=64, ffn=2816, vocab=32000)
M2B = ModelConfig("2b", n_layers=24, d_model=2048, n_heads=16, n_kv_heads=8,
                  head_dim=128, ffn=8192, vocab=128256)
# One GPU's share of the ~2B decoder under 8-way tensor parallelism: 2 query
# heads and 1 kv head (512 QKV rows), a 1024-row slice of gate/up with the
# matching 1024 input columns of down, the 256 input columns of O for those
# heads, and 16032 of the 128256 LM-head rows.  Each partial residual would be
# summed over the 8 GPUs; with the other GPUs' slots empty that sum is the
# local value, so the shard runs as a decoder of its own with these dims.
M2B_TP8 = ModelConfig("2b-tp8-shard", n_layers=24, d_model=2048, n_heads=2, n_kv_heads=1,
                      head_dim=128, ffn=1024, vocab=16032)

# Two layers of the ~2B decoder's geometry (d 2048, 16 query / 8 kv heads of
# 128, vocab cut to 4096): small enough for the float64 oracle at long
# prompts, shaped like the ~2B model in every GEMV and attention path.  The
# first keeps the ~2B SwiGLU width (8192); the second narrows it to 2048 so the
# oracle can prefill an 8192-token prompt in test time.
M2B_GEOM_L2 = ModelConfig("2b-geometry-2-layers", n_layers=2, d_model=2048, n_heads=16, n_kv_heads=8,
                          head_dim=128, ffn=8192, vocab=4096)
M2B_GEOM_L2_NARROW = ModelConfig("2b-geometry-2-layers-ffn2048", n_layers=2, d_model=2048, n_heads=16,
                                 n_kv_heads=8, head_dim=128, ffn=2048, vocab=4096)

WORKLOADS = {
    "tiny": Workload(TINY, 32, 16),
    "0.5b": Workload(M05, 128, 256),
    "2b": Workload(M2B, 512, 512),
    "2b-long": Workload(M2B, 8192, 256),
    "2b-tp8-shard": Workload(M2B_TP8, 512, 512),
}

# GEMV-tanh chain: 256 dependent stages y_i = tanh(W_i y_{i-1}), W_i 2048x2048.
CHAIN_N = 2048
CHAIN_STAGES = 256

# Stable tensor ids for seeding.
_GLOBAL_IDS = {"embed": 1, "lm_head": 2, "final_norm": 3}
_LAYER_IDS = {"attn_norm": 0, "wq": 1, "wk": 2, "wv": 3, "wo": 4,
              "mlp_norm": 5, "w_gate": 6, "w_up": 7, "w_down": 8}
LAYER_KEYS = tuple(_LAYER_IDS)


def _tensor_id(name: str, layer: int | None) -> int:
    if layer is None:
        return _GLOBAL_IDS[name]
    return 100 + 16 * layer + _LAYER_IDS[name]


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _normal_fp16(shape, std: float, seed: int, tid: int, mean: float = 0.0) -> np.ndarray:
    """Draw N(mean, std^2), round to fp16 (numpy's round-to-nearest-even)."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float16)
    nblk = (n + _BLOCK - 1) // _BLOCK

    def fill(b):
        lo, hi = b * _BLOCK, min(n, (b + 1) * _BLOCK)
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tid, b])))
        a = rng.standard_normal(hi - lo, dtype=np.float32)
        a *= np.float32(std)
        if mean:
            a += np.float32(mean)
        out[lo:hi] = a.astype(np.float16)

    if nblk == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(fill, range(nblk)))
    return out.reshape(shape)


def make_weights(cfg: ModelConfig, seed: int = 0, std: float = 0.02,
                 gains: str = "ones") -> dict:
    """Random-init fp16 weights in canonical row-major ``[out, in]`` layout.

    Returns ``{"embed": [V,d], "lm_head": [V,d], "final_norm": [d],
    "layers": [{"attn_norm","wq","wk","wv","wo","mlp_norm","w_gate","w_up","w_down"}]}``.
    ``gains="ones"`` sets every RMSNorm gain to exactly 1.0; ``"perturbed"``
    draws them from 1 + N(0, 0.1^2) (used to expose indexing mistakes).
    """
    d, f = cfg.d_model, cfg.ffn

    def gain(name, layer):
        if gains == "ones":
            return np.ones(d, dtype=np.float16)
        return _normal_fp16((d,), 0.1, seed, _tensor_id(name, layer), mean=1.0)

    w = {
        "embed": _normal_fp16((cfg.vocab, d), std, seed, _tensor_id("embed", None)),
        "lm_head": _normal_fp16((cfg.vocab, d), std, seed, _tensor_id("lm_head", None)),
        "final_norm": gain("final_norm", None),
        "layers": [],
    }
    shapes = {"wq": (cfg.q_dim, d), "wk": (cfg.kv_dim, d), "wv": (cfg.kv_dim, d),
              "wo": (d, cfg.q_dim), "w_gate": (f, d), "w_up": (f, d), "w_down": (d, f)}
    for layer in range(cfg.n_layers):
        lw = {"attn_norm": gain("attn_norm", layer), "mlp_norm": gain("mlp_norm", layer)}
        for k, shp in shapes.items():
            lw[k] = _normal_fp16(shp, std, seed, _tensor_id(k, layer))
        w["layers"].append(lw)
    return w


def make_prompt(cfg: ModelConfig, n: int, seed: int = 1) -> np.ndarray:
    """``n`` token ids drawn uniformly from ``[0, vocab)``, as int32."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 7])))
    return rng.integers(0, cfg.vocab, size=n, dtype=np.int64).astype(np.int32)


def make_chain_weights(n: int = CHAIN_N, stages: int = CHAIN_STAGES, seed: int = 0,
                       std: float = 0.02) -> np.ndarray:
    """``stages`` fp16 matrices ``[stages, n, n]`` ~ N(0, std^2), row-major ``[out, in]``."""
    return _normal_fp16((stages, n, n), std, seed, 9000 + n)


def make_chain_x0(n: int = CHAIN_N, seed: int = 2) -> np.ndarray:
    """Chain input x0 ~ N(0, 1) as float32."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 11])))
    return rng.standard_normal(n, dtype=np.float32)
