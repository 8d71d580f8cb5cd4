"""Full-recompute brute force of the decoder, used to pin ``oracle.decoder``.

TEST INFRASTRUCTURE.  Only the test suite may import this module.

It re-derives every logit from scratch over the whole prefix, with no KV cache
and with formulations deliberately different from ``oracle.decoder``:

* RoPE as multiplication of the complex numbers u_i + j u_{i+hd/2} by
  exp(j p w_i) (the same rotation of each rotate-half pair);
* attention as one masked [T, T] score matrix per head, softmax from scipy;
* grouped-query attention by repeating each kv head over its query group;
* silu as z * expit(z), RMSNorm through the vector 2-norm.

Everything is float64 except the fp16 weights and the fp16 rounding of the
cached K and V, which are part of the workload's definition.
"""
from __future__ import annotations

import numpy as np
from scipy.special import expit, softmax


def _rms(X, g, eps):
    n = X.shape[-1]
    r = np.linalg.norm(X, axis=-1, keepdims=True) / np.sqrt(n)
    return X / np.sqrt(r * r + eps) * g


def _rope_complex(U, theta):
    """U: [T, heads, hd]; position of row t is t."""
    T, _, hd = U.shape
    half = hd // 2
    w = np.array([theta ** (-(2.0 * i) / hd) for i in range(half)])
    rot = np.exp(1j * np.outer(np.arange(T), w))[:, None, :]
    z = (U[..., :half] + 1j * U[..., half:]) * rot
    return np.concatenate([z.real, z.imag], axis=-1)


def forward_all(weights: dict, ids, n_heads: int, n_kv_heads: int,
                rms_eps: float = 1e-5, rope_theta: float = 10000.0) -> np.ndarray:
    """Logits at every position of ``ids`` (shape [T, V]), recomputed from scratch."""
    ids = np.asarray(ids)
    T = len(ids)
    X = weights["embed"][ids].astype(np.float64)
    mask = np.triu(np.ones((T, T), dtype=bool), k=1)
    rep = n_heads // n_kv_heads
    for lw in weights["layers"]:
        W = {k: np.asarray(v, dtype=np.float64) for k, v in lw.items()}
        hd = W["wq"].shape[0] // n_heads
        H = _rms(X, W["attn_norm"], rms_eps)
        Q = _rope_complex((H @ W["wq"].T).reshape(T, n_heads, hd), rope_theta)
        K = _rope_complex((H @ W["wk"].T).reshape(T, n_kv_heads, hd), rope_theta)
        V = (H @ W["wv"].T).reshape(T, n_kv_heads, hd)
        K = K.astype(np.float16).astype(np.float64)
        V = V.astype(np.float16).astype(np.float64)
        K = np.repeat(K, rep, axis=1)
        V = np.repeat(V, rep, axis=1)
        scores = np.einsum("thd,shd->hts", Q, K) / np.sqrt(hd)
        scores[:, mask] = -np.inf
        A = softmax(scores, axis=-1)
        O = np.einsum("hts,shd->thd", A, V).reshape(T, n_heads * hd)
        X = X + O @ W["wo"].T
        H = _rms(X, W["mlp_norm"], rms_eps)
        G = H @ W["w_gate"].T
        X = X + ((G * expit(G)) * (H @ W["w_up"].T)) @ W["w_down"].T
    Xf = _rms(X, np.asarray(weights["final_norm"], dtype=np.float64), rms_eps)
    return Xf @ np.asarray(weights["lm_head"], dtype=np.float64).T


def chain_loops(W, x0):
    """GEMV-tanh chain with explicit Python loops (tiny sizes only)."""
    import math
    y = [float(v) for v in x0]
    out = []
    for Wi in W:
        Wi = Wi.astype(np.float64)
        y = [math.tanh(sum(float(Wi[r, c]) * y[c] for c in range(len(y))))
             for r in range(Wi.shape[0])]
        out.append(y)
    return np.array(out)
