"""CPU oracle: the batch-1 Llama-style decode step, written out plainly in float64.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this module.  It shares no code with the HIP path.

What it computes
----------------
"7 - AMD et le monokernel" (section 7.1) describes a single persistent kernel
that runs prefill, decode and sampling of a 2B-parameter FP16 model at batch 1;
"8 - Ecrire son megakernel" (section 8.2, the opcode list of the interpreter)
names the fused steps of one decode step: RMSNorm+QKV+RoPE, attention, the
attention reduction, O-projection, MLP up/gate, MLP down and the LM head.  The
pages do not write the decoder's formulas; this oracle takes the plain Llama
reading of those names:

* x = E[t] (fp16 embedding row) for token t at 0-based position p;
* per layer: h = RMSNorm(x; g1); q, k, v = Wq h, Wk h, Wv h; RoPE on q and k
  (rotate-half pairs (i, i + hd/2), angle p * theta^(-2i/hd)); K, V stored in an
  fp16 cache (round to nearest even); causal softmax attention with scale
  1/sqrt(hd), kv head of q head j = floor(j * n_kv / n_q); x += Wo o;
  h = RMSNorm(x; g2); x += Wd (silu(Wg h) * (Wu h));
* logits = Wlm RMSNorm(x; gf); greedy token = argmax, lowest index on ties.

All arithmetic is float64 except the two storage formats the workload fixes:
fp16 weights (exact in float64) and the fp16 KV cache.  Matrix products use
numpy's BLAS as a library primitive; every element is an ordinary dot product.
"""
from __future__ import annotations

import numpy as np

LAYER_KEYS = ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down")


def fp16_round(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest fp16 (ties to even); return float64."""
    with np.errstate(over="ignore"):       # values beyond 65520 round to +-inf
        return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm along the last axis: x * (mean(x^2) + eps)^(-1/2) * g."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * g


def rope_angles(pos, head_dim: int, theta: float) -> np.ndarray:
    """Angles p * theta^(-2i/hd) for i in [0, hd/2); shape [..., hd/2]."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    omega = theta ** (-2.0 * i / head_dim)
    return np.multiply.outer(np.asarray(pos, dtype=np.float64), omega)


def rope_rotate(u: np.ndarray, pos, theta: float) -> np.ndarray:
    """Rotate each (u_i, u_{i+hd/2}) pair of the last axis by its RoPE angle.

    ``u`` is [..., hd] with a scalar ``pos``, or [P, n_heads, hd] with ``pos`` of
    shape [P] (one position per row).
    """
    hd = u.shape[-1]
    half = hd // 2
    ang = rope_angles(pos, hd, theta)
    if np.ndim(pos) > 0:          # one position per row: broadcast over the head axis
        ang = ang[..., None, :]
    c, s = np.cos(ang), np.sin(ang)
    a = u[..., :half]
    b = u[..., half:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def softmax(s: np.ndarray) -> np.ndarray:
    """Softmax along the last axis (max subtracted first)."""
    e = np.exp(s - np.max(s, axis=-1, keepdims=True))
    return e / np.sum(e, axis=-1, keepdims=True)


def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z / (1 + exp(-z))."""
    return z / (1.0 + np.exp(-z))


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray) -> np.ndarray:
    """One query head over T cached positions: softmax(K q / sqrt(hd)) V."""
    a = softmax(K @ q / np.sqrt(q.shape[-1]))
    return a @ V


class Decoder:
    """KV-cached decoder.  ``step`` runs one token; ``prefill`` runs a prompt.

    ``weights`` is the canonical fp16 layout (``embed``/``lm_head`` [V, d],
    ``final_norm`` [d], per-layer ``wq`` [nq*hd, d], ``wk``/``wv`` [nkv*hd, d],
    ``wo`` [d, nq*hd], ``w_gate``/``w_up`` [f, d], ``w_down`` [d, f], norms [d]).
    """

    def __init__(self, weights: dict, n_heads: int, n_kv_heads: int,
                 rms_eps: float = 1e-5, rope_theta: float = 10000.0, max_seq: int = 4096):
        f64 = lambda a: np.asarray(a, dtype=np.float64)  # noqa: E731  (fp16 -> f64 is exact)
        self.embed = weights["embed"]                       # rows converted on use
        self.lm_head = f64(weights["lm_head"])
        self.final_norm = f64(weights["final_norm"])
        self.layers = [{k: f64(lw[k]) for k in LAYER_KEYS} for lw in weights["layers"]]
        self.n_heads, self.n_kv = n_heads, n_kv_heads
        self.eps, self.theta = rms_eps, rope_theta
        self.d = self.final_norm.shape[0]
        self.hd = self.layers[0]["wq"].shape[0] // n_heads
        self.max_seq = max_seq
        self.group = n_heads // n_kv_heads
        nl = len(self.layers)
        self.K = np.zeros((nl, max_seq, n_kv_heads, self.hd))
        self.V = np.zeros((nl, max_seq, n_kv_heads, self.hd))

    def kv_head_of(self, j: int) -> int:
        return j * self.n_kv // self.n_heads

    # -- one token ---------------------------------------------------------
    def step(self, token: int, pos: int) -> np.ndarray:
        """Run token ``token`` at position ``pos``; return the float64 logits."""
        if not 0 <= pos < self.max_seq:
            raise ValueError("position outside the cache")
        x = np.asarray(self.embed[token], dtype=np.float64)
        for li, L in enumerate(self.layers):
            h = rmsnorm(x, L["attn_norm"], self.eps)
            q = (L["wq"] @ h).reshape(self.n_heads, self.hd)
            k = (L["wk"] @ h).reshape(self.n_kv, self.hd)
            v = (L["wv"] @ h).reshape(self.n_kv, self.hd)
            q = rope_rotate(q, pos, self.theta)
            k = rope_rotate(k, pos, self.theta)
            self.K[li, pos] = fp16_round(k)
            self.V[li, pos] = fp16_round(v)
            o = np.empty((self.n_heads, self.hd))
            for j in range(self.n_heads):
                g = self.kv_head_of(j)
                o[j] = attend(q[j], self.K[li, :pos + 1, g], self.V[li, :pos + 1, g])
            x = x + L["wo"] @ o.reshape(-1)
            h = rmsnorm(x, L["mlp_norm"], self.eps)
            x = x + L["w_down"] @ (silu(L["w_gate"] @ h) * (L["w_up"] @ h))
        return self.lm_head @ rmsnorm(x, self.final_norm, self.eps)

    # -- a whole prompt, layer by layer -----------------------------------
    def prefill(self, ids) -> np.ndarray:
        """Run positions 0..P-1 of ``ids``; fill the cache; return logits at P-1."""
        ids = np.asarray(ids)
        P = len(ids)
        if not 1 <= P <= self.max_seq:
            raise ValueError("prompt length outside the cache")
        pos = np.arange(P)
        X = np.asarray(self.embed[ids], dtype=np.float64)        # [P, d]
        causal = np.tril(np.ones((P, P), dtype=bool))
        for li, L in enumerate(self.layers):
            H = rmsnorm(X, L["attn_norm"], self.eps)
            Q = (H @ L["wq"].T).reshape(P, self.n_heads, self.hd)
            Kx = (H @ L["wk"].T).reshape(P, self.n_kv, self.hd)
            Vx = (H @ L["wv"].T).reshape(P, self.n_kv, self.hd)
            Q = rope_rotate(Q, pos, self.theta)
            Kx = rope_rotate(Kx, pos, self.theta)
            self.K[li, :P] = fp16_round(Kx)
            self.V[li, :P] = fp16_round(Vx)
            O = np.empty((P, self.n_heads, self.hd))
            for j in range(self.n_heads):
                g = self.kv_head_of(j)
                S = Q[:, j] @ self.K[li, :P, g].T / np.sqrt(self.hd)   # [P, P]
                S = np.where(causal, S, -np.inf)
                O[:, j] = softmax(S) @ self.V[li, :P, g]
            X = X + O.reshape(P, -1) @ L["wo"].T
            H = rmsnorm(X, L["mlp_norm"], self.eps)
            X = X + (silu(H @ L["w_gate"].T) * (H @ L["w_up"].T)) @ L["w_down"].T
        return self.lm_head @ rmsnorm(X[-1], self.final_norm, self.eps)

    # -- drivers -------------------------------------------------------------
    def greedy(self, ids, n_steps: int):
        """Prefill ``ids`` then decode ``n_steps`` greedy tokens.

        Returns ``(t0, tokens[n_steps], logits[n_steps, V])``: ``t0`` is the
        argmax after the prompt; decode step s consumes the previous token at
        position P + s and its logits are ``logits[s]``.
        """
        P = len(ids)
        t = int(np.argmax(self.prefill(ids)))
        t0 = t
        toks, logs = [], []
        for s in range(n_steps):
            lg = self.step(t, P + s)
            t = int(np.argmax(lg))
            toks.append(t)
            logs.append(lg)
        return t0, np.array(toks, dtype=np.int32), np.array(logs)


def top2_margin(logits: np.ndarray) -> np.ndarray:
    """Difference between the largest and second-largest logit along the last axis."""
    part = np.partition(logits, -2, axis=-1)
    return part[..., -1] - part[..., -2]
