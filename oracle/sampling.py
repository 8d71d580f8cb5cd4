"""CPU oracle: drawing one token from a logit vector by top-k / temperature sampling.

TEST INFRASTRUCTURE.  Only the test suite may import this module.  It shares no
code with the HIP path.

What it computes
----------------
"7 - AMD et le monokernel" (section 7.1) lists sampling ("échantillonnage")
among what the single persistent kernel does, without saying how.  This oracle
takes the plain reading of temperature / top-k sampling:

* candidates: the k largest logits, ordered by logit, larger first; equal
  logits in order of increasing token index (the order greedy decoding uses);
* weights w_i = exp((z_i - z_max) / T) over the candidates (temperature T > 0);
* a uniform u in [0, 1): the first 32-bit output word of Philox4x32-10 (Salmon,
  Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC11)
  with key (seed mod 2^32, seed div 2^32) and counter (p, 0, 0, 0), where p is
  the 0-based position of the token the step consumes, divided by 2^32;
* the token: the first candidate whose running weight sum exceeds u * sum(w)
  (inverse-CDF draw); the last candidate if rounding leaves none.

k = 1 is greedy decoding whatever T is.  Arithmetic is float64; the RNG is exact
integer arithmetic.
"""
from __future__ import annotations

import numpy as np

# Philox4x32 round multipliers and key increments (the published constants)
PHILOX_M0, PHILOX_M1 = 0xD2511F53, 0xCD9E8D57
PHILOX_W0, PHILOX_W1 = 0x9E3779B9, 0xBB67AE85
MASK32 = 0xFFFFFFFF


def philox4x32_10(counter, key):
    """Philox4x32 with 10 rounds: 4 counter words, 2 key words -> 4 output words.

    One round: (hi0, lo0) = M0 * c0 and (hi1, lo1) = M1 * c2 as 64-bit
    products; c <- (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0).  The key is
    advanced by (W0, W1) between rounds.
    """
    c = [int(x) & MASK32 for x in counter]
    k = [int(x) & MASK32 for x in key]
    for r in range(10):
        if r:
            k = [(k[0] + PHILOX_W0) & MASK32, (k[1] + PHILOX_W1) & MASK32]
        p0 = PHILOX_M0 * c[0]
        p1 = PHILOX_M1 * c[2]
        c = [(p1 >> 32) ^ c[1] ^ k[0], p1 & MASK32, (p0 >> 32) ^ c[3] ^ k[1], p0 & MASK32]
    return c


def uniform(seed: int, position: int) -> float:
    """u in [0, 1) for the step that consumes the token at `position`."""
    w = philox4x32_10((position, 0, 0, 0), (seed & MASK32, (seed >> 32) & MASK32))[0]
    return w / 4294967296.0


def top_k_order(logits: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest logits, larger first, equal logits by increasing index."""
    z = np.asarray(logits, dtype=np.float64)
    order = np.lexsort((np.arange(z.size), -z))  # primary key: -z, then the index
    return order[:k]


def sample(logits: np.ndarray, k: int, temperature: float, u: float):
    """(token, candidates, cumulative weights, total weight) of one draw."""
    cand = top_k_order(logits, k)
    z = np.asarray(logits, dtype=np.float64)[cand]
    w = np.exp((z - z[0]) / temperature)
    cum = np.cumsum(w)
    total = cum[-1]
    hit = np.nonzero(cum > u * total)[0]
    i = int(hit[0]) if hit.size else k - 1
    return int(cand[i]), cand, cum, float(total)


def draw_ambiguity(logits: np.ndarray, k: int, temperature: float, u: float) -> float:
    """How close a draw is to flipping: the smallest of (a) the distance of u * total from
    a running-sum boundary, relative to the total, and (b) the logit gap between the k-th
    and the (k+1)-th candidates (a different candidate set).  Tests skip draws where this
    is within the GPU's rounding."""
    _, cand, cum, total = sample(logits, k, temperature, u)
    a = float(np.min(np.abs(cum - u * total)) / total)
    z = np.sort(np.asarray(logits, dtype=np.float64))[::-1]
    b = float(z[k - 1] - z[k]) if k < z.size else np.inf
    return min(a, b)
