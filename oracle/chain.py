"""CPU oracle for the dependent GEMV-tanh chain, in float64.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this module.  It shares no code with the HIP path.

The chain is the synchronisation/streaming microbenchmark of the decode
monokernel: stage i computes y_i = tanh(W_i y_{i-1}) from the previous stage's
whole output, so every stage boundary is a grid-wide data dependency.  This is
the setting in which "7 - AMD et le monokernel" (section 7.3, the measured-gain
table) compares an atomic grid synchronisation with the NaN sentinel.  Each
y_i element is one float64 dot product of an fp16 row with y_{i-1}, then tanh.
"""
from __future__ import annotations

import numpy as np


def chain(W: np.ndarray, x0: np.ndarray) -> np.ndarray:
    """Return y[S, n] with y[i] = tanh(W[i] @ y[i-1]) and y[-1] := x0."""
    W = np.asarray(W)
    y = np.asarray(x0, dtype=np.float64)
    out = np.empty((W.shape[0], W.shape[1]))
    for i in range(W.shape[0]):
        y = np.tanh(W[i].astype(np.float64) @ y)
        out[i] = y
    return out
