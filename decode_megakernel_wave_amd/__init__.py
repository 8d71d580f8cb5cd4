"""MI355X-native batch-1 decode monokernel (gfx950 HIP) behind a C ABI.

``capi`` binds ``include/mk.h`` one function per entry point; ``inputs``
draws the seeded synthetic workloads.  The HIP library ``libmk.so`` is loaded
on first use; there is no other compute path.
"""
from . import inputs  # noqa: F401
from .capi import *  # noqa: F401,F403
from .capi import MkError, lib  # noqa: F401


def to_device(weights: dict, device: int = 0) -> dict:
    """Copy an ``inputs.make_weights`` dict of fp16 numpy arrays to torch CUDA tensors."""
    import torch
    dev = torch.device("cuda", device)
    t = lambda a: torch.from_numpy(a).to(dev)  # noqa: E731
    out = {k: t(v) for k, v in weights.items() if k != "layers"}
    out["layers"] = [{k: t(v) for k, v in lw.items()} for lw in weights["layers"]]
    return out
