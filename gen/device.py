"""Upload generated inputs to device memory slice by slice (pinned staging),
so multi-GiB tensors never exist whole in host memory. Plumbing only."""
import numpy as np
import torch

import gen

_SLICE = 1 << 27  # elements per staging slice (256 MiB of bf16)


def _stage(n):
    return torch.empty(n, dtype=torch.int16, pin_memory=True)


def normal_to_device(seed, stream, shape, device="cuda", scale=1.0):
    """A [*shape] bf16 device tensor holding elements 0.. of a normal stream."""
    n = int(np.prod(shape))
    dst = torch.empty(n, dtype=torch.int16, device=device)
    stage = _stage(min(n, _SLICE))
    sv = stage.numpy().view(np.uint16)
    for e0 in range(0, n, _SLICE):
        m = min(_SLICE, n - e0)
        gen.normal(seed, stream, (m,), e0=e0, scale=scale, out=sv[:m])
        dst[e0:e0 + m].copy_(stage[:m], non_blocking=False)
    return dst.view(torch.bfloat16).view(*shape)


def idx_keys_to_device(seed, batch, L, d=64, window=0, r=4, device="cuda"):
    """Indexer keys [batch, L, d] (with planted needles) as a bf16 device tensor."""
    dst = torch.empty((batch, L, d), dtype=torch.int16, device=device)
    rows = max(1, _SLICE // d)
    stage = _stage(min(L, rows) * d)
    sv = stage.numpy().view(np.uint16)
    for b in range(batch):
        for s0 in range(0, L, rows):
            ns = min(rows, L - s0)
            gen.idx_keys(seed, b, L, s0, ns, d, window, r, out=sv[:ns * d].reshape(ns, d))
            dst[b, s0:s0 + ns].copy_(stage[:ns * d].view(ns, d), non_blocking=False)
    return dst.view(torch.bfloat16)
