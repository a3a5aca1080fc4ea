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


def paged_batch_layout(W):
    """Page table of a packed paged batch (``gen.configs.PagedBatch``): the
    pages of every sequence in one pool, dealt in a seeded shuffled order.
    Returns (table [B, max_pages] int32, n_pages, max_len)."""
    page = W.page_size
    L = W.lengths
    max_len = (max(L) + page - 1) // page * page
    pages_of = [(x + page - 1) // page for x in L]
    n_pages = sum(pages_of)
    perm = np.random.default_rng(W.seed).permutation(n_pages).astype(np.int32)
    table = np.zeros((W.batch, max_len // page), np.int32)
    nxt = 0
    for b in range(W.batch):
        table[b, :pages_of[b]] = perm[nxt:nxt + pages_of[b]]
        nxt += pages_of[b]
    return table, n_pages, max_len


def paged_batch_to_device(W, device="cuda"):
    """Device inputs of a packed paged batch: K/V pools [n_pages, page, Hkv, D]
    (streams 2, 3 over the pool), packed Q [total, Hq, D] and indexer queries
    [total, Hi, di] (streams 1, 4 over the packed rows), indexer keys
    [B, max_len, di] (stream 5 with needles), the page table, cu_q and q_pos0."""
    table, n_pages, max_len = paged_batch_layout(W)
    total = sum(W.new)
    d = {
        "table": torch.from_numpy(table).to(device),
        "kpool": normal_to_device(W.seed, 2, (n_pages, W.page_size, W.Hkv, W.D), device),
        "vpool": normal_to_device(W.seed, 3, (n_pages, W.page_size, W.Hkv, W.D), device),
        "Q": normal_to_device(W.seed, 1, (total, W.Hq, W.D), device),
        "iq": normal_to_device(W.seed, 4, (total, W.Hi, W.di), device),
        "ik": idx_keys_to_device(W.seed, W.batch, max_len, W.di, W.needle_window, W.r, device),
        "cu": torch.tensor(np.concatenate([[0], np.cumsum(W.new)]), dtype=torch.int32, device=device),
        "q_pos0": torch.tensor(W.prefix, dtype=torch.int32, device=device),
        "total": total, "max_len": max_len, "n_pages": n_pages, "table_host": table,
    }
    return d


def paged_sequence_host(W, table, b, stream, n_tok):
    """Tokens 0 .. n_tok - 1 of sequence b of a paged pool stream (2 = K,
    3 = V), gathered from their pages into one contiguous [n_tok, Hkv, D]
    array of bf16 bits (host)."""
    page = W.page_size
    row = W.Hkv * W.D
    out = np.empty((n_tok, W.Hkv, W.D), np.uint16)
    for p in range((n_tok + page - 1) // page):
        s0, s1 = p * page, min(n_tok, (p + 1) * page)
        phys = int(table[b, p])
        gen.normal(W.seed, stream, (s1 - s0, W.Hkv, W.D), e0=phys * page * row, out=out[s0:s1])
    return out
