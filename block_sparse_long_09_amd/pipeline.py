"""The QSA hot path as one call per prefill chunk or decode step.

Sequence of library calls (every step runs in the HIP kernels of libqsa.so):
  prefill chunk: qsa_compress_keys (the chunk's new complete blocks)
                 -> qsa_index_topk -> qsa_sparse_attn_prefill
  decode step:   qsa_index_topk (n_q = 1 per sequence at kv_len - 1)
                 -> qsa_sparse_attn_decode
  packed batch:  qsa_compress_keys per sequence -> qsa_index_topk_varlen
                 -> qsa_sparse_attn_prefill_paged (new rows of several
                 sequences appended to cached prefixes, K/V in pages)
  long prefill:  the prefill chunk's calls for each chunk in turn, chunk c's
                 attention on one stream beside chunk c + 1's compression and
                 indexer on another (ChunkedPrefill)
The objects below only own the caller-side buffers (workspaces, selections,
outputs) so that repeated calls allocate nothing.
"""
import torch

from . import (attn_desc, index_desc, qsa_compress_keys, qsa_index_topk, qsa_index_topk_varlen,
               qsa_index_topk_varlen_workspace_size, qsa_index_topk_workspace_size, qsa_sparse_attn_decode,
               qsa_sparse_attn_prefill, qsa_sparse_attn_prefill_paged, qsa_sparse_attn_workspace_size, workspace)


class PrefillPath:
    """Causal prefill of up to `n_q_max` queries against a prefix of at most
    `max_len` tokens, for one sequence."""

    def __init__(self, Hq, Hkv, Hi, r=4, k=512, n_q_max=8192, max_len=8192, D=128, di=64, device="cuda"):
        self.r, self.k = r, k
        self.idesc = index_desc(r, k, Hi, di)
        self.adesc = attn_desc(Hq, Hkv, D)
        self.ws_index = workspace(qsa_index_topk_workspace_size(self.idesc, 1, n_q_max, max_len), device)
        self.ws_attn = workspace(qsa_sparse_attn_workspace_size(self.adesc, 1, n_q_max, k, r), device)
        self.sel = torch.empty((n_q_max, k), dtype=torch.int32, device=device)
        self.cnt = torch.empty((n_q_max,), dtype=torch.int32, device=device)
        self.out = torch.empty((n_q_max, Hq, D), dtype=torch.bfloat16, device=device)
        self.lse = torch.empty((n_q_max, Hq), dtype=torch.float32, device=device)
        self.pos = torch.zeros((1,), dtype=torch.int32, device=device)
        self.device = device

    def compress(self, idx_k, cmp_k, q_pos0, n_q):
        """Block keys of the complete blocks that end inside this chunk."""
        first = q_pos0 // self.r
        last = (q_pos0 + n_q) // self.r
        qsa_compress_keys(idx_k, cmp_k, self.r, first, last - first)

    def select(self, idx_q, cmp_k, q_pos0, n_q):
        self.pos.fill_(q_pos0)
        qsa_index_topk(self.idesc, idx_q[:n_q], cmp_k, self.pos, q_pos0 + n_q,
                       self.sel[:n_q], self.cnt[:n_q], self.ws_index)
        return self.sel[:n_q], self.cnt[:n_q]

    def attend(self, q, k, v, q_pos0, n_q, sel=None, cnt=None):
        sel = self.sel[:n_q] if sel is None else sel
        cnt = self.cnt[:n_q] if cnt is None else cnt
        qsa_sparse_attn_prefill(self.adesc, self.r, q[:n_q], k[:q_pos0 + n_q], v[:q_pos0 + n_q], q_pos0,
                                sel, cnt, self.out[:n_q], self.lse[:n_q], self.ws_attn)
        return self.out[:n_q], self.lse[:n_q]

    def __call__(self, q, k, v, idx_q, idx_k, cmp_k, q_pos0, n_q):
        self.compress(idx_k, cmp_k, q_pos0, n_q)
        self.select(idx_q, cmp_k, q_pos0, n_q)
        return self.attend(q, k, v, q_pos0, n_q)



class ChunkedPrefill:
    """Causal prefill of `n_q` queries of one sequence in chunks of `chunk`
    queries. Chunk c's attention and chunk c + 1's key compression and
    indexer do not depend on each other (the indexer reads block keys, the
    attention K, V and its own selection), so they run on two streams side by
    side; two sets of selection buffers alternate between the chunks, and
    chunk c + 2's indexer waits until chunk c's attention has read its set.
    Outputs go to the caller's out [n_q, Hq, D] and lse [n_q, Hq]."""

    def __init__(self, Hq, Hkv, Hi, r=4, k=512, chunk=8192, max_len=8192, D=128, di=64, device="cuda"):
        self.chunk = chunk
        self.paths = [PrefillPath(Hq, Hkv, Hi, r, k, n_q_max=chunk, max_len=max_len, D=D, di=di, device=device)
                      for _ in range(2)]
        self.s_attn = torch.cuda.Stream(device)
        self.s_index = torch.cuda.Stream(device)

    def __call__(self, q, k, v, idx_q, idx_k, cmp_k, q_pos0, n_q, out, lse=None):
        cur = torch.cuda.current_stream()
        self.s_attn.wait_stream(cur)
        self.s_index.wait_stream(cur)
        n_ch = (n_q + self.chunk - 1) // self.chunk
        selected, attended = [None] * n_ch, [None] * n_ch
        for c in range(n_ch):
            c0 = c * self.chunk
            n = min(self.chunk, n_q - c0)
            p = self.paths[c % 2]
            with torch.cuda.stream(self.s_index):
                if c >= 2:
                    self.s_index.wait_event(attended[c - 2])
                p.compress(idx_k, cmp_k, q_pos0 + c0, n)
                p.select(idx_q[c0:c0 + n], cmp_k, q_pos0 + c0, n)
                selected[c] = torch.cuda.Event()
                selected[c].record(self.s_index)
            with torch.cuda.stream(self.s_attn):
                self.s_attn.wait_event(selected[c])
                end = q_pos0 + c0 + n
                qsa_sparse_attn_prefill(p.adesc, p.r, q[c0:c0 + n], k[:end], v[:end], q_pos0 + c0,
                                        p.sel[:n], p.cnt[:n], out[c0:c0 + n],
                                        None if lse is None else lse[c0:c0 + n], p.ws_attn)
                attended[c] = torch.cuda.Event()
                attended[c].record(self.s_attn)
        cur.wait_stream(self.s_attn)
        cur.wait_stream(self.s_index)
        return out, lse

class DecodePath:
    """One decode step for `batch` sequences with caches of `max_len` tokens."""

    def __init__(self, Hq, Hkv, Hi, batch, max_len, r=4, k=512, D=128, di=64, device="cuda"):
        self.r, self.k, self.batch = r, k, batch
        self.idesc = index_desc(r, k, Hi, di)
        self.adesc = attn_desc(Hq, Hkv, D)
        self.ws_index = workspace(qsa_index_topk_workspace_size(self.idesc, batch, 1, max_len), device)
        self.ws_attn = workspace(qsa_sparse_attn_workspace_size(self.adesc, batch, 1, k, r), device)
        self.sel = torch.empty((batch, 1, k), dtype=torch.int32, device=device)
        self.cnt = torch.empty((batch, 1), dtype=torch.int32, device=device)
        self.out = torch.empty((batch, Hq, D), dtype=torch.bfloat16, device=device)
        self.lse = torch.empty((batch, Hq), dtype=torch.float32, device=device)
        self.max_len = max_len

    def select(self, idx_q, cmp_k, q_pos, max_q_end=None):
        """idx_q [B, Hi, di]; q_pos int32 [B] = kv_len - 1 (device)."""
        qsa_index_topk(self.idesc, idx_q[:, None], cmp_k, q_pos, self.max_len if max_q_end is None else max_q_end,
                       self.sel, self.cnt, self.ws_index)
        return self.sel[:, 0], self.cnt[:, 0]

    def attend(self, q, k_cache, v_cache, kv_len, sel=None, cnt=None):
        sel = self.sel[:, 0] if sel is None else sel
        cnt = self.cnt[:, 0] if cnt is None else cnt
        qsa_sparse_attn_decode(self.adesc, self.r, q, k_cache, v_cache, kv_len, sel.contiguous(),
                               cnt.contiguous(), self.out, self.lse, self.ws_attn)
        return self.out, self.lse

    def __call__(self, q, k_cache, v_cache, idx_q, cmp_k, kv_len, q_pos):
        self.select(idx_q, cmp_k, q_pos)
        return self.attend(q, k_cache, v_cache, kv_len)


class PagedBatchPath:
    """Prefill of a packed batch: sequence b appends n[b] new rows at positions
    q_pos0[b] .. q_pos0[b] + n[b] - 1 to its cached prefix. K/V live in a paged
    pool ([n_pages, page_size, Hkv, D]) addressed by a page table
    ([batch, max_pages]); token and block indexer keys are cached per sequence
    ([batch, max_len, 64] and [batch, max_len / r, 64]). One row per sequence
    is a decode step of the same batch."""

    def __init__(self, Hq, Hkv, Hi, batch, max_q, max_len, r=4, k=512, D=128, di=64, device="cuda"):
        self.r, self.k, self.batch, self.max_q, self.max_len = r, k, batch, max_q, max_len
        self.idesc = index_desc(r, k, Hi, di)
        self.adesc = attn_desc(Hq, Hkv, D)
        self.ws_index = workspace(qsa_index_topk_varlen_workspace_size(self.idesc, batch, max_q, max_len), device)
        self.total_max = batch * max_q
        self.sel = torch.empty((self.total_max, k), dtype=torch.int32, device=device)
        self.cnt = torch.empty((self.total_max,), dtype=torch.int32, device=device)
        self.out = torch.empty((self.total_max, Hq, D), dtype=torch.bfloat16, device=device)
        self.lse = torch.empty((self.total_max, Hq), dtype=torch.float32, device=device)

    def compress(self, idx_k_cache, cmp_k, q_pos0_host, n_host):
        """Block keys of the blocks completed by each sequence's new rows."""
        for b, (p0, n) in enumerate(zip(q_pos0_host, n_host)):
            first, last = p0 // self.r, (p0 + n) // self.r
            if last > first:
                qsa_compress_keys(idx_k_cache[b], cmp_k[b], self.r, first, last - first)

    def select(self, idx_q, cmp_k, cu_q, q_pos0, total_q, max_q_end=None):
        qsa_index_topk_varlen(self.idesc, idx_q[:total_q], cmp_k, cu_q, q_pos0, self.max_q,
                              self.max_len if max_q_end is None else max_q_end,
                              self.sel[:total_q], self.cnt[:total_q], self.ws_index)
        return self.sel[:total_q], self.cnt[:total_q]

    def attend(self, q, k_pages, v_pages, page_table, cu_q, q_pos0, total_q, sel=None, cnt=None):
        sel = self.sel[:total_q] if sel is None else sel
        cnt = self.cnt[:total_q] if cnt is None else cnt
        qsa_sparse_attn_prefill_paged(self.adesc, self.r, q[:total_q], k_pages, v_pages, page_table, cu_q,
                                      q_pos0, sel, cnt, self.out[:total_q], self.lse[:total_q])
        return self.out[:total_q], self.lse[:total_q]

    def __call__(self, q, k_pages, v_pages, page_table, idx_q, idx_k_cache, cmp_k, cu_q, q_pos0, q_pos0_host,
                 n_host):
        total_q = int(sum(n_host))
        self.compress(idx_k_cache, cmp_k, q_pos0_host, n_host)
        self.select(idx_q, cmp_k, cu_q, q_pos0, total_q)
        return self.attend(q, k_pages, v_pages, page_table, cu_q, q_pos0, total_q)
