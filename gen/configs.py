"""Workload shapes of the five synthetic configurations (sizes, seeds, needle
rates). Shapes only: nothing here computes any step of the method.

Tensor layouts (row-major, innermost last, bf16 bits):
  prefill  Q [n_q, Hq, D], K/V [L, Hkv, D], idx_q [n_q, Hi, di], idx_k [L, di]
  decode   Q [B, Hq, D], K/V caches [B, L, Hkv, D], idx_q [B, Hi, di], idx_k [B, L, di]
Each tensor is one generator stream (see ``gen``), flat element index in the
layout above. The query of prefill row i sits at position q_pos0 + i; the
query of decode row b sits at position L - 1.
"""
from dataclasses import dataclass, field


@dataclass(frozen=True)
class Workload:
    name: str
    mode: str            # "prefill" or "decode"
    seed: int
    batch: int           # sequences (decode) or 1 (prefill)
    L: int               # context length (KV rows) per sequence
    n_q: int             # query rows per sequence (prefill); 1 for decode
    q_pos0: int          # position of the first query (prefill)
    Hq: int
    Hkv: int
    Hi: int
    D: int = 128
    di: int = 64
    r: int = 4
    k: int = 512          # kept blocks, diagonal included (budget = k * r tokens)
    needle_window: int = 0  # tokens per planted needle block (0 = none)
    chunk: int = 0        # prefill processed in chunks of this many queries (0 = one call)

    @property
    def w(self):
        return 1.0 / self.Hi

    @property
    def scale(self):
        return self.D ** -0.5

    @property
    def n_blk(self):
        return self.L // self.r


CONFIGS = {
    # 1: tiny prefill, 4K causal, budget 512 tokens, no needles
    "c1": Workload("c1_tiny_prefill_4k", "prefill", 1001, 1, 4096, 4096, 0, 16, 2, 4, k=128),
    # 2: mid prefill, 32K causal, 64 needles (one per 512 tokens)
    "c2": Workload("c2_mid_prefill_32k", "prefill", 1002, 1, 32768, 32768, 0, 32, 4, 8, needle_window=512),
    # 3: long prefill, 256K causal in 8192-query chunks, needles one per 4096 tokens
    "c3": Workload("c3_long_prefill_256k", "prefill", 1003, 1, 262144, 262144, 0, 16, 2, 4,
                   needle_window=4096, chunk=8192),
    # 4: decode, 64 sequences at 128K
    "c4": Workload("c4_decode_b64_128k", "decode", 1004, 64, 131072, 1, 131071, 32, 4, 8, needle_window=4096),
    # 5a: prefill of the last 16384 queries of a 1M causal context
    "c5a": Workload("c5a_prefill_16k_at_1m", "prefill", 1005, 1, 1048576, 16384, 1048576 - 16384, 32, 4, 8,
                    needle_window=4096),
    # 5b: decode, 4 sequences at 1M
    "c5b": Workload("c5b_decode_b4_1m", "decode", 1006, 4, 1048576, 1, 1048575, 32, 4, 8, needle_window=4096),
}


@dataclass(frozen=True)
class PagedBatch:
    """A packed serving batch: sequence b has a cached prefix of prefix[b]
    tokens and appends new[b] rows (1 = a decode step); K/V in a shared pool of
    page_size-token pages in shuffled order."""
    name: str
    seed: int
    prefix: tuple
    new: tuple
    Hq: int
    Hkv: int
    Hi: int
    page_size: int = 256
    D: int = 128
    di: int = 64
    r: int = 4
    k: int = 512
    needle_window: int = 4096

    @property
    def batch(self):
        return len(self.prefix)

    @property
    def w(self):
        return 1.0 / self.Hi

    @property
    def lengths(self):
        return [p + n for p, n in zip(self.prefix, self.new)]


PAGED = {
    # 6: 8 sequences with cached contexts of 128K .. 1M appending chunks of
    # 1 .. 4096 rows (two of them decode steps), 256-token pages
    "c6": PagedBatch("c6_paged_batch_8seq_128k_1m", 1007,
                     (131072, 262144, 393216, 524288, 655360, 786432, 917504, 1040384),
                     (2048, 1024, 512, 4096, 256, 1, 1, 2048), 32, 4, 8),
}


@dataclass(frozen=True)
class GdnWorkload:
    """A gated-delta-rule layer: B sequences of T tokens (prefill) or one
    token each on a carried state (decode); Hqk key heads, Hv value heads."""
    name: str
    mode: str
    seed: int
    batch: int
    T: int
    Hqk: int = 16
    Hv: int = 32
    dk: int = 128
    dv: int = 128

    @property
    def scale(self):
        return self.dk ** -0.5


GDN = {
    # prefill of one 32K-token sequence through one recurrent layer
    "g1": GdnWorkload("g1_gdn_prefill_32k", "prefill", 1011, 1, 32768),
    # one decode step of 64 sequences on carried states
    "g2": GdnWorkload("g2_gdn_decode_b64", "decode", 1012, 64, 1),
}
