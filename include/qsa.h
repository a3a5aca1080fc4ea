/*
 * qsa.h — C ABI of the QSA (Qwen Sparse Attention) hot path on AMD Instinct
 * MI355X (gfx950).
 *
 * The method (web pages on the Qwen3.8-Flash-Next release):
 *   - "用125亿分之6的参数，打平3970亿的旗舰模型", section
 *     "稀疏注意力：给检索建索引，也得先学会省纸": runs of r consecutive tokens
 *     form micro-blocks whose indexer key is the mean of the tokens' keys; a
 *     light multi-query indexer scores each block; the best blocks are kept,
 *     expanded back to their tokens, and exact attention runs over those
 *     tokens only.
 *   - "On the Design of Qwen3.8-Next Architecture" (agihunt.info digest of
 *     arXiv 2608.30320), token-mixing paragraph: the indexer works on
 *     micro-blocks so its cost falls from O(n^2) to O(n^2 / r); the deployed
 *     setting is a 2048-token budget with compression ratio 4.
 *
 * Conventions shared by every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller. bf16 tensors are
 *     passed as uint16_t bit patterns. Layouts are row-major, innermost
 *     dimension last, dense unless a stride argument says otherwise (strides
 *     are in elements). Every tensor pointer must be 16-byte aligned.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Calls only enqueue work: they never synchronise and never allocate.
 *     Scratch memory comes from the caller's `workspace` (size from the
 *     matching *_workspace_size query; contents need not be initialised and
 *     are clobbered; one workspace must not be used by two calls in flight).
 *   - Arguments are checked on the host before anything is enqueued. On any
 *     error nothing is launched, outputs are untouched, and a detail message
 *     is available from qsa_last_error_message() (thread-local).
 *   - Device-side faults from bad device data (e.g. out-of-range block ids
 *     passed to the attention calls) are not detected; they surface at the
 *     caller's next synchronisation.
 *   - Supported shapes: indexer dim d_i = 64, indexer heads 1..16, head dim
 *     D = 128, Hq / Hkv in 1..16 with Hkv in {1, 2, 4}, block size r in
 *     {1, 2, 4, 8, 16, 32}, 1 <= k <= 1024. Others return QSA_ERR_UNSUPPORTED.
 */
#ifndef QSA_H_
#define QSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QSA_ABI_VERSION 2

typedef enum {
  QSA_OK = 0,
  QSA_ERR_INVALID_ARGUMENT = 1, /* null pointer, negative size, inconsistent shapes */
  QSA_ERR_UNSUPPORTED = 2,      /* a shape outside the supported set above, or sizes whose launch
                                   plan does not fit the device (qsa_bench.h, diagnostics) */
  QSA_ERR_MISALIGNED = 3,       /* a tensor pointer or stride breaks 16-byte alignment */
  QSA_ERR_WORKSPACE_TOO_SMALL = 4,
  QSA_ERR_HIP = 5               /* the HIP runtime reported an error at launch */
} qsa_status_t;

/* Indexer settings. */
typedef struct {
  int32_t block_size;      /* r: tokens per micro-block */
  int32_t top_k_blocks;    /* k: blocks kept per query, the query's own block included */
  int32_t n_idx_heads;     /* H_i: indexer query heads (they share one key) */
  int32_t idx_head_dim;    /* d_i: indexer dim (64) */
  float idx_head_weight;   /* w: weight of every indexer head (1 / H_i) */
} qsa_index_desc_t;

/* Attention settings (grouped-query attention). */
typedef struct {
  int32_t n_q_heads;       /* Hq */
  int32_t n_kv_heads;      /* Hkv; query head h reads KV head h / (Hq / Hkv) */
  int32_t head_dim;        /* D (128) */
  float softmax_scale;     /* multiplies q.k before the softmax (1 / sqrt(D)) */
} qsa_attn_desc_t;

/* Micro-block key compression (explainer page, sparse-attention section:
 * the block key is the mean of its r token keys).
 *   idx_k  [batch][*][d]: token indexer keys; row b starts at idx_k + b * idx_k_batch_stride.
 *   cmp_k  [batch][*][d]: block keys; row b starts at cmp_k + b * cmp_k_batch_stride.
 * For every b < batch and block j in [first_block, first_block + n_blocks):
 *   cmp_k[b][j][i] = bf16_rne( (((k[jr][i] + k[jr+1][i]) + ...) + k[jr+r-1][i]) / r ),
 * the sum taken in fp32 left to right. Only complete blocks exist: the caller
 * passes blocks whose r tokens are all present. d = idx_head_dim must be 64. */
qsa_status_t qsa_compress_keys(const uint16_t* idx_k, int64_t idx_k_batch_stride, int32_t batch,
                               int32_t idx_head_dim, int32_t block_size, int64_t first_block,
                               int64_t n_blocks, uint16_t* cmp_k, int64_t cmp_k_batch_stride,
                               void* stream);

/* Bytes of workspace qsa_index_topk needs for these sizes (0 on bad input).
 * max_q_end: an upper bound on q_pos0[b] + n_q over the batch. The positions
 * q_pos0 live in device memory, which the host does not read (no
 * synchronisation), so the candidate range that sizes the buffers and the
 * split plan comes from this bound. */
size_t qsa_index_topk_workspace_size(const qsa_index_desc_t* desc, int32_t batch, int32_t n_q,
                                     int64_t max_q_end);

/* Indexer scoring + causal top-k block selection (explainer page,
 * sparse-attention section; digest page, token-mixing paragraph).
 *   idx_q     [batch][n_q][H_i][d_i] indexer queries; query i of row b sits at
 *             position t = q_pos0[b] + i.
 *   cmp_k     block keys of each row (see qsa_compress_keys); row b must hold
 *             at least (q_pos0[b] + n_q - 1) / r blocks.
 *   q_pos0    DEVICE int32 [batch]: position of each row's first query;
 *             q_pos0[b] + n_q <= max_q_end must hold.
 * For query t with own block b_t = t / r, the scored candidates are the
 * blocks j < b_t, each with score s = w * sum_h max(0, q_h . c_j) (fp32). The
 * min(k - 1, b_t) best candidates, ordered by (score desc, index asc), plus b_t
 * itself are kept.
 *   sel_blocks [batch][n_q][k] int32: kept blocks in ascending order, then -1.
 *   sel_count  [batch][n_q] int32: number of kept blocks, min(k, b_t + 1).
 * Decode is the case n_q = 1 with q_pos0[b] = kv_len[b] - 1. */
qsa_status_t qsa_index_topk(const qsa_index_desc_t* desc, const uint16_t* idx_q,
                            const uint16_t* cmp_k, int64_t cmp_k_batch_stride,
                            const int32_t* q_pos0, int64_t max_q_end, int32_t batch, int32_t n_q,
                            int32_t* sel_blocks, int32_t* sel_count, void* workspace,
                            size_t workspace_bytes, void* stream);

/* Bytes of workspace the sparse attention calls need (0 on bad input). The
 * decode call splits each sequence's token list (top_k_blocks * block_size
 * tokens) over several workgroups and merges their partial results in the
 * workspace, so its size depends on block_size as well. */
size_t qsa_sparse_attn_workspace_size(const qsa_attn_desc_t* desc, int32_t batch, int32_t n_q,
                                      int32_t top_k_blocks, int32_t block_size);

/* Sparse attention, prefill (news page, section 2 item 1: full-precision
 * attention on the relevant blocks only; explainer page: kept blocks are
 * expanded back to their tokens).
 *   q    [n_q][Hq][D]; query i sits at position t = q_pos0 + i.
 *   k, v [kv_len][Hkv][D]; q_pos0 + n_q <= kv_len.
 *   sel_blocks [n_q][top_k_blocks], sel_count [n_q]: as written by qsa_index_topk.
 * Tokens attended by query t: every s = j * r + m (m < r) of every listed
 * block j with s <= t. o = softmax(scale * q.K^T) V, exact, fp32 accumulation.
 *   out  [n_q][Hq][D] bf16;  lse [n_q][Hq] fp32 natural-log sum-exp of the
 *   scaled logits (may be NULL). */
qsa_status_t qsa_sparse_attn_prefill(const qsa_attn_desc_t* desc, int32_t block_size,
                                     int32_t top_k_blocks, const uint16_t* q, const uint16_t* k,
                                     const uint16_t* v, int64_t q_pos0, int32_t n_q, int64_t kv_len,
                                     const int32_t* sel_blocks, const int32_t* sel_count,
                                     uint16_t* out, float* lse, void* workspace,
                                     size_t workspace_bytes, void* stream);

/* Sparse attention, decode (news page, section 2 item 1: QSA speeds up the
 * decoding of long contexts as well as their prefill; explainer page,
 * sparse-attention section: each new token attends only to the tokens of its
 * kept blocks): one query per sequence at position kv_len[b] - 1, the newest
 * token, already in the cache.
 *   q        [batch][Hq][D]
 *   k_cache, v_cache [batch][max_len][Hkv][D]
 *   kv_len   DEVICE int32 [batch], 1 <= kv_len[b] <= max_len.
 *   sel_blocks [batch][top_k_blocks], sel_count [batch].
 *   out [batch][Hq][D] bf16; lse [batch][Hq] fp32 (may be NULL). */
qsa_status_t qsa_sparse_attn_decode(const qsa_attn_desc_t* desc, int32_t block_size,
                                    int32_t top_k_blocks, const uint16_t* q,
                                    const uint16_t* k_cache, const uint16_t* v_cache,
                                    int64_t max_len, const int32_t* kv_len, int32_t batch,
                                    const int32_t* sel_blocks, const int32_t* sel_count,
                                    uint16_t* out, float* lse, void* workspace,
                                    size_t workspace_bytes, void* stream);

/* Sparse attention, decode, for callers that cannot allocate memory (code
 * under stream or graph capture, tight serving loops, harnesses that forbid
 * allocation): the same call and results as qsa_sparse_attn_decode without a
 * workspace. The step's split partial results go to a scratch array the
 * library holds on each device (8 MiB, allocated at load, kept until the
 * process ends); nothing is allocated per call. Sizes whose partial results
 * need more than that return QSA_ERR_UNSUPPORTED. Every call on one device
 * shares that scratch: calls that may overlap on a device (other streams,
 * other threads) race, so the caller serialises them. */
qsa_status_t qsa_sparse_attn_decode_noalloc(const qsa_attn_desc_t* desc, int32_t block_size,
                                            int32_t top_k_blocks, const uint16_t* q, const uint16_t* k_cache,
                                            const uint16_t* v_cache, int64_t max_len, const int32_t* kv_len,
                                            int32_t batch, const int32_t* sel_blocks, const int32_t* sel_count,
                                            uint16_t* out, float* lse, void* stream);

/* ---- Packed variable-length batches over a paged K/V cache (serving) ----
 * A batch of `batch` sequences whose new queries are packed row after row:
 * sequence b owns rows [cu_q[b], cu_q[b + 1]) of idx_q / q / sel / out, its
 * i-th row sitting at position q_pos0[b] + i (a prefill chunk appended to a
 * cached prefix; one row per sequence is a decode step). cu_q (DEVICE int32
 * [batch + 1], cu_q[0] = 0, non-decreasing) and q_pos0 (DEVICE int32 [batch])
 * are read on the device and are not checked. */

/* Bytes of workspace qsa_index_topk_varlen needs (0 on bad input).
 * max_q: an upper bound on the rows of one sequence; max_q_end: an upper bound
 * on q_pos0[b] + rows of b. */
size_t qsa_index_topk_varlen_workspace_size(const qsa_index_desc_t* desc, int32_t batch, int32_t max_q,
                                            int64_t max_q_end);

/* qsa_index_topk over packed rows: idx_q [total_q][H_i][d_i], sel_blocks
 * [total_q][k], sel_count [total_q]; cmp_k as for qsa_index_topk (block keys
 * of sequence b at cmp_k + b * cmp_k_batch_stride, at least
 * (q_pos0[b] + rows - 1) / r of them). Same selection rule per row. */
qsa_status_t qsa_index_topk_varlen(const qsa_index_desc_t* desc, const uint16_t* idx_q,
                                   const uint16_t* cmp_k, int64_t cmp_k_batch_stride,
                                   const int32_t* cu_q, const int32_t* q_pos0, int32_t batch,
                                   int32_t max_q, int64_t max_q_end, int32_t* sel_blocks,
                                   int32_t* sel_count, void* workspace, size_t workspace_bytes,
                                   void* stream);

/* qsa_sparse_attn_prefill over packed rows and a paged K/V pool.
 *   q, out [total_q][Hq][D]; lse [total_q][Hq] (may be NULL).
 *   k_pages, v_pages [n_pages][page_size][Hkv][D]: the pool.
 *   page_table DEVICE int32 [batch][max_pages]: token s of sequence b lives at
 *   slot s % page_size of page page_table[b][s / page_size]; the pages of
 *   every token a row may attend (0 .. its position) must be listed.
 *   page_size: a power of two, at least block_size (a block never straddles
 *   pages); n_pages * page_size < 2^31.
 *   sel_blocks [total_q][top_k_blocks], sel_count [total_q] as written by
 *   qsa_index_topk_varlen. No workspace is needed (pass NULL, 0). */
qsa_status_t qsa_sparse_attn_prefill_paged(const qsa_attn_desc_t* desc, int32_t block_size,
                                           int32_t top_k_blocks, const uint16_t* q,
                                           const uint16_t* k_pages, const uint16_t* v_pages,
                                           int32_t page_size, int64_t n_pages,
                                           const int32_t* page_table, int32_t max_pages,
                                           const int32_t* cu_q, const int32_t* q_pos0, int32_t batch,
                                           int32_t total_q, const int32_t* sel_blocks,
                                           const int32_t* sel_count, uint16_t* out, float* lse,
                                           void* stream);

/* ---- Training-side forward: the indexer's dense-distillation loss ----
 * Explainer page, sparse-attention section: in the first training stage only
 * the indexer learns, pulled towards the full-attention distribution by a KL
 * divergence. For query t (position q_pos0 + i) with own block b_t:
 *   P_j = sum over query heads h and tokens s of block j of the dense causal
 *         softmax a_h(s) over s <= t, renormalised over the candidates j < b_t;
 *   Q_j = softmax over j < b_t of the indexer score s_j (the qsa_index_topk
 *         score, used as a logit);
 *   kl[i] = sum_j P_j (ln P_j - ln Q_j), 0 when b_t = 0.
 *   q [n_q][Hq][D], k [kv_len][Hkv][D] (q_pos0 + n_q <= kv_len),
 *   idx_q [n_q][H_i][d_i], cmp_k [blocks][d_i] (at least (q_pos0 + n_q - 1) / r),
 *   kl [n_q] fp32. Supported: Hq = 8 Hkv, H_i = 8, d_i = 64, D = 128.
 * Workspace: qsa_distill_kl_workspace_size bytes (the per-row log-sum-exp). */
size_t qsa_distill_kl_workspace_size(const qsa_attn_desc_t* adesc, int32_t n_q);
qsa_status_t qsa_distill_kl_prefill(const qsa_attn_desc_t* adesc, const qsa_index_desc_t* idesc,
                                    const uint16_t* q, const uint16_t* k, const uint16_t* idx_q,
                                    const uint16_t* cmp_k, int64_t q_pos0, int32_t n_q, int64_t kv_len,
                                    float* kl, void* workspace, size_t workspace_bytes, void* stream);

/* ---- Recurrent layers: the gated delta rule ----
 * Explainer page, section on the memory/efficiency trade-off, and the digest's
 * token-mixing paragraph: three of every four layers are Gated DeltaNet
 * layers, which carry a fixed-size matrix state; per token a decay gate sets
 * how much of the old state is kept and a write gate how much of the error
 * between the token's value and what the state returns for its key is
 * written. Per value head h (key head h / (Hv / Hqk)), state S (dv x dk):
 *   a_t = exp(g_t),  e_t = v_t - a_t S k_t,  S <- a_t S + beta_t e_t k_t^T,
 *   o_t = S (scale q_t).
 * q, k are expected already normalised (that happens before the mixing).
 * Supported: key_dim = value_dim = 128, n_v_heads a multiple of n_qk_heads.
 * States are fp32 [B][Hv][dv][dk]. */
typedef struct {
  int32_t n_qk_heads; /* Hqk: heads of q and k */
  int32_t n_v_heads;  /* Hv: heads of v, of the output and of the state */
  int32_t key_dim;    /* dk (128) */
  int32_t value_dim;  /* dv (128) */
  float scale;        /* read-out scale on q (e.g. 1/sqrt(dk)) */
} qsa_gdn_desc_t;

/* Prefill of B sequences of seq_len tokens: q, k [B][T][Hqk][dk], v
 * [B][T][Hv][dv] bf16 (16-byte aligned); g (log decay, <= 0) and beta (write
 * gate, in [0, 1]) [B][T][Hv] fp32; initial_state NULL (zero) or [B][Hv][dv][dk];
 * out [B][T][Hv][dv] bf16; final_state NULL or [B][Hv][dv][dk] (may be the
 * same buffer as initial_state). Runs in chunks of 64 tokens (per-chunk
 * factors in the workspace, then one ordered pass per (sequence, head)).
 * Workspace: qsa_gdn_prefill_workspace_size bytes, 16-byte aligned. */
size_t qsa_gdn_prefill_workspace_size(const qsa_gdn_desc_t* desc, int32_t batch, int64_t seq_len);
qsa_status_t qsa_gdn_prefill(const qsa_gdn_desc_t* desc, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                             const float* g, const float* beta, const float* initial_state, int32_t batch,
                             int64_t seq_len, uint16_t* out, float* final_state, void* workspace,
                             size_t workspace_bytes, void* stream);

/* One decode step of B sequences: q, k [B][Hqk][dk], v [B][Hv][dv] bf16;
 * g, beta [B][Hv] fp32; state [B][Hv][dv][dk] fp32 (16-byte aligned), updated
 * in place; out [B][Hv][dv] bf16. No workspace. */
qsa_status_t qsa_gdn_decode(const qsa_gdn_desc_t* desc, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            const float* g, const float* beta, float* state, int32_t batch, uint16_t* out,
                            void* stream);

const char* qsa_status_string(qsa_status_t status);
const char* qsa_last_error_message(void);
int qsa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QSA_H_ */
