/*
 * qsa_bench.h — dense grouped-query attention, the comparator QSA is measured
 * against (explainer page "用125亿分之6的参数，打平3970亿的旗舰模型", section
 * "稀疏注意力：给检索建索引，也得先学会省纸": the speedups are quoted against
 * GQA at a 1M-token context), and diagnostics of how the calls launch. Not
 * part of the method; same conventions as qsa.h (device pointers,
 * caller-owned workspace, async on `stream`, host-side argument checks,
 * nothing enqueued on error).
 */
#ifndef QSA_BENCH_H_
#define QSA_BENCH_H_

#include "qsa.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes of workspace the dense calls need (0 on bad input). */
size_t qsa_dense_attn_workspace_size(const qsa_attn_desc_t* desc, int32_t batch, int32_t n_q,
                                     int64_t max_len);

/* Dense causal attention, prefill: query i at position q_pos0 + i attends to
 * every token 0..q_pos0 + i. Layouts as qsa_sparse_attn_prefill. */
qsa_status_t qsa_dense_attn_prefill(const qsa_attn_desc_t* desc, const uint16_t* q,
                                    const uint16_t* k, const uint16_t* v, int64_t q_pos0,
                                    int32_t n_q, int64_t kv_len, uint16_t* out, float* lse,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* Dense attention, decode: query of sequence b at kv_len[b] - 1 attends to
 * every cached token. Layouts as qsa_sparse_attn_decode. */
qsa_status_t qsa_dense_attn_decode(const qsa_attn_desc_t* desc, const uint16_t* q,
                                   const uint16_t* k_cache, const uint16_t* v_cache,
                                   int64_t max_len, const int32_t* kv_len, int32_t batch,
                                   uint16_t* out, float* lse, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* ---- Diagnostics: the launch plan a call would use (host only, no device) ----
 * Every call checks its plan before launching and refuses one that does not
 * fit (QSA_ERR_UNSUPPORTED): every grid, workgroup size and LDS size within
 * the device's limits (grid x < 2^31, y and z <= 65535, 1024 threads, 160 KiB
 * of LDS), every value a kernel holds in a 32-bit int below 2^31 (query,
 * task, candidate and list-slot indices), every element offset into a
 * workspace region below 2^62 (the kernels form them in 64 bits). These
 * functions return that plan without launching anything. */
typedef struct {
  int32_t n_launches;       /* kernels the call enqueues (up to 3) */
  uint32_t grid[3][3];      /* grid (x, y, z) of each launch */
  uint32_t block[3];        /* threads per workgroup of each launch */
  uint64_t lds[3];          /* LDS bytes per workgroup (static upper bound + dynamic) */
  int64_t max_int32_value;  /* largest value a kernel holds in a 32-bit int */
  int64_t max_offset;       /* largest element offset into a workspace region */
  uint64_t workspace_bytes; /* the matching *_workspace_size */
  int32_t splits;           /* indexer: candidate splits; attention: token-list splits */
  int32_t cap;              /* indexer: buffer / list entries per split; attention: tokens per split */
  int32_t fits;             /* 1 when every limit above holds */
  int32_t sample_stride;    /* indexer: the many-query kernel first scores every sample_stride-th
                               64-block tile of a split to seed its thresholds (0: no sample);
                               added in ABI version 2 */
} qsa_plan_info_t;

/* Plan of qsa_index_topk (packed = 0) or qsa_index_topk_varlen (packed = 1,
 * n_q = rows of the longest sequence) for these sizes. */
qsa_status_t qsa_index_topk_plan_info(const qsa_index_desc_t* desc, int32_t batch, int32_t n_q, int64_t max_q_end,
                                      int32_t packed, qsa_plan_info_t* info);

/* Plan of the sparse attention calls: rows query rows (prefill, decode = 0)
 * or sequences (decode = 1). */
qsa_status_t qsa_sparse_attn_plan_info(const qsa_attn_desc_t* desc, int32_t rows, int32_t top_k_blocks,
                                       int32_t block_size, int32_t decode, qsa_plan_info_t* info);

#ifdef __cplusplus
}
#endif

#endif /* QSA_BENCH_H_ */
