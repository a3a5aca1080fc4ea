/*
 * qsa_bench.h — dense grouped-query attention, the comparator QSA is measured
 * against (explainer page "用125亿分之6的参数，打平3970亿的旗舰模型", section
 * "稀疏注意力：给检索建索引，也得先学会省纸": the speedups are quoted against
 * GQA at a 1M-token context). Not part of the method; same conventions as
 * qsa.h (device pointers, caller-owned workspace, async on `stream`, host-side
 * argument checks, nothing enqueued on error).
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

#ifdef __cplusplus
}
#endif

#endif /* QSA_BENCH_H_ */
