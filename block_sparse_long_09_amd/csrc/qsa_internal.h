// Host-side plans and kernel launchers of the QSA library (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qsa {

hipError_t launch_compress(const uint16_t* idx_k, int64_t k_stride, int batch, int d, int r,
                           int64_t first, int64_t n, uint16_t* cmp, int64_t c_stride,
                           hipStream_t stream);

// One kernel launch of a plan: grid, threads and LDS bytes per workgroup.
struct LaunchShape {
  uint32_t grid[3];
  uint32_t block;
  size_t lds;  // static (an upper bound from the kernel's __shared__ arrays) + dynamic
};

// The launches of a plan and the largest values its kernels hold: a plan is
// refused (the calls return QSA_ERR_UNSUPPORTED) unless every grid, block and
// LDS size is within the device's limits, every value held in a 32-bit int
// is below 2^31, and every element offset into the workspace (64-bit in the
// kernels) is below 2^62.
struct PlanCheck {
  int n;
  LaunchShape l[3];
  int64_t max_i32;     // largest value a kernel holds in an int (query, task, candidate, slot)
  int64_t max_offset;  // largest element offset into a workspace region
  const char* unfit;   // nullptr when the plan fits
};

// How qsa_index_topk cuts its work: wave tasks = (query group, candidate split).
struct IndexPlan {
  bool decode;     // one query per sequence: split scan + verified merge
  bool wide;       // >= 64 queries per sequence: LDS-pipelined workgroup kernel
  int hi;          // indexer heads
  int at;          // 32-row A tiles per wave (4 for prefill, 1 for few queries)
  int nw;          // wide kernel: compute waves per workgroup (4: two workgroups per CU, 8: one)
  int qw;          // queries per wave
  int n_qgroups;   // query groups per sequence
  int splits;      // candidate splits
  int split_len;   // candidates per split (multiple of 32)
  int cap;         // buffer entries per (query, split)
  int seed_stride; // wide kernel: sample every seed_stride-th tile to seed the thresholds (0: off)
  int64_t max_cand;
  int64_t score_stride;             // decode: floats per sequence in the score array
  int list_min, list_cap;           // decode: entries per split list (at least / room)
  size_t local_off, meta_off;       // decode: workspace offsets
  size_t buf_bytes, cnt_bytes, workspace;
  size_t stream_lds, select_lds;    // dynamic LDS bytes of the two kernels
};

// allow_decode = false keeps one query per sequence on the prefill kernels
// (packed variable-length batches)
IndexPlan plan_index(int hi, int k, int batch, int n_q, int64_t max_q_end, int r,
                     bool allow_decode = true);

PlanCheck check_index_plan(const IndexPlan& p, int batch, int n_q);

hipError_t launch_index_topk(const IndexPlan& p, const uint16_t* idx_q, const uint16_t* cmp_k,
                             int64_t cmp_stride, const int32_t* q_pos0, int batch, int n_q, int r,
                             int k, float w, int32_t* sel, int32_t* sel_cnt, void* ws,
                             hipStream_t stream, const int32_t* cu_q = nullptr);

// How the gather attention cuts its work: one workgroup per (row, split).
struct AttnPlan {
  int rows;
  int splits;
  int64_t split_tokens;
};

AttnPlan plan_attn(int batch_rows, int64_t max_tokens, bool split_kv);
size_t attn_workspace_bytes(const AttnPlan& p, int Hq);
PlanCheck check_attn_plan(const AttnPlan& p, int Hq, int Hkv, int top_k, int r);

// Packed variable-length rows over a paged K/V pool (all null: not used).
// Sequence b owns rows [cu_q[b], cu_q[b + 1]) at positions q_pos[b] + i; its
// token s is row (page_table[b * max_pages + (s >> lps)] << lps) + s % 2^lps
// of the pool.
struct PagedRows {
  const int32_t* cu_q;
  const int32_t* q_pos;
  int n_seq;
  const int32_t* page_table;
  int max_pages;
  int lps;
};

// sel == nullptr: dense (tokens 0..t). kv_len == nullptr: prefill rows at
// q_pos0 + row sharing one K/V (or packed rows of pg); else decode rows with
// their own caches.
hipError_t launch_attn(const AttnPlan& p, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                       int64_t kv_batch_stride, int64_t q_pos0, const int32_t* kv_len, int Hq,
                       int Hkv, int r, int top_k, const int32_t* sel, const int32_t* sel_cnt,
                       float scale, uint16_t* out, float* lse, void* ws, hipStream_t stream,
                       PagedRows pg = PagedRows{nullptr, nullptr, 0, nullptr, 0, 0});

// Dense causal GQA flash attention (comparator), prefill rows at q_pos0 + i.
hipError_t launch_dense_prefill(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t q_pos0,
                                int n_q, int Hq, int Hkv, float scale, uint16_t* out, float* lse,
                                hipStream_t stream);

// Forward of the indexer's dense-distillation KL per query (pass 1: the dense
// kernel's log-sum-exp into lse_ws [n_q][Hq]; pass 2: block masses, scores,
// loss). Hq = 8 Hkv, 8 indexer heads of dim 64.
hipError_t launch_distill_kl(const uint16_t* q, const uint16_t* k, const uint16_t* idx_q, const uint16_t* cmp_k,
                             int64_t q_pos0, int n_q, int Hq, int Hkv, int r, float scale, float w_idx,
                             float* lse_ws, float* kl, hipStream_t stream);

// Gated delta rule (recurrent layers): chunked prefill and one decode step.
size_t gdn_workspace_bytes(int batch, int64_t T, int Hv);
hipError_t launch_gdn_prefill(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* g,
                              const float* beta, const float* S0, int batch, int64_t T, int Hqk, int Hv,
                              float scale, uint16_t* out, float* S_out, void* ws, hipStream_t stream);
hipError_t launch_gdn_decode(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* g,
                             const float* beta, int batch, int Hqk, int Hv, float scale, float* state,
                             uint16_t* out, hipStream_t stream);

}  // namespace qsa
