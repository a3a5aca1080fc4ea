// C ABI of the QSA library: host-side argument checks, workspace sizing and
// kernel launches. Every check runs before anything is enqueued; on error
// nothing is launched and qsa_last_error_message() says why.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "qsa.h"
#include "qsa_bench.h"
#include "qsa_internal.h"

// Library-owned scratch of qsa_sparse_attn_decode_noalloc: the split-KV
// partial results of a decode step. Each device holds its own copy (zero at
// load) until the process ends; host code reaches it only through the address
// hipGetSymbolAddress returns for the current device.
constexpr size_t kNoAllocScratchBytes = 8u << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

thread_local char g_err[512] = "";

qsa_status_t fail(qsa_status_t s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

qsa_status_t ok() {
  g_err[0] = 0;
  return QSA_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool valid_block_size(int r) { return r == 1 || r == 2 || r == 4 || r == 8 || r == 16 || r == 32; }

constexpr int kMaxK = 1024;
constexpr int64_t kMaxPos = 0x7FFFFFFF;

qsa_status_t check_index_desc(const qsa_index_desc_t* d) {
  if (!d) return fail(QSA_ERR_INVALID_ARGUMENT, "index desc is NULL");
  if (!valid_block_size(d->block_size))
    return fail(QSA_ERR_UNSUPPORTED, "block_size %d not in {1,2,4,8,16,32}", d->block_size);
  if (d->top_k_blocks < 1 || d->top_k_blocks > kMaxK)
    return fail(QSA_ERR_UNSUPPORTED, "top_k_blocks %d not in [1, %d]", d->top_k_blocks, kMaxK);
  const int h = d->n_idx_heads;
  if (!(h == 1 || h == 2 || h == 4 || h == 8 || h == 16))
    return fail(QSA_ERR_UNSUPPORTED, "n_idx_heads %d not in {1,2,4,8,16}", h);
  if (d->idx_head_dim != 64) return fail(QSA_ERR_UNSUPPORTED, "idx_head_dim %d != 64", d->idx_head_dim);
  if (!(d->idx_head_weight > 0.0f) || !isfinite(d->idx_head_weight))
    return fail(QSA_ERR_INVALID_ARGUMENT, "idx_head_weight must be finite and > 0");
  return QSA_OK;
}

qsa_status_t check_attn_desc(const qsa_attn_desc_t* d) {
  if (!d) return fail(QSA_ERR_INVALID_ARGUMENT, "attn desc is NULL");
  if (d->head_dim != 128) return fail(QSA_ERR_UNSUPPORTED, "head_dim %d != 128", d->head_dim);
  const int hkv = d->n_kv_heads;
  if (!(hkv == 1 || hkv == 2 || hkv == 4))
    return fail(QSA_ERR_UNSUPPORTED, "n_kv_heads %d not in {1,2,4}", hkv);
  if (d->n_q_heads < 1 || d->n_q_heads % hkv != 0)
    return fail(QSA_ERR_INVALID_ARGUMENT, "n_q_heads %d not a positive multiple of n_kv_heads %d",
                d->n_q_heads, hkv);
  if (d->n_q_heads / hkv > 16)
    return fail(QSA_ERR_UNSUPPORTED, "group size %d > 16", d->n_q_heads / hkv);
  if (!isfinite(d->softmax_scale)) return fail(QSA_ERR_INVALID_ARGUMENT, "softmax_scale not finite");
  return QSA_OK;
}

qsa_status_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(QSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

extern "C" {

int qsa_abi_version(void) { return QSA_ABI_VERSION; }

const char* qsa_last_error_message(void) { return g_err; }

const char* qsa_status_string(qsa_status_t s) {
  switch (s) {
    case QSA_OK: return "QSA_OK";
    case QSA_ERR_INVALID_ARGUMENT: return "QSA_ERR_INVALID_ARGUMENT";
    case QSA_ERR_UNSUPPORTED: return "QSA_ERR_UNSUPPORTED";
    case QSA_ERR_MISALIGNED: return "QSA_ERR_MISALIGNED";
    case QSA_ERR_WORKSPACE_TOO_SMALL: return "QSA_ERR_WORKSPACE_TOO_SMALL";
    case QSA_ERR_HIP: return "QSA_ERR_HIP";
  }
  return "QSA_ERR_UNKNOWN";
}

qsa_status_t qsa_compress_keys(const uint16_t* idx_k, int64_t idx_k_batch_stride, int32_t batch,
                               int32_t idx_head_dim, int32_t block_size, int64_t first_block,
                               int64_t n_blocks, uint16_t* cmp_k, int64_t cmp_k_batch_stride,
                               void* stream) {
  if (batch < 0 || first_block < 0 || n_blocks < 0)
    return fail(QSA_ERR_INVALID_ARGUMENT, "negative batch/first_block/n_blocks");
  if (idx_head_dim != 64) return fail(QSA_ERR_UNSUPPORTED, "idx_head_dim %d != 64", idx_head_dim);
  if (!valid_block_size(block_size))
    return fail(QSA_ERR_UNSUPPORTED, "block_size %d not in {1,2,4,8,16,32}", block_size);
  if (batch > 65535) return fail(QSA_ERR_UNSUPPORTED, "batch %d > 65535", batch);
  if (batch == 0 || n_blocks == 0) return ok();
  if (!idx_k || !cmp_k) return fail(QSA_ERR_INVALID_ARGUMENT, "NULL tensor pointer");
  if (!aligned(idx_k, 16) || !aligned(cmp_k, 16))
    return fail(QSA_ERR_MISALIGNED, "idx_k/cmp_k must be 16-byte aligned");
  const int64_t end = first_block + n_blocks;
  if (batch > 1) {
    if (idx_k_batch_stride < end * block_size * idx_head_dim || cmp_k_batch_stride < end * idx_head_dim)
      return fail(QSA_ERR_INVALID_ARGUMENT, "batch strides do not cover %lld blocks", (long long)end);
    if (idx_k_batch_stride % 8 || cmp_k_batch_stride % 8)
      return fail(QSA_ERR_MISALIGNED, "batch strides must be multiples of 8 elements");
  }
  return hip_status(qsa::launch_compress(idx_k, idx_k_batch_stride, batch, idx_head_dim, block_size,
                                         first_block, n_blocks, cmp_k, cmp_k_batch_stride,
                                         (hipStream_t)stream),
                    "compress launch");
}

size_t qsa_index_topk_workspace_size(const qsa_index_desc_t* desc, int32_t batch, int32_t n_q,
                                     int64_t max_q_end) {
  if (check_index_desc(desc) != QSA_OK || batch < 0 || n_q < 0 || max_q_end < n_q ||
      max_q_end > kMaxPos)
    return 0;
  if (batch == 0 || n_q == 0) return 0;
  return qsa::plan_index(desc->n_idx_heads, desc->top_k_blocks, batch, n_q, max_q_end,
                         desc->block_size)
      .workspace;
}

qsa_status_t qsa_index_topk(const qsa_index_desc_t* desc, const uint16_t* idx_q,
                            const uint16_t* cmp_k, int64_t cmp_k_batch_stride,
                            const int32_t* q_pos0, int64_t max_q_end, int32_t batch, int32_t n_q,
                            int32_t* sel_blocks, int32_t* sel_count, void* workspace,
                            size_t workspace_bytes, void* stream) {
  qsa_status_t s = check_index_desc(desc);
  if (s != QSA_OK) return s;
  if (batch < 0 || n_q < 0) return fail(QSA_ERR_INVALID_ARGUMENT, "negative batch or n_q");
  if (batch > 65535) return fail(QSA_ERR_UNSUPPORTED, "batch %d > 65535", batch);
  if (max_q_end < n_q || max_q_end > kMaxPos)
    return fail(QSA_ERR_INVALID_ARGUMENT, "max_q_end %lld must be in [n_q, 2^31)", (long long)max_q_end);
  if (batch == 0 || n_q == 0) return ok();
  if (!idx_q || !cmp_k || !q_pos0 || !sel_blocks || !sel_count)
    return fail(QSA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  if (!aligned(idx_q, 16) || !aligned(cmp_k, 16))
    return fail(QSA_ERR_MISALIGNED, "idx_q/cmp_k must be 16-byte aligned");
  if (!aligned(q_pos0, 4) || !aligned(sel_blocks, 4) || !aligned(sel_count, 4))
    return fail(QSA_ERR_MISALIGNED, "int32 arrays must be 4-byte aligned");
  const int r = desc->block_size;
  const int64_t need_blocks = (max_q_end - 1) / r;
  if (batch > 1) {
    if (cmp_k_batch_stride < need_blocks * desc->idx_head_dim)
      return fail(QSA_ERR_INVALID_ARGUMENT, "cmp_k_batch_stride %lld < %lld blocks x 64",
                  (long long)cmp_k_batch_stride, (long long)need_blocks);
    if (cmp_k_batch_stride % 8) return fail(QSA_ERR_MISALIGNED, "cmp_k_batch_stride not a multiple of 8");
  }
  const qsa::IndexPlan p =
      qsa::plan_index(desc->n_idx_heads, desc->top_k_blocks, batch, n_q, max_q_end, r);
  const qsa::PlanCheck pc = qsa::check_index_plan(p, batch, n_q);
  if (pc.unfit) return fail(QSA_ERR_UNSUPPORTED, "index_topk: %s", pc.unfit);
  if (workspace_bytes < p.workspace || (p.workspace && !workspace))
    return fail(QSA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", workspace_bytes, p.workspace);
  if (!aligned(workspace, 16)) return fail(QSA_ERR_MISALIGNED, "workspace must be 16-byte aligned");
  return hip_status(qsa::launch_index_topk(p, idx_q, cmp_k, cmp_k_batch_stride, q_pos0, batch, n_q,
                                           r, desc->top_k_blocks, desc->idx_head_weight,
                                           sel_blocks, sel_count, workspace, (hipStream_t)stream),
                    "index_topk launch");
}

size_t qsa_sparse_attn_workspace_size(const qsa_attn_desc_t* desc, int32_t batch, int32_t n_q,
                                      int32_t top_k_blocks, int32_t block_size) {
  if (check_attn_desc(desc) != QSA_OK || batch < 0 || n_q < 0 || top_k_blocks < 1 ||
      top_k_blocks > kMaxK || !valid_block_size(block_size))
    return 0;
  // prefill (batch == 1, n_q rows) needs none; decode (n_q == 1) splits the token list
  if (n_q == 1 && batch >= 1) {
    const qsa::AttnPlan p = qsa::plan_attn(batch, (int64_t)top_k_blocks * block_size, true);
    return qsa::attn_workspace_bytes(p, desc->n_q_heads);
  }
  return 0;
}

static qsa_status_t check_attn_common(const qsa_attn_desc_t* desc, int32_t block_size,
                                      int32_t top_k_blocks) {
  qsa_status_t s = check_attn_desc(desc);
  if (s != QSA_OK) return s;
  if (!valid_block_size(block_size))
    return fail(QSA_ERR_UNSUPPORTED, "block_size %d not in {1,2,4,8,16,32}", block_size);
  if (top_k_blocks < 1 || top_k_blocks > kMaxK)
    return fail(QSA_ERR_UNSUPPORTED, "top_k_blocks %d not in [1, %d]", top_k_blocks, kMaxK);
  return QSA_OK;
}

qsa_status_t qsa_sparse_attn_prefill(const qsa_attn_desc_t* desc, int32_t block_size,
                                     int32_t top_k_blocks, const uint16_t* q, const uint16_t* k,
                                     const uint16_t* v, int64_t q_pos0, int32_t n_q, int64_t kv_len,
                                     const int32_t* sel_blocks, const int32_t* sel_count,
                                     uint16_t* out, float* lse, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  qsa_status_t s = check_attn_common(desc, block_size, top_k_blocks);
  if (s != QSA_OK) return s;
  if (q_pos0 < 0 || n_q < 0 || kv_len < q_pos0 + n_q || kv_len > kMaxPos)
    return fail(QSA_ERR_INVALID_ARGUMENT, "need 0 <= q_pos0, q_pos0 + n_q <= kv_len < 2^31");
  if (n_q == 0) return ok();
  if (!q || !k || !v || !sel_blocks || !sel_count || !out)
    return fail(QSA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
    return fail(QSA_ERR_MISALIGNED, "q/k/v/out must be 16-byte aligned");
  if (!aligned(sel_blocks, 4) || !aligned(sel_count, 4) || !aligned(lse, 4))
    return fail(QSA_ERR_MISALIGNED, "int32/fp32 arrays must be 4-byte aligned");
  const qsa::AttnPlan p = qsa::plan_attn(n_q, (int64_t)top_k_blocks * block_size, false);
  const qsa::PlanCheck pc = qsa::check_attn_plan(p, desc->n_q_heads, desc->n_kv_heads, top_k_blocks, block_size);
  if (pc.unfit) return fail(QSA_ERR_UNSUPPORTED, "sparse_attn_prefill: %s", pc.unfit);
  (void)workspace;
  (void)workspace_bytes;
  return hip_status(qsa::launch_attn(p, q, k, v, 0, q_pos0, nullptr, desc->n_q_heads,
                                     desc->n_kv_heads, block_size, top_k_blocks, sel_blocks,
                                     sel_count, desc->softmax_scale, out, lse, nullptr,
                                     (hipStream_t)stream),
                    "sparse_attn_prefill launch");
}

qsa_status_t qsa_sparse_attn_decode(const qsa_attn_desc_t* desc, int32_t block_size,
                                    int32_t top_k_blocks, const uint16_t* q,
                                    const uint16_t* k_cache, const uint16_t* v_cache,
                                    int64_t max_len, const int32_t* kv_len, int32_t batch,
                                    const int32_t* sel_blocks, const int32_t* sel_count,
                                    uint16_t* out, float* lse, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  qsa_status_t s = check_attn_common(desc, block_size, top_k_blocks);
  if (s != QSA_OK) return s;
  if (batch < 0 || max_len < 1 || max_len > kMaxPos)
    return fail(QSA_ERR_INVALID_ARGUMENT, "need batch >= 0 and 1 <= max_len < 2^31");
  if (batch == 0) return ok();
  if (!q || !k_cache || !v_cache || !kv_len || !sel_blocks || !sel_count || !out)
    return fail(QSA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16))
    return fail(QSA_ERR_MISALIGNED, "q/k_cache/v_cache/out must be 16-byte aligned");
  if (!aligned(kv_len, 4) || !aligned(sel_blocks, 4) || !aligned(sel_count, 4) || !aligned(lse, 4))
    return fail(QSA_ERR_MISALIGNED, "int32/fp32 arrays must be 4-byte aligned");
  const qsa::AttnPlan p = qsa::plan_attn(batch, (int64_t)top_k_blocks * block_size, true);
  const qsa::PlanCheck pc = qsa::check_attn_plan(p, desc->n_q_heads, desc->n_kv_heads, top_k_blocks, block_size);
  if (pc.unfit) return fail(QSA_ERR_UNSUPPORTED, "sparse_attn_decode: %s", pc.unfit);
  const size_t need = qsa::attn_workspace_bytes(p, desc->n_q_heads);
  if (workspace_bytes < need || (need && !workspace))
    return fail(QSA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", workspace_bytes, need);
  if (!aligned(workspace, 16)) return fail(QSA_ERR_MISALIGNED, "workspace must be 16-byte aligned");
  const int64_t stride = max_len * desc->n_kv_heads * desc->head_dim;
  return hip_status(qsa::launch_attn(p, q, k_cache, v_cache, stride, 0, kv_len, desc->n_q_heads,
                                     desc->n_kv_heads, block_size, top_k_blocks, sel_blocks,
                                     sel_count, desc->softmax_scale, out, lse, workspace,
                                     (hipStream_t)stream),
                    "sparse_attn_decode launch");
}

/* ---------------------------------------------------------- diagnostics --- */

static void fill_info(const qsa::PlanCheck& c, size_t ws, int splits, int cap, int sample_stride,
                      qsa_plan_info_t* info) {
  *info = qsa_plan_info_t{};
  info->n_launches = c.n;
  for (int i = 0; i < c.n && i < 3; ++i) {
    for (int d = 0; d < 3; ++d) info->grid[i][d] = c.l[i].grid[d];
    info->block[i] = c.l[i].block;
    info->lds[i] = c.l[i].lds;
  }
  info->max_int32_value = c.max_i32;
  info->max_offset = c.max_offset;
  info->workspace_bytes = ws;
  info->splits = splits;
  info->cap = cap;
  info->fits = c.unfit ? 0 : 1;
  info->sample_stride = sample_stride;
}

qsa_status_t qsa_index_topk_plan_info(const qsa_index_desc_t* desc, int32_t batch, int32_t n_q, int64_t max_q_end,
                                      int32_t packed, qsa_plan_info_t* info) {
  qsa_status_t s = check_index_desc(desc);
  if (s != QSA_OK) return s;
  if (!info) return fail(QSA_ERR_INVALID_ARGUMENT, "NULL info");
  if (batch < 1 || n_q < 1 || max_q_end < n_q || max_q_end > kMaxPos)
    return fail(QSA_ERR_INVALID_ARGUMENT, "need batch, n_q >= 1 and n_q <= max_q_end < 2^31");
  const qsa::IndexPlan p = qsa::plan_index(desc->n_idx_heads, desc->top_k_blocks, batch, n_q, max_q_end,
                                           desc->block_size, packed == 0);
  const qsa::PlanCheck c = qsa::check_index_plan(p, batch, n_q);
  fill_info(c, p.workspace, p.splits, p.decode ? p.list_cap : p.cap, p.decode ? 0 : p.seed_stride, info);
  return ok();
}

qsa_status_t qsa_sparse_attn_plan_info(const qsa_attn_desc_t* desc, int32_t rows, int32_t top_k_blocks,
                                       int32_t block_size, int32_t decode, qsa_plan_info_t* info) {
  qsa_status_t s = check_attn_common(desc, block_size, top_k_blocks);
  if (s != QSA_OK) return s;
  if (!info) return fail(QSA_ERR_INVALID_ARGUMENT, "NULL info");
  if (rows < 1) return fail(QSA_ERR_INVALID_ARGUMENT, "rows must be >= 1");
  const qsa::AttnPlan p = qsa::plan_attn(rows, (int64_t)top_k_blocks * block_size, decode != 0);
  const qsa::PlanCheck c = qsa::check_attn_plan(p, desc->n_q_heads, desc->n_kv_heads, top_k_blocks, block_size);
  fill_info(c, qsa::attn_workspace_bytes(p, desc->n_q_heads), p.splits, (int)p.split_tokens, 0, info);
  return ok();
}

/* --------------------------------------------------- allocation-free -------- */

namespace {
constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
static qsa_status_t scratch_address(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(QSA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(QSA_ERR_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(QSA_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return QSA_OK;
}
}  // namespace

qsa_status_t qsa_sparse_attn_decode_noalloc(const qsa_attn_desc_t* desc, int32_t block_size,
                                            int32_t top_k_blocks, const uint16_t* q, const uint16_t* k_cache,
                                            const uint16_t* v_cache, int64_t max_len, const int32_t* kv_len,
                                            int32_t batch, const int32_t* sel_blocks, const int32_t* sel_count,
                                            uint16_t* out, float* lse, void* stream) {
  qsa_status_t s = check_attn_common(desc, block_size, top_k_blocks);
  if (s != QSA_OK) return s;
  if (batch < 0 || max_len < 1 || max_len > kMaxPos)
    return fail(QSA_ERR_INVALID_ARGUMENT, "need batch >= 0 and 1 <= max_len < 2^31");
  if (batch == 0) return ok();
  if (!q || !k_cache || !v_cache || !kv_len || !sel_blocks || !sel_count || !out)
    return fail(QSA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16))
    return fail(QSA_ERR_MISALIGNED, "q/k_cache/v_cache/out must be 16-byte aligned");
  if (!aligned(kv_len, 4) || !aligned(sel_blocks, 4) || !aligned(sel_count, 4) || !aligned(lse, 4))
    return fail(QSA_ERR_MISALIGNED, "int32/fp32 arrays must be 4-byte aligned");
  const qsa::AttnPlan p = qsa::plan_attn(batch, (int64_t)top_k_blocks * block_size, true);
  const qsa::PlanCheck pc = qsa::check_attn_plan(p, desc->n_q_heads, desc->n_kv_heads, top_k_blocks, block_size);
  if (pc.unfit) return fail(QSA_ERR_UNSUPPORTED, "sparse_attn_decode_noalloc: %s", pc.unfit);
  const size_t need = qsa::attn_workspace_bytes(p, desc->n_q_heads);
  if (need > kNoAllocScratchBytes)
    return fail(QSA_ERR_UNSUPPORTED,
                "sparse_attn_decode_noalloc: the step's partial results need %zu bytes, beyond the library's "
                "%zu-byte scratch (use qsa_sparse_attn_decode with a workspace)",
                need, kNoAllocScratchBytes);
  void* ws = nullptr;
  if (need) {
    s = scratch_address(&ws);
    if (s != QSA_OK) return s;
  }
  const int64_t stride = max_len * desc->n_kv_heads * desc->head_dim;
  return hip_status(qsa::launch_attn(p, q, k_cache, v_cache, stride, 0, kv_len, desc->n_q_heads,
                                     desc->n_kv_heads, block_size, top_k_blocks, sel_blocks, sel_count,
                                     desc->softmax_scale, out, lse, ws, (hipStream_t)stream),
                    "sparse_attn_decode_noalloc launch");
}

/* ----------------------------------------------------------- comparator --- */

size_t qsa_dense_attn_workspace_size(const qsa_attn_desc_t* desc, int32_t batch, int32_t n_q,
                                     int64_t max_len) {
  if (check_attn_desc(desc) != QSA_OK || batch < 0 || n_q < 0 || max_len < 1) return 0;
  if (n_q == 1 && batch >= 1) {
    const qsa::AttnPlan p = qsa::plan_attn(batch, max_len, true);
    return qsa::attn_workspace_bytes(p, desc->n_q_heads);
  }
  return 0;
}

qsa_status_t qsa_dense_attn_prefill(const qsa_attn_desc_t* desc, const uint16_t* q,
                                    const uint16_t* k, const uint16_t* v, int64_t q_pos0,
                                    int32_t n_q, int64_t kv_len, uint16_t* out, float* lse,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  qsa_status_t s = check_attn_desc(desc);
  if (s != QSA_OK) return s;
  if (q_pos0 < 0 || n_q < 0 || kv_len < q_pos0 + n_q || kv_len > kMaxPos)
    return fail(QSA_ERR_INVALID_ARGUMENT, "need 0 <= q_pos0, q_pos0 + n_q <= kv_len < 2^31");
  if (n_q == 0) return ok();
  if (!q || !k || !v || !out) return fail(QSA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
    return fail(QSA_ERR_MISALIGNED, "q/k/v/out must be 16-byte aligned");
  if (!aligned(lse, 4)) return fail(QSA_ERR_MISALIGNED, "lse must be 4-byte aligned");
  if (32 % (desc->n_q_heads / desc->n_kv_heads))
    return fail(QSA_ERR_UNSUPPORTED, "dense prefill needs a group size dividing 32");
  (void)workspace;
  (void)workspace_bytes;
  return hip_status(qsa::launch_dense_prefill(q, k, v, q_pos0, n_q, desc->n_q_heads, desc->n_kv_heads,
                                              desc->softmax_scale, out, lse, (hipStream_t)stream),
                    "dense_attn_prefill launch");
}

qsa_status_t qsa_dense_attn_decode(const qsa_attn_desc_t* desc, const uint16_t* q,
                                   const uint16_t* k_cache, const uint16_t* v_cache,
                                   int64_t max_len, const int32_t* kv_len, int32_t batch,
                                   uint16_t* out, float* lse, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  qsa_status_t s = check_attn_desc(desc);
  if (s != QSA_OK) return s;
  if (batch < 0 || max_len < 1 || max_len > kMaxPos)
    return fail(QSA_ERR_INVALID_ARGUMENT, "need batch >= 0 and 1 <= max_len < 2^31");
  if (batch == 0) return ok();
  if (!q || !k_cache || !v_cache || !kv_len || !out)
    return fail(QSA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16))
    return fail(QSA_ERR_MISALIGNED, "q/k_cache/v_cache/out must be 16-byte aligned");
  if (!aligned(kv_len, 4) || !aligned(lse, 4))
    return fail(QSA_ERR_MISALIGNED, "int32/fp32 arrays must be 4-byte aligned");
  const qsa::AttnPlan p = qsa::plan_attn(batch, max_len, true);
  const size_t need = qsa::attn_workspace_bytes(p, desc->n_q_heads);
  if (workspace_bytes < need || (need && !workspace))
    return fail(QSA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", workspace_bytes, need);
  if (!aligned(workspace, 16)) return fail(QSA_ERR_MISALIGNED, "workspace must be 16-byte aligned");
  const int64_t stride = max_len * desc->n_kv_heads * desc->head_dim;
  return hip_status(qsa::launch_attn(p, q, k_cache, v_cache, stride, 0, kv_len, desc->n_q_heads,
                                     desc->n_kv_heads, 1, 1, nullptr, nullptr,
                                     desc->softmax_scale, out, lse, workspace,
                                     (hipStream_t)stream),
                    "dense_attn_decode launch");
}

size_t qsa_index_topk_varlen_workspace_size(const qsa_index_desc_t* desc, int32_t batch,
                                            int32_t max_q, int64_t max_q_end) {
  if (check_index_desc(desc) != QSA_OK || batch < 0 || max_q < 0 || max_q_end < max_q ||
      max_q_end > kMaxPos)
    return 0;
  if (batch == 0 || max_q == 0) return 0;
  return qsa::plan_index(desc->n_idx_heads, desc->top_k_blocks, batch, max_q, max_q_end,
                         desc->block_size, false)
      .workspace;
}

qsa_status_t qsa_index_topk_varlen(const qsa_index_desc_t* desc, const uint16_t* idx_q,
                                   const uint16_t* cmp_k, int64_t cmp_k_batch_stride,
                                   const int32_t* cu_q, const int32_t* q_pos0, int32_t batch,
                                   int32_t max_q, int64_t max_q_end, int32_t* sel_blocks,
                                   int32_t* sel_count, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  qsa_status_t s = check_index_desc(desc);
  if (s != QSA_OK) return s;
  if (batch < 0 || max_q < 0) return fail(QSA_ERR_INVALID_ARGUMENT, "negative batch or max_q");
  if (batch > 65535) return fail(QSA_ERR_UNSUPPORTED, "batch %d > 65535", batch);
  if (max_q_end < max_q || max_q_end > kMaxPos)
    return fail(QSA_ERR_INVALID_ARGUMENT, "max_q_end %lld must be in [max_q, 2^31)", (long long)max_q_end);
  if (batch == 0 || max_q == 0) return ok();
  if (!idx_q || !cmp_k || !cu_q || !q_pos0 || !sel_blocks || !sel_count)
    return fail(QSA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  if (!aligned(idx_q, 16) || !aligned(cmp_k, 16))
    return fail(QSA_ERR_MISALIGNED, "idx_q/cmp_k must be 16-byte aligned");
  if (!aligned(cu_q, 4) || !aligned(q_pos0, 4) || !aligned(sel_blocks, 4) || !aligned(sel_count, 4))
    return fail(QSA_ERR_MISALIGNED, "int32 arrays must be 4-byte aligned");
  const int r = desc->block_size;
  const int64_t need_blocks = (max_q_end - 1) / r;
  if (batch > 1) {
    if (cmp_k_batch_stride < need_blocks * desc->idx_head_dim)
      return fail(QSA_ERR_INVALID_ARGUMENT, "cmp_k_batch_stride %lld < %lld blocks x 64",
                  (long long)cmp_k_batch_stride, (long long)need_blocks);
    if (cmp_k_batch_stride % 8) return fail(QSA_ERR_MISALIGNED, "cmp_k_batch_stride not a multiple of 8");
  }
  const qsa::IndexPlan p =
      qsa::plan_index(desc->n_idx_heads, desc->top_k_blocks, batch, max_q, max_q_end, r, false);
  const qsa::PlanCheck pc = qsa::check_index_plan(p, batch, max_q);
  if (pc.unfit) return fail(QSA_ERR_UNSUPPORTED, "index_topk_varlen: %s", pc.unfit);
  if (workspace_bytes < p.workspace || (p.workspace && !workspace))
    return fail(QSA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", workspace_bytes, p.workspace);
  if (!aligned(workspace, 16)) return fail(QSA_ERR_MISALIGNED, "workspace must be 16-byte aligned");
  return hip_status(qsa::launch_index_topk(p, idx_q, cmp_k, cmp_k_batch_stride, q_pos0, batch, max_q,
                                           r, desc->top_k_blocks, desc->idx_head_weight, sel_blocks,
                                           sel_count, workspace, (hipStream_t)stream, cu_q),
                    "index_topk_varlen launch");
}

qsa_status_t qsa_sparse_attn_prefill_paged(const qsa_attn_desc_t* desc, int32_t block_size,
                                           int32_t top_k_blocks, const uint16_t* q,
                                           const uint16_t* k_pages, const uint16_t* v_pages,
                                           int32_t page_size, int64_t n_pages,
                                           const int32_t* page_table, int32_t max_pages,
                                           const int32_t* cu_q, const int32_t* q_pos0, int32_t batch,
                                           int32_t total_q, const int32_t* sel_blocks,
                                           const int32_t* sel_count, uint16_t* out, float* lse,
                                           void* stream) {
  qsa_status_t s = check_attn_common(desc, block_size, top_k_blocks);
  if (s != QSA_OK) return s;
  if (batch < 0 || total_q < 0 || max_pages < 0 || n_pages < 0)
    return fail(QSA_ERR_INVALID_ARGUMENT, "negative batch, total_q, max_pages or n_pages");
  if (page_size < block_size || page_size > (1 << 24) || (page_size & (page_size - 1)))
    return fail(QSA_ERR_INVALID_ARGUMENT, "page_size %d must be a power of two >= block_size %d",
                page_size, block_size);
  if (n_pages * (int64_t)page_size > kMaxPos)
    return fail(QSA_ERR_INVALID_ARGUMENT, "n_pages * page_size must be below 2^31");
  if (batch == 0 || total_q == 0) return ok();
  if (!q || !k_pages || !v_pages || !page_table || !cu_q || !q_pos0 || !sel_blocks || !sel_count || !out)
    return fail(QSA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  if (!aligned(q, 16) || !aligned(k_pages, 16) || !aligned(v_pages, 16) || !aligned(out, 16))
    return fail(QSA_ERR_MISALIGNED, "q/k_pages/v_pages/out must be 16-byte aligned");
  if (!aligned(page_table, 4) || !aligned(cu_q, 4) || !aligned(q_pos0, 4) || !aligned(sel_blocks, 4) ||
      !aligned(sel_count, 4) || !aligned(lse, 4))
    return fail(QSA_ERR_MISALIGNED, "int32/fp32 arrays must be 4-byte aligned");
  const qsa::AttnPlan p = qsa::plan_attn(total_q, (int64_t)top_k_blocks * block_size, false);
  const qsa::PlanCheck pc = qsa::check_attn_plan(p, desc->n_q_heads, desc->n_kv_heads, top_k_blocks, block_size);
  if (pc.unfit) return fail(QSA_ERR_UNSUPPORTED, "sparse_attn_prefill_paged: %s", pc.unfit);
  const qsa::PagedRows pg{cu_q, q_pos0, batch, page_table, max_pages, __builtin_ctz((unsigned)page_size)};
  return hip_status(qsa::launch_attn(p, q, k_pages, v_pages, 0, 0, nullptr, desc->n_q_heads,
                                     desc->n_kv_heads, block_size, top_k_blocks, sel_blocks, sel_count,
                                     desc->softmax_scale, out, lse, nullptr, (hipStream_t)stream, pg),
                    "sparse_attn_prefill_paged launch");
}

size_t qsa_distill_kl_workspace_size(const qsa_attn_desc_t* adesc, int32_t n_q) {
  if (check_attn_desc(adesc) != QSA_OK || n_q < 0) return 0;
  return (size_t)n_q * adesc->n_q_heads * sizeof(float);
}

qsa_status_t qsa_distill_kl_prefill(const qsa_attn_desc_t* adesc, const qsa_index_desc_t* idesc,
                                    const uint16_t* q, const uint16_t* k, const uint16_t* idx_q,
                                    const uint16_t* cmp_k, int64_t q_pos0, int32_t n_q, int64_t kv_len,
                                    float* kl, void* workspace, size_t workspace_bytes, void* stream) {
  qsa_status_t s = check_attn_desc(adesc);
  if (s != QSA_OK) return s;
  s = check_index_desc(idesc);
  if (s != QSA_OK) return s;
  if (adesc->n_q_heads != 8 * adesc->n_kv_heads)
    return fail(QSA_ERR_UNSUPPORTED, "distillation loss needs 8 query heads per KV head");
  if (idesc->n_idx_heads != 8) return fail(QSA_ERR_UNSUPPORTED, "distillation loss needs 8 indexer heads");
  if (q_pos0 < 0 || n_q < 0 || kv_len < q_pos0 + n_q || kv_len > kMaxPos)
    return fail(QSA_ERR_INVALID_ARGUMENT, "need 0 <= q_pos0, q_pos0 + n_q <= kv_len < 2^31");
  if (n_q == 0) return ok();
  if (!q || !k || !idx_q || !cmp_k || !kl) return fail(QSA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(idx_q, 16) || !aligned(cmp_k, 16))
    return fail(QSA_ERR_MISALIGNED, "q/k/idx_q/cmp_k must be 16-byte aligned");
  if (!aligned(kl, 4)) return fail(QSA_ERR_MISALIGNED, "kl must be 4-byte aligned");
  const size_t need = (size_t)n_q * adesc->n_q_heads * sizeof(float);
  if (workspace_bytes < need || !workspace)
    return fail(QSA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", workspace_bytes, need);
  if (!aligned(workspace, 16)) return fail(QSA_ERR_MISALIGNED, "workspace must be 16-byte aligned");
  return hip_status(qsa::launch_distill_kl(q, k, idx_q, cmp_k, q_pos0, n_q, adesc->n_q_heads, adesc->n_kv_heads,
                                           idesc->block_size, adesc->softmax_scale, idesc->idx_head_weight,
                                           reinterpret_cast<float*>(workspace), kl, (hipStream_t)stream),
                    "distill_kl launch");
}

static qsa_status_t check_gdn_desc(const qsa_gdn_desc_t* d) {
  if (!d) return fail(QSA_ERR_INVALID_ARGUMENT, "gdn desc is NULL");
  if (d->key_dim != 128 || d->value_dim != 128)
    return fail(QSA_ERR_UNSUPPORTED, "key_dim %d / value_dim %d: only 128 is supported", d->key_dim, d->value_dim);
  if (d->n_qk_heads < 1 || d->n_v_heads < 1 || d->n_v_heads % d->n_qk_heads)
    return fail(QSA_ERR_INVALID_ARGUMENT, "n_v_heads %d not a positive multiple of n_qk_heads %d", d->n_v_heads,
                d->n_qk_heads);
  if (d->n_v_heads > 65535) return fail(QSA_ERR_UNSUPPORTED, "n_v_heads %d > 65535", d->n_v_heads);
  if (!isfinite(d->scale)) return fail(QSA_ERR_INVALID_ARGUMENT, "scale not finite");
  return QSA_OK;
}

size_t qsa_gdn_prefill_workspace_size(const qsa_gdn_desc_t* desc, int32_t batch, int64_t seq_len) {
  if (check_gdn_desc(desc) != QSA_OK || batch < 0 || seq_len < 0) return 0;
  return qsa::gdn_workspace_bytes(batch, seq_len, desc->n_v_heads);
}

qsa_status_t qsa_gdn_prefill(const qsa_gdn_desc_t* desc, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                             const float* g, const float* beta, const float* initial_state, int32_t batch,
                             int64_t seq_len, uint16_t* out, float* final_state, void* workspace,
                             size_t workspace_bytes, void* stream) {
  qsa_status_t s = check_gdn_desc(desc);
  if (s != QSA_OK) return s;
  if (batch < 0 || seq_len < 0) return fail(QSA_ERR_INVALID_ARGUMENT, "negative batch or seq_len");
  if (batch > 65535) return fail(QSA_ERR_UNSUPPORTED, "batch %d > 65535", batch);
  if (seq_len > ((int64_t)1 << 37)) return fail(QSA_ERR_UNSUPPORTED, "seq_len %lld too large", (long long)seq_len);
  if (batch == 0) return ok();
  if (seq_len > 0 && (!q || !k || !v || !g || !beta || !out))
    return fail(QSA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16))
    return fail(QSA_ERR_MISALIGNED, "q/k/v must be 16-byte aligned");
  if (!aligned(g, 4) || !aligned(beta, 4) || !aligned(out, 2) || !aligned(initial_state, 4) ||
      !aligned(final_state, 4))
    return fail(QSA_ERR_MISALIGNED, "g/beta/states must be 4-byte and out 2-byte aligned");
  const size_t need = qsa::gdn_workspace_bytes(batch, seq_len, desc->n_v_heads);
  if (need > 0 && (workspace_bytes < need || !workspace))
    return fail(QSA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", workspace_bytes, need);
  if (!aligned(workspace, 16)) return fail(QSA_ERR_MISALIGNED, "workspace must be 16-byte aligned");
  if (seq_len == 0 && !final_state) return ok();
  return hip_status(qsa::launch_gdn_prefill(q, k, v, g, beta, initial_state, batch, seq_len, desc->n_qk_heads,
                                            desc->n_v_heads, desc->scale, out, final_state, workspace,
                                            (hipStream_t)stream),
                    "gdn prefill launch");
}

qsa_status_t qsa_gdn_decode(const qsa_gdn_desc_t* desc, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            const float* g, const float* beta, float* state, int32_t batch, uint16_t* out,
                            void* stream) {
  qsa_status_t s = check_gdn_desc(desc);
  if (s != QSA_OK) return s;
  if (batch < 0) return fail(QSA_ERR_INVALID_ARGUMENT, "negative batch");
  if (batch > 65535) return fail(QSA_ERR_UNSUPPORTED, "batch %d > 65535", batch);
  if (batch == 0) return ok();
  if (!q || !k || !v || !g || !beta || !state || !out) return fail(QSA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  if (!aligned(q, 8) || !aligned(k, 8) || !aligned(v, 2) || !aligned(out, 2))
    return fail(QSA_ERR_MISALIGNED, "q/k must be 8-byte and v/out 2-byte aligned");
  if (!aligned(state, 16)) return fail(QSA_ERR_MISALIGNED, "state must be 16-byte aligned");
  if (!aligned(g, 4) || !aligned(beta, 4)) return fail(QSA_ERR_MISALIGNED, "g/beta must be 4-byte aligned");
  return hip_status(qsa::launch_gdn_decode(q, k, v, g, beta, batch, desc->n_qk_heads, desc->n_v_heads, desc->scale,
                                           state, out, (hipStream_t)stream),
                    "gdn decode launch");
}

}  // extern "C"
