// Micro-block key compression: the indexer key of block j is the mean of the
// r token keys j*r .. j*r+r-1 (explainer page "用125亿分之6的参数…", section
// on sparse attention: consecutive tokens are packed into a micro-block and
// mean-pooled into one representative key).
//
// Arithmetic is fixed so the stored block key is one exact byte pattern:
// fp32 sum in token order, times 1/r (r is a power of two, so this equals the
// division), round to nearest even bf16.
//
// One thread per (block, 8 dims): r loads of 16 bytes, one 16-byte store.
// Eight neighbouring threads cover one 128-byte key row, so every wave reads
// and writes whole rows.
#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {

__global__ __launch_bounds__(256) void compress_kernel(const uint16_t* __restrict__ idx_k,
                                                       int64_t k_stride, int d, int r,
                                                       int64_t first, int64_t n,
                                                       uint16_t* __restrict__ cmp,
                                                       int64_t c_stride) {
  const int groups = d >> 3;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= n * groups) return;
  const int b = blockIdx.y;
  const int64_t j = first + gid / groups;
  const int g = (int)(gid % groups);
  const uint16_t* src = idx_k + (int64_t)b * k_stride + j * r * d + g * 8;
  float acc[8];
  {
    const u32x4 v = ld16(src);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] = bf16_bits_to_f32(v[e] & 0xFFFFu);
      acc[2 * e + 1] = bf16_bits_to_f32(v[e] >> 16);
    }
  }
  for (int m = 1; m < r; ++m) {
    const u32x4 v = ld16(src + (int64_t)m * d);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] = acc[2 * e] + bf16_bits_to_f32(v[e] & 0xFFFFu);
      acc[2 * e + 1] = acc[2 * e + 1] + bf16_bits_to_f32(v[e] >> 16);
    }
  }
  const float inv = 1.0f / (float)r;  // exact: r is a power of two
  u32x4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = pack_bf16x2(acc[2 * e] * inv, acc[2 * e + 1] * inv);
  st16(cmp + (int64_t)b * c_stride + j * d + g * 8, o);
}

hipError_t launch_compress(const uint16_t* idx_k, int64_t k_stride, int batch, int d, int r,
                           int64_t first, int64_t n, uint16_t* cmp, int64_t c_stride,
                           hipStream_t stream) {
  if (n == 0 || batch == 0) return hipSuccess;
  const int64_t threads = n * (d / 8);
  const dim3 grid((unsigned)((threads + 255) / 256), (unsigned)batch);
  hipLaunchKernelGGL(compress_kernel, grid, dim3(256), 0, stream, idx_k, k_stride, d, r, first, n,
                     cmp, c_stride);
  return hipGetLastError();
}

}  // namespace qsa
