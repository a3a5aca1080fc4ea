// Dense causal grouped-query flash attention, prefill: the comparator the
// sparse path is measured against (explainer page "用125亿分之6的参数…",
// sparse-attention section: QSA's speedups are quoted against GQA at a 1M-token
// context). Not part of the method.
//
// A workgroup (4 waves) owns 128 query rows of one KV head g: 128 / G
// consecutive queries x the G query heads that read g. Each wave holds 32 rows
// (Q^T in registers as the B operand) and streams the K/V prefix through LDS
// in 64-token tiles (double-buffered, loads for tile t+1 issued before tile t
// is computed). Per 32-token chunk, on v_mfma_f32_32x32x16_bf16:
//   S^T = K Q^T   (32 tokens x 32 rows): a lane owns one query row and 16 of
//                 its tokens, so the softmax max/sum are in-lane plus one
//                 cross-half exchange;
//   O  += P V     (32 rows x 128 dims): P leaves the S^T accumulators already in
//                 A-operand layout (the chunk's token order is permuted
//                 consistently for P and for V); the V operand is read from the
//                 row-major LDS tile with ds_read_b64_tr_b16, which hands each
//                 lane 4 consecutive tokens of one dimension (two reads per
//                 MFMA).
// Online softmax in fp32 with base-2 exponents and a lazy rescale: a row's
// reference maximum moves (and its O and l are rescaled) only when a chunk's
// maximum exceeds it by more than 2^8, so P stays below 256 and most chunks
// skip the rescale; the per-row factor goes from the S^T layout to the O
// layout through LDS.
#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {

namespace {
constexpr int kFD = 128;           // head dim
constexpr int kFTile = 64;         // tokens per LDS tile
constexpr int kFRows = 128;        // query rows per workgroup
constexpr int kKPitch = 128 + 16;  // LDS row pitch (elements): 288 B, conflict-free for both read forms
constexpr float kLazy = 8.0f;      // log2 headroom before a row's reference maximum moves

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// 4 consecutive tokens of one dimension per lane (see the header comment).
__device__ __forceinline__ uint2 ld_tr16(const uint16_t* p) {
  const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p);
  return __builtin_bit_cast(uint2, v);
}
}  // namespace

// WITH_O = false computes only the per-row log-sum-exp (no V, no P V): the
// first pass of the distillation loss.
template <bool WITH_O>
__global__ __launch_bounds__(256, 2) void dense_prefill_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    int64_t q_pos0, int n_q, int Hq, int Hkv, int G, float scale_log2, uint16_t* __restrict__ out,
    float* __restrict__ lse) {
  __shared__ __attribute__((aligned(16))) uint16_t kt[2][kFTile * kKPitch];
  __shared__ __attribute__((aligned(16))) uint16_t vt[2][kFTile * kKPitch];
  __shared__ float alpha_x[4][32];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int col = lane & 31;
  const int g = blockIdx.y;
  const int qpw = 32 / G;                      // queries per wave
  const int q_wg0 = blockIdx.x * (kFRows / G);  // first query of the workgroup
  // this lane's query row (column of S^T): query q_wg0 + wave*qpw + col/G, head col%G
  const int my_q = q_wg0 + wave * qpw + col / G;
  const int my_h = g * G + col % G;
  const bool my_valid = my_q < n_q;
  const int64_t my_t = q_pos0 + my_q;
  const int last_q = min(q_wg0 + kFRows / G, n_q) - 1;
  const int64_t t_end = q_pos0 + last_q + 1;   // tokens 0 .. t_end-1 are read by some row
  const int64_t wave_tmin = q_pos0 + q_wg0 + wave * qpw;  // smallest t of this wave

  // Q^T fragments: k index = dims 16ks + 8half .. +8, column = this lane's row
  u32x4 Qf[8];
  {
    const uint16_t* qp = q + ((int64_t)(my_valid ? my_q : 0) * Hq + my_h) * kFD + 8 * half;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) Qf[ks] = my_valid ? ld16(qp + 16 * ks) : u32x4{0u, 0u, 0u, 0u};
  }

  const int64_t kv_stride = (int64_t)Hkv * kFD;  // elements between tokens
  const uint16_t* kb = k + (int64_t)g * kFD;
  const uint16_t* vb = v + (int64_t)g * kFD;
  // tile loader: 64 tokens x 128 dims = 1024 16-byte chunks, 4 per thread
  auto load_tile = [&](int64_t t0, u32x4* RK, u32x4* RV) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = tid + 256 * u;
      const int row = c >> 4, part = c & 15;
      const int64_t s = min(t0 + row, t_end - 1);
      RK[u] = ld16(kb + s * kv_stride + part * 8);
      if (WITH_O) RV[u] = ld16(vb + s * kv_stride + part * 8);
    }
  };
  auto store_tile = [&](int buf, const u32x4* RK, const u32x4* RV) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = tid + 256 * u;
      const int row = c >> 4, part = c & 15;
      *reinterpret_cast<u32x4*>(&kt[buf][row * kKPitch + part * 8]) = RK[u];
      if (WITH_O) *reinterpret_cast<u32x4*>(&vt[buf][row * kKPitch + part * 8]) = RV[u];
    }
  };
  // transposed V reads: lane group gr = lane / 16 covers dims +16 (gr % 2) of
  // an n-tile and token half gr / 2; within the group, source lane 4j + qd
  // addresses token j, dims 4qd .. 4qd+3
  const int gr = lane >> 4, sl = lane & 15;
  const int tr_off = ((gr >> 1) * 4 + (sl >> 2)) * kKPitch + 16 * (gr & 1) + 4 * (sl & 3);

  float m_run = -INFINITY;  // this lane's row: reference maximum (log2 units)
  float l_run = 0.0f;       // this lane's share of the row sum
  f32x16 O[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) O[nt] = f32x16{};

  const int ntiles = (int)((t_end + kFTile - 1) / kFTile);
  u32x4 RK[4], RV[4];
  load_tile(0, RK, RV);
  store_tile(0, RK, RV);
  if (ntiles > 1) load_tile(kFTile, RK, RV);
  for (int tile = 0; tile < ntiles; ++tile) {
    const int buf = tile & 1;
    __syncthreads();  // tile's buffer is written; the other buffer is free
    if (tile + 1 < ntiles) {
      store_tile(buf ^ 1, RK, RV);
      if (tile + 2 < ntiles) load_tile((int64_t)(tile + 2) * kFTile, RK, RV);
    }
    const int64_t t0 = (int64_t)tile * kFTile;
    if (t0 > wave_tmin + qpw - 1) continue;  // every row of this wave is before this tile
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) {
      const int64_t c0 = t0 + 32 * ch;
      // S^T: rows = tokens c0 + col (A from LDS K rows), columns = query rows
      f32x16 S = f32x16{};
      const uint16_t* krow = &kt[buf][(32 * ch + col) * kKPitch + 8 * half];
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(krow + 16 * ks);
        S = mfma32x32x16(a, Qf[ks], S);
      }
      // this lane: row `col`, tokens c0 + 8(i/4) + 4half + i%4
      if (c0 + 31 > wave_tmin) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int64_t s = c0 + 8 * (i >> 2) + 4 * half + (i & 3);
          if (s > my_t) S[i] = -INFINITY;
        }
      }
      float cmax = S[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) cmax = fmaxf(cmax, S[i]);
      cmax = fmaxf(cmax, __shfl_xor(cmax, 32)) * scale_log2;
      const bool up = cmax > m_run + kLazy;
      if (ballot(up)) {
        const float m_new = up ? cmax : m_run;
        const float alpha = up ? exp2f(m_run - m_new) : 1.0f;
        m_run = m_new;
        l_run *= alpha;
        if (WITH_O) {
          // alpha of row `col` -> O layout (rows 8(i/4) + 4half + i%4)
          if (half == 0) alpha_x[wave][col] = alpha;
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float a = alpha_x[wave][8 * (i >> 2) + 4 * half + (i & 3)];
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) O[nt][i] *= a;
          }
          __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
          __builtin_amdgcn_wave_barrier();
        }
      }
      float psum = 0.0f;
      uint32_t pk[8];
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const float p0 = fast_exp2(fmaf(S[i], scale_log2, -m_run));
        const float p1 = fast_exp2(fmaf(S[i + 1], scale_log2, -m_run));
        psum += p0 + p1;
        pk[i >> 1] = pack_bf16x2_hw(p0, p1);
      }
      l_run += psum;
      if (!WITH_O) continue;
      // O += P V: k-step kk holds this lane's tokens i in [8kk, 8kk + 8), i.e.
      // chunk tokens 16kk + 4half + {0..3} and 16kk + 8 + 4half + {0..3}
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const u32x4 Pa = u32x4{pk[4 * kk], pk[4 * kk + 1], pk[4 * kk + 2], pk[4 * kk + 3]};
        const uint16_t* vrow = &vt[buf][(32 * ch + 16 * kk) * kKPitch + tr_off];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          const uint2 lo = ld_tr16(vrow + 32 * nt);
          const uint2 hi = ld_tr16(vrow + 8 * kKPitch + 32 * nt);
          O[nt] = mfma32x32x16(Pa, u32x4{lo.x, lo.y, hi.x, hi.y}, O[nt]);
        }
      }
    }
  }
  // finish: row sums over both halves, then O / l in bf16, lse in natural log
  float l_row = l_run + __shfl_xor(l_run, 32);
  if (!WITH_O) {
    if (lse && half == 0 && my_valid) lse[(int64_t)my_q * Hq + my_h] = (m_run + log2f(l_row)) * 0.69314718055994531f;
    return;
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
  if (half == 0) alpha_x[wave][col] = 1.0f / l_row;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int row = 8 * (i >> 2) + 4 * half + (i & 3);
    const int rq = q_wg0 + wave * qpw + row / G;
    const int rh = g * G + row % G;
    if (rq < n_q) {
      const float inv = alpha_x[wave][row];
      uint16_t* op = out + ((int64_t)rq * Hq + rh) * kFD;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) op[32 * nt + col] = (uint16_t)f32_to_bf16_bits(O[nt][i] * inv);
    }
  }
  if (lse && half == 0 && my_valid) lse[(int64_t)my_q * Hq + my_h] = (m_run + log2f(l_row)) * 0.69314718055994531f;
}

hipError_t launch_dense_prefill(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t q_pos0,
                                int n_q, int Hq, int Hkv, float scale, uint16_t* out, float* lse,
                                hipStream_t stream) {
  const int G = Hq / Hkv;
  if (32 % G) return hipErrorInvalidValue;
  const int q_per_wg = kFRows / G;
  const dim3 grid((unsigned)((n_q + q_per_wg - 1) / q_per_wg), (unsigned)Hkv);
  if (out)
    hipLaunchKernelGGL(dense_prefill_kernel<true>, grid, dim3(256), 0, stream, q, k, v, q_pos0, n_q, Hq, Hkv, G,
                       scale * 1.4426950408889634f, out, lse);
  else
    hipLaunchKernelGGL(dense_prefill_kernel<false>, grid, dim3(256), 0, stream, q, k, v, q_pos0, n_q, Hq, Hkv,
                       G, scale * 1.4426950408889634f, out, lse);
  return hipGetLastError();
}

}  // namespace qsa
