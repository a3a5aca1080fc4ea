// Forward of the indexer's dense-distillation loss (explainer page
// "用125亿分之6的参数…", sparse-attention section: in the first training stage
// only the indexer learns, pulled towards the full-attention model's attention
// distribution by a KL divergence). Per query t with own block b_t:
//   target    P_j ~ M_j = sum over the query heads h and the tokens s of block j
//             of the dense causal softmax a_h(s) (tokens s <= t), renormalised
//             over the candidate blocks j < b_t;
//   indexer   Q_j = softmax over j < b_t of the indexer score s_j;
//   loss      KL_t = sum_j P_j (ln P_j - ln Q_j)
//                  = S1 / MM - ln MM - S2 / MM + lse(s),
//             S1 = sum M ln M, S2 = sum M s, MM = sum M over the candidates.
// Pass 1 is the dense kernel without P V (per-row log-sum-exp); pass 2 below
// streams the prefix once more per group of 8 queries.
//
// Pass 2: a workgroup owns 8 consecutive queries; wave g is KV head g and
// holds two 32-row A tiles (4 queries x the 8 query heads of g) of
// v_mfma_f32_32x32x16_bf16. Per 32-token sub-chunk, S = Q K^T comes out with a
// lane per token and 4 heads x 4 queries per lane-half: the exponentials with
// the final log-sum-exp are summed over heads in-lane and across the halves,
// over the r tokens of a block across lanes, and over the KV heads through LDS
// float atomics. Every 32 blocks the indexer scores of the 8 queries (one A
// tile of 4 queries x 8 indexer heads per wave 0 / 1) are formed on the same
// MFMA and the four sums above are accumulated per lane, then reduced at the
// end. Supported: Hq / Hkv = 8 query heads per KV head, 8 indexer heads.
#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {

namespace {
constexpr int kLD = 128;  // head dim
constexpr int kLQ = 8;    // queries per workgroup

struct KlAcc {
  float s1, s2, mm, mx, z;
};

__device__ __forceinline__ void kl_merge(KlAcc& a, const KlAcc& b) {
  a.s1 += b.s1;
  a.s2 += b.s2;
  a.mm += b.mm;
  const float m = fmaxf(a.mx, b.mx);
  if (m == -INFINITY) return;
  a.z = a.z * fast_exp2(a.mx - m) + b.z * fast_exp2(b.mx - m);
  a.mx = m;
}
}  // namespace

template <int HKV>
__global__ __launch_bounds__(64 * HKV) void distill_kl_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ idx_q,
    const uint16_t* __restrict__ cmp_k, const float* __restrict__ lse_h, int64_t q_pos0, int n_q, int r,
    float scale_log2, float w_idx, float* __restrict__ kl) {
  constexpr int G = 8;
  constexpr int Hq = HKV * G;
  __shared__ float mass[kLQ][32];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int col = lane & 31;
  const int g = wave;
  const int q0 = blockIdx.x * kLQ;
  const int nq_wg = min(kLQ, n_q - q0);
  const int64_t t_last = q_pos0 + q0 + nq_wg - 1;
  const int64_t bt_last = t_last / r;
  const float log2e = 1.4426950408889634f;

  // A tiles: row m of tile T is query q0 + 4T + m / 8, head 8g + m % 8
  u32x4 Qa[2][8];
#pragma unroll
  for (int T = 0; T < 2; ++T) {
    const int qi = q0 + 4 * T + col / 8;
    const bool ok = qi < n_q;
    const uint16_t* qp = q + ((int64_t)(ok ? qi : 0) * Hq + G * g + col % 8) * kLD + 8 * half;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) Qa[T][ks] = ok ? ld16(qp + 16 * ks) : u32x4{0u, 0u, 0u, 0u};
  }
  // accumulator i of tile T: query 4T + i / 4, head 8g + 4half + i % 4
  float L2[2][16];
  const int lr = __builtin_ctz((unsigned)r);  // r is a power of two
  int64_t tq[kLQ];   // query positions
  int64_t btq[kLQ];  // their own blocks: candidates are the blocks below
#pragma unroll
  for (int x = 0; x < kLQ; ++x) {
    tq[x] = q_pos0 + q0 + x;
    btq[x] = tq[x] >> lr;
  }
#pragma unroll
  for (int T = 0; T < 2; ++T)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int qi = q0 + 4 * T + i / 4;
      L2[T][i] = qi < n_q ? lse_h[(int64_t)qi * Hq + G * g + 4 * half + (i & 3)] * log2e : INFINITY;
    }
  // indexer A tile of the tile this wave scores: row m = query 4T + m / 8, indexer head m % 8
  const int my_tile = wave < 2 ? wave : -1;
  const int T_count = HKV == 1 ? 2 : 1;  // one wave scores both tiles when it is alone
  u32x4 Ia[2][4];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int T = HKV == 1 ? u : my_tile;
    const int qi = q0 + 4 * (T < 0 ? 0 : T) + col / 8;
    const bool ok = T >= 0 && u < T_count && qi < n_q;
    const uint16_t* ip = idx_q + ((int64_t)(ok ? qi : 0) * 8 + col % 8) * 64 + 8 * half;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) Ia[u][ks] = ok ? ld16(ip + 16 * ks) : u32x4{0u, 0u, 0u, 0u};
  }
  KlAcc acc[2][4];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) acc[u][qq] = KlAcc{0.0f, 0.0f, 0.0f, -INFINITY, 0.0f};

  for (int i = tid; i < kLQ * 32; i += 64 * HKV) (&mass[0][0])[i] = 0.0f;
  __syncthreads();

  const uint16_t* kb = k + (int64_t)g * kLD + 8 * half;
  // the K fragments of the next sub-chunk of 32 tokens are in flight while the
  // current one is reduced (sub-chunks run on across block groups)
  u32x4 Kn[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) Kn[ks] = ld16(kb + min((int64_t)col, t_last) * HKV * kLD + 16 * ks);
  for (int64_t jb = 0; jb < bt_last; jb += 32) {
    // masses of blocks [jb, jb + 32): r sub-chunks of 32 tokens
    for (int u = 0; u < r; ++u) {
      const int64_t c0 = jb * r + 32 * u;
      if (c0 > t_last) break;
      u32x4 Kb[8];
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) Kb[ks] = Kn[ks];
      if (c0 + 32 <= t_last) {
        const int64_t tok = min(c0 + 32 + col, t_last);
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) Kn[ks] = ld16(kb + tok * HKV * kLD + 16 * ks);
      }
#pragma unroll
      for (int T = 0; T < 2; ++T) {
        f32x16 S = f32x16{};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) S = mfma32x32x16(Qa[T][ks], Kb[ks], S);
        float mq[4];
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          float m = 0.0f;
          if (c0 + col <= tq[4 * T + qq]) {
#pragma unroll
            for (int hh = 0; hh < 4; ++hh) m += fast_exp2(fmaf(S[4 * qq + hh], scale_log2, -L2[T][4 * qq + hh]));
          }
          mq[qq] = m + __shfl_xor(m, 32);
        }
        for (int off = 1; off < r && off < 32; off <<= 1)
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) mq[qq] += __shfl_xor(mq[qq], off);
        if (half == 0 && (col & (r - 1)) == 0) {
          const int blk = (32 * u + col) / r;
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) atomicAdd(&mass[4 * T + qq][blk], mq[qq]);
        }
      }
    }
    __syncthreads();
    // indexer scores of the same 32 blocks and the loss sums
    if (wave < 2 || HKV == 1) {
      const int64_t jrow = min(jb + col, bt_last - 1);
      u32x4 Bc[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) Bc[ks] = ld16(cmp_k + jrow * 64 + 8 * half + 16 * ks);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        if (u >= T_count) break;
        const int T = HKV == 1 ? u : my_tile;
        f32x16 C = f32x16{};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) C = mfma32x32x16(Ia[u][ks], Bc[ks], C);
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          float sc = 0.0f;
#pragma unroll
          for (int hh = 0; hh < 4; ++hh) sc += fmaxf(C[4 * qq + hh], 0.0f);
          sc = (sc + __shfl_xor(sc, 32)) * w_idx;
          const int x = 4 * T + qq;
          const int64_t j = jb + col;
          if (half == 0 && x < nq_wg && j < btq[x]) {
            const float M = mass[x][col];
            KlAcc& a = acc[u][qq];
            if (M > 0.0f) a.s1 += M * __logf(M);
            a.s2 += M * sc;
            a.mm += M;
            const float sl = sc * log2e;  // online log-sum-exp of the scores (base 2)
            if (sl > a.mx) {
              a.z = a.z * fast_exp2(a.mx - sl) + 1.0f;
              a.mx = sl;
            } else {
              a.z += fast_exp2(sl - a.mx);
            }
          }
        }
      }
    }
    __syncthreads();
    for (int i = tid; i < kLQ * 32; i += 64 * HKV) (&mass[0][0])[i] = 0.0f;
    __syncthreads();
  }
  // reduce the lanes of half 0 and write the loss
  if (wave < 2 || HKV == 1) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (u >= T_count) break;
      const int T = HKV == 1 ? u : my_tile;
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        KlAcc a = acc[u][qq];
        if (half) a = KlAcc{0.0f, 0.0f, 0.0f, -INFINITY, 0.0f};
#pragma unroll
        for (int off = 1; off < 32; off <<= 1) {
          KlAcc b;
          b.s1 = __shfl_xor(a.s1, off);
          b.s2 = __shfl_xor(a.s2, off);
          b.mm = __shfl_xor(a.mm, off);
          b.mx = __shfl_xor(a.mx, off);
          b.z = __shfl_xor(a.z, off);
          kl_merge(a, b);
        }
        const int x = 4 * T + qq;
        if (lane == 0 && x < nq_wg) {
          float v = 0.0f;
          if (btq[x] > 0 && a.mm > 0.0f) {
            const float lse_s = (a.mx + __log2f(a.z)) * 0.69314718055994531f;
            v = a.s1 / a.mm - __logf(a.mm) - a.s2 / a.mm + lse_s;
          }
          kl[q0 + x] = v;
        }
      }
    }
  }
}

hipError_t launch_distill_kl(const uint16_t* q, const uint16_t* k, const uint16_t* idx_q, const uint16_t* cmp_k,
                             int64_t q_pos0, int n_q, int Hq, int Hkv, int r, float scale, float w_idx,
                             float* lse_ws, float* kl, hipStream_t stream) {
  // pass 1: per-row log-sum-exp of the dense causal attention
  hipError_t e = launch_dense_prefill(q, k, k, q_pos0, n_q, Hq, Hkv, scale, nullptr, lse_ws, stream);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((n_q + kLQ - 1) / kLQ));
  const float sl2 = scale * 1.4426950408889634f;
  switch (Hkv) {
    case 1: hipLaunchKernelGGL(distill_kl_kernel<1>, grid, dim3(64), 0, stream, q, k, idx_q, cmp_k, lse_ws, q_pos0, n_q, r, sl2, w_idx, kl); break;
    case 2: hipLaunchKernelGGL(distill_kl_kernel<2>, grid, dim3(128), 0, stream, q, k, idx_q, cmp_k, lse_ws, q_pos0, n_q, r, sl2, w_idx, kl); break;
    case 4: hipLaunchKernelGGL(distill_kl_kernel<4>, grid, dim3(256), 0, stream, q, k, idx_q, cmp_k, lse_ws, q_pos0, n_q, r, sl2, w_idx, kl); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace qsa
