// Gated delta rule: the token mixing of the recurrent layers that sit between
// the attention layers (three of every four layers). Per value head the layer
// carries a matrix state S (dv x dk) and, for each token,
//   e_t = v_t - a_t S_{t-1} k_t,   S_t = a_t S_{t-1} + b_t e_t k_t^T,
//   o_t = S_t (scale q_t),   a_t = exp(g_t),
// i.e. it decays the memory, measures what the decayed memory already returns
// for the token's key and writes only the correction, gated by b_t.
//
// Prefill runs the chunked form of that recurrence (chunks of C = 64 tokens).
// Within a chunk with start state S, G_i the running sum of g over the chunk's
// tokens 0..i and gam_i = exp(G_i), every token's effective write
// u_j = b_j (v_j - P_j k_j) (P_j the decayed state just before token j)
// solves the unit lower-triangular system
//   (I + L) U = diag(b) V - diag(b gam) K S^T,
//   L_ij = b_i exp(G_i - G_j) k_i . k_j  (j < i),
// so with T = (I + L)^-1, W = T diag(b gam) K and U~ = T diag(b) V:
//   U = U~ - W S^T
//   O = diag(scale gam) Q S^T + M U,  M_ij = scale exp(G_i - G_j) q_i . k_j (j <= i)
//   S' = gam_C S + (diag(exp(G_C - G_j)) U)^T K.
// Every exponent is a difference G_i - G_j with i >= j (or G itself), so no
// factor exceeds 1. W, U~, M and the gates depend only on the chunk's own
// tokens: gdn_prep_kernel computes them for all chunks in parallel; then
// gdn_scan_kernel walks the chunks of each (sequence, value head) in order,
// carrying S in registers, with four waves splitting the 128 value rows.
// Decode (one token on a carried state) is gdn_decode_kernel: the recurrence
// itself, one pass over the fp32 state in HBM.
#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr int kC = 64;        // tokens per chunk
constexpr int kD = 128;       // key and value head dim
constexpr int kP = kD + 16;   // LDS pitch (elements) of 128-wide bf16 rows
constexpr int kMP = kC + 8;   // LDS pitch of 64-wide bf16 rows
constexpr int kTP = kC + 4;   // LDS pitch of 64-wide fp32 rows

// Workspace record of one (sequence, value head, chunk), byte offsets.
constexpr int64_t kRecW = 0;                     // -W, bf16 [64][128], dk order permuted (perm16)
constexpr int64_t kRecM = kRecW + kC * kD * 2;   // M, bf16 [64][64], column order permuted (perm16)
constexpr int64_t kRecG = kRecM + kC * kC * 2;   // gates, fp32 [256]: scale gam_i | exp(G_C - G_i) | gam_C
constexpr int64_t kRecU = kRecG + 256 * 4;       // U~, fp32 [64][128]
constexpr int64_t kRecBytes = kRecU + kC * kD * 4;

// Operand order of the k dimension. An MFMA 32x32x16 k-step takes, in lane
// half h, the eight k indices {4h .. 4h+3, 8+4h .. 8+4h+3} of its sixteen:
// that is the order in which an accumulator tile holds its rows, so a tile
// (the state, U) feeds the next product without a transpose. Matrices read as
// the other operand of such a product (W, M, Q) are stored with the middle
// two quads of every 16 swapped, which puts each lane's eight values in one
// 16-byte run. The map is its own inverse.
__device__ __forceinline__ int perm16(int x) {
  const int qd = (x >> 2) & 3;
  return (qd == 1 || qd == 2) ? x ^ 12 : x;
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// ds_read_b64_tr_b16: within each 16-lane group, lane l receives element l % 4
// of the 4-element chunk addressed by lane 4j + (l % 16) / 4, in slot j.
__device__ __forceinline__ uint2 ld_tr16(const uint16_t* p) {
  const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p);
  return __builtin_bit_cast(uint2, v);
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Offset (elements) of the transposed 64 x 16 read of a token-major tile with
// pitch kP: lane group gr = lane / 16 covers columns +16 (gr % 2) of a
// 32-column window and tokens +4 (gr / 2); source lane 4j + x addresses token
// j, columns 4x .. 4x+3. The lane then holds column (lane % 32) of the window,
// tokens 4 (lane / 32) + j, j = 0..3.
__device__ __forceinline__ int tr_offset(int lane) {
  const int gr = lane >> 4, sl = lane & 15;
  return ((gr >> 1) * 4 + (sl >> 2)) * kP + 16 * (gr & 1) + 4 * (sl & 3);
}

// ---------------------------------------------------------------- prep ----
// One workgroup (4 waves) per (chunk, value head, sequence).
__global__ __launch_bounds__(256, 2) void gdn_prep_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, int64_t T, int Hqk, int Hv, float scale,
    int n_chunks, uint8_t* __restrict__ ws) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kC * kP];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[kC * kP];
  __shared__ __attribute__((aligned(16))) uint16_t QTs[kC * kP];  // Q tile, then T (fp32 [64][kTP])
  __shared__ __attribute__((aligned(16))) float Lm[kC * kTP];
  __shared__ float Xs[3][16][17];
  __shared__ __attribute__((aligned(16))) float Gs[kC];
  __shared__ __attribute__((aligned(16))) float Bs[kC];
  __shared__ __attribute__((aligned(16))) float Fw[kC];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int half = lane >> 5, col = lane & 31;
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int hk = h / (Hv / Hqk);
  const int64_t t0 = (int64_t)c * kC;
  const int n = (int)min<int64_t>(kC, T - t0);
  uint8_t* rec = ws + (((int64_t)b * Hv + h) * n_chunks + c) * kRecBytes;
  float* Tm = reinterpret_cast<float*>(QTs);

  // tiles of K, Q (key head hk) and V (value head h); rows past the sequence are zero
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int idx = tid + 256 * u;
    const int r = idx >> 4, part = idx & 15;
    u32x4 kv = u32x4{0u, 0u, 0u, 0u}, qv = kv, vv = kv;
    if (r < n) {
      const int64_t tok = (int64_t)b * T + t0 + r;
      kv = ld16(k + (tok * Hqk + hk) * kD + 8 * part);
      qv = ld16(q + (tok * Hqk + hk) * kD + 8 * part);
      vv = ld16(v + (tok * Hv + h) * kD + 8 * part);
    }
    *reinterpret_cast<u32x4*>(&Ks[r * kP + 8 * part]) = kv;
    *reinterpret_cast<u32x4*>(&QTs[r * kP + 8 * part]) = qv;
    *reinterpret_cast<u32x4*>(&Vs[r * kP + 8 * part]) = vv;
  }
  if (wave == 0) {
    // running sum of the log decays over the chunk (padding adds 0)
    float x = lane < n ? g[((int64_t)b * T + t0 + lane) * Hv + h] : 0.0f;
    const float bt = lane < n ? beta[((int64_t)b * T + t0 + lane) * Hv + h] : 0.0f;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    const float gl = __shfl(x, 63);
    Gs[lane] = x;
    Bs[lane] = bt;
    Fw[lane] = bt * expf(x);
    float* gates = reinterpret_cast<float*>(rec + kRecG);
    gates[lane] = scale * expf(x);
    gates[64 + lane] = expf(gl - x);
    gates[128 + lane] = expf(gl);
    gates[192 + lane] = 0.0f;
  }
  __syncthreads();

  // K K^T -> L (fp32, LDS) and Q K^T -> M (bf16, workspace); tiles of 32 x 32
  uint16_t* Mg = reinterpret_cast<uint16_t*>(rec + kRecM);
  if (wave < 3) {
    const int ti = wave == 0 ? 0 : 1, tj = wave == 2 ? 1 : 0;
    f32x16 kk = f32x16{}, qk = f32x16{};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const u32x4 bk = *reinterpret_cast<const u32x4*>(&Ks[(32 * tj + col) * kP + 16 * ks + 8 * half]);
      const u32x4 ak = *reinterpret_cast<const u32x4*>(&Ks[(32 * ti + col) * kP + 16 * ks + 8 * half]);
      const u32x4 aq = *reinterpret_cast<const u32x4*>(&QTs[(32 * ti + col) * kP + 16 * ks + 8 * half]);
      kk = mfma32x32x16(ak, bk, kk);
      qk = mfma32x32x16(aq, bk, qk);
    }
    const int j = 32 * tj + col;
    const float gj = Gs[j];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = 32 * ti + 8 * (r >> 2) + 4 * half + (r & 3);
      const float d = expf(Gs[i] - gj);  // only read where j <= i
      Lm[i * kTP + j] = j < i ? Bs[i] * d * kk[r] : 0.0f;
      const float mv = j <= i ? scale * d * qk[r] : 0.0f;
      Mg[i * kC + perm16(j)] = (uint16_t)f32_to_bf16_bits(mv);
    }
  } else {
    // the tile above the diagonal (rows 0..31, columns 32..63) is zero
    for (int e = lane; e < 32 * 32; e += 64) {
      const int i = e >> 5, j = 32 + (e & 31);
      Mg[i * kC + perm16(j)] = 0;
    }
  }
  __syncthreads();

  // T = (I + L)^-1 in 16 x 16 blocks. Diagonal blocks first, one per wave, by
  // forward substitution (rows in order, the sum over earlier rows split over
  // the four 16-lane groups).
  {
    const int a0 = 16 * wave;
    const int cc = lane & 15, part = lane >> 4;
    for (int i = 0; i < 16; ++i) {
      float s = 0.0f;
      for (int m = part; m < i; m += 4) s += Lm[(a0 + i) * kTP + a0 + m] * Tm[(a0 + m) * kTP + a0 + cc];
      s += __shfl_xor(s, 16);
      s += __shfl_xor(s, 32);
      if (part == 0) Tm[(a0 + i) * kTP + a0 + cc] = (i == cc ? 1.0f : 0.0f) - s;
      wave_lds_sync();
    }
  }
  __syncthreads();
  // blocks below the diagonal, by distance d from it:
  // T_ab = -T_aa X, X = sum_{m in blocks b .. a-1} L_am T_mb  (a = b + d)
  for (int d = 1; d < 4; ++d) {
    const int nb = 4 - d;
    for (int e = tid; e < nb * 256; e += 256) {
      const int bb = e >> 8, i = (e >> 4) & 15, cc = e & 15;
      const int a = bb + d;
      float x = 0.0f;
      for (int m = 16 * bb; m < 16 * a; ++m) x += Lm[(16 * a + i) * kTP + m] * Tm[m * kTP + 16 * bb + cc];
      Xs[bb][i][cc] = x;
    }
    __syncthreads();
    for (int e = tid; e < nb * 256; e += 256) {
      const int bb = e >> 8, i = (e >> 4) & 15, cc = e & 15;
      const int a = bb + d;
      float x = 0.0f;
#pragma unroll
      for (int m = 0; m < 16; ++m) x += Tm[(16 * a + i) * kTP + 16 * a + m] * Xs[bb][m][cc];
      Tm[(16 * a + i) * kTP + 16 * bb + cc] = -x;
    }
    __syncthreads();
  }
  // the blocks above the diagonal of T are zero
  for (int e = tid; e < kC * kC; e += 256) {
    const int i = e >> 6, j = e & 63;
    if ((j >> 4) > (i >> 4)) Tm[i * kTP + j] = 0.0f;
  }
  __syncthreads();

  // W = T diag(b gam) K (stored negated) and U~ = T diag(b) V. The A operand
  // is a row of T scaled per column and rounded once; the B operand is the
  // token-major K or V tile read transposed. Wave w covers columns 32w..32w+31.
  {
    const int tro = tr_offset(lane);
    uint16_t* Wg = reinterpret_cast<uint16_t*>(rec + kRecW);
    float* Ug = reinterpret_cast<float*>(rec + kRecU);
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      f32x16 Wa = f32x16{}, Ua = f32x16{};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int m0 = 16 * kk + 4 * half;
        const float* trow = &Tm[(32 * rt + col) * kTP];
        const f32x4 lo = *reinterpret_cast<const f32x4*>(trow + m0);
        const f32x4 hi = *reinterpret_cast<const f32x4*>(trow + m0 + 8);
        const f32x4 fwl = *reinterpret_cast<const f32x4*>(&Fw[m0]);
        const f32x4 fwh = *reinterpret_cast<const f32x4*>(&Fw[m0 + 8]);
        const f32x4 fbl = *reinterpret_cast<const f32x4*>(&Bs[m0]);
        const f32x4 fbh = *reinterpret_cast<const f32x4*>(&Bs[m0 + 8]);
        const u32x4 aw = u32x4{pack_bf16x2_hw(lo[0] * fwl[0], lo[1] * fwl[1]), pack_bf16x2_hw(lo[2] * fwl[2], lo[3] * fwl[3]),
                               pack_bf16x2_hw(hi[0] * fwh[0], hi[1] * fwh[1]), pack_bf16x2_hw(hi[2] * fwh[2], hi[3] * fwh[3])};
        const u32x4 au = u32x4{pack_bf16x2_hw(lo[0] * fbl[0], lo[1] * fbl[1]), pack_bf16x2_hw(lo[2] * fbl[2], lo[3] * fbl[3]),
                               pack_bf16x2_hw(hi[0] * fbh[0], hi[1] * fbh[1]), pack_bf16x2_hw(hi[2] * fbh[2], hi[3] * fbh[3])};
        const uint2 kl = ld_tr16(&Ks[(16 * kk) * kP + tro + 32 * wave]);
        const uint2 kh = ld_tr16(&Ks[(16 * kk + 8) * kP + tro + 32 * wave]);
        const uint2 vl = ld_tr16(&Vs[(16 * kk) * kP + tro + 32 * wave]);
        const uint2 vh = ld_tr16(&Vs[(16 * kk + 8) * kP + tro + 32 * wave]);
        Wa = mfma32x32x16(aw, u32x4{kl.x, kl.y, kh.x, kh.y}, Wa);
        Ua = mfma32x32x16(au, u32x4{vl.x, vl.y, vh.x, vh.y}, Ua);
      }
      const int cdk = 32 * wave + col;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = 32 * rt + 8 * (r >> 2) + 4 * half + (r & 3);
        Wg[i * kD + perm16(cdk)] = (uint16_t)f32_to_bf16_bits(-Wa[r]);
        Ug[i * kD + cdk] = Ua[r];
      }
    }
  }
}

// ---------------------------------------------------------------- scan ----
// One workgroup per (value head, sequence); wave w carries value rows
// 32w .. 32w+31 of the state, held transposed (S^T, dk x dv) in four
// accumulator tiles: tile mt, value r holds S^T[32mt + 8(r/4) + 4half + r%4][32w + lane%32].
// Per chunk: K, Q, W and M are staged in LDS (double-buffered, the next
// chunk's loads in flight during the current one), U~ comes straight from the
// workspace into the accumulator layout.
struct ScanStage {
  uint16_t K[kC * kP];
  uint16_t Q[kC * kP];
  uint16_t W[kC * kP];
  uint16_t M[kC * kMP];
  float gates[256];
};

__global__ __launch_bounds__(256, 1) void gdn_scan_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const float* __restrict__ S0, int64_t T,
    int Hqk, int Hv, int n_chunks, const uint8_t* __restrict__ ws, uint16_t* __restrict__ out,
    float* __restrict__ S_out) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  ScanStage* st = reinterpret_cast<ScanStage*>(smem);

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int half = lane >> 5, col = lane & 31;
  const int h = blockIdx.x, b = blockIdx.y;
  const int hk = h / (Hv / Hqk);
  const int dv = 32 * wave + col;
  const uint8_t* recs = ws + ((int64_t)b * Hv + h) * n_chunks * kRecBytes;
  const int64_t state_base = ((int64_t)b * Hv + h) * kD * kD;

  f32x16 S[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int dk = 32 * mt + 8 * (r >> 2) + 4 * half + (r & 3);
      S[mt][r] = S0 ? S0[state_base + (int64_t)dv * kD + dk] : 0.0f;
    }
  }

  // staging of one chunk: this thread's share of K, Q (16-byte pieces), W, M,
  // the gates, and this lane's U~ values
  u32x4 RK[4], RQ[4], RW[4], RM[2], RG;
  f32x16 RU[2];
  auto load_chunk = [&](int c) {
    const int64_t t0 = (int64_t)c * kC;
    const int n = (int)min<int64_t>(kC, T - t0);
    const uint8_t* rec = recs + (int64_t)c * kRecBytes;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int idx = tid + 256 * u;
      const int r = idx >> 4, part = idx & 15;
      RK[u] = u32x4{0u, 0u, 0u, 0u};
      if (r < n) RK[u] = ld16(k + (((int64_t)b * T + t0 + r) * Hqk + hk) * kD + 8 * part);
      RW[u] = ld16(rec + kRecW + (int64_t)idx * 16);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      // Q: 32-byte pieces, stored with the middle quads swapped
      const int idx = tid + 256 * u;
      const int r = idx >> 3, pc = idx & 7;
      RQ[2 * u] = u32x4{0u, 0u, 0u, 0u};
      RQ[2 * u + 1] = RQ[2 * u];
      if (r < n) {
        const uint16_t* src = q + (((int64_t)b * T + t0 + r) * Hqk + hk) * kD + 16 * pc;
        RQ[2 * u] = ld16(src);
        RQ[2 * u + 1] = ld16(src + 8);
      }
      RM[u] = ld16(rec + kRecM + (int64_t)idx * 16);
    }
    RG = tid < 64 ? ld16(rec + kRecG + tid * 16) : u32x4{0u, 0u, 0u, 0u};
    const float* ug = reinterpret_cast<const float*>(rec + kRecU);
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = 32 * rt + 8 * (r >> 2) + 4 * half + (r & 3);
        RU[rt][r] = ug[i * kD + dv];
      }
    }
  };
  auto store_chunk = [&](ScanStage& s) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int idx = tid + 256 * u;
      const int r = idx >> 4, part = idx & 15;
      *reinterpret_cast<u32x4*>(&s.K[r * kP + 8 * part]) = RK[u];
      *reinterpret_cast<u32x4*>(&s.W[r * kP + 8 * part]) = RW[u];
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int idx = tid + 256 * u;
      const int r = idx >> 3, pc = idx & 7;
      const u32x4 a = RQ[2 * u], c2 = RQ[2 * u + 1];
      *reinterpret_cast<u32x4*>(&s.Q[r * kP + 16 * pc]) = u32x4{a.x, a.y, c2.x, c2.y};
      *reinterpret_cast<u32x4*>(&s.Q[r * kP + 16 * pc + 8]) = u32x4{a.z, a.w, c2.z, c2.w};
      const int mr = idx >> 3, mp = idx & 7;
      *reinterpret_cast<u32x4*>(&s.M[mr * kMP + 8 * mp]) = RM[u];
    }
    if (tid < 64) *reinterpret_cast<u32x4*>(&s.gates[4 * tid]) = RG;
  };

  const int tro = tr_offset(lane);
  if (n_chunks > 0) {
    load_chunk(0);
    store_chunk(st[0]);
  }
  f32x16 Ucur[2];
  for (int c = 0; c < n_chunks; ++c) {
    const int buf = c & 1;
    Ucur[0] = RU[0];
    Ucur[1] = RU[1];
    __syncthreads();  // buffer `buf` is complete; the other one is no longer read
    if (c + 1 < n_chunks) load_chunk(c + 1);
    const ScanStage& s = st[buf];

    // state as the B operand (k = dk, n = dv), bf16
    u32x4 Sb[8];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        Sb[2 * mt + u] = u32x4{pack_bf16x2_hw(S[mt][8 * u + 0], S[mt][8 * u + 1]),
                               pack_bf16x2_hw(S[mt][8 * u + 2], S[mt][8 * u + 3]),
                               pack_bf16x2_hw(S[mt][8 * u + 4], S[mt][8 * u + 5]),
                               pack_bf16x2_hw(S[mt][8 * u + 6], S[mt][8 * u + 7])};
      }
    }
    // U = U~ - W S^T and O = diag(scale gam) Q S^T (rows: tokens, columns: dv)
    f32x16 U[2], O[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      U[rt] = Ucur[rt];
      O[rt] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const u32x4 aw = *reinterpret_cast<const u32x4*>(&s.W[(32 * rt + col) * kP + 16 * ks + 8 * half]);
        const u32x4 aq = *reinterpret_cast<const u32x4*>(&s.Q[(32 * rt + col) * kP + 16 * ks + 8 * half]);
        U[rt] = mfma32x32x16(aw, Sb[ks], U[rt]);
        O[rt] = mfma32x32x16(aq, Sb[ks], O[rt]);
      }
    }
    // U as the B operand (k = token, n = dv); then its decayed copy for the state
    u32x4 Ub[4], Uh[4];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = 32 * rt + 8 * (r >> 2) + 4 * half + (r & 3);
        O[rt][r] *= s.gates[i];
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        float dec[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int r = 8 * u + j;
          dec[j] = s.gates[64 + 32 * rt + 8 * (r >> 2) + 4 * half + (r & 3)];
        }
        const f32x16& x = U[rt];
        Ub[2 * rt + u] = u32x4{pack_bf16x2_hw(x[8 * u + 0], x[8 * u + 1]), pack_bf16x2_hw(x[8 * u + 2], x[8 * u + 3]),
                               pack_bf16x2_hw(x[8 * u + 4], x[8 * u + 5]), pack_bf16x2_hw(x[8 * u + 6], x[8 * u + 7])};
        Uh[2 * rt + u] = u32x4{pack_bf16x2_hw(x[8 * u + 0] * dec[0], x[8 * u + 1] * dec[1]),
                               pack_bf16x2_hw(x[8 * u + 2] * dec[2], x[8 * u + 3] * dec[3]),
                               pack_bf16x2_hw(x[8 * u + 4] * dec[4], x[8 * u + 5] * dec[5]),
                               pack_bf16x2_hw(x[8 * u + 6] * dec[6], x[8 * u + 7] * dec[7])};
      }
    }
    // O += M U
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const u32x4 am = *reinterpret_cast<const u32x4*>(&s.M[(32 * rt + col) * kMP + 16 * kk + 8 * half]);
        O[rt] = mfma32x32x16(am, Ub[kk], O[rt]);
      }
    }
    // S^T = gam_C S^T + K^T Uh (A = K read transposed: row dk, k = token)
    const float gC = s.gates[128];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) S[mt][r] *= gC;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const uint2 lo = ld_tr16(&s.K[(16 * kk) * kP + tro + 32 * mt]);
        const uint2 hi = ld_tr16(&s.K[(16 * kk + 8) * kP + tro + 32 * mt]);
        S[mt] = mfma32x32x16(u32x4{lo.x, lo.y, hi.x, hi.y}, Uh[kk], S[mt]);
      }
    }
    // outputs of the chunk
    const int64_t t0 = (int64_t)c * kC;
    const int n = (int)min<int64_t>(kC, T - t0);
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = 32 * rt + 8 * (r >> 2) + 4 * half + (r & 3);
        if (i < n) out[(((int64_t)b * T + t0 + i) * Hv + h) * kD + dv] = (uint16_t)f32_to_bf16_bits(O[rt][r]);
      }
    }
    if (c + 1 < n_chunks) store_chunk(st[buf ^ 1]);
  }
  if (S_out) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int dk = 32 * mt + 8 * (r >> 2) + 4 * half + (r & 3);
        S_out[state_base + (int64_t)dv * kD + dk] = S[mt][r];
      }
    }
  }
}

// -------------------------------------------------------------- decode ----
// One workgroup per (value head, sequence); each half-wave updates one state
// row at a time (32 lanes x 4 columns), wave w rows 32w .. 32w+31.
__global__ __launch_bounds__(256) void gdn_decode_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, int Hqk, int Hv, float scale,
    float* __restrict__ state, uint16_t* __restrict__ out) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int half = lane >> 5, col = lane & 31;
  const int h = blockIdx.x, b = blockIdx.y;
  const int hk = h / (Hv / Hqk);
  const uint2 kr = *reinterpret_cast<const uint2*>(k + ((int64_t)b * Hqk + hk) * kD + 4 * col);
  const uint2 qr = *reinterpret_cast<const uint2*>(q + ((int64_t)b * Hqk + hk) * kD + 4 * col);
  const float k4[4] = {bf16_bits_to_f32(kr.x & 0xFFFFu), bf16_bits_to_f32(kr.x >> 16),
                       bf16_bits_to_f32(kr.y & 0xFFFFu), bf16_bits_to_f32(kr.y >> 16)};
  const float q4[4] = {bf16_bits_to_f32(qr.x & 0xFFFFu), bf16_bits_to_f32(qr.x >> 16),
                       bf16_bits_to_f32(qr.y & 0xFFFFu), bf16_bits_to_f32(qr.y >> 16)};
  const float a = expf(g[(int64_t)b * Hv + h]);
  const float bt = beta[(int64_t)b * Hv + h];
  float* srow = state + ((int64_t)b * Hv + h) * kD * kD;
  f32x4 R[16];
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    const int row = 32 * wave + 2 * s + half;
    R[s] = *reinterpret_cast<const f32x4*>(srow + (int64_t)row * kD + 4 * col);
  }
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    const int row = 32 * wave + 2 * s + half;
    float sk = R[s][0] * k4[0] + R[s][1] * k4[1] + R[s][2] * k4[2] + R[s][3] * k4[3];
#pragma unroll
    for (int off = 1; off < 32; off <<= 1) sk += __shfl_xor(sk, off);
    const float e = bf16_bits_to_f32(v[((int64_t)b * Hv + h) * kD + row]) - a * sk;
    const float w = bt * e;
    float sq = 0.0f;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      R[s][x] = a * R[s][x] + w * k4[x];
      sq += R[s][x] * q4[x];
    }
#pragma unroll
    for (int off = 1; off < 32; off <<= 1) sq += __shfl_xor(sq, off);
    *reinterpret_cast<f32x4*>(srow + (int64_t)row * kD + 4 * col) = R[s];
    if (col == 0) out[((int64_t)b * Hv + h) * kD + row] = (uint16_t)f32_to_bf16_bits(scale * sq);
  }
}

}  // namespace

size_t gdn_workspace_bytes(int batch, int64_t T, int Hv) {
  const int64_t n_chunks = (T + kC - 1) / kC;
  return (size_t)batch * Hv * n_chunks * kRecBytes;
}

hipError_t launch_gdn_prefill(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* g,
                              const float* beta, const float* S0, int batch, int64_t T, int Hqk, int Hv,
                              float scale, uint16_t* out, float* S_out, void* ws, hipStream_t stream) {
  const int64_t n_chunks = (T + kC - 1) / kC;
  if (n_chunks > 0)
    hipLaunchKernelGGL(gdn_prep_kernel, dim3((unsigned)n_chunks, Hv, batch), dim3(256), 0, stream, q, k, v, g,
                       beta, T, Hqk, Hv, scale, (int)n_chunks, reinterpret_cast<uint8_t*>(ws));
  const size_t lds = 2 * sizeof(ScanStage);  // 129 KB of the 160 KB
  hipLaunchKernelGGL(gdn_scan_kernel, dim3(Hv, batch), dim3(256), lds, stream, q, k, S0, T, Hqk, Hv,
                     (int)n_chunks, reinterpret_cast<const uint8_t*>(ws), out, S_out);
  return hipGetLastError();
}

hipError_t launch_gdn_decode(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* g,
                             const float* beta, int batch, int Hqk, int Hv, float scale, float* state,
                             uint16_t* out, hipStream_t stream) {
  hipLaunchKernelGGL(gdn_decode_kernel, dim3(Hv, batch), dim3(256), 0, stream, q, k, v, g, beta, Hqk, Hv, scale,
                     state, out);
  return hipGetLastError();
}

}  // namespace qsa
