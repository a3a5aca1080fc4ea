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
// tokens 0..i and gam_i = exp(G_i), the tokens' effective writes
// u_j = b_j (v_j - P_j k_j) (P_j the decayed state just before token j) solve
// the unit lower-triangular system (I + L) U = diag(b) R with
//   L_ij = b_i exp(G_i - G_j) k_i . k_j  (j < i),   R = V - diag(gam) K S^T.
// With Tb = (I + L)^-1 diag(b):  U = Tb R, and
//   O  = diag(scale gam) Q S^T + MT R,     MT = M Tb,
//        M_ij = scale exp(G_i - G_j) q_i . k_j  (j <= i)
//   S' = gam_C S + R^T Kt,                 Kt = Tb^T diag(exp(G_C - G_j)) K.
// Every exponent is a difference G_i - G_j with i >= j (or G itself), so no
// factor exceeds 1. MT, Kt and the gates depend only on the chunk's own
// tokens: gdn_prep_kernel computes them for every chunk in parallel. Then
// gdn_scan_kernel walks the chunks of each (sequence, value head) in order,
// the 128 value rows (independent recurrences) split over workgroups in sets
// of 16: per chunk a set's recurrence wave forms X = K S^T, R = V - gam X and
// the new state (the chain from one state to the next is two products deep)
// and its output wave forms O from the state and R handed over in LDS.
// Decode (one token on a carried state) is gdn_decode_kernel: the recurrence
// itself, one pass over the fp32 state in HBM.
#include <algorithm>
#include <atomic>
#include <cstddef>

#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr int kC = 64;        // tokens per chunk
constexpr int kD = 128;       // key and value head dim
constexpr int kP = kD + 16;   // LDS pitch (elements) of 128-wide bf16 rows
constexpr int kMP = kC + 8;   // LDS pitch of 64-wide bf16 rows
constexpr int kTP = kC + 4;   // LDS pitch of 64-wide fp32 rows (T)
constexpr int kLP = kC + 8;   // LDS pitch of 64-wide fp32 rows (L)

// Workspace record of one (sequence, value head, chunk), byte offsets. It is
// the byte image of the scan's LDS staging of these three arrays (row pitches
// included), so the scan copies it into LDS with direct global-to-LDS loads.
constexpr int64_t kRecK = 0;                     // Kt^T, bf16 [128][kMP]: rows dk in state order,
                                                 // columns tokens in accumulator order
constexpr int64_t kRecM = kRecK + kC * kP * 2;   // MT, bf16 [64][kMP], columns in accumulator order
constexpr int64_t kRecG = kRecM + kC * kMP * 2;  // gates, fp32 [256]: scale gam_i | gam_i | gam_C
constexpr int64_t kRecBytes = kRecG + 256 * 4;   // 28 KB = 7 x 256 threads x 16 B
static_assert(kD * kMP == kC * kP, "Kt^T fills the record's first part");
static_assert(kRecBytes == 7 * 256 * 16, "record copied in 7 rounds of 16 B per thread");

// Operand order of the k dimension. An MFMA 32x32x16 k-step takes, in lane
// half h, the eight k indices {4h .. 4h+3, 8+4h .. 8+4h+3} of its sixteen:
// that is the order in which an accumulator tile holds its rows, so a tile
// (the state, R) feeds the next product without a transpose. A matrix read as
// the other operand of such a product (MT) is stored with the middle two
// quads of every 16 swapped, which puts each lane's eight values in one
// 16-byte run. The map is its own inverse.
__device__ __forceinline__ int perm16(int x) {
  const int qd = (x >> 2) & 3;
  return (qd == 1 || qd == 2) ? x ^ 12 : x;
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

// ds_read_b64_tr_b16: within each 16-lane group, lane l receives element l % 4
// of the 4-element chunk addressed by lane 4j + (l % 16) / 4, in slot j.
__device__ __forceinline__ uint2 ld_tr16(const uint16_t* p) {
  const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p);
  return __builtin_bit_cast(uint2, v);
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

// Accumulator order of 32 indices for the 16x16x32 MFMA: operand slot p (lane
// group p / 8, element p % 8) of a packed pair of 16-row accumulator tiles
// holds accumulator row acc_of_slot(p); slot_of_acc is the inverse.
__device__ __forceinline__ int acc_of_slot(int p) {
  const int g = p >> 3, j = p & 7;
  return j < 4 ? 4 * g + j : 16 + 4 * g + (j - 4);
}
__device__ __forceinline__ int slot_of_acc(int x) {
  return x < 16 ? 8 * (x >> 2) + (x & 3) : 8 * ((x - 16) >> 2) + 4 + (x & 3);
}

// exp(x) for x <= 0 on the hardware exp2 (about 1 ulp; the factors it makes
// are rounded to bf16 or multiply fp32 products).
__device__ __forceinline__ float exp_hw(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }

// ---------------------------------------------------------------- prep ----
// Persistent: each workgroup (4 waves) takes (chunk, value head, sequence)
// items in turn, and loads the next item's K and Q tiles and gates into
// registers while it works on the current one.
__global__ __launch_bounds__(256, 2) void gdn_prep_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const float* __restrict__ g,
    const float* __restrict__ beta, int64_t T, int Hqk, int Hv, float scale, int n_chunks, int64_t n_items,
    uint8_t* __restrict__ ws) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kC * kP];   // K tile, natural order
  __shared__ __attribute__((aligned(16))) uint16_t QTs[kC * kP];  // Q tile, then T (fp32 [64][kTP])
  __shared__ __attribute__((aligned(16))) float Lm[kC * kLP];     // L (fp32), then Tb^T and Td^T (bf16)
  __shared__ __attribute__((aligned(16))) uint16_t Mb[kC * kMP];  // M (bf16, columns permuted)
  __shared__ __attribute__((aligned(16))) float Gs[kC];
  __shared__ __attribute__((aligned(16))) float Bs[kC];
  __shared__ __attribute__((aligned(16))) float Ds[kC];
  __shared__ __attribute__((aligned(16))) float Rg[256];  // the record's gates

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int half = lane >> 5, col = lane & 31;
  float* Tm = reinterpret_cast<float*>(QTs);
  uint16_t* TbT = reinterpret_cast<uint16_t*>(Lm);  // [64 j][kMP], i permuted: T_ij b_j
  uint16_t* TdT = TbT + kC * kMP;                   // same times exp(G_C - G_i)

  // an item's inputs in registers: thread tid holds 16-byte pieces
  // tid + 256 u (row / 16, piece % 16) of the K and Q tiles (key head h / (Hv /
  // Hqk); rows past the sequence are zero), and lane l of wave 0 token l's log
  // decay and write gate (padding 0)
  u32x4 kv[4], qv[4];
  float gx = 0.0f, bt = 0.0f;
  auto fetch = [&](int64_t it) __attribute__((always_inline)) {
    const int c = (int)(it % n_chunks), h = (int)((it / n_chunks) % Hv);
    const int64_t b = it / ((int64_t)n_chunks * Hv);
    const int hk = h / (Hv / Hqk);
    const int64_t t0 = (int64_t)c * kC;
    const int n = (int)min<int64_t>(kC, T - t0);
    gx = 0.0f;
    bt = 0.0f;
    if (wave == 0 && lane < n) {
      gx = g[(b * T + t0 + lane) * Hv + h];
      bt = beta[(b * T + t0 + lane) * Hv + h];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = (tid + 256 * u) >> 4, part = tid & 15;
      kv[u] = u32x4{0u, 0u, 0u, 0u};
      qv[u] = kv[u];
      if (r < n) {
        const int64_t tok = b * T + t0 + r;
        kv[u] = ld16(k + (tok * Hqk + hk) * kD + 8 * part);
        qv[u] = ld16(q + (tok * Hqk + hk) * kD + 8 * part);
      }
    }
  };
  // the tiles go to LDS once the previous item is done with every LDS array
  auto stage = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = (tid + 256 * u) >> 4, part = tid & 15;
      *reinterpret_cast<u32x4*>(&Ks[r * kP + 8 * part]) = kv[u];
      *reinterpret_cast<u32x4*>(&QTs[r * kP + 8 * part]) = qv[u];
    }
  };
  if ((int64_t)blockIdx.x < n_items) {
    fetch(blockIdx.x);
    stage();
  }
  for (int64_t item = blockIdx.x; item < n_items; item += gridDim.x) {
    uint8_t* rec = ws + item * kRecBytes;  // items are numbered as the records
    const bool more = item + gridDim.x < n_items;
    if (wave == 0) {
      // running sum of the log decays over the chunk (padding adds 0)
      float x = gx;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(x, off);
        if (lane >= off) x += y;
      }
      const float gl = __shfl(x, 63);
      const float gam = expf(x);
      Gs[lane] = x;
      Bs[lane] = bt;
      Ds[lane] = expf(gl - x);
      Rg[lane] = scale * gam;
      Rg[64 + lane] = gam;
      Rg[128 + lane] = expf(gl);
      Rg[192 + lane] = 0.0f;
    }
    if (more) fetch(item + gridDim.x);
    __syncthreads();

    // K K^T -> L (fp32) and Q K^T -> M (bf16), tiles of 32 x 32 on or below the diagonal
    if (wave < 3) {
      const int ti = wave == 0 ? 0 : 1, tj = wave == 2 ? 1 : 0;
      f32x16 kk = f32x16{}, qk = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const u32x4 bk = *reinterpret_cast<const u32x4*>(&Ks[(32 * tj + col) * kP + 16 * ks + 8 * half]);
        const u32x4 ak = *reinterpret_cast<const u32x4*>(&Ks[(32 * ti + col) * kP + 16 * ks + 8 * half]);
        const u32x4 aq = *reinterpret_cast<const u32x4*>(&QTs[(32 * ti + col) * kP + 16 * ks + 8 * half]);
        // the products taken transposed (K rows of tile tj as the A operand):
        // lane col then holds row i = 32 ti + col of L and M, and accumulator
        // values 4 qd .. 4 qd + 3 are its columns j = 32 tj + 8 qd + 4 half + 0..3
        kk = mfma32x32x16(bk, ak, kk);
        qk = mfma32x32x16(bk, aq, qk);
      }
      const int i = 32 * ti + col;
      const float gi = Gs[i], bi = Bs[i];
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const int j0 = 32 * tj + 8 * qd + 4 * half;
        const f32x4 gj = *reinterpret_cast<const f32x4*>(&Gs[j0]);
        f32x4 lv;
        float mv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * qd + e, j = j0 + e;
          const float d = exp_hw(gi - gj[e]);  // only used where j <= i, so the exponent is <= 0
          lv[e] = j < i ? bi * d * kk[r] : 0.0f;
          mv[e] = j <= i ? scale * d * qk[r] : 0.0f;
        }
        *reinterpret_cast<f32x4*>(&Lm[i * kLP + j0]) = lv;
        *reinterpret_cast<uint2*>(&Mb[i * kMP + perm16(j0)]) =
            make_uint2(pack_bf16x2_hw(mv[0], mv[1]), pack_bf16x2_hw(mv[2], mv[3]));
      }
    } else {
      // the tile above the diagonal (rows 0..31, columns 32..63) of M is zero
      for (int e = lane; e < 32 * 32; e += 64) Mb[(e >> 5) * kMP + perm16(32 + (e & 31))] = 0;
    }
    __syncthreads();

    // T = (I + L)^-1 in 16 x 16 blocks. The four diagonal blocks by forward
    // substitution in one wave: lane (a, c) = (lane / 16, lane % 16) keeps
    // column c of block a in registers, so each row needs only its row of L
    // (the same for the 16 lanes of a block, read once per row) and no lane
    // exchange; the entries above the diagonal come out as zeros. Four partial
    // sums keep the chain of dependent adds short.
    if (wave == 0) {
      const int a0 = 16 * (lane >> 4), cc = lane & 15;
      float t[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float* lrow = &Lm[(a0 + i) * kLP + a0];
        float part[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int m = 0; m < i; ++m) part[m & 3] += lrow[m] * t[m];
        t[i] = (i == cc ? 1.0f : 0.0f) - ((part[0] + part[1]) + (part[2] + part[3]));
      }
#pragma unroll
      for (int m = 0; m < 16; ++m) Tm[(a0 + m) * kTP + a0 + cc] = t[m];
    }
    __syncthreads();
    // The blocks below the diagonal, column block b by wave b (no exchange
    // between waves: column block b only needs its own blocks and the diagonal
    // ones): T_ab = -T_aa X, X = sum_{m = b .. a-1} L_am T_mb, for a = b+1 .. 3
    // in order, on the fp32 MFMA (16x16x4). The wave keeps its blocks T_mb in
    // accumulator layout (lane l: rows 4 (l/16) + r, column l % 16), which is
    // also the B operand of a product whose k-step s takes, in lane group g,
    // the index 4g + s: the A operand is then row l % 16, columns 4g .. 4g+3 of
    // the left factor, one 16-byte read.
    const int g4 = lane >> 4, n16 = lane & 15;
    f32x4 Tc[4];  // Tc[a] = T_{a, wave}
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      Tc[a] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      if (a == wave) {
#pragma unroll
        for (int r = 0; r < 4; ++r) Tc[a][r] = Tm[(16 * a + 4 * g4 + r) * kTP + 16 * a + n16];
      }
    }
    auto mm16 = [&](const f32x4& arow, const f32x4& bacc, f32x4 c) __attribute__((always_inline)) {
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) c = __builtin_amdgcn_mfma_f32_16x16x4f32(arow[s4], bacc[s4], c, 0, 0, 0);
      return c;
    };
#pragma unroll
    for (int a = 1; a < 4; ++a) {
      if (a > wave) {
        f32x4 x = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int mb = 0; mb < 3; ++mb) {
          if (mb >= wave && mb < a)
            x = mm16(*reinterpret_cast<const f32x4*>(&Lm[(16 * a + n16) * kLP + 16 * mb + 4 * g4]), Tc[mb], x);
        }
        const f32x4 y =
            mm16(*reinterpret_cast<const f32x4*>(&Tm[(16 * a + n16) * kTP + 16 * a + 4 * g4]), x, f32x4{0.0f, 0.0f, 0.0f, 0.0f});
        Tc[a] = -y;
      }
    }
    __syncthreads();  // L is read no more: Tb^T and Td^T take its place
    // Tb = T diag(b) and its copy scaled by the decay to the chunk end, both
    // transposed (rows j, columns i permuted) in bf16, from the registers: lane
    // (g, n) of wave b holds column j = 16b + n, rows 16a + 4g .. +3 of each
    // block (zero above the diagonal blocks); four rows go out as 8 bytes
    // (perm16 keeps a quad together).
    {
      const int j = 16 * wave + n16;
      const float bj = Bs[j];
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int i0 = 16 * a + 4 * g4;
        const f32x4 di = *reinterpret_cast<const f32x4*>(&Ds[i0]);
        const f32x4 t = Tc[a] * bj;
        *reinterpret_cast<uint2*>(&TbT[j * kMP + perm16(i0)]) =
            make_uint2(pack_bf16x2_hw(t[0], t[1]), pack_bf16x2_hw(t[2], t[3]));
        *reinterpret_cast<uint2*>(&TdT[j * kMP + perm16(i0)]) =
            make_uint2(pack_bf16x2_hw(t[0] * di[0], t[1] * di[1]), pack_bf16x2_hw(t[2] * di[2], t[3] * di[3]));
      }
    }
    __syncthreads();

    // MT = M Tb (wave w: tile (w / 2, w % 2), taken transposed so that a lane
    // holds four consecutive columns of a row) and Kt = Td^T K (wave w: dk
    // columns 32w .. 32w+31; a lane holds runs of four tokens of one dk, which
    // go to the record's transposed Kt). The record is assembled in LDS in its
    // workspace layout (Kt^T over the dead T, MT over M once every wave has
    // read M) and written out with coalesced 16-byte stores.
    f32x16 mt = f32x16{};
    {
      const int ti = wave >> 1, tj = wave & 1;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const u32x4 am = *reinterpret_cast<const u32x4*>(&Mb[(32 * ti + col) * kMP + 16 * ks + 8 * half]);
        const u32x4 bt2 = *reinterpret_cast<const u32x4*>(&TbT[(32 * tj + col) * kMP + 16 * ks + 8 * half]);
        mt = mfma32x32x16(bt2, am, mt);
      }
    }
    {
      uint16_t* KtTl = QTs;
      const int p = 32 * wave + acc_of_slot(col);  // state position of dk 32 wave + col
      const int tro = tr_offset(lane);
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        f32x16 acc = f32x16{};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const u32x4 at = *reinterpret_cast<const u32x4*>(&TdT[(32 * rt + col) * kMP + 16 * kk + 8 * half]);
          const uint2 lo = ld_tr16(&Ks[(16 * kk) * kP + tro + 32 * wave]);
          const uint2 hi = ld_tr16(&Ks[(16 * kk + 8) * kP + tro + 32 * wave]);
          acc = mfma32x32x16(at, u32x4{lo.x, lo.y, hi.x, hi.y}, acc);
        }
#pragma unroll
        for (int qd = 0; qd < 4; ++qd)
          *reinterpret_cast<uint2*>(&KtTl[p * kMP + 32 * rt + slot_of_acc(8 * qd + 4 * half)]) = make_uint2(
              pack_bf16x2_hw(acc[4 * qd], acc[4 * qd + 1]), pack_bf16x2_hw(acc[4 * qd + 2], acc[4 * qd + 3]));
      }
    }
    __syncthreads();
    {
      const int ti = wave >> 1, tj = wave & 1;
      const int i = 32 * ti + col;
#pragma unroll
      for (int qd = 0; qd < 4; ++qd)
        *reinterpret_cast<uint2*>(&Mb[i * kMP + 32 * tj + slot_of_acc(8 * qd + 4 * half)]) =
            make_uint2(pack_bf16x2_hw(mt[4 * qd], mt[4 * qd + 1]), pack_bf16x2_hw(mt[4 * qd + 2], mt[4 * qd + 3]));
    }
    __syncthreads();
    static_assert(sizeof(QTs) == kRecM - kRecK && sizeof(Mb) == kRecG - kRecM && sizeof(Rg) == kRecBytes - kRecG,
                  "LDS staging matches the record layout");
#pragma unroll
    for (int u = 0; u < 7; ++u) {
      const int ob = 16 * (tid + 256 * u);
      const uint8_t* src = ob < kRecM   ? reinterpret_cast<const uint8_t*>(QTs) + ob
                           : ob < kRecG ? reinterpret_cast<const uint8_t*>(Mb) + (ob - kRecM)
                                        : reinterpret_cast<const uint8_t*>(Rg) + (ob - kRecG);
      *reinterpret_cast<u32x4*>(rec + ob) = *reinterpret_cast<const u32x4*>(src);
    }
    if (more) {
      __syncthreads();  // every LDS array is free for the next item
      stage();
    }
  }
}

// ---------------------------------------------------------------- scan ----
// Row d of the state only ever meets column d of V and of the outputs, so the
// 128 value rows of a (sequence, value head) are independent recurrences: they
// are split over 8 / W workgroups of W sets of 16 rows, set w of part p being
// rows d0 .. d0+15, d0 = 16 (W p + w). W (1 or 2) is chosen per launch so
// that the grid still covers the chip. Each set has two compute waves: the
// recurrence wave forms X, R and the next state (the chain from one chunk to
// the next), the output wave forms O from the state and R it publishes in
// LDS; separate copy waves fill the chunk stages. The parts of a head (and
// neighbouring heads, which share a key head) are given consecutive
// workgroup slots of one XCD, so the chunk data they all copy is fetched once
// into that XCD's L2.
// A recurrence wave holds its set's rows transposed (S^T, dk x 16) in eight
// 16 x 16 accumulator tiles of the 16x16x32 MFMA. Lane l of such a tile holds rows
// 4(l/16) + r, r = 0..3, of column l % 16; a k-step reads, in lane group
// g = l/16, the eight k indices 8g .. 8g+7. Packing two row-adjacent tiles
// into an operand therefore gives lane group g rows {4g .. 4g+3, 16+4g ..
// 16+4g+3}: the "accumulator order" of each 32 indices (acc_of_slot /
// slot_of_acc above). State row position q holds dk = slot_of_acc(q), so the
// packed state meets K and Q in their natural dk order; the record holds Kt
// transposed (rows dk in state order) and MT, both with their token columns
// in accumulator order, so the state update and MT R read plain 16-byte
// rows, as prep writes them.
// Per chunk, everything the chunk reads is copied straight from memory into
// LDS (global-to-LDS loads: 16 bytes per lane, written at consecutive
// addresses from the wave's base), double-buffered so the next chunk's copies
// are in flight during the current one. K and Q rows (256 bytes) keep their
// sixteen 16-byte pieces at piece ^ (row % 16), V rows (the staged columns)
// at piece ^ (row % pieces per row), so a piece of 16 consecutive rows
// spreads over the banks; the record (Kt^T, MT, gates) is copied as the image
// prep wrote.
template <int W>
struct ScanStage {
  // V columns staged: the part's own, and at least the 32-column block that
  // holds them (one k-step of the MFMA that adds V)
  static_assert(W == 1 || W == 2, "one or two row sets per workgroup");
  static constexpr int kVC = 32;
  uint16_t K[kC * kD];
  uint16_t Q[kC * kD];
  uint16_t V[kC * kVC];
  uint16_t KtT[kD * kMP];  // Kt^T, MT and gates: the workspace record image
  uint16_t MT[kC * kMP];
  float gates[256];
  uint32_t sink[64];  // written by the L2 prefetches, never read
};

__device__ __forceinline__ f32x4 mfma16(const u32x4& a, const u32x4& b, const f32x4& c) {
  return mfma16x16x32(a, b, c);
}

// Byte offset of 16-byte piece p of row i in a swizzled tile of 256-byte rows.
__device__ __forceinline__ int swz16(int i, int p) { return i * 256 + (((p ^ i) & 15) << 4); }

// Word 3 of a raw buffer resource (32-bit data format, no swizzle).
constexpr int kBufferFlags = 0x00020000;

// s_waitcnt immediate that waits until at most n (< 64) vector memory
// operations are outstanding and does not wait on the other counters.
constexpr int vmcnt_wait(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }
// s_waitcnt immediate that waits for every LDS operation of the wave and
// does not wait on the other counters.
constexpr int kLgkmWait0 = 15 | (7 << 4) | (0 << 8) | (3 << 14);

__device__ __forceinline__ u32x4 pack_tiles(const f32x4& a, const f32x4& b) {
  return u32x4{pack_bf16x2_hw(a[0], a[1]), pack_bf16x2_hw(a[2], a[3]), pack_bf16x2_hw(b[0], b[1]),
               pack_bf16x2_hw(b[2], b[3])};
}

template <int W, int NC>
__global__ __launch_bounds__(64 * (2 * W + NC), 1) void gdn_scan_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ S0, int64_t T, int Hqk, int Hv, int n_chunks, const uint8_t* __restrict__ ws,
    uint16_t* __restrict__ out, float* __restrict__ S_out) {
  using Stage = ScanStage<W>;
  constexpr int kVC = Stage::kVC, kVB = 2 * kVC, kVP = kVB / 16;  // V row bytes, 16-byte pieces per row
  constexpr int kParts = 8 / W;
  static_assert(offsetof(Stage, MT) - offsetof(Stage, KtT) == kRecM - kRecK &&
                    offsetof(Stage, gates) - offsetof(Stage, KtT) == kRecG - kRecK,
                "stage holds the record image");
  // the two chunk stages, each named statically by the chunk loops (unrolled
  // by two)
  __shared__ __attribute__((aligned(16))) Stage st0;
  __shared__ __attribute__((aligned(16))) Stage st1;
  // handed from a set's recurrence wave to its output wave: the packed state
  // entering a chunk (two chunks' worth, by parity) and the chunk's packed R,
  // as the lanes hold them
  __shared__ __attribute__((aligned(16))) u32x4 sx[W][2][4][64];
  __shared__ __attribute__((aligned(16))) u32x4 rx[W][2][64];
  __shared__ int r_ready[W];  // chunks whose R has been handed over, per set

  const int tid = threadIdx.x;
  // the wave index as a scalar: copy, recurrence and output waves take
  // different paths, each wave as a whole (their barriers pair up one per chunk)
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  // workgroups are dealt to the eight XCDs in turn: slot L / 8 of XCD L % 8
  // takes work item (L % 8) (n / 8) + L / 8
  const int n_wg = (int)gridDim.x, L = (int)blockIdx.x;
  const int item = n_wg % 8 == 0 ? (L % 8) * (n_wg / 8) + L / 8 : L;
  const int part = item % kParts, h = (item / kParts) % Hv, b = item / (kParts * Hv);
  const int hk = h / (Hv / Hqk);
  const int vbase = kVC * ((16 * W * part) / kVC);  // first staged V column
  const uint8_t* recs = ws + ((int64_t)b * Hv + h) * n_chunks * kRecBytes;
  const int64_t kq_row = (int64_t)Hqk * kD, v_row = (int64_t)Hv * kD;

  if (wave >= 2 * W) {
    // ---- the copy waves. Copy u of copy wave w fills 1 KB at byte 1024 x,
    // x = NC u + w, of its array: K/Q rows 4x + lane / 16 (stored piece
    // lane % 16), V rows x (1024 / kVB) + lane / kVP (stored piece lane % kVP),
    // record bytes 1024 x + 16 lane; rows past the end of the sequence repeat
    // its last row.
    const int cw = wave - 2 * W;
    const uint16_t* kb = k + ((int64_t)b * T * Hqk + hk) * kD;
    const uint16_t* qb = q + ((int64_t)b * T * Hqk + hk) * kD;
    const uint16_t* vb = v + ((int64_t)b * T * Hv + h) * kD + vbase;
    auto load_chunk = [&](int c, Stage& dst) __attribute__((always_inline)) {
      const int64_t t0 = (int64_t)c * kC;
      const int n = (int)min<int64_t>(kC, T - t0);
      const uint8_t* rec = recs + (int64_t)c * kRecBytes;
      uint8_t* img = reinterpret_cast<uint8_t*>(dst.KtT);
#pragma unroll
      for (int u = 0; u < 28 / NC; ++u) {
        const int x = NC * u + cw;
        __builtin_amdgcn_global_load_lds((glb_void*)(rec + 1024 * x + 16 * lane), (lds_void*)(img + 1024 * x), 16, 0,
                                         0);
      }
#pragma unroll
      for (int u = 0; u < 16 / NC; ++u) {
        const int x = NC * u + cw;
        const int row = 4 * x + (lane >> 4);
        const int64_t src = (t0 + min(row, n - 1)) * kq_row + 8 * ((lane & 15) ^ (row & 15));
        __builtin_amdgcn_global_load_lds((glb_void*)(kb + src),
                                         (lds_void*)(reinterpret_cast<uint8_t*>(dst.K) + 1024 * x), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((glb_void*)(qb + src),
                                         (lds_void*)(reinterpret_cast<uint8_t*>(dst.Q) + 1024 * x), 16, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < kC * kVB / 1024 / NC; ++u) {
        const int x = NC * u + cw;
        const int row = x * (1024 / kVB) + lane / kVP;
        const int64_t src = (t0 + min(row, n - 1)) * v_row + 8 * ((lane % kVP) ^ (row % kVP));
        __builtin_amdgcn_global_load_lds((glb_void*)(vb + src),
                                         (lds_void*)(reinterpret_cast<uint8_t*>(dst.V) + 1024 * x), 16, 0, 0);
      }
    };
    // L2 prefetch two chunks ahead, shared out over the head's workgroups:
    // the 128-byte lines they will all copy (the record, whole V rows, K and
    // Q rows) are dealt round the copy waves of the head's parts, and each
    // wave touches one word of each of its lines (a stage's sink takes them).
    // The copies then find the chunk in L2 instead of all missing together.
    constexpr int kRecLines = (int)(kRecBytes / 128);
    constexpr int kLines = kRecLines + 2 * kC + 4 * kC;
    constexpr int kSlices = kParts * NC;
    constexpr int kPf = (kLines + 64 * kSlices - 1) / (64 * kSlices);  // prefetch loads per copy wave
    const uint16_t* vrow = v + ((int64_t)b * T * Hv + h) * kD;
    const int slice = part * NC + cw;
    auto prefetch_chunk = [&](int c, Stage& sink) __attribute__((always_inline)) {
      const int64_t t0 = (int64_t)c * kC;
      const int n = (int)min<int64_t>(kC, T - t0);
      const uint8_t* rec = recs + (int64_t)c * kRecBytes;
#pragma unroll
      for (int i = 0; i < kPf; ++i) {
        int x = slice + kSlices * (lane + 64 * i);
        if (x >= kLines) x = slice;  // a line this wave touches anyway
        const void* src;
        if (x < kRecLines) {
          src = rec + 128 * x;
        } else if (x < kRecLines + 2 * kC) {
          const int y = x - kRecLines;
          src = vrow + (t0 + min(y >> 1, n - 1)) * v_row + 64 * (y & 1);
        } else {
          const int y = x - kRecLines - 2 * kC;
          const int row = min((y & (2 * kC - 1)) >> 1, n - 1);
          src = (y < 2 * kC ? kb : qb) + (t0 + row) * kq_row + 64 * (y & 1);
        }
        __builtin_amdgcn_global_load_lds((glb_void*)src, (lds_void*)sink.sink, 4, 0, 0);
      }
    };
    // Vector memory operations complete in issue order: once at most the kPf
    // prefetches issued after this wave's copies of a chunk are outstanding,
    // the copies are in LDS, and the barrier hands them to the compute waves
    // (which by then have finished with the stage the next copies overwrite).
    auto copy_step = [&](int c, Stage& nxt) __attribute__((always_inline)) {
      __builtin_amdgcn_s_waitcnt(vmcnt_wait(kPf));
      __builtin_amdgcn_s_barrier();
      if (c + 1 < n_chunks) {
        load_chunk(c + 1, nxt);
        prefetch_chunk(min(c + 2, n_chunks - 1), nxt);
      }
    };
    if (n_chunks > 0) {
      load_chunk(0, st0);
      prefetch_chunk(min(1, n_chunks - 1), st0);
    }
    for (int c = 0; c < n_chunks; c += 2) {
      copy_step(c, st1);
      if (c + 1 < n_chunks) copy_step(c + 1, st0);
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));  // no copy into LDS outlives the workgroup
    return;
  }

  // ---- the compute waves: set `set`, recurrence (waves 0 .. W-1) or output
  // (waves W .. 2W-1); one barrier per chunk, as the copy waves. Within a
  // chunk the recurrence wave hands R to the output wave through r_ready.
  const bool recur = wave < W;
  const int set = recur ? wave : wave - W;
  const int grp = lane >> 4, cl = lane & 15;
  const int d0 = 16 * (W * part + set);  // this set's value rows
  const int dv = d0 + cl;                // this lane's
  const int64_t state_base = ((int64_t)b * Hv + h) * kD * kD;
  // (the barrier does not wait for this wave's LDS writes by itself: the
  // handed-over state and R must have landed before the other wave reads them)
  auto barrier = [&]() __attribute__((always_inline)) {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(kLgkmWait0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  if (recur) {
    // S^T tile mt, value r: state position 16mt + 4grp + r
    f32x4 S[8];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int pos = 16 * mt + 4 * grp + r;
        S[mt][r] = S0 ? S0[state_base + (int64_t)dv * kD + 32 * (pos >> 5) + slot_of_acc(pos & 31)] : 0.0f;
      }
    }
    // B operand of the identity: adds V (this set's 16 columns of a 32-column block) to an accumulator
    u32x4 ident;
    {
      const int off = 16 * ((d0 >> 4) & 1);
      uint32_t w[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const uint32_t lo = (8 * grp + 2 * x == off + cl) ? 0x3F80u : 0u;
        const uint32_t hi = (8 * grp + 2 * x + 1 == off + cl) ? 0x3F80u : 0u;
        w[x] = lo | (hi << 16);
      }
      ident = u32x4{w[0], w[1], w[2], w[3]};
    }
    const int vpiece = grp;  // the set's A-operand piece of a (32-column) V row
    // the state as the B operand (k = dk in natural order, n = dv), also
    // handed to the output wave
    u32x4 Sb[4];
    auto pack_state = [&](int parity) __attribute__((always_inline)) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        Sb[ks] = pack_tiles(S[2 * ks], S[2 * ks + 1]);
        sx[set][parity][ks][lane] = Sb[ks];
      }
    };
    pack_state(0);
    r_ready[set] = 0;
    auto step = [&](int c, const Stage& s, int parity) __attribute__((always_inline)) {
      barrier();  // the chunk is in `s`
      const uint8_t* sK = reinterpret_cast<const uint8_t*>(s.K);
      const uint8_t* sV = reinterpret_cast<const uint8_t*>(s.V);
      // X = K S^T and V, tiles of 16 tokens
      f32x4 X[4], R[4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const int row = 16 * rt + cl;
        X[rt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        R[rt] = mfma16(*reinterpret_cast<const u32x4*>(sV + row * kVB + (((vpiece ^ row) & (kVP - 1)) << 4)), ident,
                       X[rt]);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          X[rt] = mfma16(*reinterpret_cast<const u32x4*>(sK + swz16(row, 4 * ks + grp)), Sb[ks], X[rt]);
      }
      // R = V - diag(gam) X as the B operand (k = token in accumulator order)
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const f32x4 gm = *reinterpret_cast<const f32x4*>(&s.gates[64 + 16 * rt + 4 * grp]);
#pragma unroll
        for (int r = 0; r < 4; ++r) R[rt][r] -= gm[r] * X[rt][r];
      }
      u32x4 Rb[2];
      Rb[0] = pack_tiles(R[0], R[1]);
      Rb[1] = pack_tiles(R[2], R[3]);
      rx[set][0][lane] = Rb[0];
      rx[set][1][lane] = Rb[1];
      // R has landed before the flag says so (LDS operations of a wave are
      // waited for in order)
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(kLgkmWait0);
      __hip_atomic_store(&r_ready[set], c + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      // S^T = gam_C S^T + Kt^T R
      const float gC = s.gates[128];
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) S[mt][r] *= gC;
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
          S[mt] = mfma16(*reinterpret_cast<const u32x4*>(&s.KtT[(16 * mt + cl) * kMP + 32 * kk + 8 * grp]), Rb[kk],
                         S[mt]);
        }
      }
      pack_state(parity ^ 1);  // the state entering the next chunk
    };
    for (int c = 0; c < n_chunks; c += 2) {
      step(c, st0, 0);
      if (c + 1 < n_chunks) step(c + 1, st1, 1);
    }
    if (S_out) {
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int pos = 16 * mt + 4 * grp + r;
          S_out[state_base + (int64_t)dv * kD + 32 * (pos >> 5) + slot_of_acc(pos & 31)] = S[mt][r];
        }
      }
    }
    return;
  }

  // the output wave: O^T = S Q^T diag(scale gam) + R^T MT^T (the packed state
  // and R as the A operands, the Q and MT fragments as the B operands), so
  // lane l holds value columns d0 + 4 (l / 16) .. +3 of token l % 16 of each
  // 16-token tile, stored as 8 bytes; buffer stores whose range ends at the
  // chunk's last token drop the rest
  uint16_t* out_base = out + ((int64_t)b * T * Hv + h) * kD + d0;
  const int row_bytes = (int)(v_row * 2);
  auto step = [&](int c, const Stage& s, int parity) __attribute__((always_inline)) {
    barrier();  // the chunk is in `s`, its entering state in sx[set][parity]
    const uint8_t* sQ = reinterpret_cast<const uint8_t*>(s.Q);
    u32x4 Sb[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) Sb[ks] = sx[set][parity][ks][lane];
    f32x4 O[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const int row = 16 * rt + cl;
      O[rt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        O[rt] = mfma16(Sb[ks], *reinterpret_cast<const u32x4*>(sQ + swz16(row, 4 * ks + grp)), O[rt]);
      const float sg = s.gates[16 * rt + cl];
#pragma unroll
      for (int r = 0; r < 4; ++r) O[rt][r] *= sg;
    }
    // wait for the chunk's R (the recurrence wave always gets there; the
    // bound only keeps a fault from turning into a hang, and if it ever ran
    // out the chunk's output is stored as NaN rather than from a stale R)
    bool handed = false;
    for (int spin = 0; spin < (1 << 24); ++spin) {
      if (__hip_atomic_load(&r_ready[set], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) > c) {
        handed = true;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    asm volatile("" ::: "memory");
    const u32x4 Rb0 = rx[set][0][lane], Rb1 = rx[set][1][lane];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      O[rt] = mfma16(Rb0, *reinterpret_cast<const u32x4*>(&s.MT[(16 * rt + cl) * kMP + 8 * grp]), O[rt]);
      O[rt] = mfma16(Rb1, *reinterpret_cast<const u32x4*>(&s.MT[(16 * rt + cl) * kMP + 32 + 8 * grp]), O[rt]);
    }
    if (!handed) {
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) O[rt] = f32x4{NAN, NAN, NAN, NAN};
    }
    const int64_t t0 = (int64_t)c * kC;
    const int n = (int)min<int64_t>(kC, T - t0);
    const __amdgpu_buffer_rsrc_t dst =
        __builtin_amdgcn_make_buffer_rsrc(out_base + t0 * v_row, 0, (n - 1) * row_bytes + 32, kBufferFlags);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const u32x2 val = u32x2{pack_bf16x2_hw(O[rt][0], O[rt][1]), pack_bf16x2_hw(O[rt][2], O[rt][3])};
      __builtin_amdgcn_raw_buffer_store_b64(val, dst, (16 * rt + cl) * row_bytes + 8 * grp, 0, 0);
    }
  };
  for (int c = 0; c < n_chunks; c += 2) {
    step(c, st0, 0);
    if (c + 1 < n_chunks) step(c + 1, st1, 1);
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
  // the state is read once per step: non-temporal loads (measured faster when
  // the caches hold other dirty data, as after a prefill; no slower otherwise)
  f32x4 R[16];
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    const int row = 32 * wave + 2 * s + half;
    R[s] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(srow + (int64_t)row * kD + 4 * col));
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

// Compute units of the current device (cached per device).
static int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

size_t gdn_workspace_bytes(int batch, int64_t T, int Hv) {
  const int64_t n_chunks = (T + kC - 1) / kC;
  return (size_t)batch * Hv * n_chunks * kRecBytes;
}

hipError_t launch_gdn_prefill(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* g,
                              const float* beta, const float* S0, int batch, int64_t T, int Hqk, int Hv,
                              float scale, uint16_t* out, float* S_out, void* ws, hipStream_t stream) {
  const int64_t n_chunks = (T + kC - 1) / kC;
  if (n_chunks > 0) {
    const int64_t n_items = (int64_t)batch * Hv * n_chunks;  // (sequence, value head, chunk), chunk fastest
    const unsigned grid = (unsigned)std::min<int64_t>(n_items, 2 * (int64_t)device_cu_count());
    hipLaunchKernelGGL(gdn_prep_kernel, dim3(grid), dim3(256), 0, stream, q, k, g, beta, T, Hqk, Hv, scale,
                       (int)n_chunks, n_items, reinterpret_cast<uint8_t*>(ws));
  }
  // row sets per scan workgroup: two once that still gives every CU a workgroup
  const int64_t rows_sets = (int64_t)batch * Hv;  // (sequence, value head) pairs
  const int W = rows_sets * 4 >= device_cu_count() ? 2 : 1;
  const unsigned n_wg = (unsigned)(rows_sets * (8 / W));
  const uint8_t* wsb = reinterpret_cast<const uint8_t*>(ws);
  // copy waves: four beside one row set, two beside two
  if (W == 2)
    hipLaunchKernelGGL((gdn_scan_kernel<2, 2>), dim3(n_wg), dim3(64 * (4 + 2)), 0, stream, q, k, v, S0, T, Hqk, Hv,
                       (int)n_chunks, wsb, out, S_out);
  else
    hipLaunchKernelGGL((gdn_scan_kernel<1, 4>), dim3(n_wg), dim3(64 * (2 + 4)), 0, stream, q, k, v, S0, T, Hqk, Hv,
                       (int)n_chunks, wsb, out, S_out);
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
