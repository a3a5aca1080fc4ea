// Sparse attention over the kept micro-blocks, prefill and decode.
//
// Method (news page "Qwen3.8-Flash发布并开源…", section 2 item 1; explainer page
// "用125亿分之6的参数…", sparse-attention section): the kept blocks are expanded
// back to their tokens and exact, full-precision softmax attention runs over
// those tokens only. Query t attends to every s = j*r + m (m < r) of every
// kept block j with s <= t (only its own block is cut by the causal mask).
//
// Work layout. One workgroup (4 waves) serves one query row and one split of
// its token list. Each wave owns one KV head g (grouped-query attention: the
// G = Hq / Hkv query heads of g share its K and V rows), and, when Hkv < 4,
// every (4 / Hkv)-th chunk of 32 tokens. Per chunk:
//   S^T = K Q^T   on v_mfma_f32_16x16x32_bf16: K rows gathered straight from
//                 HBM into the A operand (16 B per lane, token-contiguous),
//                 Q^T (the G heads, padded to 16) held in the B operand;
//   online softmax in fp32 (base-2 exponent, scale folded in), per head;
//   O += P V      on the same MFMA: P comes out of the S^T accumulators already
//                 in A-operand layout (token order inside the chunk is permuted
//                 consistently for P and V), V goes HBM -> registers -> LDS and
//                 is read back transposed, 2 bytes per lane.
// The next chunk's K and V loads are issued as soon as the current chunk's
// K has gone through its MFMAs and its V into LDS, and are in flight during
// its softmax and P V. The kernel is bound by the HBM gather of K/V rows:
// each block of r tokens is r * Hkv * D * 2 bytes contiguous in K and in V.
//
// Decode splits the token list over many workgroups (split-KV) and a second
// kernel merges the partial (m, l, O) per head. Dense decode attention (the
// comparator) is the same kernel with the token list 0..t; dense prefill has
// its own kernel.
#include "qsa_device.h"
#include "qsa_internal.h"

#include <algorithm>

namespace qsa {

namespace {
constexpr int kD = 128;        // head dim
constexpr int kChunk = 32;     // tokens per chunk
constexpr int kVPitch = 132;   // LDS row pitch of the V tile (elements)
constexpr int kSelLds = 1024;  // kept block ids per split staged in LDS (top_k <= 1024)
}  // namespace

// Two waves per SIMD: with one chunk's K and V registers (loaded into once
// the previous chunk's are consumed) the kernel fits 256 registers, and the
// second wave hides each wave's wait for its next chunk.
template <int HKV>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void attn_gather_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, int64_t kv_batch_stride, int64_t q_pos0,
    const int32_t* __restrict__ kv_len, int Hq, int G, int r, int k,
    const int32_t* __restrict__ sel, const int32_t* __restrict__ sel_cnt, int n_splits,
    int split_tokens, float scale_log2, uint16_t* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ part_o, float2* __restrict__ part_ml, PagedRows pg) {
  constexpr int WPH = 4 / HKV;  // waves per KV head
  __shared__ uint16_t vtile[4][kChunk * kVPitch];
  __shared__ float xm[4][16], xl[4][16];
  __shared__ int32_t sblk[kSelLds];
  __shared__ int32_t sphys[kSelLds];  // paged: physical token of each kept block's first token

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int l16 = lane & 15;
  const int quad = lane >> 4;
  const int g = wave % HKV;
  const int sub = wave / HKV;
  const int64_t row = blockIdx.x;
  const int split = blockIdx.y;

  int64_t t;
  int seq = 0;
  if (pg.cu_q) {
    // packed rows: the sequence is the last b with cu_q[b] <= row
    int lo = 0, hi = pg.n_seq - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pg.cu_q[mid] <= row) lo = mid;
      else hi = mid - 1;
    }
    seq = lo;
    t = (int64_t)pg.q_pos[seq] + (row - pg.cu_q[seq]);
  } else {
    t = kv_len ? (int64_t)kv_len[row] - 1 : q_pos0 + row;
  }
  // paged K/V: token s of the sequence lives at page_table[s >> lps] << lps | s % page
  const int32_t* ptab = pg.page_table ? pg.page_table + (int64_t)seq * pg.max_pages : nullptr;
  auto phys = [&](int64_t s) -> int64_t {
    return ptab ? ((int64_t)ptab[s >> pg.lps] << pg.lps) + (s & ((1 << pg.lps) - 1)) : s;
  };
  const int64_t t_phys = phys(t);
  const uint16_t* kb = kc + (kv_len ? row * kv_batch_stride : 0);
  const uint16_t* vb = vc + (kv_len ? row * kv_batch_stride : 0);
  const int64_t n_tok = sel ? (int64_t)sel_cnt[row] * r : t + 1;
  const int64_t p_beg = (int64_t)split * split_tokens;
  const int64_t p_end = min(n_tok, p_beg + split_tokens);
  const int32_t* srow = sel ? sel + row * k : nullptr;

  // Q^T as the B operand: lane holds head l16 (zero past G), dims 32ks + 8quad.
  u32x4 Qf[4];
  {
    const uint16_t* qp = q + row * (int64_t)Hq * kD + (int64_t)(g * G + l16) * kD + 8 * quad;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) Qf[ks] = l16 < G ? ld16(qp + 32 * ks) : u32x4{0u, 0u, 0u, 0u};
  }

  // This split's kept block ids, staged in LDS once: the token gathers then
  // never wait on a global load of the selection.
  const int lr = __builtin_ctz((unsigned)r);  // r is a power of two
  const int jb0 = (int)(p_beg >> lr);
  if (srow) {
    const int jb1 = p_end > p_beg ? (int)((p_end - 1) >> lr) + 1 : jb0;
    const int nb = min(jb1 - jb0, kSelLds);
    for (int i = threadIdx.x; i < nb; i += 256) {
      const int j = srow[jb0 + i];
      sblk[i] = j;
      if (ptab) sphys[i] = (int32_t)phys((int64_t)j << lr);  // a block never straddles a page
    }
  }
  __syncthreads();

  // Storage row (token index into K/V) of list position p, and whether it is
  // attended; positions that are not attended point at a row that exists.
  auto token_of = [&](int64_t p, bool& valid) -> int64_t {
    int64_t s;
    if (p >= p_end) {
      valid = false;
      return t_phys;
    }
    if (srow) {
      const int i = (int)(p >> lr) - jb0;
      const int m = (int)(p & (r - 1));
      s = ((int64_t)sblk[i] << lr) + m;
      valid = s <= t;
      if (ptab) return (int64_t)sphys[i] + (valid ? m : 0);
    } else {
      s = p;
      valid = s <= t;
    }
    return valid ? s : t;
  };

  // Chunk loader: K fragments (rows 16mt + l16) and V rows (4x + quad).
  u32x4 Kn[2][4], Vn[8];
  uint32_t vmask_n = 0;
  auto load_chunk = [&](int64_t c) {
    bool valid;
    const int64_t s_mine = token_of(c + (lane & 31), valid);
    const uint64_t vm = ballot(valid);
    vmask_n = (uint32_t)vm;
    const int s_lo = (int)s_mine;  // positions fit in 31 bits
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int64_t s = __shfl(s_lo, 16 * mt + l16);
      const uint16_t* kp = kb + (s * HKV + g) * kD + 8 * quad;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) Kn[mt][ks] = ld16(kp + 32 * ks);
    }
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      const int64_t s = __shfl(s_lo, 4 * x + quad);
      Vn[x] = ld16(vb + (s * HKV + g) * kD + 8 * l16);
    }
  };

  float m_run = -INFINITY;  // running max (log2 units) of head l16
  float l_run = 0.0f;       // this lane's share of the running sum of head l16
  f32x4 O[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) O[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  uint16_t* vt = vtile[wave];

  int64_t c = p_beg + (int64_t)sub * kChunk;
  if (c < p_end) load_chunk(c);
  for (; c < p_end; c += (int64_t)WPH * kChunk) {
    const uint32_t vmask = vmask_n;
    // S^T for the 32 tokens of the chunk
    f32x4 S[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      S[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) S[mt] = mfma16x16x32(Kn[mt][ks], Qf[ks], S[mt]);
    }
    // stage V rows in LDS
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      uint16_t* dst = vt + (4 * x + quad) * kVPitch + 8 * l16;
      *reinterpret_cast<uint2*>(dst) = make_uint2(Vn[x][0], Vn[x][1]);
      *reinterpret_cast<uint2*>(dst + 4) = make_uint2(Vn[x][2], Vn[x][3]);
    }
    // this chunk's K and V are consumed: their registers take the next
    // chunk's loads, in flight during the softmax and P V below
    const int64_t cn = c + (int64_t)WPH * kChunk;
    if (cn < p_end) load_chunk(cn);
    // online softmax (rows of S^T are tokens 16mt + 4quad + i, column = head l16)
    float x[8];
    float cmax = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rho = 16 * mt + 4 * quad + i;
        const float v = ((vmask >> rho) & 1u) ? S[mt][i] * scale_log2 : -INFINITY;
        x[4 * mt + i] = v;
        cmax = fmaxf(cmax, v);
      }
    cmax = fmaxf(cmax, __shfl_xor(cmax, 16));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
    const float m_new = fmaxf(m_run, cmax);
    const float m_use = m_new == -INFINITY ? 0.0f : m_new;
    const float alpha = exp2f(m_run - m_use);
    float psum = 0.0f;
    float p[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p[e] = fast_exp2(x[e] - m_use);
      psum += p[e];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    // rescale O rows (heads 4quad + i) by their head's alpha
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = __shfl(alpha, 4 * quad + i);
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) O[nt][i] *= a;
    }
    const u32x4 Pf = u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                           pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    // V^T fragments: k index 8quad + e <-> token row (e < 4 ? 4quad + e : 12 + 4quad + e)
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const int dcol = 16 * nt + l16;
      uint32_t w[4];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const int e0 = 2 * e2, e1 = 2 * e2 + 1;
        const int r0 = e0 < 4 ? 4 * quad + e0 : 12 + 4 * quad + e0;
        const int r1 = e1 < 4 ? 4 * quad + e1 : 12 + 4 * quad + e1;
        w[e2] = (uint32_t)vt[r0 * kVPitch + dcol] | ((uint32_t)vt[r1 * kVPitch + dcol] << 16);
      }
      O[nt] = mfma16x16x32(Pf, u32x4{w[0], w[1], w[2], w[3]}, O[nt]);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
  }

  // per-head sum over the 4 lanes sharing head l16
  float l_head = l_run + __shfl_xor(l_run, 16);
  l_head += __shfl_xor(l_head, 32);

  if (WPH > 1) {
    // merge the waves that share KV head g: (m, l) through LDS, O through LDS
    __shared__ float xo[4][16][kD];
    if (lane < 16) {
      xm[wave][lane] = m_run;
      xl[wave][lane] = l_head;
    }
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) xo[wave][4 * quad + i][16 * nt + l16] = O[nt][i];
    __syncthreads();
    if (sub == 0) {
      // combined max and sum for head l16
      float M = -INFINITY;
      for (int u = 0; u < WPH; ++u) M = fmaxf(M, xm[g + HKV * u][l16]);
      const float Mu = M == -INFINITY ? 0.0f : M;
      float L = 0.0f;
      for (int u = 0; u < WPH; ++u) L += xl[g + HKV * u][l16] * exp2f(xm[g + HKV * u][l16] - Mu);
      m_run = M;
      l_head = L;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = 4 * quad + i;
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
          float acc = 0.0f;
          for (int u = 0; u < WPH; ++u) {
            const int wv = g + HKV * u;
            const float Mh = __shfl(Mu, h);  // same for every u; hoisted by the compiler
            acc += xo[wv][h][16 * nt + l16] * exp2f(xm[wv][h] - Mh);
          }
          O[nt][i] = acc;
        }
      }
    }
    if (sub != 0) return;
  }

  if (n_splits == 1) {
    // final: o = O / l in bf16, lse = (m + log2 l) * ln 2
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * quad + i;
      const float lh = __shfl(l_head, h);
      const float inv = 1.0f / lh;
      if (h < G) {
        uint16_t* op = out + row * (int64_t)Hq * kD + (int64_t)(g * G + h) * kD;
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) op[16 * nt + l16] = (uint16_t)f32_to_bf16_bits(O[nt][i] * inv);
      }
    }
    if (lse && lane < G) lse[row * Hq + g * G + lane] = (m_run + log2f(l_head)) * 0.69314718055994531f;
  } else {
    const int64_t base = (row * n_splits + split) * (int64_t)Hq;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * quad + i;
      if (h < G) {
        float* op = part_o + (base + g * G + h) * kD;
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) op[16 * nt + l16] = O[nt][i];
      }
    }
    if (lane < G) part_ml[base + g * G + lane] = make_float2(m_run, l_head);
  }
}

// Merge split-KV partials: one workgroup (128 threads = head dim) per (row,
// head). The per-split (m, l) pairs are read in parallel into LDS, reduced,
// and turned into weights; each thread then sums its dimension over the
// splits with independent loads.
constexpr int kMaxMergeSplits = 1024;
constexpr int kMergeBatch = 64;  // partial outputs a merge thread has in flight

__global__ __launch_bounds__(128) void attn_merge_kernel(const float* __restrict__ part_o,
                                                         const float2* __restrict__ part_ml,
                                                         int n_splits, int Hq,
                                                         uint16_t* __restrict__ out,
                                                         float* __restrict__ lse) {
  __shared__ float wsplit[kMaxMergeSplits];
  __shared__ float red[2][2];
  const int64_t row = blockIdx.x;
  const int h = blockIdx.y;
  const int d = threadIdx.x;
  const int64_t base = row * n_splits * (int64_t)Hq + h;  // index of split 0
  // with at least kMergeBatch splits, this thread's dimension of the first
  // kMergeBatch partial outputs is loaded before the weights are known (it
  // does not depend on them): one round trip for all of them
  const bool batch = n_splits >= kMergeBatch;
  float v[kMergeBatch];
  if (batch) {
    const int64_t pstride = (int64_t)Hq * kD;  // between the splits of one (row, head)
    const float* po = part_o + base * kD + d;
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) v[u] = po[u * pstride];
  }
  float m_loc = -INFINITY;
  for (int s = d; s < n_splits; s += 128) {
    const float2 ml = part_ml[base + (int64_t)s * Hq];
    wsplit[s] = ml.x;
    if (ml.y > 0.0f) m_loc = fmaxf(m_loc, ml.x);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m_loc = fmaxf(m_loc, __shfl_xor(m_loc, off));
  if ((d & 63) == 0) red[0][d >> 6] = m_loc;
  __syncthreads();
  const float M = fmaxf(red[0][0], red[0][1]);
  float l_loc = 0.0f;
  for (int s = d; s < n_splits; s += 128) {
    const float2 ml = part_ml[base + (int64_t)s * Hq];
    const float w = ml.y > 0.0f ? exp2f(wsplit[s] - M) : 0.0f;
    wsplit[s] = w;
    l_loc += ml.y * w;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) l_loc += __shfl_xor(l_loc, off);
  if ((d & 63) == 0) red[1][d >> 6] = l_loc;
  __syncthreads();
  const float L = red[1][0] + red[1][1];
  // weighted sum in split order
  float acc = 0.0f;
  int s = 0;
  if (batch) {
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) acc += v[u] * wsplit[u];
    s = kMergeBatch;
  }
  for (; s + 8 <= n_splits; s += 8) {
    float w8[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) w8[u] = part_o[(base + (int64_t)(s + u) * Hq) * kD + d];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += w8[u] * wsplit[s + u];
  }
  for (; s < n_splits; ++s) acc += part_o[(base + (int64_t)s * Hq) * kD + d] * wsplit[s];
  out[(row * Hq + h) * kD + d] = (uint16_t)f32_to_bf16_bits(acc / L);
  if (lse && d == 0) lse[row * Hq + h] = (M + log2f(L)) * 0.69314718055994531f;
}

AttnPlan plan_attn(int batch_rows, int64_t max_tokens, bool split_kv) {
  AttnPlan p{};
  p.rows = batch_rows;
  int64_t splits = 1;
  if (split_kv) {
    // about 256 workgroups: enough to spread the gathers over the chip while
    // keeping the partial (m, l, O) traffic of the merge small
    splits = (256 + batch_rows - 1) / batch_rows;
    if (splits > kMaxMergeSplits) splits = kMaxMergeSplits;
    const int64_t max_splits = (max_tokens + kChunk - 1) / kChunk;
    if (splits > max_splits) splits = max_splits;
    if (splits < 1) splits = 1;
  }
  int64_t st = (max_tokens + splits - 1) / splits;
  st = (st + kChunk - 1) / kChunk * kChunk;
  if (st < kChunk) st = kChunk;
  splits = (max_tokens + st - 1) / st;
  if (splits < 1) splits = 1;
  p.splits = (int)splits;
  p.split_tokens = st;
  return p;
}

size_t attn_workspace_bytes(const AttnPlan& p, int Hq) {
  if (p.splits == 1) return 0;
  const size_t n = (size_t)p.rows * p.splits * Hq;
  return n * kD * sizeof(float) + ((n * sizeof(float2) + 255) / 256 * 256) + 256;
}

PlanCheck check_attn_plan(const AttnPlan& p, int Hq, int Hkv, int top_k, int r) {
  PlanCheck c{};
  // static LDS of attn_gather_kernel: V tiles, block ids and their pages,
  // and (fewer than four KV heads) the cross-wave merge of (m, l, O)
  const size_t gather_lds = (size_t)4 * kChunk * kVPitch * 2 + 2 * kSelLds * 4 +
                            (Hkv < 4 ? (size_t)4 * 16 * kD * 4 + 2 * 4 * 16 * 4 : 0) + 64;
  c.n = p.splits > 1 ? 2 : 1;
  c.l[0] = LaunchShape{{p.rows > 0xFFFFFFFF ? 0xFFFFFFFFu : (uint32_t)p.rows, (uint32_t)p.splits, 1}, 256u,
                       gather_lds};
  c.l[1] = LaunchShape{{p.rows > 0xFFFFFFFF ? 0xFFFFFFFFu : (uint32_t)p.rows, (uint32_t)Hq, 1}, (uint32_t)kD,
                       (size_t)kMaxMergeSplits * 4 + 4 * 4 + 64};
  c.max_i32 = std::max<int64_t>({(int64_t)p.split_tokens, (int64_t)top_k * r, (int64_t)p.splits});
  c.max_offset = (int64_t)p.rows * p.splits * Hq * (int64_t)kD;
  c.unfit = nullptr;
  for (int i = 0; i < c.n; ++i) {
    const LaunchShape& l = c.l[i];
    if (l.grid[0] < 1 || l.grid[0] > 0x7FFFFFFFu || l.grid[1] < 1 || l.grid[1] > 65535u) c.unfit = "a launch grid exceeds the device's limits";
    else if (l.lds > 160 * 1024) c.unfit = "a workgroup exceeds 160 KiB of LDS";
  }
  if (!c.unfit && top_k > kSelLds) c.unfit = "more kept blocks than the gather stages";
  if (!c.unfit && p.splits > kMaxMergeSplits) c.unfit = "more splits than the merge takes";
  if (!c.unfit && c.max_i32 >= ((int64_t)1 << 31)) c.unfit = "a kernel index would exceed 32 bits";
  return c;
}

hipError_t launch_attn(const AttnPlan& p, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                       int64_t kv_batch_stride, int64_t q_pos0, const int32_t* kv_len, int Hq,
                       int Hkv, int r, int top_k, const int32_t* sel, const int32_t* sel_cnt,
                       float scale, uint16_t* out, float* lse, void* ws, hipStream_t stream,
                       PagedRows pg) {
  const int G = Hq / Hkv;
  if (sel && top_k > kSelLds) return hipErrorInvalidValue;
  const float scale_log2 = scale * 1.4426950408889634f;
  float* part_o = nullptr;
  float2* part_ml = nullptr;
  if (p.splits > 1) {
    const size_t n = (size_t)p.rows * p.splits * Hq;
    part_o = reinterpret_cast<float*>(ws);
    part_ml = reinterpret_cast<float2*>(reinterpret_cast<char*>(ws) + n * kD * sizeof(float));
  }
  const dim3 grid((unsigned)p.rows, (unsigned)p.splits);
#define QSA_LAUNCH_ATTN(HKV_)                                                                   \
  hipLaunchKernelGGL(attn_gather_kernel<HKV_>, grid, dim3(256), 0, stream, q, k, v,            \
                     kv_batch_stride, q_pos0, kv_len, Hq, G, r, top_k, sel, sel_cnt, p.splits, \
                     (int)p.split_tokens, scale_log2, out, lse, part_o, part_ml, pg)
  switch (Hkv) {
    case 1: QSA_LAUNCH_ATTN(1); break;
    case 2: QSA_LAUNCH_ATTN(2); break;
    case 4: QSA_LAUNCH_ATTN(4); break;
    default: return hipErrorInvalidValue;
  }
#undef QSA_LAUNCH_ATTN
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  hipLaunchKernelGGL(attn_merge_kernel, dim3((unsigned)p.rows, (unsigned)Hq), dim3(kD), 0, stream,
                     part_o, part_ml, p.splits, Hq, out, lse);
  return hipGetLastError();
}

}  // namespace qsa
