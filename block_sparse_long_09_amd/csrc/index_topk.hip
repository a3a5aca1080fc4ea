// Indexer scoring and causal top-k block selection.
//
// Method (explainer page "用125亿分之6的参数…", sparse-attention section; digest
// page "On the Design of Qwen3.8-Next Architecture", token-mixing paragraph):
// each query scores every complete micro-block before its own with a light
// multi-query indexer (H_i query heads, one shared 64-d block key); the best
// blocks are kept up to the budget. Score of query t and block j:
//   s(t, j) = w * sum_h max(0, q_{t,h} . c_j)        (fp32)
// Kept: the min(k - 1, b_t) best blocks j < b_t = t / r in (score desc,
// index asc) order, plus b_t itself; emitted in ascending block order.
//
// Kernel 1, index_stream_kernel: one wave owns QW consecutive queries (128
// indexer rows = QW x H_i) and one candidate range ("split"). It streams the
// block keys in tiles of 32 through v_mfma_f32_32x32x16_bf16 (A = query rows
// held in registers, B = 32 block keys loaded straight from global memory),
// reduces the heads in-lane (the rows of one query are placed so one lane's
// accumulators hold all its heads), and appends every candidate whose score
// beats the query's running threshold to a per-(query, split) buffer in the
// workspace. When a buffer nears capacity the wave radix-selects the exact
// (k-1)-th entry, compacts the buffer stably to the k-1 survivors and raises the
// threshold to that score. Candidates arrive in increasing block order, so a
// later candidate that only ties the threshold can never displace a kept one:
// the buffer always holds a superset of the split's exact top-(k-1).
//
// Kernel 2, index_select_kernel: one wave per query merges the split buffers
// (already in block order), radix-selects the exact (k-1)-th score, and writes
// the survivors in block order, then the query's own block, then -1 padding.
#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {

namespace {

// Exact rank selection over uint32 keys (non-negative fp32 bit patterns order
// like the floats). Finds tk, the keep-th largest key, and `need`, how many
// entries equal to tk belong to the top `keep`. Four 8-bit digit passes with a
// wave-private 256-bin histogram in LDS. Segments: (ptr, count) pairs produced
// by `seg(s)` for s < nseg, scanned in order.
template <typename SegFn>
__device__ void wave_radix_select(SegFn seg, int nseg, int keep, uint32_t* hist, uint32_t& tk,
                                  int& need_out) {
  const int lane = lane_id();
  uint32_t prefix = 0, mask = 0;
  int need = keep;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = lane; i < 256; i += kWave) hist[i] = 0;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    for (int s = 0; s < nseg; ++s) {
      const uint2* p;
      int n;
      seg(s, p, n);
      for (int i = lane; i < n; i += kWave) {
        const uint32_t key = p[i].x;
        if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
    // lane l owns bins 255-4l .. 252-4l (lane 0 holds the largest digits)
    const int top = 255 - 4 * lane;
    const uint32_t c0 = hist[top], c1 = hist[top - 1], c2 = hist[top - 2], c3 = hist[top - 3];
    const uint32_t tot = c0 + c1 + c2 + c3;
    uint32_t inc = tot;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const uint32_t v = __shfl_up(inc, off);
      if (lane >= off) inc += v;
    }
    const uint32_t exc = inc - tot;
    const bool hit = inc >= (uint32_t)need && exc < (uint32_t)need;
    const int L = __ffsll((unsigned long long)ballot(hit)) - 1;
    int dig = 0;
    uint32_t above = 0;
    if (lane == L) {
      uint32_t cum = exc;
      if (cum + c0 >= (uint32_t)need) {
        dig = top;
      } else {
        cum += c0;
        if (cum + c1 >= (uint32_t)need) {
          dig = top - 1;
        } else {
          cum += c1;
          if (cum + c2 >= (uint32_t)need) {
            dig = top - 2;
          } else {
            cum += c2;
            dig = top - 3;
          }
        }
      }
      above = cum;
    }
    dig = __shfl(dig, L);
    above = __shfl(above, L);
    prefix |= (uint32_t)dig << shift;
    mask |= 255u << shift;
    need -= (int)above;
    __builtin_amdgcn_wave_barrier();
  }
  tk = prefix;
  need_out = need;
}

// Keep, in order, entries with key > tk and the first `need` entries with
// key == tk. Writes entry e (its rank among kept is `pos`) through emit(pos, e).
template <typename SegFn, typename EmitFn>
__device__ int wave_stable_keep(SegFn seg, int nseg, uint32_t tk, int need, EmitFn emit) {
  const int lane = lane_id();
  int kept = 0, ties = 0;
  for (int s = 0; s < nseg; ++s) {
    const uint2* p;
    int n;
    seg(s, p, n);
    for (int base = 0; base < n; base += kWave) {
      const int i = base + lane;
      const bool in = i < n;
      const uint2 e = in ? p[i] : make_uint2(0u, 0u);
      const bool gt = in && e.x > tk;
      const bool eq = in && e.x == tk;
      const uint64_t me = ballot(eq);
      const int tie_rank = ties + __popcll(lanes_below(me));
      const bool keep = gt || (eq && tie_rank < need);
      const uint64_t mk = ballot(keep);
      if (keep) emit(kept + __popcll(lanes_below(mk)), e);
      kept += __popcll(mk);
      ties += __popcll(me);
    }
  }
  return kept;
}

__device__ __forceinline__ float relu_bits(float x) {
  // max on the integer view: negative values and -0.0 become +0.0
  return __int_as_float(max(__float_as_int(x), 0));
}

// Reduce one query's buffer of n entries (block order) to its exact top `keep`
// in place, keeping block order; returns the new threshold score.
__device__ __forceinline__ float compact_buffer(uint2* p, int n, int keep, uint32_t* hist) {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  auto seg = [&](int, const uint2*& sp, int& sn) {
    sp = p;
    sn = n;
  };
  uint32_t tk;
  int need;
  wave_radix_select(seg, 1, keep, hist, tk, need);
  wave_stable_keep(seg, 1, tk, need, [&](int pos, uint2 e) { p[pos] = e; });
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  return __uint_as_float(tk);
}

}  // namespace

template <int HI, int AT>
__global__ __launch_bounds__(256) void index_stream_kernel(
    const uint16_t* __restrict__ idx_q, const uint16_t* __restrict__ cmp_k, int64_t cmp_stride,
    const int32_t* __restrict__ q_pos0, int n_q, int r, int keep, float w, int n_qgroups,
    int splits, int split_len, int cap, uint2* __restrict__ buf, int* __restrict__ buf_cnt) {
  constexpr int QPH = 16 / HI;    // queries per lane-half per A tile
  constexpr int QPT = 32 / HI;    // queries per A tile
  constexpr int QW = AT * QPT;    // queries per wave
  constexpr int NS = AT * QPH;    // score slots per lane
  __shared__ uint32_t hist_all[4][256];

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5;
  const int col = lane & 31;
  const int task = blockIdx.x * 4 + wave;
  if (task >= n_qgroups * splits) return;
  const int qg = task % n_qgroups;
  const int split = task / n_qgroups;
  const int b = blockIdx.y;
  uint32_t* hist = hist_all[wave];

  const int64_t pos0 = q_pos0[b];
  const int sbeg = split * split_len;
  const int send = sbeg + split_len;

  // Query of slot s in lane-half hh.
  auto slot_query = [&](int s, int hh) { return qg * QW + (s / QPH) * QPT + hh * QPH + (s % QPH); };
  auto buf_of = [&](int qi) {
    return buf + (((int64_t)b * n_q + qi) * splits + split) * (int64_t)cap;
  };

  int lim[NS];
  float tau[NS];
  int cnt[NS];
  int maxlim = 0;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int qi = slot_query(s, half);
    int l = 0;
    if (qi < n_q) {
      const int64_t bt = (pos0 + qi) / r;
      l = (int)(bt < (int64_t)send ? bt : (int64_t)send);
    }
    lim[s] = l;
    tau[s] = -1.0f;
    cnt[s] = 0;
    maxlim = max(maxlim, l);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) maxlim = max(maxlim, __shfl_xor(maxlim, off));

  if (keep > 0 && maxlim > sbeg) {
    // A operand: row m = col of each A tile; lane-half picks k-offset 8*half.
    u32x4 A[AT][4];
    {
      const int m = col;
      const int i = 4 * (m >> 3) + (m & 3);
      const int hh = (m >> 2) & 1;
      const int qs = hh * QPH + i / HI;
      const int head = i % HI;
#pragma unroll
      for (int a = 0; a < AT; ++a) {
        const int qi = qg * QW + a * QPT + qs;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          if (qi < n_q) {
            A[a][ks] = ld16(idx_q + (((int64_t)b * n_q + qi) * HI + head) * 64 + 16 * ks + 8 * half);
          } else {
            A[a][ks] = u32x4{0u, 0u, 0u, 0u};
          }
        }
      }
    }
    const uint16_t* kb = cmp_k + (int64_t)b * cmp_stride + 8 * half;
    auto load_b = [&](int c, u32x4* B) {
      const int j = min(c + col, maxlim - 1);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) B[ks] = ld16(kb + (int64_t)j * 64 + 16 * ks);
    };
    u32x4 Bn[4];
    load_b(sbeg, Bn);
    for (int c = sbeg; c < maxlim; c += 32) {
      u32x4 B[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) B[ks] = Bn[ks];
      if (c + 32 < maxlim) load_b(c + 32, Bn);
      f32x16 acc[AT];
#pragma unroll
      for (int a = 0; a < AT; ++a) {
        acc[a] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) acc[a] = mfma32x32x16(A[a][ks], B[ks], acc[a]);
      }
      const int j = c + col;
      const uint32_t below = (1u << col) - 1u;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int a = s / QPH, qq = s % QPH;
        float sum = 0.0f;
#pragma unroll
        for (int hd = 0; hd < HI; ++hd) sum += relu_bits(acc[a][qq * HI + hd]);
        const float sc = sum * w;
        const bool pass = (j < lim[s]) && (sc > tau[s]);
        const uint64_t m64 = ballot(pass);
        if (m64) {
          const uint32_t mh = (uint32_t)(m64 >> (32 * half));
          if (pass) {
            const int pos = cnt[s] + __popc(mh & below);
            buf_of(slot_query(s, half))[pos] = make_uint2(__float_as_uint(sc), (uint32_t)j);
          }
          cnt[s] += __popc(mh);
        }
      }
      uint32_t need_mask = 0;  // bit 2s+hh: slot s of lane-half hh must be compacted
#pragma unroll
      for (int s = 0; s < NS; ++s) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          if (__shfl(cnt[s], 32 * hh) > cap - 32) need_mask |= 1u << (2 * s + hh);
      }
      while (need_mask) {
        const int bit = __ffs(need_mask) - 1;
        need_mask &= need_mask - 1;
        const int s = bit >> 1, hh = bit & 1;
        int cs = 0;
#pragma unroll
        for (int s2 = 0; s2 < NS; ++s2)
          if (s2 == s) cs = cnt[s2];
        const int ch = __shfl(cs, 32 * hh);
        const float nt = compact_buffer(buf_of(slot_query(s, hh)), ch, keep, hist);
        if (half == hh) {
#pragma unroll
          for (int s2 = 0; s2 < NS; ++s2)
            if (s2 == s) {
              cnt[s2] = keep;
              tau[s2] = nt;
            }
        }
      }
    }
  }
  if (col == 0) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int qi = slot_query(s, half);
      if (qi < n_q) buf_cnt[((int64_t)b * n_q + qi) * splits + split] = cnt[s];
    }
  }
}

__global__ __launch_bounds__(256) void index_select_kernel(
    const uint2* __restrict__ buf, const int* __restrict__ buf_cnt, const int32_t* __restrict__ q_pos0,
    int batch, int n_q, int r, int k, int splits, int cap, int32_t* __restrict__ sel,
    int32_t* __restrict__ sel_cnt) {
  __shared__ uint32_t hist_all[4][256];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int64_t gw = (int64_t)blockIdx.x * 4 + wave;
  if (gw >= (int64_t)batch * n_q) return;
  const int b = (int)(gw / n_q);
  const int qi = (int)(gw % n_q);
  uint32_t* hist = hist_all[wave];
  const int64_t t = (int64_t)q_pos0[b] + qi;
  const int64_t bt = t / r;
  const int keep = (int)((int64_t)(k - 1) < bt ? (int64_t)(k - 1) : bt);
  const uint2* qb = buf + gw * splits * (int64_t)cap;
  const int* qc = buf_cnt + gw * splits;
  int32_t* out = sel + gw * k;

  auto seg = [&](int s, const uint2*& sp, int& sn) {
    sp = qb + (int64_t)s * cap;
    sn = qc[s];
  };
  int total = 0;
  for (int s = lane; s < splits; s += kWave) total += qc[s];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) total += __shfl_xor(total, off);

  if (keep > 0) {
    uint32_t tk = 0;
    int need = 0x7FFFFFFF;
    if (total > keep) wave_radix_select(seg, splits, keep, hist, tk, need);
    wave_stable_keep(seg, splits, tk, need, [&](int pos, uint2 e) { out[pos] = (int32_t)e.y; });
  }
  if (lane == 0) {
    out[keep] = (int32_t)bt;
    sel_cnt[gw] = keep + 1;
  }
  for (int i = keep + 1 + lane; i < k; i += kWave) out[i] = -1;
}

IndexPlan plan_index(int hi, int k, int batch, int n_q, int64_t max_q_end, int r) {
  IndexPlan p{};
  p.hi = hi;
  p.at = n_q >= 64 ? 4 : 1;
  p.qw = p.at * 32 / hi;
  p.n_qgroups = (n_q + p.qw - 1) / p.qw;
  const int64_t max_cand = max_q_end > 0 ? (max_q_end - 1) / r : 0;
  p.max_cand = max_cand;
  // enough wave tasks to give every SIMD a few waves; splits no shorter than 256
  const int64_t waves = (int64_t)batch * p.n_qgroups;
  int64_t splits = (4096 + waves - 1) / waves;
  const int64_t max_splits = (max_cand + 255) / 256;
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  int64_t split_len = (max_cand + splits - 1) / splits;
  split_len = (split_len + 31) / 32 * 32;
  if (split_len < 32) split_len = 32;
  p.splits = (int)splits;
  p.split_len = (int)split_len;
  const int keep = k - 1;
  int cap = 2048;
  if (cap < 2 * keep + 64) cap = (2 * keep + 64 + 63) / 64 * 64;
  if ((int64_t)split_len + 32 <= cap) cap = (int)split_len + 32;
  p.cap = cap;
  p.buf_bytes = (size_t)batch * n_q * p.splits * (size_t)cap * sizeof(uint2);
  p.cnt_bytes = (size_t)batch * n_q * p.splits * sizeof(int);
  p.workspace = p.buf_bytes + ((p.cnt_bytes + 255) / 256 * 256);
  return p;
}

hipError_t launch_index_topk(const IndexPlan& p, const uint16_t* idx_q, const uint16_t* cmp_k,
                             int64_t cmp_stride, const int32_t* q_pos0, int batch, int n_q, int r,
                             int k, float w, int32_t* sel, int32_t* sel_cnt, void* ws,
                             hipStream_t stream) {
  uint2* buf = reinterpret_cast<uint2*>(ws);
  int* cnt = reinterpret_cast<int*>(reinterpret_cast<char*>(ws) + p.buf_bytes);
  const int tasks = p.n_qgroups * p.splits;
  const dim3 g1((tasks + 3) / 4, batch);
#define QSA_LAUNCH_STREAM(HI_, AT_)                                                               \
  hipLaunchKernelGGL((index_stream_kernel<HI_, AT_>), g1, dim3(256), 0, stream, idx_q, cmp_k,     \
                     cmp_stride, q_pos0, n_q, r, k - 1, w, p.n_qgroups, p.splits, p.split_len,   \
                     p.cap, buf, cnt)
  switch (p.hi * 10 + p.at) {
    case 14: QSA_LAUNCH_STREAM(1, 4); break;
    case 11: QSA_LAUNCH_STREAM(1, 1); break;
    case 24: QSA_LAUNCH_STREAM(2, 4); break;
    case 21: QSA_LAUNCH_STREAM(2, 1); break;
    case 44: QSA_LAUNCH_STREAM(4, 4); break;
    case 41: QSA_LAUNCH_STREAM(4, 1); break;
    case 84: QSA_LAUNCH_STREAM(8, 4); break;
    case 81: QSA_LAUNCH_STREAM(8, 1); break;
    case 164: QSA_LAUNCH_STREAM(16, 4); break;
    case 161: QSA_LAUNCH_STREAM(16, 1); break;
    default: return hipErrorInvalidValue;
  }
#undef QSA_LAUNCH_STREAM
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t nw = (int64_t)batch * n_q;
  hipLaunchKernelGGL(index_select_kernel, dim3((unsigned)((nw + 3) / 4)), dim3(256), 0, stream,
                     buf, cnt, q_pos0, batch, n_q, r, k, p.splits, p.cap, sel, sel_cnt);
  return hipGetLastError();
}

}  // namespace qsa
