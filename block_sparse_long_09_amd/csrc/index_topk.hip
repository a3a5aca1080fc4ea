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
// Prefill, few queries per sequence (n_q < 64):
//   index_stream_kernel: one wave owns QW consecutive queries (128 indexer rows
//   = QW x H_i) and one candidate range ("split"). It streams the block keys
//   in tiles of 32 through v_mfma_f32_32x32x16_bf16 (A = query rows held in
//   registers, pre-scaled by w when w is a power of two, which is exact;
//   B = 32 block keys loaded from global memory two tiles ahead), reduces the
//   heads in-lane (the rows of a query are placed so one lane's accumulators
//   hold all its heads) and appends every candidate whose score beats the
//   query's running threshold to a per-(query, split) buffer in the workspace.
//   When a buffer nears capacity the wave stages it in LDS, radix-selects the
//   exact (k-1)-th entry, compacts the buffer stably to k-1 entries and raises
//   the threshold to that score. Candidates arrive in increasing block order,
//   so a later candidate that only ties the threshold can never displace a
//   kept one: the buffer always holds a superset of the split's exact
//   top-(k-1). Each split ends compacted to at most k-1 entries.
// Prefill, many queries (n_q >= 64): index_prefill_kernel, the same scoring
//   and buffers with workgroups of compute waves that share LDS tiles of block
//   keys filled by a copy wave, approximate compactions, and thresholds seeded
//   from a strided sample of the split, checked after the scan (see there).
// Both end in index_select_kernel: one workgroup per query merges the split
//   buffers (already in block order) in LDS, selects exactly and writes the
//   output.
//
// Decode (one query per sequence):
//   index_decode_scan_kernel: one 8-wave workgroup per 2048-candidate split of
//   one sequence streams the block keys (HBM bound), writes every score to the
//   workspace and lists the split's entries at or above the lower edge of the
//   histogram bucket holding its list_min-th largest key, with the largest
//   key it left out.
//   index_decode_select_kernel: one workgroup per sequence selects the top
//   (k-1) of the union of the split lists. The result is exact when every
//   split's largest omitted key is below the selected threshold; otherwise the
//   workgroup selects exactly from the stored scores of all candidates.
#include "qsa_device.h"
#include "qsa_internal.h"
#include "select.h"

#include <algorithm>

namespace qsa {

namespace {

constexpr int kScanThreads = 512;              // decode split scan: 256 candidates per wave
constexpr int kDecodeSplit = kScanThreads * 4;  // candidates per decode split
constexpr int kMergeThreads = 1024;             // decode merge
constexpr int kSelScratch = 1024;               // keys a workgroup select gathers for its last passes
constexpr int kDecodeMaxSplits = 1024;  // decode splits per sequence
constexpr size_t kMergeMaxLds = 140 * 1024;  // merge LDS for the staged split lists

__device__ __forceinline__ float relu_bits(float x) {
  // max on the integer view: negative values and -0.0 become +0.0
  return __int_as_float(max(__float_as_int(x), 0));
}

__device__ __forceinline__ u32x4 scale_bf16x8(u32x4 v, float s) {
  u32x4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    o[e] = pack_bf16x2(bf16_bits_to_f32(v[e] & 0xFFFFu) * s, bf16_bits_to_f32(v[e] >> 16) * s);
  return o;
}

// Reduce one query's buffer of n entries (block order) to its exact top `keep`
// in place, keeping block order; returns the new threshold score.
__device__ __forceinline__ float compact_buffer(uint2* p, int n, int keep, uint32_t* hist, uint2* stage) {
  const int lane = lane_id();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  for (int base = 0; base < n; base += 8 * kWave) {
    uint2 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = base + u * kWave + lane;
      if (i < n) v[u] = p[i];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = base + u * kWave + lane;
      if (i < n) stage[i] = v[u];
    }
  }
  wave_sync();
  uint32_t tk;
  int need;
  wave_select([&](int i) { return stage[i].x; }, n, keep, hist, tk, need);
  wave_stable_keep([&](int i) { return stage[i]; }, n, tk, need, [&](int pos, uint2 e) { p[pos] = e; });
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  wave_sync();
  return __uint_as_float(tk);
}

typedef __attribute__((address_space(3))) uint32_t lds_u32;
typedef __attribute__((address_space(3))) unsigned long long lds_u64;
typedef __attribute__((address_space(1))) unsigned long long glb_u64;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// s_waitcnt immediate: at most n (< 64) vector memory operations outstanding,
// no wait on the other counters
constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

// Copy the n entries of a buffer into the wave's LDS stage (entry i to st[i])
// with global_load_lds: 16 bytes (two entries) per lane per instruction, all
// issued before one wait, no registers held. The buffer holds at least n
// rounded up to 128 entries (its capacity is a multiple of 128), so every
// load is in bounds. The wave's earlier appends to it have completed first.
__device__ __forceinline__ void stage_entries(const glb_u64* p, int n, lds_u64* st) {
  const int lane = lane_id();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  for (int base = 0; base < n; base += 128)
    __builtin_amdgcn_global_load_lds((const glb_void_t*)(p + base + 2 * lane), (lds_void_t*)(st + base), 16, 0, 0);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  wave_sync();
}

// Exact compaction: reduce one query's buffer of n entries (block order) to
// its exact top `keep` in place, keeping block order; returns the new
// threshold. The entries are staged in LDS once; the selection and the keep
// pass read them there. An entry is one 64-bit word: key low, block high. Not
// inlined (one copy serves every call site).
__device__ __noinline__ float compact_keys_staged(glb_u64* p, int n, int keep, lds_u32* hist, lds_u64* st) {
  const int lane = lane_id();
  stage_entries(p, n, st);
  uint32_t tk;
  int need;
  wave_select([&](int i) { return (uint32_t)st[i]; }, n, keep, hist, tk, need);
  int kept = 0, ties = 0;
  for (int base = 0; base < n; base += 8 * kWave) {
    unsigned long long e[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = base + u * kWave + lane;
      e[u] = i < n ? st[i] : 0ull;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = base + u * kWave + lane;
      const bool in = i < n;
      const uint32_t key = (uint32_t)e[u];
      const bool gt = in && key > tk;
      const bool eq = in && key == tk;
      const uint64_t me = ballot(eq);
      const bool keep_it = gt || (eq && ties + __popcll(lanes_below(me)) < need);
      const uint64_t mk = ballot(keep_it);
      if (keep_it) p[kept + __popcll(lanes_below(mk))] = e[u];
      kept += __popcll(mk);
      ties += __popcll(me);
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  wave_sync();
  return __uint_as_float(tk);
}

// Approximate in-loop compaction: keep, in block order, every entry whose key
// is at least L, where L is the lower edge of the histogram bucket that holds
// the keep-th largest key. The entries are staged in LDS once and bucketed by
// their key's offset from the smallest key (8 bits per pass below the
// offsets' leading zeros); further passes refine the bucket while more than
// keep + 64 entries would survive (a tight threshold lets fewer later
// candidates in, and leaves the buffer room for many before the next
// compaction). At least `keep` entries survive, so the buffer stays a
// superset of the exact top `keep`; a later candidate with key <= L can never
// enter it (at least `keep` entries with key >= L and a smaller block index
// precede it). Returns (L, the number of entries kept); a pair by value keeps
// the caller free of private (scratch) memory.
__device__ __noinline__ uint2 compact_keys_approx(glb_u64* p, int n, int keep, lds_u32* hist, lds_u64* st) {
  const int lane = lane_id();
  stage_entries(p, n, st);
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  for (int base = 0; base < n; base += 16 * kWave) {
    uint32_t v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int i = base + u * kWave + lane;
      v[u] = i < n ? (uint32_t)st[i] : 0u;
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int i = base + u * kWave + lane;
      if (i < n) {
        kmin = min(kmin, v[u]);
        kmax = max(kmax, v[u]);
      }
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, off));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, off));
  }
  // radix passes on key - kmin: the bucket [kbase, kbase + 2^hi) holds the
  // keep-th largest key
  uint32_t kbase = kmin;
  int hi = range_bits(kmin, kmax);
  uint32_t need = (uint32_t)keep;
  uint32_t above_all = 0;        // entries above the bucket
  uint32_t ge = (uint32_t)n;     // entries with key >= kbase
  for (int pass = 0; pass < 4 && hi > 0 && ge > (uint32_t)(keep + 64); ++pass) {
    const int lo = hi > 8 ? hi - 8 : 0;
    for (int i = lane; i < 256; i += kWave) hist[i] = 0;
    wave_sync();
    // eight keys per lane read before their eight atomics: the reads cannot
    // move past an LDS atomic by themselves (the compiler cannot tell the
    // stage from the histogram), and one read-then-add per key would wait out
    // the LDS latency once per key
    for (int base = 0; base < n; base += 8 * kWave) {
      uint32_t kk[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = base + u * kWave + lane;
        kk[u] = i < n ? (uint32_t)st[i] : 0u;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int d = base + u * kWave + lane < n ? range_digit(kk[u], kbase, hi, lo) : -1;
        if (d >= 0) __atomic_fetch_add(&hist[d], 1u, __ATOMIC_RELAXED);
      }
    }
    wave_sync();
    int dig;
    uint32_t above;
    wave_find_digit(hist, need, dig, above);
    const uint32_t in_bucket = hist[dig];
    wave_sync();
    kbase += (uint32_t)dig << lo;
    need -= above;
    above_all += above;
    ge = above_all + in_bucket;
    hi = lo;
  }
  const uint32_t L = kbase;
  int kept = 0;
  for (int base = 0; base < n; base += 16 * kWave) {
    unsigned long long e[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int i = base + u * kWave + lane;
      e[u] = i < n ? st[i] : 0ull;
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int i = base + u * kWave + lane;
      const bool keep_it = i < n && (uint32_t)e[u] >= L;
      const uint64_t mk = ballot(keep_it);
      if (keep_it) p[kept + __popcll(lanes_below(mk))] = e[u];
      kept += __popcll(mk);
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  wave_sync();
  return make_uint2(L, (uint32_t)kept);
}

}  // namespace

template <int HI, int AT>
__global__ __launch_bounds__(256) void index_stream_kernel(
    const uint16_t* __restrict__ idx_q, const uint16_t* __restrict__ cmp_k, int64_t cmp_stride,
    const int32_t* __restrict__ q_pos0, int n_q, int r, int keep, float a_scale, float w_epi,
    int n_qgroups, int splits, int split_len, int cap, uint2* __restrict__ buf,
    int* __restrict__ buf_cnt, const int32_t* __restrict__ cu_q) {
  constexpr int QPH = 16 / HI;    // queries per lane-half per A tile
  constexpr int QPT = 32 / HI;    // queries per A tile
  constexpr int QW = AT * QPT;    // queries per wave
  constexpr int NS = AT * QPH;    // score slots per lane
  __shared__ uint32_t hist_all[4][256];
  extern __shared__ uint2 stage_all[];

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
  uint2* stage = stage_all + (size_t)wave * cap;

  const int64_t pos0 = q_pos0[b];
  // this sequence's query rows: [row0, row0 + nqb) (packed rows when cu_q is given)
  const int64_t row0 = cu_q ? (int64_t)cu_q[b] : (int64_t)b * n_q;
  const int nqb = cu_q ? min(cu_q[b + 1] - cu_q[b], n_q) : n_q;  // n_q = rows per sequence at most
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
  int maxlim = 0, minlim = 0x7FFFFFFF;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int qi = slot_query(s, half);
    int l = 0;
    if (qi < nqb) {
      const int64_t bt = (pos0 + qi) / r;
      l = (int)(bt < (int64_t)send ? bt : (int64_t)send);
      minlim = min(minlim, l);
    }
    lim[s] = l;
    tau[s] = qi < nqb ? -1.0f : INFINITY;  // an absent query never takes a candidate
    cnt[s] = 0;
    maxlim = max(maxlim, l);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    maxlim = max(maxlim, __shfl_xor(maxlim, off));
    minlim = min(minlim, __shfl_xor(minlim, off));
  }

  if (keep > 0 && maxlim > sbeg) {
    // A operand: row m = col of each A tile; the lane-half picks k-offset 8*half.
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
          if (qi < nqb) {
            const u32x4 v = ld16(idx_q + ((row0 + qi) * HI + head) * 64 + 16 * ks + 8 * half);
            A[a][ks] = a_scale == 1.0f ? v : scale_bf16x8(v, a_scale);
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
    u32x4 B0[4], B1[4];
    load_b(sbeg, B0);
    load_b(sbeg + 32, B1);
    for (int c = sbeg; c < maxlim; c += 32) {
      u32x4 B[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        B[ks] = B0[ks];
        B0[ks] = B1[ks];
      }
      if (c + 64 < maxlim) load_b(c + 64, B1);
      f32x16 acc[AT];
#pragma unroll
      for (int a = 0; a < AT; ++a) {
        acc[a] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) acc[a] = mfma32x32x16(A[a][ks], B[ks], acc[a]);
      }
      const int j = c + col;
      const uint32_t below = (1u << col) - 1u;
      const bool interior = c + 32 <= minlim;  // every query of the wave sees the whole tile
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int a = s / QPH, qq = s % QPH;
        float sum = 0.0f;
#pragma unroll
        for (int hd = 0; hd < HI; ++hd) sum += relu_bits(acc[a][qq * HI + hd]);
        const float sc = sum * w_epi;
        const bool pass = (interior || j < lim[s]) && (sc > tau[s]);
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
      bool over = false;
#pragma unroll
      for (int s = 0; s < NS; ++s) over |= cnt[s] > cap - 32;
      if (ballot(over)) {
        uint32_t need_mask = 0;  // bit 2s+hh: slot s of lane-half hh must be compacted
#pragma unroll
        for (int s = 0; s < NS; ++s) {
#pragma unroll
          for (int hh = 0; hh < 2; ++hh)
            if (__builtin_amdgcn_readlane(cnt[s], 32 * hh) > cap - 32) need_mask |= 1u << (2 * s + hh);
        }
        while (need_mask) {
          const int bit = __ffs(need_mask) - 1;
          need_mask &= need_mask - 1;
          const int s = bit >> 1, hh = bit & 1;
          int cs = 0;
#pragma unroll
          for (int s2 = 0; s2 < NS; ++s2)
            if (s2 == s) cs = cnt[s2];
          const int ch = __builtin_amdgcn_readlane(cs, 32 * hh);
          const float nt = compact_buffer(buf_of(slot_query(s, hh)), ch, keep, hist, stage);
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
    // leave every split buffer at most `keep` long
    uint32_t need_mask = 0;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        if (__builtin_amdgcn_readlane(cnt[s], 32 * hh) > keep) need_mask |= 1u << (2 * s + hh);
    }
    while (need_mask) {
      const int bit = __ffs(need_mask) - 1;
      need_mask &= need_mask - 1;
      const int s = bit >> 1, hh = bit & 1;
      int cs = 0;
#pragma unroll
      for (int s2 = 0; s2 < NS; ++s2)
        if (s2 == s) cs = cnt[s2];
      const int ch = __builtin_amdgcn_readlane(cs, 32 * hh);
      compact_buffer(buf_of(slot_query(s, hh)), ch, keep, hist, stage);
      if (half == hh) {
#pragma unroll
        for (int s2 = 0; s2 < NS; ++s2)
          if (s2 == s) cnt[s2] = keep;
      }
    }
  }
  if (col == 0) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int qi = slot_query(s, half);
      if (qi < nqb) buf_cnt[((int64_t)b * n_q + qi) * splits + split] = cnt[s];
    }
  }
}

// Prefill indexer for many queries per sequence (n_q >= 64): a workgroup of NW
// compute waves (NW x QW queries; NW = 4, 3 or 8, chosen with the number of
// workgroups a CU holds, see plan_index) and one copy wave shares one
// candidate split.
// Block keys go HBM -> LDS directly (global_load_lds, issued by the copy wave
// into a ring of 64-candidate tiles with XOR-swizzled 16-byte parts, so the
// B-fragment reads hit distinct banks) -> B fragments: 4 slots refilled two
// tiles per barrier, or at NW = 3 3 slots refilled kPrefillDepth tiles ahead,
// one tile per barrier. Only the copy wave loads tiles and it waits on its own
// counter alone: the compute waves' appends (global stores) are never waited
// for before a tile is in place, as they would be if the compute waves loaded
// the tiles (the memory counter is in order and counts stores too).
// Per query: running threshold and a (score, block) buffer as in
// index_stream_kernel, the threshold starting from a seed taken from a sample
// of the split's tiles when seed_stride > 0 (a split whose seeded buffer ends
// short is scanned again unseeded); a wave compacts its own buffers (keys
// staged in its LDS area) when one nears capacity. Splits end with at most
// `cap` entries; the select kernel takes them as they are.
constexpr int kPrefillDepth = 2;      // tiles the copy wave keeps in flight
constexpr int prefill_vmcnt(int n) { return vmcnt_imm(n); }
template <int HI, int AT, bool SCALE_EPI, int NW>
__global__ __launch_bounds__(64 * (NW + 1)) __attribute__((amdgpu_waves_per_eu(NW == 4 ? 4 : 3)))
void index_prefill_kernel(
    const uint16_t* __restrict__ idx_q, const uint16_t* __restrict__ cmp_k, int64_t cmp_stride,
    const int32_t* __restrict__ q_pos0, int n_q, int r, int keep, float a_scale, float w_epi,
    int n_qgroups, int splits, int split_len, int cap, int seed_stride, uint2* __restrict__ buf,
    int* __restrict__ buf_cnt, const int32_t* __restrict__ cu_q) {
  constexpr int QPH = 16 / HI;
  constexpr int QPT = 32 / HI;
  constexpr int QW = AT * QPT;
  constexpr int NS = AT * QPH;
  constexpr int TILE = 64;                       // candidates per LDS tile
  constexpr int TILE_BYTES = TILE * 128;         // 8 KiB
  constexpr int PF = kPrefillDepth;
  // tiles per barrier: two, or else the compute waves wait for each other at
  // every tile (their appends vary from tile to tile); one at NW = 3, whose
  // three workgroups per CU leave no LDS for a fourth slot
  constexpr int TT = NW == 3 ? 1 : 2;
  constexpr int NSLOT = TT == 2 ? 4 : 3;         // LDS slots
  static_assert(NSLOT >= PF + 1 && NSLOT >= 2 * TT, "a slot is refilled only after its tile was processed");
  __shared__ __attribute__((aligned(16))) unsigned char ring[NSLOT * TILE_BYTES];
  __shared__ uint32_t hist_all[NW][256];
  __shared__ int wg_lim[NW];
  __shared__ int wg_compact;  // tile before which every wave compacts its fuller buffers
  __shared__ int wg_rerun;    // a seeded buffer of the workgroup ended short: scan again
  extern __shared__ unsigned long long kstage_all[];  // NW x cap entries: each wave's compaction stage

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // 4: the copy wave
  const bool copier = wave == NW;
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int col = lane & 31;
  // the last queries see the most candidates: their workgroups go out first,
  // so the short ones fill in behind them when the grid takes several rounds
  const int qg = (gridDim.x - 1 - blockIdx.x) * NW + wave;
  const int split = blockIdx.y;
  const int b = blockIdx.z;
  lds_u32* hist_l = (lds_u32*)hist_all[copier ? 0 : wave];
  lds_u64* kstage_l = (lds_u64*)(kstage_all + (copier ? 0 : wave) * cap);

  const int64_t pos0 = q_pos0[b];
  // this sequence's query rows: [row0, row0 + nqb) (packed rows when cu_q is given)
  const int64_t row0 = cu_q ? (int64_t)cu_q[b] : (int64_t)b * n_q;
  const int nqb = cu_q ? min(cu_q[b + 1] - cu_q[b], n_q) : n_q;  // n_q = rows per sequence at most
  const int sbeg = split * split_len;
  const int send = sbeg + split_len;
  auto slot_query = [&](int s, int hh) { return qg * QW + (s / QPH) * QPT + hh * QPH + (s % QPH); };
  auto buf_of = [&](int qi) {
    return buf + (((int64_t)b * n_q + qi) * splits + split) * (int64_t)cap;
  };
  const bool wave_live = !copier && qg < n_qgroups;
  // candidates of query qi in this split: [sbeg, lim_of(qi))
  auto lim_of = [&](int qi) {
    const int64_t bt = (pos0 + qi) / r;
    return (int)(bt < (int64_t)send ? bt : (int64_t)send);
  };

  float tau[NS];
  int cnt[NS];
  int lim[NS];        // candidate bound of this lane's query in slot s
  // buffer of slot 0 of this lane-half; slot s's query is d(s) queries later
  // (an absent query's buffer is never written: its threshold is +inf)
  glb_u64* const bp0 = (glb_u64*)(buf + (((int64_t)b * n_q + slot_query(0, half)) * splits + split) * (int64_t)cap);
  const int64_t qstride = (int64_t)splits * cap;
  auto buf_slot = [&](int s) { return bp0 + (int64_t)((s / QPH) * QPT + s % QPH) * qstride; };
  int maxlim = 0, minlim = 0x7FFFFFFF;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int qi = slot_query(s, half);
    int l = 0;
    if (wave_live && qi < nqb) {
      l = lim_of(qi);
      minlim = min(minlim, l);
    }
    tau[s] = (wave_live && qi < nqb) ? -1.0f : INFINITY;  // an absent query takes nothing
    cnt[s] = 0;
    lim[s] = l;
    maxlim = max(maxlim, l);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    maxlim = max(maxlim, __shfl_xor(maxlim, off));
    minlim = min(minlim, __shfl_xor(minlim, off));
  }
  minlim = __builtin_amdgcn_readfirstlane(minlim);  // wave-uniform after the reduction
  if (lane == 0 && !copier) wg_lim[wave] = maxlim;
  if (tid == 0) {
    wg_compact = -1;
    wg_rerun = 0;
  }
  __syncthreads();
  int wg_max = wg_lim[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) wg_max = max(wg_max, wg_lim[w]);

  uint32_t frozen = 0;  // bit s: slot s's count was written before a second scan
  if (keep > 0 && wg_max > sbeg) {
    u32x4 A[AT][4];
    if (!copier) {
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
          if (wave_live && qi < nqb) {
            const u32x4 v = ld16(idx_q + ((row0 + qi) * HI + head) * 64 + 16 * ks + 8 * half);
            A[a][ks] = a_scale == 1.0f ? v : scale_bf16x8(v, a_scale);
          } else {
            A[a][ks] = u32x4{0u, 0u, 0u, 0u};
          }
        }
      }
    }
    const unsigned char* kb = reinterpret_cast<const unsigned char*>(cmp_k + (int64_t)b * cmp_stride);
    const int ntiles = (wg_max - sbeg + TILE - 1) / TILE;
    // The tiles go through the LDS ring as one stream of "virtual" tiles in up
    // to three phases, each padded to whole barrier groups: [0, P1) the
    // sample (split tiles 0, rho, 2 rho, ...) that seeds the thresholds,
    // [P1, P1 + P2) the scan of every tile, [P1 + P2, P1 + 2 P2) a second scan,
    // run only when a seeded buffer ended short. Without seeding P1 = 0.
    // (not at one indexer head: its 16 queries per lane would need 64 more
    // registers for the sample's scores)
    constexpr bool kSample = NS <= 8;
    const int rho = kSample ? seed_stride : 0;
    const int n1 = rho > 0 ? (ntiles + rho - 1) / rho : 0;
    const int P1 = (n1 + TT - 1) / TT * TT;
    const int P2 = (ntiles + TT - 1) / TT * TT;
    auto real_tile = [&](int v) { return v < P1 ? v * rho : (v < P1 + P2 ? v - P1 : v - P1 - P2); };
    // Virtual tile v goes to LDS slot v % NSLOT, written by the copy wave's
    // eight 1 KiB global_load_lds: piece u of lane l lands at byte 1024u + 16l
    // of the slot, i.e. row 8u + l / 8, part l % 8, and carries the row's
    // global part (l % 8) ^ (row % 8). Rows past the workgroup's last candidate
    // (also those of the padding tiles) read that candidate instead, so every
    // load is in bounds.
    auto issue_tile = [&](int t) __attribute__((always_inline)) {
      unsigned char* dst = ring + (t % NSLOT) * TILE_BYTES;
      const int part = (lane & 7) ^ (lane >> 3);
      const int first = sbeg + real_tile(t) * TILE;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int row = min(first + 8 * u + (lane >> 3), wg_max - 1);
        __builtin_amdgcn_global_load_lds((glb_void_t*)(kb + (int64_t)row * 128 + part * 16),
                                         (lds_void_t*)(dst + 1024 * u), 16, 0, 0);
      }
    };
    // compact this wave's buffers holding more than `limit` entries
    auto compact_over = [&](int limit) {
      uint32_t need_mask = 0;  // bit 2s+hh: slot s of lane-half hh
#pragma unroll
      for (int s = 0; s < NS; ++s) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          if (__builtin_amdgcn_readlane(cnt[s], 32 * hh) > limit) need_mask |= 1u << (2 * s + hh);
      }
      while (need_mask) {
        const int bit = __ffs(need_mask) - 1;
        need_mask &= need_mask - 1;
        const int s = bit >> 1, hh = bit & 1;
        int cs = 0;
#pragma unroll
        for (int s2 = 0; s2 < NS; ++s2)
          if (s2 == s) cs = cnt[s2];
        const int ch = __builtin_amdgcn_readlane(cs, 32 * hh);
        glb_u64* cb = (glb_u64*)buf_of(slot_query(s, hh));
        const uint2 lk = compact_keys_approx(cb, ch, keep, hist_l, kstage_l);
        uint32_t L = lk.x;
        int kept = (int)lk.y;
        if (kept > keep && kept > cap - 3 * TILE) {
          // the threshold's bucket is too full (many equal keys): compact exactly
          L = __float_as_uint(compact_keys_staged(cb, kept, keep, hist_l, kstage_l));
          kept = keep;
        }
        if (half == hh) {
#pragma unroll
          for (int s2 = 0; s2 < NS; ++s2)
            if (s2 == s) {
              cnt[s2] = kept;
              tau[s2] = __uint_as_float(L);
            }
        }
      }
    };
    // The compute waves run a two-stage pipeline over 32-candidate subtiles:
    // the MFMAs of subtile u are issued next to the epilogue (ReLU, head sum,
    // threshold test) of subtile u - 1, which does not depend on them, so
    // the matrix unit and the VALU work side by side. The last subtile of a
    // barrier group is scored after the next barrier, beside the next group's
    // first MFMAs. Accumulator sets alternate: even subtiles write accA, odd
    // ones accB, so a group always ends with its last subtile pending in accB.
    f32x16 accA[AT], accB[AT];
    int cA = 0, cB = 0;    // first candidate of the subtile held in accA / accB
    bool pendB = false;    // accB holds a subtile not yet scored
    bool pending = false;  // this wave must compact before its next group
    // MFMAs of subtile nt (0, 1) of the tile in LDS slot `slot` into acc
    auto mfma_sub = [&](int slot, int nt, f32x16* acc) __attribute__((always_inline)) {
      const unsigned char* sl = ring + slot * TILE_BYTES;
      const int row = nt * 32 + col;
      u32x4 B[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int part = 2 * ks + half;
        B[ks] = *reinterpret_cast<const u32x4*>(sl + row * 128 + ((part ^ (row & 7)) * 16));
      }
#pragma unroll
      for (int a = 0; a < AT; ++a) {
        acc[a] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) acc[a] = mfma32x32x16(A[a][ks], B[ks], acc[a]);
      }
    };
    // Score the subtile at candidate c held in acc and append every candidate
    // that beats its query's threshold to the query's buffer (lanes of one
    // half share a query, so the ballot's half gives the positions). Nothing
    // passes when `live` is false (an empty pipeline stage). Returns whether
    // anything was appended.
    auto epilogue = [&](const f32x16* acc, int c, bool live) __attribute__((always_inline)) -> bool {
      const int j = c + col;
      const bool interior = c + 32 <= minlim;  // every query of the wave sees the whole subtile
      const uint64_t live_mask = live ? ~0ull : 0ull;
      float sc[NS];
      uint64_t m64[NS];
      uint64_t any = 0;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int a = s / QPH, qq = s % QPH;
        float sum = relu_bits(acc[a][qq * HI]);
#pragma unroll
        for (int hd = 1; hd < HI; ++hd) sum += relu_bits(acc[a][qq * HI + hd]);
        sc[s] = SCALE_EPI ? sum * w_epi : sum;
        m64[s] = ballot(sc[s] > tau[s]) & live_mask;
        any |= m64[s];
      }
      if (!any) return false;
      const uint32_t below = (1u << col) - 1u;
      auto append = [&](int s, uint64_t mm, bool pass) {
        if (mm) {
          const uint32_t mh = half ? (uint32_t)(mm >> 32) : (uint32_t)mm;
          if (pass)
            buf_slot(s)[cnt[s] + __popc(mh & below)] =
                (unsigned long long)__float_as_uint(sc[s]) | ((unsigned long long)(uint32_t)j << 32);
          cnt[s] += __popc(mh);
        }
      };
      if (interior) {
#pragma unroll
        for (int s = 0; s < NS; ++s) append(s, m64[s], sc[s] > tau[s]);
      } else {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const bool pass = sc[s] > tau[s] && j < lim[s];
          append(s, ballot(pass), pass);
        }
      }
      return true;
    };
    // Sample phase: each lane keeps, per slot, the four largest scores of the
    // sampled candidates it scored (descending; -1 while empty). Appends nothing.
    float top[NS][4];
#pragma unroll
    for (int s = 0; s < NS; ++s) top[s][0] = top[s][1] = top[s][2] = top[s][3] = -1.0f;
    auto seed_epi = [&](const f32x16* acc, int c, bool live) __attribute__((always_inline)) {
      const int j = c + col;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int a = s / QPH, qq = s % QPH;
        float sum = relu_bits(acc[a][qq * HI]);
#pragma unroll
        for (int hd = 1; hd < HI; ++hd) sum += relu_bits(acc[a][qq * HI + hd]);
        float y = (live && j < lim[s]) ? (SCALE_EPI ? sum * w_epi : sum) : -1.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float hi = fmaxf(top[s][i], y);
          y = fminf(top[s][i], y);
          top[s][i] = hi;
        }
      }
    };
    // One barrier group: TT tiles, 2 TT subtiles (fewer at the end). A
    // compaction one wave asked for while processing the previous group is
    // done by every wave at once, each compacting its buffers past a lower
    // mark (they fill at similar rates): otherwise the waves would wait for
    // each other at the barriers one compaction at a time. The wave that
    // asked compacts for certain (another may already have moved the flag
    // on); for the others the invitation is optional. The pending subtile is
    // scored first, so the buffers hold every candidate before the next one.
    // t: the group's first virtual tile; t0: the first of its scan (split
    // tile 0); left: tiles of the scan from t on (at least one).
    auto process_group = [&](int t, int t0, int left) __attribute__((always_inline)) {
      if (pending || wg_compact == t) {
        if (pendB) epilogue(accB, cB, true);
        pendB = false;
        // only buffers past k - 1 entries: a shorter one still needs every
        // later candidate, so its threshold must stay where it is
        compact_over(max(max(cap - 12 * TILE, cap / 2), keep));
        pending = false;
      }
      const int nsub = 2 * min(TT, left);
      bool appended = false;
#pragma unroll
      for (int u = 0; u < 2 * TT; ++u) {
        if (u < nsub) {
          const int tt = t + (u >> 1);
          const int c = sbeg + (tt - t0) * TILE + (u & 1) * 32;
          if ((u & 1) == 0) {
            mfma_sub(tt % NSLOT, 0, accA);
            cA = c;
            appended |= epilogue(accB, cB, pendB);
            pendB = false;
          } else {
            mfma_sub(tt % NSLOT, 1, accB);
            cB = c;
            appended |= epilogue(accA, cA, true);
            pendB = true;
          }
        }
      }
      // at most 32 appends per buffer per subtile: keep room for the subtiles
      // up to the next compaction point (this group's pending one, the next
      // group's, and that group's pending one, scored before a compaction)
      if (appended) {
        bool over = false;
#pragma unroll
        for (int s = 0; s < NS; ++s) over |= cnt[s] > cap - (TT * TILE + 32);
        if (ballot(over)) {
          pending = true;
          // the next group (all waves read the flag after that group's barrier)
          if (lane == 0) wg_compact = t + TT;
        }
      }
    };
    // A group of the sample phase: the same pipeline, the sample epilogue.
    auto seed_group = [&](int t, int left) __attribute__((always_inline)) {
      const int nsub = 2 * min(TT, left);
#pragma unroll
      for (int u = 0; u < 2 * TT; ++u) {
        if (u < nsub) {
          const int tt = t + (u >> 1);
          const int c = sbeg + tt * rho * TILE + (u & 1) * 32;
          if ((u & 1) == 0) {
            mfma_sub(tt % NSLOT, 0, accA);
            cA = c;
            seed_epi(accB, cB, pendB);
            pendB = false;
          } else {
            mfma_sub(tt % NSLOT, 1, accB);
            cB = c;
            seed_epi(accA, cA, true);
            pendB = true;
          }
        }
      }
    };
    // Iteration t opens with barrier B_t, after which the compute waves process
    // tile t. The copy wave issues tile t + PF right after B_t, into the slot
    // of tile t + PF - NSLOT <= t - 1 (processed before B_t), and before B_t
    // waits until tile t has landed: the memory counter is in order and the
    // 8 loads of each of tiles t + 1 .. t + PF - 1 were issued after it.
    // Loads are issued for every t (past the end they reread the last
    // candidate), so that count holds to the end.
    // With two tiles per barrier (TT = 2) the copy wave issues tiles t + 2 and
    // t + 3 right after B_t, into the slots of tiles t - 2 and t - 1 (processed
    // before B_t), and waits for both before the next barrier.
    // t runs over the virtual tiles of the sample and the scan; after the
    // scan, when seeded, one more barrier (R) tells every wave whether the
    // second scan runs; the tiles the copy wave issued last are already its
    // first ones. Both sides pass the same barriers in the same order.
    if (copier) {
      auto copy_run = [&](int t0, int t1) __attribute__((always_inline)) {
        if constexpr (TT == 1) {
          for (int t = t0; t < t1; ++t) {
            __builtin_amdgcn_s_waitcnt(prefill_vmcnt(8 * (PF - 1)));
            __builtin_amdgcn_s_barrier();
            issue_tile(t + PF);
          }
        } else {
          for (int t = t0; t < t1; t += 2) {
            __builtin_amdgcn_s_waitcnt(prefill_vmcnt(0));
            __builtin_amdgcn_s_barrier();
            issue_tile(t + 2);
            issue_tile(t + 3);
          }
        }
      };
#pragma unroll
      for (int t = 0; t < (TT == 1 ? PF : 2); ++t) issue_tile(t);
      copy_run(0, P1 + P2);
      if (P1 > 0) {
        __builtin_amdgcn_s_waitcnt(prefill_vmcnt(0));
        __syncthreads();  // R
        if (wg_rerun) copy_run(P1 + P2, P1 + 2 * P2);
      }
      __builtin_amdgcn_s_waitcnt(prefill_vmcnt(0));  // no copy into LDS outlives the workgroup
    } else {
      if constexpr (kSample) {
        for (int t = 0; t < n1; t += TT) {  // as far as P1
          __syncthreads();
          seed_group(t, n1 - t);
        }
      }
      uint32_t seeded = 0;  // bit s: slot s starts from a seeded threshold
      if (kSample && P1 > 0) {
        if (pendB) seed_epi(accB, cB, true);
        pendB = false;
        // Seed: with n candidates of this split, S of them sampled, take the
        // m-th largest sampled score, m = ceil(2.5 keep S / n), as a lower
        // estimate of the split's keep-th largest (about 2.5 keep candidates
        // reach it). The m-th largest of the lane-half's 128 kept scores is
        // at most the sample's m-th largest. The buffer takes every candidate
        // at or above it (threshold one float step below). Only for splits of
        // at least 4 keep candidates; m <= 96 of the 128.
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const int n = max(lim[s] - sbeg, 0);
          const int per = TILE * rho;
          const int S = (n / per) * TILE + min(n % per, TILE);
          const int m = (int)(((int64_t)5 * keep * S + 2 * (int64_t)n - 1) / (2 * (int64_t)max(n, 1)));
          // largest key x with at least m of the lane-half's kept scores >= x
          uint32_t x = 0;
          for (int bit = 30; bit >= 0; --bit) {
            const uint32_t tr = x | (1u << bit);
            int c = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const uint64_t bm = ballot(__float_as_int(top[s][i]) >= (int)tr);
              c += __popc(half ? (uint32_t)(bm >> 32) : (uint32_t)bm);
            }
            if (c >= m) x = tr;
          }
          if (n >= 4 * keep && m <= 96) {
            tau[s] = x > 0 ? __uint_as_float(x - 1) : -1.0f;
            seeded |= 1u << s;
          }
        }
      }
      // the scan, and once more if a seeded buffer ended short
      for (int t0 = P1;; t0 += P2) {
        for (int t = t0; t < t0 + ntiles; t += TT) {  // as far as t0 + P2
          __syncthreads();
          process_group(t, t0, t0 + ntiles - t);
        }
        if (pendB) epilogue(accB, cB, true);
        if (P1 == 0 || t0 > P1) break;
        // A seeded buffer holds every candidate at or above its seed until
        // it first compacts (then at least keep entries). One that ended
        // with fewer than keep entries may have missed some of the split's
        // best: its split is scanned again from an unseeded threshold.
        uint32_t short_m = 0;
#pragma unroll
        for (int s = 0; s < NS; ++s)
          if (((seeded >> s) & 1u) && cnt[s] < keep) short_m |= 1u << s;
        if (ballot(short_m != 0) && lane == 0) wg_rerun = 1;
        __syncthreads();  // R
        if (!wg_rerun) break;
        // the other buffers are final: their counts are written now, and
        // they take nothing more
        frozen = ~short_m & ((1u << NS) - 1u);
        if (wave_live && col == 0) {
#pragma unroll
          for (int s = 0; s < NS; ++s) {
            const int qi = slot_query(s, half);
            if (qi < nqb && ((frozen >> s) & 1u)) buf_cnt[((int64_t)b * n_q + qi) * splits + split] = cnt[s];
          }
        }
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          tau[s] = ((short_m >> s) & 1u) ? -1.0f : INFINITY;
          cnt[s] = 0;
        }
        pending = false;
        pendB = false;
        if (tid == 0) wg_compact = -1;  // read after the next barrier
      }
    }
  }
  if (wave_live && col == 0) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int qi = slot_query(s, half);
      if (qi < nqb && !((frozen >> s) & 1u)) buf_cnt[((int64_t)b * n_q + qi) * splits + split] = cnt[s];
    }
  }
}

// One workgroup (256 threads) per query: merge the split buffers in LDS.
__global__ __launch_bounds__(256) void index_select_kernel(
    const uint2* __restrict__ buf, const int* __restrict__ buf_cnt, const int32_t* __restrict__ q_pos0,
    int n_q, int r, int k, int splits, int cap, int32_t* __restrict__ sel,
    int32_t* __restrict__ sel_cnt, const int32_t* __restrict__ cu_q) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t bc[2 + 8];
  __shared__ uint32_t scratch[kSelScratch];
  __shared__ int seg_off[9];
  extern __shared__ uint2 stage[];
  const int tid = threadIdx.x;
  const int64_t gq = blockIdx.x;  // b * n_q + qi
  const int b = (int)(gq / n_q);
  const int qi = (int)(gq % n_q);
  const int64_t row = cu_q ? (int64_t)cu_q[b] + qi : gq;  // output row
  if (cu_q && qi >= cu_q[b + 1] - cu_q[b]) return;  // qi < n_q (rows per sequence at most)
  const int64_t t = (int64_t)q_pos0[b] + qi;
  const int64_t bt = t / r;
  const int keep = (int)((int64_t)(k - 1) < bt ? (int64_t)(k - 1) : bt);
  const uint2* qb = buf + gq * splits * (int64_t)cap;
  const int* qc = buf_cnt + gq * splits;
  int32_t* out = sel + row * k;

  // segment offsets (at most 8 splits, each at most keep entries)
  if (tid == 0) {
    int acc = 0;
    for (int s = 0; s < splits; ++s) {
      seg_off[s] = acc;
      acc += qc[s];
    }
    seg_off[splits] = acc;
  }
  __syncthreads();
  const int total = seg_off[splits];
  for (int s = 0; s < splits; ++s) {
    const int n = seg_off[s + 1] - seg_off[s];
    const uint2* p = qb + (int64_t)s * cap;
    for (int i = tid; i < n; i += 256) stage[seg_off[s] + i] = p[i];
  }
  __syncthreads();
  if (keep > 0) {
    uint32_t tk = 0;
    int need = 0x7FFFFFFF;
    if (total > keep)
      block_select<256>([&](int i) { return stage[i].x; }, total, keep, hist, bc, scratch, kSelScratch, tk, need);
    block_stable_keep<256>([&](int i) { return stage[i]; }, total, tk, need, bc + 2,
                           [&](int pos, uint2 e) { out[pos] = (int32_t)e.y; });
  }
  if (tid == 0) {
    out[keep] = (int32_t)bt;
    sel_cnt[row] = keep + 1;
  }
  for (int i = keep + 1 + tid; i < k; i += 256) out[i] = -1;
}

// ------------------------------------------------------------------ decode --
// Split scan: one workgroup (8 waves) per (split of kDecodeSplit candidates,
// sequence). Each wave scores 256 candidates (8 tiles of 32, 4 in flight) into
// LDS and into the score row (kept for the exact fallback). The workgroup then
// lists, in block order, the split's entries with key >= Ls, where Ls is the
// lower edge of the histogram bucket holding the split's list_min-th largest
// key, searched downwards from the largest key (bins of the distance below
// it, refined 8 bits per pass) until at most list_cap entries remain; only when those are all equal to one key is
// the list cut, in block order. The list goes to list_cap slots with keys
// shifted by one (0 marks an empty slot); meta = {entries, largest key left
// out or -1}.
template <int HI>
__global__ __launch_bounds__(kScanThreads) void index_decode_scan_kernel(
    const uint16_t* __restrict__ idx_q, const uint16_t* __restrict__ cmp_k, int64_t cmp_stride,
    const int32_t* __restrict__ q_pos0, int r, float a_scale, float w_epi, int splits, int list_min,
    int list_cap, float* __restrict__ scores, int64_t score_stride, uint2* __restrict__ local,
    int2* __restrict__ meta) {
  constexpr int NT = kScanThreads;
  constexpr int NW = NT / kWave;
  __shared__ uint32_t hist[256];
  __shared__ uint32_t bc[2 + 2 * NW];
  __shared__ float sc[kDecodeSplit];
  __shared__ uint32_t red[3][NW];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int col = lane & 31;
  const int split = blockIdx.x;
  const int b = blockIdx.y;
  const int64_t bt = (int64_t)q_pos0[b] / r;
  const int sbeg = split * kDecodeSplit;
  const int send = (int)min((int64_t)sbeg + kDecodeSplit, bt);
  const int n = max(send - sbeg, 0);
  uint2* lout = local + ((int64_t)b * splits + split) * list_cap;
  int2* mout = meta + (int64_t)b * splits + split;
  if (n == 0) {
    for (int i = tid; i < list_cap; i += NT) lout[i] = make_uint2(0u, 0u);
    if (tid == 0) *mout = make_int2(0, -1);
    return;
  }
  // A: 32 rows; the query's H_i heads sit at the rows of slot 0 of lane-half 0
  u32x4 A[4];
  {
    const int m = col;
    const int i = 4 * (m >> 3) + (m & 3);
    const int hh = (m >> 2) & 1;
    const bool mine = hh == 0 && i < HI;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (mine) {
        const u32x4 v = ld16(idx_q + ((int64_t)b * HI + i) * 64 + 16 * ks + 8 * half);
        A[ks] = a_scale == 1.0f ? v : scale_bf16x8(v, a_scale);
      } else {
        A[ks] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
  const uint16_t* kb = cmp_k + (int64_t)b * cmp_stride + 8 * half;
  const int last = send - 1;
  float* srow = scores + (int64_t)b * score_stride;
  const int wbeg = wave * 256;  // this wave's 256 candidates
  if (wbeg < n) {
    constexpr int NTILE = 8, PF = 4;  // a ring of 4 tiles in flight
    u32x4 Bq[PF][4];
    auto load = [&](int p) {
      const int j = min(sbeg + wbeg + 32 * p + col, last);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) Bq[p % PF][ks] = ld16(kb + (int64_t)j * 64 + 16 * ks);
    };
#pragma unroll
    for (int p = 0; p < PF; ++p) load(p);
#pragma unroll
    for (int p = 0; p < NTILE; ++p) {
      f32x16 acc = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) acc = mfma32x32x16(A[ks], Bq[p % PF][ks], acc);
      if (p + PF < NTILE) load(p + PF);
      float sum = 0.0f;
#pragma unroll
      for (int hd = 0; hd < HI; ++hd) sum += relu_bits(acc[hd]);
      const int jj = wbeg + 32 * p + col;
      if (half == 0 && jj < n) {
        const float sv = sum * w_epi;
        sc[jj] = sv;
        srow[sbeg + jj] = sv;
      }
    }
  }
  // The list threshold is searched downwards from the split's largest key:
  // a pass counts the keys whose distance below the maximum falls into a
  // window of 256 bins of 2^s key steps (keys further down are not counted,
  // so the few keys near the top are all the pass touches), finds the bin
  // holding the list_min-th largest, and refines inside it 8 bits at a time
  // until at most list_cap keys lie at or above its lower edge. A first
  // window too narrow to hold list_min keys is widened 256-fold.
  uint32_t kmax = 0u;
  __syncthreads();
  for (int i = tid; i < n; i += NT) kmax = max(kmax, __float_as_uint(sc[i]));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, off));
  if (lane == 0) red[1][wave] = kmax;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < NW; ++w) kmax = max(kmax, red[1][w]);
  uint32_t need = (uint32_t)min(list_min, n);
  uint32_t above_all = 0, ge = (uint32_t)n;
  uint32_t Ls = 0u;
  uint64_t wlo = 0;  // distance of the window's first bin
  int s = 14;
  bool done = n <= list_cap;
  while (!done) {
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += NT) {
      const uint64_t dist = (uint64_t)(kmax - __float_as_uint(sc[i]));
      if (dist >= wlo) {
        const uint64_t d = (dist - wlo) >> s;
        if (d < 256) atomicAdd(&hist[255 - (int)d], 1u);  // larger keys, larger digits
      }
    }
    __syncthreads();
    if (tid < kWave) {
      const int top = 255 - 4 * lane;
      uint32_t tot = hist[top] + hist[top - 1] + hist[top - 2] + hist[top - 3];
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) tot += __shfl_xor(tot, off);
      int dig = 0;
      uint32_t above = 0;
      if (tot >= need) wave_find_digit(hist, need, dig, above);
      if (tid == 0) {
        bc[0] = (uint32_t)dig;
        bc[1] = above;
        bc[2] = hist[dig];
        bc[3] = tot;
      }
    }
    __syncthreads();
    if (bc[3] < need) {  // only the first window can be short
      s += 8;
      continue;
    }
    const uint64_t db = 255u - bc[0];
    need -= bc[1];
    above_all += bc[1];
    ge = above_all + bc[2];
    const uint64_t dist_hi = wlo + ((db + 1) << s) - 1;  // the bucket's lowest key
    Ls = dist_hi >= kmax ? 0u : kmax - (uint32_t)dist_hi;
    if (ge <= (uint32_t)list_cap || s == 0) {
      done = true;
    } else {
      wlo += db << s;
      s = s >= 8 ? s - 8 : 0;
    }
  }
  // all entries >= Ls, or (many equal keys) the first slots' worth of them
  const int take = ge <= (uint32_t)list_cap ? 0x7FFFFFFF : list_cap - (int)above_all;
  const int kept = block_stable_keep<NT>(
      [&](int i) { return make_uint2(__float_as_uint(sc[i]), (uint32_t)(sbeg + i)); }, n, Ls, take, bc + 2,
      [&](int pos, uint2 e) { lout[pos] = make_uint2(e.x + 1u, e.y); });
  for (int i = kept + tid; i < list_cap; i += NT) lout[i] = make_uint2(0u, 0u);
  // largest key left out: Ls itself when equal keys were cut, else the
  // largest key below Ls
  int below = -1;
  if (take == 0x7FFFFFFF) {
    for (int i = tid; i < n; i += NT) {
      const uint32_t key = __float_as_uint(sc[i]);
      if (key < Ls) below = max(below, (int)key);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) below = max(below, __shfl_xor(below, off));
  } else {
    below = (int)Ls;
  }
  if (lane == 0) red[2][wave] = (uint32_t)below;
  __syncthreads();
  if (tid == 0) {
    int b_all = -1;
#pragma unroll
    for (int w = 0; w < NW; ++w) b_all = max(b_all, (int)red[2][w]);
    *mout = make_int2(kept, b_all);
  }
}

// Merge: one workgroup (1024 threads) per sequence. The split lists are
// staged slot by slot (block order; empty slots have key 0, the others their
// key plus one) and the top `keep` of their union is selected exactly. It is
// the exact top `keep` of all candidates when every key left out of a list is
// below the selected threshold; otherwise the stored scores of all
// candidates are selected instead.
__global__ __launch_bounds__(kMergeThreads) void index_decode_select_kernel(
    const float* __restrict__ scores, int64_t score_stride, const uint2* __restrict__ local,
    const int2* __restrict__ meta, const int32_t* __restrict__ q_pos0, int r, int k, int splits,
    int list_cap, int32_t* __restrict__ sel, int32_t* __restrict__ sel_cnt) {
  constexpr int NT = kMergeThreads;
  __shared__ uint32_t hist[256];
  __shared__ uint32_t bc[2 + 2 * (NT / kWave)];
  __shared__ uint32_t scratch[kSelScratch];
  __shared__ int red_max[NT / kWave], red_tot[NT / kWave];
  extern __shared__ uint2 stage[];
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int64_t bt = (int64_t)q_pos0[b] / r;
  const int keep = (int)((int64_t)(k - 1) < bt ? (int64_t)(k - 1) : bt);
  int32_t* out = sel + (int64_t)b * k;
  const int used = (int)min((int64_t)splits, (bt + kDecodeSplit - 1) / kDecodeSplit);
  const uint2* lb = local + (int64_t)b * splits * list_cap;
  const int2* mb = meta + (int64_t)b * splits;
  // the splits' (count, largest omitted key), reduced per wave then over waves
  int mx = -1, tot = 0;
  for (int s2 = tid; s2 < used; s2 += NT) {
    const int2 m = mb[s2];
    mx = max(mx, m.y);
    tot += m.x;
  }
  const int slots = used * list_cap;
#pragma unroll 8
  for (int i = tid; i < slots; i += NT) stage[i] = lb[i];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    mx = max(mx, __shfl_xor(mx, off));
    tot += __shfl_xor(tot, off);
  }
  if ((tid & (kWave - 1)) == 0) {
    red_max[tid / kWave] = mx;
    red_tot[tid / kWave] = tot;
  }
  __syncthreads();
  int max_omitted = -1, total = 0;
#pragma unroll
  for (int w = 0; w < NT / kWave; ++w) {
    max_omitted = max(max_omitted, red_max[w]);
    total += red_tot[w];
  }
  if (keep > 0) {
    uint32_t tk = 1u;  // shifted: every listed entry
    int need = 0x7FFFFFFF;
    bool exact;
    if (total >= keep) {
      block_select<NT, true>([&](int i) { return stage[i].x; }, slots, keep, hist, bc, scratch, kSelScratch, tk,
                             need);
      exact = max_omitted < 0 || (uint32_t)max_omitted < tk - 1u;
    } else {
      exact = max_omitted < 0;  // the lists hold every candidate
    }
    if (exact) {
      block_stable_keep<NT>([&](int i) { return stage[i]; }, slots, tk, need, bc + 2,
                            [&](int pos, uint2 e) { out[pos] = (int32_t)e.y; });
    } else {
      // exact selection over the stored scores of every candidate
      const float* srow = scores + (int64_t)b * score_stride;
      const int n = (int)bt;
      tk = 0;
      need = 0x7FFFFFFF;
      block_select<NT>([&](int i) { return __float_as_uint(srow[i]); }, n, keep, hist, bc, scratch, kSelScratch,
                       tk, need);
      block_stable_keep<NT>([&](int i) { return make_uint2(__float_as_uint(srow[i]), (uint32_t)i); }, n, tk,
                            need, bc + 2, [&](int pos, uint2 e) { out[pos] = (int32_t)e.y; });
    }
  }
  if (tid == 0) {
    out[keep] = (int32_t)bt;
    sel_cnt[b] = keep + 1;
  }
  for (int i = keep + 1 + tid; i < k; i += NT) out[i] = -1;
}

// ----------------------------------------------------------------- planning --
static bool pow2_float(float w) {
  int e;
  const float m = frexpf(w, &e);
  return m == 0.5f;
}

IndexPlan plan_index(int hi, int k, int batch, int n_q, int64_t max_q_end, int r, bool allow_decode) {
  IndexPlan p{};
  p.hi = hi;
  const int64_t max_cand = max_q_end > 0 ? (max_q_end - 1) / r : 0;
  p.max_cand = max_cand;
  const int keep = k - 1;
  const int64_t dsplits = (max_cand + kDecodeSplit - 1) / kDecodeSplit;
  // list sizes: a split of the full range holds on average mu of the top
  // `keep`; lists take at least mu + 4 sqrt(mu) + 8 entries (so that the
  // merge rarely needs the exact fallback) and have half as much room again
  const double mu = max_cand > 0 ? (double)keep * (double)kDecodeSplit / (double)max_cand : 0.0;
  int lmin = (int)ceil(mu + 4.0 * sqrt(mu) + 8.0);
  if (lmin > keep + 8) lmin = keep + 8;
  lmin = (lmin + 7) / 8 * 8;
  if (lmin < 16) lmin = 16;
  if (lmin > 1024) lmin = 1024;
  const int lcap = (lmin + max(16, lmin / 2) + 7) / 8 * 8;
  const int64_t nsplit = dsplits < 1 ? 1 : dsplits;
  if (allow_decode && n_q == 1 && nsplit <= kDecodeMaxSplits &&
      (size_t)nsplit * lcap * sizeof(uint2) <= kMergeMaxLds) {
    p.decode = true;
    p.splits = (int)nsplit;
    p.list_min = lmin;
    p.list_cap = lcap;
    p.score_stride = (max_cand + 63) / 64 * 64;
    const size_t sc = (size_t)batch * p.score_stride * sizeof(float);
    const size_t lc = (size_t)batch * p.splits * p.list_cap * sizeof(uint2);
    const size_t mc = (size_t)batch * p.splits * sizeof(int2);
    p.buf_bytes = (sc + 255) / 256 * 256;
    p.local_off = p.buf_bytes;
    p.meta_off = p.local_off + (lc + 255) / 256 * 256;
    p.workspace = p.meta_off + (mc + 255) / 256 * 256;
    p.select_lds = (size_t)p.splits * p.list_cap * sizeof(uint2);
    return p;
  }
  p.decode = false;
  p.wide = n_q >= 64;
  // A tiles per wave in the LDS-pipelined kernel: two at 8 and 16 heads (8 and
  // 4 queries per wave), one otherwise (32 / H_i queries).
  p.at = p.wide ? (hi >= 8 ? 2 : 1) : 1;
  // Compute waves per workgroup (plus one copy wave). The pipelined scan
  // keeps two accumulator sets, ~160 VGPRs at two A tiles: one 9-wave
  // workgroup per CU (168 VGPRs at most), which for a uniform batch of 8-head
  // queries at 1M fills each CU once. A packed batch of unequal sequences runs
  // many workgroups of unequal length over several rounds; there three 4-wave
  // workgroups per CU (3 compute waves each) keep more of them in flight. At 4
  // heads one A tile (~120 VGPRs) lets two 5-wave workgroups share a CU (at
  // most 128 VGPRs and 64 KiB of LDS each: a 5-wave workgroup puts two waves
  // on one SIMD, and the second workgroup's land on the same SIMD).
  p.nw = hi == 8 ? (allow_decode ? 8 : 3) : (hi == 4 ? 4 : 8);
  p.qw = p.at * 32 / hi;
  p.n_qgroups = (n_q + p.qw - 1) / p.qw;
  int64_t splits;
  if (p.wide) {
    // workgroups of kPrefillWaves query groups; about one workgroup per CU in one round.
    // A packed batch (allow_decode false) sizes n_q for its longest sequence
    // and most other workgroups are empty: size the splits for one sequence.
    const int64_t n_wg = ((int64_t)p.n_qgroups + p.nw - 1) / p.nw;
    const int64_t busy = allow_decode ? batch * n_wg : n_wg;
    const int64_t slots = p.nw == 4 ? 512 : (p.nw == 3 ? 768 : 256);  // workgroups the GPU holds at once
    splits = (slots + busy - 1) / busy;
    const int64_t max_splits = (max_cand + 1023) / 1024;
    if (splits > max_splits) splits = max_splits;
  } else {
    const int64_t waves = (int64_t)batch * p.n_qgroups;
    splits = (4096 + waves - 1) / waves;
    const int64_t max_splits = (max_cand + 255) / 256;
    if (splits > max_splits) splits = max_splits;
  }
  if (splits > 8) splits = 8;
  if (splits < 1) splits = 1;
  int64_t split_len = (max_cand + splits - 1) / splits;
  split_len = (split_len + 63) / 64 * 64;
  if (split_len < 64) split_len = 64;
  p.splits = (int)splits;
  p.split_len = (int)split_len;
  // Buffer entries per (query, split). The many-query kernel stages a whole
  // buffer in its wave's LDS to compact it (8 bytes per entry), so the
  // capacity follows the LDS left per wave: 1792 at 8 compute waves (one
  // workgroup per CU), 1280 at 4 (two per CU), 1024 at 3 (three per CU). It
  // must exceed k - 1 by room for a compaction interval (kept entries stay
  // below cap - 192, see the exact fallback) and a margin; a split shorter
  // than the capacity never needs more than its candidates. A multiple of 128:
  // staging copies whole 128-entry pieces.
  int cap = p.wide ? (p.nw == 8 ? 1792 : (p.nw == 4 ? 1280 : 1024)) : 2048;
  if (!p.wide && cap < 2 * keep + 64) cap = 2 * keep + 64;
  if (cap < keep + 448) cap = keep + 448;
  if ((int64_t)split_len + 64 <= cap) cap = (int)split_len + 64;
  cap = (cap + 127) / 128 * 128;
  p.cap = cap;
  // Seeded thresholds in the many-query kernel: every rho-th tile of a split
  // is scored first, rho the smallest power of two with 2.5 keep / rho <= 96
  // (the seed is the m-th largest of at most 128 kept sample scores per
  // query, m about 2.5 keep / rho); only where rho >= 16, so that the sample
  // adds at most 1/16 to the scoring.
  p.seed_stride = 0;
  if (p.wide && hi >= 2) {  // the kernel takes no sample at one head
    int rho = 1;
    while (5 * keep > 192 * rho) rho *= 2;
    if (rho >= 16) p.seed_stride = rho;
  }
  p.buf_bytes = (size_t)batch * n_q * p.splits * (size_t)cap * sizeof(uint2);
  p.cnt_bytes = (size_t)batch * n_q * p.splits * sizeof(int);
  p.workspace = p.buf_bytes + ((p.cnt_bytes + 255) / 256 * 256);
  // LDS per workgroup: each wave's compaction stage of cap entries (nw waves
  // in the wide kernel, 4 in the other)
  p.stream_lds = (size_t)(p.wide ? p.nw : 4) * cap * sizeof(uint2);
  // the wide kernel leaves up to `cap` entries per split; the other at most `keep`
  p.select_lds = (size_t)p.splits * (p.wide ? cap : (keep > 0 ? keep : 1)) * sizeof(uint2);
  return p;
}

// Device limits the plans are checked against (MI355X / gfx950).
constexpr int64_t kMaxGridX = 0x7FFFFFFF, kMaxGridYZ = 65535;
constexpr size_t kMaxLds = 160 * 1024;

// Upper bounds of the kernels' static LDS (their __shared__ arrays, plus
// alignment slack).
constexpr size_t kLdsSlack = 64;
constexpr size_t prefill_static_lds(int nw) {
  return (size_t)(nw == 3 ? 3 : 4) * 64 * 128 + (size_t)nw * (256 * 4 + 4) + 8 + kLdsSlack;
}
constexpr size_t kStreamStaticLds = 4 * 256 * 4 + kLdsSlack;
constexpr size_t kSelectStaticLds = (256 + 10 + kSelScratch + 9) * 4 + kLdsSlack;
constexpr size_t kDecodeScanStaticLds =
    (256 + 2 + 2 * (kScanThreads / kWave) + kDecodeSplit + 3 * (kScanThreads / kWave)) * 4 + kLdsSlack;
constexpr size_t kDecodeSelectStaticLds =
    (256 + 2 + 2 * (kMergeThreads / kWave) + kSelScratch + 2 * (kMergeThreads / kWave)) * 4 + kLdsSlack;

static PlanCheck finish_check(PlanCheck c) {
  c.unfit = nullptr;
  for (int i = 0; i < c.n; ++i) {
    const LaunchShape& l = c.l[i];
    if (l.grid[0] < 1 || (int64_t)l.grid[0] > kMaxGridX || l.grid[1] > kMaxGridYZ || l.grid[2] > kMaxGridYZ ||
        l.grid[1] < 1 || l.grid[2] < 1)
      c.unfit = "a launch grid exceeds the device's limits";
    else if (l.block > 1024)
      c.unfit = "a workgroup exceeds 1024 threads";
    else if (l.lds > kMaxLds)
      c.unfit = "a workgroup exceeds 160 KiB of LDS";
  }
  if (!c.unfit && c.max_i32 >= ((int64_t)1 << 31)) c.unfit = "a kernel index would exceed 32 bits";
  if (!c.unfit && c.max_offset >= ((int64_t)1 << 62)) c.unfit = "a workspace offset would exceed 2^62";
  return c;
}

static uint32_t grid_dim(int64_t v) { return v > 0xFFFFFFFFll ? 0xFFFFFFFFu : (uint32_t)v; }

PlanCheck check_index_plan(const IndexPlan& p, int batch, int n_q) {
  PlanCheck c{};
  if (p.decode) {
    c.n = 2;
    c.l[0] = LaunchShape{{grid_dim(p.splits), grid_dim(batch), 1}, (uint32_t)kScanThreads, kDecodeScanStaticLds};
    c.l[1] = LaunchShape{{grid_dim(batch), 1, 1}, (uint32_t)kMergeThreads, kDecodeSelectStaticLds + p.select_lds};
    c.max_i32 = std::max<int64_t>({(int64_t)p.splits * kDecodeSplit, p.max_cand, (int64_t)p.splits * p.list_cap,
                                   (int64_t)batch});
    c.max_offset = std::max<int64_t>((int64_t)batch * p.score_stride,
                                     (int64_t)batch * p.splits * (int64_t)p.list_cap);
    return finish_check(c);
  }
  c.n = 2;
  if (p.wide) {
    c.l[0] = LaunchShape{{grid_dim(((int64_t)p.n_qgroups + p.nw - 1) / p.nw), grid_dim(p.splits), grid_dim(batch)},
                         (uint32_t)(64 * (p.nw + 1)), prefill_static_lds(p.nw) + p.stream_lds};
  } else {
    c.l[0] = LaunchShape{{grid_dim(((int64_t)p.n_qgroups * p.splits + 3) / 4), grid_dim(batch), 1}, 256u,
                         kStreamStaticLds + p.stream_lds};
  }
  c.l[1] = LaunchShape{{grid_dim((int64_t)batch * n_q), 1, 1}, 256u, kSelectStaticLds + p.select_lds};
  c.max_i32 = std::max<int64_t>({(int64_t)n_q + p.qw, (int64_t)p.n_qgroups * p.splits,
                                 p.max_cand + p.split_len + 64 * ((int64_t)p.seed_stride + 2),
                                 (int64_t)p.splits * p.cap});
  c.max_offset = (int64_t)batch * n_q * p.splits * (int64_t)p.cap;
  return finish_check(c);
}

hipError_t launch_index_topk(const IndexPlan& p, const uint16_t* idx_q, const uint16_t* cmp_k,
                             int64_t cmp_stride, const int32_t* q_pos0, int batch, int n_q, int r,
                             int k, float w, int32_t* sel, int32_t* sel_cnt, void* ws,
                             hipStream_t stream, const int32_t* cu_q) {
  const bool exact_scale = pow2_float(w);
  const float a_scale = exact_scale ? w : 1.0f;
  const float w_epi = exact_scale ? 1.0f : w;
  char* wsb = reinterpret_cast<char*>(ws);
  if (p.decode) {
    float* scores = reinterpret_cast<float*>(wsb);
    uint2* local = reinterpret_cast<uint2*>(wsb + p.local_off);
    int2* meta = reinterpret_cast<int2*>(wsb + p.meta_off);
    const dim3 g1(p.splits, batch);
#define QSA_LAUNCH_DSCAN(HI_)                                                                      \
  hipLaunchKernelGGL(index_decode_scan_kernel<HI_>, g1, dim3(kScanThreads), 0, stream, idx_q,    \
                     cmp_k, cmp_stride, q_pos0, r, a_scale, w_epi, p.splits, p.list_min, p.list_cap,  \
                     scores, p.score_stride, local, meta)
    switch (p.hi) {
      case 1: QSA_LAUNCH_DSCAN(1); break;
      case 2: QSA_LAUNCH_DSCAN(2); break;
      case 4: QSA_LAUNCH_DSCAN(4); break;
      case 8: QSA_LAUNCH_DSCAN(8); break;
      case 16: QSA_LAUNCH_DSCAN(16); break;
      default: return hipErrorInvalidValue;
    }
#undef QSA_LAUNCH_DSCAN
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(index_decode_select_kernel, dim3(batch), dim3(kMergeThreads), p.select_lds, stream,
                       scores, p.score_stride, local, meta, q_pos0, r, k, p.splits, p.list_cap, sel, sel_cnt);
    return hipGetLastError();
  }
  uint2* buf = reinterpret_cast<uint2*>(wsb);
  int* cnt = reinterpret_cast<int*>(wsb + p.buf_bytes);
  if (p.wide) {
    const dim3 g1((p.n_qgroups + p.nw - 1) / p.nw, p.splits, batch);
#define QSA_LAUNCH_PREFILL(HI_, AT_, NW_)                                                           \
  hipLaunchKernelGGL((exact_scale ? index_prefill_kernel<HI_, AT_, false, NW_>                   \
                                  : index_prefill_kernel<HI_, AT_, true, NW_>), g1, dim3(64 * (NW_ + 1)), p.stream_lds, \
                     stream, idx_q, cmp_k,                                                         \
                     cmp_stride, q_pos0, n_q, r, k - 1, a_scale, w_epi, p.n_qgroups, p.splits,     \
                     p.split_len, p.cap, p.seed_stride, buf, cnt, cu_q)
    switch (p.hi) {
      case 1: QSA_LAUNCH_PREFILL(1, 1, 8); break;
      case 2: QSA_LAUNCH_PREFILL(2, 1, 8); break;
      case 4: QSA_LAUNCH_PREFILL(4, 1, 4); break;
      case 8: if (p.nw == 3) QSA_LAUNCH_PREFILL(8, 2, 3); else QSA_LAUNCH_PREFILL(8, 2, 8); break;
      case 16: QSA_LAUNCH_PREFILL(16, 2, 8); break;
      default: return hipErrorInvalidValue;
    }
#undef QSA_LAUNCH_PREFILL
  } else {
    const int tasks = p.n_qgroups * p.splits;
    const dim3 g1((tasks + 3) / 4, batch);
#define QSA_LAUNCH_STREAM(HI_)                                                                     \
  hipLaunchKernelGGL((index_stream_kernel<HI_, 1>), g1, dim3(256), p.stream_lds, stream, idx_q,    \
                     cmp_k, cmp_stride, q_pos0, n_q, r, k - 1, a_scale, w_epi, p.n_qgroups,        \
                     p.splits, p.split_len, p.cap, buf, cnt, cu_q)
    switch (p.hi) {
      case 1: QSA_LAUNCH_STREAM(1); break;
      case 2: QSA_LAUNCH_STREAM(2); break;
      case 4: QSA_LAUNCH_STREAM(4); break;
      case 8: QSA_LAUNCH_STREAM(8); break;
      case 16: QSA_LAUNCH_STREAM(16); break;
      default: return hipErrorInvalidValue;
    }
#undef QSA_LAUNCH_STREAM
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t nw = (int64_t)batch * n_q;
  hipLaunchKernelGGL(index_select_kernel, dim3((unsigned)nw), dim3(256), p.select_lds, stream, buf, cnt,
                     q_pos0, n_q, r, k, p.splits, p.cap, sel, sel_cnt, cu_q);
  return hipGetLastError();
}

}  // namespace qsa
