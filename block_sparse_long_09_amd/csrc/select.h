// Exact rank selection building blocks (wave and workgroup level).
//
// Keys are uint32: the bit patterns of non-negative fp32 scores, which order
// like the scores. "Select" finds tk, the keep-th largest key, and `need`, how
// many entries equal to tk belong to the top `keep` (the first ones in list
// order). Radix select on the offset key - kmin, where kmin and kmax are the
// smallest and largest key: the offsets' leading zero bits are skipped, and
// the rest are resolved most-significant first, 8 per pass, with a 256-bin LDS
// histogram, so even the first pass spreads the keys over the bins (fp32
// keys of similar magnitude share their top bits, and keys on both sides of
// a power of two differ in bit 30, so a plain bit prefix would not). "Stable
// keep" then emits, in list order, every entry with key > tk
// and the first `need` entries with key == tk; lists are kept in increasing
// block index, so this realises the (score desc, index asc) order exactly.
#pragma once

#include "qsa_device.h"

namespace qsa {

// One wave reads the histogram and finds the digit where the count from the
// top reaches `need`; `above` is the count of strictly larger digits.
template <typename HistPtr>
__device__ __forceinline__ void wave_find_digit(HistPtr hist, uint32_t need, int& dig, uint32_t& above) {
  const int lane = lane_id();
  const int top = 255 - 4 * lane;  // lane 0 owns the largest digits
  const uint32_t c0 = hist[top], c1 = hist[top - 1], c2 = hist[top - 2], c3 = hist[top - 3];
  const uint32_t tot = c0 + c1 + c2 + c3;
  uint32_t inc = tot;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const uint32_t v = __shfl_up(inc, off);
    if (lane >= off) inc += v;
  }
  const uint32_t exc = inc - tot;
  const bool hit = inc >= need && exc < need;
  const int L = __ffsll((unsigned long long)ballot(hit)) - 1;
  int d = 0;
  uint32_t cum = exc;
  if (cum + c0 >= need) {
    d = top;
  } else {
    cum += c0;
    if (cum + c1 >= need) {
      d = top - 1;
    } else {
      cum += c1;
      if (cum + c2 >= need) {
        d = top - 2;
      } else {
        cum += c2;
        d = top - 3;
      }
    }
  }
  dig = __shfl(d, L);
  above = __shfl(cum, L);
}

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Width in bits of the offset range [0, kmax - kmin].
__device__ __forceinline__ int range_bits(uint32_t kmin, uint32_t kmax) {
  return kmax == kmin ? 0 : 32 - __builtin_clz(kmax - kmin);
}

// Histogram digit of key k for the range [base, base + 2^w), digit bits
// [lo, w) of the offset; -1 when k is outside the range. Keys are below 2^31
// (non-negative fp32 bit patterns), so a key below base wraps to an offset of
// at least 2^31, out of every range.
__device__ __forceinline__ int range_digit(uint32_t k, uint32_t base, int w, int lo) {
  const uint32_t d = (k - base) >> lo;  // wraps to a large value below base
  return d < (1u << (w - lo)) ? (int)d : -1;
}

// Wave-level select over n keys given by key(i) (cheap to read, e.g. LDS).
template <typename KeyFn, typename HistPtr>
__device__ void wave_select(KeyFn key, int n, int keep, HistPtr hist, uint32_t& tk, int& need_out,
                            uint32_t* ties_out = nullptr) {
  const int lane = lane_id();
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  for (int i = lane; i < n; i += kWave) {
    const uint32_t k = key(i);
    kmin = min(kmin, k);
    kmax = max(kmax, k);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, off));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, off));
  }
  uint32_t base = kmin;
  int w = range_bits(kmin, kmax);
  uint32_t need = (uint32_t)keep;
  uint32_t ties = (uint32_t)n;  // every key equals kmin when the range is empty
  while (w > 0) {
    const int lo = w > 8 ? w - 8 : 0;
    for (int i = lane; i < 256; i += kWave) hist[i] = 0;
    wave_sync();
    // eight keys per lane read before their eight atomics (one read-then-add
    // per key would wait out the read latency once per key)
    for (int b0 = 0; b0 < n; b0 += 8 * kWave) {
      uint32_t kk[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = b0 + u * kWave + lane;
        kk[u] = i < n ? key(i) : 0u;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int d = b0 + u * kWave + lane < n ? range_digit(kk[u], base, w, lo) : -1;
        if (d >= 0) __atomic_fetch_add(&hist[d], 1u, __ATOMIC_RELAXED);
      }
    }
    wave_sync();
    int dig;
    uint32_t above;
    wave_find_digit(hist, need, dig, above);
    if (lo == 0) ties = hist[dig];
    base += (uint32_t)dig << lo;
    need -= above;
    w = lo;
    wave_sync();
  }
  tk = base;
  need_out = (int)need;
  if (ties_out) *ties_out = ties;
}

// Wave-level stable keep over entries get(i), i < n, emitting emit(pos, e).
template <typename GetFn, typename EmitFn>
__device__ int wave_stable_keep(GetFn get, int n, uint32_t tk, int need, EmitFn emit) {
  const int lane = lane_id();
  int kept = 0, ties = 0;
  for (int base = 0; base < n; base += kWave) {
    const int i = base + lane;
    const bool in = i < n;
    const uint2 e = in ? get(i) : make_uint2(0u, 0u);
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
  return kept;
}

// Workgroup-level (NT threads) select. LDS: hist 256 bins, bc 3 words,
// scratch `scratch_cap` keys. One radix pass over all n keys finds the bucket
// of the keep-th largest; when the bucket holds at most scratch_cap keys they
// are gathered into scratch and the first wave finishes the selection alone
// (a few short passes, no workgroup barriers); otherwise workgroup passes
// continue. SKIP_ZERO leaves keys equal to 0 out of the key range (they mark
// empty slots and must never be the keep-th largest).
template <int NT, bool SKIP_ZERO = false, typename KeyFn>
__device__ void block_select(KeyFn key, int n, int keep, uint32_t* hist, uint32_t* bc, uint32_t* scratch,
                             int scratch_cap, uint32_t& tk, int& need_out) {
  constexpr int NW = NT / kWave;
  const int tid = threadIdx.x;
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  for (int i = tid; i < n; i += NT) {
    const uint32_t k = key(i);
    if (!SKIP_ZERO || k != 0u) kmin = min(kmin, k);
    kmax = max(kmax, k);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, off));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, off));
  }
  __syncthreads();  // hist may still be read by a previous call
  if (lane_id() == 0) {
    hist[tid / kWave] = kmin;
    hist[NW + tid / kWave] = kmax;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    kmin = min(kmin, hist[w]);
    kmax = max(kmax, hist[NW + w]);
  }
  if (kmin > kmax) kmin = kmax;  // every key skipped
  uint32_t base = kmin;
  int w = range_bits(kmin, kmax);
  uint32_t need = (uint32_t)keep;
  while (w > 0) {
    const int lo = w > 8 ? w - 8 : 0;
    __syncthreads();
    for (int i = tid; i < 256; i += NT) hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += NT) {
      const int d = range_digit(key(i), base, w, lo);
      if (d >= 0) atomicAdd(&hist[d], 1u);
    }
    __syncthreads();
    if (tid < kWave) {
      int dig;
      uint32_t above;
      wave_find_digit(hist, need, dig, above);
      if (tid == 0) {
        bc[0] = (uint32_t)dig;
        bc[1] = above;
        bc[2] = hist[dig];
      }
    }
    __syncthreads();
    base += bc[0] << lo;
    need -= bc[1];
    w = lo;
    const uint32_t in_bucket = bc[2];
    if (w > 0 && in_bucket <= (uint32_t)scratch_cap) {
      // gather the bucket [base, base + 2^w) and finish in one wave
      __syncthreads();
      if (tid == 0) bc[2] = 0;
      __syncthreads();
      for (int i = tid; i < n; i += NT) {
        const uint32_t k = key(i);
        if (range_digit(k, base, w, 0) >= 0) scratch[atomicAdd(&bc[2], 1u)] = k;
      }
      __syncthreads();
      if (tid < kWave) {
        uint32_t t2;
        int n2;
        wave_select([&](int i) { return scratch[i]; }, (int)in_bucket, (int)need, hist, t2, n2);
        if (tid == 0) {
          bc[0] = t2;
          bc[1] = (uint32_t)n2;
        }
      }
      __syncthreads();
      base = bc[0];
      need = bc[1];
      w = 0;
    }
  }
  __syncthreads();
  tk = base;
  need_out = (int)need;
}

// Workgroup-level stable keep: thread t handles the consecutive entries
// [t * ipt, (t + 1) * ipt); one exclusive scan of its (> tk, == tk) counts
// gives every thread its output position. cnt: 2 * (NT / 64) words of LDS.
template <int NT, typename GetFn, typename EmitFn>
__device__ int block_stable_keep(GetFn get, int n, uint32_t tk, int need, uint32_t* cnt, EmitFn emit) {
  constexpr int NW = NT / kWave;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int w = tid / kWave;
  const int ipt = (n + NT - 1) / NT;
  const int i0 = min(tid * ipt, n), i1 = min(i0 + ipt, n);
  int gt = 0, eq = 0;
  for (int i = i0; i < i1; ++i) {
    const uint32_t k = get(i).x;
    gt += k > tk;
    eq += k == tk;
  }
  int gi = gt, ei = eq;  // inclusive scans within the wave
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int g2 = __shfl_up(gi, off), e2 = __shfl_up(ei, off);
    if (lane >= off) {
      gi += g2;
      ei += e2;
    }
  }
  __syncthreads();  // cnt may still be read by a previous call
  if (lane == kWave - 1) {
    cnt[w] = (uint32_t)gi;
    cnt[NW + w] = (uint32_t)ei;
  }
  __syncthreads();
  int g_before = gi - gt, e_before = ei - eq, g_all = 0, e_all = 0;
#pragma unroll
  for (int v = 0; v < NW; ++v) {
    const int gv = (int)cnt[v], ev = (int)cnt[NW + v];
    if (v < w) {
      g_before += gv;
      e_before += ev;
    }
    g_all += gv;
    e_all += ev;
  }
  int pos = g_before + min(e_before, need);
  int er = e_before;
  for (int i = i0; i < i1; ++i) {
    const uint2 e = get(i);
    const bool is_eq = e.x == tk;
    if (e.x > tk || (is_eq && er < need)) emit(pos++, e);
    er += is_eq;
  }
  return g_all + min(e_all, need);
}

}  // namespace qsa
