// Workgroup-level building blocks for 1024-thread workgroups (16 waves of 64):
// flag scans in index order, integer reductions, an MSB-first radix select of
// the k-th largest 64-bit key, and a stable LSD radix sort (descending) of
// (key, index) lists.  Wave-level work uses ballots; cross-wave work goes
// through LDS.  Every function must be reached by all 1024 threads.
#pragma once

#include "internal.h"

namespace twinkv {

constexpr int kBT = 1024;
constexpr int kBW = kBT / 64;

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }
__device__ __forceinline__ uint64_t lanes_below() { return (1ull << lane_id()) - 1ull; }

// fp64 -> unsigned key with the same order (-0.0 and +0.0 map together)
__device__ __forceinline__ uint64_t ordered_bits(double x) {
  x += 0.0;
  const uint64_t u = (uint64_t)__double_as_longlong(x);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

struct ScanSmem {
  int wave[kBW];
};

// Exclusive prefix (in thread order) of 0/1 flags over the workgroup; the
// workgroup total goes to *total.
__device__ __forceinline__ int block_scan_flag(bool f, ScanSmem& s, int* total) {
  const uint64_t m = __ballot(f);
  const int pre = __popcll(m & lanes_below());
  if (lane_id() == 0) s.wave[wave_id()] = __popcll(m);
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kBW; ++w) {
    const int v = s.wave[w];
    off += (w < wave_id()) ? v : 0;
    tot += v;
  }
  __syncthreads();
  *total = tot;
  return off + pre;
}

struct ScanSmem2 {
  int wave[2][kBW];
};

// Both exclusive prefixes of two 0/1 flags in one round of barriers.
__device__ __forceinline__ void block_scan_flag2(bool f0, bool f1, ScanSmem2& s, int* pre0, int* pre1, int* tot0,
                                                 int* tot1) {
  const uint64_t m0 = __ballot(f0);
  const uint64_t m1 = __ballot(f1);
  if (lane_id() == 0) {
    s.wave[0][wave_id()] = __popcll(m0);
    s.wave[1][wave_id()] = __popcll(m1);
  }
  __syncthreads();
  int o0 = 0, o1 = 0, t0 = 0, t1 = 0;
#pragma unroll
  for (int w = 0; w < kBW; ++w) {
    const int v0 = s.wave[0][w];
    const int v1 = s.wave[1][w];
    o0 += (w < wave_id()) ? v0 : 0;
    o1 += (w < wave_id()) ? v1 : 0;
    t0 += v0;
    t1 += v1;
  }
  __syncthreads();
  *pre0 = o0 + __popcll(m0 & lanes_below());
  *pre1 = o1 + __popcll(m1 & lanes_below());
  *tot0 = t0;
  *tot1 = t1;
}

__device__ __forceinline__ long long block_sum(long long v, long long* s_red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  if (lane_id() == 0) s_red[wave_id()] = v;
  __syncthreads();
  long long t = 0;
#pragma unroll
  for (int w = 0; w < kBW; ++w) t += s_red[w];
  __syncthreads();
  return t;
}

struct SelectSmem {
  unsigned hist[256];
  unsigned dstar, above, neq;
};

// Wave 0 finds the digit d* with (#digits above d*) < k <= (#digits >= d*).
__device__ __forceinline__ void find_digit(SelectSmem& s, unsigned k) {
  if (wave_id() == 0) {
    const int l = lane_id();
    unsigned loc[4];
    unsigned lsum = 0;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      loc[t] = s.hist[255 - 4 * l - t];
      lsum += loc[t];
    }
    unsigned incl = lsum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const unsigned v = __shfl_up(incl, off);
      if (l >= off) incl += v;
    }
    const unsigned excl = incl - lsum;
    if (excl < k && k <= incl) {
      unsigned cum = excl;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if (cum + loc[t] >= k) {
          s.dstar = 255 - 4 * l - t;
          s.above = cum;
          s.neq = loc[t];
          break;
        }
        cum += loc[t];
      }
    }
  }
}

// MSB-first radix select over positions [lo, hi) with pred(i) true, for the
// k largest keys (1 <= k <= number of eligible positions).  Returns T such
// that the selection is every key > T plus the first *k_rem keys == T (in
// any order the caller fixes); *n_eq >= *k_rem.  Normally T is the k-th
// largest key, *k_rem = k - #(key > T) and *n_eq = #(key == T).  The passes
// stop early once every key sharing the digits found so far is selected:
// then T is that prefix with the lower bits zero and *k_rem = *n_eq = the
// number of keys sharing it, so all of them are either > T or == T and
// taken, and no key outside the prefix lies between.
template <class KeyOf, class Pred>
__device__ uint64_t block_radix_select(int64_t lo, int64_t hi, unsigned k, KeyOf key_of, Pred pred, SelectSmem& s,
                                       unsigned* k_rem, unsigned* n_eq) {
  uint64_t prefix = 0, mask = 0;
  unsigned neq = 0;
  for (int shift = 56; shift >= 0; shift -= 8) {
    if (threadIdx.x < 256) s.hist[threadIdx.x] = 0;
    __syncthreads();
    for (int64_t i = lo + threadIdx.x; i < hi; i += kBT) {
      if (!pred(i)) continue;
      const uint64_t kk = key_of(i);
      if ((kk & mask) != prefix) continue;
      atomicAdd(&s.hist[(kk >> shift) & 255u], 1u);
    }
    __syncthreads();
    find_digit(s, k);
    __syncthreads();
    prefix |= (uint64_t)s.dstar << shift;
    mask |= 255ull << shift;
    k -= s.above;
    neq = s.neq;
    __syncthreads();
    if (neq == k) break;  // uniform: read from LDS after the barrier
  }
  *k_rem = k;
  *n_eq = neq;
  return prefix;
}

struct SortSmem {
  unsigned hist[256];
  unsigned off[256];
  unsigned tot[256];
  unsigned wave_cnt[kBW][256];
  unsigned single;
};

// Stable descending sort of L (key, idx) pairs by key with 8-bit LSD passes.
// Data starts in (ka, ia); (kb, ib) is scratch of the same size.  Passes in
// which every key has the same digit are skipped.  The result ends in (ka, ia).
__device__ void block_sort_desc(uint64_t* ka, int32_t* ia, uint64_t* kb, int32_t* ib, int L, SortSmem& s) {
  uint64_t* sk = ka;
  int32_t* si = ia;
  uint64_t* dk = kb;
  int32_t* di = ib;
  for (int shift = 0; shift < 64; shift += 8) {
    if (threadIdx.x < 256) s.hist[threadIdx.x] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < L; i += kBT) atomicAdd(&s.hist[(sk[i] >> shift) & 255u], 1u);
    __syncthreads();
    if (threadIdx.x == 0) s.single = 0;
    __syncthreads();
    if (threadIdx.x < 256 && s.hist[threadIdx.x] == (unsigned)L) s.single = 1;
    // exclusive offsets in descending digit order
    if (wave_id() == 0) {
      const int l = lane_id();
      unsigned loc[4];
      unsigned lsum = 0;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        loc[t] = s.hist[255 - 4 * l - t];
        lsum += loc[t];
      }
      unsigned incl = lsum;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const unsigned v = __shfl_up(incl, off);
        if (l >= off) incl += v;
      }
      unsigned cum = incl - lsum;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        s.off[255 - 4 * l - t] = cum;
        cum += loc[t];
      }
    }
    for (int t = threadIdx.x; t < kBW * 256; t += kBT) (&s.wave_cnt[0][0])[t] = 0;
    __syncthreads();
    if (s.single) continue;  // identity permutation: nothing to move
    for (int base = 0; base < L; base += kBT) {
      const int i = base + (int)threadIdx.x;
      const bool valid = i < L;
      uint64_t key = 0;
      int32_t idx = 0;
      unsigned dg = 0;
      if (valid) {
        key = sk[i];
        idx = si[i];
        dg = (unsigned)(key >> shift) & 255u;
      }
      uint64_t peers = __ballot(valid);
#pragma unroll
      for (int bit = 0; bit < 8; ++bit) {
        const bool on = (dg >> bit) & 1u;
        const uint64_t bb = __ballot(valid && on);
        peers &= on ? bb : ~bb;
      }
      const unsigned rank = __popcll(peers & lanes_below());
      if (valid && rank == 0) s.wave_cnt[wave_id()][dg] = __popcll(peers);
      __syncthreads();
      if (threadIdx.x < 256) {
        unsigned run = 0;
#pragma unroll
        for (int w = 0; w < kBW; ++w) {
          const unsigned v = s.wave_cnt[w][threadIdx.x];
          s.wave_cnt[w][threadIdx.x] = run;
          run += v;
        }
        s.tot[threadIdx.x] = run;
      }
      __syncthreads();
      if (valid) {
        const unsigned dst = s.off[dg] + s.wave_cnt[wave_id()][dg] + rank;
        dk[dst] = key;
        di[dst] = idx;
      }
      __syncthreads();
      if (threadIdx.x < 256) {
        s.off[threadIdx.x] += s.tot[threadIdx.x];
#pragma unroll
        for (int w = 0; w < kBW; ++w) s.wave_cnt[w][threadIdx.x] = 0;
      }
      __syncthreads();
    }
    uint64_t* tk = sk;
    sk = dk;
    dk = tk;
    int32_t* ti = si;
    si = di;
    di = ti;
  }
  if (sk != ka) {
    __syncthreads();
    for (int i = threadIdx.x; i < L; i += kBT) {
      ka[i] = sk[i];
      ia[i] = si[i];
    }
  }
  __syncthreads();
}

}  // namespace twinkv
