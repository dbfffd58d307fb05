// Exact-budget per-head selection ("Small Frequency Corrections Can Change
// What Survives KV Cache Compression", sections 3.1, 3.2 and 3.4):
// keep the protected sinks and recent positions, clipped against the head's
// capacity (sinks first), and the u = b - s - r unprotected positions ranked
// first by (score desc, energy desc, position asc).
//
// One 1024-thread workgroup per head.  Scores and energies are non-negative
// fp64, so their bit patterns order like the values.  An MSB-first radix
// select (up to 8 passes of 8-bit digits; it stops as soon as the bucket of
// the boundary digit is taken whole) finds the threshold of the u largest
// scores; only if the boundary value is shared by more positions than remain
// to be taken does a second select run on the energies of those ties, and
// only if that boundary is shared too are the remaining slots given to the
// lowest positions.  A
// final pass in position order writes the keep mask and the ascending list of
// retained positions.
#include "blockops.h"

namespace twinkv {
namespace {

__device__ __forceinline__ uint64_t dbits(double x) { return (uint64_t)__double_as_longlong(x + 0.0); }

__global__ __launch_bounds__(kBT) void select_kernel(SelectArgs a) {
  __shared__ SelectSmem ss;
  __shared__ ScanSmem2 sc;

  const int64_t g = blockIdx.x;
  const int64_t N = a.N;
  const double* sc_g = a.score + g * N;
  const double* en_g = a.energy + g * N;

  int64_t cap = a.capacity[g];
  cap = cap < 0 ? 0 : (cap > N ? N : cap);
  const int64_t s_cnt = a.sink < cap ? a.sink : cap;
  const int64_t r_cnt = a.recent < cap - s_cnt ? a.recent : cap - s_cnt;
  const int64_t u = cap - s_cnt - r_cnt;
  const int64_t lo = s_cnt, hi = N - r_cnt;  // unprotected candidates [lo, hi)

  // this head's run of the kept list: [kept_off[g], kept_off[g+1]), clipped
  // to the list's length kept_off[G], so inconsistent offsets can give wrong
  // entries but never a write outside [0, kept_off[G])
  const long long total = a.kept_off[a.G];
  const long long off_g = a.kept_off[g];
  long long off_end = a.kept_off[g + 1];
  off_end = off_end < total ? off_end : total;

  // level 0: take no candidate; 1: all; 2: score > T1, ties resolved below
  int level;
  uint64_t T1 = 0, T2 = 0;
  unsigned k1 = 0, k2 = 0, n1 = 0, n2 = 0;
  bool lvl_energy = false, lvl_index = false;
  if (u == 0) {
    level = 0;
  } else if (u == hi - lo) {
    level = 1;
  } else {
    level = 2;
    T1 = block_radix_select(
        lo, hi, (unsigned)u, [&](int64_t i) { return dbits(sc_g[i]); }, [](int64_t) { return true; }, ss, &k1, &n1);
    if (k1 < n1) {
      lvl_energy = true;
      T2 = block_radix_select(
          lo, hi, k1, [&](int64_t i) { return dbits(en_g[i]); }, [&](int64_t i) { return dbits(sc_g[i]) == T1; }, ss,
          &k2, &n2);
      lvl_index = k2 < n2;
    }
  }

  // final pass in position order
  int tie_base = 0, kept_base = 0;
  for (int64_t base = 0; base < N; base += kBT) {
    const int64_t i = base + threadIdx.x;
    const bool in = i < N;
    const bool prot = in && (i < lo || i >= hi);
    const bool cand = in && !prot;
    bool take = prot;
    bool tie = false;
    if (cand) {
      if (level == 1) {
        take = true;
      } else if (level == 2) {
        const uint64_t s1 = dbits(sc_g[i]);
        if (s1 > T1) {
          take = true;
        } else if (s1 == T1) {
          if (!lvl_energy) {
            take = true;
          } else {
            const uint64_t e1 = dbits(en_g[i]);
            if (e1 > T2) take = true;
            else if (e1 == T2) {
              if (!lvl_index) take = true;
              else tie = true;
            }
          }
        }
      }
    }
    // the index-level ties kept are the first k2 of all such ties in
    // position order, so in this chunk the first `rem` of its ties; a kept
    // position's place is the other kept positions before it plus the kept
    // ties before it
    int trank = 0, krank = 0, tie_tot = 0, kept_tot = 0;
    block_scan_flag2(tie, take, sc, &trank, &krank, &tie_tot, &kept_tot);
    const int rem = (int)k2 > tie_base ? (int)k2 - tie_base : 0;
    if (tie && trank < rem) take = true;
    if (in) a.keep[g * N + i] = take ? 1 : 0;
    if (take) {
      const long long dst = off_g + kept_base + krank + (trank < rem ? trank : rem);
      if (dst >= 0 && dst < off_end) a.kept_idx[dst] = (int32_t)i;
    }
    kept_base += kept_tot + (tie_tot < rem ? tie_tot : rem);
    tie_base += tie_tot;
  }
}

// Start of each head's run in the kept list: kept_off[0] = 0 and
// kept_off[g+1] = kept_off[g] + clamp(capacity[g], 0, N).  One workgroup scans
// the heads in chunks of kBT: an inclusive scan inside each wave by shuffles,
// then the wave totals through LDS.
__global__ __launch_bounds__(kBT) void offsets_kernel(const int32_t* __restrict__ capacity, int64_t G, int64_t N,
                                                      int64_t* __restrict__ kept_off) {
  __shared__ long long wsum[kBW];
  long long base = 0;
  if (threadIdx.x == 0) kept_off[0] = 0;
  for (int64_t c0 = 0; c0 < G; c0 += kBT) {
    const int64_t q = c0 + threadIdx.x;
    long long v = 0;
    if (q < G) {
      const long long c = capacity[q];
      v = c < 0 ? 0 : (c > N ? N : c);
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const long long u = __shfl_up(v, off);
      if (lane_id() >= off) v += u;
    }
    if (lane_id() == 63) wsum[wave_id()] = v;
    __syncthreads();
    long long before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kBW; ++w) {
      const long long t = wsum[w];
      before += (w < wave_id()) ? t : 0;
      tot += t;
    }
    __syncthreads();
    if (q < G) kept_off[q + 1] = base + before + v;
    base += tot;
  }
}

// Selection keys of the score variants (TwinKV page, section 3.2, Eq. 3;
// frequency-correction page, sections 5.3 and 5.5): from the count c (of
// position perm[i] when a permutation is given) and the energy e of each
// position, with disc = ln((N+1)/(c+1)):
//   twin:   score e * disc,           tie e
//   value:  score e,                  tie e
//   rarity: score disc / ln(N+1),     tie 0  (equal counts: lower position)
// The expressions are the ones the score kernel evaluates, so the twin
// variant without a permutation reproduces its scores bit for bit.
__global__ __launch_bounds__(256) void variant_kernel(const int32_t* __restrict__ count,
                                                     const double* __restrict__ energy,
                                                     const int32_t* __restrict__ perm, int64_t G, int64_t N,
                                                     int variant, double* __restrict__ score,
                                                     double* __restrict__ tie) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= G * N) return;
  int64_t src = i;
  if (perm) {
    int64_t p = perm[i];
    p = p < 0 ? 0 : (p >= N ? N - 1 : p);
    src = (i / N) * N + p;
  }
  const int c = count[src];
  const double e = energy[i];
  const double disc = log((double)(N + 1) / (double)(c + 1));
  if (variant == 0) {
    score[i] = e * disc;
    tie[i] = e;
  } else if (variant == 1) {
    score[i] = e;
    tie[i] = e;
  } else {
    score[i] = disc / log((double)(N + 1));
    tie[i] = 0.0;
  }
}

}  // namespace

hipError_t launch_variant(const int32_t* count, const double* energy, const int32_t* perm, int64_t G, int64_t N,
                          int variant, double* score, double* tie, hipStream_t stream) {
  const int64_t n = G * N;
  const int64_t blocks = (n + 255) / 256;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(variant_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, count, energy, perm, G, N, variant,
                     score, tie);
  return hipGetLastError();
}

hipError_t launch_offsets(const int32_t* capacity, int64_t G, int64_t N, int64_t* kept_off, hipStream_t stream) {
  hipLaunchKernelGGL(offsets_kernel, dim3(1), dim3(kBT), 0, stream, capacity, G, N, kept_off);
  return hipGetLastError();
}

hipError_t launch_select(const SelectArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(select_kernel, dim3((unsigned)a.G), dim3(kBT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace twinkv
