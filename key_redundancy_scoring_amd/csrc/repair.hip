// Repair-pass kernels ("TwinKV: A Composable Repair Pass for KV Cache Eviction
// via Pairwise Key Redundancy", section 3.4).
//
// compact_kernel: the retained positions of each head in ascending order and
//   their number K = |S0|; the restricted Gram sweep reads column keys through
//   this list, so only the K retained columns are compared (the O(nKd) form
//   the page's complexity section describes).
//
// swap_kernel (one 1024-thread workgroup per head), given b_i = b_i(S0):
//   orphans O = { i not in S0 : b_i < tau }, ranked by (b asc, i asc);
//   donors  D = { j in S0, outside the sink/recent regions clipped against K :
//                 b_j >= tau }, ranked by (b desc, j asc);
//   m = min(|O|, |D|); S1 = S0 - D[:m] + O[:m]; pairs (O[k], D[k]).
//   Both rankings become "descending 64-bit key, ascending position": the key
//   is the order-preserving bit image of b for donors and its complement for
//   orphans.  On the side with more than m members a radix select finds the
//   m-th key (or a prefix of it that only the chosen share); the m chosen members of each side are gathered in position
//   order and put in rank order by a stable LSD radix sort, which keeps equal
//   keys in position order.
#include <limits.h>

#include "blockops.h"

namespace twinkv {
namespace {

__global__ __launch_bounds__(kBT) void compact_kernel(const uint8_t* __restrict__ keep_in, int64_t N,
                                                      int32_t* __restrict__ pos, int32_t* __restrict__ ncols) {
  __shared__ ScanSmem sc;
  const int64_t g = blockIdx.x;
  const uint8_t* in = keep_in + g * N;
  int32_t* out = pos + g * N;
  int base = 0;
  for (int64_t b = 0; b < N; b += kBT) {
    const int64_t i = b + threadIdx.x;
    const bool f = i < N && in[i] != 0;
    int tot = 0;
    const int r = block_scan_flag(f, sc, &tot);
    if (f) out[base + r] = (int32_t)i;
    base += tot;
  }
  if (threadIdx.x == 0) ncols[g] = base;
}

// The rows of the restricted sweep.  The prior (prior_sim, prior_idx) is the
// unrestricted best nonlocal twin of each position, from the score pass over
// the same keys and window.  If it is retained, it is also b_i(S0) with its
// position: the lowest position attaining the maximum over all nonlocal j
// lies in S0, so it attains the maximum over S0's nonlocal j, and no lower
// position of S0 does.  If there is no nonlocal j at all (prior_idx = -1),
// S0 has none either.  Those rows take the prior and are not swept; the
// others are listed in ascending order.  Without a prior every row is
// listed.  A prior index outside [0, N) other than -1 is treated as not
// retained, so its row is swept.  The head's count of rows queued for the
// exact resolve is zeroed here, before the sweep that fills the queue.
__global__ __launch_bounds__(kBT) void rows_kernel(const uint8_t* __restrict__ keep_in,
                                                   const double* __restrict__ prior_sim,
                                                   const int32_t* __restrict__ prior_idx, int64_t N,
                                                   int32_t* __restrict__ row_pos, int32_t* __restrict__ nrows,
                                                   double* __restrict__ best_sim, int32_t* __restrict__ best_idx,
                                                   int32_t* __restrict__ qcount) {
  __shared__ ScanSmem sc;
  const int64_t g = blockIdx.x;
  const size_t o = (size_t)g * N;
  int base = 0;
  for (int64_t b = 0; b < N; b += kBT) {
    const int64_t i = b + threadIdx.x;
    bool f = i < N;
    if (f && prior_idx) {
      const int32_t j = prior_idx[o + i];
      if (j == -1 || (j >= 0 && j < N && keep_in[o + j] != 0)) {
        f = false;
        best_sim[o + i] = prior_sim[o + i];
        best_idx[o + i] = j;
      }
    }
    int tot = 0;
    const int r = block_scan_flag(f, sc, &tot);
    if (f) row_pos[o + base + r] = (int32_t)i;
    base += tot;
  }
  if (threadIdx.x == 0) {
    nrows[g] = base;
    qcount[g] = 0;
  }
}

// Copy retained key rows (and their inverse norms) into column order, so the
// restricted Gram sweep streams contiguous rows: ckeys[g][k] = keys[g][pos[g][k]]
// for k < ncols[g].  One 16-byte chunk per thread and step.
template <int D>
__global__ __launch_bounds__(256) void gather_kernel(const uint4* __restrict__ keys, const float* __restrict__ rinv,
                                                     const int32_t* __restrict__ pos,
                                                     const int32_t* __restrict__ ncols, int64_t N, int64_t bph,
                                                     uint4* __restrict__ ckeys, float* __restrict__ crinv) {
  constexpr int CH = D / 8;
  constexpr int STEPS = 4;
  const int64_t g = blockIdx.x / bph;
  const int64_t bx = blockIdx.x % bph;
  const int64_t lim = (int64_t)ncols[g] * CH;
  const int32_t* pg = pos + g * N;
  const uint4* kg = keys + g * N * CH;
  uint4* cg = ckeys + g * N * CH;
#pragma unroll
  for (int t = 0; t < STEPS; ++t) {
    const int64_t q = (bx * STEPS + t) * 256 + threadIdx.x;
    if (q < lim) {
      const int64_t k = q / CH;
      const int c = (int)(q % CH);
      const int64_t src = pg[k];
      cg[q] = kg[src * CH + c];
      if (c == 0) crinv[g * N + k] = rinv[g * N + src];
    }
  }
}

// Gather the top-m members of one side, in position order, into (lk, li).
template <class KeyOf, class Pred>
__device__ void collect_side(int64_t N, unsigned m, long long count, KeyOf key_of, Pred pred, uint64_t* lk,
                             int32_t* li, SelectSmem& ss, ScanSmem2& sc) {
  const bool all = (long long)m == count;
  uint64_t T = 0;
  unsigned k_rem = 0, n_eq = 0;
  if (!all) T = block_radix_select(0, N, m, key_of, pred, ss, &k_rem, &n_eq);
  int tie_base = 0, base = 0;
  for (int64_t b = 0; b < N; b += kBT) {
    const int64_t i = b + threadIdx.x;
    bool take = false, tie = false;
    uint64_t key = 0;
    if (i < N && pred(i)) {
      key = key_of(i);
      if (all || key > T) take = true;
      else if (key == T) tie = true;
    }
    // the ties taken are the first k_rem of all ties in position order, so
    // in this chunk the first `rem` of its ties; a member's place among the
    // chunk's chosen is the plain takes before it plus the taken ties before it
    int tr = 0, kr = 0, tt = 0, kt = 0;
    block_scan_flag2(tie, take, sc, &tr, &kr, &tt, &kt);
    const int rem = (int)k_rem > tie_base ? (int)k_rem - tie_base : 0;
    if (take || (tie && tr < rem)) {
      const int r = kr + (tr < rem ? tr : rem);
      lk[base + r] = key;
      li[base + r] = (int32_t)i;
    }
    base += kt + (tt < rem ? tt : rem);
    tie_base += tt;
  }
  __syncthreads();
}

__global__ __launch_bounds__(kBT) void swap_kernel(SwapArgs a) {
  __shared__ SelectSmem ss;
  __shared__ ScanSmem2 sc;
  __shared__ SortSmem so;
  __shared__ long long red[kBW];

  const int64_t g = blockIdx.x;
  const int64_t N = a.N;
  const int64_t K = a.ncols[g];
  const int64_t s_cnt = a.sink < K ? a.sink : K;
  const int64_t r_cnt = a.recent < K - s_cnt ? a.recent : K - s_cnt;
  const uint8_t* in = a.keep_in + g * N;
  const double* bs = a.best + g * N;
  uint8_t* out = a.keep_out + g * N;
  const double tau = a.tau;

  auto is_orphan = [&](int64_t i) { return in[i] == 0 && bs[i] < tau; };
  auto is_donor = [&](int64_t i) { return in[i] != 0 && i >= s_cnt && i < N - r_cnt && bs[i] >= tau; };
  auto orphan_key = [&](int64_t i) { return ~ordered_bits(bs[i]); };
  auto donor_key = [&](int64_t i) { return ordered_bits(bs[i]); };

  long long no = 0, nd = 0;
  for (int64_t i = threadIdx.x; i < N; i += kBT) {
    no += is_orphan(i) ? 1 : 0;
    nd += is_donor(i) ? 1 : 0;
    out[i] = in[i] != 0 ? 1 : 0;
  }
  no = block_sum(no, red);
  nd = block_sum(nd, red);
  const long long m = no < nd ? no : nd;
  __syncthreads();

  int32_t* pairs = a.pairs + g * (N / 2) * 2;
  if (m > 0) {
    uint64_t* ka = a.keys_a + g * N;
    int32_t* ia = a.idx_a + g * N;
    uint64_t* kb = a.keys_b + g * N;
    int32_t* ib = a.idx_b + g * N;
    collect_side(N, (unsigned)m, no, orphan_key, is_orphan, ka, ia, ss, sc);
    collect_side(N, (unsigned)m, nd, donor_key, is_donor, ka + m, ia + m, ss, sc);
    block_sort_desc(ka, ia, kb, ib, (int)m, so);
    block_sort_desc(ka + m, ia + m, kb + m, ib + m, (int)m, so);
    for (int64_t k = threadIdx.x; k < m; k += kBT) {
      const int32_t o = ia[k];
      const int32_t dn = ia[m + k];
      out[dn] = 0;
      out[o] = 1;
      pairs[2 * k] = o;
      pairs[2 * k + 1] = dn;
    }
  }
  for (int64_t k = m + threadIdx.x; k < N / 2; k += kBT) {
    pairs[2 * k] = -1;
    pairs[2 * k + 1] = -1;
  }
  if (threadIdx.x == 0) {
    a.n_orphans[g] = (int32_t)no;
    a.n_donors[g] = (int32_t)nd;
    a.n_swaps[g] = (int32_t)m;
  }
}

}  // namespace

hipError_t launch_compact(const uint8_t* keep_in, int64_t G, int64_t N, int32_t* pos, int32_t* ncols,
                          hipStream_t stream) {
  hipLaunchKernelGGL(compact_kernel, dim3((unsigned)G), dim3(kBT), 0, stream, keep_in, N, pos, ncols);
  return hipGetLastError();
}

hipError_t launch_rows(const uint8_t* keep_in, const double* prior_sim, const int32_t* prior_idx, int64_t G,
                       int64_t N, int32_t* row_pos, int32_t* nrows, double* best_sim, int32_t* best_idx,
                       int32_t* qcount, hipStream_t stream) {
  hipLaunchKernelGGL(rows_kernel, dim3((unsigned)G), dim3(kBT), 0, stream, keep_in, prior_sim, prior_idx, N, row_pos,
                     nrows, best_sim, best_idx, qcount);
  return hipGetLastError();
}

hipError_t launch_gather(const uint16_t* keys, const float* rinv, const int32_t* pos, const int32_t* ncols, int64_t G,
                         int64_t N, int d, uint16_t* ckeys, float* crinv, hipStream_t stream) {
  const int64_t chunks = N * (d / 8);
  const int64_t bph = (chunks + 1023) / 1024;
  if (bph * G > INT_MAX) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(bph * G));
  if (d == 64)
    hipLaunchKernelGGL((gather_kernel<64>), grid, dim3(256), 0, stream, (const uint4*)keys, rinv, pos, ncols, N, bph,
                       (uint4*)ckeys, crinv);
  else
    hipLaunchKernelGGL((gather_kernel<128>), grid, dim3(256), 0, stream, (const uint4*)keys, rinv, pos, ncols, N, bph,
                       (uint4*)ckeys, crinv);
  return hipGetLastError();
}

hipError_t launch_swap(const SwapArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(swap_kernel, dim3((unsigned)a.G), dim3(kBT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace twinkv
