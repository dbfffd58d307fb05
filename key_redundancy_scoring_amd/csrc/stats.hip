// Count statistics of each head over its unprotected positions ("TwinKV: A
// Composable Repair Pass ...", Figure 1(b); "Small Frequency Corrections Can
// Change What Survives KV Cache Compression", sections 2.1 and 5.5 and
// appendix B.2): positions with a nonlocal twin, the six-bin count
// histogram, the sum of normalised discounts, how the Twin selection differs
// from value-only selection, and the energy margins |e/e_cut - 1| of the
// changed positions and of the whole pool around value-only's cut.
//
// One 1024-thread workgroup per head, two passes over the head's N
// positions (the margins need the cut, a minimum over the first pass).
// Everything but the discount sum is an integer count; the bins compare the
// same fp64 quantities the definition names.

#include "blockops.h"

namespace twinkv {
namespace {

__device__ __forceinline__ double block_min(double v, double* s) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmin(v, __shfl_xor(v, off));
  if (lane_id() == 0) s[wave_id()] = v;
  __syncthreads();
  double t = s[0];
#pragma unroll
  for (int w = 1; w < kBW; ++w) t = fmin(t, s[w]);
  __syncthreads();
  return t;
}

__device__ __forceinline__ double block_sumd(double v, double* s) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  if (lane_id() == 0) s[wave_id()] = v;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int w = 0; w < kBW; ++w) t += s[w];
  __syncthreads();
  return t;
}

__device__ __forceinline__ int margin_bin(double dev) {
  return (dev >= 0.05) + (dev >= 0.10) + (dev >= 0.25) + (dev >= 0.50);
}

__global__ __launch_bounds__(kBT) void stats_kernel(StatsArgs a) {
  __shared__ long long red[kBW];
  __shared__ double redd[kBW];
  const int64_t g = blockIdx.x;
  const int64_t N = a.N;
  int64_t cap = a.capacity[g];
  cap = cap < 0 ? 0 : (cap > N ? N : cap);
  const int64_t s_cnt = a.sink < cap ? a.sink : cap;
  const int64_t r_cnt = a.recent < cap - s_cnt ? a.recent : cap - s_cnt;
  const int64_t lo = s_cnt, hi = N - r_cnt;
  const int32_t* cg = a.count + g * N;
  const double* eg = a.energy + g * N;
  const uint8_t* kt = a.keep_twin ? a.keep_twin + g * N : nullptr;
  const uint8_t* kv = a.keep_value ? a.keep_value + g * N : nullptr;
  const double lnN1 = log((double)(N + 1));

  long long n = 0, twin = 0, hist[6] = {0, 0, 0, 0, 0, 0}, kept = 0, added = 0, removed = 0;
  double osum = 0.0, ecut = __builtin_inf();
  for (int64_t i = lo + threadIdx.x; i < hi; i += kBT) {
    const int c = cg[i];
    ++n;
    twin += c >= 1;
    hist[0] += c == 0;
    hist[1] += c == 1;
    hist[2] += c == 2;
    hist[3] += c >= 3 && c <= 4;
    hist[4] += c >= 5 && c <= 8;
    hist[5] += c >= 9;
    osum += log((double)(N + 1) / (double)(c + 1)) / lnN1;
    if (kt) {
      const bool t = kt[i] != 0, v = kv[i] != 0;
      kept += t;
      added += t && !v;
      removed += v && !t;
      if (v) ecut = fmin(ecut, eg[i]);
    }
  }
  int64_t* out = a.stats + g * kStatInts;
  const long long vals[11] = {n, twin, hist[0], hist[1], hist[2], hist[3], hist[4], hist[5], kept, added, removed};
#pragma unroll
  for (int k = 0; k < 11; ++k) {
    const long long t = block_sum(vals[k], red);
    if (threadIdx.x == 0) out[k] = t;
  }
  osum = block_sumd(osum, redd);
  ecut = block_min(ecut, redd);
  if (!(ecut < __builtin_inf())) ecut = 0.0;  // value-only keeps no unprotected position

  long long mb[15];
#pragma unroll
  for (int k = 0; k < 15; ++k) mb[k] = 0;
  if (kt && ecut > 0.0) {
    for (int64_t i = lo + threadIdx.x; i < hi; i += kBT) {
      const double dev = fabs(eg[i] / ecut - 1.0);
      const int b = margin_bin(dev);
      const bool t = kt[i] != 0, v = kv[i] != 0;
#pragma unroll
      for (int k = 0; k < 5; ++k) {
        mb[k] += (t && !v && b == k);
        mb[5 + k] += (v && !t && b == k);
        mb[10 + k] += (b == k);
      }
    }
  }
#pragma unroll
  for (int k = 0; k < 15; ++k) {
    const long long t = block_sum(mb[k], red);
    if (threadIdx.x == 0) out[11 + k] = t;
  }
  if (threadIdx.x == 0) {
    a.fstats[g * 2] = osum;
    a.fstats[g * 2 + 1] = ecut;
  }
}

}  // namespace

hipError_t launch_stats(const StatsArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(stats_kernel, dim3((unsigned)a.G), dim3(kBT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace twinkv
