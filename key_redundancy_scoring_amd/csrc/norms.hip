// Streaming pass over keys (and values): squared key norms in fp64, the fp32
// inverse norm used by the Gram sweep, and the value energy ||v||^2 in fp64.
//
// Value energy is e_{h,i} = ||v_{h,i}||_2^2 ("Small Frequency Corrections Can
// Change What Survives KV Cache Compression", section 3.2); the key norm
// normalises keys for the cosine of "TwinKV: A Composable Repair Pass ...",
// section 3.2, Eq. 1.
//
// Products of two bf16 numbers are exact in fp32 (8-bit significands), so nsq
// and energy are fp64 sums of d exact non-negative terms: exact when the
// squares of a row span less than about 2^31 in magnitude, and otherwise
// within (d-1) fp64 roundings of the exact sum.
//
// Layout: one key row is d bf16 = d/8 chunks of 16 bytes; d/8 consecutive
// lanes read one row, so a wave reads 1 KiB of contiguous memory per load.
#include "internal.h"

namespace twinkv {

namespace {

__device__ __forceinline__ double sumsq8(uint4 u) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
  double acc = 0.0;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const float lo = __uint_as_float(w[t] << 16);
    const float hi = __uint_as_float(w[t] & 0xffff0000u);
    acc += (double)(lo * lo);  // exact in fp32
    acc += (double)(hi * hi);
  }
  return acc;
}

template <int LPK>
__device__ __forceinline__ double group_sum(double v) {
#pragma unroll
  for (int off = LPK / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, LPK);
  return v;
}

template <int D, bool WITH_V>
__global__ __launch_bounds__(256) void norms_energy_kernel(const uint4* __restrict__ K, const uint4* __restrict__ V,
                                                           int64_t nkeys, double* __restrict__ nsq,
                                                           float* __restrict__ rinv, double* __restrict__ energy) {
  constexpr int LPK = D / 8;         // lanes per key row
  constexpr int KPB = 256 / LPK;     // key rows per block per step
  const int sub = threadIdx.x % LPK;
  const int64_t stride = (int64_t)gridDim.x * KPB;
  for (int64_t key = (int64_t)blockIdx.x * KPB + threadIdx.x / LPK; key < nkeys; key += stride) {
    // a whole LPK-lane group is either inside or outside the range, so the
    // group-wide shuffles below always see active partners
    const uint4 kv = K[key * LPK + sub];
    double n = group_sum<LPK>(sumsq8(kv));
    double e = 0.0;
    if (WITH_V) {
      const uint4 vv = V[key * LPK + sub];
      e = group_sum<LPK>(sumsq8(vv));
    }
    if (sub == 0) {
      nsq[key] = n;
      rinv[key] = n > 0.0 ? (float)(1.0 / sqrt(n)) : 0.0f;
      if (WITH_V) energy[key] = e;
    }
  }
}

template <int D>
hipError_t launch_d(const uint16_t* keys, const uint16_t* values, int64_t nkeys, double* nsq, float* rinv,
                    double* energy, hipStream_t stream) {
  constexpr int KPB = 256 / (D / 8);
  int64_t blocks = (nkeys + KPB - 1) / KPB;
  if (blocks > 256 * 64) blocks = 256 * 64;
  if (blocks < 1) blocks = 1;
  if (values)
    hipLaunchKernelGGL((norms_energy_kernel<D, true>), dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const uint4*)keys, (const uint4*)values, nkeys, nsq, rinv, energy);
  else
    hipLaunchKernelGGL((norms_energy_kernel<D, false>), dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const uint4*)keys, (const uint4*)nullptr, nkeys, nsq, rinv, (double*)nullptr);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_norms(const uint16_t* keys, const uint16_t* values, int64_t nkeys, int d, double* nsq,
                        float* rinv, double* energy, hipStream_t stream) {
  if (d == 64) return launch_d<64>(keys, values, nkeys, nsq, rinv, energy, stream);
  return launch_d<128>(keys, values, nkeys, nsq, rinv, energy, stream);
}

}  // namespace twinkv
