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

// Each LPK-lane group takes kRows consecutive key rows per step and issues
// all their loads, keys and values, before the first sum: 2 * kRows 16-byte
// loads in flight per lane.  Lane u of the group then writes row u's
// results, so a wave's stores cover consecutive keys.  Keys and values are
// read once here, so the loads are nontemporal.
constexpr int kRows = 4;

__device__ __forceinline__ uint4 load_nt(const uint4* p) {
  typedef unsigned u4 __attribute__((ext_vector_type(4)));
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u4*>(p)));
}

template <int D, bool WITH_V>
__global__ __launch_bounds__(256) void norms_energy_kernel(const uint4* __restrict__ K, const uint4* __restrict__ V,
                                                           int64_t nkeys, double* __restrict__ nsq,
                                                           float* __restrict__ rinv, double* __restrict__ energy) {
  constexpr int LPK = D / 8;           // lanes per key row
  constexpr int GPB = 256 / LPK;       // lane groups per block
  static_assert(kRows <= LPK, "one writing lane per row of the group");
  const int sub = threadIdx.x % LPK;
  const int64_t stride = (int64_t)gridDim.x * GPB * kRows;
  for (int64_t key0 = ((int64_t)blockIdx.x * GPB + threadIdx.x / LPK) * kRows; key0 < nkeys; key0 += stride) {
    // a whole LPK-lane group is either inside or outside the range, so the
    // group-wide shuffles below always see active partners
    uint4 kv[kRows], vv[kRows];
#pragma unroll
    for (int u = 0; u < kRows; ++u) {
      const int64_t key = key0 + u;
      kv[u] = key < nkeys ? load_nt(K + key * LPK + sub) : make_uint4(0u, 0u, 0u, 0u);
      if (WITH_V) vv[u] = key < nkeys ? load_nt(V + key * LPK + sub) : make_uint4(0u, 0u, 0u, 0u);
    }
    double n_mine = 0.0, e_mine = 0.0;
#pragma unroll
    for (int u = 0; u < kRows; ++u) {
      const double n = group_sum<LPK>(sumsq8(kv[u]));
      const double e = WITH_V ? group_sum<LPK>(sumsq8(vv[u])) : 0.0;
      n_mine = sub == u ? n : n_mine;
      e_mine = sub == u ? e : e_mine;
    }
    const int64_t key = key0 + sub;
    if (sub < kRows && key < nkeys) {
      nsq[key] = n_mine;
      rinv[key] = n_mine > 0.0 ? (float)(1.0 / sqrt(n_mine)) : 0.0f;
      if (WITH_V) energy[key] = e_mine;
    }
  }
}

template <int D>
hipError_t launch_d(const uint16_t* keys, const uint16_t* values, int64_t nkeys, double* nsq, float* rinv,
                    double* energy, hipStream_t stream) {
  constexpr int KPB = 256 / (D / 8) * kRows;  // keys per block per step
  int64_t blocks = (nkeys + KPB - 1) / KPB;
  if (blocks > (1 << 20)) blocks = 1 << 20;  // a grid-stride loop covers the rest
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
