// Head capacities from prefix attention ("Small Frequency Corrections Can
// Change What Survives KV Cache Compression", section 3.3, Equation 5, and
// appendices A.2 and A.3).
//
// For every KV head g the Gq query heads that share it observe the prefix
// from its last W positions t = N-W .. N-1.  With the causal softmax
//   a[q,t,i] = exp(s_{q,t,i} - m_{q,t}) / Z_{q,t},   s = q.k_i / sqrt(d),  i <= t,
// the statistic of position i is the average over the query heads of the
// sum over the W queries of a[q,t,i], max-pooled over a centred window of
// `pool` positions and rounded once to fp32: z[g][i].  Per layer (H KV heads
// sharing the per-head budget B = P + U), g_h counts head h's positions among
// the H*U largest unprotected z of the layer (ties to the lower head, then
// the lower position; an all-zero pool gives g_h = U), and
//   u~_h = (g_h + U)/2,  u_h = floor(u~_h) + delta_h,  b_h = P + u_h,
// where the first R = H*U - sum floor(u~_h) heads with fractional part 1/2
// get delta_h = 1.
//
// Kernels:
//   attn_kernel<D, 1>  one block of 256 keys of one head: every key against
//                      every observing query, logits in fp64 (bf16 products
//                      are exact in fp32, summed in fp64); per query the
//                      block's max logit and sum of exp(s - max);
//   combine_kernel     per query, the block partials merged into (m, Z);
//   attn_kernel<D, 2>  per key, sum over queries of exp(s - m)/Z, over Gq;
//   pool_kernel        the width-`pool` max, fp32 z, and the layer's pool of
//                      unprotected scores in (head, position) order;
//   the selection kernel over each layer's pool with capacity H*U (score
//   descending, then pool index ascending = head, then position);
//   alloc_kernel       per layer: g_h from the selected pool, Equation 5.
// The logits are recomputed in the second pass rather than stored: storing
// them would take Gq*W*N*8 bytes per head, while recomputing is FMA work the
// CUs have to spare.

#include "blockops.h"
#include "internal.h"

namespace twinkv {
namespace {

constexpr int kAT = 256;  // threads (keys) per attention block

__device__ __forceinline__ double wave_max(double v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmax(v, __shfl_xor(v, off));
  return v;
}
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// d = 64: the queries sit in LDS widened to fp64 (64 KiB) and the key in
// fp64 registers, so each product is one fp64 FMA of exact operands.  d = 128
// (whose fp64 key would not fit the registers) keeps bf16 queries in LDS and
// forms each exact product in fp32 before the fp64 sum.  Both sum the d
// products in order with one rounding each, so they give the same logits.
template <int D, int PHASE>
__global__ __launch_bounds__(kAT) void attn_kernel(AttnArgs a) {
  constexpr int CH = D / 8;
  constexpr bool F64 = D == 64;
  __shared__ uint4 qs[F64 ? 1 : kMaxQueries * CH];
  __shared__ double qd[F64 ? kMaxQueries * D : 2];
  __shared__ double pm[kAT / 64][kMaxQueries];
  __shared__ double pz[kAT / 64][kMaxQueries];
  __shared__ double sm[kMaxQueries];
  __shared__ double sr[kMaxQueries];  // 1 / Z

  const int64_t g = blockIdx.x / a.nchunk;
  const int64_t chunk = blockIdx.x % a.nchunk;
  const int Q = a.Gq * a.W;
  const int tid = threadIdx.x;
  const uint4* qg = reinterpret_cast<const uint4*>(a.queries) + (size_t)g * Q * CH;
  if (F64) {
    const uint16_t* qh = a.queries + (size_t)g * Q * D;
    for (int e = tid; e < Q * D; e += kAT) qd[e] = (double)__uint_as_float((uint32_t)qh[e] << 16);
  } else {
    for (int e = tid; e < Q * CH; e += kAT) qs[e] = qg[e];
  }
  if (PHASE == 2) {
    for (int q = tid; q < Q; q += kAT) {
      sm[q] = a.mz[((size_t)g * Q + q) * 2];
      sr[q] = 1.0 / a.mz[((size_t)g * Q + q) * 2 + 1];
    }
  }
  __syncthreads();

  const int64_t N = a.N;
  const int64_t j = chunk * kAT + tid;
  const bool valid = j < N;
  float kf[F64 ? 1 : D];
  double kd[F64 ? D : 1];
  {
    const uint4* kj = reinterpret_cast<const uint4*>(a.keys) + ((size_t)g * N + (valid ? j : 0)) * CH;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const uint4 u = kj[c];
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float lo = __uint_as_float(w[t] << 16), hi = __uint_as_float(w[t] & 0xffff0000u);
        if (F64) {
          kd[8 * c + 2 * t] = (double)lo;
          kd[8 * c + 2 * t + 1] = (double)hi;
        } else {
          kf[8 * c + 2 * t] = lo;
          kf[8 * c + 2 * t + 1] = hi;
        }
      }
    }
  }
  const double scale = a.inv_sqrt_d;
  double acc = 0.0;
#pragma unroll 1
  for (int q = 0; q < Q; ++q) {
    double s = 0.0;
    if (F64) {
      const double2* q2 = reinterpret_cast<const double2*>(qd + q * D);
#pragma unroll
      for (int c = 0; c < D / 2; ++c) {
        const double2 qq = q2[c];  // the same address in every lane: a broadcast
        s = fma(qq.x, kd[2 * c], s);
        s = fma(qq.y, kd[2 * c + 1], s);
      }
    } else {
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const uint4 u = qs[q * CH + c];
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          s += (double)(__uint_as_float(w[t] << 16) * kf[8 * c + 2 * t]);  // exact in fp32
          s += (double)(__uint_as_float(w[t] & 0xffff0000u) * kf[8 * c + 2 * t + 1]);
        }
      }
    }
    s *= scale;
    const int64_t tq = N - a.W + (q % a.W);
    const bool ok = valid && j <= tq;
    if (PHASE == 1) {
      const double m = wave_max(ok ? s : -__builtin_inf());
      const double e = (ok && m > -__builtin_inf()) ? exp(s - m) : 0.0;
      const double z = wave_sum(e);
      if ((tid & 63) == 0) {
        pm[tid >> 6][q] = m;
        pz[tid >> 6][q] = z;
      }
    } else {
      if (ok) acc += exp(s - sm[q]) * sr[q];
    }
  }
  if (PHASE == 1) {
    __syncthreads();
    for (int q = tid; q < Q; q += kAT) {
      double m = -__builtin_inf();
#pragma unroll
      for (int w = 0; w < kAT / 64; ++w) m = fmax(m, pm[w][q]);
      double z = 0.0;
      if (m > -__builtin_inf()) {
#pragma unroll
        for (int w = 0; w < kAT / 64; ++w)
          if (pm[w][q] > -__builtin_inf()) z += pz[w][q] * exp(pm[w][q] - m);
      }
      double* dst = a.part + (((size_t)g * a.nchunk + chunk) * Q + q) * 2;
      dst[0] = m;
      dst[1] = z;
    }
  } else if (valid) {
    a.agg[(size_t)g * N + j] = acc * a.inv_gq;
  }
}

// Per query: merge the block partials (max, sum of exp(s - max)) into (m, Z).
__global__ __launch_bounds__(kMaxQueries) void combine_kernel(AttnArgs a) {
  const int64_t g = blockIdx.x;
  const int Q = a.Gq * a.W;
  const int q = threadIdx.x;
  if (q >= Q) return;
  double m = -__builtin_inf();
  for (int64_t c = 0; c < a.nchunk; ++c) m = fmax(m, a.part[(((size_t)g * a.nchunk + c) * Q + q) * 2]);
  double z = 0.0;
  for (int64_t c = 0; c < a.nchunk; ++c) {
    const double* p = a.part + (((size_t)g * a.nchunk + c) * Q + q) * 2;
    if (p[0] > -__builtin_inf()) z += p[1] * exp(p[0] - m);
  }
  a.mz[((size_t)g * Q + q) * 2] = m;
  a.mz[((size_t)g * Q + q) * 2 + 1] = z;
}

// z = fp32(max of agg over the centred window), and the layer's pool of
// unprotected scores, head after head.
__global__ __launch_bounds__(kAT) void pool_kernel(AttnArgs a) {
  const int64_t N = a.N;
  const int64_t nb = (N + kAT - 1) / kAT;
  const int64_t g = blockIdx.x / nb;
  const int64_t j = (blockIdx.x % nb) * kAT + threadIdx.x;
  if (j >= N) return;
  const int h = a.pool / 2;
  const int64_t lo = j - h > 0 ? j - h : 0;
  const int64_t hi = j + h < N - 1 ? j + h : N - 1;
  const double* ag = a.agg + (size_t)g * N;
  double m = ag[lo];
  for (int64_t i = lo + 1; i <= hi; ++i) m = fmax(m, ag[i]);
  const float z = (float)m;
  a.z[(size_t)g * N + j] = z;
  if (j >= a.s_cnt && j < N - a.r_cnt) {
    const int64_t width = N - a.s_cnt - a.r_cnt;
    a.pool_score[(size_t)g * width + (j - a.s_cnt)] = (double)z;
  }
}

// One block per layer: g_h from the selected pool, then Equation 5.
__global__ __launch_bounds__(kBT) void alloc_kernel(AllocArgs a) {
  __shared__ long long red[kBW];
  __shared__ int cnt[kMaxHeads];
  __shared__ int anynz;
  const int64_t layer = blockIdx.x;
  const int H = a.H;
  const int64_t width = a.width;
  const uint8_t* keep = a.pool_keep + (size_t)layer * H * width;
  const double* sc = a.pool_score + (size_t)layer * H * width;
  if (threadIdx.x == 0) anynz = 0;
  __syncthreads();
  long long nz = 0;
  for (int64_t e = threadIdx.x; e < (int64_t)H * width; e += kBT) nz |= (sc[e] != 0.0) ? 1 : 0;
  nz = block_sum(nz, red);
  for (int hh = 0; hh < H; ++hh) {
    long long c = 0;
    for (int64_t e = threadIdx.x; e < width; e += kBT) c += keep[(size_t)hh * width + e];
    c = block_sum(c, red);
    if (threadIdx.x == 0) cnt[hh] = (int)c;
  }
  if (threadIdx.x == 0) anynz = nz != 0;
  __syncthreads();
  if (threadIdx.x != 0) return;
  const int64_t U = a.U;
  int64_t floor_sum = 0;
  for (int hh = 0; hh < H; ++hh) {
    if (!anynz) cnt[hh] = (int)U;
    floor_sum += (cnt[hh] + U) / 2;
  }
  int64_t R = (int64_t)H * U - floor_sum;
  for (int hh = 0; hh < H; ++hh) {
    const int64_t twice = cnt[hh] + U;
    int64_t u = twice / 2;
    if ((twice & 1) && R > 0) {
      u += 1;
      --R;
    }
    const size_t o = (size_t)layer * H + hh;
    a.capacity[o] = (int32_t)(a.P + u);
    if (a.g_count) a.g_count[o] = cnt[hh];
  }
}

// Allocation skipped (U = 0) or no layer pool: every head keeps B.
__global__ void fill_kernel(int32_t* capacity, int32_t* g_count, int64_t G, int32_t B) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= G) return;
  capacity[i] = B;
  if (g_count) g_count[i] = 0;
}

}  // namespace

hipError_t launch_attn(const AttnArgs& a, int d, int phase, hipStream_t stream) {
  const int64_t blocks = a.G * a.nchunk;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (phase == 1) {
    if (d == 64) hipLaunchKernelGGL((attn_kernel<64, 1>), dim3((unsigned)blocks), dim3(kAT), 0, stream, a);
    else hipLaunchKernelGGL((attn_kernel<128, 1>), dim3((unsigned)blocks), dim3(kAT), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)a.G), dim3(kMaxQueries), 0, stream, a);
  } else {
    if (d == 64) hipLaunchKernelGGL((attn_kernel<64, 2>), dim3((unsigned)blocks), dim3(kAT), 0, stream, a);
    else hipLaunchKernelGGL((attn_kernel<128, 2>), dim3((unsigned)blocks), dim3(kAT), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t nb = (a.N + kAT - 1) / kAT;
    hipLaunchKernelGGL(pool_kernel, dim3((unsigned)(a.G * nb)), dim3(kAT), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_alloc(const AllocArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(alloc_kernel, dim3((unsigned)a.L), dim3(kBT), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_fill_capacity(int32_t* capacity, int32_t* g_count, int64_t G, int32_t B, hipStream_t stream) {
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)((G + 255) / 256)), dim3(256), 0, stream, capacity, g_count, G, B);
  return hipGetLastError();
}

}  // namespace twinkv
