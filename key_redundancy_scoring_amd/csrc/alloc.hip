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
//                      every observing query, logits on the fp64 matrix
//                      cores (exact bf16 products, fp64 sums); per query the
//                      block's max logit and sum of exp(s - max);
//   combine_kernel     per query, the block partials merged into (m, Z);
//   attn_kernel<D, 2>  per key, sum over queries of exp(s - m)/Z, over Gq;
//   pool_kernel        the width-`pool` max, fp32 z;
//   rank_*_kernel      per layer, the threshold of the H*U largest
//                      unprotected z (three radix passes over many blocks),
//                      per head the counts above and at it, then g_h (ties
//                      to the lower head, then position) and Equation 5.
// The logits are recomputed in the second pass rather than stored: storing
// them would take Gq*W*N*8 bytes per head, while recomputing is matrix-core
// work that runs beside the exponentials on the vector units.

#include "internal.h"

namespace twinkv {
namespace {

constexpr int kAT = 256;            // keys per attention block
constexpr int kQG = kMaxQueries / 16;

// Waves per attention block and key groups of 16 per wave (256 keys per
// block either way).  A wave's key operands, widened to fp64, take
// 2*(d/4)*KG registers per lane and its two accumulator sets 16*KG; the
// d = 64 statistics pass keeps four key groups (each query operand read
// feeds four MFMAs), the other passes take two so they keep two waves per
// SIMD.
template <int D, int PHASE>
struct AttnShape {
  static constexpr int KG = (D == 64 && PHASE == 1) ? 4 : 2;
  static constexpr int WAVES = kAT / (16 * KG);
};

typedef double v4d __attribute__((ext_vector_type(4)));

// fp64 DPP moves within rows of 16 lanes (both 32-bit halves).
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)b, CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(b >> 32), CTRL, 0xF, 0xF, false);
  return __longlong_as_double(((long long)hi << 32) | (long long)(unsigned)lo);
}
// Max and sum over the 16 lanes of a row (lane xor 1, xor 2, half-row mirror,
// row mirror); every lane of the row ends with the same value.
__device__ __forceinline__ double row16_max(double v) {
  v = fmax(v, dpp_f64<0xB1>(v));
  v = fmax(v, dpp_f64<0x4E>(v));
  v = fmax(v, dpp_f64<0x141>(v));
  return fmax(v, dpp_f64<0x140>(v));
}
__device__ __forceinline__ double row16_sum(double v) {
  v += dpp_f64<0xB1>(v);
  v += dpp_f64<0x4E>(v);
  v += dpp_f64<0x141>(v);
  return v + dpp_f64<0x140>(v);
}

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// The logits of one block: 256 keys of one head against its Q = Gq*W
// observing queries, on the fp64 matrix cores (v_mfma_f64_16x16x4f64: lane l
// supplies A[l%16][l/16] and B[l/16][l%16] and holds D[l/16 + 4r][l%16],
// r = 0..3, as measured on gfx950).  A tile is 16 queries x 16 keys; a wave
// owns KG key groups (16*KG keys) and walks the query groups.  The feature
// index of step s in lane
// group k is (d/4)k + s, so a lane's operands are contiguous slices of a row.
// The bf16 products are exact in fp64; only the sums round.  The queries are
// staged once per block in LDS as fp32 (exact), in operand order, so each
// wave reads one contiguous 1 KiB per four steps; the keys stay in registers
// as fp32.  Both are widened to fp64 at the matrix core's input.
template <int D, int PHASE>
__global__ __launch_bounds__((64 * AttnShape<D, PHASE>::WAVES)) void attn_kernel(AttnArgs a) {
  constexpr int KS = D / 4;  // k-steps per tile
  constexpr int C8 = D / 8;  // 16-byte chunks per bf16 row
  constexpr int kKG = AttnShape<D, PHASE>::KG;
  constexpr int NW = AttnShape<D, PHASE>::WAVES;
  constexpr int NT = 64 * NW;
  __shared__ float4 qa[kQG * (KS / 4) * 64];
  __shared__ double pm[NW][kMaxQueries];
  __shared__ double pz[NW][kMaxQueries];
  __shared__ double2 smr[kMaxQueries];  // (max, 1 / normaliser)

  const int64_t g = blockIdx.x / a.nchunk;
  const int64_t chunk = blockIdx.x % a.nchunk;
  const int Q = a.Gq * a.W;
  const int nqg = (Q + 15) / 16;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6, kq = lane >> 4;

  {
    const uint4* qsrc = reinterpret_cast<const uint4*>(a.queries) + (size_t)g * Q * C8;
    for (int e = tid; e < nqg * 16 * C8; e += NT) {
      const int qq = e / C8, c = e % C8;
      const uint4 u = qq < Q ? qsrc[(size_t)qq * C8 + c] : make_uint4(0u, 0u, 0u, 0u);
      const int f0 = 8 * c;
      float4* dst = qa + ((qq >> 4) * (KS / 4) + (f0 % KS) / 4) * 64 + (qq & 15) + 16 * (f0 / KS);
      dst[0] = make_float4(bf_lo(u.x), bf_hi(u.x), bf_lo(u.y), bf_hi(u.y));
      dst[64] = make_float4(bf_lo(u.z), bf_hi(u.z), bf_lo(u.w), bf_hi(u.w));
    }
    if (PHASE == 2) {
      for (int q = tid; q < nqg * 16; q += NT) {
        double2 v = make_double2(0.0, 0.0);
        if (q < Q) {
          v.x = a.mz[((size_t)g * Q + q) * 2];
          v.y = 1.0 / a.mz[((size_t)g * Q + q) * 2 + 1];
        }
        smr[q] = v;
      }
    }
  }

  const int64_t N = a.N;
  const int64_t j0 = chunk * kAT + wv * (16 * kKG) + (lane & 15);
  float kb[kKG][KS];
#pragma unroll
  for (int kg = 0; kg < kKG; ++kg) {
    const int64_t j = j0 + 16 * kg;
    const int64_t jl = j < N ? j : N - 1;
    const uint4* src = reinterpret_cast<const uint4*>(a.keys + ((size_t)g * N + jl) * D + KS * kq);
#pragma unroll
    for (int c = 0; c < KS / 8; ++c) {
      const uint4 u = src[c];
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        kb[kg][8 * c + 2 * t] = bf_lo(w[t]);
        kb[kg][8 * c + 2 * t + 1] = bf_hi(w[t]);
      }
    }
  }
  __syncthreads();

  const double scale = a.inv_sqrt_d;
  double agg[kKG] = {};
  // The logits of query group qg into acc.
  auto mfma_group = [&](int qg, v4d(&acc)[kKG]) __attribute__((always_inline)) {
#pragma unroll
    for (int kg = 0; kg < kKG; ++kg) acc[kg] = v4d{0.0, 0.0, 0.0, 0.0};
    const float4* ap = qa + qg * (KS / 4) * 64 + lane;
#pragma unroll
    for (int s4 = 0; s4 < KS / 4; ++s4) {
      const float4 av = ap[s4 * 64];
      const float af[4] = {av.x, av.y, av.z, av.w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int kg = 0; kg < kKG; ++kg)
          acc[kg] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)af[u], (double)kb[kg][4 * s4 + u], acc[kg], 0, 0, 0);
      }
    }
  };
  // The softmax work of query group qg, without branches: a masked logit
  // enters the exponential as -inf, which gives 0.  Phase 1 leaves each
  // row's (max, sum) in pmv/pzv for store().
  double pmv[4], pzv[4];
  auto epilogue = [&](int qg, const v4d(&acc)[kKG]) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int q = qg * 16 + kq + 4 * r;
      const int64_t tq = N - a.W + (q % a.W);
      double v[kKG];
      bool ok[kKG];
#pragma unroll
      for (int kg = 0; kg < kKG; ++kg) {
        const int64_t j = j0 + 16 * kg;
        ok[kg] = q < Q && j < N && j <= tq;
        v[kg] = acc[kg][r] * scale;
      }
      if (PHASE == 1) {
        double m = -__builtin_inf();
#pragma unroll
        for (int kg = 0; kg < kKG; ++kg) m = fmax(m, ok[kg] ? v[kg] : -__builtin_inf());
        m = row16_max(m);
        double z = 0.0;
#pragma unroll
        for (int kg = 0; kg < kKG; ++kg) z += exp(ok[kg] ? v[kg] - m : -__builtin_inf());
        pmv[r] = m;
        pzv[r] = row16_sum(z);
      } else {
        const double2 mr = smr[q];
#pragma unroll
        for (int kg = 0; kg < kKG; ++kg) agg[kg] += exp(ok[kg] ? v[kg] - mr.x : -__builtin_inf()) * mr.y;
      }
    }
  };
  auto store = [&](int qg) __attribute__((always_inline)) {
    if (PHASE == 1 && (lane & 15) == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int q = qg * 16 + kq + 4 * r;
        if (q < Q) {
          pm[wv][q] = pmv[r];
          pz[wv][q] = pzv[r];
        }
      }
    }
  };
  // Spread one query group's epilogue over the next group's MFMAs.
  auto interleave = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < KS * kKG; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // up to six VALU
    }
  };
  // Software pipeline over the query groups: the MFMAs of group qg+1 run
  // while the vector units do group qg's exponentials.
  v4d accA[kKG], accB[kKG];
  mfma_group(0, accA);
  int qg = 0;
#pragma unroll 1
  for (; qg + 2 < nqg; qg += 2) {
    mfma_group(qg + 1, accB);
    epilogue(qg, accA);
    interleave();
    store(qg);
    mfma_group(qg + 2, accA);
    epilogue(qg + 1, accB);
    interleave();
    store(qg + 1);
  }
  if (qg + 1 < nqg) {
    mfma_group(qg + 1, accB);
    epilogue(qg, accA);
    interleave();
    store(qg);
    epilogue(qg + 1, accB);
    store(qg + 1);
  } else {
    epilogue(qg, accA);
    store(qg);
  }

  if (PHASE == 1) {
    __syncthreads();
    for (int q = tid; q < Q; q += NT) {
      double m = -__builtin_inf();
#pragma unroll
      for (int w = 0; w < NW; ++w) m = fmax(m, pm[w][q]);
      double z = 0.0;
      if (m > -__builtin_inf()) {
#pragma unroll
        for (int w = 0; w < NW; ++w)
          if (pm[w][q] > -__builtin_inf()) z += pz[w][q] * exp(pm[w][q] - m);
      }
      double* dst = a.part + (((size_t)g * a.nchunk + chunk) * Q + q) * 2;
      dst[0] = m;
      dst[1] = z;
    }
  } else {
    // the four lane groups of a column hold disjoint query rows of one key
#pragma unroll
    for (int kg = 0; kg < kKG; ++kg) {
      agg[kg] += __shfl_xor(agg[kg], 16);
      agg[kg] += __shfl_xor(agg[kg], 32);
      const int64_t j = j0 + 16 * kg;
      if (kq == 0 && j < N) a.agg[(size_t)g * N + j] = agg[kg] * a.inv_gq;
    }
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

// z = fp32(max of agg over the centred window).
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
  a.z[(size_t)g * N + j] = (float)m;
}

// The layer-wide ranking of the unprotected z, by a radix select on their
// fp32 bit patterns (z >= 0, so the bits order as the values).  Three passes
// over bits 31..21, 20..10 and 9..0 find T, the (H*U)-th largest unprotected
// z of each layer, and `need`, how many of the entries equal to T the top
// H*U takes.  Then each head counts its entries above and equal to T.  Equal
// scores go to the lower head first (then the lower position, which does not
// change a count), so g_h = above_h + the part of `need` that the heads
// before h have not used, capped at equal_h.
constexpr int kRankBins = 2048;
constexpr int kRT = 256;
constexpr int kRPer = 16;
constexpr int kRChunk = kRT * kRPer;  // entries per ranking block

__device__ __forceinline__ int rank_shift(int pass) { return pass == 0 ? 21 : (pass == 1 ? 10 : 0); }
__device__ __forceinline__ int rank_bits(int pass) { return pass == 2 ? 10 : 11; }

__global__ void rank_init_kernel(AllocArgs a) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < a.L * kRankBins) a.hist[i] = 0u;
  if (i < a.G * 3) a.counts[i] = 0u;
  if (i < a.L) {
    a.prefix[i] = 0u;
    a.need[i] = (int64_t)a.H * a.U;
  }
}

// Digit histogram of the entries that match the threshold bits found so far.
__global__ __launch_bounds__(kRT) void rank_hist_kernel(AllocArgs a, int pass) {
  __shared__ uint32_t h[kRankBins];
  const int64_t nb = (a.width + kRChunk - 1) / kRChunk;
  const int64_t g = blockIdx.x / nb;
  const int64_t e0 = (blockIdx.x % nb) * kRChunk;
  const int64_t layer = g / a.H;
  for (int i = threadIdx.x; i < kRankBins; i += kRT) h[i] = 0u;
  __syncthreads();
  const int sh = rank_shift(pass), top = sh + rank_bits(pass);
  const uint32_t mask = (1u << rank_bits(pass)) - 1u;
  const uint32_t pre = a.prefix[layer];
  const float* zg = a.z + (size_t)g * a.N + a.s_cnt;
  for (int t = 0; t < kRPer; ++t) {
    const int64_t e = e0 + t * kRT + threadIdx.x;
    if (e < a.width) {
      const uint32_t key = __float_as_uint(zg[e]);
      if (top == 32 || (key >> top) == (pre >> top)) atomicAdd(&h[(key >> sh) & mask], 1u);
    }
  }
  __syncthreads();
  uint32_t* gh = a.hist + (size_t)layer * kRankBins;
  for (int i = threadIdx.x; i < kRankBins; i += kRT)
    if (h[i]) atomicAdd(&gh[i], h[i]);
}

// One block per layer: the digit of the bin that holds the need-th largest
// matching entry, and what remains to take inside it; clears the histogram
// for the next pass.
__global__ __launch_bounds__(kRT) void rank_scan_kernel(AllocArgs a, int pass) {
  __shared__ uint32_t wsum[kRT / 64];
  const int64_t layer = blockIdx.x;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int nb = 1 << rank_bits(pass), per = nb / kRT;
  uint32_t* gh = a.hist + (size_t)layer * kRankBins;
  const int64_t need = a.need[layer];
  const uint32_t pre = a.prefix[layer];
  // thread t owns bins nb-1-per*t down to nb-per*(t+1), highest first
  uint32_t c[kRankBins / kRT];
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < kRankBins / kRT; ++i) {
    c[i] = i < per ? gh[nb - 1 - per * t - i] : 0u;
    s += c[i];
  }
  uint32_t inc = s;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t v = __shfl_up(inc, off);
    if (lane >= off) inc += v;
  }
  if (lane == 63) wsum[wv] = inc;
  __syncthreads();
  uint32_t before = 0;
  for (int w = 0; w < wv; ++w) before += wsum[w];
  const int64_t excl = (int64_t)before + inc - s;
  if (excl < need && need <= excl + (int64_t)s) {
    int64_t run = excl;
    for (int i = 0; i < per; ++i) {
      if (run + c[i] >= need) {
        a.prefix[layer] = pre | ((uint32_t)(nb - 1 - per * t - i) << rank_shift(pass));
        a.need[layer] = need - run;
        break;
      }
      run += c[i];
    }
  }
  for (int i = 0; i < per; ++i) gh[nb - 1 - per * t - i] = 0u;
}

// Per head: entries above the layer's threshold, equal to it, and nonzero.
__global__ __launch_bounds__(kRT) void rank_count_kernel(AllocArgs a) {
  __shared__ uint32_t red[3][kRT / 64];
  const int64_t nb = (a.width + kRChunk - 1) / kRChunk;
  const int64_t g = blockIdx.x / nb;
  const int64_t e0 = (blockIdx.x % nb) * kRChunk;
  const uint32_t T = a.prefix[g / a.H];
  const float* zg = a.z + (size_t)g * a.N + a.s_cnt;
  uint32_t v[3] = {0u, 0u, 0u};
  for (int t = 0; t < kRPer; ++t) {
    const int64_t e = e0 + t * kRT + threadIdx.x;
    if (e < a.width) {
      const uint32_t key = __float_as_uint(zg[e]);
      v[0] += key > T;
      v[1] += key == T;
      v[2] += key != 0u;
    }
  }
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int k = 0; k < 3; ++k) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v[k] += __shfl_xor(v[k], off);
    if (lane == 0) red[k][wv] = v[k];
  }
  __syncthreads();
  if (threadIdx.x < 3) {
    uint32_t tot = 0;
    for (int w = 0; w < kRT / 64; ++w) tot += red[threadIdx.x][w];
    if (tot) atomicAdd(&a.counts[(size_t)g * 3 + threadIdx.x], tot);
  }
}

// One thread per layer: g_h from the counts and the threshold's remaining
// take, then Equation 5.
__global__ void rank_alloc_kernel(AllocArgs a) {
  const int64_t layer = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (layer >= a.L) return;
  const int H = a.H;
  const uint32_t* cnt = a.counts + (size_t)layer * H * 3;
  bool anynz = false;
  for (int hh = 0; hh < H; ++hh) anynz |= cnt[3 * hh + 2] != 0u;
  const int64_t U = a.U;
  int64_t floor_sum = 0;
  int64_t need = a.need[layer];
  for (int hh = 0; hh < H; ++hh) {
    const int64_t take = need < (int64_t)cnt[3 * hh + 1] ? need : (int64_t)cnt[3 * hh + 1];
    need -= take;
    const int64_t gh = anynz ? (int64_t)cnt[3 * hh] + take : U;
    floor_sum += (gh + U) / 2;
  }
  int64_t R = (int64_t)H * U - floor_sum;
  need = a.need[layer];
  for (int hh = 0; hh < H; ++hh) {
    const int64_t take = need < (int64_t)cnt[3 * hh + 1] ? need : (int64_t)cnt[3 * hh + 1];
    need -= take;
    const int64_t gh = anynz ? (int64_t)cnt[3 * hh] + take : U;
    const int64_t twice = gh + U;
    int64_t u = twice / 2;
    if ((twice & 1) && R > 0) {
      u += 1;
      --R;
    }
    const size_t o = (size_t)layer * H + hh;
    a.capacity[o] = (int32_t)(a.P + u);
    if (a.g_count) a.g_count[o] = (int32_t)gh;
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
    if (d == 64)
      hipLaunchKernelGGL((attn_kernel<64, 1>), dim3((unsigned)blocks), dim3(64 * AttnShape<64, 1>::WAVES), 0, stream, a);
    else
      hipLaunchKernelGGL((attn_kernel<128, 1>), dim3((unsigned)blocks), dim3(64 * AttnShape<128, 1>::WAVES), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)a.G), dim3(kMaxQueries), 0, stream, a);
  } else {
    if (d == 64)
      hipLaunchKernelGGL((attn_kernel<64, 2>), dim3((unsigned)blocks), dim3(64 * AttnShape<64, 2>::WAVES), 0, stream, a);
    else
      hipLaunchKernelGGL((attn_kernel<128, 2>), dim3((unsigned)blocks), dim3(64 * AttnShape<128, 2>::WAVES), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t nb = (a.N + kAT - 1) / kAT;
    hipLaunchKernelGGL(pool_kernel, dim3((unsigned)(a.G * nb)), dim3(kAT), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_alloc(const AllocArgs& a, hipStream_t stream) {
  const int64_t nb = (a.width + kRChunk - 1) / kRChunk;
  const int64_t blocks = a.G * nb;
  if (blocks < 1 || blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  int64_t init = a.L * kRankBins;
  if (a.G * 3 > init) init = a.G * 3;
  hipLaunchKernelGGL(rank_init_kernel, dim3((unsigned)((init + 255) / 256)), dim3(256), 0, stream, a);
  for (int pass = 0; pass < 3; ++pass) {
    hipLaunchKernelGGL(rank_hist_kernel, dim3((unsigned)blocks), dim3(kRT), 0, stream, a, pass);
    hipLaunchKernelGGL(rank_scan_kernel, dim3((unsigned)a.L), dim3(kRT), 0, stream, a, pass);
  }
  hipLaunchKernelGGL(rank_count_kernel, dim3((unsigned)blocks), dim3(kRT), 0, stream, a);
  hipLaunchKernelGGL(rank_alloc_kernel, dim3((unsigned)((a.L + 63) / 64)), dim3(64), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_fill_capacity(int32_t* capacity, int32_t* g_count, int64_t G, int32_t B, hipStream_t stream) {
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)((G + 255) / 256)), dim3(256), 0, stream, capacity, g_count, G, B);
  return hipGetLastError();
}

}  // namespace twinkv
