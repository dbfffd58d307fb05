// Physical cache layout after selection ("Small Frequency Corrections Can
// Change What Survives KV Cache Compression", section 3.4): the retained
// keys and values of every head, in sequence order, packed head after head
// with no padding, so equal-quota heads form contiguous slices of one tensor
// and the payload is exactly 2*d*sum(b_h) elements.  Keys are copied as they
// are (no re-rotation) and values unchanged.
//
// A copy kernel bound by HBM bandwidth: CH = d/8 consecutive lanes move one
// key row (d bf16 = CH 16-byte chunks), so every wave reads and writes whole
// contiguous rows.  The grid is folded over heads: block (g, x) copies rows
// [x*RPB, (x+1)*RPB) of head g's retained list; blocks past the head's count
// exit at once.  Every index is clamped to the sizes the caller states, so
// inconsistent offsets cannot send an access outside the buffers.

#include "internal.h"

namespace twinkv {
namespace {

constexpr int kGT = 256;  // threads per block
constexpr int kPasses = 4;

typedef unsigned u4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_nt(const uint4* p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u4v*>(p)));
}
__device__ __forceinline__ void store_nt(uint4* p, uint4 v) {
  __builtin_nontemporal_store(__builtin_bit_cast(u4v, v), reinterpret_cast<u4v*>(p));
}

template <int CH>
__global__ __launch_bounds__(kGT) void gather_kv_kernel(const uint4* __restrict__ keys, const uint4* __restrict__ values,
                                                        const int32_t* __restrict__ kept_idx,
                                                        const int64_t* __restrict__ kept_off, int64_t G, int64_t N,
                                                        int64_t total, int64_t bph, uint4* __restrict__ out_keys,
                                                        uint4* __restrict__ out_values) {
  constexpr int RPP = kGT / CH;  // rows per pass
  constexpr int RPB = RPP * kPasses;
  const int64_t g = blockIdx.x / bph;
  const int64_t x = blockIdx.x % bph;
  if (g >= G) return;
  int64_t o0 = kept_off[g];
  int64_t o1 = kept_off[g + 1];
  o0 = o0 < 0 ? 0 : (o0 > total ? total : o0);
  o1 = o1 < o0 ? o0 : (o1 > total ? total : o1);
  const int64_t cnt = (o1 - o0) < N ? (o1 - o0) : N;
  const int64_t r0 = x * RPB;
  if (r0 >= cnt) return;
  const int c = threadIdx.x % CH;
  // the indices, then every row's loads, then the stores: 2 * kPasses
  // 16-byte loads in flight per lane; source and destination are touched
  // once, so loads and stores are nontemporal
  int64_t src[kPasses];
  bool ok[kPasses];
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const int64_t row = r0 + p * RPP + threadIdx.x / CH;
    ok[p] = row < cnt;
    int64_t i = ok[p] ? kept_idx[o0 + row] : 0;
    i = i < 0 ? 0 : (i >= N ? N - 1 : i);
    src[p] = (g * N + i) * CH + c;
  }
  uint4 kv[kPasses], vv[kPasses];
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    if (ok[p]) {
      kv[p] = load_nt(keys + src[p]);
      if (values) vv[p] = load_nt(values + src[p]);
    }
  }
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    if (ok[p]) {
      const int64_t dst = (o0 + r0 + p * RPP + threadIdx.x / CH) * CH + c;
      store_nt(out_keys + dst, kv[p]);
      if (values) store_nt(out_values + dst, vv[p]);
    }
  }
}

}  // namespace

hipError_t launch_gather_kv(const uint16_t* keys, const uint16_t* values, const int32_t* kept_idx,
                            const int64_t* kept_off, int64_t G, int64_t N, int d, int64_t total, uint16_t* out_keys,
                            uint16_t* out_values, hipStream_t stream) {
  if (total == 0) return hipSuccess;
  const int CH = d / 8;
  const int64_t rpb = (kGT / CH) * kPasses;
  const int64_t bph = (N + rpb - 1) / rpb;
  const int64_t blocks = G * bph;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const uint4* k = reinterpret_cast<const uint4*>(keys);
  const uint4* v = reinterpret_cast<const uint4*>(values);
  uint4* ok = reinterpret_cast<uint4*>(out_keys);
  uint4* ov = reinterpret_cast<uint4*>(out_values);
  if (d == 64)
    gather_kv_kernel<8><<<dim3((unsigned)blocks), dim3(kGT), 0, stream>>>(k, v, kept_idx, kept_off, G, N, total, bph,
                                                                         ok, ov);
  else
    gather_kv_kernel<16><<<dim3((unsigned)blocks), dim3(kGT), 0, stream>>>(k, v, kept_idx, kept_off, G, N, total, bph,
                                                                          ok, ov);
  return hipGetLastError();
}

}  // namespace twinkv
