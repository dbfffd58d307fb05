// Fused Gram sweep: for every row i of a head, reduce the row of cosine
// similarities against a column set to
//   * the nonlocal twin count c_i = #{ j : |i-j| > w, sim(i,j) > tau }
//     ("TwinKV: A Composable Repair Pass ...", section 3.2, Eq. 2; "Small
//     Frequency Corrections ...", section 3.2), score mode only;
//   * the best nonlocal twin b_i = max sim(i,j) over the same j and its lowest
//     position a_i; in repair mode the columns are the retained set S0, which
//     gives b_i(S0) of Eq. 4 ("TwinKV ...", section 3.4);
// and, in score mode, the discounted score e_i * ln((N+1)/(c_i+1)) ("Small
// Frequency Corrections ...", section 3.2).  The N x N similarity matrix is
// never written anywhere.
//
// Mapping onto gfx950:
//   * A workgroup is 4 waves and owns 512 consecutive rows of one head; each
//     wave owns 4 blocks of 32 rows whose bf16 keys stay in VGPRs as MFMA
//     B operands for the whole sweep.
//   * Column keys stream through LDS in stages of 64 columns (double
//     buffered, one barrier per stage).  16-byte chunks are XOR-swizzled by
//     the column's low 3 bits so the MFMA A-operand reads are spread over banks.
//   * v_mfma_f32_32x32x16_bf16 with A = 32 column keys, B = 32 row keys gives
//     lane l the row (l mod 32) and 16 columns 8*(r/4) + 4*(l/32) + (r mod 4)
//     in accumulator r, so all reductions over columns stay inside a lane.
//   * Epilogue per 32x32 tile and lane: y = dot * (1/||k_j||) (16 mul), the
//     tile maximum by a 3-input max tree (8 ops), then one compare and two
//     selects record (running max, tile index).  The count needs y > tau*||k_i||
//     and runs only when the tile maximum crosses that threshold (rare: twins
//     are sparse).  The |i-j| <= w band and the ragged tail take a masked
//     variant on the few tiles that touch them.
//   * Which of the 16 columns of the winning tile holds the maximum is not
//     tracked in the sweep; after it, each lane recomputes its 16 candidates
//     exactly in fp64 (bf16 products are exact) and keeps the largest, lowest
//     position on ties; the two half-waves that share a row then merge.  This
//     also makes b_i the exact fp64 cosine dot/sqrt(n_i*n_j) of the chosen pair.
//   * Workgroup ids are remapped so each XCD (ids are dealt round-robin over
//     8 XCDs) receives a contiguous run of row blocks: the blocks of one head
//     sweep its key stream together out of one L2.
#include <limits.h>

#include "internal.h"

namespace twinkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWaves = 4;
constexpr int kRowBlocks = 4;  // 32-row blocks per wave
constexpr int kStageCols = 64;
constexpr int kTilesPerStage = kStageCols / 32;
static_assert(kWaves * kRowBlocks * 32 == kGramRowsPerWG, "row split");

template <int D>
struct Smem {
  uint4 keys[2][kStageCols * (D / 8)];
  float rinv[2][kStageCols];
  int32_t pos[2][kStageCols];
};

__device__ __forceinline__ float max3f(float a, float b, float c) { return __builtin_fmaxf(a, __builtin_fmaxf(b, c)); }

__device__ __forceinline__ double dot8_exact(uint4 a, uint4 b) {
  const uint32_t x[4] = {a.x, a.y, a.z, a.w};
  const uint32_t y[4] = {b.x, b.y, b.z, b.w};
  double s = 0.0;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    s += (double)(__uint_as_float(x[t] << 16) * __uint_as_float(y[t] << 16));
    s += (double)(__uint_as_float(x[t] & 0xffff0000u) * __uint_as_float(y[t] & 0xffff0000u));
  }
  return s;
}

// column offset (within a 32-column tile) of accumulator r in half-wave h
__device__ __forceinline__ int tile_col(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

template <int D, int MODE>
__global__ __launch_bounds__(256, 1) void gram_kernel(GramArgs a) {
  constexpr int CH = D / 8;       // 16-byte chunks per key row
  constexpr int KS = D / 16;      // MFMA k-steps
  constexpr int LOADS = kStageCols * CH / 256;
  __shared__ Smem<D> sm;

  const int64_t N = a.N;
  const int64_t bph = (N + kGramRowsPerWG - 1) / kGramRowsPerWG;
  const int64_t total = a.G * bph;
  const int64_t per_xcd = (total + 7) / 8;
  const int64_t logical = (int64_t)(blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (logical >= total) return;
  const int64_t g = logical / bph;
  const int64_t rb = logical % bph;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;
  const int lrow = lane & 31;
  const int w = a.window;
  const int row0 = (int)(rb * kGramRowsPerWG) + wave * (kRowBlocks * 32);

  const uint4* Kg = reinterpret_cast<const uint4*>(a.keys) + (size_t)g * N * CH;
  const float* rinv_g = a.rinv + (size_t)g * N;
  const int32_t* pos_g = (MODE == GRAM_REPAIR) ? a.pos + (size_t)g * N : nullptr;
  const int ncols = (MODE == GRAM_REPAIR) ? a.ncols[g] : (int)N;

  // ---- row keys as MFMA B operands, row state
  bf16x8 brow[kRowBlocks][KS];
  float thr[kRowBlocks], best[kRowBlocks];
  int btile[kRowBlocks], cnt[kRowBlocks];
#pragma unroll
  for (int b = 0; b < kRowBlocks; ++b) {
    const int i = row0 + 32 * b + lrow;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      uint4 v = {0u, 0u, 0u, 0u};
      if (i < N) v = Kg[(size_t)i * CH + 2 * s + h];
      brow[b][s] = __builtin_bit_cast(bf16x8, v);
    }
    thr[b] = (i < N) ? (float)(a.tau * sqrt(a.nsq[(size_t)g * N + i])) : __builtin_inff();
    best[b] = -__builtin_inff();
    btile[b] = -1;
    cnt[b] = 0;
  }

  // ---- stage loader: global -> registers -> LDS
  uint4 pre[LOADS];
  float pre_r = 0.0f;
  int32_t pre_p = INT_MAX;
  auto fetch = [&](int64_t col0) {
#pragma unroll
    for (int t = 0; t < LOADS; ++t) {
      const int q = tid + 256 * t;
      const int c = q / CH, k = q % CH;
      const int64_t col = col0 + c;
      uint4 v = {0u, 0u, 0u, 0u};
      if (col < ncols) {
        const int64_t row = (MODE == GRAM_REPAIR) ? pos_g[col] : col;
        v = Kg[(size_t)row * CH + k];
      }
      pre[t] = v;
    }
    if (tid < kStageCols) {
      const int64_t col = col0 + tid;
      pre_r = 0.0f;
      pre_p = INT_MAX;
      if (col < ncols) {
        const int64_t row = (MODE == GRAM_REPAIR) ? pos_g[col] : col;
        pre_r = rinv_g[row];
        pre_p = (int32_t)row;
      }
    }
  };
  auto commit = [&](int buf) {
#pragma unroll
    for (int t = 0; t < LOADS; ++t) {
      const int q = tid + 256 * t;
      const int c = q / CH, k = q % CH;
      sm.keys[buf][c * CH + (k ^ (c & 7))] = pre[t];
    }
    if (tid < kStageCols) {
      sm.rinv[buf][tid] = pre_r;
      sm.pos[buf][tid] = pre_p;
    }
  };

  const int nstages = (ncols + kStageCols - 1) / kStageCols;
  if (nstages > 0) {
    fetch(0);
    commit(0);
  }
  __syncthreads();

  for (int st = 0; st < nstages; ++st) {
    const int buf = st & 1;
    if (st + 1 < nstages) fetch((int64_t)(st + 1) * kStageCols);

#pragma unroll
    for (int tt = 0; tt < kTilesPerStage; ++tt) {
      const int cb = tt * 32;  // first column of the tile inside the stage
      const int tile = st * kTilesPerStage + tt;
      const int c0 = tile * 32;
      bf16x8 A[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int c = cb + lrow;
        const int k = 2 * s + h;
        A[s] = __builtin_bit_cast(bf16x8, sm.keys[buf][c * CH + (k ^ (c & 7))]);
      }
      float rv[16];
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const float4 r4 = *reinterpret_cast<const float4*>(&sm.rinv[buf][cb + 8 * gq + 4 * h]);
        rv[4 * gq + 0] = r4.x;
        rv[4 * gq + 1] = r4.y;
        rv[4 * gq + 2] = r4.z;
        rv[4 * gq + 3] = r4.w;
      }
      int pmin, pmax;
      if (MODE == GRAM_REPAIR) {
        pmin = __builtin_amdgcn_readfirstlane(sm.pos[buf][cb]);
        pmax = __builtin_amdgcn_readfirstlane(sm.pos[buf][cb + 31]);
      } else {
        pmin = c0;
        pmax = c0 + 31;
      }
      const bool tail = (c0 + 31 >= ncols);

#pragma unroll
      for (int b = 0; b < kRowBlocks; ++b) {
        f32x16 acc = {};
#pragma unroll
        for (int s = 0; s < KS; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[s], brow[b][s], acc, 0, 0, 0);
        float y[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) y[r] = acc[r] * rv[r];

        const int r0 = row0 + 32 * b;
        const bool masked = tail || (pmin <= r0 + 31 + w && pmax >= r0 - w);
        if (masked) {
          const int i = r0 + lrow;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int q = tile_col(r, h);
            const int col = c0 + q;
            const int j = (MODE == GRAM_REPAIR) ? sm.pos[buf][cb + q] : col;
            const int dist = i > j ? i - j : j - i;
            if (!(col < ncols && dist > w)) y[r] = -__builtin_inff();
          }
        }
        const float m01 = max3f(y[0], y[1], y[2]);
        const float m02 = max3f(y[3], y[4], y[5]);
        const float m03 = max3f(y[6], y[7], y[8]);
        const float m04 = max3f(y[9], y[10], y[11]);
        const float m05 = max3f(y[12], y[13], y[14]);
        const float m11 = max3f(m01, m02, m03);
        const float m12 = max3f(m04, m05, y[15]);
        const float m = __builtin_fmaxf(m11, m12);
        if (m > best[b]) {
          best[b] = m;
          btile[b] = tile;
        }
        if (MODE == GRAM_SCORE) {
          if (m > thr[b]) {
            int c = 0;
#pragma unroll
            for (int r = 0; r < 16; ++r) c += (y[r] > thr[b]) ? 1 : 0;
            cnt[b] += c;
          }
        }
      }
    }

    if (st + 1 < nstages) commit(buf ^ 1);
    __syncthreads();
  }

  // ---- exact fp64 fixup of the best twin, merge of half-waves, outputs
#pragma unroll 1
  for (int b = 0; b < kRowBlocks; ++b) {
    const int i = row0 + 32 * b + lrow;
    const bool row_ok = i < N;
    double bb = -1.0;
    int aa = -1;
    if (row_ok && btile[b] >= 0) {
      const double ni = a.nsq[(size_t)g * N + i];
      const uint4* ki = Kg + (size_t)i * CH;
#pragma unroll 1
      for (int r = 0; r < 16; ++r) {
        const int col = btile[b] * 32 + tile_col(r, h);
        if (col >= ncols) continue;
        const int j = (MODE == GRAM_REPAIR) ? pos_g[col] : col;
        const int dist = i > j ? i - j : j - i;
        if (dist <= w) continue;
        const uint4* kj = Kg + (size_t)j * CH;
        double dot = 0.0;
#pragma unroll
        for (int k = 0; k < CH; ++k) dot += dot8_exact(ki[k], kj[k]);
        const double nn = ni * a.nsq[(size_t)g * N + j];
        double sim = nn > 0.0 ? dot / sqrt(nn) : 0.0;
        sim += 0.0;
        if (aa < 0 || sim > bb || (sim == bb && j < aa)) {
          bb = sim;
          aa = j;
        }
      }
    }
    const double pb = __shfl_xor(bb, 32);
    const int pa = __shfl_xor(aa, 32);
    if (pa >= 0 && (aa < 0 || pb > bb || (pb == bb && pa < aa))) {
      bb = pb;
      aa = pa;
    }
    int c = 0;
    if (MODE == GRAM_SCORE) c = cnt[b] + __shfl_xor(cnt[b], 32);
    if (h == 0 && row_ok) {
      const size_t o = (size_t)g * N + i;
      a.best_sim[o] = bb;
      a.best_idx[o] = aa;
      if (MODE == GRAM_SCORE) {
        if (a.tau < 0.0 && a.nsq[o] == 0.0) {
          // a zero key has cosine 0 with every key: all nonlocal positions count
          const int64_t lo = i - w > 0 ? i - w : 0;
          const int64_t hi = i + w < N - 1 ? i + w : N - 1;
          c = (int)(N - (hi - lo + 1));
        }
        a.count[o] = c;
        const double disc = log((double)(N + 1) / (double)(c + 1));
        a.score[o] = a.energy[o] * disc;
        if (a.omega) a.omega[o] = disc / log((double)(N + 1));
      }
    }
  }
}

template <int D, int MODE>
hipError_t launch_dm(const GramArgs& a, hipStream_t stream) {
  const int64_t bph = (a.N + kGramRowsPerWG - 1) / kGramRowsPerWG;
  const int64_t total = a.G * bph;
  const int64_t grid = 8 * ((total + 7) / 8);
  if (grid > INT_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gram_kernel<D, MODE>), dim3((unsigned)grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gram(const GramArgs& a, int mode, hipStream_t stream) {
  if (a.d == 64) return mode == GRAM_SCORE ? launch_dm<64, GRAM_SCORE>(a, stream) : launch_dm<64, GRAM_REPAIR>(a, stream);
  return mode == GRAM_SCORE ? launch_dm<128, GRAM_SCORE>(a, stream) : launch_dm<128, GRAM_REPAIR>(a, stream);
}

}  // namespace twinkv
