// Single-order score sweep: the nonlocal twin count c_i = #{ j : |i-j| > w,
// sim(i,j) > tau } and the best nonlocal twin (b_i, a_i) of every position
// ("TwinKV: A Composable Repair Pass ...", section 3.2, Eq. 1 and Eq. 2;
// "Small Frequency Corrections ...", section 3.2), with every unordered
// nonlocal pair {i, j} evaluated once, and the discounted score
// e_i * ln((N+1)/(c_i+1)) ("Small Frequency Corrections ...", section 3.2).
//
// A pair i < j with j - i > w is evaluated in the workgroup that owns i's
// row block, which sweeps the columns from its own first row to the end.
// Its value serves both ends:
//   * the row side (i's maximum over later j, the count of i) stays in the
//     lane that holds row i, as in the repair pass's sweep: y = dot / ||k_j||,
//     a 3-input max tree per 32x32 block and a running (maximum, first tile)
//     per half-row;
//   * the column side (j's maximum over the block's rows) is scaled to the
//     cosine, merged over the wave's row blocks in each lane, then over the
//     32 lanes that share a column set (DPP row mirrors whose bank masks
//     write each column only into the lanes that keep it, a
//     v_permlane16_swap step across rows, then quad reductions), then over
//     the workgroup's waves in LDS, and stored per (row block, column); its
//     counts are added atomically (rare: only when some element of a block
//     crosses tau).
// The resolve kernels then take, for every position, the largest of its row
// side and of the column maxima of the row blocks before it, mark the
// blocks whose maximum is within a margin of it, and re-sweep each such
// block against just those positions to find the exact fp64 best twin.  The
// row side's own best is made exact at the end of the sweep (the fused
// fixup) over the first tile attaining each half-row's maximum; a row where
// another tile comes within twice the fp32 error of that maximum is queued
// for the exact resolve of resolve.hip instead.  Both sides merge through a
// 64-bit atomic maximum of (exact cosine, position) in which the low bits of
// the order-preserving image of the cosine carry the position, so equal
// cosines go to the lowest position.  A workgroup sweeps two row blocks, rb
// and nb-1-rb, so every workgroup covers about the same number of columns.
#include <limits.h>

#include "sweep.h"

namespace twinkv {
namespace {

// d = 64: three row blocks of 32 per wave (96 rows), 384 rows per workgroup,
// 256-column stages; 256 VGPRs at two waves per SIMD.  Four row blocks spill
// with the column-side registers (and one wave per SIMD is slower).
using TriShape64 = GramShape<64, 3, 4, 256, 2>;
using TriShape128 = GramShape<128, 2, 4, 128, 2>;

// screening margin in cosine units: far above the fp32 error of a dot product
// of at most 128 exact bf16 products scaled by fp32 inverse norms (below 1e-5)
constexpr float kMargin = 8e-5f;
// A tile whose fp32 maximum stays more than this (cosine units) below the
// row's cannot hold the exact best: it exceeds twice the fp32 error of one
// candidate (below 7.7e-6 at d = 128).  Rows where another tile comes closer
// go to the exact resolve.
constexpr float kTieMargin = 2e-5f;

// Column maxima of a tile over the 32 lanes of each half-wave.  The 16
// accumulator values of a lane are 16 columns (tile_col(r, h)) of the lane's
// row; the 32 lanes of a half-wave share those columns.  Inside a 16-lane
// row, lane p pairs with 15 - p and then with 7 - p (DPP mirrors): of each
// pair of values the lanes keep one column, and the DPP bank mask (a bank is
// a group of four lanes of a row) writes each column only into the lanes
// that keep it, so no lane selects are needed.  A swap across the rows then
// pairs lanes l and l^16 on the four values left, and the last two pairings,
// inside 4-lane quads, reduce fully.  On return every lane holds the maxima
// of column slots s and s + 8, s = 4*b4 + 2*b2 + b3 (bk: bit k of the lane
// id).  The DPP reads follow their inputs' writes by the two wait states the
// hardware requires.
__device__ __forceinline__ void reduce_cols(const float (&v)[16], float& c0, float& c1) {
  float a0, a1, a2, a3, a4, a5, a6, a7;
  // lanes 0-7 of a row keep the even slot of each pair, lanes 8-15 the odd
  asm("s_nop 1\n\t"
      "v_max_f32_dpp %0, %8, %8 row_mirror row_mask:0xf bank_mask:0x3\n\t"
      "v_max_f32_dpp %0, %9, %9 row_mirror row_mask:0xf bank_mask:0xc\n\t"
      "v_max_f32_dpp %1, %10, %10 row_mirror row_mask:0xf bank_mask:0x3\n\t"
      "v_max_f32_dpp %1, %11, %11 row_mirror row_mask:0xf bank_mask:0xc\n\t"
      "v_max_f32_dpp %2, %12, %12 row_mirror row_mask:0xf bank_mask:0x3\n\t"
      "v_max_f32_dpp %2, %13, %13 row_mirror row_mask:0xf bank_mask:0xc\n\t"
      "v_max_f32_dpp %3, %14, %14 row_mirror row_mask:0xf bank_mask:0x3\n\t"
      "v_max_f32_dpp %3, %15, %15 row_mirror row_mask:0xf bank_mask:0xc\n\t"
      "v_max_f32_dpp %4, %16, %16 row_mirror row_mask:0xf bank_mask:0x3\n\t"
      "v_max_f32_dpp %4, %17, %17 row_mirror row_mask:0xf bank_mask:0xc\n\t"
      "v_max_f32_dpp %5, %18, %18 row_mirror row_mask:0xf bank_mask:0x3\n\t"
      "v_max_f32_dpp %5, %19, %19 row_mirror row_mask:0xf bank_mask:0xc\n\t"
      "v_max_f32_dpp %6, %20, %20 row_mirror row_mask:0xf bank_mask:0x3\n\t"
      "v_max_f32_dpp %6, %21, %21 row_mirror row_mask:0xf bank_mask:0xc\n\t"
      "v_max_f32_dpp %7, %22, %22 row_mirror row_mask:0xf bank_mask:0x3\n\t"
      "v_max_f32_dpp %7, %23, %23 row_mirror row_mask:0xf bank_mask:0xc"
      : "=&v"(a0), "=&v"(a1), "=&v"(a2), "=&v"(a3), "=&v"(a4), "=&v"(a5), "=&v"(a6), "=&v"(a7)
      : "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]), "v"(v[6]), "v"(v[7]), "v"(v[8]),
        "v"(v[9]), "v"(v[10]), "v"(v[11]), "v"(v[12]), "v"(v[13]), "v"(v[14]), "v"(v[15]));
  float b0, b1, b2, b3;
  // lanes 0-3 and 8-11 (banks 0, 2) keep the even one of each pair
  asm("s_nop 1\n\t"
      "v_max_f32_dpp %0, %4, %4 row_half_mirror row_mask:0xf bank_mask:0x5\n\t"
      "v_max_f32_dpp %0, %5, %5 row_half_mirror row_mask:0xf bank_mask:0xa\n\t"
      "v_max_f32_dpp %1, %6, %6 row_half_mirror row_mask:0xf bank_mask:0x5\n\t"
      "v_max_f32_dpp %1, %7, %7 row_half_mirror row_mask:0xf bank_mask:0xa\n\t"
      "v_max_f32_dpp %2, %8, %8 row_half_mirror row_mask:0xf bank_mask:0x5\n\t"
      "v_max_f32_dpp %2, %9, %9 row_half_mirror row_mask:0xf bank_mask:0xa\n\t"
      "v_max_f32_dpp %3, %10, %10 row_half_mirror row_mask:0xf bank_mask:0x5\n\t"
      "v_max_f32_dpp %3, %11, %11 row_half_mirror row_mask:0xf bank_mask:0xa"
      : "=&v"(b0), "=&v"(b1), "=&v"(b2), "=&v"(b3)
      : "v"(a0), "v"(a1), "v"(a2), "v"(a3), "v"(a4), "v"(a5), "v"(a6), "v"(a7));
  // rows of 16 lanes: even rows keep b0 / b2, odd rows b1 / b3
  auto r0 = __builtin_amdgcn_permlane16_swap(__float_as_uint(b0), __float_as_uint(b1), false, false);
  auto r1 = __builtin_amdgcn_permlane16_swap(__float_as_uint(b2), __float_as_uint(b3), false, false);
  float x0 = __builtin_fmaxf(__uint_as_float(r0[0]), __uint_as_float(r0[1]));
  float x1 = __builtin_fmaxf(__uint_as_float(r1[0]), __uint_as_float(r1[1]));
  asm("s_nop 1\n\t"
      "v_max_f32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %1, %1, %1 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_max_f32_dpp %0, %0, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %1, %1, %1 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf"
      : "+v"(x0), "+v"(x1));
  c0 = x0;
  c1 = x1;
}

// fp32 <-> int with the same order (for atomic maxima of signed values)
__device__ __forceinline__ int ordered_f32(float v) {
  const int b = __float_as_int(v + 0.0f);
  return b >= 0 ? b : b ^ 0x7FFFFFFF;
}
__device__ __forceinline__ float unordered_f32(int o) { return __int_as_float(o >= 0 ? o : o ^ 0x7FFFFFFF); }

__device__ __forceinline__ int64_t part_offset(int64_t g, int64_t rb, int64_t N, int64_t nb, int rows) {
  const int64_t per_head = nb * N - (int64_t)rows * nb * (nb - 1) / 2;
  return g * per_head + rb * N - (int64_t)rows * rb * (rb - 1) / 2;
}

// Exact best of row i over the 16 columns of tile tp in half p (positions
// j = tp*32 + tile_col(r, p), those with j < ncols and |i - j| > w): an fp32
// screen, then fp64 for those within the margin of the largest.  Both lanes
// of a row run it (each over the feature chunks 2s+h it holds) and combine
// partial sums, so they reach identical results.  Column index c is
// position pos_of(c).
template <int D, class PosOf>
__device__ __forceinline__ void exact_tile(const uint4* Kg, const double* nsq_g, const float* rinv_g, int i, double ni,
                                           int tp, int p, int ncols, int w, int h, float margin, PosOf pos_of,
                                           double& bb, int& aa) {
  constexpr int CH = D / 8;
  constexpr int KS = D / 16;
  uint4 kr[KS];
#pragma unroll
  for (int s2 = 0; s2 < KS; ++s2) kr[s2] = Kg[(size_t)i * CH + 2 * s2 + h];
  constexpr int BATCH = CH == 8 ? 4 : 2;
  float ya[16];
  float ymax = -__builtin_inff();
#pragma unroll
  for (int r0 = 0; r0 < 16; r0 += BATCH) {
    uint4 q[BATCH][KS];
    float rj[BATCH];
    int jj[BATCH];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const int col = tp * 32 + tile_col(r0 + u, p);
      const int cc = col < ncols ? col : ncols - 1;
      const int j = pos_of(cc);
      jj[u] = j;
      const uint4* kj = Kg + (size_t)j * CH;
#pragma unroll
      for (int s2 = 0; s2 < KS; ++s2) q[u][s2] = kj[2 * s2 + h];
      rj[u] = rinv_g[j];
    }
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const int col = tp * 32 + tile_col(r0 + u, p);
      const int j = jj[u];
      const int dist = i > j ? i - j : j - i;
      float part = 0.0f;
#pragma unroll
      for (int s2 = 0; s2 < KS; ++s2) {
        part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, kr[s2].x), __builtin_bit_cast(bf16x2, q[u][s2].x), part, false);
        part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, kr[s2].y), __builtin_bit_cast(bf16x2, q[u][s2].y), part, false);
        part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, kr[s2].z), __builtin_bit_cast(bf16x2, q[u][s2].z), part, false);
        part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, kr[s2].w), __builtin_bit_cast(bf16x2, q[u][s2].w), part, false);
      }
      const float dotf = part + __shfl_xor(part, 32);
      ya[r0 + u] = (col < ncols && dist > w) ? dotf * rj[u] : -__builtin_inff();
      ymax = __builtin_fmaxf(ymax, ya[r0 + u]);
    }
  }
  unsigned cm = 0u;
#pragma unroll
  for (int r = 0; r < 16; ++r) cm |= (ya[r] > -__builtin_inff() && ya[r] >= ymax - margin) ? 1u << r : 0u;
#pragma unroll 1
  while (cm != 0u) {
    const int r = __builtin_ctz(cm);
    cm &= cm - 1u;
    const int j = pos_of(tp * 32 + tile_col(r, p));
    const uint4* kj = Kg + (size_t)j * CH;
    double part = 0.0;
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) part += dot8_exact(kr[s2], kj[2 * s2 + h]);
    const double dot = part + __shfl_xor(part, 32);
    const double nn = ni * nsq_g[j];
    double sim = nn > 0.0 ? dot / sqrt(nn) : 0.0;
    sim += 0.0;
    if (aa < 0 || sim > bb || (sim == bb && j < aa)) {
      bb = sim;
      aa = j;
    }
  }
}

// ---------------------------------------------------------------------------
// the sweep

template <class S>
__global__ __launch_bounds__(64 * S::WAVES, S::OCC) void tri_sweep_kernel(TriArgs a) {
  constexpr int D = S::D;
  constexpr int RB = S::RB;
  constexpr int WAVES = S::WAVES;
  constexpr int SC = S::SC;
  constexpr int NT = 64 * WAVES;
  constexpr int ROWS = S::ROWS;
  constexpr int CH = D / 8;
  constexpr int KS = D / 16;
  constexpr int LOADS = SC * CH / NT;
  constexpr int TILES = SC / 32;
  static_assert(LOADS * NT == SC * CH, "stage load split");
  static_assert(SC % 64 == 0 && SC / 64 <= WAVES, "stage columns: whole waves load rinv");
  __shared__ StageK<D, SC> buf0;
  __shared__ StageK<D, SC> buf1;
  // per wave and stage column, the wave's column maximum; three buffers, so a
  // stage's maxima are merged one barrier after its last tile was written
  __shared__ float colpart[3][WAVES][SC];

  const int64_t N = a.N;
  const int64_t nb = a.nb;
  const int64_t npair = (nb + 1) / 2;
  const int64_t total = a.G * npair;
  const int64_t per_xcd = (total + 7) / 8;
  const int64_t logical = (int64_t)(blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (logical >= total) return;
  const int64_t g = logical / npair;
  const int64_t pidx = logical % npair;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  const int lrow = lane & 31;
  const int w = a.window;
  const uint4* Kg = reinterpret_cast<const uint4*>(a.keys) + (size_t)g * N * CH;
  const float* rinv_g = a.rinv + (size_t)g * N;
  const double* nsq_g = a.nsq + (size_t)g * N;
  int32_t* ccount_g = a.ccount + (size_t)g * N;

  // stage-load and A-operand offsets: load t of a stage reads column
  // (tid + NT*t)/CH at a swizzled chunk, the A operand of tile tt reads column
  // 32*tt + lrow; the swizzle repeats within both strides, so the per-lane
  // part of either address is the same for every t and tt
  static_assert((NT / CH) % kSwzPeriod == 0 && 32 % kSwzPeriod == 0, "swizzle period");
  uint32_t ld_off, a_off[KS];
  {
    const int c = tid / CH;
    ld_off = (uint32_t)((c * CH + ((tid % CH) ^ swz<CH>(c))) * 16);
#pragma unroll
    for (int s = 0; s < KS; ++s) a_off[s] = (uint32_t)((lrow * CH + ((2 * s + h) ^ swz<CH>(lrow))) * 16);
  }

#pragma unroll 1
  for (int pass = 0; pass < 2; ++pass) {
    const int64_t rb = pass == 0 ? pidx : nb - 1 - pidx;
    if (pass == 1 && rb == pidx) break;  // the middle block of an odd count: once
    const int col_start = (int)(rb * ROWS);
    const int ncols = (int)N - col_start;  // this block sweeps columns col_start .. N-1
    const int row0 = col_start + wave * (RB * 32);
    int32_t* part_rb = a.part + part_offset(g, rb, N, nb, ROWS);

    // ---- row keys (rows past the end repeat the last row: their values
    // duplicate a real row's, so column maxima are unaffected; they count nothing)
    bf16x8 brow[RB][KS];
    float thr[RB], best[RB], second[RB], rinvr[RB];  // second: the largest maximum of the other tiles
    int btile[RB], cnt[RB];
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      const int r = row0 + 32 * b + lrow;
      const int i = r < N ? r : (int)N - 1;
#pragma unroll
      for (int s = 0; s < KS; ++s) brow[b][s] = __builtin_bit_cast(bf16x8, Kg[(size_t)i * CH + 2 * s + h]);
      const double ni = nsq_g[i];
      // y = dot/||k_j|| is ||k_i|| cos, so cos > tau is y > tau*||k_i||; a zero
      // key has cosine 0 with every key, which exceeds a negative tau; + 0.0f
      // turns a -0 threshold into +0
      thr[b] = r >= N ? __builtin_inff()
                      : (ni == 0.0 && a.tau < 0.0) ? -__builtin_inff() : (float)(a.tau * sqrt(ni)) + 0.0f;
      rinvr[b] = rinv_g[i];
      best[b] = -__builtin_inff();
      second[b] = -__builtin_inff();
      btile[b] = -1;
      cnt[b] = 0;
    }

    const uint4* Cg = Kg + (size_t)col_start * CH;
    const float* crinv = rinv_g + col_start;
    auto issue = [&](int col0, StageK<D, SC>& sb) TWINKV_INLINE {
      if (col0 + SC <= ncols) {
        const char* base = reinterpret_cast<const char*>(Cg + (size_t)col0 * CH);
#pragma unroll
        for (int u = 0; u < LOADS; ++u) dma16(base + (size_t)NT * 16 * u + ld_off, &sb.keys[NT * u + wave * 64]);
        if (wave < SC / 64) dma4(crinv + col0 + tid, &sb.rinv[wave * 64]);
        return;
      }
      const int lastc = ncols - 1;
#pragma unroll
      for (int u = 0; u < LOADS; ++u) {
        const int c = col0 + tid / CH + (NT / CH) * u;
        const int col = c < lastc ? c : lastc;
        dma16(reinterpret_cast<const char*>(Cg + (size_t)col * CH) + (ld_off & (CH * 16 - 1)),
              &sb.keys[NT * u + wave * 64]);
      }
      if (wave < SC / 64) {
        const int col = col0 + tid < lastc ? col0 + tid : lastc;
        dma4(crinv + col, &sb.rinv[wave * 64]);
      }
    };
    auto load_a = [&](const StageK<D, SC>& sb, int tt, bf16x8 (&A)[KS]) TWINKV_INLINE {
      const char* kb = reinterpret_cast<const char*>(sb.keys) + tt * 32 * CH * 16;
#pragma unroll
      for (int s = 0; s < KS; ++s)
        A[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(kb + a_off[s]));
    };
    auto load_rv = [&](const StageK<D, SC>& sb, int tt, float (&rv)[16]) TWINKV_INLINE {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const float4 r4 = *reinterpret_cast<const float4*>(&sb.rinv[tt * 32 + 8 * gq + 4 * h]);
        rv[4 * gq + 0] = r4.x;
        rv[4 * gq + 1] = r4.y;
        rv[4 * gq + 2] = r4.z;
        rv[4 * gq + 3] = r4.w;
      }
    };
    // first and last row position of the wave (rows past the end clamped)
    const int rlo = __builtin_amdgcn_readfirstlane(row0 < N ? row0 : (int)N - 1);
    const int rhi = __builtin_amdgcn_readfirstlane(row0 + RB * 32 - 1 < N ? row0 + RB * 32 - 1 : (int)N - 1);
    // counts of y > tau*||k_i|| over the 16 values of block b: the row's,
    // and, one atomic per twin, each column's.  Excluded entries hold -inf,
    // and a zero key under a negative tau has thr = -inf, so the test is a
    // compare (the sign of thr - y would be a NaN's there)
    auto count16 = [&](const auto& y, int b, int c0) TWINKV_INLINE {
      uint32_t msk = 0;
#pragma unroll
      for (int r = 0; r < 16; ++r) msk |= (y[r] > thr[b] ? 1u : 0u) << r;
      cnt[b] += __popc(msk);
      while (msk != 0u) {
        const int r = __builtin_ctz(msk);
        msk &= msk - 1u;
        atomicAdd(&ccount_g[c0 + tile_col(r, h)], 1);
      }
    };
    auto mfma_block = [&](const bf16x8 (&A)[KS], int b, f32x16& acc) TWINKV_INLINE {
      acc = (f32x16){};
#pragma unroll
      for (int s = 0; s < KS; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[s], brow[b][s], acc, 0, 0, 0);
    };
    float colmax[16];
    // block b of a tile whose dots are in acc: y = dot/||k_j|| and its block
    // maximum for the row side; z = y/||k_i|| (the cosine) merged into the
    // column maxima over the wave's blocks
    auto epilogue = [&](f32x16& acc, int b, const float (&rv)[16], bool live, int tile, int c0) TWINKV_INLINE {
      float yy[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        acc[r] *= rv[r];
        yy[r] = acc[r];
      }
      const float m = max16(yy);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float z = yy[r] * rinvr[b];
        colmax[r] = (b == 0) ? z : __builtin_fmaxf(colmax[r], z);
      }
      if (live) {  // wave-uniform
        second[b] = __builtin_amdgcn_fmed3f(m, best[b], second[b]);  // second <= best: max(second, min(m, best))
        btile[b] = m > best[b] ? tile : btile[b];
        best[b] = __builtin_fmaxf(best[b], m);
        if (__ballot(m > thr[b]) != 0ull) count16(acc, b, c0);
      }
    };
    // one lane of each quad writes the quad's two column maxima
    const int qcol = tile_col(4 * ((lane >> 4) & 1) + 2 * ((lane >> 2) & 1) + ((lane >> 3) & 1), h);
    auto write_cols = [&](int st, int tt, float c0, float c1) TWINKV_INLINE {
      if ((lane & 3) == 0) {
        colpart[st % 3][wave][tt * 32 + qcol] = c0;
        colpart[st % 3][wave][tt * 32 + qcol + 16] = c1;
      }
    };
    auto flush_cols = [&](int st, int tt, bool live) TWINKV_INLINE {
      float c0, c1;
      reduce_cols(colmax, c0, c1);
      if (!live) c0 = c1 = -__builtin_inff();  // a masked tile is added after the sweep
      write_cols(st, tt, c0, c1);
    };
    auto merge_stage = [&](int st) TWINKV_INLINE {
      for (int c = tid; c < SC; c += NT) {
        const int col = st * SC + c;  // relative to col_start
        if (col < ncols) {
          float v = colpart[st % 3][0][c];
#pragma unroll
          for (int wv = 1; wv < WAVES; ++wv) v = __builtin_fmaxf(v, colpart[st % 3][wv][c]);
          part_rb[col] = ordered_f32(v);
        }
      }
    };
    auto interleave = [&]() TWINKV_INLINE {
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 7, 0);  // up to seven VALU
      }
    };

    // ---- the sweep.  The stages at the start that hold a pair with j - i <=
    // w for some row of the workgroup (the diagonal) and a ragged last stage
    // run tile by tile from LDS, masking pairs with j - i <= w, columns past
    // the end and rows past the end; the clean stages between them (every tile
    // past the band of every row) run the rolling pipeline of the repair
    // sweep unmasked.  Tiles are visited in column order, so the first tile
    // attaining a row's maximum is kept.
    const int nstages = (ncols + SC - 1) / SC;
    const int tile0 = col_start >> 5;
    const int wg_rhi = col_start + ROWS - 1 < N ? col_start + ROWS - 1 : (int)N - 1;
    // leading stages that reach the band, rounded up to an even count so the
    // pipelined stages start in the first buffer
    const int nd0 = ((wg_rhi + w - col_start) / SC + 2) & ~1;
    const int nd = nd0 < nstages ? nd0 : nstages;
    const int nce = (ncols % SC == 0) ? nstages : nstages - 1;  // stages before a ragged last one
    f32x16 acc[RB];
    bf16x8 A[KS];
    float rv[16];

    // one tile's epilogue with every pair tested
    auto masked_epilogue = [&](f32x16& accb, int b, int tile, int c0) TWINKV_INLINE {
      const int i = row0 + 32 * b + lrow;
      // entry r is column base + o, o = 8*(r>>2) + (r&3): a pair when o > lo
      // (j - i > w) and o <= hi (j < N); a row past the end has none
      const int base = c0 + 4 * h;
      const int lo = i < N ? i + w - base : 64;
      const int hi = (int)N - 1 - base;
      float yy[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int o = 8 * (r >> 2) + (r & 3);
        const bool ok = o > lo && o <= hi;
        yy[r] = ok ? accb[r] * rv[r] : -__builtin_inff();
        const float z = ok ? yy[r] * rinvr[b] : -__builtin_inff();
        colmax[r] = (b == 0) ? z : __builtin_fmaxf(colmax[r], z);
      }
      const float m = max16(yy);
      second[b] = __builtin_amdgcn_fmed3f(m, best[b], second[b]);
      btile[b] = m > best[b] ? tile : btile[b];
      best[b] = __builtin_fmaxf(best[b], m);
      if (__ballot(m > thr[b]) != 0ull) count16(yy, b, c0);  // excluded entries are -inf
    };
    // a stage run tile by tile; its data was issued before (into the buffer
    // of its parity)
    auto masked_stage = [&](int st) TWINKV_INLINE {
      StageK<D, SC>& cur = (st & 1) ? buf1 : buf0;
      StageK<D, SC>& nxt = (st & 1) ? buf0 : buf1;
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      __syncthreads();
      if (st >= 1) merge_stage(st - 1);
      if (st + 1 < nstages) issue((st + 1) * SC, nxt);
#pragma unroll 1
      for (int tt = 0; tt < TILES; ++tt) {
        const int tile = tile0 + st * TILES + tt;
        const int c0 = tile * 32;
        if (c0 >= N) break;  // past the end (wave-uniform); these columns are never merged
        if (c0 + 31 <= rlo + w) {  // no pair of this tile has j - i > w for this wave
          write_cols(st, tt, -__builtin_inff(), -__builtin_inff());
          continue;
        }
        const bool live = c0 > rhi + w && c0 + 31 < N;  // wave-uniform
        load_a(cur, tt, A);
        load_rv(cur, tt, rv);
#pragma unroll
        for (int b = 0; b < RB; ++b) {
          f32x16 y;
          mfma_block(A, b, y);
          if (live) epilogue(y, b, rv, true, tile, c0);
          else masked_epilogue(y, b, tile, c0);
        }
        flush_cols(st, tt, true);
      }
    };
    // the rolling pipeline over a clean stage: after block b's epilogue for
    // tile t its accumulator takes the MFMAs of tile t+1; the last tile's
    // epilogue overlaps the next stage's first MFMAs when that stage is clean
    auto stage = [&](int st, StageK<D, SC>& cur, const StageK<D, SC>& nxt) TWINKV_INLINE {
#pragma unroll 1
      for (int tt = 0; tt < TILES - 1; ++tt) {
        const int tile = tile0 + st * TILES + tt;
        load_a(cur, tt + 1, A);
#pragma unroll
        for (int b = 0; b < RB; ++b) {
          epilogue(acc[b], b, rv, true, tile, tile * 32);
          mfma_block(A, b, acc[b]);
          interleave();
        }
        flush_cols(st, tt, true);
        load_rv(cur, tt + 1, rv);
      }
      const bool more = st + 1 < nce;
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      __syncthreads();
      if (st >= 1) merge_stage(st - 1);
      if (st + 2 < nstages) issue((st + 2) * SC, cur);
      if (more) load_a(nxt, 0, A);
      const int tile = tile0 + st * TILES + TILES - 1;
#pragma unroll
      for (int b = 0; b < RB; ++b) {
        epilogue(acc[b], b, rv, true, tile, tile * 32);
        if (more) mfma_block(A, b, acc[b]);
        interleave();
      }
      flush_cols(st, TILES - 1, true);
      if (more) load_rv(nxt, 0, rv);
    };

    // stages [0, nd) and [max(nd, nce), nstages) run masked, tile by tile
    auto masked_run = [&](int from, int to) TWINKV_INLINE {
#pragma unroll 1
      for (int st = from; st < to; ++st) masked_stage(st);
    };
    issue(0, buf0);
    int st_m = 0, st_end = nd;  // the masked range to run next
#pragma unroll 1
    for (int part = 0; part < 2; ++part) {
      masked_run(st_m, st_end);
      if (part == 1) break;
      if (nd < nce) {
        // stage nd (even: the first buffer) was issued by the last diagonal stage
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
        __syncthreads();
        if (nd + 1 < nstages) issue((nd + 1) * SC, buf1);
        load_a(buf0, 0, A);
#pragma unroll
        for (int b = 0; b < RB; ++b) mfma_block(A, b, acc[b]);
        load_rv(buf0, 0, rv);
#pragma unroll 1
        for (int st = nd; st < nce; st += 2) {
          stage(st, buf0, buf1);
          if (st + 1 >= nce) break;
          stage(st + 1, buf1, buf0);
        }
      }
      // then the stages past both: a ragged last stage (or none)
      st_m = nd > nce ? nd : nce;
      st_end = nstages;
    }
    __syncthreads();
    if (nstages > 0) merge_stage(nstages - 1);

    // ---- exact row side: per half-row, the fp32 maximum and its first tile;
    // a half within the margin of the row's maximum is screened and its
    // near-maximal columns recomputed in fp64
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      const int i = row0 + 32 * b + lrow;
      const bool row_ok = i < N;
      const int ic = row_ok ? i : (int)N - 1;
      double bb = -1.0;
      int aa = -1;
      const double ni = nsq_g[ic];
      const float margin = 8e-5f * (float)sqrt(ni) + 1e-30f;  // y units (||k_i|| cos)
      const float other = __shfl_xor(best[b], 32);
      const bool look = row_ok && btile[b] >= 0 && best[b] >= other - margin;
      const bool look_o = __shfl_xor((int)look, 32) != 0;
      const int tile_o = __shfl_xor(btile[b], 32);
      const bool look0 = (h == 0) ? look : look_o;
      const bool look1 = (h == 1) ? look : look_o;
#pragma unroll
      for (int ps = 0; ps < 2; ++ps) {
        const int p = (ps == 0 && look0) ? 0 : 1;
        const bool lk = ps == 0 ? (look0 || look1) : (look0 && look1);
        const int tp = (h == p) ? btile[b] : tile_o;
        if (__ballot(lk) == 0ull) continue;
        if (lk) exact_tile<D>(Kg, nsq_g, rinv_g, ic, ni, tp, p, (int)N, w, h, margin, [](int c) { return c; }, bb, aa);
      }
      const int c = cnt[b] + __shfl_xor(cnt[b], 32);
      const float ymax = __builtin_fmaxf(best[b], __shfl_xor(best[b], 32));
      // another tile of either half within twice the fp32 error of the
      // row's maximum may hold the exact best: queue the row for the exact
      // resolve, with candidates down to the screening margin below the
      // maximum.  A zero key is settled here: all its cosines are exactly 0
      // and the first tile holds the lowest eligible position.
      const bool near = second[b] >= ymax - kTieMargin * (float)sqrt(ni);
      const bool near_o = __shfl_xor((int)near, 32) != 0;  // both lanes of the row take part in the shuffle
      const bool amb = row_ok && ni > 0.0 && ymax > -__builtin_inff() && (near || near_o);
      if (h == 0 && row_ok) {
        const size_t o = (size_t)g * N + i;
        a.best64[o] = aa >= 0 ? pack_best(bb, aa, a.idx_mask) : 0ull;
        a.best_sim[o] = bb;  // the row side's exact result, kept for the finalize
        a.best_idx[o] = aa;
        a.rowcos[o] = ymax > -__builtin_inff() ? ymax * rinvr[b] : -__builtin_inff();
        a.rcount[o] = c;
        if (amb) {
          const int k = atomicAdd(&a.q.count[g], 1);
          a.q.row[(size_t)g * N + k] = i;
          a.q.thr[(size_t)g * N + k] = ymax * rinvr[b] - kMargin;
        }
      }
    }
    __syncthreads();  // LDS is reused by the next pass
  }
}

// ---------------------------------------------------------------------------
// resolve: the largest of each position's row side and column maxima, and
// the row blocks within the margin of it

template <int ROWS>
__global__ __launch_bounds__(256) void tri_colmax_kernel(TriArgs a) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= a.G * a.N) return;
  const int64_t N = a.N;
  const int64_t g = q / N;
  const int64_t k = q % N;
  const int rbk = (int)(k / ROWS);  // row blocks 0..rbk swept column k
  // column k of block rb sits at part_offset(g, rb) + k - rb*ROWS; the next
  // block's entry is N - (rb+1)*ROWS further on
  const int32_t* p0 = a.part + part_offset(g, 0, N, a.nb, ROWS) + k;
  float p1 = -__builtin_inff(), p2 = -__builtin_inff();
  int r1 = -1;
  {
    const int32_t* pp = p0;
#pragma unroll 4
    for (int rb = 0; rb <= rbk; ++rb) {
      const float p = unordered_f32(*pp);
      pp += N - (int64_t)(rb + 1) * ROWS;
      const bool top = p > p1;
      p2 = top ? p1 : __builtin_fmaxf(p2, p);
      r1 = top ? rb : r1;
      p1 = top ? p : p1;
    }
  }
  const float m = __builtin_fmaxf(a.rowcos[q], p1);
  a.colmax[q] = m;
  if (!(p1 > -__builtin_inff()) || p1 < m - kMargin) return;
  uint32_t* bits = a.cbits + (size_t)g * a.nb * a.words + (k >> 5);
  const uint32_t bit = 1u << (k & 31);
  if (!(p2 >= m - kMargin)) {  // the usual case: one block within the margin
    atomicOr(bits + (size_t)r1 * a.words, bit);
    return;
  }
  const int32_t* pp = p0;
  for (int rb = 0; rb <= rbk; ++rb) {
    const float p = unordered_f32(*pp);
    pp += N - (int64_t)(rb + 1) * ROWS;
    if (p > -__builtin_inff() && p >= m - kMargin) atomicOr(bits + (size_t)rb * a.words, bit);
  }
}

// Exact best twin of the marked positions over one row block.  The block's
// rows are staged in LDS as MFMA A operands (with their squared and inverse
// norms); the marked positions are gathered as B operands, 32 per wave and
// round, rounds kept full by queueing the positions of several candidate
// words.  A row is a candidate when its fp32 value reaches the position's
// overall maximum minus the margin: usually one row per position, the one
// that attains the maximum.  Each half-row lane notes its first candidate;
// afterwards the candidates are recomputed exactly in fp64 from the staged
// row and the position's own chunks (the two lanes that hold a position add
// their halves), and a position with more than one candidate in a half has
// its tiles swept again with every candidate recomputed.  The best goes to
// the 64-bit atomic maximum.  Pairs with |i - k| <= w and rows past the end
// are excluded (a pair also on k's row side changes no maximum).
template <class S>
__global__ __launch_bounds__(256, S::D == 64 ? 2 : 1) void tri_colres_kernel(TriArgs a) {
  constexpr int D = S::D;
  constexpr int ROWS = S::ROWS;
  constexpr int NT = 256;
  constexpr int CH = D / 8;
  constexpr int KS = D / 16;
  constexpr int TILES = ROWS / 32;
  constexpr int WCHUNK = NT / 2;              // candidate words expanded at a time (by the first half)
  constexpr int ROUND = 4 * 32;               // positions per round
  constexpr int QCAP = WCHUNK * 32 + ROUND;   // a chunk's positions plus a partial round carried over
  static_assert((ROWS * CH) % NT == 0, "block load split");
  __shared__ StageK<D, ROWS> blk;
  __shared__ double bnsq[ROWS];
  __shared__ int32_t queue[QCAP];
  __shared__ int32_t qcount;
  __shared__ int32_t wsum[NT / 64];

  const int64_t N = a.N;
  const int64_t g = blockIdx.x / a.nb;
  const int64_t rb = blockIdx.x % a.nb;
  const int base = (int)(rb * ROWS);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;
  const int lrow = lane & 31;
  const int w = a.window;
  const uint4* Kg = reinterpret_cast<const uint4*>(a.keys) + (size_t)g * N * CH;
  const uint32_t* bits = a.cbits + ((size_t)g * a.nb + rb) * a.words;
  const int nrows = (int)N - base < ROWS ? (int)N - base : ROWS;  // rows of this block

  // the block's rows (past the end: the last row) straight into LDS with the
  // sweep's swizzle: slot s = c*CH + (chunk ^ swz(c)) is written by the lane
  // that fetches that chunk of row c
  {
    constexpr int LD = ROWS * CH / NT;
#pragma unroll
    for (int u = 0; u < LD; ++u) {
      const int sl = NT * u + tid;
      const int c = sl / CH;
      const int chunk = (sl % CH) ^ swz<CH>(c);
      dma16(Kg + (size_t)(base + (c < nrows ? c : nrows - 1)) * CH + chunk, &blk.keys[NT * u + wave * 64]);
    }
    for (int c = tid; c < ROWS; c += NT) {
      const int src = base + (c < nrows ? c : nrows - 1);
      blk.rinv[c] = a.rinv[(size_t)g * N + src];
      bnsq[c] = a.nsq[(size_t)g * N + src];
    }
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
  }
  if (tid == 0) qcount = 0;
  __syncthreads();

  uint32_t a_off[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) a_off[s] = (uint32_t)((lrow * CH + ((2 * s + h) ^ swz<CH>(lrow))) * 16);

  // exact cosine of position k (chunks kc of this lane's half) with staged row
  // c; both lanes of the position call it together
  auto exact = [&](const uint4 (&kc)[KS], double nk, int c) TWINKV_INLINE {
    double part = 0.0;
#pragma unroll
    for (int s = 0; s < KS; ++s) part += dot8_exact(kc[s], blk.keys[c * CH + ((2 * s + h) ^ swz<CH>(c))]);
    const double dot = part + __shfl_xor(part, 32);
    const double nn = nk * bnsq[c];
    const double sim = nn > 0.0 ? dot / sqrt(nn) : 0.0;
    return sim + 0.0;
  };
  auto tile_dots = [&](int tt, const bf16x8 (&bk)[KS]) TWINKV_INLINE {
    bf16x8 A[KS];
    const char* kb = reinterpret_cast<const char*>(blk.keys) + tt * 32 * CH * 16;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      A[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(kb + a_off[s]));
    f32x16 acc = (f32x16){};
#pragma unroll
    for (int s = 0; s < KS; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[s], bk[s], acc, 0, 0, 0);
    return acc;
  };
  // candidate rows of a tile: y = dot/||k_row|| >= thr; the window and the
  // end of the block are tested only on tiles that reach them
  auto cand_mask = [&](const f32x16& acc, int tt, int k, float thr) TWINKV_INLINE {
    float rv[16];
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const float4 r4 = *reinterpret_cast<const float4*>(&blk.rinv[tt * 32 + 8 * gq + 4 * h]);
      rv[4 * gq + 0] = r4.x;
      rv[4 * gq + 1] = r4.y;
      rv[4 * gq + 2] = r4.z;
      rv[4 * gq + 3] = r4.w;
    }
    uint32_t m = 0;
#pragma unroll
    for (int r = 0; r < 16; ++r) m |= (uint32_t)(acc[r] * rv[r] >= thr) << r;
    const int lo = base + tt * 32;  // rows lo .. lo + 31
    const bool edge = lo + 31 >= k - w && lo <= k + w;
    if (__ballot(edge || tt * 32 + 31 >= nrows) != 0ull) {
      uint32_t keep = 0;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int c = tt * 32 + tile_col(r, h);
        const int i = base + c;
        const int dist = i > k ? i - k : k - i;
        keep |= (uint32_t)(c < nrows && dist > w) << r;
      }
      m &= keep;
    }
    return m;
  };
  auto process = [&](int q0, int qn) TWINKV_INLINE {
    const int qi = q0 + wave * 32 + lrow;
    const bool ok = qi < qn;
    const int k = queue[ok ? qi : q0];  // a lane without a position repeats one; its result is dropped
    uint4 kc[KS];
    bf16x8 bk[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      kc[s] = Kg[(size_t)k * CH + 2 * s + h];
      bk[s] = __builtin_bit_cast(bf16x8, kc[s]);
    }
    const double nk = a.nsq[(size_t)g * N + k];
    // y = dot/||k_row|| = ||k|| cos: rows within the margin of k's overall maximum
    const float thr = ok ? (a.colmax[(size_t)g * N + k] - kMargin) * (float)sqrt(nk) : __builtin_inff();
    int first = -1;  // this half's first candidate (staged row), -2: more than one
#pragma unroll 1
    for (int tt = 0; tt < TILES; ++tt) {
      const f32x16 acc = tile_dots(tt, bk);
      const uint32_t m = cand_mask(acc, tt, k, thr);
      if (m != 0u) first = (first == -1 && (m & (m - 1u)) == 0u) ? tt * 32 + tile_col(__builtin_ctz(m), h) : -2;
    }
    double bb = -1.0;
    int aa = -1;
    auto take = [&](double sim, int c) TWINKV_INLINE {
      const int j = base + c;
      if (aa < 0 || sim > bb || (sim == bb && j < aa)) {
        bb = sim;
        aa = j;
      }
    };
    const int other = __shfl_xor(first, 32);
    // the single candidates of half 0, then half 1
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int c = (h == p) ? first : other;
      if (__ballot(c >= 0) == 0ull) continue;
      if (c >= 0) take(exact(kc, nk, c), c);
    }
    // positions with several candidates in a half: every candidate, exactly
    if (__ballot(first == -2 || other == -2) != 0ull) {
      const bool redo = first == -2 || other == -2;
#pragma unroll 1
      for (int tt = 0; tt < TILES; ++tt) {
        const f32x16 acc = tile_dots(tt, bk);
        const uint32_t mine = redo ? cand_mask(acc, tt, k, thr) : 0u;
        const uint32_t oth = (uint32_t)__shfl_xor((int)mine, 32);
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          uint32_t cm = (h == p) ? mine : oth;
          while (cm != 0u) {
            const int r = __builtin_ctz(cm);
            cm &= cm - 1u;
            const int c = tt * 32 + tile_col(r, p);
            take(exact(kc, nk, c), c);
          }
        }
      }
    }
    if (h == 0 && ok && aa >= 0)
      atomicMax((unsigned long long*)&a.best64[(size_t)g * N + k], (unsigned long long)pack_best(bb, aa, a.idx_mask));
  };

#pragma unroll 1
  for (int64_t c0 = base >> 5; c0 < a.words; c0 += WCHUNK) {  // base is a multiple of 32
    // each of the first WCHUNK threads expands one word; a workgroup scan
    // places its positions
    const int64_t wi = c0 + tid;
    const uint32_t word = (tid < WCHUNK && wi < a.words) ? bits[wi] : 0u;
    const int cw = __popc(word);
    int incl = cw;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_up(incl, off);
      if (lane >= off) incl += v;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    const int q = qcount;  // fewer than ROUND carried over
    int before = 0, total = 0;
#pragma unroll
    for (int wv = 0; wv < NT / 64; ++wv) {
      before += wv < wave ? wsum[wv] : 0;
      total += wsum[wv];
    }
    int pos = q + before + incl - cw;
    uint32_t wb = word;
    while (wb != 0u) {
      const int bt = __builtin_ctz(wb);
      wb &= wb - 1u;
      queue[pos++] = (int32_t)(wi * 32 + bt);
    }
    __syncthreads();
    const int qn = q + total;
    const bool last = c0 + WCHUNK >= a.words;
    const int full = last ? qn : qn - qn % ROUND;  // whole rounds now, the rest with the next chunk
#pragma unroll 1
    for (int q0 = 0; q0 < full; q0 += ROUND) process(q0, full);
    __syncthreads();
    if (!last) {  // carry the partial round to the front
      const int rest = qn - full;
      int v = 0;
      if (tid < rest) v = queue[full + tid];
      __syncthreads();
      if (tid < rest) queue[tid] = v;
      if (tid == 0) qcount = rest;
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------------------
// outputs: the exact cosine of the winning pair, counts, scores

template <int D>
__global__ __launch_bounds__(256) void tri_finalize_kernel(TriArgs a) {
  constexpr int CH = D / 8;
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= a.G * a.N) return;
  const int64_t N = a.N;
  const int64_t g = q / N;
  const uint64_t u = a.best64[q];
  double bb = -1.0;
  int aa = -1;
  // the sweep's fixup left its own exact result in best_sim / best_idx: when
  // the packed best still names that position, its cosine is already exact
  const int aa_row = a.best_idx[q];
  if (u != 0ull && unpack_idx(u, a.idx_mask) == aa_row) {
    aa = aa_row;
    bb = a.best_sim[q];
  } else if (u != 0ull) {
    aa = unpack_idx(u, a.idx_mask);
    const uint4* ki = reinterpret_cast<const uint4*>(a.keys) + (size_t)q * CH;
    const uint4* kj = reinterpret_cast<const uint4*>(a.keys) + ((size_t)g * N + aa) * CH;
    double dot = 0.0;
#pragma unroll
    for (int c = 0; c < CH; ++c) dot += dot8_exact(ki[c], kj[c]);
    const double nn = a.nsq[q] * a.nsq[(size_t)g * N + aa];
    bb = (nn > 0.0 ? dot / sqrt(nn) : 0.0) + 0.0;
  }
  const int c = a.rcount[q] + a.ccount[q];
  a.best_sim[q] = bb;
  a.best_idx[q] = aa;
  a.count[q] = c;
  const double disc = log((double)(N + 1) / (double)(c + 1));
  a.score[q] = a.energy[q] * disc;
  if (a.omega) a.omega[q] = disc / log((double)(N + 1));
}

__global__ __launch_bounds__(256) void tri_clear_kernel(int32_t* ccount, int64_t n, uint32_t* cbits, int64_t nbits,
                                                        int32_t* qcount, int64_t G) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < n; q += stride) ccount[q] = 0;
  for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < nbits; q += stride) cbits[q] = 0u;
  for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < G; q += stride) qcount[q] = 0;
}

template <class S>
hipError_t launch_d(const TriArgs& a, hipStream_t stream, hipEvent_t mark) {
  const int64_t n = a.G * a.N;
  const int64_t nbits = a.G * a.nb * a.words;
  int64_t cb = (n > nbits ? n : nbits) / 256 + 1;
  cb = cb < 8192 ? cb : 8192;
  const int64_t total = a.G * ((a.nb + 1) / 2);
  const int64_t grid = 8 * ((total + 7) / 8);
  if (grid > INT_MAX || a.G * a.nb > INT_MAX || (n + 255) / 256 > INT_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(tri_clear_kernel, dim3((unsigned)cb), dim3(256), 0, stream, a.ccount, n, a.cbits, nbits,
                     a.q.count, a.G);
  hipLaunchKernelGGL((tri_sweep_kernel<S>), dim3((unsigned)grid), dim3(64 * S::WAVES), 0, stream, a);
  if (mark && hipEventRecord(mark, stream) != hipSuccess) return hipErrorInvalidValue;
  RowResArgs r{};
  r.keys = a.keys;
  r.nsq = a.nsq;
  r.rinv = a.rinv;
  r.col_keys = a.keys;
  r.col_rinv = a.rinv;
  r.q = a.q;
  r.G = a.G;
  r.N = a.N;
  r.d = a.d;
  r.window = a.window;
  r.best64 = a.best64;
  r.idx_mask = a.idx_mask;
  r.cand_row = a.cand_row;
  r.cand_col = a.cand_col;
  r.cand_count = a.cand_count;
  r.cand_cap = a.cand_cap;
  const hipError_t e = launch_rowres(r, stream);
  if (e != hipSuccess) return e;
  const unsigned kb = (unsigned)((n + 255) / 256);
  hipLaunchKernelGGL((tri_colmax_kernel<S::ROWS>), dim3(kb), dim3(256), 0, stream, a);
  hipLaunchKernelGGL((tri_colres_kernel<S>), dim3((unsigned)(a.G * a.nb)), dim3(256), 0, stream, a);
  hipLaunchKernelGGL((tri_finalize_kernel<S::D>), dim3(kb), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

int tri_rows(int d) { return d == 64 ? TriShape64::ROWS : TriShape128::ROWS; }

int64_t tri_part_per_head(int64_t N, int rows) {
  const int64_t nb = (N + rows - 1) / rows;
  return nb * N - (int64_t)rows * nb * (nb - 1) / 2;
}

hipError_t launch_tri(const TriArgs& a, hipStream_t stream, hipEvent_t mark) {
  if (a.d == 64) return launch_d<TriShape64>(a, stream, mark);
  return launch_d<TriShape128>(a, stream, mark);
}

}  // namespace twinkv
