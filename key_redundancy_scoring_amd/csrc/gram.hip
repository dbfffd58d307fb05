// Restricted Gram sweep of the repair pass: for every listed row i of a head,
// the best surviving twin b_i(S0) = max sim(i, j) over the retained columns
// j in S0 with |i - j| > w, and its lowest position a_i(S0) ("TwinKV: A
// Composable Repair Pass ...", section 3.4, Eq. 4).  The rows are all
// positions, or those whose unrestricted best twin was not retained.  This
// is the O(nKd) form of that section: rows meet only the K retained columns,
// and the similarity matrix is never written anywhere.
//
// Mapping onto gfx950:
//   * A workgroup of WAVES waves owns WAVES*RB*32 consecutive entries of the
//     row list (their positions ascend, and the band test below uses the
//     first and last of a wave); each wave owns RB blocks of 32 rows whose
//     bf16 keys stay in VGPRs as MFMA B operands for the whole sweep.  Three
//     workgroups share a CU at d = 64 (two at d = 128), so one workgroup's
//     prologue and fp64 fixup overlap another's sweep.
//   * Column keys (a compacted copy of the retained keys, with their
//     positions) stream HBM/L2 -> LDS in stages of SC columns with
//     global_load_lds (no VGPR round trip), into two LDS buffers: stage s+1
//     is in flight while stage s is computed, and the one wait per stage sits
//     before the barrier.  Each lane of a direct load writes 16 bytes at
//     base + 16*lane, so the XOR swizzle that spreads the MFMA A-operand reads
//     over the LDS banks (16-byte chunk k of column c sits at slot
//     c*CH + (k ^ swz(c))) is applied by choosing which global chunk each
//     lane fetches.  Columns past the end are clamped to the last one; the
//     tiles that hold them are handled by the masked path below.
//   * v_mfma_f32_32x32x16_bf16 with A = 32 column keys, B = 32 row keys gives
//     lane l the row (l mod 32) and 16 columns 8*(r/4) + 4*(l/32) + (r mod 4)
//     in accumulator r, so all reductions over columns stay inside a lane.
//     Products of bf16 values are exact; the dot products are fp32 sums.
//   * Epilogue per 32x32 block and lane, in registers: y = dot * (1/||k_j||)
//     (16 multiplies), the block maximum by a 3-input max tree, then one
//     compare and two selects keep (running max, first tile attaining it).
//   * Tiles that touch the |i-j| <= w band or the ragged tail (a few per row
//     block) leave the state unchanged in the sweep (branch-free: their
//     maximum is taken as -inf) and are recomputed with masking at the end of
//     the sweep, in tile order; there an exact tie with the running maximum
//     goes to the lower tile, as it would in column order.
//   * Which of the 16 columns of the winning tile holds the maximum is not
//     tracked in the sweep; after it, a lane whose half-row maximum can be the
//     row's screens its 16 candidates in fp32 and recomputes the near-maximal
//     ones exactly in fp64 (bf16 products are exact), keeping the largest,
//     lowest position on ties; the two half-waves that share a row then
//     merge.  This also makes b_i the exact fp64 cosine dot/sqrt(n_i*n_j) of
//     the chosen pair.  The sweep also keeps the largest maximum of the other
//     tiles; a row where it comes within twice the fp32 error (2e-5 in
//     cosine units) of the row's maximum is queued for the exact resolve of
//     resolve.hip, which settles it over every retained column.
//   * Workgroup ids are remapped so each XCD (ids are dealt round-robin over
//     8 XCDs) receives a contiguous run of row blocks: the blocks of one head
//     sweep its key stream together out of one L2.
#include <limits.h>

#include "sweep.h"

namespace twinkv {
namespace {

// d = 64: two row blocks per wave at three waves per SIMD (at most 168
// VGPRs).  The restricted sweep covers only the retained columns, often a
// few thousand, so the per-workgroup tail (masked tiles, fixup) weighs more,
// and a third wave per SIMD hides it better than the column reuse of four
// row blocks pays.  d = 128: three row blocks per wave at two waves per SIMD
// (242 VGPRs), so each A operand read from LDS feeds 24 MFMAs (7 % faster
// than two blocks; a second A buffer read a tile ahead no longer fits).
using Shape64 = GramShape<64, 2, 4, 128, 3>;
using Shape128 = GramShape<128, 3, 4, 128, 2>;

template <class S>
__global__ __launch_bounds__(64 * S::WAVES, S::OCC) void gram_kernel(GramArgs a) {
  constexpr int D = S::D;
  constexpr int RB = S::RB;
  constexpr int WAVES = S::WAVES;
  constexpr int SC = S::SC;
  constexpr int NT = 64 * WAVES;   // threads
  constexpr int ROWS = S::ROWS;
  constexpr int CH = D / 8;        // 16-byte chunks per key row
  constexpr int KS = D / 16;       // MFMA k-steps
  constexpr int LOADS = SC * CH / NT;
  constexpr int TILES = SC / 32;
  static_assert(LOADS * NT == SC * CH, "stage load split");
  static_assert(SC % 64 == 0 && SC / 64 <= WAVES, "stage columns: whole waves load rinv");
  // distinct LDS objects, so the compiler can tell the buffer being read
  // from the ones being filled
  __shared__ Stage<D, SC> buf0;
  __shared__ Stage<D, SC> buf1;

  const int64_t N = a.N;
  const int64_t bph = (N + ROWS - 1) / ROWS;
  const int64_t total = a.G * bph;
  const int64_t per_xcd = (total + 7) / 8;
  const int64_t logical = (int64_t)(blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (logical >= total) return;
  const int64_t g = logical / bph;
  const int64_t rb = logical % bph;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  const int lrow = lane & 31;
  const int w = a.window;
  const int row0 = (int)(rb * ROWS) + wave * (RB * 32);

  const uint4* Kg = reinterpret_cast<const uint4*>(a.keys) + (size_t)g * N * CH;
  const uint4* Cg = reinterpret_cast<const uint4*>(a.col_keys) + (size_t)g * N * CH;
  const float* crinv_g = a.col_rinv + (size_t)g * N;
  const int32_t* cpos_g = a.col_pos + (size_t)g * N;
  const int ncols = a.ncols[g];
  // the rows listed in row_pos (ascending positions); row r of the list is
  // position row_of(r), clamped to the last listed row
  const int nrows = a.nrows[g];
  if ((int64_t)rb * ROWS >= nrows) return;  // the whole workgroup, before any barrier
  const int32_t* rpos_g = a.row_pos + (size_t)g * N;
  auto row_of = [&](int r) TWINKV_INLINE { return rpos_g[r < nrows ? r : nrows - 1]; };

  // ---- row keys as MFMA B operands, row state
  bf16x8 brow[RB][KS];
  float best[RB], second[RB];  // second: the largest maximum of the other tiles
  int btile[RB];
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    const int r = row0 + 32 * b + lrow;
    const int i = row_of(r);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      uint4 v = {0u, 0u, 0u, 0u};
      if (r < nrows) v = Kg[(size_t)i * CH + 2 * s + h];
      brow[b][s] = __builtin_bit_cast(bf16x8, v);
    }
    best[b] = -__builtin_inff();
    second[b] = -__builtin_inff();
    btile[b] = -1;
  }

  // ---- byte offsets of this lane's stage loads and A-operand reads.  Load t
  // of a stage reads column (tid + NT*t)/CH at a swizzled chunk, and the
  // A operand of tile tt reads column 32*tt + lrow.  The swizzle repeats
  // every 16 columns, so the per-lane part of either address is the same for
  // every t and tt; the rest is a uniform stride (an SGPR base or an
  // instruction offset).
  static_assert((NT / CH) % kSwzPeriod == 0 && 32 % kSwzPeriod == 0, "swizzle period");
  uint32_t ld_off, a_off[KS];
  {
    const int c = tid / CH;
    ld_off = (uint32_t)((c * CH + ((tid % CH) ^ swz<CH>(c))) * 16);
#pragma unroll
    for (int s = 0; s < KS; ++s) a_off[s] = (uint32_t)((lrow * CH + ((2 * s + h) ^ swz<CH>(lrow))) * 16);
  }

  // ---- stage issue: direct loads into one LDS buffer.  A stage whose
  // columns all exist takes uniform bases and the per-lane offsets above; the
  // last, partial stage clamps its columns to the last one (every address
  // valid; the tiles past the end are masked).
  auto issue = [&](int col0, Stage<D, SC>& sb) TWINKV_INLINE {
    if (col0 + SC <= ncols) {
      const char* base = reinterpret_cast<const char*>(Cg + (size_t)col0 * CH);
#pragma unroll
      for (int t = 0; t < LOADS; ++t) dma16(base + (size_t)NT * 16 * t + ld_off, &sb.keys[NT * t + wave * 64]);
      if (wave < SC / 64) {
        dma4(crinv_g + col0 + tid, &sb.rinv[wave * 64]);
        dma4(cpos_g + col0 + tid, &sb.pos[wave * 64]);
      }
      return;
    }
    const int lastc = ncols - 1;
#pragma unroll
    for (int t = 0; t < LOADS; ++t) {
      // column tid/CH + (NT/CH)*t of the stage, chunk as in ld_off
      const int c = col0 + tid / CH + (NT / CH) * t;
      const int col = c < lastc ? c : lastc;
      dma16(reinterpret_cast<const char*>(Cg + (size_t)col * CH) + (ld_off & (CH * 16 - 1)),
            &sb.keys[NT * t + wave * 64]);
    }
    if (wave < SC / 64) {
      const int col = col0 + tid < lastc ? col0 + tid : lastc;
      dma4(crinv_g + col, &sb.rinv[wave * 64]);
      dma4(cpos_g + col, &sb.pos[wave * 64]);
    }
  };

  // ---- per-tile pieces
  auto load_a = [&](const Stage<D, SC>& sb, int tt, bf16x8 (&A)[KS]) TWINKV_INLINE {
    const char* kb = reinterpret_cast<const char*>(sb.keys) + tt * 32 * CH * 16;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      A[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(kb + a_off[s]));
  };
  auto load_rv = [&](const Stage<D, SC>& sb, int tt, float (&rv)[16]) TWINKV_INLINE {
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const float4 r4 = *reinterpret_cast<const float4*>(&sb.rinv[tt * 32 + 8 * gq + 4 * h]);
      rv[4 * gq + 0] = r4.x;
      rv[4 * gq + 1] = r4.y;
      rv[4 * gq + 2] = r4.z;
      rv[4 * gq + 3] = r4.w;
    }
  };
  // first and last row position of the wave (wave-uniform)
  const int rlo = __builtin_amdgcn_readfirstlane(row_of(row0));
  const int rhi = __builtin_amdgcn_readfirstlane(row_of(row0 + RB * 32 - 1));
  // Bit tt set: some block of the wave's rows meets the |i-j| <= w band or
  // the ragged tail in tile tt of stage st (wave-uniform).
  auto masked_tiles = [&](const Stage<D, SC>& sb, int st) TWINKV_INLINE {
    unsigned bits = 0;
#pragma unroll
    for (int tt = 0; tt < TILES; ++tt) {
      const int c0 = (st * TILES + tt) * 32;
      const int pmin = __builtin_amdgcn_readfirstlane(sb.pos[tt * 32]);
      const int pmax = __builtin_amdgcn_readfirstlane(sb.pos[tt * 32 + 31]);
      const bool mk = (c0 + 31 >= ncols) || (pmin <= rhi + w && pmax >= rlo - w);
      bits |= (unsigned)mk << tt;
    }
    return bits;
  };
  // Bit tt set: tile tt of stage st reaches past the last column.
  auto tail_tiles = [&](int st) TWINKV_INLINE {
    unsigned bits = 0;
#pragma unroll
    for (int tt = 0; tt < TILES; ++tt) bits |= (unsigned)((st * TILES + tt) * 32 + 31 >= ncols) << tt;
    return bits;
  };
  auto mfma_block = [&](const bf16x8 (&A)[KS], int b, f32x16& acc) TWINKV_INLINE {
    acc = (f32x16){};
#pragma unroll
    for (int s = 0; s < KS; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[s], brow[b][s], acc, 0, 0, 0);
  };
  // Epilogue of block b of a tile whose dots are in acc: y = dot * rinv_j, the
  // block maximum, running maximum and first tile (a masked tile leaves the
  // state alone).
  auto epilogue = [&](f32x16& acc, int b, const float (&rv)[16], bool live, int tile) TWINKV_INLINE {
    float yy[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      acc[r] *= rv[r];
      yy[r] = acc[r];
    }
    const float m = max16(yy);
    if (live) {  // wave-uniform: a masked tile leaves the state alone
      second[b] = __builtin_amdgcn_fmed3f(m, best[b], second[b]);  // second <= best: max(second, min(m, best))
      btile[b] = m > best[b] ? tile : btile[b];
      best[b] = __builtin_fmaxf(best[b], m);
    }
  };
  // Keep the next tile's MFMAs between the epilogue's vector instructions.
  auto interleave = [&]() TWINKV_INLINE {
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 7, 0);  // up to seven VALU
    }
  };

  // ---- the sweep: a rolling pipeline over (tile, block).  After block b's
  // epilogue for tile t its accumulator takes the MFMAs of block b for tile
  // t+1, which run while block b+1's epilogue executes.  The epilogue reads
  // only registers, so once the last tile's operands of stage s are read the
  // one wait and barrier of the stage publish stage s+1, the loads of stage
  // s+2 go into stage s's buffer, and the last tile's epilogue overlaps the
  // next stage's first MFMAs.  Masked tiles only leave the state unchanged
  // here; the band tiles are contiguous, their range is recorded.
  const int nstages = (ncols + SC - 1) / SC;
  f32x16 acc[RB];
  bf16x8 A[KS];
  float rv[16];
  int band_lo = INT_MAX, band_hi = -1;  // masked tiles other than the tail
  if (nstages > 0) issue(0, buf0);
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();
  if (nstages > 1) issue(SC, buf1);
  if (nstages > 0) {
    load_a(buf0, 0, A);
#pragma unroll
    for (int b = 0; b < RB; ++b) mfma_block(A, b, acc[b]);
    load_rv(buf0, 0, rv);
  }
  auto stage = [&](int st, Stage<D, SC>& cur, const Stage<D, SC>& nxt) TWINKV_INLINE {
    const unsigned mbits = __builtin_amdgcn_readfirstlane(masked_tiles(cur, st));
    const unsigned tailbits = __builtin_amdgcn_readfirstlane(tail_tiles(st));
    const unsigned bbits = mbits & ~tailbits;
    if (bbits != 0u) {
      band_lo = min(band_lo, st * TILES + __builtin_ctz(bbits));
      band_hi = max(band_hi, st * TILES + 31 - __builtin_clz(bbits));
    }
#pragma unroll
    for (int tt = 0; tt < TILES - 1; ++tt) {
      const int tile = st * TILES + tt;
      load_a(cur, tt + 1, A);
      const bool live = ((mbits >> tt) & 1u) == 0u;
#pragma unroll
      for (int b = 0; b < RB; ++b) {
        epilogue(acc[b], b, rv, live, tile);
        mfma_block(A, b, acc[b]);
        interleave();
      }
      // this tile's inverse norms are no longer needed: fetch the next tile's
      // into the same registers while the last block's MFMAs run
      load_rv(cur, tt + 1, rv);
    }
    // every operand of this stage has been read: publish the next one
    const bool more = st + 1 < nstages;
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
    if (st + 2 < nstages) issue((st + 2) * SC, cur);
    if (more) load_a(nxt, 0, A);
    const int tile = st * TILES + TILES - 1;
    const bool live = ((mbits >> (TILES - 1)) & 1u) == 0u;
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      epilogue(acc[b], b, rv, live, tile);
      if (more) mfma_block(A, b, acc[b]);
      interleave();
    }
    if (more) load_rv(nxt, 0, rv);
  };
#pragma unroll 1
  for (int st = 0; st < nstages; st += 2) {
    stage(st, buf0, buf1);
    if (st + 1 >= nstages) break;
    stage(st + 1, buf1, buf0);
  }

  // ---- masked tiles (the band range and the partial last tile), recomputed
  // from global memory with the band and the tail excluded.  They come after
  // later tiles: an exact tie with the running maximum goes to the lower
  // tile, as it would have in column order.  The whole wave is active (the
  // MFMA reads every lane).
  {
    const int ntiles = (ncols + 31) / 32;
    const int last = ntiles - 1;
    const int nband = band_hi >= 0 ? band_hi - band_lo + 1 : 0;
    const bool last_extra = ntiles > 0 && (ncols & 31) != 0 && !(nband > 0 && last >= band_lo && last <= band_hi);
    const int nproc = nband + (last_extra ? 1 : 0);
#pragma unroll 1
    for (int k = 0; k < nproc; ++k) {
      const int t = k < nband ? band_lo + k : last;
      const int c0 = t * 32;
      bf16x8 Am[KS];
      {
        const int c = c0 + lrow < ncols ? c0 + lrow : ncols - 1;  // clamped; masked below
#pragma unroll
        for (int s = 0; s < KS; ++s) Am[s] = __builtin_bit_cast(bf16x8, Cg[(size_t)c * CH + 2 * s + h]);
      }
      float rvm[16];
      int jpos[16];
      bool cval[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int col = c0 + tile_col(r, h);
        cval[r] = col < ncols;
        const int cc = cval[r] ? col : ncols - 1;
        rvm[r] = crinv_g[cc];
        jpos[r] = cpos_g[cc];
      }
#pragma unroll
      for (int b = 0; b < RB; ++b) {
        f32x16 y;
        mfma_block(Am, b, y);
        const int i = row_of(row0 + 32 * b + lrow);
        float yy[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int dist = i > jpos[r] ? i - jpos[r] : jpos[r] - i;
          y[r] = (cval[r] && dist > w) ? y[r] * rvm[r] : -__builtin_inff();
          yy[r] = y[r];
        }
        const float m = max16(yy);
        second[b] = __builtin_amdgcn_fmed3f(m, best[b], second[b]);
        if (m > best[b] || (m == best[b] && t < btile[b])) {
          best[b] = m;
          btile[b] = t;
        }
      }
    }
  }

  // ---- exact fp64 fixup of the best twin and outputs (unrolled: the
  // per-block state stays in registers).  Each half-wave holds, for its row,
  // the fp32 maximum over its 16 columns of every tile and the first tile
  // attaining it.  Only a half whose maximum can be the row's is looked at:
  // its 16 candidates are screened with fp32 dot products and those within a
  // safe margin of the largest, which always include the exact maximum, are
  // evaluated exactly in fp64.  Both lanes of the row do the work, each over
  // the feature chunks it holds as MFMA operands (chunks 2s+h), and
  // add their partial sums: the two lanes obtain identical values and
  // decisions, so the row's result needs no further merge.
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    const int i = row_of(row0 + 32 * b + lrow);
    const bool row_ok = row0 + 32 * b + lrow < nrows;
    double bb = -1.0;
    int aa = -1;
    const double ni = row_ok ? a.nsq[(size_t)g * N + i] : 0.0;
    // |fp32 value - exact| stays below 1e-5 * ||k_i|| for the sweep's and
    // this screen's sums of at most 128 exact products (then scaled by
    // rinv_j); the margin is eight times that
    const float margin = 8e-5f * (float)sqrt(ni) + 1e-30f;
    const float other = __shfl_xor(best[b], 32);
    const bool look = row_ok && btile[b] >= 0 && best[b] >= other - margin;
    const bool look_o = __shfl_xor((int)look, 32) != 0;
    const int tile_o = __shfl_xor(btile[b], 32);
    // the halves of the row to examine, the same in both lanes of the row:
    // the first pass takes each row's lower looking half, the second (rare)
    // its upper half when both halves are within the margin
    const bool look0 = (h == 0) ? look : look_o;
    const bool look1 = (h == 1) ? look : look_o;
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      const int p = (pass == 0 && look0) ? 0 : 1;
      const bool lk = pass == 0 ? (look0 || look1) : (look0 && look1);
      const int tp = (h == p) ? btile[b] : tile_o;
      if (__ballot(lk) == 0ull) continue;
      if (lk) {
        // this lane's feature chunks of row i, reloaded (the sweep's copy is
        // not kept alive this long)
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
#pragma unroll
          for (int u = 0; u < BATCH; ++u) {
            const int col = tp * 32 + tile_col(r0 + u, p);
            const int cc = col < ncols ? col : ncols - 1;
            const int j = cpos_g[cc];
            const uint4* kj = Kg + (size_t)j * CH;
#pragma unroll
            for (int s2 = 0; s2 < KS; ++s2) q[u][s2] = kj[2 * s2 + h];
            rj[u] = crinv_g[cc];
          }
#pragma unroll
          for (int u = 0; u < BATCH; ++u) {
            const int col = tp * 32 + tile_col(r0 + u, p);
            const int cc = col < ncols ? col : ncols - 1;
            const int j = cpos_g[cc];
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
        // the candidates as a bit set (invalid ones are -inf); the loop runs
        // as often as the most candidates any lane has, usually once or twice
        unsigned cm = 0u;
#pragma unroll
        for (int r = 0; r < 16; ++r) cm |= (ya[r] > -__builtin_inff() && ya[r] >= ymax - margin) ? 1u << r : 0u;
#pragma unroll 1
        while (cm != 0u) {
          const int r = __builtin_ctz(cm);
          cm &= cm - 1u;
          const int col = tp * 32 + 8 * (r >> 2) + 4 * p + (r & 3);
          const int j = cpos_g[col];
          const uint4* kj = Kg + (size_t)j * CH;
          double part = 0.0;
#pragma unroll
          for (int s2 = 0; s2 < KS; ++s2) part += dot8_exact(kr[s2], kj[2 * s2 + h]);
          const double dot = part + __shfl_xor(part, 32);
          const double nn = ni * a.nsq[(size_t)g * N + j];
          double sim = nn > 0.0 ? dot / sqrt(nn) : 0.0;
          sim += 0.0;
          if (aa < 0 || sim > bb || (sim == bb && j < aa)) {
            bb = sim;
            aa = j;
          }
        }
      }
    }
    // another tile of either half within twice the fp32 error of the row's
    // maximum may hold the exact best: queue the row for the exact resolve,
    // with candidates down to the screening margin below the maximum (in
    // cosine units).  A zero key is settled here: all its cosines are exactly
    // 0 and the first tile holds the lowest eligible position.
    const float ymax = __builtin_fmaxf(best[b], other);
    const bool near = second[b] >= ymax - 2e-5f * (float)sqrt(ni);
    const bool near_o = __shfl_xor((int)near, 32) != 0;  // both lanes of the row take part in the shuffle
    const bool amb = row_ok && ni > 0.0 && ymax > -__builtin_inff() && (near || near_o);
    if (h == 0 && row_ok) {
      const size_t o = (size_t)g * N + i;
      a.best_sim[o] = bb;
      a.best_idx[o] = aa;
      if (amb) {
        const int k = atomicAdd(&a.q.count[g], 1);
        a.q.row[o - i + k] = i;
        a.q.thr[o - i + k] = (float)((double)ymax / sqrt(ni)) - 8e-5f;
      }
    }
  }
}

template <class S>
hipError_t launch_dm(const GramArgs& a, hipStream_t stream) {
  const int64_t bph = (a.N + S::ROWS - 1) / S::ROWS;
  const int64_t total = a.G * bph;
  const int64_t grid = 8 * ((total + 7) / 8);
  if (grid > INT_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gram_kernel<S>), dim3((unsigned)grid), dim3(64 * S::WAVES), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gram(const GramArgs& a, hipStream_t stream) {
  return a.d == 64 ? launch_dm<Shape64>(a, stream) : launch_dm<Shape128>(a, stream);
}

}  // namespace twinkv
