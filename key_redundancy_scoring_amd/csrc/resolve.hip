// Exact resolve of the rows a sweep's fp32 screen cannot settle.
//
// Both sweeps ("TwinKV: A Composable Repair Pass ...", section 3.2 Eq. 2 and
// section 3.4 Eq. 4: the best twin is the largest cosine over the row's
// nonlocal, and in the repair pass retained, columns, at its lowest
// position) keep per half-row only the fp32 maximum and the first tile that
// attains it, and settle that tile's columns in fp64.  Beside it they track
// the largest maximum of the other tiles; when it comes within twice the
// fp32 error of the row's maximum, another tile may hold the exact best, and
// the row is queued with a cosine threshold a safe margin below its fp32
// maximum.
//
// Here the columns of each head are cut into segments of kSegCols, one
// workgroup per (head, segment).  Its waves take the head's queued rows 32
// at a time as an MFMA B operand and sweep the segment's columns: the A
// operands are read straight from memory, the next tile's while the current
// tile is tested, and the columns' inverse norms and positions come from
// LDS.  Every column with |i - j| > w whose fp32 cosine reaches the row's
// threshold is listed; the threshold lies below the true maximum by more
// than the fp32 error, so the exact best is always among those candidates.
// A second kernel evaluates the listed candidates in fp64, one per thread,
// so their loads overlap; a row whose candidates do not fit the list is
// evaluated over all its columns by a third.  Results merge through a 64-bit
// atomic maximum of (exact cosine, position) packed as in the score pass:
// into the score pass's own packed best, or, for the repair pass, into a
// scratch array that a last kernel turns back into (b, a) for the queued
// rows.
#include "sweep.h"

namespace twinkv {
namespace {

constexpr int kSegCols = 1024;
constexpr int kWaves = 4;

template <int D>
__global__ __launch_bounds__(64 * kWaves, D == 64 ? 4 : 2) void rowres_kernel(RowResArgs a, int64_t nseg) {
  constexpr int CH = D / 8;
  constexpr int KS = D / 16;
  const int64_t g = blockIdx.x / nseg;
  const int seg = (int)(blockIdx.x % nseg);
  const int64_t N = a.N;
  const int nq = a.q.count[g];
  const int nc = a.ncols ? a.ncols[g] : (int)N;
  const int c_lo = seg * kSegCols;
  const int c_hi = c_lo + kSegCols < nc ? c_lo + kSegCols : nc;
  if (nq <= 0 || c_lo >= c_hi) return;  // the whole workgroup
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int h = lane >> 5;
  const int lrow = lane & 31;
  const int w = a.window;
  const uint4* Kg = reinterpret_cast<const uint4*>(a.keys) + (size_t)g * N * CH;
  const uint4* Cg = reinterpret_cast<const uint4*>(a.col_keys) + (size_t)g * N * CH;
  const float* crinv_g = a.col_rinv + (size_t)g * N;
  const int32_t* cpos_g = a.col_pos ? a.col_pos + (size_t)g * N : nullptr;
  const int32_t* qrow = a.q.row + (size_t)g * N;
  const float* qthr = a.q.thr + (size_t)g * N;

  // the segment's inverse norms and positions, staged once (positions past
  // the segment's end read as -1)
  __shared__ float s_rinv[kSegCols];
  __shared__ int s_pos[kSegCols];
  for (int t = threadIdx.x; t < kSegCols; t += 64 * kWaves) {
    const int col = c_lo + t;
    s_rinv[t] = col < c_hi ? crinv_g[col] : 0.0f;
    s_pos[t] = col < c_hi ? (cpos_g ? cpos_g[col] : col) : -1;
  }
  __syncthreads();

  // one tile's A operand: the chunks 2s+h of column c0 + lrow
  struct Tile {
    bf16x8 A[KS];
  };
  auto load = [&](int c0, Tile& t) TWINKV_INLINE {
    const int ca = c0 + lrow < c_hi ? c0 + lrow : c_hi - 1;
#pragma unroll
    for (int s = 0; s < KS; ++s) t.A[s] = __builtin_bit_cast(bf16x8, Cg[(size_t)ca * CH + 2 * s + h]);
  };

#pragma unroll 1
  for (int c = wave; c * 32 < nq; c += kWaves) {  // wave-uniform
    const int k = c * 32 + lrow;
    const bool valid = k < nq;
    const int i = qrow[valid ? k : nq - 1];
    const float thr = valid ? qthr[k] : __builtin_inff();  // a padding lane takes no candidate
    const float ri = a.rinv[(size_t)g * N + i];
    bf16x8 B[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) B[s] = __builtin_bit_cast(bf16x8, Kg[(size_t)i * CH + 2 * s + h]);
    // one tile: the MFMAs on loaded operands, then (while the next tile's
    // loads are in flight) the candidate test and the rare fp64 path
    auto process = [&](int c0, const Tile& t, Tile& next, bool more) TWINKV_INLINE {
      f32x16 acc = {};
#pragma unroll
      for (int s = 0; s < KS; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(t.A[s], B[s], acc, 0, 0, 0);
      if (more) load(c0 + 32, next);
      // the lane's 16 columns are four runs of four (8q + 4h + 0..3)
      float rj[16];
      int pj[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int lc = c0 - c_lo + 8 * q + 4 * h;
        const float4 r4 = *reinterpret_cast<const float4*>(&s_rinv[lc]);
        const int4 p4 = *reinterpret_cast<const int4*>(&s_pos[lc]);
        rj[4 * q + 0] = r4.x;
        rj[4 * q + 1] = r4.y;
        rj[4 * q + 2] = r4.z;
        rj[4 * q + 3] = r4.w;
        pj[4 * q + 0] = p4.x;
        pj[4 * q + 1] = p4.y;
        pj[4 * q + 2] = p4.z;
        pj[4 * q + 3] = p4.w;
      }
      unsigned cm = 0u;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = pj[r];
        const int dist = i > j ? i - j : j - i;
        if (j >= 0 && dist > w && acc[r] * rj[r] * ri >= thr) cm |= 1u << r;
      }
#pragma unroll 1
      while (cm != 0u) {
        const int r = __builtin_ctz(cm);
        cm &= cm - 1u;
        // the position again from r (a run-time index into pj would move it
        // to scratch memory)
        const int j = s_pos[c0 - c_lo + tile_col(r, h)];
        const int slot = atomicAdd(&a.cand_count[g], 1);
        if (slot < a.cand_cap) {
          a.cand_row[g * a.cand_cap + slot] = i;
          a.cand_col[g * a.cand_cap + slot] = j;
        } else {
          // the list is full: the whole row goes to the exhaustive pass
          a.q.thr[(size_t)g * N + k] = -__builtin_inff();
        }
      }
    };
    Tile t0, t1;
    load(c_lo, t0);
#pragma unroll 1
    for (int c0 = c_lo; c0 < c_hi; c0 += 64) {  // two tiles per trip, the buffers alternating
      process(c0, t0, t1, c0 + 32 < c_hi);
      if (c0 + 32 >= c_hi) break;
      process(c0 + 32, t1, t0, c0 + 64 < c_hi);
    }
  }
}

// The heads' candidate counts start at 0; in the repair pass the queued
// rows' entries of the scratch packed array start at 0 too (below every key).
__global__ __launch_bounds__(256) void rowres_clear_kernel(RowResArgs a, bool repair) {
  const int64_t g = blockIdx.x;
  if (threadIdx.x == 0) a.cand_count[g] = 0;
  if (!repair) return;
  const int nq = a.q.count[g];
  for (int k = threadIdx.x; k < nq; k += 256) a.best64[(size_t)g * a.N + a.q.row[(size_t)g * a.N + k]] = 0ull;
}

// fp64 cosine of every listed candidate, merged into its row's packed best;
// one workgroup per head.
template <int D>
__global__ __launch_bounds__(256) void rowres_eval_kernel(RowResArgs a) {
  constexpr int CH = D / 8;
  const int64_t g = blockIdx.x;
  const int64_t N = a.N;
  const int64_t n = a.cand_count[g] < a.cand_cap ? a.cand_count[g] : a.cand_cap;
  const uint4* Kg = reinterpret_cast<const uint4*>(a.keys) + (size_t)g * N * CH;
  for (int64_t k = threadIdx.x; k < n; k += 256) {
    const int i = a.cand_row[g * a.cand_cap + k];
    const int j = a.cand_col[g * a.cand_cap + k];
    double dot = 0.0;
#pragma unroll
    for (int cc = 0; cc < CH; ++cc) dot += dot8_exact(Kg[(size_t)i * CH + cc], Kg[(size_t)j * CH + cc]);
    const double nn = a.nsq[(size_t)g * N + i] * a.nsq[(size_t)g * N + j];
    const double sim = (nn > 0.0 ? dot / sqrt(nn) : 0.0) + 0.0;
    atomicMax((unsigned long long*)&a.best64[(size_t)g * N + i], (unsigned long long)pack_best(sim, j, a.idx_mask));
  }
}

// Rows whose candidates overflowed the list (threshold set to -inf): every
// column of the row's set with |i - j| > w in fp64, one workgroup per head
// taking such rows one at a time.  Only reached when many columns tie within
// the margin of a row's maximum (e.g. many identical keys).
template <int D>
__global__ __launch_bounds__(256) void rowres_exhaustive_kernel(RowResArgs a) {
  constexpr int CH = D / 8;
  __shared__ uint64_t red[4];
  const int64_t g = blockIdx.x;
  const int64_t N = a.N;
  const int nq = a.q.count[g];
  const int nc = a.ncols ? a.ncols[g] : (int)N;
  const uint4* Kg = reinterpret_cast<const uint4*>(a.keys) + (size_t)g * N * CH;
  const int32_t* cpos_g = a.col_pos ? a.col_pos + (size_t)g * N : nullptr;
  for (int k = 0; k < nq; ++k) {  // uniform
    if (a.q.thr[(size_t)g * N + k] != -__builtin_inff()) continue;
    const int i = a.q.row[(size_t)g * N + k];
    const double ni = a.nsq[(size_t)g * N + i];
    uint64_t best = 0ull;
    for (int c = threadIdx.x; c < nc; c += 256) {
      const int j = cpos_g ? cpos_g[c] : c;
      if ((i > j ? i - j : j - i) <= a.window) continue;
      double dot = 0.0;
#pragma unroll
      for (int cc = 0; cc < CH; ++cc) dot += dot8_exact(Kg[(size_t)i * CH + cc], Kg[(size_t)j * CH + cc]);
      const double nn = ni * a.nsq[(size_t)g * N + j];
      const uint64_t u = pack_best((nn > 0.0 ? dot / sqrt(nn) : 0.0) + 0.0, j, a.idx_mask);
      best = u > best ? u : best;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const uint64_t o = (uint64_t)__shfl_xor((long long)best, off);
      best = o > best ? o : best;
    }
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = best;
    __syncthreads();
    if (threadIdx.x == 0) {
      uint64_t m = red[0];
      for (int t = 1; t < 4; ++t) m = red[t] > m ? red[t] : m;
      if (m != 0ull) atomicMax((unsigned long long*)&a.best64[(size_t)g * N + i], (unsigned long long)m);
    }
    __syncthreads();
  }
}

// Repair pass: (b, a) of each queued row from its packed best, the cosine
// recomputed exactly for the position found.
template <int D>
__global__ __launch_bounds__(256) void rowres_finish_kernel(RowResArgs a) {
  constexpr int CH = D / 8;
  const int64_t g = blockIdx.x;
  const int64_t N = a.N;
  const int nq = a.q.count[g];
  const uint4* Kg = reinterpret_cast<const uint4*>(a.keys) + (size_t)g * N * CH;
  for (int k = threadIdx.x; k < nq; k += 256) {
    const int i = a.q.row[(size_t)g * N + k];
    const size_t o = (size_t)g * N + i;
    const uint64_t u = a.best64[o];
    if (u == 0ull) continue;  // not reached: a queued row has a candidate
    const int j = unpack_idx(u, a.idx_mask);
    double dot = 0.0;
#pragma unroll
    for (int cc = 0; cc < CH; ++cc) dot += dot8_exact(Kg[(size_t)i * CH + cc], Kg[(size_t)j * CH + cc]);
    const double nn = a.nsq[o] * a.nsq[(size_t)g * N + j];
    a.best_sim[o] = (nn > 0.0 ? dot / sqrt(nn) : 0.0) + 0.0;
    a.best_idx[o] = j;
  }
}

}  // namespace

int64_t rowres_cand_cap(int64_t N) {
  const int64_t c = N / 8;
  return c > 256 ? c : 256;
}

hipError_t launch_rowres(const RowResArgs& a, hipStream_t stream) {
  const int64_t nseg = (a.N + kSegCols - 1) / kSegCols;
  if (a.G > 0x7fffffffLL || a.G * nseg > 0x7fffffffLL) return hipErrorInvalidValue;
  const bool repair = a.best_sim != nullptr;
  hipLaunchKernelGGL(rowres_clear_kernel, dim3((unsigned)a.G), dim3(256), 0, stream, a, repair);
  if (a.d == 64) {
    hipLaunchKernelGGL(rowres_kernel<64>, dim3((unsigned)(a.G * nseg)), dim3(64 * kWaves), 0, stream, a, nseg);
    hipLaunchKernelGGL(rowres_eval_kernel<64>, dim3((unsigned)a.G), dim3(256), 0, stream, a);
    hipLaunchKernelGGL(rowres_exhaustive_kernel<64>, dim3((unsigned)a.G), dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL(rowres_kernel<128>, dim3((unsigned)(a.G * nseg)), dim3(64 * kWaves), 0, stream, a, nseg);
    hipLaunchKernelGGL(rowres_eval_kernel<128>, dim3((unsigned)a.G), dim3(256), 0, stream, a);
    hipLaunchKernelGGL(rowres_exhaustive_kernel<128>, dim3((unsigned)a.G), dim3(256), 0, stream, a);
  }
  if (repair) {
    if (a.d == 64)
      hipLaunchKernelGGL(rowres_finish_kernel<64>, dim3((unsigned)a.G), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL(rowres_finish_kernel<128>, dim3((unsigned)a.G), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace twinkv
