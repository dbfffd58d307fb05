// Internal declarations shared by the library's HIP translation units.
// Not part of the public ABI (include/twinkv.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace twinkv {

// Rows whose best twin the fp32 screen of a sweep cannot settle: another
// tile than the first one attaining a half-row's maximum comes within twice
// the fp32 error of it.  Each head's queue holds the positions of such rows
// and, per entry, the cosine threshold of the candidates to evaluate exactly.
struct RowQueue {
  int32_t* row;    // [G][N] queued positions of head g at g*N + k, k < count[g]
  float* thr;      // [G][N] candidate threshold (cosine) of entry k
  int32_t* count;  // [G] entries per head; zeroed before the sweep that fills it
};

// Exact resolve of queued rows (resolve.hip): every column j of the row's
// column set with |i - j| > w whose fp32 cosine reaches the entry's threshold
// is evaluated in fp64, the largest (lowest position on ties) wins.
struct RowResArgs {
  const uint16_t* keys;      // bf16 [G][N][d]
  const double* nsq;         // ||k||^2 [G][N]
  const float* rinv;         // 1/||k|| [G][N]
  const uint16_t* col_keys;  // bf16 [G][N][d]: the columns (all keys, or the retained keys compacted)
  const float* col_rinv;     // [G][N] inverse norms of the columns
  const int32_t* col_pos;    // [G][N] position of each compacted column; null: column c is position c
  const int32_t* ncols;      // [G] columns per head; null: N
  RowQueue q;
  int64_t G, N;
  int32_t d, window;
  // outputs: the atomic maximum of each queued row's packed result (positions
  // in the idx_mask bits) in best64 [G][N]; when best_sim is not null (the
  // repair pass) best64 is scratch whose queued entries are zeroed first, and
  // (b, a) of the queued rows are written to best_sim / best_idx at the end
  uint64_t* best64;
  uint64_t idx_mask;
  double* best_sim;
  int32_t* best_idx;
  // candidates found by the sweep, evaluated in fp64 by a second kernel:
  // head g's entry k < min(cand_count[g], cand_cap) is row cand_row[g*cand_cap
  // + k] and column position cand_col[g*cand_cap + k]; a row with a
  // candidate past the capacity is evaluated over all its columns instead
  int32_t* cand_row;
  int32_t* cand_col;
  int32_t* cand_count;  // [G]
  int64_t cand_cap;     // entries per head
};
// Candidate-list capacity per head of the exact resolve for N positions.
int64_t rowres_cand_cap(int64_t N);
hipError_t launch_rowres(const RowResArgs& a, hipStream_t stream);

// Restricted Gram sweep of the repair pass (gram.hip).
struct GramArgs {
  const uint16_t* keys;      // bf16 [G][N][d]: the rows (and the fp64 fixup's operands)
  const double* nsq;         // ||k||^2 in fp64 [G][N]
  const uint16_t* col_keys;  // bf16 [G][N][d]: the retained keys, compacted in position order
  const float* col_rinv;     // 1/||k|| in fp32 of each column [G][N] (0 for a zero key)
  const int32_t* col_pos;    // original position of each compacted column, ascending [G][N]
  const int32_t* ncols;      // number of retained positions per head [G]
  const int32_t* row_pos;    // positions of the rows to sweep, ascending [G][N]
  const int32_t* nrows;      // number of rows to sweep per head [G]
  int64_t G, N;
  int32_t d, window;
  RowQueue q;  // rows left to the exact resolve (count zeroed by the rows pass)
  // outputs
  double* best_sim;
  int32_t* best_idx;
};

// Single-order score sweep (tri.hip).  Each unordered nonlocal pair is
// computed once, in the workgroup of its lower position's row block: the
// row side (the lower position's maximum over later columns) is tracked per
// row in registers, the column side (each later position's
// maximum over the block's rows) is reduced across lanes and stored per
// (row block, column), and a resolve pass finds the exact best twin.
struct TriArgs {
  const uint16_t* keys;  // bf16 [G][N][d]
  const double* nsq;     // ||k||^2 [G][N]
  const float* rinv;     // 1/||k|| [G][N]
  const double* energy;  // ||v||^2 [G][N]
  int64_t G, N;
  int32_t d, window;
  double tau;
  int64_t nb;            // row blocks per head
  uint64_t idx_mask;     // 2^b - 1, the smallest with 2^b >= N: position bits of a packed best
  int64_t words;         // 32-bit candidate words per (head, row block): ceil(N/32)
  // workspace
  int32_t* part;         // column maxima per (head, row block), order-preserving fp32 bits; block rb
                         // of head g holds columns rb*ROWS .. N-1 (see tri_part_offset)
  float* rowcos;         // [G][N] fp32 row-side maximum cosine, -inf if none
  int32_t* rcount;       // [G][N] row-side counts
  int32_t* ccount;       // [G][N] column-side counts (cleared before the sweep)
  uint64_t* best64;      // [G][N] packed (exact cosine, position) of the best twin found so far; 0 = none
  float* colmax;         // [G][N] fp32 maximum cosine over both sides
  uint32_t* cbits;       // [G][nb][words] candidate row blocks of each position (cleared before the sweep)
  RowQueue q;            // rows whose row side the sweep cannot settle (count cleared before the sweep)
  int32_t* cand_row;     // candidate lists of the exact resolve (see RowResArgs)
  int32_t* cand_col;
  int32_t* cand_count;
  int64_t cand_cap;
  // outputs
  int32_t* count;
  double* best_sim;
  int32_t* best_idx;
  double* score;
  double* omega;         // may be null
};
// Rows per row block of the single-order sweep at head dim d (64 or 128).
int tri_rows(int d);
// Entries of the column-maximum array per head.
int64_t tri_part_per_head(int64_t N, int rows);
// Clear, sweep, then resolve (queued rows, column maxima, candidate blocks,
// exact column side, final outputs).  `mark` (may be null) is recorded between the sweep
// and the resolve kernels.
hipError_t launch_tri(const TriArgs& a, hipStream_t stream, hipEvent_t mark);

// nsq = ||k||^2 (fp64), rinv = 1/||k|| (fp32, 0 for a zero key) and energy =
// ||v||^2 (fp64; skipped when values is null).
hipError_t launch_norms(const uint16_t* keys, const uint16_t* values, int64_t nkeys, int d, double* nsq,
                        float* rinv, double* energy, hipStream_t stream);
hipError_t launch_gram(const GramArgs& a, hipStream_t stream);


struct SelectArgs {
  const double* score;
  const double* energy;
  const int32_t* capacity;
  const int64_t* kept_off;  // [G+1] start of each head's run in kept_idx
  uint8_t* keep;
  int32_t* kept_idx;
  int64_t G, N;
  int32_t sink, recent;
};
hipError_t launch_select(const SelectArgs& a, hipStream_t stream);
// kept_off[0] = 0, kept_off[g+1] = kept_off[g] + clamp(capacity[g], 0, N).
hipError_t launch_offsets(const int32_t* capacity, int64_t G, int64_t N, int64_t* kept_off, hipStream_t stream);
// Selection keys of a score variant (0 twin, 1 value, 2 rarity), optionally
// with permuted counts.
hipError_t launch_variant(const int32_t* count, const double* energy, const int32_t* perm, int64_t G, int64_t N,
                          int variant, double* score, double* tie, hipStream_t stream);

hipError_t launch_compact(const uint8_t* keep_in, int64_t G, int64_t N, int32_t* pos, int32_t* ncols,
                          hipStream_t stream);
// The rows the restricted sweep must visit (all rows without a prior); rows
// whose unrestricted best twin is retained or absent take it as b_i(S0).
hipError_t launch_rows(const uint8_t* keep_in, const double* prior_sim, const int32_t* prior_idx, int64_t G,
                       int64_t N, int32_t* row_pos, int32_t* nrows, double* best_sim, int32_t* best_idx,
                       int32_t* qcount, hipStream_t stream);
// Copy the retained keys and their inverse norms into column order.
hipError_t launch_gather(const uint16_t* keys, const float* rinv, const int32_t* pos, const int32_t* ncols, int64_t G,
                         int64_t N, int d, uint16_t* ckeys, float* crinv, hipStream_t stream);

// Pack the retained keys (and values, if not null) of every head in sequence
// order: head g's rows kept_idx[kept_off[g] .. kept_off[g+1]) go to rows
// kept_off[g].. of out_keys / out_values ([total][d]).
hipError_t launch_gather_kv(const uint16_t* keys, const uint16_t* values, const int32_t* kept_idx,
                            const int64_t* kept_off, int64_t G, int64_t N, int d, int64_t total, uint16_t* out_keys,
                            uint16_t* out_values, hipStream_t stream);

// Head allocation from prefix attention (alloc.hip).
constexpr int kMaxQueries = 128;  // Gq * W observing queries per KV head
constexpr int kMaxHeads = 1024;   // KV heads per layer

struct AttnArgs {
  const uint16_t* keys;     // bf16 [G][N][d]
  const uint16_t* queries;  // bf16 [G][Gq][W][d]
  int64_t G, N;
  int32_t Gq, W, pool;
  int64_t nchunk;           // blocks of 256 keys per head
  double inv_sqrt_d, inv_gq;
  double* part;             // [G][nchunk][Gq*W][2] block (max, sum of exp)
  double* mz;               // [G][Gq*W][2] per query (max, normaliser)
  double* agg;              // [G][N] attention summed over queries, averaged over query heads
  float* z;                 // [G][N] pooled fp32 scores
  int64_t s_cnt, r_cnt;     // protected leading / trailing positions
};
struct AllocArgs {
  const float* z;           // [G][N] pooled fp32 scores
  int64_t G, N, L;          // heads, positions, layers
  int32_t H;                // KV heads per layer
  int64_t s_cnt, width;     // unprotected positions s_cnt .. s_cnt + width - 1 of a head
  int64_t U, P;
  uint32_t* hist;           // [L][2048] digit histograms (workspace)
  uint32_t* prefix;         // [L] threshold bits (workspace)
  int64_t* need;            // [L] entries still to take at the threshold (workspace)
  uint32_t* counts;         // [G][3] above, at the threshold, nonzero (workspace)
  int32_t* capacity;        // [G] out
  int32_t* g_count;         // [G] out, may be null
};
hipError_t launch_attn(const AttnArgs& a, int d, int phase, hipStream_t stream);
hipError_t launch_alloc(const AllocArgs& a, hipStream_t stream);
hipError_t launch_fill_capacity(int32_t* capacity, int32_t* g_count, int64_t G, int32_t B, hipStream_t stream);

// Count statistics (stats.hip): int64 [G][kStatInts] counts and double
// [G][2] (sum of normalised discounts, value-only energy cut) per head.
constexpr int kStatInts = 26;
struct StatsArgs {
  const int32_t* count;
  const double* energy;
  const uint8_t* keep_twin;   // may be null (then keep_value is null too)
  const uint8_t* keep_value;
  const int32_t* capacity;
  int64_t* stats;
  double* fstats;
  int64_t G, N;
  int32_t sink, recent;
};
hipError_t launch_stats(const StatsArgs& a, hipStream_t stream);

struct SwapArgs {
  const uint8_t* keep_in;
  const double* best;
  const int32_t* ncols;  // |S0| per head
  uint8_t* keep_out;
  int32_t* n_orphans;
  int32_t* n_donors;
  int32_t* n_swaps;
  int32_t* pairs;        // [G][N/2][2]
  uint64_t* keys_a;      // workspace [G][N]
  int32_t* idx_a;        // workspace [G][N]
  uint64_t* keys_b;      // workspace [G][N]
  int32_t* idx_b;        // workspace [G][N]
  int64_t G, N;
  double tau;
  int32_t sink, recent;
};
hipError_t launch_swap(const SwapArgs& a, hipStream_t stream);

}  // namespace twinkv
