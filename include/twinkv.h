/*
 * twinkv.h - C ABI of the MI355X (gfx950) key-redundancy scoring library.
 *
 * The library computes, independently for every (batch, layer, KV head) --
 * called a "head" below, G of them, each with N positions and head dim d --
 * the quantities of TwinKV-style KV-cache compression:
 *
 *   twinkv_score   nonlocal near-duplicate counts, best nonlocal twin
 *                  (similarity and position), value energy and the
 *                  frequency-discounted score;
 *   twinkv_select  exact-budget per-head retention with protected sink and
 *                  recent positions;
 *   twinkv_variant_score  selection keys of the score variants (value only,
 *                  rarity only, permuted counts);
 *   twinkv_repair  the one-shot orphan/donor swap on a given retained set at
 *                  a fixed budget;
 *   twinkv_gather_kv  the packed, unpadded cache of the retained keys and
 *                  values in sequence order;
 *   twinkv_allocate  per-head capacities of a layer from the attention of
 *                  its last observed prefix queries;
 *   twinkv_count_stats  per-head count statistics (twin fraction, count
 *                  histogram, discount mean, selection change, margins).
 *
 * Sources (page title and section/equation):
 *   [P1] "TwinKV: A Composable Repair Pass for KV Cache Eviction via Pairwise
 *        Key Redundancy" (arXiv HTML): section 3.1, section 3.2 (Eq. 1, Eq. 2,
 *        Eq. 3, protected regions), section 3.4 (Eq. 4, orphans, donors, swap),
 *        Figure 1(b) (fraction of keys with a twin).
 *   [P2] "Small Frequency Corrections Can Change What Survives KV Cache
 *        Compression" (paperpeel): section 3.1 (budget, protection), section
 *        3.2 (count, energy, score, ties), section 3.3 (head allocation,
 *        Equation 5), section 3.4 (selection order and physical cache
 *        layout), sections 2.1, 5.3 and 5.5 (count statistics, score
 *        ablations), appendices A.2, A.3 (prefix attention, budget proof),
 *        B.2 (measured frequency statistics).
 *
 * Conventions for every entry point:
 *   - Array arguments are DEVICE pointers owned by the caller; the library
 *     never allocates, frees or keeps them after the call returns.
 *   - Per-head arrays are dense, row-major, heads outermost: element (g, i)
 *     of a [G][N] array is at g*N + i; keys/values [G][N][d] put feature t of
 *     position i of head g at (g*N + i)*d + t.  Keys and values are bfloat16
 *     (raw 16-bit patterns), finite.  Pointers must be 16-byte aligned.
 *   - Positions are 0-based; "|i - j| > window" is shift-invariant, so the
 *     pages' 1-based formulas carry over unchanged.
 *   - All work is enqueued asynchronously on `stream` (a hipStream_t, may be
 *     NULL for the null stream); the call returns before the GPU finishes.
 *     Arguments are checked on the host first: on any error nothing is
 *     launched and a negative twinkv_status is returned.  Faults inside the
 *     kernels surface at the caller's next synchronisation.
 *   - `workspace` is caller-owned device scratch of at least
 *     twinkv_workspace_bytes(op, params) bytes (256-byte aligned); it may be
 *     NULL when that size is 0.  Concurrent calls need distinct workspaces.
 *   - `marks` is optional (NULL to skip): an array of hipEvent_t created by
 *     the caller.  When given, the library records marks[k] on `stream`
 *     immediately before launching phase k and marks[P] after the last
 *     launch, where P is the phase count documented per entry point.  It
 *     serves only to time the phases.
 *   - No exception crosses the ABI.  The only global state is the
 *     per-device static scratch of twinkv_score_noalloc.
 */
#ifndef TWINKV_H
#define TWINKV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum twinkv_status {
  TWINKV_OK = 0,
  TWINKV_ERR_ARG = -1,         /* a null pointer, a size out of range, a bad parameter */
  TWINKV_ERR_UNSUPPORTED = -2, /* head dim other than 64 or 128                        */
  TWINKV_ERR_WORKSPACE = -3,   /* workspace smaller than twinkv_workspace_bytes()       */
  TWINKV_ERR_HIP = -4,         /* the HIP runtime refused a launch or an event record   */
  TWINKV_ERR_TOO_LARGE = -5    /* workspace beyond the static scratch of twinkv_score_noalloc */
} twinkv_status;

/* Problem description shared by all entry points. */
typedef struct twinkv_params {
  int64_t G;      /* number of independent heads (batch * layers * KV heads), >= 1          */
  int64_t N;      /* prefix length of every head, 1 <= N <= 2^30                             */
  int32_t d;      /* head dim: 64 or 128                                                    */
  int32_t window; /* local exclusion w >= 0: j is a twin candidate of i only if |i-j| > w
                     ([P1] section 3.2; the pages' second page calls it l); any w >= N - 1
                     leaves no candidate                                                     */
  double tau;     /* similarity threshold, -1 < tau < 1 ([P1] Eq. 2 uses sim > tau)          */
  int32_t sink;   /* leading protected positions before clipping, >= 0 ([P2] section 3.1)   */
  int32_t recent; /* trailing protected positions before clipping, >= 0                     */
} twinkv_params;

enum { TWINKV_OP_SCORE = 0, TWINKV_OP_SELECT = 1, TWINKV_OP_REPAIR = 2 };

/* Phase counts for the `marks` argument. */
enum { TWINKV_SCORE_PHASES = 3, TWINKV_SELECT_PHASES = 1, TWINKV_REPAIR_PHASES = 4, TWINKV_GATHER_PHASES = 1,
       TWINKV_ALLOC_PHASES = 3, TWINKV_VARIANT_PHASES = 1, TWINKV_STATS_PHASES = 1 };

/* Number of int64 counts per head written by twinkv_count_stats. */
enum { TWINKV_STAT_INTS = 26 };

/* Score variants for twinkv_variant_score. */
enum { TWINKV_VARIANT_TWIN = 0, TWINKV_VARIANT_VALUE = 1, TWINKV_VARIANT_RARITY = 2 };

/* Bytes of workspace an operation needs for these parameters; 0 if the
 * parameters are invalid (see the entry points) or the op needs none. */
size_t twinkv_workspace_bytes(int op, const twinkv_params* params);

/* Uniform per-head capacity B = floor(N * (1 - removal)) ([P2] section 3.1,
 * "Equation 1").  Returns -1 if N < 0 or removal is outside [0, 1]. */
int64_t twinkv_uniform_capacity(int64_t N, double removal);

/* Capacity ceil(N * (1 - removal)) of [P1] section 3.1 (evaluated in
 * double precision as written).  Returns -1 if N < 0 or removal is outside
 * [0, 1]. */
int64_t twinkv_uniform_capacity_ceil(int64_t N, double removal);

/* Human-readable text for a twinkv_status value (static storage). */
const char* twinkv_status_string(int status);

/*
 * twinkv_score - per position i of every head:
 *   count[g][i]    = #{ j : |i-j| > window, sim(i,j) > tau }           ([P1] Eq. 2, [P2] 3.2)
 *   best_sim[g][i] = max over j with |i-j| > window of sim(i,j), or -1 if no such j;
 *                    computed exactly in fp64 as dot/sqrt(n_i*n_j) for the chosen j
 *   best_idx[g][i] = the lowest j attaining best_sim, or -1 if no such j
 *   energy[g][i]   = ||v_i||^2, fp64 sum of exact squares               ([P2] 3.2)
 *   score[g][i]    = energy * ln((N+1)/(count+1)), fp64                  ([P2] 3.2)
 *   omega[g][i]    = ln((N+1)/(count+1)) / ln(N+1) (optional: may be NULL)
 * where sim(i,j) = k_i.k_j / (||k_i|| ||k_j||) is the cosine of the
 * post-RoPE keys ([P1] Eq. 1) and is 0 when either key is zero.
 * Protected positions take part in the counts ([P2] 3.2).
 * keys, values: bf16 [G][N][d].  count, best_idx: int32 [G][N].
 * best_sim, energy, score, omega: double [G][N].
 * Each unordered nonlocal pair is evaluated once (on the MFMA matrix cores,
 * bf16 products exact, fp32 sums); every candidate within the fp32 error of
 * a position's maximum is then evaluated in fp64, so best_idx is the exact
 * argmax of the fp64 cosines at its lowest position, except that cosines
 * closer than 2^(b-52) relative (b = ceil(log2 N)) rank as equal and the
 * lower position wins.  The workspace grows with N: about 52 bytes per key
 * plus 2N/R + N/(8R) bytes per key (R = 384 rows per block at d = 64, 256
 * at d = 128) for the column maxima and candidate bits of each row block.
 * Phases for `marks`: 0 = norms and energies, 1 = single-order Gram sweep
 * (counts, row-side best twin, column maxima), 2 = resolve (exact best twin
 * of the rows two tiles nearly tie, exact column-side best twin, outputs and
 * scores).
 */
int twinkv_score(const twinkv_params* params, const void* keys, const void* values,
                 int32_t* count, double* best_sim, int32_t* best_idx, double* energy,
                 double* score, double* omega, void* workspace, size_t workspace_bytes,
                 hipStream_t stream, hipEvent_t* marks);

/*
 * twinkv_score_noalloc - twinkv_score for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same kernels and the same outputs,
 * bit for bit, with the workspace twinkv_score takes (squared and inverse
 * norms, the sweep's column maxima, counters and candidate bits) carved from
 * a static device array of the library instead.  Neither this call nor the
 * library allocates or frees anything; the array,
 * TWINKV_NOALLOC_SCRATCH_BYTES (64 MiB), is part of the library's device
 * code and each device it runs on holds its own copy until the process
 * ends.  The scratch used is the current device's (hipGetDevice), so
 * `stream` must belong to it; its address is looked up on the first call on
 * each device.  Every call on a device shares that device's scratch and it
 * keeps the last call's contents (each call writes every entry it reads
 * before reading it): calls that overlap on one device, on different
 * streams or from different threads, race and give wrong results.
 * Arguments and outputs as twinkv_score; a problem whose workspace
 * (twinkv_workspace_bytes(TWINKV_OP_SCORE, params)) exceeds the array
 * returns TWINKV_ERR_TOO_LARGE before anything is launched (at d = 64 that
 * admits, e.g., 256 heads of N = 8192 or 32 heads of N = 32768).
 * Phases for `marks`: as twinkv_score.
 */
enum { TWINKV_NOALLOC_SCRATCH_BYTES = 64 << 20 };
int twinkv_score_noalloc(const twinkv_params* params, const void* keys, const void* values, int32_t* count,
                         double* best_sim, int32_t* best_idx, double* energy, double* score, double* omega,
                         hipStream_t stream, hipEvent_t* marks);

/*
 * twinkv_select - per head g with capacity b = capacity[g] (0 <= b <= N;
 * values outside are clamped): protect the first s = min(sink, b) and the
 * last r = min(recent, b - s) positions, then keep the u = b - s - r
 * unprotected positions ranked first by (score desc, energy desc, position
 * asc) ([P2] 3.1, 3.2 tie rule, 3.4).
 *   keep[g][i]  (uint8 [G][N])  1 if retained, else 0
 *   kept_idx    (int32 [kept_off[G]])  the retained positions of head g in
 *               ascending (sequence) order at kept_idx[kept_off[g] ..
 *               kept_off[g+1]) ([P2] 3.4: the kept indices stay in order)
 * score, energy: double [G][N] (as produced by twinkv_score; must be finite
 * and >= 0).  capacity: int32 [G].  kept_off: int64 [G+1] device array of
 * prefix sums of the clamped capacities (twinkv_capacity_offsets writes it).
 * Writes to kept_idx stay inside [kept_off[g], min(kept_off[g+1],
 * kept_off[G])), so offsets that do not match the capacities give wrong
 * lists, never a write outside kept_idx's kept_off[G] entries.  Of the
 * parameters only G, N, sink and recent are read; workspace may be NULL
 * (twinkv_workspace_bytes is 0).
 * Phases for `marks`: 0 = select.
 */
int twinkv_select(const twinkv_params* params, const double* score, const double* energy,
                  const int32_t* capacity, const int64_t* kept_off, uint8_t* keep, int32_t* kept_idx,
                  void* workspace, size_t workspace_bytes, hipStream_t stream, hipEvent_t* marks);

/*
 * twinkv_capacity_offsets - the kept_off array of twinkv_select and
 * twinkv_gather_kv, on the device: kept_off[0] = 0 and kept_off[g+1] =
 * kept_off[g] + clamp(capacity[g], 0, N) for g < G ([P2] 3.4: heads packed
 * one after another).  capacity: int32 [G]; kept_off: int64 [G+1] (out).
 * Requires 1 <= G < 2^31 and 1 <= N <= 2^30.  Asynchronous on `stream`.
 */
int twinkv_capacity_offsets(const int32_t* capacity, int64_t G, int64_t N, int64_t* kept_off, hipStream_t stream);

/*
 * twinkv_repair - one-shot repair of the retained set S0 = {i : keep_in[g][i] != 0}
 * of every head at its own budget K = |S0| ([P1] section 3.4):
 *   best_sim[g][i] = b_i(S0) = max over j in S0, |i-j| > window of sim(i,j), or -1
 *                    (exact fp64 for the chosen j)                       ([P1] Eq. 4)
 *   best_idx[g][i] = the lowest such j attaining it, or -1 (every candidate
 *                    within the fp32 error of the maximum is evaluated in fp64)
 *   orphans  O = { i not in S0 : b_i < tau } ranked by (b asc, i asc)
 *   donors   D = { j in S0 outside the protected regions : b_j >= tau } ranked by
 *              (b desc, j asc); the protected regions are the first
 *              min(sink, K) and the last min(recent, K - min(sink, K)) positions
 *   m = min(|O|, |D|);  S1 = S0 - D[0:m] + O[0:m], so |S1| = |S0|.
 *   keep_out[g][i]   (uint8 [G][N]) S1
 *   n_orphans, n_donors, n_swaps: int32 [G]  |O|, |D|, m
 *   swap_pairs: int32 [G][N/2][2]: (O[k], D[k]) for k < m, then (-1, -1)
 *     (m <= N/2 always: m <= min(N - K, K)).
 * keys: bf16 [G][N][d]; keep_in: uint8 [G][N].
 * prior_sim, prior_idx (double / int32 [G][N], both NULL or both given): the
 *   unrestricted best twin (best_sim, best_idx) that twinkv_score wrote for the
 *   same keys, window and tau.  Where prior_idx[g][i] is retained (or is -1:
 *   no nonlocal position exists), it is b_i(S0) with its position, since the
 *   lowest position attaining the maximum over all nonlocal j is then in S0;
 *   those rows are copied and only the others are swept.  The outputs are the
 *   same as without a prior.  An index outside [0, N) other than -1 counts as
 *   not retained (that row is swept); any other inconsistent prior gives wrong
 *   results, never an access outside the stated sizes.  Both NULL: every row
 *   is swept.
 * Phases for `marks`: 0 = norms, 1 = compaction of S0 (retained positions and a
 * contiguous copy of their keys) and of the rows to sweep, 2 = restricted
 * Gram, fixup and exact resolve of near-tied rows, 3 = classification, ranking
 * and swap.
 */
int twinkv_repair(const twinkv_params* params, const void* keys, const uint8_t* keep_in,
                  const double* prior_sim, const int32_t* prior_idx, uint8_t* keep_out,
                  double* best_sim, int32_t* best_idx, int32_t* n_orphans, int32_t* n_donors,
                  int32_t* n_swaps, int32_t* swap_pairs, void* workspace, size_t workspace_bytes,
                  hipStream_t stream, hipEvent_t* marks);

/*
 * twinkv_variant_score - selection keys of a score variant for twinkv_select,
 * from the counts and energies twinkv_score wrote ([P1] section 3.2, Eq. 3;
 * [P2] section 3.2 and the ablations of sections 5.3 and 5.5).  With
 * c = count[g][perm[g][i]] (or count[g][i] when perm is NULL) and
 * disc = ln((N+1)/(c+1)):
 *   TWINKV_VARIANT_TWIN:   score = energy * disc,    tie = energy
 *   TWINKV_VARIANT_VALUE:  score = energy,           tie = energy   (frequency removed)
 *   TWINKV_VARIANT_RARITY: score = disc / ln(N+1),   tie = 0        (value removed: equal
 *                          counts fall to the lower position; the order of [P1]'s -r/n)
 * twinkv_select ranks by (score desc, tie desc, position asc), so passing
 * score and tie as its score and energy arguments selects by the variant.
 * The twin variant without perm reproduces twinkv_score's scores bit for bit;
 * with perm it is [P2]'s permuted-frequency control (perm[g] a permutation of
 * the head's unprotected positions, identity elsewhere; entries are clamped
 * to [0, N)).  [P1]'s standalone score is the rarity variant with the
 * capacity twinkv_uniform_capacity_ceil().
 *   count: int32 [G][N] (>= 0); energy: double [G][N]; perm: int32 [G][N] or NULL
 *   score, tie: double [G][N] (out; distinct from each other and from energy)
 * Of the parameters only G and N are read.  Phases for `marks`: 0 = variant.
 */
int twinkv_variant_score(const twinkv_params* params, int variant, const int32_t* count, const double* energy,
                         const int32_t* perm, double* score, double* tie, hipStream_t stream, hipEvent_t* marks);

/*
 * twinkv_count_stats - statistics of every head over its unprotected
 * positions (the protection of twinkv_select, clipped against capacity[g])
 * ([P1] Figure 1(b); [P2] sections 2.1 and 5.5, appendix B.2).  Per head g,
 * stats[g][k] (int64):
 *   0  n        unprotected positions
 *   1  twin     of them with count >= 1
 *   2-7         six-bin count histogram: {0}, {1}, {2}, {3,4}, {5..8}, {9+}
 *   8  kept     unprotected positions kept by keep_twin
 *   9  added    kept by keep_twin, not by keep_value
 *   10 removed  kept by keep_value, not by keep_twin
 *   11-15       |e/e_cut - 1| of the added positions in five bins with edges
 *               0.05, 0.10, 0.25, 0.50 (bin k: edges <= value, counted)
 *   16-20       the same for the removed positions
 *   21-25       the same for all unprotected positions
 * and fstats[g][0] = sum of ln((N+1)/(c+1))/ln(N+1) over the unprotected
 * positions, fstats[g][1] = e_cut, the lowest energy among the unprotected
 * positions keep_value keeps (0 if none; margins are then all 0).
 * [P2] measures selection change as added / kept and the discount mean as
 * fstats[0] / n.  The page's bin edges are not printed; these are readings.
 *   count: int32 [G][N] (>= 0); energy: double [G][N]; capacity: int32 [G]
 *   keep_twin, keep_value: uint8 [G][N] (both NULL: entries 8-25 are 0)
 *   stats: int64 [G][TWINKV_STAT_INTS]; fstats: double [G][2]
 * Of the parameters G, N, sink and recent are read.  Phases: 0 = statistics.
 */
int twinkv_count_stats(const twinkv_params* params, const int32_t* count, const double* energy,
                       const uint8_t* keep_twin, const uint8_t* keep_value, const int32_t* capacity, int64_t* stats,
                       double* fstats, hipStream_t stream, hipEvent_t* marks);

/*
 * twinkv_gather_kv - physical cache layout of a selection ([P2] section 3.4):
 * the retained keys (and values) of every head, in sequence order, packed
 * head after head with no padding.  Head g's retained positions are
 * kept_idx[kept_off[g] .. kept_off[g+1]) (ascending, as twinkv_select writes
 * them); row kept_off[g] + r of out_keys / out_values is row kept_idx[kept_off[g]
 * + r] of head g, copied bit for bit (keys are not re-rotated, values are
 * unchanged).  Heads with equal quotas therefore form contiguous slices of
 * one tensor and the payload is exactly 2 * d * total elements.
 *   keys, values:  bf16 [G][N][d] (values may be NULL: keys only)
 *   kept_idx:      int32 [total]
 *   kept_off:      int64 [G+1] device array, kept_off[0] = 0 and
 *                  kept_off[g+1] - kept_off[g] = that head's count (0..N),
 *                  kept_off[G] = total
 *   out_keys, out_values: bf16 [total][d] (out_values NULL iff values NULL;
 *                  both may be NULL when total is 0)
 * Of the parameters only G, N and d are read.  The kernel clamps every
 * offset and index to [0, total] / [0, N), so inconsistent offsets produce
 * wrong rows, never an access outside the stated sizes.
 * Phases for `marks`: 0 = gather.
 */
int twinkv_gather_kv(const twinkv_params* params, const void* keys, const void* values, const int32_t* kept_idx,
                     const int64_t* kept_off, int64_t total, void* out_keys, void* out_values, hipStream_t stream,
                     hipEvent_t* marks);

/*
 * twinkv_allocate - per-head capacities from prefix attention ([P2] section
 * 3.3, Equation 5; appendices A.2, A.3).  The G = L*H heads form L layers of
 * H consecutive KV heads that share the per-head budget B (0 <= B <= N).
 * For KV head g, its Gq query heads observe the prefix from the last W
 * positions t = N-W .. N-1 (queries[g][q][w] is query head q at position
 * N-W+w, post-RoPE):
 *   a[q,w,i] = exp(q.k_i/sqrt(d)) / sum_{j<=t} exp(q.k_j/sqrt(d))  for i <= t, else 0
 *   z[g][i]  = fp32( max over |i'-i| <= pool/2 of  (1/Gq) sum_q sum_w a[q,w,i'] )
 * (logits and sums evaluated in fp64, bf16 products exact; the window is cut
 * at the ends of the prefix).  With s = min(sink, B), r = min(recent, B-s),
 * P = s + r and U = B - P, g_h counts head h's positions among the H*U
 * largest unprotected z of its layer (ties to the lower head, then the lower
 * position; a layer whose unprotected z are all zero gives g_h = U), and
 *   capacity[h] = P + floor((g_h + U)/2) + delta_h,
 * where the first R = H*U - sum floor((g_h+U)/2) heads of the layer with an
 * odd g_h + U get delta_h = 1.  So every layer's capacities sum to H*B and
 * each is at least P + floor(U/2).  U = 0 skips the allocation: capacity = B.
 *   keys:     bf16 [G][N][d];  queries: bf16 [G][Gq][W][d]
 *   capacity: int32 [G] (out);  g_count: int32 [G] (out, may be NULL; 0 when skipped)
 *   z:        float [G][N] (out, may be NULL)
 * Requirements (else TWINKV_ERR_ARG): 1 <= H <= 1024 dividing G, Gq >= 1,
 * 1 <= W <= N, Gq*W <= 128, pool odd, H*N <= 2^30.  Of the parameters G, N,
 * d, sink and recent are read.  Workspace: twinkv_allocate_workspace_bytes().
 * Phases for `marks`: 0 = per-query softmax statistics, 1 = attention
 * aggregation and pooling, 2 = layer-wide ranking and Equation 5.
 */
size_t twinkv_allocate_workspace_bytes(const twinkv_params* params, int32_t H, int32_t Gq, int32_t W, int32_t pool,
                                       int64_t B);
int twinkv_allocate(const twinkv_params* params, int32_t H, int32_t Gq, int32_t W, int32_t pool, int64_t B,
                    const void* keys, const void* queries, int32_t* capacity, int32_t* g_count, float* z,
                    void* workspace, size_t workspace_bytes, hipStream_t stream, hipEvent_t* marks);

#ifdef __cplusplus
}
#endif

#endif /* TWINKV_H */
