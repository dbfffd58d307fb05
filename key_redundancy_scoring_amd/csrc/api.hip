// C ABI of the key-redundancy scoring library (declared in include/twinkv.h).
// Host-side argument checks, workspace carving and kernel launches on the
// caller's stream.  Nothing here allocates device memory.
#include <math.h>
#include <string.h>

#include <mutex>

#include "twinkv.h"
#include "internal.h"

namespace {

using namespace twinkv;

constexpr size_t kAlign = 256;

constexpr size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Sizes and protection counts, the part of the parameters every op reads.
int check_sizes(const twinkv_params* p) {
  if (!p) return TWINKV_ERR_ARG;
  if (p->G < 1 || p->N < 1 || p->N > (int64_t(1) << 30)) return TWINKV_ERR_ARG;
  if (p->G > (int64_t(1) << 31) - 1) return TWINKV_ERR_ARG;
  if (p->sink < 0 || p->recent < 0) return TWINKV_ERR_ARG;
  return TWINKV_OK;
}

// Everything the similarity sweep reads as well.
int check_params(const twinkv_params* p) {
  const int rc = check_sizes(p);
  if (rc != TWINKV_OK) return rc;
  if (p->window < 0) return TWINKV_ERR_ARG;
  if (!(p->tau > -1.0 && p->tau < 1.0)) return TWINKV_ERR_ARG;  // also rejects NaN
  if (p->d != 64 && p->d != 128) return TWINKV_ERR_UNSUPPORTED;
  return TWINKV_OK;
}

// The window the kernels see.  A window of N or more leaves no nonlocal pair,
// exactly as N itself does, and keeps the kernels' int32 band arithmetic
// (position + window, position - window with positions below 2^30) in range.
int32_t kernel_window(const twinkv_params* p) { return p->window < p->N ? p->window : (int32_t)p->N; }

struct Carve {
  char* base;
  size_t off = 0;
  template <class T>
  T* take(size_t count) {
    T* r = reinterpret_cast<T*>(base + off);
    off = align_up(off + count * sizeof(T));
    return r;
  }
};

// Candidate lists of the exact resolve: rows, columns, counts per head.
size_t cand_ws(const twinkv_params* p) {
  const size_t cap = (size_t)p->G * (size_t)rowres_cand_cap(p->N);
  return 2 * align_up(cap * sizeof(int32_t)) + align_up((size_t)p->G * sizeof(int32_t));
}

// Score workspace: squared norms, inverse norms, then the single-order
// sweep's column maxima, row-side results, column counts, packed best twins,
// overall maxima, candidate bits, the queue of rows for the exact resolve
// (positions, thresholds, counts) and its candidate list, carved in this
// order by score_launch.
size_t score_ws(const twinkv_params* p) {
  const size_t G = (size_t)p->G, N = (size_t)p->N;
  const size_t n = G * N;
  const int rows = tri_rows(p->d);
  const size_t nb = (N + rows - 1) / rows;
  const size_t words = (N + 31) / 32;
  return align_up(n * sizeof(double)) + align_up(n * sizeof(float)) +
         align_up(G * (size_t)tri_part_per_head(p->N, rows) * sizeof(int32_t)) + 3 * align_up(n * sizeof(int32_t)) +
         align_up(n * sizeof(uint64_t)) + align_up(n * sizeof(float)) + align_up(G * nb * words * sizeof(uint32_t)) +
         align_up(n * sizeof(int32_t)) + align_up(n * sizeof(float)) + align_up(G * sizeof(int32_t)) + cand_ws(p);
}

// Repair workspace: norms, compacted positions and their counts, rows to
// sweep and their counts, the swap's key/index scratch (two pairs; the first
// index array and the second key array also hold the queue of rows for the
// exact resolve before the swap runs), the compacted keys and their inverse
// norms, the queue counts and the resolve's candidate list.
size_t repair_ws(const twinkv_params* p) {
  const size_t n = (size_t)p->G * (size_t)p->N;
  return align_up(n * sizeof(double)) + align_up(n * sizeof(float)) + 2 * align_up(n * sizeof(int32_t)) +
         2 * align_up((size_t)p->G * sizeof(int32_t)) +
         2 * (align_up(n * sizeof(uint64_t)) + align_up(n * sizeof(int32_t))) +
         align_up(n * (size_t)p->d * sizeof(uint16_t)) + align_up(n * sizeof(float)) +
         align_up((size_t)p->G * sizeof(int32_t)) + cand_ws(p);
}

// 2^b - 1 for the smallest b with 2^b >= N: the position bits of a packed best.
uint64_t index_mask(int64_t N) {
  uint64_t m = 1;
  while (m < (uint64_t)N) m <<= 1;
  return m - 1;
}

struct AllocShape {
  int64_t Q, nchunk, width, s_cnt, r_cnt, P, U, L;
};

AllocShape alloc_shape(const twinkv_params* p, int32_t H, int32_t Gq, int32_t W, int64_t B) {
  AllocShape a{};
  a.Q = (int64_t)Gq * W;
  a.nchunk = (p->N + 255) / 256;
  a.s_cnt = p->sink < B ? p->sink : B;
  a.r_cnt = p->recent < B - a.s_cnt ? p->recent : B - a.s_cnt;
  a.P = a.s_cnt + a.r_cnt;
  a.U = B - a.P;
  a.width = p->N - a.P;
  a.L = p->G / H;
  return a;
}

int check_alloc(const twinkv_params* p, int32_t H, int32_t Gq, int32_t W, int32_t pool, int64_t B) {
  const int rc = check_sizes(p);
  if (rc != TWINKV_OK) return rc;
  if (p->d != 64 && p->d != 128) return TWINKV_ERR_UNSUPPORTED;
  if (H < 1 || H > kMaxHeads || p->G % H != 0) return TWINKV_ERR_ARG;
  if (Gq < 1 || W < 1 || W > p->N || (int64_t)Gq * W > kMaxQueries) return TWINKV_ERR_ARG;
  if (pool < 1 || (pool & 1) == 0) return TWINKV_ERR_ARG;
  if (B < 0 || B > p->N) return TWINKV_ERR_ARG;
  if ((int64_t)H * p->N > (int64_t(1) << 30)) return TWINKV_ERR_ARG;
  return TWINKV_OK;
}

size_t alloc_ws(const twinkv_params* p, int32_t H, int32_t Gq, int32_t W, int64_t B) {
  const AllocShape s = alloc_shape(p, H, Gq, W, B);
  const size_t G = (size_t)p->G, N = (size_t)p->N;
  return align_up(G * s.nchunk * s.Q * 2 * sizeof(double)) + align_up(G * s.Q * 2 * sizeof(double)) +
         align_up(G * N * sizeof(double)) + align_up(G * N * sizeof(float)) +
         align_up((size_t)s.L * 2048 * sizeof(uint32_t)) + align_up((size_t)s.L * sizeof(uint32_t)) +
         align_up((size_t)s.L * sizeof(int64_t)) + align_up(G * 3 * sizeof(uint32_t));
}

int record(hipEvent_t* marks, int k, hipStream_t s) {
  if (!marks) return TWINKV_OK;
  return hipEventRecord(marks[k], s) == hipSuccess ? TWINKV_OK : TWINKV_ERR_HIP;
}

#define TRY_HIP(expr)                                  \
  do {                                                 \
    if ((expr) != hipSuccess) return TWINKV_ERR_HIP;   \
  } while (0)
#define TRY(expr)                   \
  do {                              \
    int _rc = (expr);               \
    if (_rc != TWINKV_OK) return _rc; \
  } while (0)

int check_score_args(const twinkv_params* p, const void* keys, const void* values, const int32_t* count,
                     const double* best_sim, const int32_t* best_idx, const double* energy, const double* score) {
  TRY(check_params(p));
  if (!keys || !values || !count || !best_sim || !best_idx || !energy || !score) return TWINKV_ERR_ARG;
  if (!aligned16(keys) || !aligned16(values)) return TWINKV_ERR_ARG;
  return TWINKV_OK;
}

// Norms pass, then the single-order Gram sweep and its resolve kernels, over
// caller-checked arguments, with the workspace at `base` (score_ws bytes).
int score_launch(const twinkv_params* p, const void* keys, const void* values, int32_t* count, double* best_sim,
                 int32_t* best_idx, double* energy, double* score, double* omega, char* base, hipStream_t stream,
                 hipEvent_t* marks) {
  const size_t G = (size_t)p->G, N = (size_t)p->N;
  const size_t n = G * N;
  const int rows = tri_rows(p->d);
  Carve cv{base};
  double* nsq = cv.take<double>(n);
  float* rinv = cv.take<float>(n);
  TriArgs t{};
  t.part = cv.take<int32_t>(G * (size_t)tri_part_per_head(p->N, rows));
  t.rowcos = cv.take<float>(n);
  t.rcount = cv.take<int32_t>(n);
  t.ccount = cv.take<int32_t>(n);
  t.best64 = cv.take<uint64_t>(n);
  t.colmax = cv.take<float>(n);
  t.nb = (p->N + rows - 1) / rows;
  t.words = (p->N + 31) / 32;
  t.cbits = cv.take<uint32_t>(G * (size_t)t.nb * (size_t)t.words);
  t.q.row = cv.take<int32_t>(n);
  t.q.thr = cv.take<float>(n);
  t.q.count = cv.take<int32_t>(G);
  t.cand_cap = rowres_cand_cap(p->N);
  t.cand_row = cv.take<int32_t>(G * (size_t)t.cand_cap);
  t.cand_col = cv.take<int32_t>(G * (size_t)t.cand_cap);
  t.cand_count = cv.take<int32_t>(G);
  t.idx_mask = index_mask(p->N);
  TRY(record(marks, 0, stream));
  TRY_HIP(launch_norms(static_cast<const uint16_t*>(keys), static_cast<const uint16_t*>(values), (int64_t)n, p->d,
                       nsq, rinv, energy, stream));
  TRY(record(marks, 1, stream));
  t.keys = static_cast<const uint16_t*>(keys);
  t.nsq = nsq;
  t.rinv = rinv;
  t.energy = energy;
  t.G = p->G;
  t.N = p->N;
  t.d = p->d;
  t.window = kernel_window(p);
  t.tau = p->tau;
  t.count = count;
  t.best_sim = best_sim;
  t.best_idx = best_idx;
  t.score = score;
  t.omega = omega;
  TRY_HIP(launch_tri(t, stream, marks ? marks[2] : nullptr));
  TRY(record(marks, 3, stream));
  return TWINKV_OK;
}

// Scratch of twinkv_score_noalloc: TWINKV_NOALLOC_SCRATCH_BYTES carved like
// a score workspace.  Each device the library runs on holds its own copy for the
// life of the process.  In host code `scratch` names a host-side stand-in,
// never the device memory: its device address is looked up once per device
// with hipGetSymbolAddress and only that address is handed to kernels.
constexpr size_t kScratchBytes = TWINKV_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_addr[kMaxDevices];  // device address of `scratch`, per device; null until looked up

// Device address of the current device's scratch, looked up on the first
// call on that device (with it current) and kept.
int scratch_of_current_device(char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return TWINKV_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return TWINKV_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* addr = nullptr;
    if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || addr == nullptr) return TWINKV_ERR_HIP;
    g_scratch_addr[dev] = static_cast<char*>(addr);
  }
  *out = g_scratch_addr[dev];
  return TWINKV_OK;
}

}  // namespace

extern "C" {

const char* twinkv_status_string(int status) {
  switch (status) {
    case TWINKV_OK: return "ok";
    case TWINKV_ERR_ARG: return "invalid argument";
    case TWINKV_ERR_UNSUPPORTED: return "unsupported head dimension (64 or 128 only)";
    case TWINKV_ERR_WORKSPACE: return "workspace too small";
    case TWINKV_ERR_HIP: return "HIP runtime error";
    case TWINKV_ERR_TOO_LARGE: return "problem larger than the static scratch (workspace > TWINKV_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int64_t twinkv_uniform_capacity(int64_t N, double removal) {
  if (N < 0 || !(removal >= 0.0 && removal <= 1.0)) return -1;
  return (int64_t)floor((double)N * (1.0 - removal));
}

int64_t twinkv_uniform_capacity_ceil(int64_t N, double removal) {
  if (N < 0 || !(removal >= 0.0 && removal <= 1.0)) return -1;
  return (int64_t)ceil((double)N * (1.0 - removal));
}

int twinkv_variant_score(const twinkv_params* p, int variant, const int32_t* count, const double* energy,
                         const int32_t* perm, double* score, double* tie, hipStream_t stream, hipEvent_t* marks) {
  TRY(check_sizes(p));
  if (variant < TWINKV_VARIANT_TWIN || variant > TWINKV_VARIANT_RARITY) return TWINKV_ERR_ARG;
  if (!count || !energy || !score || !tie) return TWINKV_ERR_ARG;
  if (score == tie || score == energy || tie == energy) return TWINKV_ERR_ARG;
  TRY(record(marks, 0, stream));
  TRY_HIP(launch_variant(count, energy, perm, p->G, p->N, variant, score, tie, stream));
  TRY(record(marks, 1, stream));
  return TWINKV_OK;
}

int twinkv_count_stats(const twinkv_params* p, const int32_t* count, const double* energy, const uint8_t* keep_twin,
                       const uint8_t* keep_value, const int32_t* capacity, int64_t* stats, double* fstats,
                       hipStream_t stream, hipEvent_t* marks) {
  TRY(check_sizes(p));
  if (!count || !energy || !capacity || !stats || !fstats) return TWINKV_ERR_ARG;
  if ((keep_twin == nullptr) != (keep_value == nullptr)) return TWINKV_ERR_ARG;
  StatsArgs sa{};
  sa.count = count;
  sa.energy = energy;
  sa.keep_twin = keep_twin;
  sa.keep_value = keep_value;
  sa.capacity = capacity;
  sa.stats = stats;
  sa.fstats = fstats;
  sa.G = p->G;
  sa.N = p->N;
  sa.sink = p->sink;
  sa.recent = p->recent;
  TRY(record(marks, 0, stream));
  TRY_HIP(launch_stats(sa, stream));
  TRY(record(marks, 1, stream));
  return TWINKV_OK;
}

size_t twinkv_workspace_bytes(int op, const twinkv_params* p) {
  switch (op) {
    case TWINKV_OP_SCORE: return check_params(p) == TWINKV_OK ? score_ws(p) : 0;
    case TWINKV_OP_SELECT: return 0;
    case TWINKV_OP_REPAIR: return check_params(p) == TWINKV_OK ? repair_ws(p) : 0;
    default: return 0;
  }
}

int twinkv_score(const twinkv_params* p, const void* keys, const void* values, int32_t* count, double* best_sim,
                 int32_t* best_idx, double* energy, double* score, double* omega, void* workspace,
                 size_t workspace_bytes, hipStream_t stream, hipEvent_t* marks) {
  TRY(check_score_args(p, keys, values, count, best_sim, best_idx, energy, score));
  const size_t need = score_ws(p);
  if (!workspace || workspace_bytes < need) return TWINKV_ERR_WORKSPACE;
  if (((uintptr_t)workspace & (kAlign - 1)) != 0) return TWINKV_ERR_ARG;
  return score_launch(p, keys, values, count, best_sim, best_idx, energy, score, omega,
                      static_cast<char*>(workspace), stream, marks);
}

int twinkv_score_noalloc(const twinkv_params* p, const void* keys, const void* values, int32_t* count,
                         double* best_sim, int32_t* best_idx, double* energy, double* score, double* omega,
                         hipStream_t stream, hipEvent_t* marks) {
  TRY(check_score_args(p, keys, values, count, best_sim, best_idx, energy, score));
  if (score_ws(p) > kScratchBytes) return TWINKV_ERR_TOO_LARGE;
  char* base = nullptr;
  TRY(scratch_of_current_device(&base));
  // the same carving as a workspace; every entry a kernel reads is written
  // earlier in the same call (the clear kernel zeroes the counters)
  return score_launch(p, keys, values, count, best_sim, best_idx, energy, score, omega, base, stream, marks);
}

int twinkv_capacity_offsets(const int32_t* capacity, int64_t G, int64_t N, int64_t* kept_off, hipStream_t stream) {
  if (!capacity || !kept_off) return TWINKV_ERR_ARG;
  if (G < 1 || G > (int64_t(1) << 31) - 1 || N < 1 || N > (int64_t(1) << 30)) return TWINKV_ERR_ARG;
  TRY_HIP(launch_offsets(capacity, G, N, kept_off, stream));
  return TWINKV_OK;
}

int twinkv_select(const twinkv_params* p, const double* score, const double* energy, const int32_t* capacity,
                  const int64_t* kept_off, uint8_t* keep, int32_t* kept_idx, void* workspace, size_t workspace_bytes,
                  hipStream_t stream, hipEvent_t* marks) {
  (void)workspace;
  (void)workspace_bytes;
  TRY(check_sizes(p));
  if (!score || !energy || !capacity || !kept_off || !keep || !kept_idx) return TWINKV_ERR_ARG;
  SelectArgs sa{};
  sa.score = score;
  sa.energy = energy;
  sa.capacity = capacity;
  sa.kept_off = kept_off;
  sa.keep = keep;
  sa.kept_idx = kept_idx;
  sa.G = p->G;
  sa.N = p->N;
  sa.sink = p->sink;
  sa.recent = p->recent;
  TRY(record(marks, 0, stream));
  TRY_HIP(launch_select(sa, stream));
  TRY(record(marks, 1, stream));
  return TWINKV_OK;
}

int twinkv_gather_kv(const twinkv_params* p, const void* keys, const void* values, const int32_t* kept_idx,
                     const int64_t* kept_off, int64_t total, void* out_keys, void* out_values, hipStream_t stream,
                     hipEvent_t* marks) {
  TRY(check_sizes(p));
  if (p->d != 64 && p->d != 128) return TWINKV_ERR_UNSUPPORTED;
  if (!keys || !kept_off || total < 0) return TWINKV_ERR_ARG;
  if (total > p->G * p->N) return TWINKV_ERR_ARG;
  if (total > 0 && (!kept_idx || !out_keys)) return TWINKV_ERR_ARG;
  if (total > 0 && (values == nullptr) != (out_values == nullptr)) return TWINKV_ERR_ARG;
  if (!aligned16(keys) || (values && !aligned16(values)) || (out_keys && !aligned16(out_keys)) ||
      (out_values && !aligned16(out_values)))
    return TWINKV_ERR_ARG;
  TRY(record(marks, 0, stream));
  TRY_HIP(launch_gather_kv(static_cast<const uint16_t*>(keys), static_cast<const uint16_t*>(values), kept_idx,
                           kept_off, p->G, p->N, p->d, total, static_cast<uint16_t*>(out_keys),
                           static_cast<uint16_t*>(out_values), stream));
  TRY(record(marks, 1, stream));
  return TWINKV_OK;
}

size_t twinkv_allocate_workspace_bytes(const twinkv_params* p, int32_t H, int32_t Gq, int32_t W, int32_t pool,
                                       int64_t B) {
  return check_alloc(p, H, Gq, W, pool, B) == TWINKV_OK ? alloc_ws(p, H, Gq, W, B) : 0;
}

int twinkv_allocate(const twinkv_params* p, int32_t H, int32_t Gq, int32_t W, int32_t pool, int64_t B,
                    const void* keys, const void* queries, int32_t* capacity, int32_t* g_count, float* z,
                    void* workspace, size_t workspace_bytes, hipStream_t stream, hipEvent_t* marks) {
  TRY(check_alloc(p, H, Gq, W, pool, B));
  if (!keys || !queries || !capacity) return TWINKV_ERR_ARG;
  if (!aligned16(keys) || !aligned16(queries)) return TWINKV_ERR_ARG;
  const size_t need = alloc_ws(p, H, Gq, W, B);
  if (!workspace || workspace_bytes < need) return TWINKV_ERR_WORKSPACE;
  if (((uintptr_t)workspace & (kAlign - 1)) != 0) return TWINKV_ERR_ARG;
  const AllocShape sh = alloc_shape(p, H, Gq, W, B);
  const size_t G = (size_t)p->G, N = (size_t)p->N;
  Carve cv{static_cast<char*>(workspace)};
  AttnArgs aa{};
  aa.part = cv.take<double>(G * sh.nchunk * sh.Q * 2);
  aa.mz = cv.take<double>(G * sh.Q * 2);
  aa.agg = cv.take<double>(G * N);
  float* zbuf = cv.take<float>(G * N);
  AllocArgs al{};
  al.hist = cv.take<uint32_t>((size_t)sh.L * 2048);
  al.prefix = cv.take<uint32_t>((size_t)sh.L);
  al.need = cv.take<int64_t>((size_t)sh.L);
  al.counts = cv.take<uint32_t>(G * 3);
  aa.keys = static_cast<const uint16_t*>(keys);
  aa.queries = static_cast<const uint16_t*>(queries);
  aa.G = p->G;
  aa.N = p->N;
  aa.Gq = Gq;
  aa.W = W;
  aa.pool = pool;
  aa.nchunk = sh.nchunk;
  aa.inv_sqrt_d = 1.0 / sqrt((double)p->d);
  aa.inv_gq = 1.0 / (double)Gq;
  aa.z = z ? z : zbuf;
  aa.s_cnt = sh.s_cnt;
  aa.r_cnt = sh.r_cnt;

  TRY(record(marks, 0, stream));
  TRY_HIP(launch_attn(aa, p->d, 1, stream));
  TRY(record(marks, 1, stream));
  TRY_HIP(launch_attn(aa, p->d, 2, stream));
  TRY(record(marks, 2, stream));
  if (sh.U == 0) {
    // no unprotected slots: allocation is skipped and every head keeps B
    TRY_HIP(launch_fill_capacity(capacity, g_count, p->G, (int32_t)B, stream));
  } else {
    al.z = aa.z;
    al.G = p->G;
    al.N = p->N;
    al.L = sh.L;
    al.H = H;
    al.s_cnt = sh.s_cnt;
    al.width = sh.width;
    al.U = sh.U;
    al.P = sh.P;
    al.capacity = capacity;
    al.g_count = g_count;
    TRY_HIP(launch_alloc(al, stream));
  }
  TRY(record(marks, 3, stream));
  return TWINKV_OK;
}

int twinkv_repair(const twinkv_params* p, const void* keys, const uint8_t* keep_in, const double* prior_sim,
                  const int32_t* prior_idx, uint8_t* keep_out, double* best_sim, int32_t* best_idx,
                  int32_t* n_orphans, int32_t* n_donors, int32_t* n_swaps, int32_t* swap_pairs, void* workspace,
                  size_t workspace_bytes, hipStream_t stream, hipEvent_t* marks) {
  TRY(check_params(p));
  if (!keys || !keep_in || !keep_out || !best_sim || !best_idx || !n_orphans || !n_donors || !n_swaps)
    return TWINKV_ERR_ARG;
  if ((prior_sim == nullptr) != (prior_idx == nullptr)) return TWINKV_ERR_ARG;
  if (p->N >= 2 && !swap_pairs) return TWINKV_ERR_ARG;
  if (!aligned16(keys)) return TWINKV_ERR_ARG;
  if (keep_in == keep_out) return TWINKV_ERR_ARG;
  const size_t need = repair_ws(p);
  if (!workspace || workspace_bytes < need) return TWINKV_ERR_WORKSPACE;
  if (((uintptr_t)workspace & (kAlign - 1)) != 0) return TWINKV_ERR_ARG;

  Carve cv{static_cast<char*>(workspace)};
  const size_t n = (size_t)p->G * (size_t)p->N;
  double* nsq = cv.take<double>(n);
  float* rinv = cv.take<float>(n);
  int32_t* pos = cv.take<int32_t>(n);
  int32_t* ncols = cv.take<int32_t>((size_t)p->G);
  int32_t* row_pos = cv.take<int32_t>(n);
  int32_t* nrows = cv.take<int32_t>((size_t)p->G);
  uint64_t* keys_a = cv.take<uint64_t>(n);
  int32_t* idx_a = cv.take<int32_t>(n);
  uint64_t* keys_b = cv.take<uint64_t>(n);
  int32_t* idx_b = cv.take<int32_t>(n);
  uint16_t* ckeys = cv.take<uint16_t>(n * (size_t)p->d);
  float* crinv = cv.take<float>(n);
  int32_t* qcount = cv.take<int32_t>((size_t)p->G);
  const int64_t cand_cap = rowres_cand_cap(p->N);
  int32_t* cand_row = cv.take<int32_t>((size_t)p->G * (size_t)cand_cap);
  int32_t* cand_col = cv.take<int32_t>((size_t)p->G * (size_t)cand_cap);
  int32_t* cand_count = cv.take<int32_t>((size_t)p->G);
  const uint16_t* kin = static_cast<const uint16_t*>(keys);

  TRY(record(marks, 0, stream));
  TRY_HIP(launch_norms(kin, nullptr, (int64_t)n, p->d, nsq, rinv, nullptr, stream));
  TRY(record(marks, 1, stream));
  TRY_HIP(launch_compact(keep_in, p->G, p->N, pos, ncols, stream));
  TRY_HIP(launch_gather(kin, rinv, pos, ncols, p->G, p->N, p->d, ckeys, crinv, stream));
  TRY_HIP(launch_rows(keep_in, prior_sim, prior_idx, p->G, p->N, row_pos, nrows, best_sim, best_idx, qcount, stream));
  TRY(record(marks, 2, stream));
  GramArgs ga{};
  ga.keys = kin;
  ga.nsq = nsq;
  ga.col_keys = ckeys;
  ga.col_rinv = crinv;
  ga.col_pos = pos;
  ga.ncols = ncols;
  ga.row_pos = row_pos;
  ga.nrows = nrows;
  ga.G = p->G;
  ga.N = p->N;
  ga.d = p->d;
  ga.window = kernel_window(p);
  ga.q.row = idx_a;  // free until the swap
  ga.q.thr = reinterpret_cast<float*>(keys_b);
  ga.q.count = qcount;
  ga.best_sim = best_sim;
  ga.best_idx = best_idx;
  TRY_HIP(launch_gram(ga, stream));
  RowResArgs rr{};
  rr.keys = kin;
  rr.nsq = nsq;
  rr.rinv = rinv;
  rr.col_keys = ckeys;
  rr.col_rinv = crinv;
  rr.col_pos = pos;
  rr.ncols = ncols;
  rr.q = ga.q;
  rr.G = p->G;
  rr.N = p->N;
  rr.d = p->d;
  rr.window = ga.window;
  rr.best64 = keys_a;  // scratch, free until the swap
  rr.idx_mask = index_mask(p->N);
  rr.best_sim = best_sim;
  rr.best_idx = best_idx;
  rr.cand_row = cand_row;
  rr.cand_col = cand_col;
  rr.cand_count = cand_count;
  rr.cand_cap = cand_cap;
  TRY_HIP(launch_rowres(rr, stream));
  TRY(record(marks, 3, stream));
  SwapArgs sw{};
  sw.keep_in = keep_in;
  sw.best = best_sim;
  sw.ncols = ncols;
  sw.keep_out = keep_out;
  sw.n_orphans = n_orphans;
  sw.n_donors = n_donors;
  sw.n_swaps = n_swaps;
  sw.pairs = swap_pairs;
  sw.keys_a = keys_a;
  sw.idx_a = idx_a;
  sw.keys_b = keys_b;
  sw.idx_b = idx_b;
  sw.G = p->G;
  sw.N = p->N;
  sw.tau = p->tau;
  sw.sink = p->sink;
  sw.recent = p->recent;
  TRY_HIP(launch_swap(sw, stream));
  TRY(record(marks, 4, stream));
  return TWINKV_OK;
}

}  // extern "C"
