// Batch-level draft scheduler (one workgroup) and the online verify-cost table
// (host state + HIP event pairs).  C ABI declared in include/dspark_verify.h.
//
// Scheduler [P2 "MTP Heads and Confidence Heads" §9, "Why It Is Called Prefix
// Survival Probability"; P3 "Teaching the Speculator What a Draft Costs", "The
// controller, and the table it reads from"]: the (stream, slot) candidates are
// ranked by prefix survival, the greedy prefix of that ranking that earns the
// most expected tokens per millisecond of verify is kept.
//
// Online table [P3, "What we changed"]: every bracketed verify step is timed by
// an event pair that is read back only once it has completed, filed under the
// step's token count, and the served table is rebuilt at a fixed cadence from
// the boot curve with the live medians laid over it.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <climits>
#include <deque>
#include <new>
#include <vector>

#include "../../include/dspark_verify.h"

namespace dspark {
namespace {

constexpr int kSchedThreads = 1024;
constexpr int kSchedWaves = kSchedThreads / 64;
constexpr int kSchedMax = DSPARK_MAX_SCHEDULE;

struct SchedArgs {
  const float* c;        // [B, k]
  const float* ms;       // [n_ms]
  int B, k;
  int32_t* n_out;        // [B]
  int32_t* total_out;    // [1] or null
  double* expected_out;  // [1] or null
};

constexpr int kFixBits = 40;                      // survivals in units of 2^-40 tokens
constexpr int kIdxBits = 12;                      // candidate index j * B + b < 4096
constexpr int kPer = kSchedMax / kSchedThreads;   // sorted positions per thread in the scan
static_assert(kSchedMax == (1 << kIdxBits), "candidate index must fit the key's low bits");
static_assert(kSchedMax % kSchedThreads == 0, "whole positions per thread");

// a in [0, 1] (NaN -> 0) rounded to the nearest multiple of 2^-40, as an integer.
__device__ __forceinline__ int64_t fixed_survival(double a) {
  a = a > 0.0 ? (a < 1.0 ? a : 1.0) : 0.0;
  return (int64_t)rint(a * 1099511627776.0);
}

// Bottom-up merge sort of sorted runs of length k (positions [r k, r k + k)) in
// buf0, ping-ponging with buf1; returns which buffer holds the result.  Each key
// finds its place in its merged pair directly: its index in its own run plus the
// number of keys of the partner run below it (keys are unique), counted by binary
// lifting over the partner run.  Runs have length k 2^level, so key i sits in run
// (i / k) >> level.  Thread t handles keys t + T r for r < RC, in lockstep so
// that their loads overlap; loads use indices clamped to [0, N).
template <int RC>
__device__ int merge_runs(uint64_t* buf0, uint64_t* buf1, int N, int k, int tid, int T) {
  int ik[RC];
#pragma unroll
  for (int r = 0; r < RC; ++r) ik[r] = (tid + r * T) / k;
  int src = 0;
  for (int L = k, lv = 0; L < N; L <<= 1, ++lv) {
    const uint64_t* in = src == 0 ? buf0 : buf1;
    uint64_t* out = src == 0 ? buf1 : buf0;
    const int top = 1 << (31 - __clz(L));   // largest power of two <= L
    uint64_t x[RC];
    int os[RC], len[RC], cnt[RC];
#pragma unroll
    for (int r = 0; r < RC; ++r) {
      const int i = tid + r * T;
      const int q = ik[r] >> lv;
      os[r] = (q ^ 1) * L;
      len[r] = i < N ? max(0, min(L, N - os[r])) : 0;
      x[r] = in[min(i, N - 1)];
      cnt[r] = 0;
    }
    for (int step = top; step > 0; step >>= 1) {
      uint64_t y[RC];
#pragma unroll
      for (int r = 0; r < RC; ++r) y[r] = in[min(os[r] + cnt[r] + step - 1, N - 1)];
#pragma unroll
      for (int r = 0; r < RC; ++r)   // bitwise &: both sides evaluated, no branch around the load
        cnt[r] += ((int)(cnt[r] + step - 1 < len[r]) & (int)(y[r] < x[r])) ? step : 0;
    }
#pragma unroll
    for (int r = 0; r < RC; ++r) {
      const int i = tid + r * T;
      const int q = ik[r] >> lv;
      if (i < N) out[(q >> 1) * (2 * L) + (i - q * L) + cnt[r]] = x[r];
    }
    src ^= 1;
    __syncthreads();
  }
  return src;
}

__global__ __launch_bounds__(kSchedThreads) void schedule_kernel(SchedArgs s) {
  // sort key: (2^40 - a_fixed) in the high bits, j * B + b in the low 12, so that
  // ascending keys give descending survival, then slot, then stream (keys are unique)
  __shared__ uint64_t keys[2][kSchedMax];   // merge sort, ping-pong
  __shared__ int cnt[kSchedMax];
  __shared__ int64_t wtot[kSchedWaves];
  __shared__ double rs[kSchedWaves], re[kSchedWaves];
  __shared__ int ri[kSchedWaves];
  // T = blockDim.x, a multiple of 64 with kPer T >= N (sized by the launcher)
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, T = blockDim.x, nw = T >> 6;
  const int B = s.B, k = s.k, N = B * k;

  // the costs of the batch sizes this thread scores (m = kPer tid + 1 + r), and m = 0
  float msr[kPer];
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int m = kPer * tid + 1 + r;
    msr[r] = m <= N ? s.ms[B + m] : 1.f;
  }
  const float ms0 = s.ms[B];

  // prefix survival of every stream, multiplied left to right in fp64.  A stream's
  // keys ascend with j (survival never grows along a stream, ties go to the lower
  // slot), so stream b's k positions [b k, b k + k) start out as one sorted run.
  for (int b = tid; b < B; b += T) {
    double run = 1.0;
    for (int j = 0; j < k; ++j) {
      run = run * (double)s.c[(size_t)b * k + j];
      const int i = j * B + b;
      keys[0][b * k + j] = ((uint64_t)((int64_t(1) << kFixBits) - fixed_survival(run)) << kIdxBits) | (uint64_t)i;
    }
  }
  __syncthreads();

  // bottom-up merge sort of the runs
  const int rc = (N + T - 1) / T;   // keys per thread
  int src;
  switch (rc) {
    case 1: src = merge_runs<1>(keys[0], keys[1], N, k, tid, T); break;
    case 2: src = merge_runs<2>(keys[0], keys[1], N, k, tid, T); break;
    case 3: src = merge_runs<3>(keys[0], keys[1], N, k, tid, T); break;
    default: src = merge_runs<4>(keys[0], keys[1], N, k, tid, T); break;
  }
  uint64_t kv[kPer];
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int p = kPer * tid + r;
    kv[r] = p < N ? (src == 0 ? keys[0][p] : keys[1][p]) : ~uint64_t(0);
  }

  // E(m) = B + the first m survivals, exactly, in 2^-40 units: thread sums of kPer
  // consecutive positions, a wave scan of those, and the wave totals before it
  int64_t incl[kPer];
  int64_t run = 0;
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int p = kPer * tid + r;
    run += p < N ? (int64_t(1) << kFixBits) - (int64_t)(kv[r] >> kIdxBits) : 0;
    incl[r] = run;
  }
  int64_t x = run;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) wtot[w] = x;
  __syncthreads();
  int64_t base = ((int64_t)B << kFixBits) + (x - run);
  for (int ww = 0; ww < w; ++ww) base += wtot[ww];

  // the best m in [0, N] of E(m) / verify_ms[B + m], smallest m on ties.  Thread t
  // scores m = 4t + 1 .. 4t + 4 in order (thread 0 also m = 0), so the first lane of
  // a wave, and the first wave, holding the maximum hold its smallest m.
  const double unit = 1.0 / 1099511627776.0;   // 2^-40
  double best = -1.0, bestE = 0.0;
  int mbest = INT_MAX;
  if (tid == 0) {
    best = (double)B / (double)ms0;
    bestE = (double)B;
    mbest = 0;
  }
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int m = kPer * tid + 1 + r;
    if (m <= N) {
      const double E = (double)(base + incl[r]) * unit;   // exact: below 2^53 units
      const double q = E / (double)msr[r];
      if (q > best) { best = q; bestE = E; mbest = m; }
    }
  }
  double wmax = best;
  for (int off = 32; off >= 1; off >>= 1) wmax = fmax(wmax, __shfl_xor(wmax, off));
  const uint64_t hit = __ballot(best == wmax);
  const int first = __builtin_ctzll(hit);
  if (lane == first) { rs[w] = best; re[w] = bestE; ri[w] = mbest; }
  for (int b = tid; b < B; b += T) cnt[b] = 0;
  __syncthreads();
  best = rs[0]; bestE = re[0]; mbest = ri[0];
#pragma unroll
  for (int ww = 1; ww < nw; ++ww)
    if (rs[ww] > best) { best = rs[ww]; bestE = re[ww]; mbest = ri[ww]; }
  if (mbest > N) { mbest = 0; bestE = (double)B; }   // no ratio above -1 (a caller's invalid table)

  // per-stream counts of the first mbest candidates (integer atomics: order-free)
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int p = kPer * tid + r;
    if (p < mbest) atomicAdd(&cnt[(int)(kv[r] & ((1u << kIdxBits) - 1)) % B], 1);
  }
  __syncthreads();
  for (int b = tid; b < B; b += T) s.n_out[b] = cnt[b];
  if (tid == 0) {
    if (s.total_out != nullptr) s.total_out[0] = B + mbest;
    if (s.expected_out != nullptr) s.expected_out[0] = bestE;
  }
}

}  // namespace
}  // namespace dspark

// ---------------------------------------------------------------------------
// online verify-cost table (host)
// ---------------------------------------------------------------------------
struct dspark_cost_table {
  std::vector<float> boot, table;
  int window = 32, min_samples = 3, rebuild_every = 32;
  std::vector<std::deque<float>> live;   // per token count: the last `window` times
  std::vector<int32_t> touched;          // token counts with at least one time
  int64_t filed = 0, dropped = 0;
  std::vector<int32_t> log_tokens;
  std::vector<float> log_ms;
  // event pairs, created on first use on the then-current device
  bool events_ready = false;
  hipEvent_t ev_start[DSPARK_COST_EVENTS] = {};
  hipEvent_t ev_stop[DSPARK_COST_EVENTS] = {};
  int32_t ev_tokens[DSPARK_COST_EVENTS] = {};
  int head = 0, count = 0;               // ring of pairs awaiting their read-back
  bool open = false, open_dropped = false;
  int32_t open_tokens = 0;

  void rebuild() {
    table = boot;
    std::vector<float> v;
    for (int32_t t : touched) {
      const std::deque<float>& d = live[t];
      if ((int)d.size() < min_samples) continue;
      v.assign(d.begin(), d.end());
      std::sort(v.begin(), v.end());
      const size_t h = v.size() / 2;
      const double med = (v.size() & 1) ? (double)v[h] : ((double)v[h - 1] + (double)v[h]) / 2.0;
      table[t] = (float)med;
    }
  }

  void file(int32_t t, float ms) {
    if (t < 0 || t >= (int32_t)boot.size()) { ++dropped; return; }
    std::deque<float>& d = live[t];
    if (d.empty()) touched.push_back(t);
    d.push_back(ms);
    while ((int)d.size() > window) d.pop_front();
    if (log_tokens.size() < (size_t)DSPARK_COST_LOG_MAX) {
      log_tokens.push_back(t);
      log_ms.push_back(ms);
    }
    ++filed;
    if (filed % rebuild_every == 0) rebuild();
  }

  // Reads back every completed pair at the front of the ring; never waits.
  hipError_t poll(int32_t* n_filed) {
    int32_t n = 0;
    while (count > 0) {
      const hipError_t q = hipEventQuery(ev_stop[head]);
      if (q == hipErrorNotReady) break;
      if (q != hipSuccess) return q;
      float ms = 0.f;
      const hipError_t e = hipEventElapsedTime(&ms, ev_start[head], ev_stop[head]);
      if (e != hipSuccess) return e;
      file(ev_tokens[head], ms);
      ++n;
      head = (head + 1) % DSPARK_COST_EVENTS;
      --count;
    }
    if (n_filed != nullptr) *n_filed = n;
    return hipSuccess;
  }

  hipError_t make_events() {
    for (int i = 0; i < DSPARK_COST_EVENTS; ++i) {
      hipError_t e = hipEventCreate(&ev_start[i]);
      if (e == hipSuccess) e = hipEventCreate(&ev_stop[i]);
      if (e != hipSuccess) return e;
    }
    events_ready = true;
    return hipSuccess;
  }

  ~dspark_cost_table() {
    for (int i = 0; i < DSPARK_COST_EVENTS; ++i) {
      if (ev_start[i] != nullptr) (void)hipEventDestroy(ev_start[i]);
      if (ev_stop[i] != nullptr) (void)hipEventDestroy(ev_stop[i]);
    }
  }
};

extern "C" {

dspark_status dspark_schedule_batch(const float* c, int32_t B, int32_t k, const float* verify_ms, int32_t n_ms,
                                    int32_t* n_out, int32_t* total_out, double* expected_out, void* stream) {
  if (c == nullptr || verify_ms == nullptr || n_out == nullptr || B <= 0 || k <= 0) return DSPARK_ERR_INVALID_ARG;
  if ((int64_t)B * k > DSPARK_MAX_SCHEDULE) return DSPARK_ERR_UNSUPPORTED;
  if ((int64_t)n_ms < (int64_t)B * (k + 1) + 1) return DSPARK_ERR_INVALID_ARG;
  dspark::SchedArgs s{c, verify_ms, B, k, n_out, total_out, expected_out};
  // keys per thread rc <= 4, threads a multiple of 64 with rc threads >= B k
  const int N = B * k, rc = (N + dspark::kSchedThreads - 1) / dspark::kSchedThreads;
  const int threads = ((N + rc - 1) / rc + 63) / 64 * 64;
  hipLaunchKernelGGL(dspark::schedule_kernel, dim3(1), dim3(threads), 0, reinterpret_cast<hipStream_t>(stream), s);
  return hipGetLastError() == hipSuccess ? DSPARK_OK : DSPARK_ERR_HIP;
}

dspark_status dspark_cost_table_create(const float* boot_ms, int32_t n, int32_t window, int32_t min_samples,
                                       int32_t rebuild_every, dspark_cost_table** out) {
  if (out == nullptr) return DSPARK_ERR_INVALID_ARG;
  *out = nullptr;
  if (boot_ms == nullptr || n <= 0 || window <= 0 || min_samples <= 0 || min_samples > window || rebuild_every <= 0)
    return DSPARK_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n; ++i)
    if (!(boot_ms[i] > 0.f) || boot_ms[i] == INFINITY) return DSPARK_ERR_INVALID_ARG;
  try {
    dspark_cost_table* t = new dspark_cost_table();
    t->boot.assign(boot_ms, boot_ms + n);
    t->table = t->boot;
    t->live.resize(n);
    t->window = window;
    t->min_samples = min_samples;
    t->rebuild_every = rebuild_every;
    *out = t;
  } catch (const std::bad_alloc&) {
    return DSPARK_ERR_NO_MEMORY;
  }
  return DSPARK_OK;
}

void dspark_cost_table_destroy(dspark_cost_table* t) { delete t; }

dspark_status dspark_cost_table_begin(dspark_cost_table* t, int32_t num_tokens, void* stream) {
  if (t == nullptr || t->open) return DSPARK_ERR_INVALID_ARG;
  if (!t->events_ready && t->make_events() != hipSuccess) return DSPARK_ERR_HIP;
  try {
    if (t->poll(nullptr) != hipSuccess) return DSPARK_ERR_HIP;
  } catch (const std::bad_alloc&) {
    return DSPARK_ERR_NO_MEMORY;
  }
  t->open = true;
  t->open_tokens = num_tokens;
  t->open_dropped = t->count == DSPARK_COST_EVENTS;   // every pair still in flight: skip this step
  if (t->open_dropped) {
    ++t->dropped;
    return DSPARK_OK;
  }
  const int slot = (t->head + t->count) % DSPARK_COST_EVENTS;
  return hipEventRecord(t->ev_start[slot], reinterpret_cast<hipStream_t>(stream)) == hipSuccess ? DSPARK_OK
                                                                                                  : DSPARK_ERR_HIP;
}

dspark_status dspark_cost_table_end(dspark_cost_table* t, void* stream) {
  if (t == nullptr || !t->open) return DSPARK_ERR_INVALID_ARG;
  t->open = false;
  if (t->open_dropped) return DSPARK_OK;
  const int slot = (t->head + t->count) % DSPARK_COST_EVENTS;
  if (hipEventRecord(t->ev_stop[slot], reinterpret_cast<hipStream_t>(stream)) != hipSuccess) return DSPARK_ERR_HIP;
  t->ev_tokens[slot] = t->open_tokens;
  ++t->count;
  return DSPARK_OK;
}

dspark_status dspark_cost_table_poll(dspark_cost_table* t, int32_t* filed) {
  if (filed != nullptr) *filed = 0;
  if (t == nullptr) return DSPARK_ERR_INVALID_ARG;
  if (!t->events_ready) return DSPARK_OK;
  try {
    return t->poll(filed) == hipSuccess ? DSPARK_OK : DSPARK_ERR_HIP;
  } catch (const std::bad_alloc&) {
    return DSPARK_ERR_NO_MEMORY;
  }
}

dspark_status dspark_cost_table_observe(dspark_cost_table* t, int32_t num_tokens, float ms) {
  if (t == nullptr || !(ms >= 0.f) || ms == INFINITY) return DSPARK_ERR_INVALID_ARG;
  try {
    t->file(num_tokens, ms);
  } catch (const std::bad_alloc&) {
    return DSPARK_ERR_NO_MEMORY;
  }
  return DSPARK_OK;
}

dspark_status dspark_cost_table_read(const dspark_cost_table* t, float* out, int32_t n) {
  if (t == nullptr || out == nullptr || n <= 0 || n > (int32_t)t->table.size()) return DSPARK_ERR_INVALID_ARG;
  memcpy(out, t->table.data(), (size_t)n * sizeof(float));
  return DSPARK_OK;
}

dspark_status dspark_cost_table_stats(const dspark_cost_table* t, int64_t* filed, int64_t* dropped,
                                      int32_t* in_flight) {
  if (t == nullptr) return DSPARK_ERR_INVALID_ARG;
  if (filed != nullptr) *filed = t->filed;
  if (dropped != nullptr) *dropped = t->dropped;
  if (in_flight != nullptr) *in_flight = t->count;
  return DSPARK_OK;
}

int32_t dspark_cost_table_log(const dspark_cost_table* t, int32_t* tokens, float* ms, int32_t cap) {
  if (t == nullptr || cap <= 0) return 0;
  const int32_t n = std::min<int32_t>(cap, (int32_t)t->log_tokens.size());
  if (tokens != nullptr) memcpy(tokens, t->log_tokens.data(), (size_t)n * sizeof(int32_t));
  if (ms != nullptr) memcpy(ms, t->log_ms.data(), (size_t)n * sizeof(float));
  return n;
}

}  // extern "C"
