// Device helpers for the gfx950 verify sampler: Philox4x32-10, logit loads,
// wave64 cross-lane reductions and the workspace layout shared by the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dspark {

constexpr int kGroup = 256;        // vocab ids per race group (and per pass workgroup)
constexpr int kWaveCols = 64;      // vocab ids per wave inside a group
constexpr int kWaves = 4;          // waves per pass workgroup
constexpr int kThreads = kWaves * 64;
constexpr int kMaxK = 32;
constexpr int kChunk = 16;         // rows per MFMA chunk

// Counters in the workspace's `nitems` region: [0] residual rows and [1] bonus rows of
// the pass-2 list, then pass 1's target-item counters, kQueueStride ints (a 128-byte
// line) apart from each other (workgroup g draws from counter g % min(kQueues, grid),
// items of its own residue class).  All are cleared by the pack launch.
constexpr int kQueues = 8;
constexpr int kQueueStride = 32;
constexpr int kCounterInts = kQueueStride * (1 + kQueues);

constexpr double kLog2e = 1.4426950408889634074;
constexpr double kLn2 = 0.69314718055994530942;

enum Purpose : uint32_t { kPurposeDraft = 0, kPurposeAccept = 1, kPurposeSample = 3 };
// The drafter walk's race clocks for slot j: purpose 16 + j.
__host__ __device__ constexpr uint32_t walk_purpose(int j) { return 16u + (uint32_t)j; }
enum Dtype : int { kF32 = 0, kBF16 = 1 };

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of
// (c0,c1,c2,c3) -> (hi(M1 c2)^c1^k0, lo(M1 c2), hi(M0 c0)^c3^k1, lo(M0 c0)),
// the key advancing by the Weyl constants between rounds.  Only word 0 is used.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t philox_word0(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                                 uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    // one 32 x 32 -> 64-bit product per multiplier (v_mad_u64_u32 gives both halves)
    const uint64_t p0 = (uint64_t)c0 * 0xD2511F53u, p1 = (uint64_t)c2 * 0xCD9E8D57u;
    const uint32_t lo0 = (uint32_t)p0, hi0 = (uint32_t)(p0 >> 32);
    const uint32_t lo1 = (uint32_t)p1, hi1 = (uint32_t)(p1 >> 32);
    const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
    k0 += 0x9E3779B9u; k1 += 0xBB67AE85u;
  }
  return c0;
}

// All four output words of one counter.
__device__ __forceinline__ uint4 philox4(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                         uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    // one 32 x 32 -> 64-bit product per multiplier (v_mad_u64_u32 gives both halves)
    const uint64_t p0 = (uint64_t)c0 * 0xD2511F53u, p1 = (uint64_t)c2 * 0xCD9E8D57u;
    const uint32_t lo0 = (uint32_t)p0, hi0 = (uint32_t)(p0 >> 32);
    const uint32_t lo1 = (uint32_t)p1, hi1 = (uint32_t)(p1 >> 32);
    const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
    k0 += 0x9E3779B9u; k1 += 0xBB67AE85u;
  }
  return make_uint4(c0, c1, c2, c3);
}

// The sampler's clocks: one per vocabulary id, from the generator's output stream for
// (stream b, purpose, step): id v reads word v mod 4 of counter (b, v div 4, purpose,
// step), E_v = -ln U_v with U_v = ((x >> 8) + 1/2) 2^-24.
__device__ __forceinline__ uint32_t stream_word(uint32_t k0, uint32_t k1, uint32_t b, uint32_t v, uint32_t purpose,
                                                uint32_t step) {
  const uint4 w = philox4(b, v >> 2, purpose, step, k0, k1);
  const uint32_t i = v & 3u;
  return i == 0 ? w.x : (i == 1 ? w.y : (i == 2 ? w.z : w.w));
}

// log2 E in fp64 (the exact comparison of candidates).
__device__ __forceinline__ double clock_log2_f64(uint32_t x) {
  const double U = ((double)(x >> 8) + 0.5) * 0x1.0p-24;
  return log2(-log(U));
}

// E = -ln U in fp32 with one logarithm, relative error <= ~2^-16: U <= 1/2 is exact in
// fp32; for U > 1/2, d = 1 - U is exact, and -ln(1 - d) is a three-term series below
// 2^-8 (where the rounded 1 - d would lose E) and -ln of the rounded 1 - d above.
__device__ __forceinline__ float clock_f32(uint32_t x) {
  const uint32_t m = x >> 8;
  const float U = ((float)m + 0.5f) * 0x1.0p-24f;
  const float d = ((float)((1u << 24) - 1u - m) + 0.5f) * 0x1.0p-24f;
  const bool upper = m >= (1u << 23);
  const float t = upper ? 1.0f - d : U;
  const float e = -__builtin_amdgcn_logf(t) * 0.69314718055994530942f;   // v_log_f32 is log2
  const float series = d * (1.0f + d * (0.5f + d * (1.0f / 3.0f)));
  return (upper && d < 0x1.0p-8f) ? series : e;
}

// log2 E of clock word x (E = -ln U, U = ((x >> 8) + 1/2) 2^-24) in units of 2^-10,
// rounded, as an int16 value (log2 E lies in [-25, 4.2]): absolute error below 2^-10,
// far inside the margin the candidate pass leaves for the fp64 check.  For U > 1 - 2^-8
// the exact d = 1 - U gives log2 E = log2 d + d / (2 ln 2) + O(d^2); otherwise
// E = -ln U from one logarithm of U.
__device__ __forceinline__ int clock_log2_q10(uint32_t x) {
  const uint32_t m = x >> 8;
  const float U = ((float)m + 0.5f) * 0x1.0p-24f;
  const float d = ((float)((1u << 24) - 1u - m) + 0.5f) * 0x1.0p-24f;   // exact
  const bool small = d < 0x1.0p-8f;
  const float E = small ? d : -__builtin_amdgcn_logf(U) * 0.69314718055994530942f;
  const float L = __builtin_amdgcn_logf(E) + (small ? d * 0.72134752044448170368f : 0.f);
  return (int)__builtin_rintf(L * 1024.f);
}

// Accept uniform u = ((x >> 8) + 1) * 2^-24, in (0, 1], exact in fp32 and fp64.
__device__ __forceinline__ double accept_uniform(uint32_t k0, uint32_t k1, uint32_t b, uint32_t j, uint32_t step) {
  const uint32_t x = philox_word0(b, j, kPurposeAccept, step, k0, k1);
  return (double)((x >> 8) + 1u) * 0x1.0p-24;
}


// ---------------------------------------------------------------------------
// Workspace data that one launch phase writes and another reads -- in the fused
// verify launch, a workgroup possibly on another XCD -- goes through agent-coherent
// accesses (relaxed atomics at agent scope, the sc1 bit): stores write through to
// the device's coherence point and loads do not take stale L2 lines, so no cache
// write-back or invalidate is needed between phases.  Types of 4 or 8k bytes.
// ---------------------------------------------------------------------------
template <class T>
__device__ __forceinline__ T ld_c(const T* p) {
  static_assert(sizeof(T) % 4 == 0, "coherent accesses move whole 32-bit words");
  T v;
  if constexpr (sizeof(T) % 8 == 0) {
    uint64_t w[sizeof(T) / 8];
    uint64_t* q = reinterpret_cast<uint64_t*>(const_cast<T*>(p));
#pragma unroll
    for (int i = 0; i < (int)(sizeof(T) / 8); ++i)
      w[i] = __hip_atomic_load(q + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_memcpy(&v, w, sizeof(T));
  } else {
    uint32_t w[sizeof(T) / 4];
    uint32_t* q = reinterpret_cast<uint32_t*>(const_cast<T*>(p));
#pragma unroll
    for (int i = 0; i < (int)(sizeof(T) / 4); ++i)
      w[i] = __hip_atomic_load(q + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_memcpy(&v, w, sizeof(T));
  }
  return v;
}

template <class T>
__device__ __forceinline__ void st_c(T* p, const T& v) {
  static_assert(sizeof(T) % 4 == 0, "coherent accesses move whole 32-bit words");
  if constexpr (sizeof(T) % 8 == 0) {
    uint64_t w[sizeof(T) / 8];
    __builtin_memcpy(w, &v, sizeof(T));
    uint64_t* q = reinterpret_cast<uint64_t*>(p);
#pragma unroll
    for (int i = 0; i < (int)(sizeof(T) / 8); ++i) __hip_atomic_store(q + i, w[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    uint32_t w[sizeof(T) / 4];
    __builtin_memcpy(w, &v, sizeof(T));
    uint32_t* q = reinterpret_cast<uint32_t*>(p);
#pragma unroll
    for (int i = 0; i < (int)(sizeof(T) / 4); ++i) __hip_atomic_store(q + i, w[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Wait until this wave's memory operations have completed (s_waitcnt vmcnt(0)).
__device__ __forceinline__ void wait_memory() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// ---------------------------------------------------------------------------
// Loads.  bf16 -> fp32 is a 16-bit shift.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// 16 consecutive logits of one row, columns [c0, c0+16), -inf beyond V.
// `vec` says the row base is 16-byte aligned and V is a multiple of the vector width.
template <int DT>
__device__ __forceinline__ void load16(const void* __restrict__ row, int c0, int V, bool vec, float (&x)[16]) {
  if (DT == kBF16) {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(row);
    if (vec && c0 + 16 <= V) {
      const uint4 a = *reinterpret_cast<const uint4*>(p + c0);
      const uint4 b = *reinterpret_cast<const uint4*>(p + c0 + 8);
      const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) { x[2 * i] = bf16lo(w[i]); x[2 * i + 1] = bf16hi(w[i]); }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = (c0 + i < V) ? bf16_to_f32(p[c0 + i]) : -INFINITY;
    }
  } else {
    const float* p = reinterpret_cast<const float*>(row);
    if (vec && c0 + 16 <= V) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 a = *reinterpret_cast<const float4*>(p + c0 + 4 * i);
        x[4 * i] = a.x; x[4 * i + 1] = a.y; x[4 * i + 2] = a.z; x[4 * i + 3] = a.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = (c0 + i < V) ? p[c0 + i] : -INFINITY;
    }
  }
}

template <int DT>
__device__ __forceinline__ float load1(const void* __restrict__ row, int c) {
  if (DT == kBF16) return bf16_to_f32(reinterpret_cast<const uint16_t*>(row)[c]);
  return reinterpret_cast<const float*>(row)[c];
}

// ---------------------------------------------------------------------------
// Cross-lane reductions inside the 4 lanes {n, n+16, n+32, n+48} of a wave, on
// the gfx950 row swaps (VALU, no LDS round trip).  permlane16_swap(v, v) returns
// rows (0,0,2,2) and (1,1,3,3) of v, permlane32_swap(v, v) halves (lo,lo) and
// (hi,hi); combining the two results gives every lane the same value.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float max4lanes(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum4lanes(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// One row of the residual pass, prepared by the scan: the target/draft rows, the
// Markov previous token, the stream, the row maxima, the temperature constant
// (hi + lo) and the exponent constants of P p and q in log2 units (hi + lo).
struct Item {
  int32_t dr, tr, prev, b;
  float Mt, Md, chi, clo;
  float kph, kpl, kqh, kql;
};

// The two best race candidates of one listed row within one 256-id group: log2
// scores (log2 w - log2 E, fp32) and ids; larger score first, the smaller id among
// equal scores.  Empty slots hold (-inf, INT_MAX).
struct Top2 {
  float s1;
  int32_t v1;
  float s2;
  int32_t v2;
};

// The walk's race candidates: a row's best two (score, id) in a group, each with its
// biased logit y = d + bias in fp64 (d exact; bias from the fp32 MFMA started from a
// zero accumulator, absolute error of order 1e-9 for weights of the drafter's scale),
// so that the draw scores them exactly without reading them again.
struct WalkTop2 {
  float s1;
  int32_t v1;
  float s2;
  int32_t v2;
  double y1, y2;
};

// ---------------------------------------------------------------------------
// Workspace (carved on the host, 256-byte aligned regions).
// ---------------------------------------------------------------------------
struct Workspace {
  float2* tpart;      // [NG][B*(k+1)]   target row group partials (raw max, sum 2^((l-m)c))
  float2* dpart;      // [NG][B*k]       draft row group partials on biased logits
  float* wgrp;        // [NG][B*k]       residual group masses of pass-2 rows
  float* tm;          // [B*(k+1)]     target row max (raw logits)
  double* tl2s;       // [B*(k+1)]     log2 of sum 2^((l-m)c)
  float* dm;          // [B*k]         draft row max (biased logits)
  double* dl2s;       // [B*k]
  double* logP;       // [B*(k+1)]     log P_j (clipped prefix)
  double* lpx;        // [B*k]         log p_j(x_j)
  double* lqx;        // [B*k]         log q_j(x_j)
  int32_t* info;      // [B*4]         gamma, stop (token-wise t / block provisional), f, flags
  int32_t* info2;     // [B*4]         first list index of the stream's residual rows, list index of its bonus row
  uint32_t* rowmask;  // [B]           pass-2 rows of each stream (bit i = slot i)
  Item* items;        // [B*k]         pass-2 list: residual rows from the front, bonus rows from the back
  int32_t* nitems;    // [kCounterInts] list counts and work counters (see kQueues)
  uint4* btile;       // [ceil(B*k/16)][R/32][64] W1 tiles of every draft row in MFMA lane order (pass 1)
  Top2* race;         // [NG][B*k]       race candidates of the pass-2 rows (by list index); the walk:
                      //                 [NG][B] WalkTop2
  uint2* clk;         // [B][NG*64]      race clocks of sampled streams: log2 E in units of 2^-10 as
                      //                 int16, four ids to a uint2 (ids 4i .. 4i+3 of the stream);
                      //                 the resident walk: its drawing workgroups' clocks
  int32_t* sync;      // [kSyncInts]     resident launches: error word at [1], arrival counters on
                      //                 lines 1 .. kGridCountLines, go-word copies from [kGoBase];
                      //                 cleared by pack (verify) or sync_clear_kernel (walk)
};

// Clock bytes of one resident-walk workgroup's block of rows (64 rows x 256 ids, int16).
constexpr size_t kWalkClockBytes = 64 * 256 * 2;
// The resident launches' wait words: the error word at [1]; the arrival counters,
// kGridSubs per phase parity and a top counter each, one 64-byte line apiece (lines
// 1 .. kGridCountLines of kSyncStride words); then kGoCopies copies of the go word, one
// 128-byte line apart (workgroup g waits on copy g % kGoCopies, so that hundreds of
// waiting workgroups do not all poll one line).
constexpr int kSyncStride = 16;
constexpr int kGridSubs = 16;
constexpr int kGridCountLines = 2 * (kGridSubs + 1);
constexpr int kMaxFusedGrid = 2048;   // workgroups of a resident launch, at most
constexpr int kGoCopies = 16;
constexpr int kGoStride = 32;
constexpr int kGoBase = kSyncStride * (1 + kGridCountLines);
constexpr int kSyncInts = kGoBase + kGoCopies * kGoStride;

struct Args {
  int B, k, V, R, NG, dtype;
  int vec_ok;                     // 1 if V is a multiple of the 16-byte vector width
  const void* target;
  const void* draft;
  const int32_t* tokens;
  const int32_t* num_drafts;
  const float* temperature;
  const uint16_t* W1;
  const uint16_t* W2t;
  const int32_t* anchor;
  uint32_t key0, key1, step;
  int method;                     // 0 token-wise, 1 block
  int fused_grid;                 // > 0: workgroups of the fused launch (0: separate launches)
  int32_t* accepted_len;
  int32_t* out_tokens;
  double* diag;
  Workspace ws;
};

__device__ __forceinline__ int stream_gamma(const Args& a, int b) {
  if (a.num_drafts == nullptr) return a.k;
  const int g = a.num_drafts[b];
  return g < 0 ? 0 : (g > a.k ? a.k : g);
}

__device__ __forceinline__ float stream_temp(const Args& a, int b) {
  return a.temperature == nullptr ? 1.0f : a.temperature[b];
}

__device__ __forceinline__ int clamp_tok(int x, int V) { return x < 0 ? 0 : (x >= V ? V - 1 : x); }

// Previous token conditioning draft slot j of stream b (-1: no bias).
__device__ __forceinline__ int draft_prev(const Args& a, int b, int j) {
  int prev = (j == 0) ? (a.anchor ? a.anchor[b] : -1) : a.tokens[b * a.k + j - 1];
  return (prev >= 0 && prev < a.V) ? prev : -1;
}

struct BiasArgs {
  const uint16_t* W1;
  const uint16_t* W2t;
  int V, R, rows, dtype, vec_ok;
  const int32_t* prev;
  const void* logits_in;
  float* out;
};

constexpr int kMaxMs = 256;
struct AdaptArgs {
  const uint16_t* hidden;
  const uint16_t* w;
  float bias;
  int B, k, H, n_ms, vec_ok;
  int32_t* n_out;
  float* c_out;
  float* a_out;
  float ms[kMaxMs];
};

// Dynamic LDS of pass 1 (the per-stream table, 12 bytes a stream and 16 more); calls
// needing more than kMaxPassLds (B > 4096) are rejected as unsupported.
size_t verify_lds_bytes(int B);
constexpr size_t kMaxPassLds = 12 * 4096 + 16;

// launchers (kernels.hip)
hipError_t launch_verify(const Args& a, hipStream_t st, void* const* events);
hipError_t launch_walk(const Args& a, int32_t* tokens_out, double* logq_out, hipStream_t st);
// Launches a walk of this problem takes on the current device: 2 (the sync words are
// cleared, then one resident launch) or 2 k (two per slot).
int walk_launches(const Args& a);
hipError_t launch_markov_bias(const BiasArgs& ba, int NG, hipStream_t st);
hipError_t launch_adaptive(const AdaptArgs& aa, hipStream_t st);
hipError_t launch_random_words(uint64_t seed, uint32_t b, uint32_t purpose, uint32_t step, uint32_t idx0, int n,
                               int kind, uint32_t* out, hipStream_t st);
hipError_t launch_w2_transpose(const uint16_t* w2, int R, int V, uint16_t* w2t, hipStream_t st);
int verify_fused_grid(const Args& a);   // workgroups of the fused verify launch, 0: separate launches
hipError_t launch_scatter(const void* in, const int32_t* ids, int rows, int K, int V, int dtype, void* out,
                          hipStream_t st);

}  // namespace dspark
