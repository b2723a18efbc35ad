// gfx950 kernels of the DSpark verify sampler and the drafter's walk.
//
// Sources (page titles): [P1] "MTP, DSpark and Block Verification, Explained";
// [P2] "MTP Heads and Confidence Heads"; [P3] "Teaching the Speculator What a Draft Costs".
//
// A verify call is a pack launch and then either one resident launch of one workgroup
// per 256-id group (all resident; its four phases below are separated by grid-wide
// waits) or the same four phases as four launches:
//   pack      the B operand of the Markov product [P2 §6; P1 §3 "The Markov fix-up"]:
//             W1[prev] of every draft row, 16 rows per tile, stored in MFMA lane
//             order so that a wave reads one k-step of a tile as one contiguous
//             1 KB load; clears the counters of the launches below.
//   pass1     one workgroup per 256-id vocabulary group g.  Draft rows (slots
//             0..gamma_b-1): each wave keeps its 64 columns of W2 as MFMA A operands,
//             streams the packed W1 tiles through the B operand (staged in LDS) and
//             adds the bias; the wave partials meet in LDS once every 16 chunks.
//             Then target rows (slots 0..gamma_b-1): a 16-lane row reduces a group's
//             256 ids to a partial (max, sum 2^((l - max) log2e / T)), in items drawn
//             from shared counters so that all workgroups finish together.
//   scan      one workgroup per stream: the logits at the draft tokens (bias in
//             fp64), row normalisers from the partials (fp64), log p_j(x_j),
//             log q_j(x_j), the token-wise stop and the clipped prefix P_i [P1 §4],
//             and the list of rows pass 2 needs.  Block verification needs R_i only
//             where u_{i-1} <= P_i (h_i <= P_i always), plus the row the sampler may
//             land on.  The workgroups without a stream compute the race clocks
//             meanwhile (int16 log2 E of every id of every sampled stream).
//   pass2     like the draft half of pass1 over the listed rows only: per group,
//             the residual mass sum max(0, P_i p_i - q_i) (Markov bias recomputed)
//             and the two best race candidates (score log2 w - log2 E).
//   finalize  one workgroup per stream: R_i, h_i, tau (top-down), then the one-level
//             exponential race: the best group candidate, every candidate within a
//             window of it scored again in fp64; the outputs.
// The walk is one resident launch for its k slots (or two launches per slot): per
// slot, group partials and race candidates of the biased draft logits, then one
// workgroup per stream draws x_j.
//
// Partials are group-major ([group or segment][row]): a stream's rows are adjacent,
// so the per-stream scan and finalize read short contiguous runs.  Full windows take
// unconditional 16-byte loads (VEC); only the last, ragged window masks columns.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "common.hpp"

namespace dspark {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}
__device__ __forceinline__ bf16x8 zero_bf16x8() { return __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0)); }

// Temperature constant c = log2(e) / T split into hi + lo floats with chi <= c
// and clo > 0, so that fma(t, chi, t * clo) stays -inf (not NaN) for t = -inf.
__device__ __forceinline__ void temp_split(float T, float& chi, float& clo) {
  const double c = kLog2e / (double)T;
  chi = (float)c;
  if ((double)chi > c) chi = nextafterf(chi, 0.0f);
  clo = (float)(c - (double)chi);
  if (!(clo > 0.0f)) clo = 1e-30f;
}

// This wave's W2 columns as MFMA A operands.  Lane (n = l&15, q = l>>4) supplies
// A row m = n of subtile s, i.e. vocabulary id cb + 16(n>>2) + 4s + (n&3), k-range
// 8q + 32kk.  With that permutation the 16x16 output puts columns cb + 16q + [0,16)
// of draft row n into lane (n, q), in order (acc[s][i] -> column cb + 16q + 4s + i).
// VEC: each 16-column window starts at min(start, V - 16) (the kernels mask the
// columns a clamped window repeats); otherwise columns past V are clamped to V - 1
// and masked after the product.
template <int KS, bool VEC = false>
__device__ __forceinline__ void load_w2_slab(const Args& a, int cb, int n, int q, bf16x8 (&A)[4][KS]) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    int vr;
    if (VEC) {
      vr = min(cb + 16 * (n >> 2), a.V - 16) + 4 * s + (n & 3);
    } else {
      vr = cb + 16 * (n >> 2) + 4 * s + (n & 3);
      vr = vr < a.V ? vr : a.V - 1;
    }
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) A[s][kk] = load_bf16x8(a.W2t + (size_t)vr * a.R + kk * 32 + 8 * q);
  }
}

// Bias of draft row n (previous token `prev`, -1 = none) at this lane's 16 columns,
// B operand straight from global memory.
template <int KS>
__device__ __forceinline__ void markov_tile(const Args& a, const bf16x8 (&A)[4][KS], int prev, int q, float (&bias)[16]) {
  bf16x8 Bop[KS];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk)
    Bop[kk] = prev >= 0 ? load_bf16x8(a.W1 + (size_t)prev * a.R + kk * 32 + 8 * q) : zero_bf16x8();
  f32x4 acc[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) acc[s] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < KS; ++kk)
#pragma unroll
    for (int s = 0; s < 4; ++s) acc[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[s][kk], Bop[kk], acc[s], 0, 0, 0);
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int i = 0; i < 4; ++i) bias[4 * s + i] = acc[s][i];
}

// ---------------------------------------------------------------------------
// Cross-lane reductions.  DPP within a 16-lane row: quad_perm [1,0,3,2],
// quad_perm [2,3,0,1], row_half_mirror, row_mirror; every lane ends with the
// row's result, and every lane computes it in the same order.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dppf<0xB1>(v));
  v = fmaxf(v, dppf<0x4E>(v));
  v = fmaxf(v, dppf<0x141>(v));
  v = fmaxf(v, dppf<0x140>(v));
  return v;
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dppf<0xB1>(v);
  v += dppf<0x4E>(v);
  v += dppf<0x141>(v);
  v += dppf<0x140>(v);
  return v;
}
// Whole-wave reductions on VALU lane moves only (every lane gets the result): DPP
// within rows of 16 (xor 1, xor 2, half-row mirror, row mirror), then the gfx950 row
// swaps (permlane16_swap, permlane32_swap) across the four rows.
__device__ __forceinline__ float wave_max_dpp(float v) { return max4lanes(row16_max(v)); }
template <int CTRL>
__device__ __forceinline__ double dppd(double v) {
  const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), CTRL, 0xF, 0xF, false);
  return __hiloint2double(hi, lo);
}
template <int CTRL>
__device__ __forceinline__ int dppi(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ double swap_sum16(double v) {
  const auto lo = __builtin_amdgcn_permlane16_swap(__double2loint(v), __double2loint(v), false, false);
  const auto hi = __builtin_amdgcn_permlane16_swap(__double2hiint(v), __double2hiint(v), false, false);
  return __hiloint2double(hi[0], lo[0]) + __hiloint2double(hi[1], lo[1]);
}
__device__ __forceinline__ double swap_sum32(double v) {
  const auto lo = __builtin_amdgcn_permlane32_swap(__double2loint(v), __double2loint(v), false, false);
  const auto hi = __builtin_amdgcn_permlane32_swap(__double2hiint(v), __double2hiint(v), false, false);
  return __hiloint2double(hi[0], lo[0]) + __hiloint2double(hi[1], lo[1]);
}
__device__ __forceinline__ double wave_sum(double v) {
  v += dppd<0xB1>(v);
  v += dppd<0x4E>(v);
  v += dppd<0x141>(v);
  v += dppd<0x140>(v);
  return swap_sum32(swap_sum16(v));
}
__device__ __forceinline__ double wave_max_f64(double v) {
  v = fmax(v, dppd<0xB1>(v));
  v = fmax(v, dppd<0x4E>(v));
  v = fmax(v, dppd<0x141>(v));
  v = fmax(v, dppd<0x140>(v));
  {
    const auto lo = __builtin_amdgcn_permlane16_swap(__double2loint(v), __double2loint(v), false, false);
    const auto hi = __builtin_amdgcn_permlane16_swap(__double2hiint(v), __double2hiint(v), false, false);
    v = fmax(__hiloint2double(hi[0], lo[0]), __hiloint2double(hi[1], lo[1]));
  }
  const auto lo = __builtin_amdgcn_permlane32_swap(__double2loint(v), __double2loint(v), false, false);
  const auto hi = __builtin_amdgcn_permlane32_swap(__double2hiint(v), __double2hiint(v), false, false);
  return fmax(__hiloint2double(hi[0], lo[0]), __hiloint2double(hi[1], lo[1]));
}
// (score, index) arg-max over the wave: larger score, then smaller index.
__device__ __forceinline__ void take_better(double& s, int& i, double os, int oi) {
  if (os > s || (os == s && oi < i)) { s = os; i = oi; }
}
template <int CTRL>
__device__ __forceinline__ void argmax_step(double& s, int& i) {
  const double os = dppd<CTRL>(s);
  const int oi = dppi<CTRL>(i);
  take_better(s, i, os, oi);
}
__device__ __forceinline__ void wave_argmax(double& s, int& i) {
  argmax_step<0xB1>(s, i);
  argmax_step<0x4E>(s, i);
  argmax_step<0x141>(s, i);
  argmax_step<0x140>(s, i);
  {
    const auto lo = __builtin_amdgcn_permlane16_swap(__double2loint(s), __double2loint(s), false, false);
    const auto hi = __builtin_amdgcn_permlane16_swap(__double2hiint(s), __double2hiint(s), false, false);
    const auto ix = __builtin_amdgcn_permlane16_swap(i, i, false, false);
    s = __hiloint2double(hi[0], lo[0]);
    i = ix[0];
    take_better(s, i, __hiloint2double(hi[1], lo[1]), ix[1]);
  }
  {
    const auto lo = __builtin_amdgcn_permlane32_swap(__double2loint(s), __double2loint(s), false, false);
    const auto hi = __builtin_amdgcn_permlane32_swap(__double2hiint(s), __double2hiint(s), false, false);
    const auto ix = __builtin_amdgcn_permlane32_swap(i, i, false, false);
    s = __hiloint2double(hi[0], lo[0]);
    i = ix[0];
    take_better(s, i, __hiloint2double(hi[1], lo[1]), ix[1]);
  }
}

// 16 logits kept packed until use: bf16 as 8 words, fp32 as 16 floats.
template <int DT> struct Raw16;
template <> struct Raw16<kBF16> { uint32_t w[8]; };
template <> struct Raw16<kF32> { float f[16]; };

// VEC: columns [c0, c0+16) are inside the row and 16-byte aligned (the caller clamps
// the window): plain vector loads.  Otherwise each element is checked against V and
// -inf fills the rest.
template <int DT, bool VEC>
__device__ __forceinline__ void raw_load(Raw16<DT>& r, const char* __restrict__ row, int c0, int V) {
  if (DT == kBF16) {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(row);
    auto& w = reinterpret_cast<Raw16<kBF16>&>(r).w;
    if (VEC) {
      const uint4 a = *reinterpret_cast<const uint4*>(p + c0);
      const uint4 b = *reinterpret_cast<const uint4*>(p + c0 + 8);
      w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w; w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t lo = (c0 + 2 * i < V) ? p[c0 + 2 * i] : 0xFF80u;      // bf16 -inf
        const uint32_t hi = (c0 + 2 * i + 1 < V) ? p[c0 + 2 * i + 1] : 0xFF80u;
        w[i] = lo | (hi << 16);
      }
    }
  } else {
    const float* p = reinterpret_cast<const float*>(row);
    auto& f = reinterpret_cast<Raw16<kF32>&>(r).f;
    if (VEC) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 a = *reinterpret_cast<const float4*>(p + c0 + 4 * i);
        f[4 * i] = a.x; f[4 * i + 1] = a.y; f[4 * i + 2] = a.z; f[4 * i + 3] = a.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) f[i] = (c0 + i < V) ? p[c0 + i] : -INFINITY;
    }
  }
}

template <int DT>
__device__ __forceinline__ void raw_to_f32(const Raw16<DT>& r, float (&x)[16]) {
  if (DT == kBF16) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t w = reinterpret_cast<const Raw16<kBF16>&>(r).w[i];
      x[2 * i] = bf16lo(w);
      x[2 * i + 1] = bf16hi(w);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = reinterpret_cast<const Raw16<kF32>&>(r).f[i];
  }
}

// Element e of a raw 16-id window as fp32.
template <int DT>
__device__ __forceinline__ float raw_elem(const Raw16<DT>& r, int e) {
  if (DT == kBF16) {
    const uint32_t w = reinterpret_cast<const Raw16<kBF16>&>(r).w[e >> 1];
    return (e & 1) ? bf16hi(w) : bf16lo(w);
  }
  return reinterpret_cast<const Raw16<kF32>&>(r).f[e];
}

// Columns a clamped window repeats (the first `shift` of 16) do not count.
__device__ __forceinline__ void mask_shift(float (&x)[16], int shift) {
#pragma unroll
  for (int i = 0; i < 16; ++i) x[i] = i < shift ? -INFINITY : x[i];
}

// Partial (max, sum 2^((x - max) c)) of 16 values; RED selects the lanes that share
// the row: 0 = the 4 lanes {n, n+16, n+32, n+48} (MFMA layout), 1 = a 16-lane DPP row.
// With m c = mh + ml exactly (mh = fl(m c), ml = fma(m, c, -mh)), each term is
// 2^(fma(x, c, -mh)) and the common factor 2^-ml is applied once: three operations
// per value.  c is log2(e)/T rounded to fp32; its rounding moves a term by a relative
// (x - m) c 2^-24, so the terms that carry the sum are exact to fp32 rounding.
template <int RED>
__device__ __forceinline__ float2 row_partial(const float (&x)[16], float c) {
  float m = x[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) m = fmaxf(m, x[i]);
  m = RED == 0 ? max4lanes(m) : row16_max(m);
  float s = 0.f;
  if (m != -INFINITY) {
    const float mh = m * c;
    const float ml = fmaf(m, c, -mh);
#pragma unroll
    for (int i = 0; i < 16; ++i) s += __builtin_amdgcn_exp2f(fmaf(x[i], c, -mh));
    s *= __builtin_amdgcn_exp2f(-ml);
  }
  s = RED == 0 ? sum4lanes(s) : row16_sum(s);
  return make_float2(m, s);
}

// floor(i / d) for 0 <= i < 2^22 and 1 <= d <= 64, from hd = 0.5f / d: (2i + 1) / (2d)
// lies at least 1/(2d) from an integer and the two fp32 roundings move it by less.
__device__ __forceinline__ int div_small(int i, float hd) { return (int)((float)(2 * i + 1) * hd); }

// ---------------------------------------------------------------------------
// pack: one wave per 16 draft rows (lane n + 16 q: row n, quarter q of each k-step).
// The W1 rows of the rows' previous tokens go into `btile` in MFMA lane order, so
// that pass 1 reads a k-step of 16 rows as one contiguous 1 KB load; gathered here,
// before pass 1 floods memory with logits, the scattered W1 rows arrive fast.  Rows
// with no previous token get a zero tile.  Also clears the pass-2 list counts and
// pass 1's item counters.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void pack_kernel(Args a) {
  const int c = blockIdx.x, l = threadIdx.x, n = l & 15, q = l >> 4;
  if (c == 0 && l < 2) st_c(&a.ws.nitems[l], 0);
  if (c == 0 && l < kQueues) st_c(&a.ws.nitems[kQueueStride * (1 + l)], 0);
  if (a.fused_grid > 0 && c == 0) {   // the fused launch's go and error words and counters
    if (l < 4) st_c(&a.ws.sync[l], 0);
    if (l < kGoCopies) st_c(&a.ws.sync[kGoBase + kGoStride * l], 0);
    for (int i = l; i <= kGridCountLines; i += 64) st_c(&a.ws.sync[kSyncStride * i], 0);
  }
  if (a.W1 == nullptr) return;
  const int ND = a.B * a.k;
  const int drc = min(c * kChunk + n, ND - 1);
  const int b = drc / a.k, j = drc - b * a.k;
  const int pv = draft_prev(a, b, j);
  const int ks = a.R / 32;   // <= 8
  uint4 v[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {   // unconditional loads (clamped row), masked after
    const int kc = kk < ks ? kk : 0;
    v[kk] = *reinterpret_cast<const uint4*>(a.W1 + (size_t)max(pv, 0) * a.R + kc * 32 + 8 * q);
  }
  uint4* dst = a.ws.btile + (size_t)c * ks * 64 + l;
#pragma unroll
  for (int kk = 0; kk < 8; ++kk)
    if (kk < ks) dst[kk * 64] = pv >= 0 ? v[kk] : make_uint4(0, 0, 0, 0);
}

// x + bias at the lane's row and 16 columns: A = this wave's W2 slab, B = a packed
// tile; the accumulator starts from x (the logits), so the add is free.
template <int KS>
__device__ __forceinline__ void markov_mma(const bf16x8 (&A)[4][KS], const bf16x8 (&B)[KS], float (&x)[16]) {
  f32x4 acc[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) acc[s] = f32x4{x[4 * s], x[4 * s + 1], x[4 * s + 2], x[4 * s + 3]};
#pragma unroll
  for (int kk = 0; kk < KS; ++kk)
#pragma unroll
    for (int s = 0; s < 4; ++s) acc[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[s][kk], B[kk], acc[s], 0, 0, 0);
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int i = 0; i < 4; ++i) x[4 * s + i] = acc[s][i];
}

// Per-stream constants of a pass in LDS: c = log2(e)/T (fp32) and gamma_b.
__host__ __device__ __forceinline__ size_t align16(size_t x) { return (x + 15) & ~(size_t)15; }

__host__ __device__ __forceinline__ size_t stream_table_bytes(int B) {
  return 2 * align16((size_t)B * sizeof(float)) + align16((size_t)B * sizeof(int)) + 16;
}

// Stand-in temperature constant of a greedy stream (T = 0) in the stream table; no
// sampled stream comes near it (log2(e) / T < 1e-20 would need T > 1e20).
constexpr float kGreedyTcValue = 1e-30f;
constexpr float kGreedyTc = 1e-20f;

// tc[b] = log2(e) / T_b (fp32; a stand-in for a greedy stream), gam[b] = gamma_b, a
// flag word (any greedy stream), and T[b] itself (the fused launch's scan and
// finalize read T_b and gamma_b from here instead of from global memory).
struct StreamTable {
  const float* tc;
  const int* gam;
  bool any_greedy;
  const float* T;
};
__device__ __forceinline__ const float* stream_table_T(const Args& a, const char* smem) {
  return reinterpret_cast<const float*>(smem + align16((size_t)a.B * sizeof(float)) +
                                        align16((size_t)a.B * sizeof(int)) + 16);
}
__device__ __forceinline__ const int* stream_table_gam(const Args& a, const char* smem) {
  return reinterpret_cast<const int*>(smem + align16((size_t)a.B * sizeof(float)));
}

// T0, gam0: stream threadIdx.x's temperature and draft count when the caller has
// loaded them already (pass 1 issues those loads ahead of its W2 slab); NaN = not loaded.
__device__ __forceinline__ StreamTable build_stream_table(const Args& a, char* smem, float T0 = NAN, int gam0 = 0) {
  float* tc = reinterpret_cast<float*>(smem);
  int* gam = reinterpret_cast<int*>(smem + align16((size_t)a.B * sizeof(float)));
  int* flag = reinterpret_cast<int*>(smem + align16((size_t)a.B * sizeof(float)) + align16((size_t)a.B * sizeof(int)));
  if (threadIdx.x == 0) flag[0] = 0;
  __syncthreads();
  float* tt = const_cast<float*>(stream_table_T(a, smem));
  auto put = [&](int b, float T, int gm) {
    // T = 0 (greedy) only needs the row maxima: any finite positive c keeps the sums finite
    tc[b] = T > 0.f ? (float)(kLog2e / (double)T) : kGreedyTcValue;
    gam[b] = gm;
    tt[b] = T;
    if (!(T > 0.f)) flag[0] = 1;
  };
  const bool pre = !isnan(T0);
  if (pre && (int)threadIdx.x < a.B) put(threadIdx.x, T0, gam0);
  for (int b = threadIdx.x + (pre ? kThreads : 0); b < a.B; b += kThreads) put(b, stream_temp(a, b), stream_gamma(a, b));
  __syncthreads();
  return StreamTable{tc, gam, flag[0] != 0, tt};
}

// ---------------------------------------------------------------------------
// pass1: row statistics.  Workgroup g owns vocabulary ids [256g, 256g + 256).
// ---------------------------------------------------------------------------
// Draft rows, 16 per chunk: the logits of the next PD chunks and the next W1 tile
// are in flight while the current chunk goes through the MFMA and the reduction.
// The 4 wave partials of a row (64 ids each) meet in LDS; every 16 chunks one
// barrier pair turns them into group partials.
constexpr int kFlush = 16;   // chunks per LDS flush (256 rows, one per thread)

__device__ __forceinline__ float2 combine_waves(const float2 (&p)[kWaves], float c) {
  float M = p[0].x;
#pragma unroll
  for (int w = 1; w < kWaves; ++w) M = fmaxf(M, p[w].x);
  float S = 0.f;
  if (M != -INFINITY) {
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
      if (p[w].x != -INFINITY) S += p[w].y * __builtin_amdgcn_exp2f((p[w].x - M) * c);
  }
  return make_float2(M, S);
}

// W1 tiles reach the B operand through LDS: the workgroup copies a block of tiles at
// a time from `btile` (thread t moves 16-byte units t, t + 256, ...), two blocks in
// LDS, the next block's loads in flight while the current one is used.  A wave then
// reads a k-step of a tile with one conflict-free ds_read_b128 per lane.  Blocks of
// two tiles (at least one unit per thread: four at R = 32): the staged loads hold 16
// VGPRs at R = 256 rather than 32, which measured ~1.5 us less per call than blocks
// of four despite twice the barriers.
template <int KS>
constexpr int kStageOf = KS >= 2 ? 2 : 4;   // tiles (chunks) per staged block

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));   // a native vector: stays in registers

template <int KS>
struct TileStage {
  static constexpr int kStage = kStageOf<KS>;
  static constexpr int kUnits = kStage * KS * 64;   // 16-byte units per block
  static constexpr int kPer = kUnits / kThreads;    // units per thread (= KS)
  u32x4 v[kPer];
};

template <int KS>
__device__ __forceinline__ void tile_stage_load(const Args& a, int blk, int nch, TileStage<KS>& t) {
  const u32x4* src = reinterpret_cast<const u32x4*>(a.ws.btile);
#pragma unroll
  for (int i = 0; i < TileStage<KS>::kPer; ++i) {
    const int u = threadIdx.x + kThreads * i;
    const int tile = min(blk * TileStage<KS>::kStage + u / (KS * 64), nch - 1);
    t.v[i] = src[(size_t)tile * KS * 64 + u % (KS * 64)];
  }
}

template <int KS>
__device__ __forceinline__ void tile_stage_store(const TileStage<KS>& t, uint4* dst) {
  u32x4* d = reinterpret_cast<u32x4*>(dst);
#pragma unroll
  for (int i = 0; i < TileStage<KS>::kPer; ++i) d[threadIdx.x + kThreads * i] = t.v[i];
}

// Draft rows, 16 per chunk, in blocks of kStage chunks: the logits of the next PD
// chunks are in flight while the current chunk goes through the MFMA (B operand from
// LDS) and the reduction.  The 4 wave partials of a row (64 ids each) meet in LDS and
// every 16 chunks one barrier pair turns them into group partials.  Chunks past the
// batch (at most kStage - 1) run with clamped loads and write nothing.
template <int DT, int KS, bool MARKOV, bool VEC>
__device__ __forceinline__ void pass1_draft(const Args& a, const StreamTable& st, int g,
                                            float2 (*part)[kWaves], uint4* bst, const bf16x8 (&A)[4][KS],
                                            TileStage<KS>& stage) {
  constexpr int PD = 2;   // logits prefetch distance (chunks)
  constexpr int kStage = TileStage<KS>::kStage;
  static_assert(kStage % PD == 0 && kFlush % kStage == 0, "block, ring and flush sizes must nest");
  static_assert(TileStage<KS>::kUnits % kThreads == 0, "a staged block must split evenly");
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, n = l & 15, q = l >> 4;
  const int cb = g * kGroup + w * kWaveCols;
  const int cw = cb + 16 * q;                                // this lane's 16-column window
  const int c0 = VEC ? min(cw, a.V - 16) : cw;               // where it is loaded from
  const int shift = VEC ? (cw >= a.V ? 16 : cw - c0) : 0;    // columns of the window owned elsewhere
  const bool rag = VEC && cb + kWaveCols > a.V;              // wave-uniform
  const int ND = a.B * a.k;
  const int nch = (ND + kChunk - 1) / kChunk;
  const int nblk = (nch + kStage - 1) / kStage;
  const size_t rb = (size_t)a.V * (DT == kBF16 ? 2 : 4);
  const char* base = reinterpret_cast<const char*>(a.draft);
  const float hk = 0.5f / (float)a.k;
  auto row_of_dr = [&](int dr, int& b) {   // false if draft row dr is past the batch or inactive
    b = div_small(dr, hk);
    return dr < ND && dr - b * a.k < st.gam[b < a.B ? b : a.B - 1];
  };
  auto row_of = [&](int c, int& b) { return row_of_dr(c * kChunk + n, b); };
  // Loads are unconditional (no branch around them, so the wait counters stay exact):
  // an inactive row reads its stream's first draft row, a chunk past the end the last row.
  auto load_x = [&](int c, Raw16<DT>& x) {
    int b;
    const int dr = min(c * kChunk + n, ND - 1);
    const int src = row_of_dr(dr, b) ? dr : b * a.k;
    raw_load<DT, VEC>(x, base + (size_t)src * rb, c0, a.V);
  };

  auto chunk = [&](int c, const uint4* tiles, Raw16<DT>& xb) {
    float x[16];
    raw_to_f32<DT>(xb, x);
    load_x(c + PD, xb);
    if (MARKOV) {
      bf16x8 Bop[KS];
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) Bop[kk] = __builtin_bit_cast(bf16x8, tiles[kk * 64 + l]);
      markov_mma<KS>(A, Bop, x);   // x += bias
    }
    int b;
    const bool act = row_of(c, b);
    if (rag) mask_shift(x, shift);
    const float2 pw = row_partial<0>(x, act ? st.tc[b] : 0.f);
    if (q == 0) part[(c % kFlush) * kChunk + n][w] = pw;
    if (c % kFlush == kFlush - 1 || c == nch - 1) {   // uniform: every wave runs the same chunks
      __syncthreads();
      const int dr = (c - c % kFlush) * kChunk + tid;
      int bb;
      if (tid < (c % kFlush + 1) * kChunk && row_of_dr(dr, bb)) {
        float2 p[kWaves];
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) p[ww] = part[tid][ww];
        st_c(&a.ws.dpart[(size_t)g * ND + dr], combine_waves(p, st.tc[bb]));
      }
      __syncthreads();
    }
  };
  // the first chunks' logits go out before the wait for the W2 slab and tile block 0
  // (issued by the kernel before the stream table), so they arrive meanwhile
  Raw16<DT> xb[PD];   // ring of logits buffers, indexed at compile time
#pragma unroll
  for (int i = 0; i < PD; ++i) load_x(i, xb[i]);
  if (MARKOV) {
    tile_stage_store<KS>(stage, bst);
    tile_stage_load<KS>(a, 1, nch, stage);
  }
  __syncthreads();   // block 0 of the tiles is in LDS
  for (int j = 0; j < nblk; ++j) {
    const uint4* tiles = bst + (j & 1) * TileStage<KS>::kUnits;
#pragma unroll
    for (int cc = 0; cc < kStage; ++cc) chunk(j * kStage + cc, tiles + cc * KS * 64, xb[cc % PD]);
    if (MARKOV) {
      tile_stage_store<KS>(stage, bst + ((j + 1) & 1) * TileStage<KS>::kUnits);
      tile_stage_load<KS>(a, j + 2, nch, stage);
    }
    __syncthreads();   // block j + 1 is in LDS; nobody reads block j any more
  }
}

// Target rows, after the workgroup's draft rows, in items of kItemRows rows of one
// group handed out by counters (zeroed by pack): the second workgroup resident on a
// compute unit issues behind the first (its waves are younger), and with a fixed
// split it would finish ~10 us after it; taking items until none is left, both end
// together.  Item i covers group i % NG and rows [kItemRows (i / NG), +kItemRows) of
// the row list: rows 0..gamma-1 of every stream, enumerated as p = b k + j; then, only
// if the batch has a greedy stream, one more row per stream: the bonus row gamma of a
// greedy stream (its argmax is needed by the scan).  A sampled stream's bonus row is
// read by pass 2, and only when the verifier stops there.  A 16-lane DPP row covers
// the group's 256 ids of one row; a workgroup step takes 16 rows, U steps an item.
// Workgroup g draws from counter g % min(kQueues, grid), whose items are the indices
// of that residue class (one counter for the whole grid serialises ~2500 atomics on
// one address).  Thread 0 claims one item ahead (in `pend`), so the counter's round
// trip is hidden behind an item's loads.
// One claim: a plain single-lane atomic.  The address goes through a VGPR the compiler
// cannot see into, so the atomic optimizer (which rewrites an atomic on a uniform
// address into a wave-level one whose result is read back at once) leaves it alone,
// and the result is waited for only where it is used, one item later.
typedef __attribute__((address_space(1))) int global_int;   // a global (not flat) address

__device__ __forceinline__ int claim_add(int* p) {
  uintptr_t v = reinterpret_cast<uintptr_t>(p);
  asm volatile("" : "+v"(v));
  return __hip_atomic_fetch_add(reinterpret_cast<global_int*>(v), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// An item is 16 U rows of one group: 32 rows (measured at the headline shape: 64-row
// items end the phase less evenly, 16-row items keep too few loads in flight).
template <int DT>
struct TargetQueue {
  static constexpr int U = 2;
  static constexpr int kRS = kThreads / 16;      // rows per step
  static constexpr int kItemRows = kRS * U;
  int* slot;   // LDS [2]: the claimed index, seen by the whole workgroup
  int par;     // which slot the next claim uses
  int pend;    // thread 0: the index claimed for the next item
};

template <int DT, bool VEC>
__device__ __forceinline__ void pass1_target(const Args& a, const StreamTable& st, TargetQueue<DT>& tq, int g,
                                             int ng1) {
  using Q = TargetQueue<DT>;
  constexpr int U = Q::U, RS = Q::kRS, IR = Q::kItemRows;
  const int tid = threadIdx.x, rq = tid >> 4, l16 = tid & 15;
  const int k1 = a.k + 1;
  const int NT = a.B * k1, NS = a.B * a.k;
  const int NR = NS + (st.any_greedy ? a.B : 0);
  const int NI = (NR + IR - 1) / IR * a.NG;
  const size_t rb = (size_t)a.V * (DT == kBF16 ? 2 : 4);
  const char* base = reinterpret_cast<const char*>(a.target);
  const float hk = 0.5f / (float)a.k;
  // row p of the list -> stream b, target row tr, and whether it is needed
  auto map = [&](int p, int& b, int& tr) {
    if (p < NS) {
      b = min(div_small(p, hk), a.B - 1);
      const int j = p - b * a.k;
      tr = b * k1 + j;
      return j < st.gam[b];
    }
    b = min(p - NS, a.B - 1);
    tr = b * k1 + st.gam[b];
    return p < NR && st.tc[b] < kGreedyTc;
  };
  const int nq = min(kQueues, ng1), qx = g % nq;
  auto claim = [&]() {
    if (tid == 0) {
      tq.slot[tq.par] = tq.pend;
      tq.pend = claim_add(a.ws.nitems + kQueueStride * (1 + qx));
    }
    __syncthreads();
    const int i = qx + nq * __builtin_amdgcn_readfirstlane(tq.slot[tq.par]);
    tq.par ^= 1;
    return i;
  };
  // unconditional loads, as in the draft phase: an unneeded row re-reads its stream's
  // first row
  auto load_item = [&](int i, Raw16<DT>(&raw)[U]) {
    const int gi = i % a.NG, r0 = i / a.NG * IR;
    const int cw = gi * kGroup + 16 * l16;
    const int c0 = VEC ? min(cw, a.V - 16) : cw;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int b, tr;
      const bool act = map(min(r0 + RS * u + rq, NR - 1), b, tr);
      raw_load<DT, VEC>(raw[u], base + (size_t)(act ? tr : b * k1) * rb, c0, a.V);
    }
  };
  auto consume = [&](int i, const Raw16<DT>(&raw)[U]) {
    const int gi = i % a.NG, r0 = i / a.NG * IR;
    const int cw = gi * kGroup + 16 * l16;
    const int c0 = VEC ? min(cw, a.V - 16) : cw;
    const int shift = VEC ? (cw >= a.V ? 16 : cw - c0) : 0;   // columns of the window owned elsewhere
    const bool rag = VEC && (gi + 1) * kGroup > a.V;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int b = 0, tr = 0;
      const int p = r0 + RS * u + rq;
      const bool act = p < NR && map(p, b, tr);
      float x[16];
      raw_to_f32<DT>(raw[u], x);
      if (rag) mask_shift(x, shift);
      const float2 pw = row_partial<1>(x, act ? st.tc[b] : 0.f);
      if (l16 == 0 && act) st_c(&a.ws.tpart[(size_t)gi * NT + tr], pw);
    }
  };
  int cur = claim();
  if (cur >= NI) return;
  Raw16<DT> ra[U], rbuf[U];
  load_item(cur, ra);
  for (;;) {   // past the last item, the current one is loaded again (cache hits), unused
    const int nx = claim();
    load_item(nx < NI ? nx : cur, rbuf);
    consume(cur, ra);
    if (nx >= NI) break;
    const int nx2 = claim();
    load_item(nx2 < NI ? nx2 : nx, ra);
    consume(nx, rbuf);
    if (nx2 >= NI) break;
    cur = nx2;
  }
}


// LDS of pass 1: the wave partials of a flush, the staged W1 tiles (32 KB at R = 256)
// and the item claim slots; the per-stream table (8 bytes a stream) lives in the
// launch's dynamic LDS.
template <int KS, bool MARKOV>
struct Pass1Lds {
  float2 part[kFlush * kChunk][kWaves];
  uint4 bst[MARKOV ? 2 * TileStage<KS>::kUnits : 1];
  int qslot[2];
};

// Pass 1 for vocabulary group g of a pass of ng1 workgroups (one per group).  A
// receives this workgroup's W2 slab (the fused launch keeps it for pass 2).
// VEC (rows 16-byte aligned, V >= 16) is a whole-launch choice made on the host.
template <int DT, int KS, bool MARKOV, bool VEC>
__device__ __forceinline__ void pass1_body(const Args& a, int g, int ng1, Pass1Lds<KS, MARKOV>& sh, char* table,
                                           bf16x8 (&A)[4][KS]) {
  // Issue order: this thread's stream's temperature and draft count, then the W2 slab
  // and the first W1 tile block (which do not depend on the stream table), so that
  // building the table waits only for its own two loads and the slab, the launch's
  // longest wait, starts at once.
  const int tb = min((int)threadIdx.x, a.B - 1);
  const float T0 = a.temperature != nullptr ? a.temperature[tb] : 1.0f;    // raw: used after the
  const int n0 = a.num_drafts != nullptr ? a.num_drafts[tb] : a.k;          // slab loads below
  TileStage<KS> stage;
  if (MARKOV) {
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    load_w2_slab<KS, VEC>(a, g * kGroup + w * kWaveCols, l & 15, l >> 4, A);
    tile_stage_load<KS>(a, 0, (a.B * a.k + kChunk - 1) / kChunk, stage);
  }
  __builtin_amdgcn_sched_barrier(0);   // keep the uses of T0 and n0 after the loads above
  const StreamTable st = build_stream_table(a, table, (int)threadIdx.x < a.B ? T0 : NAN,
                                            n0 < 0 ? 0 : (n0 > a.k ? a.k : n0));
  TargetQueue<DT> tq{sh.qslot, 0, 0};
  if (threadIdx.x == 0) tq.pend = claim_add(a.ws.nitems + kQueueStride * (1 + g % min(kQueues, ng1)));
  pass1_draft<DT, KS, MARKOV, VEC>(a, st, g, sh.part, sh.bst, A, stage);
  pass1_target<DT, VEC>(a, st, tq, g, ng1);
}

template <int DT, int KS, bool MARKOV, bool VEC>
__global__ __launch_bounds__(kThreads, 2) void pass1_kernel(Args a) {
  extern __shared__ __align__(16) char table[];
  __shared__ Pass1Lds<KS, MARKOV> sh;
  bf16x8 A[4][KS];
  pass1_body<DT, KS, MARKOV, VEC>(a, blockIdx.x, gridDim.x, sh, table, A);
}

// Row normalisers from the group partials (m_g, s_g) of pass 1: M = max_g m_g and
// S = sum_g s_g 2^((m_g - M) c), returned as (M, log2 S).  A stream's partials of one
// group are contiguous (its target rows, then, in the other buffer, its draft rows),
// so the workgroup first copies up to 6 target and 6 draft rows of 512 groups into
// LDS, row-major, with consecutive lanes on consecutive 8-byte words (a wave
// instruction touches ~11 groups' worth of lines instead of 64); then each wave
// reduces 3 rows from LDS.  The terms use pass 1's fp32 c and its three-operation
// exponent (M c split into hi + lo exactly), so each moves by a relative
// (m_g - M) c 2^-24 at most and S is within ~2e-7 relative, summed in fp64.
constexpr int kScanRows = 6;                               // target (and draft) rows per pass
constexpr int kScanGroups = 256;                           // groups per pass
constexpr int kStageIter = kScanRows * kScanGroups / kThreads;
struct ScanLds {
  float2 t[kScanRows][kScanGroups + 1];   // +1: stores of one instruction spread over banks
  float2 d[kScanRows][kScanGroups + 1];
};
struct StageRegs {
  float2 t[kStageIter], d[kStageIter];
};

// Loads rows [r0, r0 + nt) of the stream's target partials and [r0, r0 + nd) of its
// draft partials for groups [g0, g0 + ng); element e = tid + 256 i is group e / 6,
// row e % 6.  Rows or groups past the range re-read a valid word (ignored).
__device__ __forceinline__ void stage_load(StageRegs& sr, const Args& a, int b, int r0, int nt, int nd, int g0,
                                           int ng, int tid) {
  const int k1 = a.k + 1, NT = a.B * k1, ND = a.B * a.k;
#pragma unroll
  for (int i = 0; i < kStageIter; ++i) {
    const int e = tid + kThreads * i;
    const int gl = min(e / kScanRows, ng - 1), r = e % kScanRows;
    const size_t gg = (size_t)(g0 + gl);
    sr.t[i] = ld_c(&a.ws.tpart[gg * NT + b * k1 + r0 + (r < nt ? r : 0)]);
    sr.d[i] = ld_c(&a.ws.dpart[gg * ND + b * a.k + min(r0 + (r < nd ? r : 0), a.k - 1)]);
  }
}

__device__ __forceinline__ void stage_store(const StageRegs& sr, ScanLds& sh, int tid) {
#pragma unroll
  for (int i = 0; i < kStageIter; ++i) {
    const int e = tid + kThreads * i;
    const int gl = e / kScanRows, r = e % kScanRows;
    sh.t[r][gl] = sr.t[i];
    sh.d[r][gl] = sr.d[i];
  }
}

// One pass of groups [g0, g0 + ng) over one LDS row, folded into its running (M, S).
// Every term, and the rescaling of S when the pass raises M, is 2^((m - M) cf) in
// the three-operation form 2^(fma(m, cf, -mh)) 2^(-ml) with M cf = mh + ml exactly
// (cf = log2(e) / T in fp32, as pass 1 used inside each group); an empty group
// (m_g = -inf, s_g = 0) adds 0.
__device__ __forceinline__ void stage_reduce_row(const float2* row, int l, int ng, float cf, float& M, double& S) {
  float2 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int g = l + 64 * i;
    v[i] = g < ng ? row[g] : make_float2(-INFINITY, 0.f);
  }
  float m = v[0].x;
#pragma unroll
  for (int i = 1; i < 8; ++i) m = fmaxf(m, v[i].x);
  m = wave_max_dpp(m);
  if (m > M) {
    if (M != -INFINITY) {
      const float mh = m * cf, ml = fmaf(m, cf, -mh);
      S *= (double)__builtin_amdgcn_exp2f(fmaf(M, cf, -mh)) * (double)__builtin_amdgcn_exp2f(-ml);
    }
    M = m;
  }
  const float mh = M * cf, ml = fmaf(M, cf, -mh);
  double part = 0.0;
#pragma unroll
  for (int i = 0; i < 8; ++i) part += (double)v[i].y * (double)__builtin_amdgcn_exp2f(fmaf(v[i].x, cf, -mh));
  S += part * (double)__builtin_amdgcn_exp2f(-ml);
}

// The 3 LDS rows of this wave (slot q: row w + 4q of the 12, target rows first), one
// after the other (a scheduling barrier keeps their registers apart).
__device__ __forceinline__ void stage_reduce(const ScanLds& sh, int w, int l, int ng, double c, float (&M)[3],
                                             double (&S)[3]) {
  const float cf = (float)c;
#pragma unroll
  for (int q = 0; q < 3; ++q) {
    const int slot = w + kWaves * q;
    stage_reduce_row(slot < kScanRows ? sh.t[slot] : sh.d[slot - kScanRows], l, ng, cf, M[q], S[q]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Temperature 0 [P1 §4 "Greedy is a different code path"]: a draft is kept iff it is
// the target's argmax at its slot (first id among equal maxima); the first mismatch
// stops the block and the target's argmax there is emitted (the bonus position's when
// every draft is kept).  The argmax of a target row comes from its group maxima (raw
// logits, exact): the first group that reaches the row maximum, then the first id of
// that group holding it.  No residual pass and no sampler are involved.
constexpr int kLoadsInFlight = 8;   // per lane, in the per-wave loops over group partials

template <int DT>
__device__ __forceinline__ void greedy_scan(const Args& a, int b, int gamma, int* s_am) {
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int k1 = a.k + 1, NT = a.B * k1, NG = a.NG;
  const size_t rb = (size_t)a.V * (DT == kBF16 ? 2 : 4);
  for (int r = w; r <= gamma; r += kWaves) {   // one wave per target row
    const int row = b * k1 + r;
    // the group maxima of lane l are groups l + 64 u: loaded 8 at a time (clamped
    // index, masked after), kept for the index search when they all fit
    float gm[kLoadsInFlight];
    auto load_maxima = [&](int g0) {
#pragma unroll
      for (int u = 0; u < kLoadsInFlight; ++u)
        gm[u] = ld_c(&a.ws.tpart[(size_t)min(g0 + l + 64 * u, NG - 1) * NT + row]).x;
    };
    load_maxima(0);
    float M = -INFINITY;
    for (int g0 = 0;;) {
#pragma unroll
      for (int u = 0; u < kLoadsInFlight; ++u)
        if (g0 + l + 64 * u < NG) M = fmaxf(M, gm[u]);
      g0 += 64 * kLoadsInFlight;
      if (g0 >= NG) break;
      load_maxima(g0);
    }
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    int gs = 0x7fffffff;
    if (NG > 64 * kLoadsInFlight) load_maxima(0);
    for (int g0 = 0;;) {
#pragma unroll
      for (int u = 0; u < kLoadsInFlight; ++u)
        if (g0 + l + 64 * u < NG && gm[u] == M) gs = min(gs, g0 + l + 64 * u);
      g0 += 64 * kLoadsInFlight;
      if (g0 >= NG) break;
      load_maxima(g0);
    }
    for (int off = 32; off >= 1; off >>= 1) gs = min(gs, __shfl_xor(gs, off));
    gs = gs < NG ? gs : 0;
    int vs = 0x7fffffff;
    const char* rowp = reinterpret_cast<const char*>(a.target) + (size_t)row * rb;
#pragma unroll
    for (int i = 0; i < kGroup / 64; ++i) {
      const int v = gs * kGroup + (kGroup / 64) * l + i;
      if (v < a.V && load1<DT>(rowp, v) == M) vs = min(vs, v);
    }
    for (int off = 32; off >= 1; off >>= 1) vs = min(vs, __shfl_xor(vs, off));
    if (l == 0) s_am[r] = vs < a.V ? vs : gs * kGroup;
  }
  __syncthreads();
  if (tid == 0) {
    int t = gamma;
    for (int j = 0; j < gamma; ++j)
      if (s_am[j] != a.tokens[b * a.k + j]) { t = j; break; }
    // gamma, the stop (no residual mass is needed), 0, the emitted token
    st_c(reinterpret_cast<int4*>(a.ws.info + 4 * b), make_int4(gamma, t, 0, s_am[t]));
    st_c(&a.ws.rowmask[b], 0u);
  }
  if (tid <= gamma) st_c(&a.ws.logP[b * k1 + tid], (double)NAN);
  if (tid < gamma) {
    st_c(&a.ws.lpx[b * a.k + tid], (double)NAN);
    st_c(&a.ws.lqx[b * a.k + tid], (double)NAN);
  }
}

// LDS of the scan of one stream.
struct ScanPhaseLds {
  ScanLds sh[2];   // the group passes in turn (the first two loaded at the start)
  float s_M[2 * kMaxK + 1];
  double s_l2s[2 * kMaxK + 1];
  double s_lt[kMaxK], s_ld[kMaxK], s_u[kMaxK], s_lr[kMaxK], s_lp[kMaxK + 1];
  double s_thr[kMaxK], s_eP[kMaxK + 1];
  int s_am[kMaxK + 1];
  int s_base;
  uint32_t s_mask;
};

// The scan of stream b.  Every thread of the workgroup calls it.
template <int DT>
// tT, tgam: the stream table's T_b and gamma_b in LDS (the fused launch), or null (read
// from the inputs).
__device__ __forceinline__ void scan_body(const Args& a, int b, ScanPhaseLds& L, const float* tT = nullptr,
                                          const int* tgam = nullptr) {
  float* s_M = L.s_M;
  double* s_l2s = L.s_l2s;
  double *s_lt = L.s_lt, *s_ld = L.s_ld, *s_u = L.s_u, *s_lr = L.s_lr, *s_lp = L.s_lp;
  double *s_thr = L.s_thr, *s_eP = L.s_eP;
  int& s_base = L.s_base;
  uint32_t& s_mask = L.s_mask;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  // The row statistics of the first two group passes go out first: they depend on b
  // alone (rows 0 .. min(6, k) - 1, a bound on gamma_b: the rows at and past gamma_b
  // are loaded and not used; a second pass past the last group re-reads group NG - 1),
  // and the stream's draft count and temperature arrive meanwhile.
  const int kr = min(kScanRows, a.k);
  const int ngp = min(a.NG, kScanGroups);
  const int ng2 = min(a.NG - kScanGroups, kScanGroups);   // groups of the second pass (<= 0: none)
  StageRegs sreg, sreg2;
  stage_load(sreg, a, b, 0, kr, kr, 0, ngp, tid);
  stage_load(sreg2, a, b, 0, kr, kr, min(kScanGroups, a.NG - 1), max(ng2, 1), tid);
  const int gamma = tgam != nullptr ? tgam[b] : stream_gamma(a, b);
  const float Tf = tT != nullptr ? tT[b] : stream_temp(a, b);
  if (Tf == 0.f) {   // the whole workgroup takes the greedy branch
    greedy_scan<DT>(a, b, gamma, L.s_am);
    return;
  }
  const double T = (double)Tf;
  const double c = kLog2e / T;
  const int k1 = a.k + 1;
  const int NT = a.B * k1, ND = a.B * a.k;
  const size_t esz = DT == kBF16 ? 2 : 4;
  // the first two passes into LDS now (issued before the temperature, so arrived):
  // their registers are free for the gathers
  stage_store(sreg, L.sh[0], tid);
  stage_store(sreg2, L.sh[1], tid);

  if (tid < gamma) s_u[tid] = accept_uniform(a.key0, a.key1, (uint32_t)b, (uint32_t)tid, a.step);

  // the logits at the drafts, t_j(x_j) and d_j(x_j) + W1[prev_j] . W2t[x_j] (the bias in
  // fp64): wave w takes slots w and w + 4 at a time, lane l ranks 4l .. 4l + 3
  for (int j0 = w; j0 < gamma; j0 += 2 * kWaves) {
    int x[2], pv[2];
    uint2 p1[2], p2[2];
    float lt[2], ld[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int j = min(j0 + kWaves * u, gamma - 1);
      x[u] = clamp_tok(a.tokens[b * a.k + j], a.V);
      pv[u] = a.W1 != nullptr ? draft_prev(a, b, j) : -1;
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int j = min(j0 + kWaves * u, gamma - 1);
      lt[u] = load1<DT>(reinterpret_cast<const char*>(a.target) + (size_t)(b * k1 + j) * a.V * esz, x[u]);
      ld[u] = load1<DT>(reinterpret_cast<const char*>(a.draft) + (size_t)(b * a.k + j) * a.V * esz, x[u]);
      const int r = min(4 * l, max(a.R - 4, 0));   // lanes past R / 4 re-read a valid piece, unused
      p1[u] = p2[u] = make_uint2(0, 0);
      if (a.W1 != nullptr) {
        p1[u] = *reinterpret_cast<const uint2*>(a.W1 + (size_t)max(pv[u], 0) * a.R + r);
        p2[u] = *reinterpret_cast<const uint2*>(a.W2t + (size_t)x[u] * a.R + r);
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      double acc = 0.0;
      if (pv[u] >= 0 && 4 * l < a.R)
        acc = (double)bf16lo(p1[u].x) * (double)bf16lo(p2[u].x) + (double)bf16hi(p1[u].x) * (double)bf16hi(p2[u].x) +
              (double)bf16lo(p1[u].y) * (double)bf16lo(p2[u].y) + (double)bf16hi(p1[u].y) * (double)bf16hi(p2[u].y);
      acc = wave_sum(acc);
      const int j = j0 + kWaves * u;
      if (l == 0 && j < gamma) {
        s_lt[j] = lt[u];
        s_ld[j] = (double)ld[u] + acc;
      }
    }
  }

  // row normalisers of target and draft rows 0..gamma-1 (the bonus row's statistics
  // are taken by pass 2 if the verifier stops there): passes of 6 target and 6 draft
  // rows (the first pass's loads were issued above), each over groups in runs of 512
  // staged through LDS
  for (int r0 = 0; r0 < gamma; r0 += kScanRows) {
    const int nt = min(kScanRows, gamma - r0), nd = nt;
    float M[3] = {-INFINITY, -INFINITY, -INFINITY};
    double S[3] = {0.0, 0.0, 0.0};
    for (int g0 = 0; g0 < a.NG; g0 += kScanGroups) {
      const int ng = min(kScanGroups, a.NG - g0);
      // rows 0..5 of groups 0..511 were loaded at the start (buffers 0 and 1); any other
      // pass is loaded now into buffer 0, once its readers are done with it
      const bool pre = r0 == 0 && g0 <= kScanGroups;
      ScanLds& sh = L.sh[pre && g0 == kScanGroups ? 1 : 0];
      if (!pre) {
        stage_load(sreg, a, b, r0, nt, nd, g0, ng, tid);
        __syncthreads();
        stage_store(sreg, sh, tid);
      }
      __syncthreads();
      stage_reduce(sh, w, l, ng, c, M, S);
    }
#pragma unroll
    for (int q = 0; q < 3; ++q) S[q] = wave_sum(S[q]);
    // one log2 per wave: lane q takes row q
    const double l2s = log2(l == 0 ? S[0] : (l == 1 ? S[1] : S[2]));
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      const int slot = w + kWaves * q;
      const bool is_t = slot < kScanRows;
      const int j = r0 + (is_t ? slot : slot - kScanRows);   // slot within the stream
      if (l == q && j < gamma) {
        const int r = is_t ? j : gamma + 1 + j;                 // index into s_M / s_l2s
        s_M[r] = M[q];
        s_l2s[r] = l2s;
        if (is_t) { st_c(&a.ws.tm[b * k1 + j], M[q]); st_c(&a.ws.tl2s[b * k1 + j], l2s); }
        else { st_c(&a.ws.dm[b * a.k + j], M[q]); st_c(&a.ws.dl2s[b * a.k + j], l2s); }
      }
    }
  }
  __syncthreads();

  // per slot, in parallel: log p_j(x_j), log q_j(x_j), log r_j
  if (tid < gamma) {
    const int j = tid;
    const double lpx = (s_lt[j] - (double)s_M[j]) / T - s_l2s[j] * kLn2;
    const double lqx = (s_ld[j] - (double)s_M[gamma + 1 + j]) / T - s_l2s[gamma + 1 + j] * kLn2;
    st_c(&a.ws.lpx[b * a.k + j], lpx);
    st_c(&a.ws.lqx[b * a.k + j], lqx);
    s_lr[j] = lpx - lqx;
    s_thr[j] = s_lr[j] >= 0.0 ? 1.0 : exp(s_lr[j]);   // token-wise threshold min(1, r_j)
  }
  __syncthreads();
  // clipped prefix log P_i (each slot recomputes it, in the same order) and P_i itself
  if (tid <= gamma) {
    double lp = 0.0;
    for (int i = 1; i <= tid; ++i) {
      const double v = lp + s_lr[i - 1];
      lp = v < 0.0 ? v : 0.0;
    }
    s_lp[tid] = lp;
    s_eP[tid] = exp(lp);
  }
  __syncthreads();
  if (tid == 0) {
    // token-wise stop t: first j with u_j > min(1, r_j)
    int t = gamma;
    for (int j = 0; j < gamma; ++j)
      if (!(s_u[j] <= s_thr[j])) { t = j; break; }
    uint32_t mask = 0;
    int stop = 0, f = 0;
    if (a.method == 0) {
      stop = t;
      if (t < gamma) mask = 1u << t;
    } else {
      if (gamma == 0 || s_u[gamma - 1] <= s_eP[gamma]) {
        stop = gamma;   // top test passed (or no drafts): tau = gamma
      } else {
        for (int i = gamma - 1; i >= 0; --i) if (s_lp[i] == 0.0) { f = i; break; }
        mask = 1u << f;  // tau >= f; row f may be sampled
        for (int i = f + 1; i < gamma; ++i)
          if (s_u[i - 1] <= s_eP[i]) mask |= 1u << i;   // h_i <= P_i: only these can pass
        stop = -1;
      }
    }
    st_c(reinterpret_cast<int4*>(a.ws.info + 4 * b), make_int4(gamma, stop, f, t));
    st_c(&a.ws.rowmask[b], mask);
    s_mask = mask;
    s_base = mask ? atomicAdd(a.ws.nitems, __popc(mask)) : 0;
    int bonus_item = -1;
    if (stop == gamma) {   // the bonus row is sampled: pass 2 races over it
      const int ib = atomicAdd(a.ws.nitems + 1, 1);
      Item it{};
      it.dr = -1;
      it.tr = b * k1 + gamma;
      it.prev = -1;
      it.b = b;
      temp_split((float)T, it.chi, it.clo);
      bonus_item = a.B * a.k - 1 - ib;
      st_c(&a.ws.items[bonus_item], it);
    }
    st_c(reinterpret_cast<int2*>(a.ws.info2 + 4 * b), make_int2(s_base, bonus_item));
  }
  __syncthreads();
  if (tid <= gamma) st_c(&a.ws.logP[b * k1 + tid], s_lp[tid]);
  const uint32_t mask = s_mask;
  if (tid < gamma && ((mask >> tid) & 1u)) {
    const int i = tid;
    Item it;
    it.dr = b * a.k + i;
    it.tr = b * k1 + i;
    it.prev = a.W1 != nullptr ? draft_prev(a, b, i) : -1;
    it.b = b;
    it.Mt = s_M[i];
    it.Md = s_M[gamma + 1 + i];
    temp_split((float)T, it.chi, it.clo);
    const double kp = (a.method == 1 ? s_lp[i] * kLog2e : 0.0) - s_l2s[i];
    const double kq = -s_l2s[gamma + 1 + i];
    it.kph = (float)kp;
    it.kpl = (float)(kp - (double)it.kph);
    it.kqh = (float)kq;
    it.kql = (float)(kq - (double)it.kqh);
    st_c(&a.ws.items[s_base + __popc(mask & ((1u << i) - 1u))], it);
  }
}

// ---------------------------------------------------------------------------
// Race clocks ahead of pass 2.  Row (b, grp) holds log2 E of the sampler's clocks of
// stream b at ids grp * 256 .. + 255 (ws.clk, int16 in units of 2^-10): one generator
// block of four ids per lane, one row per wave.  Workgroup `slot` of `nslots` takes
// an equal share of the B NG rows.
// ---------------------------------------------------------------------------
// Four rows per turn, computed side by side (four independent generator chains); a
// row past the share is computed from a clamped row and not stored.  Greedy streams'
// rows are computed too (unused): the loop reads nothing from memory.
__device__ __forceinline__ void clock_rows(const Args& a, int slot, int nslots) {
  constexpr int kU = 4;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int rows = a.B * a.NG;
  const int per = (rows + nslots - 1) / nslots;
  const int r0 = slot * per, r1 = min(r0 + per, rows);
  for (int rb = r0 + kU * w; rb < r1; rb += kU * kWaves) {
    int b = rb / a.NG, grp = rb - b * a.NG;   // row rb; the next ones step from it
    uint2 out[kU];
    int dst[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (u > 0) {
        ++grp;
        while (grp >= a.NG) {   // at most once unless NG < 4
          grp -= a.NG;
          ++b;
        }
      }
      const uint32_t bb = (uint32_t)min(b, a.B - 1);
      dst[u] = rb + u < r1 ? (int)bb * a.NG * 64 + grp * 64 + l : -1;
      const uint4 x = philox4(bb, (uint32_t)(grp * 64 + l), kPurposeSample, a.step, a.key0, a.key1);
      const uint32_t q0 = (uint32_t)clock_log2_q10(x.x) & 0xffffu, q1 = (uint32_t)clock_log2_q10(x.y) & 0xffffu;
      const uint32_t q2 = (uint32_t)clock_log2_q10(x.z) & 0xffffu, q3 = (uint32_t)clock_log2_q10(x.w) & 0xffffu;
      out[u] = make_uint2(q0 | (q1 << 16), q2 | (q3 << 16));
    }
#pragma unroll
    for (int u = 0; u < kU; ++u)
      if (dst[u] >= 0) st_c(&a.ws.clk[(size_t)dst[u]], out[u]);
  }
}

// Workgroups 0..B-1 scan their stream; the rest compute the race clocks.
template <int DT>
__global__ __launch_bounds__(kThreads) void scan_kernel(Args a) {
  __shared__ ScanPhaseLds L;
  if ((int)blockIdx.x >= a.B) {
    clock_rows(a, (int)blockIdx.x - a.B, (int)gridDim.x - a.B);
    return;
  }
  scan_body<DT>(a, blockIdx.x, L);
}

// threadIdx.x through a register the compiler cannot see into: index math formed from
// it inside a loop is recomputed there (a few VALU) instead of being kept live across
// the loop, where it would take registers or spill.
__device__ __forceinline__ int opaque_tid() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// ---------------------------------------------------------------------------
// Race candidates.  The sampler draws Y = argmax_v w_v / E_v over the whole
// vocabulary, one Exp(1) clock per id (an exponential race picks v with probability
// w_v / sum w).  The kernels rank log2 w - log2 E in fp32 and keep, per listed row
// and 256-id group, the two best (score, id); the per-stream kernels then take the
// best group and re-evaluate every candidate within kRaceWindow of it in fp64.
// ---------------------------------------------------------------------------
constexpr float kRaceWindow = 0x1.0p-6f;   // log2 units: far above the fp32 ranking error (~1e-5)

__device__ __forceinline__ Top2 top2_empty() { return Top2{-INFINITY, INT_MAX, -INFINITY, INT_MAX}; }
// Bitwise, not short-circuit: the comparisons become lane masks combined on the scalar
// unit, with no branch.
__device__ __forceinline__ bool top_better(float s, int v, float t, int u) {
  return (int)(s > t) | ((int)(s == t) & (int)(v < u));
}
// Branch-free (selects only): (-inf, INT_MAX) is never inserted.
__device__ __forceinline__ void top2_add(Top2& a, float s, int v) {
  const bool b1 = top_better(s, v, a.s1, a.v1);
  const bool b2 = top_better(s, v, a.s2, a.v2);
  const float s2 = b1 ? a.s1 : (b2 ? s : a.s2);
  const int v2 = b1 ? a.v1 : (b2 ? v : a.v2);
  a.s1 = b1 ? s : a.s1;
  a.v1 = b1 ? v : a.v1;
  a.s2 = s2;
  a.v2 = v2;
}
__device__ __forceinline__ void top2_merge(Top2& a, const Top2& o) {
  top2_add(a, o.s1, o.v1);
  top2_add(a, o.s2, o.v2);
}
// The race of pass 2's rows, listed or bonus: a lane's best score over its 16 ids
// c0 .. c0 + 15 in increasing order (a later id replaces an earlier one only with a
// strictly larger score, so the smaller id wins ties), from 16 clocks L (int16, units
// of 2^-10, two to a word).  A listed row's y are residual weights w >= 0 (score
// log2 w - log2 E), a bonus row's y are y = x c, the logits scaled to log2 units
// (-inf: none; score y - log2 E); either way the scores share the row's scale across
// lanes, waves and groups.  Lanes keep one candidate each and the best two of a row's
// 16 lanes go on (merged at the flush): two ids of one lane trade places only
// when their scores agree to the fp32 rounding, which the fp64 check of every
// candidate near the best does not need.
__device__ __forceinline__ Top2 race16_row(const float (&y)[16], const uint2 (&L)[4], bool bonus, int c0) {
  float best = -INFINITY;
  int bv = INT_MAX;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const uint32_t word = (e & 2) ? L[e >> 2].y : L[e >> 2].x;
    const int q = (e & 1) ? ((int32_t)word >> 16) : ((int32_t)(word << 16) >> 16);
    const float lq = (float)q * 0x1.0p-10f;
    // computed on every lane and selected (a branch per id costs more than the log):
    // a residual weight is +0 or positive and log2(+0) = -inf
    const float lg = __builtin_amdgcn_logf(y[e]);
    const float sc = (bonus ? y[e] : lg) - lq;
    const bool better = sc > best;
    best = better ? sc : best;
    bv = better ? c0 + e : bv;
  }
  Top2 r = top2_empty();
  r.s1 = best;
  r.v1 = best > -INFINITY ? bv : INT_MAX;
  return r;
}

// This lane's 16 clocks of stream b at ids c0 .. c0 + 15 (c0 a multiple of 4).
__device__ __forceinline__ void load_clocks(const Args& a, uint32_t b, int c0, uint2 (&L)[4]) {
  const uint2* p = a.ws.clk + (size_t)b * a.NG * 64 + (c0 >> 2);
#pragma unroll
  for (int i = 0; i < 4; ++i) L[i] = ld_c(&p[i]);
}

// ---------------------------------------------------------------------------
// pass2: per listed row and group, the residual mass sum max(0, P_i p_i - q_i) and
// the race candidates of w = max(0, P_i p_i - q_i); then, for the bonus rows the
// verifiers stop at (listed from the back), the race candidates of w = p_gamma.
// The scan prepared one Item per listed row (row indices and exponent constants)
// and its packed W1 tile.  Waves reduce 64 ids each; the 4 wave results of a row
// meet in LDS and are flushed every 256 rows.
// ---------------------------------------------------------------------------
constexpr int kItemWords = (int)(sizeof(Item) / sizeof(int32_t));
static_assert(kItemWords == 12, "Item is 12 words: dr, tr, prev, b, Mt, Md, chi, clo, kph, kpl, kqh, kql");
constexpr int kStageWords = kChunk * kItemWords;   // one chunk's items: 192 words, 3 per lane
struct Pass2Lds {
  float part[kFlush * kChunk][kWaves];
  uint2 cand[kFlush * kChunk][17];   // a row's 16 lane candidates (score bits, id); padded
  int32_t items[kWaves][4][kStageWords];    // per wave, the items of chunks c .. c + 2 (ring of 4)
  uint4 btile[2][8 * 64];                   // the W1 tiles of chunks c and c + 1 (R <= 256)
};

// x + bias with the B operand read from LDS one k-step at a time (unit kk * 64 + l).
template <int KS>
__device__ __forceinline__ void markov_mma_lds(const bf16x8 (&A)[4][KS], const uint4* bt, int l, float (&x)[16]) {
  f32x4 acc[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) acc[s] = f32x4{x[4 * s], x[4 * s + 1], x[4 * s + 2], x[4 * s + 3]};
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    const bf16x8 b = __builtin_bit_cast(bf16x8, bt[kk * 64 + l]);
#pragma unroll
    for (int s = 0; s < 4; ++s) acc[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[s][kk], b, acc[s], 0, 0, 0);
  }
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int i = 0; i < 4; ++i) x[4 * s + i] = acc[s][i];
}

// Pass 2 for vocabulary group g.  slab_loaded: A already holds this workgroup's W2
// slab (the fused launch's pass 1 left it there).
template <int DT, int KS, bool MARKOV, bool VEC>
__device__ __forceinline__ void pass2_body(const Args& a, int g, Pass2Lds& L, bf16x8 (&A)[4][KS], bool slab_loaded) {
  auto& part = L.part;
  auto& cand = L.cand;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, n = l & 15, q = l >> 4;
  const int cb = (g * kWaves + w) * kWaveCols;
  const int cw = cb + 16 * q;
  const int c0 = VEC ? min(cw, a.V - 16) : cw;
  const int shift = VEC ? (cw >= a.V ? 16 : cw - c0) : 0;
  const bool rag = VEC && cb + kWaveCols > a.V;
  const size_t rb = (size_t)a.V * (DT == kBF16 ? 2 : 4);
  const int ND = a.B * a.k;

  // the W2 slab does not depend on the list: its loads go out before the count is read
  if (MARKOV && !slab_loaded) load_w2_slab<KS, VEC>(a, cb, n, q, A);
  // The rows in list order: the NI residual rows (items 0 .. NI-1), then the NB bonus
  // rows (items ND-1, ND-2, ...), chunk c holding positions 16c .. 16c + 15.  Each wave
  // stages the item records of its chunks in LDS, two chunks ahead: lane l holds words
  // l, l + 64, l + 128 of a later chunk's 16 records across a chunk, and the rows and
  // constants are read from LDS when they are needed (no registers held through the
  // products, no load waited on in the loop).  Positions past the list read a clamped
  // record: stale, indices clamped to valid rows, nothing computed from it written back.
  const int NT = a.B * (a.k + 1);
  const int NI = ld_c(&a.ws.nitems[0]), NB = ld_c(&a.ws.nitems[1]);
  const int NV = NI + NB;
  auto item_of = [&](int i) { return i < NI ? i : ND - 1 - min(i - NI, ND - 1); };
  int32_t* stage = &L.items[w][0][0];
  int32_t words[3];
  const int32_t* item_words = reinterpret_cast<const int32_t*>(a.ws.items);
  auto load_words = [&](int c) {
    const int lo = opaque_tid() & 63;
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      const int e = lo + 64 * u;   // record e / 12 of the chunk, word e % 12
      const int r = min(c * kChunk + e / kItemWords, ND - 1);
      words[u] = ld_c(item_words + (size_t)item_of(r) * kItemWords + e % kItemWords);
    }
  };
  auto store_words = [&](int c) {
#pragma unroll
    for (int u = 0; u < 3; ++u) stage[(c & 3) * kStageWords + l + 64 * u] = words[u];
    __builtin_amdgcn_wave_barrier();
  };
  auto record = [&](int c) { return stage + (c & 3) * kStageWords + n * kItemWords; };
  auto rows_of = [&](int c) {   // (dr, tr) of this lane's row in chunk c, clamped
    const int32_t* r = record(c);
    return make_int2(min(max(r[0], 0), ND - 1), min(max(r[1], 0), NT - 1));
  };
  auto fetch = [&](int2 h, Raw16<DT>& t, Raw16<DT>& d) {
    raw_load<DT, VEC>(t, reinterpret_cast<const char*>(a.target) + (size_t)h.y * rb, c0, a.V);
    raw_load<DT, VEC>(d, reinterpret_cast<const char*>(a.draft) + (size_t)h.x * rb, c0, a.V);
  };
  // pipeline: records three chunks ahead (registers), two ahead in LDS; the logits of
  // chunk c in ring buffer c & 1, loaded two chunks ahead (the ring is indexed at
  // compile time: the loop runs two chunks per turn).  The prologue issues its loads in
  // the order the loop's first waits need them (the logits last), so that those waits
  // never have to drain the logits.
  // The W1 tile of a chunk (the B operand, the same for the 4 waves: row n's previous
  // token's W1 row in MFMA lane order, zero for a row with no previous token) goes
  // through LDS, double-buffered: each thread gathers its share of the tile two chunks
  // ahead (unit u: k-step u / 64, lane u % 64, from the chunk's records in this wave's
  // stage) and stores it one chunk ahead; the workgroup barrier at the top of each
  // chunk publishes it (and frees the buffer the previous chunk read).  Loads are
  // unconditional (a row with no previous token reads W1 row 0), masked at the store.
  constexpr int kBtUnits = KS * 64, kBtPer = (kBtUnits + kThreads - 1) / kThreads;
  uint4 bt[kBtPer];
  bool btv[kBtPer];
  // (a share is whole when the tile is a multiple of the workgroup: no branch then)
  auto bt_load = [&](int c) {
#pragma unroll
    for (int i = 0; i < kBtPer; ++i) {
      const int u = tid + kThreads * i;
      if (kBtUnits % kThreads == 0 || u < kBtUnits) {
        const int kk = u >> 6, ll = u & 63;
        const int prev = stage[(c & 3) * kStageWords + (ll & 15) * kItemWords + 2];
        btv[i] = prev >= 0 && prev < a.V;
        bt[i] = *reinterpret_cast<const uint4*>(a.W1 + (size_t)(btv[i] ? prev : 0) * a.R + kk * 32 + 8 * (ll >> 4));
      }
    }
  };
  auto bt_store = [&](int c) {
#pragma unroll
    for (int i = 0; i < kBtPer; ++i) {
      const int u = tid + kThreads * i;
      if (kBtUnits % kThreads == 0 || u < kBtUnits) L.btile[c & 1][u] = btv[i] ? bt[i] : make_uint4(0, 0, 0, 0);
    }
  };
  load_words(0);
  store_words(0);
  load_words(1);
  if (MARKOV) bt_load(0);
  store_words(1);
  if (MARKOV) {
    bt_store(0);
    bt_load(1);
  }
  load_words(2);
  Raw16<DT> tr0, dr0, tr1, dr1;
  fetch(rows_of(0), tr0, dr0);
  fetch(rows_of(1), tr1, dr1);
  const int nch = (NV + kChunk - 1) / kChunk;
  auto step = [&](int c, Raw16<DT>& tb, Raw16<DT>& db) {
    // Two workgroups share a CU and run the same number of chunks; the older one's waves
    // win the issue arbitration and finish first, leaving the other to finish alone.
    // Waves take a priority that falls with each chunk done, so the one behind catches up.
    // (levels 3, 2, 1, 0 over the first chunks, so that they differ from the start)
    const int lvl = c;   // uniform
    if (lvl == 0) __builtin_amdgcn_s_setprio(3);
    else if (lvl == 1) __builtin_amdgcn_s_setprio(2);
    else if (lvl == 2) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
    store_words(c + 2);   // loaded a chunk ago: the registers are free for the products
    if (MARKOV) {
      __syncthreads();
      bt_store(c + 1);
    }
    float bias[16];       // the bias alone (not folded into the draft logits: the residual
                          // compares P p with q and keeps their rounding apart)
    if (MARKOV) {
#pragma unroll
      for (int e = 0; e < 16; ++e) bias[e] = 0.f;
      markov_mma_lds<KS>(A, L.btile[c & 1], l, bias);
      __builtin_amdgcn_sched_barrier(0);
      bt_load(c + 2);
    }
    load_words(c + 3);
    const int32_t* rc = record(c);
    const bool bonus = rc[0] < 0;   // a bonus row: no draft row, raced over p_gamma
    const float4 k0 = make_float4(__int_as_float(rc[4]), __int_as_float(rc[5]), __int_as_float(rc[6]),
                                  __int_as_float(rc[7]));   // (Mt, Md, chi, clo)
    const float4 k1 = make_float4(__int_as_float(rc[8]), __int_as_float(rc[9]), __int_as_float(rc[10]),
                                  __int_as_float(rc[11]));  // (kph, kpl, kqh, kql)
    const uint32_t sb = (uint32_t)min(max(rc[3], 0), a.B - 1);
    uint2 ck[4];   // the row's clocks at this lane's ids, used by the race at the end
    load_clocks(a, sb, c0, ck);
    // a residual row: weights w = max(0, P p - q) (normalised) and their sum; a bonus
    // row: y = x log2(e) / T (unnormalised: every group of the row uses the same scale,
    // which is all the race needs).  Straight from the raw logits (the buffers are
    // refilled after); then the race over them.
    // The sum takes every lane's weight times 0 or 1 (a bonus row's sum is never read),
    // so that the weight is needed on every lane and is computed without a branch on
    // the kind of row: the lanes of a chunk mix kinds, and a branch per id costs more
    // than the work it would skip.
    const float res = bonus ? 0.f : 1.f;
    float s = 0.f;
    float y[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float xte = (rag && e < shift) ? -INFINITY : raw_elem<DT>(tb, e);
      const float tp = xte - k0.x;
      const float d = MARKOV ? raw_elem<DT>(db, e) + bias[e] : raw_elem<DT>(db, e);
      const float tq = d - k0.y;
      const float ep = fmaf(tp, k0.z, k1.x) + fmaf(tp, k0.w, k1.y);
      const float eq = fmaf(tq, k0.z, k1.z) + fmaf(tq, k0.w, k1.w);
      const float wv = __builtin_amdgcn_exp2f(ep) - __builtin_amdgcn_exp2f(eq);
      const bool in = VEC || c0 + e < a.V;
      const float wr = (in && wv > 0.f) ? wv : 0.f;
      y[e] = bonus ? (in ? xte * (k0.z + k0.w) : -INFINITY) : wr;
      s = fmaf(res, wr, s);
    }
    fetch(rows_of(c + 2), tb, db);
    s = sum4lanes(s);
    // every lane's best id of the chunk goes to LDS; a row's 16 are merged at the flush
    const Top2 rt = race16_row(y, ck, bonus, c0);
    {
      const int t = opaque_tid(), rr = (c % kFlush) * kChunk + (t & 15), ww = t >> 6;
      cand[rr][4 * ww + ((t & 63) >> 4)] = make_uint2(__float_as_uint(rt.s1), (uint32_t)rt.v1);
      if (q == 0) part[rr][ww] = s;
    }
    if (c % kFlush == kFlush - 1 || c == nch - 1) {
      __syncthreads();
      const int t = opaque_tid();   // addresses formed here, not kept through the loop
      const int i = (c - c % kFlush) * kChunk + t;
      if (t < (c % kFlush + 1) * kChunk && i < NV) {
        const int it = item_of(i);
        if (i < NI) {
          const int dr = min(max(ld_c(&a.ws.items[it].dr), 0), ND - 1);
          st_c(&a.ws.wgrp[(size_t)g * ND + dr], (part[t][0] + part[t][1]) + (part[t][2] + part[t][3]));
        }
        Top2 r = top2_empty();
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const uint2 e = cand[t][u];
          top2_add(r, __uint_as_float(e.x), (int)e.y);
        }
        st_c(&a.ws.race[(size_t)g * ND + it], r);
      }
      __syncthreads();
    }
  };
  for (int c = 0; c < nch; c += 2) {   // uniform: every wave runs the same chunks
    step(c, tr0, dr0);
    if (c + 1 < nch) step(c + 1, tr1, dr1);
  }
}

template <int DT, int KS, bool MARKOV, bool VEC>
__global__ __launch_bounds__(kThreads, 2) void pass2_kernel(Args a) {
  __shared__ Pass2Lds L;
  bf16x8 A[4][KS];
  pass2_body<DT, KS, MARKOV, VEC>(a, blockIdx.x, L, A, false);
}

// ---------------------------------------------------------------------------
// finalize: tau, the race, outputs.  One workgroup per stream.
// ---------------------------------------------------------------------------
__device__ __forceinline__ double block_sum(double v, double* red) {
  const int tid = threadIdx.x;
  v = wave_sum(v);
  if ((tid & 63) == 0) red[tid >> 6] = v;
  __syncthreads();
  const double r = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return r;
}

// Arg-max of score with the lowest index on ties; score < 0 means "not a contestant".
__device__ __forceinline__ void block_argmax(double& score, int& idx, double* rs, int* ri) {
  const int tid = threadIdx.x;
  wave_argmax(score, idx);
  if ((tid & 63) == 0) { rs[tid >> 6] = score; ri[tid >> 6] = idx; }
  __syncthreads();
  score = rs[0]; idx = ri[0];
  for (int ww = 1; ww < kWaves; ++ww) take_better(score, idx, rs[ww], ri[ww]);
  __syncthreads();
}

// Markov bias of the 256 ids of group gsel after one previous token, by the whole
// workgroup: sum_r W1[prev, r] W2t[v, r] (R = 32 KS).  A row of W2t is 4 KS slices of
// 16 bytes; lane l reads slice l mod 4KS of consecutive rows, so one wave instruction
// covers 16 / KS whole rows, and dots it with the same slice of W1[prev] (each bf16
// product is exact in fp32; v_dot2c_f32_bf16 adds two per instruction).  The slice
// sums of a row meet in LDS (rows padded by one float against bank conflicts) and
// thread t returns the bias of id 256 gsel + t.  The bias carries an absolute error of
// a few 1e-9 for weights of the drafter's scale, as fine as the fp32 row statistics it
// is combined with.  Contains a barrier: every thread of the workgroup must call it.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot8_bf16(const uint4& p, const uint4& q) {
  float acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p.x), __builtin_bit_cast(bf16x2, q.x), 0.f,
                                              false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p.y), __builtin_bit_cast(bf16x2, q.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p.z), __builtin_bit_cast(bf16x2, q.z), acc, false);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p.w), __builtin_bit_cast(bf16x2, q.w), acc, false);
}

template <int KS>
struct GroupBiasLds {
  float part[kGroup * (4 * KS + 1)];
};

template <int KS>
__device__ __forceinline__ float group_bias(const Args& a, int prev, int gsel, GroupBiasLds<KS>& sh) {
  constexpr int SL = 4 * KS;                      // 16-byte slices per row
  constexpr int RPI = 64 / SL;                    // rows per wave instruction
  constexpr int NI = kGroup / kWaves / RPI;       // instructions per wave
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int sl = l % SL, ri = l / SL;
  const uint4 w1 = *reinterpret_cast<const uint4*>(a.W1 + (size_t)prev * (32 * KS) + 8 * sl);
  constexpr int NB = NI < 8 ? NI : 8;             // loads in flight per batch
#pragma unroll 1
  for (int n0 = 0; n0 < NI; n0 += NB) {
    uint4 x[NB];
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      const int v = min(gsel * kGroup + w * 64 + (n0 + n) * RPI + ri, a.V - 1);   // rows past V: ignored
      x[n] = *reinterpret_cast<const uint4*>(a.W2t + (size_t)v * (32 * KS) + 8 * sl);
    }
#pragma unroll
    for (int n = 0; n < NB; ++n) sh.part[(w * 64 + (n0 + n) * RPI + ri) * (SL + 1) + sl] = dot8_bf16(w1, x[n]);
  }
  __syncthreads();
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < SL; ++e) acc += sh.part[tid * (SL + 1) + e];
  return acc;
}

// The Markov bias of one id in fp64, by a whole wave: sum_r W1[prev, r] W2t[v, r]
// (prev < 0: 0); every lane gets the result.
__device__ __forceinline__ double bias_f64_wave(const Args& a, int prev, int v) {
  double acc = 0.0;
  if (prev >= 0) {
    const int l = threadIdx.x & 63;
    for (int r = l; r < a.R; r += 64)
      acc += (double)bf16_to_f32(a.W1[(size_t)prev * a.R + r]) * (double)bf16_to_f32(a.W2t[(size_t)v * a.R + r]);
  }
  return wave_sum(acc);
}

// Race winner of one row from the per-group candidates race[g][it] (g < NG): the best
// fp32 score, then every candidate within kRaceWindow of it scored again in fp64 by
// `score64(v)` (called by a whole wave, result in every lane; -inf for no weight).
// Returns the id with the largest fp64 score (the smallest id among equal ones), or
// -1 if no group has a candidate.  Every thread of the workgroup must call it.
constexpr int kMaxCand = 256;
struct RaceLds {
  int cand[kMaxCand];
  double sc[kMaxCand];
  int n;
  float best[kWaves];
};

template <class Score64>
__device__ __forceinline__ int race_pick(const Args& a, int it, int ND, RaceLds& sh, double* rs, int* ri, Score64 score64) {
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int NG = a.NG;
  // every thread's first two groups are loaded at once (clamped, masked after)
  Top2 t0 = ld_c(&a.ws.race[(size_t)min(tid, NG - 1) * ND + it]);
  Top2 t1 = ld_c(&a.ws.race[(size_t)min(tid + kThreads, NG - 1) * ND + it]);
  if (tid >= NG) t0 = top2_empty();
  if (tid + kThreads >= NG) t1 = top2_empty();
  float best = fmaxf(t0.s1, t1.s1);
  for (int gi = tid + 2 * kThreads; gi < NG; gi += kThreads) best = fmaxf(best, ld_c(&a.ws.race[(size_t)gi * ND + it]).s1);
  best = wave_max_dpp(best);
  if (tid == 0) sh.n = 0;
  if (l == 0) sh.best[w] = best;
  __syncthreads();
  best = fmaxf(fmaxf(sh.best[0], sh.best[1]), fmaxf(sh.best[2], sh.best[3]));
  if (best == -INFINITY) return -1;   // uniform
  const float floor_ = best - kRaceWindow;
  auto offer = [&](float sc, int v) {
    if (sc >= floor_ && v >= 0 && v < a.V) {
      const int k = atomicAdd(&sh.n, 1);
      if (k < kMaxCand) sh.cand[k] = v;
    }
  };
  offer(t0.s1, t0.v1); offer(t0.s2, t0.v2);
  offer(t1.s1, t1.v1); offer(t1.s2, t1.v2);
  for (int gi = tid + 2 * kThreads; gi < NG; gi += kThreads) {
    const Top2 t = ld_c(&a.ws.race[(size_t)gi * ND + it]);
    offer(t.s1, t.v1); offer(t.s2, t.v2);
  }
  __syncthreads();
  const int nc = min(sh.n, kMaxCand);
  for (int c = w; c < nc; c += kWaves) {
    const double sc = score64(sh.cand[c]);
    if (l == 0) sh.sc[c] = sc;
  }
  __syncthreads();
  double bs = -INFINITY;
  int bv = 0x7fffffff;
  for (int c = tid; c < nc; c += kThreads) take_better(bs, bv, sh.sc[c], sh.cand[c]);
  block_argmax(bs, bv, rs, ri);
  return bv < a.V ? bv : -1;
}

// The race over a whole target row in fp64 (w = exp2(x c) up to a common factor):
// only when a residual has no mass anywhere (rounding; the verifiers then draw from p_s).
template <int DT>
__device__ __forceinline__ int full_row_race(const Args& a, const char* row, uint32_t b, double c, double* rs, int* ri) {
  double bs = -INFINITY;
  int bv = 0x7fffffff;
  for (int v0 = 4 * threadIdx.x; v0 < a.V; v0 += 4 * kThreads) {
    const uint4 x = philox4(b, (uint32_t)(v0 >> 2), kPurposeSample, a.step, a.key0, a.key1);
    const uint32_t xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (v0 + i >= a.V) break;
      const double lt = load1<DT>(row, v0 + i);
      if (lt == -INFINITY) continue;
      take_better(bs, bv, lt * c - clock_log2_f64(xs[i]), v0 + i);
    }
  }
  block_argmax(bs, bv, rs, ri);
  return bv < a.V ? bv : 0;
}

struct FinalLds {
  RaceLds rl;
  double rs[kWaves];
  int ri[kWaves];
  double s_R[kMaxK], s_h[kMaxK + 1];
};

// Finalize of stream b.  Every thread of the workgroup calls it.
template <int DT, int KS>
// err: the fused launch's error word (set when a grid-wide wait gave up), or null: when
// set, the stream's outputs are marked invalid (accepted length -1, tokens -1).
__device__ __forceinline__ void finalize_body(const Args& a, int b, FinalLds& L, const float* tT = nullptr,
                                              const int32_t* err = nullptr) {
  RaceLds& rl = L.rl;
  double* rs = L.rs;
  int* ri = L.ri;
  double *s_R = L.s_R, *s_h = L.s_h;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int k1 = a.k + 1;
  const int NG = a.NG;
  const int ND = a.B * a.k;
  const int4 info = ld_c(reinterpret_cast<const int4*>(a.ws.info + 4 * b));
  const int2 info2 = ld_c(reinterpret_cast<const int2*>(a.ws.info2 + 4 * b));
  const bool failed = err != nullptr && ld_c(err) != 0;
  const int gamma = info.x, f = info.z;
  int stop = info.y;
  const uint32_t mask = ld_c(&a.ws.rowmask[b]);
  const float Tf = tT != nullptr ? tT[b] : stream_temp(a, b);
  if (Tf == 0.f || failed) {   // greedy: the scan decided the stop and the token
    if (tid <= a.k) {
      const int s = failed ? -1 : stop;
      a.out_tokens[b * k1 + tid] = failed ? -1 : (tid < s ? a.tokens[b * a.k + tid] : (tid == s ? info.w : -1));
      if (a.diag != nullptr) {
        double* dg = a.diag + ((size_t)b * k1 + tid) * 5;
        for (int e = 0; e < 5; ++e) dg[e] = NAN;
      }
    }
    if (tid == 0) a.accepted_len[b] = failed ? -1 : stop;
    return;
  }
  const double T = (double)Tf;
  const double c = kLog2e / T;
  const size_t esz = DT == kBF16 ? 2 : 4;
  if (tid <= kMaxK) s_h[tid] = NAN;
  if (tid < kMaxK) s_R[tid] = NAN;
  __syncthreads();

  // residual masses R_i of the candidate rows above f, one wave per row
  if (a.method == 1 && stop < 0) {
    int ci = 0;
    for (int i = f + 1; i < gamma; ++i) {
      if (!((mask >> i) & 1u)) continue;
      if ((ci & (kWaves - 1)) == w) {
        const int dr = b * a.k + i;
        // 8 loads in flight per lane (clamped index, masked after); each lane still
        // adds its groups l, l + 64, ... in increasing order
        double v = 0.0;
        for (int g0 = 0; g0 < NG; g0 += 64 * kLoadsInFlight) {
          float x[kLoadsInFlight];
#pragma unroll
          for (int u = 0; u < kLoadsInFlight; ++u)
            x[u] = ld_c(&a.ws.wgrp[(size_t)min(g0 + l + 64 * u, NG - 1) * ND + dr]);
#pragma unroll
          for (int u = 0; u < kLoadsInFlight; ++u)
            if (g0 + l + 64 * u < NG) v += (double)x[u];
        }
        v = wave_sum(v);
        if (l == 0) {
          s_R[i] = v;
          s_h[i] = v / (v - expm1(ld_c(&a.ws.logP[b * k1 + i])));
        }
      }
      ++ci;
    }
    __syncthreads();
    // tau: the highest i whose test passes; rows outside the mask cannot pass (u > P_i >= h_i)
    stop = f;
    for (int i = gamma - 1; i > f; --i) {
      if (!((mask >> i) & 1u)) continue;
      if (accept_uniform(a.key0, a.key1, (uint32_t)b, (uint32_t)(i - 1), a.step) <= s_h[i]) { stop = i; break; }
    }
  }
  const int s = stop;
  const int tr = b * k1 + s;
  const int dr = b * a.k + (s < gamma ? s : 0);
  const bool resid = s < gamma;
  // the sampled row's place in the pass-2 list
  const int it = min(max(resid ? info2.x + __popc(mask & ((1u << s) - 1u)) : info2.y, 0), ND - 1);
  const char* trow = reinterpret_cast<const char*>(a.target) + (size_t)tr * a.V * esz;
  const char* drow = reinterpret_cast<const char*>(a.draft) + (size_t)dr * a.V * esz;
  int Y;
  if (resid) {
    // w(v) = max(0, P_s p_s(v) - q_s(v)) in fp64 from the exact logits, the fp64 row
    // normalisers and the fp64 Markov bias at v
    const double Mt = (double)ld_c(&a.ws.tm[tr]), tl2s = ld_c(&a.ws.tl2s[tr]);
    const double Md = (double)ld_c(&a.ws.dm[dr]), dl2s = ld_c(&a.ws.dl2s[dr]);
    const double lpP = a.method == 1 ? ld_c(&a.ws.logP[tr]) * kLog2e : 0.0;
    const int prev = a.W1 != nullptr ? draft_prev(a, b, s) : -1;
    Y = race_pick(a, it, ND, rl, rs, ri, [&](int v) {
      const double bias = a.W1 != nullptr ? bias_f64_wave(a, prev, v) : 0.0;
      const double lt = load1<DT>(trow, v), ld = load1<DT>(drow, v);
      const double pv = exp2((lt - Mt) * c - tl2s + lpP);
      const double qv = exp2((ld + bias - Md) * c - dl2s);
      const double wv = pv - qv;
      const uint32_t x = stream_word(a.key0, a.key1, (uint32_t)b, (uint32_t)v, kPurposeSample, a.step);
      return wv > 0.0 ? log2(wv) - clock_log2_f64(x) : -INFINITY;
    });
    if (Y < 0) Y = full_row_race<DT>(a, trow, (uint32_t)b, c, rs, ri);   // no residual mass: draw from p_s
  } else {
    Y = race_pick(a, it, ND, rl, rs, ri, [&](int v) {
      const double lt = load1<DT>(trow, v);
      const uint32_t x = stream_word(a.key0, a.key1, (uint32_t)b, (uint32_t)v, kPurposeSample, a.step);
      return lt != -INFINITY ? lt * c - clock_log2_f64(x) : -INFINITY;
    });
    if (Y < 0) Y = full_row_race<DT>(a, trow, (uint32_t)b, c, rs, ri);
  }

  // outputs
  if (tid <= a.k) {
    int o = -1;
    if (tid < s) o = a.tokens[b * a.k + tid];
    else if (tid == s) o = Y;
    a.out_tokens[b * k1 + tid] = o;
    if (a.diag != nullptr) {
      double* dg = a.diag + ((size_t)b * k1 + tid) * 5;
      const bool slot = tid < gamma;
      const double lP = tid <= gamma ? ld_c(&a.ws.logP[b * k1 + tid]) : 0.0;
      dg[0] = slot ? ld_c(&a.ws.lpx[b * a.k + tid]) : NAN;
      dg[1] = slot ? ld_c(&a.ws.lqx[b * a.k + tid]) : NAN;
      dg[2] = tid <= gamma ? exp(lP) : NAN;
      dg[3] = (a.method == 1 && tid < kMaxK) ? s_R[tid] : NAN;
      double h = (a.method == 1 && tid <= kMaxK) ? s_h[tid] : NAN;
      if (a.method == 1 && tid == gamma && gamma >= 1) h = exp(lP);
      if (a.method == 1 && tid >= 1 && tid < gamma && lP == 0.0) h = 1.0;
      dg[4] = h;
    }
  }
  if (tid == 0) a.accepted_len[b] = s;
}

template <int DT, int KS>
__global__ __launch_bounds__(kThreads) void finalize_kernel(Args a) {
  __shared__ FinalLds L;
  finalize_body<DT, KS>(a, blockIdx.x, L);
}

// ---------------------------------------------------------------------------
// The fused verify launch: pass 1, scan, pass 2 and finalize as phases of one
// launch of G >= NG workgroups, all resident at once (the host checks occupancy):
//   phase 1  pass 1 for group g (g < NG); the workgroup keeps its W2 slab
//   phase 2  the scan of streams g, g + G, ... (workgroups g < B, which load their
//            slab again afterwards: the scan needs the registers); the race clocks
//            of every sampled stream, by the workgroups without a stream
//   phase 3  pass 2 for group g, on the slab still in registers (W2 is read once
//            but for the scanning workgroups' slabs)
//   phase 4  finalize of streams g, g + G, ...
// with a grid barrier between phases.  Data one phase leaves for another goes
// through agent-coherent accesses (ld_c / st_c), so the barrier needs no cache
// maintenance: each wave waits for its own memory operations, workgroup g then
// writes its arrival word, workgroup 0 waits for all of them and writes the go word
// (its copies: workgroup g waits on copy g % kGoCopies).
// A wait gives up after ~0.2 s (s_memrealtime counts at 100 MHz), sets the error
// word and goes on; finalize then marks its streams' outputs invalid (accepted
// length -1).  That can only happen if the workgroups are not all resident (for
// example another kernel on the device holding compute units), never as part of a
// normal call.
// ---------------------------------------------------------------------------
constexpr uint64_t kBarrierTicks = 20000000ull;

__device__ __forceinline__ void spin_until_ge(int* p, int v, int* err) {
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  while (ld_c(p) < v) {
    if (__builtin_amdgcn_s_memrealtime() - t0 > kBarrierTicks) {
      st_c(err, 1);
      break;
    }
  }
}

// A workgroup announces that its part of a phase is done (grid_arrive), may do work
// that depends on no other workgroup, then waits until every workgroup has announced
// (grid_wait).  Announcing is an atomic increment of one of kGridSubs counters of the
// phase's parity (workgroup g: counter g % kGridSubs, each on its own line, so that
// no one address serialises the whole grid's increments); the increment that
// completes a counter's count increments the parity's top counter, and the one that
// completes the top count writes the go words, so no workgroup polls the others.
// Every workgroup announces every phase once and none can announce phase p + 2
// before all have announced p, so after phase p = 2j + 1 or 2j + 2 a counter holds
// (j + 1) times its workgroup count.  A later announcement by any workgroup begins by
// waiting for its own stores, so the go words of phase p have landed before those of
// p + 1 are written.
__device__ __forceinline__ void grid_arrive(const Args& a, int phase) {
  wait_memory();
  __syncthreads();
  if (threadIdx.x == 0) {
    int* sync = a.ws.sync;
    const int G = (int)gridDim.x, g = (int)blockIdx.x, rounds = (phase + 1) >> 1;
    const int nsub = G < kGridSubs ? G : kGridSubs, sub = g % kGridSubs;
    int* base = sync + kSyncStride * (1 + (phase & 1) * (kGridSubs + 1));
    const int members = (G - sub + kGridSubs - 1) / kGridSubs;
    if (claim_add(base + kSyncStride * sub) == members * rounds - 1 &&
        claim_add(base + kSyncStride * kGridSubs) == nsub * rounds - 1)
      for (int c = 0; c < kGoCopies; ++c) st_c(&sync[kGoBase + kGoStride * c], phase);
  }
}

__device__ __forceinline__ void grid_wait(const Args& a, int phase) {
  int* sync = a.ws.sync;
  if (threadIdx.x == 0) spin_until_ge(&sync[kGoBase + kGoStride * (blockIdx.x % kGoCopies)], phase, &sync[1]);
  __syncthreads();
}

__device__ __forceinline__ void grid_barrier(const Args& a, int phase) {
  grid_arrive(a, phase);
  grid_wait(a, phase);
}

template <int KS, bool MARKOV>
__host__ __device__ constexpr size_t fused_lds_bytes() {
  size_t m = sizeof(Pass1Lds<KS, MARKOV>);
  m = m > sizeof(ScanPhaseLds) ? m : sizeof(ScanPhaseLds);
  m = m > sizeof(Pass2Lds) ? m : sizeof(Pass2Lds);
  m = m > sizeof(FinalLds) ? m : sizeof(FinalLds);
  return (m + 15) / 16 * 16;
}

template <int DT, int KS, bool MARKOV, bool VEC>
__global__ __launch_bounds__(kThreads, 2) void verify_fused_kernel(Args a) {
  extern __shared__ __align__(16) char table[];   // pass 1's stream table
  __shared__ __align__(16) char lds[fused_lds_bytes<KS, MARKOV>()];
  const int g = blockIdx.x, G = gridDim.x;
  bf16x8 A[4][KS];
  if (g < a.NG) pass1_body<DT, KS, MARKOV, VEC>(a, g, a.NG, *reinterpret_cast<Pass1Lds<KS, MARKOV>*>(lds), table, A);
  grid_barrier(a, 1);
  const bool has_table = g < a.NG;   // pass 1 built the stream table in this workgroup's LDS
  // workgroups without a stream to scan compute the race clocks meanwhile; when every
  // workgroup scans, each takes its share of the clocks after its streams
  const int nscan = a.B < G ? a.B : G;
  const bool spare = G > nscan;
  if (g < a.B) {
    // a workgroup with streams to scan gives its slab's registers to the scan and loads
    // the slab again afterwards (at B = 64 of 505 groups: 8 MB of W2), while it waits for
    // the others; the others keep theirs through phase 2
    for (int b = g; b < a.B; b += G) {
      scan_body<DT>(a, b, *reinterpret_cast<ScanPhaseLds*>(lds), has_table ? stream_table_T(a, table) : nullptr,
                    has_table ? stream_table_gam(a, table) : nullptr);
      __syncthreads();
    }
    if (!spare) clock_rows(a, g, G);
    grid_arrive(a, 2);
    if (MARKOV) {   // A is defined on every path here, so the old slab is dead during the scan
      if (g < a.NG) {
        const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
        load_w2_slab<KS, VEC>(a, g * kGroup + w * kWaveCols, l & 15, l >> 4, A);
      } else {
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
          for (int kk = 0; kk < KS; ++kk) A[s4][kk] = zero_bf16x8();
      }
    }
    grid_wait(a, 2);
  } else {
    clock_rows(a, g - nscan, G - nscan);
    grid_barrier(a, 2);
  }
  if (g < a.NG) pass2_body<DT, KS, MARKOV, VEC>(a, g, *reinterpret_cast<Pass2Lds*>(lds), A, true);
  grid_barrier(a, 3);
  for (int b = g; b < a.B; b += G) {
    finalize_body<DT, KS>(a, b, *reinterpret_cast<FinalLds*>(lds), has_table ? stream_table_T(a, table) : nullptr,
                          &a.ws.sync[1]);
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// The drafter's Markov walk [P2 §6 "Why the Markov Head Helps"; P1 §3 "The Markov
// fix-up", Figure 2]: x_j ~ softmax((d_j + W1[x_{j-1}] . W2) / T), x_{-1} = anchor,
// drawn by the exponential race over every id with the clocks of purpose 16 + j.
// Slot j needs x_{j-1}, so a slot has two parts: the group partials and race
// candidates of every stream's biased logits (one workgroup per 256-id group, MFMA
// as in pass 1's draft rows), then one workgroup per stream that draws x_j (every
// candidate near the best one scored again in fp64).  One resident launch runs all k
// slots, with grid-wide waits between the parts, and every workgroup keeps its
// group's W2 columns in registers throughout, so a walk reads W2 once; when the
// workgroups cannot all be resident, the walk takes two launches per slot.
// ---------------------------------------------------------------------------
// threadIdx.x through an empty asm: values derived from it are computed where they are
// used instead of being kept live (and spilled) across the walk's slot loop.
constexpr int kWalkRows = 64;                      // streams per block of the partial part
constexpr int kWalkChunks = kWalkRows / kChunk;    // MFMA chunks per block
static_assert(kThreads == 4 * kWalkRows, "a block's candidates are merged by one quad of threads per row");

template <int KS, bool MARKOV>
struct WalkRowsLds {
  float2 part[kWalkRows][kWaves];
  int prev[kWalkRows];
  float c[kWalkRows];
  uint4 w1s[MARKOV ? kWalkRows * (4 * KS + 1) : 1];   // W1 rows, padded stride
};

// The race clocks of one block of rows, each thread's own: [cc][i][t] holds the int16
// log2 clocks (units of 2^-10, two to a word) of the ids c0 + 4i .. c0 + 4i + 3 that
// thread t covers in chunk cc.
typedef uint2 WalkClocks[kWalkChunks][4][kThreads];

// A thread's 16-id window in its group: ids c0 .. c0 + 15 (VEC: clamped inside the row,
// its first `shift` ids belonging to the previous lane; rag: the wave's columns pass V).
struct WalkLane {
  int c0, shift;
  bool rag;
};
template <bool VEC>
__device__ __forceinline__ WalkLane walk_lane(const Args& a, int g) {
  const int tid = opaque_tid(), w = tid >> 6, q = (tid & 63) >> 4;
  const int cb = g * kGroup + w * kWaveCols;
  const int cw = cb + 16 * q;
  WalkLane r;
  r.c0 = VEC ? min(cw, a.V - 16) : cw;
  r.shift = VEC ? (cw >= a.V ? 16 : cw - r.c0) : 0;
  r.rag = VEC && cb + kWaveCols > a.V;
  return r;
}

// The slot-j draft logits of rows r0 .. r0 + 63 at this thread's window (rows past B
// clamped to the last stream, their results unused).
template <int DT, bool VEC>
__device__ __forceinline__ void walk_load_rows(const Args& a, int j, int r0, int c0, Raw16<DT> (&xr)[kWalkChunks]) {
  const int n = opaque_tid() & 15;
  const size_t rb = (size_t)a.V * (DT == kBF16 ? 2 : 4);
  const char* base = reinterpret_cast<const char*>(a.draft);
#pragma unroll
  for (int cc = 0; cc < kWalkChunks; ++cc)
    raw_load<DT, VEC>(xr[cc], base + ((size_t)min(r0 + cc * kChunk + n, a.B - 1) * a.k + j) * rb, c0, a.V);
}

// The four clocks of one generator block, two to a word.
__device__ __forceinline__ uint2 clock_words(const uint4& x) {
  const uint32_t q0 = (uint32_t)clock_log2_q10(x.x) & 0xffffu, q1 = (uint32_t)clock_log2_q10(x.y) & 0xffffu;
  const uint32_t q2 = (uint32_t)clock_log2_q10(x.z) & 0xffffu, q3 = (uint32_t)clock_log2_q10(x.w) & 0xffffu;
  return make_uint2(q0 | (q1 << 16), q2 | (q3 << 16));
}

// The slot-j clocks of rows r0 .. r0 + 63 at this thread's window: they depend on
// nothing the walk draws, so a resident walk computes them while it waits.
__device__ __forceinline__ void walk_fill_clocks(const Args& a, int j, int r0, int c0, WalkClocks& clk) {
  const int tid = opaque_tid(), n = tid & 15;
  asm volatile("" : "+v"(c0));   // computed here, not kept from the kernel's start
#pragma unroll 1
  for (int cc = 0; cc < kWalkChunks; ++cc) {
    const uint32_t b = (uint32_t)min(r0 + cc * kChunk + n, a.B - 1);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      clk[cc][i][tid] = clock_words(philox4(b, (uint32_t)(c0 >> 2) + i, walk_purpose(j), a.step, a.key0, a.key1));
  }
}

// Chunk cc of the first block's slot-j clocks of another workgroup's group, at the
// window thread t covers there (window start c0), into dst[i][t] (coherent stores).
__device__ __forceinline__ void walk_clock_chunk(const Args& a, int j, int cc, int c0, uint2* dst) {
  const int tid = opaque_tid(), n = tid & 15;
  asm volatile("" : "+v"(c0));
  const uint32_t b = (uint32_t)min(cc * kChunk + n, a.B - 1);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    st_c(&dst[i * kThreads + tid],
         clock_words(philox4(b, (uint32_t)(c0 >> 2) + i, walk_purpose(j), a.step, a.key0, a.key1)));
}

// A lane's best race score y c - log2 E over its 16 ids c0 .. c0 + 15 in increasing
// order (the smaller id wins ties), x = d + bias the biased logits (-inf: none), with
// that id's d (exact, from the raw logits) + bias in fp64.
struct WalkCand {
  float s;
  int32_t v;
  double y;
};
// (Scores are formed in units of 2^-10, x (1024 c) - q, and scaled back once: scaling by
// a power of two commutes with the rounding, so the result is bit for bit the same.)
template <int DT>
__device__ __forceinline__ WalkCand walk_race16(const float (&x)[16], const float (&bias)[16], const Raw16<DT>& d,
                                                const uint2 (&L)[4], float c, int c0) {
  float best = -INFINITY, bd = 0.f, bb = 0.f;
  int bv = INT_MAX;
  const float c10 = c * 1024.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const uint32_t word = (e & 2) ? L[e >> 2].y : L[e >> 2].x;
    const int q = (e & 1) ? ((int32_t)word >> 16) : ((int32_t)(word << 16) >> 16);
    const float sc = fmaf(x[e], c10, -(float)q);
    const bool better = sc > best;
    best = better ? sc : best;
    bv = better ? c0 + e : bv;
    bd = better ? raw_elem<DT>(d, e) : bd;
    bb = better ? bias[e] : bb;
  }
  return WalkCand{best * 0x1.0p-10f, best > -INFINITY ? bv : INT_MAX, (double)bd + (double)bb};
}

__device__ __forceinline__ WalkTop2 wtop2_empty() { return WalkTop2{-INFINITY, INT_MAX, -INFINITY, INT_MAX, 0.0, 0.0}; }
// As top2_add, carrying each candidate's y.
__device__ __forceinline__ void wtop2_add(WalkTop2& a, float s, int v, double y) {
  const bool b1 = top_better(s, v, a.s1, a.v1);
  const bool b2 = top_better(s, v, a.s2, a.v2);
  const float s2 = b1 ? a.s1 : (b2 ? s : a.s2);
  const int v2 = b1 ? a.v1 : (b2 ? v : a.v2);
  const double y2 = b1 ? a.y1 : (b2 ? y : a.y2);
  a.s1 = b1 ? s : a.s1;
  a.v1 = b1 ? v : a.v1;
  a.y1 = b1 ? y : a.y1;
  a.s2 = s2;
  a.v2 = v2;
  a.y2 = y2;
}
__device__ __forceinline__ void wtop2_merge(WalkTop2& a, const WalkTop2& o) {
  wtop2_add(a, o.s1, o.v1, o.y1);
  wtop2_add(a, o.s2, o.v2, o.y2);
}
// The best two of a quad's best twos (lanes 4r .. 4r + 3: DPP xor 1, then xor 2); every
// lane of the quad ends with the same set.
template <int CTRL>
__device__ __forceinline__ WalkTop2 wtop2_dpp(const WalkTop2& t) {
  return WalkTop2{dppf<CTRL>(t.s1), dppi<CTRL>(t.v1), dppf<CTRL>(t.s2), dppi<CTRL>(t.v2), dppd<CTRL>(t.y1),
                  dppd<CTRL>(t.y2)};
}
__device__ __forceinline__ WalkTop2 walk_top2_quad(WalkTop2 t) {
  wtop2_merge(t, wtop2_dpp<0xB1>(t));
  wtop2_merge(t, wtop2_dpp<0x4E>(t));
  return t;
}

// Group partials (max, sum) and race candidates of slot j for rows r0 .. r0 + 63 of
// group g, from their draft logits xr and clocks clk; written to tpart / race [g][b].
// csrc: when not null, the clocks are first copied into clk from there (another
// workgroup computed them: coherent loads, issued with the block's other loads).
// sums: whether the partials' sums are formed (only log q needs them; the race and the
// greedy branch's maxima do not); without, a partial is (max, 1).
// Every thread of the workgroup calls it.
template <int DT, int KS, bool MARKOV, bool VEC>
__device__ __forceinline__ void walk_block(const Args& a, int g, int j, int r0, const WalkLane& wl,
                                           const Raw16<DT> (&xr)[kWalkChunks], const bf16x8 (&A)[4][KS],
                                           WalkRowsLds<KS, MARKOV>& L, WalkClocks& clk, bool sums,
                                           const uint2* csrc = nullptr) {
  const int tid = opaque_tid(), w = tid >> 6, l = tid & 63, n = l & 15, q = l >> 4;
  uint2 cw[kWalkChunks * 4];
  if (csrc != nullptr) {   // uniform
#pragma unroll
    for (int u = 0; u < kWalkChunks * 4; ++u) cw[u] = ld_c(&csrc[u * kThreads + tid]);
  }
  if (tid < kWalkRows) {
    const int b = min(r0 + tid, a.B - 1);
    // an absent input reads a stand-in word (the stream's first token slot), replaced
    const int32_t* standin = a.tokens + (size_t)b * a.k;
    const float T = *(a.temperature != nullptr ? a.temperature + b : reinterpret_cast<const float*>(standin));
    // x_{j-1} was drawn by another workgroup (of this launch, or of the previous one)
    const int pv = ld_c(j > 0 ? a.tokens + (size_t)b * a.k + j - 1 : (a.anchor != nullptr ? a.anchor + b : standin));
    const bool has = j > 0 || a.anchor != nullptr;
    L.prev[tid] = (has && pv >= 0 && pv < a.V) ? pv : -1;   // as draft_prev
    const float Tb = a.temperature != nullptr ? T : 1.f;      // as stream_temp
    L.c[tid] = Tb > 0.f ? (float)(kLog2e / (double)Tb) : 1e-30f;
  }
  if (csrc != nullptr) {
#pragma unroll
    for (int u = 0; u < kWalkChunks * 4; ++u) clk[u >> 2][u & 3][tid] = cw[u];
  }
  __syncthreads();
  if (MARKOV) {   // the block's W1 rows: whole rows per wave instruction, all in flight
    constexpr int kPer = kWalkRows * 4 * KS / kThreads;
    u32x4* d = reinterpret_cast<u32x4*>(L.w1s);
    u32x4 v[kPer];
    int pv[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int u = tid + i * kThreads, row = u / (4 * KS), piece = u % (4 * KS);
      pv[i] = L.prev[row];
      v[i] = *reinterpret_cast<const u32x4*>(a.W1 + (size_t)(pv[i] >= 0 ? pv[i] : 0) * a.R + 8 * piece);
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int u = tid + i * kThreads, row = u / (4 * KS), piece = u % (4 * KS);
      d[row * (4 * KS + 1) + piece] = pv[i] >= 0 ? v[i] : u32x4{0u, 0u, 0u, 0u};
    }
    __syncthreads();
  }
#pragma unroll
  for (int cc = 0; cc < kWalkChunks; ++cc) {
    const int rr = cc * kChunk + n;   // row within the block
    // two workgroups share a CU with the same chunks: the waves' issue priority falls
    // with each chunk done, so the one behind catches up (as in pass 2)
    if (cc == 0) __builtin_amdgcn_s_setprio(3);
    else if (cc == 1) __builtin_amdgcn_s_setprio(2);
    else if (cc == 2) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
    float x[16], bias[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) bias[e] = 0.f;
    if (MARKOV) {   // the bias alone (a zero accumulator, B operand read one k-step at a time)
      f32x4 acc[4];
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) acc[s4] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const bf16x8 bop = __builtin_bit_cast(bf16x8, L.w1s[rr * (4 * KS + 1) + 4 * kk + q]);
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4)
          acc[s4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[s4][kk], bop, acc[s4], 0, 0, 0);
      }
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
        for (int i = 0; i < 4; ++i) bias[4 * s4 + i] = acc[s4][i];
    }
    raw_to_f32<DT>(xr[cc], x);
#pragma unroll
    for (int e = 0; e < 16; ++e) x[e] += bias[e];
    if (wl.rag) mask_shift(x, wl.shift);
    const float c = L.c[rr];
    float2 pw;
    if (sums) {   // uniform
      pw = row_partial<0>(x, c);
    } else {
      float m = x[0];
#pragma unroll
      for (int e = 1; e < 16; ++e) m = fmaxf(m, x[e]);
      pw = make_float2(max4lanes(m), 1.f);
    }
    // race scores of q_j: y c - log2 E with y c = log2 of the weight on the row's scale
#pragma unroll
    for (int e = 0; e < 16; ++e) x[e] = (VEC || wl.c0 + e < a.V) ? x[e] : -INFINITY;
    uint2 ck[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) ck[i] = clk[cc][i][tid];
    // the lane's best id of the chunk goes into two of its own clock slots, read above
    // and dead from here: (score, id) and y
    const WalkCand wc = walk_race16<DT>(x, bias, xr[cc], ck, c, wl.c0);
    clk[cc][0][tid] = make_uint2(__float_as_uint(wc.s), (uint32_t)wc.v);
    clk[cc][1][tid] = make_uint2((uint32_t)__double2loint(wc.y), (uint32_t)__double2hiint(wc.y));
    if (q == 0) L.part[rr][w] = pw;
    __builtin_amdgcn_sched_barrier(0);   // one chunk's values at a time
  }
  __builtin_amdgcn_s_setprio(0);
  __syncthreads();
  {   // a row's 16 lane candidates (lanes n + 16 q of the 4 waves): 4 per thread of a quad,
      // then across the quad; the quad's first thread stores the row's best two
    const int row = tid >> 2, wv = tid & 3, cc = row >> 4, n = row & 15;
    WalkTop2 r = wtop2_empty();
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const int t = 64 * wv + 16 * qq + n;
      const uint2 sv = clk[cc][0][t], yy = clk[cc][1][t];
      wtop2_add(r, __uint_as_float(sv.x), (int)sv.y, __hiloint2double((int)yy.y, (int)yy.x));
    }
    r = walk_top2_quad(r);
    if (wv == 0 && r0 + row < a.B) st_c(&reinterpret_cast<WalkTop2*>(a.ws.race)[(size_t)g * a.B + r0 + row], r);
  }
  if (tid < kWalkRows && r0 + tid < a.B) {
    float2 p[kWaves];
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) p[ww] = L.part[tid][ww];
    st_c(&a.ws.tpart[(size_t)g * a.B + r0 + tid], combine_waves(p, L.c[tid]));
  }
  __syncthreads();
}

// ln x for x > 0 from x = f 2^e, f in [1/2, 1): (e + log2 f) ln 2 with the hardware
// log2 of f, absolute error of order 1e-7; and e^d for d <= 0 with the hardware exp2,
// relative error of order 1e-7 near 0 (2e-6 at d = -30).  The walk's normaliser of
// log q takes these in place of library fp64 calls, far inside its 1e-5 budget.
__device__ __forceinline__ double ln_split(float x) {
  int e;
  const float f = frexpf(x, &e);
  return ((double)e + (double)__builtin_amdgcn_logf(f)) * kLn2;
}
__device__ __forceinline__ double exp_neg(double d) { return (double)__builtin_amdgcn_exp2f((float)(d * kLog2e)); }

template <int KS>
struct WalkPickLds {
  GroupBiasLds<KS> gb;   // the greedy branch's group bias
  int cand[kMaxCand];
  double sc[kMaxCand];   // fp64 race scores of the candidates
  double yv[kMaxCand];   // and their biased logits
  int n;
  float best[kWaves];
  double lmax[kWaves], red[kWaves], rs[kWaves];
  int ri[kWaves];
};

// x_j of stream b from the slot's group partials and race candidates (written by other
// workgroups: coherent loads).  Sampled: the race winner, every candidate within
// kRaceWindow of the best fp32 score scored again in fp64 as y c - log2 E from the y
// its record carries and its exact clock; log q_j(x) = y_x / T - ln sum_v exp(y_v / T),
// the sum from the fp32 group partials.  Greedy (T = 0): the largest biased logit, the
// smallest id among equals.  err: the resident walk's error word, or null; once set,
// the slot's outputs are marked invalid (token -1, log q NaN).  Every thread of the
// workgroup calls it.
template <int DT, int KS>
__device__ __forceinline__ void walk_pick_body(const Args& a, int b, int j, int32_t* tokens_out, double* logq_out,
                                               WalkPickLds<KS>& L, const int32_t* err) {
  const int tid = opaque_tid(), w = tid >> 6, l = tid & 63;
  const int NG = a.NG;
  const size_t ND = (size_t)a.B;
  const WalkTop2* race = reinterpret_cast<const WalkTop2*>(a.ws.race);
  const int g0 = min(tid, NG - 1), g1 = min(tid + kThreads, NG - 1);
  // the stream's inputs and a thread's first two groups go out together: branch-free
  // addresses (a stand-in word for an absent input, replaced after)
  const int32_t* standin = a.tokens + (size_t)b * a.k;
  const int graw = *(a.num_drafts != nullptr ? a.num_drafts + b : standin);
  const float traw = *(a.temperature != nullptr ? a.temperature + b : reinterpret_cast<const float*>(standin));
  float2 p0 = ld_c(&a.ws.tpart[(size_t)g0 * ND + b]), p1 = ld_c(&a.ws.tpart[(size_t)g1 * ND + b]);
  WalkTop2 t0 = ld_c(&race[(size_t)g0 * ND + b]), t1 = ld_c(&race[(size_t)g1 * ND + b]);
  const int failed = err != nullptr ? ld_c(err) : 0;
  __builtin_amdgcn_sched_barrier(0);
  const int gamma = a.num_drafts != nullptr ? (graw < 0 ? 0 : (graw > a.k ? a.k : graw)) : a.k;
  if (j >= gamma || failed != 0) {   // uniform
    if (tid == 0) {
      st_c(&tokens_out[(size_t)b * a.k + j], -1);
      if (logq_out != nullptr) logq_out[(size_t)b * a.k + j] = NAN;
    }
    return;
  }
  if (tid >= NG) {
    p0 = make_float2(-INFINITY, 0.f);
    t0 = wtop2_empty();
  }
  if (tid + kThreads >= NG) {
    p1 = make_float2(-INFINITY, 0.f);
    t1 = wtop2_empty();
  }
  const float Tf = a.temperature != nullptr ? traw : 1.0f;
  int x;
  if (Tf == 0.f) {
    // the group with the largest maximum, then inside it the biased logits in fp64 (the
    // group's Markov bias from one cooperative pass over its W2t rows); x_{j-1} was
    // drawn by this launch or the previous one (a coherent load)
    const int praw = ld_c(j > 0 ? a.tokens + (size_t)b * a.k + j - 1 : (a.anchor != nullptr ? a.anchor + b : standin));
    const int pr = (j > 0 || a.anchor != nullptr) ? praw : -1;
    const int prev = (a.W1 != nullptr && pr >= 0 && pr < a.V) ? pr : -1;
    const size_t esz = DT == kBF16 ? 2 : 4;
    const char* drow = reinterpret_cast<const char*>(a.draft) + ((size_t)b * a.k + j) * a.V * esz;
    double best = -INFINITY;
    int gbest = 0x7fffffff;
    auto max_group = [&](int gi, float2 p) {
      if (p.x != -INFINITY && (double)p.x > best) { best = (double)p.x; gbest = gi; }
    };
    max_group(tid, p0);
    max_group(tid + kThreads, p1);
    for (int gi = tid + 2 * kThreads; gi < NG; gi += kThreads) max_group(gi, ld_c(&a.ws.tpart[(size_t)gi * ND + b]));
    block_argmax(best, gbest, L.rs, L.ri);
    const int gsel = gbest < NG ? gbest : 0;
    const int v = gsel * kGroup + tid;
    const float bias = prev >= 0 ? group_bias<KS>(a, prev, gsel, L.gb) : 0.f;
    double xv = v < a.V ? (double)load1<DT>(drow, v) + (double)bias : -INFINITY;
    int vbest = v < a.V ? v : 0x7fffffff;
    block_argmax(xv, vbest, L.rs, L.ri);
    x = vbest < a.V ? vbest : gsel * kGroup;
    if (tid == 0 && logq_out != nullptr) logq_out[(size_t)b * a.k + j] = NAN;
  } else {
    const double invT = 1.0 / (double)Tf;
    const double c = kLog2e * invT;
    const bool want = logq_out != nullptr;   // the normaliser is for log q only
    // a group's log weight for the normaliser: m_g / T + ln s_g
    auto lw = [&](float2 p) { return p.x != -INFINITY ? (double)p.x * invT + ln_split(p.y) : -INFINITY; };
    const double lw0 = want ? lw(p0) : -INFINITY, lw1 = want ? lw(p1) : -INFINITY;
    float best = fmaxf(t0.s1, t1.s1);
    double lm = fmax(lw0, lw1);
    for (int gi = tid + 2 * kThreads; gi < NG; gi += kThreads) {
      best = fmaxf(best, ld_c(&race[(size_t)gi * ND + b]).s1);
      if (want) lm = fmax(lm, lw(ld_c(&a.ws.tpart[(size_t)gi * ND + b])));
    }
    best = wave_max_dpp(best);
    if (want) lm = wave_max_f64(lm);
    if (tid == 0) L.n = 0;
    if (l == 0) {
      L.best[w] = best;
      L.lmax[w] = lm;
    }
    __syncthreads();
    best = fmaxf(fmaxf(L.best[0], L.best[1]), fmaxf(L.best[2], L.best[3]));
    lm = fmax(fmax(L.lmax[0], L.lmax[1]), fmax(L.lmax[2], L.lmax[3]));
    // candidates within the window of the best fp32 score; the normaliser's terms
    const float floor_ = best - kRaceWindow;
    auto offer = [&](float s, int v, double y) {
      if (s >= floor_ && v >= 0 && v < a.V) {
        const int k = atomicAdd(&L.n, 1);
        if (k < kMaxCand) {
          L.cand[k] = v;
          L.yv[k] = y;
        }
      }
    };
    offer(t0.s1, t0.v1, t0.y1);
    offer(t0.s2, t0.v2, t0.y2);
    offer(t1.s1, t1.v1, t1.y1);
    offer(t1.s2, t1.v2, t1.y2);
    double sum = (lw0 != -INFINITY ? exp_neg(lw0 - lm) : 0.0) + (lw1 != -INFINITY ? exp_neg(lw1 - lm) : 0.0);
    for (int gi = tid + 2 * kThreads; gi < NG; gi += kThreads) {
      const WalkTop2 t = ld_c(&race[(size_t)gi * ND + b]);
      offer(t.s1, t.v1, t.y1);
      offer(t.s2, t.v2, t.y2);
      if (want) {
        const double lg = lw(ld_c(&a.ws.tpart[(size_t)gi * ND + b]));
        if (lg != -INFINITY) sum += exp_neg(lg - lm);
      }
    }
    if (want) sum = wave_sum(sum);
    if (l == 0) L.red[w] = sum;
    __syncthreads();
    const int nc = min(L.n, kMaxCand);
    sum = (L.red[0] + L.red[1]) + (L.red[2] + L.red[3]);
    int bv = nc == 1 ? L.cand[0] : 0x7fffffff;
    // A lone candidate is the winner: every id whose exact score could reach the best
    // fp32 score's lies within the window, and so does any id of its group that ranks
    // above it.  Otherwise each candidate's exact score, one per thread.
    if (nc > 1) {   // uniform
      for (int ci = tid; ci < nc; ci += kThreads) {
        const double y = L.yv[ci];
        const uint32_t xw = stream_word(a.key0, a.key1, (uint32_t)b, (uint32_t)L.cand[ci], walk_purpose(j), a.step);
        L.sc[ci] = y != -INFINITY ? y * c - clock_log2_f64(xw) : -INFINITY;
      }
      __syncthreads();
      double bs = -INFINITY;
      for (int ci = tid; ci < nc; ci += kThreads) take_better(bs, bv, L.sc[ci], L.cand[ci]);
      block_argmax(bs, bv, L.rs, L.ri);
    }
    x = bv < a.V ? bv : 0;   // 0: a row with no finite logit (excluded by the caller's contract)
    if (tid == 0 && logq_out != nullptr) {
      double y = NAN;
      for (int ci = 0; ci < nc; ++ci)
        if (L.cand[ci] == bv) y = L.yv[ci];
      logq_out[(size_t)b * a.k + j] = y * invT - (lm + ln_split((float)sum));
    }
  }
  if (tid == 0) st_c(&tokens_out[(size_t)b * a.k + j], x);
}

// Two launches per slot: the partial part (one workgroup per group), then the draws.
template <int DT, int KS, bool MARKOV, bool VEC>
__global__ __launch_bounds__(kThreads, 2) void walk_partials_kernel(Args a, int j, bool sums) {
  __shared__ WalkRowsLds<KS, MARKOV> L;
  __shared__ WalkClocks clk;
  const int g = blockIdx.x;
  const int tid = opaque_tid();
  const WalkLane wl = walk_lane<VEC>(a, g);
  Raw16<DT> xr[kWalkChunks];
  walk_load_rows<DT, VEC>(a, j, 0, wl.c0, xr);   // before the slab: staged while it is in flight
  bf16x8 A[4][KS];
  if (MARKOV) load_w2_slab<KS, VEC>(a, g * kGroup + (tid >> 6) * kWaveCols, tid & 15, (tid & 63) >> 4, A);
  walk_fill_clocks(a, j, 0, wl.c0, clk);
  for (int r0 = 0; r0 < a.B; r0 += kWalkRows) {
    if (r0 > 0) {
      walk_load_rows<DT, VEC>(a, j, r0, wl.c0, xr);
      walk_fill_clocks(a, j, r0, wl.c0, clk);
    }
    walk_block<DT, KS, MARKOV, VEC>(a, g, j, r0, wl, xr, A, L, clk, sums);
  }
}

template <int DT, int KS>
__global__ __launch_bounds__(kThreads) void walk_pick_kernel(Args a, int j, int32_t* tokens_out, double* logq_out) {
  __shared__ WalkPickLds<KS> L;
  walk_pick_body<DT, KS>(a, blockIdx.x, j, tokens_out, logq_out, L, nullptr);
}

// The go and error words and the counter lines of a resident launch.
__global__ __launch_bounds__(kThreads) void sync_clear_kernel(int32_t* sync) {
  const int t = threadIdx.x;
  if (t < 4) st_c(&sync[t], 0);
  if (t < kGoCopies) st_c(&sync[kGoBase + kGoStride * t], 0);
  for (int i = t; i <= kGridCountLines; i += kThreads) st_c(&sync[kSyncStride * i], 0);
}

template <int KS, bool MARKOV>
__host__ __device__ constexpr size_t walk_lds_bytes() {
  const size_t m = sizeof(WalkRowsLds<KS, MARKOV>) > sizeof(WalkPickLds<KS>) ? sizeof(WalkRowsLds<KS, MARKOV>)
                                                                             : sizeof(WalkPickLds<KS>);
  return (m + 15) / 16 * 16;
}

// The whole walk in one launch of NG workgroups (all resident).  Slot j: every
// workgroup computes its group's partials and candidates (phase 2j + 1); the first
// P = min(B, NG) workgroups then wait for all of them and draw (workgroup g draws
// streams g, g + NG, ...), while the others compute the drawing workgroups' clocks
// for slot j + 1 (their first block of rows, into the clock region, one buffer per
// slot parity: a slot's buffer is written only after every reader of its previous
// contents has passed a wait) and then their own; everyone waits for the draws
// (phase 2j + 2).
template <int DT, int KS, bool MARKOV, bool VEC>
__global__ __launch_bounds__(kThreads, 2) void walk_fused_kernel(Args a, int32_t* tokens_out, double* logq_out) {
  __shared__ __align__(16) char lds[walk_lds_bytes<KS, MARKOV>()];
  __shared__ WalkClocks clk;
  auto& L = *reinterpret_cast<WalkRowsLds<KS, MARKOV>*>(lds);
  auto& P = *reinterpret_cast<WalkPickLds<KS>*>(lds);
  const int g = blockIdx.x, G = gridDim.x;
  const int tid = opaque_tid();
  const int NP = a.B < G ? a.B : G;   // drawing workgroups
  const int NO = G - NP;              // the others
  const bool picker = g < NP;
  // [2][NP][kWalkChunks][4][kThreads]: the drawing workgroups' clocks by slot parity
  uint2* const pclk = a.ws.clk;
  auto pbuf = [&](int slot, int pg) { return pclk + ((size_t)(slot & 1) * NP + pg) * kWalkChunks * 4 * kThreads; };
  const WalkLane wl = walk_lane<VEC>(a, g);
  Raw16<DT> xr[kWalkChunks];
  walk_load_rows<DT, VEC>(a, 0, 0, wl.c0, xr);
  bf16x8 A[4][KS];
  if (MARKOV) load_w2_slab<KS, VEC>(a, g * kGroup + (tid >> 6) * kWaveCols, tid & 15, (tid & 63) >> 4, A);
  walk_fill_clocks(a, 0, 0, wl.c0, clk);
  for (int j = 0; j < a.k; ++j) {
    for (int r0 = 0; r0 < a.B; r0 += kWalkRows) {
      if (r0 > 0) {
        walk_load_rows<DT, VEC>(a, j, r0, wl.c0, xr);
        walk_fill_clocks(a, j, r0, wl.c0, clk);
      }
      // the first block's clocks of a drawing workgroup were computed by the others
      walk_block<DT, KS, MARKOV, VEC>(a, g, j, r0, wl, xr, A, L, clk, logq_out != nullptr,
                                      (picker && j > 0 && NO > 0 && r0 == 0) ? pbuf(j, g) : nullptr);
    }
    const int ph1 = 2 * j + 1, ph2 = 2 * j + 2;
    const bool last = j + 1 == a.k;
    grid_arrive(a, ph1);
    if (picker) {
      grid_wait(a, ph1);
      for (int b = g; b < a.B; b += G) {
        walk_pick_body<DT, KS>(a, b, j, tokens_out, logq_out, P, &a.ws.sync[1]);
        __syncthreads();
      }
      if (!last) {
        grid_arrive(a, ph2);
        walk_load_rows<DT, VEC>(a, j + 1, 0, wl.c0, xr);
        if (NO == 0) walk_fill_clocks(a, j + 1, 0, wl.c0, clk);
        grid_wait(a, ph2);
      }
    } else if (!last) {
      // a share of the drawing workgroups' clocks (task t: workgroup t / 4, chunk t % 4)
      for (int t = g - NP; t < NP * kWalkChunks; t += NO) {
        const int pg = t / kWalkChunks, cc = t % kWalkChunks;
        walk_clock_chunk(a, j + 1, cc, walk_lane<VEC>(a, pg).c0, pbuf(j + 1, pg) + cc * 4 * kThreads);
      }
      grid_arrive(a, ph2);
      walk_load_rows<DT, VEC>(a, j + 1, 0, wl.c0, xr);
      walk_fill_clocks(a, j + 1, 0, wl.c0, clk);
      grid_wait(a, ph2);
    }
  }
}

// ---------------------------------------------------------------------------
// The generator words the sampler draws, for callers that replay or audit a call:
// kind 0, word 0 of counter (b, idx0 + i, purpose, step) (the accept uniforms' words);
// kind 1, word idx0 + i of the stream of (b, purpose, step), i.e. word v mod 4 of
// counter (b, v div 4, purpose, step) for v = idx0 + i (the race clocks' words).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void random_words_kernel(uint32_t k0, uint32_t k1, uint32_t b, uint32_t purpose,
                                                                uint32_t step, uint32_t idx0, int n, int kind,
                                                                uint32_t* out) {
  const int i = blockIdx.x * kThreads + opaque_tid();
  if (i >= n) return;
  const uint32_t idx = idx0 + (uint32_t)i;
  out[i] = kind == 0 ? philox_word0(b, idx, purpose, step, k0, k1) : stream_word(k0, k1, b, idx, purpose, step);
}

hipError_t launch_random_words(uint64_t seed, uint32_t b, uint32_t purpose, uint32_t step, uint32_t idx0, int n,
                               int kind, uint32_t* out, hipStream_t st) {
  hipLaunchKernelGGL(random_words_kernel, dim3((n + kThreads - 1) / kThreads), dim3(kThreads), 0, st,
                     (uint32_t)(seed & 0xffffffffu), (uint32_t)(seed >> 32), b, purpose, step, idx0, n, kind, out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// W2 [R, V] -> W2t [V, R]: 64 x 64 tiles through LDS, reads coalesced along v and
// writes along r.  Elements are moved as 16-bit words (bf16 bits).
// ---------------------------------------------------------------------------
constexpr int kTrTile = 64;

__global__ __launch_bounds__(kThreads) void w2_transpose_kernel(const uint16_t* __restrict__ w2, int R, int V,
                                                                 uint16_t* __restrict__ w2t) {
  __shared__ uint32_t tile[kTrTile][kTrTile + 1];   // +1: column reads spread over banks
  const int v0 = blockIdx.x * kTrTile, r0 = blockIdx.y * kTrTile;
  const int tx = opaque_tid() & 63, ty = opaque_tid() >> 6;
#pragma unroll
  for (int i = 0; i < kTrTile / kWaves; ++i) {
    const int r = r0 + ty + kWaves * i, v = v0 + tx;
    tile[ty + kWaves * i][tx] = (r < R && v < V) ? w2[(size_t)r * V + v] : 0u;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kTrTile / kWaves; ++i) {
    const int v = v0 + ty + kWaves * i, r = r0 + tx;
    if (v < V && r < R) w2t[(size_t)v * R + r] = (uint16_t)tile[tx][ty + kWaves * i];
  }
}

hipError_t launch_w2_transpose(const uint16_t* w2, int R, int V, uint16_t* w2t, hipStream_t st) {
  const dim3 grid((V + kTrTile - 1) / kTrTile, (R + kTrTile - 1) / kTrTile);
  hipLaunchKernelGGL(w2_transpose_kernel, grid, dim3(kThreads), 0, st, w2, R, V, w2t);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Reduced draft vocabulary [P1 §3 "The Markov fix-up": the drafter scores a reduced
// vocabulary and scatters its logits into target-vocabulary columns]: every other
// column is -inf, so q = 0 there and the residual keeps the target's mass.
// ---------------------------------------------------------------------------
template <int DT>
__global__ __launch_bounds__(kThreads) void fill_ninf_kernel(void* out, size_t n) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  for (size_t i = (size_t)blockIdx.x * kThreads + opaque_tid(); i < n; i += stride) {
    if (DT == kBF16) reinterpret_cast<uint16_t*>(out)[i] = 0xFF80u;   // bf16 -inf
    else reinterpret_cast<float*>(out)[i] = -INFINITY;
  }
}

template <int DT>
__global__ __launch_bounds__(kThreads) void scatter_kernel(const void* in, const int32_t* ids, int rows, int K, int V,
                                                           void* out) {
  const size_t n = (size_t)rows * K;
  const size_t stride = (size_t)gridDim.x * kThreads;
  for (size_t i = (size_t)blockIdx.x * kThreads + opaque_tid(); i < n; i += stride) {
    const int r = (int)(i / K), c = (int)(i - (size_t)r * K);
    const int v = ids[c];
    if (v < 0 || v >= V) continue;   // ids are the caller's: out-of-range ones are dropped
    if (DT == kBF16)
      reinterpret_cast<uint16_t*>(out)[(size_t)r * V + v] = reinterpret_cast<const uint16_t*>(in)[i];
    else
      reinterpret_cast<float*>(out)[(size_t)r * V + v] = reinterpret_cast<const float*>(in)[i];
  }
}

// ---------------------------------------------------------------------------
// Markov bias alone: out[i, v] = logits_in[i, v] + W1[prev_i] . W2[:, v]
// ---------------------------------------------------------------------------
template <int DT, int KS>
__global__ __launch_bounds__(kThreads) void markov_bias_kernel(BiasArgs ba) {
  Args a{};
  a.V = ba.V; a.R = ba.R; a.W1 = ba.W1; a.W2t = ba.W2t;
  const int g = blockIdx.x;
  const int tid = opaque_tid(), w = tid >> 6, l = tid & 63, n = l & 15, q = l >> 4;
  const int cb = g * kGroup + w * kWaveCols;
  const int c0 = cb + 16 * q;
  bf16x8 A[4][KS];
  load_w2_slab<KS>(a, cb, n, q, A);
  const size_t esz = DT == kBF16 ? 2 : 4;
  for (int ch = 0; ch < ba.rows; ch += kChunk) {
    const int r = ch + n;
    const bool active = r < ba.rows;
    int prev = active ? ba.prev[r] : -1;
    prev = (prev >= 0 && prev < ba.V) ? prev : -1;
    float bias[16];
    markov_tile<KS>(a, A, prev, q, bias);
    if (!active) continue;
    float x[16];
    if (ba.logits_in != nullptr) {
      load16<DT>(reinterpret_cast<const char*>(ba.logits_in) + (size_t)r * ba.V * esz, c0, ba.V, ba.vec_ok != 0, x);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = 0.f;
    }
    float* o = ba.out + (size_t)r * ba.V;
    if (ba.vec_ok && c0 + 16 <= ba.V && (ba.V % 4) == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<float4*>(o + c0 + 4 * i) =
            make_float4(x[4 * i] + bias[4 * i], x[4 * i + 1] + bias[4 * i + 1], x[4 * i + 2] + bias[4 * i + 2],
                        x[4 * i + 3] + bias[4 * i + 3]);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (c0 + i < ba.V) o[c0 + i] = x[i] + bias[i];
    }
  }
}

// ---------------------------------------------------------------------------
// Confidence head + adaptive count.  One workgroup per stream: for 4 slots at a time
// every thread takes 8 consecutive hidden features per step (2048 per step), so the
// loads of all 4 slots are in flight together; the dot products accumulate in fp64.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void adaptive_kernel(AdaptArgs aa) {
  constexpr int kSlots = 8;   // slots whose hidden states are in flight together (k <= 8: one round)
  __shared__ double s_part[kWaves][kMaxK];
  __shared__ double s_c[kMaxK];
  const int b = blockIdx.x;
  const int tid = opaque_tid(), w = tid >> 6, l = tid & 63;
  // w . h for every slot: the whole workgroup splits H, each wave sums its share in
  // fp64 and the 4 wave sums meet in LDS
  for (int j0 = 0; j0 < aa.k; j0 += kSlots) {
    double acc[kSlots];
#pragma unroll
    for (int sl = 0; sl < kSlots; ++sl) acc[sl] = 0.0;
    const uint16_t* h[kSlots];
#pragma unroll
    for (int sl = 0; sl < kSlots; ++sl) h[sl] = aa.hidden + ((size_t)b * aa.k + min(j0 + sl, aa.k - 1)) * aa.H;
    if (aa.vec_ok) {   // H % 8 == 0 and 16-byte aligned rows
      // two steps of 8 ids per thread at a time (H = 4096: all of a slot's loads at
      // once): clamped addresses, the past-the-end step masked after
      constexpr int kSteps = 2;
      for (int c00 = 8 * tid; c00 < aa.H; c00 += 8 * kThreads * kSteps) {
        uint4 wv[kSteps], hv[kSteps][kSlots];
#pragma unroll
        for (int it = 0; it < kSteps; ++it) {
          const int cc = min(c00 + 8 * kThreads * it, aa.H - 8);
          wv[it] = *reinterpret_cast<const uint4*>(aa.w + cc);
#pragma unroll
          for (int sl = 0; sl < kSlots; ++sl) hv[it][sl] = *reinterpret_cast<const uint4*>(h[sl] + cc);
        }
        __builtin_amdgcn_sched_barrier(0);   // every load above goes out before any use
#pragma unroll
        for (int it = 0; it < kSteps; ++it) {
          if (c00 + 8 * kThreads * it >= aa.H) continue;
          const uint32_t ww[4] = {wv[it].x, wv[it].y, wv[it].z, wv[it].w};
#pragma unroll
          for (int sl = 0; sl < kSlots; ++sl) {
            const uint32_t hh[4] = {hv[it][sl].x, hv[it][sl].y, hv[it][sl].z, hv[it][sl].w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
              acc[sl] += (double)bf16lo(hh[i]) * (double)bf16lo(ww[i]) + (double)bf16hi(hh[i]) * (double)bf16hi(ww[i]);
          }
        }
      }
    } else {
      for (int c = tid; c < aa.H; c += kThreads) {
        const double wc = (double)bf16_to_f32(aa.w[c]);
#pragma unroll
        for (int sl = 0; sl < kSlots; ++sl) acc[sl] += (double)bf16_to_f32(h[sl][c]) * wc;
      }
    }
#pragma unroll
    for (int sl = 0; sl < kSlots; ++sl) acc[sl] = wave_sum(acc[sl]);
    if (l == 0)
#pragma unroll
      for (int sl = 0; sl < kSlots; ++sl)
        if (j0 + sl < aa.k) s_part[w][j0 + sl] = acc[sl];
  }
  __syncthreads();
  if (tid < aa.k) {
    const double z = (s_part[0][tid] + s_part[1][tid]) + (s_part[2][tid] + s_part[3][tid]);
    const double cj = 1.0 / (1.0 + exp(-(z + (double)aa.bias)));
    s_c[tid] = cj;
    if (aa.c_out) aa.c_out[b * aa.k + tid] = (float)cj;
  }
  __syncthreads();
  if (tid == 0) {
    double surv = 1.0, expected = 1.0;
    double best = 1.0 / (double)aa.ms[1];
    int nbest = 0;
    for (int j = 0; j < aa.k; ++j) {
      surv *= s_c[j];
      expected += surv;                      // 1 + sum_{i<=j} a_i = E(n = j + 1)
      if (aa.a_out) aa.a_out[b * aa.k + j] = (float)surv;
      const double ratio = expected / (double)aa.ms[j + 2];
      if (ratio > best) { best = ratio; nbest = j + 1; }
    }
    aa.n_out[b] = nbest;
  }
}

// ---------------------------------------------------------------------------
// launch wrappers (host side of this translation unit)
// ---------------------------------------------------------------------------
// Workgroups of the fused launch for this problem on the current device, or 0 when
// they could not all be resident at once (then the call uses separate launches).
// The resident count per CU comes from the runtime's occupancy calculator and is
// cached per device for each kernel instance.  DSPARK_VERIFY_LAUNCH=separate in the
// environment forces separate launches.
template <int DT, int KS, bool MARKOV, bool VEC>
static int fused_grid_for(const Args& a) {
  const char* env = getenv("DSPARK_VERIFY_LAUNCH");
  if (env != nullptr && strcmp(env, "separate") == 0) return 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  static int cus[64], occ[64][2];   // occ[dev][0]: table bytes it was computed for (+1)
  static std::mutex mu;
  const size_t table = stream_table_bytes(a.B);
  int resident;
  {
    std::lock_guard<std::mutex> lock(mu);
    if (cus[dev] == 0 && hipDeviceGetAttribute(&cus[dev], hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    if (occ[dev][0] != (int)table + 1) {
      int o = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, verify_fused_kernel<DT, KS, MARKOV, VEC>, kThreads,
                                                       table) != hipSuccess)
        return 0;
      occ[dev][0] = (int)table + 1;
      occ[dev][1] = o;
    }
    resident = occ[dev][1] * cus[dev];
  }
  if (a.NG > resident) return 0;
  const int G = a.NG > a.B ? a.NG : (a.B < resident ? a.B : resident);
  return G <= kMaxFusedGrid ? G : 0;
}

template <int DT, int KS, bool MARKOV, bool VEC>
static hipError_t launch_passes(const Args& a0, hipStream_t st, void* const* ev) {
  auto mark = [&](int i) {
    if (ev != nullptr && ev[i] != nullptr) (void)hipEventRecord(reinterpret_cast<hipEvent_t>(ev[i]), st);
  };
  Args a = a0;
  a.fused_grid = 0;
  if constexpr (VEC) a.fused_grid = fused_grid_for<DT, KS, MARKOV, VEC>(a);   // aligned rows only
  const int nchd = (a.B * a.k + kChunk - 1) / kChunk;
  mark(0);
  hipLaunchKernelGGL(pack_kernel, dim3(nchd), dim3(64), 0, st, a);
  mark(1);
  if constexpr (VEC) {
    if (a.fused_grid > 0) {   // the four other stages in one launch: their events coincide
      hipLaunchKernelGGL((verify_fused_kernel<DT, KS, MARKOV, VEC>), dim3(a.fused_grid), dim3(kThreads),
                         stream_table_bytes(a.B), st, a);
      for (int i = 2; i <= 5; ++i) mark(i);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((pass1_kernel<DT, KS, MARKOV, VEC>), dim3(a.NG), dim3(kThreads), stream_table_bytes(a.B), st, a);
  mark(2);
  hipLaunchKernelGGL((scan_kernel<DT>), dim3(a.B + a.NG), dim3(kThreads), 0, st, a);
  mark(3);
  hipLaunchKernelGGL((pass2_kernel<DT, KS, MARKOV, VEC>), dim3(a.NG), dim3(kThreads), 0, st, a);
  mark(4);
  hipLaunchKernelGGL((finalize_kernel<DT, KS>), dim3(a.B), dim3(kThreads), 0, st, a);
  mark(5);
  return hipGetLastError();
}

template <int DT, bool VEC>
static hipError_t launch_vec(const Args& a, hipStream_t st, void* const* ev) {
  if (a.W1 == nullptr) return launch_passes<DT, 1, false, VEC>(a, st, ev);
  switch (a.R) {
    case 32: return launch_passes<DT, 1, true, VEC>(a, st, ev);
    case 64: return launch_passes<DT, 2, true, VEC>(a, st, ev);
    case 128: return launch_passes<DT, 4, true, VEC>(a, st, ev);
    default: return launch_passes<DT, 8, true, VEC>(a, st, ev);
  }
}

template <int DT>
static hipError_t launch_dt(const Args& a, hipStream_t st, void* const* ev) {
  return (a.vec_ok && a.V >= 16) ? launch_vec<DT, true>(a, st, ev) : launch_vec<DT, false>(a, st, ev);
}

template <int DT>
static int fused_grid_dt(const Args& a) {
  if (!(a.vec_ok && a.V >= 16)) return 0;
  if (a.W1 == nullptr) return fused_grid_for<DT, 1, false, true>(a);
  switch (a.R) {
    case 32: return fused_grid_for<DT, 1, true, true>(a);
    case 64: return fused_grid_for<DT, 2, true, true>(a);
    case 128: return fused_grid_for<DT, 4, true, true>(a);
    default: return fused_grid_for<DT, 8, true, true>(a);
  }
}

int verify_fused_grid(const Args& a) { return a.dtype == kBF16 ? fused_grid_dt<kBF16>(a) : fused_grid_dt<kF32>(a); }

hipError_t launch_verify(const Args& a, hipStream_t st, void* const* ev) {
  return a.dtype == kBF16 ? launch_dt<kBF16>(a, st, ev) : launch_dt<kF32>(a, st, ev);
}

// Workgroups of the resident walk (NG) when they can all be resident on the current
// device, else 0 (two launches per slot).  DSPARK_WALK_LAUNCH=separate in the
// environment forces the two launches per slot.
template <int DT, int KS, bool MARKOV, bool VEC>
static int walk_grid_for(const Args& a) {
  const char* env = getenv("DSPARK_WALK_LAUNCH");
  if (env != nullptr && strcmp(env, "separate") == 0) return 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  static int cus[64], occ[64];   // occ: resident workgroups per CU, + 1 once computed
  static std::mutex mu;
  int resident;
  {
    std::lock_guard<std::mutex> lock(mu);
    if (cus[dev] == 0 && hipDeviceGetAttribute(&cus[dev], hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    if (occ[dev] == 0) {
      int o = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, walk_fused_kernel<DT, KS, MARKOV, VEC>, kThreads, 0) !=
          hipSuccess)
        return 0;
      occ[dev] = o + 1;
    }
    resident = (occ[dev] - 1) * cus[dev];
  }
  return (a.NG <= resident && a.NG <= kMaxFusedGrid) ? a.NG : 0;
}

template <int DT, int KS, bool MARKOV, bool VEC>
static hipError_t launch_walk_t(const Args& a, int32_t* tokens_out, double* logq_out, hipStream_t st, int* launches) {
  const int G = walk_grid_for<DT, KS, MARKOV, VEC>(a);
  if (launches != nullptr) {   // the plan only
    *launches = G > 0 ? 2 : 2 * a.k;
    return hipSuccess;
  }
  if (G > 0) {
    // the resident walk writes its wait words and, when some workgroups draw nothing,
    // the drawing workgroups' clocks
    if (a.ws.sync == nullptr || a.ws.clk == nullptr || a.ws.tpart == nullptr || a.ws.race == nullptr)
      return hipErrorInvalidValue;
    hipLaunchKernelGGL(sync_clear_kernel, dim3(1), dim3(kThreads), 0, st, a.ws.sync);
    hipLaunchKernelGGL((walk_fused_kernel<DT, KS, MARKOV, VEC>), dim3(G), dim3(kThreads), 0, st, a, tokens_out,
                       logq_out);
    return hipGetLastError();
  }
  if (a.ws.tpart == nullptr || a.ws.race == nullptr) return hipErrorInvalidValue;
  for (int j = 0; j < a.k; ++j) {
    hipLaunchKernelGGL((walk_partials_kernel<DT, KS, MARKOV, VEC>), dim3(a.NG), dim3(kThreads), 0, st, a, j,
                       logq_out != nullptr);
    hipLaunchKernelGGL((walk_pick_kernel<DT, KS>), dim3(a.B), dim3(kThreads), 0, st, a, j, tokens_out, logq_out);
  }
  return hipGetLastError();
}

template <int DT, bool VEC>
static hipError_t launch_walk_vec(const Args& a, int32_t* t, double* lq, hipStream_t st, int* n) {
  if (a.W1 == nullptr) return launch_walk_t<DT, 1, false, VEC>(a, t, lq, st, n);
  switch (a.R) {
    case 32: return launch_walk_t<DT, 1, true, VEC>(a, t, lq, st, n);
    case 64: return launch_walk_t<DT, 2, true, VEC>(a, t, lq, st, n);
    case 128: return launch_walk_t<DT, 4, true, VEC>(a, t, lq, st, n);
    default: return launch_walk_t<DT, 8, true, VEC>(a, t, lq, st, n);
  }
}

template <int DT>
static hipError_t launch_walk_dt(const Args& a, int32_t* t, double* lq, hipStream_t st, int* n) {
  return (a.vec_ok && a.V >= 16) ? launch_walk_vec<DT, true>(a, t, lq, st, n)
                                 : launch_walk_vec<DT, false>(a, t, lq, st, n);
}

hipError_t launch_walk(const Args& a, int32_t* tokens_out, double* logq_out, hipStream_t st) {
  return a.dtype == kBF16 ? launch_walk_dt<kBF16>(a, tokens_out, logq_out, st, nullptr)
                          : launch_walk_dt<kF32>(a, tokens_out, logq_out, st, nullptr);
}

int walk_launches(const Args& a) {
  int n = 0;
  const hipError_t e = a.dtype == kBF16 ? launch_walk_dt<kBF16>(a, nullptr, nullptr, nullptr, &n)
                                        : launch_walk_dt<kF32>(a, nullptr, nullptr, nullptr, &n);
  return e == hipSuccess ? n : 0;
}

size_t verify_lds_bytes(int B) { return stream_table_bytes(B); }

template <int DT>
static hipError_t launch_bias_dt(const BiasArgs& ba, int NG, hipStream_t st) {
  switch (ba.R) {
    case 32: hipLaunchKernelGGL((markov_bias_kernel<DT, 1>), dim3(NG), dim3(kThreads), 0, st, ba); break;
    case 64: hipLaunchKernelGGL((markov_bias_kernel<DT, 2>), dim3(NG), dim3(kThreads), 0, st, ba); break;
    case 128: hipLaunchKernelGGL((markov_bias_kernel<DT, 4>), dim3(NG), dim3(kThreads), 0, st, ba); break;
    default: hipLaunchKernelGGL((markov_bias_kernel<DT, 8>), dim3(NG), dim3(kThreads), 0, st, ba); break;
  }
  return hipGetLastError();
}

hipError_t launch_markov_bias(const BiasArgs& ba, int NG, hipStream_t st) {
  return ba.dtype == kBF16 ? launch_bias_dt<kBF16>(ba, NG, st) : launch_bias_dt<kF32>(ba, NG, st);
}

hipError_t launch_scatter(const void* in, const int32_t* ids, int rows, int K, int V, int dtype, void* out,
                          hipStream_t st) {
  const size_t n_out = (size_t)rows * V, n_in = (size_t)rows * K;
  auto grid = [](size_t n) { const size_t g = (n + kThreads - 1) / kThreads; return (int)(g < 4096 ? g : 4096); };
  const int g1 = grid(n_out), g2 = grid(n_in);
  if (dtype == kBF16) {
    hipLaunchKernelGGL(fill_ninf_kernel<kBF16>, dim3(g1), dim3(kThreads), 0, st, out, n_out);
    hipLaunchKernelGGL(scatter_kernel<kBF16>, dim3(g2), dim3(kThreads), 0, st, in, ids, rows, K, V, out);
  } else {
    hipLaunchKernelGGL(fill_ninf_kernel<kF32>, dim3(g1), dim3(kThreads), 0, st, out, n_out);
    hipLaunchKernelGGL(scatter_kernel<kF32>, dim3(g2), dim3(kThreads), 0, st, in, ids, rows, K, V, out);
  }
  return hipGetLastError();
}

hipError_t launch_adaptive(const AdaptArgs& aa, hipStream_t st) {
  hipLaunchKernelGGL(adaptive_kernel, dim3(aa.B), dim3(kThreads), 0, st, aa);
  return hipGetLastError();
}

}  // namespace dspark
