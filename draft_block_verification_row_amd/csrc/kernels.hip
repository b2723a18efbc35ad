// gfx950 kernels of the DSpark verify sampler.
//
// Sources (page titles): [P1] "MTP, DSpark and Block Verification, Explained";
// [P2] "MTP Heads and Confidence Heads"; [P3] "Teaching the Speculator What a Draft Costs".
//
// A call is four launches on one stream:
//   pass1     one workgroup per 256-id vocabulary group g; every target row
//             (slots 0..gamma_b) and every draft row (slots 0..gamma_b-1) gets a
//             partial (max, sum 2^((l - max) log2e / T)) over the group.  Draft rows
//             get the Markov bias W1[prev] . W2 from MFMA tiles held in registers:
//             the wave keeps its 64 columns of W2 as the A operand for the whole
//             launch and streams draft rows through the B operand [P2 §6; P1 §3].
//   scan      one workgroup per stream: row normalisers from the partials (fp64),
//             log p_j(x_j), log q_j(x_j) (gathered bias in fp64), the token-wise stop
//             and the clipped prefix P_i [P1 §4], and the rows whose residual mass
//             is needed.  Block verification needs R_i only where u_{i-1} <= P_i
//             (h_i <= P_i always), plus the row the sampler may land on.
//   pass2     like pass1 over the listed rows only: per group, the residual mass
//             sum max(0, P_i p_i - q_i) (Markov bias recomputed on MFMA).
//   finalize  one workgroup per stream: R_i, h_i, tau (top-down), then the
//             two-level exponential race over group masses and within the winning
//             group (weights recomputed in fp64), and the outputs.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "common.hpp"

namespace dspark {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kSuper = 256;   // rows per LDS flush (one per thread)

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
template <int KS>
__device__ __forceinline__ void load_w2_slab(const Args& a, int cb, int n, int q, bf16x8 (&A)[4][KS]) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    int vr = cb + 16 * (n >> 2) + 4 * s + (n & 3);
    vr = vr < a.V ? vr : a.V - 1;   // columns past V are masked after the product
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) A[s][kk] = load_bf16x8(a.W2t + (size_t)vr * a.R + kk * 32 + 8 * q);
  }
}

// Bias of draft row n (previous token `prev`, -1 = none) at this lane's 16 columns.
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

// Partial (max, sum 2^((x - max) c)) of 16 values of one row, reduced over the 4
// lanes holding the wave's 64 columns of that row.
__device__ __forceinline__ float2 row_partial(const float (&x)[16], float chi, float clo) {
  float m = x[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) m = fmaxf(m, x[i]);
  m = max4lanes(m);
  float s = 0.f;
  if (m != -INFINITY) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float t = x[i] - m;
      s += __builtin_amdgcn_exp2f(fmaf(t, chi, t * clo));
    }
  }
  s = sum4lanes(s);
  return make_float2(m, s);
}

// Combine the 4 wave partials of one row into the group partial.
__device__ __forceinline__ float2 combine_waves(const float2 (&p)[kWaves], float chi, float clo) {
  float M = p[0].x;
#pragma unroll
  for (int w = 1; w < kWaves; ++w) M = fmaxf(M, p[w].x);
  float S = 0.f;
  if (M != -INFINITY) {
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      if (p[w].x == -INFINITY) continue;
      const float t = p[w].x - M;
      S += p[w].y * __builtin_amdgcn_exp2f(fmaf(t, chi, t * clo));
    }
  }
  return make_float2(M, S);
}

// ---------------------------------------------------------------------------
// pass1: row statistics, per 256-id group.
// ---------------------------------------------------------------------------
template <int DT, int KS, bool MARKOV>
__global__ __launch_bounds__(kThreads) void pass1_kernel(Args a) {
  __shared__ float2 part[kSuper][kWaves];
  const int g = blockIdx.x;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, n = l & 15, q = l >> 4;
  const int cb = g * kGroup + w * kWaveCols;
  const int c0 = cb + 16 * q;
  const bool vec = a.vec_ok != 0;
  if (g == 0 && tid == 0) *a.ws.nitems = 0;   // pass-2 list is rebuilt by scan

  // draft rows (b, j), j < gamma_b
  const int ND = a.B * a.k;
  if (ND > 0) {
    bf16x8 A[4][KS];
    if (MARKOV) load_w2_slab<KS>(a, cb, n, q, A);
    for (int r0 = 0; r0 < ND; r0 += kSuper) {
      for (int ch = r0; ch < r0 + kSuper && ch < ND; ch += kChunk) {
        const int dr = ch + n;
        const int b = dr / a.k, j = dr - b * a.k;
        const bool active = dr < ND && j < stream_gamma(a, b < a.B ? b : 0);
        float x[16];
        float bias[16];
        if (MARKOV) markov_tile<KS>(a, A, active ? draft_prev(a, b, j) : -1, q, bias);
        float chi = 0.f, clo = 0.f;
        if (active) {
          const char* row = reinterpret_cast<const char*>(a.draft) + (size_t)dr * a.V * (DT == kBF16 ? 2 : 4);
          load16<DT>(row, c0, a.V, vec, x);
          temp_split(stream_temp(a, b), chi, clo);
          if (MARKOV) {
#pragma unroll
            for (int i = 0; i < 16; ++i) x[i] += bias[i];
          }
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) x[i] = -INFINITY;
        }
        const float2 pw = row_partial(x, chi, clo);
        if (q == 0) part[ch - r0 + n][w] = pw;
      }
      __syncthreads();
      const int dr = r0 + tid;
      if (dr < ND) {
        const int b = dr / a.k, j = dr - b * a.k;
        if (j < stream_gamma(a, b)) {
          float chi, clo;
          temp_split(stream_temp(a, b), chi, clo);
          float2 p[kWaves];
#pragma unroll
          for (int ww = 0; ww < kWaves; ++ww) p[ww] = part[tid][ww];
          a.ws.dpart[(size_t)dr * a.NG + g] = combine_waves(p, chi, clo);
        }
      }
      __syncthreads();
    }
  }

  // target rows (b, j), j <= gamma_b
  const int NT = a.B * (a.k + 1);
  for (int r0 = 0; r0 < NT; r0 += kSuper) {
    for (int ch = r0; ch < r0 + kSuper && ch < NT; ch += kChunk) {
      const int tr = ch + n;
      const int b = tr / (a.k + 1), j = tr - b * (a.k + 1);
      const bool active = tr < NT && j <= stream_gamma(a, b < a.B ? b : 0);
      float x[16];
      float chi = 0.f, clo = 0.f;
      if (active) {
        const char* row = reinterpret_cast<const char*>(a.target) + (size_t)tr * a.V * (DT == kBF16 ? 2 : 4);
        load16<DT>(row, c0, a.V, vec, x);
        temp_split(stream_temp(a, b), chi, clo);
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = -INFINITY;
      }
      const float2 pw = row_partial(x, chi, clo);
      if (q == 0) part[ch - r0 + n][w] = pw;
    }
    __syncthreads();
    const int tr = r0 + tid;
    if (tr < NT) {
      const int b = tr / (a.k + 1), j = tr - b * (a.k + 1);
      if (j <= stream_gamma(a, b)) {
        float chi, clo;
        temp_split(stream_temp(a, b), chi, clo);
        float2 p[kWaves];
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) p[ww] = part[tid][ww];
        a.ws.tpart[(size_t)tr * a.NG + g] = combine_waves(p, chi, clo);
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// scan: one workgroup per stream.
// ---------------------------------------------------------------------------
// Row normaliser from the group partials: M = max m_g, log2 S = log2 sum s_g 2^((m_g - M) c).
__device__ void row_norm(const float2* __restrict__ parts, int NG, double c, int l, float& M_out, double& l2s_out) {
  float M = -INFINITY;
  for (int gi = l; gi < NG; gi += 64) M = fmaxf(M, parts[gi].x);
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  double S = 0.0;
  for (int gi = l; gi < NG; gi += 64) {
    const float2 p = parts[gi];
    if (p.x != -INFINITY) S += (double)p.y * exp2(((double)p.x - (double)M) * c);
  }
  for (int off = 32; off >= 1; off >>= 1) S += __shfl_xor(S, off);
  M_out = M;
  l2s_out = log2(S);
}

template <int DT>
__global__ __launch_bounds__(kThreads) void scan_kernel(Args a) {
  __shared__ double s_lpx[kMaxK], s_lqx[kMaxK];
  const int b = blockIdx.x;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int gamma = stream_gamma(a, b);
  const double T = (double)stream_temp(a, b);
  const double c = kLog2e / T;
  const int k1 = a.k + 1;

  // normalisers: rows handled one per wave
  for (int r = w; r < 2 * gamma + 1; r += kWaves) {
    float M; double l2s;
    if (r <= gamma) {
      const int tr = b * k1 + r;
      row_norm(a.ws.tpart + (size_t)tr * a.NG, a.NG, c, l, M, l2s);
      if (l == 0) { a.ws.tm[tr] = M; a.ws.tl2s[tr] = l2s; }
    } else {
      const int dr = b * a.k + (r - gamma - 1);
      row_norm(a.ws.dpart + (size_t)dr * a.NG, a.NG, c, l, M, l2s);
      if (l == 0) { a.ws.dm[dr] = M; a.ws.dl2s[dr] = l2s; }
    }
  }
  __syncthreads();

  // gathered log-probabilities of the drafts, one wave per slot
  const size_t esz = DT == kBF16 ? 2 : 4;
  for (int j = w; j < gamma; j += kWaves) {
    const int x = clamp_tok(a.tokens[b * a.k + j], a.V);
    double bias = 0.0;
    if (a.W1 != nullptr) {
      const int prev = draft_prev(a, b, j);
      if (prev >= 0) {
        for (int r = l; r < a.R; r += 64)
          bias += (double)bf16_to_f32(a.W1[(size_t)prev * a.R + r]) * (double)bf16_to_f32(a.W2t[(size_t)x * a.R + r]);
      }
      for (int off = 32; off >= 1; off >>= 1) bias += __shfl_xor(bias, off);
    }
    if (l == 0) {
      const int tr = b * k1 + j, dr = b * a.k + j;
      const double lt = load1<DT>(reinterpret_cast<const char*>(a.target) + (size_t)tr * a.V * esz, x);
      const double ld = (double)load1<DT>(reinterpret_cast<const char*>(a.draft) + (size_t)dr * a.V * esz, x) + bias;
      const double lpx = (lt - (double)a.ws.tm[tr]) / T - a.ws.tl2s[tr] * kLn2;
      const double lqx = (ld - (double)a.ws.dm[dr]) / T - a.ws.dl2s[dr] * kLn2;
      s_lpx[j] = lpx; s_lqx[j] = lqx;
      a.ws.lpx[dr] = lpx; a.ws.lqx[dr] = lqx;
    }
  }
  __syncthreads();

  if (tid == 0) {
    // token-wise stop t: first j with u_j > min(1, r_j)
    int t = gamma;
    for (int j = 0; j < gamma; ++j) {
      const double lr = s_lpx[j] - s_lqx[j];
      const double thr = lr >= 0.0 ? 1.0 : exp(lr);
      const double u = accept_uniform(a.key0, a.key1, (uint32_t)b, (uint32_t)j, a.step);
      if (!(u <= thr)) { t = j; break; }
    }
    // clipped prefix log P_i
    double lp[kMaxK + 1];
    lp[0] = 0.0;
    for (int i = 1; i <= gamma; ++i) {
      const double v = lp[i - 1] + (s_lpx[i - 1] - s_lqx[i - 1]);
      lp[i] = v < 0.0 ? v : 0.0;
    }
    for (int i = 0; i <= gamma; ++i) a.ws.logP[b * k1 + i] = lp[i];
    uint32_t mask = 0;
    int stop = 0, f = 0;
    if (a.method == 0) {
      stop = t;
      if (t < gamma) mask = 1u << t;
    } else {
      if (gamma == 0 || accept_uniform(a.key0, a.key1, (uint32_t)b, (uint32_t)(gamma - 1), a.step) <= exp(lp[gamma])) {
        stop = gamma;   // top test passed (or no drafts): tau = gamma
      } else {
        for (int i = gamma - 1; i >= 0; --i) if (lp[i] == 0.0) { f = i; break; }
        mask = 1u << f;  // tau >= f; row f may be sampled
        for (int i = f + 1; i < gamma; ++i) {
          const double u = accept_uniform(a.key0, a.key1, (uint32_t)b, (uint32_t)(i - 1), a.step);
          if (u <= exp(lp[i])) mask |= 1u << i;   // h_i <= P_i: only these can pass
        }
        stop = -1;
      }
    }
    a.ws.info[4 * b + 0] = gamma;
    a.ws.info[4 * b + 1] = stop;
    a.ws.info[4 * b + 2] = f;
    a.ws.info[4 * b + 3] = t;
    a.ws.rowmask[b] = mask;
    for (int i = 0; i < gamma; ++i)
      if (mask & (1u << i)) {
        const int slot = atomicAdd(a.ws.nitems, 1);
        a.ws.items[slot] = b * a.k + i;
      }
  }
}

// ---------------------------------------------------------------------------
// pass2: residual group masses sum max(0, P_i p_i - q_i) of the listed rows.
// ---------------------------------------------------------------------------
template <int DT, int KS, bool MARKOV>
__global__ __launch_bounds__(kThreads) void pass2_kernel(Args a) {
  __shared__ float part[kSuper][kWaves];
  const int g = blockIdx.x;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, n = l & 15, q = l >> 4;
  const int cb = g * kGroup + w * kWaveCols;
  const int c0 = cb + 16 * q;
  const bool vec = a.vec_ok != 0;
  const int NI = *a.ws.nitems;
  if (NI == 0) return;
  const int k1 = a.k + 1;
  const size_t esz = DT == kBF16 ? 2 : 4;

  bf16x8 A[4][KS];
  if (MARKOV) load_w2_slab<KS>(a, cb, n, q, A);
  for (int r0 = 0; r0 < NI; r0 += kSuper) {
    for (int ch = r0; ch < r0 + kSuper && ch < NI; ch += kChunk) {
      const int it = ch + n;
      const bool active = it < NI;
      const int dr = active ? a.ws.items[it] : 0;
      const int b = dr / a.k, i = dr - b * a.k;
      float bias[16];
      if (MARKOV) markov_tile<KS>(a, A, active ? draft_prev(a, b, i) : -1, q, bias);
      float s = 0.f;
      if (active) {
        const int tr = b * k1 + i;
        float xt[16], xd[16];
        load16<DT>(reinterpret_cast<const char*>(a.target) + (size_t)tr * a.V * esz, c0, a.V, vec, xt);
        load16<DT>(reinterpret_cast<const char*>(a.draft) + (size_t)dr * a.V * esz, c0, a.V, vec, xd);
        float chi, clo;
        temp_split(stream_temp(a, b), chi, clo);
        const float Mt = a.ws.tm[tr], Md = a.ws.dm[dr];
        // exponent constants in log2 units, split hi + lo
        const double kp = (a.method == 1 ? a.ws.logP[tr] * kLog2e : 0.0) - a.ws.tl2s[tr];
        const double kq = -a.ws.dl2s[dr];
        const float kph = (float)kp, kpl = (float)(kp - (double)kph);
        const float kqh = (float)kq, kql = (float)(kq - (double)kqh);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float tp = xt[e] - Mt;
          const float d = MARKOV ? xd[e] + bias[e] : xd[e];
          const float tq = d - Md;
          const float ep = fmaf(tp, chi, kph) + fmaf(tp, clo, kpl);
          const float eq = fmaf(tq, chi, kqh) + fmaf(tq, clo, kql);
          const float pv = __builtin_amdgcn_exp2f(ep), qv = __builtin_amdgcn_exp2f(eq);
          const float wv = pv - qv;
          s += (c0 + e < a.V && wv > 0.f) ? wv : 0.f;
        }
      }
      s = sum4lanes(s);
      if (q == 0) part[ch - r0 + n][w] = s;
    }
    __syncthreads();
    const int it = r0 + tid;
    if (it < NI) {
      const int dr = a.ws.items[it];
      a.ws.wgrp[(size_t)dr * a.NG + g] = (part[tid][0] + part[tid][1]) + (part[tid][2] + part[tid][3]);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// finalize: tau, the race, outputs.  One workgroup per stream.
// ---------------------------------------------------------------------------
__device__ double block_sum(double v, double* red) {
  const int tid = threadIdx.x;
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  if ((tid & 63) == 0) red[tid >> 6] = v;
  __syncthreads();
  const double r = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return r;
}

// Arg-max of score with the lowest index on ties; score < 0 means "not a contestant".
__device__ void block_argmax(double& score, int& idx, double* rs, int* ri) {
  const int tid = threadIdx.x;
  for (int off = 32; off >= 1; off >>= 1) {
    const double os = __shfl_xor(score, off);
    const int oi = __shfl_xor(idx, off);
    if (os > score || (os == score && oi < idx)) { score = os; idx = oi; }
  }
  if ((tid & 63) == 0) { rs[tid >> 6] = score; ri[tid >> 6] = idx; }
  __syncthreads();
  score = rs[0]; idx = ri[0];
  for (int ww = 1; ww < kWaves; ++ww)
    if (rs[ww] > score || (rs[ww] == score && ri[ww] < idx)) { score = rs[ww]; idx = ri[ww]; }
  __syncthreads();
}

template <int DT>
__global__ __launch_bounds__(kThreads) void finalize_kernel(Args a) {
  __shared__ double red[kWaves];
  __shared__ double rs[kWaves];
  __shared__ int ri[kWaves];
  __shared__ double s_R[kMaxK], s_h[kMaxK + 1];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int k1 = a.k + 1;
  const int gamma = a.ws.info[4 * b + 0];
  int stop = a.ws.info[4 * b + 1];
  const int f = a.ws.info[4 * b + 2];
  const uint32_t mask = a.ws.rowmask[b];
  const double T = (double)stream_temp(a, b);
  const double c = kLog2e / T;
  const size_t esz = DT == kBF16 ? 2 : 4;

  if (tid <= kMaxK) s_h[tid] = NAN;
  if (tid < kMaxK) s_R[tid] = NAN;
  __syncthreads();
  // residual masses R_i of the candidate rows above f
  if (a.method == 1 && stop < 0) {
    for (int i = f + 1; i < gamma; ++i) {
      if (!(mask & (1u << i))) continue;
      const float* wr = a.ws.wgrp + (size_t)(b * a.k + i) * a.NG;
      double v = 0.0;
      for (int gi = tid; gi < a.NG; gi += kThreads) v += (double)wr[gi];
      const double R = block_sum(v, red);
      if (tid == 0) {
        const double lp = a.ws.logP[b * k1 + i];
        s_R[i] = R;
        s_h[i] = R / (R - expm1(lp));
      }
    }
    __syncthreads();
    // tau: the highest i whose test passes; rows outside the mask cannot pass (u > P_i >= h_i)
    stop = f;
    for (int i = gamma - 1; i > f; --i) {
      if (!(mask & (1u << i))) continue;
      const double u = accept_uniform(a.key0, a.key1, (uint32_t)b, (uint32_t)(i - 1), a.step);
      if (u <= s_h[i]) { stop = i; break; }
    }
  }
  const int s = stop;

  // weights of the sampled row: bonus / fallback use the target's own group partials
  bool use_p = (s == gamma);
  const float* wr = a.ws.wgrp + (size_t)(b * a.k + (s < gamma ? s : 0)) * a.NG;
  if (!use_p) {
    double v = 0.0;
    for (int gi = tid; gi < a.NG; gi += kThreads) v += (double)wr[gi];
    const double tot = block_sum(v, red);
    if (!(tot > 0.0)) use_p = true;   // all-zero residual: draw from p_s
  }
  const int tr = b * k1 + s;
  const float2* tp = a.ws.tpart + (size_t)tr * a.NG;
  const double Mt = (double)a.ws.tm[tr];

  // group race
  double best = -1.0;
  int gbest = 0x7fffffff;
  for (int gi = tid; gi < a.NG; gi += kThreads) {
    double W;
    if (use_p) {
      const float2 p = tp[gi];
      W = p.x == -INFINITY ? 0.0 : (double)p.y * exp2(((double)p.x - Mt) * c);
    } else {
      W = (double)wr[gi];
    }
    if (W > 0.0) {
      const double sc = W / race_clock(a.key0, a.key1, (uint32_t)b, (uint32_t)gi, kPurposeRaceGroup, a.step);
      if (sc > best) { best = sc; gbest = gi; }
    }
  }
  block_argmax(best, gbest, rs, ri);
  const int gsel = gbest < a.NG ? gbest : 0;

  // race inside the group, weights recomputed in fp64
  const int v = gsel * kGroup + tid;
  double sc = -1.0;
  if (v < a.V) {
    const double lt = load1<DT>(reinterpret_cast<const char*>(a.target) + (size_t)tr * a.V * esz, v);
    double wv;
    if (use_p) {
      wv = exp2((lt - Mt) * c);
    } else {
      const int dr = b * a.k + s;
      double d = load1<DT>(reinterpret_cast<const char*>(a.draft) + (size_t)dr * a.V * esz, v);
      if (a.W1 != nullptr) {
        const int prev = draft_prev(a, b, s);
        if (prev >= 0) {
          double bias = 0.0;
          for (int r = 0; r < a.R; ++r)
            bias += (double)bf16_to_f32(a.W1[(size_t)prev * a.R + r]) * (double)bf16_to_f32(a.W2t[(size_t)v * a.R + r]);
          d += bias;
        }
      }
      const double lpP = (a.method == 1 ? a.ws.logP[tr] * kLog2e : 0.0);
      const double pv = exp2((lt - Mt) * c - a.ws.tl2s[tr] + lpP);
      const double qv = exp2((d - (double)a.ws.dm[dr]) * c - a.ws.dl2s[dr]);
      wv = pv - qv;
    }
    if (wv > 0.0) sc = wv / race_clock(a.key0, a.key1, (uint32_t)b, (uint32_t)v, kPurposeRaceItem, a.step);
  }
  int vbest = sc >= 0.0 ? v : 0x7fffffff;
  block_argmax(sc, vbest, rs, ri);
  const int Y = vbest < a.V ? vbest : gsel * kGroup;

  // outputs
  if (tid <= a.k) {
    int o = -1;
    if (tid < s) o = a.tokens[b * a.k + tid];
    else if (tid == s) o = Y;
    a.out_tokens[b * k1 + tid] = o;
    if (a.diag != nullptr) {
      double* dg = a.diag + ((size_t)b * k1 + tid) * 5;
      const bool slot = tid < gamma;
      dg[0] = slot ? a.ws.lpx[b * a.k + tid] : NAN;
      dg[1] = slot ? a.ws.lqx[b * a.k + tid] : NAN;
      dg[2] = tid <= gamma ? exp(a.ws.logP[b * k1 + tid]) : NAN;
      dg[3] = (a.method == 1 && tid < kMaxK) ? s_R[tid] : NAN;
      double h = (a.method == 1 && tid <= kMaxK) ? s_h[tid] : NAN;
      if (a.method == 1 && tid == gamma && gamma >= 1) h = exp(a.ws.logP[b * k1 + gamma]);
      if (a.method == 1 && tid >= 1 && tid < gamma && a.ws.logP[b * k1 + tid] == 0.0) h = 1.0;
      dg[4] = h;
    }
  }
  if (tid == 0) a.accepted_len[b] = s;
}

// ---------------------------------------------------------------------------
// Markov bias alone: out[i, v] = logits_in[i, v] + W1[prev_i] . W2[:, v]
// ---------------------------------------------------------------------------
template <int DT, int KS>
__global__ __launch_bounds__(kThreads) void markov_bias_kernel(BiasArgs ba) {
  Args a{};
  a.V = ba.V; a.R = ba.R; a.W1 = ba.W1; a.W2t = ba.W2t;
  const int g = blockIdx.x;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, n = l & 15, q = l >> 4;
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
// Confidence head + adaptive count.  One wave per stream.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void adaptive_kernel(AdaptArgs aa) {
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int b = blockIdx.x * kWaves + w;
  if (b >= aa.B) return;
  double surv = 1.0, expected = 1.0;
  double best = 1.0 / (double)aa.ms[1];
  int nbest = 0;
  for (int j = 0; j < aa.k; ++j) {
    const uint16_t* h = aa.hidden + ((size_t)b * aa.k + j) * aa.H;
    double z = 0.0;
    for (int e = l; e < aa.H; e += 64) z += (double)bf16_to_f32(h[e]) * (double)bf16_to_f32(aa.w[e]);
    for (int off = 32; off >= 1; off >>= 1) z += __shfl_xor(z, off);
    z += (double)aa.bias;
    const double cj = 1.0 / (1.0 + exp(-z));
    surv *= cj;
    expected += surv;                         // 1 + sum_{i<=j} a_i = E(n = j + 1)
    const double ratio = expected / (double)aa.ms[j + 2];
    if (ratio > best) { best = ratio; nbest = j + 1; }
    if (l == 0) {
      if (aa.c_out) aa.c_out[b * aa.k + j] = (float)cj;
      if (aa.a_out) aa.a_out[b * aa.k + j] = (float)surv;
    }
  }
  if (l == 0) aa.n_out[b] = nbest;
}

// ---------------------------------------------------------------------------
// launch wrappers (host side of this translation unit)
// ---------------------------------------------------------------------------
template <int DT, int KS, bool MARKOV>
static hipError_t launch_passes(const Args& a, hipStream_t st, void* const* ev) {
  auto mark = [&](int i) {
    if (ev != nullptr && ev[i] != nullptr) (void)hipEventRecord(reinterpret_cast<hipEvent_t>(ev[i]), st);
  };
  mark(0);
  hipLaunchKernelGGL((pass1_kernel<DT, KS, MARKOV>), dim3(a.NG), dim3(kThreads), 0, st, a);
  mark(1);
  hipLaunchKernelGGL((scan_kernel<DT>), dim3(a.B), dim3(kThreads), 0, st, a);
  mark(2);
  hipLaunchKernelGGL((pass2_kernel<DT, KS, MARKOV>), dim3(a.NG), dim3(kThreads), 0, st, a);
  mark(3);
  hipLaunchKernelGGL((finalize_kernel<DT>), dim3(a.B), dim3(kThreads), 0, st, a);
  mark(4);
  return hipGetLastError();
}

template <int DT>
static hipError_t launch_dt(const Args& a, hipStream_t st, void* const* ev) {
  if (a.W1 == nullptr) return launch_passes<DT, 1, false>(a, st, ev);
  switch (a.R) {
    case 32: return launch_passes<DT, 1, true>(a, st, ev);
    case 64: return launch_passes<DT, 2, true>(a, st, ev);
    case 128: return launch_passes<DT, 4, true>(a, st, ev);
    default: return launch_passes<DT, 8, true>(a, st, ev);
  }
}

hipError_t launch_verify(const Args& a, hipStream_t st, void* const* ev) {
  return a.dtype == kBF16 ? launch_dt<kBF16>(a, st, ev) : launch_dt<kF32>(a, st, ev);
}

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

hipError_t launch_adaptive(const AdaptArgs& aa, hipStream_t st) {
  hipLaunchKernelGGL(adaptive_kernel, dim3((aa.B + kWaves - 1) / kWaves), dim3(kThreads), 0, st, aa);
  return hipGetLastError();
}

}  // namespace dspark
