// Host side of the C ABI declared in include/dspark_verify.h: argument checks,
// workspace carve-up and the launches.  No allocation, no synchronisation.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "../../include/dspark_verify.h"
#include "common.hpp"

using namespace dspark;

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool rank_ok(int R) { return R == 32 || R == 64 || R == 128 || R == 256; }

// Offsets of every workspace region, in the order of dspark::Workspace.
struct Layout {
  size_t off[19];
  size_t total;
};

Layout layout(int B, int k, int V) {
  const size_t NG = (size_t)(V + kGroup - 1) / kGroup;
  const size_t BT = (size_t)B * (k + 1), BD = (size_t)B * k;
  const size_t tiles = (BD + kChunk - 1) / kChunk;
  const size_t sizes[19] = {
      BT * NG * sizeof(float2),           // tpart
      BD * NG * sizeof(float2),           // dpart
      BD * NG * sizeof(float),            // wgrp
      BT * sizeof(float),        // tm
      BT * sizeof(double),       // tl2s
      BD * sizeof(float),        // dm
      BD * sizeof(double),       // dl2s
      BT * sizeof(double),       // logP
      BD * sizeof(double),       // lpx
      BD * sizeof(double),       // lqx
      (size_t)B * 4 * sizeof(int32_t),  // info
      (size_t)B * 4 * sizeof(int32_t),  // info2
      (size_t)B * sizeof(uint32_t),     // rowmask
      BD * sizeof(Item),                // items
      kCounterInts * sizeof(int32_t),   // nitems: list counts and pass-1 item counters
      tiles * 8 * 64 * sizeof(uint4),   // btile (sized for the largest rank, R = 256)
      std::max(BD * NG * sizeof(Top2), (size_t)B * NG * sizeof(WalkTop2)),   // race candidates
      // race clocks; the resident walk: the drawing workgroups' next-slot clocks
      std::max((size_t)B * NG * kGroup * sizeof(int16_t), 2 * std::min((size_t)B, NG) * kWalkClockBytes),
      kSyncInts * sizeof(int32_t),      // barrier words of the fused launch
  };
  Layout L;
  size_t o = 0;
  for (int i = 0; i < 19; ++i) {
    L.off[i] = o;
    o += align_up(sizes[i] > 0 ? sizes[i] : 1);
  }
  L.total = o;
  return L;
}

bool problem_sizes_ok(const dspark_verify_problem* p) {
  if (p == nullptr) return false;
  if (p->B < 1 || p->k < 1 || p->k > DSPARK_MAX_K || p->V < 1) return false;
  if (p->dtype != DSPARK_F32 && p->dtype != DSPARK_BF16) return false;
  // row offsets are computed in size_t; the int32 token ids bound V
  return true;
}

// The kernel arguments a problem fixes (inputs, sizes, generator key); outputs and
// workspace are filled in by the caller.
Args problem_args(const dspark_verify_problem* p) {
  Args a;
  memset(&a, 0, sizeof(a));
  a.B = p->B; a.k = p->k; a.V = p->V; a.R = p->W1 ? p->R : 0;
  a.NG = (p->V + kGroup - 1) / kGroup;
  a.dtype = p->dtype;
  const int esz = p->dtype == DSPARK_BF16 ? 2 : 4;
  a.vec_ok = ((size_t)p->V * esz) % 16 == 0 && aligned16(p->target_logits) && aligned16(p->draft_logits);
  a.target = p->target_logits;
  a.draft = p->draft_logits;
  a.tokens = p->draft_tokens;
  a.num_drafts = p->num_drafts;
  a.temperature = p->temperature;
  a.W1 = p->W1;
  a.W2t = p->W1 ? p->W2t : nullptr;
  a.anchor = p->anchor_tokens;
  a.key0 = (uint32_t)(p->seed & 0xffffffffu);
  a.key1 = (uint32_t)(p->seed >> 32);
  a.step = p->step;
  return a;
}

dspark_status verify_common(const dspark_verify_problem* p, const dspark_verify_outputs* o, void* ws,
                            size_t ws_bytes, void* stream, int method) {
  if (!problem_sizes_ok(p) || o == nullptr) return DSPARK_ERR_INVALID_ARG;
  if (!p->target_logits || !p->draft_logits || !p->draft_tokens || !o->accepted_len || !o->out_tokens)
    return DSPARK_ERR_INVALID_ARG;
  if (p->W1 != nullptr) {
    if (p->W2t == nullptr) return DSPARK_ERR_INVALID_ARG;
    if (!rank_ok(p->R)) return DSPARK_ERR_UNSUPPORTED;
    if (!aligned16(p->W1) || !aligned16(p->W2t)) return DSPARK_ERR_UNSUPPORTED;
  }
  if (verify_lds_bytes(p->B) > kMaxPassLds) return DSPARK_ERR_UNSUPPORTED;
  const Layout L = layout(p->B, p->k, p->V);
  if (ws == nullptr || ws_bytes < L.total || (reinterpret_cast<uintptr_t>(ws) % kAlign) != 0)
    return DSPARK_ERR_WORKSPACE;

  Args a = problem_args(p);
  a.method = method;
  a.accepted_len = o->accepted_len;
  a.out_tokens = o->out_tokens;
  a.diag = o->diag;
  char* base = reinterpret_cast<char*>(ws);
  a.ws.tpart = reinterpret_cast<float2*>(base + L.off[0]);
  a.ws.dpart = reinterpret_cast<float2*>(base + L.off[1]);
  a.ws.wgrp = reinterpret_cast<float*>(base + L.off[2]);
  a.ws.tm = reinterpret_cast<float*>(base + L.off[3]);
  a.ws.tl2s = reinterpret_cast<double*>(base + L.off[4]);
  a.ws.dm = reinterpret_cast<float*>(base + L.off[5]);
  a.ws.dl2s = reinterpret_cast<double*>(base + L.off[6]);
  a.ws.logP = reinterpret_cast<double*>(base + L.off[7]);
  a.ws.lpx = reinterpret_cast<double*>(base + L.off[8]);
  a.ws.lqx = reinterpret_cast<double*>(base + L.off[9]);
  a.ws.info = reinterpret_cast<int32_t*>(base + L.off[10]);
  a.ws.info2 = reinterpret_cast<int32_t*>(base + L.off[11]);
  a.ws.rowmask = reinterpret_cast<uint32_t*>(base + L.off[12]);
  a.ws.items = reinterpret_cast<Item*>(base + L.off[13]);
  a.ws.nitems = reinterpret_cast<int32_t*>(base + L.off[14]);
  a.ws.btile = reinterpret_cast<uint4*>(base + L.off[15]);
  a.ws.race = reinterpret_cast<Top2*>(base + L.off[16]);
  a.ws.clk = reinterpret_cast<uint2*>(base + L.off[17]);
  a.ws.sync = reinterpret_cast<int32_t*>(base + L.off[18]);
  if (launch_verify(a, reinterpret_cast<hipStream_t>(stream), o->stage_events) != hipSuccess)
    return DSPARK_ERR_HIP;
  return DSPARK_OK;
}

// The drafter walk: the verify problem's shapes, draft logits, temperatures, Markov
// factors, anchors, num_drafts, seed and step; no target logits or draft tokens.
dspark_status walk_check(const dspark_verify_problem* p) {
  if (!problem_sizes_ok(p) || !p->draft_logits) return DSPARK_ERR_INVALID_ARG;
  if (p->W1 != nullptr) {
    if (p->W2t == nullptr) return DSPARK_ERR_INVALID_ARG;
    if (!rank_ok(p->R)) return DSPARK_ERR_UNSUPPORTED;
    if (!aligned16(p->W1) || !aligned16(p->W2t)) return DSPARK_ERR_UNSUPPORTED;
  }
  return DSPARK_OK;
}

Args walk_args(const dspark_verify_problem* p, int32_t* tokens_out) {
  Args a;
  memset(&a, 0, sizeof(a));
  a.B = p->B; a.k = p->k; a.V = p->V; a.R = p->W1 ? p->R : 0;
  a.NG = (p->V + kGroup - 1) / kGroup;
  a.dtype = p->dtype;
  const int esz = p->dtype == DSPARK_BF16 ? 2 : 4;
  a.vec_ok = ((size_t)p->V * esz) % 16 == 0 && aligned16(p->draft_logits);
  a.draft = p->draft_logits;
  a.tokens = tokens_out;          // slot j reads x_{j-1} from the tokens drawn so far
  a.num_drafts = p->num_drafts;
  a.temperature = p->temperature;
  a.W1 = p->W1;
  a.W2t = p->W1 ? p->W2t : nullptr;
  a.anchor = p->anchor_tokens;
  a.key0 = (uint32_t)(p->seed & 0xffffffffu);
  a.key1 = (uint32_t)(p->seed >> 32);
  a.step = p->step;
  return a;
}

dspark_status walk_common(const dspark_verify_problem* p, int32_t* tokens_out, double* logq_out, void* ws,
                          size_t ws_bytes, void* stream) {
  const dspark_status st = walk_check(p);
  if (st != DSPARK_OK) return st;
  if (!tokens_out) return DSPARK_ERR_INVALID_ARG;
  const Layout L = layout(p->B, p->k, p->V);
  if (ws == nullptr || ws_bytes < L.total || (reinterpret_cast<uintptr_t>(ws) % kAlign) != 0)
    return DSPARK_ERR_WORKSPACE;
  Args a = walk_args(p, tokens_out);
  char* base = reinterpret_cast<char*>(ws);
  a.ws.tpart = reinterpret_cast<float2*>(base + L.off[0]);    // [NG][B] partials
  a.ws.race = reinterpret_cast<Top2*>(base + L.off[16]);      // [NG][B] candidates
  a.ws.clk = reinterpret_cast<uint2*>(base + L.off[17]);     // the resident walk's offloaded clocks
  a.ws.sync = reinterpret_cast<int32_t*>(base + L.off[18]);   // the resident walk's grid-wide waits
  if (launch_walk(a, tokens_out, logq_out, reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return DSPARK_ERR_HIP;
  return DSPARK_OK;
}

// Scratch of the allocation-free verify entry point: one copy per device, held until
// the process ends.  Host code never passes `scratch` itself to a kernel (in host code
// the name is a stand-in, not a device address); it uses the address that
// hipGetSymbolAddress returns for the current device, looked up once per device.
constexpr size_t kScratchBytes = (size_t)DSPARK_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

dspark_status scratch_for_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DSPARK_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return DSPARK_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DSPARK_OK;
}

}  // namespace

extern "C" {

dspark_status dspark_verify_noalloc(const dspark_verify_problem* p, const dspark_verify_outputs* o, int32_t method,
                                    void* stream) {
  if (method != 0 && method != 1) return DSPARK_ERR_INVALID_ARG;
  if (!problem_sizes_ok(p)) return DSPARK_ERR_INVALID_ARG;
  if (layout(p->B, p->k, p->V).total > kScratchBytes) return DSPARK_ERR_TOO_LARGE;
  void* ws = nullptr;
  const dspark_status st = scratch_for_current_device(&ws);
  if (st != DSPARK_OK) return st;
  return verify_common(p, o, ws, kScratchBytes, stream, method);
}

dspark_status dspark_draft_sample(const dspark_verify_problem* p, int32_t* tokens_out, double* logq_out,
                                  void* ws, size_t ws_bytes, void* stream) {
  return walk_common(p, tokens_out, logq_out, ws, ws_bytes, stream);
}

dspark_status dspark_draft_launches(const dspark_verify_problem* p, int32_t* launches) {
  if (launches == nullptr) return DSPARK_ERR_INVALID_ARG;
  const dspark_status st = walk_check(p);
  if (st != DSPARK_OK) return st;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return DSPARK_ERR_HIP;
  const int n = walk_launches(walk_args(p, nullptr));
  if (n <= 0) return DSPARK_ERR_HIP;
  *launches = n;
  return DSPARK_OK;
}

size_t dspark_workspace_bytes(const dspark_verify_problem* p) {
  if (!problem_sizes_ok(p)) return 0;
  return layout(p->B, p->k, p->V).total;
}

dspark_status dspark_verify_launches(const dspark_verify_problem* p, int32_t* launches) {
  if (!problem_sizes_ok(p) || launches == nullptr) return DSPARK_ERR_INVALID_ARG;
  if (p->W1 != nullptr && !rank_ok(p->R)) return DSPARK_ERR_UNSUPPORTED;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return DSPARK_ERR_HIP;
  *launches = verify_fused_grid(problem_args(p)) > 0 ? 2 : 1 + 4;
  return DSPARK_OK;
}

dspark_status dspark_verify_tokenwise(const dspark_verify_problem* p, const dspark_verify_outputs* o,
                                      void* ws, size_t ws_bytes, void* stream) {
  return verify_common(p, o, ws, ws_bytes, stream, 0);
}

dspark_status dspark_verify_block(const dspark_verify_problem* p, const dspark_verify_outputs* o,
                                  void* ws, size_t ws_bytes, void* stream) {
  return verify_common(p, o, ws, ws_bytes, stream, 1);
}

dspark_status dspark_markov_bias(const uint16_t* W1, const uint16_t* W2t, int32_t V, int32_t R,
                                 const int32_t* prev_tokens, int32_t rows, const void* logits_in,
                                 int32_t dtype, float* out, void* stream) {
  if (!W1 || !W2t || !prev_tokens || !out || V < 1 || rows < 0) return DSPARK_ERR_INVALID_ARG;
  if (dtype != DSPARK_F32 && dtype != DSPARK_BF16) return DSPARK_ERR_INVALID_ARG;
  if (!rank_ok(R) || !aligned16(W1) || !aligned16(W2t)) return DSPARK_ERR_UNSUPPORTED;
  if (rows == 0) return DSPARK_OK;
  BiasArgs ba;
  ba.W1 = W1; ba.W2t = W2t; ba.V = V; ba.R = R; ba.rows = rows; ba.dtype = dtype;
  const int esz = dtype == DSPARK_BF16 ? 2 : 4;
  ba.vec_ok = ((size_t)V * esz) % 16 == 0 && ((size_t)V * 4) % 16 == 0 && aligned16(out) &&
              (logits_in == nullptr || aligned16(logits_in));
  ba.prev = prev_tokens;
  ba.logits_in = logits_in;
  ba.out = out;
  const int NG = (V + kGroup - 1) / kGroup;
  if (launch_markov_bias(ba, NG, reinterpret_cast<hipStream_t>(stream)) != hipSuccess) return DSPARK_ERR_HIP;
  return DSPARK_OK;
}

dspark_status dspark_adaptive_k(const uint16_t* hidden, const uint16_t* w, float bias, int32_t B, int32_t k,
                                int32_t H, const float* verify_ms, int32_t n_ms, int32_t* n_out, float* c_out,
                                float* a_out, void* stream) {
  if (!hidden || !w || !verify_ms || !n_out || B < 1 || k < 1 || k > DSPARK_MAX_K || H < 1)
    return DSPARK_ERR_INVALID_ARG;
  if (n_ms < k + 2 || n_ms > kMaxMs) return DSPARK_ERR_INVALID_ARG;
  AdaptArgs aa;
  memset(&aa, 0, sizeof(aa));
  aa.hidden = hidden; aa.w = w; aa.bias = bias; aa.B = B; aa.k = k; aa.H = H; aa.n_ms = n_ms;
  aa.n_out = n_out; aa.c_out = c_out; aa.a_out = a_out;
  aa.vec_ok = (H % 8) == 0 && aligned16(hidden) && aligned16(w);
  for (int i = 0; i < n_ms; ++i) {
    if (!(verify_ms[i] > 0.0f)) return DSPARK_ERR_INVALID_ARG;
    aa.ms[i] = verify_ms[i];
  }
  if (launch_adaptive(aa, reinterpret_cast<hipStream_t>(stream)) != hipSuccess) return DSPARK_ERR_HIP;
  return DSPARK_OK;
}

dspark_status dspark_draft_scatter(const void* reduced, const int32_t* vocab_ids, int32_t rows, int32_t K,
                                   int32_t V, int32_t dtype, void* out, void* stream) {
  if (!reduced || !vocab_ids || !out || rows < 0 || K < 1 || V < 1 || K > V) return DSPARK_ERR_INVALID_ARG;
  if (dtype != DSPARK_F32 && dtype != DSPARK_BF16) return DSPARK_ERR_INVALID_ARG;
  if (rows == 0) return DSPARK_OK;
  if (launch_scatter(reduced, vocab_ids, rows, K, V, dtype, out, reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return DSPARK_ERR_HIP;
  return DSPARK_OK;
}

dspark_status dspark_random_words(uint64_t seed, uint32_t b, uint32_t purpose, uint32_t step, uint32_t idx0, int32_t n,
                                  int32_t kind, uint32_t* out, void* stream) {
  if (out == nullptr || n < 0 || (kind != 0 && kind != 1)) return DSPARK_ERR_INVALID_ARG;
  if (n == 0) return DSPARK_OK;
  if (launch_random_words(seed, b, purpose, step, idx0, n, kind, out, reinterpret_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return DSPARK_ERR_HIP;
  return DSPARK_OK;
}

dspark_status dspark_w2_transpose(const uint16_t* W2, int32_t R, int32_t V, uint16_t* W2t, void* stream) {
  if (W2 == nullptr || W2t == nullptr || R < 1 || V < 1) return DSPARK_ERR_INVALID_ARG;
  if ((size_t)R * (size_t)V > ((size_t)1 << 40)) return DSPARK_ERR_INVALID_ARG;
  const char *a = reinterpret_cast<const char*>(W2), *b = reinterpret_cast<const char*>(W2t);
  const size_t bytes = (size_t)R * V * sizeof(uint16_t);
  if (a < b + bytes && b < a + bytes) return DSPARK_ERR_INVALID_ARG;   // no in-place transpose
  if (launch_w2_transpose(W2, R, V, W2t, reinterpret_cast<hipStream_t>(stream)) != hipSuccess) return DSPARK_ERR_HIP;
  return DSPARK_OK;
}

int32_t dspark_k_for_batch(const int32_t* schedule, int32_t n, int32_t batch, int32_t k_default) {
  if (schedule == nullptr) return k_default;
  for (int32_t i = 0; i < n; ++i)
    if (schedule[3 * i] <= batch && batch <= schedule[3 * i + 1]) return schedule[3 * i + 2];
  return k_default;
}

const char* dspark_status_string(dspark_status s) {
  switch (s) {
    case DSPARK_OK: return "ok";
    case DSPARK_ERR_INVALID_ARG: return "invalid argument";
    case DSPARK_ERR_UNSUPPORTED: return "unsupported configuration";
    case DSPARK_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case DSPARK_ERR_HIP: return "HIP launch failed";
    case DSPARK_ERR_NO_MEMORY: return "host allocation failed";
    case DSPARK_ERR_TOO_LARGE: return "problem needs more scratch than the static per-device buffer holds";
  }
  return "unknown status";
}

}  // extern "C"
