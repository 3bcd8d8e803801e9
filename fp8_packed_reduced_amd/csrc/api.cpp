// C interface of libfpr.so (declared in include/fpr.h): argument checks,
// the memory plan of the caller-provided buffers, and the launch sequence of
// each call on the caller's stream.  No allocation, no synchronisation.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <mutex>

#include "../../include/fpr.h"
#include "common.hpp"
#include "launch.hpp"

namespace {

using fpr::ceil_div;
using fpr::round_up;

constexpr size_t kAlign = 256;
constexpr int kPartsW = 768;     // amax blocks for W_packed (one row each at D = 768)
constexpr int kPartsAct = 256;   // amax blocks for x
using fpr::kMaxTokens;
constexpr size_t kMaxDynLds = 64 * 1024;  // dynamic LDS of one epilogue block

struct Plan {
  int D, H, dqk, dv, qs, nq, nqk2, N;
  int64_t T, Tp;
  bool fused;  // norm/RoPE in the forward GEMM's epilogue (else qk_pre in the workspace)
  bool two_pass;  // backward without dQK (fpr_dims.bwd_passes = 2)
  size_t s_x8, s_rho, s_xsc, saved_total;
  size_t f_part, f_qk, fwd_total;
  int f_parts;
  size_t b_part, b_gsc, b_dqkv, b_g8, b_dwpart, bwd_total;
  int b_parts, b_nr_parts, b_dv_parts;  // all amax partials = norm/RoPE's, then dv's
  size_t p_part, pack_total;
};

bool dims_ok(const fpr_dims* d) {
  if (!d) return false;
  if (d->d_model <= 0 || d->n_heads <= 0 || d->d_qk <= 0 || d->d_v <= 0) return false;
  if (!(d->eps >= 0.0f) || !(d->rope_base > 0.0f)) return false;
  if (d->qk_stride < 0) return false;
  if (d->grad_format != FPR_FORMAT_E4M3 && d->grad_format != FPR_FORMAT_E5M2) return false;
  if (d->bwd_passes < 0 || d->bwd_passes > 2) return false;
  return true;
}

int shape_check(const fpr_dims* d) {
  if (!dims_ok(d)) return FPR_ERR_ARG;
  const int64_t N = (int64_t)d->n_heads * (2 * d->d_qk + d->d_v);
  if (d->d_model % 64 || d->d_qk % 16 || d->d_v % 16 || N % 64) return FPR_ERR_SHAPE;
  if (d->n_heads > 64 || d->d_qk > 512 || d->d_v > 4096 || N > (1 << 20) ||
      d->d_model > (1 << 16))
    return FPR_ERR_SHAPE;
  if (d->qk_stride && (d->qk_stride < d->d_qk || d->qk_stride % 8 || d->qk_stride > 1024))
    return FPR_ERR_SHAPE;
  if (d->bwd_passes == 2 && !fpr::norm_rope_bwd_two_pass(d->d_qk)) return FPR_ERR_SHAPE;
  if (fpr::norm_rope_fwd_lds(d->n_heads, d->d_qk) > kMaxDynLds ||
      fpr::norm_rope_bwd_lds(d->n_heads, d->d_qk) > kMaxDynLds)
    return FPR_ERR_SHAPE;
  return FPR_OK;
}

size_t take(size_t& cursor, size_t bytes) {
  const size_t at = cursor;
  cursor = (size_t)round_up((int64_t)(cursor + bytes), kAlign);
  return at;
}

Plan make_plan(const fpr_dims* d, int64_t T) {
  Plan p{};
  p.D = d->d_model;
  p.H = d->n_heads;
  p.dqk = d->d_qk;
  p.dv = d->d_v;
  p.qs = d->qk_stride ? d->qk_stride : d->d_qk;
  p.nq = p.H * p.dqk;
  p.nqk2 = 2 * p.nq;
  p.N = p.nqk2 + p.H * p.dv;
  p.T = T;
  p.Tp = round_up(T > 0 ? T : 1, 128);
  p.fused = fpr::fused_forward(p.dqk, p.N, p.D);
  p.two_pass = d->bwd_passes == 2;
  size_t c = 0;
  p.s_x8 = take(c, fpr::act_blocked_bytes(T, p.D));
  p.s_rho = take(c, (size_t)T * 2 * p.H * sizeof(float));
  p.s_xsc = take(c, 4 * sizeof(float));
  p.saved_total = c;
  c = 0;
  // one amax block per 256 x 16-byte vectors of x, at most kPartsAct
  p.f_parts = (int)std::max<int64_t>(1, std::min<int64_t>(kPartsAct, ceil_div(T * p.D / 8, fpr::kThreads)));
  p.f_part = take(c, (size_t)p.f_parts * 4);
  p.f_qk = p.fused ? (size_t)-1 : take(c, (size_t)T * p.nqk2 * 2);
  p.fwd_total = c;
  c = 0;
  p.b_nr_parts = fpr::norm_rope_bwd_blocks(T > 0 ? T : 1, p.H, p.dqk);
  p.b_dv_parts = (int)std::max<int64_t>(
      1, std::min<int64_t>(kPartsAct, ceil_div(T * p.H * p.dv / 8, fpr::kThreads)));
  p.b_parts = p.b_nr_parts + p.b_dv_parts;  // <= kMaxPartials, checked by plan_ok()
  p.b_part = take(c, (size_t)p.b_parts * 4);
  p.b_gsc = take(c, 4 * sizeof(float));
  p.b_dqkv = p.two_pass ? (size_t)-1 : take(c, (size_t)T * p.nqk2 * 2);
  p.b_g8 = take(c, fpr::act_blocked_bytes(T, p.N));
  p.b_dwpart = take(c, fpr::dw_partial_bytes(p.D, p.N, p.Tp));
  p.bwd_total = c;
  c = 0;
  p.p_part = take(c, (size_t)kPartsW * 4);
  p.pack_total = c;
  return p;
}

// Every quantiser block re-reduces all amax partials of its tensor, so their
// number must stay bounded at any token count.
bool plan_ok(const Plan& p) { return p.b_parts <= fpr::kMaxPartials && p.f_parts <= fpr::kMaxPartials; }

// ---- FP8 ReLU^2 MLP: shapes and memory plan

bool al16(const void* p);

struct MlpPlan {
  int D, F;
  int64_t T, Tp;
  size_t s_x8, s_h8, s_xsc, s_hsc, saved_total;
  int x_parts;
  size_t f_xpart, f_h, f_hpart, fwd_total;
  size_t b_dypart, b_dysc, b_dy8, b_dpre, b_dppart, b_dpsc, b_dp8, b_dwpart, bwd_total;
  size_t p_part, pack_total;
};

int mlp_shape_check(const fpr_mlp_dims* d) {
  if (!d || d->d_model <= 0 || d->d_ff <= 0) return FPR_ERR_ARG;
  if (d->grad_format != FPR_FORMAT_E4M3 && d->grad_format != FPR_FORMAT_E5M2) return FPR_ERR_ARG;
  if (d->d_model % 64 || d->d_ff % 64 || d->d_model > (1 << 16) || d->d_ff > (1 << 16))
    return FPR_ERR_SHAPE;
  return FPR_OK;
}

MlpPlan make_mlp_plan(const fpr_mlp_dims* d, int64_t T) {
  MlpPlan p{};
  p.D = d->d_model;
  p.F = d->d_ff;
  p.T = T;
  p.Tp = round_up(T > 0 ? T : 1, 128);
  const size_t slots = (size_t)fpr::gemm_amax_slots_max() * 4;
  size_t c = 0;
  p.s_x8 = take(c, fpr::act_blocked_bytes(T, p.D));
  p.s_h8 = take(c, fpr::act_blocked_bytes(T, p.F));
  p.s_xsc = take(c, 4 * sizeof(float));
  p.s_hsc = take(c, 4 * sizeof(float));
  p.saved_total = c;
  // one amax block per 256 x 16-byte vectors of x (or dy), at most kPartsAct
  p.x_parts =
      (int)std::max<int64_t>(1, std::min<int64_t>(kPartsAct, ceil_div(T * p.D / 8, fpr::kThreads)));
  c = 0;
  p.f_xpart = take(c, (size_t)p.x_parts * 4);
  p.f_h = take(c, (size_t)T * p.F * 2);
  p.f_hpart = take(c, slots);
  p.fwd_total = c;
  c = 0;
  p.b_dypart = take(c, (size_t)p.x_parts * 4);
  p.b_dysc = take(c, 4 * sizeof(float));
  p.b_dy8 = take(c, fpr::act_blocked_bytes(T, p.D));
  p.b_dpre = take(c, (size_t)T * p.F * 2);
  p.b_dppart = take(c, slots);
  p.b_dpsc = take(c, 4 * sizeof(float));
  p.b_dp8 = take(c, fpr::act_blocked_bytes(T, p.F));
  p.b_dwpart = take(c, std::max(fpr::dw_partial_bytes(p.D, p.F, p.Tp),
                                fpr::dw_partial_bytes(p.F, p.D, p.Tp)));
  p.bwd_total = c;
  c = 0;
  p.p_part = take(c, (size_t)kPartsW * 4);
  p.pack_total = c;
  return p;
}

// mlp_pack_forward's workspace: W1's and W2's amax partials, then the
// forward's.
size_t mlp_pack_forward_off() { return (size_t)round_up(2 * (int64_t)kPartsW * 4, kAlign); }
size_t mlp_pack_forward_bytes(const MlpPlan& p) { return mlp_pack_forward_off() + p.fwd_total; }

int mlp_cache_check(const fpr_mlp_cache* c) {
  if (!c || !c->w1 || !c->w1_t || !c->w2 || !c->w2_t || !c->scales || !c->status)
    return FPR_ERR_ARG;
  if (!al16(c->w1) || !al16(c->w1_t) || !al16(c->w2) || !al16(c->w2_t) ||
      (uintptr_t)c->scales % 4 || (uintptr_t)c->status % 4)
    return FPR_ERR_ALIGN;
  return FPR_OK;
}

int mlp_tokens_check(int64_t T) {
  if (T <= 0) return FPR_ERR_ARG;
  return T > kMaxTokens ? FPR_ERR_SHAPE : FPR_OK;
}

thread_local fpr_trace* t_trace = nullptr;

bool same_name(const char* a, const char* b) {
  while (*a && *a == *b) ++a, ++b;
  return *a == *b;
}

// Launch one stage, bracketed by the caller's events when a trace is set.
template <class F>
void stage(const char* name, hipStream_t s, F&& launch) {
  fpr_trace* t = t_trace;
  if (t && t->count < t->capacity && t->count < FPR_TRACE_MAX &&
      (!t->only || same_name(t->only, name))) {
    const int i = t->count;
    (void)hipEventRecord(static_cast<hipEvent_t>(t->events[2 * i]), s);
    launch();
    (void)hipEventRecord(static_cast<hipEvent_t>(t->events[2 * i + 1]), s);
    t->names[i] = name;
    t->count = i + 1;
  } else {
    launch();
  }
}

bool al16(const void* p) { return p && ((uintptr_t)p % 16 == 0); }

int finish() { return hipGetLastError() == hipSuccess ? FPR_OK : FPR_ERR_LAUNCH; }

template <class T>
T* at(void* base, size_t off) {
  return reinterpret_cast<T*>(static_cast<uint8_t*>(base) + off);
}
template <class T>
const T* at(const void* base, size_t off) {
  return reinterpret_cast<const T*>(static_cast<const uint8_t*>(base) + off);
}

int cache_check(const fpr_weight_cache* c) {
  if (!c || !c->w_packed || !c->w_packed_t || !c->scales || !c->status) return FPR_ERR_ARG;
  if (!al16(c->w_packed) || !al16(c->w_packed_t) || (uintptr_t)c->scales % 4 ||
      (uintptr_t)c->status % 4)
    return FPR_ERR_ALIGN;
  return FPR_OK;
}

int tokens_check(int32_t n_seq, int32_t seq_len, int64_t* T) {
  if (n_seq <= 0 || seq_len <= 0) return FPR_ERR_ARG;
  *T = (int64_t)n_seq * seq_len;
  if (*T > kMaxTokens) return FPR_ERR_SHAPE;
  return FPR_OK;
}

int ld_check(int64_t ld, int64_t cols, const void* p) {
  if (!p || ld < cols) return FPR_ERR_ARG;
  if (!al16(p) || ld % 4) return FPR_ERR_ALIGN;
  return FPR_OK;
}

// ---- the fixed scratch of qkv_forward_noalloc
//
// For callers that cannot allocate: the forward's workspace (with the norm
// and RoPE fused into the GEMM, only the x amax partials) lives in this
// array, one copy per device, held until the process ends.  Host code never
// uses the array's name as an address: each device's copy is looked up once
// with hipGetSymbolAddress and that pointer is what the kernels get.
constexpr size_t kNoAllocScratch = 64 * 1024;
constexpr int kMaxDevices = 64;
__device__ __attribute__((aligned(256))) uint8_t scratch[kNoAllocScratch];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// This device's copy of the scratch array, or null on failure.
void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

// qkv_pack_forward's workspace: the weight pack's, then the forward's.
size_t pack_forward_off(const Plan& p) { return (size_t)round_up((int64_t)p.pack_total, kAlign); }
size_t pack_forward_bytes(const Plan& p) { return pack_forward_off(p) + p.fwd_total; }

// The forward after x8 and its scales exist: the packed GEMM with the norm,
// RoPE and head-major stores in its epilogue, or, for other head widths,
// the GEMM and then the norm/RoPE kernel.
void forward_gemm(const fpr_dims* dims, const Plan& p, int32_t n_seq, int32_t seq_len,
                  const fpr_weight_cache* cache, uint16_t* q, uint16_t* k, uint16_t* v,
                  void* saved, void* workspace, hipStream_t s) {
  const int64_t T = p.T;
  float* xsc = at<float>(saved, p.s_xsc);
  uint8_t* x8 = at<uint8_t>(saved, p.s_x8);
  float* rho = at<float>(saved, p.s_rho);
  if (p.fused) {
    stage("gemm_fwd", s, [&] {
      fpr::launch_gemm_qkv_fwd(x8, cache->w_packed_t, n_seq, seq_len, p.D, p.H, p.dqk, p.dv, p.qs,
                               dims->eps, dims->rope_base, xsc, cache->scales, q, k, v, rho, s);
    });
  } else {
    uint16_t* qk = at<uint16_t>(workspace, p.f_qk);
    stage("gemm_fwd", s, [&] {
      fpr::launch_gemm_fwd(x8, cache->w_packed_t, (int)T, p.N, p.D, xsc, cache->scales, qk,
                           p.nqk2, v, p.H, p.dv, seq_len, s);
    });
    stage("norm_rope_fwd", s, [&] {
      fpr::launch_norm_rope_fwd(qk, T, seq_len, p.H, p.dqk, p.qs, dims->eps, dims->rope_base, q,
                                k, rho, s);
    });
  }
}

// The MLP forward after x8 and its scales exist: the up-projection with
// relu^2 and the amax of h in its epilogue, h's quantiser, the down-projection.
void mlp_forward_gemms(const MlpPlan& p, const fpr_mlp_cache* cache, uint16_t* y, void* saved,
                       void* workspace, hipStream_t s) {
  const int64_t T = p.T;
  uint32_t* hparts = at<uint32_t>(workspace, p.f_hpart);
  uint16_t* h = at<uint16_t>(workspace, p.f_h);
  uint8_t* x8 = at<uint8_t>(saved, p.s_x8);
  uint8_t* h8 = at<uint8_t>(saved, p.s_h8);
  float* xsc = at<float>(saved, p.s_xsc);
  float* hsc = at<float>(saved, p.s_hsc);
  int nh = 0;
  stage("mlp_gemm_up", s, [&] {
    nh = fpr::launch_gemm_relu2(x8, cache->w1_t, (int)T, p.F, p.D, xsc, cache->scales, h,
                                hparts, s);
  });
  stage("mlp_quantize_h", s, [&] {
    fpr::launch_quantize_act(h, T, p.F, hparts, nh, hsc, cache->status, FPR_STATUS_H_NONFINITE,
                             h8, p.Tp, s);
  });
  stage("mlp_gemm_down", s, [&] {
    fpr::launch_gemm_dx(h8, cache->w2_t, (int)T, p.D, p.F, hsc, cache->scales + 2, y, s);
  });
}

}  // namespace

extern "C" {

size_t fpr_workspace_bytes(const fpr_dims* dims, int64_t tokens, int which) {
  if (shape_check(dims) != FPR_OK) return 0;
  if (which == FPR_CALL_PACK) return make_plan(dims, 1).pack_total;
  if (tokens <= 0 || tokens > kMaxTokens) return 0;
  const Plan p = make_plan(dims, tokens);
  if (!plan_ok(p)) return 0;
  if (which == FPR_CALL_FORWARD) return p.fwd_total;
  if (which == FPR_CALL_BACKWARD) return p.bwd_total;
  if (which == FPR_CALL_PACK_FORWARD) return pack_forward_bytes(p);
  return 0;
}

size_t fpr_saved_bytes(const fpr_dims* dims, int64_t tokens) {
  if (shape_check(dims) != FPR_OK || tokens <= 0 || tokens > kMaxTokens) return 0;
  return make_plan(dims, tokens).saved_total;
}

int fpr_get_layout(const fpr_dims* dims, int64_t tokens, fpr_layout* out) {
  int rc = shape_check(dims);
  if (rc) return rc;
  if (!out || tokens <= 0) return FPR_ERR_ARG;
  if (tokens > kMaxTokens) return FPR_ERR_SHAPE;
  const Plan p = make_plan(dims, tokens);
  out->tokens = p.T;
  out->tokens_padded = p.Tp;
  out->saved_x8 = p.s_x8;
  out->saved_rho = p.s_rho;
  out->saved_x_scales = p.s_xsc;
  out->fwd_qk_pre = p.f_qk;
  out->bwd_dqkv = p.b_dqkv;
  out->bwd_g_scales = p.b_gsc;
  out->bwd_g8 = p.b_g8;
  out->bwd_dw_part = p.b_dwpart;
  out->dw_splits = fpr::dw_splits(p.D, p.N, p.Tp);
  out->bwd_amax_partials = p.b_parts;
  out->k_block = fpr::kKBlock;
  out->act_block_rows = fpr::kActRows;
  return FPR_OK;
}

int pack_quantize_weights(const fpr_dims* dims, const float* wq, int64_t ldq, const float* wk,
                          int64_t ldk, const float* wv, int64_t ldv,
                          const fpr_weight_cache* cache, void* workspace,
                          size_t workspace_bytes, void* stream) {
  int rc = shape_check(dims);
  if (rc) return rc;
  const Plan p = make_plan(dims, 1);
  if ((rc = ld_check(ldq, p.nq, wq)) || (rc = ld_check(ldk, p.nq, wk)) ||
      (rc = ld_check(ldv, (int64_t)p.H * p.dv, wv)) || (rc = cache_check(cache)))
    return rc;
  if (!workspace) return FPR_ERR_ARG;
  if (!al16(workspace)) return FPR_ERR_ALIGN;
  if (workspace_bytes < p.pack_total) return FPR_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  uint32_t* parts = at<uint32_t>(workspace, p.p_part);
  stage("amax_w", s, [&] {
    fpr::launch_amax_w(wq, ldq, wk, ldk, wv, ldv, p.D, p.nq, p.N, parts, kPartsW, s);
  });
  stage("quantize_w", s, [&] {
    fpr::launch_quantize_w(wq, ldq, wk, ldk, wv, ldv, p.D, p.nq, p.N, parts, kPartsW,
                           cache->scales, cache->status, FPR_STATUS_W_NONFINITE, cache->w_packed,
                           cache->w_packed_t, s);
  });
  return finish();
}

int qkv_forward(const fpr_dims* dims, int32_t n_seq, int32_t seq_len, const uint16_t* x,
                const fpr_weight_cache* cache, uint16_t* q, uint16_t* k, uint16_t* v,
                void* saved, size_t saved_bytes, void* workspace, size_t workspace_bytes,
                void* stream) {
  int rc = shape_check(dims);
  if (rc) return rc;
  int64_t T;
  if ((rc = tokens_check(n_seq, seq_len, &T)) || (rc = cache_check(cache))) return rc;
  if (!x || !q || !k || !v || !saved || !workspace) return FPR_ERR_ARG;
  if (!al16(x) || !al16(q) || !al16(k) || !al16(v) || !al16(saved) || !al16(workspace))
    return FPR_ERR_ALIGN;
  const Plan p = make_plan(dims, T);
  if (!plan_ok(p)) return FPR_ERR_SHAPE;
  if (saved_bytes < p.saved_total || workspace_bytes < p.fwd_total) return FPR_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  uint32_t* parts = at<uint32_t>(workspace, p.f_part);
  float* xsc = at<float>(saved, p.s_xsc);
  uint8_t* x8 = at<uint8_t>(saved, p.s_x8);
  stage("amax_x", s, [&] { fpr::launch_amax_bf16(x, T * p.D, parts, p.f_parts, s); });
  stage("quantize_x", s, [&] {
    fpr::launch_quantize_act(x, T, p.D, parts, p.f_parts, xsc, cache->status,
                             FPR_STATUS_X_NONFINITE, x8, p.Tp, s);
  });
  forward_gemm(dims, p, n_seq, seq_len, cache, q, k, v, saved, workspace, s);
  return finish();
}

int qkv_pack_forward(const fpr_dims* dims, const float* wq, int64_t ldq, const float* wk,
                     int64_t ldk, const float* wv, int64_t ldv, const fpr_weight_cache* cache,
                     int32_t n_seq, int32_t seq_len, const uint16_t* x, uint16_t* q, uint16_t* k,
                     uint16_t* v, void* saved, size_t saved_bytes, void* workspace,
                     size_t workspace_bytes, void* stream) {
  int rc = shape_check(dims);
  if (rc) return rc;
  int64_t T;
  if ((rc = tokens_check(n_seq, seq_len, &T)) || (rc = cache_check(cache))) return rc;
  const Plan p = make_plan(dims, T);
  if ((rc = ld_check(ldq, p.nq, wq)) || (rc = ld_check(ldk, p.nq, wk)) ||
      (rc = ld_check(ldv, (int64_t)p.H * p.dv, wv)))
    return rc;
  if (!x || !q || !k || !v || !saved || !workspace) return FPR_ERR_ARG;
  if (!al16(x) || !al16(q) || !al16(k) || !al16(v) || !al16(saved) || !al16(workspace))
    return FPR_ERR_ALIGN;
  if (!plan_ok(p)) return FPR_ERR_SHAPE;
  if (saved_bytes < p.saved_total || workspace_bytes < pack_forward_bytes(p))
    return FPR_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  void* fws = static_cast<uint8_t*>(workspace) + pack_forward_off(p);
  uint32_t* px = at<uint32_t>(fws, p.f_part);
  float* xsc = at<float>(saved, p.s_xsc);
  uint8_t* x8 = at<uint8_t>(saved, p.s_x8);
  const fpr::WeightJob job{wq, ldq, wk, ldk, wv, ldv, p.D, p.nq, p.N,
                           at<uint32_t>(workspace, p.p_part), cache->scales, cache->w_packed,
                           cache->w_packed_t};
  stage("amax_wx", s, [&] {
    fpr::launch_amax_wx(&job, 1, kPartsW, x, T * p.D, px, p.f_parts, cache->status, s);
  });
  stage("quantize_wx", s, [&] {
    fpr::launch_quantize_wx(&job, 1, kPartsW, FPR_STATUS_W_NONFINITE, x, T, p.D, px, p.f_parts,
                            xsc, FPR_STATUS_X_NONFINITE, x8, p.Tp, cache->status, s);
  });
  forward_gemm(dims, p, n_seq, seq_len, cache, q, k, v, saved, fws, s);
  return finish();
}

int qkv_forward_noalloc(const fpr_dims* dims, int32_t n_seq, int32_t seq_len, const uint16_t* x,
                        const fpr_weight_cache* cache, uint16_t* q, uint16_t* k, uint16_t* v,
                        void* saved, size_t saved_bytes, void* stream) {
  int rc = shape_check(dims);
  if (rc) return rc;
  int64_t T;
  if ((rc = tokens_check(n_seq, seq_len, &T))) return rc;
  if (make_plan(dims, T).fwd_total > kNoAllocScratch) return FPR_ERR_SCRATCH;
  void* ws = device_scratch();
  if (!ws) return FPR_ERR_LAUNCH;
  return qkv_forward(dims, n_seq, seq_len, x, cache, q, k, v, saved, saved_bytes, ws,
                     kNoAllocScratch, stream);
}

size_t fpr_noalloc_scratch_bytes(void) { return kNoAllocScratch; }

int qkv_backward(const fpr_dims* dims, int32_t n_seq, int32_t seq_len, const uint16_t* q,
                 const uint16_t* k, const uint16_t* dq, const uint16_t* dk, const uint16_t* dv,
                 const void* saved, size_t saved_bytes,
                 const fpr_weight_cache* cache, uint16_t* dx, float* dwq, int64_t ldq,
                 float* dwk, int64_t ldk, float* dwv, int64_t ldv, void* workspace,
                 size_t workspace_bytes, void* stream) {
  int rc = shape_check(dims);
  if (rc) return rc;
  int64_t T;
  if ((rc = tokens_check(n_seq, seq_len, &T)) || (rc = cache_check(cache))) return rc;
  const Plan p = make_plan(dims, T);
  if (!plan_ok(p)) return FPR_ERR_SHAPE;
  if ((rc = ld_check(ldq, p.nq, dwq)) || (rc = ld_check(ldk, p.nq, dwk)) ||
      (rc = ld_check(ldv, (int64_t)p.H * p.dv, dwv)))
    return rc;
  if (!q || !k || !dq || !dk || !dv || !saved || !dx || !workspace) return FPR_ERR_ARG;
  if (!al16(q) || !al16(k) || !al16(dq) || !al16(dk) || !al16(dv) || !al16(saved) || !al16(dx) ||
      !al16(workspace))
    return FPR_ERR_ALIGN;
  if (saved_bytes < p.saved_total || workspace_bytes < p.bwd_total) return FPR_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const float* xsc = at<float>(saved, p.s_xsc);
  const uint8_t* x8 = at<uint8_t>(saved, p.s_x8);
  const float* rho = at<float>(saved, p.s_rho);
  uint32_t* parts = at<uint32_t>(workspace, p.b_part);
  float* gsc = at<float>(workspace, p.b_gsc);
  uint8_t* g8 = at<uint8_t>(workspace, p.b_g8);
  float* dwpart = at<float>(workspace, p.b_dwpart);
  stage("amax_dv", s, [&] {
    // dv is read again only after the norm/RoPE backward's 450 MB
    fpr::launch_amax_bf16(dv, T * p.H * p.dv, parts + p.b_nr_parts, p.b_dv_parts, s, true);
  });
  const bool e5 = dims->grad_format == FPR_FORMAT_E5M2;
  if (p.two_pass) {  // "Eight seconds", What generalizes: dQK never reaches memory
    stage("norm_rope_bwd", s, [&] {
      fpr::launch_norm_rope_bwd_amax(dq, dk, q, k, rho, T, seq_len, p.H, p.dqk, p.qs,
                                     dims->rope_base, parts, s);
    });
    stage("quantize_g", s, [&] {
      fpr::launch_norm_rope_bwd_codes(dq, dk, q, k, rho, T, seq_len, p.H, p.dqk, p.qs,
                                      dims->rope_base, parts, p.b_parts, g8, p.N, s, e5);
      fpr::launch_quantize_act_split(nullptr, p.nqk2, dv, p.dv, p.H, seq_len, T, p.N, parts,
                                     p.b_parts, gsc, cache->status, FPR_STATUS_G_NONFINITE, g8,
                                     p.Tp, s, e5);
    });
  } else {
    uint16_t* dqkv = at<uint16_t>(workspace, p.b_dqkv);
    stage("norm_rope_bwd", s, [&] {
      fpr::launch_norm_rope_bwd(dq, dk, q, k, rho, T, seq_len, p.H, p.dqk, p.qs,
                                dims->rope_base, dqkv, parts, s);
    });
    stage("quantize_g", s, [&] {
      fpr::launch_quantize_act_split(dqkv, p.nqk2, dv, p.dv, p.H, seq_len, T, p.N, parts,
                                     p.b_parts, gsc, cache->status, FPR_STATUS_G_NONFINITE, g8,
                                     p.Tp, s, e5);
    });
  }
  stage("gemm_dx", s, [&] {
    fpr::launch_gemm_dx(g8, cache->w_packed, (int)T, p.D, p.N, gsc, cache->scales, dx, s, e5);
  });
  stage("gemm_dw", s, [&] { fpr::launch_gemm_dw(x8, g8, p.D, p.N, p.Tp, dwpart, s, e5); });
  stage("dw_reduce", s, [&] {
    fpr::launch_dw_reduce(dwpart, p.D, p.N, p.Tp, xsc, gsc, dwq, ldq, dwk, ldk, dwv, ldv, p.nq, s);
  });
  return finish();
}

void fpr_trace_set(fpr_trace* trace) { t_trace = trace; }

const char* fpr_status_string(int code) {
  switch (code) {
    case FPR_OK: return "ok";
    case FPR_ERR_ARG: return "invalid argument (null pointer, non-positive size or ld < columns)";
    case FPR_ERR_SHAPE: return "unsupported shape";
    case FPR_ERR_ALIGN: return "misaligned pointer or leading dimension";
    case FPR_ERR_WORKSPACE: return "workspace or saved buffer too small";
    case FPR_ERR_LAUNCH: return "kernel launch failed";
    case FPR_ERR_SCRATCH:
      return "the call needs more workspace than the library's fixed scratch "
             "(fpr_noalloc_scratch_bytes)";
    default: return "unknown status code";
  }
}

// ---- FP8 ReLU^2 MLP

size_t fpr_mlp_workspace_bytes(const fpr_mlp_dims* dims, int64_t tokens, int which) {
  if (mlp_shape_check(dims) != FPR_OK) return 0;
  if (which == FPR_CALL_PACK) return make_mlp_plan(dims, 1).pack_total;
  if (mlp_tokens_check(tokens) != FPR_OK) return 0;
  const MlpPlan p = make_mlp_plan(dims, tokens);
  if (which == FPR_CALL_FORWARD) return p.fwd_total;
  if (which == FPR_CALL_BACKWARD) return p.bwd_total;
  if (which == FPR_CALL_PACK_FORWARD) return mlp_pack_forward_bytes(p);
  return 0;
}

size_t fpr_mlp_saved_bytes(const fpr_mlp_dims* dims, int64_t tokens) {
  if (mlp_shape_check(dims) != FPR_OK || mlp_tokens_check(tokens) != FPR_OK) return 0;
  return make_mlp_plan(dims, tokens).saved_total;
}

int fpr_mlp_get_layout(const fpr_mlp_dims* dims, int64_t tokens, fpr_mlp_layout* out) {
  int rc = mlp_shape_check(dims);
  if (rc || (rc = mlp_tokens_check(tokens))) return rc;
  if (!out) return FPR_ERR_ARG;
  const MlpPlan p = make_mlp_plan(dims, tokens);
  out->tokens = p.T;
  out->tokens_padded = p.Tp;
  out->saved_x8 = p.s_x8;
  out->saved_h8 = p.s_h8;
  out->saved_x_scales = p.s_xsc;
  out->saved_h_scales = p.s_hsc;
  out->fwd_h = p.f_h;
  out->bwd_dy8 = p.b_dy8;
  out->bwd_dy_scales = p.b_dysc;
  out->bwd_dpre = p.b_dpre;
  out->bwd_dpre8 = p.b_dp8;
  out->bwd_dpre_scales = p.b_dpsc;
  out->bwd_dw_part = p.b_dwpart;
  out->dw1_splits = fpr::dw_splits(p.D, p.F, p.Tp);
  out->dw2_splits = fpr::dw_splits(p.F, p.D, p.Tp);
  return FPR_OK;
}

int mlp_pack_quantize_weights(const fpr_mlp_dims* dims, const float* w1, int64_t ld1,
                              const float* w2, int64_t ld2, const fpr_mlp_cache* cache,
                              void* workspace, size_t workspace_bytes, void* stream) {
  int rc = mlp_shape_check(dims);
  if (rc) return rc;
  const MlpPlan p = make_mlp_plan(dims, 1);
  if ((rc = ld_check(ld1, p.F, w1)) || (rc = ld_check(ld2, p.D, w2)) ||
      (rc = mlp_cache_check(cache)))
    return rc;
  if (!workspace) return FPR_ERR_ARG;
  if (!al16(workspace)) return FPR_ERR_ALIGN;
  if (workspace_bytes < p.pack_total) return FPR_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  uint32_t* parts = at<uint32_t>(workspace, p.p_part);
  // a single matrix is the packed-weight case with all columns in one piece
  stage("mlp_amax_w", s, [&] {
    fpr::launch_amax_w(w1, ld1, w1, ld1, w1, ld1, p.D, p.F, p.F, parts, kPartsW, s);
  });
  stage("mlp_quantize_w", s, [&] {
    fpr::launch_quantize_w(w1, ld1, w1, ld1, w1, ld1, p.D, p.F, p.F, parts, kPartsW,
                           cache->scales, cache->status, FPR_STATUS_W_NONFINITE, cache->w1,
                           cache->w1_t, s, true);
  });
  stage("mlp_amax_w", s, [&] {
    fpr::launch_amax_w(w2, ld2, w2, ld2, w2, ld2, p.F, p.D, p.D, parts, kPartsW, s);
  });
  stage("mlp_quantize_w", s, [&] {
    fpr::launch_quantize_w(w2, ld2, w2, ld2, w2, ld2, p.F, p.D, p.D, parts, kPartsW,
                           cache->scales + 2, cache->status, FPR_STATUS_W_NONFINITE, cache->w2,
                           cache->w2_t, s, false);
  });
  return finish();
}

int mlp_forward(const fpr_mlp_dims* dims, int64_t tokens, const uint16_t* x,
                const fpr_mlp_cache* cache, uint16_t* y, void* saved, size_t saved_bytes,
                void* workspace, size_t workspace_bytes, void* stream) {
  int rc = mlp_shape_check(dims);
  if (rc || (rc = mlp_tokens_check(tokens)) || (rc = mlp_cache_check(cache))) return rc;
  if (!x || !y || !saved || !workspace) return FPR_ERR_ARG;
  if (!al16(x) || !al16(y) || !al16(saved) || !al16(workspace)) return FPR_ERR_ALIGN;
  const MlpPlan p = make_mlp_plan(dims, tokens);
  if (saved_bytes < p.saved_total || workspace_bytes < p.fwd_total) return FPR_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const int64_t T = p.T;
  uint32_t* xparts = at<uint32_t>(workspace, p.f_xpart);
  uint8_t* x8 = at<uint8_t>(saved, p.s_x8);
  float* xsc = at<float>(saved, p.s_xsc);
  stage("mlp_amax_x", s, [&] { fpr::launch_amax_bf16(x, T * p.D, xparts, p.x_parts, s); });
  stage("mlp_quantize_x", s, [&] {
    fpr::launch_quantize_act(x, T, p.D, xparts, p.x_parts, xsc, cache->status,
                             FPR_STATUS_X_NONFINITE, x8, p.Tp, s);
  });
  mlp_forward_gemms(p, cache, y, saved, workspace, s);
  return finish();
}

int mlp_pack_forward(const fpr_mlp_dims* dims, const float* w1, int64_t ld1, const float* w2,
                     int64_t ld2, const fpr_mlp_cache* cache, int64_t tokens, const uint16_t* x,
                     uint16_t* y, void* saved, size_t saved_bytes, void* workspace,
                     size_t workspace_bytes, void* stream) {
  int rc = mlp_shape_check(dims);
  if (rc || (rc = mlp_tokens_check(tokens)) || (rc = mlp_cache_check(cache))) return rc;
  const MlpPlan p = make_mlp_plan(dims, tokens);
  if ((rc = ld_check(ld1, p.F, w1)) || (rc = ld_check(ld2, p.D, w2))) return rc;
  if (!x || !y || !saved || !workspace) return FPR_ERR_ARG;
  if (!al16(x) || !al16(y) || !al16(saved) || !al16(workspace)) return FPR_ERR_ALIGN;
  if (saved_bytes < p.saved_total || workspace_bytes < mlp_pack_forward_bytes(p))
    return FPR_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const int64_t T = p.T;
  void* fws = static_cast<uint8_t*>(workspace) + mlp_pack_forward_off();
  uint32_t* xparts = at<uint32_t>(fws, p.f_xpart);
  uint8_t* x8 = at<uint8_t>(saved, p.s_x8);
  float* xsc = at<float>(saved, p.s_xsc);
  uint32_t* wparts = at<uint32_t>(workspace, 0);
  // each matrix is the packed-weight case with all columns in one piece
  const fpr::WeightJob jobs[2] = {
      {w1, ld1, w1, ld1, w1, ld1, p.D, p.F, p.F, wparts, cache->scales, cache->w1, cache->w1_t},
      {w2, ld2, w2, ld2, w2, ld2, p.F, p.D, p.D, wparts + kPartsW, cache->scales + 2, cache->w2,
       cache->w2_t}};
  stage("mlp_amax_wx", s, [&] {
    fpr::launch_amax_wx(jobs, 2, kPartsW, x, T * p.D, xparts, p.x_parts, cache->status, s);
  });
  stage("mlp_quantize_wx", s, [&] {
    fpr::launch_quantize_wx(jobs, 2, kPartsW, FPR_STATUS_W_NONFINITE, x, T, p.D, xparts,
                            p.x_parts, xsc, FPR_STATUS_X_NONFINITE, x8, p.Tp, cache->status, s);
  });
  mlp_forward_gemms(p, cache, y, saved, fws, s);
  return finish();
}

int mlp_backward(const fpr_mlp_dims* dims, int64_t tokens, const uint16_t* dy,
                 const void* saved, size_t saved_bytes, const fpr_mlp_cache* cache,
                 uint16_t* dx, float* dw1, int64_t ld1, float* dw2, int64_t ld2,
                 void* workspace, size_t workspace_bytes, void* stream) {
  int rc = mlp_shape_check(dims);
  if (rc || (rc = mlp_tokens_check(tokens)) || (rc = mlp_cache_check(cache))) return rc;
  const MlpPlan p = make_mlp_plan(dims, tokens);
  if ((rc = ld_check(ld1, p.F, dw1)) || (rc = ld_check(ld2, p.D, dw2))) return rc;
  if (!dy || !saved || !dx || !workspace) return FPR_ERR_ARG;
  if (!al16(dy) || !al16(saved) || !al16(dx) || !al16(workspace)) return FPR_ERR_ALIGN;
  if (saved_bytes < p.saved_total || workspace_bytes < p.bwd_total) return FPR_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const int64_t T = p.T;
  const uint8_t* x8 = at<uint8_t>(saved, p.s_x8);
  const uint8_t* h8 = at<uint8_t>(saved, p.s_h8);
  const float* xsc = at<float>(saved, p.s_xsc);
  const float* hsc = at<float>(saved, p.s_hsc);
  uint32_t* dyparts = at<uint32_t>(workspace, p.b_dypart);
  float* dysc = at<float>(workspace, p.b_dysc);
  uint8_t* dy8 = at<uint8_t>(workspace, p.b_dy8);
  uint16_t* dpre = at<uint16_t>(workspace, p.b_dpre);
  uint32_t* dpparts = at<uint32_t>(workspace, p.b_dppart);
  float* dpsc = at<float>(workspace, p.b_dpsc);
  uint8_t* dp8 = at<uint8_t>(workspace, p.b_dp8);
  float* dwpart = at<float>(workspace, p.b_dwpart);
  int np = 0;
  const bool e5 = dims->grad_format == FPR_FORMAT_E5M2;
  stage("mlp_amax_dy", s, [&] { fpr::launch_amax_bf16(dy, T * p.D, dyparts, p.x_parts, s); });
  stage("mlp_quantize_dy", s, [&] {
    fpr::launch_quantize_act_split(dy, p.D, nullptr, 1, 1, 1, T, p.D, dyparts, p.x_parts, dysc,
                                   cache->status, FPR_STATUS_G_NONFINITE, dy8, p.Tp, s, e5);
  });
  stage("mlp_gemm_dh", s, [&] {
    np = fpr::launch_gemm_dpre(dy8, cache->w2, (int)T, p.F, p.D, dysc, cache->scales + 2, h8,
                               hsc, dpre, dpparts, s, e5);
  });
  stage("mlp_quantize_dpre", s, [&] {
    fpr::launch_quantize_act_split(dpre, p.F, nullptr, 1, 1, 1, T, p.F, dpparts, np, dpsc,
                                   cache->status, FPR_STATUS_H_NONFINITE, dp8, p.Tp, s, e5);
  });
  stage("mlp_gemm_dx", s, [&] {
    fpr::launch_gemm_dx(dp8, cache->w1, (int)T, p.D, p.F, dpsc, cache->scales, dx, s, e5);
  });
  // one column block covers the whole output (nq = its width)
  stage("mlp_gemm_dw1", s, [&] {
    fpr::launch_gemm_dw(x8, dp8, p.D, p.F, p.Tp, dwpart, s, e5);
  });
  stage("mlp_dw1_reduce", s, [&] {
    fpr::launch_dw_reduce(dwpart, p.D, p.F, p.Tp, xsc, dpsc, dw1, ld1, dw1, ld1, dw1, ld1, p.F,
                          s);
  });
  stage("mlp_gemm_dw2", s, [&] {
    fpr::launch_gemm_dw(h8, dy8, p.F, p.D, p.Tp, dwpart, s, e5);
  });
  stage("mlp_dw2_reduce", s, [&] {
    fpr::launch_dw_reduce(dwpart, p.F, p.D, p.Tp, hsc, dysc, dw2, ld2, dw2, ld2, dw2, ld2, p.D,
                          s);
  });
  return finish();
}

int fpr_e4m3_encode(const float* in, int64_t n, float inv_scale, uint8_t* out, void* stream) {
  if (!in || !out || n <= 0) return FPR_ERR_ARG;
  if (!al16(in) || !al16(out) || n % 16) return FPR_ERR_ALIGN;
  (void)hipGetLastError();
  fpr::launch_encode(in, n, inv_scale, out, static_cast<hipStream_t>(stream), false);
  return finish();
}

int fpr_probe_copy(const void* src, void* dst, int64_t bytes, int blocks, void* stream) {
  if (!src || !dst || bytes <= 0 || blocks <= 0) return FPR_ERR_ARG;
  if (!al16(src) || !al16(dst) || bytes % 16) return FPR_ERR_ALIGN;
  (void)hipGetLastError();
  fpr::launch_probe_copy(src, dst, bytes, blocks, static_cast<hipStream_t>(stream));
  return finish();
}

int fpr_probe_read(const void* src, int64_t bytes, uint32_t* out, int blocks, void* stream) {
  if (!src || !out || bytes <= 0 || blocks <= 0) return FPR_ERR_ARG;
  if (!al16(src) || bytes % 16) return FPR_ERR_ALIGN;
  (void)hipGetLastError();
  fpr::launch_probe_read(src, bytes, out, blocks, static_cast<hipStream_t>(stream));
  return finish();
}

int64_t fpr_probe_mfma(int blocks, int iters, float* out, void* stream) {
  if (!out || blocks <= 0 || iters <= 0) return -FPR_ERR_ARG;
  (void)hipGetLastError();
  fpr::launch_probe_mfma(blocks, iters, out, static_cast<hipStream_t>(stream));
  return finish() == FPR_OK ? fpr::probe_mfma_flop(blocks, iters) : -FPR_ERR_LAUNCH;
}

int fpr_e5m2_encode(const float* in, int64_t n, float inv_scale, uint8_t* out, void* stream) {
  if (!in || !out || n <= 0) return FPR_ERR_ARG;
  if (!al16(in) || !al16(out) || n % 16) return FPR_ERR_ALIGN;
  (void)hipGetLastError();
  fpr::launch_encode(in, n, inv_scale, out, static_cast<hipStream_t>(stream), true);
  return finish();
}

}  // extern "C"
