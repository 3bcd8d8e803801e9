// Host-side launchers of the gfx950 kernels (internal to libfpr.so).
// Every launcher enqueues on `s` and returns; errors surface through
// hipGetLastError() in the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace fpr {

// Largest token count a call accepts.  The GEMMs address a tile's rows by
// 32-bit offsets from its first row, (tile rows - 1) * stride + 128 bytes,
// and the dW stride is the padded token count.
constexpr int64_t kMaxTokens = int64_t(1) << 24;

// ---- quantize.hip --------------------------------------------------------

// Per-block max |w| over the logical W_packed [D][N] read from its three
// pieces; writes `parts` fp32 bit patterns (as uint32) to `partials`.
void launch_amax_w(const float* wq, int64_t ldq, const float* wk, int64_t ldk,
                   const float* wv, int64_t ldv, int D, int nq, int N,
                   uint32_t* partials, int parts, hipStream_t s);

// Per-block max |x| of n bf16 values (n % 8 == 0).  stream: non-temporal
// loads, for a tensor whose quantiser does not follow at once.
void launch_amax_bf16(const uint16_t* x, int64_t n, uint32_t* partials, int parts,
                      hipStream_t s, bool stream = false);

// The quantisers below take the `parts` amax partials of their tensor and
// reduce them to the scales (scales[0] = s, scales[1] = inv, which they also
// write); a non-finite amax sets `status_bit` in *status (the weight
// quantiser overwrites *status, the activation one ORs into it).

// Quantise W_packed and write both layouts: w_packed [D][N], w_packed_t [N][D].
// A single matrix is the case nq = N (all three pieces the same pointer).
// With reset_status false the status bit is ORed in rather than *status
// overwritten (the second of two weights quantised into one cache).
void launch_quantize_w(const float* wq, int64_t ldq, const float* wk, int64_t ldk,
                       const float* wv, int64_t ldv, int D, int nq, int N,
                       const uint32_t* partials, int parts, float* scales, int32_t* status,
                       int status_bit, uint8_t* w_packed, uint8_t* w_packed_t, hipStream_t s,
                       bool reset_status = true);

// The weight pack and x's quantiser sharing launches: one launch takes both
// amaxes (parts_w W blocks, then parts_x x blocks; block 0 clears *status),
// the next writes both codes (W's both layouts and scales with bit w_bit,
// x8 and its scales with x_bit, as the separate launchers do).
// The weight pack and x's quantiser in two shared launches, for one weight
// (the packed QKV weight) or two (the MLP's W1 and W2; njobs <= 2).  A job
// names a weight as launch_amax_w does, its parts_w amax partials, its
// scales and both code layouts.  The amax launch clears *status first.
struct WeightJob {
  const float* wq;
  int64_t ldq;
  const float* wk;
  int64_t ldk;
  const float* wv;
  int64_t ldv;
  int D, nq, N;
  uint32_t* partials;
  float* scales;
  uint8_t* packed;
  uint8_t* packed_t;
};
void launch_amax_wx(const WeightJob* jobs, int njobs, int parts_w, const uint16_t* x, int64_t n,
                    uint32_t* px, int parts_x, int32_t* status, hipStream_t s);
void launch_quantize_wx(const WeightJob* jobs, int njobs, int parts_w, int w_bit,
                        const uint16_t* x, int64_t rows, int cols, const uint32_t* px,
                        int parts_x, float* x_scales, int x_bit, uint8_t* x8,
                        int64_t tokens_padded, int32_t* status, hipStream_t s);

// Blocked layout of the FP8 activation copies x8 and g8, which only the
// GEMMs read.  A matrix of R rows (tokens) and K columns (K contiguous) is
// stored as blocks of kActRows rows x kKBlock bytes: block
// (R / kActRows, K / kKBlock) at ((r_blk * ceil(K / kKBlock) + k_blk) *
// kActRows) * kKBlock, rows kKBlock bytes apart inside.  One K step of a
// forward / dX tile (the A operand) is one contiguous block, and one K step
// of dW (128 tokens of x8 and g8) is half a block row.
constexpr int kKBlock = 128, kActRows = 256;
inline size_t act_blocked_bytes(int64_t rows, int64_t cols) {
  return (size_t)round_up(rows, kActRows) * (size_t)round_up(cols, kKBlock);
}

// Quantise a [rows][cols] bf16 matrix with its per-tensor scale (from the
// partials, as above) into dst (blocked row layout; columns cols .. multiple
// of kKBlock and rows rows .. tokens_padded written as zero, the latter
// being the dW GEMM's K tail).  cols % 16 == 0, tokens_padded % kKBlock ==
// 0.  Rows from tokens_padded to the end of the last block of rows are left
// unwritten: no GEMM reads them.
void launch_quantize_act(const uint16_t* src, int64_t rows, int cols, const uint32_t* partials,
                         int parts, float* scales, int32_t* status, int status_bit, uint8_t* dst,
                         int64_t tokens_padded, hipStream_t s);

// The same for rows whose first `split` columns come from src [rows][split]
// and the rest from head-major rows: column split + h * vw + j of token t is
// element j of row (t / vs * vh + h) * vs + t % vs of vsrc (the packed
// gradient: dQK, then dv [n_seq][H][S][d_v]).  split % 16 == 0, vw % 16 == 0.
// With src null, columns below split of the rows < rows are neither read nor
// written (another kernel writes their codes); their padding rows still are.
void launch_quantize_act_split(const uint16_t* src, int split, const uint16_t* vsrc, int vw,
                               int vh, int vs, int64_t rows, int cols, const uint32_t* partials,
                               int parts, float* scales, int32_t* status, int status_bit,
                               uint8_t* dst, int64_t tokens_padded, hipStream_t s,
                               bool e5m2 = false);

// e4m3 (or e5m2) codes of in[i] * inv, no amax: the encoder hooks.
void launch_encode(const float* in, int64_t n, float inv, uint8_t* out, hipStream_t s,
                   bool e5m2 = false);

// ---- gemm.hip --------------------------------------------------------------

// Forward: Y = s_x s_w x8 @ W_packed, M = T rows, N packed columns, K = D.
// Q|K columns go to qk_pre [T][nqk2] bf16; V columns to v head-major.  (The
// path for head widths without a fused forward, below.)
void launch_gemm_fwd(const uint8_t* x8, const uint8_t* w_packed_t, int T, int N, int D,
                     const float* x_scales, const float* w_scales, uint16_t* qk_pre, int nqk2,
                     uint16_t* v, int H, int d_v, int seq_len, hipStream_t s);

// Whether the forward GEMM carries the norm and RoPE in its epilogue: head
// widths 64, 96 and 128, packed weight (N x D bytes) under 2 GiB.
bool fused_forward(int d_qk, int64_t N, int D);

// Forward with RMSNorm and RoPE in the GEMM's epilogue: q, k head-major rows
// of qs >= d_qk elements (columns d_qk .. qs - 1 written as zero), v
// head-major, and rho [2][n_seq][H][S] fp32 = 1 / rms of every q, then every
// k head row (of the bf16-rounded product).
void launch_gemm_qkv_fwd(const uint8_t* x8, const uint8_t* w_packed_t, int n_seq, int seq_len,
                         int D, int H, int d_qk, int d_v, int qs, float eps, float base,
                         const float* x_scales, const float* w_scales, uint16_t* q, uint16_t* k,
                         uint16_t* v, float* rho, hipStream_t s);

// dX = s_g s_w g8 @ W_packed^T: M = T, N = D, K = N_packed; dx [T][D] bf16.
// g_e5m2: g8 holds e5m2 codes (else e4m3); the weight codes are e4m3.
void launch_gemm_dx(const uint8_t* g8, const uint8_t* w_packed, int T, int D, int Np,
                    const float* g_scales, const float* w_scales, uint16_t* dx, hipStream_t s,
                    bool g_e5m2 = false);

// FP8 ReLU^2 MLP (W1 [D][F], W2 [F][D]; activations in the blocked row
// layout).  h = relu(s_x s_w1 x8 @ W1)^2 into h [T][F] bf16, through the
// cached W1^T codes w1_t [F][D]; and dpre = 2 (s_dy s_w2 dy8 @ W2^T)
// sqrt(s_h dec(h8)) into dpre [T][F] bf16, through the cached W2 codes
// w2 [F][D].  Both write one amax partial per matrix wave and return how
// many (at most gemm_amax_slots_max()).  The MLP's y = h8 @ W2 and
// dX = dpre8 @ W1^T are launch_gemm_dx with B = W2^T codes [D][F] and
// W1 codes [D][F].
int gemm_amax_slots_max();
int launch_gemm_relu2(const uint8_t* x8, const uint8_t* w1_t, int T, int F, int D,
                      const float* x_scales, const float* w_scales, uint16_t* h,
                      uint32_t* partials, hipStream_t s);
int launch_gemm_dpre(const uint8_t* dy8, const uint8_t* w2, int T, int F, int D,
                     const float* dy_scales, const float* w_scales, const uint8_t* h8,
                     const float* h_scales, uint16_t* dpre, uint32_t* partials, hipStream_t s,
                     bool dy_e5m2 = false);

// Number of K splits the dW GEMM uses, and its partial-buffer size.
int dw_splits(int D, int Np, int64_t tokens_padded);
size_t dw_partial_bytes(int D, int Np, int64_t tokens_padded);

// dW = s_x s_g x^T g: M = D, N = N_packed, K = tokens (padded, zero tail).
// x8 [T][D], g8 [T][Np] in the blocked row layout, rows T .. Tp - 1 zero;
// unscaled split-K partial sums go to `part` [dw_splits][D][Np] fp32 ...
void launch_gemm_dw(const uint8_t* x8, const uint8_t* g8, int D, int Np, int64_t Tp,
                    float* part, hipStream_t s,
                    bool g_e5m2 = false);
// ... and are summed in split order, scaled by s_x s_g and written into the
// three column blocks dwq [D][nq] (ldq), dwk, dwv [D][N - 2nq] (ldv).
void launch_dw_reduce(const float* part, int D, int Np, int64_t Tp, const float* x_scales,
                      const float* g_scales, float* dwq, int64_t ldq, float* dwk, int64_t ldk,
                      float* dwv, int64_t ldv, int nq, hipStream_t s);

// ---- epilogue.hip ----------------------------------------------------------

// Dynamic LDS bytes of the two epilogue kernels (callers keep them <= 64 KiB);
// 0 for d_qk = 64, 96, 128, whose kernels use only static LDS.
size_t norm_rope_fwd_lds(int H, int d_qk);
size_t norm_rope_bwd_lds(int H, int d_qk);

// Forward norm/RoPE for head widths without a fused forward: pre-norm Q|K
// rows (qk_pre [T][2*H*d_qk] bf16) -> RMSNorm -> RoPE -> head-major q, k
// with rows of qs >= d_qk elements (a multiple of 8), columns d_qk .. qs - 1
// written as zero, and rho [2][n_seq][H][S] = 1 / rms of each row.
void launch_norm_rope_fwd(const uint16_t* qk_pre, int64_t T, int seq_len, int H, int d_qk,
                          int qs, float eps, float base, uint16_t* q, uint16_t* k, float* rho,
                          hipStream_t s);

// Backward epilogue from the forward's outputs: dq, dk, q, k (head-major,
// rows of qs elements of which the first d_qk are read) and rho -> the Q|K
// part of the packed gradient, dQK [T][2 H d_qk] bf16, plus one amax partial
// per block over dQK; norm_rope_bwd_blocks() is that block count (at most
// 1024).  (dv's amax is taken by launch_amax_bf16.)
int norm_rope_bwd_blocks(int64_t T, int H, int d_qk);
void launch_norm_rope_bwd(const uint16_t* dq, const uint16_t* dk, const uint16_t* q,
                          const uint16_t* k, const float* rho, int64_t T, int seq_len, int H,
                          int d_qk, int qs, float base, uint16_t* dqkv, uint32_t* partials,
                          hipStream_t s);

// The same backward in two passes that never write dQK (d_qk 64, 96, 128
// only, norm_rope_bwd_two_pass()): the first leaves only the amax partials;
// the second, after dv's partials are in too, recomputes every row and
// encodes it with the gradient scale straight into the Q|K columns of the
// gradient codes g8 (blocked row layout, N columns), the same codes the
// quantiser would write from dQK.  Rows T .. of g8 are not written.
bool norm_rope_bwd_two_pass(int d_qk);
void launch_norm_rope_bwd_amax(const uint16_t* dq, const uint16_t* dk, const uint16_t* q,
                               const uint16_t* k, const float* rho, int64_t T, int seq_len, int H,
                               int d_qk, int qs, float base, uint32_t* partials, hipStream_t s);
void launch_norm_rope_bwd_codes(const uint16_t* dq, const uint16_t* dk, const uint16_t* q,
                                const uint16_t* k, const float* rho, int64_t T, int seq_len,
                                int H, int d_qk, int qs, float base, const uint32_t* partials,
                                int parts, uint8_t* g8, int N, hipStream_t s, bool e5m2);

// ---- probe.hip: measured ceilings -------------------------------------------

// Streaming copy of `bytes` (a multiple of 16) from src to dst.
void launch_probe_copy(const void* src, void* dst, int64_t bytes, int blocks, hipStream_t s);
// Streaming read of `bytes` (a multiple of 16); one word per block to out.
void launch_probe_read(const void* src, int64_t bytes, uint32_t* out, int blocks, hipStream_t s);
// `blocks` blocks of 8 waves, each `iters` rounds of 4 independent FP8 MFMAs;
// one float per wave to out (blocks * 8).
void launch_probe_mfma(int blocks, int iters, float* out, hipStream_t s);
int64_t probe_mfma_flop(int blocks, int iters);

}  // namespace fpr
