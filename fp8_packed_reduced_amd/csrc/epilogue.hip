// Fused layout kernels around the packed GEMM, for gfx950.
//
// Forward ("96 is enough", "The change": split, rms_norm(q), rms_norm(k),
// rope(q), rope(k); PR #344 page, "Changes": norm, RoPE and layout
// conversion fused, lane swaps kept in registers): pre-norm Q|K rows ->
// u = a / sqrt(mean(a^2) + eps) -> rotate pairs (i, i + d/2) by
// p * base^(-2i/d) -> head-major q, k, whose rows may be padded with zeros
// to a stride qs > d for an attention kernel that wants equal Q/K/V widths
// (the FA3 padding of the PR #344 page, "Changes").
//
// Backward ("Where the eight seconds were hiding", "The inventory": the norm,
// RoPE and backward shuffles): du = R_{-p} dq; da = rho * (du - u <u,du>/d)
// into the Q|K part of the packed gradient, dQK [T][2H d] bf16, with one
// amax partial per block over dQK for the gradient quantiser, which reads
// the V columns straight from dv (whose amax a separate pass takes).
//
// Main kernels (d = 64, 96, 128): four consecutive lanes own one head row
// and every access is a whole 16-byte chunk (below); the row sums take two
// cross-lane steps (DPP quad permutes).  Rotation angles are formed in
// revolutions: position * theta_j / (2 pi) in double, reduced to its
// fractional part, then the hardware sin/cos of that fraction, once per
// token and pair into an LDS table that all heads share.
//
// Fallback kernels (other head widths): work item = (token, head row,
// chunk c), a thread owns the 8 elements [8c, 8c+8) of a row and their
// rotation partners; row sums go through per-item partials in LDS, summed
// in a fixed order.
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace fpr {

// cos/sin of p * base^(-2j/d) for the block's tokens: the angle is formed
// and reduced modulo 2 pi in double (positions reach 65535 rad), then fp32
// sincos of the reduced angle.
__device__ inline void build_rope_table(float2* cs, int tt_count, int64_t t0, int64_t T,
                                        int seq_len, int h, int d, float base) {
  const double two_pi = 6.283185307179586476925286766559;
  const double lg = log2((double)base);
  for (int i = threadIdx.x; i < tt_count * h; i += kThreads) {
    const int tt = i / h, j = i - tt * h;
    const int64_t t = t0 + tt;
    const double p = t < T ? (double)(t % seq_len) : 0.0;
    const double theta = exp2(-(2.0 * j / d) * lg);
    const double phi = p * theta;
    const double r = fma(-rint(phi / two_pi), two_pi, phi);
    float sn, cn;
    sincosf((float)r, &sn, &cn);
    cs[i] = make_float2(cn, sn);
  }
}

__device__ inline void unpack8(uint4 v, float* f) {
  f[0] = bf16_to_f32(v.x & 0xffffu); f[1] = bf16_to_f32(v.x >> 16);
  f[2] = bf16_to_f32(v.y & 0xffffu); f[3] = bf16_to_f32(v.y >> 16);
  f[4] = bf16_to_f32(v.z & 0xffffu); f[5] = bf16_to_f32(v.z >> 16);
  f[6] = bf16_to_f32(v.w & 0xffffu); f[7] = bf16_to_f32(v.w >> 16);
}

__device__ inline uint4 pack8(const float* f) {
  return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                    pack_bf16x2(f[6], f[7]));
}

__device__ inline uint32_t absmax8(uint4 v) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w}, m = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t lo = w[j] & 0x7fffu, hi = (w[j] >> 16) & 0x7fffu;
    m = m > lo ? m : lo;
    m = m > hi ? m : hi;
  }
  return m;
}

// ------------------------------------------------------- shared helpers

// theta_j / (2 pi) = base^(-2j/d) / (2 pi), j < h, for the block.
__device__ inline void build_rev_table(double* rev, int h, int d, float base) {
  const double lg = log2((double)base);
  for (int j = threadIdx.x; j < h; j += kThreads)
    rev[j] = exp2(-(2.0 * j / d) * lg) * 0.15915494309189533576888376337251;
  __syncthreads();
}

// cos / sin of the angle pos * theta_j, from its fractional revolution.
__device__ inline void rope_cs(double rev_j, int64_t pos, float& c, float& s) {
  double r = (double)pos * rev_j;
  r -= rint(r);
  const float f = (float)r;
  s = __builtin_amdgcn_sinf(f);  // sin(2 pi f)
  c = __builtin_amdgcn_cosf(f);
}

__device__ inline float quad_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));  // lane ^ 1
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));  // lane ^ 2
  return v;
}

// ------------------------------------------------- quad-chunk kernels
//
// Four lanes per head row, every access a whole 16-byte chunk (8-byte
// lane accesses split each memory instruction over many partial lines and
// ran ~25% slower here): of the CH = d / 8 chunks of a row, lane l owns
// chunks l, l + 4, l + 8, ... (M = CH / 4 of them), so each load or store
// instruction covers 64 consecutive bytes of every row in the wave.  The
// RoPE partner of chunk c (elements i + d/2 of its elements i) is chunk
// c +- CH/2: for d = 64 and 128 that is another chunk of the same lane;
// for d = 96 it is a chunk of lane l ^ 2, which one DPP quad permute per
// word brings over.  A block takes TT tokens at a time and first builds the
// cos/sin table of their positions (shared by all heads) in LDS.

constexpr int kQuadTT = 16;         // tokens per block iteration
constexpr int kQuadTileBlocks = 1024;

template <int D>
struct QuadChunks {
  static constexpr int CH = D / 8, HC = CH / 2, M = CH / 4, h = D / 2;
  static_assert(CH % 4 == 0, "four lanes per row");
  // chunk of lane l, own slot m
  __device__ static int chunk(int l, int m) { return l + 4 * m; }
  // the slot (in lane l ^ 2 for d = 96, else in lane l) holding the partner of slot m
  __device__ static int partner_slot(int l, int m) {
    if (CH == 12) return (m + (l < 2 ? 1 : 2)) % 3;
    return (m + M / 2) % M;
  }
};

__device__ __forceinline__ uint32_t dpp_quad_xor2(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true);  // [2,3,0,1]
}

// Partner chunks of the lane's M chunks.
template <int D>
__device__ __forceinline__ void quad_partners(const uint4 (&own)[QuadChunks<D>::M],
                                              uint4 (&par)[QuadChunks<D>::M], int l) {
  using Q = QuadChunks<D>;
  if constexpr (Q::CH == 12) {
    uint4 x[3];
#pragma unroll
    for (int m = 0; m < 3; ++m)
      x[m] = make_uint4(dpp_quad_xor2(own[m].x), dpp_quad_xor2(own[m].y), dpp_quad_xor2(own[m].z),
                        dpp_quad_xor2(own[m].w));
    // lanes 0, 1 take slot (m + 1) % 3 of lane l ^ 2, lanes 2, 3 slot (m + 2) % 3
#pragma unroll
    for (int m = 0; m < 3; ++m) par[m] = l < 2 ? x[(m + 1) % 3] : x[(m + 2) % 3];
  } else {
#pragma unroll
    for (int m = 0; m < Q::M; ++m) par[m] = own[(m + Q::M / 2) % Q::M];
  }
}

__device__ __forceinline__ uint4 pack8_rn(const float* f) {
  return make_uint4(cvt_bf16x2_rn(f[0], f[1]), cvt_bf16x2_rn(f[2], f[3]),
                    cvt_bf16x2_rn(f[4], f[5]), cvt_bf16x2_rn(f[6], f[7]));
}

// cos/sin of pairs j < h at the positions of tokens t0 .. t0 + nt - 1, and
// the tokens' sequence indices and positions.
__device__ inline void quad_table(float2* cs, int64_t* bq, int* sp, const double* rev, int64_t t0,
                                  int nt, int h, int seq_len) {
  for (int i = threadIdx.x; i < nt * h; i += kThreads) {
    const int tt = i / h, j = i - tt * h;
    const int64_t t = t0 + tt;
    float cn, sn;
    rope_cs(rev[j], t - (t / seq_len) * seq_len, cn, sn);
    cs[i] = make_float2(cn, sn);
  }
  if (threadIdx.x < nt) {
    const int64_t t = t0 + threadIdx.x;
    bq[threadIdx.x] = t / seq_len;
    sp[threadIdx.x] = (int)(t - (t / seq_len) * seq_len);
  }
}

template <int D>
struct QcFwdRow {
  uint4 own[QuadChunks<D>::M];
  int tt, rr;
  bool ok;
};

template <int D>
__device__ __forceinline__ void qc_fwd_load(QcFwdRow<D>& r, int row, int rows, int R, int64_t t0,
                                            const uint16_t* __restrict__ qk_pre, int l) {
  using Q = QuadChunks<D>;
  r.ok = row < rows;
  if (!r.ok) return;
  r.tt = row / R;
  r.rr = row - r.tt * R;
  const uint16_t* src = qk_pre + ((t0 + r.tt) * R + r.rr) * D;
#pragma unroll
  for (int m = 0; m < Q::M; ++m) r.own[m] = *reinterpret_cast<const uint4*>(src + 8 * Q::chunk(l, m));
}

template <int D>
__device__ __forceinline__ void qc_fwd_finish(const QcFwdRow<D>& r, const float2* cs,
                                              const int64_t* bq, const int* sp, int H,
                                              int seq_len, int qs, float eps,
                                              uint16_t* __restrict__ q,
                                              uint16_t* __restrict__ k, int l) {
  using Q = QuadChunks<D>;
  constexpr int h = Q::h, M = Q::M, HC = Q::HC;
  if (!r.ok) return;
  float ss = 0.f;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    float x[8];
    unpack8(r.own[m], x);
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
  }
  ss = quad_sum(ss);
  const float rho = 1.0f / sqrtf(ss / (float)D + eps);
  uint4 par[M];
  quad_partners<D>(r.own, par, l);
  const int tt = r.tt, rr = r.rr, hh = rr < H ? rr : rr - H;
  uint16_t* dst = (rr < H ? q : k) + ((bq[tt] * H + hh) * seq_len + sp[tt]) * qs;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int c = Q::chunk(l, m);
    const bool lower = c < HC;
    const float2* tab = cs + tt * h + 8 * (lower ? c : c - HC);
    float x[8], y[8], o[8];
    unpack8(r.own[m], x);
    unpack8(par[m], y);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float u = x[e] * rho, w = y[e] * rho, cn = tab[e].x, sn = tab[e].y;
      o[e] = lower ? u * cn - w * sn : u * cn + w * sn;
    }
    *reinterpret_cast<uint4*>(dst + 8 * c) = pack8_rn(o);
  }
  // zero padding chunks CH .. qs / 8 - 1, dealt round the quad like the row's
  for (int c = Q::CH + l; c < qs / 8; c += 4)
    *reinterpret_cast<uint4*>(dst + 8 * c) = make_uint4(0, 0, 0, 0);
}

template <int D>
__global__ __launch_bounds__(kThreads) void norm_rope_fwd_qc(
    const uint16_t* __restrict__ qk_pre, int64_t T, int seq_len, int H, int qs, float eps,
    float base, uint16_t* __restrict__ q, uint16_t* __restrict__ k) {
  using Q = QuadChunks<D>;
  constexpr int h = Q::h, QUADS = kThreads / 4;
  __shared__ double rev[h];
  __shared__ float2 cs[kQuadTT * h];
  __shared__ int64_t bq[kQuadTT];
  __shared__ int sp[kQuadTT];
  build_rev_table(rev, h, D, base);
  const int R = 2 * H, l = threadIdx.x & 3;
  const int64_t groups = ceil_div(T, kQuadTT);
  for (int64_t gi = blockIdx.x; gi < groups; gi += gridDim.x) {
    const int64_t t0 = gi * kQuadTT;
    const int nt = (int)min<int64_t>(kQuadTT, T - t0), rows = nt * R;
    quad_table(cs, bq, sp, rev, t0, nt, h, seq_len);
    __syncthreads();
    for (int row = threadIdx.x >> 2; row < rows; row += 2 * QUADS) {
      QcFwdRow<D> r0, r1;  // two rows' loads in flight per thread
      qc_fwd_load<D>(r0, row, rows, R, t0, qk_pre, l);
      qc_fwd_load<D>(r1, row + QUADS, rows, R, t0, qk_pre, l);
      qc_fwd_finish<D>(r0, cs, bq, sp, H, seq_len, qs, eps, q, k, l);
      qc_fwd_finish<D>(r1, cs, bq, sp, H, seq_len, qs, eps, q, k, l);
    }
    __syncthreads();
  }
}

template <int D>
struct QcBwdRow {
  uint4 a[QuadChunks<D>::M], g[QuadChunks<D>::M];
  int tt, rr;
  bool ok;
};

// Token t (< 2^24, so 32-bit) of the packed rows is position t % seq_len of
// sequence t / seq_len.
template <int D>
__device__ __forceinline__ void qc_bwd_load(QcBwdRow<D>& r, int row, int rows, int R, int H,
                                            int seq_len, int qs, int64_t t0,
                                            const uint16_t* __restrict__ dq,
                                            const uint16_t* __restrict__ dk,
                                            const uint16_t* __restrict__ qk_pre, int l) {
  using Q = QuadChunks<D>;
  r.ok = row < rows;
  if (!r.ok) return;
  const int tt = row / R, rr = row - tt * R, hh = rr < H ? rr : rr - H;
  r.tt = tt;
  r.rr = rr;
  const int t = (int)t0 + tt, b = t / seq_len, sp = t - b * seq_len;
  const uint16_t* asrc = qk_pre + ((t0 + tt) * R + rr) * D;
  const uint16_t* gsrc = (rr < H ? dq : dk) + (((int64_t)b * H + hh) * seq_len + sp) * qs;
#pragma unroll
  for (int m = 0; m < Q::M; ++m) {
    r.a[m] = *reinterpret_cast<const uint4*>(asrc + 8 * Q::chunk(l, m));
    r.g[m] = *reinterpret_cast<const uint4*>(gsrc + 8 * Q::chunk(l, m));
  }
}

// Finishes the row into dQK (rows of N elements) and returns the largest
// |bf16| bit pattern.
template <int D>
__device__ __forceinline__ uint32_t qc_bwd_finish(const QcBwdRow<D>& r, const float2* cs,
                                                  int64_t t0, int N, float eps,
                                                  uint16_t* __restrict__ dqkv, int l) {
  using Q = QuadChunks<D>;
  constexpr int h = Q::h, M = Q::M, HC = Q::HC;
  if (!r.ok) return 0;
  uint4 pg[M];
  quad_partners<D>(r.g, pg, l);
  // own element e of slot m is a_i (lower chunks) or b_i, i = 8 (c mod HC) + e;
  // du = R_{-p} dq
  float du[M][8], ss = 0.f, sd = 0.f;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int c = Q::chunk(l, m);
    const bool lower = c < HC;
    const float2* tab = cs + r.tt * h + 8 * (lower ? c : c - HC);
    float x[8], gx[8], gp[8];
    unpack8(r.a[m], x);
    unpack8(r.g[m], gx);
    unpack8(pg[m], gp);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float cn = tab[e].x, sn = tab[e].y;
      du[m][e] = lower ? gx[e] * cn + gp[e] * sn : gx[e] * cn - gp[e] * sn;
      ss += x[e] * x[e];
      sd += x[e] * du[m][e];
    }
  }
  ss = quad_sum(ss);
  sd = quad_sum(sd);
  const float rho = 1.0f / sqrtf(ss / (float)D + eps);
  // rho^2 <u,du> / d, where <u,du> = rho * sum(a du)
  const float coef = rho * rho * rho * sd / (float)D;
  uint16_t* dst = dqkv + (t0 + r.tt) * N + r.rr * D;
  uint32_t amax = 0;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    float x[8], o[8];
    unpack8(r.a[m], x);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = rho * du[m][e] - coef * x[e];
    const uint4 pk = pack8_rn(o);
    amax = max(amax, absmax8(pk));
    *reinterpret_cast<uint4*>(dst + 8 * Q::chunk(l, m)) = pk;
  }
  return amax;
}

// Per token group, every load is issued before anything waits on one: the
// lane's bwd_rows<D>() head rows (for d = 96 and H = 6, the group's 192
// rows are exactly 3 per quad); the cos/sin table of the group is built
// while they are in flight.  Three rows of d = 128 would not fit two waves
// per SIMD in registers.  The V gradient's amax is a separate streaming
// pass over dv (launch_amax_bf16): reading it here, head-major beside four
// other streams, cost more than that pass.
template <int D>
constexpr int bwd_rows() { return D == 128 ? 2 : 3; }

template <int D>
__global__ __launch_bounds__(kThreads) void norm_rope_bwd_qc(
    const uint16_t* __restrict__ dq, const uint16_t* __restrict__ dk,
    const uint16_t* __restrict__ qk_pre, int64_t T, int seq_len, int H, int qs, float eps,
    float base, uint16_t* __restrict__ dqkv, uint32_t* __restrict__ partials) {
  using Q = QuadChunks<D>;
  constexpr int h = Q::h, QUADS = kThreads / 4, RB = bwd_rows<D>();
  __shared__ double rev[h];
  __shared__ float2 cs[kQuadTT * h];
  __shared__ int64_t bq[kQuadTT];
  __shared__ int sp[kQuadTT];
  __shared__ uint32_t red[4];
  build_rev_table(rev, h, D, base);
  const int R = 2 * H, qkw = R * D, l = threadIdx.x & 3, quad = threadIdx.x >> 2;
  uint32_t amax = 0;
  const int64_t groups = ceil_div(T, kQuadTT);
  for (int64_t gi = blockIdx.x; gi < groups; gi += gridDim.x) {
    const int64_t t0 = gi * kQuadTT;
    const int nt = (int)min<int64_t>(kQuadTT, T - t0), rows = nt * R;
    for (int rb = 0; rb < rows; rb += RB * QUADS) {
      QcBwdRow<D> r[RB];
#pragma unroll
      for (int j = 0; j < RB; ++j)
        qc_bwd_load<D>(r[j], rb + quad + j * QUADS, rows, R, H, seq_len, qs, t0, dq, dk, qk_pre,
                       l);
      if (rb == 0) {  // the same for every thread: rows > 0
        quad_table(cs, bq, sp, rev, t0, nt, h, seq_len);
        __syncthreads();
      }
#pragma unroll
      for (int j = 0; j < RB; ++j)
        amax = max(amax, qc_bwd_finish<D>(r[j], cs, t0, qkw, eps, dqkv, l));
    }
    __syncthreads();
  }
  amax = block_max_u32(amax << 16, red);
  if (threadIdx.x == 0) partials[blockIdx.x] = amax;
}

// ------------------------------------------------------------- forward

template <int TT>
__global__ __launch_bounds__(kThreads) void norm_rope_fwd_kernel(
    const uint16_t* __restrict__ qk_pre, int64_t T, int seq_len, int H, int d, int qs,
    float eps, float base, uint16_t* __restrict__ q, uint16_t* __restrict__ k) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int h = d / 2, C = h / 8, R = 2 * H, rowlen = R * d;
  const int items = TT * R * C;
  uint4* data = reinterpret_cast<uint4*>(smem);                  // [items][2]
  float* part = reinterpret_cast<float*>(data + 2 * items);      // [items]
  float2* cs = reinterpret_cast<float2*>(part + items);          // [TT][h]
  const int64_t t0 = (int64_t)blockIdx.x * TT;

  build_rope_table(cs, TT, t0, T, seq_len, h, d, base);
  for (int it = threadIdx.x; it < items; it += kThreads) {
    const int c = it % C, rr = (it / C) % R, tt = it / (C * R);
    const int64_t t = t0 + tt;
    uint4 lo = make_uint4(0, 0, 0, 0), hi = lo;
    if (t < T) {
      const uint16_t* row = qk_pre + t * rowlen + rr * d;
      lo = *reinterpret_cast<const uint4*>(row + 8 * c);
      hi = *reinterpret_cast<const uint4*>(row + h + 8 * c);
    }
    float a[8], b[8];
    unpack8(lo, a);
    unpack8(hi, b);
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) ss += a[j] * a[j] + b[j] * b[j];
    data[2 * it] = lo;
    data[2 * it + 1] = hi;
    part[it] = ss;
  }
  __syncthreads();
  for (int it = threadIdx.x; it < items; it += kThreads) {
    const int c = it % C, rr = (it / C) % R, tt = it / (C * R);
    const int64_t t = t0 + tt;
    if (t >= T) continue;
    float ss = 0.f;
    const int first = it - c;
    for (int j = 0; j < C; ++j) ss += part[first + j];
    const float rho = 1.0f / sqrtf(ss / (float)d + eps);
    float a[8], b[8], oa[8], ob[8];
    unpack8(data[2 * it], a);
    unpack8(data[2 * it + 1], b);
    const float2* tab = cs + tt * h + 8 * c;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float ua = a[j] * rho, ub = b[j] * rho;
      const float cn = tab[j].x, sn = tab[j].y;
      oa[j] = ua * cn - ub * sn;
      ob[j] = ub * cn + ua * sn;
    }
    const int64_t bseq = t / seq_len, s = t - bseq * seq_len;
    uint16_t* dst = rr < H ? q + ((bseq * H + rr) * seq_len + s) * qs
                           : k + ((bseq * H + (rr - H)) * seq_len + s) * qs;
    *reinterpret_cast<uint4*>(dst + 8 * c) = pack8(oa);
    *reinterpret_cast<uint4*>(dst + h + 8 * c) = pack8(ob);
  }
  // zero padding columns d .. qs - 1 of every row
  const int pc = (qs - d) / 8, pitems = TT * R * pc;
  for (int it = threadIdx.x; it < pitems; it += kThreads) {
    const int c = it % pc, rr = (it / pc) % R, tt = it / (pc * R);
    const int64_t t = t0 + tt;
    if (t >= T) continue;
    const int64_t bseq = t / seq_len, s = t - bseq * seq_len;
    uint16_t* dst = (rr < H ? q : k) + ((bseq * H + (rr < H ? rr : rr - H)) * seq_len + s) * qs;
    *reinterpret_cast<uint4*>(dst + d + 8 * c) = make_uint4(0, 0, 0, 0);
  }
}

// ------------------------------------------------------------ backward

template <int TT>
__global__ __launch_bounds__(kThreads) void norm_rope_bwd_kernel(
    const uint16_t* __restrict__ dq, const uint16_t* __restrict__ dk,
    const uint16_t* __restrict__ qk_pre, int64_t T, int seq_len, int H, int d, int qs,
    float eps, float base, uint16_t* __restrict__ dqkv, uint32_t* __restrict__ partials) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ uint32_t red[4];
  const int h = d / 2, C = h / 8, R = 2 * H, qkw = R * d;
  const int items = TT * R * C;
  uint4* data = reinterpret_cast<uint4*>(smem);                  // [items][4]: a lo/hi, g lo/hi
  float* part = reinterpret_cast<float*>(data + 4 * items);      // [items][2]: sum a^2, sum a.du
  float2* cs = reinterpret_cast<float2*>(part + 2 * items);      // [TT][h]
  const int64_t t0 = (int64_t)blockIdx.x * TT;
  uint32_t amax = 0;

  build_rope_table(cs, TT, t0, T, seq_len, h, d, base);
  __syncthreads();
  for (int it = threadIdx.x; it < items; it += kThreads) {
    const int c = it % C, rr = (it / C) % R, tt = it / (C * R);
    const int64_t t = t0 + tt;
    uint4 alo = make_uint4(0, 0, 0, 0), ahi = alo, glo = alo, ghi = alo;
    if (t < T) {
      const uint16_t* arow = qk_pre + t * qkw + rr * d;
      alo = *reinterpret_cast<const uint4*>(arow + 8 * c);
      ahi = *reinterpret_cast<const uint4*>(arow + h + 8 * c);
      const int64_t bseq = t / seq_len, s = t - bseq * seq_len;
      const uint16_t* grow = rr < H ? dq + ((bseq * H + rr) * seq_len + s) * qs
                                    : dk + ((bseq * H + (rr - H)) * seq_len + s) * qs;
      glo = *reinterpret_cast<const uint4*>(grow + 8 * c);
      ghi = *reinterpret_cast<const uint4*>(grow + h + 8 * c);
    }
    float a[8], b[8], ga[8], gb[8];
    unpack8(alo, a);
    unpack8(ahi, b);
    unpack8(glo, ga);
    unpack8(ghi, gb);
    const float2* tab = cs + tt * h + 8 * c;
    float ss = 0.f, sd = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float cn = tab[j].x, sn = tab[j].y;
      const float dua = ga[j] * cn + gb[j] * sn;   // R_{-p}
      const float dub = gb[j] * cn - ga[j] * sn;
      ss += a[j] * a[j] + b[j] * b[j];
      sd += a[j] * dua + b[j] * dub;
    }
    data[4 * it] = alo;
    data[4 * it + 1] = ahi;
    data[4 * it + 2] = glo;
    data[4 * it + 3] = ghi;
    part[2 * it] = ss;
    part[2 * it + 1] = sd;
  }
  __syncthreads();
  for (int it = threadIdx.x; it < items; it += kThreads) {
    const int c = it % C, rr = (it / C) % R, tt = it / (C * R);
    const int64_t t = t0 + tt;
    if (t >= T) continue;
    float ss = 0.f, sd = 0.f;
    const int first = it - c;
    for (int j = 0; j < C; ++j) {
      ss += part[2 * (first + j)];
      sd += part[2 * (first + j) + 1];
    }
    const float rho = 1.0f / sqrtf(ss / (float)d + eps);
    // rho^2 <u,du> / d, where <u,du> = rho * sum(a du)
    const float coef = rho * rho * rho * sd / (float)d;
    float a[8], b[8], ga[8], gb[8], oa[8], ob[8];
    unpack8(data[4 * it], a);
    unpack8(data[4 * it + 1], b);
    unpack8(data[4 * it + 2], ga);
    unpack8(data[4 * it + 3], gb);
    const float2* tab = cs + tt * h + 8 * c;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float cn = tab[j].x, sn = tab[j].y;
      const float dua = ga[j] * cn + gb[j] * sn;
      const float dub = gb[j] * cn - ga[j] * sn;
      oa[j] = rho * dua - coef * a[j];
      ob[j] = rho * dub - coef * b[j];
    }
    const uint4 plo = pack8(oa), phi = pack8(ob);
    amax = max(amax, max(absmax8(plo), absmax8(phi)));
    uint16_t* dst = dqkv + t * qkw + rr * d;
    *reinterpret_cast<uint4*>(dst + 8 * c) = plo;
    *reinterpret_cast<uint4*>(dst + h + 8 * c) = phi;
  }
  amax = block_max_u32(amax << 16, red);
  if (threadIdx.x == 0) partials[blockIdx.x] = amax;
}

// ------------------------------------------------------------- launchers

constexpr int kFwdTT = 16, kBwdTT = 8;

static bool quad_width(int d) { return d == 64 || d == 96 || d == 128; }


// The quad-chunk kernels use static LDS only: 0 for their widths.
size_t norm_rope_fwd_lds(int H, int d) {
  if (quad_width(d)) return 0;
  const size_t items = (size_t)kFwdTT * 2 * H * (d / 16);
  return items * (32 + 4) + (size_t)kFwdTT * (d / 2) * 8;
}

size_t norm_rope_bwd_lds(int H, int d) {
  if (quad_width(d)) return 0;
  const size_t items = (size_t)kBwdTT * 2 * H * (d / 16);
  return items * (64 + 8) + (size_t)kBwdTT * (d / 2) * 8;
}

void launch_norm_rope_fwd(const uint16_t* qk_pre, int64_t T, int seq_len, int H, int d, int qs,
                          float eps, float base, uint16_t* q, uint16_t* k, hipStream_t s) {
  const unsigned grid =
      (unsigned)std::min<int64_t>(kQuadTileBlocks, std::max<int64_t>(1, ceil_div(T, kQuadTT)));
  switch (d) {
    case 64:
      norm_rope_fwd_qc<64><<<grid, kThreads, 0, s>>>(qk_pre, T, seq_len, H, qs, eps, base, q, k);
      return;
    case 96:
      norm_rope_fwd_qc<96><<<grid, kThreads, 0, s>>>(qk_pre, T, seq_len, H, qs, eps, base, q, k);
      return;
    case 128:
      norm_rope_fwd_qc<128><<<grid, kThreads, 0, s>>>(qk_pre, T, seq_len, H, qs, eps, base, q,
                                                       k);
      return;
    default:
      break;
  }
  const size_t lds = norm_rope_fwd_lds(H, d);
  norm_rope_fwd_kernel<kFwdTT><<<(unsigned)ceil_div(T, kFwdTT), kThreads, lds, s>>>(
      qk_pre, T, seq_len, H, d, qs, eps, base, q, k);
}

int norm_rope_bwd_blocks(int64_t T, int H, int d) {
  (void)H;
  return quad_width(d)
             ? (int)std::min<int64_t>(kQuadTileBlocks, std::max<int64_t>(1, ceil_div(T, kQuadTT)))
             : (int)ceil_div(T, kBwdTT);
}

void launch_norm_rope_bwd(const uint16_t* dq, const uint16_t* dk, const uint16_t* qk_pre,
                          int64_t T, int seq_len, int H, int d, int qs, float eps, float base,
                          uint16_t* dqkv, uint32_t* partials, hipStream_t s) {
  const unsigned grid = (unsigned)norm_rope_bwd_blocks(T, H, d);
  switch (d) {
    case 64:
      norm_rope_bwd_qc<64><<<grid, kThreads, 0, s>>>(dq, dk, qk_pre, T, seq_len, H, qs, eps,
                                                        base, dqkv, partials);
      return;
    case 96:
      norm_rope_bwd_qc<96><<<grid, kThreads, 0, s>>>(dq, dk, qk_pre, T, seq_len, H, qs, eps,
                                                        base, dqkv, partials);
      return;
    case 128:
      norm_rope_bwd_qc<128><<<grid, kThreads, 0, s>>>(dq, dk, qk_pre, T, seq_len, H, qs, eps,
                                                        base, dqkv, partials);
      return;
    default:
      break;
  }
  const size_t lds = norm_rope_bwd_lds(H, d);
  norm_rope_bwd_kernel<kBwdTT><<<grid, kThreads, lds, s>>>(dq, dk, qk_pre, T, seq_len, H, d, qs,
                                                          eps, base, dqkv, partials);
}

}  // namespace fpr
