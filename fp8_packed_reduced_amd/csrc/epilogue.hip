// Fused layout kernels around the packed GEMM, for gfx950.
//
// Forward ("96 is enough", "The change": split, rms_norm(q), rms_norm(k),
// rope(q), rope(k); PR #344 page, "Changes": norm, RoPE and layout
// conversion fused, lane swaps kept in registers): pre-norm Q|K rows ->
// u = a / sqrt(mean(a^2) + eps) -> rotate pairs (i, i + d/2) by
// p * base^(-2i/d) -> head-major q, k.
//
// Backward ("Where the eight seconds were hiding", "The inventory": the norm,
// RoPE and backward shuffles): du = R_{-p} dq; da = rho * (du - u <u,du>/d);
// the V gradient is re-laid out; everything is packed into dQKV [T][N] bf16
// with one amax partial per block for the gradient quantiser.
//
// Main kernels (d = 64, 96, 128): four consecutive lanes own one head row,
// lane q the P = d/8 pairs (i, i + d/2) for i in [qP, qP + P), so a RoPE
// pair never leaves a thread and the row sums take two cross-lane steps
// (DPP quad permutes) with no LDS.  Rotation angles are formed in
// revolutions: position * theta_j / (2 pi) in double, reduced to its
// fractional part, then the hardware sin/cos of that fraction.
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

// ------------------------------------------------- quad-lane kernels

constexpr int kQuadBlocks = 2048;  // grid of the grid-stride quad kernels

// Work of the forward quad kernel: a wave's 16 quads (one head row each)
// cover TG consecutive tokens x HG consecutive head rows (4 x 4, or 8 x 2
// when the 2H head rows are not a multiple of 4), so each token's rows that
// a wave reads, and each head's rows it writes head-major, are runs of HG
// (resp. TG) whole rows: 768 contiguous bytes for 96-wide heads, whole
// cache lines, where rows of 192 bytes alone would leave lines half
// written.  The backward kernel, whose large streams (pre-norm rows in,
// dQKV out) are both token-major, takes head rows in plain row order.
__host__ __device__ inline int quad_heads(int R) { return R % 4 == 0 ? 4 : 2; }
__host__ __device__ inline int64_t quad_units(int64_t T, int R) {
  const int HG = quad_heads(R);
  return ceil_div(T, 16 / HG) * (R / HG) * 64;
}

// Token and head row of quad-kernel unit u (lane u % 4 of its quad).
__device__ inline void quad_row(int64_t u, int R, int64_t& t, int& rr) {
  const int HG = quad_heads(R), TG = 16 / HG, n_hg = R / HG;
  const int64_t w = u >> 6;
  const int qd = (int)((u >> 2) & 15);
  const int64_t tg = w / n_hg;
  const int hg = (int)(w - tg * n_hg);
  t = tg * TG + qd % TG;
  rr = hg * HG + qd / TG;
}

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

template <int P>
__device__ inline void load_bf16(const uint16_t* p, float (&f)[P]) {
#pragma unroll
  for (int i = 0; i < P / 4; ++i) {
    const uint2 w = *reinterpret_cast<const uint2*>(p + 4 * i);
    f[4 * i] = bf16_to_f32(w.x & 0xffffu);
    f[4 * i + 1] = bf16_to_f32(w.x >> 16);
    f[4 * i + 2] = bf16_to_f32(w.y & 0xffffu);
    f[4 * i + 3] = bf16_to_f32(w.y >> 16);
  }
}

// Stores P values as bf16 and returns the largest |bf16| bit pattern.
template <int P>
__device__ inline uint32_t store_bf16(uint16_t* p, const float (&f)[P]) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < P / 4; ++i) {
    const uint2 w = make_uint2(pack_bf16x2(f[4 * i], f[4 * i + 1]),
                               pack_bf16x2(f[4 * i + 2], f[4 * i + 3]));
    *reinterpret_cast<uint2*>(p + 4 * i) = w;
    m = max(m, max(max(w.x & 0x7fffu, (w.x >> 16) & 0x7fffu),
                   max(w.y & 0x7fffu, (w.y >> 16) & 0x7fffu)));
  }
  return m;
}

// One head row of the forward quad kernel: loaded first, finished later,
// so a thread can have several rows' loads in flight.
template <int P>
struct FwdRow {
  float a[P], b[P];
  int64_t t;
  int rr;
  bool ok;
};

template <int P>
__device__ __forceinline__ void fwd_load(FwdRow<P>& r, int64_t u, int64_t units, int64_t T, int R,
                                         const uint16_t* __restrict__ qk_pre, int lq) {
  constexpr int h = 4 * P, d = 2 * h;
  r.ok = false;
  if (u >= units) return;
  quad_row(u, R, r.t, r.rr);
  if (r.t >= T) return;  // the whole quad
  r.ok = true;
  const uint16_t* src = qk_pre + (r.t * R + r.rr) * d + lq * P;  // row t, head row rr
  load_bf16<P>(src, r.a);
  load_bf16<P>(src + h, r.b);
}

template <int P>
__device__ __forceinline__ void fwd_finish(FwdRow<P>& r, const double* rev, int seq_len, int H,
                                           float eps, uint16_t* __restrict__ q,
                                           uint16_t* __restrict__ k, int lq) {
  constexpr int h = 4 * P, d = 2 * h;
  if (!r.ok) return;
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < P; ++i) ss += r.a[i] * r.a[i] + r.b[i] * r.b[i];
  ss = quad_sum(ss);
  const float rho = 1.0f / sqrtf(ss / (float)d + eps);
  const int64_t bseq = r.t / seq_len, s = r.t - bseq * seq_len;
#pragma unroll
  for (int i = 0; i < P; ++i) {
    float cn, sn;
    rope_cs(rev[lq * P + i], s, cn, sn);
    const float ua = r.a[i] * rho, ub = r.b[i] * rho;
    r.a[i] = ua * cn - ub * sn;
    r.b[i] = ub * cn + ua * sn;
  }
  const int rr = r.rr;
  uint16_t* dst = (rr < H ? q + ((bseq * H + rr) * seq_len + s) * d
                          : k + ((bseq * H + (rr - H)) * seq_len + s) * d) + lq * P;
  store_bf16<P>(dst, r.a);
  store_bf16<P>(dst + h, r.b);
}

template <int P>
__global__ __launch_bounds__(kThreads) void norm_rope_fwd_quad(
    const uint16_t* __restrict__ qk_pre, int64_t T, int seq_len, int H, float eps, float base,
    uint16_t* __restrict__ q, uint16_t* __restrict__ k) {
  constexpr int h = 4 * P, d = 2 * h;
  __shared__ double rev[h];
  build_rev_table(rev, h, d, base);
  const int R = 2 * H, lq = threadIdx.x & 3;
  const int64_t units = quad_units(T, R), stride = (int64_t)gridDim.x * kThreads;
  for (int64_t u = blockIdx.x * (int64_t)kThreads + threadIdx.x; u < units; u += 2 * stride) {
    FwdRow<P> r0, r1;  // two rows' loads in flight per thread
    fwd_load<P>(r0, u, units, T, R, qk_pre, lq);
    fwd_load<P>(r1, u + stride, units, T, R, qk_pre, lq);
    fwd_finish<P>(r0, rev, seq_len, H, eps, q, k, lq);
    fwd_finish<P>(r1, rev, seq_len, H, eps, q, k, lq);
  }
}

// One head row of the backward quad kernel, loaded first and finished
// later (as FwdRow).
template <int P>
struct BwdRow {
  float a[P], b[P], ga[P], gb[P];
  int64_t t, s;
  int rr;
  bool ok;
};

template <int P>
__device__ __forceinline__ void bwd_load(BwdRow<P>& r, int64_t u, int64_t units, int R, int H,
                                         int seq_len, const uint16_t* __restrict__ dq,
                                         const uint16_t* __restrict__ dk,
                                         const uint16_t* __restrict__ qk_pre, int lq) {
  constexpr int h = 4 * P, d = 2 * h;
  r.ok = u < units;
  if (!r.ok) return;
  const int64_t row = u >> 2;
  r.t = row / R;
  r.rr = (int)(row - r.t * R);
  const int64_t bseq = r.t / seq_len;
  r.s = r.t - bseq * seq_len;
  const int rr = r.rr;
  const uint16_t* asrc = qk_pre + row * d + lq * P;
  const uint16_t* gsrc = (rr < H ? dq + ((bseq * H + rr) * seq_len + r.s) * d
                                 : dk + ((bseq * H + (rr - H)) * seq_len + r.s) * d) + lq * P;
  load_bf16<P>(asrc, r.a);
  load_bf16<P>(asrc + h, r.b);
  load_bf16<P>(gsrc, r.ga);
  load_bf16<P>(gsrc + h, r.gb);
}

// Finishes the row and returns the largest |bf16| bit pattern it wrote.
template <int P>
__device__ __forceinline__ uint32_t bwd_finish(BwdRow<P>& r, const double* rev, int N,
                                               float eps, uint16_t* __restrict__ dqkv, int lq) {
  constexpr int h = 4 * P, d = 2 * h;
  if (!r.ok) return 0;
  float ss = 0.f, sd = 0.f;
#pragma unroll
  for (int i = 0; i < P; ++i) {
    float cn, sn;
    rope_cs(rev[lq * P + i], r.s, cn, sn);
    const float dua = r.ga[i] * cn + r.gb[i] * sn;  // R_{-p}
    const float dub = r.gb[i] * cn - r.ga[i] * sn;
    r.ga[i] = dua;
    r.gb[i] = dub;
    ss += r.a[i] * r.a[i] + r.b[i] * r.b[i];
    sd += r.a[i] * dua + r.b[i] * dub;
  }
  ss = quad_sum(ss);
  sd = quad_sum(sd);
  const float rho = 1.0f / sqrtf(ss / (float)d + eps);
  // rho^2 <u,du> / d, where <u,du> = rho * sum(a du)
  const float coef = rho * rho * rho * sd / (float)d;
#pragma unroll
  for (int i = 0; i < P; ++i) {
    r.ga[i] = rho * r.ga[i] - coef * r.a[i];
    r.gb[i] = rho * r.gb[i] - coef * r.b[i];
  }
  uint16_t* dst = dqkv + r.t * N + r.rr * d + lq * P;
  const uint32_t m = store_bf16<P>(dst, r.ga);
  return max(m, store_bf16<P>(dst + h, r.gb));
}

// Backward, then the V gradient re-laid out into the packed rows; one amax
// partial per block.
template <int P>
__global__ __launch_bounds__(kThreads) void norm_rope_bwd_quad(
    const uint16_t* __restrict__ dq, const uint16_t* __restrict__ dk,
    const uint16_t* __restrict__ dv, const uint16_t* __restrict__ qk_pre, int64_t T,
    int seq_len, int H, int dvw, float eps, float base, uint16_t* __restrict__ dqkv,
    uint32_t* __restrict__ partials) {
  constexpr int h = 4 * P, d = 2 * h;
  __shared__ double rev[h];
  __shared__ uint32_t red[4];
  build_rev_table(rev, h, d, base);
  const int R = 2 * H, qkw = R * d, N = qkw + H * dvw, lq = threadIdx.x & 3;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  uint32_t amax = 0;
  const int64_t units = T * R * 4;
  for (int64_t u = blockIdx.x * (int64_t)kThreads + threadIdx.x; u < units; u += 2 * stride) {
    BwdRow<P> r0, r1;  // two rows' loads in flight per thread
    bwd_load<P>(r0, u, units, R, H, seq_len, dq, dk, qk_pre, lq);
    bwd_load<P>(r1, u + stride, units, R, H, seq_len, dq, dk, qk_pre, lq);
    amax = max(amax, bwd_finish<P>(r0, rev, N, eps, dqkv, lq));
    amax = max(amax, bwd_finish<P>(r1, rev, N, eps, dqkv, lq));
  }
  const int cv = dvw / 8;
  const int64_t vunits = T * H * cv;
  for (int64_t u = blockIdx.x * (int64_t)kThreads + threadIdx.x; u < vunits; u += stride) {
    const int64_t th = u / cv;
    const int c = (int)(u - th * cv);
    const int64_t t = th / H;
    const int hh = (int)(th - t * H);
    const int64_t bseq = t / seq_len, s = t - bseq * seq_len;
    const uint4 g =
        *reinterpret_cast<const uint4*>(dv + ((bseq * H + hh) * seq_len + s) * dvw + 8 * c);
    amax = max(amax, absmax8(g));
    *reinterpret_cast<uint4*>(dqkv + t * N + qkw + hh * dvw + 8 * c) = g;
  }
  amax = block_max_u32(amax << 16, red);
  if (threadIdx.x == 0) partials[blockIdx.x] = amax;
}

// ------------------------------------------------------------- forward

template <int TT>
__global__ __launch_bounds__(kThreads) void norm_rope_fwd_kernel(
    const uint16_t* __restrict__ qk_pre, int64_t T, int seq_len, int H, int d, float eps,
    float base, uint16_t* __restrict__ q, uint16_t* __restrict__ k) {
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
    uint16_t* dst = rr < H ? q + ((bseq * H + rr) * seq_len + s) * d
                           : k + ((bseq * H + (rr - H)) * seq_len + s) * d;
    *reinterpret_cast<uint4*>(dst + 8 * c) = pack8(oa);
    *reinterpret_cast<uint4*>(dst + h + 8 * c) = pack8(ob);
  }
}

// ------------------------------------------------------------ backward

template <int TT>
__global__ __launch_bounds__(kThreads) void norm_rope_bwd_kernel(
    const uint16_t* __restrict__ dq, const uint16_t* __restrict__ dk,
    const uint16_t* __restrict__ dv, const uint16_t* __restrict__ qk_pre, int64_t T,
    int seq_len, int H, int d, int dvw, float eps, float base, uint16_t* __restrict__ dqkv,
    uint32_t* __restrict__ partials) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ uint32_t red[4];
  const int h = d / 2, C = h / 8, R = 2 * H, qkw = R * d, N = qkw + H * dvw;
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
      const uint16_t* grow = rr < H ? dq + ((bseq * H + rr) * seq_len + s) * d
                                    : dk + ((bseq * H + (rr - H)) * seq_len + s) * d;
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
    uint16_t* dst = dqkv + t * N + rr * d;
    *reinterpret_cast<uint4*>(dst + 8 * c) = plo;
    *reinterpret_cast<uint4*>(dst + h + 8 * c) = phi;
  }
  // V gradient: re-lay out head-major dv into the packed rows
  const int cv = dvw / 8, vitems = TT * H * cv;
  for (int it = threadIdx.x; it < vitems; it += kThreads) {
    const int c = it % cv, hh = (it / cv) % H, tt = it / (cv * H);
    const int64_t t = t0 + tt;
    if (t >= T) continue;
    const int64_t bseq = t / seq_len, s = t - bseq * seq_len;
    const uint4 g = *reinterpret_cast<const uint4*>(dv + ((bseq * H + hh) * seq_len + s) * dvw + 8 * c);
    amax = max(amax, absmax8(g));
    *reinterpret_cast<uint4*>(dqkv + t * N + qkw + hh * dvw + 8 * c) = g;
  }
  amax = block_max_u32(amax << 16, red);
  if (threadIdx.x == 0) partials[blockIdx.x] = amax;
}

// ------------------------------------------------------------- launchers

constexpr int kFwdTT = 16, kBwdTT = 8;

static bool quad_width(int d) { return d == 64 || d == 96 || d == 128; }

static unsigned quad_grid(int64_t units) {
  return (unsigned)std::min<int64_t>(kQuadBlocks, std::max<int64_t>(1, ceil_div(units, kThreads)));
}

size_t norm_rope_fwd_lds(int H, int d) {
  const size_t items = (size_t)kFwdTT * 2 * H * (d / 16);
  return items * (32 + 4) + (size_t)kFwdTT * (d / 2) * 8;
}

size_t norm_rope_bwd_lds(int H, int d) {
  const size_t items = (size_t)kBwdTT * 2 * H * (d / 16);
  return items * (64 + 8) + (size_t)kBwdTT * (d / 2) * 8;
}

void launch_norm_rope_fwd(const uint16_t* qk_pre, int64_t T, int seq_len, int H, int d, float eps,
                          float base, uint16_t* q, uint16_t* k, hipStream_t s) {
  const unsigned grid = quad_grid(quad_units(T, 2 * H));
  switch (d) {
    case 64:
      norm_rope_fwd_quad<8><<<grid, kThreads, 0, s>>>(qk_pre, T, seq_len, H, eps, base, q, k);
      return;
    case 96:
      norm_rope_fwd_quad<12><<<grid, kThreads, 0, s>>>(qk_pre, T, seq_len, H, eps, base, q, k);
      return;
    case 128:
      norm_rope_fwd_quad<16><<<grid, kThreads, 0, s>>>(qk_pre, T, seq_len, H, eps, base, q, k);
      return;
    default:
      break;
  }
  const size_t lds = norm_rope_fwd_lds(H, d);
  norm_rope_fwd_kernel<kFwdTT><<<(unsigned)ceil_div(T, kFwdTT), kThreads, lds, s>>>(
      qk_pre, T, seq_len, H, d, eps, base, q, k);
}

int norm_rope_bwd_blocks(int64_t T, int H, int d) {
  return quad_width(d) ? (int)quad_grid(T * 2 * H * 4) : (int)ceil_div(T, kBwdTT);
}

void launch_norm_rope_bwd(const uint16_t* dq, const uint16_t* dk, const uint16_t* dv,
                          const uint16_t* qk_pre, int64_t T, int seq_len, int H, int d, int d_v,
                          float eps, float base, uint16_t* dqkv, uint32_t* partials,
                          hipStream_t s) {
  const unsigned grid = (unsigned)norm_rope_bwd_blocks(T, H, d);
  switch (d) {
    case 64:
      norm_rope_bwd_quad<8><<<grid, kThreads, 0, s>>>(dq, dk, dv, qk_pre, T, seq_len, H, d_v, eps,
                                                      base, dqkv, partials);
      return;
    case 96:
      norm_rope_bwd_quad<12><<<grid, kThreads, 0, s>>>(dq, dk, dv, qk_pre, T, seq_len, H, d_v,
                                                       eps, base, dqkv, partials);
      return;
    case 128:
      norm_rope_bwd_quad<16><<<grid, kThreads, 0, s>>>(dq, dk, dv, qk_pre, T, seq_len, H, d_v,
                                                       eps, base, dqkv, partials);
      return;
    default:
      break;
  }
  const size_t lds = norm_rope_bwd_lds(H, d);
  norm_rope_bwd_kernel<kBwdTT><<<grid, kThreads, lds, s>>>(dq, dk, dv, qk_pre, T, seq_len, H, d,
                                                          d_v, eps, base, dqkv, partials);
}

}  // namespace fpr
