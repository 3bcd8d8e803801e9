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
// Work item = (token, head row, chunk c): a thread owns the 8 elements
// [8c, 8c+8) of a row together with their rotation partners [h+8c, h+8c+8),
// h = d/2, so a RoPE pair never leaves the thread's registers.  The row sums
// are combined through per-item partials in LDS, summed in a fixed order.
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
  const size_t lds = norm_rope_fwd_lds(H, d);
  norm_rope_fwd_kernel<kFwdTT><<<(unsigned)ceil_div(T, kFwdTT), kThreads, lds, s>>>(
      qk_pre, T, seq_len, H, d, eps, base, q, k);
}

int norm_rope_bwd_blocks(int64_t T) { return (int)ceil_div(T, kBwdTT); }

void launch_norm_rope_bwd(const uint16_t* dq, const uint16_t* dk, const uint16_t* dv,
                          const uint16_t* qk_pre, int64_t T, int seq_len, int H, int d, int d_v,
                          float eps, float base, uint16_t* dqkv, uint32_t* partials,
                          hipStream_t s) {
  const size_t lds = norm_rope_bwd_lds(H, d);
  norm_rope_bwd_kernel<kBwdTT><<<(unsigned)norm_rope_bwd_blocks(T), kThreads, lds, s>>>(
      dq, dk, dv, qk_pre, T, seq_len, H, d, d_v, eps, base, dqkv, partials);
}

}  // namespace fpr
