// Norm/RoPE kernels around the packed GEMM, for gfx950.
//
// Forward ("96 is enough", "The change": split, rms_norm(q), rms_norm(k),
// rope(q), rope(k); PR #344 page, "Changes": norm, RoPE and layout
// conversion fused).  For head widths 64, 96 and 128 all of it runs in the
// forward GEMM's epilogue (gemm.hip), which stores q, k, v and one fp32
// rho = 1 / rms per Q/K head row.  For other widths the GEMM stores the
// pre-norm Q|K rows in the forward workspace and norm_rope_fwd_kernel below
// turns them into q, k and rho: u = a / sqrt(mean(a^2) + eps), pairs
// (i, i + d/2) rotated by p * base^(-2i/d), head-major rows that may be
// padded with zeros to a stride qs > d (the FA3 padding of the PR #344
// page, "Changes").
//
// Backward ("Where the eight seconds were hiding", "The inventory": the norm,
// RoPE and backward shuffles), from the forward's own outputs: with
// u = R_{-p} q the normalised row and du = R_{-p} dq, the gradient of the
// pre-norm row is da = rho (du - u <u,du> / d).  A rotation keeps inner
// products, so <u,du> = <q,dq>, and da = rho R_{-p} (dq - q <q,dq> / d):
// one row sum, one inverse rotation, no pre-norm row.  The result is the
// Q|K part of the packed gradient, dQK [T][2H d] bf16, with one amax
// partial per block over dQK for the gradient quantiser, which reads the V
// columns straight from dv (whose amax a separate pass takes).
//
// Main backward kernel (d = 64, 96, 128): four consecutive lanes own one
// head row and every access is a whole 16-byte chunk (below); the row sum
// takes two cross-lane steps (DPP quad permutes).  Rotation angles come
// once per token and pair into an LDS table that all heads share.  The
// same kernel also runs the two-pass form that keeps dQK out of memory
// ("Where the eight seconds were hiding", "What generalizes": bytes that
// carry nothing new): a pass that only takes the amax, then one that
// re-derives every row and writes its gradient codes with the scale of the
// whole of dQKV, which that amax (and dv's) decides.
//
// Fallback kernels (other head widths): work item = (token, head row,
// chunk c), a thread owns the 8 elements [8c, 8c+8) of a row and their
// rotation partners; row sums go through per-item partials in LDS, summed
// in a fixed order.
#include <algorithm>
#include <atomic>

#include "common.hpp"
#include "launch.hpp"

namespace fpr {

// cos/sin of p * base^(-2j/d) for the block's tokens: the angle is formed
// and reduced modulo 2 pi in double (positions reach 2^24 rad), then fp32
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

// Element offset of head row (b, hh, s) in a head-major [n_seq][H][S][w] tensor.
__device__ inline int64_t head_row(int64_t b, int hh, int H, int S, int64_t s, int w) {
  return ((b * H + hh) * S + s) * w;
}

// ------------------------------------------------------- shared helpers

// theta_j / (2 pi), j < h, for the block.
__device__ inline void build_rev_table(double* rev, int h, int d, float base) {
  for (int j = threadIdx.x; j < h; j += kThreads) rev[j] = rope_rev(j, d, base);
  __syncthreads();
}

__device__ inline float quad_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));  // lane ^ 1
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));  // lane ^ 2
  return v;
}

// ------------------------------------------------- quad-chunk backward
//
// Four lanes per head row, every access a whole 16-byte chunk (8-byte
// lane accesses split each memory instruction over many partial lines and
// ran ~25% slower here): of the CH = d / 8 chunks of a row, lane l owns
// chunks l, l + 4, l + 8, ... (M = CH / 4 of them), so each load or store
// instruction covers 64 consecutive bytes of every row in the wave.  The
// RoPE partner of chunk c (elements i + d/2 of its elements i) is chunk
// c +- CH/2: for d = 64 and 128 that is another chunk of the same lane;
// for d = 96 it is a chunk of lane l ^ 2, which one DPP quad permute per
// word brings over.  A block takes TT tokens at a time and builds the
// cos/sin table of their positions (shared by all heads) in LDS.

constexpr int kQuadTT = 16;         // tokens per block iteration
constexpr int kQuadTileBlocks = 1024;

template <int D>
struct QuadChunks {
  static constexpr int CH = D / 8, HC = CH / 2, M = CH / 4, h = D / 2;
  static_assert(CH % 4 == 0, "four lanes per row");
  // chunk of lane l, own slot m
  __device__ static int chunk(int l, int m) { return l + 4 * m; }
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

// cos/sin of pairs j < h at the positions of tokens t0 .. t0 + nt - 1.
__device__ inline void quad_table(float2* cs, const double* rev, int64_t t0, int nt, int h,
                                  int seq_len) {
  for (int i = threadIdx.x; i < nt * h; i += kThreads) {
    const int tt = i / h, j = i - tt * h;
    const int64_t t = t0 + tt;
    float cn, sn;
    rope_cs(rev[j], t - (t / seq_len) * seq_len, cn, sn);
    cs[i] = make_float2(cn, sn);
  }
}

// The forward's outputs a backward row needs: q / k rows and their rho.
struct FwdRows {
  const uint16_t* q;
  const uint16_t* k;
  const float* rho;  // [2][n_seq][H][S]
  int n_seq;
};

template <int D>
struct QcBwdRow {
  uint4 q[QuadChunks<D>::M], g[QuadChunks<D>::M];
  float rho;
  int tt, rr;
  bool ok;
};

// Token t (< 2^24, so 32-bit) of the packed rows is position t % seq_len of
// sequence t / seq_len.
template <int D>
__device__ __forceinline__ void qc_bwd_load(QcBwdRow<D>& r, int row, int rows, int R, int H,
                                            int seq_len, int qs, int64_t t0,
                                            const uint16_t* __restrict__ dq,
                                            const uint16_t* __restrict__ dk, const FwdRows& f,
                                            int l) {
  using Q = QuadChunks<D>;
  r.ok = row < rows;
  if (!r.ok) return;
  const int tt = row / R, rr = row - tt * R;
  const bool isq = rr < H;
  const int hh = isq ? rr : rr - H;
  r.tt = tt;
  r.rr = rr;
  const int t = (int)t0 + tt, b = t / seq_len, sp = t - b * seq_len;
  const int64_t row_i = ((int64_t)b * H + hh) * seq_len + sp;
  const uint16_t* qsrc = (isq ? f.q : f.k) + row_i * qs;
  const uint16_t* gsrc = (isq ? dq : dk) + row_i * qs;
#pragma unroll
  for (int m = 0; m < Q::M; ++m) {
    r.q[m] = *reinterpret_cast<const uint4*>(qsrc + 8 * Q::chunk(l, m));
    r.g[m] = *reinterpret_cast<const uint4*>(gsrc + 8 * Q::chunk(l, m));
  }
  r.rho = f.rho[(isq ? 0 : (int64_t)f.n_seq * H * seq_len) + row_i];
}

// What the quad-chunk backward does with a finished row: write it to dQK
// (rows of N bf16), only fold it into the amax, or encode it into the
// gradient codes (the blocked row layout the GEMMs read, as the gradient
// quantiser writes it, from the same bf16 values and scale).
enum { kBwdWrite = 0, kBwdAmax = 1, kBwdCodes = 2 };

struct GradCodes {
  uint8_t* g8;               // [Tp / kActRows][kblocks][kActRows][kKBlock]
  int kblocks;
  const uint32_t* partials;  // every amax partial of dQKV, for the scale
  int parts;
};

// Finishes the row and returns the largest |bf16| bit pattern of it.
template <int D, int MODE, bool E5>
__device__ __forceinline__ uint32_t qc_bwd_finish(const QcBwdRow<D>& r, const float2* cs,
                                                  int64_t t0, int N, uint16_t* __restrict__ dqkv,
                                                  int l, const GradCodes& gc, float inv) {
  using Q = QuadChunks<D>;
  constexpr int h = Q::h, M = Q::M, HC = Q::HC;
  if (!r.ok) return 0;
  // <q, dq> over the row, bf16 pairs at a time
  float sd = 0.f;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    sd = dot2_bf16(r.q[m].x, r.g[m].x, sd);
    sd = dot2_bf16(r.q[m].y, r.g[m].y, sd);
    sd = dot2_bf16(r.q[m].z, r.g[m].z, sd);
    sd = dot2_bf16(r.q[m].w, r.g[m].w, sd);
  }
  uint4 pq[M], pg[M];
  quad_partners<D>(r.q, pq, l);
  quad_partners<D>(r.g, pg, l);
  sd = quad_sum(sd);
  const float c = sd / (float)D;
  const int64_t t = t0 + r.tt;
  uint32_t amax = 0;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    // own element e of slot m is element i (lower chunks) or i + d/2 of the
    // row, i = 8 (chunk mod HC) + e; its partner the other one.
    // w = dq - c q; da = rho R_{-p} w
    const int ch = Q::chunk(l, m);
    const bool lower = ch < HC;
    const float2* tab = cs + r.tt * h + 8 * (lower ? ch : ch - HC);
    float x[8], gx[8], xp[8], gp[8], o[8];
    unpack8(r.q[m], x);
    unpack8(r.g[m], gx);
    unpack8(pq[m], xp);
    unpack8(pg[m], gp);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float cn = tab[e].x, sn = tab[e].y;
      const float w = gx[e] - c * x[e], wp = gp[e] - c * xp[e];
      o[e] = r.rho * (lower ? w * cn + wp * sn : w * cn - wp * sn);
    }
    const uint4 pk = pack8_rn(o);
    amax = max(amax, absmax8(pk));
    if constexpr (MODE == kBwdWrite) {
      *reinterpret_cast<uint4*>(dqkv + t * N + r.rr * D + 8 * ch) = pk;
    } else if constexpr (MODE == kBwdCodes) {
      const uint32_t lo = fp8x4<E5>(bf16_to_f32(pk.x & 0xffffu) * inv, bf16_to_f32(pk.x >> 16) * inv,
                                    bf16_to_f32(pk.y & 0xffffu) * inv, bf16_to_f32(pk.y >> 16) * inv);
      const uint32_t hi = fp8x4<E5>(bf16_to_f32(pk.z & 0xffffu) * inv, bf16_to_f32(pk.z >> 16) * inv,
                                    bf16_to_f32(pk.w & 0xffffu) * inv, bf16_to_f32(pk.w >> 16) * inv);
      const int col = r.rr * D + 8 * ch;  // < 2^16
      const int64_t blk = (t / kActRows) * gc.kblocks + col / kKBlock;
      *reinterpret_cast<uint2*>(gc.g8 + (blk * kActRows + t % kActRows) * kKBlock +
                                col % kKBlock) = make_uint2(lo, hi);
    }
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

//
// The grid is what fits on the device at once (at most `nparts` blocks),
// and the blocks deal the groups of kQuadTT tokens round-robin, so that at
// any moment they work on neighbouring tokens (ranges of tokens per block,
// 768 streams of 12 head rows each far apart, ran ~10% slower).  Block b
// writes amax partial b; block 0 zeroes the slots [gridDim.x, nparts) that
// no block owns.
// With MODE = kBwdCodes the block first folds every partial into the
// gradient scale and writes no partial itself.
template <int D, int MODE, bool E5>
__global__ __launch_bounds__(kThreads) void norm_rope_bwd_qc(
    const uint16_t* __restrict__ dq, const uint16_t* __restrict__ dk, FwdRows f, int64_t T,
    int seq_len, int H, int qs, float base, uint16_t* __restrict__ dqkv,
    uint32_t* __restrict__ partials, int nparts, GradCodes gc) {
  using Q = QuadChunks<D>;
  constexpr int h = Q::h, QUADS = kThreads / 4, RB = bwd_rows<D>();
  __shared__ double rev[h];
  __shared__ float2 cs[kQuadTT * h];
  __shared__ uint32_t red[4];
  float inv = 1.0f;
  if constexpr (MODE == kBwdCodes)
    inv = tensor_scales(gc.partials, gc.parts, red, false, nullptr, nullptr, 0, false,
                        E5 ? kE5m2Max : kE4m3Max).y;
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
        qc_bwd_load<D>(r[j], rb + quad + j * QUADS, rows, R, H, seq_len, qs, t0, dq, dk, f, l);
      if (rb == 0) {  // the same for every thread: rows > 0
        quad_table(cs, rev, t0, nt, h, seq_len);
        __syncthreads();
      }
#pragma unroll
      for (int j = 0; j < RB; ++j)
        amax = max(amax, qc_bwd_finish<D, MODE, E5>(r[j], cs, t0, qkw, dqkv, l, gc, inv));
    }
    __syncthreads();
  }
  if constexpr (MODE != kBwdCodes) {
    amax = block_max_u32(amax << 16, red);
    if (threadIdx.x == 0) partials[blockIdx.x] = amax;
    if (blockIdx.x == 0)
      for (int i = gridDim.x + threadIdx.x; i < nparts; i += kThreads) partials[i] = 0;
  }
}

// ------------------------------------------------- forward (other widths)

template <int TT>
__global__ __launch_bounds__(kThreads) void norm_rope_fwd_kernel(
    const uint16_t* __restrict__ qk_pre, int64_t T, int seq_len, int n_seq, int H, int d, int qs,
    float eps, float base, uint16_t* __restrict__ q, uint16_t* __restrict__ k,
    float* __restrict__ rho_out) {
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
    const bool isq = rr < H;
    const int hh = isq ? rr : rr - H;
    uint16_t* dst = (isq ? q : k) + head_row(bseq, hh, H, seq_len, s, qs);
    *reinterpret_cast<uint4*>(dst + 8 * c) = pack8(oa);
    *reinterpret_cast<uint4*>(dst + h + 8 * c) = pack8(ob);
    if (c == 0)
      rho_out[(isq ? 0 : (int64_t)n_seq * H * seq_len) + head_row(bseq, hh, H, seq_len, s, 1)] =
          rho;
  }
  // zero padding columns d .. qs - 1 of every row
  const int pc = (qs - d) / 8, pitems = TT * R * pc;
  for (int it = threadIdx.x; it < pitems; it += kThreads) {
    const int c = it % pc, rr = (it / pc) % R, tt = it / (pc * R);
    const int64_t t = t0 + tt;
    if (t >= T) continue;
    const int64_t bseq = t / seq_len, s = t - bseq * seq_len;
    uint16_t* dst =
        (rr < H ? q : k) + head_row(bseq, rr < H ? rr : rr - H, H, seq_len, s, qs);
    *reinterpret_cast<uint4*>(dst + d + 8 * c) = make_uint4(0, 0, 0, 0);
  }
}

// ------------------------------------------------ backward (other widths)

// Persistent: at most kQuadTileBlocks blocks walk the groups of TT tokens,
// so the amax partials (one per block) stay few at any token count.
template <int TT>
__global__ __launch_bounds__(kThreads) void norm_rope_bwd_kernel(
    const uint16_t* __restrict__ dq, const uint16_t* __restrict__ dk, FwdRows f, int64_t T,
    int seq_len, int H, int d, int qs, float base, uint16_t* __restrict__ dqkv,
    uint32_t* __restrict__ partials) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ uint32_t red[4];
  const int h = d / 2, C = h / 8, R = 2 * H, qkw = R * d;
  const int items = TT * R * C;
  uint4* data = reinterpret_cast<uint4*>(smem);                  // [items][4]: q lo/hi, g lo/hi
  float* part = reinterpret_cast<float*>(data + 4 * items);      // [items]: sum q.dq
  float2* cs = reinterpret_cast<float2*>(part + items);          // [TT][h]
  uint32_t amax = 0;
  const int64_t groups = ceil_div(T, TT);
  for (int64_t gi = blockIdx.x; gi < groups; gi += gridDim.x) {
    const int64_t t0 = gi * TT;
    build_rope_table(cs, TT, t0, T, seq_len, h, d, base);
    for (int it = threadIdx.x; it < items; it += kThreads) {
      const int c = it % C, rr = (it / C) % R, tt = it / (C * R);
      const int64_t t = t0 + tt;
      uint4 qlo = make_uint4(0, 0, 0, 0), qhi = qlo, glo = qlo, ghi = qlo;
      if (t < T) {
        const int64_t bseq = t / seq_len, s = t - bseq * seq_len;
        const bool isq = rr < H;
        const int64_t row = head_row(bseq, isq ? rr : rr - H, H, seq_len, s, qs);
        const uint16_t* qrow = (isq ? f.q : f.k) + row;
        const uint16_t* grow = (isq ? dq : dk) + row;
        qlo = *reinterpret_cast<const uint4*>(qrow + 8 * c);
        qhi = *reinterpret_cast<const uint4*>(qrow + h + 8 * c);
        glo = *reinterpret_cast<const uint4*>(grow + 8 * c);
        ghi = *reinterpret_cast<const uint4*>(grow + h + 8 * c);
      }
      float a[8], b[8], ga[8], gb[8];
      unpack8(qlo, a);
      unpack8(qhi, b);
      unpack8(glo, ga);
      unpack8(ghi, gb);
      float sd = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) sd += a[j] * ga[j] + b[j] * gb[j];
      data[4 * it] = qlo;
      data[4 * it + 1] = qhi;
      data[4 * it + 2] = glo;
      data[4 * it + 3] = ghi;
      part[it] = sd;
    }
    __syncthreads();
    for (int it = threadIdx.x; it < items; it += kThreads) {
      const int c = it % C, rr = (it / C) % R, tt = it / (C * R);
      const int64_t t = t0 + tt;
      if (t >= T) continue;
      float sd = 0.f;
      const int first = it - c;
      for (int j = 0; j < C; ++j) sd += part[first + j];
      const float cf = sd / (float)d;
      const int64_t bseq = t / seq_len, s = t - bseq * seq_len;
      const bool isq = rr < H;
      const float rho = f.rho[(isq ? 0 : (int64_t)f.n_seq * H * seq_len) +
                              head_row(bseq, isq ? rr : rr - H, H, seq_len, s, 1)];
      float a[8], b[8], ga[8], gb[8], oa[8], ob[8];
      unpack8(data[4 * it], a);
      unpack8(data[4 * it + 1], b);
      unpack8(data[4 * it + 2], ga);
      unpack8(data[4 * it + 3], gb);
      const float2* tab = cs + tt * h + 8 * c;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float cn = tab[j].x, sn = tab[j].y;
        const float wa = ga[j] - cf * a[j], wb = gb[j] - cf * b[j];  // dq - q <q,dq> / d
        oa[j] = rho * (wa * cn + wb * sn);                           // rho R_{-p} (...)
        ob[j] = rho * (wb * cn - wa * sn);
      }
      const uint4 plo = pack8(oa), phi = pack8(ob);
      amax = max(amax, max(absmax8(plo), absmax8(phi)));
      uint16_t* dst = dqkv + t * qkw + rr * d;
      *reinterpret_cast<uint4*>(dst + 8 * c) = plo;
      *reinterpret_cast<uint4*>(dst + h + 8 * c) = phi;
    }
    __syncthreads();
  }
  amax = block_max_u32(amax << 16, red);
  if (threadIdx.x == 0) partials[blockIdx.x] = amax;
}

// ------------------------------------------------------------- launchers

constexpr int kFwdTT = 16, kBwdTT = 8;

static bool quad_width(int d) { return d == 64 || d == 96 || d == 128; }

// The quad-chunk backward uses static LDS only, and the fused forward has no
// norm/RoPE kernel: 0 for their widths.
size_t norm_rope_fwd_lds(int H, int d) {
  if (quad_width(d)) return 0;
  const size_t items = (size_t)kFwdTT * 2 * H * (d / 16);
  return items * (32 + 4) + (size_t)kFwdTT * (d / 2) * 8;
}

size_t norm_rope_bwd_lds(int H, int d) {
  if (quad_width(d)) return 0;
  const size_t items = (size_t)kBwdTT * 2 * H * (d / 16);
  return items * (64 + 4) + (size_t)kBwdTT * (d / 2) * 8;
}

void launch_norm_rope_fwd(const uint16_t* qk_pre, int64_t T, int seq_len, int H, int d, int qs,
                          float eps, float base, uint16_t* q, uint16_t* k, float* rho,
                          hipStream_t s) {
  const size_t lds = norm_rope_fwd_lds(H, d);
  norm_rope_fwd_kernel<kFwdTT><<<(unsigned)ceil_div(T, kFwdTT), kThreads, lds, s>>>(
      qk_pre, T, seq_len, (int)(T / seq_len), H, d, qs, eps, base, q, k, rho);
}

int norm_rope_bwd_blocks(int64_t T, int H, int d) {
  (void)H;
  const int64_t tt = quad_width(d) ? kQuadTT : kBwdTT;
  return (int)std::min<int64_t>(kQuadTileBlocks, std::max<int64_t>(1, ceil_div(T, tt)));
}

// Blocks of the quad backward for width D that the current device holds at
// once, over all its CUs (queried once per device).
template <int D, int MODE, bool E5>
static int quad_bwd_resident() {
  constexpr int kDevs = 64;
  static std::atomic<int> cached[kDevs] = {};  // 0: not yet queried
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDevs) dev = -1;
  if (dev >= 0) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev < 0 ? 0 : dev) !=
          hipSuccess || cus <= 0)
    cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, norm_rope_bwd_qc<D, MODE, E5>,
                                                   kThreads, 0) !=
          hipSuccess || per_cu <= 0)
    per_cu = 1;
  const int n = cus * per_cu;
  if (dev >= 0) cached[dev].store(n, std::memory_order_relaxed);  // same value from any thread
  return n;
}

template <int D, int MODE, bool E5>
static void launch_bwd_qc_as(const uint16_t* dq, const uint16_t* dk, const FwdRows& f, int64_t T,
                             int seq_len, int H, int qs, float base, uint16_t* dqkv,
                             uint32_t* partials, int nparts, const GradCodes& gc, hipStream_t s) {
  const unsigned grid = (unsigned)std::min(nparts, quad_bwd_resident<D, MODE, E5>());
  norm_rope_bwd_qc<D, MODE, E5><<<grid, kThreads, 0, s>>>(dq, dk, f, T, seq_len, H, qs, base,
                                                          dqkv, partials, nparts, gc);
}

template <int D>
static void launch_bwd_qc(const uint16_t* dq, const uint16_t* dk, const FwdRows& f, int64_t T,
                          int seq_len, int H, int qs, float base, uint16_t* dqkv,
                          uint32_t* partials, int nparts, int mode, const GradCodes& gc,
                          bool e5, hipStream_t s) {
  if (mode == kBwdWrite)
    launch_bwd_qc_as<D, kBwdWrite, false>(dq, dk, f, T, seq_len, H, qs, base, dqkv, partials,
                                          nparts, gc, s);
  else if (mode == kBwdAmax)
    launch_bwd_qc_as<D, kBwdAmax, false>(dq, dk, f, T, seq_len, H, qs, base, dqkv, partials,
                                         nparts, gc, s);
  else if (e5)
    launch_bwd_qc_as<D, kBwdCodes, true>(dq, dk, f, T, seq_len, H, qs, base, dqkv, partials,
                                         nparts, gc, s);
  else
    launch_bwd_qc_as<D, kBwdCodes, false>(dq, dk, f, T, seq_len, H, qs, base, dqkv, partials,
                                          nparts, gc, s);
}

void launch_norm_rope_bwd(const uint16_t* dq, const uint16_t* dk, const uint16_t* q,
                          const uint16_t* k, const float* rho, int64_t T, int seq_len, int H,
                          int d, int qs, float base, uint16_t* dqkv, uint32_t* partials,
                          hipStream_t s) {
  const int nparts = norm_rope_bwd_blocks(T, H, d);
  const FwdRows f{q, k, rho, (int)(T / seq_len)};
  const GradCodes none{nullptr, 0, nullptr, 0};
  switch (d) {
    case 64:
      return launch_bwd_qc<64>(dq, dk, f, T, seq_len, H, qs, base, dqkv, partials, nparts,
                               kBwdWrite, none, false, s);
    case 96:
      return launch_bwd_qc<96>(dq, dk, f, T, seq_len, H, qs, base, dqkv, partials, nparts,
                               kBwdWrite, none, false, s);
    case 128:
      return launch_bwd_qc<128>(dq, dk, f, T, seq_len, H, qs, base, dqkv, partials, nparts,
                                kBwdWrite, none, false, s);
    default:
      break;
  }
  const size_t lds = norm_rope_bwd_lds(H, d);
  norm_rope_bwd_kernel<kBwdTT><<<(unsigned)nparts, kThreads, lds, s>>>(
      dq, dk, f, T, seq_len, H, d, qs, base, dqkv, partials);
}

bool norm_rope_bwd_two_pass(int d) { return d == 64 || d == 96 || d == 128; }

void launch_norm_rope_bwd_amax(const uint16_t* dq, const uint16_t* dk, const uint16_t* q,
                               const uint16_t* k, const float* rho, int64_t T, int seq_len, int H,
                               int d, int qs, float base, uint32_t* partials, hipStream_t s) {
  const int nparts = norm_rope_bwd_blocks(T, H, d);
  const FwdRows f{q, k, rho, (int)(T / seq_len)};
  const GradCodes none{nullptr, 0, nullptr, 0};
  if (d == 64)
    launch_bwd_qc<64>(dq, dk, f, T, seq_len, H, qs, base, nullptr, partials, nparts, kBwdAmax,
                      none, false, s);
  else if (d == 96)
    launch_bwd_qc<96>(dq, dk, f, T, seq_len, H, qs, base, nullptr, partials, nparts, kBwdAmax,
                      none, false, s);
  else if (d == 128)
    launch_bwd_qc<128>(dq, dk, f, T, seq_len, H, qs, base, nullptr, partials, nparts, kBwdAmax,
                       none, false, s);
}

void launch_norm_rope_bwd_codes(const uint16_t* dq, const uint16_t* dk, const uint16_t* q,
                                const uint16_t* k, const float* rho, int64_t T, int seq_len,
                                int H, int d, int qs, float base, const uint32_t* partials,
                                int parts, uint8_t* g8, int N, hipStream_t s, bool e5m2) {
  const int nparts = norm_rope_bwd_blocks(T, H, d);
  const FwdRows f{q, k, rho, (int)(T / seq_len)};
  const GradCodes gc{g8, (int)ceil_div(N, kKBlock), partials, parts};
  if (d == 64)
    launch_bwd_qc<64>(dq, dk, f, T, seq_len, H, qs, base, nullptr, nullptr, nparts, kBwdCodes,
                      gc, e5m2, s);
  else if (d == 96)
    launch_bwd_qc<96>(dq, dk, f, T, seq_len, H, qs, base, nullptr, nullptr, nparts, kBwdCodes,
                      gc, e5m2, s);
  else if (d == 128)
    launch_bwd_qc<128>(dq, dk, f, T, seq_len, H, qs, base, nullptr, nullptr, nparts, kBwdCodes,
                       gc, e5m2, s);
}

}  // namespace fpr
