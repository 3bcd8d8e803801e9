// Per-tensor e4m3 quantisers for gfx950: the packed weight (both cached
// layouts from one read of W, PR #344 page, "Changes"), and bf16 activations
// / gradients (the GEMMs' blocked row layout, which all three GEMMs read:
// forward and dX as K-contiguous rows, dW token by token).
//
// The scale needs the whole tensor's amax before any code can be written,
// so each quantiser is two kernels: per-block partial amax, then quantize,
// whose every block first reduces the (few KB of, L2-resident) partials to
// the scales itself; one of its blocks also publishes them.  Partials are
// fp32 bit patterns of |v| held as uint32: for non-negative floats the
// integer order is the float order, and any NaN or Inf pattern compares
// above every finite value.
#include "common.hpp"
#include "launch.hpp"

namespace fpr {

// ------------------------------------------------------------- amax of W

__device__ inline float4 load_w4(const float* wq, int64_t ldq, const float* wk, int64_t ldk,
                                 const float* wv, int64_t ldv, int nq, int d, int n) {
  const float* p = n < nq       ? wq + d * ldq + n
                   : n < 2 * nq ? wk + d * ldk + (n - nq)
                                : wv + d * ldv + (n - 2 * nq);
  return *reinterpret_cast<const float4*>(p);
}

// The three pieces of the logical W_packed [D][N]: columns [0, nq) from wq,
// [nq, 2 nq) from wk, the rest from wv, each with its own row stride.
struct WSrc {
  const float* wq;
  int64_t ldq;
  const float* wk;
  int64_t ldk;
  const float* wv;
  int64_t ldv;
  int D, nq, N;
};

// Block b of nb takes rows b, b + nb, ... of the logical [D][N] matrix; its
// threads stride over a row's float4s (no index division), four loads in
// flight per thread where the row is long enough.
__device__ __forceinline__ void amax_w_block(const WSrc& w, int b, int nb,
                                             uint32_t* __restrict__ partials, uint32_t* red) {
  const int quads = w.N / 4;
  uint32_t m = 0;
  auto fold = [&](float4 v) {
    uint32_t a = __float_as_uint(v.x) & 0x7fffffffu;
    uint32_t c = __float_as_uint(v.y) & 0x7fffffffu;
    uint32_t e = __float_as_uint(v.z) & 0x7fffffffu;
    uint32_t f = __float_as_uint(v.w) & 0x7fffffffu;
    a = a > c ? a : c;
    e = e > f ? e : f;
    a = a > e ? a : e;
    m = m > a ? m : a;
  };
  auto ld = [&](int d, int n) { return load_w4(w.wq, w.ldq, w.wk, w.ldk, w.wv, w.ldv, w.nq, d, n); };
  for (int d = b; d < w.D; d += nb) {
    int q = threadIdx.x;
    for (; q + 3 * kThreads < quads; q += 4 * kThreads) {
      const float4 w0 = ld(d, 4 * q);
      const float4 w1 = ld(d, 4 * (q + kThreads));
      const float4 w2 = ld(d, 4 * (q + 2 * kThreads));
      const float4 w3 = ld(d, 4 * (q + 3 * kThreads));
      fold(w0);
      fold(w1);
      fold(w2);
      fold(w3);
    }
    for (; q < quads; q += kThreads) fold(ld(d, 4 * q));
  }
  m = block_max_u32(m, red);
  if (threadIdx.x == 0) partials[b] = m;
}

__global__ __launch_bounds__(kThreads) void amax_w_kernel(WSrc w, uint32_t* __restrict__ partials) {
  __shared__ uint32_t red[4];
  amax_w_block(w, blockIdx.x, gridDim.x, partials, red);
}

// --------------------------------------------------------- amax of bf16

__device__ inline uint32_t absmax_bits8(uint4 v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t lo = w[j] & 0x7fffu, hi = (w[j] >> 16) & 0x7fffu;
    const uint32_t a = lo > hi ? lo : hi;
    m = m > a ? m : a;
  }
  return m;
}

// Block b of nb: eight independent 16-byte loads in flight per thread.  NT
// streams the tensor past the caches (for a tensor that nothing reads again
// soon); otherwise the last-level cache keeps part of it for the quantiser.
template <bool NT>
__device__ __forceinline__ void amax_bf16_block(const uint16_t* __restrict__ x, int64_t n, int b,
                                                int nb, uint32_t* __restrict__ partials,
                                                uint32_t* red) {
  const int64_t vecs = n / 8, stride = (int64_t)nb * kThreads;
  const uint4* v = reinterpret_cast<const uint4*>(x);
  uint32_t m = 0;
  int64_t i = b * (int64_t)kThreads + threadIdx.x;
  for (; i + 7 * stride < vecs; i += 8 * stride) {
    uint4 a[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) a[j] = NT ? load_stream(v + i + j * stride) : v[i + j * stride];
#pragma unroll
    for (int j = 0; j < 8; ++j) m = max(m, absmax_bits8(a[j]));
  }
  for (; i < vecs; i += stride) m = max(m, absmax_bits8(v[i]));
  m = block_max_u32(m << 16, red);
  if (threadIdx.x == 0) partials[b] = m;
}

template <bool NT>
__global__ __launch_bounds__(kThreads) void amax_bf16_kernel(const uint16_t* __restrict__ x,
                                                             int64_t n,
                                                             uint32_t* __restrict__ partials) {
  __shared__ uint32_t red[4];
  amax_bf16_block<NT>(x, n, blockIdx.x, gridDim.x, partials, red);
}

// ----------------------------------------------- W_packed, both layouts

// One 64 (d) x 64 (n) tile per block, (bx, by) = (n / 64, d / 64).  Each
// fp32 weight is read once; its code goes straight to w_packed[d][n] and,
// through an LDS transpose, to w_packed_t[n][d].
__device__ __forceinline__ void quantize_w_block(
    const WSrc& w, int bx, int by, const uint32_t* __restrict__ partials, int parts,
    float* __restrict__ scales, int32_t* __restrict__ status, int status_bit,
    uint8_t* __restrict__ w_packed, uint8_t* __restrict__ w_packed_t, bool publish, bool reset,
    uint8_t (*tile_t)[64 + 4], uint32_t* red) {
  const int D = w.D, N = w.N;
  const int n0 = bx * 64, d0 = by * 64;
  const float inv = tensor_scales(partials, parts, red, publish, scales, status, status_bit,
                                  reset).y;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = threadIdx.x + kThreads * i;
    const int r = idx >> 4, c = (idx & 15) * 4;
    const int d = d0 + r, n = n0 + c;
    uint32_t code = 0;
    if (d < D && n < N) {
      float4 v = load_w4(w.wq, w.ldq, w.wk, w.ldk, w.wv, w.ldv, w.nq, d, n);
      code = e4m3x4(v.x * inv, v.y * inv, v.z * inv, v.w * inv);
      *reinterpret_cast<uint32_t*>(w_packed + (int64_t)d * N + n) = code;
    }
    tile_t[c + 0][r] = (uint8_t)(code);
    tile_t[c + 1][r] = (uint8_t)(code >> 8);
    tile_t[c + 2][r] = (uint8_t)(code >> 16);
    tile_t[c + 3][r] = (uint8_t)(code >> 24);
  }
  __syncthreads();
  {
    const int r = threadIdx.x >> 2, c = (threadIdx.x & 3) * 16;  // r: n_local, c: d_local
    const int n = n0 + r, d = d0 + c;
    if (n < N && d < D) {
      uint32_t q[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        q[j] = (uint32_t)tile_t[r][c + 4 * j] | ((uint32_t)tile_t[r][c + 4 * j + 1] << 8) |
               ((uint32_t)tile_t[r][c + 4 * j + 2] << 16) |
               ((uint32_t)tile_t[r][c + 4 * j + 3] << 24);
      *reinterpret_cast<uint4*>(w_packed_t + (int64_t)n * D + d) = make_uint4(q[0], q[1], q[2], q[3]);
    }
  }
}

__global__ __launch_bounds__(kThreads) void quantize_w_kernel(
    WSrc w, const uint32_t* __restrict__ partials, int parts, float* __restrict__ scales,
    int32_t* __restrict__ status, int status_bit, uint8_t* __restrict__ w_packed,
    uint8_t* __restrict__ w_packed_t, bool reset) {
  __shared__ uint8_t tile_t[64][64 + 4];
  __shared__ uint32_t red[4];
  quantize_w_block(w, blockIdx.x, blockIdx.y, partials, parts, scales, status, status_bit,
                   w_packed, w_packed_t, blockIdx.x == 0 && blockIdx.y == 0, reset, tile_t, red);
}

// ------------------------------ bf16 rows -> e4m3, blocked row layout

// One block per 128 tokens x 128 columns (one K block of the row layout).
// The source rows are the tokens' first `split` columns, `split` elements
// apart, followed by the columns of V-like head-major rows: column
// split + h * vw + j of token t is element j of row
// (t / vs * vh + h) * vs + t % vs of `vsrc` (vw elements per row, vh heads,
// sequences of vs tokens).  Thread (rg, cc) owns tokens 8rg..8rg+7 and
// columns 8cc..8cc+7: it reads 8 x 16 bytes of bf16 and writes 8 x 8 bytes
// of codes (16 threads cover a block row's 128 bytes).
struct ActSrc {
  const uint16_t* src;   // [rows][split], or null: those columns of rows < rows are
  int split;             // written by another kernel (neither read nor written here)
  const uint16_t* vsrc;  // head-major rows of the remaining columns
  int vw, vh, vs;
};

// Block (bx, by) of a (., gy) grid: tokens 128 bx .. and K block by; block
// (0, gy - 1) publishes the scale (the last K block holds columns it
// writes, also when src is null).
template <bool E5>
__device__ __forceinline__ void quantize_act_block(
    const ActSrc& as, int64_t rows, int cols, int bx, int by, int gy,
    const uint32_t* __restrict__ partials, int parts, float* __restrict__ scales,
    int32_t* __restrict__ status, int status_bit, uint8_t* __restrict__ dst,
    int64_t tokens_padded, uint32_t* red) {
  const int64_t t0 = (int64_t)bx * kKBlock;                // first token
  const int kb = by, c0 = kb * kKBlock;                    // K block of the row layout
  const int cc = threadIdx.x & 15, rg = threadIdx.x >> 4;
  const int kblocks = (int)ceil_div(cols, kKBlock);
  const int c = c0 + 8 * cc;
  // a block with only columns left to another kernel and no padding rows
  if (!as.src && c0 + kKBlock <= as.split && t0 + kKBlock <= rows) return;
  uint4 in[8];  // the tile's loads go out before the scale reduction
  const bool head_major = c >= as.split;
  const bool skip = !as.src && !head_major;  // real rows of these columns are not ours
  const int hv = head_major ? (c - as.split) / as.vw : 0;
  const int jv = head_major ? c - as.split - hv * as.vw : 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t t = t0 + 8 * rg + i;
    in[i] = make_uint4(0, 0, 0, 0);
    if (t < rows && c < cols && !skip) {
      const uint16_t* p;
      if (head_major) {  // tokens < 2^24: 32-bit division
        const int b = (int)t / as.vs;
        p = as.vsrc + (((int64_t)b * as.vh + hv) * as.vs + ((int)t - b * as.vs)) * as.vw + jv;
      } else {
        p = as.src + t * as.split + c;
      }
      in[i] = load_stream(p);  // read once: streamed past the caches
    }
  }
  const float inv = tensor_scales(partials, parts, red, bx == 0 && by == gy - 1, scales, status,
                                  status_bit, false, E5 ? kE5m2Max : kE4m3Max).y;
  // rows rows .. tokens_padded - 1 (zero input) are written as zero codes:
  // the dW GEMM reads them as its K tail
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t t = t0 + 8 * rg + i;
    const uint4 v = in[i];
    const uint32_t lo = fp8x4<E5>(bf16_to_f32(v.x & 0xffffu) * inv, bf16_to_f32(v.x >> 16) * inv,
                                  bf16_to_f32(v.y & 0xffffu) * inv, bf16_to_f32(v.y >> 16) * inv);
    const uint32_t hi = fp8x4<E5>(bf16_to_f32(v.z & 0xffffu) * inv, bf16_to_f32(v.z >> 16) * inv,
                                  bf16_to_f32(v.w & 0xffffu) * inv, bf16_to_f32(v.w >> 16) * inv);
    if (t < tokens_padded && !(skip && t < rows)) {
      const int64_t blk = (t / kActRows) * kblocks + kb;
      *reinterpret_cast<uint2*>(dst + (blk * kActRows + t % kActRows) * kKBlock + 8 * cc) =
          make_uint2(lo, hi);
    }
  }
}

template <bool E5>
__global__ __launch_bounds__(kThreads) void quantize_act_kernel(
    ActSrc as, int64_t rows, int cols, const uint32_t* __restrict__ partials, int parts,
    float* __restrict__ scales, int32_t* __restrict__ status, int status_bit,
    uint8_t* __restrict__ dst, int64_t tokens_padded) {
  __shared__ uint32_t red[4];
  quantize_act_block<E5>(as, rows, cols, blockIdx.x, blockIdx.y, gridDim.y, partials, parts,
                         scales, status, status_bit, dst, tokens_padded, red);
}

// ------------------------------- the weight pack and x in shared launches
//
// For a step that packs fresh weights and then runs the forward: the amax
// blocks of one or two weights and of x run in one launch, then the
// weights' quantiser tiles and x's quantiser blocks in the next, so the
// small, latency-bound weight work overlaps the activation streams instead
// of running before them.  Each tensor keeps its own partials, scales and
// status bit; block 0 of the amax launch clears the status word (the
// weight pack's reset) before either quantiser can set a bit.

// One weight: its pieces, parts_w amax partials, scales and both layouts.
struct WJob {
  WSrc w;
  uint32_t* partials;
  float* scales;
  uint8_t* packed;
  uint8_t* packed_t;
};

__device__ __forceinline__ int w_tiles_x(const WSrc& w) { return (int)ceil_div(w.N, 64); }
__device__ __forceinline__ int w_tiles(const WSrc& w) {
  return w_tiles_x(w) * (int)ceil_div(w.D, 64);
}

// Blocks [0, nw parts_w): weight b / parts_w, its block b % parts_w; the
// rest x, parts_x blocks.
__global__ __launch_bounds__(kThreads) void amax_wx_kernel(WJob a, WJob b, int nw, int parts_w,
                                                           const uint16_t* __restrict__ x,
                                                           int64_t n, int parts_x,
                                                           uint32_t* __restrict__ px,
                                                           int32_t* __restrict__ status) {
  __shared__ uint32_t red[4];
  const int blk = blockIdx.x;
  if (blk == 0 && threadIdx.x == 0) *status = 0;
  if (blk < nw * parts_w) {
    const WJob& j = blk < parts_w ? a : b;
    amax_w_block(j.w, blk % parts_w, parts_w, j.partials, red);
  } else {
    amax_bf16_block<false>(x, n, blk - nw * parts_w, parts_x, px, red);
  }
}

// Blocks [0, tiles of a): a's 64 x 64 tiles in row order, then b's (nw =
// 2), then x's, gy_x consecutive blocks per 128 tokens.  Each weight's
// first tile publishes its scale.
__global__ __launch_bounds__(kThreads) void quantize_wx_kernel(
    WJob a, WJob b, int nw, int parts_w, int w_bit, ActSrc as, int64_t rows, int cols, int gy_x,
    const uint32_t* __restrict__ px, int parts_x, float* __restrict__ x_scales, int x_bit,
    uint8_t* __restrict__ x8, int64_t tokens_padded, int32_t* __restrict__ status) {
  __shared__ uint8_t tile_t[64][64 + 4];
  __shared__ uint32_t red[4];
  const int na = w_tiles(a.w), nb = nw > 1 ? w_tiles(b.w) : 0;
  const int blk = blockIdx.x;
  if (blk < na + nb) {
    const bool first = blk < na;
    const WJob& j = first ? a : b;
    const int t = first ? blk : blk - na, gx = w_tiles_x(j.w);
    quantize_w_block(j.w, t % gx, t / gx, j.partials, parts_w, j.scales, status, w_bit, j.packed,
                     j.packed_t, t == 0, false, tile_t, red);
  } else {
    const int bb = blk - na - nb;
    quantize_act_block<false>(as, rows, cols, bb / gy_x, bb % gy_x, gy_x, px, parts_x, x_scales,
                              status, x_bit, x8, tokens_padded, red);
  }
}

template <bool E5>
__global__ __launch_bounds__(kThreads) void encode_kernel(const float* __restrict__ in, int64_t n,
                                                          float inv, uint8_t* __restrict__ out) {
  const int64_t i = (blockIdx.x * (int64_t)kThreads + threadIdx.x) * 16;
  if (i >= n) return;
  const float4* p = reinterpret_cast<const float4*>(in + i);
  uint32_t w[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float4 f = p[j];
    w[j] = fp8x4<E5>(f.x * inv, f.y * inv, f.z * inv, f.w * inv);
  }
  *reinterpret_cast<uint4*>(out + i) = make_uint4(w[0], w[1], w[2], w[3]);
}

// --------------------------------------------------------------- launchers

void launch_amax_w(const float* wq, int64_t ldq, const float* wk, int64_t ldk, const float* wv,
                   int64_t ldv, int D, int nq, int N, uint32_t* partials, int parts,
                   hipStream_t s) {
  amax_w_kernel<<<parts, kThreads, 0, s>>>(WSrc{wq, ldq, wk, ldk, wv, ldv, D, nq, N}, partials);
}

void launch_amax_bf16(const uint16_t* x, int64_t n, uint32_t* partials, int parts,
                      hipStream_t s, bool stream) {
  if (stream)
    amax_bf16_kernel<true><<<parts, kThreads, 0, s>>>(x, n, partials);
  else
    amax_bf16_kernel<false><<<parts, kThreads, 0, s>>>(x, n, partials);
}

void launch_quantize_w(const float* wq, int64_t ldq, const float* wk, int64_t ldk,
                       const float* wv, int64_t ldv, int D, int nq, int N,
                       const uint32_t* partials, int parts, float* scales, int32_t* status,
                       int status_bit, uint8_t* w_packed, uint8_t* w_packed_t, hipStream_t s,
                       bool reset_status) {
  dim3 grid((unsigned)ceil_div(N, 64), (unsigned)ceil_div(D, 64));
  quantize_w_kernel<<<grid, kThreads, 0, s>>>(WSrc{wq, ldq, wk, ldk, wv, ldv, D, nq, N}, partials,
                                              parts, scales, status, status_bit, w_packed,
                                              w_packed_t, reset_status);
}

namespace {
WJob to_job(const WeightJob& j) {
  return WJob{WSrc{j.wq, j.ldq, j.wk, j.ldk, j.wv, j.ldv, j.D, j.nq, j.N}, j.partials, j.scales,
              j.packed, j.packed_t};
}
}  // namespace

void launch_amax_wx(const WeightJob* jobs, int njobs, int parts_w, const uint16_t* x, int64_t n,
                    uint32_t* px, int parts_x, int32_t* status, hipStream_t s) {
  const WJob a = to_job(jobs[0]), b = to_job(jobs[njobs > 1 ? 1 : 0]);
  amax_wx_kernel<<<njobs * parts_w + parts_x, kThreads, 0, s>>>(a, b, njobs, parts_w, x, n,
                                                                parts_x, px, status);
}

void launch_quantize_wx(const WeightJob* jobs, int njobs, int parts_w, int w_bit,
                        const uint16_t* x, int64_t rows, int cols, const uint32_t* px,
                        int parts_x, float* x_scales, int x_bit, uint8_t* x8,
                        int64_t tokens_padded, int32_t* status, hipStream_t s) {
  const WJob a = to_job(jobs[0]), b = to_job(jobs[njobs > 1 ? 1 : 0]);
  int64_t blocks = 0;
  for (int i = 0; i < njobs; ++i)
    blocks += ceil_div(jobs[i].N, 64) * ceil_div(jobs[i].D, 64);
  const int gy_x = (int)ceil_div(cols, kKBlock);
  blocks += (tokens_padded / kKBlock) * gy_x;
  const ActSrc as{x, cols, nullptr, 1, 1, 1};
  quantize_wx_kernel<<<(unsigned)blocks, kThreads, 0, s>>>(a, b, njobs, parts_w, w_bit, as, rows,
                                                           cols, gy_x, px, parts_x, x_scales,
                                                           x_bit, x8, tokens_padded, status);
}

void launch_quantize_act(const uint16_t* src, int64_t rows, int cols, const uint32_t* partials,
                         int parts, float* scales, int32_t* status, int status_bit, uint8_t* dst,
                         int64_t tokens_padded, hipStream_t s) {
  launch_quantize_act_split(src, cols, nullptr, 1, 1, 1, rows, cols, partials, parts, scales,
                            status, status_bit, dst, tokens_padded, s, false);
}

void launch_quantize_act_split(const uint16_t* src, int split, const uint16_t* vsrc, int vw,
                               int vh, int vs, int64_t rows, int cols, const uint32_t* partials,
                               int parts, float* scales, int32_t* status, int status_bit,
                               uint8_t* dst, int64_t tokens_padded, hipStream_t s, bool e5m2) {
  dim3 grid((unsigned)(tokens_padded / kKBlock), (unsigned)ceil_div(cols, kKBlock));
  const ActSrc as{src, split, vsrc, vw, vh, vs};
  if (e5m2)
    quantize_act_kernel<true><<<grid, kThreads, 0, s>>>(as, rows, cols, partials, parts, scales,
                                                        status, status_bit, dst, tokens_padded);
  else
    quantize_act_kernel<false><<<grid, kThreads, 0, s>>>(as, rows, cols, partials, parts, scales,
                                                         status, status_bit, dst, tokens_padded);
}

void launch_encode(const float* in, int64_t n, float inv, uint8_t* out, hipStream_t s,
                   bool e5m2) {
  const int64_t blocks = ceil_div(n / 16, kThreads);
  if (e5m2)
    encode_kernel<true><<<(unsigned)blocks, kThreads, 0, s>>>(in, n, inv, out);
  else
    encode_kernel<false><<<(unsigned)blocks, kThreads, 0, s>>>(in, n, inv, out);
}

}  // namespace fpr
