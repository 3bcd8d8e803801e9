// FP8 (e4m3 x e4m3 -> fp32) GEMMs of the packed QKV projection on the gfx950
// matrix cores: forward x @ W_packed ("96 is enough", "The change": one FP8
// matmul, one launch, one weight read), dX through the cached row-major
// W_packed codes and dW = x^T dQKV (PR #344 page, "Changes": FP8 backward;
// "Where the eight seconds were hiding", "The inventory": the cached
// transposed view serves the backward pass).
//
// All three are C[m][n] = sum_k A[m][k] * B[n][k] with both operands
// K-contiguous in memory.  A block of 4 waves computes a BM x BN tile; each
// wave a (BM/2) x (BN/2) sub-tile from 16x16x128 MFMAs.  K advances 128 bytes
// per step through a double-buffered LDS stage; the 16-byte chunks of each
// 128-byte LDS row are XOR-swizzled by the row index so that the 16 rows a
// fragment read touches fall on distinct banks.
//
// The MFMA's first operand is fed from B (n rows) and its second from A (m
// rows).  Its 16x16 result then lands with lane l holding four consecutive n
// (4*(l/16) .. +3) of one m (l % 16): each lane stores 8 contiguous bytes of
// a row-major bf16 output (or 16 bytes of fp32).  Which k each byte of a
// lane's 32-byte operand stands for does not matter, as long as both
// operands use the same assignment, which they do.
#include "common.hpp"
#include "launch.hpp"

namespace fpr {

constexpr int kBK = 128;  // bytes (= e4m3 elements) of K per step

template <int BM, int BN>
struct TileCfg {
  static constexpr int WM = BM / 2, WN = BN / 2;        // 2 x 2 waves
  static constexpr int FM = WM / 16, FN = WN / 16;      // 16x16 fragments per wave
  static constexpr int A_CH = BM * (kBK / 16) / kThreads;  // 16 B chunks per thread
  static constexpr int B_CH = BN * (kBK / 16) / kThreads;
  static constexpr int STAGE = (BM + BN) * kBK;
  static_assert(A_CH * kThreads == BM * 8 && B_CH * kThreads == BN * 8, "tile/threads");
};

__device__ inline int swz(int row, int chunk) { return row * kBK + ((chunk ^ (row & 7)) << 4); }

// Workgroups are dispatched round-robin over the 8 XCDs (block b -> XCD b % 8).
// Give each XCD a contiguous run of tiles so that the N tiles of one M tile,
// which share their A rows, run on the same XCD and share its L2.
__device__ inline int xcd_contiguous(int b, int nblocks) {
  const int per = nblocks / 8, rem = nblocks % 8;
  const int xcd = b % 8, local = b / 8;
  return xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
}

__device__ inline v8i as_v8i(uint4 lo, uint4 hi) {
  v8i r;
  r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
  r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
  return r;
}

// splits == 1: tiles mapped XCD-contiguously.  splits > 1 (split-K): block b
// takes split b % splits of tile b / splits, so with 8 splits every XCD
// streams one K range for all tiles and the A/B rows are shared in its L2.
template <int BM, int BN, class Epi>
__global__ __launch_bounds__(kThreads) void gemm_e4m3_kernel(
    const uint8_t* __restrict__ A, int64_t lda, const uint8_t* __restrict__ B, int64_t ldb,
    int M, int N, int K, int n_tiles, int splits, int ksteps_per_split, Epi epi) {
  using C = TileCfg<BM, BN>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * C::STAGE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  int split = 0, tile;
  if (splits > 1) {
    split = blockIdx.x % splits;
    tile = blockIdx.x / splits;
  } else {
    tile = xcd_contiguous(blockIdx.x, gridDim.x);
  }
  const int m0 = (tile / n_tiles) * BM, n0 = (tile % n_tiles) * BN;
  const int nk = (K + kBK - 1) / kBK;
  const int ks0 = split * ksteps_per_split;
  const int ks1 = min(nk, ks0 + ksteps_per_split);

  v4f acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  uint4 ra[C::A_CH], rb[C::B_CH];
  // Rows past M / N are clamped to the last valid row (their results are
  // never stored); K chunks past K are zero.
  auto gload = [&](int ks) {
    const int k0 = ks * kBK;
#pragma unroll
    for (int i = 0; i < C::A_CH; ++i) {
      const int q = tid + kThreads * i, row = q >> 3, ch = q & 7;
      const int64_t grow = min(m0 + row, M - 1);
      const int kc = k0 + ch * 16;
      ra[i] = kc < K ? *reinterpret_cast<const uint4*>(A + grow * lda + kc) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < C::B_CH; ++i) {
      const int q = tid + kThreads * i, row = q >> 3, ch = q & 7;
      const int64_t grow = min(n0 + row, N - 1);
      const int kc = k0 + ch * 16;
      rb[i] = kc < K ? *reinterpret_cast<const uint4*>(B + grow * ldb + kc) : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&](int buf) {
    uint8_t* As = lds + buf * C::STAGE;
    uint8_t* Bs = As + BM * kBK;
#pragma unroll
    for (int i = 0; i < C::A_CH; ++i) {
      const int q = tid + kThreads * i;
      *reinterpret_cast<uint4*>(As + swz(q >> 3, q & 7)) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < C::B_CH; ++i) {
      const int q = tid + kThreads * i;
      *reinterpret_cast<uint4*>(Bs + swz(q >> 3, q & 7)) = rb[i];
    }
  };

  if (ks0 < ks1) {
    gload(ks0);
    sstore(0);
    __syncthreads();
    const int g = lane >> 4, r16 = lane & 15;
    for (int ks = ks0; ks < ks1; ++ks) {
      const int buf = (ks - ks0) & 1;
      if (ks + 1 < ks1) gload(ks + 1);
      const uint8_t* As = lds + buf * C::STAGE;
      const uint8_t* Bs = As + BM * kBK;
      v8i fb[C::FN];
#pragma unroll
      for (int j = 0; j < C::FN; ++j) {
        const int row = wn * C::WN + j * 16 + r16;
        fb[j] = as_v8i(*reinterpret_cast<const uint4*>(Bs + swz(row, 2 * g)),
                       *reinterpret_cast<const uint4*>(Bs + swz(row, 2 * g + 1)));
      }
#pragma unroll
      for (int i = 0; i < C::FM; ++i) {
        const int row = wm * C::WM + i * 16 + r16;
        const v8i fa = as_v8i(*reinterpret_cast<const uint4*>(As + swz(row, 2 * g)),
                              *reinterpret_cast<const uint4*>(As + swz(row, 2 * g + 1)));
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              fb[j], fa, acc[i][j], 0, 0, 0, 127, 0, 127);  // e4m3 x e4m3, unit E8M0 scales
      }
      if (ks + 1 < ks1) sstore(buf ^ 1);
      __syncthreads();
    }
  }

  Epi e = epi;
  e.prepare();
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
      const int m = m0 + wm * C::WM + i * 16 + (lane & 15);
      const int n = n0 + wn * C::WN + j * 16 + 4 * (lane >> 4);
      e(split, m, n, acc[i][j]);
    }
}

// ------------------------------------------------------------- epilogues

// Forward: scale, round to bf16; Q|K columns to the saved pre-norm rows,
// V columns straight into the head-major v output.
struct EpiFwd {
  const float* sx;
  const float* sw;
  uint16_t* qk_pre;
  uint16_t* v;
  int M, N, nqk2, H, dv, S;
  float alpha;
  __device__ void prepare() { alpha = sx[0] * sw[0]; }
  __device__ void operator()(int, int m, int n, v4f a) const {
    if (m >= M || n >= N) return;
    const uint2 p = make_uint2(pack_bf16x2(a[0] * alpha, a[1] * alpha),
                               pack_bf16x2(a[2] * alpha, a[3] * alpha));
    if (n < nqk2) {
      *reinterpret_cast<uint2*>(qk_pre + (int64_t)m * nqk2 + n) = p;
    } else {
      const int nn = n - nqk2, h = nn / dv, j = nn - h * dv;
      const int b = m / S, s = m - b * S;
      *reinterpret_cast<uint2*>(v + (((int64_t)b * H + h) * S + s) * dv + j) = p;
    }
  }
};

struct EpiDx {
  const float* sg;
  const float* sw;
  uint16_t* dx;
  int M, N;
  float alpha;
  __device__ void prepare() { alpha = sg[0] * sw[0]; }
  __device__ void operator()(int, int m, int n, v4f a) const {
    if (m >= M || n >= N) return;
    *reinterpret_cast<uint2*>(dx + (int64_t)m * N + n) =
        make_uint2(pack_bf16x2(a[0] * alpha, a[1] * alpha), pack_bf16x2(a[2] * alpha, a[3] * alpha));
  }
};

// dW split-K: unscaled fp32 partial sums, part[split][m][n].
struct EpiDwPart {
  float* part;
  int M, N;
  __device__ void prepare() {}
  __device__ void operator()(int split, int m, int n, v4f a) const {
    if (m >= M || n >= N) return;
    *reinterpret_cast<float4*>(part + ((int64_t)split * M + m) * N + n) =
        make_float4(a[0], a[1], a[2], a[3]);
  }
};

// Sum the split-K partials in split order (deterministic), scale, and write
// the three column blocks of dW.
__global__ __launch_bounds__(kThreads) void dw_reduce_kernel(
    const float* __restrict__ part, int splits, int D, int N, const float* __restrict__ sx,
    const float* __restrict__ sg, int nq, float* __restrict__ dwq, int64_t ldq,
    float* __restrict__ dwk, int64_t ldk, float* __restrict__ dwv, int64_t ldv) {
  const int64_t i = blockIdx.x * (int64_t)kThreads + threadIdx.x;  // float4 index
  const int64_t quads = (int64_t)D * N / 4;
  if (i >= quads) return;
  const int d = (int)(i / (N / 4)), n = (int)(i % (N / 4)) * 4;
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int k = 0; k < splits; ++k) {
    const float4 p = reinterpret_cast<const float4*>(part + ((int64_t)k * D + d) * N)[n / 4];
    s.x += p.x; s.y += p.y; s.z += p.z; s.w += p.w;
  }
  const float alpha = sx[0] * sg[0];
  s = make_float4(s.x * alpha, s.y * alpha, s.z * alpha, s.w * alpha);
  float* dst = n < nq ? dwq + d * ldq + n : n < 2 * nq ? dwk + d * ldk + (n - nq)
                                                       : dwv + d * ldv + (n - 2 * nq);
  *reinterpret_cast<float4*>(dst) = s;
}

// ------------------------------------------------------------- launchers

constexpr int kBM = 256, kBN = 192;

template <class Epi>
static void launch_gemm(const uint8_t* A, int64_t lda, const uint8_t* B, int64_t ldb, int M,
                        int N, int K, int splits, int ksteps_per_split, const Epi& epi,
                        hipStream_t s) {
  const int m_tiles = (int)ceil_div(M, kBM), n_tiles = (int)ceil_div(N, kBN);
  const int blocks = m_tiles * n_tiles * splits;
  gemm_e4m3_kernel<kBM, kBN, Epi><<<blocks, kThreads, 0, s>>>(A, lda, B, ldb, M, N, K, n_tiles,
                                                              splits, ksteps_per_split, epi);
}

void launch_gemm_fwd(const uint8_t* x8, const uint8_t* w_packed_t, int T, int N, int D,
                     const float* x_scales, const float* w_scales, uint16_t* qk_pre, int nqk2,
                     uint16_t* v, int H, int d_v, int seq_len, hipStream_t s) {
  EpiFwd e{x_scales, w_scales, qk_pre, v, T, N, nqk2, H, d_v, seq_len, 0.f};
  const int nk = (int)ceil_div(D, kBK);
  launch_gemm(x8, D, w_packed_t, D, T, N, D, 1, nk, e, s);
}

void launch_gemm_dx(const uint8_t* g8, const uint8_t* w_packed, int T, int D, int Np,
                    const float* g_scales, const float* w_scales, uint16_t* dx, hipStream_t s) {
  EpiDx e{g_scales, w_scales, dx, T, D, 0.f};
  const int nk = (int)ceil_div(Np, kBK);
  launch_gemm(g8, Np, w_packed, Np, T, D, Np, 1, nk, e, s);
}

int dw_splits(int64_t tokens_padded) {
  const int64_t nk = ceil_div(tokens_padded, kBK);
  return (int)(nk < 8 ? nk : 8);
}

size_t dw_partial_bytes(int D, int Np, int64_t tokens_padded) {
  return (size_t)dw_splits(tokens_padded) * D * Np * sizeof(float);
}

void launch_gemm_dw(const uint8_t* x8t, const uint8_t* g8t, int D, int Np, int64_t Tp,
                    float* part, hipStream_t s) {
  const int splits = dw_splits(Tp);
  const int nk = (int)ceil_div(Tp, kBK);
  const int per = (int)ceil_div(nk, splits);
  EpiDwPart e{part, D, Np};
  launch_gemm(x8t, Tp, g8t, Tp, D, Np, (int)Tp, splits, per, e, s);
}

void launch_dw_reduce(const float* part, int D, int Np, int64_t Tp, const float* x_scales,
                      const float* g_scales, float* dwq, int64_t ldq, float* dwk, int64_t ldk,
                      float* dwv, int64_t ldv, int nq, hipStream_t s) {
  const int64_t quads = (int64_t)D * Np / 4;
  dw_reduce_kernel<<<(unsigned)ceil_div(quads, kThreads), kThreads, 0, s>>>(
      part, dw_splits(Tp), D, Np, x_scales, g_scales, nq, dwq, ldq, dwk, ldk, dwv, ldv);
}

}  // namespace fpr
