// Measurement probes for gfx950: the ceilings the path's kernels are held
// against next to the published peaks, measured on the same device in the
// same run.
//  - copy: a streaming copy (16-byte non-temporal loads and stores, four in
//    flight per thread, grid-stride), the practical HBM ceiling of the
//    read-and-write kernels;
//  - read: a streaming read (16-byte non-temporal loads, four in flight,
//    folded into one word per block), that of the read-only (amax) kernels.
//    Of the forms tried (plain or non-temporal, four to sixteen loads in
//    flight, 4 to 64 blocks per CU, grid-stride or one contiguous chunk per
//    block) these were the fastest, by up to 20% over plain loads;
//  - mfma: back-to-back v_mfma_scale_f32_32x32x64_f8f6f4 on register
//    operands, four independent accumulators per wave and two waves per
//    SIMD, the practical FP8 matrix-core ceiling (no loads, no LDS).
#include "common.hpp"
#include "launch.hpp"

namespace fpr {

typedef float v16f_p __attribute__((ext_vector_type(16)));

typedef unsigned v4u_p __attribute__((ext_vector_type(4)));

// Four 16-byte non-temporal loads in flight per thread, then four
// streaming stores.
__global__ __launch_bounds__(kThreads) void probe_copy_kernel(const uint4* __restrict__ src,
                                                              uint4* __restrict__ dst,
                                                              int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    uint4 a[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] = load_stream(src + i + j * stride);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const v4u_p x = {a[j].x, a[j].y, a[j].z, a[j].w};
      __builtin_nontemporal_store(x, reinterpret_cast<v4u_p*>(dst + i + j * stride));
    }
  }
  for (; i < n; i += stride) dst[i] = src[i];
}

__global__ __launch_bounds__(kThreads) void probe_read_kernel(const uint4* __restrict__ src,
                                                              int64_t n,
                                                              uint32_t* __restrict__ out) {
  __shared__ uint32_t red[4];
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t x = 0;
  for (; i + 3 * stride < n; i += 4 * stride) {
    uint4 a[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] = load_stream(src + i + j * stride);
#pragma unroll
    for (int j = 0; j < 4; ++j) x ^= a[j].x ^ a[j].y ^ a[j].z ^ a[j].w;
  }
  for (; i < n; i += stride) {
    const uint4 a = src[i];
    x ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  x = block_max_u32(x, red);
  if (threadIdx.x == 0) out[blockIdx.x] = x;
}

// Each wave runs `iters` rounds of four independent MFMAs; the sums go to
// out[wave] so that nothing is optimised away.
__global__ __launch_bounds__(512, 1) void probe_mfma_kernel(int iters, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  v8i a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = 0x38383838 ^ (lane * 0x01010101 + j);  // e4m3 codes near 1.0
    b[j] = 0x38383838 ^ (j * 0x00010001);
  }
  v16f_p acc[4] = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      acc[q] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[q], 0, 0, 0, 127, 0, 127);
  }
  float s = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[q][e];
  if (lane == 0) out[blockIdx.x * 8 + (threadIdx.x >> 6)] = s;
}

void launch_probe_copy(const void* src, void* dst, int64_t bytes, int blocks, hipStream_t s) {
  probe_copy_kernel<<<blocks, kThreads, 0, s>>>(static_cast<const uint4*>(src),
                                                static_cast<uint4*>(dst), bytes / 16);
}

void launch_probe_read(const void* src, int64_t bytes, uint32_t* out, int blocks,
                       hipStream_t s) {
  probe_read_kernel<<<blocks, kThreads, 0, s>>>(static_cast<const uint4*>(src), bytes / 16, out);
}

int64_t probe_mfma_flop(int blocks, int iters) {
  return (int64_t)blocks * 8 * iters * 4 * (2 * 32 * 32 * 64);
}

void launch_probe_mfma(int blocks, int iters, float* out, hipStream_t s) {
  probe_mfma_kernel<<<blocks, 512, 0, s>>>(iters, out);
}

}  // namespace fpr
