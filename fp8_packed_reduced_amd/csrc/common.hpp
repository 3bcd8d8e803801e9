// Device helpers shared by the gfx950 kernels of libfpr.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fpr {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;        // every kernel runs 256-thread blocks (4 waves)
constexpr int kMaxPartials = 4096;   // upper bound on per-block amax partials

__host__ __device__ inline int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }
__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ------------------------------------------------------------------ bf16

__device__ inline float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN.
__device__ inline uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

typedef float v2f_t __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf_t __attribute__((ext_vector_type(2)));

// fp32 pair -> packed bf16 pair with the gfx950 converter: round to nearest
// even (the same bits as f32_to_bf16 for every non-NaN input).
__device__ inline uint32_t cvt_bf16x2_rn(float a, float b) {
  const v2f_t x = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, v2bf_t));
}

__device__ inline uint32_t pack_bf16x2(float a, float b) {
  return f32_to_bf16(a) | (f32_to_bf16(b) << 16);
}

// Sum of the products of two packed bf16 pairs, added to c in fp32
// (v_dot2_f32_bf16: each bf16 product is exact in fp32).
typedef __bf16 v2bf16_t __attribute__((ext_vector_type(2)));
__device__ inline float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2bf16_t, a),
                                        __builtin_bit_cast(v2bf16_t, b), c, false);
}

// ------------------------------------------------------------------ e4m3
//
// OCP E4M3 through the gfx950 converter (round to nearest even).  The
// explicit clamp to +-448 makes the conversion saturating for any input; a
// per-tensor amax scale never produces more than 448 * (1 + 2^-24) anyway.
__device__ inline float sat448(float v) { return __builtin_amdgcn_fmed3f(v, -448.0f, 448.0f); }

// Four fp32 values -> four e4m3 bytes, a in the lowest byte.
__device__ inline uint32_t e4m3x4(float a, float b, float c, float d) {
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(a), sat448(b), 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(sat448(c), sat448(d), lo, true);
}

// OCP E5M2 (the optional gradient format) through the gfx950 converter,
// clamped to +-57344 first so that it saturates instead of overflowing.
constexpr float kE4m3Max = 448.0f, kE5m2Max = 57344.0f;
__device__ inline float sat57344(float v) { return __builtin_amdgcn_fmed3f(v, -kE5m2Max, kE5m2Max); }

__device__ inline uint32_t e5m2x4(float a, float b, float c, float d) {
  int lo = __builtin_amdgcn_cvt_pk_bf8_f32(sat57344(a), sat57344(b), 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(sat57344(c), sat57344(d), lo, true);
}

// Four fp32 values -> four codes of format E5 (e5m2) or e4m3.
template <bool E5>
__device__ inline uint32_t fp8x4(float a, float b, float c, float d) {
  if constexpr (E5)
    return e5m2x4(a, b, c, d);
  else
    return e4m3x4(a, b, c, d);
}

// ------------------------------------------------------------------ RoPE
//
// "96 is enough", "The change": rope(q), rope(k).  Pair (i, i + d/2) of a
// head row at position p turns by p * base^(-2i/d).  The angle is formed in
// revolutions, p * theta_i / (2 pi) in double (positions reach 2^24 and the
// angle 2^24 rad), reduced to its fractional part, and the hardware sin/cos
// (v_sin_f32 / v_cos_f32 take revolutions) of that fraction in fp32.

// theta_i / (2 pi) = base^(-2i/d) / (2 pi)
__device__ inline double rope_rev(int i, int d, float base) {
  return exp2(-(2.0 * i / d) * log2((double)base)) * 0.15915494309189533576888376337251;
}

__device__ inline void rope_cs(double rev_i, int64_t pos, float& c, float& s) {
  const float f = (float)__builtin_amdgcn_fract((double)pos * rev_i);  // in [0, 1)
  s = __builtin_amdgcn_sinf(f);  // sin(2 pi f)
  c = __builtin_amdgcn_cosf(f);
}

// ------------------------------------------------------------ reductions

__device__ inline uint32_t wave_max_u32(uint32_t v) {
  for (int off = 32; off >= 1; off >>= 1) {
    uint32_t o = __shfl_xor(v, off, 64);
    v = v > o ? v : o;
  }
  return v;
}

// Max over the 256 threads of a block; every thread gets the result.
// A 16-byte load marked non-temporal: data read once and streamed past the
// caches, which then keep what the next kernels reuse.
__device__ inline uint4 load_stream(const void* p) {
  typedef unsigned v4u_l __attribute__((ext_vector_type(4)));
  const v4u_l v = __builtin_nontemporal_load(reinterpret_cast<const v4u_l*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ inline uint32_t block_max_u32(uint32_t v, uint32_t* lds4) {
  v = wave_max_u32(v);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) lds4[wave] = v;
  __syncthreads();
  uint32_t r = lds4[0];
  for (int i = 1; i < kThreads / 64; ++i) r = r > lds4[i] ? r : lds4[i];
  __syncthreads();
  return r;
}

// ---------------------------------------------------------------- scales

// The per-tensor scales from the amax partials (block-wide; every thread
// gets them): s = fl(amax / fmax), inv = fl(fmax / amax) with IEEE-correct
// fp32 divisions, fmax the format's largest finite value (448 for e4m3,
// 57344 for e5m2); (1, 1) for amax = 0, an inverse that overflows, or a
// non-finite amax.  The block that `publishes` writes scales[0..1] and, for
// a non-finite amax, sets `status_bit` in *status (overwriting *status
// when `reset`).
__device__ inline float2 tensor_scales(const uint32_t* __restrict__ partials, int parts,
                                       uint32_t* red, bool publish, float* __restrict__ scales,
                                       int32_t* __restrict__ status, int status_bit, bool reset,
                                       float fmax = kE4m3Max) {
  uint32_t m = 0;
#pragma unroll 8
  for (int i = threadIdx.x; i < parts; i += kThreads) m = m > partials[i] ? m : partials[i];
  m = block_max_u32(m, red);
  float sc = 1.0f, inv = 1.0f;
  const bool finite = m < 0x7f800000u;
  if (finite) {
    const float amax = __uint_as_float(m);
    const float i = fmax / amax;
    if (amax != 0.0f && i <= 3.40282347e38f) {
      sc = amax / fmax;
      inv = i;
    }
  }
  if (publish && threadIdx.x == 0) {
    scales[0] = sc;
    scales[1] = inv;
    if (reset)
      *status = finite ? 0 : status_bit;
    else if (!finite)
      atomicOr(status, status_bit);
  }
  return make_float2(sc, inv);
}

}  // namespace fpr
