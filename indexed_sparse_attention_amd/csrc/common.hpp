// Device helpers shared by the DSA kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

constexpr int kWave = 64;

// Number formats (values of dsa_dtype).
constexpr int kF32 = 0, kBF16 = 1, kE4M3 = 2;
// E4M3 elements with scales kept beside them: one E8M0 byte per 32 elements
// of a row (MXFP8, index keys), one fp32 per 128 elements (latent rows)
constexpr int kMXE4M3 = 3, kE4M3T128 = 4;

// Top-K histogram: the top 12 bits of the order-preserving score key.
constexpr int kHistBits = 12;
constexpr int kHistBins = 1 << kHistBits;
constexpr int kHistShift = 32 - kHistBits;

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;
typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);  // v_cvt_pk_bf16_f32: round to nearest even
}

// Two fp32 -> bf16 (round to nearest even) packed lo | hi << 16: one instruction.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f2v __attribute__((ext_vector_type(2)));
  typedef __bf16 b2v __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2v){lo, hi}, b2v));
}

// OCP E4M3 code -> f32 (exact).  s eeee mmm: e == 0 gives m * 2^-9, otherwise
// (1 + m/8) * 2^(e-7); s 1111 111 is NaN.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  uint32_t mag = c & 0x7Fu;
  float v;
  if (mag >= 8u) v = __uint_as_float((mag << 20) + (120u << 23));
  else v = (float)mag * 0.001953125f;  // 2^-9
  if (mag == 0x7Fu) v = __uint_as_float(0x7FC00000u);
  return (c & 0x80u) ? -v : v;
}

// Nearest E4M3 value of x (ties to even), saturating at +-448.  Used to
// quantise the index query when the index keys are E4M3.
__device__ __forceinline__ float e4m3_quantize(float x) {
  float a = fabsf(x);
  float r;
  if (a >= 448.0f) {
    r = 448.0f;
  } else if (a < 0.015625f) {  // subnormal range: spacing 2^-9
    r = rintf(a * 512.0f) * 0.001953125f;
  } else {
    int e;
    frexpf(a, &e);  // a = f * 2^e, f in [0.5, 1): spacing of e4m3 there is 2^(e-4)
    float spacing = ldexpf(1.0f, e - 4);
    r = rintf(a / spacing) * spacing;
  }
  return copysignf(r, x);
}

// E4M3 code of a value that is exactly representable (output of e4m3_quantize).
__device__ __forceinline__ uint32_t e4m3_code_exact(float v) {
  uint32_t s = (__float_as_uint(v) >> 24) & 0x80u;
  float a = fabsf(v);
  if (a < 0.015625f) return s | (uint32_t)(a * 512.0f);
  uint32_t u = __float_as_uint(a);
  return s | ((((u >> 23) - 120u) << 3) | ((u >> 20) & 7u));
}

// Order-preserving unsigned key of an fp32 score (larger score -> larger key);
// -0 and +0 share the key of +0.
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = (s == 0.0f) ? 0u : __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Stores that write through the L2 to memory (device-scope coherent: the
// `sc1` policy), for results a later kernel reads.  The eight XCDs' L2s are
// not coherent with one another, so the release at a kernel's end writes
// every line its ordinary stores left dirty back to memory before the next
// kernel may start: megabytes of results then leave after the last
// workgroup has finished.  Stored through, they leave while the kernel still
// runs.
__device__ __forceinline__ void store_through(void* p, i32x4 v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1" ::"v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ void store_through(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_through(int32_t* p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Stamps a workgroup's start (construction) and its first thread's exit
// (destruction) into a wg_trace region; nothing when the region is null.
struct WgTrace {
  uint64_t* tr;
  __device__ __forceinline__ void stamp(int which) const {
    if (tr && threadIdx.x == 0) {
      const int64_t w = blockIdx.x + (int64_t)gridDim.x * (blockIdx.y + (int64_t)gridDim.y * blockIdx.z);
      tr[2 * w + which] = __builtin_amdgcn_s_memrealtime();
    }
  }
  __device__ __forceinline__ explicit WgTrace(uint64_t* t) : tr(t) { stamp(0); }
  __device__ __forceinline__ ~WgTrace() { stamp(1); }
};

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ int clamp_len(int32_t len, int64_t lmax) {
  int64_t l = len < 0 ? 0 : (int64_t)len;
  return (int)(l > lmax ? lmax : l);
}

// Rows a launch treats as filled: seq_lens[b] clamped to [0, Lmax], less
// `sub` rows (a launch over a tile of a sequence's query tokens that ends
// `sub` tokens before the last one sees exactly as those tokens do), never
// below 0.
__device__ __forceinline__ int filled_rows(int32_t len, int64_t lmax, int sub) {
  const int l = clamp_len(len, lmax) - sub;
  return l > 0 ? l : 0;
}

}  // namespace dsa
