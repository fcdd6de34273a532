// Internal declarations shared by the HIP translation units of librabit.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "rabit.h"

namespace rabit {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// streaming (non-temporal) 16-byte load
__device__ __forceinline__ uint4 load_nt(const uint4* p) {
  const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// ---------------------------------------------------------------------------
// Format helpers (device)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// Single direct round-to-nearest-even of a float64 to a 16-bit binary float
// with MANT stored mantissa bits, exponent bias BIAS, smallest normal
// exponent EMIN and largest binade EMAX (fp16: 10, 15, -14, 15; bf16: 7, 127,
// -126, 127). Written from the IEEE 754 definition: the magnitude is cut at
// the target quantum 2^(max(e, EMIN) - MANT) and rounded half to even;
// a carry out of the mantissa moves into the exponent field by addition.
template <int MANT, int BIAS, int EMIN, int EMAX, uint16_t QNAN>
__device__ __forceinline__ uint16_t f64_to_small_rne(double d) {
  const uint64_t b = (uint64_t)__double_as_longlong(d);
  const uint16_t sign = (uint16_t)((b >> 63) << 15);
  const uint64_t a = b & 0x7FFFFFFFFFFFFFFFull;
  const uint16_t inf = (uint16_t)(((2 * BIAS + 1) & ((1 << (15 - MANT)) - 1)) << MANT);
  if (a >= 0x7FF0000000000000ull) return sign | (a > 0x7FF0000000000000ull ? QNAN : inf);
  if (a == 0) return sign;
  const int ebits = (int)(a >> 52);
  if (ebits == 0) return sign;  // float64 subnormal: far below every 16-bit quantum
  const int e = ebits - 1023;
  if (e > EMAX) return sign | inf;
  const uint64_t sig = (a & ((1ull << 52) - 1)) | (1ull << 52);
  const int s = 52 - MANT + (e < EMIN ? EMIN - e : 0);
  if (s > 62) return sign;  // below half of the smallest subnormal
  uint64_t keep = sig >> s;
  const uint64_t rem = sig & ((1ull << s) - 1);
  const uint64_t half = 1ull << (s - 1);
  keep += (rem > half || (rem == half && (keep & 1))) ? 1 : 0;
  uint32_t bits = (e >= EMIN) ? ((uint32_t)(e + BIAS - 1) << MANT) + (uint32_t)keep : (uint32_t)keep;
  if (bits > inf) bits = inf;
  return sign | (uint16_t)bits;
}

__device__ __forceinline__ uint16_t f64_to_f16_rne(double d) {
  return f64_to_small_rne<10, 15, -14, 15, 0x7E00>(d);
}
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double d) {
  return f64_to_small_rne<7, 127, -126, 127, 0x7FC0>(d);
}
// float32 -> bfloat16, round to nearest even (NaN kept quiet)
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ---------------------------------------------------------------------------
// Geometry of the V1 plane layout
// ---------------------------------------------------------------------------
__host__ __device__ __forceinline__ int row_groups(int out) { return (out + 63) / 64; }
__host__ __device__ __forceinline__ int col_groups(int in) { return (in + 127) / 128; }
__host__ __device__ __forceinline__ size_t unit_index(int rg, int kg, int p, int r, int KG) {
  return (((size_t)rg * KG + kg) * 2 + p) * 64 + r;
}

// ---------------------------------------------------------------------------
// Host-side launchers (each returns hipSuccess or the launch error)
// ---------------------------------------------------------------------------
size_t pack_workspace_bytes(int out, int in);
hipError_t launch_pack(const float* W, int out, int in, bool meanabs, uint16_t* g, uint16_t* h,
                       uint4* planes, void* ws, hipStream_t st);
hipError_t launch_unpack(const uint4* planes, int out, int in, uint32_t* words, hipStream_t st);

size_t gemv_workspace_bytes(int out, int in, int batch);
hipError_t launch_gemv(const uint4* planes, const uint16_t* g, const uint16_t* h, int out, int in,
                       const uint16_t* x, int batch, void* y, int y_dtype, void* ws, hipStream_t st);
hipError_t launch_gemv_partial(const uint4* planes, const uint16_t* g, const uint16_t* h, int out,
                               int in, const uint16_t* x, int batch, void* ws, hipStream_t st);
hipError_t launch_gemv_reduce(int out, int in, int batch, void* y, int y_dtype, const void* ws,
                              hipStream_t st);

size_t gemm_workspace_bytes(int out, int in, int m);
hipError_t launch_gemm(const uint4* planes, const uint16_t* g, const uint16_t* h, int out, int in,
                       const uint16_t* X, int m, void* Y, int y_dtype, void* ws, hipStream_t st);

// decode glue (plain bf16 stand-ins around the binary linear layers)
hipError_t launch_rmsnorm(const uint16_t* x, uint16_t* y, int batch, int n, float eps, hipStream_t st);
hipError_t launch_attn_1tok(const float* v, int kv_rows, uint16_t* a, int batch, int n_heads,
                            int n_kv_heads, int head_dim, hipStream_t st);
hipError_t launch_silu_mul(const float* gate, const float* up, uint16_t* z, int batch, int n,
                           hipStream_t st);
hipError_t launch_residual_add(const uint16_t* x, const float* d, uint16_t* out, int batch, int n,
                               hipStream_t st);
hipError_t launch_test_f64_to_16(const double* in, uint16_t* out, int n, int bf16, hipStream_t st);

}  // namespace rabit
