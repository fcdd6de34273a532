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

// Wave-wide reductions with DPP row operations (no LDS round trips): xor 1,
// xor 2, half-row mirror, row mirror, then the row broadcasts 15 and 31; the
// result is in lane 63 and is returned to every lane. The combination order
// is fixed, so every workgroup computing the same reduction gets the same bits.
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_i32(int v, int ident) {
  return __builtin_amdgcn_update_dpp(ident, v, CTRL, ROWS, 0xf, false);
}
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_f64(double v, double ident) {
  const long long b = __double_as_longlong(v), o = __double_as_longlong(ident);
  const int lo = __builtin_amdgcn_update_dpp((int)o, (int)b, CTRL, ROWS, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp((int)(o >> 32), (int)(b >> 32), CTRL, ROWS, 0xf, false);
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}
__device__ __forceinline__ double lane63_f64(double v) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane((int)b, 63), hi = __builtin_amdgcn_readlane((int)(b >> 32), 63);
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}
__device__ __forceinline__ double wave_max_f64(double v) {
  const double z = 0.0;  // identity: only non-negative values are reduced
  v = fmax(v, dpp_f64<0xB1, 0xf>(v, z));
  v = fmax(v, dpp_f64<0x4E, 0xf>(v, z));
  v = fmax(v, dpp_f64<0x141, 0xf>(v, z));
  v = fmax(v, dpp_f64<0x140, 0xf>(v, z));
  v = fmax(v, dpp_f64<0x142, 0xa>(v, z));
  v = fmax(v, dpp_f64<0x143, 0xc>(v, z));
  return lane63_f64(v);
}
__device__ __forceinline__ int wave_max_i32(int v) {
  const int lo = -2147483647 - 1;
  v = max(v, dpp_i32<0xB1, 0xf>(v, lo));
  v = max(v, dpp_i32<0x4E, 0xf>(v, lo));
  v = max(v, dpp_i32<0x141, 0xf>(v, lo));
  v = max(v, dpp_i32<0x140, 0xf>(v, lo));
  v = max(v, dpp_i32<0x142, 0xa>(v, lo));
  v = max(v, dpp_i32<0x143, 0xc>(v, lo));
  return __builtin_amdgcn_readlane(v, 63);
}
__device__ __forceinline__ int wave_sum_i32(int v) {
  v += dpp_i32<0xB1, 0xf>(v, 0);
  v += dpp_i32<0x4E, 0xf>(v, 0);
  v += dpp_i32<0x141, 0xf>(v, 0);
  v += dpp_i32<0x140, 0xf>(v, 0);
  v += dpp_i32<0x142, 0xa>(v, 0);
  v += dpp_i32<0x143, 0xc>(v, 0);
  return __builtin_amdgcn_readlane(v, 63);
}

__device__ __forceinline__ double wave_sum_f64(double v) {
  v += dpp_f64<0xB1, 0xf>(v, 0.0);
  v += dpp_f64<0x4E, 0xf>(v, 0.0);
  v += dpp_f64<0x141, 0xf>(v, 0.0);
  v += dpp_f64<0x140, 0xf>(v, 0.0);
  v += dpp_f64<0x142, 0xa>(v, 0.0);
  v += dpp_f64<0x143, 0xc>(v, 0.0);
  return lane63_f64(v);
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
// out of line: the rare general case stays out of the hot instruction stream
static __device__ __attribute__((noinline)) uint16_t f64_to_bf16_rne_slow(double d) {
  return f64_to_bf16_rne(d);
}

// Same result as f64_to_bf16_rne, with a short branch-free path for values
// whose bfloat16 rounding lies in the normal range (float64 binades -126 ..
// 127): the exponent is rebiased and the 52-bit mantissa rounded half to even
// at bit 45; a carry out of the mantissa moves into the exponent (up to the
// infinity pattern). Everything else takes the general conversion.
__device__ __forceinline__ uint16_t f64_to_bf16_rne_fast(double d) {
  const uint64_t b = (uint64_t)__double_as_longlong(d);
  const uint32_t e = (uint32_t)(b >> 52) & 0x7FFu;
  if (e >= 897u && e <= 1150u) {
    const uint64_t r = (b & 0x7FFFFFFFFFFFFFFFull) - ((uint64_t)896 << 52);
    const uint64_t q = (r + 0xFFFFFFFFFFFull + ((r >> 45) & 1)) >> 45;  // + 2^44 - 1 + lsb: half to even
    return (uint16_t)(((b >> 63) << 15) | q);
  }
  return f64_to_bf16_rne_slow(d);
}

// float32 -> bfloat16, round to nearest even (NaN kept quiet)
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ---------------------------------------------------------------------------
// Direct buffer-to-LDS loads
// ---------------------------------------------------------------------------
// Raw (untyped, unswizzled) buffer resource word 3.
constexpr int kBufWord3 = 0x00020000;
typedef __attribute__((address_space(3))) void lds_void;

// Direct buffer-to-LDS loads of 16 and 4 bytes per lane: lane l writes its
// bytes at dst + size * l. (Plain device functions: inside a kernel template
// the builtin keeps the host pass from emitting the kernel's launch handle.)
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t r, lds_void* dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ void lds_load4(__amdgpu_buffer_rsrc_t r, lds_void* dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 4, voff, 0, 0, 0);
}

// s_waitcnt immediate: at most n vector-memory loads of this wave in flight
// and (lgkm0) none of its LDS accesses; expcnt unconstrained
__host__ __device__ constexpr int vmcnt_imm(int n, bool lgkm0 = false) {
  return (n & 15) | ((n >> 4) << 14) | (7 << 4) | ((lgkm0 ? 0 : 15) << 8);
}

// Workgroup barrier after this wave's loads but the last N have landed in
// LDS and its own LDS reads are done. A fence (__syncthreads) would wait for
// every load in flight, direct-to-LDS ones included; the empty asm
// statements keep the compiler from moving memory accesses across the
// barrier instead.
template <int N>
__device__ __forceinline__ void ring_barrier() {
  __builtin_amdgcn_sched_barrier(0);  // no instruction moves across a step boundary
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(N, true));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// ---------------------------------------------------------------------------
// Geometry of the V1 plane layout
// ---------------------------------------------------------------------------
__host__ __device__ __forceinline__ int row_groups(int out) { return (out + 63) / 64; }
__host__ __device__ __forceinline__ int col_groups(int in) { return (in + 127) / 128; }
// 16-byte unit (rg, kg, p, r) of a layer with P paths (layout V1)
__host__ __device__ __forceinline__ size_t unit_index(int rg, int kg, int p, int r, int KG, int P = 2) {
  return (((size_t)rg * KG + kg) * P + p) * 64 + r;
}

// ---------------------------------------------------------------------------
// Host-side launchers (each returns hipSuccess or the launch error)
// ---------------------------------------------------------------------------
size_t pack_workspace_bytes(int out, int in);
// normalized (with meanabs): h divided by the global mean |.| of the matrix
hipError_t launch_pack(const float* W, int out, int in, int P, bool meanabs, uint16_t* g,
                       uint16_t* h, uint4* planes, void* ws, hipStream_t st, bool normalized = false);
hipError_t launch_unpack(const uint4* planes, int out, int in, int P, uint32_t* words, hipStream_t st);

size_t gemv_workspace_bytes(int out, int in, int batch);
// paths: 2, or 3 for the 3-bit variant
hipError_t launch_gemv(const uint4* planes, const uint16_t* g, const uint16_t* h, int out, int in,
                       const uint16_t* x, int batch, void* y, int y_dtype, void* ws, hipStream_t st,
                       int paths = 2);
hipError_t launch_gemv_partial(const uint4* planes, const uint16_t* g, const uint16_t* h, int out,
                               int in, const uint16_t* x, int batch, void* ws, hipStream_t st,
                               int paths = 2);
hipError_t launch_gemv_reduce(int out, int in, int batch, void* y, int y_dtype, const void* ws,
                              hipStream_t st, int paths = 2);


// Several matrices that read the same input in one launch (q/k/v, gate/up):
// each leaves its partial buffer (header, then float32 partials
// [batch][slices][64*ceil(out/64)], slices at most ceil(in/512)) in part.
// With stats != nullptr the input is RMSNorm(x) (unit weight, eps), rounded to
// bfloat16, with stats[b][RABIT_STAT_PARTS] the partial sums of x^2 of row b.
struct LinSeg {
  const uint4* planes;
  const uint16_t* g;
  const uint16_t* h;
  int out;
  double* part;
  int paths = 2;  // every segment of a launch has the same number of paths
};
#define RABIT_STAT_PARTS 32

// A GEMV launch's partial buffer for one matrix: a 256-byte header whose
// first int32 is the number of partial slices per output row, then the
// float32 partials [batch][slices][64*ceil(out/64)] (the digit path writes one
// slice per range of 512 columns, the fp16 path one per chunk of ranges).
constexpr int kPartHdrDoubles = 32;
__host__ __device__ __forceinline__ int part_slices(const double* part) { return *(const int*)part; }
__host__ __device__ __forceinline__ const float* part_data(const double* part) {
  return (const float*)(part + kPartHdrDoubles);
}

// Σ_r part[b][r][i] over the S slices of a GEMV's partials (row
// stride `stride`), added in ascending r, with the loads of C ranges in flight
// together (clamped index, masked). sum_ranges, which the attention and
// SiLU consumers use, takes C = 8; the residual consumer takes C = 32 beyond
// 8 slices (measured: 64 in flight was slower than either).
template <int C>
__device__ __forceinline__ double sum_ranges_by(const float* __restrict__ pp, int S, int stride) {
  double v = 0.0;
  for (int r = 0; r < S; r += C) {
    double t[C];
#pragma unroll
    for (int u = 0; u < C; ++u) t[u] = (double)pp[(size_t)min(r + u, S - 1) * stride];
#pragma unroll
    for (int u = 0; u < C; ++u) v += r + u < S ? t[u] : 0.0;
  }
  return v;
}
// (part: the matrix's whole partial buffer, header included)
__device__ __forceinline__ double sum_ranges(const double* __restrict__ part, int b, int stride, int i) {
  const int S = part_slices(part);
  const size_t at = (size_t)b * S * stride + i;
  return sum_ranges_by<8>(part_data(part) + at, S, stride);
}
size_t gemv_part_bytes(int out, int in, int batch);

// Where a decode GEMV launch takes its input from (batch 1): the op between
// two linear layers is formed per column inside the second one, from the
// first one's partial buffers (slices summed in ascending order, as
// rabit_gemv_reduce does), instead of in a launch of its own.
enum GemvXMode { XSRC_X = 0, XSRC_ATTN = 1, XSRC_SILU = 2 };
struct GemvXSrc {
  int mode = XSRC_X;
  // XSRC_ATTN: column c = head h, dim d is bf16(v[(h / rep) head_dim + d])
  // (one-token attention), v = Σ of pa's slices; XSRC_SILU: column c is
  // bf16(silu(Σ pa) Σ pb) (gate, up)
  const double* pa = nullptr;
  const double* pb = nullptr;
  int head_dim = 1, rep = 1;
  // XSRC_ATTN: the q and k sums, fp32 into qk [n_q + kv], spread over the
  // launch's workgroups
  const double* pq = nullptr;
  const double* pk = nullptr;
  float* qk = nullptr;
  int n_q = 0, kv = 0;
};
hipError_t launch_gemv_multi(const LinSeg* segs, int nseg, int in, const uint16_t* x, int batch,
                             const double* stats, float eps, hipStream_t st,
                             const GemvXSrc* xs = nullptr);

size_t gemm_workspace_bytes(int out, int in, int m);
// weff: form the effective weight per tile in fp16 (one matrix op per tile
// instead of one per path)
hipError_t launch_gemm(const uint4* planes, const uint16_t* g, const uint16_t* h, int out, int in,
                       const uint16_t* X, int m, void* Y, int y_dtype, void* ws, hipStream_t st,
                       int paths = 2, bool weff = false);

// training side (dW, dg, dh; dX through the GEMM of the transposed layer)
size_t grad_weight_workspace_bytes(int out, int in, int P);
size_t grad_input_workspace_bytes(int out, int in, int m, int P);
hipError_t launch_transpose_planes(const uint4* planes, int out, int in, int P, uint4* planes_t,
                                   hipStream_t st);
hipError_t launch_grad_input(const uint4* planes, const uint16_t* g, const uint16_t* h, int out,
                             int in, int P, const uint16_t* dY, int m, void* dX, int dx_dtype,
                             void* ws, hipStream_t st, bool weff = false);
hipError_t launch_grad_weight(const uint4* planes, const uint16_t* g, const uint16_t* h, int out,
                              int in, int P, const uint16_t* X, const uint16_t* dY, int m, float* dW,
                              float* dg, float* dh, int accumulate, void* ws, hipStream_t st);

// initialisation: iterative residual SVID (g, h float32 [P][out], [P][in])
size_t svid_workspace_bytes(int out, int in);
hipError_t launch_svid(const float* W, int out, int in, int P, int sweeps, int passes,
                       const float* f_out, const float* f_in, bool cont, float* g, float* h,
                       uint4* planes, void* ws, hipStream_t st);

// decode glue (plain bf16 stand-ins around the binary linear layers)
hipError_t launch_rmsnorm(const uint16_t* x, uint16_t* y, int batch, int n, float eps, hipStream_t st);
hipError_t launch_attn_1tok(const float* v, int kv_rows, uint16_t* a, int batch, int n_heads,
                            int n_kv_heads, int head_dim, hipStream_t st);
hipError_t launch_silu_mul(const float* gate, const float* up, uint16_t* z, int batch, int n,
                           hipStream_t st);
hipError_t launch_residual_add(const uint16_t* x, const float* d, uint16_t* out, int batch, int n,
                               hipStream_t st);
// fused consumers of GEMV partial buffers (header with the slice count, row stride 64*ceil(out/64))
// x_out = bf16(x + Σ part) (part == nullptr: x_out unused, x itself), and the
// RABIT_STAT_PARTS partial sums of x_out^2 per row
hipError_t launch_resid_stats(const double* part, const uint16_t* x, uint16_t* x_out,
                              double* stats, int batch, int n, hipStream_t st);
// a = bf16(silu(Σ gate part) * Σ up part)
hipError_t launch_reduce_silu(const double* pg, const double* pu, uint16_t* a,
                              int batch, int n, hipStream_t st);
// q, k: fp32 sums (kept in qk); v = bf16(Σ part); attention over a one-token
// context returns, per head, its key/value group's v
hipError_t launch_reduce_attn(const double* pq, const double* pk, const double* pv,
                              float* qk, uint16_t* attn, int batch, int n_heads,
                              int n_kv_heads, int head_dim, hipStream_t st);
hipError_t launch_test_f64_to_16(const double* in, uint16_t* out, int n, int bf16, hipStream_t st);
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t st);

}  // namespace rabit
