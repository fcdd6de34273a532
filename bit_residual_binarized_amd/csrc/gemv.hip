// Decode GEMV on packed planes: y = Σ_p g_p ⊙ (B_p (h_p ⊙ x)).
//
// RaBiT paper App. E.1 describes a CUDA GEMV that expands sign bits with
// shifts/XOR into fp16 FMAs; it notes the limit moves toward register
// throughput. On gfx950 the sign expansion is instead done by the int8
// matrix cores:
//
//  * u_p = h_p ⊙ x is formed exactly (float64), then held as a signed 31-bit
//    fixed-point integer u_fx = rint(u_p * 2^sh), sh chosen per (batch row,
//    path) so that max|u_fx| lies in [2^29, 2^30). u_fx is split into four
//    signed bytes (digits) d_0..d_3 with u_fx = Σ 256^i d_i.
//  * Σ_j s_j u_j = Σ_j u_j − 2 Σ_{bit_j = 1} u_j (s_j = 1 − 2 bit_j, paper
//    §5.4: additions and element-wise scaling).
//  * The masked sum Σ bit_j u_j is an int8 dot product: for a stored word w
//    of 32 columns and a slice t in 0..7, (w & (0x01010101 << t)) is a dword
//    of four int8 values bit * 2^t (t = 7: bit * -128) for the columns
//    8r + t, r = 0..3. One v_and per four weights feeds the MFMA
//    V_MFMA_I32_4X4X4_16B_I8 with the A operand broadcast from one of its 16
//    blocks: B block k (lanes 4k..4k+3) = one row per lane, A = the 4 digit
//    rows of the 4 columns of one (word, slice) combination. Per lane the
//    result is the 4 digit sums of that lane's row, kept per slice (8
//    int32 accumulators x 4 digits x 2 paths).
//  * All sums are exact integers; split-K partials are combined with int64
//    atomics (order-independent), and y = g_1 S_1 + g_2 S_2 is formed in
//    float64 and rounded once.
#include <algorithm>

#include "rabit_internal.h"

namespace rabit {

namespace {

// ---------------------------------------------------------------------------
// Workspace layout for the batch-1-style kernel, per batch row b:
//   abuf  uint32 [batch][KG][64 lanes][2 paths][2 vgprs]   (1 KiB per kg)
//   shift int32  [batch][2]
//   usum  int64  [batch][2]      Σ_j u_fx
//   acc   int64  [batch][2][RG*64]  split-K accumulators (zeroed by prep)
//   cnt   uint32 [batch][RG]        split-K arrival counters (zeroed by prep)
// ---------------------------------------------------------------------------
struct GemvWs {
  uint32_t* abuf;
  int* shift;
  long long* usum;
  long long* acc;
  unsigned* cnt;
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

__host__ inline GemvWs carve(void* ws, int out, int in, int batch) {
  const int KG = col_groups(in), RG = row_groups(out);
  char* p = (char*)ws;
  GemvWs w;
  w.abuf = (uint32_t*)p;
  p += align256((size_t)batch * KG * 64 * 4 * 4);
  w.shift = (int*)p;
  p += align256((size_t)batch * 2 * sizeof(int));
  w.usum = (long long*)p;
  p += align256((size_t)batch * 2 * sizeof(long long));
  w.acc = (long long*)p;
  p += align256((size_t)batch * 2 * RG * 64 * sizeof(long long));
  w.cnt = (unsigned*)p;
  return w;
}

__host__ inline size_t ws_bytes(int out, int in, int batch) {
  const int KG = col_groups(in), RG = row_groups(out);
  return align256((size_t)batch * KG * 64 * 4 * 4) + align256((size_t)batch * 2 * sizeof(int)) +
         align256((size_t)batch * 2 * sizeof(long long)) +
         align256((size_t)batch * 2 * RG * 64 * sizeof(long long)) +
         align256((size_t)batch * RG * sizeof(unsigned));
}

__device__ __forceinline__ double u_exact(const uint16_t* __restrict__ h, const uint16_t* __restrict__ x,
                                          int j) {
  return (double)f16_bits_to_f32(h[j]) * (double)bf16_bits_to_f32(x[j]);
}

// fixed point value of column j (0 past the end)
__device__ __forceinline__ int ufx_at(const uint16_t* __restrict__ h, const uint16_t* __restrict__ x,
                                      int in, int j, int sh) {
  if (j >= in) return 0;
  return (int)rint(ldexp(u_exact(h, x, j), sh));
}

// digit i (signed byte) of the balanced base-256 expansion of v
__device__ __forceinline__ uint32_t digit_byte(int v, int i) {
  int d = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    d = (int)(int8_t)(v & 0xFF);
    if (k == i) break;
    v = (v - d) >> 8;
  }
  return (uint32_t)(uint8_t)(int8_t)d;
}

// One workgroup per (batch row, path): max |u|, shift, digits, Σ u_fx; also
// clears the split-K accumulators and counters used by the main kernel.
__global__ __launch_bounds__(1024) void k_gemv_prep(const uint16_t* __restrict__ x,
                                                    const uint16_t* __restrict__ h, int in, int KG,
                                                    int out_pad, int RG, GemvWs ws) {
  const int b = blockIdx.x >> 1, p = blockIdx.x & 1;
  const uint16_t* xb = x + (size_t)b * in;
  const uint16_t* hp = h + (size_t)p * in;
  const int tid = threadIdx.x;
  __shared__ double smax[16];
  __shared__ long long ssum[16];
  __shared__ int s_sh;

  double m = 0.0;
  for (int j = tid; j < in; j += 1024) m = fmax(m, fabs(u_exact(hp, xb, j)));
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) m = fmax(m, __shfl_xor(m, s, 64));
  if ((tid & 63) == 0) smax[tid >> 6] = m;
  __syncthreads();
  if (tid == 0) {
    double mm = 0.0;
    for (int i = 0; i < 16; ++i) mm = fmax(mm, smax[i]);
    s_sh = (mm > 0.0) ? 29 - ilogb(mm) : 0;
  }
  __syncthreads();
  const int sh = s_sh;

  long long su = 0;
  for (int j = tid; j < in; j += 1024) su += (long long)ufx_at(hp, xb, in, j, sh);
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) su += __shfl_xor(su, s, 64);
  if ((tid & 63) == 0) ssum[tid >> 6] = su;

  // A operand dwords of this path: (kg, lane L, vgpr v)
  uint32_t* ab = ws.abuf + (size_t)b * KG * 256;
  const int ndw = KG * 128;
  for (int d = tid; d < ndw; d += 1024) {
    const int kg = d >> 7, L = (d >> 1) & 63, v = d & 1;
    const int c = 16 * v + (L >> 2);  // (word, slice) combination
    const int q = c >> 3, t = c & 7, i = L & 3;
    const int base = 128 * kg + 32 * q + t;
    uint32_t dw = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) dw |= digit_byte(ufx_at(hp, xb, in, base + 8 * r, sh), i) << (8 * r);
    ab[((size_t)kg * 64 + L) * 4 + p * 2 + v] = dw;
  }
  // clear split-K state
  long long* acc = ws.acc + ((size_t)b * 2 + p) * out_pad;
  for (int r = tid; r < out_pad; r += 1024) acc[r] = 0;
  if (p == 0)
    for (int r = tid; r < RG; r += 1024) ws.cnt[(size_t)b * RG + r] = 0;
  __syncthreads();
  if (tid == 0) {
    long long t = 0;
    for (int i = 0; i < 16; ++i) t += ssum[i];
    ws.usum[b * 2 + p] = t;
    ws.shift[b * 2 + p] = sh;
  }
}

// exact integer masked sum of one lane's row from its 8 slice accumulators
__device__ __forceinline__ long long combine_slices(const v4i (&acc)[8]) {
  long long m = 0;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    long long xd = 0;
#pragma unroll
    for (int t = 0; t < 7; ++t) xd += (long long)(acc[t][d] >> t);
    xd -= (long long)(acc[7][d] >> 7);  // slice 7 carries the factor -128
    m += xd * (1ll << (8 * d));
  }
  return m;
}

__device__ __forceinline__ void store_y(void* y, int y_dtype, size_t idx, double v) {
  if (y_dtype == RABIT_OUT_F32)
    ((float*)y)[idx] = (float)v;
  else
    ((uint16_t*)y)[idx] = f64_to_bf16_rne(v);
}

// One wave = one 64-row group x one K range; lane = row.
template <int KSPLIT>
__global__ __launch_bounds__(256) void k_gemv_b1(const uint4* __restrict__ planes,
                                                 const uint16_t* __restrict__ g, int out, int RG,
                                                 int KG, int S, int kg_per, GemvWs ws, void* y,
                                                 int y_dtype, int b) {
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int l = threadIdx.x & 63;
  if (wid >= RG * S) return;
  const int rg = wid / S, sp = wid - rg * S;
  const int kg0 = sp * kg_per;
  const int kg1 = min(KG, kg0 + kg_per);
  const uint4* __restrict__ ab = (const uint4*)(ws.abuf + (size_t)b * KG * 256);

  v4i acc[2][8];
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[p][t] = (v4i){0, 0, 0, 0};

  const uint4* pl = planes + unit_index(rg, 0, 0, l, KG);
  uint4 w0 = make_uint4(0, 0, 0, 0), w1 = w0, av = w0;
  if (kg0 < kg1) {
    w0 = load_nt(pl + (size_t)kg0 * 128);
    w1 = load_nt(pl + (size_t)kg0 * 128 + 64);
    av = ab[(size_t)kg0 * 64 + l];
  }
  for (int kg = kg0; kg < kg1; ++kg) {
    uint4 nw0 = w0, nw1 = w1, nav = av;
    if (kg + 1 < kg1) {
      nw0 = load_nt(pl + (size_t)(kg + 1) * 128);
      nw1 = load_nt(pl + (size_t)(kg + 1) * 128 + 64);
      nav = ab[(size_t)(kg + 1) * 64 + l];
    }
    const uint32_t ws0[4] = {w0.x, w0.y, w0.z, w0.w};
    const uint32_t ws1[4] = {w1.x, w1.y, w1.z, w1.w};
    const int a0[2] = {(int)av.x, (int)av.y};  // path 0: vgpr 0 (q = 0,1), vgpr 1 (q = 2,3)
    const int a1[2] = {(int)av.z, (int)av.w};  // path 1
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#define RABIT_SLICE(T)                                                                       \
  {                                                                                          \
    const int bw0 = (int)(ws0[q] & (0x01010101u << (T)));                                   \
    const int bw1 = (int)(ws1[q] & (0x01010101u << (T)));                                   \
    if (q & 1) {                                                                             \
      acc[0][T] = __builtin_amdgcn_mfma_i32_4x4x4i8(a0[q >> 1], bw0, acc[0][T], 4, 8 + (T), 0); \
      acc[1][T] = __builtin_amdgcn_mfma_i32_4x4x4i8(a1[q >> 1], bw1, acc[1][T], 4, 8 + (T), 0); \
    } else {                                                                                 \
      acc[0][T] = __builtin_amdgcn_mfma_i32_4x4x4i8(a0[q >> 1], bw0, acc[0][T], 4, (T), 0);  \
      acc[1][T] = __builtin_amdgcn_mfma_i32_4x4x4i8(a1[q >> 1], bw1, acc[1][T], 4, (T), 0);  \
    }                                                                                        \
  }
      RABIT_SLICE(0) RABIT_SLICE(1) RABIT_SLICE(2) RABIT_SLICE(3)
      RABIT_SLICE(4) RABIT_SLICE(5) RABIT_SLICE(6) RABIT_SLICE(7)
#undef RABIT_SLICE
    }
    w0 = nw0;
    w1 = nw1;
    av = nav;
  }

  const long long m0 = combine_slices(acc[0]);
  const long long m1 = combine_slices(acc[1]);
  const int row = rg * 64 + l;
  const int out_pad = RG * 64;
  long long M0 = m0, M1 = m1;
  if (KSPLIT) {
    long long* accp = ws.acc + (size_t)b * 2 * out_pad;
    atomicAdd((unsigned long long*)&accp[row], (unsigned long long)m0);
    atomicAdd((unsigned long long*)&accp[out_pad + row], (unsigned long long)m1);
    __threadfence();
    unsigned old = 0;
    if (l == 0) old = atomicAdd(&ws.cnt[(size_t)b * RG + rg], 1u);
    old = __shfl(old, 0, 64);
    if (old != (unsigned)(S - 1)) return;
    __threadfence();
    M0 = (long long)__hip_atomic_load((unsigned long long*)&accp[row], __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
    M1 = (long long)__hip_atomic_load((unsigned long long*)&accp[out_pad + row], __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
  }
  if (row < out) {
    const long long U0 = ws.usum[b * 2 + 0], U1 = ws.usum[b * 2 + 1];
    const int sh0 = ws.shift[b * 2 + 0], sh1 = ws.shift[b * 2 + 1];
    const double s0 = ldexp((double)(U0 - 2 * M0), -sh0);
    const double s1 = ldexp((double)(U1 - 2 * M1), -sh1);
    const double g0 = (double)f16_bits_to_f32(g[row]);
    const double g1 = (double)f16_bits_to_f32(g[out + row]);
    store_y(y, y_dtype, (size_t)b * out + row, g0 * s0 + g1 * s1);
  }
}

}  // namespace

size_t gemv_workspace_bytes(int out, int in, int batch) { return ws_bytes(out, in, batch); }

static void split_k(int RG, int KG, int* S_out, int* kg_per_out) {
  // split K so that the grid has about 2048 waves, at least 2 column groups each
  int S = std::max(1, std::min(KG / 2, (2048 + RG - 1) / RG));
  const int kg_per = (KG + S - 1) / S;
  S = (KG + kg_per - 1) / kg_per;
  *S_out = S;
  *kg_per_out = kg_per;
}

hipError_t launch_gemv_prepare(const uint16_t* h, int out, int in, const uint16_t* x, int batch,
                               void* ws, hipStream_t st) {
  const int KG = col_groups(in), RG = row_groups(out);
  GemvWs w = carve(ws, out, in, batch);
  hipLaunchKernelGGL(k_gemv_prep, dim3(2 * batch), dim3(1024), 0, st, x, h, in, KG, RG * 64, RG, w);
  return hipGetLastError();
}

hipError_t launch_gemv_run(const uint4* planes, const uint16_t* g, int out, int in, int batch,
                           void* y, int y_dtype, void* ws, hipStream_t st) {
  const int KG = col_groups(in), RG = row_groups(out);
  GemvWs w = carve(ws, out, in, batch);
  int S, kg_per;
  split_k(RG, KG, &S, &kg_per);
  const int blocks = (RG * S + 3) / 4;
  for (int b = 0; b < batch; ++b) {
    if (S > 1)
      hipLaunchKernelGGL(k_gemv_b1<1>, dim3(blocks), dim3(256), 0, st, planes, g, out, RG, KG, S,
                         kg_per, w, y, y_dtype, b);
    else
      hipLaunchKernelGGL(k_gemv_b1<0>, dim3(blocks), dim3(256), 0, st, planes, g, out, RG, KG, S,
                         kg_per, w, y, y_dtype, b);
  }
  return hipGetLastError();
}

hipError_t launch_gemv(const uint4* planes, const uint16_t* g, const uint16_t* h, int out, int in,
                       const uint16_t* x, int batch, void* y, int y_dtype, void* ws,
                       hipStream_t st) {
  hipError_t e = launch_gemv_prepare(h, out, in, x, batch, ws, st);
  if (e != hipSuccess) return e;
  return launch_gemv_run(planes, g, out, in, batch, y, y_dtype, ws, st);
}

}  // namespace rabit
