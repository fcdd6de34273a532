// Decode GEMV on packed planes: y = Σ_p g_p ⊙ (B_p (h_p ⊙ x)).
//
// RaBiT paper App. E.1 describes a CUDA GEMV that expands sign bits with
// shifts/XOR into fp16 FMAs and notes that the limit moves toward register
// throughput. On gfx950 the sign expansion is done by the int8 matrix cores:
//
//  * Σ_j s_j u_j = Σ_j u_j − 2 Σ_{bit_j = 1} u_j with s_j = 1 − 2 bit_j and
//    u = h_p ⊙ x (paper §5.4: additions and element-wise scaling).
//  * u is formed exactly (float64) and held as a fixed-point integer
//    u_fx = rint(u * 2^sh), with one exponent per (batch row, path, K range)
//    chosen so that the range's max |u_fx| lies in [2^29, 2^30); u_fx is
//    split into four signed bytes d_0..d_3, u_fx = Σ_i 256^i d_i.
//  * For a stored word w (32 columns of one row) and a slice t in 0..7,
//    (w & (0x01010101 << t)) is a dword of four int8 values bit * 2^t
//    (t = 7: bit * -128) for the columns 8r + t, r = 0..3. One v_and per four
//    weights feeds V_MFMA_I32_4X4X4_16B_I8 with the A operand broadcast from
//    one of its 16 blocks: lane = output row, A block = the 4 digit rows of
//    the 4 columns of one (word, slice) pair. Per lane and slice the result
//    is the 4 digit sums of that lane's row: 8 int32 accumulators x 4 digits.
//  * Per K range the sums are exact integers; the range result
//    g_1 S_1 + g_2 S_2 is formed in float64. Ranges are reduced in a fixed
//    order (4 waves of a workgroup through LDS, then workgroups by a small
//    kernel), so the output is bitwise repeatable. No atomics, no fences.
#include <algorithm>

#include "rabit_internal.h"

namespace rabit {

namespace {

constexpr int kWaves = 4;    // waves per workgroup; they share a row group and split K
constexpr int kMaxRing = 3;  // column groups (both paths) in flight per wave

// K split of one GEMV: S = kWaves * SG ranges of kg_per column groups (a
// multiple of the ring depth, so only the last range is ragged).
struct Plan {
  int RG, KG, SG, S, kg_per, ring;
};

__host__ inline Plan make_plan(int out, int in) {
  Plan p;
  p.RG = row_groups(out);
  p.KG = col_groups(in);
  const int target_waves = 2048;
  const int max_sg = std::max(1, (p.KG + kWaves - 1) / kWaves);
  p.SG = std::max(1, std::min(max_sg, (target_waves + kWaves * p.RG - 1) / (kWaves * p.RG)));
  p.S = kWaves * p.SG;
  const int kg_per = (p.KG + p.S - 1) / p.S;
  p.ring = std::min(kMaxRing, kg_per);
  p.kg_per = ((kg_per + p.ring - 1) / p.ring) * p.ring;
  return p;
}

// Workspace (all offsets 256-byte aligned):
//   abuf   uint32 [batch][KG+1][64 lanes][2 paths][2 vgprs] A operand images;
//                 slot KG is all zero (read by surplus ring slots)
//   rshift int32  [batch][2][S]                             per-range exponent
//   rusum  int64  [batch][2][S]                             per-range Σ u_fx
//   part   double [batch][SG][RG*64]                        per-workgroup partials
struct GemvWs {
  uint32_t* abuf;
  int* rshift;
  long long* rusum;
  double* part;
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

__host__ inline size_t ws_layout(const Plan& P, int batch, void* base, GemvWs* w) {
  const size_t sz[4] = {align256((size_t)batch * (P.KG + 1) * 64 * 4 * 4),
                        align256((size_t)batch * 2 * P.S * sizeof(int)),
                        align256((size_t)batch * 2 * P.S * sizeof(long long)),
                        align256((size_t)batch * P.SG * P.RG * 64 * sizeof(double))};
  char* p = (char*)base;
  if (w) {
    w->abuf = (uint32_t*)p;
    w->rshift = (int*)(p + sz[0]);
    w->rusum = (long long*)(p + sz[0] + sz[1]);
    w->part = (double*)(p + sz[0] + sz[1] + sz[2]);
  }
  return sz[0] + sz[1] + sz[2] + sz[3];
}

__device__ __forceinline__ double u_exact(const uint16_t* __restrict__ h,
                                          const uint16_t* __restrict__ x, int j) {
  return (double)f16_bits_to_f32(h[j]) * (double)bf16_bits_to_f32(x[j]);
}

__device__ __forceinline__ int ufx_at(const uint16_t* __restrict__ h,
                                      const uint16_t* __restrict__ x, int in, int j, int sh) {
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

__device__ __forceinline__ double wave_max(double v) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) v = fmax(v, __shfl_xor(v, s, 64));
  return v;
}
__device__ __forceinline__ long long wave_sum(long long v) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) v += __shfl_xor(v, s, 64);
  return v;
}

// One workgroup per (K range r, path p, batch row b): exponent, Σ u_fx and
// the A-operand images of the range's column groups.
__global__ __launch_bounds__(256) void k_gemv_prep(const uint16_t* __restrict__ x,
                                                   const uint16_t* __restrict__ h, int in, Plan P,
                                                   GemvWs ws) {
  const int r = blockIdx.x, p = blockIdx.y, b = blockIdx.z;
  const uint16_t* xb = x + (size_t)b * in;
  const uint16_t* hp = h + (size_t)p * in;
  const int kgA = min(P.KG, r * P.kg_per), kgB = min(P.KG, kgA + P.kg_per);
  const int c0 = kgA * 128, c1 = min(in, kgB * 128);
  __shared__ double smax[4];
  __shared__ long long ssum[4];

  double m = 0.0;
  for (int j = c0 + (int)threadIdx.x; j < c1; j += 256) m = fmax(m, fabs(u_exact(hp, xb, j)));
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) smax[threadIdx.x >> 6] = m;
  __syncthreads();
  m = fmax(fmax(smax[0], smax[1]), fmax(smax[2], smax[3]));
  const int sh = (m > 0.0) ? 29 - ilogb(m) : 0;

  long long su = 0;
  for (int j = c0 + (int)threadIdx.x; j < c1; j += 256) su += (long long)ufx_at(hp, xb, in, j, sh);
  su = wave_sum(su);
  if ((threadIdx.x & 63) == 0) ssum[threadIdx.x >> 6] = su;
  __syncthreads();
  if (threadIdx.x == 0) {
    ws.rshift[((size_t)b * 2 + p) * P.S + r] = sh;
    ws.rusum[((size_t)b * 2 + p) * P.S + r] = ((ssum[0] + ssum[1]) + ssum[2]) + ssum[3];
  }

  const int ndw = (kgB - kgA) * 128;
  for (int d = threadIdx.x; d < ndw; d += 256) {
    const int kg = kgA + (d >> 7), L = (d >> 1) & 63, v = d & 1;
    const int c = 16 * v + (L >> 2);  // (word, slice) pair of this A image
    const int q = c >> 3, t = c & 7, i = L & 3;
    const int base = 128 * kg + 32 * q + t;
    uint32_t dw = 0;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
      dw |= digit_byte(ufx_at(hp, xb, in, base + 8 * rr, sh), i) << (8 * rr);
    ws.abuf[(((size_t)b * (P.KG + 1) + kg) * 64 + L) * 4 + p * 2 + v] = dw;
  }
  if (r == 0 && p == 0) ws.abuf[((size_t)b * (P.KG + 1) + P.KG) * 256 + threadIdx.x] = 0;
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

// 32 MFMAs: one 128-column unit of one path (4 words x 8 slices)
__device__ __forceinline__ void mfma_unit(v4i (&acc)[8], const uint4& w, const uint2& a) {
  const uint32_t ws4[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int av = (int)((q < 2) ? a.x : a.y);
#define RABIT_SLICE(T)                                                                     \
  {                                                                                        \
    const int bw = (int)(ws4[q] & (0x01010101u << (T)));                                  \
    if (q & 1)                                                                             \
      acc[T] = __builtin_amdgcn_mfma_i32_4x4x4i8(av, bw, acc[T], 4, 8 + (T), 0);         \
    else                                                                                   \
      acc[T] = __builtin_amdgcn_mfma_i32_4x4x4i8(av, bw, acc[T], 4, (T), 0);             \
  }
    RABIT_SLICE(0) RABIT_SLICE(1) RABIT_SLICE(2) RABIT_SLICE(3)
    RABIT_SLICE(4) RABIT_SLICE(5) RABIT_SLICE(6) RABIT_SLICE(7)
#undef RABIT_SLICE
  }
}

// Workgroup = 4 waves on one 64-row group, wave w takes K range 4*sg + w.
// blockIdx.y = batch row. RING column groups (both paths) are in flight per
// wave. The loop has no data-dependent branch: the trip count is rounded up
// to a multiple of RING, and surplus groups read their A operand from a zero
// image (their weights are a clamped re-read), so they add exactly 0.
template <int RING>
__global__ __launch_bounds__(256) void k_gemv_main(const uint4* __restrict__ planes,
                                                   const uint16_t* __restrict__ g, int out,
                                                   Plan P, GemvWs ws, void* y, int y_dtype) {
  const int rg = blockIdx.x / P.SG, sg = blockIdx.x - rg * P.SG;
  const int b = blockIdx.y;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), l = threadIdx.x & 63;
  const int r = sg * kWaves + w;
  const int kgA = min(P.KG, r * P.kg_per), kgB = min(P.KG, kgA + P.kg_per);
  const int nk = __builtin_amdgcn_readfirstlane(kgB - kgA);
  const int nkr = __builtin_amdgcn_readfirstlane(((nk + RING - 1) / RING) * RING);

  const uint4* __restrict__ wbase = planes + unit_index(rg, kgA, 0, l, P.KG);
  const uint4* __restrict__ abase = (const uint4*)(ws.abuf + (((size_t)b * (P.KG + 1) + kgA) * 64 + l) * 4);
  const uint4* __restrict__ azero = (const uint4*)(ws.abuf + (((size_t)b * (P.KG + 1) + P.KG) * 64 + l) * 4);

  v4i acc0[8], acc1[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) acc0[t] = acc1[t] = (v4i){0, 0, 0, 0};
  long long M0 = 0, M1 = 0;
  if (nk > 0) {
    uint4 w0[RING], w1[RING], av[RING];
#pragma unroll
    for (int i = 0; i < RING; ++i) {
      const int k = min(i, nk - 1);
      av[i] = *((i < nk) ? abase + (size_t)i * 64 : azero);
      w0[i] = load_nt(wbase + (size_t)k * 128);
      w1[i] = load_nt(wbase + (size_t)k * 128 + 64);
      __builtin_amdgcn_sched_barrier(0);
    }
    for (int k0 = 0; k0 < nkr; k0 += RING) {
#pragma unroll
      for (int i = 0; i < RING; ++i) {
        mfma_unit(acc0, w0[i], make_uint2(av[i].x, av[i].y));
        mfma_unit(acc1, w1[i], make_uint2(av[i].z, av[i].w));
        // keep each slot's three loads together and in ring order: loads
        // complete in order, so the wait before a slot then covers only it
        __builtin_amdgcn_sched_barrier(0);
        const int kn = k0 + i + RING;
        const int k = min(kn, nk - 1);
        av[i] = *((kn < nk) ? abase + (size_t)kn * 64 : azero);
        w0[i] = load_nt(wbase + (size_t)k * 128);
        w1[i] = load_nt(wbase + (size_t)k * 128 + 64);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    M0 = combine_slices(acc0);
    M1 = combine_slices(acc1);
  }

  const int row = rg * 64 + l;
  const size_t ri0 = ((size_t)b * 2 + 0) * P.S + r, ri1 = ((size_t)b * 2 + 1) * P.S + r;
  double part = 0.0;
  if (nk > 0 && row < out) {
    const double s0 = ldexp((double)(ws.rusum[ri0] - 2 * M0), -ws.rshift[ri0]);
    const double s1 = ldexp((double)(ws.rusum[ri1] - 2 * M1), -ws.rshift[ri1]);
    part = (double)f16_bits_to_f32(g[row]) * s0 + (double)f16_bits_to_f32(g[out + row]) * s1;
  }
  __shared__ double red[kWaves][64];
  red[w][l] = part;
  __syncthreads();
  if (w == 0) {
    double v = red[0][l];
    v += red[1][l];
    v += red[2][l];
    v += red[3][l];
    if (P.SG == 1) {
      if (row < out) store_y(y, y_dtype, (size_t)b * out + row, v);
    } else {
      ws.part[((size_t)b * P.SG + sg) * P.RG * 64 + row] = v;
    }
  }
}

// y = Σ_sg part (ascending sg)
__global__ __launch_bounds__(256) void k_gemv_reduce(int out, Plan P, GemvWs ws, void* y,
                                                     int y_dtype) {
  const int row = blockIdx.x * 256 + threadIdx.x, b = blockIdx.y;
  if (row >= out) return;
  const double* pp = ws.part + (size_t)b * P.SG * P.RG * 64 + row;
  double v = 0.0;
  for (int s = 0; s < P.SG; ++s) v += pp[(size_t)s * P.RG * 64];
  store_y(y, y_dtype, (size_t)b * out + row, v);
}

}  // namespace

size_t gemv_workspace_bytes(int out, int in, int batch) {
  return ws_layout(make_plan(out, in), batch, nullptr, nullptr);
}

hipError_t launch_gemv_prepare(const uint16_t* h, int out, int in, const uint16_t* x, int batch,
                               void* ws, hipStream_t st) {
  const Plan P = make_plan(out, in);
  GemvWs w;
  ws_layout(P, batch, ws, &w);
  hipLaunchKernelGGL(k_gemv_prep, dim3(P.S, 2, batch), dim3(256), 0, st, x, h, in, P, w);
  return hipGetLastError();
}

hipError_t launch_gemv_run(const uint4* planes, const uint16_t* g, int out, int in, int batch,
                           void* y, int y_dtype, void* ws, hipStream_t st) {
  const Plan P = make_plan(out, in);
  GemvWs w;
  ws_layout(P, batch, ws, &w);
  const dim3 grid(P.RG * P.SG, batch);
  if (P.ring == 1)
    hipLaunchKernelGGL(k_gemv_main<1>, grid, dim3(256), 0, st, planes, g, out, P, w, y, y_dtype);
  else if (P.ring == 2)
    hipLaunchKernelGGL(k_gemv_main<2>, grid, dim3(256), 0, st, planes, g, out, P, w, y, y_dtype);
  else
    hipLaunchKernelGGL(k_gemv_main<3>, grid, dim3(256), 0, st, planes, g, out, P, w, y, y_dtype);
  if (P.SG > 1)
    hipLaunchKernelGGL(k_gemv_reduce, dim3((out + 255) / 256, batch), dim3(256), 0, st, out, P, w,
                       y, y_dtype);
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
