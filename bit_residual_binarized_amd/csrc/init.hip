// Initialisation of the scales (RaBiT paper §4.3): iterative residual SVID,
// optionally on the importance-preconditioned matrix.
//
// Sweep t re-fits path i to R_i = W' − Σ_{j≠i} g_j ⊙ B_j ⊙ h_j (paths before
// i already re-fitted in this sweep), with B_i = sign(R_i) and g_i h_iᵀ the
// leading rank-1 term of |R_i|. The rank-1 term comes from power iteration on
// |R_i|, warm-started from the path's previous h_i: a rows pass u = |R_i| v,
// then alternating columns passes v = |R_i|ᵀ u and rows passes, each pass
// one read of W (R_i is rebuilt on the fly from W and the other paths' bits
// and scales; nothing the size of W is stored). The first rows pass of a
// re-fit also writes the bits of B_i. With σ = ||u|| / ||v|| after the last
// rows pass, g_i = u / (sqrt(σ) ||v||) and h_i = sqrt(σ) v / ||v||.
//
// Arithmetic: R in float32 (W' = fl(fl(f_out W) f_in), then each other path's
// fl(g_j h_j) subtracted in path order), pass sums in float32 inside a tile,
// tiles added in float64 (four interleaved slices in ascending order, then
// the slices in order), vectors stored in float32.
#include <algorithm>
#include <math.h>

#include "rabit_internal.h"

namespace rabit {

namespace {

constexpr int kR = 64;    // tile rows
constexpr int kC = 256;   // tile columns
constexpr int kRedWg = 256;

__host__ inline size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }

struct SvidWs {
  float* gp;        // [P][out] scales in the preconditioned domain
  float* hp;        // [P][in]
  float* u;         // [out]
  float* v;         // [in]
  float* part;      // pass partials: rows pass [ceil(in/256)][out], columns pass [ceil(out/64)][in]
  double* sq_u;     // [ceil(out/64)] partial Σ u²
  double* sq_v;     // [ceil(in/64)] partial Σ v²
};

__host__ inline size_t part_elems(int out, int in) {
  return std::max((size_t)((in + kC - 1) / kC) * out, (size_t)((out + kR - 1) / kR) * in);
}

__host__ inline SvidWs carve_svid(void* ws, int out, int in, int P) {
  char* p = (char*)ws;
  SvidWs w;
  w.gp = (float*)p;  p += a256((size_t)P * out * 4);
  w.hp = (float*)p;  p += a256((size_t)P * in * 4);
  w.u = (float*)p;   p += a256((size_t)out * 4);
  w.v = (float*)p;   p += a256((size_t)in * 4);
  w.part = (float*)p; p += a256(part_elems(out, in) * 4);
  w.sq_u = (double*)p; p += a256((size_t)((out + 63) / 64) * 8);
  w.sq_v = (double*)p;
  return w;
}

__host__ inline size_t svid_ws_bytes(int out, int in, int P) {
  return a256((size_t)P * out * 4) + a256((size_t)P * in * 4) + a256((size_t)out * 4) +
         a256((size_t)in * 4) + a256(part_elems(out, in) * 4) +
         a256((size_t)((out + 63) / 64) * 8) + a256((size_t)((in + 63) / 64) * 8);
}

// One pass over a 64 x 256 tile. Thread (c4 = tid % 64, q = tid / 64) holds
// columns i0 + 4 c4 .. + 3 of rows o0 + 16 q .. + 15.
//   ROWS: part[tile column][o] = Σ_{tile columns} |R[o][i]| vec[i]
//   COLS: part[tile row][i]    = Σ_{tile rows}    |R[o][i]| vec[o]
// With bits, the sign bits of R (path i) are written into the planes.
template <bool ROWS>
__global__ __launch_bounds__(256) void k_svid_pass(const float* __restrict__ W,
                                                   const float* __restrict__ f_out,
                                                   const float* __restrict__ f_in, int out, int in,
                                                   int P, int path, uint32_t* planes, SvidWs ws,
                                                   int bits) {
  const int nct = (in + kC - 1) / kC;
  const int ct = blockIdx.x % nct, rt = blockIdx.x / nct;
  const int o0 = rt * kR, i0 = ct * kC;
  const int tid = threadIdx.x, c4 = tid & 63, q = tid >> 6;
  const int ic = i0 + 4 * c4, icc = min(ic, in - 1);
  const int KG = col_groups(in);
  const bool vec = (in & 3) == 0 && ic + 4 <= in;
  const float* vecin = ROWS ? ws.v : ws.u;

  float fin[4], vin[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int i = min(ic + c, in - 1);
    fin[c] = f_in ? f_in[i] : 1.0f;
    vin[c] = ROWS ? vecin[i] : 0.f;
  }
  // other paths' column scales
  float hj[3][4];
#pragma unroll
  for (int j = 0; j < 3; ++j)
#pragma unroll
    for (int c = 0; c < 4; ++c) hj[j][c] = (j < P && j != path) ? ws.hp[(size_t)j * in + min(ic + c, in - 1)] : 0.f;

  float colacc[4] = {0.f, 0.f, 0.f, 0.f};
  float rv[16];                    // ROWS: this thread's share of each row
  __shared__ float s_row[kR];      // ROWS: per row of the tile
  __shared__ float s_col[4][kC];   // COLS: per wave, per column

  for (int rr = 0; rr < 16; ++rr) {
    const int o = o0 + 16 * q + rr;
    const bool orow = o < out;
    const int oc = min(o, out - 1);
    float w[4];
    if (vec) {
      const float4 t = *(const float4*)(W + (size_t)oc * in + ic);
      w[0] = t.x; w[1] = t.y; w[2] = t.z; w[3] = t.w;
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) w[c] = ic + c < in ? W[(size_t)oc * in + min(ic + c, in - 1)] : 0.f;
    }
    const float fo = f_out ? f_out[oc] : 1.0f;
    float r[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) r[c] = (w[c] * fo) * fin[c];
    // subtract the other paths in path order
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      if (j >= P || j == path) continue;
      const float gj = ws.gp[(size_t)j * out + oc];
      // (columns past in: the word of the last column, unused since |R| is masked)
      const uint32_t word = planes[4 * unit_index(oc >> 6, icc >> 7, j, oc & 63, KG, P) + ((icc >> 5) & 3)];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float e = gj * hj[j][c];
        const bool neg = (word >> ((ic + c) & 31)) & 1u;
        r[c] = neg ? r[c] + e : r[c] - e;
      }
    }
    uint32_t nib = 0;
    float a[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const bool ok = orow && ic + c < in;
      a[c] = ok ? fabsf(r[c]) : 0.f;
      nib |= (ok && r[c] < 0.f) ? (1u << c) : 0u;
    }
    if (ROWS) {
      rv[rr] = ((a[0] * vin[0] + a[1] * vin[1]) + a[2] * vin[2]) + a[3] * vin[3];
    } else {
      const float uo = orow ? vecin[o] : 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c) colacc[c] += a[c] * uo;
    }
    if (bits) {
      // 8 lanes x 4 bits -> one 32-column word in lane 8w (columns 32 w ..)
      uint32_t x = nib | (__shfl_down(nib, 1, 64) << 4);
      x |= __shfl_down(x, 2, 64) << 8;
      x |= __shfl_down(x, 4, 64) << 16;
      const int col = i0 + 32 * (c4 >> 3);
      if ((c4 & 7) == 0 && (o >> 6) < row_groups(out) && (col >> 7) < KG)
        planes[4 * unit_index(o >> 6, col >> 7, path, o & 63, KG, P) + ((col >> 5) & 3)] = x;
    }
  }
  if (ROWS) {
    // sum each of the 16 rows over the 64 lanes: a butterfly that halves the
    // number of rows a lane holds at each of the xor 32, 16, 8, 4 steps, then
    // xor 2 and 1; lane l ends with row 8 b5 + 4 b4 + 2 b3 + b2 (bits of l)
    const int l = c4;
    float t8[8], t4[4], t2[2];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const bool hi = l & 32;
      t8[k] = (hi ? rv[8 + k] : rv[k]) + __shfl_xor(hi ? rv[k] : rv[8 + k], 32, 64);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const bool hi = l & 16;
      t4[k] = (hi ? t8[4 + k] : t8[k]) + __shfl_xor(hi ? t8[k] : t8[4 + k], 16, 64);
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const bool hi = l & 8;
      t2[k] = (hi ? t4[2 + k] : t4[k]) + __shfl_xor(hi ? t4[k] : t4[2 + k], 8, 64);
    }
    const bool hi = l & 4;
    float t1 = (hi ? t2[1] : t2[0]) + __shfl_xor(hi ? t2[0] : t2[1], 4, 64);
    t1 += __shfl_xor(t1, 2, 64);
    t1 += __shfl_xor(t1, 1, 64);
    const int row = 8 * ((l >> 5) & 1) + 4 * ((l >> 4) & 1) + 2 * ((l >> 3) & 1) + ((l >> 2) & 1);
    if ((l & 3) == 0) s_row[16 * q + row] = t1;
    __syncthreads();
    if (tid < kR) {
      const int o = o0 + tid;
      if (o < out) ws.part[(size_t)ct * out + o] = s_row[tid];
    }
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) s_col[q][4 * c4 + c] = colacc[c];
    __syncthreads();
    const int i = i0 + tid;
    if (i < in) ws.part[(size_t)rt * in + i] = ((s_col[0][tid] + s_col[1][tid]) + s_col[2][tid]) + s_col[3][tid];
  }
}

// vec[e] = Σ_t part[t][e] in float64: slice k (of 4) adds the partials
// t ≡ k (mod 4) in ascending t, eight loads in flight, and the four slice sums
// are added in slice order; Σ vec² per workgroup of 64 elements
__global__ __launch_bounds__(256) void k_svid_reduce(const float* __restrict__ part, int nt, int n,
                                                     float* vec, double* sq) {
  const int k = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int e = blockIdx.x * 64 + l;
  const int ec = min(e, n - 1);
  double acc = 0.0;
  for (int t0 = k; t0 < nt; t0 += 32) {
    float x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int t = t0 + 4 * u;
      x[u] = part[(size_t)min(t, nt - 1) * n + ec];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += t0 + 4 * u < nt ? (double)x[u] : 0.0;
  }
  __shared__ double sl[4][64];
  sl[k][l] = acc;
  __syncthreads();
  if (k == 0) {
    const double v = ((sl[0][l] + sl[1][l]) + sl[2][l]) + sl[3][l];
    const float f = (float)v;
    if (e < n) vec[e] = f;
    double s2 = e < n ? (double)f * f : 0.0;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) s2 += __shfl_xor(s2, m, 64);
    if (l == 0) sq[blockIdx.x] = s2;
  }
}

// v = the path's h (warm start) or ones (cold start), and Σ v² per 64 elements
__global__ __launch_bounds__(64) void k_svid_start(SvidWs ws, int in, int path, int cold) {
  const int e = blockIdx.x * 64 + threadIdx.x;
  float x = 0.f;
  if (e < in) {
    x = cold ? 1.0f : ws.hp[(size_t)path * in + e];
    ws.v[e] = x;
  }
  double s = (double)x * x;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor(s, m, 64);
  if (threadIdx.x == 0) ws.sq_v[blockIdx.x] = s;
}

// g_path = u / (sqrt(σ) ||v||), h_path = sqrt(σ) v / ||v||, σ = ||u|| / ||v||
__global__ __launch_bounds__(kRedWg) void k_svid_extract(SvidWs ws, int out, int in, int path) {
  // ||u||², ||v||²: thread t adds entries t, t + 256, ... of the per-64
  // partial arrays, then a fixed tree over the workgroup (the same bits in
  // every workgroup)
  const int nsu = (out + 63) / 64, nsv = (in + 63) / 64;
  double a = 0.0, b = 0.0;
  for (int k = threadIdx.x; k < nsu; k += kRedWg) a += ws.sq_u[k];
  for (int k = threadIdx.x; k < nsv; k += kRedWg) b += ws.sq_v[k];
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    a += __shfl_xor(a, m, 64);
    b += __shfl_xor(b, m, 64);
  }
  __shared__ double s_a[kRedWg / 64], s_b[kRedWg / 64];
  if ((threadIdx.x & 63) == 0) {
    s_a[threadIdx.x >> 6] = a;
    s_b[threadIdx.x >> 6] = b;
  }
  __syncthreads();
  const double nu = sqrt(((s_a[0] + s_a[1]) + s_a[2]) + s_a[3]);
  const double nv = sqrt(((s_b[0] + s_b[1]) + s_b[2]) + s_b[3]);
  const bool ok = nu > 0.0 && nv > 0.0;
  const double sig = ok ? nu / nv : 0.0, rs = sqrt(sig);
  const int e = blockIdx.x * kRedWg + threadIdx.x;
  if (e < out) ws.gp[(size_t)path * out + e] = ok ? (float)((double)ws.u[e] / (rs * nv)) : 0.f;
  if (e < in) ws.hp[(size_t)path * in + e] = ok ? (float)((double)ws.v[e] * rs / nv) : 0.f;
}

// state in the preconditioned domain: from the caller's scales (continue) or zero
__global__ __launch_bounds__(256) void k_svid_setup(SvidWs ws, const float* g, const float* h,
                                                    const float* f_out, const float* f_in, int out,
                                                    int in, int P, int cont) {
  const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t ng = (size_t)P * out;
  if (e < ng) {
    const int o = (int)(e % out);
    ws.gp[e] = cont ? g[e] * (f_out ? f_out[o] : 1.0f) : 0.f;
  } else if (e < ng + (size_t)P * in) {
    const size_t k = e - ng;
    const int i = (int)(k % in);
    ws.hp[k] = cont ? h[k] * (f_in ? f_in[i] : 1.0f) : 0.f;
  }
}

__global__ __launch_bounds__(256) void k_fill_zero_u32(uint32_t* p, size_t n) {
  const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (e < n) p[e] = 0u;
}

// g = g' / f_out, h = h' / f_in
__global__ __launch_bounds__(256) void k_svid_finish(SvidWs ws, float* g, float* h,
                                                     const float* f_out, const float* f_in, int out,
                                                     int in, int P) {
  const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t ng = (size_t)P * out;
  if (e < ng) {
    const int o = (int)(e % out);
    g[e] = f_out ? ws.gp[e] / f_out[o] : ws.gp[e];
  } else if (e < ng + (size_t)P * in) {
    const size_t k = e - ng;
    const int i = (int)(k % in);
    h[k] = f_in ? ws.hp[k] / f_in[i] : ws.hp[k];
  }
}

}  // namespace

size_t svid_workspace_bytes(int out, int in) {
  return std::max(svid_ws_bytes(out, in, 2), svid_ws_bytes(out, in, 3));
}

hipError_t launch_svid(const float* W, int out, int in, int P, int sweeps, int passes,
                       const float* f_out, const float* f_in, bool cont, float* g, float* h,
                       uint4* planes, void* ws, hipStream_t st) {
  SvidWs w = carve_svid(ws, out, in, P);
  const size_t nsc = (size_t)P * (out + in);
  hipLaunchKernelGGL(k_svid_setup, dim3((unsigned)((nsc + 255) / 256)), dim3(256), 0, st, w, g, h,
                     f_out, f_in, out, in, P, cont ? 1 : 0);
  if (!cont) {
    const size_t nw = (size_t)row_groups(out) * col_groups(in) * P * 64 * 4;
    hipLaunchKernelGGL(k_fill_zero_u32, dim3((unsigned)((nw + 255) / 256)), dim3(256), 0, st,
                       (uint32_t*)planes, nw);
  }
  const int nct = (in + kC - 1) / kC, nrt = (out + kR - 1) / kR;
  const dim3 tiles(nct * nrt), blk(256);
  const dim3 gu((out + 63) / 64), gv((in + 63) / 64);
  const dim3 ge((std::max(out, in) + kRedWg - 1) / kRedWg);
  for (int t = 0; t < sweeps; ++t) {
    for (int i = 0; i < P; ++i) {
      hipLaunchKernelGGL(k_svid_start, gv, dim3(64), 0, st, w, in, i, (!cont && t == 0) ? 1 : 0);
      for (int k = 0; k < passes; ++k) {
        if ((k & 1) == 0) {  // rows pass: u = |R| v (the first also writes the bits of B_i)
          hipLaunchKernelGGL(k_svid_pass<true>, tiles, blk, 0, st, W, f_out, f_in, out, in, P, i,
                             (uint32_t*)planes, w, k == 0 ? 1 : 0);
          hipLaunchKernelGGL(k_svid_reduce, gu, dim3(256), 0, st, w.part, nct, out, w.u, w.sq_u);
        } else {             // columns pass: v = |R|ᵀ u
          hipLaunchKernelGGL(k_svid_pass<false>, tiles, blk, 0, st, W, f_out, f_in, out, in, P, i,
                             (uint32_t*)planes, w, 0);
          hipLaunchKernelGGL(k_svid_reduce, gv, dim3(256), 0, st, w.part, nrt, in, w.v, w.sq_v);
        }
      }
      hipLaunchKernelGGL(k_svid_extract, ge, dim3(kRedWg), 0, st, w, out, in, i);
    }
  }
  hipLaunchKernelGGL(k_svid_finish, dim3((unsigned)((nsc + 255) / 256)), dim3(256), 0, st, w, g, h,
                     f_out, f_in, out, in, P);
  return hipGetLastError();
}

}  // namespace rabit
