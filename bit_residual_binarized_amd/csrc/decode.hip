// Plain bf16 stand-ins around the binary linear layers of a decode step
// (RMSNorm with unit weight, attention over a one-token context, SiLU * up,
// residual add). The pages time Llama2 decoding (RaBiT paper Table 7, App.
// E.2) without defining these ops; they are not part of the timed linear
// layers. Each rounds its result once to bfloat16 from float64.
#include <algorithm>

#include "rabit_internal.h"

namespace rabit {

namespace {

__global__ __launch_bounds__(1024) void k_rmsnorm(const uint16_t* __restrict__ x,
                                                  uint16_t* __restrict__ y, int n, float eps) {
  const int b = blockIdx.x;
  const uint16_t* xb = x + (size_t)b * n;
  double ss = 0.0;
  for (int j = threadIdx.x; j < n; j += blockDim.x) {
    const double v = (double)bf16_bits_to_f32(xb[j]);
    ss += v * v;
  }
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) ss += __shfl_xor(ss, s, 64);
  __shared__ double part[16];
  __shared__ double s_inv;
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
    for (int i = 0; i < (int)(blockDim.x >> 6); ++i) t += part[i];
    s_inv = 1.0 / sqrt(t / (double)n + (double)eps);
  }
  __syncthreads();
  const double inv = s_inv;
  for (int j = threadIdx.x; j < n; j += blockDim.x)
    y[(size_t)b * n + j] = f64_to_bf16_rne((double)bf16_bits_to_f32(xb[j]) * inv);
}

// v: float32 [batch][kv_rows]; head h reads the value vector of group h / rep
__global__ void k_attn_1tok(const float* __restrict__ v, int kv_rows, uint16_t* __restrict__ a,
                            int n_heads, int rep, int head_dim) {
  const int b = blockIdx.y;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  const int n = n_heads * head_dim;
  if (i >= n) return;
  const int h = i / head_dim, d = i - h * head_dim;
  const float* vb = v + (size_t)b * kv_rows;
  a[(size_t)b * n + i] = f64_to_bf16_rne((double)vb[(h / rep) * head_dim + d]);
}

__global__ void k_silu_mul(const float* __restrict__ gate, const float* __restrict__ up,
                           uint16_t* __restrict__ z, size_t total) {
  const size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  if (i >= total) return;
  const double g = (double)gate[i];
  z[i] = f64_to_bf16_rne(g / (1.0 + exp(-g)) * (double)up[i]);
}

__global__ void k_residual_add(const uint16_t* __restrict__ x, const float* __restrict__ d,
                               uint16_t* __restrict__ out, size_t total) {
  const size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  if (i >= total) return;
  out[i] = f64_to_bf16_rne((double)bf16_bits_to_f32(x[i]) + (double)d[i]);
}

// ---- consumers of GEMV partials (fused with the ops that follow a layer) ----
// part: the producing GEMV launch's partial buffer of the matrix (a header
// with the slice count S, then float32 [batch][S][stride], stride =
// 64 ceil(n/64); slices are 512-column ranges or chunks of them);
// sum_ranges adds the slices in ascending order, as rabit_gemv_reduce does.
// Block (i, b) covers elements [i span, (i + 1) span) of row b: x_out =
// bf16(x + Σ part) (or x itself without part) and the sum of x_out^2 over
// the block, combined in a fixed order, into stats[b][i]. Beyond 8 slices
// (the 16 and 56 ranges of a batch-1 layer) the loads of 32 slices are in
// flight together: 0.5-1 us per layer less at batch 1 than 8 at a time
// (64 at a time was slower).
__global__ __launch_bounds__(256) void k_resid_stats(const double* __restrict__ part,
                                                     const uint16_t* x, uint16_t* x_out,
                                                     double* __restrict__ stats, int n) {
  const int i = blockIdx.x, b = blockIdx.y;
  const int span = (n + RABIT_STAT_PARTS - 1) / RABIT_STAT_PARTS;
  const int e0 = min(n, i * span), e1 = min(n, e0 + span);
  const int stride = 64 * ((n + 63) / 64);
  double ss = 0.0;
  for (int e = e0 + (int)threadIdx.x; e < e1; e += 256) {
    double v = (double)bf16_bits_to_f32(x[(size_t)b * n + e]);
    if (part) {
      const int S = part_slices(part);
      const float* pp = part_data(part) + (size_t)b * S * stride + e;
      const uint16_t o = f64_to_bf16_rne(v + (S <= 8 ? sum_ranges_by<8>(pp, S, stride) : sum_ranges_by<32>(pp, S, stride)));
      x_out[(size_t)b * n + e] = o;
      v = (double)bf16_bits_to_f32(o);
    }
    ss += v * v;
  }
  ss = wave_sum_f64(ss);
  __shared__ double s_w[4];
  if ((threadIdx.x & 63) == 0) s_w[threadIdx.x >> 6] = ss;
  __syncthreads();
  if (threadIdx.x == 0) stats[(size_t)b * RABIT_STAT_PARTS + i] = ((s_w[0] + s_w[1]) + s_w[2]) + s_w[3];
}

__global__ __launch_bounds__(256) void k_reduce_silu(const double* __restrict__ pg,
                                                     const double* __restrict__ pu,
                                                     uint16_t* __restrict__ a, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x, b = blockIdx.y;
  if (i >= n) return;
  const int stride = 64 * ((n + 63) / 64);
  const double g = sum_ranges(pg, b, stride, i), u = sum_ranges(pu, b, stride, i);
  a[(size_t)b * n + i] = f64_to_bf16_rne(g / (1.0 + exp(-g)) * u);
}

// qk: [batch][n_q + kv] fp32 (q then k); attn: [batch][n_q] bf16
__global__ __launch_bounds__(256) void k_reduce_attn(const double* __restrict__ pq,
                                                     const double* __restrict__ pk,
                                                     const double* __restrict__ pv,
                                                     float* __restrict__ qk,
                                                     uint16_t* __restrict__ attn, int n_q, int kv,
                                                     int rep, int head_dim) {
  const int i = blockIdx.x * 256 + threadIdx.x, b = blockIdx.y;
  const int sq = 64 * ((n_q + 63) / 64), skv = 64 * ((kv + 63) / 64);
  if (i < n_q) {
    qk[(size_t)b * (n_q + kv) + i] = (float)sum_ranges(pq, b, sq, i);
    const int h = i / head_dim, d = i - h * head_dim;
    attn[(size_t)b * n_q + i] = f64_to_bf16_rne(sum_ranges(pv, b, skv, (h / rep) * head_dim + d));
  }
  if (i < kv) qk[(size_t)b * (n_q + kv) + n_q + i] = (float)sum_ranges(pk, b, skv, i);
}

}  // namespace

hipError_t launch_resid_stats(const double* part, const uint16_t* x, uint16_t* x_out,
                              double* stats, int batch, int n, hipStream_t st) {
  hipLaunchKernelGGL(k_resid_stats, dim3(RABIT_STAT_PARTS, batch), dim3(256), 0, st, part, x,
                     x_out, stats, n);
  return hipGetLastError();
}

hipError_t launch_reduce_silu(const double* pg, const double* pu, uint16_t* a,
                              int batch, int n, hipStream_t st) {
  hipLaunchKernelGGL(k_reduce_silu, dim3((n + 255) / 256, batch), dim3(256), 0, st, pg, pu, a, n);
  return hipGetLastError();
}

hipError_t launch_reduce_attn(const double* pq, const double* pk, const double* pv,
                              float* qk, uint16_t* attn, int batch, int n_heads,
                              int n_kv_heads, int head_dim, hipStream_t st) {
  const int n_q = n_heads * head_dim, kv = n_kv_heads * head_dim;
  hipLaunchKernelGGL(k_reduce_attn, dim3((std::max(n_q, kv) + 255) / 256, batch), dim3(256), 0, st,
                     pq, pk, pv, qk, attn, n_q, kv, n_heads / n_kv_heads,
                     head_dim);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(const uint16_t* x, uint16_t* y, int batch, int n, float eps,
                          hipStream_t st) {
  hipLaunchKernelGGL(k_rmsnorm, dim3(batch), dim3(1024), 0, st, x, y, n, eps);
  return hipGetLastError();
}

hipError_t launch_attn_1tok(const float* v, int kv_rows, uint16_t* a, int batch, int n_heads,
                            int n_kv_heads, int head_dim, hipStream_t st) {
  const int n = n_heads * head_dim;
  hipLaunchKernelGGL(k_attn_1tok, dim3((n + 255) / 256, batch), dim3(256), 0, st, v, kv_rows, a,
                     n_heads, n_heads / n_kv_heads, head_dim);
  return hipGetLastError();
}

hipError_t launch_silu_mul(const float* gate, const float* up, uint16_t* z, int batch, int n,
                           hipStream_t st) {
  const size_t total = (size_t)batch * n;
  hipLaunchKernelGGL(k_silu_mul, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, gate, up,
                     z, total);
  return hipGetLastError();
}

hipError_t launch_residual_add(const uint16_t* x, const float* d, uint16_t* out, int batch, int n,
                               hipStream_t st) {
  const size_t total = (size_t)batch * n;
  hipLaunchKernelGGL(k_residual_add, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, x, d,
                     out, total);
  return hipGetLastError();
}

}  // namespace rabit
