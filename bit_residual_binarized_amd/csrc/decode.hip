// Plain bf16 stand-ins around the binary linear layers of a decode step
// (RMSNorm with unit weight, attention over a one-token context, SiLU * up,
// residual add). The pages time Llama2 decoding (RaBiT paper Table 7, App.
// E.2) without defining these ops; they are not part of the timed linear
// layers. Each rounds its result once to bfloat16 from float64.
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

}  // namespace

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
