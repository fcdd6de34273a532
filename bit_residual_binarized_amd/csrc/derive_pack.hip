// Derive and pack both binary paths of a layer from one shared fp32 weight.
//
// RaBiT paper §4.2 ("The Coupled Forward Pass"): B_1 = sign(W);
// R_1 = W − g_1 ⊙ B_1 ⊙ h_1; B_2 = sign(R_1). Paper App. E.1 ("Weight
// Packing"): 32 columns per uint32, +1 -> 0, -1 -> 1.
//
// Passes (each reads W once, HBM-bound at 4 B per weight):
//   S1  |W| partial sums per (column tile, row) and (row tile, column)
//   F   finalize: ordered sums of the partials, IEEE f64 divide, f64->fp16 RNE
//   D   B_1, R_1 (fp32, one rounding), B_2, |R_1| partial sums, packed planes
//   F   finalize g_2, h_2
// The partial-sum structure is the canonical scale-sum order of rabit.h, so
// the fp16 scales and hence B_2 are bit-exact and independent of the launch.
#include "rabit_internal.h"

namespace rabit {

namespace {

constexpr int kTileRows = 64;   // rows per tile (4 waves x 16-row segments)
constexpr int kTileCols = 256;  // columns per tile (lane l: l + 64c, c = 0..3)

// One workgroup = one 64 x 256 tile, 4 waves; wave w owns rows 16w..16w+15.
template <bool PASS_D, bool SUMS>
__global__ __launch_bounds__(256) void k_derive_tile(
    const float* __restrict__ W, int out, int in,
    const uint16_t* __restrict__ g1h, const uint16_t* __restrict__ h1h,
    double* __restrict__ rowpart, double* __restrict__ colpart,
    uint4* __restrict__ planes, int KG) {
  const int ct = blockIdx.x, rt = blockIdx.y;
  const int wv = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int col0 = ct * kTileCols;

  __shared__ double scol[4][kTileCols];
  __shared__ uint32_t swords[2][2][64][4];  // [kg local][path][row][word]

  int cols[4];
  bool cval[4];
  float h1f[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    cols[c] = col0 + l + 64 * c;
    cval[c] = cols[c] < in;
    h1f[c] = (PASS_D && cval[c]) ? f16_bits_to_f32(h1h[cols[c]]) : 0.0f;
  }
  double cp[4] = {0.0, 0.0, 0.0, 0.0};

#pragma unroll 4
  for (int rr = 0; rr < 16; ++rr) {
    const int rloc = wv * 16 + rr;
    const int row = rt * kTileRows + rloc;
    const bool rv = row < out;
    const float* wrow = W + (size_t)(rv ? row : 0) * in;
    const float g1f = (PASS_D && rv) ? f16_bits_to_f32(g1h[row]) : 0.0f;
    float a[4];
    bool b1[4], b2[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float v = (rv && cval[c]) ? __builtin_nontemporal_load(wrow + cols[c]) : 0.0f;
      if (PASS_D) {
        const float e = g1f * h1f[c];           // exact: fp16 x fp16 fits fp32
        b1[c] = v < 0.0f;
        const float r = v - (b1[c] ? -e : e);   // one rounding
        b2[c] = r < 0.0f;
        a[c] = fabsf(r);
      } else {
        a[c] = fabsf(v);
      }
    }
    if (SUMS) {
      double lv = (double)a[0];
      lv += (double)a[1];
      lv += (double)a[2];
      lv += (double)a[3];
      // halving tree: lane l and lane l^s form the same sum, so lane 0 ends
      // with v[0] of the tree v[l] += v[l+s], s = 32..1
#pragma unroll
      for (int s = 32; s >= 1; s >>= 1) lv += __shfl_xor(lv, s, 64);
      if (l == 0 && rv) rowpart[(size_t)ct * out + row] = lv;
#pragma unroll
      for (int c = 0; c < 4; ++c) cp[c] += (double)a[c];
    }
    if (PASS_D) {
      // ballot(c) bit l <-> column col0 + 64c + l: low half = word 2c,
      // high half = word 2c + 1 of the tile (8 words = 2 column groups)
      uint32_t myword = 0;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint64_t m1 = __ballot(b1[c]);
        const uint64_t m2 = __ballot(b2[c]);
        if (l == 2 * c) myword = (uint32_t)m1;
        if (l == 2 * c + 1) myword = (uint32_t)(m1 >> 32);
        if (l == 8 + 2 * c) myword = (uint32_t)m2;
        if (l == 8 + 2 * c + 1) myword = (uint32_t)(m2 >> 32);
      }
      if (l < 16) {
        const int p = l >> 3, k = l & 7;
        swords[k >> 2][p][rloc][k & 3] = myword;
      }
    }
  }

  if (SUMS) {
#pragma unroll
    for (int c = 0; c < 4; ++c) scol[wv][l + 64 * c] = cp[c];
  }
  __syncthreads();
  if (SUMS) {
    const int x = threadIdx.x;
    const int col = col0 + x;
    if (col < in) {
      double t = scol[0][x];
      t += scol[1][x];
      t += scol[2][x];
      t += scol[3][x];
      colpart[(size_t)rt * in + col] = t;
    }
  }
  if (PASS_D) {
    const int t = threadIdx.x;
    const int kgl = t >> 7, p = (t >> 6) & 1, r = t & 63;
    const int kg = 2 * ct + kgl;
    if (kg < KG) {
      const uint32_t* s = swords[kgl][p][r];
      planes[unit_index(rt, kg, p, r, KG)] = make_uint4(s[0], s[1], s[2], s[3]);
    }
  }
}

// Ordered reduction of the partials and rounding to fp16.
__global__ __launch_bounds__(256) void k_finalize(const double* __restrict__ rowpart,
                                                  const double* __restrict__ colpart, int out,
                                                  int in, int nct, int nrt,
                                                  uint16_t* __restrict__ g_out,
                                                  uint16_t* __restrict__ h_out) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= out + in) return;
  const bool row = t < out;
  const double* p = row ? rowpart + t : colpart + (t - out);
  const int n = row ? nct : nrt;
  const size_t stride = row ? (size_t)out : (size_t)in;
  // the tile partials are added strictly in order; the loads of 32 of them
  // are in flight at a time (clamped index, masked)
  double s = 0.0;
  for (int c0 = 0; c0 < n; c0 += 32) {
    double v[32];
#pragma unroll
    for (int u = 0; u < 32; ++u) v[u] = p[(size_t)min(c0 + u, n - 1) * stride];
#pragma unroll
    for (int u = 0; u < 32; ++u) s += c0 + u < n ? v[u] : 0.0;
  }
  if (row)
    g_out[t] = f64_to_f16_rne(s / (double)in);
  else
    h_out[t - out] = f64_to_f16_rne(s / (double)out);
}

// Device layout -> canonical words (test hook).
__global__ __launch_bounds__(256) void k_unpack(const uint4* __restrict__ planes, int out, int in,
                                                uint32_t* __restrict__ words) {
  const int KG = col_groups(in);
  const int nw = (in + 31) / 32;
  const size_t total = (size_t)2 * out * nw;
  for (size_t idx = blockIdx.x * (size_t)blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    const int k = (int)(idx % nw);
    const int row = (int)((idx / nw) % out);
    const int p = (int)(idx / ((size_t)nw * out));
    const uint4 u = planes[unit_index(row >> 6, k >> 2, p, row & 63, KG)];
    const int q = k & 3;
    words[idx] = q == 0 ? u.x : (q == 1 ? u.y : (q == 2 ? u.z : u.w));
  }
}

__global__ void k_test_f64_to_16(const double* __restrict__ in, uint16_t* __restrict__ out, int n,
                                 int bf16) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = bf16 ? f64_to_bf16_rne(in[i]) : f64_to_f16_rne(in[i]);
}

}  // namespace

size_t pack_workspace_bytes(int out, int in) {
  const size_t nct = (size_t)(in + kTileCols - 1) / kTileCols;
  const size_t nrt = (size_t)(out + kTileRows - 1) / kTileRows;
  return (nct * out + nrt * in) * sizeof(double);
}

hipError_t launch_pack(const float* W, int out, int in, bool meanabs, uint16_t* g, uint16_t* h,
                       uint4* planes, void* ws, hipStream_t st) {
  const int nct = (in + kTileCols - 1) / kTileCols;
  const int nrt = (out + kTileRows - 1) / kTileRows;
  const int KG = col_groups(in);
  double* rowpart = (double*)ws;
  double* colpart = rowpart + (size_t)nct * out;
  const dim3 grid(nct, nrt), block(256);
  const int fin_blocks = (out + in + 255) / 256;
  if (meanabs) {
    hipLaunchKernelGGL((k_derive_tile<false, true>), grid, block, 0, st, W, out, in, nullptr,
                       nullptr, rowpart, colpart, nullptr, KG);
    hipLaunchKernelGGL(k_finalize, dim3(fin_blocks), block, 0, st, rowpart, colpart, out, in, nct,
                       nrt, g, h);
    hipLaunchKernelGGL((k_derive_tile<true, true>), grid, block, 0, st, W, out, in, g, h, rowpart,
                       colpart, planes, KG);
    hipLaunchKernelGGL(k_finalize, dim3(fin_blocks), block, 0, st, rowpart, colpart, out, in, nct,
                       nrt, g + out, h + in);
  } else {
    hipLaunchKernelGGL((k_derive_tile<true, false>), grid, block, 0, st, W, out, in, g, h,
                       nullptr, nullptr, planes, KG);
  }
  return hipGetLastError();
}

hipError_t launch_unpack(const uint4* planes, int out, int in, uint32_t* words, hipStream_t st) {
  const size_t total = (size_t)2 * out * ((in + 31) / 32);
  const int blocks = (int)std::min<size_t>((total + 255) / 256, 65535);
  hipLaunchKernelGGL(k_unpack, dim3(blocks), dim3(256), 0, st, planes, out, in, words);
  return hipGetLastError();
}

hipError_t launch_test_f64_to_16(const double* in, uint16_t* out, int n, int bf16,
                                 hipStream_t st) {
  hipLaunchKernelGGL(k_test_f64_to_16, dim3((n + 255) / 256), dim3(256), 0, st, in, out, n, bf16);
  return hipGetLastError();
}

}  // namespace rabit
