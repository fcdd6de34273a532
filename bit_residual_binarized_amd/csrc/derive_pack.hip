// Derive and pack the binary paths of a layer from one shared fp32 weight.
//
// RaBiT paper §4.2 ("The Coupled Forward Pass"): B_1 = sign(W);
// R_1 = W − g_1 ⊙ B_1 ⊙ h_1; B_2 = sign(R_1). For the 3-bit variant (three
// paths) the same step once more, each path correcting the residual of its
// predecessor (paper §1): R_2 = R_1 − g_2 ⊙ B_2 ⊙ h_2, B_3 = sign(R_2).
// Paper App. E.1 ("Weight Packing"): 32 columns per uint32, +1 -> 0, -1 -> 1.
//
// Passes (each reads W once, HBM-bound at 4 B per weight):
//   S1  |W| partial sums per (column tile, row) and (row tile, column)
//   F   finalize: ordered sums of the partials, IEEE f64 divide, f64->fp16 RNE
//   D   B_1, R_1 (fp32, one rounding), B_2, |R_1| partial sums, packed planes
//   F   finalize g_2, h_2
//   and with three paths:
//   E   R_1 again, R_2 (fp32, one rounding), B_3, |R_2| partial sums, plane 3
//   F   finalize g_3, h_3
// With given scales one pass (D) writes every plane.
// The partial-sum structure is the canonical scale-sum order of rabit.h, so
// the fp16 scales and hence B_2 are bit-exact and independent of the launch.
#include "rabit_internal.h"

namespace rabit {

namespace {

constexpr int kTileRows = 64;   // rows per tile (4 waves x 16-row segments)
constexpr int kTileCols = 256;  // columns per tile (lane l: l + 64c, c = 0..3)

// One workgroup = one 64 x 256 tile, 4 waves; wave w owns rows 16w..16w+15.
// STAGE 0: |W| sums. STAGE 1: B_1, B_2 (and B_3 with three paths and given
// scales), |R_1| sums. STAGE 2 (three paths): B_3, |R_2| sums. P: paths of the
// layer (the plane stride of the device layout). g, h: the scales of every
// path ([P][out], [P][in]), as far as they are known at this stage.
template <int STAGE, bool SUMS, int P>
__global__ __launch_bounds__(256) void k_derive_tile(
    const float* __restrict__ W, int out, int in,
    const uint16_t* __restrict__ gh, const uint16_t* __restrict__ hh,
    double* __restrict__ rowpart, double* __restrict__ colpart,
    uint4* __restrict__ planes, int KG) {
  // paths written by this stage: [pb, pb + NP)
  constexpr bool kB3 = P == 3 && (STAGE == 2 || (STAGE == 1 && !SUMS));
  constexpr int pb = STAGE == 2 ? 2 : 0;
  constexpr int NP = STAGE == 0 ? 0 : STAGE == 2 ? 1 : (kB3 ? 3 : 2);
  const int ct = blockIdx.x, rt = blockIdx.y;
  const int wv = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int col0 = ct * kTileCols;

  __shared__ double scol[4][kTileCols];
  __shared__ uint32_t swords[2][NP > 0 ? NP : 1][64][4];  // [kg local][path - pb][row][word]

  // Every load below is issued unconditionally from a clamped index and
  // masked afterwards: a load under a condition becomes a branch that waits
  // for it, which left one row of loads in flight per wave.
  int cols[4], cc[4];
  bool cval[4];
  uint16_t hr1[4], hr2[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    cols[c] = col0 + l + 64 * c;
    cval[c] = cols[c] < in;
    cc[c] = min(cols[c], in - 1);
    hr1[c] = STAGE > 0 ? hh[cc[c]] : (uint16_t)0;
    hr2[c] = kB3 ? hh[in + cc[c]] : (uint16_t)0;
  }
  // g of the wave's 16 rows: lane rr < 16 holds row 16 wv + rr (read per row
  // with readlane)
  const int grow = min(rt * kTileRows + wv * 16 + (l & 15), out - 1);
  const uint32_t gr1 = STAGE > 0 ? gh[grow] : 0u;
  const uint32_t gr2 = kB3 ? gh[out + grow] : 0u;
  float h1f[4], h2f[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    h1f[c] = (STAGE > 0 && cval[c]) ? f16_bits_to_f32(hr1[c]) : 0.0f;
    h2f[c] = (kB3 && cval[c]) ? f16_bits_to_f32(hr2[c]) : 0.0f;
  }
  double cp[4] = {0.0, 0.0, 0.0, 0.0};

  // rows in batches of kBatch: the batch's loads are all issued before its
  // rows are processed (the per-row word writes are branches that the
  // compiler does not move loads across)
  constexpr int kBatch = 4;
#pragma unroll 1  // one batch of loads in registers at a time
  for (int rb = 0; rb < 16; rb += kBatch) {
  float wb[kBatch][4];
  double lvb[kBatch];  // this lane's share (4 columns) of the batch's row sums
#pragma unroll
  for (int k = 0; k < kBatch; ++k) {
    const int row = min(rt * kTileRows + wv * 16 + rb + k, out - 1);
#pragma unroll
    for (int c = 0; c < 4; ++c) wb[k][c] = __builtin_nontemporal_load(W + (size_t)row * in + cc[c]);
  }
#pragma unroll
  for (int k = 0; k < kBatch; ++k) {
    const int rr = rb + k;
    const int rloc = wv * 16 + rr;
    const int row = rt * kTileRows + rloc;
    const bool rv = row < out;
    const float g1f = (STAGE > 0 && rv) ? f16_bits_to_f32((uint16_t)__builtin_amdgcn_readlane(gr1, rr)) : 0.0f;
    const float g2f = (kB3 && rv) ? f16_bits_to_f32((uint16_t)__builtin_amdgcn_readlane(gr2, rr)) : 0.0f;
    const float* wv4 = wb[k];
    float a[4];
    bool b1[4], b2[4], b3[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float v = (rv && cval[c]) ? wv4[c] : 0.0f;
      b3[c] = false;
      if (STAGE > 0) {
        const float e = g1f * h1f[c];           // exact: fp16 x fp16 fits fp32
        b1[c] = v < 0.0f;
        const float r = v - (b1[c] ? -e : e);   // one rounding
        b2[c] = r < 0.0f;
        a[c] = fabsf(r);
        if (kB3) {
          const float e2 = g2f * h2f[c];
          const float r2 = r - (b2[c] ? -e2 : e2);  // one rounding
          b3[c] = r2 < 0.0f;
          if (STAGE == 2) a[c] = fabsf(r2);
        }
      } else {
        a[c] = fabsf(v);
      }
    }
    if (SUMS) {
      double lv = (double)a[0];
      lv += (double)a[1];
      lv += (double)a[2];
      lv += (double)a[3];
      lvb[k] = lv;
#pragma unroll
      for (int c = 0; c < 4; ++c) cp[c] += (double)a[c];
    }
    if (NP > 0) {
      // ballot(c) bit l <-> column col0 + 64c + l: low half = word 2c,
      // high half = word 2c + 1 of the tile (8 words = 2 column groups);
      // lane 8 q + k keeps word k of written path pb + q
      uint32_t myword = 0;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
#pragma unroll
        for (int q = 0; q < NP; ++q) {
          const int path = pb + q;
          const uint64_t m = __ballot(path == 0 ? b1[c] : path == 1 ? b2[c] : b3[c]);
          if (l == 8 * q + 2 * c) myword = (uint32_t)m;
          if (l == 8 * q + 2 * c + 1) myword = (uint32_t)(m >> 32);
        }
      }
      if (l < 8 * NP) {
        const int q = l >> 3, k = l & 7;
        swords[k >> 2][q][rloc][k & 3] = myword;
      }
    }
  }
  if (SUMS) {
    // The batch's 4 row sums over the 64 lanes by the halving tree
    // v[l] += v[l + s], s = 32 .. 1, rows together: at s = 32 and 16 each lane
    // keeps half of the rows it holds and adds the partner's share of them
    // (the tree's two operands, in either order: IEEE addition commutes
    // exactly); s = 8 .. 1 finish the one row left. Lane l ends with row
    // 2 b5 + b4 of the batch (bits of l).
    static_assert(kBatch == 4, "butterfly for four rows");
    double t2[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const bool hi = l & 32;
      t2[k] = (hi ? lvb[2 + k] : lvb[k]) + __shfl_xor(hi ? lvb[k] : lvb[2 + k], 32, 64);
    }
    const bool hi = l & 16;
    double t1 = (hi ? t2[1] : t2[0]) + __shfl_xor(hi ? t2[0] : t2[1], 16, 64);
#pragma unroll
    for (int s = 8; s >= 1; s >>= 1) t1 += __shfl_xor(t1, s, 64);
    const int row = rt * kTileRows + wv * 16 + rb + 2 * ((l >> 5) & 1) + ((l >> 4) & 1);
    if ((l & 15) == 0 && row < out) rowpart[(size_t)ct * out + row] = t1;
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
  // units (kg local, written path, row): 2 * NP * 64 of them
#pragma unroll
  for (int u = threadIdx.x; u < 2 * NP * 64; u += 256) {
    constexpr int NPs = NP > 0 ? NP : 1;  // (no units when a stage writes no path)
    const int kgl = u / (NPs * 64), q = (u / 64) % NPs, r = u & 63;
    const int kg = 2 * ct + kgl;
    if (kg < KG) {
      const uint32_t* s = swords[kgl][q][r];
      planes[unit_index(rt, kg, pb + q, r, KG, P)] = make_uint4(s[0], s[1], s[2], s[3]);
    }
  }
}

// Ordered reduction of the partials and rounding to fp16.
// One wave per workgroup: the column sums read 8 B x (rows / 64) per thread,
// and small workgroups spread those reads over many CUs.
// With tot != nullptr (normalized scales) the totals are also written to
// tot[0 .. out + in) and h is left to k_norm_h.
__global__ __launch_bounds__(64) void k_finalize(const double* __restrict__ rowpart,
                                                  const double* __restrict__ colpart, int out,
                                                  int in, int nct, int nrt,
                                                  uint16_t* __restrict__ g_out,
                                                  uint16_t* __restrict__ h_out,
                                                  double* __restrict__ tot) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= out + in) return;
  const bool row = t < out;
  const double* p = row ? rowpart + t : colpart + (t - out);
  const int n = row ? nct : nrt;
  const size_t stride = row ? (size_t)out : (size_t)in;
  // the tile partials are added strictly in order; the loads of 96 of them
  // are in flight at a time (clamped index, masked): a 64-row tiling of an
  // 11008-row layer has 172 column partials, two round trips
  constexpr int kFly = 96;
  double s = 0.0;
  for (int c0 = 0; c0 < n; c0 += kFly) {
    double v[kFly];
#pragma unroll
    for (int u = 0; u < kFly; ++u) v[u] = p[(size_t)min(c0 + u, n - 1) * stride];
#pragma unroll
    for (int u = 0; u < kFly; ++u) s += c0 + u < n ? v[u] : 0.0;
  }
  if (row)
    g_out[t] = f64_to_f16_rne(s / (double)in);
  else if (!tot)
    h_out[t - out] = f64_to_f16_rne(s / (double)out);
  if (tot) tot[t] = s;  // normalized scales: row then column totals for k_norm_h
}

// Normalized scales: h[j] = fp16((S_col[j] / out) / mu) with mu = T / (out in)
// and T the canonical total of the row sums: lane l of one wave sums rows l,
// l + 64, ... in ascending order, then the halving tree v[l] += v[l + s],
// s = 32 .. 1 (a xor butterfly leaves the tree's value in lane 0). Every
// workgroup computes T the same way and then its 1024 columns.
__global__ __launch_bounds__(256) void k_norm_h(const double* __restrict__ tot, int out, int in,
                                                uint16_t* __restrict__ h_out) {
  __shared__ double s_mu;
  if (threadIdx.x < 64) {
    const int l = threadIdx.x;
    double v = 0.0;
    constexpr int kFly = 8;
    for (int r0 = l; r0 < out; r0 += 64 * kFly) {
      double t[kFly];
#pragma unroll
      for (int u = 0; u < kFly; ++u) t[u] = tot[min(r0 + 64 * u, out - 1)];
#pragma unroll
      for (int u = 0; u < kFly; ++u) v += r0 + 64 * u < out ? t[u] : 0.0;
    }
#pragma unroll
    for (int sh = 32; sh >= 1; sh >>= 1) v += __shfl_xor(v, sh, 64);
    if (l == 0) s_mu = v / ((double)out * (double)in);
  }
  __syncthreads();
  const double mu = s_mu;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int j = blockIdx.x * 1024 + k * 256 + threadIdx.x;
    if (j < in) h_out[j] = mu != 0.0 ? f64_to_f16_rne((tot[out + j] / (double)out) / mu) : (uint16_t)0;
  }
}

// Device layout -> canonical words (test hook).
__global__ __launch_bounds__(256) void k_unpack(const uint4* __restrict__ planes, int out, int in,
                                                int P, uint32_t* __restrict__ words) {
  const int KG = col_groups(in);
  const int nw = (in + 31) / 32;
  const size_t total = (size_t)P * out * nw;
  for (size_t idx = blockIdx.x * (size_t)blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    const int k = (int)(idx % nw);
    const int row = (int)((idx / nw) % out);
    const int p = (int)(idx / ((size_t)nw * out));
    const uint4 u = planes[unit_index(row >> 6, k >> 2, p, row & 63, KG, P)];
    const int q = k & 3;
    words[idx] = q == 0 ? u.x : (q == 1 ? u.y : (q == 2 ? u.z : u.w));
  }
}

__global__ void k_test_f64_to_16(const double* __restrict__ in, uint16_t* __restrict__ out, int n,
                                 int bf16) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = bf16 == 2 ? f64_to_bf16_rne_fast(in[i]) : bf16 ? f64_to_bf16_rne(in[i]) : f64_to_f16_rne(in[i]);
}

}  // namespace

size_t pack_workspace_bytes(int out, int in) {
  const size_t nct = (size_t)(in + kTileCols - 1) / kTileCols;
  const size_t nrt = (size_t)(out + kTileRows - 1) / kTileRows;
  // tile partials, then the row and column totals (normalized scales)
  return (nct * out + nrt * in + (size_t)out + in) * sizeof(double);
}

hipError_t launch_pack(const float* W, int out, int in, int P, bool meanabs, uint16_t* g,
                       uint16_t* h, uint4* planes, void* ws, hipStream_t st, bool normalized) {
  if (P != 2 && P != 3) return hipErrorInvalidValue;
  const int nct = (in + kTileCols - 1) / kTileCols;
  const int nrt = (out + kTileRows - 1) / kTileRows;
  const int KG = col_groups(in);
  double* rowpart = (double*)ws;
  double* colpart = rowpart + (size_t)nct * out;
  double* tot = normalized ? colpart + (size_t)nrt * in : nullptr;
  const dim3 grid(nct, nrt), block(256);
  const int fin_blocks = (out + in + 63) / 64;
  auto finalize = [&](int p) {
    hipLaunchKernelGGL(k_finalize, dim3(fin_blocks), dim3(64), 0, st, rowpart, colpart, out, in, nct,
                       nrt, g + (size_t)p * out, h + (size_t)p * in, tot);
    if (normalized)
      hipLaunchKernelGGL(k_norm_h, dim3((in + 1023) / 1024), dim3(256), 0, st, tot, out, in,
                         h + (size_t)p * in);
  };
  if (meanabs) {
    hipLaunchKernelGGL((k_derive_tile<0, true, 2>), grid, block, 0, st, W, out, in, nullptr,
                       nullptr, rowpart, colpart, nullptr, KG);
    finalize(0);
    if (P == 2) {
      hipLaunchKernelGGL((k_derive_tile<1, true, 2>), grid, block, 0, st, W, out, in, g, h, rowpart,
                         colpart, planes, KG);
      finalize(1);
    } else {
      hipLaunchKernelGGL((k_derive_tile<1, true, 3>), grid, block, 0, st, W, out, in, g, h, rowpart,
                         colpart, planes, KG);
      finalize(1);
      hipLaunchKernelGGL((k_derive_tile<2, true, 3>), grid, block, 0, st, W, out, in, g, h, rowpart,
                         colpart, planes, KG);
      finalize(2);
    }
  } else if (P == 2) {
    hipLaunchKernelGGL((k_derive_tile<1, false, 2>), grid, block, 0, st, W, out, in, g, h,
                       nullptr, nullptr, planes, KG);
  } else {
    hipLaunchKernelGGL((k_derive_tile<1, false, 3>), grid, block, 0, st, W, out, in, g, h,
                       nullptr, nullptr, planes, KG);
  }
  return hipGetLastError();
}

hipError_t launch_unpack(const uint4* planes, int out, int in, int P, uint32_t* words, hipStream_t st) {
  const size_t total = (size_t)P * out * ((in + 31) / 32);
  const int blocks = (int)std::min<size_t>((total + 255) / 256, 65535);
  hipLaunchKernelGGL(k_unpack, dim3(blocks), dim3(256), 0, st, planes, out, in, P, words);
  return hipGetLastError();
}

hipError_t launch_test_f64_to_16(const double* in, uint16_t* out, int n, int bf16,
                                 hipStream_t st) {
  hipLaunchKernelGGL(k_test_f64_to_16, dim3((n + 255) / 256), dim3(256), 0, st, in, out, n, bf16);
  return hipGetLastError();
}

}  // namespace rabit
