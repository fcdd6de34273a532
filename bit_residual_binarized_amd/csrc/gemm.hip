// Prefill GEMM on packed planes: Y = Σ_p (X ⊙ h_p) B_pᵀ ⊙ g_p.
//
// The pages' kernel (RaBiT paper App. E.1) covers only the decode GEMV; this
// prefill path is a dense contraction and runs on the fp16 matrix cores:
//   * B tile = ±h_p[k] in fp16, exact: the sign bit of h_p is flipped where
//     the plane bit is 1 (two columns k, k+16 of a 32-column word per dword).
//   * A tile = X in fp16; each row of X is first scaled by a power of two so
//     that its largest |x| lies in [2^14, 2^15) (exact for bf16 inputs above
//     the fp16 subnormal range), the scale is undone in the epilogue.
//   * fp32 accumulation, one accumulator set per path; g_p applied in the
//     epilogue (paper §4.1 eq.: W_hat = g ⊙ B ⊙ h).
// Inside a 32-column block the contraction index κ is permuted so that
// dword m of a fragment holds columns (m, m + 16): κ = 2m + hh <-> column
// m + 16 hh. A and B use the same κ order, so the MFMA sums the same pairs.
#include <algorithm>
#include <type_traits>

#include "rabit_internal.h"

namespace rabit {

namespace {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 h2v __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kBN = 128, kBK = 64;
// token rows per workgroup: 128 with two paths; 64 with three (the third
// accumulator set would not fit the registers of two waves per SIMD)
__host__ __device__ constexpr int bm_of(int P) { return P == 2 ? 128 : 64; }
constexpr int kLdsStride = 36;  // dwords per 64-column row in LDS (32 + 4 padding)

struct GemmWs {
  uint16_t* xh;      // fp16 [m][Kp], κ-permuted inside 32-column blocks
  int* rowexp;       // [m] power-of-two exponent applied to row m
  uint32_t* hpairs;  // [P][Kp/32][16] fp16 pairs (h[32b+m], h[32b+m+16])
  float* part;       // split K: [Z][m][out] partial Σ_p g_p acc_p
};

__host__ inline size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }

// split of K over grid.z: enough workgroups to fill the chip, at least four
// 64-column steps per slice
__host__ inline int split_k(int out, int in, int m, int bm, int bn = kBN) {
  const int Kp = col_groups(in) * 128;
  const int tiles = ((out + bn - 1) / bn) * ((m + bm - 1) / bm);
  int z = std::max(1, (512 + tiles - 1) / tiles);
  z = std::min(z, std::max(1, Kp / (4 * kBK)));
  return std::min(z, 16);
}

__host__ inline GemmWs carve(void* ws, int out, int in, int m, int P) {
  const size_t Kp = (size_t)col_groups(in) * 128;
  char* p = (char*)ws;
  GemmWs w;
  w.xh = (uint16_t*)p;
  p += a256((size_t)m * Kp * 2);
  w.rowexp = (int*)p;
  p += a256((size_t)m * 4);
  w.hpairs = (uint32_t*)p;
  p += a256((size_t)P * (Kp / 32) * 16 * 4);
  w.part = (float*)p;
  return w;
}

__host__ inline size_t ws_bytes_p(int out, int in, int m, int P) {
  const size_t Kp = (size_t)col_groups(in) * 128;
  // the exact path's tiles (bm_of(P) rows) or the effective-weight path's (128)
  const int z = std::max(split_k(out, in, m, bm_of(P)), split_k(out, in, m, 128, 2 * kBN));
  return a256((size_t)m * Kp * 2) + a256((size_t)m * 4) + a256((size_t)P * (Kp / 32) * 16 * 4) +
         (z > 1 ? a256((size_t)z * m * out * 4) : 0);
}

// enough for a layer of two or of three paths
__host__ inline size_t ws_bytes(int out, int in, int m) {
  return std::max(ws_bytes_p(out, in, m, 2), ws_bytes_p(out, in, m, 3));
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}
__device__ __forceinline__ uint32_t f16_to_bits(float f) { return f32_to_f16_bits(f); }

// One wave per row of X: row maximum, exponent, scaled fp16 copy. Lane l
// handles 32-column blocks l, l + 64, ...: four 16-byte loads of bf16, then
// the block's κ order (dword m = columns m, m + 16) in four 16-byte stores.
__global__ __launch_bounds__(256) void k_gemm_prep_x(const uint16_t* __restrict__ X, int in, int Kp,
                                                     int M, GemmWs ws) {
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6), l = threadIdx.x & 63;
  if (m >= M) return;
  const uint16_t* xr = X + (size_t)m * in;
  const int nblk = Kp / 32;
  const bool vec = (in & 7) == 0;  // rows 16-byte aligned
  float mx = 0.0f;
  for (int b = l; b < nblk; b += 64) {
    const int c0 = 32 * b;
    if (vec && c0 + 32 <= in) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 t = *(const uint4*)(xr + c0 + 8 * q);
        const uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
        for (int k = 0; k < 4; ++k)
          mx = fmaxf(mx, fmaxf(fabsf(__uint_as_float(w[k] << 16)), fabsf(__uint_as_float(w[k] & 0xFFFF0000u))));
      }
    } else {
      for (int c = c0; c < min(c0 + 32, in); ++c) mx = fmaxf(mx, fabsf(bf16_bits_to_f32(xr[c])));
    }
  }
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) mx = fmaxf(mx, __shfl_xor(mx, s, 64));
  const int e = (mx > 0.0f) ? 14 - ilogbf(mx) : 0;
  uint16_t* xo = ws.xh + (size_t)m * Kp;
  for (int b = l; b < nblk; b += 64) {
    const int c0 = 32 * b;
    float v[32];
    if (vec && c0 + 32 <= in) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 t = *(const uint4*)(xr + c0 + 8 * q);
        const uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          v[8 * q + 2 * k] = __uint_as_float(w[k] << 16);
          v[8 * q + 2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
        }
      }
    } else {
#pragma unroll
      for (int c = 0; c < 32; ++c) v[c] = c0 + c < in ? bf16_bits_to_f32(xr[min(c0 + c, in - 1)]) : 0.0f;
    }
    // dword mm of the block = (column mm, column mm + 16), scaled by 2^e
    uint32_t o[16];
#pragma unroll
    for (int mm = 0; mm < 16; ++mm)
      o[mm] = (uint32_t)f32_to_f16_bits(ldexpf(v[mm], e)) |
              ((uint32_t)f32_to_f16_bits(ldexpf(v[mm + 16], e)) << 16);
    uint4* dst = (uint4*)(xo + c0);
#pragma unroll
    for (int q = 0; q < 4; ++q) dst[q] = make_uint4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
  }
  if (l == 0) ws.rowexp[m] = e;
}

__global__ void k_gemm_prep_h(const uint16_t* __restrict__ h, int in, int Kp, int P, GemmWs ws) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;  // (p, blk, pair)
  const int nb = Kp / 32;
  if (idx >= P * nb * 16) return;
  const int pr = idx & 15, blk = (idx >> 4) % nb, p = idx / (16 * nb);
  const int c0 = blk * 32 + pr, c1 = c0 + 16;
  const uint32_t lo = c0 < in ? h[(size_t)p * in + c0] : 0;
  const uint32_t hi = c1 < in ? h[(size_t)p * in + c1] : 0;
  ws.hpairs[idx] = lo | (hi << 16);
}

// 128 x 128 output tile per workgroup and K slice blockIdx.z, 64 columns per
// step. Wave w owns output columns [32 w, 32 w + 32) for all 128 rows, and
// builds its own ±h_p fragments in registers from the plane words (no LDS for
// the weights): lane (fr, fg) of fragment (p, j, sub) holds rows κ = 8 fg ..
// 8 fg + 7 of column n0 + 32 w + 16 j + fr, i.e. pairs (m, m + 16), m = 4 fg + c,
// of the 32-column block. X goes through a double-buffered LDS tile (one
// barrier per step). The next step's X rows, plane words and h pairs are
// loaded into registers while the current step runs on the matrix cores.
//
// WEFF: the effective weight of the tile, Σ_p g_p[n] (±h_p[k]), is formed in
// fp16 before the matrix op instead of one matrix op per path: with
// f[n] = max_p |g_p[n]| and r_p = g_p / f (fp16, in [-1, 1]), the B fragment is
// e = Σ_p r_p (±h_p) by packed fp16 multiply-adds (path order) and f[n] is
// applied in the epilogue. One accumulator set; 128 x 256 tiles for any P,
// each wave 64 output columns.
template <int P, bool WEFF>
__global__ __launch_bounds__(256, 2) void k_gemm(const uint4* __restrict__ planes,
                                              const uint16_t* __restrict__ g, int out, int M,
                                              int Kp, int ksteps, GemmWs ws, void* Y, int y_dtype) {
  constexpr int kBM = WEFF ? 128 : bm_of(P), MT = kBM / 16;  // 16-row matrix tiles per wave
  constexpr int NA = WEFF ? 1 : P;                             // accumulator sets
  // 16-column fragments per wave: 2 (exact path), 4 (WEFF: one fragment
  // build feeds four matrix ops per X fragment read, as in the exact path)
  constexpr int NJ = WEFF ? 4 : 2;
  const int n0 = blockIdx.x * (64 * NJ), m0 = blockIdx.y * kBM;
  const int tid = threadIdx.x, l = tid & 63;
  const int wn = __builtin_amdgcn_readfirstlane(tid >> 6) * (16 * NJ);
  const int KG = Kp / 128;
  const int nb = Kp / 32;
  const int out_pad = row_groups(out) * 64;
  const int ks0 = blockIdx.z * ksteps, ks1 = min(Kp / kBK, ks0 + ksteps);
  // 16-row MFMA tiles of the workgroup that hold rows of X (uniform)
  const int mtiles = __builtin_amdgcn_readfirstlane(min(MT, max(0, (M - m0 + 15) / 16)));
  const int fr = l & 15, fg = l >> 4;

  __shared__ __align__(16) uint32_t sA[2][kBM * kLdsStride];
  __shared__ __align__(16) uint32_t sH[2][P][2][16];  // [buffer][p][sub]: the step's h pairs

  v4f acc[NA][MT][NJ];
#pragma unroll
  for (int p = 0; p < NA; ++p)
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[p][i][j] = (v4f){0.f, 0.f, 0.f, 0.f};

  // A loader: thread -> row m0 + (tid >> 1), half (tid & 1) of the 64 columns
  const int am = m0 + (tid >> 1), ah = tid & 1;
  const bool aload = (tid >> 1) < kBM;  // all threads with 128 rows, half with 64
  const bool avalid = aload && am < M;
  const uint4* asrc = (const uint4*)(ws.xh + (size_t)min(am, M - 1) * Kp) + ah * 4;
  // B: the words of rows n0 + wn + 16 j + fr. These rows lie in one 64-row
  // group (n0 + wn is a multiple of 16 NJ), so one base pointer per path
  // serves every j (row 16 j is 16 j units further); a group past the last
  // is clamped to it (those columns are not stored).
  const uint32_t* wsrc[P];
  {
    const int base = n0 + wn;
    const int rg = min(base >> 6, out_pad / 64 - 1);
#pragma unroll
    for (int p = 0; p < P; ++p)
      wsrc[p] = (const uint32_t*)(planes + unit_index(rg, 0, p, (base & 63) + fr, KG, P));
  }
  // h pairs of the step, staged through LDS by threads 0 .. 32 P - 1: (p, sub, pair)
  const bool hload = tid < 32 * P;
  const int hp = hload ? tid >> 5 : 0, hs = (tid >> 4) & 1, hq = tid & 15;
  const uint32_t* hsrc = ws.hpairs + (size_t)hp * nb * 16 + hs * 16 + hq;

  // WEFF: per fragment column n (j = 0, 1), f = max_p g_p[n] and the fp16
  // ratios r_p = g_p / f, duplicated into both halves of a dword
  uint32_t rpair[P][NJ];
  if (WEFF) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int n = min(n0 + wn + 16 * j + fr, out - 1);
      float gv[P], f = 0.f;
#pragma unroll
      for (int p = 0; p < P; ++p) {
        gv[p] = f16_bits_to_f32(g[(size_t)p * out + n]);
        f = fmaxf(f, fabsf(gv[p]));
      }
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const uint32_t rb = f16_to_bits(f > 0.f ? gv[p] / f : 0.f);
        rpair[p][j] = rb | (rb << 16);
      }
    }
  }

  // WEFF: the step's plane words of the workgroup's 256 rows go through LDS
  // (thread t loads row n0 + t of every path), which keeps the registers of
  // four fragments per wave free for the accumulators
  constexpr int NW = WEFF ? 2 : 1;
  __shared__ __align__(16) uint2 sW[NW][WEFF ? P : 1][WEFF ? 256 : 1];
  const uint32_t* wrow[P];
  if (WEFF) {
    const int r = n0 + tid;
    const int rg = min(r >> 6, out_pad / 64 - 1);
#pragma unroll
    for (int p = 0; p < P; ++p)
      wrow[p] = (const uint32_t*)(planes + unit_index(rg, 0, p, r & 63, KG, P));
  }

  uint4 ra[4];
  uint2 rw[P][WEFF ? 1 : NJ];  // [p][j]: words 2 ks, 2 ks + 1 of the row (the two 32-column blocks)
  uint32_t rh = 0;
  auto load = [&](int ks) {
#pragma unroll
    for (int q = 0; q < 4; ++q) ra[q] = asrc[(size_t)ks * 8 + q];
    // column group ks / 2 is P x 64 units (4 dwords each) after group 0
    const size_t wo = (size_t)(ks >> 1) * (P * 64 * 4) + 2 * (ks & 1);
#pragma unroll
    for (int p = 0; p < P; ++p) {
      if (WEFF) {
        rw[p][0] = *(const uint2*)(wrow[p] + wo);
      } else {
#pragma unroll
        for (int j = 0; j < NJ; ++j) rw[p][j] = *(const uint2*)(wsrc[p] + 64 * j + wo);
      }
    }
    if (hload) rh = hsrc[(size_t)ks * 32];
  };
  auto store_a = [&](int buf) {
    if (aload) {
      uint32_t* da = sA[buf] + (tid >> 1) * kLdsStride + ah * 16;
#pragma unroll
      for (int q = 0; q < 4; ++q) *(uint4*)(da + 4 * q) = avalid ? ra[q] : make_uint4(0, 0, 0, 0);
    }
    if (hload) sH[buf][hp][hs][hq] = rh;
    if (WEFF) {
#pragma unroll
      for (int p = 0; p < P; ++p) sW[buf & (NW - 1)][p][tid] = rw[p][0];
    }
  };
  if (ks0 < ks1) {
    load(ks0);
    store_a(0);
  }
  __syncthreads();

  // the main loop, in a copy without per-tile guards for full 128-row tiles
  // (a guard per matrix op splits the loop into small blocks that the
  // scheduler cannot overlap)
  auto run = [&](auto full_tag) {
  constexpr bool kFull = decltype(full_tag)::value;
  for (int ks = ks0; ks < ks1; ++ks) {
    const int buf = (ks - ks0) & 1;
    uint2 cw[P][WEFF ? 1 : NJ];  // WEFF reads its words from LDS where it uses them
    if (!WEFF) {
#pragma unroll
      for (int p = 0; p < P; ++p)
#pragma unroll
        for (int j = 0; j < NJ; ++j) cw[p][WEFF ? 0 : j] = rw[p][WEFF ? 0 : j];
    }
    if (ks + 1 < ks1) load(ks + 1);  // in flight during the matrix ops

    const uint32_t* a0 = sA[buf] + fr * kLdsStride + 4 * fg;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      v8h fa[MT];
#pragma unroll
      for (int i = 0; i < MT; ++i) fa[i] = *(const v8h*)(a0 + 16 * i * kLdsStride + 16 * sub);
      // dword c of a fragment holds columns (m, m + 16), m = 4 fg + c: the
      // sign bits are bits m and m + 16 of the word, moved to bits 15 and 31
      const int sh = 15 - 4 * fg;
      if (WEFF) {
        uint4 hh[P];
#pragma unroll
        for (int p = 0; p < P; ++p) hh[p] = *(const uint4*)(&sH[buf][p][sub][4 * fg]);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          uint32_t e[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            h2v t;
#pragma unroll
            for (int p = 0; p < P; ++p) {
              const uint32_t w = ((const uint32_t*)&sW[buf & (NW - 1)][p][wn + 16 * j + fr])[sub];
              const h2v x = __builtin_bit_cast(h2v, (&hh[p].x)[c] ^ ((w << (sh - c)) & 0x80008000u));
              const h2v r = __builtin_bit_cast(h2v, rpair[p][j]);
              t = p == 0 ? r * x : __builtin_elementwise_fma(r, x, t);
            }
            e[c] = __builtin_bit_cast(uint32_t, t);
          }
          const v8h fb = __builtin_bit_cast(v8h, make_uint4(e[0], e[1], e[2], e[3]));
#pragma unroll
          for (int i = 0; i < MT; ++i)
            if (kFull || i < mtiles)
              acc[0][i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa[i], fb, acc[0][i][j], 0, 0, 0);
        }
      } else {
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const uint4 hh = *(const uint4*)(&sH[buf][p][sub][4 * fg]);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const uint32_t w = sub ? cw[p][WEFF ? 0 : j].y : cw[p][WEFF ? 0 : j].x;
          uint4 e;
          e.x = hh.x ^ ((w << sh) & 0x80008000u);
          e.y = hh.y ^ ((w << (sh - 1)) & 0x80008000u);
          e.z = hh.z ^ ((w << (sh - 2)) & 0x80008000u);
          e.w = hh.w ^ ((w << (sh - 3)) & 0x80008000u);
          const v8h fb = __builtin_bit_cast(v8h, e);
#pragma unroll
          for (int i = 0; i < MT; ++i)
            if (kFull || i < mtiles)
              acc[p][i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa[i], fb, acc[p][i][j], 0, 0, 0);
        }
      }
      }
    }
    if (ks + 1 < ks1) store_a(buf ^ 1);
    __syncthreads();
  }
  };
  if (mtiles == MT)
    run(std::true_type{});
  else
    run(std::false_type{});

  // epilogue: C[i][j] of a 16x16 tile: lane l, reg r -> row 4(l/16)+r, col l%16
  const bool split = gridDim.z > 1;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int n = n0 + wn + 16 * j + (l & 15);
    if (n >= out) continue;
    float g0 = f16_bits_to_f32(g[n]);
    if (WEFF) {  // f[n] = max_p |g_p[n]|, as in the prologue
      g0 = fabsf(g0);
#pragma unroll
      for (int p = 1; p < P; ++p) g0 = fmaxf(g0, fabsf(f16_bits_to_f32(g[(size_t)p * out + n])));
    }
    const float g1 = (!WEFF) ? f16_bits_to_f32(g[out + n]) : 0.f;
    const float g2 = (!WEFF && P == 3) ? f16_bits_to_f32(g[2 * out + n]) : 0.f;
#pragma unroll
    for (int i = 0; i < MT; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + 16 * i + 4 * (l >> 4) + r;
        if (m >= M) continue;
        float v = g0 * acc[0][i][j][r];
        if (!WEFF) v += g1 * acc[NA > 1 ? 1 : 0][i][j][r];
        if (!WEFF && P == 3) v += g2 * acc[NA - 1][i][j][r];
        if (split) {
          ws.part[((size_t)blockIdx.z * M + m) * out + n] = v;
        } else {
          const float y = ldexpf(v, -ws.rowexp[m]);
          if (y_dtype == RABIT_OUT_F32)
            ((float*)Y)[(size_t)m * out + n] = y;
          else
            ((uint16_t*)Y)[(size_t)m * out + n] = f32_to_bf16_rne(y);
        }
      }
    }
  }
}

// split K: Y = 2^-rowexp Σ_z part[z] (ascending z)
__global__ __launch_bounds__(256) void k_gemm_reduce(GemmWs ws, int out, int M, int Z, void* Y,
                                                     int y_dtype) {
  const size_t idx = blockIdx.x * (size_t)256 + threadIdx.x;
  if (idx >= (size_t)M * out) return;
  const int m = (int)(idx / out);
  float v = 0.f;
  for (int z = 0; z < Z; ++z) v += ws.part[(size_t)z * M * out + idx];
  const float y = ldexpf(v, -ws.rowexp[m]);
  if (y_dtype == RABIT_OUT_F32)
    ((float*)Y)[idx] = y;
  else
    ((uint16_t*)Y)[idx] = f32_to_bf16_rne(y);
}

}  // namespace

size_t gemm_workspace_bytes(int out, int in, int m) { return ws_bytes(out, in, m); }

hipError_t launch_gemm(const uint4* planes, const uint16_t* g, const uint16_t* h, int out, int in,
                       const uint16_t* X, int m, void* Y, int y_dtype, void* ws, hipStream_t st,
                       int paths, bool weff) {
  if (paths != 2 && paths != 3) return hipErrorInvalidValue;
  const int Kp = col_groups(in) * 128;
  GemmWs w = carve(ws, out, in, m, paths);
  hipLaunchKernelGGL(k_gemm_prep_x, dim3((m + 3) / 4), dim3(256), 0, st, X, in, Kp, m, w);
  const int nh = paths * (Kp / 32) * 16;
  hipLaunchKernelGGL(k_gemm_prep_h, dim3((nh + 255) / 256), dim3(256), 0, st, h, in, Kp, paths, w);
  const int bm = weff ? 128 : bm_of(paths), bn = weff ? 2 * kBN : kBN;
  const int Z = split_k(out, in, m, bm, bn);
  const int steps = Kp / kBK;
  const int per = (steps + Z - 1) / Z;
  const dim3 grid((out + bn - 1) / bn, (m + bm - 1) / bm, Z);
  auto kern = paths == 3 ? (weff ? k_gemm<3, true> : k_gemm<3, false>)
                         : (weff ? k_gemm<2, true> : k_gemm<2, false>);
  hipLaunchKernelGGL(kern, grid, dim3(256), 0, st, planes, g, out, m, Kp, per, w, Y, y_dtype);
  if (Z > 1) {
    const size_t n = (size_t)m * out;
    hipLaunchKernelGGL(k_gemm_reduce, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, w, out,
                       m, Z, Y, y_dtype);
  }
  return hipGetLastError();
}

}  // namespace rabit
