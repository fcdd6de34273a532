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
// Small token counts (decode batches, M <= 32): 32-row token tiles and 256
// output columns per workgroup (64 per wave), K split up to 32 ways. The
// ±h fragments are built once per weight whatever M, so a 128-row tile
// would spend the same fragment work on at most a quarter of its rows.
constexpr int kSmallM = 32, kSmallBM = 32, kSmallBN = 256, kSmallZcap = 32;
// output columns per workgroup: 128 on the exact path; 256 on the
// effective-weight path with two paths, 128 with three (the three ratio
// registers per fragment column would spill with four fragments per wave)
__host__ __device__ constexpr int bn_of(int P, bool weff) { return weff && P == 2 ? 256 : 128; }

struct GemmWs {
  uint16_t* xh;      // fp16 [m][Kp], κ-permuted inside 32-column blocks
  int* rowexp;       // [m] power-of-two exponent applied to row m
  uint32_t* hpairs;  // [P][Kp/32][16] fp16 pairs (h[32b+m], h[32b+m+16])
  float* part;       // split K: [Z][m][out] partial Σ_p g_p acc_p
};

__host__ inline size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }

// split of K over grid.z (1..16 slices of at least four 64-column steps):
// the z with the least modelled time, in units of one workgroup step. The
// kernel takes ceil(z tiles / 512) rounds (two workgroups on each of 256 CUs)
// of ceil(steps / z) steps plus about two for filling the ring and the
// epilogue; a split adds the ordered reduce, which reads z and writes one
// fp32 partial per output (about (z + 1) m out / 1.5e6 steps at 4 TB/s and
// 1.5 us per step). Among equal kernel times the smallest z wins, so no
// slice is ever empty.
__host__ inline int split_k(int out, int in, int m, int bm, int bn = kBN, int zcap = 16) {
  const int Kp = col_groups(in) * 128;
  const int steps = Kp / kBK;
  const long long tiles = (long long)((out + bn - 1) / bn) * ((m + bm - 1) / bm);
  const int zmax = std::min(zcap, std::max(1, steps / 4));
  int best = 1;
  double best_cost = 0.0;
  for (int z = 1; z <= zmax; ++z) {
    const double rounds = (double)((z * tiles + 511) / 512);
    double cost = rounds * (double)((steps + z - 1) / z + 2);
    if (z > 1) cost += (double)(z + 1) * (double)m * (double)out / 1.5e6;
    if (z == 1 || cost < best_cost) {
      best = z;
      best_cost = cost;
    }
  }
  return best;
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
  int z = std::max(split_k(out, in, m, bm_of(P)), split_k(out, in, m, 128, bn_of(P, true)));
  if (m <= kSmallM) z = std::max(z, split_k(out, in, m, kSmallBM, kSmallBN, kSmallZcap));
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
__device__ __forceinline__ void prep_x(const uint16_t* __restrict__ X, int in, int Kp, int M, GemmWs ws,
                                       int blk) {
  const int m = blk * 4 + (threadIdx.x >> 6), l = threadIdx.x & 63;
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

// h pairs (h[32 b + m], h[32 b + m + 16]) of every path and 32-column block
__device__ __forceinline__ void prep_h(const uint16_t* __restrict__ h, int in, int Kp, int P, GemmWs ws,
                                       int wg) {
  const int idx = wg * 256 + threadIdx.x;  // (p, blk, pair)
  const int nb = Kp / 32;
  if (idx >= P * nb * 16) return;
  const int pr = idx & 15, blk = (idx >> 4) % nb, p = idx / (16 * nb);
  const int c0 = blk * 32 + pr, c1 = c0 + 16;
  const uint32_t lo = c0 < in ? h[(size_t)p * in + c0] : 0;
  const uint32_t hi = c1 < in ? h[(size_t)p * in + c1] : 0;
  ws.hpairs[idx] = lo | (hi << 16);
}

// The two preparations of a call in one launch: workgroups [0, nbx) take the
// X rows (four per workgroup), the rest the h pairs (256 per workgroup).
__global__ __launch_bounds__(256) void k_gemm_prep(const uint16_t* __restrict__ X, const uint16_t* __restrict__ h,
                                                   int in, int Kp, int M, int P, int nbx, GemmWs ws) {
  if ((int)blockIdx.x < nbx)
    prep_x(X, in, Kp, M, ws, blockIdx.x);
  else
    prep_h(h, in, Kp, P, ws, blockIdx.x - nbx);
}

// LDS bytes of one stage of the main loop's ring (X rows, plane words and h
// pairs of one 64-column step), and the ring depth: four stages where two
// workgroups fit a CU's 160 KiB of LDS, else three
__host__ __device__ constexpr int stage_bytes(int BM, int BN, int P) { return BM * 128 + P * BN * 8 + 1024; }
__host__ __device__ constexpr int n_stages(int BM, int BN, int P) {
  return 2 * 4 * stage_bytes(BM, BN, P) <= 160 * 1024 ? 4 : 3;
}

// kBM x kBN output tile per workgroup and K slice blockIdx.z, 64 columns per
// step. Wave w owns output columns [16 NJ w, 16 NJ (w + 1)) for all kBM rows,
// and builds its own ±h_p fragments in registers from the plane words: lane
// (fr, fg) of fragment (p, j, sub) holds rows κ = 8 fg .. 8 fg + 7 of column
// n0 + 16 NJ w + 16 j + fr, i.e. pairs (m, m + 16), m = 4 fg + c, of the
// 32-column block.
//
// Operands flow through a ring of NS LDS stages filled by direct
// buffer-to-LDS loads, NS - 1 steps ahead of the matrix ops: no staging
// registers and no per-step address arithmetic (the step selects the buffer
// descriptor's base; rows past M and steps past the slice read as zero from
// the descriptor's bound). Every wave issues the same number of loads per
// stage, so one vmcnt value waits for a stage; one barrier per step publishes
// the stage and frees the one the next loads overwrite.
//
// WEFF: the effective weight of the tile, Σ_p g_p[n] (±h_p[k]), is formed in
// fp16 before the matrix op instead of one matrix op per path: with
// f[n] = max_p |g_p[n]| and r_p = g_p / f (fp16, in [-1, 1]), the B fragment is
// e = Σ_p r_p (±h_p) by packed fp16 multiply-adds (path order) and f[n] is
// applied in the epilogue. One accumulator set; 128-row tiles of 256 output
// columns with two paths (64 per wave) and 128 with three (32 per wave).
template <int P, bool WEFF, bool SMALL = false>
__global__ __launch_bounds__(256, 2) void k_gemm(const uint4* __restrict__ planes,
                                              const uint16_t* __restrict__ g, int out, int M,
                                              int Kp, int ksteps, GemmWs ws, void* Y, int y_dtype) {
  static_assert(!(SMALL && WEFF), "the small-M tiles are for the exact path");
  constexpr int kBM = SMALL ? kSmallBM : WEFF ? 128 : bm_of(P), MT = kBM / 16;  // 16-row tiles per wave
  constexpr int kBNt = SMALL ? kSmallBN : bn_of(P, WEFF);
  constexpr int NA = WEFF ? 1 : P;  // accumulator sets
  constexpr int NJ = kBNt / 64;     // 16-column fragments per wave
  constexpr int NS = n_stages(kBM, kBNt, P);
  // loads per wave and stage: X in 16-byte units (4 KiB per workgroup-wide
  // load), words in 4-byte units (1 KiB), h pairs in one load (8 P lanes
  // carry pairs, the others read zeros: no lane is masked off, since a
  // masked load is a branch that costs the compiler its count of the loads
  // in flight)
  constexpr int LA = kBM / 32, LW = P * kBNt / 128, NL = LA + LW + 1;
  // each part of each stage is an object of its own, so that the compiler
  // sees that reading one stage does not wait for loads into the others
  __shared__ __align__(16) uint32_t sa0[kBM * 32], sa1[kBM * 32], sa2[kBM * 32], sa3[kBM * 32];
  __shared__ __align__(16) uint2 sw0[P * kBNt], sw1[P * kBNt], sw2[P * kBNt], sw3[P * kBNt];
  __shared__ __align__(16) uint32_t sh0[256], sh1[256], sh2[256], sh3[256];
  struct SP {
    uint32_t* a;  // row r: 128 bytes; 16-byte slot s holds column block s ^ (r & 7): the 8
                  // rows that one 128-byte phase of a fragment read touches hit 8 slots
    uint2* w;     // [p][n]: words 2 ks, 2 ks + 1 of row n0 + n, path p
    uint32_t* h;  // h pair e = 32 p + 16 sub + q (the step's two 32-column blocks) at
                  // 64 (e / 8 P) + e % 8 P: 8 P pairs per wave's 64-dword slot
  };
  auto stage = [&](auto U) __attribute__((always_inline)) -> SP {
    constexpr int u = decltype(U)::value;
    if constexpr (u == 0) return SP{sa0, sw0, sh0};
    else if constexpr (u == 1) return SP{sa1, sw1, sh1};
    else if constexpr (u == 2) return SP{sa2, sw2, sh2};
    else return SP{sa3, sw3, sh3};
  };

  const int n0 = blockIdx.x * kBNt, m0 = blockIdx.y * kBM;
  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = w * (16 * NJ);
  const int KG = Kp / 128;
  const int nb = Kp / 32;
  const int out_pad = row_groups(out) * 64;
  const int ks0 = blockIdx.z * ksteps, ks1 = min(Kp / kBK, ks0 + ksteps);
  // 16-row MFMA tiles of the workgroup that hold rows of X (uniform)
  const int mtiles = __builtin_amdgcn_readfirstlane(min(MT, max(0, (M - m0 + 15) / 16)));
  const int fr = l & 15, fg = l >> 4;

  v4f acc[NA][MT][NJ];
#pragma unroll
  for (int p = 0; p < NA; ++p)
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[p][i][j] = (v4f){0.f, 0.f, 0.f, 0.f};

  // ---- loader: per-lane byte offsets, the same for every step ----
  // X: load i of wave w fills rows 8 (4 i + w) .. + 7; lane l: row
  // 8 (4 i + w) + (l >> 3), LDS slot l & 7, column block (l & 7) ^ (row & 7)
  uint32_t offA[LA];
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    const int r = 8 * (4 * i + w) + (l >> 3);
    offA[i] = (uint32_t)r * (uint32_t)Kp * 2u + 16u * (uint32_t)((l & 7) ^ (r & 7));
  }
  // words: load i of wave w, lane l: element e = 64 (4 i + w) + l of [P][kBNt][2]
  // (rows past the last 64-row group read that group; they are not stored)
  uint32_t offW[LW];
#pragma unroll
  for (int i = 0; i < LW; ++i) {
    const int e = 64 * (4 * i + w) + l;
    const int p = e / (2 * kBNt), n = (e >> 1) % kBNt, d = e & 1;
    const int rg = min((n0 + n) >> 6, out_pad / 64 - 1);
    offW[i] = (uint32_t)(unit_index(rg, 0, p, n & 63, KG, P) * 16 + 4 * d);
  }
  // h pairs: lane l < 8 P of wave w loads pair e = 8 P w + l of [P][2][16];
  // the other lanes read past the descriptor's bound (zeros)
  const uint32_t offH = l < 8 * P ? 4u * (uint32_t)(((8 * P * w + l) >> 5) * nb * 16 + ((8 * P * w + l) & 31))
                                  : 0x7FFFFFF0u;
  const size_t plane_bytes = (size_t)(out_pad / 64) * KG * P * 1024;
  const size_t x_bytes = (size_t)(M - m0) * Kp * 2;
  auto issue = [&](SP S, int k) __attribute__((always_inline)) {
    const bool live = k < ks1;  // uniform: later steps only keep the load count
    {
      const size_t kb = (size_t)k * kBK * 2;
      const uint32_t n = live ? (uint32_t)min(x_bytes - kb, (size_t)0xFFFFFFFFu) : 0u;
      const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
          (void*)((const char*)(ws.xh + (size_t)m0 * Kp) + kb), (short)0, (int)n, kBufWord3);
#pragma unroll
      for (int i = 0; i < LA; ++i)
        lds_load16(r, (lds_void*)(S.a + (4 * i + w) * 256), offA[i]);
    }
    {
      const size_t kb = (size_t)(k >> 1) * P * 1024 + 8 * (k & 1);
      const uint32_t n = live ? (uint32_t)(plane_bytes - kb) : 0u;
      const __amdgpu_buffer_rsrc_t r =
          __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)planes + kb), (short)0, (int)n, kBufWord3);
#pragma unroll
      for (int i = 0; i < LW; ++i)
        lds_load4(r, (lds_void*)((uint32_t*)S.w + (4 * i + w) * 64), offW[i]);
    }
    {
      const size_t kb = (size_t)k * 32 * 4;
      const uint32_t n = live ? (uint32_t)((size_t)P * nb * 16 * 4 - kb) : 0u;
      const __amdgpu_buffer_rsrc_t r =
          __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)ws.hpairs + kb), (short)0, (int)n, kBufWord3);
      lds_load4(r, (lds_void*)(S.h + 64 * w), offH);
    }
  };

  // WEFF: per fragment column n (j = 0 .. NJ - 1), f = max_p |g_p[n]| and the
  // fp16 ratios r_p = g_p / f, duplicated into both halves of a dword
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

  auto hpos = [](int e) { return 64 * (e / (8 * P)) + e % (8 * P); };
  // the matrix ops of one step from stage S
  const int xsw = fr & 7;  // this lane's X rows 16 i + fr share the slot swizzle
  auto compute = [&](SP S, auto full_tag) __attribute__((always_inline)) {
    constexpr bool kFull = decltype(full_tag)::value;
    uint2 cw[P][WEFF ? 1 : NJ];  // exact path: this lane's words, both 32-column blocks
    if (!WEFF) {
#pragma unroll
      for (int p = 0; p < P; ++p)
#pragma unroll
        for (int j = 0; j < NJ; ++j) cw[p][WEFF ? 0 : j] = S.w[p * kBNt + wn + 16 * j + fr];
    }
    const uint32_t* a0 = S.a + fr * 32;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      // two paths: one half's X fragments live at a time (two halves' did
      // not fit the registers of two waves per SIMD); three paths leave the
      // scheduler free to overlap the halves
      if (sub && P == 2 && !SMALL) __builtin_amdgcn_sched_barrier(0);
      v8h fa[MT];
#pragma unroll
      for (int i = 0; i < MT; ++i) fa[i] = *(const v8h*)(a0 + 512 * i + 4 * ((fg + 4 * sub) ^ xsw));
      // dword c of a fragment holds columns (m, m + 16), m = 4 fg + c: the
      // sign bits are bits m and m + 16 of the word, moved to bits 15 and 31
      const int sh = 15 - 4 * fg;
      if (WEFF) {
        uint4 hh[P];
#pragma unroll
        for (int p = 0; p < P; ++p) hh[p] = *(const uint4*)(S.h + hpos(32 * p + 16 * sub + 4 * fg));
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          uint32_t e[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            h2v t;
#pragma unroll
            for (int p = 0; p < P; ++p) {
              const uint32_t wd = ((const uint32_t*)(S.w + p * kBNt + wn + 16 * j + fr))[sub];
              const h2v x = __builtin_bit_cast(h2v, (&hh[p].x)[c] ^ ((wd << (sh - c)) & 0x80008000u));
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
          const uint4 hh = *(const uint4*)(S.h + hpos(32 * p + 16 * sub + 4 * fg));
#pragma unroll
          for (int j = 0; j < NJ; ++j) {
            const uint32_t wd = sub ? cw[p][WEFF ? 0 : j].y : cw[p][WEFF ? 0 : j].x;
            uint4 e;
            e.x = hh.x ^ ((wd << sh) & 0x80008000u);
            e.y = hh.y ^ ((wd << (sh - 1)) & 0x80008000u);
            e.z = hh.z ^ ((wd << (sh - 2)) & 0x80008000u);
            e.w = hh.w ^ ((wd << (sh - 3)) & 0x80008000u);
            const v8h fb = __builtin_bit_cast(v8h, e);
#pragma unroll
            for (int i = 0; i < MT; ++i)
              if (kFull || i < mtiles)
                acc[p][i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa[i], fb, acc[p][i][j], 0, 0, 0);
          }
        }
      }
    }
  };

  // step k from stage U: wait for this wave's loads of the stage (NS - 2
  // later stages stay in flight), barrier (every wave's loads have landed and
  // every wave is done with step k - 1), the matrix ops, then refill the
  // stage step k - 1 used with step k + NS - 1 (issued after this step's LDS
  // reads, the compiler adds no wait of its own for the loads in flight)
  auto step = [&](auto U, int k, auto full_tag) __attribute__((always_inline)) {
    constexpr int u = decltype(U)::value;
    ring_barrier<(NS - 2) * NL>();
    issue(stage(std::integral_constant<int, (u + NS - 1) % NS>{}), k + NS - 1);
    compute(stage(U), full_tag);
  };
  issue(stage(std::integral_constant<int, 0>{}), ks0);
  issue(stage(std::integral_constant<int, 1>{}), ks0 + 1);
  if constexpr (NS == 4) issue(stage(std::integral_constant<int, 2>{}), ks0 + 2);
  // the main loop, in a copy without per-tile guards for full tiles (a guard
  // per matrix op splits the loop into small blocks that the scheduler cannot
  // overlap), unrolled over the ring so that each stage is a distinct object.
  // The unrolled steps run unconditionally: a step past the slice reads the
  // zeros its zero-length descriptors return and adds exactly zero (a branch
  // per step made the compiler wait for every load in flight at the joins).
  auto run = [&](auto full_tag) __attribute__((always_inline)) {
    for (int ks = ks0; ks < ks1; ks += NS) {
      step(std::integral_constant<int, 0>{}, ks, full_tag);
      step(std::integral_constant<int, 1>{}, ks + 1, full_tag);
      step(std::integral_constant<int, 2>{}, ks + 2, full_tag);
      if constexpr (NS == 4) step(std::integral_constant<int, 3>{}, ks + 3, full_tag);
    }
  };
  if (mtiles == MT)
    run(std::true_type{});
  else
    run(std::false_type{});
  // no load may still write this workgroup's LDS when it ends
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));

  // epilogue: C[i][j] of a 16x16 tile: lane l, reg r -> row 4(l/16)+r, col l%16.
  // The scales and row exponents are all loaded first (clamped indices), so
  // that no load waits behind a store's bounds check.
  const bool split = gridDim.z > 1;
  uint16_t gq[NJ][P];
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int p = 0; p < P; ++p) gq[j][p] = g[(size_t)p * out + min(n0 + wn + 16 * j + (l & 15), out - 1)];
  int rex[MT][4];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) rex[i][r] = split ? 0 : ws.rowexp[min(m0 + 16 * i + 4 * (l >> 4) + r, M - 1)];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int n = n0 + wn + 16 * j + (l & 15);
    if (n >= out) continue;
    float g0 = f16_bits_to_f32(gq[j][0]);
    if (WEFF) {  // f[n] = max_p |g_p[n]|, as in the prologue
      g0 = fabsf(g0);
#pragma unroll
      for (int p = 1; p < P; ++p) g0 = fmaxf(g0, fabsf(f16_bits_to_f32(gq[j][p])));
    }
    const float g1 = (!WEFF) ? f16_bits_to_f32(gq[j][P > 1 ? 1 : 0]) : 0.f;
    const float g2 = (!WEFF && P == 3) ? f16_bits_to_f32(gq[j][P - 1]) : 0.f;
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
          const float y = ldexpf(v, -rex[i][r]);
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
  const int nbx = (m + 3) / 4, nh = paths * (Kp / 32) * 16;
  hipLaunchKernelGGL(k_gemm_prep, dim3(nbx + (nh + 255) / 256), dim3(256), 0, st, X, h, in, Kp, m, paths, nbx, w);
  const bool small = !weff && m <= kSmallM;
  const int bm = small ? kSmallBM : weff ? 128 : bm_of(paths), bn = small ? kSmallBN : bn_of(paths, weff);
  const int Z = small ? split_k(out, in, m, bm, bn, kSmallZcap) : split_k(out, in, m, bm, bn);
  const int steps = Kp / kBK;
  const int per = (steps + Z - 1) / Z;
  const dim3 grid((out + bn - 1) / bn, (m + bm - 1) / bm, Z);
  auto kern = paths == 3 ? (weff ? k_gemm<3, true> : small ? k_gemm<3, false, true> : k_gemm<3, false>)
                         : (weff ? k_gemm<2, true> : small ? k_gemm<2, false, true> : k_gemm<2, false>);
  hipLaunchKernelGGL(kern, grid, dim3(256), 0, st, planes, g, out, m, Kp, per, w, Y, y_dtype);
  if (Z > 1) {
    const size_t n = (size_t)m * out;
    hipLaunchKernelGGL(k_gemm_reduce, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, w, out,
                       m, Z, Y, y_dtype);
  }
  return hipGetLastError();
}

}  // namespace rabit
