// Training side of one layer (RaBiT paper §4.2, "Backward Pass and Parameter
// Updates"): the straight-through gradient to the shared weight, the scale
// gradients with the cores held constant, and the gradient to the layer input.
//
//   dW[o][i]  = Σ_n dY[n][o] X[n][i]                       (gradient of W_hat)
//   dg_p[o]   = Σ_i dW[o][i] B_p[o][i] h_p[i]              (= Σ_n dY ⊙ B_p (h_p ⊙ x_n))
//   dh_p[i]   = Σ_o dW[o][i] B_p[o][i] g_p[o]              (= Σ_n x_n ⊙ B_pᵀ (g_p ⊙ dY_n))
//   dX        = dY W_hat = the prefill GEMM of the layer W_hatᵀ (cores B_pᵀ,
//               output scales h_p, input scales g_p)
//
// k_grad_w computes 256 x 128 tiles of dW on the bf16 matrix cores (MFMA
// 16x16x32, fp32 accumulation; bf16 x bf16 products are exact in fp32) and,
// from the same accumulators, the tile's partial sums of dg and dh: dW is
// written once and never read back. The contraction runs over the tokens n,
// which are the slow index of both X [N][in] and dY [N][out]; the loaders
// turn 8 token rows of 4 columns into 4 column chunks of 8 tokens (the MFMA
// operand order) on the way into LDS.
#include <algorithm>
#include <type_traits>

#include "rabit_internal.h"

namespace rabit {

namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kTI = 256;  // dW tile: columns i
constexpr int kTO = 128;  // dW tile: rows o (128: wave tiles 128 x 64 at two waves per SIMD;
                          // 256: 128 x 128 at one wave per SIMD, accumulators in AGPRs)
constexpr int kBO = kTO / 32;   // 16-row matrix tiles per wave along o
constexpr int kCY = kTO / 64;   // dY columns per loader thread
constexpr int kK = 32;    // tokens per step

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// word 3 of a raw buffer descriptor on this architecture family (no format
// conversion, no swizzle): out-of-range reads return 0
constexpr int kBufferWord3 = 0x00020000;

__host__ inline size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }

// 16-byte chunk slot of column q inside one 8-token group: an XOR
// swizzle so that the loaders' stores (lanes 4 columns apart) and the
// fragment reads (16 consecutive columns) both spread over the LDS banks
__device__ __forceinline__ int slot(int q) { return q ^ ((q >> 3) & 3); }

struct GradWs {
  float* prow;  // [ceil(in/256)][P][128*ceil(out/128)]: per column tile, Σ over its columns
  float* pcol;  // [ceil(out/128)][P][256*ceil(in/256)]: per row tile, Σ over its rows
};

__host__ inline GradWs carve_grad(void* ws, int out, int in, int P) {
  const size_t to = (out + kTO - 1) / kTO, ti = (in + kTI - 1) / kTI;
  GradWs w;
  w.prow = (float*)ws;
  w.pcol = (float*)((char*)ws + a256(ti * P * to * kTO * 4));
  return w;
}

__host__ inline size_t grad_ws_bytes(int out, int in, int P) {
  const size_t to = (out + kTO - 1) / kTO, ti = (in + kTI - 1) / kTI;
  return a256(ti * P * to * kTO * 4) + a256(to * P * ti * kTI * 4);
}

// ---------------------------------------------------------------------------
// Bit transpose of the planes: the layer W_hatᵀ (out' = in, in' = out).
// One wave per destination slab (rg', kg', p): destination rows i in
// [64 rg', 64 rg' + 64) are source columns, destination columns o in
// [128 kg', 128 kg' + 128) are source rows. Lane l holds 64 source bits of
// rows 128 kg' + l and 128 kg' + 64 + l; ballot c over the wave collects
// column c of both 64-row blocks, which lane c stores as its unit.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_transpose_planes(const uint32_t* __restrict__ src, int out,
                                                          int in, int P, uint4* __restrict__ dst) {
  const int RGt = row_groups(in), KGt = col_groups(out), KGs = col_groups(in);
  const int RGs = row_groups(out);
  const int slab = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (slab >= RGt * KGt * P) return;
  const int l = threadIdx.x & 63;
  const int p = slab % P, kgt = (slab / P) % KGt, rgt = slab / (P * KGt);
  const int kgs = rgt >> 1, half = rgt & 1;
  uint2 w[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int o = 128 * kgt + 64 * b + l;
    w[b] = make_uint2(0, 0);
    if ((o >> 6) < RGs)
      w[b] = *(const uint2*)(src + 4 * unit_index(o >> 6, kgs, p, o & 63, KGs, P) + 2 * half);
  }
  uint4 mine = make_uint4(0, 0, 0, 0);
#pragma unroll 8
  for (int c = 0; c < 64; ++c) {
    const uint32_t s0 = c < 32 ? w[0].x >> c : w[0].y >> (c - 32);
    const uint32_t s1 = c < 32 ? w[1].x >> c : w[1].y >> (c - 32);
    const uint64_t m0 = __ballot(s0 & 1u), m1 = __ballot(s1 & 1u);
    if (l == c) mine = make_uint4((uint32_t)m0, (uint32_t)(m0 >> 32), (uint32_t)m1, (uint32_t)(m1 >> 32));
  }
  dst[unit_index(rgt, kgt, p, l, KGt, P)] = mine;
}

// ---------------------------------------------------------------------------
// Ring loader of the dW kernel (out and in multiples of 8, so that every
// token row starts on a 16-byte boundary): each 32-token step is a stage of
// raw token rows, X [32][256] then dY [32][128] bf16, filled by direct
// buffer-to-LDS loads two steps ahead (a ring of three stages, each an LDS
// object of its own, no staging registers). The matrix operands (8 tokens of
// one column per lane) come from LDS transposed reads (DS_READ_B64_TR_B16):
// in each group of 16 lanes, lane 4 q + m points at 4 columns (4 m ..) of
// token row q of a 4 x 16 block, and lane i receives column i of the 4 rows;
// two such reads give the 8 tokens of a fragment.
// ---------------------------------------------------------------------------
constexpr int kXRowB = kTI * 2;                        // bytes per token row of the X stage
constexpr int kYRowB = kTO * 2;                        // and of the dY stage
constexpr int kStageBytes = kK * (kXRowB + kYRowB);    // 24 KiB

// 16-byte slot of chunk c (8 columns) in token row r of a stage: bits 1-3 of
// c XORed with (r & 3) | (bit 3 of r) << 2, so that the 16 rows x 32 bytes
// of one transposed read spread over all banks (row strides are multiples of
// the bank width); an involution, so it also maps a slot to its chunk
__device__ __forceinline__ int rslot(int c, int r) { return c ^ (2 * ((r & 3) | ((r >> 1) & 4))); }

typedef short v4s __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4s lds_v4s;
typedef __attribute__((address_space(3))) unsigned char lds_u8;

__device__ __forceinline__ void grad_w_ring(v4f (&acc)[8][kBO], const uint16_t* X, const uint16_t* dY,
                                            int M, int out, int in, int i0, int o0, unsigned char* s0,
                                            unsigned char* s1, unsigned char* s2) {
  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wi = w & 1, wo = w >> 1, fr = l & 15, fg = l >> 4;
  auto stage = [&](auto U) __attribute__((always_inline)) -> lds_u8* {
    constexpr int u = decltype(U)::value;
    return (lds_u8*)(u == 0 ? s0 : u == 1 ? s1 : s2);
  };

  // stage <- tokens [32 ks, 32 ks + 32): wave w loads token rows 8 w .. 8 w + 7
  // of X (two rows per load) and of dY (four per load); rows past M, and
  // every row of a step past the end, read 0 (the descriptors end at row M)
  auto issue = [&](lds_u8* st, int ks) __attribute__((always_inline)) {
    const int n0 = ks * kK;
    const uint64_t left = (uint64_t)max(M - n0, 0);
    const uint64_t xb = left * in * 2, yb = left * out * 2;
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(X + (size_t)min(n0, M) * in), (short)0, (int)(xb > 0xFFFFFFFFull ? 0xFFFFFFFFu : xb),
        kBufferWord3);
    const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(dY + (size_t)min(n0, M) * out), (short)0, (int)(yb > 0xFFFFFFFFull ? 0xFFFFFFFFu : yb),
        kBufferWord3);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int r = 8 * w + 2 * k + (l >> 5), c = rslot(l & 31, r);
      lds_load16(rx, (lds_void*)(st + (8 * w + 2 * k) * kXRowB), (uint32_t)(r * in + i0 + 8 * c) * 2u);
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int r = 8 * w + 4 * k + (l >> 4), c = rslot(l & 15, r);
      lds_load16(ry, (lds_void*)(st + kK * kXRowB + (8 * w + 4 * k) * kYRowB),
                 (uint32_t)(r * out + o0 + 8 * c) * 2u);
    }
  };
  constexpr int kLoads = 6;  // loads per stage and wave

  // per-lane offsets of the transposed reads inside a stage: fragment a of X
  // (columns 128 wi + 16 a + .., tokens 8 fg ..) and b of dY (rows 64 wo +
  // 16 b + ..); lane 4 q + m of its group reads token row 8 fg + q, columns
  // 4 m .. 4 m + 3 of the fragment, and the second read the row 4 below
  const int q = fr >> 2, m = fr & 3, r0 = 8 * fg + q;
  const int sw = 2 * ((r0 & 3) | ((r0 >> 1) & 4));  // rslot's XOR for rows r0 and r0 + 4
  int offA[8], offB[kBO];
#pragma unroll
  for (int a = 0; a < 8; ++a)
    offA[a] = r0 * kXRowB + ((((128 * wi + 16 * a) >> 3) + (m >> 1)) ^ sw) * 16 + (m & 1) * 8;
#pragma unroll
  for (int b = 0; b < kBO; ++b)
    offB[b] = kK * kXRowB + r0 * kYRowB + (((((kTO / 2) * wo + 16 * b) >> 3) + (m >> 1)) ^ sw) * 16 +
              (m & 1) * 8;
  auto frag = [&](lds_u8* p, int rowb) __attribute__((always_inline)) {
    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)p);
    const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p + 4 * rowb));
    return __builtin_bit_cast(v8bf, (v8s)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // step ks from stage U: this wave's loads of the stage have landed (the
  // next stage's may be in flight), barrier (every wave's loads have landed
  // and every wave is done with step ks - 1), refill the stage step ks - 1
  // used with step ks + 2, then the matrix ops. The steps run unconditionally
  // over the ring: a step past the end reads zeros and adds exactly zero.
  auto step = [&](auto U, int ks) __attribute__((always_inline)) {
    constexpr int u = decltype(U)::value;
    ring_barrier<kLoads>();
    issue(stage(std::integral_constant<int, (u + 2) % 3>()), ks + 2);
    lds_u8* st = stage(U);
    v8bf fb[kBO];
#pragma unroll
    for (int b = 0; b < kBO; ++b) fb[b] = frag(st + offB[b], kYRowB);
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      const v8bf fa = frag(st + offA[a], kXRowB);
#pragma unroll
      for (int b = 0; b < kBO; ++b)
        acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, fb[b], acc[a][b], 0, 0, 0);
    }
  };
  const int nsteps = (M + kK - 1) / kK;
  issue(stage(std::integral_constant<int, 0>()), 0);
  issue(stage(std::integral_constant<int, 1>()), 1);
#pragma unroll 1
  for (int ks = 0; ks < nsteps; ks += 3) {
    step(std::integral_constant<int, 0>(), ks);
    step(std::integral_constant<int, 1>(), ks + 1);
    step(std::integral_constant<int, 2>(), ks + 2);
  }
  // no load may still write the ring when the epilogue reuses it
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
}

// ---------------------------------------------------------------------------
// dW tile (256 columns i x 128 rows o) and the tile's scale-gradient partials.
//
// Wave w of the workgroup owns i in [128 (w & 1), +128) and o in
// [64 (w >> 1), +64) of the tile: 8 x 4 matrix tiles of 16 x 16 (a wave tile
// of 128 x 64 reads 12 KiB of LDS per 32 matrix ops; the LDS read rate, not
// the matrix cores, bounds smaller wave tiles). MFMA rows are columns i of dW
// (A = X chunks), MFMA columns are rows o (B = dY chunks), the contraction is
// 32 tokens: lane (fr, fg) supplies tokens 8 fg .. 8 fg + 7 of column fr. The
// result lane l, register r holds dW[o = l % 16][i = 4 (l / 16) + r] of each
// 16 x 16 tile: four consecutive i, one 16-byte store.
// ---------------------------------------------------------------------------
template <int P, bool RING>
__global__ __launch_bounds__(256, kTO == 256 ? 1 : 2) void k_grad_w(const uint16_t* __restrict__ X,
                                                   const uint16_t* __restrict__ dY, int M, int out,
                                                   int in, const uint32_t* __restrict__ planes,
                                                   const uint16_t* __restrict__ g,
                                                   const uint16_t* __restrict__ h, float* dW,
                                                   int accumulate, GradWs ws) {
  const int nbx = (in + kTI - 1) / kTI, nby = (out + kTO - 1) / kTO;
  // Tile order: bands of G tile rows, column-major inside a band; each XCD
  // (workgroup id mod 8, each with its own L2) takes a contiguous run of that
  // order when the count divides by 8. An XCD's run then spans about G rows
  // by T / (8 G) columns of tiles, which read G dY panels (128 rows each) and
  // T / (8 G) X panels (256 columns, twice the bytes per token): G near
  // sqrt(T / 4) keeps that union smallest, and the tiles an XCD runs at once
  // (a few columns of one band) share their panels in its L2.
  const int T = nbx * nby;
  int o = blockIdx.x;
  if ((T & 7) == 0) o = (blockIdx.x & 7) * (T >> 3) + (blockIdx.x >> 3);
  const int G = max(1, min(nby, (int)sqrtf((float)T * 0.25f)));
  const int band = o / (G * nbx), rem = o - band * G * nbx;
  const int gb = min(G, nby - band * G);
  const int bx = rem / gb, by = band * G + rem % gb;
  const int i0 = bx * kTI, o0 = by * kTO;
  const int tid = threadIdx.x, l = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wi = wv & 1, wo = wv >> 1;
  const int fr = l & 15, fg = l >> 4;
  const int KG = col_groups(in);

  v4f acc[8][kBO];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < kBO; ++b) acc[a][b] = (v4f){0.f, 0.f, 0.f, 0.f};

  // the main loop; the epilogue's side arrays are then laid over its operand
  // buffers
  unsigned char* side;
  if constexpr (RING) {
    __shared__ __align__(16) unsigned char st0[kStageBytes], st1[kStageBytes], st2[kStageBytes];
    grad_w_ring(acc, X, dY, M, out, in, i0, o0, st0, st1, st2);
    side = st0;
  } else {
    __shared__ __align__(16) uint4 sA[2][4][kTI];  // [buf][token group][slot(i)]: X
    __shared__ __align__(16) uint4 sB[2][4][kTO];  // [buf][token group][slot(o)]: dY
    // loaders, per thread and step: X columns i0 + 4 qx .. + 3 and dY columns
    // o0 + kCY qy .. + kCY - 1, each for tokens 8 ng .. 8 ng + 7 of the step
    // token group = wave: the rows of a load are uniform (scalar addresses)
    const int ng = __builtin_amdgcn_readfirstlane(tid >> 6), qx = tid & 63, qy = tid & 63;
    const int cx = i0 + 4 * qx, cy = o0 + kCY * qy;
    const bool vx = (in & 3) == 0 && cx + 4 <= in;
    const bool vy = (out % kCY) == 0 && cy + kCY <= out;
    uint2 rx[8];
    uint2 ry[8];  // kCY = 2: .x only
    // Full-width columns: raw buffer loads from a per-step scalar base, the
    // lane's column as the only per-lane offset and the token row as the scalar
    // offset; the descriptor covers rows up to M only, so rows past M read 0.
    // Ragged columns: element loads with clamped indices, masked.
    auto load = [&](int ks) {
      const int n0 = ks * kK;
      const uint32_t left = (uint32_t)(M - n0);  // rows from n0 to M (>= 1)
      if (vx) {
        const uint64_t nbytes = (uint64_t)left * in * 2;
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(X + (size_t)n0 * in), (short)0, (int)(nbytes > 0xFFFFFFFFull ? 0xFFFFFFFFu : nbytes),
            kBufferWord3);
  #pragma unroll
        for (int j = 0; j < 8; ++j) {
          const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, 2 * cx,
                                                               (8 * ng + j) * in * 2, 0);
          rx[j] = make_uint2(v.x, v.y);
        }
      } else {
  #pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int n = n0 + 8 * ng + j;
          const size_t row = (size_t)min(n, M - 1) * in;
          uint32_t e[4];
  #pragma unroll
          for (int c = 0; c < 4; ++c) e[c] = cx + c < in ? X[row + min(cx + c, in - 1)] : 0u;
          rx[j] = n < M ? make_uint2(e[0] | (e[1] << 16), e[2] | (e[3] << 16)) : make_uint2(0, 0);
        }
      }
      if (vy) {
        const uint64_t nbytes = (uint64_t)left * out * 2;
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(dY + (size_t)n0 * out), (short)0, (int)(nbytes > 0xFFFFFFFFull ? 0xFFFFFFFFu : nbytes),
            kBufferWord3);
  #pragma unroll
        for (int j = 0; j < 8; ++j) {
          if (kCY == 4) {
            const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, 2 * cy, (8 * ng + j) * out * 2, 0);
            ry[j] = make_uint2(v.x, v.y);
          } else {
            ry[j] = make_uint2(__builtin_amdgcn_raw_buffer_load_b32(r, 2 * cy, (8 * ng + j) * out * 2, 0), 0u);
          }
        }
      } else {
  #pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int n = n0 + 8 * ng + j;
          const size_t row = (size_t)min(n, M - 1) * out;
          uint32_t e[4] = {0u, 0u, 0u, 0u};
  #pragma unroll
          for (int c = 0; c < kCY; ++c) e[c] = cy + c < out ? dY[row + min(cy + c, out - 1)] : 0u;
          ry[j] = n < M ? make_uint2(e[0] | (e[1] << 16), e[2] | (e[3] << 16)) : make_uint2(0u, 0u);
        }
      }
    };
    // 8 token rows of a column pair -> two chunks of 8 tokens (one per column):
    // dword k of a chunk holds tokens 2k, 2k + 1 (one byte permute each)
    auto chunks = [](const uint32_t (&v)[8], uint4& lo, uint4& hi) {
  #pragma unroll
      for (int k = 0; k < 4; ++k) {
        (&lo.x)[k] = __builtin_amdgcn_perm(v[2 * k + 1], v[2 * k], 0x05040100u);
        (&hi.x)[k] = __builtin_amdgcn_perm(v[2 * k + 1], v[2 * k], 0x07060302u);
      }
    };
    auto store = [&](int buf) {
      uint32_t t[8];
      uint4 c0, c1;
  #pragma unroll
      for (int j = 0; j < 8; ++j) t[j] = rx[j].x;
      chunks(t, c0, c1);
      sA[buf][ng][slot(4 * qx)] = c0;
      sA[buf][ng][slot(4 * qx + 1)] = c1;
  #pragma unroll
      for (int j = 0; j < 8; ++j) t[j] = rx[j].y;
      chunks(t, c0, c1);
      sA[buf][ng][slot(4 * qx + 2)] = c0;
      sA[buf][ng][slot(4 * qx + 3)] = c1;
  #pragma unroll
      for (int h2 = 0; h2 < kCY / 2; ++h2) {
  #pragma unroll
        for (int j = 0; j < 8; ++j) t[j] = h2 ? ry[j].y : ry[j].x;
        chunks(t, c0, c1);
        sB[buf][ng][slot(kCY * qy + 2 * h2)] = c0;
        sB[buf][ng][slot(kCY * qy + 2 * h2 + 1)] = c1;
      }
    };

    const int nsteps = (M + kK - 1) / kK;
    if (nsteps > 0) {
      load(0);
      store(0);
    }
    __syncthreads();
    for (int ks = 0; ks < nsteps; ++ks) {
      const int buf = ks & 1;
      if (ks + 1 < nsteps) load(ks + 1);  // in flight during the matrix ops
      v8bf fb[kBO];
  #pragma unroll
      for (int b = 0; b < kBO; ++b)
        fb[b] = __builtin_bit_cast(v8bf, sB[buf][fg][slot((kTO / 2) * wo + 16 * b + fr)]);
  #pragma unroll
      for (int a = 0; a < 8; ++a) {
        const v8bf fa = __builtin_bit_cast(v8bf, sA[buf][fg][slot(128 * wi + 16 * a + fr)]);
  #pragma unroll
        for (int b = 0; b < kBO; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, fb[b], acc[a][b], 0, 0, 0);
      }
      if (ks + 1 < nsteps) store(buf ^ 1);
      __syncthreads();
    }
    side = (unsigned char*)&sA[0][0][0];
  }
  constexpr int kRed = kTI > kTO ? kTI : kTO;
  static_assert(P * (2 * 4 * kTO + kTO + kTI + 2 * kRed) * 4 <= (kStageBytes < 2 * 4 * kTI * 16 ? kStageBytes : 2 * 4 * kTI * 16),
                "the side arrays fit over the operand buffers");
  // [p][column group of the tile][word][row o], [p][o], [p][i], [wave half][p][.]
  uint32_t (*sBitsW)[2][4][kTO] = reinterpret_cast<uint32_t (*)[2][4][kTO]>(side);
  float (*sG)[kTO] = reinterpret_cast<float (*)[kTO]>(side + P * 2 * 4 * kTO * 4);
  float (*sH)[kTI] = reinterpret_cast<float (*)[kTI]>(side + P * (2 * 4 * kTO + kTO) * 4);
  float (*sRed)[P][kRed] = reinterpret_cast<float (*)[P][kRed]>(side + P * (2 * 4 * kTO + kTO + kTI) * 4);
  __syncthreads();  // every wave is done with the operand buffers
  // side loads for the epilogue
  for (int t = tid; t < P * 2 * kTO; t += 256) {
    const int p = t / (2 * kTO), c = (t / kTO) & 1, r = t % kTO, o = o0 + r;
    uint4 u = make_uint4(0, 0, 0, 0);
    if ((o >> 6) < row_groups(out) && 2 * bx + c < KG)
      u = ((const uint4*)planes)[unit_index(o >> 6, 2 * bx + c, p, o & 63, KG, P)];
    sBitsW[p][c][0][r] = u.x;
    sBitsW[p][c][1][r] = u.y;
    sBitsW[p][c][2][r] = u.z;
    sBitsW[p][c][3][r] = u.w;
  }
  for (int t = tid; t < P * kTO; t += 256) {
    const int p = t / kTO, r = t % kTO, o = o0 + r;
    sG[p][r] = o < out ? f16_bits_to_f32(g[(size_t)p * out + o]) : 0.f;
  }
  for (int t = tid; t < P * kTI; t += 256) {
    const int p = t / kTI, r = t % kTI, i = i0 + r;
    sH[p][r] = i < in ? f16_bits_to_f32(h[(size_t)p * in + i]) : 0.f;
  }
  __syncthreads();

  // ---- scale-gradient partials, one 16-column block a at a time. Lane
  // (fr, fg) of tile (a, b) holds row o = o0 + 64 wo + 16 b + fr, columns
  // i = i0 + 128 wi + 16 a + 4 fg + r. The bit of (o, i) is bit i % 32 of
  // word (i % 128) / 32 = a / 2 of the row's unit in column group 2 bx + wi.
  // Row sums (dg): each lane adds its columns, then the 4 lane groups
  // (xor 16, 32), then the two waves that share the rows (in LDS, wave wi = 0
  // first). Column sums (dh): each lane adds its 4 rows, then the 16 lanes of
  // its DPP row, then the two waves that share the columns.
  // pass 1, column sums (dh). The two passes are split by a barrier: with both
  // sums in one pass the scheduler keeps every accumulator alive to the end
  // and the kernel spills.
#pragma unroll
  for (int a = 0; a < 8; ++a) {
    const int il = 128 * wi + 16 * a + 4 * fg;  // tile column of register r = 0
#pragma unroll
    for (int p = 0; p < P; ++p) {
      float cs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int b = 0; b < kBO; ++b) {
        const int ol = (kTO / 2) * wo + 16 * b + fr;
        const uint32_t word = sBitsW[p][wi][a >> 1][ol];
        const float go = sG[p][ol];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          // B_p = -1 flips the sign of the scale factor, not of dW
          const uint32_t sgn = ((word >> ((16 * a + 4 * fg + r) & 31)) & 1u) << 31;
          cs[r] += acc[a][b][r] * __uint_as_float(__float_as_uint(go) ^ sgn);
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = cs[r];
        v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xf, 0xf, false));
        v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xf, 0xf, false));
        v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xf, 0xf, false));
        v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xf, 0xf, false));
        cs[r] = v;
      }
      if (fr == 0) *(float4*)&sRed[wo][p][il] = make_float4(cs[0], cs[1], cs[2], cs[3]);
    }
  }
  __syncthreads();
  for (int t = tid; t < P * kTI; t += 256) {
    const int p = t / kTI, r = t % kTI;
    ws.pcol[((size_t)by * P + p) * ((size_t)nbx * kTI) + i0 + r] = sRed[0][p][r] + sRed[1][p][r];
  }
  __syncthreads();

  // pass 2, dW stores and row sums (dg), one 16-row block b at a time (its
  // sums reduced before the next block starts, so few values stay live). A
  // full tile without accumulation stores 16 bytes per lane and tile with no
  // guards; the other copy guards every element.
  auto pass2 = [&](auto fast_tag) {
    constexpr bool kFast = decltype(fast_tag)::value;
#pragma unroll
    for (int b = 0; b < kBO; ++b) {
      const int ol = (kTO / 2) * wo + 16 * b + fr;
      const int o = o0 + ol;
      float rs[P];
#pragma unroll
      for (int p = 0; p < P; ++p) rs[p] = 0.f;
#pragma unroll
      for (int a = 0; a < 8; ++a) {
        const int il = 128 * wi + 16 * a + 4 * fg;
        const int i = i0 + il;
        float* d = dW + (size_t)o * in + i;
        if (kFast) {
          *(float4*)d = make_float4(acc[a][b][0], acc[a][b][1], acc[a][b][2], acc[a][b][3]);
        } else if (o < out) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (i + r < in) d[r] = accumulate ? d[r] + acc[a][b][r] : acc[a][b][r];
        }
#pragma unroll
        for (int p = 0; p < P; ++p) {
          const float4 hv = *(const float4*)&sH[p][il];
          const uint32_t word = sBitsW[p][wi][a >> 1][ol];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const uint32_t sgn = ((word >> ((16 * a + 4 * fg + r) & 31)) & 1u) << 31;
            rs[p] += acc[a][b][r] * __uint_as_float(__float_as_uint((&hv.x)[r]) ^ sgn);
          }
        }
      }
#pragma unroll
      for (int p = 0; p < P; ++p) {
        float v = rs[p];
        v += __shfl_xor(v, 16, 64);
        v += __shfl_xor(v, 32, 64);
        if (fg == 0) sRed[wi][p][ol] = v;
      }
    }
  };
  if ((in & 3) == 0 && i0 + kTI <= in && o0 + kTO <= out && !accumulate)
    pass2(std::true_type{});
  else
    pass2(std::false_type{});
  __syncthreads();
  for (int t = tid; t < P * kTO; t += 256) {
    const int p = t / kTO, r = t % kTO;
    ws.prow[((size_t)bx * P + p) * ((size_t)nby * kTO) + o0 + r] = sRed[0][p][r] + sRed[1][p][r];
  }
}

// dg[p][o] = Σ_bx prow[bx][p][o], dh[p][i] = Σ_by pcol[by][p][i], ascending
__global__ __launch_bounds__(256) void k_grad_reduce(GradWs ws, int out, int in, int P,
                                                     float* dg, float* dh, int accumulate) {
  const int nbx = (in + kTI - 1) / kTI, nby = (out + kTO - 1) / kTO;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  const int ng = P * out;
  if (idx < ng) {
    const int p = idx / out, o = idx % out;
    float v = 0.f;
    for (int b = 0; b < nbx; ++b) v += ws.prow[((size_t)b * P + p) * ((size_t)nby * kTO) + o];
    dg[idx] = accumulate ? dg[idx] + v : v;
  } else if (idx < ng + P * in) {
    const int k = idx - ng, p = k / in, i = k % in;
    float v = 0.f;
    for (int b = 0; b < nby; ++b) v += ws.pcol[((size_t)b * P + p) * ((size_t)nbx * kTI) + i];
    dh[k] = accumulate ? dh[k] + v : v;
  }
}

}  // namespace

size_t grad_weight_workspace_bytes(int out, int in, int P) { return grad_ws_bytes(out, in, P); }

size_t grad_input_workspace_bytes(int out, int in, int m, int P) {
  // transposed planes, then the prefill GEMM's workspace for the layer W_hatᵀ
  size_t planes_t = (size_t)row_groups(in) * col_groups(out) * P * 64 * 16;
  return a256(planes_t) + gemm_workspace_bytes(in, out, m);
}

hipError_t launch_transpose_planes(const uint4* planes, int out, int in, int P, uint4* planes_t,
                                   hipStream_t st) {
  const int slabs = row_groups(in) * col_groups(out) * P;
  hipLaunchKernelGGL(k_transpose_planes, dim3((slabs + 3) / 4), dim3(256), 0, st,
                     (const uint32_t*)planes, out, in, P, planes_t);
  return hipGetLastError();
}

hipError_t launch_grad_input(const uint4* planes, const uint16_t* g, const uint16_t* h, int out,
                             int in, int P, const uint16_t* dY, int m, void* dX, int dx_dtype,
                             void* ws, hipStream_t st, bool weff) {
  uint4* pt = (uint4*)ws;
  const size_t planes_t = (size_t)row_groups(in) * col_groups(out) * P * 64 * 16;
  hipError_t e = launch_transpose_planes(planes, out, in, P, pt, st);
  if (e != hipSuccess) return e;
  // W_hatᵀ: out' = in, in' = out, output scales h, input scales g
  return launch_gemm(pt, h, g, in, out, dY, m, dX, dx_dtype, (char*)ws + a256(planes_t), st, P, weff);
}

hipError_t launch_grad_weight(const uint4* planes, const uint16_t* g, const uint16_t* h, int out,
                              int in, int P, const uint16_t* X, const uint16_t* dY, int m, float* dW,
                              float* dg, float* dh, int accumulate, void* ws, hipStream_t st) {
  GradWs w = carve_grad(ws, out, in, P);
  const int tiles = ((out + kTO - 1) / kTO) * ((in + kTI - 1) / kTI);
  // the ring loader moves 16-byte chunks of token rows (X and dY themselves
  // are 16-byte aligned at the boundary)
  const bool ring = in % 8 == 0 && out % 8 == 0;
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(tiles), dim3(256), 0, st, X, dY, m, out, in, (const uint32_t*)planes, g,
                       h, dW, accumulate, w);
  };
  if (P == 3)
    ring ? go(k_grad_w<3, true>) : go(k_grad_w<3, false>);
  else
    ring ? go(k_grad_w<2, true>) : go(k_grad_w<2, false>);
  const int n = P * (out + in);
  hipLaunchKernelGGL(k_grad_reduce, dim3((n + 255) / 256), dim3(256), 0, st, w, out, in, P, dg, dh,
                     accumulate);
  return hipGetLastError();
}

}  // namespace rabit
