// Decode GEMV on packed planes: y = Σ_p g_p ⊙ (B_p (h_p ⊙ x)).
//
// RaBiT paper App. E.1 describes a CUDA GEMV that expands sign bits with
// shifts/XOR into fp16 FMAs and notes that the limit moves toward register
// throughput. On gfx950 the ±1 contraction runs on the matrix cores, with the
// plane bits used directly as fp4 operands:
//
//  * Σ_j s_j u_j = Σ_j u_j − 2 Σ_{bit_j = 1} u_j with s_j = 1 − 2 bit_j and
//    u = h_p ⊙ x (paper §5.4: additions and element-wise scaling).
//  * The input columns are cut into K ranges of 512 (one "chunk"). Per
//    (batch row, path, range), u is formed exactly (float64) and held as a
//    fixed-point integer v = rint(u · 2^sh), sh chosen so that the range's
//    largest |u| maps into [2^18, 2^19); v + 2^20 is written in 7 base-8
//    digits 0..7.
//  * A stored word w (32 columns of one row, bit t of nibble e = column
//    4e + t) gives four fp4 slices with one VALU op each: w & 0x1..1 (value
//    0.5 per set bit), w & 0x2..2 (1.0), w & 0x4..4 (2.0) and
//    (w & 0x8..8) | 0x1..1 (+0.5 for a clear bit, -0.5 for a set one).
//  * V_MFMA_SCALE_F32_16X16X128_F8F6F4 multiplies one slice (16 rows x 128
//    columns, fp4) by an fp6 e2m3 operand whose rows are the digits: codes
//    2d, d, d and -d (values d/4, d/8, d/8, -d/8; e2m3 codes below 16 are
//    linear), with the per-row E8M0 operand scale 2^(3 (digit + 1)) (halved
//    for the 2.0 slice), so a set bit in column j adds 8^k d_k(j) to row k.
//    The fourth slice's constant part (-d/16 per column) is removed exactly
//    by starting the accumulators from one product against all -0.5. One
//    extra row of ones yields the set-bit count. Every fp32 partial sum is an
//    exact multiple of a power of two with few significant bits, so Σ bit·v
//    is recovered exactly as an integer.
//  * Each workgroup builds the digit operand of its own range in LDS from x
//    and h (no separate activation pass), then its 4 waves stream 64-row
//    groups of planes through the matrix cores (one 8 KiB slab per wave and
//    row group, prefetched one row group ahead).
//  * Per range, g_1 S_1 + g_2 S_2 is formed in float64 from exact integers;
//    the ranges' partials are summed in a fixed order by the consumer (a
//    small reduce kernel, or the fused op that follows the layer), so the
//    output is bitwise repeatable. No atomics, no fences.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "rabit_internal.h"

namespace rabit {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kChunk = 512;                    // columns per K range
constexpr int kImgDw = 6;                      // dwords per lane of one fp6 image (32 x 6 bits)
constexpr int kImgDwords = 64 * kImgDw;        // one (path, slice) image
// P paths x 4 slices, one batch pair (12 KiB with two paths)
template <int P>
constexpr int kPairDwords = P * 4 * kImgDwords;
constexpr int kFxTop = 18;                     // max |v| of a range in [2^18, 2^19]
constexpr int kOff = 1 << 20;                  // v + kOff in [0, 2^21): 7 digits of base 8
constexpr int kNoExp = -100000;                // exponent of an all-zero range
constexpr int kStatParts = RABIT_STAT_PARTS;   // partial sums of x^2 per row (RMSNorm input)

// One matrix of a launch. All segments of a launch share the input x (and so
// in_features); their row blocks are numbered consecutively.
struct Seg {
  const uint4* planes;
  const uint16_t* g;
  const uint16_t* h;
  double* part;  // partials [batch][S][RG*64]
  int out, RG, rb0;
};

constexpr int kMaxSeg = 3;

struct Args {
  Seg seg[kMaxSeg];
  const uint16_t* x;      // bf16 [batch][in]
  const double* stats;    // norm mode: [batch][kStatParts] partial sums of x^2
  int nseg, in, KG, S, m, batch, norm;
  int items, ngrp;        // work items (row block, range); batch groups along x
  float eps;
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

constexpr int kMaxRounds = 8;   // row groups per wave and launch
constexpr int kMaxDevices = 64;

struct Plan {
  int KG, S, m, paths;
  int RB[kMaxSeg];    // row blocks per segment (4 m row groups each)
};


__host__ inline size_t part_bytes(int out, int S, int batch) {
  return align256((size_t)batch * S * row_groups(out) * 64 * sizeof(double));
}

// 6 dwords of 32 fp6 fields, every field = code
__device__ __forceinline__ void fill_code(uint32_t (&dw)[kImgDw], uint32_t code) {
#pragma unroll
  for (int d = 0; d < kImgDw; ++d) dw[d] = 0;
#pragma unroll
  for (int x = 0; x < 32; ++x) {
    const int bit = 6 * x;
    dw[bit >> 5] |= code << (bit & 31);
    if ((bit & 31) > 26) dw[(bit >> 5) + 1] |= code >> (32 - (bit & 31));
  }
}

// digit row: field x = digit `dig` of src[x] (code d, value d/8); the 32
// values are read from LDS in two halves to bound the live registers
__device__ __forceinline__ void deposit_digits(uint32_t (&dw)[kImgDw], const int* src, int dig) {
#pragma unroll
  for (int d = 0; d < kImgDw; ++d) dw[d] = 0;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    int vals[16];
#pragma unroll
    for (int x = 0; x < 16; x += 4) {
      const int4 v4 = *(const int4*)(src + 16 * half + x);
      vals[x] = v4.x;
      vals[x + 1] = v4.y;
      vals[x + 2] = v4.z;
      vals[x + 3] = v4.w;
    }
#pragma unroll
    for (int xx = 0; xx < 16; ++xx) {
      const int x = 16 * half + xx;
      const uint32_t f = __builtin_amdgcn_ubfe((uint32_t)vals[xx], 3 * dig, 3);
      const int bit = 6 * x;
      dw[bit >> 5] |= f << (bit & 31);
      if ((bit & 31) > 29) dw[(bit >> 5) + 1] |= f >> (32 - (bit & 31));
    }
  }
}

// Workgroup: 4 waves; segment/row block rbg, K range r (512 columns), batch
// pairs [NBP grp, NBP grp + NBP). Every launch uses NBP = 1: a workgroup that
// carries several pairs shares one weight load among them, but needs more
// registers (fewer resident waves) and was measured slower than one-pair
// workgroups that share the weights through L2. Round k: wave w takes row
// group 4 m rb + 4 k + w. Lane l = j + 16 g loads, per tile tau and path p,
// the 16-byte unit (rg, 4 r + g, p, 16 tau + j): 128 columns of row
// 16 tau + j, bit 4e + t of dword q being column 32 q + 4 e + t of the group.
template <int NBP, bool RING, bool GROUPED, int P>
__global__ __launch_bounds__(256) void k_gemv(Args A) {
  // Work item (row block, range) and batch group of this workgroup. With
  // several batch groups (GROUPED), the groups of one item are adjacent in
  // launch order and share blockIdx.x % 8 (workgroups are dealt to the 8 XCDs
  // in launch order), so that the item's weights come from HBM once and from
  // that XCD's L2 for the other groups.
  int wid = blockIdx.x, grp = 0;
  if (GROUPED) {
    const int hi = blockIdx.x >> 3;
    grp = hi % A.ngrp;
    wid = (hi / A.ngrp) * 8 + (blockIdx.x & 7);
    if (wid >= A.items) return;
  }
  const int r = wid % A.S;
  const int rbg = wid / A.S;
  // segment of this row block (uniform selects, no indexing of the arguments)
  const int si = (A.nseg > 2 && rbg >= A.seg[2].rb0) ? 2 : (A.nseg > 1 && rbg >= A.seg[1].rb0) ? 1 : 0;
  const uint4* planes = si == 2 ? A.seg[2].planes : si == 1 ? A.seg[1].planes : A.seg[0].planes;
  const uint16_t* gsc = si == 2 ? A.seg[2].g : si == 1 ? A.seg[1].g : A.seg[0].g;
  const uint16_t* hsc = si == 2 ? A.seg[2].h : si == 1 ? A.seg[1].h : A.seg[0].h;
  double* part = si == 2 ? A.seg[2].part : si == 1 ? A.seg[1].part : A.seg[0].part;
  const int out = si == 2 ? A.seg[2].out : si == 1 ? A.seg[1].out : A.seg[0].out;
  const int RG = si == 2 ? A.seg[2].RG : si == 1 ? A.seg[1].RG : A.seg[0].RG;
  const int rb = rbg - (si == 2 ? A.seg[2].rb0 : si == 1 ? A.seg[1].rb0 : A.seg[0].rb0);

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;
  const int j = l & 15, gl = l >> 4;
  const int bp0 = grp * NBP;
  const int in = A.in, batch = A.batch, m = A.m;
  const int col0 = r * kChunk;

  // weights of round k (clamped row group: loads stay in bounds, results unused)
  // and the row scales g_p of this lane's 4 output rows
  auto load_round = [&](uint4 (&wt)[4 * P], uint16_t (&gt)[4 * P], int k) {
    const int rg = min(RG - 1, 4 * m * rb + 4 * k + w);
    const int kg = min(A.KG - 1, 4 * r + gl);
#pragma unroll
    for (int tau = 0; tau < 4; ++tau)
#pragma unroll
      for (int p = 0; p < P; ++p) wt[tau * P + p] = load_nt(planes + unit_index(rg, kg, p, 16 * tau + j, A.KG, P));
#pragma unroll
    for (int tau = 0; tau < 4; ++tau)
#pragma unroll
      for (int p = 0; p < P; ++p) gt[tau * P + p] = gsc[(size_t)p * out + min(rg * 64 + 16 * tau + j, out - 1)];
  };

  __shared__ __align__(16) uint32_t s_img[NBP * kPairDwords<P>];
  __shared__ __align__(16) int s_v[2][P][kChunk];     // [hb][p][t*128 + g*32 + x] = v + kOff
  __shared__ int s_ex[4][2][P];         // per wave [hb][p]
  __shared__ int s_sum[4][2][P];
  __shared__ int s_sh[NBP][2][P];
  __shared__ int s_U[NBP][2][P];

  // ---- digit operand of this range, pair by pair ---------------------------
  // element e = tid + 256 k (k = 0, 1) of the range: column col0 + e
  // loads are unconditional (clamped indices) and masked afterwards, so that
  // no branch separates them and they are all in flight together
  uint16_t hv[P][2], xv[NBP][2][2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int col = col0 + tid + 256 * k;
    const int cc = min(col, in - 1);
#pragma unroll
    for (int p = 0; p < P; ++p) hv[p][k] = hsc[(size_t)p * in + cc];
#pragma unroll
    for (int q = 0; q < NBP; ++q)
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const int b = 2 * (bp0 + q) + hb;
        xv[q][hb][k] = A.x[(size_t)min(b, batch - 1) * in + cc];
      }
  }
  // RMSNorm input: lane l < kStatParts holds partial sum l of x^2 of each
  // batch row (added by a fixed DPP tree below)
  double stp[NBP][2];
  if (A.norm) {
#pragma unroll
    for (int q = 0; q < NBP; ++q)
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
        stp[q][hb] = A.stats[(size_t)min(2 * (bp0 + q) + hb, batch - 1) * kStatParts + (l & (kStatParts - 1))];
  }
  // the first round's weights are issued after x and h: waiting for those
  // (loads complete in order) then does not wait for the weights
  uint4 w0[4 * P], w1[4 * P];
  uint16_t g0[4 * P], g1[4 * P];
  __builtin_amdgcn_sched_barrier(0);
  load_round(w0, g0, 0);
  __builtin_amdgcn_sched_barrier(0);  // keep every load above the first use of x and h
  if (A.norm) {
    // x <- bf16(x / sqrt(mean(x^2) + eps)), the partial sums added in order
#pragma unroll
    for (int q = 0; q < NBP; ++q)
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const double ss = wave_sum_f64(l < kStatParts ? stp[q][hb] : 0.0);
        const double den = sqrt(ss / (double)in + (double)A.eps);
#pragma unroll
        for (int k = 0; k < 2; ++k) xv[q][hb][k] = f64_to_bf16_rne_fast((double)bf16_bits_to_f32(xv[q][hb][k]) / den);
      }
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const bool ok = col0 + tid + 256 * k < in;
#pragma unroll
    for (int p = 0; p < P; ++p) hv[p][k] = ok ? hv[p][k] : (uint16_t)0;
#pragma unroll
    for (int q = 0; q < NBP; ++q)
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
        xv[q][hb][k] = (ok && 2 * (bp0 + q) + hb < batch) ? xv[q][hb][k] : (uint16_t)0;
  }

#pragma unroll
  for (int q = 0; q < NBP; ++q) {
    // which rows of this pair exist (uniform); absent rows get zero operands
    const bool live0 = 2 * (bp0 + q) < batch, live1 = 2 * (bp0 + q) + 1 < batch;
    // range exponent: the largest binary exponent of a nonzero |u| (frexp:
    // |u| = f 2^e, f in [1/2, 1)), so that max |u| 2^sh lies in [2^18, 2^19)
    double u[2][P][2];
    int ex[2][P];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int p = 0; p < P; ++p) {
        ex[hb][p] = kNoExp;
        if (hb == 1 && !live1) continue;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          u[hb][p][k] = (double)f16_bits_to_f32(hv[p][k]) * (double)bf16_bits_to_f32(xv[q][hb][k]);
          int e;
          frexp(u[hb][p][k], &e);
          ex[hb][p] = max(ex[hb][p], u[hb][p][k] != 0.0 ? e : kNoExp);
        }
        ex[hb][p] = wave_max_i32(ex[hb][p]);
      }
    if (l == 0)
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int p = 0; p < P; ++p) s_ex[w][hb][p] = ex[hb][p];
    __syncthreads();
    int sh[2][P];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const int E = max(max(s_ex[0][hb][p], s_ex[1][hb][p]), max(s_ex[2][hb][p], s_ex[3][hb][p]));
        sh[hb][p] = E == kNoExp ? 0 : kFxTop + 1 - E;
        if (hb == 1 && !live1) continue;
        int su = 0;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int v = (int)rint(ldexp(u[hb][p][k], sh[hb][p]));
          su += v;
          const int e = tid + 256 * k;
          const int t = e & 3, g = e >> 7, x = 8 * ((e >> 5) & 3) + ((e >> 2) & 7);
          s_v[hb][p][t * 128 + g * 32 + x] = v + kOff;
        }
        su = wave_sum_i32(su);
        if (l == 0) s_sum[w][hb][p] = su;
      }
    __syncthreads();
    if (tid < 2 * P) {
      const int hb = tid / P, p = tid % P;
      // same value as sh[hb][p], selected without indexing a register array
      int shs = 0;
#pragma unroll
      for (int hb2 = 0; hb2 < 2; ++hb2)
#pragma unroll
        for (int p2 = 0; p2 < P; ++p2) shs = (hb2 == hb && p2 == p) ? sh[hb2][p2] : shs;
      const bool lv = hb ? live1 : live0;
      s_sh[q][hb][p] = shs;
      s_U[q][hb][p] = lv ? ((s_sum[0][hb][p] + s_sum[1][hb][p]) + s_sum[2][hb][p]) + s_sum[3][hb][p] : 0;
    }
    // image rows: wave w builds slice t = w, row unit u = (p, g, dr) the row
    // L = 8 hb + dr + 16 g of image (p, t) for each batch row hb of the pair;
    // the 32 P units of a slice take the wave's 64 lanes once (two paths) or
    // twice (three)
#pragma unroll
    for (int u0 = 0; u0 < 32 * P; u0 += 64) {
      const int uu = u0 + l;
      if (uu >= 32 * P) break;
      const int t = w, p = uu >> 5, g = (uu >> 3) & 3, dr = uu & 7;
      const bool dbl = t == 0;  // slice of value 0.5: code 2d
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const bool lv = hb ? live1 : live0;
        uint32_t* dst = s_img + q * kPairDwords<P> + (p * 4 + t) * kImgDwords + (8 * hb + dr + 16 * g) * kImgDw;
        if (!lv) {
#pragma unroll
          for (int d = 0; d < kImgDw; d += 2) *(uint2*)(dst + d) = make_uint2(0u, 0u);
          continue;
        }
        const int* src = &s_v[hb][p][t * 128 + g * 32];
        uint32_t dw[kImgDw];
        deposit_digits(dw, src, dr);
        if (dr == 7) fill_code(dw, 1u);  // row of ones: set-bit count
        if (dbl) {
          // codes 2d: shift the lane's 192-bit field vector left by one (each
          // digit sits in the low 3 bits of its 6-bit field, so none crosses)
#pragma unroll
          for (int d = kImgDw - 1; d > 0; --d) dw[d] = (dw[d] << 1) | (dw[d - 1] >> 31);
          dw[0] <<= 1;
        } else if (t == 3) {
          // sign bit in every field: values -d/8 against the +-0.5 slice
          uint32_t sg[kImgDw];
          fill_code(sg, 32u);
#pragma unroll
          for (int d = 0; d < kImgDw; ++d) dw[d] |= sg[d];
        }
#pragma unroll
        for (int d = 0; d < kImgDw; d += 2) *(uint2*)(dst + d) = make_uint2(dw[d], dw[d + 1]);
      }
    }
    __syncthreads();
  }

  // ---- stream the planes -----------------------------------------------------
  // C lane l, reg k = row i = 4 gl + k of the digit operand (digit i % 8 of
  // batch row 2 q + i / 8; i % 8 == 7 is the ones row), column j = row 16 tau + j.
  // Row i of the digit operand carries the E8M0 scale 2^(3 (i % 8 + 1)) for
  // digit rows (lane i + 16 g supplies the scale of row i, K block g) and
  // 2^0 for the ones row, so accumulator rows are 8^d D_d (D_d = Σ bit·digit_d,
  // an integer) and P/8 (P = set-bit count). In fp32, exactly: lanes gl even
  // hold digits 0..3 (sum below 2^22), lanes gl odd digits 4..6 and the count
  // term -kOff P (multiples of 4096 in (-2^30, 2^30)); with the partner lane
  // (l + 16) they give Σ bit·v exactly.
  const int hbl = gl >> 1;
  const int arow = l & 7;  // digit of operand row l & 15 (7: the ones row)
  const int ascale = arow == 7 ? 127 : 127 + 3 * (arow + 1);
  const float kc3 = (gl & 1) ? -8.f * kOff : 1.f;
  // this lane's row of image (pair q, path/slice ps)
  auto image_row = [&](int q, int ps) -> v8i {
    const uint32_t* s = s_img + q * kPairDwords<P> + ps * kImgDwords + l * kImgDw;
    const uint2 a0 = *(const uint2*)(s), a1 = *(const uint2*)(s + 2), a2 = *(const uint2*)(s + 4);
    return (v8i){(int)a0.x, (int)a0.y, (int)a1.x, (int)a1.y, (int)a2.x, (int)a2.y, 0, 0};
  };
  // with one batch pair and two paths the 8 operand rows of this lane stay in
  // registers (with the ring); without it they are read from LDS per use,
  // which frees 48 registers for more resident waves
  constexpr bool kAreg = NBP == 1 && RING && P == 2;
  v8i areg[kAreg ? 8 : 1];
#pragma unroll
  for (int ps = 0; ps < (kAreg ? 8 : 1); ++ps) areg[ps] = kAreg ? image_row(0, ps) : (v8i){};

  // Slice 3 is read as (0.5 - bit) against digits coded -d/8, which adds a
  // constant -(1/16) Σ d per operand row over the chunk's slice-3 columns; the
  // accumulators start from that constant's negation, computed exactly by one
  // matrix op against an all -0.5 operand (fp4 code 0b1001).
  v4f ainit[NBP][P];
#pragma unroll
  for (int q = 0; q < NBP; ++q)
#pragma unroll
    for (int p = 0; p < P; ++p)
      ainit[q][p] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
          kAreg ? areg[(p * 4 + 3) % (kAreg ? 8 : 1)] : image_row(q, p * 4 + 3),
          (v8i){(int)0x99999999u, (int)0x99999999u, (int)0x99999999u, (int)0x99999999u, 0, 0, 0, 0},
          (v4f){0.f, 0.f, 0.f, 0.f}, 2, 4, 0, ascale, 0, 127);

  // one round: row group 4 m rb + 4 k + w from the weights in wt
  auto round = [&](const uint4 (&wt)[4 * P], const uint16_t (&gt)[4 * P], int k) {
    const int rg = 4 * m * rb + 4 * k + w;
    // per lane and path: this lane's exact share of Σ bit·v (see above)
    int mv[NBP][P][4];
#pragma unroll
    for (int p = 0; p < P; ++p) {
      v4f acc[NBP][4];
#pragma unroll
      for (int q = 0; q < NBP; ++q)
#pragma unroll
        for (int tau = 0; tau < 4; ++tau) acc[q][tau] = ainit[q][p];
      // slice T of a stored word (see the header comment)
      auto slice_step = [&](auto tc) {
        constexpr int T = decltype(tc)::value;
        // T0: w & 0x1..1 (0.5), T1: w & 0x2..2 (1.0), T2: w & 0x4..4 (2.0, the
        // operand scale halved), T3: (w & 0x8..8) | 0x1..1 (+0.5 or -0.5)
        constexpr uint32_t mT = T == 0 ? 0x11111111u : T == 1 ? 0x22222222u : T == 2 ? 0x44444444u : 0x88888888u;
        constexpr uint32_t oT = T == 3 ? 0x11111111u : 0u;
        const int sc = T == 2 ? ascale - 1 : ascale;
        v8i a[NBP];
#pragma unroll
        for (int q = 0; q < NBP; ++q) a[q] = kAreg ? areg[(p * 4 + T) % (kAreg ? 8 : 1)] : image_row(q, p * 4 + T);
#pragma unroll
        for (int tau = 0; tau < 4; ++tau) {
          const uint4 wv = wt[tau * P + p];
          const v8i bv = (v8i){(int)((wv.x & mT) | oT), (int)((wv.y & mT) | oT),
                               (int)((wv.z & mT) | oT), (int)((wv.w & mT) | oT), 0, 0, 0, 0};
#pragma unroll
          for (int q = 0; q < NBP; ++q)
            acc[q][tau] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                a[q], bv, acc[q][tau], 2 /*A: fp6 e2m3*/, 4 /*B: fp4 e2m1*/, 0, sc, 0, 127);
        }
      };
      slice_step(std::integral_constant<int, 0>());
      slice_step(std::integral_constant<int, 1>());
      slice_step(std::integral_constant<int, 2>());
      slice_step(std::integral_constant<int, 3>());

#pragma unroll
      for (int q = 0; q < NBP; ++q)
#pragma unroll
        for (int tau = 0; tau < 4; ++tau) {
          const v4f c = acc[q][tau];
          mv[q][p][tau] = (int)__builtin_fmaf(c[3], kc3, (c[0] + c[1]) + c[2]);
        }
    }

    // lanes of rows 0 and 2 (gl even) add the share of the lane 16 above
    // (a VALU row swap) and form Σ_p g_p S_p in float64 (each product exact,
    // paths added in order)
    double res[NBP][4];
#pragma unroll
    for (int q = 0; q < NBP; ++q) {
      int shp[P], Up[P];
#pragma unroll
      for (int p = 0; p < P; ++p) {
        shp[p] = s_sh[q][hbl][p];
        Up[p] = s_U[q][hbl][p];
      }
#pragma unroll
      for (int tau = 0; tau < 4; ++tau) {
        double acc = 0.0;
#pragma unroll
        for (int p = 0; p < P; ++p) {
          const int mp = mv[q][p][tau] + (int)__builtin_amdgcn_permlane16_swap(mv[q][p][tau], mv[q][p][tau], false, false)[1];
          const double gp = ldexp((double)f16_bits_to_f32(gt[tau * P + p]), -shp[p]);
          acc = p == 0 ? gp * (double)(Up[p] - 2 * mp) : acc + gp * (double)(Up[p] - 2 * mp);
        }
        res[q][tau] = acc;
      }
    }

    if (rg < RG && (gl & 1) == 0) {
#pragma unroll
      for (int q = 0; q < NBP; ++q) {
        const int b = 2 * (bp0 + q) + hbl;
        if (b >= batch) continue;
#pragma unroll
        for (int tau = 0; tau < 4; ++tau) {
          const int row = rg * 64 + 16 * tau + j;
          if (row >= out) continue;
            part[((size_t)b * A.S + r) * RG * 64 + row] = res[q][tau];
        }
      }
    }
  };

  // rounds in pairs, so that each ring buffer is a fixed register array
#pragma unroll 1
  for (int k = 0; k < m; k += 2) {
    if (!RING) {
      // one buffer: the next round's weights are loaded after this round
      // (fewer registers, more resident waves to cover the latency)
      round(w0, g0, k);
      if (k + 1 < m) {
        load_round(w0, g0, k + 1);
        round(w0, g0, k + 1);
        if (k + 2 < m) load_round(w0, g0, k + 2);
      }
      continue;
    }
    if (k + 1 < m) load_round(w1, g1, k + 1);
    round(w0, g0, k);
    if (k + 1 < m) {
      if (k + 2 < m) load_round(w0, g0, k + 2);
      round(w1, g1, k + 1);
    }
  }
}

// y = Σ_r part (ascending r)
__global__ __launch_bounds__(256) void k_gemv_reduce(const double* __restrict__ part, int out,
                                                     int RG, int S, void* y, int y_dtype) {
  const int row = blockIdx.x * 256 + threadIdx.x, b = blockIdx.y;
  if (row >= out) return;
  // many ranges (wide layers): 32 loads in flight per round trip
  const double* pp = part + (size_t)b * S * RG * 64 + row;
  const double v = S <= 8 ? sum_ranges_by<8>(pp, S, RG * 64) : sum_ranges_by<32>(pp, S, RG * 64);
  if (y_dtype == RABIT_OUT_F32)
    ((float*)y)[(size_t)b * out + row] = (float)v;
  else
    ((uint16_t*)y)[(size_t)b * out + row] = f64_to_bf16_rne(v);
}

// Workgroups of one variant that fit on the device at once (occupancy from
// the runtime, queried once per device and variant).
int resident_wgs(bool ring, int paths) {
  static std::atomic<int> cache[kMaxDevices][2][2];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
  std::atomic<int>& slot = cache[dev][ring ? 1 : 0][paths == 3 ? 1 : 0];
  int c = slot.load(std::memory_order_relaxed);
  if (c == 0) {
    int cus = 0, per = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
      cus = 256;
    const void* fn = paths == 3
        ? (ring ? (const void*)k_gemv<1, true, false, 3> : (const void*)k_gemv<1, false, false, 3>)
        : (ring ? (const void*)k_gemv<1, true, false, 2> : (const void*)k_gemv<1, false, false, 2>);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, fn, 256, 0) != hipSuccess || per < 1) per = 1;
    c = cus * per;
    slot.store(c, std::memory_order_relaxed);
  }
  return c;
}

// Rows per workgroup (4 m row groups). A workgroup builds the digit operand
// of its range once and then streams m row groups. With one batch pair and
// m > 1 the next round's weights are in flight during a round, so all
// workgroups of a launch should be resident together: a second pass of a few
// workgroups runs its m rounds with most of the device idle. Cost model:
// passes x (m rounds + one for the digit build), ties to the smaller m (more
// workgroups). With more batch pairs (one buffer, rounds not overlapped) the
// rounds stay short: enough workgroups to fill the device a few times over.
__host__ inline Plan make_plan(const int* outs, int nseg, int in, int batch, int paths) {
  Plan P;
  P.paths = paths;
  P.KG = col_groups(in);
  P.S = (in + kChunk - 1) / kChunk;
  const int groups = (batch + 1) / 2;  // one batch pair per workgroup
  long best = -1;
  P.m = 1;
  for (int m = 1; m <= kMaxRounds; ++m) {
    long wgs = 0;
    for (int s = 0; s < nseg; ++s) wgs += (row_groups(outs[s]) + 4 * m - 1) / (4 * m);
    wgs *= (long)P.S * groups;
    const long cap = resident_wgs(m > 1, paths);
    const long cost = (wgs + cap - 1) / cap * (m + 1);
    if (best < 0 || cost < best) {
      best = cost;
      P.m = m;
    }
  }
  for (int s = 0; s < nseg; ++s) P.RB[s] = (row_groups(outs[s]) + 4 * P.m - 1) / (4 * P.m);
  return P;
}

hipError_t launch_main(const Plan& P, const Args& A, int batch, hipStream_t st) {
  int nrb = 0;
  for (int s = 0; s < A.nseg; ++s) nrb += P.RB[s];
  const int groups = (batch + 1) / 2;
  const dim3 grid(groups > 1 ? (nrb * P.S + 7) / 8 * 8 * groups : nrb * P.S);
  Args B = A;
  B.items = nrb * P.S;
  B.ngrp = groups;
  auto go = [&](auto paths_tag) {
    constexpr int NP = decltype(paths_tag)::value;
    if (groups > 1) {
      if (A.m > 1)
        hipLaunchKernelGGL((k_gemv<1, true, true, NP>), grid, dim3(256), 0, st, B);
      else
        hipLaunchKernelGGL((k_gemv<1, false, true, NP>), grid, dim3(256), 0, st, B);
    } else {
      if (A.m > 1)
        hipLaunchKernelGGL((k_gemv<1, true, false, NP>), grid, dim3(256), 0, st, B);
      else
        hipLaunchKernelGGL((k_gemv<1, false, false, NP>), grid, dim3(256), 0, st, B);
    }
  };
  if (P.paths == 3)
    go(std::integral_constant<int, 3>());
  else
    go(std::integral_constant<int, 2>());
  return hipGetLastError();
}

Args make_args(const Plan& P, const uint4* planes, const uint16_t* g, const uint16_t* h, int out,
               int in, const uint16_t* x, int batch, void* ws) {
  Args A = {};
  A.seg[0].planes = planes;
  A.seg[0].g = g;
  A.seg[0].h = h;
  A.seg[0].part = (double*)ws;
  A.seg[0].out = out;
  A.seg[0].RG = row_groups(out);
  A.seg[0].rb0 = 0;
  A.x = x;
  A.nseg = 1;
  A.in = in;
  A.KG = P.KG;
  A.S = P.S;
  A.m = P.m;
  A.batch = batch;
  A.norm = 0;
  A.stats = nullptr;
  A.eps = 0.f;
  return A;
}

}  // namespace

size_t gemv_workspace_bytes(int out, int in, int batch) {
  const int S = (in + kChunk - 1) / kChunk;
  return part_bytes(out, S, batch);
}

hipError_t launch_gemv_partial(const uint4* planes, const uint16_t* g, const uint16_t* h, int out,
                               int in, const uint16_t* x, int batch, void* ws, hipStream_t st,
                               int paths) {
  if (paths != 2 && paths != 3) return hipErrorInvalidValue;
  const Plan P = make_plan(&out, 1, in, batch, paths);
  const Args A = make_args(P, planes, g, h, out, in, x, batch, ws);
  return launch_main(P, A, batch, st);
}

hipError_t launch_gemv_reduce(int out, int in, int batch, void* y, int y_dtype, const void* ws,
                              hipStream_t st) {
  const int S = (in + kChunk - 1) / kChunk;
  hipLaunchKernelGGL(k_gemv_reduce, dim3((out + 255) / 256, batch), dim3(256), 0, st,
                     (const double*)ws, out, row_groups(out), S, y, y_dtype);
  return hipGetLastError();
}

size_t gemv_part_bytes(int out, int in, int batch) {
  return part_bytes(out, (in + kChunk - 1) / kChunk, batch);
}

hipError_t launch_gemv_multi(const LinSeg* segs, int nseg, int in, const uint16_t* x, int batch,
                             const double* stats, float eps, hipStream_t st) {
  if (nseg < 1 || nseg > kMaxSeg) return hipErrorInvalidValue;
  int outs[kMaxSeg];
  for (int s = 0; s < nseg; ++s) {
    outs[s] = segs[s].out;
    if (segs[s].paths != segs[0].paths) return hipErrorInvalidValue;
  }
  if (segs[0].paths != 2 && segs[0].paths != 3) return hipErrorInvalidValue;
  const Plan P = make_plan(outs, nseg, in, batch, segs[0].paths);
  Args A = {};
  int rb0 = 0;
  for (int s = 0; s < nseg; ++s) {
    A.seg[s].planes = segs[s].planes;
    A.seg[s].g = segs[s].g;
    A.seg[s].h = segs[s].h;
    A.seg[s].part = segs[s].part;
    A.seg[s].out = segs[s].out;
    A.seg[s].RG = row_groups(segs[s].out);
    A.seg[s].rb0 = rb0;
    rb0 += P.RB[s];
  }
  A.x = x;
  A.stats = stats;
  A.nseg = nseg;
  A.in = in;
  A.KG = P.KG;
  A.S = P.S;
  A.m = P.m;
  A.batch = batch;
  A.norm = stats ? 1 : 0;
  A.eps = eps;
  return launch_main(P, A, batch, st);
}

hipError_t launch_gemv(const uint4* planes, const uint16_t* g, const uint16_t* h, int out, int in,
                       const uint16_t* x, int batch, void* y, int y_dtype, void* ws,
                       hipStream_t st, int paths) {
  hipError_t e = launch_gemv_partial(planes, g, h, out, in, x, batch, ws, st, paths);
  if (e != hipSuccess) return e;
  return launch_gemv_reduce(out, in, batch, y, y_dtype, ws, st);
}

}  // namespace rabit
