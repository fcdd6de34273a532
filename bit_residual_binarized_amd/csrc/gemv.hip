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
//  * Per range, g_1 S_1 + g_2 S_2 is formed in float64 from exact integers
//    and stored as one float32 partial (half the bytes of a float64 one for
//    the launch that reads it next); the ranges' partials are summed in
//    float64 in a fixed order by the consumer (a small reduce kernel, the op
//    that follows the layer, or the next GEMV forming its input), so the
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
  double* part;  // partial buffer: header (slice count), then [batch][slices][RG*64]
  uint32_t* hp;  // fp16 path: the matrix's h pairs in the contraction order
  int out, RG, rb0;
};

constexpr int kMaxSeg = 3;

struct Args {
  Seg seg[kMaxSeg];
  const uint16_t* x;      // bf16 [batch][in]
  const double* stats;    // norm mode: [batch][kStatParts] partial sums of x^2
  int nseg, in, KG, S, m, batch, norm;
  int items, ngrp;        // work items (row block, range); batch groups along x
  int kr, nck;            // fp16 path: ranges per chunk, chunks per row block
  uint16_t* xh;           // fp16 path: prepared x [batch][Kp] (contraction order)
  int* rowexp;            // fp16 path: per token, the power of two applied to x
  float eps;
  GemvXSrc xs;            // digit path: input formed from partial buffers
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

constexpr int kMaxRounds = 8;   // row groups per wave and launch
constexpr int kMaxDevices = 64;

struct Plan {
  int KG, S, m, paths;
  int RB[kMaxSeg];    // row blocks per segment (4 m row groups each)
};


__host__ inline size_t part_bytes(int out, int S, int batch) {
  return kPartHdrDoubles * sizeof(double) + align256((size_t)batch * S * row_groups(out) * 64 * sizeof(float));
}

// fp16 path (batches from RABIT_GEMV_FP16_MIN_BATCH on): after each matrix's
// partial buffer, the launch's prepared x (used in the first matrix's area),
// the per-token exponents and the matrix's h pairs (up to 3 paths).
// The prepared rows span whole ranges, S = ceil(in / 512) of them, zero past
// in: a range's columns past in meet zeros there, whatever weights the
// clamped plane loads bring.
__host__ inline int f16_cols(int in) { return (in + kChunk - 1) / kChunk * kChunk; }
__host__ inline size_t xh_bytes(int in) { return align256((size_t)RABIT_MAX_GEMV_BATCH * f16_cols(in) * 2); }
constexpr size_t kRowExpBytes = 256;
__host__ inline size_t hp_bytes(int in) { return align256((size_t)3 * (f16_cols(in) / 32) * 64); }
__host__ inline size_t prep_bytes(int in) { return xh_bytes(in) + kRowExpBytes + hp_bytes(in); }

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
template <int NBP, bool RING, bool GROUPED, int P, int XM = XSRC_X>
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
  if (blockIdx.x == 0 && threadIdx.x < A.nseg) {
    // the partial buffers' headers: one slice per range
    double* hp = threadIdx.x == 2 ? A.seg[2].part : threadIdx.x == 1 ? A.seg[1].part : A.seg[0].part;
    ((int*)hp)[0] = A.S;
  }
  part += kPartHdrDoubles;

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

  // ---- input formed from the previous launch's partials (batch 1) ----------
  // Their loads go out first, ahead of h and the weights, so that they do not
  // queue behind the weight stream: 16 slices of each of the NS sums (2
  // columns per thread, and gate and up for SiLU), and for the attention
  // input this workgroup's share of the q and k sums (kept in fp32). The
  // partials are this path's float32 ranges (the launches that form their
  // inputs follow digit-path launches of the same step).
  constexpr int NS = XM == XSRC_ATTN ? 2 : XM == XSRC_SILU ? 4 : 1;
  constexpr int kFormC = XM == XSRC_X ? 1 : 16;  // slices per batch of loads
  float ft[NS][kFormC];
  double acc[NS];
  const float* fsrc[NS];
  int fS = 0, fstride = 1;
  float sq[XM == XSRC_ATTN ? kFormC : 1];
  int sq_row = -1, sq_S = 0, sq_stride = 1;
  const float* sq_src = nullptr;
  if constexpr (XM != XSRC_X) {
    fS = part_slices(A.xs.pa);
    fstride = 64 * (((XM == XSRC_ATTN ? A.xs.kv : A.in) + 63) / 64);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int cc = min(col0 + tid + 256 * k, A.in - 1);
      if constexpr (XM == XSRC_ATTN) {
        const int hd = A.xs.head_dim, hh = cc / hd, d = cc - hh * hd;
        fsrc[k] = part_data(A.xs.pa) + (hh / A.xs.rep) * hd + d;
      } else {
        fsrc[k] = part_data(A.xs.pa) + cc;
        fsrc[k + 2] = part_data(A.xs.pb) + cc;
      }
    }
#pragma unroll
    for (int i = 0; i < NS; ++i)
#pragma unroll
      for (int u = 0; u < kFormC; ++u) ft[i][u] = fsrc[i][(size_t)min(u, fS - 1) * fstride];
    if constexpr (XM == XSRC_ATTN) {
      // rows [wid per, wid per + per) of q then k: the first 256 preloaded
      // here, one per thread (any further ones after the rounds)
      const int rows = A.xs.n_q + A.xs.kv, per = (rows + A.items - 1) / A.items;
      const int row = wid * per + tid;
      if (grp == 0 && tid < per && row < rows) {
        const bool isq = row < A.xs.n_q;
        sq_row = row;
        sq_src = part_data(isq ? A.xs.pq : A.xs.pk) + (isq ? row : row - A.xs.n_q);
        sq_S = part_slices(isq ? A.xs.pq : A.xs.pk);
        sq_stride = 64 * (((isq ? A.xs.n_q : A.xs.kv) + 63) / 64);
#pragma unroll
        for (int u = 0; u < kFormC; ++u) sq[u] = sq_src[(size_t)min(u, sq_S - 1) * sq_stride];
      }
    }
  }

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
    if constexpr (XM == XSRC_X)
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
  if constexpr (XM != XSRC_X) {
    // the formed input: each sum's slices added in ascending order (the
    // batch in flight, then any further ones)
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      acc[i] = 0.0;
#pragma unroll
      for (int u = 0; u < kFormC; ++u) acc[i] += u < fS ? (double)ft[i][u] : 0.0;
    }
    for (int r = kFormC; r < fS; r += kFormC) {
#pragma unroll
      for (int i = 0; i < NS; ++i)
#pragma unroll
        for (int u = 0; u < kFormC; ++u) ft[i][u] = fsrc[i][(size_t)min(r + u, fS - 1) * fstride];
#pragma unroll
      for (int i = 0; i < NS; ++i)
#pragma unroll
        for (int u = 0; u < kFormC; ++u) acc[i] += r + u < fS ? (double)ft[i][u] : 0.0;
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      if constexpr (XM == XSRC_ATTN)
        xv[0][0][k] = f64_to_bf16_rne(acc[k]);
      else
        xv[0][0][k] = f64_to_bf16_rne(acc[k] / (1.0 + exp(-acc[k])) * acc[k + 2]);
      xv[0][1][k] = 0;
    }
  }
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

  // masks of slice 3, set once outside the rounds
  const uint32_t m3s = 0x88888888u, o3v = 0x11111111u;
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
        constexpr uint32_t mT = T == 0 ? 0x11111111u : T == 1 ? 0x22222222u : 0x44444444u;
        const int sc = T == 2 ? ascale - 1 : ascale;
        v8i a[NBP];
#pragma unroll
        for (int q = 0; q < NBP; ++q) a[q] = kAreg ? areg[(p * 4 + T) % (kAreg ? 8 : 1)] : image_row(q, p * 4 + T);
#pragma unroll
        for (int tau = 0; tau < 4; ++tau) {
          const uint4 wv = wt[tau * P + p];
          v8i bv;
          if constexpr (T == 3) {
            // (w & 0x8..8) | 0x1..1 as one bitfield insert (the compiler emits an
            // AND and an OR, each with a literal); the mask in a scalar register,
            // the inserted constant in a vector one (one scalar operand per
            // instruction on this target)
            uint32_t r[4];
            const uint32_t wd[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
            for (int d = 0; d < 4; ++d) asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r[d]) : "s"(m3s), "v"(wd[d]), "v"(o3v));
            bv = (v8i){(int)r[0], (int)r[1], (int)r[2], (int)r[3], 0, 0, 0, 0};
          } else {
            bv = (v8i){(int)(wv.x & mT), (int)(wv.y & mT), (int)(wv.z & mT), (int)(wv.w & mT), 0, 0, 0, 0};
          }
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
            ((float*)part)[((size_t)b * A.S + r) * RG * 64 + row] = (float)res[q][tau];
        }
      }
    }
  };

  if constexpr (XM == XSRC_ATTN) {
    // this thread's q or k row (batch 1), slices in ascending order
    if (sq_row >= 0) {
      double v = 0.0;
#pragma unroll
      for (int u = 0; u < kFormC; ++u) v += u < sq_S ? (double)sq[u] : 0.0;
      for (int r = kFormC; r < sq_S; r += kFormC)
        for (int u = 0; u < kFormC && r + u < sq_S; ++u) v += (double)sq_src[(size_t)(r + u) * sq_stride];
      A.xs.qk[sq_row] = (float)v;
    }
  }

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

  if constexpr (XM == XSRC_ATTN) {
    // rows of this work item's q/k share beyond the first 256 (small launches)
    const int rows = A.xs.n_q + A.xs.kv, per = (rows + A.items - 1) / A.items;
    if (grp == 0)
      for (int e = 256 + tid; e < per; e += 256) {
        const int row = wid * per + e;
        if (row >= rows) break;
        const bool isq = row < A.xs.n_q;
        const int stride = 64 * (((isq ? A.xs.n_q : A.xs.kv) + 63) / 64);
        A.xs.qk[row] = (float)sum_ranges(isq ? A.xs.pq : A.xs.pk, 0, stride, isq ? row : row - A.xs.n_q);
      }
  }
}

// ---------------------------------------------------------------------------
// Batches from kF16MinBatch on: fp16 matrix cores, every weight decoded once
// for all the batch's tokens.
//
// The digit path above spends its matrix and slice work per batch pair; from
// a few pairs on, a dense fp16 contraction is cheaper. Per token, x is scaled
// by a power of two and rounded to fp16 (k_gemv16_prep, below); the B operand
// holds ±h_p (exact in fp16); the products are exact in fp32 and the matrix
// cores accumulate them in fp32. A workgroup covers a chunk of kr consecutive
// ranges of 512 columns and, per chunk and output, forms Σ_p g_p acc_p 2^-e in
// float64 and leaves it as one float32 partial (so the partials, written and
// read again by the consumer, shrink kr-fold, and are half the bytes of the
// digit path's).
//
// Inside a 32-column block the contraction index is permuted so that dword c
// of a lane's 8 fp16 values holds the columns (m, m + 16), m = 4 t + c, of
// quarter t (paper App. E.1 packs 32 columns per word: the sign bits of that
// dword are bits m and m + 16 of the stored word, moved to bits 15 and 31 by
// one shift, which serves two words at once as a 64-bit shift). A and B use
// the same order.
//
// Workgroup: 4 waves, one row group (64 rows) each, 4 consecutive row groups.
// Lane (j, gl) holds, per range, the 16-byte unit (rg, 4 r + gl, p, 16 tau + j)
// of each path and 16-row slice tau (as in k_gemv); matrix step s of a range
// takes word s / 4, quarter s % 4 of that unit.
// ---------------------------------------------------------------------------
constexpr int kF16MinBatch = RABIT_GEMV_FP16_MIN_BATCH;
constexpr int kXRow = 260;  // dwords per staged token row (256 + 4: conflict-free 16-byte reads)

typedef _Float16 v8h __attribute__((ext_vector_type(8)));

// v << n as one V_LSHLREV_B64 (full rate here); the compiler otherwise splits
// a 64-bit shift into a 32-bit shift and an align, two instructions
__device__ __forceinline__ uint64_t shl64(uint64_t v, int n) {
  uint64_t r;
  asm volatile("v_lshlrev_b64 %0, %1, %2" : "=v"(r) : "v"(n), "v"(v));
  return r;
}

__device__ __forceinline__ uint32_t f16_pair(float lo, float hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)lo) |
         ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)hi) << 16);
}

// The prepared input (k_gemv16_prep, one launch before the GEMV): token b's
// x (RMSNorm applied when the launch has statistics) scaled by 2^e_b so that
// the row's largest |value| lies in [2^14, 2^15) and rounded to fp16 (exact
// for every value above 2^-32 of that largest one; the rest off by at most
// 2^-25 2^-e_b), in the contraction order: dword m of each 32-column block
// holds columns (m, m + 16); Kp = 512 ceil(in / 512) columns (whole ranges),
// zero past in. Every matrix's h pairs in the same order.
// Workgroup (b, s) for s < xs = ceil(Kp / 2048): token b's row maximum (each
// of the row's workgroups reads the whole row), then columns [2048 s, 2048 s
// + 2048): thread t writes dwords 4 q .. 4 q + 3 (q = t % 4) of block
// 64 s + t / 4. Workgroups from hwg0 on: the h pairs.
constexpr int kPrepCols = 2048;

__global__ __launch_bounds__(256) void k_gemv16_prep(Args A, int P, int hwg0) {
  const int Kp = A.S * kChunk, nblk = Kp / 32;
  const int in = A.in, tid = threadIdx.x, l = tid & 63, w = tid >> 6;
  if ((int)blockIdx.x >= hwg0) {
    const int idx = ((int)blockIdx.x - hwg0) * 256 + tid;  // (segment, path, block, m)
    const int per = P * nblk * 16;
    const int sg = idx / per;
    if (sg >= A.nseg) return;
    const int rem = idx - sg * per, pth = rem / (nblk * 16), blk = (rem >> 4) % nblk, m = rem & 15;
    const uint16_t* h = sg == 2 ? A.seg[2].h : sg == 1 ? A.seg[1].h : A.seg[0].h;
    uint32_t* hp = sg == 2 ? A.seg[2].hp : sg == 1 ? A.seg[1].hp : A.seg[0].hp;
    const int c0 = 32 * blk + m, c1 = c0 + 16;
    const uint32_t lo = c0 < in ? h[(size_t)pth * in + c0] : 0u, hi = c1 < in ? h[(size_t)pth * in + c1] : 0u;
    hp[(size_t)(pth * nblk + blk) * 16 + m] = lo | (hi << 16);
    return;
  }
  const int xs = (Kp + kPrepCols - 1) / kPrepCols;
  const int b = blockIdx.x / xs, sl = blockIdx.x % xs;
  const uint16_t* xb = A.x + (size_t)b * in;
  __shared__ double s_den;
  __shared__ float s_m[4];
  if (A.norm && w == 0) {
    // the sum of x^2 from its kStatParts partials, by the digit path's DPP tree
    const double v = A.stats[(size_t)b * kStatParts + (l & (kStatParts - 1))];
    const double ss = wave_sum_f64(l < kStatParts ? v : 0.0);
    if (l == 0) s_den = sqrt(ss / (double)in + (double)A.eps);
  }
  const bool vec = (in & 7) == 0;
  float m = 0.0f;
  if (vec) {
    const int ng = in / 8;
    for (int g0 = tid; g0 < ng; g0 += 256 * 8) {
      uint4 v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = ((const uint4*)xb)[min(g0 + 256 * k, ng - 1)];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const uint32_t d[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
        float mk = 0.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          mk = fmaxf(mk, fmaxf(fabsf(__uint_as_float(d[q] << 16)), fabsf(__uint_as_float(d[q] & 0xFFFF0000u))));
        m = g0 + 256 * k < ng ? fmaxf(m, mk) : m;
      }
    }
  } else {
    for (int c = tid; c < in; c += 256) m = fmaxf(m, fabsf(bf16_bits_to_f32(xb[c])));
  }
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) m = fmaxf(m, __shfl_xor(m, sh, 64));
  if (l == 0) s_m[w] = m;
  __syncthreads();
  m = fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3]));
  const double den = A.norm ? s_den : 1.0;
  // with RMSNorm the largest input is the rounding of the largest |x| / den
  // (both steps are monotonic)
  if (A.norm && m > 0.0f) m = bf16_bits_to_f32(f64_to_bf16_rne_fast((double)m / den));
  const int e = m > 0.0f ? 14 - ilogbf(m) : 0;
  if (tid == 0 && sl == 0) A.rowexp[b] = e;
  const int blk = sl * (kPrepCols / 32) + (tid >> 2), q = tid & 3;
  if (blk >= nblk) return;
  const int c0 = 32 * blk + 4 * q;  // columns c0 + c and c0 + c + 16, c < 4
  uint32_t lo[4], hi[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    lo[c] = c0 + c < in ? xb[c0 + c] : 0u;
    hi[c] = c0 + c + 16 < in ? xb[c0 + c + 16] : 0u;
  }
  auto val = [&](uint32_t v) -> float {
    return A.norm ? bf16_bits_to_f32(f64_to_bf16_rne_fast((double)bf16_bits_to_f32((uint16_t)v) / den))
                  : bf16_bits_to_f32((uint16_t)v);
  };
  uint32_t o[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) o[c] = f16_pair(ldexpf(val(lo[c]), e), ldexpf(val(hi[c]), e));
  *(uint4*)(A.xh + (size_t)b * Kp + 32 * blk + 8 * q) = make_uint4(o[0], o[1], o[2], o[3]);
}

// The contraction: the prepared x and h pairs of a range reach LDS by direct
// buffer-to-LDS loads into a ring of two stages, issued one range ahead
// together with that range's weights (no staging registers, one barrier per
// range).
template <int MT, int P>
__global__ __launch_bounds__(256, P == 3 && MT == 2 ? 1 : 2) void k_gemv16(Args A) {
  constexpr int NB = 16 * MT;   // token rows held (batch <= NB)
  const int ck = blockIdx.x % A.nck, rbg = blockIdx.x / A.nck;
  const int si = (A.nseg > 2 && rbg >= A.seg[2].rb0) ? 2 : (A.nseg > 1 && rbg >= A.seg[1].rb0) ? 1 : 0;
  const uint4* planes = si == 2 ? A.seg[2].planes : si == 1 ? A.seg[1].planes : A.seg[0].planes;
  const uint16_t* gsc = si == 2 ? A.seg[2].g : si == 1 ? A.seg[1].g : A.seg[0].g;
  const uint32_t* hps = si == 2 ? A.seg[2].hp : si == 1 ? A.seg[1].hp : A.seg[0].hp;
  double* part = si == 2 ? A.seg[2].part : si == 1 ? A.seg[1].part : A.seg[0].part;
  const int out = si == 2 ? A.seg[2].out : si == 1 ? A.seg[1].out : A.seg[0].out;
  const int RG = si == 2 ? A.seg[2].RG : si == 1 ? A.seg[1].RG : A.seg[0].RG;
  const int rb = rbg - (si == 2 ? A.seg[2].rb0 : si == 1 ? A.seg[1].rb0 : A.seg[0].rb0);
  if (blockIdx.x == 0 && threadIdx.x < A.nseg) {
    // the partial buffers' headers: one slice per chunk of ranges
    double* hp = threadIdx.x == 2 ? A.seg[2].part : threadIdx.x == 1 ? A.seg[1].part : A.seg[0].part;
    ((int*)hp)[0] = A.nck;
  }
  part += kPartHdrDoubles;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;
  const int j = l & 15, gl = l >> 4;
  const int batch = A.batch;
  const int Kp = A.S * kChunk, nblk = Kp / 32;  // the prepared rows (whole ranges)
  const int r0 = ck * A.kr, r1 = min(A.S, r0 + A.kr);
  const int rg = 4 * rb + w;            // this wave's row group
  const int rgc = min(rg, RG - 1);      // clamped: loads stay in bounds, results unused

  __shared__ __align__(16) uint32_t s_x[2][NB * kXRow];
  __shared__ __align__(16) uint32_t s_h[2][P][256];

  auto load_w = [&](uint4 (&wt)[4 * P], int r) {
    const int kg = min(A.KG - 1, 4 * r + gl);
#pragma unroll
    for (int tau = 0; tau < 4; ++tau)
#pragma unroll
      for (int p = 0; p < P; ++p) wt[tau * P + p] = load_nt(planes + unit_index(rgc, kg, p, 16 * tau + j, A.KG, P));
  };
  // range r's x (wave w: tokens w, w + 4, ...) and h pairs (path w % P) into
  // stage u: every wave issues NB / 4 + 1 loads of 1 KiB
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      (void*)A.xh, (short)0, (int)((size_t)batch * Kp * 2), kBufWord3);
  const __amdgpu_buffer_rsrc_t rh = __builtin_amdgcn_make_buffer_rsrc(
      (void*)hps, (short)0, (int)((size_t)P * nblk * 64), kBufWord3);
  auto issue = [&](int r, auto U) {
    constexpr int u = decltype(U)::value;
#pragma unroll
    for (int k = 0; k < NB / 4; ++k) {
      const int b = w + 4 * k;
      lds_load16(rx, (lds_void*)(s_x[u] + b * kXRow),
                 (uint32_t)(((size_t)min(b, batch - 1) * Kp + (size_t)r * kChunk) * 2) + 16u * l);
    }
    const int hpth = w % P;
    lds_load16(rh, (lds_void*)(s_h[u][hpth]), (uint32_t)((hpth * nblk + 16 * r) * 64) + 16u * l);
  };

  v4f acc[P][4][MT];
#pragma unroll
  for (int p = 0; p < P; ++p)
#pragma unroll
    for (int tau = 0; tau < 4; ++tau)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[p][tau][mt] = (v4f){0.f, 0.f, 0.f, 0.f};

  // the matrix ops of stage u with the range's weights wt
  auto compute = [&](const uint4 (&wt)[4 * P], auto U) {
    constexpr int u = decltype(U)::value;
    // steps (q, t4) and (q + 1, t4) together: words q and q + 1 of a unit sit
    // in adjacent registers, and one 64-bit shift by 15 - 4 t4 - c brings the
    // sign bits of dword c of both steps to bits 15 and 31 of each half (no
    // bit of the low word reaches those positions of the high word)
    // the LDS operands of step pair sp (qq = 2 (sp / 4), t4 = sp % 4) are read
    // one step pair ahead, into the other of two register sets
    v8h fx0[2][MT], fx1[2][MT];
    uint4 hx0[2][P], hx1[2][P];
    auto rd = [&](int sp) {
      const int off0 = 16 * (4 * gl + 2 * (sp >> 2)) + 4 * (sp & 3), off1 = off0 + 16;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        fx0[sp & 1][mt] = *(const v8h*)(s_x[u] + (16 * mt + j) * kXRow + off0);
        fx1[sp & 1][mt] = *(const v8h*)(s_x[u] + (16 * mt + j) * kXRow + off1);
      }
#pragma unroll
      for (int p = 0; p < P; ++p) {
        hx0[sp & 1][p] = *(const uint4*)(s_h[u][p] + off0);
        hx1[sp & 1][p] = *(const uint4*)(s_h[u][p] + off1);
      }
    };
    rd(0);
#pragma unroll
    for (int qq = 0; qq < 4; qq += 2)
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
        // one step pair at a time (the scheduler would otherwise hoist every
        // step's LDS reads), with the next pair's reads issued first
        __builtin_amdgcn_sched_barrier(0);
        const int sp = 2 * qq + t4;
        if (sp + 1 < 8) rd(sp + 1);
        const int sh = 15 - 4 * t4;
        v8h fa0[MT], fa1[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          fa0[mt] = fx0[sp & 1][mt];
          fa1[mt] = fx1[sp & 1][mt];
        }
#pragma unroll
        for (int p = 0; p < P; ++p) {
          const uint4 h0 = hx0[sp & 1][p];
          const uint4 h1 = hx1[sp & 1][p];
          if constexpr (MT == 2) {
            // all four slices' operands first, then the low step's matrix
            // ops, then the high step's: the two ops on one accumulator are
            // eight apart (same accumulation order as below; 24 more registers,
            // which cost occupancy with one token tile)
            v8h fb0[4], fb1[4];
#pragma unroll
            for (int tau = 0; tau < 4; ++tau) {
              const uint4 wv = wt[tau * P + p];
              const uint64_t pr = qq == 0 ? (((uint64_t)wv.y << 32) | wv.x) : (((uint64_t)wv.w << 32) | wv.z);
              const uint64_t s0 = shl64(pr, sh), s1 = shl64(pr, sh - 1), s2 = shl64(pr, sh - 2),
                             s3 = shl64(pr, sh - 3);
              uint4 e0, e1;
              e0.x = h0.x ^ ((uint32_t)s0 & 0x80008000u);
              e0.y = h0.y ^ ((uint32_t)s1 & 0x80008000u);
              e0.z = h0.z ^ ((uint32_t)s2 & 0x80008000u);
              e0.w = h0.w ^ ((uint32_t)s3 & 0x80008000u);
              e1.x = h1.x ^ ((uint32_t)(s0 >> 32) & 0x80008000u);
              e1.y = h1.y ^ ((uint32_t)(s1 >> 32) & 0x80008000u);
              e1.z = h1.z ^ ((uint32_t)(s2 >> 32) & 0x80008000u);
              e1.w = h1.w ^ ((uint32_t)(s3 >> 32) & 0x80008000u);
              fb0[tau] = __builtin_bit_cast(v8h, e0);
              fb1[tau] = __builtin_bit_cast(v8h, e1);
            }
#pragma unroll
            for (int tau = 0; tau < 4; ++tau)
#pragma unroll
              for (int mt = 0; mt < MT; ++mt)
                acc[p][tau][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa0[mt], fb0[tau], acc[p][tau][mt], 0, 0, 0);
#pragma unroll
            for (int tau = 0; tau < 4; ++tau)
#pragma unroll
              for (int mt = 0; mt < MT; ++mt)
                acc[p][tau][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa1[mt], fb1[tau], acc[p][tau][mt], 0, 0, 0);
            // issue order: the first slice's operands (6 VALU), then one
            // matrix op and two VALU instructions at a time, so that the
            // operand builds run beside the matrix ops
            __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
              __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
            }
            continue;
          }
#pragma unroll
          for (int tau = 0; tau < 4; ++tau) {
            const uint4 wv = wt[tau * P + p];
            const uint64_t pr = qq == 0 ? (((uint64_t)wv.y << 32) | wv.x) : (((uint64_t)wv.w << 32) | wv.z);
            const uint64_t s0 = shl64(pr, sh), s1 = shl64(pr, sh - 1), s2 = shl64(pr, sh - 2),
                           s3 = shl64(pr, sh - 3);
            uint4 e0, e1;
            e0.x = h0.x ^ ((uint32_t)s0 & 0x80008000u);
            e0.y = h0.y ^ ((uint32_t)s1 & 0x80008000u);
            e0.z = h0.z ^ ((uint32_t)s2 & 0x80008000u);
            e0.w = h0.w ^ ((uint32_t)s3 & 0x80008000u);
            e1.x = h1.x ^ ((uint32_t)(s0 >> 32) & 0x80008000u);
            e1.y = h1.y ^ ((uint32_t)(s1 >> 32) & 0x80008000u);
            e1.z = h1.z ^ ((uint32_t)(s2 >> 32) & 0x80008000u);
            e1.w = h1.w ^ ((uint32_t)(s3 >> 32) & 0x80008000u);
            const v8h fb0 = __builtin_bit_cast(v8h, e0), fb1 = __builtin_bit_cast(v8h, e1);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
              acc[p][tau][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa0[mt], fb0, acc[p][tau][mt], 0, 0, 0);
              acc[p][tau][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa1[mt], fb1, acc[p][tau][mt], 0, 0, 0);
            }
          }
        }
      }
  };

  // ranges in pairs (stages 0 and 1, weight buffers wa and wb). Before the
  // matrix ops of range r: this wave's stage loads of r have landed (only
  // r's NB/4... weight loads, issued after them, may still be in flight) and
  // every wave is done with range r - 1, whose stage the loads of r + 1 reuse
  uint4 wa[4 * P], wb[4 * P];
  issue(r0, std::integral_constant<int, 0>());
  load_w(wa, r0);
#pragma unroll 1
  for (int r = r0; r < r1; r += 2) {
    ring_barrier<4 * P>();
    const bool n1 = r + 1 < r1;
    if (n1) {
      issue(r + 1, std::integral_constant<int, 1>());
      load_w(wb, r + 1);
    }
    compute(wa, std::integral_constant<int, 0>());
    if (!n1) break;
    ring_barrier<4 * P>();
    const bool n2 = r + 2 < r1;
    if (n2) {
      issue(r + 2, std::integral_constant<int, 0>());
      load_w(wa, r + 2);
    }
    compute(wb, std::integral_constant<int, 1>());
    if (!n2) break;
  }

  // tokens 16 mt + 4 gl + i of row 16 tau + j: Σ_p g_p acc_p 2^-e_b in float64,
  // stored rounded to float32
  if (rg < RG) {
    int eb[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) eb[mt][i] = A.rowexp[min(16 * mt + 4 * gl + i, batch - 1)];
#pragma unroll
    for (int tau = 0; tau < 4; ++tau) {
      const int row = rg * 64 + 16 * tau + j;
      double gp[P];
#pragma unroll
      for (int p = 0; p < P; ++p) gp[p] = (double)f16_bits_to_f32(gsc[(size_t)p * out + min(row, out - 1)]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int b = 16 * mt + 4 * gl + i;
          if (b >= batch || row >= out) continue;
          double v = gp[0] * (double)acc[0][tau][mt][i];
#pragma unroll
          for (int p = 1; p < P; ++p) v += gp[p] * (double)acc[p][tau][mt][i];
          // streaming (nontemporal) store: measured 1-2 us shorter [q,k,v], o
          // and down launches at batch 16-32; on the digit path (batch 1) the
          // same stores made the decode step slower, so it keeps plain ones
          __builtin_nontemporal_store((float)ldexp(v, -eb[mt][i]), &((float*)part)[((size_t)b * A.nck + ck) * RG * 64 + row]);
        }
    }
  }
}

// y = Σ_r part (ascending r)
__global__ __launch_bounds__(256) void k_gemv_reduce(const double* __restrict__ part, int out,
                                                     int RG, void* y, int y_dtype) {
  const int row = blockIdx.x * 256 + threadIdx.x, b = blockIdx.y;
  if (row >= out) return;
  const int S = part_slices(part);
  // many ranges (wide layers): 32 loads in flight per round trip
  const size_t at = (size_t)b * S * RG * 64 + row;
  const float* pp = part_data(part) + at;
  const double v = S <= 8 ? sum_ranges_by<8>(pp, S, RG * 64) : sum_ranges_by<32>(pp, S, RG * 64);
  if (y_dtype == RABIT_OUT_F32)
    ((float*)y)[(size_t)b * out + row] = (float)v;
  else
    ((uint16_t*)y)[(size_t)b * out + row] = f64_to_bf16_rne(v);
}

// Workgroups of one variant that fit on the device at once (occupancy from
// the runtime, queried once per device and variant).
template <int XM>
const void* gemv_fn(bool ring, int paths) {
  return paths == 3 ? (ring ? (const void*)k_gemv<1, true, false, 3, XM> : (const void*)k_gemv<1, false, false, 3, XM>)
                    : (ring ? (const void*)k_gemv<1, true, false, 2, XM> : (const void*)k_gemv<1, false, false, 2, XM>);
}

int resident_wgs(bool ring, int paths, int xm) {
  static std::atomic<int> cache[kMaxDevices][2][2][3];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
  std::atomic<int>& slot = cache[dev][ring ? 1 : 0][paths == 3 ? 1 : 0][xm];
  int c = slot.load(std::memory_order_relaxed);
  if (c == 0) {
    int cus = 0, per = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
      cus = 256;
    const void* fn = xm == XSRC_ATTN ? gemv_fn<XSRC_ATTN>(ring, paths)
                   : xm == XSRC_SILU ? gemv_fn<XSRC_SILU>(ring, paths) : gemv_fn<XSRC_X>(ring, paths);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, fn, 256, 0) != hipSuccess || per < 1) per = 1;
    c = cus * per;
    slot.store(c, std::memory_order_relaxed);
  }
  return c;
}

// Workgroups of k_gemv16<MT, P> resident at once (runtime occupancy query,
// once per device and variant).
int resident_wgs16(int mt, int paths) {
  static std::atomic<int> cache[kMaxDevices][2][2];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
  std::atomic<int>& slot = cache[dev][mt == 2 ? 1 : 0][paths == 3 ? 1 : 0];
  int c = slot.load(std::memory_order_relaxed);
  if (c == 0) {
    int cus = 0, per = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
      cus = 256;
    const void* fn = paths == 3 ? (mt == 2 ? (const void*)k_gemv16<2, 3> : (const void*)k_gemv16<1, 3>)
                                : (mt == 2 ? (const void*)k_gemv16<2, 2> : (const void*)k_gemv16<1, 2>);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, fn, 256, 0) != hipSuccess || per < 1) per = 1;
    c = cus * per;
    slot.store(c, std::memory_order_relaxed);
  }
  return c;
}

// The fp16 path's launch: row blocks of 4 row groups, chunks of kr ranges.
// Cost model as for the digit path: passes x (kr ranges + one for staging),
// ties to the larger kr (fewer partials to write and read back).
struct Plan16 {
  int S, kr, nck, mt, paths;
  int RB[kMaxSeg];
};

__host__ inline Plan16 make_plan16(const int* outs, int nseg, int in, int batch, int paths) {
  Plan16 P;
  P.paths = paths;
  P.mt = batch > 16 ? 2 : 1;
  P.S = (in + kChunk - 1) / kChunk;
  long rbs = 0;
  for (int s = 0; s < nseg; ++s) {
    P.RB[s] = (row_groups(outs[s]) + 3) / 4;
    rbs += P.RB[s];
  }
  const long cap = resident_wgs16(P.mt, paths);
  long best = -1;
  P.kr = P.S;
  for (int kr = P.S; kr >= 1; --kr) {
    const long nck = (P.S + kr - 1) / kr;
    const long cost = (rbs * nck + cap - 1) / cap * (kr + 1);
    if (best < 0 || cost < best) {
      best = cost;
      P.kr = kr;
    }
  }
  P.nck = (P.S + P.kr - 1) / P.kr;
  return P;
}

// Rows per workgroup (4 m row groups). A workgroup builds the digit operand
// of its range once and then streams m row groups. With one batch pair and
// m > 1 the next round's weights are in flight during a round, so all
// workgroups of a launch should be resident together: a second pass of a few
// workgroups runs its m rounds with most of the device idle. Cost model:
// passes x (m rounds + one for the digit build), ties to the smaller m (more
// workgroups). With more batch pairs (one buffer, rounds not overlapped) the
// rounds stay short: enough workgroups to fill the device a few times over.
__host__ inline Plan make_plan(const int* outs, int nseg, int in, int batch, int paths, int xm = XSRC_X) {
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
    const long cap = resident_wgs(m > 1, paths, xm);
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
  auto go = [&](auto paths_tag, auto xm_tag) {
    constexpr int NP = decltype(paths_tag)::value, XM = decltype(xm_tag)::value;
    if (groups > 1) {
      if (A.m > 1)
        hipLaunchKernelGGL((k_gemv<1, true, true, NP, XM>), grid, dim3(256), 0, st, B);
      else
        hipLaunchKernelGGL((k_gemv<1, false, true, NP, XM>), grid, dim3(256), 0, st, B);
    } else {
      if (A.m > 1)
        hipLaunchKernelGGL((k_gemv<1, true, false, NP, XM>), grid, dim3(256), 0, st, B);
      else
        hipLaunchKernelGGL((k_gemv<1, false, false, NP, XM>), grid, dim3(256), 0, st, B);
    }
  };
  auto go_p = [&](auto xm_tag) {
    if (P.paths == 3)
      go(std::integral_constant<int, 3>(), xm_tag);
    else
      go(std::integral_constant<int, 2>(), xm_tag);
  };
  if (A.xs.mode == XSRC_ATTN)
    go_p(std::integral_constant<int, XSRC_ATTN>());
  else if (A.xs.mode == XSRC_SILU)
    go_p(std::integral_constant<int, XSRC_SILU>());
  else
    go_p(std::integral_constant<int, XSRC_X>());
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
  return part_bytes(out, S, batch) + (batch >= kF16MinBatch ? prep_bytes(in) : 0);
}

hipError_t launch_16(const Plan16& P, Args A, int batch, hipStream_t st) {
  int nrb = 0;
  for (int s = 0; s < A.nseg; ++s) {
    A.seg[s].rb0 = nrb;
    nrb += P.RB[s];
    // the fp16 path's area after the matrix's partial buffer
    char* prep = (char*)A.seg[s].part + part_bytes(A.seg[s].out, P.S, batch);
    A.seg[s].hp = (uint32_t*)(prep + xh_bytes(A.in) + kRowExpBytes);
    if (s == 0) {
      A.xh = (uint16_t*)prep;
      A.rowexp = (int*)(prep + xh_bytes(A.in));
    }
  }
  A.kr = P.kr;
  A.nck = P.nck;
  const int hthreads = A.nseg * P.paths * (P.S * kChunk / 32) * 16;
  const int xwgs = batch * ((P.S * kChunk + kPrepCols - 1) / kPrepCols);
  hipLaunchKernelGGL(k_gemv16_prep, dim3(xwgs + (hthreads + 255) / 256), dim3(256), 0, st, A, P.paths,
                     xwgs);
  const dim3 grid(nrb * P.nck);
  if (P.paths == 3) {
    if (P.mt == 2)
      hipLaunchKernelGGL((k_gemv16<2, 3>), grid, dim3(256), 0, st, A);
    else
      hipLaunchKernelGGL((k_gemv16<1, 3>), grid, dim3(256), 0, st, A);
  } else {
    if (P.mt == 2)
      hipLaunchKernelGGL((k_gemv16<2, 2>), grid, dim3(256), 0, st, A);
    else
      hipLaunchKernelGGL((k_gemv16<1, 2>), grid, dim3(256), 0, st, A);
  }
  return hipGetLastError();
}

hipError_t launch_gemv_partial(const uint4* planes, const uint16_t* g, const uint16_t* h, int out,
                               int in, const uint16_t* x, int batch, void* ws, hipStream_t st,
                               int paths) {
  if (paths != 2 && paths != 3) return hipErrorInvalidValue;
  const LinSeg seg{planes, g, h, out, (double*)ws, paths};
  return launch_gemv_multi(&seg, 1, in, x, batch, nullptr, 0.f, st);
}

hipError_t launch_gemv_reduce(int out, int in, int batch, void* y, int y_dtype, const void* ws,
                              hipStream_t st, int paths) {
  (void)in;
  (void)paths;
  hipLaunchKernelGGL(k_gemv_reduce, dim3((out + 255) / 256, batch), dim3(256), 0, st,
                     (const double*)ws, out, row_groups(out), y, y_dtype);
  return hipGetLastError();
}

size_t gemv_part_bytes(int out, int in, int batch) { return gemv_workspace_bytes(out, in, batch); }

hipError_t launch_gemv_multi(const LinSeg* segs, int nseg, int in, const uint16_t* x, int batch,
                             const double* stats, float eps, hipStream_t st, const GemvXSrc* xs) {
  if (nseg < 1 || nseg > kMaxSeg) return hipErrorInvalidValue;
  if (xs && xs->mode != XSRC_X) {
    // formed inputs: digit path only, no RMSNorm, the partial buffers they read
    if (batch != 1 || stats || !xs->pa) return hipErrorInvalidValue;
    if (xs->mode == XSRC_ATTN &&
        (xs->head_dim < 1 || xs->rep < 1 || !xs->pq || !xs->pk || !xs->qk || xs->n_q != in || xs->kv < 1 ||
         xs->kv != in / xs->rep || in % (xs->rep * xs->head_dim)))
      return hipErrorInvalidValue;
    if (xs->mode == XSRC_SILU && !xs->pb) return hipErrorInvalidValue;
  }
  int outs[kMaxSeg];
  for (int s = 0; s < nseg; ++s) {
    outs[s] = segs[s].out;
    if (segs[s].paths != segs[0].paths) return hipErrorInvalidValue;
  }
  if (segs[0].paths != 2 && segs[0].paths != 3) return hipErrorInvalidValue;
  if (batch >= kF16MinBatch) {
    const Plan16 P = make_plan16(outs, nseg, in, batch, segs[0].paths);
    Args A = {};
    for (int s = 0; s < nseg; ++s) {
      A.seg[s].planes = segs[s].planes;
      A.seg[s].g = segs[s].g;
      A.seg[s].h = segs[s].h;
      A.seg[s].part = segs[s].part;
      A.seg[s].out = segs[s].out;
      A.seg[s].RG = row_groups(segs[s].out);
    }
    A.x = x;
    A.stats = stats;
    A.nseg = nseg;
    A.in = in;
    A.KG = col_groups(in);
    A.S = P.S;
    A.batch = batch;
    A.norm = stats ? 1 : 0;
    A.eps = eps;
    return launch_16(P, A, batch, st);
  }
  const Plan P = make_plan(outs, nseg, in, batch, segs[0].paths, xs ? xs->mode : XSRC_X);
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
  if (xs) A.xs = *xs;
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
  return launch_gemv_reduce(out, in, batch, y, y_dtype, ws, st, paths);
}

}  // namespace rabit
