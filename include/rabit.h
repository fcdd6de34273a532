/*
 * rabit.h - C ABI of the MI355X (gfx950) hot path for RaBiT-style 2-path
 * residual binarization.
 *
 * Method (the pages about "RaBiT: Residual-Aware Binarization Training for
 * Accurate and Efficient LLMs", arXiv 2602.05367):
 *   - paper §4.1, "Binary Building Blocks": W_hat = g ⊙ B ⊙ h, B in {±1}
 *   - paper §4.1, "Multi-bit Approximation via Stacking": W_hat^(2) =
 *     Σ_{p=1,2} g_p ⊙ B_p ⊙ h_p; g_p is per output row, h_p per input column
 *     (paper §4.3 maps g to the output side and h to the input side)
 *   - paper §4.2, "The Coupled Forward Pass": B_1 = sign(W), R_1 = W − W_hat_1,
 *     B_2 = sign(R_1); after training the cores are derived once from W and
 *     frozen and W is discarded
 *   - paper App. E.1, "Weight Packing": 32 columns per uint32, +1 -> 0, -1 -> 1
 *   - paper §5.4: the layer is additions plus element-wise scaling
 *
 * Conventions for every entry point
 *   - Every pointer named "device" is a device pointer owned by the caller;
 *     the library keeps no pointer after a call returns and allocates nothing.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream). Argument errors are returned before anything is enqueued.
 *   - Device pointers must be 16-byte aligned (RABIT_EALIGN otherwise).
 *   - Calls that take a workspace need at least rabit_*_workspace_bytes()
 *     bytes of it (RABIT_EWORKSPACE otherwise). The workspace is scratch: its
 *     contents need not be initialised and are undefined afterwards. Two calls
 *     that overlap in time must not share a workspace.
 *   - Inputs containing NaN or Inf are not supported (results unspecified).
 *   - Launch failures are reported as RABIT_EDEVICE.
 *
 * Readings where the pages are silent (the oracle implements the same):
 *   - sign(v) = +1 unless v < 0, so +0, -0 give +1 (bit 0).
 *   - Canonical word k of a row holds columns 32k .. 32k+31, column 32k+t in
 *     bit t (LSB first); bits past the last column are 0.
 *   - Mean-|.| scales: g[i] = fp16_rne(S_row(i) / in), h[j] =
 *     fp16_rne(S_col(j) / out) where S are float64 sums of |M| in this order:
 *       S_col: rows in tiles of 64, tiles in 4 segments of 16 rows; a segment
 *         is summed in ascending row order from +0.0, the 4 segment sums of a
 *         tile left to right, tile sums left to right.
 *       S_row: columns in tiles of 256; lane l (0..63) of a tile sums tile
 *         columns l, l+64, l+128, l+192 left to right; the lane values are
 *         combined by v[l] += v[l+s] for s = 32,16,8,4,2,1 (result v[0]);
 *         tile results are added left to right from +0.0.
 *     The divide is one IEEE float64 division and the conversion a single
 *     direct round-to-nearest-even to fp16 (overflow gives +inf).
 *   - R_1 = fl32(W − B_1 * (g_1 * h_1)): the fp16 product is exact in fp32,
 *     the subtraction rounds once.
 */
#ifndef RABIT_H_
#define RABIT_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RABIT_LAYOUT_V1 1

typedef enum {
  RABIT_OK = 0,
  RABIT_EINVAL = -1,        /* null pointer, bad enum, aliasing, bad layout version */
  RABIT_ESHAPE = -2,        /* dimension < 1 or above the supported maximum */
  RABIT_EALIGN = -3,        /* device pointer not 16-byte aligned */
  RABIT_EUNSUPPORTED = -4,  /* n_paths != 2, or an unsupported option */
  RABIT_EDEVICE = -5,       /* a HIP launch or runtime call failed */
  RABIT_EWORKSPACE = -6,    /* workspace missing or too small */
  RABIT_ESCRATCH = -7       /* rabit_gemv_noalloc: the call needs more than its
                               fixed scratch buffer (RABIT_NOALLOC_SCRATCH_BYTES) */
} rabit_status;

enum {
  RABIT_SCALES_GIVEN = 0,   /* g_1, h_1 are inputs; g_2, h_2 are not touched */
  RABIT_SCALES_MEANABS = 1, /* all four scales written as mean |.| (see above) */
  /* as MEANABS, with each h divided by the global mean |.| of the matrix
     being binarised (see rabit_pack) */
  RABIT_SCALES_MEANABS_NORMALIZED = 2
};

enum {
  RABIT_OUT_F32 = 0,        /* y as float32 */
  RABIT_OUT_BF16 = 1        /* y rounded once (RNE) to bfloat16 */
};

/* Largest supported dimensions (out_features, in_features, batch, M). */
#define RABIT_MAX_FEATURES (1 << 19)
#define RABIT_MAX_GEMV_BATCH 32
/* Batches from this size on run the decode GEMV on fp16 matrix cores (see
   rabit_gemv); smaller ones on the exact fixed-point path. */
#define RABIT_GEMV_FP16_MIN_BATCH 8
#define RABIT_MAX_GEMM_M (1 << 20)

/*
 * One frozen layer of n_paths binary paths (paper §4.2: cores derived once,
 * W discarded). n_paths is 2 (the 2-bit model) or 3 (the 3-bit variant: a
 * third path from the residual of the second, paper §1 and App. E.1).
 *
 * planes  device, rabit_planes_bytes(out, in, n_paths) bytes. Device layout
 *         V1: a sequence of 16-byte units indexed (rg, kg, p, r) in row-major
 *         order, rg in [0, ceil(out/64)) = group of 64 output rows,
 *         kg in [0, ceil(in/128)) = group of 128 input columns,
 *         p in [0, n_paths) = path, r in [0, 64) = row inside the group.
 *         Unit (rg, kg, p, r) holds, as 4 little-endian uint32, the canonical
 *         words 4*kg + 0, +1, +2, +3 of row 64*rg + r of path p. Rows >= out
 *         and words past ceil(in/32) are zero. (A wave of 64 lanes loads one
 *         (rg, kg, p) slab of 1 KiB with one 16-byte load per lane.)
 * g       device, fp16 bit patterns [n_paths][out]: g_1, g_2(, g_3) (per
 *         output row)
 * h       device, fp16 bit patterns [n_paths][in]: h_1, h_2(, h_3) (per input
 *         column)
 * Every call takes both (the layers of one call all with the same n_paths;
 * RABIT_EUNSUPPORTED otherwise).
 */
typedef struct {
  int32_t layout_version;   /* RABIT_LAYOUT_V1 */
  int32_t out_features;     /* rows of W (outputs) */
  int32_t in_features;      /* columns of W (inputs) */
  int32_t n_paths;          /* 2 or 3 */
  void *planes;
  uint16_t *g;
  uint16_t *h;
} rabit_layer;

/* Bytes of the plane buffer: n_paths * ceil(out/64)*64 * ceil(in/128) * 16
   (0 for n_paths other than 2 and 3, or unsupported dimensions). */
size_t rabit_planes_bytes(int32_t out_features, int32_t in_features, int32_t n_paths);

/* Workspace needed by rabit_pack / rabit_gemv / rabit_gemm for these sizes. */
size_t rabit_pack_workspace_bytes(int32_t out_features, int32_t in_features);
size_t rabit_gemv_workspace_bytes(int32_t out_features, int32_t in_features, int32_t batch);
size_t rabit_gemm_workspace_bytes(int32_t out_features, int32_t in_features, int32_t m);

/*
 * Derive and pack every path of one layer (paper §4.2 steps 1-3, App. E.1;
 * with three paths one more step: R_2 = fl32(R_1 − g_2 B_2 h_2),
 * B_3 = sign(R_2)).
 *
 * W           device float32 [out][in], row-major, contiguous (read only).
 * scale_mode  RABIT_SCALES_MEANABS: writes g_1, h_1 = mean |W| per row/column,
 *             then g_2, h_2 = mean |R_1| (and g_3, h_3 = mean |R_2|), and the
 *             planes. W is read 2 times (3 with three paths).
 *             RABIT_SCALES_MEANABS_NORMALIZED: as MEANABS with h[j] =
 *             fp16((S_col(j) / out) / mu), mu = T / (out * in), where T is
 *             the canonical total of the row sums S_row: lane l (0..63) adds
 *             S_row(l), S_row(l+64), ... in ascending order from +0.0, then
 *             v[l] += v[l+s] for s = 32,16,8,4,2,1 (result v[0]); each
 *             division one IEEE float64 division (h = 0 where T = 0). Then
 *             g_p h_p tracks |M| itself rather than mean|M|^2 (a reading that
 *             fits paper App. B, Corollary 1: the second path approximates
 *             the first path's residual).
 *             RABIT_SCALES_GIVEN: reads g_1, h_1 (and with three paths g_2,
 *             h_2) from layer->g, layer->h; writes only the planes (one read
 *             of W).
 * layer       host pointer; its device buffers are written as described.
 * Errors: RABIT_EINVAL (null, bad mode, W aliasing an output),
 * RABIT_ESHAPE, RABIT_EALIGN, RABIT_EUNSUPPORTED, RABIT_EWORKSPACE,
 * RABIT_EDEVICE.
 */
int rabit_pack(const float *W, uint32_t scale_mode, const rabit_layer *layer,
               void *workspace, size_t workspace_bytes, void *stream);

/*
 * Test hook: write the canonical words of every plane.
 * words  device uint32 [n_paths][out][ceil(in/32)] (path 1 first).
 */
int rabit_unpack(const rabit_layer *layer, uint32_t *words, void *stream);

/*
 * Decode GEMV (paper App. E.1, "binary GEMV operations"):
 *   y[b][i] = Σ_p g_p[i] * Σ_j B_p[i][j] * h_p[j] * x[b][j]
 *
 * x       device bfloat16 bit patterns [batch][in], row-major.
 * batch   1 .. RABIT_MAX_GEMV_BATCH.
 * y       device [batch][out], float32 (RABIT_OUT_F32) or bfloat16
 *         (RABIT_OUT_BF16), written entirely.
 * Arithmetic, batch < RABIT_GEMV_FP16_MIN_BATCH: h_p*x is formed exactly and
 * held as a fixed-point integer per (batch row, path, range of 512 input
 * columns), scaled by a power of two so that the range's largest |h_p*x| maps
 * into [2^18, 2^19) (per-element error <= 2^-19 of that largest value); the
 * signed sums are exact integers; each range's g_1 S_1 + g_2 S_2 is formed in
 * float64 and rounded to float32 (within 2^-24 of Σ_p |g_p| Σ_range |h_p x|
 * plus the grid error), the ranges are summed in float64 in ascending order
 * and the result is rounded once.
 * Arithmetic, batch >= RABIT_GEMV_FP16_MIN_BATCH: each token row of x is
 * scaled by a power of two 2^e so that its largest |x| lies in [2^14, 2^15)
 * and rounded to fp16 (exact for values above 2^-32 of that largest one, the
 * rest off by at most 2^-25 2^-e); the products with ±h_p are exact and
 * summed in fp32 over chunks of consecutive 512-column ranges (at most
 * in_features + 16 ceil(in/512) roundings, each within 2^-24 of a running sum
 * bounded by Σ_j |h_p[j] x[j]|); per chunk Σ_p g_p acc_p 2^-e is formed in
 * float64 and rounded to float32 (one more rounding per chunk, within 2^-24
 * of Σ_p |g_p| Σ_j |h_p[j] x[j]|), the chunks are summed in float64 in
 * ascending order and the result is rounded once.
 * Result is bitwise repeatable (no order-dependent arithmetic); a batch row's
 * result depends only on that row, for batches of the same arithmetic and
 * token tile (up to 16 rows, or 17 to 32).
 * workspace must not overlap x or y.
 */
int rabit_gemv(const rabit_layer *layer, const uint16_t *x, int32_t batch,
               void *y, int32_t y_dtype, void *workspace, size_t workspace_bytes,
               void *stream);

/*
 * rabit_gemv without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). Same arithmetic, kernels and result bits as
 * rabit_gemv; nothing is allocated. The per-range partials live in a fixed
 * scratch array of RABIT_NOALLOC_SCRATCH_BYTES in device memory that the
 * library holds on every GPU it runs on until the process ends (its address
 * is looked up once per device, on the first call there).
 * Limit: rabit_gemv_workspace_bytes(out, in, batch) <= RABIT_NOALLOC_SCRATCH_BYTES
 * (e.g. a 28672 x 8192 or 8192 x 28672 layer up to batch 8), else
 * RABIT_ESCRATCH before anything is enqueued.
 * Every call on one GPU shares that GPU's scratch: calls that may overlap on
 * one GPU (different streams without ordering between them, or several host
 * threads) race and must be serialised by the caller. Each call overwrites
 * every partial it reads, so nothing needs clearing between calls.
 * Errors: as rabit_gemv (no workspace errors), RABIT_ESCRATCH, RABIT_EDEVICE
 * (the scratch address could not be obtained).
 */
#define RABIT_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int rabit_gemv_noalloc(const rabit_layer *layer, const uint16_t *x, int32_t batch, void *y,
                       int32_t y_dtype, void *stream);

/*
 * The two halves of rabit_gemv, for callers that time or schedule them apart.
 * rabit_gemv_partial streams every plane byte in one kernel launch and leaves
 * in the workspace the partial result, in float32, of each range of 512
 * input columns (from RABIT_GEMV_FP16_MIN_BATCH on, of each chunk of
 * ranges), after a header that records their count;
 * rabit_gemv_reduce sums those partials (ascending order) into y.
 * A reduce consumes the workspace of the last partial for the same layer and
 * batch; the pair gives the same bits as rabit_gemv. Errors as rabit_gemv.
 */
int rabit_gemv_partial(const rabit_layer *layer, const uint16_t *x, int32_t batch,
                       void *workspace, size_t workspace_bytes, void *stream);
int rabit_gemv_reduce(const rabit_layer *layer, int32_t batch, void *y, int32_t y_dtype,
                      void *workspace, size_t workspace_bytes, void *stream);

/*
 * rabit_gemv_partial for n = 1..3 layers that read the same x (equal
 * in_features; e.g. q/k/v or gate/up of a decoder layer), in one kernel
 * launch. workspace holds the layers' partial buffers back to back: layer i's
 * starts at the sum of rabit_gemv_workspace_bytes(out_k, in, batch) over
 * k < i (each a multiple of 256), and rabit_gemv_reduce on layer i with a
 * pointer to its buffer gives the same bits as rabit_gemv. workspace_bytes
 * must cover all n buffers. Errors as rabit_gemv; RABIT_ESHAPE if n is out of
 * range or in_features differ.
 */
int rabit_gemv_partial_multi(const rabit_layer *layers, int32_t n, const uint16_t *x,
                             int32_t batch, void *workspace, size_t workspace_bytes,
                             void *stream);

/*
 * Prefill GEMM: Y[m][i] = Σ_p g_p[i] * Σ_j B_p[i][j] * h_p[j] * X[m][j].
 *
 * X       device bfloat16 bit patterns [M][in], row-major.
 * M       1 .. RABIT_MAX_GEMM_M.
 * Y       device [M][out] float32 or bfloat16.
 * Arithmetic: MFMA fp16 x fp16 -> fp32. The B tile holds ±h_p (exact in
 * fp16); each X row is scaled by a power of two so that its largest |x| is
 * in [2^14, 2^15), rounded to fp16, and unscaled in the epilogue, where g_p
 * is applied in fp32.
 * Errors: RABIT_ESHAPE also when the layer's planes take 4 GiB or more (the
 * kernel addresses them with 32-bit offsets; rabit_grad_input likewise).
 */
int rabit_gemm(const rabit_layer *layer, const uint16_t *X, int32_t m,
               void *Y, int32_t y_dtype, void *workspace, size_t workspace_bytes,
               void *stream);

/*
 * Training side of one layer (paper §4.2, "The Coupled Forward Pass" and
 * "Backward Pass and Parameter Updates"). A training step derives the cores
 * from the shared weight W_FP with the current scales (rabit_pack with
 * RABIT_SCALES_GIVEN) and runs the forward with rabit_gemm; the calls below
 * are its backward, for the loss gradient dY at the layer output. The pages
 * omit the formulas; the reading used here:
 *   dW   = Σ_n dY[n] X[n]ᵀ, the gradient of the effective weight W_hat, handed
 *          to W_FP unchanged (the straight-through estimator), d_out x d_in;
 *   dg_p = Σ_n dY[n] ⊙ (B_p (h_p ⊙ X[n])), dh_p = Σ_n X[n] ⊙ (B_pᵀ (g_p ⊙ dY[n]))
 *          (chain rule with the cores B_p held constant, summed over the
 *          samples of the batch);
 *   dX   = dY W_hat (the gradient passed to the layer below).
 * The scales are the layer's fp16 values.
 */
#define RABIT_GRAD_ACCUMULATE 1u  /* add into dW, dg, dh instead of overwriting */

/* Workspace bytes of rabit_grad_input / rabit_grad_weight (2 or 3 paths). */
size_t rabit_grad_input_workspace_bytes(int32_t out_features, int32_t in_features, int32_t m);
size_t rabit_grad_weight_workspace_bytes(int32_t out_features, int32_t in_features);

/*
 * The planes of the layer W_hatᵀ (out' = in_features, in' = out_features,
 * cores B_pᵀ; its scales are the layer's h as g' and g as h', used in place):
 * bit (o, i) of B_p is written as bit (i, o) of path p in layout V1.
 * planes_t  device, rabit_planes_bytes(in_features, out_features, n_paths)
 *           bytes, written entirely; must not overlap the layer's buffers.
 * Errors: RABIT_EINVAL, RABIT_ESHAPE, RABIT_EALIGN, RABIT_EUNSUPPORTED,
 * RABIT_EDEVICE.
 */
int rabit_transpose_planes(const rabit_layer *layer, void *planes_t, void *stream);

/*
 * dX[n][j] = Σ_i dY[n][i] W_hat[i][j]: the planes are transposed into the
 * workspace, then the prefill GEMM of W_hatᵀ runs (same arithmetic as
 * rabit_gemm, with dY in the role of X).
 * dY   device bfloat16 bit patterns [M][out], row-major.
 * M    1 .. RABIT_MAX_GEMM_M.
 * dX   device [M][in] float32 or bfloat16 (dx_dtype), written entirely; must
 *      not overlap dY or the layer's buffers.
 * Errors as rabit_gemm.
 */
int rabit_grad_input(const rabit_layer *layer, const uint16_t *dY, int32_t m, void *dX,
                     int32_t dx_dtype, void *workspace, size_t workspace_bytes, void *stream);
/* rabit_grad_input with the options of rabit_gemm_ex (RABIT_GEMM_WEFF). */
int rabit_grad_input_ex(const rabit_layer *layer, const uint16_t *dY, int32_t m, void *dX,
                        int32_t dx_dtype, uint32_t flags, void *workspace, size_t workspace_bytes,
                        void *stream);

/*
 * dW, dg and dh of the layer for one batch.
 * X     device bfloat16 bit patterns [M][in] (the layer input of the forward).
 * dY    device bfloat16 bit patterns [M][out].
 * M     1 .. RABIT_MAX_GEMM_M.
 * dW    device float32 [out][in], row-major.
 * dg    device float32 [n_paths][out];  dh  device float32 [n_paths][in].
 * flags 0 (overwrite) or RABIT_GRAD_ACCUMULATE (add to the values present,
 *       e.g. over micro-batches).
 * Arithmetic: dW on the bf16 matrix cores (products exact, fp32 sums);
 * dg, dh from the fp32 dW values of each 128 x 128 tile (fp32 sums, tiles
 * added in ascending order). Outputs must not overlap each other, X, dY or
 * the layer's buffers.
 * Errors: RABIT_EINVAL (null, flags, aliasing), RABIT_ESHAPE, RABIT_EALIGN,
 * RABIT_EUNSUPPORTED, RABIT_EWORKSPACE, RABIT_EDEVICE.
 */
int rabit_grad_weight(const rabit_layer *layer, const uint16_t *X, const uint16_t *dY,
                      int32_t m, float *dW, float *dg, float *dh, uint32_t flags,
                      void *workspace, size_t workspace_bytes, void *stream);

/*
 * Initial scales of a layer (paper §4.3 "Iterative Residual SVID" eq. and
 * "I/O Channel Importance-Scaled Preconditioning" eqs.; App. F.1/F.3: 20
 * sweeps). Sweep t re-fits path i = 1..n_paths in order to
 * R_i = W' − Σ_{j≠i} g_j ⊙ B_j ⊙ h_j (paths before i from this sweep, after i
 * from the previous one; all zero before the first sweep, so sweep 1 is the
 * greedy fit) with SVID(R_i): B_i = sign(R_i) and g_i h_iᵀ the leading
 * rank-1 term of |R_i| (SVID is not defined on the pages; this is the plain
 * reading, the exact minimiser of ||R_i − g_i ⊙ B_i ⊙ h_i|| over signs and
 * non-negative rank-1 scales). W' = f_out ⊙ W ⊙ f_in (f = s^a, the channel
 * importance factors; NULL = 1), and the scales are mapped back:
 * g_i = g_i' / f_out, h_i = h_i' / f_in.
 *
 * The rank-1 term is computed by power iteration on |R_i|, warm-started
 * from h_i: power_passes (odd, 1..63; 5 reach the exact SVID to about 1e-9
 * on the synthetic layers, 3 leave about 1e-2 after 20 sweeps) reads of W
 * per re-fit, alternating
 * rows (u = |R_i| v) and columns (v = |R_i|ᵀ u), starting and ending with
 * rows; then with σ = ||u|| / ||v||, g_i = u / (sqrt(σ) ||v||) and
 * h_i = sqrt(σ) v / ||v||. R is formed in float32: fl(fl(f_out W) f_in), then
 * each other path's fl(g_j h_j) subtracted in path order.
 *
 * W       device float32 [out][in].
 * f_out   device float32 [out] or NULL;  f_in  device float32 [in] or NULL
 *         (positive).
 * flags   0, or RABIT_SVID_CONTINUE: g, h and planes hold a previous result
 *         (original domain) that stands for the paths before the first sweep.
 * g, h    device float32 [n_paths][out], [n_paths][in]: the scales (written;
 *         read first with RABIT_SVID_CONTINUE).
 * planes  device, rabit_planes_bytes(out, in, n_paths) bytes, layout V1: the
 *         bits of each B_i of the last sweep.
 * The scales are float32, as learnable parameters; a packed layer takes them
 * rounded to fp16 (rabit_pack with RABIT_SCALES_GIVEN re-derives the cores).
 * Errors: RABIT_EINVAL (null, flags, aliasing), RABIT_ESHAPE (sizes, sweeps
 * < 1 or > 1000, power_passes even or out of range), RABIT_EALIGN,
 * RABIT_EUNSUPPORTED (n_paths), RABIT_EWORKSPACE, RABIT_EDEVICE.
 */
#define RABIT_SVID_CONTINUE 1u

size_t rabit_svid_workspace_bytes(int32_t out_features, int32_t in_features);
int rabit_svid_init(const float *W, int32_t out_features, int32_t in_features, int32_t n_paths,
                    int32_t sweeps, int32_t power_passes, const float *f_out, const float *f_in,
                    uint32_t flags, float *g, float *h, void *planes, void *workspace,
                    size_t workspace_bytes, void *stream);

/*
 * rabit_gemm with options (flags 0 = rabit_gemm).
 * RABIT_GEMM_WEFF: the effective weight W_hat (paper §4.1 "Multi-bit
 *   Approximation via Stacking") of each tile is formed in fp16 and the
 *   matrix cores run once per tile instead of once per path: with
 *   f[i] = max_p |g_p[i]| and r_p = fp16(g_p[i] / f[i]), the tile holds
 *   e[i][j] = Σ_p r_p (±h_p[j]) by fp16 multiply-adds in path order, and
 *   Y = f ⊙ (X eᵀ) with fp32 accumulation. Each weight is rounded (about
 *   2^-11 relative), so Y is no longer the exact ±h contraction; half the
 *   matrix work of the exact path with two paths, a third with three.
 * Errors as rabit_gemm; RABIT_EINVAL for unknown flags.
 */
#define RABIT_GEMM_WEFF 1u
int rabit_gemm_ex(const rabit_layer *layer, const uint16_t *X, int32_t m, void *Y,
                  int32_t y_dtype, uint32_t flags, void *workspace, size_t workspace_bytes,
                  void *stream);

/*
 * Decoder configuration for rabit_decode_step (a Llama-style block; the pages
 * time Llama2 decoding, Table 7, without defining the block).
 */
typedef struct {
  int32_t hidden;       /* model width */
  int32_t ffn;          /* MLP width */
  int32_t n_heads;      /* query heads */
  int32_t n_kv_heads;   /* key/value heads (GQA) */
  int32_t head_dim;
  int32_t n_layers;
  float rms_eps;        /* RMSNorm epsilon (unit weight) */
  int32_t mlp_only;     /* 1: blocks have no attention (q/k/v/o unused) */
} rabit_decoder_cfg;

size_t rabit_decode_workspace_bytes(const rabit_decoder_cfg *cfg, int32_t batch);

/*
 * One decode step through cfg->n_layers blocks, one token per batch row.
 *
 * layers   host array [n_layers * 7] of layers in the order
 *          q, k, v, o, gate, up, down (q/k/v/o ignored when mlp_only).
 * x        device bf16 [batch][hidden] input hidden state.
 * out      device bf16 [batch][hidden] output hidden state (may equal x).
 * Per block (bf16 at each arrow that stores an activation):
 *   n = rmsnorm(x) -> [q,k,v = W n] -> a = attention over a one-token
 *   context (each head returns its KV group's v) -> x = x + W_o a ->
 *   n = rmsnorm(x) -> z = silu(W_gate n) * (W_up n) -> x = x + W_down z.
 * batch    1 .. RABIT_MAX_GEMV_BATCH uses the GEMV; larger batches the GEMM.
 * Errors: as the ops above; RABIT_ESHAPE if a layer's shape does not match
 * cfg (q, o: hidden x hidden; k, v: n_kv_heads*head_dim x hidden; gate, up:
 * ffn x hidden; down: hidden x ffn).
 */
int rabit_decode_step(const rabit_decoder_cfg *cfg, const rabit_layer *layers,
                      const uint16_t *x, int32_t batch, uint16_t *out,
                      void *workspace, size_t workspace_bytes, void *stream);

const char *rabit_status_string(int status);
int32_t rabit_layout_version(void);

/*
 * Test hook: the library's float64 -> fp16 (bf16 = 0) or -> bfloat16
 * (bf16 = 1) round-to-nearest-even, as used for the scales and outputs;
 * bf16 = 2: the short bfloat16 path the RMSNorm prologues use (same result).
 * in: device float64 [n]; out: device uint16 [n].
 */
int rabit_test_f64_to_16(const double *in, uint16_t *out, int32_t n, int32_t bf16, void *stream);

/*
 * Measurement hook: reads `bytes` of device memory once with 16-byte loads
 * (eight in flight per thread, each load instruction covering 4 KiB of
 * consecutive memory) and keeps nothing. It gives the practical HBM ceiling
 * for a read-only stream of a given size, next to the GEMV (which streams
 * its planes the same way). Not part of the method.
 * src   device, 16-byte aligned; bytes a multiple of 16 (0: nothing runs).
 * sink  device uint32, 16-byte aligned; may be overwritten with an
 *       unspecified value.
 * Errors: RABIT_EINVAL (null pointer), RABIT_EALIGN (alignment or bytes).
 */
int rabit_stream_read(const void *src, size_t bytes, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* RABIT_H_ */
