// extern "C" entry points of librabit: argument validation, workspace
// carving and dispatch to the HIP launchers. Nothing here allocates device
// memory; every call enqueues on the caller's stream.
#include <algorithm>
#include <mutex>

#include "rabit_internal.h"

using namespace rabit;

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return na && nb && x < y + nb && y < x + na;
}

int dev_status(hipError_t e) { return e == hipSuccess ? RABIT_OK : RABIT_EDEVICE; }

int check_dims(int64_t out, int64_t in) {
  if (out < 1 || in < 1 || out > RABIT_MAX_FEATURES || in > RABIT_MAX_FEATURES) return RABIT_ESHAPE;
  return RABIT_OK;
}

// layer header checks shared by every op that reads a packed layer
// the prefill GEMM addresses a layer's planes with 32-bit buffer offsets
bool gemm_planes_fit(const rabit_layer* L) {
  return rabit_planes_bytes(L->out_features, L->in_features, L->n_paths) <= 0xFFFFFFFFull;
}

int check_layer(const rabit_layer* L) {
  if (!L) return RABIT_EINVAL;
  if (L->layout_version != RABIT_LAYOUT_V1) return RABIT_EINVAL;
  if (L->n_paths != 2 && L->n_paths != 3) return RABIT_EUNSUPPORTED;
  int s = check_dims(L->out_features, L->in_features);
  if (s) return s;
  if (!L->planes || !L->g || !L->h) return RABIT_EINVAL;
  if (!aligned16(L->planes) || !aligned16(L->g) || !aligned16(L->h)) return RABIT_EALIGN;
  const int P = L->n_paths;
  const size_t pb = rabit_planes_bytes(L->out_features, L->in_features, P);
  const size_t gb = (size_t)P * L->out_features * 2, hb = (size_t)P * L->in_features * 2;
  if (overlap(L->planes, pb, L->g, gb) || overlap(L->planes, pb, L->h, hb) ||
      overlap(L->g, gb, L->h, hb))
    return RABIT_EINVAL;
  return RABIT_OK;
}

// does [p, p + n) overlap any buffer of the layer (every path's plane, g and h)?
bool overlaps_layer(const void* p, size_t n, const rabit_layer* L) {
  const int P = L->n_paths, out = L->out_features, in = L->in_features;
  return overlap(p, n, L->planes, rabit_planes_bytes(out, in, P)) ||
         overlap(p, n, L->g, (size_t)2 * P * out) || overlap(p, n, L->h, (size_t)2 * P * in);
}

}  // namespace

extern "C" {

int32_t rabit_layout_version(void) { return RABIT_LAYOUT_V1; }

const char* rabit_status_string(int status) {
  switch (status) {
    case RABIT_OK: return "ok";
    case RABIT_EINVAL: return "invalid argument";
    case RABIT_ESHAPE: return "unsupported shape";
    case RABIT_EALIGN: return "device pointer not 16-byte aligned";
    case RABIT_EUNSUPPORTED: return "unsupported option";
    case RABIT_EDEVICE: return "HIP launch or runtime error";
    case RABIT_EWORKSPACE: return "workspace missing or too small";
    case RABIT_ESCRATCH: return "call needs more than the fixed scratch buffer of rabit_gemv_noalloc";
    default: return "unknown status";
  }
}

size_t rabit_planes_bytes(int32_t out, int32_t in, int32_t n_paths) {
  if (check_dims(out, in) || (n_paths != 2 && n_paths != 3)) return 0;
  return (size_t)n_paths * row_groups(out) * 64 * col_groups(in) * 16;
}

size_t rabit_pack_workspace_bytes(int32_t out, int32_t in) {
  if (check_dims(out, in)) return 0;
  return pack_workspace_bytes(out, in);
}

size_t rabit_gemv_workspace_bytes(int32_t out, int32_t in, int32_t batch) {
  if (check_dims(out, in) || batch < 1 || batch > RABIT_MAX_GEMV_BATCH) return 0;
  return gemv_workspace_bytes(out, in, batch);
}

size_t rabit_gemm_workspace_bytes(int32_t out, int32_t in, int32_t m) {
  if (check_dims(out, in) || m < 1 || m > RABIT_MAX_GEMM_M) return 0;
  return gemm_workspace_bytes(out, in, m);
}

int rabit_pack(const float* W, uint32_t scale_mode, const rabit_layer* L, void* workspace,
               size_t workspace_bytes, void* stream) {
  if (!L || !W) return RABIT_EINVAL;
  if (scale_mode != RABIT_SCALES_GIVEN && scale_mode != RABIT_SCALES_MEANABS &&
      scale_mode != RABIT_SCALES_MEANABS_NORMALIZED)
    return RABIT_EINVAL;
  int s = check_layer(L);
  if (s) return s;
  if (!aligned16(W)) return RABIT_EALIGN;
  const int out = L->out_features, in = L->in_features, P = L->n_paths;
  const size_t wb = (size_t)out * in * 4;
  if (overlap(W, wb, L->planes, rabit_planes_bytes(out, in, P)) ||
      overlap(W, wb, L->g, (size_t)2 * P * out) || overlap(W, wb, L->h, (size_t)2 * P * in))
    return RABIT_EINVAL;
  const bool meanabs = scale_mode != RABIT_SCALES_GIVEN;
  if (meanabs) {
    if (!workspace) return RABIT_EWORKSPACE;
    if (workspace_bytes < pack_workspace_bytes(out, in)) return RABIT_EWORKSPACE;
    if (!aligned16(workspace)) return RABIT_EALIGN;
  }
  return dev_status(launch_pack(W, out, in, P, meanabs, L->g, L->h, (uint4*)L->planes, workspace,
                                (hipStream_t)stream, scale_mode == RABIT_SCALES_MEANABS_NORMALIZED));
}

int rabit_unpack(const rabit_layer* L, uint32_t* words, void* stream) {
  int s = check_layer(L);
  if (s) return s;
  if (!words) return RABIT_EINVAL;
  if (!aligned16(words)) return RABIT_EALIGN;
  return dev_status(launch_unpack((const uint4*)L->planes, L->out_features, L->in_features,
                                  L->n_paths, words, (hipStream_t)stream));
}

namespace {
int check_gemv_common(const rabit_layer* L, int32_t batch, void* workspace, size_t workspace_bytes) {
  int s = check_layer(L);
  if (s) return s;
  if (batch < 1 || batch > RABIT_MAX_GEMV_BATCH) return RABIT_ESHAPE;
  if (!workspace || workspace_bytes < gemv_workspace_bytes(L->out_features, L->in_features, batch))
    return RABIT_EWORKSPACE;
  if (!aligned16(workspace)) return RABIT_EALIGN;
  return RABIT_OK;
}
int check_gemv_x(const rabit_layer* L, const uint16_t* x) {
  if (!x) return RABIT_EINVAL;
  if (!aligned16(x)) return RABIT_EALIGN;
  (void)L;
  return RABIT_OK;
}
int check_gemv_y(const rabit_layer* L, int32_t batch, void* y, int32_t y_dtype, const void* x) {
  if (!y) return RABIT_EINVAL;
  if (y_dtype != RABIT_OUT_F32 && y_dtype != RABIT_OUT_BF16) return RABIT_EINVAL;
  if (!aligned16(y)) return RABIT_EALIGN;
  const int out = L->out_features, in = L->in_features;
  const size_t yb = (size_t)batch * out * (y_dtype == RABIT_OUT_F32 ? 4 : 2);
  if ((x && overlap(y, yb, x, (size_t)batch * in * 2)) || overlaps_layer(y, yb, L))
    return RABIT_EINVAL;
  return RABIT_OK;
}
}  // namespace

int rabit_gemv(const rabit_layer* L, const uint16_t* x, int32_t batch, void* y, int32_t y_dtype,
               void* workspace, size_t workspace_bytes, void* stream) {
  int s = check_layer(L);
  if (s) return s;
  if (!x || !y) return RABIT_EINVAL;
  if (y_dtype != RABIT_OUT_F32 && y_dtype != RABIT_OUT_BF16) return RABIT_EINVAL;
  if (batch < 1 || batch > RABIT_MAX_GEMV_BATCH) return RABIT_ESHAPE;
  if ((s = check_gemv_x(L, x)) || (s = check_gemv_y(L, batch, y, y_dtype, x))) return s;
  if ((s = check_gemv_common(L, batch, workspace, workspace_bytes))) return s;
  const size_t wsb = gemv_workspace_bytes(L->out_features, L->in_features, batch);
  const size_t yb = (size_t)batch * L->out_features * (y_dtype == RABIT_OUT_F32 ? 4 : 2);
  if (overlap(workspace, wsb, x, (size_t)batch * L->in_features * 2) ||
      overlap(workspace, wsb, y, yb) || overlaps_layer(workspace, wsb, L))
    return RABIT_EINVAL;
  return dev_status(launch_gemv((const uint4*)L->planes, L->g, L->h, L->out_features,
                                L->in_features, x, batch, y, y_dtype, workspace,
                                (hipStream_t)stream, L->n_paths));
}

}  // extern "C"

// ---- the allocation-free GEMV's scratch ------------------------------------
// One file-scope device array per GPU the library runs on. Host code never
// uses the name `scratch` as an address: its device address is looked up per
// device (hipGetSymbolAddress, with that device current) on the first call
// there and kept in scratch_dev[].
namespace {
constexpr int kScratchDevices = 64;
__device__ __align__(256) unsigned char scratch[RABIT_NOALLOC_SCRATCH_BYTES];
std::mutex scratch_mu;
void* scratch_dev[kScratchDevices] = {};

void* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_dev[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    scratch_dev[dev] = p;
  }
  return scratch_dev[dev];
}
}  // namespace

extern "C" {

int rabit_gemv_noalloc(const rabit_layer* L, const uint16_t* x, int32_t batch, void* y,
                       int32_t y_dtype, void* stream) {
  int s = check_layer(L);
  if (s) return s;
  if (!x || !y) return RABIT_EINVAL;
  if (y_dtype != RABIT_OUT_F32 && y_dtype != RABIT_OUT_BF16) return RABIT_EINVAL;
  if (batch < 1 || batch > RABIT_MAX_GEMV_BATCH) return RABIT_ESHAPE;
  if ((s = check_gemv_x(L, x)) || (s = check_gemv_y(L, batch, y, y_dtype, x))) return s;
  if (gemv_workspace_bytes(L->out_features, L->in_features, batch) > RABIT_NOALLOC_SCRATCH_BYTES)
    return RABIT_ESCRATCH;
  void* ws = scratch_address();
  if (!ws) return RABIT_EDEVICE;
  return dev_status(launch_gemv((const uint4*)L->planes, L->g, L->h, L->out_features,
                                L->in_features, x, batch, y, y_dtype, ws, (hipStream_t)stream,
                                L->n_paths));
}

int rabit_gemv_partial(const rabit_layer* L, const uint16_t* x, int32_t batch, void* workspace,
                       size_t workspace_bytes, void* stream) {
  int s = check_gemv_common(L, batch, workspace, workspace_bytes);
  if (s) return s;
  if ((s = check_gemv_x(L, x))) return s;
  const size_t wsb = gemv_workspace_bytes(L->out_features, L->in_features, batch);
  if (overlap(workspace, wsb, x, (size_t)batch * L->in_features * 2) ||
      overlaps_layer(workspace, wsb, L))
    return RABIT_EINVAL;
  return dev_status(launch_gemv_partial((const uint4*)L->planes, L->g, L->h, L->out_features,
                                        L->in_features, x, batch, workspace, (hipStream_t)stream,
                                        L->n_paths));
}

int rabit_gemv_partial_multi(const rabit_layer* Ls, int32_t n, const uint16_t* x, int32_t batch,
                             void* workspace, size_t workspace_bytes, void* stream) {
  if (!Ls) return RABIT_EINVAL;
  if (n < 1 || n > 3) return RABIT_ESHAPE;
  if (batch < 1 || batch > RABIT_MAX_GEMV_BATCH) return RABIT_ESHAPE;
  int s;
  if ((s = check_gemv_x(&Ls[0], x))) return s;
  const int in = Ls[0].in_features;
  LinSeg segs[3];
  size_t off = 0;
  for (int i = 0; i < n; ++i) {
    if ((s = check_layer(&Ls[i]))) return s;
    if (Ls[i].in_features != in) return RABIT_ESHAPE;
    if (Ls[i].n_paths != Ls[0].n_paths) return RABIT_EUNSUPPORTED;
    segs[i] = LinSeg{(const uint4*)Ls[i].planes, Ls[i].g, Ls[i].h, Ls[i].out_features,
                     (double*)((char*)workspace + off), Ls[i].n_paths};
    off += gemv_workspace_bytes(Ls[i].out_features, in, batch);
  }
  if (!workspace || workspace_bytes < off) return RABIT_EWORKSPACE;
  if (!aligned16(workspace)) return RABIT_EALIGN;
  if (overlap(workspace, off, x, (size_t)batch * in * 2)) return RABIT_EINVAL;
  for (int i = 0; i < n; ++i)
    if (overlaps_layer(workspace, off, &Ls[i])) return RABIT_EINVAL;
  return dev_status(launch_gemv_multi(segs, n, in, x, batch, nullptr, 0.f, (hipStream_t)stream));
}

int rabit_gemv_reduce(const rabit_layer* L, int32_t batch, void* y, int32_t y_dtype, void* workspace,
                      size_t workspace_bytes, void* stream) {
  int s = check_gemv_common(L, batch, workspace, workspace_bytes);
  if (s) return s;
  if ((s = check_gemv_y(L, batch, y, y_dtype, nullptr))) return s;
  const size_t yb = (size_t)batch * L->out_features * (y_dtype == RABIT_OUT_F32 ? 4 : 2);
  const size_t wsb = gemv_workspace_bytes(L->out_features, L->in_features, batch);
  if (overlap(workspace, wsb, y, yb) || overlaps_layer(workspace, wsb, L)) return RABIT_EINVAL;
  return dev_status(launch_gemv_reduce(L->out_features, L->in_features, batch, y, y_dtype,
                                       workspace, (hipStream_t)stream, L->n_paths));
}

int rabit_gemm(const rabit_layer* L, const uint16_t* X, int32_t m, void* Y, int32_t y_dtype,
               void* workspace, size_t workspace_bytes, void* stream) {
  return rabit_gemm_ex(L, X, m, Y, y_dtype, 0u, workspace, workspace_bytes, stream);
}

int rabit_gemm_ex(const rabit_layer* L, const uint16_t* X, int32_t m, void* Y, int32_t y_dtype,
                  uint32_t flags, void* workspace, size_t workspace_bytes, void* stream) {
  if (flags & ~RABIT_GEMM_WEFF) return RABIT_EINVAL;
  int s = check_layer(L);
  if (s) return s;
  if (!gemm_planes_fit(L)) return RABIT_ESHAPE;
  if (!X || !Y) return RABIT_EINVAL;
  if (y_dtype != RABIT_OUT_F32 && y_dtype != RABIT_OUT_BF16) return RABIT_EINVAL;
  if (m < 1 || m > RABIT_MAX_GEMM_M) return RABIT_ESHAPE;
  if (!aligned16(X) || !aligned16(Y)) return RABIT_EALIGN;
  const int out = L->out_features, in = L->in_features;
  const size_t yb = (size_t)m * out * (y_dtype == RABIT_OUT_F32 ? 4 : 2);
  if (overlap(Y, yb, X, (size_t)m * in * 2) ||
      overlap(Y, yb, L->planes, rabit_planes_bytes(out, in, L->n_paths)))
    return RABIT_EINVAL;
  if (!workspace || workspace_bytes < gemm_workspace_bytes(out, in, m)) return RABIT_EWORKSPACE;
  if (!aligned16(workspace)) return RABIT_EALIGN;
  return dev_status(launch_gemm((const uint4*)L->planes, L->g, L->h, out, in, X, m, Y, y_dtype,
                                workspace, (hipStream_t)stream, L->n_paths,
                                (flags & RABIT_GEMM_WEFF) != 0));
}

// --------------------------------------------------------------------------
// training side
// --------------------------------------------------------------------------
size_t rabit_grad_input_workspace_bytes(int32_t out, int32_t in, int32_t m) {
  if (check_dims(out, in) || m < 1 || m > RABIT_MAX_GEMM_M) return 0;
  return std::max(grad_input_workspace_bytes(out, in, m, 2), grad_input_workspace_bytes(out, in, m, 3));
}

size_t rabit_grad_weight_workspace_bytes(int32_t out, int32_t in) {
  if (check_dims(out, in)) return 0;
  return std::max(grad_weight_workspace_bytes(out, in, 2), grad_weight_workspace_bytes(out, in, 3));
}

int rabit_transpose_planes(const rabit_layer* L, void* planes_t, void* stream) {
  int s = check_layer(L);
  if (s) return s;
  if (!planes_t) return RABIT_EINVAL;
  if (!aligned16(planes_t)) return RABIT_EALIGN;
  const int out = L->out_features, in = L->in_features, P = L->n_paths;
  if (overlaps_layer(planes_t, rabit_planes_bytes(in, out, P), L)) return RABIT_EINVAL;
  return dev_status(launch_transpose_planes((const uint4*)L->planes, out, in, P, (uint4*)planes_t,
                                            (hipStream_t)stream));
}

int rabit_grad_input(const rabit_layer* L, const uint16_t* dY, int32_t m, void* dX,
                     int32_t dx_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return rabit_grad_input_ex(L, dY, m, dX, dx_dtype, 0u, workspace, workspace_bytes, stream);
}

int rabit_grad_input_ex(const rabit_layer* L, const uint16_t* dY, int32_t m, void* dX,
                        int32_t dx_dtype, uint32_t flags, void* workspace, size_t workspace_bytes,
                        void* stream) {
  if (flags & ~RABIT_GEMM_WEFF) return RABIT_EINVAL;
  int s = check_layer(L);
  if (s) return s;
  if (!gemm_planes_fit(L)) return RABIT_ESHAPE;
  if (!dY || !dX) return RABIT_EINVAL;
  if (dx_dtype != RABIT_OUT_F32 && dx_dtype != RABIT_OUT_BF16) return RABIT_EINVAL;
  if (m < 1 || m > RABIT_MAX_GEMM_M) return RABIT_ESHAPE;
  if (!aligned16(dY) || !aligned16(dX)) return RABIT_EALIGN;
  const int out = L->out_features, in = L->in_features, P = L->n_paths;
  const size_t xb = (size_t)m * in * (dx_dtype == RABIT_OUT_F32 ? 4 : 2);
  if (overlap(dX, xb, dY, (size_t)m * out * 2) || overlaps_layer(dX, xb, L)) return RABIT_EINVAL;
  if (!workspace || workspace_bytes < grad_input_workspace_bytes(out, in, m, P))
    return RABIT_EWORKSPACE;
  if (!aligned16(workspace)) return RABIT_EALIGN;
  return dev_status(launch_grad_input((const uint4*)L->planes, L->g, L->h, out, in, P, dY, m, dX,
                                      dx_dtype, workspace, (hipStream_t)stream,
                                      (flags & RABIT_GEMM_WEFF) != 0));
}

int rabit_grad_weight(const rabit_layer* L, const uint16_t* X, const uint16_t* dY, int32_t m,
                      float* dW, float* dg, float* dh, uint32_t flags, void* workspace,
                      size_t workspace_bytes, void* stream) {
  int s = check_layer(L);
  if (s) return s;
  if (!X || !dY || !dW || !dg || !dh) return RABIT_EINVAL;
  if (flags & ~RABIT_GRAD_ACCUMULATE) return RABIT_EINVAL;
  if (m < 1 || m > RABIT_MAX_GEMM_M) return RABIT_ESHAPE;
  if (!aligned16(X) || !aligned16(dY) || !aligned16(dW) || !aligned16(dg) || !aligned16(dh))
    return RABIT_EALIGN;
  const int out = L->out_features, in = L->in_features, P = L->n_paths;
  const size_t wb = (size_t)out * in * 4, gb = (size_t)P * out * 4, hb = (size_t)P * in * 4;
  const size_t xb = (size_t)m * in * 2, yb = (size_t)m * out * 2;
  const void* outs[3] = {dW, dg, dh};
  const size_t ob[3] = {wb, gb, hb};
  for (int a = 0; a < 3; ++a) {
    if (overlap(outs[a], ob[a], X, xb) || overlap(outs[a], ob[a], dY, yb) ||
        overlaps_layer(outs[a], ob[a], L))
      return RABIT_EINVAL;
    for (int b = a + 1; b < 3; ++b)
      if (overlap(outs[a], ob[a], outs[b], ob[b])) return RABIT_EINVAL;
  }
  if (!workspace || workspace_bytes < grad_weight_workspace_bytes(out, in, P))
    return RABIT_EWORKSPACE;
  if (!aligned16(workspace)) return RABIT_EALIGN;
  return dev_status(launch_grad_weight((const uint4*)L->planes, L->g, L->h, out, in, P, X, dY, m,
                                       dW, dg, dh, (flags & RABIT_GRAD_ACCUMULATE) ? 1 : 0,
                                       workspace, (hipStream_t)stream));
}

// --------------------------------------------------------------------------
// initialisation (iterative residual SVID)
// --------------------------------------------------------------------------
size_t rabit_svid_workspace_bytes(int32_t out, int32_t in) {
  if (check_dims(out, in)) return 0;
  return svid_workspace_bytes(out, in);
}

int rabit_svid_init(const float* W, int32_t out, int32_t in, int32_t n_paths, int32_t sweeps,
                    int32_t passes, const float* f_out, const float* f_in, uint32_t flags, float* g,
                    float* h, void* planes, void* workspace, size_t workspace_bytes, void* stream) {
  if (n_paths != 2 && n_paths != 3) return RABIT_EUNSUPPORTED;
  int s = check_dims(out, in);
  if (s) return s;
  if (sweeps < 1 || sweeps > 1000 || passes < 1 || passes > 63 || (passes & 1) == 0)
    return RABIT_ESHAPE;
  if (!W || !g || !h || !planes) return RABIT_EINVAL;
  if (flags & ~RABIT_SVID_CONTINUE) return RABIT_EINVAL;
  if (!aligned16(W) || !aligned16(g) || !aligned16(h) || !aligned16(planes) ||
      (f_out && !aligned16(f_out)) || (f_in && !aligned16(f_in)))
    return RABIT_EALIGN;
  const size_t wb = (size_t)out * in * 4, gb = (size_t)n_paths * out * 4,
               hb = (size_t)n_paths * in * 4, pb = rabit_planes_bytes(out, in, n_paths);
  const void* outs[3] = {g, h, planes};
  const size_t ob[3] = {gb, hb, pb};
  for (int a = 0; a < 3; ++a) {
    if (overlap(outs[a], ob[a], W, wb) || (f_out && overlap(outs[a], ob[a], f_out, (size_t)out * 4)) ||
        (f_in && overlap(outs[a], ob[a], f_in, (size_t)in * 4)))
      return RABIT_EINVAL;
    for (int b = a + 1; b < 3; ++b)
      if (overlap(outs[a], ob[a], outs[b], ob[b])) return RABIT_EINVAL;
  }
  if (!workspace || workspace_bytes < svid_workspace_bytes(out, in)) return RABIT_EWORKSPACE;
  if (!aligned16(workspace)) return RABIT_EALIGN;
  return dev_status(launch_svid(W, out, in, n_paths, sweeps, passes, f_out, f_in,
                                (flags & RABIT_SVID_CONTINUE) != 0, g, h, (uint4*)planes, workspace,
                                (hipStream_t)stream));
}

// --------------------------------------------------------------------------
// decode step
// --------------------------------------------------------------------------
namespace {

struct DecodeWs {
  uint16_t *xa, *xb, *n, *attn, *z;
  float *q, *k, *v, *o, *gate, *up, *down;
  // GEMV path (batch <= RABIT_MAX_GEMV_BATCH): partials and row statistics
  double *stats, *pq, *pk, *pv, *po, *pg, *pu, *pd;
  float* qk;
  void* lin;
  size_t lin_bytes;
};

size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }

int check_cfg(const rabit_decoder_cfg* c) {
  if (!c) return RABIT_EINVAL;
  if (c->hidden < 1 || c->ffn < 1 || c->n_layers < 1 || c->hidden > RABIT_MAX_FEATURES ||
      c->ffn > RABIT_MAX_FEATURES)
    return RABIT_ESHAPE;
  if (!c->mlp_only) {
    if (c->n_heads < 1 || c->n_kv_heads < 1 || c->head_dim < 1 || c->n_heads % c->n_kv_heads)
      return RABIT_ESHAPE;
    if ((int64_t)c->n_heads * c->head_dim != c->hidden) return RABIT_ESHAPE;
  }
  if (!(c->rms_eps > 0.0f)) return RABIT_EINVAL;
  return RABIT_OK;
}

size_t lin_ws(const rabit_decoder_cfg* c, int batch) {
  const int kv = c->mlp_only ? 0 : c->n_kv_heads * c->head_dim;
  size_t mx = 0;
  const int shapes[5][2] = {{c->hidden, c->hidden}, {kv, c->hidden}, {c->ffn, c->hidden},
                            {c->hidden, c->ffn}, {c->hidden, c->hidden}};
  for (auto& sh : shapes) {
    if (sh[0] < 1) continue;
    const size_t b = batch <= RABIT_MAX_GEMV_BATCH ? gemv_workspace_bytes(sh[0], sh[1], batch)
                                                   : gemm_workspace_bytes(sh[0], sh[1], batch);
    mx = std::max(mx, b);
  }
  return mx;
}

size_t decode_ws(const rabit_decoder_cfg* c, int batch, DecodeWs* w, void* base) {
  const int H = c->hidden, F = c->ffn;
  const int kv = c->mlp_only ? 0 : c->n_kv_heads * c->head_dim;
  const int kv1 = std::max(kv, 1);
  const bool gv = batch <= RABIT_MAX_GEMV_BATCH;
  size_t off = 0;
  char* p = (char*)base;
  auto take = [&](void** slot, size_t bytes) {
    *slot = (base && bytes) ? (void*)(p + off) : nullptr;
    off += a256(bytes);
  };
  take((void**)&w->xa, (size_t)batch * H * 2);
  take((void**)&w->xb, (size_t)batch * H * 2);
  take((void**)&w->attn, (size_t)batch * H * 2);
  take((void**)&w->z, (size_t)batch * F * 2);
  // GEMM path: normalised input and fp32 outputs of every linear layer
  take((void**)&w->n, gv ? 0 : (size_t)batch * H * 2);
  take((void**)&w->q, gv ? 0 : (size_t)batch * H * 4);
  take((void**)&w->k, gv ? 0 : (size_t)batch * kv1 * 4);
  take((void**)&w->v, gv ? 0 : (size_t)batch * kv1 * 4);
  take((void**)&w->o, gv ? 0 : (size_t)batch * H * 4);
  take((void**)&w->gate, gv ? 0 : (size_t)batch * F * 4);
  take((void**)&w->up, gv ? 0 : (size_t)batch * F * 4);
  take((void**)&w->down, gv ? 0 : (size_t)batch * H * 4);
  // GEMV path: x^2 partial sums, q/k outputs and the per-range partials
  take((void**)&w->stats, gv ? (size_t)batch * RABIT_STAT_PARTS * 8 : 0);
  take((void**)&w->qk, gv ? (size_t)batch * (H + kv1) * 4 : 0);
  take((void**)&w->pq, gv && kv ? gemv_part_bytes(H, H, batch) : 0);
  take((void**)&w->pk, gv && kv ? gemv_part_bytes(kv, H, batch) : 0);
  take((void**)&w->pv, gv && kv ? gemv_part_bytes(kv, H, batch) : 0);
  take((void**)&w->po, gv && kv ? gemv_part_bytes(H, H, batch) : 0);
  take((void**)&w->pg, gv ? gemv_part_bytes(F, H, batch) : 0);
  take((void**)&w->pu, gv ? gemv_part_bytes(F, H, batch) : 0);
  take((void**)&w->pd, gv ? gemv_part_bytes(H, F, batch) : 0);
  w->lin_bytes = gv ? 0 : lin_ws(c, batch);
  w->lin = (base && w->lin_bytes) ? p + off : nullptr;
  return off + w->lin_bytes;
}

extern "C++" LinSeg seg_of(const rabit_layer& L, double* part) {
  return LinSeg{(const uint4*)L.planes, L.g, L.h, L.out_features, part, L.n_paths};
}

// One decode step at batch <= RABIT_MAX_GEMV_BATCH. Per layer: [q,k,v] GEMV
// on RMSNorm(x) -> q/k/v sums + attention -> o GEMV -> x + o and its x^2
// sums -> [gate,up] GEMV on RMSNorm -> SiLU(gate)*up -> down GEMV -> x + down
// and its x^2 sums, plus one launch for the statistics of the step input.
// At batch 1 the o and down GEMVs form their inputs (attention, SiLU(gate)*up)
// from the previous launch's partials themselves: 6 launches per layer (3
// without attention); otherwise 8 (4).
hipError_t decode_gemv_path(const rabit_decoder_cfg* cfg, const rabit_layer* layers,
                            const uint16_t* x, int batch, uint16_t* out, const DecodeWs& w,
                            hipStream_t st) {
  const int H = cfg->hidden, F = cfg->ffn;
  const bool formed = batch == 1;
  hipError_t e = launch_resid_stats(nullptr, x, nullptr, w.stats, batch, H, st);
  const uint16_t* cur = x;
  for (int l = 0; l < cfg->n_layers && e == hipSuccess; ++l) {
    const rabit_layer* Ls = layers + l * 7;
    uint16_t* nxt = (l == cfg->n_layers - 1) ? out : (cur == w.xa ? w.xb : w.xa);
    if (!cfg->mlp_only) {
      const LinSeg qkv[3] = {seg_of(Ls[0], w.pq), seg_of(Ls[1], w.pk), seg_of(Ls[2], w.pv)};
      if (!e) e = launch_gemv_multi(qkv, 3, H, cur, batch, w.stats, cfg->rms_eps, st);
      const LinSeg o = seg_of(Ls[3], w.po);
      if (formed) {
        GemvXSrc xs;
        xs.mode = XSRC_ATTN;
        xs.pa = w.pv;
        xs.head_dim = cfg->head_dim;
        xs.rep = cfg->n_heads / cfg->n_kv_heads;
        xs.pq = w.pq;
        xs.pk = w.pk;
        xs.qk = w.qk;
        xs.n_q = H;
        xs.kv = cfg->n_kv_heads * cfg->head_dim;
        if (!e) e = launch_gemv_multi(&o, 1, H, nullptr, batch, nullptr, 0.f, st, &xs);
      } else {
        if (!e) e = launch_reduce_attn(w.pq, w.pk, w.pv, w.qk, w.attn, batch, cfg->n_heads,
                                       cfg->n_kv_heads, cfg->head_dim, st);
        if (!e) e = launch_gemv_multi(&o, 1, H, w.attn, batch, nullptr, 0.f, st);
      }
      if (!e) e = launch_resid_stats(w.po, cur, nxt, w.stats, batch, H, st);
      cur = nxt;
    }
    const LinSeg gu[2] = {seg_of(Ls[4], w.pg), seg_of(Ls[5], w.pu)};
    if (!e) e = launch_gemv_multi(gu, 2, H, cur, batch, w.stats, cfg->rms_eps, st);
    const LinSeg dn = seg_of(Ls[6], w.pd);
    if (formed) {
      GemvXSrc xs;
      xs.mode = XSRC_SILU;
      xs.pa = w.pg;
      xs.pb = w.pu;
      if (!e) e = launch_gemv_multi(&dn, 1, F, nullptr, batch, nullptr, 0.f, st, &xs);
    } else {
      if (!e) e = launch_reduce_silu(w.pg, w.pu, w.z, batch, F, st);
      if (!e) e = launch_gemv_multi(&dn, 1, F, w.z, batch, nullptr, 0.f, st);
    }
    // x + down may be written in place (cur == nxt when attention ran)
    if (!e) e = launch_resid_stats(w.pd, cur, nxt, w.stats, batch, H, st);
    cur = nxt;
  }
  return e;
}

hipError_t linear(const rabit_layer& L, const uint16_t* x, int batch, float* y, const DecodeWs& w,
                  hipStream_t st) {
  if (batch <= RABIT_MAX_GEMV_BATCH)
    return launch_gemv((const uint4*)L.planes, L.g, L.h, L.out_features, L.in_features, x, batch,
                       y, RABIT_OUT_F32, w.lin, st, L.n_paths);
  return launch_gemm((const uint4*)L.planes, L.g, L.h, L.out_features, L.in_features, x, batch, y,
                     RABIT_OUT_F32, w.lin, st, L.n_paths);
}

}  // namespace

size_t rabit_decode_workspace_bytes(const rabit_decoder_cfg* cfg, int32_t batch) {
  if (check_cfg(cfg) || batch < 1 || batch > RABIT_MAX_GEMM_M) return 0;
  DecodeWs w;
  return decode_ws(cfg, batch, &w, nullptr);
}

int rabit_decode_step(const rabit_decoder_cfg* cfg, const rabit_layer* layers, const uint16_t* x,
                      int32_t batch, uint16_t* out, void* workspace, size_t workspace_bytes,
                      void* stream) {
  int s = check_cfg(cfg);
  if (s) return s;
  if (!layers || !x || !out) return RABIT_EINVAL;
  if (batch < 1 || batch > RABIT_MAX_GEMM_M) return RABIT_ESHAPE;
  if (!aligned16(x) || !aligned16(out)) return RABIT_EALIGN;
  const int H = cfg->hidden, F = cfg->ffn;
  const int kv = cfg->mlp_only ? 0 : cfg->n_kv_heads * cfg->head_dim;
  for (int l = 0; l < cfg->n_layers; ++l) {
    for (int m = cfg->mlp_only ? 4 : 0; m < 7; ++m) {
      const rabit_layer& L = layers[l * 7 + m];
      // 2 or 3 paths, the same number in every layer
      if ((s = check_layer(&L))) return s;
      if (L.n_paths != layers[(cfg->mlp_only ? 4 : 0)].n_paths) return RABIT_EUNSUPPORTED;
      static const int kOut[7] = {0, 1, 1, 0, 2, 2, 0}, kIn[7] = {0, 0, 0, 0, 0, 0, 2};
      const int want_out = kOut[m] == 0 ? H : (kOut[m] == 1 ? kv : F);
      const int want_in = kIn[m] == 0 ? H : F;
      if (L.out_features != want_out || L.in_features != want_in) return RABIT_ESHAPE;
    }
  }
  DecodeWs w;
  const size_t need = decode_ws(cfg, batch, &w, nullptr);
  if (!workspace || workspace_bytes < need) return RABIT_EWORKSPACE;
  if (!aligned16(workspace)) return RABIT_EALIGN;
  decode_ws(cfg, batch, &w, workspace);
  hipStream_t st = (hipStream_t)stream;
  if (batch <= RABIT_MAX_GEMV_BATCH)
    return dev_status(decode_gemv_path(cfg, layers, x, batch, out, w, st));
  hipError_t e = hipSuccess;
  const uint16_t* cur = x;
  for (int l = 0; l < cfg->n_layers && e == hipSuccess; ++l) {
    const rabit_layer* Ls = layers + l * 7;
    uint16_t* nxt = (l == cfg->n_layers - 1) ? out : (cur == w.xa ? w.xb : w.xa);
    if (!cfg->mlp_only) {
      if (!e) e = launch_rmsnorm(cur, w.n, batch, H, cfg->rms_eps, st);
      if (!e) e = linear(Ls[0], w.n, batch, w.q, w, st);
      if (!e) e = linear(Ls[1], w.n, batch, w.k, w, st);
      if (!e) e = linear(Ls[2], w.n, batch, w.v, w, st);
      if (!e) e = launch_attn_1tok(w.v, kv, w.attn, batch, cfg->n_heads, cfg->n_kv_heads,
                                   cfg->head_dim, st);
      if (!e) e = linear(Ls[3], w.attn, batch, w.o, w, st);
      if (!e) e = launch_residual_add(cur, w.o, nxt, batch, H, st);
      cur = nxt;
    }
    if (!e) e = launch_rmsnorm(cur, w.n, batch, H, cfg->rms_eps, st);
    if (!e) e = linear(Ls[4], w.n, batch, w.gate, w, st);
    if (!e) e = linear(Ls[5], w.n, batch, w.up, w, st);
    if (!e) e = launch_silu_mul(w.gate, w.up, w.z, batch, F, st);
    if (!e) e = linear(Ls[6], w.z, batch, w.down, w, st);
    // the residual may write in place (cur == nxt when attention ran)
    if (!e) e = launch_residual_add(cur, w.down, nxt, batch, H, st);
    cur = nxt;
  }
  return dev_status(e);
}

int rabit_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (!src || !sink) return RABIT_EINVAL;
  if (!aligned16(src) || !aligned16(sink) || bytes % 16) return RABIT_EALIGN;
  return dev_status(launch_stream_read(src, bytes, sink, (hipStream_t)stream));
}

int rabit_test_f64_to_16(const double* in, uint16_t* out, int32_t n, int32_t bf16, void* stream) {
  if (!in || !out || n < 1) return RABIT_EINVAL;
  return dev_status(launch_test_f64_to_16(in, out, n, bf16, (hipStream_t)stream));
}

}  // extern "C"
