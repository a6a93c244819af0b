// gdn_api.hip -- the C ABI of libgdn.so: argument checks on the host, then
// the launchers.  Nothing here allocates, synchronises or reads environment
// variables; a failed check returns before anything is enqueued.
#include <math.h>
#include <string.h>

#include <mutex>

#include "gdn.h"
#include "gdn_launch.h"

namespace {

using gdn::Dims;

gdn_status_t resolve(const gdn_config_t* cfg, Dims* d) {
  if (!cfg) return GDN_ERR_INVALID_ARG;
  if (cfg->num_k_heads <= 0 || cfg->num_v_heads <= 0) return GDN_ERR_INVALID_ARG;
  if (cfg->num_v_heads % cfg->num_k_heads != 0) return GDN_ERR_INVALID_ARG;
  if (cfg->head_k_dim != 128 || cfg->head_v_dim != 128) return GDN_ERR_UNSUPPORTED;
  if (cfg->conv_width != 4 || cfg->chunk_size != 64) return GDN_ERR_UNSUPPORTED;
  if (cfg->conv_act != 0 && cfg->conv_act != 1) return GDN_ERR_INVALID_ARG;
  if (cfg->decay_per_key_channel != 0 && cfg->decay_per_key_channel != 1) return GDN_ERR_INVALID_ARG;
  if (cfg->qk_l2norm != 0 && cfg->qk_l2norm != 1) return GDN_ERR_INVALID_ARG;
  if (!(cfg->l2_eps >= 0.0f) || !(cfg->rms_eps >= 0.0f)) return GDN_ERR_INVALID_ARG;
  d->hk = cfg->num_k_heads;
  d->hv = cfg->num_v_heads;
  d->dk = cfg->head_k_dim;
  d->dv = cfg->head_v_dim;
  d->cc = 2 * d->hk * d->dk + d->hv * d->dv;
  d->act = cfg->conv_act;
  d->per_channel = cfg->decay_per_key_channel;
  d->l2norm = cfg->qk_l2norm;
  d->l2_eps = cfg->l2_eps;
  d->rms_eps = cfg->rms_eps;
  d->q_scale = cfg->q_scale > 0.0f ? cfg->q_scale : 1.0f / sqrtf((float)cfg->head_k_dim);
  return GDN_OK;
}

bool valid_dtype(gdn_dtype_t t) { return t == GDN_F32 || t == GDN_BF16; }
size_t dsize(gdn_dtype_t t) { return t == GDN_BF16 ? 2 : 4; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Byte ranges [a, a+na) and [b, b+nb) overlap.
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return na && nb && pa < pb + nb && pb < pa + na;
}

gdn_status_t check_seqlens(const int32_t* cu_host, int32_t n, int32_t t) {
  if (!cu_host || n < 0 || t < 0) return GDN_ERR_INVALID_ARG;
  if (cu_host[0] != 0 || cu_host[n] != t) return GDN_ERR_SEQLENS;
  for (int32_t i = 0; i < n; ++i)
    if (cu_host[i + 1] < cu_host[i]) return GDN_ERR_SEQLENS;
  return GDN_OK;
}

gdn_status_t hip_status(hipError_t e) { return e == hipSuccess ? GDN_OK : GDN_ERR_HIP; }

size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

// The gates of a call: fp32 g / beta (g 16-byte aligned, it is read as vectors
// with per-key-channel decay), or the a / b projections with A_log and dt_bias
// (scalar decay only).
gdn_status_t check_gates(const Dims& d, const gdn::Gates& gt, bool any_rows) {
  if (gt.a || gt.b || gt.A_log || gt.dt_bias) {
    if (d.per_channel) return GDN_ERR_UNSUPPORTED;
    if (any_rows && (!gt.a || !gt.b || !gt.A_log || !gt.dt_bias)) return GDN_ERR_INVALID_ARG;
    return GDN_OK;
  }
  if (any_rows && (!gt.g || !gt.beta)) return GDN_ERR_INVALID_ARG;
  if (any_rows && !aligned16(gt.g)) return GDN_ERR_INVALID_ARG;
  return GDN_OK;
}

gdn::Gates given_gates(const float* g, const float* beta) { return gdn::Gates{g, beta, nullptr, nullptr, nullptr, nullptr}; }
gdn::Gates derived_gates(const void* a, const void* b, const float* A_log, const float* dt_bias) {
  return gdn::Gates{nullptr, nullptr, a, b, A_log, dt_bias};
}

// gdn_prefill workspace: the conv output [T][Cc] | the chunk workspace | the
// fp32 pre-norm output [T][Hv][dv] when the chunk kernels do not apply the norm
struct PrefillWs {
  size_t y, chunk, o, total;
};
PrefillWs prefill_ws(const Dims& d, bool bf16, int32_t n, int32_t t) {
  PrefillWs w;
  w.y = 0;
  w.chunk = round256((size_t)t * d.cc * (bf16 ? 2 : 4));
  w.o = w.chunk + round256(gdn::chunk_workspace_bytes(d, n, t));
  w.total = w.o + (gdn::chunk_fuses_norm(d, bf16, n) ? 0 : (size_t)t * d.hv * d.dv * sizeof(float));
  return w;
}

}  // namespace

extern "C" {

int gdn_abi_version(void) { return GDN_ABI_VERSION; }

const char* gdn_status_string(gdn_status_t s) {
  switch (s) {
    case GDN_OK: return "ok";
    case GDN_ERR_INVALID_ARG: return "invalid argument";
    case GDN_ERR_UNSUPPORTED: return "unsupported geometry or dtype";
    case GDN_ERR_SEQLENS: return "invalid cu_seqlens";
    case GDN_ERR_WORKSPACE: return "workspace missing or too small";
    case GDN_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

gdn_status_t gdn_config_default(gdn_config_t* cfg) {
  if (!cfg) return GDN_ERR_INVALID_ARG;
  cfg->num_k_heads = 16;
  cfg->num_v_heads = 48;
  cfg->head_k_dim = 128;
  cfg->head_v_dim = 128;
  cfg->conv_width = 4;
  cfg->chunk_size = 64;
  cfg->conv_act = 1;
  cfg->decay_per_key_channel = 0;
  cfg->qk_l2norm = 1;
  cfg->l2_eps = 1e-6f;
  cfg->rms_eps = 1e-6f;
  cfg->q_scale = 1.0f / sqrtf(128.0f);
  return GDN_OK;
}

gdn_status_t gdn_conv1d_prefill(const gdn_config_t* cfg, gdn_dtype_t dtype, const void* x,
                                int64_t x_stride, const float* w, const void* conv_state_in,
                                void* conv_state_out, void* y, int64_t y_stride,
                                const int32_t* cu_dev, const int32_t* cu_host, int32_t N,
                                int32_t T, gdn_stream_t stream) {
  Dims d;
  gdn_status_t st = resolve(cfg, &d);
  if (st != GDN_OK) return st;
  if (!valid_dtype(dtype)) return GDN_ERR_UNSUPPORTED;
  if (N < 0 || T < 0) return GDN_ERR_INVALID_ARG;
  if (!cu_dev || !w) return GDN_ERR_INVALID_ARG;
  if (T > 0 && (!x || !y)) return GDN_ERR_INVALID_ARG;
  if (x_stride < d.cc || y_stride < d.cc || x_stride % 8 || y_stride % 8) return GDN_ERR_INVALID_ARG;
  if (T > 0 && (!aligned16(x) || !aligned16(y) || !aligned16(w))) return GDN_ERR_INVALID_ARG;
  st = check_seqlens(cu_host, N, T);
  if (st != GDN_OK) return st;
  const size_t es = dsize(dtype);
  if (T > 0 && overlaps(x, ((size_t)(T - 1) * x_stride + d.cc) * es, y, ((size_t)(T - 1) * y_stride + d.cc) * es))
    return GDN_ERR_INVALID_ARG;
  if (conv_state_in && !aligned16(conv_state_in)) return GDN_ERR_INVALID_ARG;
  return hip_status(gdn::launch_conv1d_prefill(d, dtype == GDN_BF16, x, x_stride, w, conv_state_in,
                                               conv_state_out, y, y_stride, cu_dev, N, T,
                                               static_cast<hipStream_t>(stream)));
}

gdn_status_t gdn_conv1d_step(const gdn_config_t* cfg, gdn_dtype_t dtype, const void* x,
                             int64_t x_stride, const float* w, void* conv_state, void* y,
                             int64_t y_stride, int32_t B, gdn_stream_t stream) {
  Dims d;
  gdn_status_t st = resolve(cfg, &d);
  if (st != GDN_OK) return st;
  if (!valid_dtype(dtype)) return GDN_ERR_UNSUPPORTED;
  if (B < 0) return GDN_ERR_INVALID_ARG;
  if (B > 0 && (!x || !w || !conv_state || !y)) return GDN_ERR_INVALID_ARG;
  if (x_stride < d.cc || y_stride < d.cc) return GDN_ERR_INVALID_ARG;
  if (B > 0 && !aligned16(w)) return GDN_ERR_INVALID_ARG;
  if (B > 65535) return GDN_ERR_INVALID_ARG;
  return hip_status(gdn::launch_conv1d_step(d, dtype == GDN_BF16, x, x_stride, w, conv_state, y,
                                            y_stride, B, static_cast<hipStream_t>(stream)));
}

gdn_status_t gdn_chunk_prefill_workspace_size(const gdn_config_t* cfg, int32_t N, int32_t T,
                                              size_t* bytes) {
  Dims d;
  gdn_status_t st = resolve(cfg, &d);
  if (st != GDN_OK) return st;
  if (!bytes || N < 0 || T < 0) return GDN_ERR_INVALID_ARG;
  *bytes = gdn::chunk_workspace_bytes(d, N, T);
  return GDN_OK;
}

static gdn_status_t chunk_prefill_checked(const gdn_config_t* cfg, gdn_dtype_t in_dtype,
                                          gdn_dtype_t out_dtype, const void* q, const void* k,
                                          int64_t qk_stride, const void* v, int64_t v_stride,
                                          const gdn::Gates& gt, const float* initial_state,
                                          const int32_t* cu_dev, const int32_t* cu_host, int32_t N,
                                          int32_t T, void* out, float* final_state, void* ws,
                                          size_t ws_bytes, gdn_stream_t stream) {
  Dims d;
  gdn_status_t st = resolve(cfg, &d);
  if (st != GDN_OK) return st;
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype)) return GDN_ERR_UNSUPPORTED;
  if (N < 0 || T < 0) return GDN_ERR_INVALID_ARG;
  if (!cu_dev) return GDN_ERR_INVALID_ARG;
  st = check_gates(d, gt, T > 0);
  if (st != GDN_OK) return st;
  if (T > 0 && (!q || !k || !v || !out)) return GDN_ERR_INVALID_ARG;
  const int64_t vec = in_dtype == GDN_BF16 ? 8 : 4;   // elements per 16-byte load
  if (qk_stride < (int64_t)d.hk * d.dk || v_stride < (int64_t)d.hv * d.dv) return GDN_ERR_INVALID_ARG;
  if (qk_stride % vec || v_stride % vec) return GDN_ERR_INVALID_ARG;
  if (T > 0 && (!aligned16(q) || !aligned16(k) || !aligned16(v))) return GDN_ERR_INVALID_ARG;
  if ((initial_state && !aligned16(initial_state)) || (final_state && !aligned16(final_state)))
    return GDN_ERR_INVALID_ARG;
  st = check_seqlens(cu_host, N, T);
  if (st != GDN_OK) return st;
  if ((size_t)N * d.hk > (size_t)1 << 24) return GDN_ERR_INVALID_ARG;
  const size_t need = gdn::chunk_workspace_bytes(d, N, T);
  if (N > 0 && (!ws || ws_bytes < need || !aligned16(ws))) return GDN_ERR_WORKSPACE;
  const size_t out_bytes = (size_t)T * d.hv * d.dv * dsize(out_dtype);
  const size_t state_bytes = (size_t)N * d.hv * d.dv * d.dk * sizeof(float);
  if (overlaps(out, out_bytes, ws, need) || overlaps(final_state, state_bytes, ws, need))
    return GDN_ERR_INVALID_ARG;
  return hip_status(gdn::launch_chunk_prefill(d, in_dtype == GDN_BF16, out_dtype == GDN_BF16, q, k,
                                              qk_stride, v, v_stride, gt, initial_state,
                                              cu_dev, cu_host, N, T, out, final_state, ws,
                                              ws_bytes, nullptr, nullptr,
                                              static_cast<hipStream_t>(stream)));
}

gdn_status_t gdn_prefill_workspace_size(const gdn_config_t* cfg, gdn_dtype_t dtype, int32_t N,
                                        int32_t T, size_t* bytes) {
  Dims d;
  gdn_status_t st = resolve(cfg, &d);
  if (st != GDN_OK) return st;
  if (!valid_dtype(dtype)) return GDN_ERR_UNSUPPORTED;
  if (!bytes || N < 0 || T < 0) return GDN_ERR_INVALID_ARG;
  *bytes = prefill_ws(d, dtype == GDN_BF16, N, T).total;
  return GDN_OK;
}

static gdn_status_t prefill_checked(const gdn_config_t* cfg, gdn_dtype_t dtype, gdn_dtype_t out_dtype,
                                    const void* x, int64_t x_stride, const float* conv_w,
                                    const void* conv_state_in, void* conv_state_out, const gdn::Gates& gt,
                                    const void* z, const float* norm_w, const float* initial_state,
                                    const int32_t* cu_dev, const int32_t* cu_host, int32_t N, int32_t T,
                                    void* out, float* final_state, void* ws, size_t ws_bytes,
                                    gdn_stream_t stream) {
  Dims d;
  gdn_status_t st = resolve(cfg, &d);
  if (st != GDN_OK) return st;
  if (!valid_dtype(dtype) || !valid_dtype(out_dtype)) return GDN_ERR_UNSUPPORTED;
  if (N < 0 || T < 0 || !cu_dev || !conv_w) return GDN_ERR_INVALID_ARG;
  st = check_gates(d, gt, T > 0);
  if (st != GDN_OK) return st;
  if (T > 0 && (!x || !z || !norm_w || !out)) return GDN_ERR_INVALID_ARG;
  if (x_stride < d.cc || x_stride % 8) return GDN_ERR_INVALID_ARG;
  if (T > 0 && (!aligned16(x) || !aligned16(conv_w) || !aligned16(z) || !aligned16(norm_w) ||
                !aligned16(out)))
    return GDN_ERR_INVALID_ARG;
  if ((conv_state_in && !aligned16(conv_state_in)) || (initial_state && !aligned16(initial_state)) ||
      (final_state && !aligned16(final_state)))
    return GDN_ERR_INVALID_ARG;
  st = check_seqlens(cu_host, N, T);
  if (st != GDN_OK) return st;
  if ((size_t)N * d.hk > (size_t)1 << 24) return GDN_ERR_INVALID_ARG;
  const bool bf16 = dtype == GDN_BF16;
  const PrefillWs wl = prefill_ws(d, bf16, N, T);
  if (N > 0 && (!ws || ws_bytes < wl.total || !aligned16(ws))) return GDN_ERR_WORKSPACE;
  const size_t es = dsize(dtype);
  const size_t out_bytes = (size_t)T * d.hv * d.dv * dsize(out_dtype);
  const size_t state_bytes = (size_t)N * d.hv * d.dv * d.dk * sizeof(float);
  const size_t x_bytes = T > 0 ? ((size_t)(T - 1) * x_stride + d.cc) * es : 0;
  const size_t z_bytes = (size_t)T * d.hv * d.dv * es;
  if (overlaps(out, out_bytes, ws, wl.total) || overlaps(out, out_bytes, x, x_bytes) ||
      overlaps(out, out_bytes, z, z_bytes) || overlaps(final_state, state_bytes, ws, wl.total) ||
      overlaps(ws, wl.total, x, x_bytes) || overlaps(ws, wl.total, z, z_bytes) ||
      overlaps(conv_state_out, (size_t)N * 3 * d.cc * es, ws, wl.total))
    return GDN_ERR_INVALID_ARG;
  if (N == 0) return GDN_OK;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* w8 = static_cast<uint8_t*>(ws);
  void* y = w8 + wl.y;
  hipError_t e = gdn::launch_conv1d_prefill(d, bf16, x, x_stride, conv_w, conv_state_in,
                                            conv_state_out, y, d.cc, cu_dev, N, T, s);
  if (e != hipSuccess) return GDN_ERR_HIP;
  // q | k | v are column blocks of the conv output rows
  const size_t kq = (size_t)d.hk * d.dk * es;
  const void* q = y;
  const void* k = static_cast<uint8_t*>(y) + kq;
  const void* v = static_cast<uint8_t*>(y) + 2 * kq;
  if (gdn::chunk_fuses_norm(d, bf16, N)) {
    // bf16 here: the gate comes in the activations' dtype
    return hip_status(gdn::launch_chunk_prefill(d, bf16, out_dtype == GDN_BF16, q, k, d.cc, v, d.cc,
                                                gt, initial_state, cu_dev, cu_host, N, T, out,
                                                final_state, w8 + wl.chunk, wl.o - wl.chunk,
                                                static_cast<const uint16_t*>(z), norm_w, s));
  }
  // the pre-norm output: fp16 where the spine rounds its operands to fp16 anyway
  // (half the bytes of the round trip through memory), else fp32
  void* o = w8 + wl.o;
  const bool o_f16 = gdn::chunk_out_f16(d, bf16, N);
  e = gdn::launch_chunk_prefill(d, bf16, false, q, k, d.cc, v, d.cc, gt, initial_state, cu_dev,
                                cu_host, N, T, o, final_state, w8 + wl.chunk, wl.o - wl.chunk,
                                nullptr, nullptr, s, o_f16);
  if (e != hipSuccess) return GDN_ERR_HIP;
  if (o_f16)
    return hip_status(gdn::launch_gated_rmsnorm_f16o(d, bf16, out_dtype == GDN_BF16, o, z, norm_w, out, T, s));
  return hip_status(gdn::launch_gated_rmsnorm(d, false, bf16, out_dtype == GDN_BF16, o, z, norm_w,
                                              out, T, s));
}

gdn_status_t gdn_gated_rmsnorm(const gdn_config_t* cfg, gdn_dtype_t o_dtype, gdn_dtype_t z_dtype,
                               gdn_dtype_t out_dtype, const void* o, const void* z,
                               const float* w, void* out, int64_t rows, gdn_stream_t stream) {
  Dims d;
  gdn_status_t st = resolve(cfg, &d);
  if (st != GDN_OK) return st;
  if (!valid_dtype(o_dtype) || !valid_dtype(z_dtype) || !valid_dtype(out_dtype)) return GDN_ERR_UNSUPPORTED;
  if (rows < 0) return GDN_ERR_INVALID_ARG;
  if (rows > 0 && (!o || !z || !w || !out)) return GDN_ERR_INVALID_ARG;
  if (rows > 0 && (!aligned16(o) || !aligned16(z) || !aligned16(w) || !aligned16(out)))
    return GDN_ERR_INVALID_ARG;
  if (out != o && rows > 0) {
    const size_t n = (size_t)rows * d.hv * d.dv;
    if (overlaps(out, n * dsize(out_dtype), o, n * dsize(o_dtype))) return GDN_ERR_INVALID_ARG;
  }
  if (rows == 0) return GDN_OK;   // (empty buffers may share a null address)
  if (out == o && o_dtype != out_dtype) return GDN_ERR_INVALID_ARG;
  return hip_status(gdn::launch_gated_rmsnorm(d, o_dtype == GDN_BF16, z_dtype == GDN_BF16,
                                              out_dtype == GDN_BF16, o, z, w, out, rows,
                                              static_cast<hipStream_t>(stream)));
}

static gdn_status_t decode_step_checked(const gdn_config_t* cfg, gdn_dtype_t dtype, gdn_dtype_t out_dtype,
                                        const void* x, const float* conv_w, void* conv_state,
                                        const gdn::Gates& gt, const void* z, const float* norm_w,
                                        void* state, bool state_f16, void* out, int32_t B,
                                        gdn_stream_t stream) {
  Dims d;
  gdn_status_t st = resolve(cfg, &d);
  if (st != GDN_OK) return st;
  if (!valid_dtype(dtype) || !valid_dtype(out_dtype)) return GDN_ERR_UNSUPPORTED;
  // the q / k conv-state shift that follows the step (Hk < Hv) puts the
  // sequences on grid.y: checked here so that a refused launch can never leave
  // a half-applied step behind
  if (B < 0 || B > 65535) return GDN_ERR_INVALID_ARG;
  if ((int64_t)B * d.hv > INT32_MAX) return GDN_ERR_INVALID_ARG;   // one workgroup per (sequence, value head)
  st = check_gates(d, gt, B > 0);
  if (st != GDN_OK) return st;
  if (B > 0 && (!x || !conv_w || !conv_state || !z || !norm_w || !state || !out))
    return GDN_ERR_INVALID_ARG;
  if (B > 0 && (!aligned16(conv_w) || !aligned16(state))) return GDN_ERR_INVALID_ARG;
  return hip_status(gdn::launch_decode_step(d, dtype == GDN_BF16, out_dtype == GDN_BF16, x, conv_w,
                                            conv_state, gt, z, norm_w, state, state_f16, out, B,
                                            static_cast<hipStream_t>(stream)));
}


gdn_status_t gdn_chunk_prefill(const gdn_config_t* cfg, gdn_dtype_t in_dtype,
                               gdn_dtype_t out_dtype, const void* q, const void* k,
                               int64_t qk_stride, const void* v, int64_t v_stride,
                               const float* g, const float* beta, const float* initial_state,
                               const int32_t* cu_dev, const int32_t* cu_host, int32_t N,
                               int32_t T, void* out, float* final_state, void* ws,
                               size_t ws_bytes, gdn_stream_t stream) {
  return chunk_prefill_checked(cfg, in_dtype, out_dtype, q, k, qk_stride, v, v_stride, given_gates(g, beta),
                               initial_state, cu_dev, cu_host, N, T, out, final_state, ws, ws_bytes, stream);
}

// ---------------------------------------------------------------------------
// gdn_chunk_prefill_noalloc: the chunk workspace in a fixed device array.
// Each GPU the library runs on holds its own copy of `scratch` from module load
// until the process ends.  In host code the array's name is not a device
// address, so its address is looked up once per device (with that device
// current) and only that pointer is ever handed to the kernels.
// ---------------------------------------------------------------------------
namespace {
constexpr int kMaxDevices = 64;
static __device__ __align__(256) uint8_t scratch[GDN_NOALLOC_SCRATCH_BYTES];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

gdn_status_t scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GDN_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return GDN_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return GDN_OK;
}
}  // namespace

gdn_status_t gdn_chunk_prefill_noalloc(const gdn_config_t* cfg, gdn_dtype_t in_dtype,
                                       gdn_dtype_t out_dtype, const void* q, const void* k,
                                       int64_t qk_stride, const void* v, int64_t v_stride,
                                       const float* g, const float* beta, const float* initial_state,
                                       const int32_t* cu_dev, const int32_t* cu_host, int32_t N,
                                       int32_t T, void* out, float* final_state, gdn_stream_t stream) {
  Dims d;
  gdn_status_t st = resolve(cfg, &d);
  if (st != GDN_OK) return st;
  if (N < 0 || T < 0) return GDN_ERR_INVALID_ARG;
  if (gdn::chunk_workspace_bytes(d, N, T) > (size_t)GDN_NOALLOC_SCRATCH_BYTES) return GDN_ERR_WORKSPACE;
  if (N == 0) return GDN_OK;
  void* ws = nullptr;
  st = scratch_on_current_device(&ws);
  if (st != GDN_OK) return st;
  return chunk_prefill_checked(cfg, in_dtype, out_dtype, q, k, qk_stride, v, v_stride, given_gates(g, beta),
                               initial_state, cu_dev, cu_host, N, T, out, final_state, ws,
                               (size_t)GDN_NOALLOC_SCRATCH_BYTES, stream);
}

gdn_status_t gdn_chunk_prefill_ab(const gdn_config_t* cfg, gdn_dtype_t in_dtype,
                                  gdn_dtype_t out_dtype, const void* q, const void* k,
                                  int64_t qk_stride, const void* v, int64_t v_stride,
                                  const void* a, const void* b, const float* A_log,
                                  const float* dt_bias, const float* initial_state,
                                  const int32_t* cu_dev, const int32_t* cu_host, int32_t N,
                                  int32_t T, void* out, float* final_state, void* ws,
                                  size_t ws_bytes, gdn_stream_t stream) {
  return chunk_prefill_checked(cfg, in_dtype, out_dtype, q, k, qk_stride, v, v_stride,
                               derived_gates(a, b, A_log, dt_bias), initial_state, cu_dev, cu_host, N, T,
                               out, final_state, ws, ws_bytes, stream);
}

gdn_status_t gdn_prefill(const gdn_config_t* cfg, gdn_dtype_t dtype, gdn_dtype_t out_dtype,
                         const void* x, int64_t x_stride, const float* conv_w,
                         const void* conv_state_in, void* conv_state_out, const float* g,
                         const float* beta, const void* z, const float* norm_w,
                         const float* initial_state, const int32_t* cu_dev, const int32_t* cu_host,
                         int32_t N, int32_t T, void* out, float* final_state, void* ws,
                         size_t ws_bytes, gdn_stream_t stream) {
  return prefill_checked(cfg, dtype, out_dtype, x, x_stride, conv_w, conv_state_in, conv_state_out,
                         given_gates(g, beta), z, norm_w, initial_state, cu_dev, cu_host, N, T, out,
                         final_state, ws, ws_bytes, stream);
}

gdn_status_t gdn_prefill_ab(const gdn_config_t* cfg, gdn_dtype_t dtype, gdn_dtype_t out_dtype,
                            const void* x, int64_t x_stride, const float* conv_w,
                            const void* conv_state_in, void* conv_state_out, const void* a,
                            const void* b, const float* A_log, const float* dt_bias, const void* z,
                            const float* norm_w, const float* initial_state, const int32_t* cu_dev,
                            const int32_t* cu_host, int32_t N, int32_t T, void* out,
                            float* final_state, void* ws, size_t ws_bytes, gdn_stream_t stream) {
  return prefill_checked(cfg, dtype, out_dtype, x, x_stride, conv_w, conv_state_in, conv_state_out,
                         derived_gates(a, b, A_log, dt_bias), z, norm_w, initial_state, cu_dev, cu_host,
                         N, T, out, final_state, ws, ws_bytes, stream);
}

gdn_status_t gdn_decode_step(const gdn_config_t* cfg, gdn_dtype_t dtype, gdn_dtype_t out_dtype,
                             const void* x, const float* conv_w, void* conv_state, const float* g,
                             const float* beta, const void* z, const float* norm_w, float* state,
                             void* out, int32_t B, gdn_stream_t stream) {
  return decode_step_checked(cfg, dtype, out_dtype, x, conv_w, conv_state, given_gates(g, beta), z, norm_w,
                             state, false, out, B, stream);
}

gdn_status_t gdn_decode_step_h16(const gdn_config_t* cfg, gdn_dtype_t dtype, gdn_dtype_t out_dtype,
                                 const void* x, const float* conv_w, void* conv_state, const float* g,
                                 const float* beta, const void* z, const float* norm_w, void* state,
                                 void* out, int32_t B, gdn_stream_t stream) {
  return decode_step_checked(cfg, dtype, out_dtype, x, conv_w, conv_state, given_gates(g, beta), z, norm_w,
                             state, true, out, B, stream);
}

gdn_status_t gdn_state_convert(const void* src, gdn_dtype_t src_dtype, void* dst, gdn_dtype_t dst_dtype,
                               int64_t n, gdn_stream_t stream) {
  const bool widen = src_dtype == GDN_F16 && dst_dtype == GDN_F32;
  const bool narrow = src_dtype == GDN_F32 && dst_dtype == GDN_F16;
  if (!widen && !narrow) return GDN_ERR_UNSUPPORTED;
  if (n < 0) return GDN_ERR_INVALID_ARG;
  if (n == 0) return GDN_OK;
  if (!src || !dst || !aligned16(src) || !aligned16(dst)) return GDN_ERR_INVALID_ARG;
  if (overlaps(src, (size_t)n * (widen ? 2 : 4), dst, (size_t)n * (widen ? 4 : 2))) return GDN_ERR_INVALID_ARG;
  return hip_status(gdn::launch_state_convert(src, widen, dst, n, static_cast<hipStream_t>(stream)));
}

gdn_status_t gdn_decode_step_ab(const gdn_config_t* cfg, gdn_dtype_t dtype, gdn_dtype_t out_dtype,
                                const void* x, const float* conv_w, void* conv_state, const void* a,
                                const void* b, const float* A_log, const float* dt_bias,
                                const void* z, const float* norm_w, float* state, void* out,
                                int32_t B, gdn_stream_t stream) {
  return decode_step_checked(cfg, dtype, out_dtype, x, conv_w, conv_state, derived_gates(a, b, A_log, dt_bias),
                             z, norm_w, state, false, out, B, stream);
}

gdn_status_t gdn_verify_workspace_size(const gdn_config_t* cfg, int32_t B, int32_t K, size_t* bytes) {
  Dims d;
  gdn_status_t st = resolve(cfg, &d);
  if (st != GDN_OK) return st;
  if (!bytes || B < 0 || K < 1 || K > GDN_MAX_VERIFY_ROWS) return GDN_ERR_INVALID_ARG;
  *bytes = gdn::verify_workspace_bytes(d, B, K);
  return GDN_OK;
}

gdn_status_t gdn_verify(const gdn_config_t* cfg, gdn_dtype_t dtype, gdn_dtype_t out_dtype,
                        const void* x, const float* conv_w, const void* conv_state, const float* g,
                        const float* beta, const void* z, const float* norm_w, const float* state,
                        void* out, int32_t B, int32_t K, void* ws, size_t ws_bytes,
                        gdn_stream_t stream) {
  Dims d;
  gdn_status_t st = resolve(cfg, &d);
  if (st != GDN_OK) return st;
  if (!valid_dtype(dtype) || !valid_dtype(out_dtype)) return GDN_ERR_UNSUPPORTED;
  if (B < 0 || (int64_t)B * d.hv > INT32_MAX || K < 1 || K > GDN_MAX_VERIFY_ROWS) return GDN_ERR_INVALID_ARG;
  if (B == 0) return GDN_OK;
  if (!x || !conv_w || !conv_state || !g || !beta || !z || !norm_w || !state || !out) return GDN_ERR_INVALID_ARG;
  if (!aligned16(conv_w) || !aligned16(state) || (d.per_channel && !aligned16(g))) return GDN_ERR_INVALID_ARG;
  const size_t need = gdn::verify_workspace_bytes(d, B, K);
  if (!ws || ws_bytes < need || !aligned16(ws)) return GDN_ERR_WORKSPACE;
  const size_t state_bytes = (size_t)B * d.hv * d.dv * d.dk * sizeof(float);
  const size_t out_bytes = (size_t)B * K * d.hv * d.dv * dsize(out_dtype);
  if (overlaps(out, out_bytes, state, state_bytes) || overlaps(out, out_bytes, ws, need) ||
      overlaps(ws, need, state, state_bytes))
    return GDN_ERR_INVALID_ARG;
  return hip_status(gdn::launch_verify(d, dtype == GDN_BF16, out_dtype == GDN_BF16, x, conv_w, conv_state, g,
                                       beta, z, norm_w, state, out, B, K, ws, static_cast<hipStream_t>(stream)));
}

gdn_status_t gdn_verify_commit(const gdn_config_t* cfg, gdn_dtype_t dtype, const int32_t* accepted,
                               const void* x, const float* g, void* conv_state, float* state,
                               int32_t B, int32_t K, const void* ws, size_t ws_bytes,
                               gdn_stream_t stream) {
  Dims d;
  gdn_status_t st = resolve(cfg, &d);
  if (st != GDN_OK) return st;
  if (!valid_dtype(dtype)) return GDN_ERR_UNSUPPORTED;
  if (B < 0 || B > 65535 || K < 1 || K > GDN_MAX_VERIFY_ROWS) return GDN_ERR_INVALID_ARG;
  if (B == 0) return GDN_OK;
  if (!accepted || !x || !g || !conv_state || !state) return GDN_ERR_INVALID_ARG;
  if (!aligned16(state) || (d.per_channel && !aligned16(g))) return GDN_ERR_INVALID_ARG;
  const size_t need = gdn::verify_workspace_bytes(d, B, K);
  if (!ws || ws_bytes < need || !aligned16(ws)) return GDN_ERR_WORKSPACE;
  const size_t state_bytes = (size_t)B * d.hv * d.dv * d.dk * sizeof(float);
  if (overlaps(ws, need, state, state_bytes)) return GDN_ERR_INVALID_ARG;
  return hip_status(gdn::launch_verify_commit(d, dtype == GDN_BF16, accepted, x, g, conv_state, state, B, K, ws,
                                              static_cast<hipStream_t>(stream)));
}

}  // extern "C"
