// gdn_launch.h -- internal launchers behind the C ABI.  Each takes already
// validated arguments and only enqueues kernels on the stream.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

// Where g and beta of a call come from: fp32 arrays, or (a non-null) derived
// per element from the a / b projections [rows][Hv] in the activations'
// dtype with the per-head A_log and dt_bias (scalar decay only).
struct Gates {
  const float* g;
  const float* beta;
  const void* a;
  const void* b;
  const float* A_log;
  const float* dt_bias;
};

// Geometry resolved from gdn_config_t.
struct Dims {
  int hk, hv, dk, dv;
  int cc;           // conv channels 2*hk*dk + hv*dv
  int act;          // conv activation: 0 none, 1 SiLU
  int per_channel;  // decay per key channel
  int l2norm;       // 1: q, k L2-normalised in the kernels; 0: used as given
  float l2_eps, rms_eps, q_scale;
};

hipError_t launch_conv1d_prefill(const Dims& d, bool bf16, const void* x, int64_t x_stride,
                                 const float* w, const void* cs_in, void* cs_out, void* y,
                                 int64_t y_stride, const int32_t* cu, int n, int t,
                                 hipStream_t s);
hipError_t launch_conv1d_step(const Dims& d, bool bf16, const void* x, int64_t x_stride,
                              const float* w, void* cs, void* y, int64_t y_stride, int b,
                              hipStream_t s);
hipError_t launch_gated_rmsnorm(const Dims& d, bool o_bf16, bool z_bf16, bool out_bf16,
                                const void* o, const void* z, const float* w, void* out,
                                int64_t rows, hipStream_t s);
// state: fp32, or fp16 (state_f16) widened on load and rounded on store
hipError_t launch_decode_step(const Dims& d, bool bf16, bool out_bf16, const void* x,
                              const float* conv_w, void* conv_state, const Gates& gt,
                              const void* z, const float* norm_w, void* state, bool state_f16,
                              void* out, int b, hipStream_t s);
// n state values fp32 -> fp16 (rounded to nearest even) or fp16 -> fp32
hipError_t launch_state_convert(const void* src, bool src_f16, void* dst, int64_t n, hipStream_t s);

// Speculative verify transaction (gdn_verify.hip).  The workspace holds the
// per-row update vectors the commit replays: u [b][k][hv][dv] then the
// normalised keys [b][k][hk][dk], fp32.
size_t verify_workspace_bytes(const Dims& d, int b, int k);
hipError_t launch_verify(const Dims& d, bool bf16, bool out_bf16, const void* x, const float* conv_w,
                         const void* conv_state, const float* g, const float* beta, const void* z,
                         const float* norm_w, const float* state, void* out, int b, int k, void* ws,
                         hipStream_t s);
hipError_t launch_verify_commit(const Dims& d, bool bf16, const int32_t* accepted, const void* x,
                                const float* g, void* conv_state, float* state, int b, int k,
                                const void* ws, hipStream_t s);

// Chunk prefill.  Workspace layout is private to gdn_chunk.hip.
size_t chunk_workspace_bytes(const Dims& d, int n, int t);
// Whether the chunk prefill for n sequences can apply the gated norm to its
// output itself (norm_z / norm_w of launch_chunk_prefill); the answer depends
// only on the geometry, the input dtype and n.
bool chunk_fuses_norm(const Dims& d, bool in_bf16, int n);
// Whether the chunk prefill for n sequences can write its output as fp16
// (out_f16): the register-resident spine with 32 value rows per workgroup,
// whose products already round their operands to fp16; the one-call prefill
// keeps its pre-norm output in that form when it does not fuse the norm.
bool chunk_out_f16(const Dims& d, bool in_bf16, int n);
// norm_z (bf16 [T][Hv][dv]) and norm_w non-null: out receives the gated norm
// of the chunk output (requires chunk_fuses_norm).  out_f16: out is fp16
// (requires chunk_out_f16; out_bf16 is then ignored).
hipError_t launch_chunk_prefill(const Dims& d, bool in_bf16, bool out_bf16, const void* q,
                                const void* k, int64_t qk_stride, const void* v,
                                int64_t v_stride, const Gates& gt, const float* init_state, const int32_t* cu_dev,
                                const int32_t* cu_host, int n, int t, void* out,
                                float* final_state, void* ws, size_t ws_bytes,
                                const uint16_t* norm_z, const float* norm_w, hipStream_t s,
                                bool out_f16 = false);
// The gated norm of an fp16 o (the one-call prefill's pre-norm output), z bf16 or fp32.
hipError_t launch_gated_rmsnorm_f16o(const Dims& d, bool z_bf16, bool out_bf16, const void* o,
                                     const void* z, const float* w, void* out, int64_t rows,
                                     hipStream_t s);

}  // namespace gdn
