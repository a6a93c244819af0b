/*
 * gdn.h -- C ABI of libgdn.so, the Gated DeltaNet (GDN) sublayer hot path for
 * AMD Instinct MI355X (gfx950).
 *
 * The sublayer (as the golden PR for the Qwen3.8-Flash-Next GDN sublayer and
 * the Qwen3.8 / GLM-5.3 kernel TDD ledgers describe it):
 *   1. depthwise causal conv1d of width 4 over the projected [Q|K|V] rows;
 *   2. q and k L2-normalised per head, q scaled by 1/sqrt(dk), key heads
 *      repeat-interleaved onto the value heads;
 *   3. the gated delta rule with an fp32 [value,key] state per value head,
 *      either chunk-wise (WY form, 64-token chunks, state carried across
 *      chunks and packed variable-length sequences) or one decode token;
 *   4. an RMSNorm over each value head, gated by sigmoid(z).
 *
 * Conventions shared by every call
 *   - All tensor arguments are DEVICE pointers unless the name ends in _host.
 *     The caller owns every buffer (including the workspace); the library
 *     never allocates, frees, synchronises or keeps a pointer after the call.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream).  Results are valid once the stream has reached them.
 *   - Arguments are checked on the host before anything is launched; a
 *     failed check returns a status and launches nothing.  After launching,
 *     a HIP launch error is reported as GDN_ERR_HIP.  There is no silent
 *     fallback: an unsupported shape or dtype is an error.
 *   - Dtype GDN_BF16 means bfloat16 storage; arithmetic is fp32 throughout,
 *     with matrix products on bf16 MFMA using hi/lo splitting of fp32
 *     operands, or fp32 MFMA on the GDN_F32 path.
 *   - Recurrent states are fp32, laid out [seq][value head][dv][dk] (value
 *     index major), as the GLM-5.3 ledger's KDA decode slice fixes.
 *   - Preconditions documented, not checked on the device: g <= 0 (a log
 *     decay), 0 <= beta <= 1, all inputs finite.
 *
 * Supported geometry: head_k_dim = head_v_dim = 128, conv_width = 4,
 * chunk_size = 64, num_v_heads a multiple of num_k_heads.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 2

typedef enum {
  GDN_OK = 0,
  GDN_ERR_INVALID_ARG = 1,  /* null pointer, bad count or stride, aliasing      */
  GDN_ERR_UNSUPPORTED = 2,  /* head dim / conv width / chunk / dtype not built  */
  GDN_ERR_SEQLENS = 3,      /* cu_seqlens not 0-based, non-decreasing, ending T */
  GDN_ERR_WORKSPACE = 4,    /* workspace missing or smaller than required       */
  GDN_ERR_HIP = 5           /* a HIP launch or runtime call failed              */
} gdn_status_t;

/* GDN_F16 (IEEE half) is a storage type of recurrent states only
 * (gdn_decode_step_h16, gdn_state_convert); activations are fp32 or bf16. */
typedef enum { GDN_F32 = 0, GDN_BF16 = 1, GDN_F16 = 2 } gdn_dtype_t;

typedef void* gdn_stream_t; /* a hipStream_t */

/* Geometry and numerics of one GDN sublayer; passed by pointer, checked on
 * every call.  gdn_config_default fills the pages' model geometry. */
typedef struct {
  int32_t num_k_heads;           /* Hk: 16 on the pages' model                      */
  int32_t num_v_heads;           /* Hv: 48; Hv % Hk == 0 (repeat-interleave ratio)   */
  int32_t head_k_dim;            /* dk: 128 (only value built)                       */
  int32_t head_v_dim;            /* dv: 128 (only value built)                       */
  int32_t conv_width;            /* 4 (only value built)                             */
  int32_t chunk_size;            /* 64 (only value built)                            */
  int32_t conv_act;              /* 0: none, 1: SiLU after the conv (default 1)      */
  int32_t decay_per_key_channel; /* 0: g is [T][Hv]; 1: g is [T][Hv][dk]             */
  int32_t qk_l2norm;             /* 1 (default): q, k L2-normalised inside the calls; */
                                 /* 0: q, k used as given (the caller's separate unit- */
                                 /* L2 stage, GLM ledger row I2a); q_scale applies     */
  float l2_eps;                  /* q,k: x / sqrt(sum x^2 + l2_eps); default 1e-6    */
  float rms_eps;                 /* gated norm: rsqrt(mean o^2 + rms_eps); 1e-6      */
  float q_scale;                 /* <= 0 selects 1/sqrt(head_k_dim)                  */
} gdn_config_t;

/* ABI version of the library (GDN_ABI_VERSION it was built with). */
int gdn_abi_version(void);

/* Static, never-NULL description of a status code. */
const char* gdn_status_string(gdn_status_t status);

/* Fill *cfg with Hk=16, Hv=48, dk=dv=128, conv 4, chunk 64, SiLU, scalar
 * decay, eps 1e-6 / 1e-6, q_scale 1/sqrt(128).  Host only. */
gdn_status_t gdn_config_default(gdn_config_t* cfg);

/*
 * Depthwise causal conv1d prefill over N packed sequences (the conv leg of
 * the golden PR's Consumer section; the GLM ledger's conv slice fixes that a
 * step equals the full width-4 conv).  Channel c of token t:
 *     y[t][c] = act( sum_{i=0..3} w[c][i] * x[t-3+i][c] )
 * where positions before the start of t's sequence read that sequence's
 * carried conv state (rows oldest first), or zero when conv_state_in is NULL.
 *   dtype            GDN_F32 or GDN_BF16 for x, y and the conv states
 *   x                [T][Cc] with row stride x_stride (elements, >= Cc), where
 *                    Cc = 2*Hk*dk + Hv*dv and a row is [Q heads | K heads | V heads]
 *   w                [Cc][4] fp32, w[c][3] multiplies the current token
 *   conv_state_in    [N][3][Cc] or NULL
 *   conv_state_out   [N][3][Cc] or NULL: the last three inputs of each sequence
 *                    (carried rows when the sequence is shorter than 3); may
 *                    equal conv_state_in
 *   y                [T][Cc] with row stride y_stride (>= Cc); must not overlap x
 *   cu_dev, cu_host  [N+1] int32 sequence offsets, the same values on device
 *                    and host; cu[0] = 0, non-decreasing, cu[N] = T
 */
gdn_status_t gdn_conv1d_prefill(const gdn_config_t* cfg, gdn_dtype_t dtype, const void* x,
                                int64_t x_stride, const float* w, const void* conv_state_in,
                                void* conv_state_out, void* y, int64_t y_stride,
                                const int32_t* cu_dev, const int32_t* cu_host, int32_t N,
                                int32_t T, gdn_stream_t stream);

/*
 * One conv step for B sequences of one token each: window (state rows 0..2,
 * x) gives y; the state becomes (rows 1, 2, x).
 *   x [B][Cc] (row stride x_stride), conv_state [B][3][Cc] updated in place,
 *   y [B][Cc] (row stride y_stride).
 */
gdn_status_t gdn_conv1d_step(const gdn_config_t* cfg, gdn_dtype_t dtype, const void* x,
                             int64_t x_stride, const float* w, void* conv_state, void* y,
                             int64_t y_stride, int32_t B, gdn_stream_t stream);

/* Bytes of device workspace gdn_chunk_prefill needs for N sequences and T
 * tokens in total.  Host only; pure. */
gdn_status_t gdn_chunk_prefill_workspace_size(const gdn_config_t* cfg, int32_t N, int32_t T,
                                              size_t* bytes);

/*
 * Chunk-wise gated delta rule over N packed sequences (the golden PR's
 * prepare -> cumsum -> A -> solve -> recompute -> state -> output sequence;
 * the TDD ledger's batched/prefill recurrence).  Per sequence and value head
 * h, with S the fp32 [dv][dk] state started from initial_state (or zero) and
 * khat = L2(k), qtil = L2(q) * q_scale from key head h / (Hv/Hk), each token
 * computes, in exact arithmetic,
 *     S <- S * exp(g)           (per key channel: column j scaled by exp(g[j]))
 *     u  = beta * (v - S khat);  S <- S + u khat^T;  o = S qtil
 * The library evaluates this in 64-token chunks in the WY form.  Precision:
 * with bf16 inputs the chunk products round their operands (normalised rows,
 * the chunk-start state, the per-chunk intermediates) once to fp16 and
 * accumulate in fp32, the state staying fp32 (max-relative error ~1e-3 against
 * exact arithmetic); values, states and outputs must then stay within fp16
 * range (|x| < 65504).  fp32 inputs take fp32 products throughout (~1e-6).
 *   in_dtype         dtype of q, k, v
 *   out_dtype        dtype of out
 *   q, k             [T][Hk][dk] with row stride qk_stride (elements per token)
 *   v                [T][Hv][dv] with row stride v_stride
 *   g                fp32 [T][Hv], or [T][Hv][dk] with decay_per_key_channel
 *   beta             fp32 [T][Hv]
 *   initial_state    fp32 [N][Hv][dv][dk] or NULL (zero)
 *   cu_dev, cu_host  as for gdn_conv1d_prefill; sequences may be empty
 *   out              [T][Hv][dv] (the pre-norm output)
 *   final_state      fp32 [N][Hv][dv][dk] or NULL; may equal initial_state
 *   ws, ws_bytes     device workspace of at least
 *                    gdn_chunk_prefill_workspace_size(cfg, N, T) bytes
 */
gdn_status_t gdn_chunk_prefill(const gdn_config_t* cfg, gdn_dtype_t in_dtype,
                               gdn_dtype_t out_dtype, const void* q, const void* k,
                               int64_t qk_stride, const void* v, int64_t v_stride,
                               const float* g, const float* beta, const float* initial_state,
                               const int32_t* cu_dev, const int32_t* cu_host, int32_t N,
                               int32_t T, void* out, float* final_state, void* ws,
                               size_t ws_bytes, gdn_stream_t stream);

/*
 * gdn_chunk_prefill for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments without ws / ws_bytes.  The workspace is a fixed device
 * array of GDN_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held
 * from the library's load on that GPU until the process ends; its address is
 * looked up once per device (on the first call with that device current).
 * The call allocates nothing.
 *   - Sizes whose gdn_chunk_prefill_workspace_size exceeds the array return
 *     GDN_ERR_WORKSPACE before anything is enqueued (128 MiB covers, e.g., one
 *     4096-token sequence at 48 value heads: 105 MB).
 *   - Every call on one GPU shares that GPU's array and overwrites it (nothing
 *     in it needs clearing: each call writes before it reads).  Calls that
 *     overlap on one GPU (other streams, other host threads) race on it and
 *     must be serialised by the caller.
 *   - The current device must be the one `stream` belongs to.
 * Results are bit-identical to gdn_chunk_prefill (the same kernels).
 */
#define GDN_NOALLOC_SCRATCH_BYTES (128u << 20)
gdn_status_t gdn_chunk_prefill_noalloc(const gdn_config_t* cfg, gdn_dtype_t in_dtype,
                                       gdn_dtype_t out_dtype, const void* q, const void* k,
                                       int64_t qk_stride, const void* v, int64_t v_stride,
                                       const float* g, const float* beta, const float* initial_state,
                                       const int32_t* cu_dev, const int32_t* cu_host, int32_t N,
                                       int32_t T, void* out, float* final_state, gdn_stream_t stream);

/*
 * The gates of a call from the a / b projections.  The golden PR's prepare
 * stage derives the raw g/beta from the in_proj_a / in_proj_b outputs with the
 * layer's A_log and dt_bias vectors, and the TDD ledger lists the GDN
 * alpha/beta transform kernels; neither page prints the transform.  This
 * library reads it as, per token (or sequence) t and value head h,
 *     g[t][h]    = -exp(A_log[h]) * softplus(a[t][h] + dt_bias[h])
 *     beta[t][h] = sigmoid(b[t][h]),        softplus(x) = log(1 + exp(x)).
 * The *_ab calls below take a, b ([rows][Hv], in the activations' dtype) and
 * A_log, dt_bias (fp32 [Hv]) in place of g and beta and derive the gates
 * inside their kernels (no g / beta pass).  Scalar decay only:
 * GDN_ERR_UNSUPPORTED with decay_per_key_channel.
 */

/* gdn_chunk_prefill with derived gates; a, b [T][Hv] in in_dtype. */
gdn_status_t gdn_chunk_prefill_ab(const gdn_config_t* cfg, gdn_dtype_t in_dtype,
                                  gdn_dtype_t out_dtype, const void* q, const void* k,
                                  int64_t qk_stride, const void* v, int64_t v_stride,
                                  const void* a, const void* b, const float* A_log,
                                  const float* dt_bias, const float* initial_state,
                                  const int32_t* cu_dev, const int32_t* cu_host, int32_t N,
                                  int32_t T, void* out, float* final_state, void* ws,
                                  size_t ws_bytes, gdn_stream_t stream);

/*
 * Gated RMSNorm with the sigmoid gate (the golden PR: sigmoid, not SiLU;
 * rsqrt(variance + eps)) over rows * Hv vectors of length dv:
 *     out[i] = o[i] * rsqrt(mean(o^2) + rms_eps) * w[i] * sigmoid(z[i])
 *   o     [rows][Hv][dv] in o_dtype;  z [rows][Hv][dv] in z_dtype
 *   w     fp32 [dv], shared by every head;  out [rows][Hv][dv] in out_dtype
 * out may equal o when o_dtype == out_dtype.  o, z, w and out are 16-byte
 * aligned (GDN_ERR_INVALID_ARG otherwise).
 */
gdn_status_t gdn_gated_rmsnorm(const gdn_config_t* cfg, gdn_dtype_t o_dtype, gdn_dtype_t z_dtype,
                               gdn_dtype_t out_dtype, const void* o, const void* z,
                               const float* w, void* out, int64_t rows, gdn_stream_t stream);

/* Bytes of device workspace gdn_prefill needs for N sequences and T tokens
 * in total with activations of `dtype`.  Host only; pure. */
gdn_status_t gdn_prefill_workspace_size(const gdn_config_t* cfg, gdn_dtype_t dtype, int32_t N,
                                        int32_t T, size_t* bytes);

/*
 * The whole sublayer prefill over N packed sequences (the golden PR's
 * Consumer section: conv, then the chunked delta rule, then the gated norm):
 * gdn_conv1d_prefill over x, q | k | v taken from the conv output rows,
 * gdn_chunk_prefill, and gdn_gated_rmsnorm of its output, with the same
 * arithmetic as those calls made in that order.  Where a workgroup of the
 * chunk kernels holds a whole value head (many sequences), they apply the
 * gated norm to each chunk's output themselves and the pre-norm output is
 * never stored; otherwise it goes through the workspace, as fp16 for bf16
 * inputs (whose chunk products already round their operands to fp16) and
 * fp32 for fp32 inputs.
 *   dtype            dtype of x, the conv states and z
 *   out_dtype        dtype of out
 *   x                [T][Cc] raw projected rows, row stride x_stride (>= Cc,
 *                    a multiple of 8)
 *   conv_w           fp32 [Cc][4]
 *   conv_state_in    [N][3][Cc] or NULL (zero);  conv_state_out [N][3][Cc] or
 *                    NULL, may equal conv_state_in
 *   g, beta          as for gdn_chunk_prefill
 *   z                [T][Hv][dv] gate;  norm_w fp32 [dv]
 *   initial_state    fp32 [N][Hv][dv][dk] or NULL;  final_state the same or
 *                    NULL, may equal initial_state
 *   cu_dev, cu_host  as for gdn_conv1d_prefill
 *   out              [T][Hv][dv]
 *   ws, ws_bytes     device workspace of at least
 *                    gdn_prefill_workspace_size(cfg, dtype, N, T) bytes; it
 *                    must not overlap x, z, out or the states
 * x, conv_w, g, z, norm_w, out and the workspace are 16-byte aligned.
 */
gdn_status_t gdn_prefill(const gdn_config_t* cfg, gdn_dtype_t dtype, gdn_dtype_t out_dtype,
                         const void* x, int64_t x_stride, const float* conv_w,
                         const void* conv_state_in, void* conv_state_out, const float* g,
                         const float* beta, const void* z, const float* norm_w,
                         const float* initial_state, const int32_t* cu_dev, const int32_t* cu_host,
                         int32_t N, int32_t T, void* out, float* final_state, void* ws,
                         size_t ws_bytes, gdn_stream_t stream);

/* gdn_prefill with derived gates; a, b [T][Hv] in dtype.  Workspace as for
 * gdn_prefill (gdn_prefill_workspace_size). */
gdn_status_t gdn_prefill_ab(const gdn_config_t* cfg, gdn_dtype_t dtype, gdn_dtype_t out_dtype,
                            const void* x, int64_t x_stride, const float* conv_w,
                            const void* conv_state_in, void* conv_state_out, const void* a,
                            const void* b, const float* A_log, const float* dt_bias, const void* z,
                            const float* norm_w, const float* initial_state, const int32_t* cu_dev,
                            const int32_t* cu_host, int32_t N, int32_t T, void* out,
                            float* final_state, void* ws, size_t ws_bytes, gdn_stream_t stream);

/*
 * One fused decode step for B sequences (the TDD ledger's scalar recurrence
 * with fused output gate; the Qwen3SsmLayer conv + recurrence + norm decode
 * kernels): conv step over all Cc channels, L2/q-scale, the recurrence for the
 * single token, and the sigmoid gated norm.
 *   dtype        dtype of x, conv_state and z
 *   out_dtype    dtype of out
 *   x            [B][Cc] raw projected [Q|K|V] row per sequence (contiguous)
 *   conv_w       fp32 [Cc][4]
 *   conv_state   [B][3][Cc], updated in place
 *   g            fp32 [B][Hv] (or [B][Hv][dk] with decay_per_key_channel)
 *   beta         fp32 [B][Hv]
 *   z            [B][Hv][dv];  norm_w fp32 [dv]
 *   state        fp32 [B][Hv][dv][dk], updated in place
 *   out          [B][Hv][dv]
 * 0 <= B <= 65535, else GDN_ERR_INVALID_ARG before anything is enqueued.  When Hk < Hv the
 * key head's q / k conv-state channels are read by all its value heads, and
 * the step is two launches on the stream: the fused step, then a shift of
 * those channels.
 */
gdn_status_t gdn_decode_step(const gdn_config_t* cfg, gdn_dtype_t dtype, gdn_dtype_t out_dtype,
                             const void* x, const float* conv_w, void* conv_state, const float* g,
                             const float* beta, const void* z, const float* norm_w, float* state,
                             void* out, int32_t B, gdn_stream_t stream);

/*
 * gdn_decode_step with the recurrent state stored in fp16 (the Qwen3SsmLayer
 * field notes' FP16 h-state: the same expressions and accumulation order as
 * the fp32 kernel, the state widened to fp32 on load and rounded to the
 * nearest fp16 once per token on store).  state is fp16 [B][Hv][dv][dk],
 * 16-byte aligned; every other argument as for gdn_decode_step.  This changes
 * the numerics: the state carries a relative rounding of at most 2^-11 per
 * token on top of the fp32 path (the tests state the bound they check).
 */
gdn_status_t gdn_decode_step_h16(const gdn_config_t* cfg, gdn_dtype_t dtype, gdn_dtype_t out_dtype,
                                 const void* x, const float* conv_w, void* conv_state, const float* g,
                                 const float* beta, const void* z, const float* norm_w, void* state,
                                 void* out, int32_t B, gdn_stream_t stream);

/*
 * Width converter of recurrent states (the field notes' matched pair around
 * the fp32 prefill kernels for an fp16-sized state pool): n values from src to
 * dst, GDN_F16 -> GDN_F32 (exact) or GDN_F32 -> GDN_F16 (round to nearest
 * even).  src and dst 16-byte aligned, not overlapping.
 */
gdn_status_t gdn_state_convert(const void* src, gdn_dtype_t src_dtype, void* dst, gdn_dtype_t dst_dtype,
                               int64_t n, gdn_stream_t stream);

/* gdn_decode_step with derived gates; a, b [B][Hv] in dtype. */
gdn_status_t gdn_decode_step_ab(const gdn_config_t* cfg, gdn_dtype_t dtype, gdn_dtype_t out_dtype,
                                const void* x, const float* conv_w, void* conv_state, const void* a,
                                const void* b, const float* A_log, const float* dt_bias,
                                const void* z, const float* norm_w, float* state, void* out,
                                int32_t B, gdn_stream_t stream);

/*
 * Speculative verify transaction (the Qwen3.8 TDD ledger's transaction rules:
 * the verified rows are computed from the prior logical state; a commit
 * publishes only the state after the accepted rows; abort leaves the prior
 * state; rejected rows are never read.  The Qwen3SsmLayer field notes give
 * the WY verify kernels of K = 2..17 rows and their write-on-accept twin with
 * a post-verdict fold, the form built here).  One transaction is one
 * gdn_verify followed by exactly one gdn_verify_commit on the same workspace
 * (accepted = 0 everywhere is the abort).
 */
#define GDN_MAX_VERIFY_ROWS 64

/* Bytes of workspace a transaction of B sequences x K rows needs.  Host only. */
gdn_status_t gdn_verify_workspace_size(const gdn_config_t* cfg, int32_t B, int32_t K, size_t* bytes);

/*
 * Verify: row t of sequence b gets the output decode step t would produce
 * after rows 0..t-1 of that sequence, starting from (conv_state, state) --
 * the same arithmetic as gdn_decode_step, row by row.  conv_state and state
 * are only read.  The workspace receives what the commit replays.
 *   dtype, out_dtype   as for gdn_decode_step
 *   x                  [B][K][Cc] raw projected rows (contiguous)
 *   conv_state         [B][3][Cc];  state fp32 [B][Hv][dv][dk]
 *   g                  fp32 [B][K][Hv] (or [B][K][Hv][dk]);  beta fp32 [B][K][Hv]
 *   z                  [B][K][Hv][dv];  norm_w fp32 [dv]
 *   out                [B][K][Hv][dv]
 *   K                  1 .. GDN_MAX_VERIFY_ROWS
 */
gdn_status_t gdn_verify(const gdn_config_t* cfg, gdn_dtype_t dtype, gdn_dtype_t out_dtype,
                        const void* x, const float* conv_w, const void* conv_state, const float* g,
                        const float* beta, const void* z, const float* norm_w, const float* state,
                        void* out, int32_t B, int32_t K, void* ws, size_t ws_bytes,
                        gdn_stream_t stream);

/*
 * Commit: sequence b advances by its first c = clamp(accepted[b], 0, K) rows,
 * exactly as c decode steps would leave conv_state and state (the recurrent
 * state is the verify's own value after row c, bit for bit); c = 0 leaves
 * both untouched.  Reads x and g rows 0..c-1 of each sequence only.
 *   accepted   DEVICE int32 [B]
 *   x, g       the verify's (unchanged since)
 *   conv_state, state   updated in place
 */
gdn_status_t gdn_verify_commit(const gdn_config_t* cfg, gdn_dtype_t dtype, const int32_t* accepted,
                               const void* x, const float* g, void* conv_state, float* state,
                               int32_t B, int32_t K, const void* ws, size_t ws_bytes,
                               gdn_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
