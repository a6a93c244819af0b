// gdn_decode.hip -- one fused GDN decode step for B sequences: conv step,
// L2 / q scale, the gated delta rule for the single token, and the sigmoid
// gated RMSNorm, with the conv state and the fp32 recurrent state updated in
// place.
//
// Follows the Qwen3.8 kernel TDD ledger (dense kernel map: scalar GDN
// recurrence with fused output gate), the Qwen3SsmLayer field notes on the
// fused conv + recurrence + norm decode kernels and their state traffic (two
// reads and one write of the state cut to one read and one write), and the
// GLM-5.3 ledger's KDA decode slice (fp32 [value,key] state, decay by
// exp(g), beta-scaled delta, separate q output scale 1/sqrt(dk)).
//
// Per value head h with state S [dv][dk] and per-column decay a_j = exp(g)
// (or exp(g_j) per key channel), the token gives, in one pass over S:
//     Sd  = S diag(a)                       (decayed state, kept in registers)
//     p   = Sd khat,  r = Sd qtil           (two row sums per row of S)
//     u   = beta (v - p)
//     S'  = Sd + u khat^T                   (written back)
//     o   = S' qtil = r + u (khat . qtil)
// so S is read once and written once.
//
// Work split: one 512-thread workgroup per (sequence, value head), so a
// 64-sequence batch at 48 value heads is 3072 equal workgroups, each streaming
// one contiguous 64 KiB state (measured on gfx950: in-place streams of one
// 64 KiB block per workgroup reach ~5.9 TB/s, against ~5.4 TB/s for 768-thread
// workgroups over a key head's three blocks).  At eight waves per SIMD four
// such workgroups share a CU, so the 3072 run as three full rounds of 1024
// (256-thread workgroups, eight per CU, left the last of 1.5 rounds half
// empty).  The 64 KiB state of the head is spread as 8 rows x one float4 per
// thread; a wavefront loads two full 512-byte rows per instruction.  Rows are independent: each row's two dot
// products are reduced across the 32 lanes that hold it (DPP and a swizzle, no
// LDS), and the row is updated and stored as soon as its loads land.
// Conv state: each workgroup shifts its value head's v channels in place (it
// is their only reader).  The key head's q and k channels are read by all of
// its value heads, so when the key head is shared (ratio > 1) every workgroup
// only reads them, and a second small kernel shifts them after the step.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

constexpr int kGroup = 256;             // threads per workgroup of the small kernels
constexpr int kD = 128;                 // head_k_dim == head_v_dim
constexpr int kStepThreads = 512;       // threads per value head (the step kernel)
constexpr int kRowGroups = kStepThreads / 32;
constexpr int kRowsPerThread = kD / kRowGroups;
constexpr int kWindow = 4;              // state rows in flight per thread

// Four state values at a buffer offset, streamed (non-temporal: the state is
// touched once per step); fp16 is widened on load and rounded to nearest even
// on store.
template <typename TS>
__device__ __forceinline__ f32x4_t state_buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  if constexpr (sizeof(TS) == 4) {
    return __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 2));
  } else {
    return __builtin_convertvector(__builtin_bit_cast(f16x4_t, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 2)),
                                   f32x4_t);
  }
}
template <typename TS>
__device__ __forceinline__ void state_buf_store4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, f32x4_t v) {
  typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
  if constexpr (sizeof(TS) == 4) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, voff, soff, 2);
  } else {
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2_t, __builtin_convertvector(v, f16x4_t)), r, voff, soff, 2);
  }
}

// Conv of one channel for one token: y = act(w . (s0, s1, s2, x)); with `shift`
// the channel's state rows become (s1, s2, x).  The loads are issued by
// load() and the arithmetic and stores done by finish(), so that other loads
// can be issued in between.
template <typename T>
struct ConvTap {
  float s0, s1, s2, xv;
  f32x4_t w;
  __device__ __forceinline__ void load(const T* x_row, const float* conv_w, const T* cs_row, int c, int cc) {
    const T* p = cs_row + c;
    s0 = ld(p);
    s1 = ld(p + cc);
    s2 = ld(p + 2 * cc);
    xv = ld(x_row + c);
    w = *reinterpret_cast<const f32x4_t*>(conv_w + (int64_t)c * 4);
  }
  __device__ __forceinline__ float finish(T* cs_row, int c, int cc, int act, bool shift) const {
    float y = w[0] * s0;
    y = fmaf(w[1], s1, y);
    y = fmaf(w[2], s2, y);
    y = fmaf(w[3], xv, y);
    if (shift) {
      T* p = cs_row + c;
      st(p, s1);
      st(p + cc, s2);
      st(p + 2 * cc, xv);
    }
    return act ? silu_conv(y) : y;
  }
};

template <typename T, typename To, typename TS, bool kPerChannel>
__global__ __launch_bounds__(kStepThreads, kStepThreads / 64) void decode_step_kernel(
    const T* __restrict__ x, const float* __restrict__ conv_w, T* __restrict__ conv_state,
    Gates gates, const T* __restrict__ z,
    const float* __restrict__ norm_w, TS* __restrict__ state, To* __restrict__ out, int hk,
    int hv, int cc, int act, int l2norm, float l2_eps, float q_scale, float rms_eps) {
  const int b = blockIdx.x / hv;
  const int h = blockIdx.x % hv;
  const int ratio = hv / hk;
  const int kh = h / ratio;
  const int tid = threadIdx.x;
  const int gwave = tid / kWave;
  const int lane = tid % kWave;
  const int cg = tid % 32;                // column group: columns 4cg .. 4cg+3
  const int rg = tid / 32;                // row group: rows rg + kRowGroups m

  __shared__ float s_q[kD], s_k[kD], s_scal[2];
  __shared__ float s_v[kD], s_o[kD], s_nrm[2];

  // The conv inputs are loaded first and then a window of kWindow state rows:
  // loads complete in issue order, so the conv (which gates the first barrier)
  // waits only for its own loads while the state rows are still in flight.
  // Each processed row issues the load of the row kWindow after it, so the
  // state (fp32, or fp16 widened to fp32) is streamed once per step.  A short
  // window keeps a thread within 64 registers: eight waves per SIMD (four
  // workgroups per CU) keep as many rows in flight as a longer window would.
  // Every thread loads a q / k and a v conv input (threads past the channels
  // repeat one, unused): no branch before the state loads.
  const T* x_row = x + (int64_t)b * cc;
  T* cs_row = conv_state + (int64_t)b * 3 * cc;
  const int tq = tid % (2 * kD);
  const int c_qk = tq < kD ? kh * kD + tq : hk * kD + kh * kD + (tq - kD);   // the key head's q / k channel
  const int c_v = 2 * hk * kD + h * kD + (tid % kD);                             // this head's v channel (tid < kD)
  ConvTap<T> tap_qk, tap_v;
  tap_qk.load(x_row, conv_w, cs_row, c_qk, cc);
  tap_v.load(x_row, conv_w, cs_row, c_v, cc);

  // raw gates (given, or the a / b projections they are derived from)
  GateRaw<T> graw{};
  f32x4_t gv;
  if constexpr (kPerChannel) {
    gv = *reinterpret_cast<const f32x4_t*>(gates.g + ((int64_t)b * hv + h) * kD + 4 * cg);
    graw.beta = gates.beta[(int64_t)b * hv + h];
  } else {
    graw = gate_raw<T>(gates, b, hv, h);
  }

  // the head's state through a buffer descriptor: a 32-bit lane offset and the
  // row step in the scalar offset, so that no 64-bit address is held per row
  TS* S = state + ((int64_t)b * hv + h) * kD * kD;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(S, (short)0, kD * kD * (int)sizeof(TS), 0x00020000);
  const uint32_t voff = (uint32_t)(rg * kD + 4 * cg) * sizeof(TS);
  auto load_row = [&](int m) { return state_buf_load4<TS>(rs, voff, (uint32_t)(kRowGroups * m * kD * sizeof(TS))); };
  f32x4_t sreg[kRowsPerThread];
#pragma unroll
  for (int m = 0; m < kWindow; ++m) sreg[m] = load_row(m);
  // nothing that uses the conv or gate loads may move above the state loads
  __builtin_amdgcn_sched_barrier(0);

  // decay factors a and beta
  float a[4], bt;
  if constexpr (kPerChannel) {
#pragma unroll
    for (int e = 0; e < 4; ++e) a[e] = __expf(gv[e]);
    bt = graw.beta;
  } else {
    float gs;
    gate_resolve(gates, graw, gs, bt);
    const float av = __expf(gs);
#pragma unroll
    for (int e = 0; e < 4; ++e) a[e] = av;
  }

  if (tid < 2 * kD) {  // q / k are shifted here only when this head is their sole reader
    const float y = tap_qk.finish(cs_row, c_qk, cc, act, ratio == 1);
    if (tid < kD) s_q[tid] = y; else s_k[tid - kD] = y;
  }
  if (tid < kD) s_v[tid] = tap_v.finish(cs_row, c_v, cc, act, true);
  __syncthreads();
  if (tid < 2 * kWave) {
    const int w = tid / kWave;
    const float* src = w == 0 ? s_q : s_k;
    const float a0 = src[2 * lane], a1 = src[2 * lane + 1];
    const float ss = wave_sum(a0 * a0 + a1 * a1);
    if (lane == 0) s_scal[w] = l2norm ? 1.0f / sqrtf(ss + l2_eps) : 1.0f;
  }
  __syncthreads();
  const float rq = s_scal[0] * q_scale, rk = s_scal[1];
  // khat . qtil, computed by every wave (no exchange needed)
  const float kq = wave_sum(s_k[2 * lane] * s_q[2 * lane] + s_k[2 * lane + 1] * s_q[2 * lane + 1]) * rq * rk;
  // this thread's normalised key / query columns
  float kcol[4], qcol[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) { kcol[e] = s_k[4 * cg + e] * rk; qcol[e] = s_q[4 * cg + e] * rq; }

  // per row: decay, the two dot products reduced over the row's 32 lanes,
  // u = beta (v - p), o = r + u (khat . qtil), then the row is updated and
  // written back: S' = Sd + u khat^T
#pragma unroll
  for (int m = 0; m < kRowsPerThread; ++m) {
    if (m + kWindow < kRowsPerThread) sreg[m + kWindow] = load_row(m + kWindow);
    const int row = rg + kRowGroups * m;
    float pk = 0.0f, pq = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sreg[m][e] *= a[e];
      pk = fmaf(sreg[m][e], kcol[e], pk);
      pq = fmaf(sreg[m][e], qcol[e], pq);
    }
    pk = row32_sum(pk);
    pq = row32_sum(pq);
    const float u = bt * (s_v[row] - pk);
    if (cg == 0) s_o[row] = fmaf(u, kq, pq);
#pragma unroll
    for (int e = 0; e < 4; ++e) sreg[m][e] = fmaf(u, kcol[e], sreg[m][e]);
    state_buf_store4<TS>(rs, voff, (uint32_t)(kRowGroups * m * kD * sizeof(TS)), sreg[m]);
  }
  __syncthreads();

  // the sigmoid gated RMSNorm of the head's 128 outputs
  if (tid < kD) {
    const float o = s_o[tid];
    const float ss = wave_sum(o * o);
    if (lane == 0) s_nrm[gwave] = ss;
  }
  __syncthreads();
  if (tid < kD) {
    const float o = s_o[tid];
    const float r = rsqrtf((s_nrm[0] + s_nrm[1]) * (1.0f / kD) + rms_eps);
    const int64_t off = ((int64_t)b * hv + h) * kD + tid;
    st(out + off, o * r * norm_w[tid] * sigmoidf_(ld(z + off)));
  }
}

// Shift of the shared q / k conv state channels after a step whose workgroups
// only read them: rows (s0, s1, s2) become (s1, s2, x).  One channel per
// thread; values move bit for bit.
template <typename T>
__global__ __launch_bounds__(kGroup) void conv_shift_kernel(const T* __restrict__ x, T* __restrict__ conv_state,
                                                            int cc, int n_ch) {
  const int c = blockIdx.x * kGroup + threadIdx.x;
  if (c >= n_ch) return;
  const int64_t b = blockIdx.y;
  T* p = conv_state + b * 3 * cc + c;
  const T s1 = p[cc], s2 = p[2 * cc], xv = x[b * cc + c];
  p[0] = s1;
  p[cc] = s2;
  p[2 * cc] = xv;
}

template <typename T, typename To, typename TS, bool kPC>
hipError_t decode_ratio(const Dims& d, const void* x, const float* conv_w, void* conv_state,
                        const Gates& gt, const void* z, const float* norm_w,
                        void* state, void* out, int b, hipStream_t s) {
  hipLaunchKernelGGL((decode_step_kernel<T, To, TS, kPC>), dim3(b * d.hv), dim3(kStepThreads), 0, s,
                     static_cast<const T*>(x), conv_w, static_cast<T*>(conv_state), gt,
                     static_cast<const T*>(z), norm_w, static_cast<TS*>(state),
                     static_cast<To*>(out), d.hk, d.hv, d.cc, d.act, d.l2norm, d.l2_eps, d.q_scale, d.rms_eps);
  if (d.hv != d.hk) {   // shared q / k channels: shifted once, after every head has read them
    const int n_ch = 2 * d.hk * kD;
    hipLaunchKernelGGL(conv_shift_kernel<T>, dim3((n_ch + kGroup - 1) / kGroup, b), dim3(kGroup), 0, s,
                       static_cast<const T*>(x), static_cast<T*>(conv_state), d.cc, n_ch);
  }
  return hipGetLastError();
}

template <typename T, typename To>
hipError_t decode_impl(const Dims& d, const void* x, const float* conv_w, void* conv_state,
                       const Gates& gt, const void* z, const float* norm_w,
                       void* state, bool state_f16, void* out, int b, hipStream_t s) {
  if (state_f16)
    return d.per_channel ? decode_ratio<T, To, _Float16, true>(d, x, conv_w, conv_state, gt, z, norm_w, state, out, b, s)
                         : decode_ratio<T, To, _Float16, false>(d, x, conv_w, conv_state, gt, z, norm_w, state, out, b, s);
  return d.per_channel ? decode_ratio<T, To, float, true>(d, x, conv_w, conv_state, gt, z, norm_w, state, out, b, s)
                       : decode_ratio<T, To, float, false>(d, x, conv_w, conv_state, gt, z, norm_w, state, out, b, s);
}

// Recurrent state width conversion, fp32 <-> fp16 (narrowing rounds to
// nearest even).  Four values per thread, grid-stride.
template <typename Ts, typename Td>
__global__ __launch_bounds__(kGroup) void state_convert_kernel(const Ts* __restrict__ src, Td* __restrict__ dst,
                                                               int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * kGroup * 4;
  for (int64_t i = ((int64_t)blockIdx.x * kGroup + threadIdx.x) * 4; i < n; i += stride) {
    if (i + 4 <= n) {
      state_store4(dst + i, state_load4(src + i));
    } else {
      for (int64_t j = i; j < n; ++j) dst[j] = (Td)(float)src[j];
    }
  }
}

}  // namespace

hipError_t launch_decode_step(const Dims& d, bool bf16, bool out_bf16, const void* x,
                              const float* conv_w, void* conv_state, const Gates& gt,
                              const void* z, const float* norm_w, void* state, bool state_f16,
                              void* out, int b, hipStream_t s) {
  if (b == 0) return hipSuccess;
  if (bf16)
    return out_bf16 ? decode_impl<uint16_t, uint16_t>(d, x, conv_w, conv_state, gt, z, norm_w, state, state_f16, out, b, s)
                    : decode_impl<uint16_t, float>(d, x, conv_w, conv_state, gt, z, norm_w, state, state_f16, out, b, s);
  return out_bf16 ? decode_impl<float, uint16_t>(d, x, conv_w, conv_state, gt, z, norm_w, state, state_f16, out, b, s)
                  : decode_impl<float, float>(d, x, conv_w, conv_state, gt, z, norm_w, state, state_f16, out, b, s);
}

hipError_t launch_state_convert(const void* src, bool src_f16, void* dst, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int64_t want = (n + 4 * kGroup - 1) / (4 * kGroup);
  const unsigned blocks = (unsigned)(want < 8192 ? want : 8192);
  if (src_f16)
    hipLaunchKernelGGL((state_convert_kernel<_Float16, float>), dim3(blocks), dim3(kGroup), 0, s,
                       static_cast<const _Float16*>(src), static_cast<float*>(dst), n);
  else
    hipLaunchKernelGGL((state_convert_kernel<float, _Float16>), dim3(blocks), dim3(kGroup), 0, s,
                       static_cast<const float*>(src), static_cast<_Float16*>(dst), n);
  return hipGetLastError();
}

}  // namespace gdn
