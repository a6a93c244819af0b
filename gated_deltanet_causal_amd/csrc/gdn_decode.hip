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
// Work split: one workgroup per (sequence, key head) with one 256-thread group
// per value head of that key head (768 threads for the pages' ratio of 3), so
// a 64-sequence batch is 1024 equal workgroups.  The workgroup owns the key
// head's q/k conv channels and its value heads' v channels, so each conv-state
// element has exactly one writer and is shifted in place.  Within a group, the
// 64 KiB state of the head is spread as 16 rows x one float4 per thread; a
// wavefront loads two full 512-byte rows per instruction.  Rows are
// independent: each row's two dot products are reduced across the 32 lanes
// that hold it (DPP and a swizzle, no LDS), and the row is updated and stored
// as soon as its loads land.  The small LDS footprint lets two workgroups share
// a CU, so one streams its state while the other computes.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

constexpr int kGroup = 256;             // threads per value head
constexpr int kD = 128;                 // head_k_dim == head_v_dim
constexpr int kRowsPerThread = 16;      // 128 rows over 8 row groups
constexpr int kWindow = 8;              // state rows in flight per thread

// Conv of one channel for one token: y = act(w . (s0, s1, s2, x)); the
// channel's state rows become (s1, s2, x).
template <typename T>
__device__ __forceinline__ float conv_channel(const T* x_row, const float* conv_w, T* cs_row,
                                              int c, int cc, int act) {
  T* p = cs_row + c;
  const float s0 = ld(p), s1 = ld(p + cc), s2 = ld(p + 2 * cc);
  const float xv = ld(x_row + c);
  const f32x4_t w = *reinterpret_cast<const f32x4_t*>(conv_w + (int64_t)c * 4);
  float y = w[0] * s0;
  y = fmaf(w[1], s1, y);
  y = fmaf(w[2], s2, y);
  y = fmaf(w[3], xv, y);
  st(p, s1);
  st(p + cc, s2);
  st(p + 2 * cc, xv);
  return act ? y * sigmoidf_(y) : y;
}

template <typename T, typename To, typename TS, bool kPerChannel, int kRatio>
__global__ __launch_bounds__(kGroup * kRatio, kRatio <= 3 ? 2 * kRatio : kRatio) void decode_step_kernel(
    const T* __restrict__ x, const float* __restrict__ conv_w, T* __restrict__ conv_state,
    Gates gates, const T* __restrict__ z,
    const float* __restrict__ norm_w, TS* __restrict__ state, To* __restrict__ out, int hk,
    int hv, int cc, int act, float l2_eps, float q_scale, float rms_eps) {
  const int b = blockIdx.x / hk;
  const int kh = blockIdx.x % hk;
  const int tid = threadIdx.x;
  const int hh = tid / kGroup;            // value head within the key head
  const int h = kh * kRatio + hh;
  const int gt = tid % kGroup;            // thread within the value head's group
  const int gwave = gt / kWave;
  const int lane = tid % kWave;
  const int cg = gt % 32;                 // column group: columns 4cg .. 4cg+3
  const int rg = gt / 32;                 // row group: rows rg + 8m

  __shared__ float s_q[kD], s_k[kD], s_scal[2];
  __shared__ float s_v[kRatio][kD], s_o[kRatio][kD], s_nrm[kRatio][2];

  // issue the state loads first; the conv and norms below overlap their latency.
  // The state (fp32, or fp16 widened to fp32) is streamed once per step.
  // A window of kWindow rows is in flight: the first rows are issued here and
  // each processed row issues the load of the row kWindow after it, which keeps
  // the registers of two workgroups per CU within the register file.
  TS* S = state + ((int64_t)b * hv + h) * kD * kD;
  auto load_row = [&](int m) { return state_load4(S + (rg + 8 * m) * kD + 4 * cg); };
  f32x4_t sreg[kRowsPerThread];
#pragma unroll
  for (int m = 0; m < kWindow; ++m) sreg[m] = load_row(m);

  const T* x_row = x + (int64_t)b * cc;
  T* cs_row = conv_state + (int64_t)b * 3 * cc;
  if (tid < 2 * kD) {   // the key head's q and k channels
    const int c = tid < kD ? kh * kD + tid : hk * kD + kh * kD + (tid - kD);
    const float y = conv_channel(x_row, conv_w, cs_row, c, cc, act);
    if (tid < kD) s_q[tid] = y; else s_k[tid - kD] = y;
  }
  if (gt < kD) s_v[hh][gt] = conv_channel(x_row, conv_w, cs_row, 2 * hk * kD + h * kD + gt, cc, act);
  __syncthreads();
  if (tid < 2 * kWave) {
    const int w = tid / kWave;
    const float* src = w == 0 ? s_q : s_k;
    const float a0 = src[2 * lane], a1 = src[2 * lane + 1];
    const float ss = wave_sum(a0 * a0 + a1 * a1);
    if (lane == 0) s_scal[w] = 1.0f / sqrtf(ss + l2_eps);
  }
  __syncthreads();
  const float rq = s_scal[0] * q_scale, rk = s_scal[1];
  // khat . qtil, computed by every wave (no exchange needed)
  const float kq = wave_sum(s_k[2 * lane] * s_q[2 * lane] + s_k[2 * lane + 1] * s_q[2 * lane + 1]) * rq * rk;
  // this thread's normalised key / query columns and decay factors
  float kcol[4], qcol[4], a[4], bt;
#pragma unroll
  for (int e = 0; e < 4; ++e) { kcol[e] = s_k[4 * cg + e] * rk; qcol[e] = s_q[4 * cg + e] * rq; }
  if constexpr (kPerChannel) {
    const f32x4_t gv = *reinterpret_cast<const f32x4_t*>(gates.g + ((int64_t)b * hv + h) * kD + 4 * cg);
#pragma unroll
    for (int e = 0; e < 4; ++e) a[e] = __expf(gv[e]);
    bt = gates.beta[(int64_t)b * hv + h];
  } else {
    float gs;
    gate_pair<T>(gates, b, hv, h, gs, bt);   // given, or derived from the a / b projections
    const float av = __expf(gs);
#pragma unroll
    for (int e = 0; e < 4; ++e) a[e] = av;
  }

  // per row: decay, the two dot products reduced over the row's 32 lanes,
  // u = beta (v - p), o = r + u (khat . qtil), then the row is updated and
  // written back: S' = Sd + u khat^T
#pragma unroll
  for (int m = 0; m < kRowsPerThread; ++m) {
    if (m + kWindow < kRowsPerThread) sreg[m + kWindow] = load_row(m + kWindow);
    const int row = rg + 8 * m;
    float pk = 0.0f, pq = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sreg[m][e] *= a[e];
      pk = fmaf(sreg[m][e], kcol[e], pk);
      pq = fmaf(sreg[m][e], qcol[e], pq);
    }
    pk = row32_sum(pk);
    pq = row32_sum(pq);
    const float u = bt * (s_v[hh][row] - pk);
    if (cg == 0) s_o[hh][row] = fmaf(u, kq, pq);
#pragma unroll
    for (int e = 0; e < 4; ++e) sreg[m][e] = fmaf(u, kcol[e], sreg[m][e]);
    state_store4(S + row * kD + 4 * cg, sreg[m]);
  }
  __syncthreads();

  // the sigmoid gated RMSNorm of the head's 128 outputs
  if (gt < kD) {
    const float o = s_o[hh][gt];
    const float ss = wave_sum(o * o);
    if (lane == 0) s_nrm[hh][gwave] = ss;
  }
  __syncthreads();
  if (gt < kD) {
    const float o = s_o[hh][gt];
    const float r = rsqrtf((s_nrm[hh][0] + s_nrm[hh][1]) * (1.0f / kD) + rms_eps);
    const int64_t off = ((int64_t)b * hv + h) * kD + gt;
    st(out + off, o * r * norm_w[gt] * sigmoidf_(ld(z + off)));
  }
}

template <typename T, typename To, typename TS, bool kPC>
hipError_t decode_ratio(const Dims& d, const void* x, const float* conv_w, void* conv_state,
                        const Gates& gt, const void* z, const float* norm_w,
                        void* state, void* out, int b, hipStream_t s) {
  const int ratio = d.hv / d.hk;
  dim3 grid(b * d.hk);
#define GDN_DECODE_LAUNCH(R)                                                                      \
  hipLaunchKernelGGL((decode_step_kernel<T, To, TS, kPC, R>), grid, dim3(kGroup * (R)), 0, s,     \
                     static_cast<const T*>(x), conv_w, static_cast<T*>(conv_state), gt,          \
                     static_cast<const T*>(z), norm_w, static_cast<TS*>(state),                  \
                     static_cast<To*>(out), d.hk, d.hv,                                          \
                     d.cc, d.act, d.l2_eps, d.q_scale, d.rms_eps)
  switch (ratio) {
    case 1: GDN_DECODE_LAUNCH(1); break;
    case 2: GDN_DECODE_LAUNCH(2); break;
    case 3: GDN_DECODE_LAUNCH(3); break;
    case 4: GDN_DECODE_LAUNCH(4); break;
    default: return hipErrorInvalidValue;
  }
#undef GDN_DECODE_LAUNCH
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
