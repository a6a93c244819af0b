// gdn_conv.hip -- depthwise causal conv1d (width 4) over the projected
// [Q|K|V] rows: token-parallel prefill over packed sequences, the carried
// conv-state write-back, and the one-token decode step.
//
// Follows the conv leg of pegainfer PR #1152 (Consumer section: Qwen3.5 causal
// conv1d prefill kernel, bit-exact leg) and the GLM-5.3 kernel TDD ledger's
// conv slice (a step equals the full width-4 causal conv).  Tap w[c][3] meets
// the current token; carried state rows are oldest first.
//
// Memory: each thread owns 4 adjacent channels (8 bytes of bf16, 16 of fp32)
// and a tile of 16 tokens (with 8 channels the 19 rows held 136 VGPRs and
// three waves per SIMD, and a 4096-token prefill's 1,280 workgroups ran in
// 1.7 rounds; with 4, twice the workgroups at higher occupancy: -3.5 us).  Inside a sequence it loads the tile's 16 rows and the 3
// before it at once and then computes, so x is read about once (19 rows per 16
// tokens, the extra 3 mostly from L2) and y written once (HBM-bound: 2 + 2 bytes
// per element in bf16).  Tiles that meet a sequence start walk token by token,
// taking the rows before the start from the carried conv state.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

constexpr int kConvTile = 16;     // tokens per thread
constexpr int kConvVec = 4;       // channels per thread
constexpr int kConvThreads = 256;

template <typename T>
__device__ __forceinline__ void load4(const T* p, float (&v)[kConvVec]) {
  if constexpr (sizeof(T) == 2) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    v[0] = __uint_as_float(u.x << 16);
    v[1] = __uint_as_float(u.x & 0xffff0000u);
    v[2] = __uint_as_float(u.y << 16);
    v[3] = __uint_as_float(u.y & 0xffff0000u);
  } else {
    const f32x4_t a = *reinterpret_cast<const f32x4_t*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = a[i];
  }
}

template <typename T>
__device__ __forceinline__ void store4(T* p, const float (&v)[kConvVec]) {
  if constexpr (sizeof(T) == 2) {
    uint2 u;   // pairs through one conversion each (round to nearest even)
    u.x = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{v[0], v[1]}, bf16x2_t));
    u.y = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{v[2], v[3]}, bf16x2_t));
    *reinterpret_cast<uint2*>(p) = u;
  } else {
    *reinterpret_cast<f32x4_t*>(p) = f32x4_t{v[0], v[1], v[2], v[3]};
  }
}

__device__ __forceinline__ float conv_activation(float y, int act) {
  return act ? silu_conv(y) : y;
}

// Sequence holding token t: the n with cu[n] <= t < cu[n+1] (empty sequences skipped).
__device__ __forceinline__ int find_sequence(const int32_t* cu, int n_seq, int t) {
  int lo = 0, hi = n_seq - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

template <typename T>
__global__ __launch_bounds__(kConvThreads) void conv1d_prefill_kernel(
    const T* __restrict__ x, int64_t x_stride, const float* __restrict__ w,
    const T* __restrict__ cs_in, T* __restrict__ y, int64_t y_stride,
    const int32_t* __restrict__ cu, int n_seq, int n_tok, int cc, int act) {
  const int c0 = (blockIdx.x * kConvThreads + threadIdx.x) * kConvVec;
  if (c0 >= cc) return;
  const int t_begin = blockIdx.y * kConvTile;
  const int t_end = min(t_begin + kConvTile, n_tok);

  float wt[4][kConvVec];
#pragma unroll
  for (int e = 0; e < kConvVec; ++e) {
    const f32x4_t wv = *reinterpret_cast<const f32x4_t*>(w + (int64_t)(c0 + e) * 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) wt[i][e] = wv[i];
  }

  int n = find_sequence(cu, n_seq, t_begin);
  int seq_start = cu[n], seq_end = cu[n + 1];

  // Common case: the tile and its three history rows lie inside one sequence.
  // All 19 rows are loaded before any is used, so each thread keeps 19 loads
  // in flight instead of one per token.
  if (t_begin - 3 >= seq_start && t_end <= seq_end) {
    constexpr int kRows = kConvTile + 3;
    float rows[kRows][kConvVec];
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
      const int pos = min(t_begin - 3 + i, t_end - 1);   // rows past the tile end are never used
      load4(x + (int64_t)pos * x_stride + c0, rows[i]);
    }
#pragma unroll
    for (int i = 0; i < kConvTile; ++i) {
      if (t_begin + i < t_end) {
        float out[kConvVec];
#pragma unroll
        for (int e = 0; e < kConvVec; ++e) {
          float acc = wt[0][e] * rows[i][e];
          acc = fmaf(wt[1][e], rows[i + 1][e], acc);
          acc = fmaf(wt[2][e], rows[i + 2][e], acc);
          acc = fmaf(wt[3][e], rows[i + 3][e], acc);
          out[e] = conv_activation(acc, act);
        }
        store4(y + (int64_t)(t_begin + i) * y_stride + c0, out);
      }
    }
    return;
  }

  // hist[j] holds the input at position t - 3 + j of the current token t.
  float hist[3][kConvVec];
  auto fill_history = [&](int t) {
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const int pos = t - 3 + j;
      if (pos >= seq_start) {
        load4(x + (int64_t)pos * x_stride + c0, hist[j]);
      } else if (cs_in) {
        load4(cs_in + ((int64_t)n * 3 + (3 + pos - seq_start)) * cc + c0, hist[j]);
      } else {
#pragma unroll
        for (int e = 0; e < kConvVec; ++e) hist[j][e] = 0.0f;
      }
    }
  };
  fill_history(t_begin);
  for (int t = t_begin; t < t_end; ++t) {
    if (t >= seq_end) {
      while (cu[n + 1] <= t) ++n;
      seq_start = cu[n];
      seq_end = cu[n + 1];
      fill_history(t);
    }
    float cur[kConvVec], out[kConvVec];
    load4(x + (int64_t)t * x_stride + c0, cur);
#pragma unroll
    for (int e = 0; e < kConvVec; ++e) {
      float acc = wt[0][e] * hist[0][e];
      acc = fmaf(wt[1][e], hist[1][e], acc);
      acc = fmaf(wt[2][e], hist[2][e], acc);
      acc = fmaf(wt[3][e], cur[e], acc);
      out[e] = conv_activation(acc, act);
      hist[0][e] = hist[1][e];
      hist[1][e] = hist[2][e];
      hist[2][e] = cur[e];
    }
    store4(y + (int64_t)t * y_stride + c0, out);
  }
}

// Last three inputs of each sequence (carried rows when it is shorter than 3).
// Runs after the prefill kernel so that conv_state_out may alias conv_state_in:
// each thread reads its three values before writing them.
template <typename T>
__global__ __launch_bounds__(kConvThreads) void conv1d_state_out_kernel(
    const T* __restrict__ x, int64_t x_stride, const T* cs_in, T* cs_out,
    const int32_t* __restrict__ cu, int cc) {
  const int c = blockIdx.x * kConvThreads + threadIdx.x;
  const int n = blockIdx.y;
  if (c >= cc) return;
  const int start = cu[n];
  const int len = cu[n + 1] - start;
  float keep[3];
#pragma unroll
  for (int r = 0; r < 3; ++r) {
    const int pos = len - 3 + r;
    if (pos >= 0) keep[r] = ld(x + (int64_t)(start + pos) * x_stride + c);
    else keep[r] = cs_in ? ld(cs_in + ((int64_t)n * 3 + (3 + pos)) * cc + c) : 0.0f;
  }
#pragma unroll
  for (int r = 0; r < 3; ++r) st(cs_out + ((int64_t)n * 3 + r) * cc + c, keep[r]);
}

template <typename T>
__global__ __launch_bounds__(kConvThreads) void conv1d_step_kernel(
    const T* __restrict__ x, int64_t x_stride, const float* __restrict__ w, T* cs,
    T* __restrict__ y, int64_t y_stride, int cc, int act) {
  const int c = blockIdx.x * kConvThreads + threadIdx.x;
  const int b = blockIdx.y;
  if (c >= cc) return;
  T* row = cs + (int64_t)b * 3 * cc + c;
  const float s0 = ld(row), s1 = ld(row + cc), s2 = ld(row + 2 * cc);
  const float xv = ld(x + (int64_t)b * x_stride + c);
  const f32x4_t wv = *reinterpret_cast<const f32x4_t*>(w + (int64_t)c * 4);
  float acc = wv[0] * s0;
  acc = fmaf(wv[1], s1, acc);
  acc = fmaf(wv[2], s2, acc);
  acc = fmaf(wv[3], xv, acc);
  st(y + (int64_t)b * y_stride + c, conv_activation(acc, act));
  st(row, s1);
  st(row + cc, s2);
  st(row + 2 * cc, xv);
}

template <typename T>
hipError_t conv_prefill_impl(const Dims& d, const void* x, int64_t x_stride, const float* w,
                             const void* cs_in, void* cs_out, void* y, int64_t y_stride,
                             const int32_t* cu, int n, int t, hipStream_t s) {
  if (t > 0) {
    const int per_block = kConvThreads * kConvVec;
    dim3 grid((d.cc + per_block - 1) / per_block, (t + kConvTile - 1) / kConvTile);
    hipLaunchKernelGGL(conv1d_prefill_kernel<T>, grid, dim3(kConvThreads), 0, s,
                       static_cast<const T*>(x), x_stride, w, static_cast<const T*>(cs_in),
                       static_cast<T*>(y), y_stride, cu, n, t, d.cc, d.act);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (cs_out && n > 0) {
    dim3 grid((d.cc + kConvThreads - 1) / kConvThreads, n);
    hipLaunchKernelGGL(conv1d_state_out_kernel<T>, grid, dim3(kConvThreads), 0, s,
                       static_cast<const T*>(x), x_stride, static_cast<const T*>(cs_in),
                       static_cast<T*>(cs_out), cu, d.cc);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_conv1d_prefill(const Dims& d, bool bf16, const void* x, int64_t x_stride,
                                 const float* w, const void* cs_in, void* cs_out, void* y,
                                 int64_t y_stride, const int32_t* cu, int n, int t,
                                 hipStream_t s) {
  return bf16 ? conv_prefill_impl<uint16_t>(d, x, x_stride, w, cs_in, cs_out, y, y_stride, cu, n, t, s)
              : conv_prefill_impl<float>(d, x, x_stride, w, cs_in, cs_out, y, y_stride, cu, n, t, s);
}

hipError_t launch_conv1d_step(const Dims& d, bool bf16, const void* x, int64_t x_stride,
                              const float* w, void* cs, void* y, int64_t y_stride, int b,
                              hipStream_t s) {
  if (b == 0) return hipSuccess;
  dim3 grid((d.cc + kConvThreads - 1) / kConvThreads, b);
  if (bf16)
    hipLaunchKernelGGL(conv1d_step_kernel<uint16_t>, grid, dim3(kConvThreads), 0, s,
                       static_cast<const uint16_t*>(x), x_stride, w, static_cast<uint16_t*>(cs),
                       static_cast<uint16_t*>(y), y_stride, d.cc, d.act);
  else
    hipLaunchKernelGGL(conv1d_step_kernel<float>, grid, dim3(kConvThreads), 0, s,
                       static_cast<const float*>(x), x_stride, w, static_cast<float*>(cs),
                       static_cast<float*>(y), y_stride, d.cc, d.act);
  return hipGetLastError();
}

}  // namespace gdn
