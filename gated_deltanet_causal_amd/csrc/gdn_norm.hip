// gdn_norm.hip -- gated RMSNorm with the sigmoid gate over [rows][Hv][dv]
// vectors, all rows and heads in one launch.
//
// Follows pegainfer PR #1152 (Summary and Negative controls: the checkpoint's
// output gate is sigmoid, not SiLU; code review: rsqrt(variance + eps), eps
// 1e-6) and the Qwen3SsmLayer field notes on the strided gated norm (one launch
// walks every sequence instead of one launch per row).
//
//   out[i] = o[i] * rsqrt(mean_i o^2 + eps) * w[i] * sigmoid(z[i])
//
// Sixteen lanes per vector of dv = 128: each lane owns eight adjacent elements
// (16- or 32-byte accesses, coalesced across the wave), a wave covers four
// vectors per step and takes two steps at once so each lane keeps two sets of
// loads in flight.  The sum of squares is reduced inside each 16-lane row with
// DPP.  Pure streaming: HBM-bound.
#include <type_traits>

#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

constexpr int kNormThreads = 256;
constexpr int kVecPerWaveStep = kWave / 16;                   // 4
constexpr int kSteps = 2;                                     // vector groups per wave
constexpr int kVecPerBlock = kNormThreads / kWave * kVecPerWaveStep * kSteps;   // 32

template <typename T>
__device__ __forceinline__ void ld8(const T* p, float (&v)[8]) {
  if constexpr (std::is_same_v<T, _Float16>) {
    const f16x8_t h = load_f16x8(reinterpret_cast<const uint16_t*>(p));
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (float)h[i];
  } else if constexpr (sizeof(T) == 2) {
    const u32x4_t u = *reinterpret_cast<const u32x4_t*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(u[i] << 16);
      v[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    }
  } else {
    const f32x4_t a = *reinterpret_cast<const f32x4_t*>(p);
    const f32x4_t b = *reinterpret_cast<const f32x4_t*>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
  }
}

template <typename T>
__device__ __forceinline__ void st8(T* p, const float (&v)[8]) {
  if constexpr (sizeof(T) == 2) {
    u32x4_t u;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      u[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{v[2 * i], v[2 * i + 1]}, bf16x2_t));
    *reinterpret_cast<u32x4_t*>(p) = u;
  } else {
    *reinterpret_cast<f32x4_t*>(p) = f32x4_t{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4_t*>(p + 4) = f32x4_t{v[4], v[5], v[6], v[7]};
  }
}

// Sum over each row of 16 lanes (quad sums, then rotations by 4 and 8 lanes).
template <typename Ti, typename Tz, typename To>
__global__ __launch_bounds__(kNormThreads) void gated_rmsnorm_kernel(
    const Ti* o, const Tz* __restrict__ z, const float* __restrict__ w, To* out,
    int64_t vectors, float eps) {
  const int lane = threadIdx.x % kWave, q = lane & 15;
  const int64_t first = (int64_t)blockIdx.x * kVecPerBlock +
                        (threadIdx.x / kWave) * kVecPerWaveStep * kSteps + (lane >> 4);
  float wv[8];
  {
    const f32x4_t a = *reinterpret_cast<const f32x4_t*>(w + 8 * q);
    const f32x4_t b = *reinterpret_cast<const f32x4_t*>(w + 8 * q + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) { wv[i] = a[i]; wv[4 + i] = b[i]; }
  }
  // vectors handled by this lane's row: first, first + 4 (rows of 16 lanes are
  // all active or all inactive, so the row reduction never reads an idle lane)
  float ov[kSteps][8], zv[kSteps][8];
#pragma unroll
  for (int s = 0; s < kSteps; ++s) {
    const int64_t vec = first + s * kVecPerWaveStep;
    if (vec < vectors) {
      ld8(o + vec * 128 + 8 * q, ov[s]);
      ld8(z + vec * 128 + 8 * q, zv[s]);
    }
  }
#pragma unroll
  for (int s = 0; s < kSteps; ++s) {
    const int64_t vec = first + s * kVecPerWaveStep;
    if (vec < vectors) {
      float ss = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) ss = fmaf(ov[s][i], ov[s][i], ss);
      ss = row16_sum(ss);
      const float r = rsqrtf(ss * (1.0f / 128.0f) + eps);
      float y[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = ov[s][i] * r * wv[i] * sigmoidf_(zv[s][i]);
      st8(out + vec * 128 + 8 * q, y);
    }
  }
}

template <typename Ti, typename Tz, typename To>
hipError_t norm_impl(const Dims& d, const void* o, const void* z, const float* w, void* out,
                     int64_t rows, hipStream_t s) {
  const int64_t vectors = rows * d.hv;
  if (vectors == 0) return hipSuccess;
  const int64_t blocks = (vectors + kVecPerBlock - 1) / kVecPerBlock;
  hipLaunchKernelGGL((gated_rmsnorm_kernel<Ti, Tz, To>), dim3((unsigned)blocks),
                     dim3(kNormThreads), 0, s, static_cast<const Ti*>(o), static_cast<const Tz*>(z), w,
                     static_cast<To*>(out), vectors, d.rms_eps);
  return hipGetLastError();
}

}  // namespace

template <typename Ti, typename Tz>
hipError_t norm_out(const Dims& d, bool out_bf16, const void* o, const void* z, const float* w,
                    void* out, int64_t rows, hipStream_t s) {
  return out_bf16 ? norm_impl<Ti, Tz, uint16_t>(d, o, z, w, out, rows, s)
                  : norm_impl<Ti, Tz, float>(d, o, z, w, out, rows, s);
}

hipError_t launch_gated_rmsnorm_f16o(const Dims& d, bool z_bf16, bool out_bf16, const void* o,
                                     const void* z, const float* w, void* out, int64_t rows,
                                     hipStream_t s) {
  return z_bf16 ? norm_out<_Float16, uint16_t>(d, out_bf16, o, z, w, out, rows, s)
                : norm_out<_Float16, float>(d, out_bf16, o, z, w, out, rows, s);
}

hipError_t launch_gated_rmsnorm(const Dims& d, bool o_bf16, bool z_bf16, bool out_bf16,
                                const void* o, const void* z, const float* w, void* out,
                                int64_t rows, hipStream_t s) {
  if (o_bf16)
    return z_bf16 ? norm_out<uint16_t, uint16_t>(d, out_bf16, o, z, w, out, rows, s)
                  : norm_out<uint16_t, float>(d, out_bf16, o, z, w, out, rows, s);
  return z_bf16 ? norm_out<float, uint16_t>(d, out_bf16, o, z, w, out, rows, s)
                : norm_out<float, float>(d, out_bf16, o, z, w, out, rows, s);
}

}  // namespace gdn
