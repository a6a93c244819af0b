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
// One wavefront per vector of dv = 128: each lane owns two adjacent elements
// (one 8-byte fp32 or 4-byte bf16 access, coalesced across the wave).  Pure
// streaming: HBM-bound.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

constexpr int kNormThreads = 256;
constexpr int kVecPerBlock = kNormThreads / kWave;

template <typename Ti, typename Tz, typename To>
__global__ __launch_bounds__(kNormThreads) void gated_rmsnorm_kernel(
    const Ti* o, const Tz* __restrict__ z, const float* __restrict__ w, To* out,
    int64_t vectors, float eps) {
  const int lane = threadIdx.x % kWave;
  const int64_t vec = (int64_t)blockIdx.x * kVecPerBlock + threadIdx.x / kWave;
  if (vec >= vectors) return;
  const int64_t base = vec * 128 + 2 * lane;
  const float o0 = ld(o + base), o1 = ld(o + base + 1);
  const float ss = wave_sum(o0 * o0 + o1 * o1);
  const float r = rsqrtf(ss * (1.0f / 128.0f) + eps);
  const float y0 = o0 * r * w[2 * lane] * sigmoidf_(ld(z + base));
  const float y1 = o1 * r * w[2 * lane + 1] * sigmoidf_(ld(z + base + 1));
  st(out + base, y0);
  st(out + base + 1, y1);
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
