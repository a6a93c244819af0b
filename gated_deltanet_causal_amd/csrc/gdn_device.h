// gdn_device.h -- device helpers for the gfx950 GDN kernels: bf16 storage
// conversion, hi/lo splitting of fp32 operands, MFMA tile wrappers and
// wavefront reductions.  Internal to libgdn.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_launch.h"

namespace gdn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Storage types.  bf16 values are carried as raw 16-bit patterns (uint16_t)
// in memory; arithmetic is always fp32.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round to nearest even (the hardware conversion of gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

template <typename T> struct Storage;
template <> struct Storage<float> {
  __device__ static __forceinline__ float load(const float* p) { return *p; }
  __device__ static __forceinline__ void store(float* p, float v) { *p = v; }
};
template <> struct Storage<uint16_t> {
  __device__ static __forceinline__ float load(const uint16_t* p) { return bf16_bits_to_f32(*p); }
  __device__ static __forceinline__ void store(uint16_t* p, float v) { *p = f32_to_bf16_bits(v); }
};

template <typename T> __device__ __forceinline__ float ld(const T* p) { return Storage<T>::load(p); }
template <typename T> __device__ __forceinline__ void st(T* p, float v) { Storage<T>::store(p, v); }

// ---------------------------------------------------------------------------
// hi/lo split of an fp32 value into two bf16 values with hi + lo equal to x
// up to 2^-17 relative: hi = rne(x), lo = rne(x - hi); x - hi is exact.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void split_bf16(float x, __bf16& hi, __bf16& lo) {
  hi = static_cast<__bf16>(x);
  lo = static_cast<__bf16>(x - static_cast<float>(hi));
}

// Two fp32 values -> their bf16 hi parts and bf16 lo parts (x = hi + lo up to
// 2^-17 relative), each pair packed in one dword: three VALU ops per value.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void split2(float a, float b, uint32_t& hp, uint32_t& lp) {
  hp = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
  const float ha = __uint_as_float(hp << 16), hb = __uint_as_float(hp & 0xffff0000u);
  lp = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a - ha, b - hb}, bf16x2_t));
}

// ---------------------------------------------------------------------------
// MFMA 16x16 output tiles.  Accumulator layout (both instructions): lane l
// holds C[4*(l/16) + r][l%16] in element r (r = 0..3).  Operand layout: lane l
// holds A[l%16][k0 + E*(l/16) + e] and B[k0 + E*(l/16) + e][l%16], e < E, with
// E = 8 (bf16, K = 32 per instruction) or E = 1 (fp32, K = 4).  Only the
// pairing of A's and B's k slots matters for the product, and both operands
// are always loaded with the same k mapping.
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x4_t mfma_bf16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma_f32(float a, float b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// fp16 operands (the register-resident chunk spines): 11 significant bits, so a
// single rounding of an fp32 operand costs at most 2^-11 relative.
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ f32x4_t mfma_f16(f16x8_t a, f16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
// Two fp32 values rounded to fp16 (nearest even), packed low-first in one dword.
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, f16x2_t));
}
__device__ __forceinline__ f16x8_t as_f16x8(u32x4_t u) { return __builtin_bit_cast(f16x8_t, u); }
__device__ __forceinline__ f16x8_t load_f16x8(const uint16_t* p) {  // 16-byte aligned
  return __builtin_bit_cast(f16x8_t, *reinterpret_cast<const u32x4_t*>(p));
}

__device__ __forceinline__ bf16x8_t load_bf16x8(const uint16_t* p) {  // 16-byte aligned
  return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(p));
}
__device__ __forceinline__ bf16x8_t load_bf16x8(const __bf16* p) {
  return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(p));
}

// ---------------------------------------------------------------------------
// Wavefront reductions (64 lanes).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Sum over aligned groups of `width` lanes (width a power of two <= 64).
template <int width>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = width / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Sum over aligned groups of 4 lanes with DPP quad permutes (no LDS crossbar).
__device__ __forceinline__ float quad_sum(float v) {
  // quad_perm [1,0,3,2] then [2,3,0,1]
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));
  return v;
}

// sigmoid(x) = 1 / (1 + 2^(-x log2 e)) on the hardware exp2 and reciprocal (each within 1 ulp),
// not an IEEE division, which was half the conv's instructions where the conv is VALU-bound.
// Every sigmoid of the library (the conv's SiLU, the norm's output gate, beta from b) is this
// one, so that the paths that compute the same value agree.
__device__ __forceinline__ float sigmoidf_(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.44269504f * x));
}

// The conv's SiLU activation, y sigmoid(y).
__device__ __forceinline__ float silu_conv(float y) { return y * sigmoidf_(y); }

// Four consecutive values of a recurrent state, stored as fp32 or as fp16
// (the fp16 h-state: widened on load, rounded to nearest even on store, so
// the arithmetic stays fp32 and the state is rounded once per token).  The
// state is streamed once per step, hence non-temporal.
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4_t state_load4(const float* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
}
__device__ __forceinline__ f32x4_t state_load4(const _Float16* p) {
  return __builtin_convertvector(__builtin_nontemporal_load(reinterpret_cast<const f16x4_t*>(p)), f32x4_t);
}
__device__ __forceinline__ void state_store4(float* p, f32x4_t v) {
  __builtin_nontemporal_store(v, reinterpret_cast<f32x4_t*>(p));
}
__device__ __forceinline__ void state_store4(_Float16* p, f32x4_t v) {
  __builtin_nontemporal_store(__builtin_convertvector(v, f16x4_t), reinterpret_cast<f16x4_t*>(p));
}

// Sum over the 32 lanes holding one state row (aligned halves of the wave):
// quad_perm swaps for lane distance 1 and 2, the half-row and row mirrors for
// 4 and 8, and a swizzle exchanging lane i with i ^ 16 for the last step.
template <int kCtrl>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, 0xf, 0xf, false));
}
// Sum over each row of 16 lanes (quad sums, then rotations by 4 and 8 within the row).
__device__ __forceinline__ float row16_sum(float v) {
  v = quad_sum(v);
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x124, 0xF, 0xF, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x128, 0xF, 0xF, true));
  return v;
}

__device__ __forceinline__ float row32_sum(float v) {
  v = dpp_add<0xB1>(v);    // quad_perm [1,0,3,2]
  v = dpp_add<0x4E>(v);    // quad_perm [2,3,0,1]
  v = dpp_add<0x141>(v);   // row_half_mirror
  v = dpp_add<0x140>(v);   // row_mirror
  return v + __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
}

// Gates of one token and value head from the a / b projections (the prepare
// stage's gate derivation, as read from the golden PR and the TDD ledger's
// alpha/beta transforms): g = -exp(A_log) softplus(a + dt_bias), beta =
// sigmoid(b); softplus(x) = log(1 + e^x), as x + log1p(e^-x) for x > 0.
__device__ __forceinline__ void derive_gates(float a, float b, float A_log, float dt_bias, float& g,
                                             float& beta) {
  const float x = a + dt_bias;
  const float sp = x > 0.0f ? x + log1pf(__expf(-x)) : log1pf(__expf(x));
  g = -__expf(A_log) * sp;
  beta = sigmoidf_(b);
}

// The raw gate inputs of row t, value head h (scalar decay): a, b (storage
// type, unconverted), A_log, dt_bias when the gates are derived, else g and
// beta.  Loaded apart from gate_resolve() so that a kernel can issue the loads
// early: nothing in the loading branch uses a loaded value, so no wait for
// them is placed there.
template <typename T>
struct GateRaw {
  T a, b;
  float g, beta, A_log, dt_bias;
};
template <typename T>
__device__ __forceinline__ GateRaw<T> gate_raw(const Gates& gt, int64_t t, int hv, int h) {
  const int64_t i = t * hv + h;
  GateRaw<T> r{};
  if (gt.a) {
    r.a = static_cast<const T*>(gt.a)[i];
    r.b = static_cast<const T*>(gt.b)[i];
    r.A_log = gt.A_log[h];
    r.dt_bias = gt.dt_bias[h];
  } else {
    r.g = gt.g[i];
    r.beta = gt.beta[i];
  }
  return r;
}
// Branch-free (both forms computed, one selected), so that a compiler cannot
// merge it into gate_raw's branch and pull the arithmetic up to the loads.
template <typename T>
__device__ __forceinline__ void gate_resolve(const Gates& gt, const GateRaw<T>& r, float& g, float& beta) {
  float gd, bd;
  derive_gates(ld(&r.a), ld(&r.b), r.A_log, r.dt_bias, gd, bd);
  const bool derived = gt.a != nullptr;
  g = derived ? gd : r.g;
  beta = derived ? bd : r.beta;
}

// g and beta of row t, value head h (scalar decay)
template <typename T>
__device__ __forceinline__ void gate_pair(const Gates& gt, int64_t t, int hv, int h, float& g, float& beta) {
  gate_resolve(gt, gate_raw<T>(gt, t, hv, h), g, beta);
}

}  // namespace gdn
