// gdn_chunk.hip -- chunk-wise (WY form, 64-token chunks) gated delta rule
// prefill over packed variable-length sequences, for gfx950.
//
// Follows pegainfer PR #1152 (Consumer / shipped-line diff: prepare = head
// expansion + L2 norm + split v, then cumsum -> A -> solve -> recompute ->
// state -> output, with the recurrent state carried across chunks) and the
// Qwen3SsmLayer field notes on the chunked prefill's state spine (tensor-core
// products with bf16 operands and an fp32 accumulator that is the state; the
// triangular solve and output square moved onto matrix units).
//
// Per chunk of L <= 64 tokens of one value head, with S0 the [dv][dk] state
// entering the chunk, gam the within-chunk cumulative log decay, rk = 1/|k|,
// rq = q_scale/|q| (K, Q the raw key / query rows), the exact identities used
// are (derivation: the state after token r is
// S0 e^{gam_r} + sum_{j<=r} e^{gam_r - gam_j} u_j khat_j^T):
//   A[r][j]  = beta_r e^{gam_r-gam_j} rk_r rk_j (K K^T)[r][j]      (j < r)
//   Tt       = (I + A)^-1 diag(beta)
//   R        = V - diag(e^{gam} rk) (K S0^T)
//   Vnew     = Tt R                                   (the u_j of the chunk)
//   O        = diag(rq e^{gam}) (Q S0^T) + Pt Vnew,
//              Pt[r][j] = rq_r rk_j e^{gam_r-gam_j} (Q K^T)[r][j]   (j <= r)
//   S_L      = e^{gam_L} S0 + (diag(rk e^{gam_L - gam}) Vnew)^T K
// Decay factors are always formed as e^{difference} (all exponents <= 0).
//
// Kernels
//   plan   prefix sum of chunks per sequence (device side, from cu_seqlens).
//   intra  one workgroup per (chunk, key head): K K^T and Q K^T on MFMA once
//          for the key head, then per value head A, the unit-lower triangular
//          inverse, Tt and Pt.  Tt and Pt are written to the workspace already
//          in the MFMA A-operand lane layout (hi/lo bf16 pairs, or fp32).
//   spine  one workgroup per (sequence, value head, 32-row dv tile): walks the
//          sequence's chunks in order with the fp32 state tile in LDS, running
//          the four products above on MFMA.
// Numerics: the raw bf16 K, Q and V enter MFMA exactly; every fp32 operand
// (state, R, Vnew, Tt, Pt) is split into hi + lo bf16 and multiplied as
// hi*hi + hi*lo + lo*hi (exact-input products need two terms), so products are
// accurate to ~2^-16 relative with fp32 accumulation.  The fp32 input path
// uses fp32 MFMA instead.
#include <algorithm>

#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

constexpr int kC = 64;           // chunk
constexpr int kD = 128;          // head dim (k and v)
constexpr int kTile = 32;        // dv rows per spine workgroup
constexpr int kThreads = 256;
constexpr size_t kFragBytes = 16384;           // one 64x64 operand in lane layout
constexpr size_t kRecBytes = 2 * kFragBytes + 1024;  // Tt, Pt, vectors
constexpr int kSortMax = 4096;                 // longest-first order up to this many sequences
constexpr int kXcds = 8;                       // XCDs; workgroups are dealt to them round-robin

__host__ __device__ constexpr size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Workspace: first[N+1] | order[N] | per-(chunk, value head) records.
__host__ __device__ inline size_t records_offset(int n_seq) {
  return align_up(sizeof(int32_t) * (2 * (size_t)n_seq + 1), 256);
}

template <bool F32> struct Ops;
template <> struct Ops<false> {
  using E = uint16_t;            // storage element in LDS (bf16 bits)
  using F = bf16x8_t;            // MFMA operand fragment
  static constexpr int kEpl = 8, kKs = 32;
  static constexpr int kPadK = 8;     // row padding (elements) of k-contiguous LDS tiles
};
template <> struct Ops<true> {
  using E = float;
  using F = float;
  static constexpr int kEpl = 1, kKs = 4;
  static constexpr int kPadK = 4;
};

template <bool F32>
__device__ __forceinline__ typename Ops<F32>::F frag(const typename Ops<F32>::E* m, int pitch,
                                                      int idx0, int k0) {
  const int l = threadIdx.x % kWave;
  const typename Ops<F32>::E* p = m + (idx0 + (l & 15)) * pitch + k0 + Ops<F32>::kEpl * (l >> 4);
  if constexpr (F32) return *p;
  else return load_bf16x8(p);
}

template <bool F32>
__device__ __forceinline__ f32x4_t mma(typename Ops<F32>::F a, typename Ops<F32>::F b, f32x4_t c) {
  if constexpr (F32) return mfma_f32(a, b, c);
  else return mfma_bf16(a, b, c);
}

// hi/lo fragment pair of an fp32 matrix row segment m[idx][k0 .. k0+E-1] (k contiguous).
template <bool F32>
__device__ __forceinline__ void frag_split_f32(const float* m, int pitch, int idx0, int k0,
                                               typename Ops<F32>::F& hi, typename Ops<F32>::F& lo) {
  const int l = threadIdx.x % kWave;
  const float* p = m + (idx0 + (l & 15)) * pitch + k0 + Ops<F32>::kEpl * (l >> 4);
  if constexpr (F32) {
    hi = *p;
    lo = 0.0f;
  } else {
    const f32x4_t a = *reinterpret_cast<const f32x4_t*>(p);
    const f32x4_t b = *reinterpret_cast<const f32x4_t*>(p + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      __bf16 h0, l0, h1, l1;
      split_bf16(a[e], h0, l0);
      split_bf16(b[e], h1, l1);
      hi[e] = h0; lo[e] = l0; hi[4 + e] = h1; lo[4 + e] = l1;
    }
  }
}

// Store the four accumulator rows of a lane (rows t0+4(l/16)+r, column c) transposed:
// mt[c][t0 + 4(l/16) + r] for r = 0..3, as hi/lo bf16 (or one fp32 array).
template <bool F32>
__device__ __forceinline__ void store_acc_transposed(typename Ops<F32>::E* hi, typename Ops<F32>::E* lo,
                                                     int pitch, int c0, int t0, f32x4_t v) {
  const int l = threadIdx.x % kWave;
  const int off = (c0 + (l & 15)) * pitch + t0 + 4 * (l >> 4);
  if constexpr (F32) {
    *reinterpret_cast<f32x4_t*>(hi + off) = v;
  } else {
    uint32_t h2[2], l2[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      __bf16 ha, la, hb, lb;
      split_bf16(v[2 * e], ha, la);
      split_bf16(v[2 * e + 1], hb, lb);
      h2[e] = __builtin_bit_cast(uint16_t, ha) | (uint32_t(__builtin_bit_cast(uint16_t, hb)) << 16);
      l2[e] = __builtin_bit_cast(uint16_t, la) | (uint32_t(__builtin_bit_cast(uint16_t, lb)) << 16);
    }
    *reinterpret_cast<uint2*>(hi + off) = make_uint2(h2[0], h2[1]);
    *reinterpret_cast<uint2*>(lo + off) = make_uint2(l2[0], l2[1]);
  }
}

// Chunk index -> sequence: largest n with first[n] <= c (first is a prefix sum).
__device__ __forceinline__ int chunk_sequence(const int32_t* first, int n_seq, int c) {
  int lo = 0, hi = n_seq - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (first[mid] <= c) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// ---------------------------------------------------------------------------
// plan: first[n] = sum_{m<n} ceil(len_m / 64), n = 0..N
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void chunk_plan_kernel(const int32_t* __restrict__ cu,
                                                              int n_seq, int32_t* __restrict__ first,
                                                              int32_t* __restrict__ order) {
  __shared__ int32_t part[kThreads];
  const int per = (n_seq + kThreads - 1) / kThreads;
  const int beg = threadIdx.x * per;
  const int end = min(beg + per, n_seq);
  int32_t sum = 0;
  for (int n = beg; n < end; ++n) sum += (cu[n + 1] - cu[n] + kC - 1) / kC;
  part[threadIdx.x] = sum;
  __syncthreads();
  if (threadIdx.x == 0) {
    int32_t run = 0;
    for (int i = 0; i < kThreads; ++i) { const int32_t v = part[i]; part[i] = run; run += v; }
    first[n_seq] = run;
  }
  __syncthreads();
  int32_t run = part[threadIdx.x];
  for (int n = beg; n < end; ++n) {
    first[n] = run;
    run += (cu[n + 1] - cu[n] + kC - 1) / kC;
  }
  // Spine order: longest sequence first (ties by index), so the longest serial
  // chains start earliest.  Quadratic rank count; identity order past kSortMax.
  for (int n = threadIdx.x; n < n_seq; n += kThreads) {
    int rank = n;
    if (n_seq <= kSortMax) {
      const int len = cu[n + 1] - cu[n];
      rank = 0;
      for (int m = 0; m < n_seq; ++m) {
        const int lm = cu[m + 1] - cu[m];
        rank += (lm > len) || (lm == len && m < n);
      }
    }
    order[rank] = n;
  }
}

// Load a 64 x 128 tile of raw key or query rows (zero rows past L) into LDS.
template <bool F32, typename Tin>
__device__ __forceinline__ void load_rows(typename Ops<F32>::E* dst, int pitch, const Tin* src,
                                          int64_t stride, int L) {
  // each thread moves 16-byte pieces: 8 bf16 (bf16 input) or 4 fp32 (fp32 input)
  constexpr int kPer = 16 / sizeof(Tin);
  constexpr int kPieces = kC * kD / kPer;
  for (int p = threadIdx.x; p < kPieces; p += kThreads) {
    const int r = p / (kD / kPer);
    const int c = (p % (kD / kPer)) * kPer;
    typename Ops<F32>::E* d = dst + r * pitch + c;
    if constexpr (F32) {
      f32x4_t v = {0.f, 0.f, 0.f, 0.f};
      if (r < L) v = *reinterpret_cast<const f32x4_t*>(src + r * stride + c);
      *reinterpret_cast<f32x4_t*>(d) = v;
    } else {
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (r < L) v = *reinterpret_cast<const u32x4_t*>(src + r * stride + c);
      *reinterpret_cast<u32x4_t*>(d) = v;
    }
  }
}


// Number of (row tile, k step) fragment slots of a lower-triangular 64x64
// operand in lane layout: k steps up to the diagonal of each 16-row tile.
template <bool F32> struct Tri;
template <> struct Tri<false> {            // bf16: k step 32 -> 1,1,2,2 steps
  static constexpr int kSlots = 6;
  __device__ static constexpr int slot(int mt, int ks) { return mt < 2 ? mt : 2 + 2 * (mt - 2) + ks; }
};
template <> struct Tri<true> {             // fp32: k step 4 -> 4,8,12,16 steps
  static constexpr int kSlots = 40;
  __device__ static constexpr int slot(int mt, int ks) { return 2 * mt * (mt + 1) + ks; }
};

// All of this lane's fragments of a triangular operand record (hi and lo).
template <bool F32>
__device__ __forceinline__ void load_tri_frags(const uint8_t* src, int lane, typename Ops<F32>::F* fh,
                                               typename Ops<F32>::F* fl) {
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
    for (int ks = 0; ks * Ops<F32>::kKs <= 16 * mt + 15; ++ks) {
      const int sl = Tri<F32>::slot(mt, ks);
      if constexpr (F32) {
        fh[sl] = reinterpret_cast<const float*>(src)[(mt * 16 + ks) * kWave + lane];
      } else {
        const int f = mt * 2 + ks;
        fh[sl] = *reinterpret_cast<const bf16x8_t*>(src + ((size_t)(f * 2 + 0) * kWave + lane) * 16);
        fl[sl] = *reinterpret_cast<const bf16x8_t*>(src + ((size_t)(f * 2 + 1) * kWave + lane) * 16);
      }
    }
  }
}

// 64 x 32 value tile (rows past L zero) as fp32 into LDS, 16-byte loads.
template <typename Tin>
__device__ __forceinline__ void load_values(float* sV, int pitch, const Tin* src, int64_t stride, int L) {
  constexpr int kPer = 16 / sizeof(Tin);
  for (int p = threadIdx.x; p < kC * (kTile / kPer); p += kThreads) {
    const int t = p / (kTile / kPer);
    const int i = (p % (kTile / kPer)) * kPer;
    float vals[kPer];
    if constexpr (sizeof(Tin) == 2) {
      u32x4_t u = {0u, 0u, 0u, 0u};
      if (t < L) u = *reinterpret_cast<const u32x4_t*>(src + (int64_t)t * stride + i);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vals[2 * e] = __uint_as_float(u[e] << 16);
        vals[2 * e + 1] = __uint_as_float(u[e] & 0xffff0000u);
      }
    } else {
      f32x4_t u = {0.f, 0.f, 0.f, 0.f};
      if (t < L) u = *reinterpret_cast<const f32x4_t*>(src + (int64_t)t * stride + i);
#pragma unroll
      for (int e = 0; e < 4; ++e) vals[e] = u[e];
    }
#pragma unroll
    for (int e = 0; e < kPer; ++e) sV[t * pitch + i + e] = vals[e];
  }
}


// 16x16x16 fp32 product on fp32 MFMA: acc += X Y with X, Y in LDS (pitches px, py).
__device__ __forceinline__ f32x4_t mm16_f32(const float* X, int px, const float* Y, int py, f32x4_t acc) {
  const int l = threadIdx.x % kWave;
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4)
    acc = mfma_f32(X[(l & 15) * px + 4 * s4 + (l >> 4)], Y[(4 * s4 + (l >> 4)) * py + (l & 15)], acc);
  return acc;
}

// Store a 16x16 accumulator tile to LDS (pitch p), scaled.
__device__ __forceinline__ void st16(float* M, int p, f32x4_t acc, float scale) {
  const int l = threadIdx.x % kWave;
#pragma unroll
  for (int i = 0; i < 4; ++i) M[(4 * (l >> 4) + i) * p + (l & 15)] = scale * acc[i];
}

// T = (I + A)^-1 for the strictly lower 64x64 A in LDS (pitch kAP), written to
// sT (same pitch; the strictly upper 16x16 blocks are left unwritten).  Blocked:
// the four 16x16 diagonal blocks by forward substitution (one wave each, lane =
// (column, quarter of the rows)), then the off-diagonal blocks level by level,
//   T[b+1][b] = -D[b+1] A[b+1][b] D[b]
//   T[b+2][b] = -D[b+2] (A[b+2][b] D[b] + A[b+2][b+1] T[b+1][b])
//   T[3][0]   = -D[3] (A[3][0] D[0] + A[3][1] T[1][0] + A[3][2] T[2][0])
// on exact-product fp32 MFMA.  Called by all threads of the block.
template <int kAP>
__device__ __forceinline__ void unit_lower_inverse(const float* sA, float* sT, float* sM) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  {
    const int b = wave, c = lane >> 2, part = lane & 3;
    const float* Ab = sA + 16 * b * kAP + 16 * b;
    float tc[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) tc[m] = (4 * m + part == c) ? 1.0f : 0.0f;
#pragma unroll
    for (int r = 1; r < 16; ++r) {
      float acc = 0.0f;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        if (4 * m < r) {
          const float a = Ab[r * kAP + 4 * m + part];
          acc = fmaf(4 * m + part < r ? a : 0.0f, tc[m], acc);
        }
      }
      acc = group_sum<4>(acc);
      if (r > c && (r & 3) == part) tc[r >> 2] = -acc;
    }
    float* Tb = sT + 16 * b * kAP + 16 * b;
#pragma unroll
    for (int m = 0; m < 4; ++m) Tb[(4 * m + part) * kAP + c] = tc[m];
  }
  constexpr int kMP = 17;
  auto blk = [](const float* base, int i, int j) { return base + 16 * i * kAP + 16 * j; };
  const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
  for (int lvl = 1; lvl < 4; ++lvl) {
    __syncthreads();
    const int b = wave;                      // block row b + lvl, column b
    const bool on = b + lvl < 4;
    if (on) {
      f32x4_t m = zero;
      m = mm16_f32(blk(sA, b + lvl, b), kAP, blk(sT, b, b), kAP, m);
      for (int j = b + 1; j < b + lvl; ++j) m = mm16_f32(blk(sA, b + lvl, j), kAP, blk(sT, j, b), kAP, m);
      st16(sM + b * 16 * kMP, kMP, m, 1.0f);
    }
    __syncthreads();
    if (on) {
      f32x4_t t = zero;
      t = mm16_f32(blk(sT, b + lvl, b + lvl), kAP, sM + b * 16 * kMP, kMP, t);
      st16(const_cast<float*>(blk(sT, b + lvl, b)), kAP, t, -1.0f);
    }
  }
  __syncthreads();
}


// Register staging of one chunk's bf16 K, Q, V rows and its vectors, so the
// next chunk's global loads are in flight while the current chunk computes.
// Piece maps: K = 2 x (8 columns of a row pair), consecutive lanes on
// consecutive row pairs; Q = 4 x 16 bytes of a row; V = 16 bytes of a row's
// 32-column tile; one vector element.
struct ChunkStage {
  u32x4_t k0[2], k1[2], q[4], v;
  float vec;
};

__device__ __forceinline__ void stage_issue(ChunkStage& cs, const uint16_t* k, const uint16_t* q,
                                            int64_t qk_stride, const uint16_t* v, int64_t v_stride,
                                            const float* vec, int L) {
  const int tid = threadIdx.x;
  const u32x4_t z = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int p = tid + i * kThreads;
    const int t = 2 * (p % (kC / 2)), j0 = 8 * (p / (kC / 2));
    cs.k0[i] = t < L ? *reinterpret_cast<const u32x4_t*>(k + (int64_t)t * qk_stride + j0) : z;
    cs.k1[i] = t + 1 < L ? *reinterpret_cast<const u32x4_t*>(k + (int64_t)(t + 1) * qk_stride + j0) : z;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = tid + i * kThreads;
    const int t = p / (kD / 8), j0 = 8 * (p % (kD / 8));
    cs.q[i] = t < L ? *reinterpret_cast<const u32x4_t*>(q + (int64_t)t * qk_stride + j0) : z;
  }
  {
    const int t = tid / (kTile / 8), i0 = 8 * (tid % (kTile / 8));
    cs.v = t < L ? *reinterpret_cast<const u32x4_t*>(v + (int64_t)t * v_stride + i0) : z;
  }
  cs.vec = tid < 3 * kC + 1 ? vec[tid] : 0.0f;
}

__device__ __forceinline__ void stage_commit(const ChunkStage& cs, uint16_t* sK, int pitch, uint16_t* sKt,
                                             int tpitch, uint16_t* sQ, float* sV, int vpitch, float* s_vec) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int p = tid + i * kThreads;
    const int t = 2 * (p % (kC / 2)), j0 = 8 * (p / (kC / 2));
    *reinterpret_cast<u32x4_t*>(sK + t * pitch + j0) = cs.k0[i];
    *reinterpret_cast<u32x4_t*>(sK + (t + 1) * pitch + j0) = cs.k1[i];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t a = (cs.k0[i][e / 2] >> (16 * (e % 2))) & 0xffffu;
      const uint32_t b = (cs.k1[i][e / 2] >> (16 * (e % 2))) & 0xffffu;
      *reinterpret_cast<uint32_t*>(sKt + (j0 + e) * tpitch + t) = a | (b << 16);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = tid + i * kThreads;
    const int t = p / (kD / 8), j0 = 8 * (p % (kD / 8));
    *reinterpret_cast<u32x4_t*>(sQ + t * pitch + j0) = cs.q[i];
  }
  {
    const int t = tid / (kTile / 8), i0 = 8 * (tid % (kTile / 8));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sV[t * vpitch + i0 + 2 * e] = __uint_as_float(cs.v[e] << 16);
      sV[t * vpitch + i0 + 2 * e + 1] = __uint_as_float(cs.v[e] & 0xffff0000u);
    }
  }
  if (tid < 3 * kC + 1) s_vec[tid] = cs.vec;
}

// ---------------------------------------------------------------------------
// intra: per (chunk, key head) -> Tt, Pt, vectors for each of its value heads
// ---------------------------------------------------------------------------
template <bool F32, typename Tin>
__global__ __launch_bounds__(kThreads) void chunk_intra_kernel(
    const Tin* __restrict__ q, const Tin* __restrict__ k, int64_t qk_stride,
    const float* __restrict__ g, const float* __restrict__ beta, const int32_t* __restrict__ cu,
    int n_seq, int hk, int hv, float l2_eps, float q_scale, uint8_t* __restrict__ ws) {
  using O = Ops<F32>;
  using E = typename O::E;
  constexpr int kPitch = kD + O::kPadK;
  constexpr int kAP = kC + 1;        // fp32 64x64 scratch pitch
  // K / Q tiles are dead once the Gram tiles are in registers, so the 64x64
  // scratch (A, Pt, T) reuses their LDS.
  constexpr int kKQBytes = 2 * kC * kPitch * (int)sizeof(E);
  constexpr int kScratchBytes = 3 * kC * kAP * (int)sizeof(float);
  __shared__ __attribute__((aligned(16))) uint8_t s_pool[kKQBytes > kScratchBytes ? kKQBytes : kScratchBytes];
  E* sK = reinterpret_cast<E*>(s_pool);
  E* sQ = sK + kC * kPitch;
  float* sA = reinterpret_cast<float*>(s_pool);
  float* sP = sA + kC * kAP;
  float* sT = sP + kC * kAP;
  __shared__ float sM[3 * 16 * 17];
  __shared__ float s_rk[kC], s_rq[kC], s_gam[kC], s_beta[kC];

  const int32_t* first = reinterpret_cast<const int32_t*>(ws);
  const int c = blockIdx.x;
  const int kh = blockIdx.y;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int n = chunk_sequence(first, n_seq, c);
  const int t0 = cu[n] + (c - first[n]) * kC;
  const int L = min(kC, cu[n + 1] - t0);
  const int ratio = hv / hk;

  load_rows<F32>(sK, kPitch, k + (int64_t)t0 * qk_stride + kh * kD, qk_stride, L);
  load_rows<F32>(sQ, kPitch, q + (int64_t)t0 * qk_stride + kh * kD, qk_stride, L);
  __syncthreads();

  // row norms: 4 threads per row, 32 elements each
  {
    const int r = tid / 4, part = tid % 4;
    float sk = 0.f, sq = 0.f;
    for (int e = 0; e < 32; ++e) {
      float kv, qv;
      if constexpr (F32) { kv = sK[r * kPitch + part * 32 + e]; qv = sQ[r * kPitch + part * 32 + e]; }
      else { kv = bf16_bits_to_f32(sK[r * kPitch + part * 32 + e]); qv = bf16_bits_to_f32(sQ[r * kPitch + part * 32 + e]); }
      sk = fmaf(kv, kv, sk);
      sq = fmaf(qv, qv, sq);
    }
    sk = group_sum<4>(sk);
    sq = group_sum<4>(sq);
    if (part == 0) {
      s_rk[r] = r < L ? 1.0f / sqrtf(sk + l2_eps) : 0.0f;
      s_rq[r] = r < L ? q_scale / sqrtf(sq + l2_eps) : 0.0f;
    }
  }

  // G = K K^T and H = Q K^T, lower-triangular tiles of row-tile `wave`
  f32x4_t accG[4], accH[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    accG[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    accH[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  for (int ks = 0; ks < kD; ks += O::kKs) {
    const auto ak = frag<F32>(sK, kPitch, 16 * wave, ks);
    const auto aq = frag<F32>(sQ, kPitch, 16 * wave, ks);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      if (nt <= wave) {
        const auto b = frag<F32>(sK, kPitch, 16 * nt, ks);
        accG[nt] = mma<F32>(ak, b, accG[nt]);
        accH[nt] = mma<F32>(aq, b, accH[nt]);
      }
    }
  }

  for (int hh = 0; hh < ratio; ++hh) {
    const int h = kh * ratio + hh;
    // cumulative log decay within the chunk (padded tokens decay by 1, beta 0)
    if (wave == 0) {
      float gv = lane < L ? g[(int64_t)(t0 + lane) * hv + h] : 0.0f;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const float up = __shfl_up(gv, o, kWave);
        if (lane >= o) gv += up;
      }
      s_gam[lane] = gv;
      s_beta[lane] = lane < L ? beta[(int64_t)(t0 + lane) * hv + h] : 0.0f;
    }
    __syncthreads();

    // A (strictly lower) and Pt (lower incl. diagonal) from the Gram tiles
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      if (nt <= wave) {
        const int j = 16 * nt + (lane & 15);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * wave + 4 * (lane >> 4) + e;
          const float dec = __expf(s_gam[r] - s_gam[j]);
          sA[r * kAP + j] = j < r ? s_beta[r] * dec * s_rk[r] * s_rk[j] * accG[nt][e] : 0.0f;
          sP[r * kAP + j] = j <= r ? s_rq[r] * s_rk[j] * dec * accH[nt][e] : 0.0f;
        }
      }
    }
    __syncthreads();

    // T = (I + A)^-1; Tt = T diag(beta) is formed while writing the fragments
    unit_lower_inverse<kAP>(sA, sT, sM);

    // write Tt and Pt in A-operand lane layout, masked to the lower triangle
    uint8_t* rec = ws + records_offset(n_seq) + ((size_t)c * hv + h) * kRecBytes;
    for (int which = 0; which < 2; ++which) {
      const float* src = which == 0 ? sT : sP;
      const bool scale_cols = which == 0;
      uint8_t* dst = rec + which * kFragBytes;
      if constexpr (F32) {
        // fragment (mt, ks): lane l holds src[16mt + l%16][4ks + l/16]
        for (int p = tid; p < 16 * 4 * kWave; p += kThreads) {
          const int l = p % kWave, f = p / kWave;   // f = mt * 16 + ks
          const int mt = f / 16, ks = f % 16;
          const int r = 16 * mt + (l & 15), kk = 4 * ks + (l >> 4);
          reinterpret_cast<float*>(dst)[p] =
              kk <= r ? src[r * kAP + kk] * (scale_cols ? s_beta[kk] : 1.0f) : 0.0f;
        }
      } else {
        // fragment (mt, ks, term): lane l holds src[16mt + l%16][32ks + 8(l/16) + e]
        for (int p = tid; p < 8 * kWave; p += kThreads) {
          const int l = p % kWave, f = p / kWave;   // f = mt * 2 + ks
          const int mt = f / 2, ks = f % 2;
          const int r = 16 * mt + (l & 15), k0 = 32 * ks + 8 * (l >> 4);
          bf16x8_t hi, lo;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float v = (k0 + e) <= r ? src[r * kAP + k0 + e] * (scale_cols ? s_beta[k0 + e] : 1.0f) : 0.0f;
            __bf16 a, b;
            split_bf16(v, a, b);
            hi[e] = a;
            lo[e] = b;
          }
          *reinterpret_cast<bf16x8_t*>(dst + ((size_t)(f * 2 + 0) * kWave + l) * 16) = hi;
          *reinterpret_cast<bf16x8_t*>(dst + ((size_t)(f * 2 + 1) * kWave + l) * 16) = lo;
        }
      }
    }
    // vectors: a = e^gam rk, b = rq e^gam, c = rk e^{gam_L - gam}, d = e^{gam_L}
    if (tid < kC) {
      float* vec = reinterpret_cast<float*>(rec + 2 * kFragBytes);
      const float gl = s_gam[kC - 1];
      vec[tid] = __expf(s_gam[tid]) * s_rk[tid];
      vec[kC + tid] = s_rq[tid] * __expf(s_gam[tid]);
      vec[2 * kC + tid] = s_rk[tid] * __expf(gl - s_gam[tid]);
      if (tid == 0) vec[3 * kC] = __expf(gl);
    }
    __syncthreads();   // sA, sP, s_gam, s_beta are rewritten for the next value head
  }
}

// ---------------------------------------------------------------------------
// spine: per (sequence, value head, dv tile), sequential over chunks
// ---------------------------------------------------------------------------
template <bool F32, typename Tin, typename To>
__global__ __launch_bounds__(kThreads) void chunk_spine_kernel(
    const Tin* __restrict__ q, const Tin* __restrict__ k, int64_t qk_stride,
    const Tin* __restrict__ v, int64_t v_stride, const float* __restrict__ init_state,
    const int32_t* __restrict__ cu, int n_seq, int hk, int hv, const uint8_t* __restrict__ ws,
    To* __restrict__ out, float* final_state) {
  using O = Ops<F32>;
  using E = typename O::E;
  using F = typename O::F;
  constexpr int kPitch = kD + O::kPadK;          // K, Q rows
  constexpr int kTP = kC + O::kPadK;             // transposed [i][t] tiles
  constexpr int kSP = kD + 4;                    // fp32 state pitch
  constexpr int kVP = kTile + 1;                 // fp32 V tile pitch
  __shared__ __attribute__((aligned(16))) E sK[kC * kPitch];
  __shared__ __attribute__((aligned(16))) E sQ[kC * kPitch];
  __shared__ __attribute__((aligned(16))) E sKt[F32 ? 1 : kD * kTP];
  __shared__ __attribute__((aligned(16))) float sS[kTile * kSP];
  __shared__ float sV[kC * kVP];
  __shared__ __attribute__((aligned(16))) E sRh[kTile * kTP], sRl[F32 ? 1 : kTile * kTP];
  __shared__ __attribute__((aligned(16))) E sNh[kTile * kTP], sNl[F32 ? 1 : kTile * kTP];
  __shared__ __attribute__((aligned(16))) E sWh[kTile * kTP], sWl[F32 ? 1 : kTile * kTP];
  __shared__ float s_vec[3 * kC + 4];

  // Block -> (sequence, key head) group and member (value head of the group,
  // dv tile).  All members of a group share the key head's K/Q tiles, so they
  // are given block ids congruent mod kXcds: they run on one XCD and share its L2.
  const int ratio = hv / hk;
  const int members = ratio * (kD / kTile);
  const int xcd = blockIdx.x % kXcds;
  const int rest = blockIdx.x / kXcds;
  const int grp = (rest / members) * kXcds + xcd;
  if (grp >= n_seq * hk) return;
  const int member = rest % members;
  const int32_t* first = reinterpret_cast<const int32_t*>(ws);
  const int32_t* order = first + n_seq + 1;
  const int n = order[grp / hk];
  const int kh = grp % hk;
  const int h = kh * ratio + member / (kD / kTile);
  const int tile = member % (kD / kTile);
  const int i0 = tile * kTile;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const uint8_t* recs = ws + records_offset(n_seq);
  const int seq_beg = cu[n], seq_end = cu[n + 1];
  const int chunk0 = first[n];

  float* s_out = final_state ? final_state + (((int64_t)n * hv + h) * kD + i0) * kD : nullptr;
  {
    const float* s_in = init_state ? init_state + (((int64_t)n * hv + h) * kD + i0) * kD : nullptr;
    for (int p = tid; p < kTile * kD / 4; p += kThreads) {
      const int i = p / (kD / 4), j = (p % (kD / 4)) * 4;
      f32x4_t val = {0.f, 0.f, 0.f, 0.f};
      if (s_in) val = *reinterpret_cast<const f32x4_t*>(s_in + i * kD + j);
      *reinterpret_cast<f32x4_t*>(sS + i * kSP + j) = val;
    }
  }

  // product roles: waves 0,1 own Y / R / Vnew for dv sub-tile (wave & 1);
  // waves 2,3 own Z / O for the same sub-tiles; all four share the state update.
  const int sub = wave & 1;
  const bool y_role = wave < 2;

  // bf16 inputs: chunk c+1's K / Q / V / vectors are loaded into registers
  // while chunk c computes (ChunkStage); fp32 inputs stage synchronously.
  [[maybe_unused]] ChunkStage stage;
  auto chunk_ptrs = [&](int t0c, int cidx, const Tin*& kp, const Tin*& qp, const Tin*& vp, const float*& vecp) {
    kp = k + (int64_t)t0c * qk_stride + kh * kD;
    qp = q + (int64_t)t0c * qk_stride + kh * kD;
    vp = v + (int64_t)t0c * v_stride + h * kD + i0;
    vecp = reinterpret_cast<const float*>(recs + ((size_t)cidx * hv + h) * kRecBytes + 2 * kFragBytes);
  };
  if constexpr (!F32) {
    if (seq_beg < seq_end) {
      const Tin *kp, *qp, *vp;
      const float* vecp;
      chunk_ptrs(seq_beg, chunk0, kp, qp, vp, vecp);
      stage_issue(stage, kp, qp, qk_stride, vp, v_stride, vecp, min(kC, seq_end - seq_beg));
    }
  }
  for (int t0 = seq_beg, c = chunk0; t0 < seq_end; t0 += kC, ++c) {
    const int L = min(kC, seq_end - t0);
    const uint8_t* rec = recs + ((size_t)c * hv + h) * kRecBytes;
    // this wave's triangular operand (Tt for waves 0,1, Pt for waves 2,3):
    // issued first, in flight while K / Q / V are committed and product 1 runs
    F fh[Tri<F32>::kSlots], fl[Tri<F32>::kSlots];
    load_tri_frags<F32>(rec + (y_role ? 0 : kFragBytes), lane, fh, fl);
    __syncthreads();   // previous chunk finished with sK / sQ / sV / tiles
    if constexpr (F32) {
      load_rows<F32>(sK, kPitch, k + (int64_t)t0 * qk_stride + kh * kD, qk_stride, L);
      load_rows<F32>(sQ, kPitch, q + (int64_t)t0 * qk_stride + kh * kD, qk_stride, L);
      load_values(sV, kVP, v + (int64_t)t0 * v_stride + h * kD + i0, v_stride, L);
      if (tid < 3 * kC + 1) s_vec[tid] = reinterpret_cast<const float*>(rec + 2 * kFragBytes)[tid];
    } else {
      stage_commit(stage, sK, kPitch, sKt, kTP, sQ, sV, kVP, s_vec);
      if (t0 + kC < seq_end) {
        const Tin *kp, *qp, *vp;
        const float* vecp;
        chunk_ptrs(t0 + kC, c + 1, kp, qp, vp, vecp);
        stage_issue(stage, kp, qp, qk_stride, vp, v_stride, vecp, min(kC, seq_end - t0 - kC));
      }
    }
    __syncthreads();

    // ---- Y = K S0^T (waves 0,1) and Z = Q S0^T (waves 2,3): 64 x 16 each ----
    f32x4_t acc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    {
      const E* a_src = y_role ? sK : sQ;
      for (int ks = 0; ks < kD; ks += O::kKs) {
        F bh, bl;
        frag_split_f32<F32>(sS, kSP, 16 * sub, ks, bh, bl);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const F a = frag<F32>(a_src, kPitch, 16 * mt, ks);
          acc[mt] = mma<F32>(a, bh, acc[mt]);
          if constexpr (!F32) acc[mt] = mma<F32>(a, bl, acc[mt]);
        }
      }
    }
    if (y_role) {
      // R = V - a_t Y, stored transposed [i][t] as hi/lo
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        f32x4_t rv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 16 * mt + 4 * (lane >> 4) + e;
          rv[e] = sV[t * kVP + 16 * sub + (lane & 15)] - s_vec[t] * acc[mt][e];
        }
        store_acc_transposed<F32>(sRh, sRl, kTP, 16 * sub, 16 * mt, rv);
      }
    }
    __syncthreads();

    // ---- Vnew = Tt R (waves 0,1) ----
    if (y_role) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        f32x4_t vn = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks * O::kKs <= 16 * mt + 15; ++ks) {
          const int sl = Tri<F32>::slot(mt, ks);
          const F bh = frag<F32>(sRh, kTP, 16 * sub, ks * O::kKs);
          vn = mma<F32>(fh[sl], bh, vn);
          if constexpr (!F32) {
            const F bl = frag<F32>(sRl, kTP, 16 * sub, ks * O::kKs);
            vn = mma<F32>(fh[sl], bl, vn);
            vn = mma<F32>(fl[sl], bh, vn);
          }
        }
        store_acc_transposed<F32>(sNh, sNl, kTP, 16 * sub, 16 * mt, vn);
        f32x4_t w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = s_vec[2 * kC + 16 * mt + 4 * (lane >> 4) + e] * vn[e];
        store_acc_transposed<F32>(sWh, sWl, kTP, 16 * sub, 16 * mt, w);
      }
    }
    __syncthreads();

    // ---- O = b_t Z + Pt Vnew (waves 2,3) ----
    if (!y_role) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[mt][e] *= s_vec[kC + 16 * mt + 4 * (lane >> 4) + e];
#pragma unroll
        for (int ks = 0; ks * O::kKs <= 16 * mt + 15; ++ks) {
          const int sl = Tri<F32>::slot(mt, ks);
          const F bh = frag<F32>(sNh, kTP, 16 * sub, ks * O::kKs);
          acc[mt] = mma<F32>(fh[sl], bh, acc[mt]);
          if constexpr (!F32) {
            const F bl = frag<F32>(sNl, kTP, 16 * sub, ks * O::kKs);
            acc[mt] = mma<F32>(fh[sl], bl, acc[mt]);
            acc[mt] = mma<F32>(fl[sl], bh, acc[mt]);
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 16 * mt + 4 * (lane >> 4) + e;
          if (t < L) st(out + ((int64_t)(t0 + t) * hv + h) * kD + i0 + 16 * sub + (lane & 15), acc[mt][e]);
        }
      }
    }

    // ---- S <- d S + W^T K, W = c_t Vnew  (all waves: rows 16*sub.., 4 column tiles) ----
    {
      const float d = s_vec[3 * kC];
      const int nj0 = (wave >> 1) * 4;
      f32x4_t sacc[4];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int j = 16 * (nj0 + q4) + (lane & 15);
#pragma unroll
        for (int e = 0; e < 4; ++e) sacc[q4][e] = d * sS[(16 * sub + 4 * (lane >> 4) + e) * kSP + j];
      }
      for (int ks = 0; ks < kC; ks += O::kKs) {
        const F ah = frag<F32>(sWh, kTP, 16 * sub, ks);
        F al;
        if constexpr (!F32) al = frag<F32>(sWl, kTP, 16 * sub, ks);
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          F b;
          if constexpr (F32) b = sK[(ks + (lane >> 4)) * kPitch + 16 * (nj0 + q4) + (lane & 15)];
          else b = frag<F32>(sKt, kTP, 16 * (nj0 + q4), ks);
          sacc[q4] = mma<F32>(ah, b, sacc[q4]);
          if constexpr (!F32) sacc[q4] = mma<F32>(al, b, sacc[q4]);
        }
      }
      __syncthreads();   // all reads of the old state (Y/Z and the d*S term) are done
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int j = 16 * (nj0 + q4) + (lane & 15);
#pragma unroll
        for (int e = 0; e < 4; ++e) sS[(16 * sub + 4 * (lane >> 4) + e) * kSP + j] = sacc[q4][e];
      }
    }
  }
  __syncthreads();
  if (s_out) {
    for (int p = tid; p < kTile * kD / 4; p += kThreads) {
      const int i = p / (kD / 4), j = (p % (kD / 4)) * 4;
      *reinterpret_cast<f32x4_t*>(s_out + i * kD + j) = *reinterpret_cast<const f32x4_t*>(sS + i * kSP + j);
    }
  }
}

template <bool F32, typename Tin, typename To>
hipError_t chunk_impl(const Dims& d, const void* q, const void* k, int64_t qk_stride, const void* v,
                      int64_t v_stride, const float* g, const float* beta, const float* init_state,
                      const int32_t* cu_dev, int n, int total_chunks, void* out,
                      float* final_state, void* ws, hipStream_t s) {
  uint8_t* w = static_cast<uint8_t*>(ws);
  hipLaunchKernelGGL(chunk_plan_kernel, dim3(1), dim3(kThreads), 0, s, cu_dev, n,
                     reinterpret_cast<int32_t*>(w), reinterpret_cast<int32_t*>(w) + n + 1);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (total_chunks > 0) {
    hipLaunchKernelGGL((chunk_intra_kernel<F32, Tin>), dim3(total_chunks, d.hk), dim3(kThreads), 0, s,
                       static_cast<const Tin*>(q), static_cast<const Tin*>(k), qk_stride, g, beta,
                       cu_dev, n, d.hk, d.hv, d.l2_eps, d.q_scale, w);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int groups = n * d.hk;
  const int members = (d.hv / d.hk) * (kD / kTile);
  const int blocks = (groups + kXcds - 1) / kXcds * kXcds * members;
  hipLaunchKernelGGL((chunk_spine_kernel<F32, Tin, To>), dim3(blocks), dim3(kThreads), 0, s,
                     static_cast<const Tin*>(q), static_cast<const Tin*>(k), qk_stride,
                     static_cast<const Tin*>(v), v_stride, init_state, cu_dev, n, d.hk, d.hv, w,
                     static_cast<To*>(out), final_state);
  return hipGetLastError();
}

}  // namespace

size_t chunk_workspace_bytes(const Dims& d, int n, int t) {
  const size_t max_chunks = (size_t)t / kC + (size_t)n;
  return records_offset(n) + max_chunks * d.hv * kRecBytes;
}

hipError_t launch_chunk_prefill(const Dims& d, bool in_bf16, bool out_bf16, const void* q,
                                const void* k, int64_t qk_stride, const void* v,
                                int64_t v_stride, const float* g, const float* beta,
                                const float* init_state, const int32_t* cu_dev,
                                const int32_t* cu_host, int n, int t, void* out,
                                float* final_state, void* ws, size_t ws_bytes, hipStream_t s) {
  (void)t;
  (void)ws_bytes;
  if (n == 0) return hipSuccess;
  int total = 0;
  for (int i = 0; i < n; ++i) total += (cu_host[i + 1] - cu_host[i] + kC - 1) / kC;
  if (in_bf16)
    return out_bf16 ? chunk_impl<false, uint16_t, uint16_t>(d, q, k, qk_stride, v, v_stride, g, beta, init_state, cu_dev, n, total, out, final_state, ws, s)
                    : chunk_impl<false, uint16_t, float>(d, q, k, qk_stride, v, v_stride, g, beta, init_state, cu_dev, n, total, out, final_state, ws, s);
  return out_bf16 ? chunk_impl<true, float, uint16_t>(d, q, k, qk_stride, v, v_stride, g, beta, init_state, cu_dev, n, total, out, final_state, ws, s)
                  : chunk_impl<true, float, float>(d, q, k, qk_stride, v, v_stride, g, beta, init_state, cu_dev, n, total, out, final_state, ws, s);
}

}  // namespace gdn
