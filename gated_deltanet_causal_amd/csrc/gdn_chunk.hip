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
//          inverse, Tt and Pt (per-key-channel decay: one workgroup per (chunk,
//          value head), decayed Gram tiles).  Tt and Pt are written to the
//          workspace already in the MFMA A-operand lane layout: fp16 for the
//          register-resident spines (bf16 inputs), fp32 for the LDS spine.
//   spine  walks a sequence's chunks in order with the fp32 state in MFMA
//          accumulators, running the products above on MFMA: register-
//          resident (bf16 inputs, 16 value rows per wave, every product
//          chained through registers) or through LDS (fp32 inputs).
// Numerics.  The Gram products K K^T and Q K^T take the raw bf16 rows exactly.
// bf16 inputs with scalar decay (the register-resident spines): every operand
// of the state and output products -- khat = rk K and qtil = rq Q (formed once
// per chunk and key head by the intra kernel), the chunk-start state, R,
// Vnew, Tt, Pt -- is rounded once to fp16 (2^-11 relative) and multiplied on
// fp16 MFMA with fp32 accumulation; the state itself stays fp32 in the
// accumulators.  A numpy model of these rounding points put the error at
// 6-9e-4 max-relative over 1-4k tokens (with and without decay), inside the
// 2e-3 bound; operands must stay within fp16 range (|x| < 65504), which holds
// for normalised rows, decay factors <= 1 and values and states of the
// activations' scale.  Per-key-channel decay multiplies Kt = khat e^{gam_t},
// Qt = qtil e^{gam_t} and Kb = khat e^{gam_L - gam_t} instead (fp16, factors
// <= 1), formed by its intra kernel, whose decayed Gram tiles split every
// fp32 operand into hi + lo bf16 (hi*hi + hi*lo + lo*hi, ~2^-16 relative).
// The fp32 input path uses fp32 MFMA throughout.
#include <algorithm>
#include <type_traits>
#include <utility>

#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

constexpr int kC = 64;           // chunk
constexpr int kD = 128;          // head dim (k and v)
constexpr int kTile = 32;        // dv rows per spine workgroup
constexpr int kThreads = 256;
constexpr int kIntraMinWaves = 4;   // intra: waves per SIMD the register budget must allow (bf16: 128 VGPRs)
constexpr size_t kFragBytes = 16384;           // one 64x64 operand in lane layout
constexpr size_t kRecBytes = 2 * kFragBytes + 1024;  // Tt, Pt, vectors
// Records of the register-resident spines (bf16 inputs, scalar decay): the six
// Tt fragments that are not all zero, then the six of Pt, each one fp16 operand
// of 16 x 32 in lane layout (1 KB), then the chunk vectors.  The normalised key
// and query rows these spines multiply follow the records in the workspace.
constexpr size_t kHFrag = 1024;
constexpr size_t kHRecP = 6 * kHFrag;
constexpr size_t kHRecVec = 12 * kHFrag;
constexpr size_t kHRecBytes = kHRecVec + 1024;
// Tt / Pt fragments (mt, ks) with ks <= mt / 2 (the rest of the 64 x 64 is zero)
constexpr int kNF = 6;
__host__ __device__ constexpr int frag_mt(int x) { return x < 4 ? x : x - 2; }     // 0 1 2 3 2 3
__host__ __device__ constexpr int frag_ks(int x) { return x < 4 ? 0 : 1; }         // 0 0 0 0 1 1
constexpr int kSortMax = 4096;                 // longest-first order up to this many sequences
constexpr int kXcds = 8;                       // XCDs; workgroups are dealt to them round-robin
// Spine kernels (the sequential walk over a sequence's chunks)
constexpr int kSpineLds = 0;    // 8 waves per 32 value rows, intermediates through LDS (fp32, per key channel)
constexpr int kSpineWave = 1;   // register-resident, a value head per workgroup
constexpr int kSpineRows = 2;   // register-resident, 32 value rows per workgroup
constexpr int kRowsNW = 2;        // kSpineRows: compute waves (16 value rows each)
constexpr int kRowsLoaders = 4;   // kSpineRows: loader waves staging the next chunk
constexpr int kWaveSpineMinBlocks = 256;   // value heads x sequences from which kSpineWave is used

__host__ __device__ constexpr size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Workspace: first[N+1] | order[N] | per-(chunk, value head) records; for the
// register-resident spines the normalised rows khat [T][Hk][dk] and qtil
// [T][Hk][dk] (fp16) follow their records.  Records are laid out for the upper
// bound T / 64 + N of a batch's chunks.
__host__ __device__ inline size_t records_offset(int n_seq) {
  return align_up(sizeof(int32_t) * (2 * (size_t)n_seq + 1), 256);
}
inline size_t hat_offset(int n_seq, int t, int hv) {
  return align_up(records_offset(n_seq) + ((size_t)t / kC + (size_t)n_seq) * hv * kHRecBytes, 256);
}

template <bool F32> struct Ops;
template <> struct Ops<false> {
  using E = uint16_t;            // storage element in LDS (bf16 bits)
  using F = bf16x8_t;            // MFMA operand fragment
  static constexpr int kEpl = 8, kKs = 32;
  // row padding (elements) of k-contiguous LDS tiles: 32 bytes, so that the
  // 16-byte fragment reads of 16 rows (128 or 256 bytes per row) hit distinct
  // banks; a 16-byte pad makes those reads two-way bank conflicted
  static constexpr int kPadK = 16;
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
    for (int e = 0; e < 2; ++e) split2(v[2 * e], v[2 * e + 1], h2[e], l2[e]);
    *reinterpret_cast<uint2*>(hi + off) = make_uint2(h2[0], h2[1]);
    *reinterpret_cast<uint2*>(lo + off) = make_uint2(l2[0], l2[1]);
  }
}

// The plan's outputs.  A single sequence needs no plan: its chunks start at 0
// and it is the whole order, so the plan kernel is not launched for it and
// its workspace entries are never read.
__device__ __forceinline__ int plan_first(const int32_t* first, int n_seq, int n) {
  return n_seq == 1 ? 0 : first[n];
}
__device__ __forceinline__ int plan_order(const int32_t* order, int n_seq, int i) {
  return n_seq == 1 ? 0 : order[i];
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

// Paired-tile k order.  The 32 k slots of a bf16 MFMA are (g, e): lane group
// g = l/16 and operand element e < 8.  Slot (g, e) of k step ks stands for
// index 32 ks + 16 (e/4) + 4 g + e%4, which is exactly where two vertically
// adjacent 16x16 accumulator tiles (rows 32 ks .. +15 and +16 .. +31) keep
// their rows in lane l (rows 4g .. 4g+3 of each).  A pair of accumulator tiles
// is therefore a B operand as it stands, and an A operand only needs its
// columns in the same order.
__host__ __device__ constexpr int pair_k(int ks, int g, int e) {
  return 32 * ks + 16 * (e >> 2) + 4 * g + (e & 3);
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
    // A's row r, columns 4m + part (independent of the recurrence): the first
    // eight rows up front, each later one eight rows ahead of its use, which
    // keeps the bf16 intra kernel within its 128 registers without spilling
    float ar[16][4];
    auto read_row = [&](int r) {
#pragma unroll
      for (int m = 0; m < 4; ++m) ar[r][m] = (4 * m < r && 4 * m + part < r) ? Ab[r * kAP + 4 * m + part] : 0.0f;
    };
#pragma unroll
    for (int r = 1; r < 9; ++r) read_row(r);
#pragma unroll
    for (int r = 1; r < 16; ++r) {
      if (r + 8 < 16) read_row(r + 8);
      float acc = 0.0f;
#pragma unroll
      for (int m = 0; m < 4; ++m)
        if (4 * m < r) acc = fmaf(ar[r][m], tc[m], acc);
      acc = quad_sum(acc);
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



// Shared tail of the intra kernels: T = (I + A)^-1 from sA, then Tt = T diag(beta)
// and (kWithP) Pt (sP) written to the record in MFMA A-operand lane layout, masked
// to the lower triangle: hi/lo bf16 fragment pairs (bf16 inputs) or fp32, in the
// plain k order (element e of lane l in k step ks holds column 32 ks + 8 (l/16) + e);
// kPairK writes the register-resident spines' records instead: single fp16
// fragments in the paired-tile k order (column pair_k(ks, l/16, e)).  All threads.
template <bool F32, int kAP, bool kPairK = false, bool kWithP = true>
__device__ __forceinline__ void write_operands(const float* sA, const float* sP, float* sT, float* sM,
                                               const float* s_beta, uint8_t* rec) {
  const int tid = threadIdx.x;
  unit_lower_inverse<kAP>(sA, sT, sM);
  for (int which = 0; which < (kWithP ? 2 : 1); ++which) {
    const float* src = which == 0 ? sT : sP;
    const bool scale_cols = which == 0;
    uint8_t* dst = rec + which * kFragBytes;
    if constexpr (F32) {
      // fragment (mt, ks): lane l holds src[16mt + l%16][4ks + l/16]
      for (int p = tid; p < 16 * 4 * kWave; p += kThreads) {
        const int l = p % kWave, f = p / kWave;   // f = mt * 16 + ks
        const int mt = f / 16, ks = f % 16;
        const int r = 16 * mt + (l & 15), kk = 4 * ks + (l >> 4);
        reinterpret_cast<float*>(dst)[p] = kk <= r ? src[r * kAP + kk] * (scale_cols ? s_beta[kk] : 1.0f) : 0.0f;
      }
    } else if constexpr (kPairK) {
      // the register-resident spines' records: the six fragments (mt, ks) that are
      // not all zero, compact index x = mt + 2 ks, each a single fp16 operand in the
      // paired-tile k order: lane l holds src[16mt + l%16][pair_k(ks, l/16, e)]
#pragma unroll 1
      for (int p = tid; p < kNF * kWave; p += kThreads) {
        const int l = p % kWave, x = p / kWave;
        const int mt = frag_mt(x), ks = frag_ks(x);
        const int r = 16 * mt + (l & 15);
        uint32_t hp[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const int k0 = pair_k(ks, l >> 4, e), k1 = pair_k(ks, l >> 4, e + 1);
          const float v0 = src[r * kAP + k0] * (scale_cols ? s_beta[k0] : 1.0f);
          const float v1 = src[r * kAP + k1] * (scale_cols ? s_beta[k1] : 1.0f);
          hp[e / 2] = pack_f16x2(k0 <= r ? v0 : 0.0f, k1 <= r ? v1 : 0.0f);
        }
        *reinterpret_cast<u32x4_t*>(rec + which * kHRecP + (size_t)p * 16) = u32x4_t{hp[0], hp[1], hp[2], hp[3]};
      }
    } else {
      // fragment (mt, ks, term): lane l holds src[16mt + l%16][32ks + 8(l/16) + e], as
      // hi/lo bf16; entries above the diagonal are zero.
      // All loads are issued unconditionally (the upper part of sT is never
      // written; the select drops those values).
#pragma unroll 1
      for (int it = 0; it < 8 * kWave / kThreads; ++it) {
        const int p = tid + it * kThreads;
        const int l = p % kWave, f = p / kWave;   // f = mt * 2 + ks
        const int mt = f / 2, ks = f % 2;
        // fragments (0, 1) and (1, 1) lie above the diagonal: all zero, never read
        if (ks == 1 && mt < 2) continue;   // uniform per wave
        const int r = 16 * mt + (l & 15);
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int kk = 32 * ks + 8 * (l >> 4) + e;
          v[e] = src[r * kAP + kk] * (scale_cols ? s_beta[kk] : 1.0f);
        }
        uint32_t hp[4], lp[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const int k0 = 32 * ks + 8 * (l >> 4) + e;
          split2(k0 <= r ? v[e] : 0.0f, k0 + 1 <= r ? v[e + 1] : 0.0f, hp[e / 2], lp[e / 2]);
        }
        *reinterpret_cast<u32x4_t*>(dst + ((size_t)(f * 2 + 0) * kWave + l) * 16) = u32x4_t{hp[0], hp[1], hp[2], hp[3]};
        *reinterpret_cast<u32x4_t*>(dst + ((size_t)(f * 2 + 1) * kWave + l) * 16) = u32x4_t{lp[0], lp[1], lp[2], lp[3]};
      }
    }
  }
}

// Operand fragment of X[row][c] = raw[row][c] * rs[row] * exp(sgn * (gam[row][c] - ref[c]))
// (ref = 0 when null), rows row0.., columns k0.. in the operand lane layout, split into
// hi/lo bf16 (fp32: hi only).  raw k-contiguous (pitch), gam (gpitch) fp32, or fp64 on
// the fp32 path, where the difference is then formed without cancellation.
template <bool F32, typename GT = float>
__device__ __forceinline__ void decayed_frag(const typename Ops<F32>::E* raw, int pitch, const GT* gam,
                                             int gpitch, const GT* ref, const float* rs, int row0, int k0,
                                             float sgn, typename Ops<F32>::F& hi, typename Ops<F32>::F& lo) {
  const int l = threadIdx.x % kWave;
  const int r = row0 + (l & 15);
  const int c0 = k0 + Ops<F32>::kEpl * (l >> 4);
  const float s = rs[r];
  if constexpr (F32) {
    const float e = (float)(gam[r * gpitch + c0] - (ref ? ref[c0] : GT(0)));
    hi = raw[r * pitch + c0] * s * __expf(sgn * e);
    lo = 0.0f;
  } else {
    static_assert(sizeof(GT) == sizeof(float), "bf16 operands take fp32 log decays");
    const u32x4_t u = *reinterpret_cast<const u32x4_t*>(raw + r * pitch + c0);
    const f32x4_t g0 = *reinterpret_cast<const f32x4_t*>(gam + r * gpitch + c0);
    const f32x4_t g1 = *reinterpret_cast<const f32x4_t*>(gam + r * gpitch + c0 + 4);
    f32x4_t f0 = {0.f, 0.f, 0.f, 0.f}, f1 = {0.f, 0.f, 0.f, 0.f};
    if (ref) {
      f0 = *reinterpret_cast<const f32x4_t*>(ref + c0);
      f1 = *reinterpret_cast<const f32x4_t*>(ref + c0 + 4);
    }
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float kv = (e & 1) ? __uint_as_float(u[e / 2] & 0xffff0000u) : __uint_as_float(u[e / 2] << 16);
      const float ge = e < 4 ? g0[e] - f0[e] : g1[e - 4] - f1[e - 4];
      x[e] = kv * s * __expf(sgn * ge);
    }
    uint32_t hp[4], lp[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) split2(x[2 * e], x[2 * e + 1], hp[e], lp[e]);
    hi = __builtin_bit_cast(bf16x8_t, u32x4_t{hp[0], hp[1], hp[2], hp[3]});
    lo = __builtin_bit_cast(bf16x8_t, u32x4_t{lp[0], lp[1], lp[2], lp[3]});
  }
}

// The same operand for bf16 inputs as one fp16 fragment, for tiles whose
// factors are all e^{<= 0} (|x| <= |raw| rs, inside fp16 range).
__device__ __forceinline__ f16x8_t decayed_frag_h(const uint16_t* raw, int pitch, const float* gam, int gpitch,
                                                 const float* ref, const float* rs, int row0, int k0, float sgn) {
  const int l = threadIdx.x % kWave;
  const int r = row0 + (l & 15);
  const int c0 = k0 + 8 * (l >> 4);
  const float s = rs[r];
  const u32x4_t u = *reinterpret_cast<const u32x4_t*>(raw + r * pitch + c0);
  const f32x4_t g0 = *reinterpret_cast<const f32x4_t*>(gam + r * gpitch + c0);
  const f32x4_t g1 = *reinterpret_cast<const f32x4_t*>(gam + r * gpitch + c0 + 4);
  const f32x4_t f0 = *reinterpret_cast<const f32x4_t*>(ref + c0);
  const f32x4_t f1 = *reinterpret_cast<const f32x4_t*>(ref + c0 + 4);
  uint32_t hp[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float ga = e < 2 ? g0[2 * e] - f0[2 * e] : g1[2 * e - 4] - f1[2 * e - 4];
    const float gb = e < 2 ? g0[2 * e + 1] - f0[2 * e + 1] : g1[2 * e - 3] - f1[2 * e - 3];
    hp[e] = pack_f16x2(__uint_as_float(u[e] << 16) * s * __expf(sgn * ga),
                       __uint_as_float(u[e] & 0xffff0000u) * s * __expf(sgn * gb));
  }
  return as_f16x8(u32x4_t{hp[0], hp[1], hp[2], hp[3]});
}

// product with both operands split: hi*hi + hi*lo + lo*hi (fp32: one exact product)
template <bool F32>
__device__ __forceinline__ f32x4_t mma3(typename Ops<F32>::F ah, typename Ops<F32>::F al,
                                        typename Ops<F32>::F bh, typename Ops<F32>::F bl, f32x4_t c) {
  c = mma<F32>(ah, bh, c);
  if constexpr (!F32) {
    c = mma<F32>(ah, bl, c);
    c = mma<F32>(al, bh, c);
  }
  return c;
}

// ---------------------------------------------------------------------------
// intra, per-key-channel decay: per (chunk, value head).  With gam[r][c] the
// within-chunk cumulative log decay of channel c (non-increasing in r, since
// g <= 0), each 16x16 tile (row tile i, column tile n <= i) of
//   A[r][j]  = beta_r sum_c (khat_r[c] e^{gam_r[c]-gam_b[c]}) (khat_j[c] e^{gam_b[c]-gam_j[c]})   j < r
//   Pt[r][j] =        sum_c (qtil_r[c] e^{gam_r[c]-gam_b[c]}) (khat_j[c] e^{gam_b[c]-gam_j[c]})   j <= r
// is one MFMA product over channels with its own reference token b:
//   n < i  b = 16 i, the first row of the later tile: r >= b > j, so both
//          factors are e^{<= 0} for any decay (underflow only where the exact
//          product is below the smallest normal);
//   n = i  b = 16 i + 8: a factor is e^{+-(at most 8 tokens of log decay)}.
//          Where some channel of the tile decays by more than kDiagLim over
//          those 8 tokens (|g| > ~10 per token sustained), the tile is
//          instead summed element by element with e^{gam_r - gam_j} <= 1.
// The operands are formed in registers from raw K / Q and gam: for bf16 inputs
// single fp16 fragments left of the diagonal (every factor e^{<= 0}) and hi/lo
// bf16 pairs on the diagonal (factors up to e^{kDiagLim}, beyond fp16 range);
// fp32 fragments on the fp32 path.
// bf16 inputs: the kernel also writes what the register-resident spine
// multiplies, each rounded once to fp16 (every factor e^{<= 0}):
//   Kt[t] = khat_t e^{gam_t},  Qt[t] = qtil_t e^{gam_t},  Kb[t] = khat_t e^{gam_L - gam_t}
// ([T][Hv][dk] each, Qt and Kb after Kt), its records (Tt, Pt as fp16
// fragments) and d = e^{gam_L} per channel; the fp32 path keeps the LDS spine.
// ---------------------------------------------------------------------------
constexpr float kDiagLim = 80.0f;   // largest exponent of a diagonal-tile factor (e^80 ~ 5.5e34)
template <bool F32, typename Tin>
__global__ __launch_bounds__(kThreads) void chunk_intra_pc_kernel(
    const Tin* __restrict__ q, const Tin* __restrict__ k, int64_t qk_stride,
    const float* __restrict__ g, const float* __restrict__ beta, const int32_t* __restrict__ cu,
    int n_seq, int hk, int hv, int l2norm, float l2_eps, float q_scale, uint8_t* __restrict__ ws,
    uint16_t* __restrict__ kpc) {
  using O = Ops<F32>;
  using E = typename O::E;
  using F = typename O::F;
  constexpr int kPitch = kD + O::kPadK;
  // cumulative log decays: fp32, or fp64 on the fp32 path (a difference of two
  // sums taken after a strong decay would otherwise lose ~|gam| 2^-24 absolute)
  using GT = std::conditional_t<F32, double, float>;
  constexpr int kGP = kD + 4;        // gam pitch (elements)
  constexpr int kAP = kC + 1;
  constexpr int kPhase1 = 2 * kC * kPitch * (int)sizeof(E) + kC * kGP * (int)sizeof(GT);
  constexpr int kScratchBytes = 3 * kC * kAP * (int)sizeof(float);
  __shared__ __attribute__((aligned(16))) uint8_t s_pool[kPhase1 > kScratchBytes ? kPhase1 : kScratchBytes];
  E* sK = reinterpret_cast<E*>(s_pool);
  E* sQ = sK + kC * kPitch;
  GT* sGam = reinterpret_cast<GT*>(s_pool + 2 * kC * kPitch * sizeof(E));
  float* sA = reinterpret_cast<float*>(s_pool);
  float* sP = sA + kC * kAP;
  float* sT = sP + kC * kAP;
  __shared__ float sM[3 * 16 * 17];
  __shared__ float s_rk[kC], s_rq[kC], s_beta[kC];
  __shared__ GT s_tot[kD];
  __shared__ float s_dl[F32 ? 1 : kD];   // e^{gam_L} per channel (bf16 inputs)

  const int32_t* first = reinterpret_cast<const int32_t*>(ws);
  const int c = blockIdx.x;
  const int h = blockIdx.y;
  const int kh = h / (hv / hk);
  const int tid = threadIdx.x, wave = tid / kWave;
  const int n = chunk_sequence(first, n_seq, c);
  const int t0 = cu[n] + (c - plan_first(first, n_seq, n)) * kC;
  const int L = min(kC, cu[n + 1] - t0);

  // K, Q and g rows: every load issued before the first LDS store (a load, wait,
  // store loop puts one memory round trip per piece on the workgroup's path);
  // rows past L are read at row L - 1 and stored as zero
  {
    constexpr int kPer = 16 / sizeof(Tin);
    constexpr int kIt = kC * kD / kPer / kThreads;
    constexpr int kItG = kC * kD / 4 / kThreads;
    u32x4_t rk_[kIt], rq_[kIt];
    f32x4_t rg_[kItG];
    const Tin* kb = k + (int64_t)t0 * qk_stride + kh * kD;
    const Tin* qb = q + (int64_t)t0 * qk_stride + kh * kD;
    const float* gb = g + ((int64_t)t0 * hv + h) * kD;
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
      const int p = tid + it * kThreads, r = p / (kD / kPer), c = (p % (kD / kPer)) * kPer;
      const int rr = min(r, L - 1);
      rk_[it] = *reinterpret_cast<const u32x4_t*>(kb + (int64_t)rr * qk_stride + c);
      rq_[it] = *reinterpret_cast<const u32x4_t*>(qb + (int64_t)rr * qk_stride + c);
    }
#pragma unroll
    for (int it = 0; it < kItG; ++it) {
      const int p = tid + it * kThreads, r = p / (kD / 4), c4 = 4 * (p % (kD / 4));
      rg_[it] = *reinterpret_cast<const f32x4_t*>(gb + (int64_t)min(r, L - 1) * hv * kD + c4);
    }
    const float bv = tid < L ? beta[(int64_t)(t0 + tid) * hv + h] : 0.0f;
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
      const int p = tid + it * kThreads, r = p / (kD / kPer), c = (p % (kD / kPer)) * kPer;
      const u32x4_t z = {0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4_t*>(sK + r * kPitch + c) = r < L ? rk_[it] : z;
      *reinterpret_cast<u32x4_t*>(sQ + r * kPitch + c) = r < L ? rq_[it] : z;
    }
#pragma unroll
    for (int it = 0; it < kItG; ++it) {
      const int p = tid + it * kThreads, r = p / (kD / 4), c4 = 4 * (p % (kD / 4));
      const f32x4_t gv = r < L ? rg_[it] : f32x4_t{0.f, 0.f, 0.f, 0.f};
      if constexpr (F32) {
#pragma unroll
        for (int e = 0; e < 4; ++e) sGam[r * kGP + c4 + e] = gv[e];
      } else {
        *reinterpret_cast<f32x4_t*>(sGam + r * kGP + c4) = gv;
      }
    }
    if (tid < kC) s_beta[tid] = bv;
  }
  __syncthreads();

  {  // row norms: 4 threads per row
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
      s_rk[r] = r < L ? (l2norm ? 1.0f / sqrtf(sk + l2_eps) : 1.0f) : 0.0f;
      s_rq[r] = r < L ? (l2norm ? q_scale / sqrtf(sq + l2_eps) : q_scale) : 0.0f;
    }
  }
  {  // per-channel cumulative sum over the chunk: thread (channel, half of the rows)
    const int ch = tid % kD, half = tid / kD;
    GT v[kC / 2];
#pragma unroll
    for (int r = 0; r < kC / 2; ++r) v[r] = sGam[(half * (kC / 2) + r) * kGP + ch];
#pragma unroll
    for (int r = 1; r < kC / 2; ++r) v[r] += v[r - 1];
    if (half == 0) s_tot[ch] = v[kC / 2 - 1];
    __syncthreads();
    const GT off = half ? s_tot[ch] : GT(0);
#pragma unroll
    for (int r = 0; r < kC / 2; ++r) sGam[(half * (kC / 2) + r) * kGP + ch] = v[r] + off;
  }
  __syncthreads();
  if constexpr (!F32) {
    // the register-resident spine's operands Kt, Qt, Kb of rows r < L (rows past
    // the chunk's end belong to the next sequence); gam_L = gam of row 63
    const int64_t plane = (int64_t)cu[n_seq] * hv * kD;   // [T][Hv][dk]
    if (tid < kD) s_dl[tid] = __expf(sGam[(kC - 1) * kGP + tid]);
#pragma unroll
    for (int p = tid; p < kC * kD / 8; p += kThreads) {
      const int r = p / (kD / 8), c8 = 8 * (p % (kD / 8));
      if (r >= L) continue;
      const u32x4_t ku = *reinterpret_cast<const u32x4_t*>(sK + r * kPitch + c8);
      const u32x4_t qu = *reinterpret_cast<const u32x4_t*>(sQ + r * kPitch + c8);
      const f32x4_t ga = *reinterpret_cast<const f32x4_t*>(sGam + r * kGP + c8);
      const f32x4_t gb = *reinterpret_cast<const f32x4_t*>(sGam + r * kGP + c8 + 4);
      const f32x4_t la = *reinterpret_cast<const f32x4_t*>(sGam + (kC - 1) * kGP + c8);
      const f32x4_t lb = *reinterpret_cast<const f32x4_t*>(sGam + (kC - 1) * kGP + c8 + 4);
      const float rk = s_rk[r], rq = s_rq[r];
      u32x4_t kt, qt, kb;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float g0 = w < 2 ? ga[2 * w] : gb[2 * w - 4], g1 = w < 2 ? ga[2 * w + 1] : gb[2 * w - 3];
        const float l0 = w < 2 ? la[2 * w] : lb[2 * w - 4], l1 = w < 2 ? la[2 * w + 1] : lb[2 * w - 3];
        const float e0 = __expf(g0), e1 = __expf(g1);
        const float f0 = __expf(l0 - g0), f1 = __expf(l1 - g1);
        const float k0 = __uint_as_float(ku[w] << 16) * rk, k1 = __uint_as_float(ku[w] & 0xffff0000u) * rk;
        const float q0 = __uint_as_float(qu[w] << 16) * rq, q1 = __uint_as_float(qu[w] & 0xffff0000u) * rq;
        kt[w] = pack_f16x2(k0 * e0, k1 * e1);
        qt[w] = pack_f16x2(q0 * e0, q1 * e1);
        kb[w] = pack_f16x2(k0 * f0, k1 * f1);
      }
      uint16_t* dst = kpc + ((int64_t)(t0 + r) * hv + h) * kD + c8;
      *reinterpret_cast<u32x4_t*>(dst) = kt;
      *reinterpret_cast<u32x4_t*>(dst + plane) = qt;
      *reinterpret_cast<u32x4_t*>(dst + 2 * plane) = kb;
    }
  }
  // references of this wave's row tile (rows past L carry gam_{L-1}: g is zero there)
  const GT* ref_off = sGam + 16 * wave * kGP;
  const GT* ref_dia = sGam + (16 * wave + 8) * kGP;
  // the diagonal tile's factors stay finite when no channel decays by more than
  // kDiagLim between the tile's first row and b or between b and its last row.
  // On the fp32 path the tile is always summed element by element: a factor
  // e^{+x} times one e^{-y} carries ~(x + y) 2^-24 of relative error from the
  // exponent's rounding, above that path's bound for strong decays.
  bool dia_mfma = !F32;
  if constexpr (!F32) {
    const int lane = tid % kWave;
    float worst = 0.0f;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int ch = lane + kWave * h2;
      const float gb = ref_dia[ch];
      worst = fmaxf(worst, fmaxf(fabsf(ref_off[ch] - gb), fabsf(gb - sGam[(16 * wave + 15) * kGP + ch])));
    }
    dia_mfma = !__any(worst > kDiagLim);
  }

  // decayed Gram tiles of row tile `wave`: G~ = Ka Kb^T, H~ = Qa Kb^T
  f32x4_t accG[4], accH[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    accG[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    accH[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  for (int ks = 0; ks < kD; ks += O::kKs) {
    F kah, kal, qah, qal;
    if constexpr (F32) {
      if (wave > 0) {   // row side of the tiles left of the diagonal (reference 16 wave)
        decayed_frag<F32, GT>(sK, kPitch, sGam, kGP, ref_off, s_rk, 16 * wave, ks, 1.0f, kah, kal);
        decayed_frag<F32, GT>(sQ, kPitch, sGam, kGP, ref_off, s_rq, 16 * wave, ks, 1.0f, qah, qal);
      }
#pragma unroll
      for (int nt = 0; nt < 3; ++nt) {
        if (nt < wave) {
          F bh, bl;
          decayed_frag<F32, GT>(sK, kPitch, sGam, kGP, ref_off, s_rk, 16 * nt, ks, -1.0f, bh, bl);
          accG[nt] = mma3<F32>(kah, kal, bh, bl, accG[nt]);
          accH[nt] = mma3<F32>(qah, qal, bh, bl, accH[nt]);
        }
      }
    } else if (wave > 0) {
      // bf16 inputs: the tiles left of the diagonal (every factor e^{<= 0}) on
      // single fp16 operands, as the spine that consumes them rounds Tt and Pt
      const f16x8_t ka = decayed_frag_h(sK, kPitch, sGam, kGP, ref_off, s_rk, 16 * wave, ks, 1.0f);
      const f16x8_t qa = decayed_frag_h(sQ, kPitch, sGam, kGP, ref_off, s_rq, 16 * wave, ks, 1.0f);
#pragma unroll
      for (int nt = 0; nt < 3; ++nt) {
        if (nt < wave) {
          const f16x8_t kb = decayed_frag_h(sK, kPitch, sGam, kGP, ref_off, s_rk, 16 * nt, ks, -1.0f);
          accG[nt] = mfma_f16(ka, kb, accG[nt]);
          accH[nt] = mfma_f16(qa, kb, accH[nt]);
        }
      }
    }
    if (dia_mfma) {   // the diagonal tile (reference 16 wave + 8)
      F bh, bl;
      decayed_frag<F32, GT>(sK, kPitch, sGam, kGP, ref_dia, s_rk, 16 * wave, ks, 1.0f, kah, kal);
      decayed_frag<F32, GT>(sQ, kPitch, sGam, kGP, ref_dia, s_rq, 16 * wave, ks, 1.0f, qah, qal);
      decayed_frag<F32, GT>(sK, kPitch, sGam, kGP, ref_dia, s_rk, 16 * wave, ks, -1.0f, bh, bl);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        if (nt == wave) {
          accG[nt] = mma3<F32>(kah, kal, bh, bl, accG[nt]);
          accH[nt] = mma3<F32>(qah, qal, bh, bl, accH[nt]);
        }
      }
    }
  }
  if (!dia_mfma) {
    // the diagonal tile element by element, e^{gam_r - gam_j} <= 1 per channel:
    // lane (g, m) holds rows 16 wave + 4 g + e, column 16 wave + m (j <= r only)
    const int lane = tid % kWave;
    const int j = 16 * wave + (lane & 15);
    f32x4_t gd = {0.f, 0.f, 0.f, 0.f}, hd = {0.f, 0.f, 0.f, 0.f};
    for (int ch = 0; ch < kD; ++ch) {
      float kj;
      if constexpr (F32) kj = sK[j * kPitch + ch];
      else kj = bf16_bits_to_f32(sK[j * kPitch + ch]);
      const GT gj = sGam[j * kGP + ch];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * wave + 4 * (lane >> 4) + e;
        float kr, qr;
        if constexpr (F32) { kr = sK[r * kPitch + ch]; qr = sQ[r * kPitch + ch]; }
        else { kr = bf16_bits_to_f32(sK[r * kPitch + ch]); qr = bf16_bits_to_f32(sQ[r * kPitch + ch]); }
        const float w = j <= r ? kj * __expf((float)(sGam[r * kGP + ch] - gj)) : 0.0f;
        gd[e] = fmaf(kr, w, gd[e]);
        hd[e] = fmaf(qr, w, hd[e]);
      }
    }
    const float rkj = s_rk[j];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * wave + 4 * (lane >> 4) + e;
      gd[e] *= s_rk[r] * rkj;
      hd[e] *= s_rq[r] * rkj;
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
      if (nt == wave) { accG[nt] = gd; accH[nt] = hd; }
  }
  __syncthreads();   // the pool's K / Q / gam are dead from here on
  {
    const int lane = tid % kWave;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      if (nt <= wave) {
        const int j = 16 * nt + (lane & 15);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * wave + 4 * (lane >> 4) + e;
          sA[r * kAP + j] = j < r ? s_beta[r] * accG[nt][e] : 0.0f;
          sP[r * kAP + j] = j <= r ? accH[nt][e] : 0.0f;
        }
      }
    }
  }
  __syncthreads();
  uint8_t* rec = ws + records_offset(n_seq) + ((size_t)c * hv + h) * (F32 ? kRecBytes : kHRecBytes);
  write_operands<F32, kAP, !F32>(sA, sP, sT, sM, s_beta, rec);
  if constexpr (F32) {
    // vectors for the LDS spine: rk, rq
    if (tid < kC) {
      float* vec = reinterpret_cast<float*>(rec + 2 * kFragBytes);
      vec[tid] = s_rk[tid];
      vec[kC + tid] = s_rq[tid];
    }
  } else {
    // the register-resident spine's decay of the state over the chunk, per channel
    if (tid < kD) reinterpret_cast<float*>(rec + kHRecVec)[tid] = s_dl[tid];
  }
}

// ---------------------------------------------------------------------------
// intra: per (chunk, key head) -> Tt, Pt, vectors for each of its value heads
// ---------------------------------------------------------------------------
template <bool F32, typename Tin, bool kPairK>
__global__ __launch_bounds__(kThreads, F32 ? 2 : kIntraMinWaves) void chunk_intra_kernel(
    const Tin* __restrict__ q, const Tin* __restrict__ k, int64_t qk_stride,
    Gates gates, const int32_t* __restrict__ cu,
    int n_seq, int hk, int hv, int l2norm, float l2_eps, float q_scale, uint8_t* __restrict__ ws,
    uint16_t* __restrict__ khat) {
  using O = Ops<F32>;
  using E = typename O::E;
  constexpr int kPitch = kD + O::kPadK;
  constexpr int kAP = kC + 1;        // fp32 64x64 scratch pitch
  // K / Q tiles are dead once the Gram tiles are in registers, so the 64x64
  // scratch (A, T and, in the plain k order, Pt) reuses their LDS.  In the
  // paired-tile k order Pt goes from the Gram registers straight to the record
  // (below).  The diagonal-block scratch of write_operands sits after A and T in
  // the same pool, so bf16 inputs take 38.4 KB of LDS: with at most 128 VGPRs
  // (kIntraMinWaves) four workgroups share a CU, and a 4096-token sequence's
  // 1024 (chunk, key head) workgroups run in one round instead of 1.33.
  constexpr int kKQBytes = 2 * kC * kPitch * (int)sizeof(E);
  constexpr int kScratchBytes = (kPairK ? 2 : 3) * kC * kAP * (int)sizeof(float);
  __shared__ __attribute__((aligned(16))) uint8_t s_pool[kKQBytes > kScratchBytes ? kKQBytes : kScratchBytes];
  E* sK = reinterpret_cast<E*>(s_pool);
  E* sQ = sK + kC * kPitch;
  float* sA = reinterpret_cast<float*>(s_pool);
  float* sT = sA + kC * kAP;
  float* sP = sT + kC * kAP;   // plain k order only
  // write_operands' 16x16 blocks, after the scratch in the same pool (used only
  // once the K / Q tiles are dead)
  static_assert(kScratchBytes + 3 * 16 * 17 * (int)sizeof(float) <= (kKQBytes > kScratchBytes ? kKQBytes : kScratchBytes),
                "the pool holds the scratch and the blocks");
  float* sM = reinterpret_cast<float*>(s_pool + kScratchBytes);
  __shared__ __attribute__((aligned(16))) float s_rk[kC], s_rq[kC];
  // cumulative log decay per value head (double-buffered): fp64 on the fp32 path,
  // whose factors e^{gam_r - gam_j} would otherwise lose ~|gam| 2^-24 to cancellation
  using GT = std::conditional_t<F32, double, float>;
  __shared__ __attribute__((aligned(16))) GT s_gam[2][kC];
  __shared__ __attribute__((aligned(16))) float s_beta[2][kC];

  const int32_t* first = reinterpret_cast<const int32_t*>(ws);
  const int c = blockIdx.x;
  const int kh = blockIdx.y;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int n = chunk_sequence(first, n_seq, c);
  const int t0 = cu[n] + (c - plan_first(first, n_seq, n)) * kC;
  const int L = min(kC, cu[n + 1] - t0);
  const int ratio = hv / hk;

  // cumulative log decay and beta of value head kh * ratio + hh (padded tokens
  // decay by 1 and have beta 0), by wave 0: lane = token.  The gates are given,
  // or derived here from the a / b projections.
  auto gb_load = [&](int hh, float& gv, float& bv) {
    const int h = kh * ratio + hh;
    gv = bv = 0.0f;
    if (lane < L) gate_pair<Tin>(gates, t0 + lane, hv, h, gv, bv);
  };
  auto gb_store = [&](int buf, float gv_in, float bv) {
    GT gv = gv_in;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const GT up = __shfl_up(gv, o, kWave);
      if (lane >= o) gv += up;
    }
    s_gam[buf][lane] = gv;
    s_beta[buf][lane] = bv;
  };
  float gv_next = 0.f, bv_next = 0.f;
  if (wave == 0) gb_load(0, gv_next, bv_next);

  // K and Q rows: all loads issued before the first store (rows past L read as zero)
  {
    constexpr int kPer = 16 / sizeof(Tin);
    constexpr int kIt = kC * kD / kPer / kThreads;
    u32x4_t rk_[kIt], rq_[kIt];
    const Tin* kb = k + (int64_t)t0 * qk_stride + kh * kD;
    const Tin* qb = q + (int64_t)t0 * qk_stride + kh * kD;
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
      const int p = tid + it * kThreads, r = p / (kD / kPer), c = (p % (kD / kPer)) * kPer;
      const int rr = min(r, L - 1);
      rk_[it] = *reinterpret_cast<const u32x4_t*>(kb + (int64_t)rr * qk_stride + c);
      rq_[it] = *reinterpret_cast<const u32x4_t*>(qb + (int64_t)rr * qk_stride + c);
    }
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
      const int p = tid + it * kThreads, r = p / (kD / kPer), c = (p % (kD / kPer)) * kPer;
      const u32x4_t z = {0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4_t*>(sK + r * kPitch + c) = r < L ? rk_[it] : z;
      *reinterpret_cast<u32x4_t*>(sQ + r * kPitch + c) = r < L ? rq_[it] : z;
    }
  }
  if (wave == 0) gb_store(0, gv_next, bv_next);
  __syncthreads();

  // row norms: 4 threads per row, 32 elements each (16-byte reads)
  {
    const int r = tid / 4, part = tid % 4;
    float sk = 0.f, sq = 0.f;
#pragma unroll
    for (int e4 = 0; e4 < 32; e4 += 16 / (int)sizeof(E)) {
      const u32x4_t ku = *reinterpret_cast<const u32x4_t*>(sK + r * kPitch + part * 32 + e4);
      const u32x4_t qu = *reinterpret_cast<const u32x4_t*>(sQ + r * kPitch + part * 32 + e4);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        if constexpr (F32) {
          sk = fmaf(__uint_as_float(ku[w]), __uint_as_float(ku[w]), sk);
          sq = fmaf(__uint_as_float(qu[w]), __uint_as_float(qu[w]), sq);
        } else {
          const float k0 = __uint_as_float(ku[w] << 16), k1 = __uint_as_float(ku[w] & 0xffff0000u);
          const float q0 = __uint_as_float(qu[w] << 16), q1 = __uint_as_float(qu[w] & 0xffff0000u);
          sk = fmaf(k0, k0, fmaf(k1, k1, sk));
          sq = fmaf(q0, q0, fmaf(q1, q1, sq));
        }
      }
    }
    sk = quad_sum(sk);
    sq = quad_sum(sq);
    const float rkv = l2norm ? 1.0f / sqrtf(sk + l2_eps) : 1.0f;
    const float rqv = l2norm ? q_scale / sqrtf(sq + l2_eps) : q_scale;
    if (part == 0) {
      s_rk[r] = r < L ? rkv : 0.0f;
      s_rq[r] = r < L ? rqv : 0.0f;
    }
    if constexpr (kPairK) {
      // the rows the register-resident spines multiply, normalised and rounded
      // once to fp16: khat = rk k and qtil = rq q (q_scale included), the
      // lane's 32 columns of its row (rows past the chunk's end belong to the
      // next sequence and are not written)
      if (r < L) {
        // qtil [T][Hk][dk] follows khat (cu[n_seq] = T)
        uint16_t* qhat = khat + (int64_t)cu[n_seq] * hk * kD;
        const int64_t off = ((int64_t)(t0 + r) * hk + kh) * kD + part * 32;
#pragma unroll
        for (int e8 = 0; e8 < 32; e8 += 8) {
          const u32x4_t ku = *reinterpret_cast<const u32x4_t*>(sK + r * kPitch + part * 32 + e8);
          const u32x4_t qu = *reinterpret_cast<const u32x4_t*>(sQ + r * kPitch + part * 32 + e8);
          u32x4_t kh16, qh16;
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            kh16[w] = pack_f16x2(__uint_as_float(ku[w] << 16) * rkv, __uint_as_float(ku[w] & 0xffff0000u) * rkv);
            qh16[w] = pack_f16x2(__uint_as_float(qu[w] << 16) * rqv, __uint_as_float(qu[w] & 0xffff0000u) * rqv);
          }
          *reinterpret_cast<u32x4_t*>(khat + off + e8) = kh16;
          *reinterpret_cast<u32x4_t*>(qhat + off + e8) = qh16;
        }
      }
    }
  }

  // G = K K^T (tiles (wave, nt), nt <= wave) and H = Q K^T: in the paired-tile
  // k order H is formed transposed, tiles (nt, wave) of H^T = K Q^T, whose
  // accumulators pairs are Pt's operand fragments as they stand
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
        if constexpr (kPairK) accH[nt] = mma<F32>(b, aq, accH[nt]);
        else accH[nt] = mma<F32>(aq, b, accH[nt]);
      }
    }
  }

  __syncthreads();   // every wave's Gram tiles are in registers: the K / Q LDS becomes scratch

  for (int hh = 0; hh < ratio; ++hh) {
    const int h = kh * ratio + hh;
    const int buf = hh & 1;
    if (wave == 0 && hh + 1 < ratio) gb_load(hh + 1, gv_next, bv_next);   // lands during this head
    const GT* gam = s_gam[buf];
    const float* bet = s_beta[buf];

    uint8_t* rec = ws + records_offset(n_seq) + ((size_t)c * hv + h) * (kPairK ? kHRecBytes : kRecBytes);
    // A (strictly lower) and Pt (lower incl. diagonal) from the Gram tiles
    {
      const int r0 = 16 * wave + 4 * (lane >> 4);
      GT gr[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) gr[e] = gam[r0 + e];
      const f32x4_t br = *reinterpret_cast<const f32x4_t*>(bet + r0);
      const f32x4_t rkr = *reinterpret_cast<const f32x4_t*>(s_rk + r0);
      const f32x4_t rqr = *reinterpret_cast<const f32x4_t*>(s_rq + r0);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        if (nt <= wave) {
          const int j = 16 * nt + (lane & 15);
          const GT gj = gam[j];
          const float rkj = s_rk[j];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = r0 + e;
            const float dec = __expf((float)(gr[e] - gj));
            const float a = br[e] * dec * rkr[e] * rkj * accG[nt][e];
            sA[r * kAP + j] = j < r ? a : 0.0f;
            if constexpr (!kPairK) {
              const float pv = rqr[e] * rkj * dec * accH[nt][e];
              sP[r * kAP + j] = j <= r ? pv : 0.0f;
            }
          }
        }
      }
    }
    if constexpr (kPairK) {
      // Pt fragments (mt = wave, ks) straight from the H^T tiles (2 ks, wave) and
      // (2 ks + 1, wave): lane l holds Pt[r][j], r = 16 wave + l%16,
      // j = 16 nt + 4 (l/16) + e (the record's paired-tile k order)
      static_assert(!kPairK || !F32, "the paired-tile order is the bf16 records'");
      const int r = 16 * wave + (lane & 15);
      const float gr = gam[r], rqr = s_rq[r];
      f32x4_t pv[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        pv[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if (nt <= wave) {
          const int j0 = 16 * nt + 4 * (lane >> 4);
          const f32x4_t gj = *reinterpret_cast<const f32x4_t*>(gam + j0);
          const f32x4_t rkj = *reinterpret_cast<const f32x4_t*>(s_rk + j0);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            pv[nt][e] = j0 + e <= r ? rqr * rkj[e] * __expf(gr - gj[e]) * accH[nt][e] : 0.0f;
        }
      }
      // single fp16 fragments, compact index x = wave + 2 ks; (mt, ks) = (0, 1) and
      // (1, 1) lie above the diagonal and are not written
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        if (ks == 1 && wave < 2) continue;   // uniform per wave
        const u32x4_t hp = {pack_f16x2(pv[2 * ks][0], pv[2 * ks][1]), pack_f16x2(pv[2 * ks][2], pv[2 * ks][3]),
                            pack_f16x2(pv[2 * ks + 1][0], pv[2 * ks + 1][1]),
                            pack_f16x2(pv[2 * ks + 1][2], pv[2 * ks + 1][3])};
        *reinterpret_cast<u32x4_t*>(rec + kHRecP + (size_t)(wave + 2 * ks) * kHFrag + 16 * lane) = hp;
      }
    }
    __syncthreads();

    // T = (I + A)^-1; Tt = T diag(beta) is formed while writing the fragments
    write_operands<F32, kAP, kPairK, !kPairK>(sA, sP, sT, sM, bet, rec);

    // vectors: a = e^gam rk, b = rq e^gam, c = rk e^{gam_L - gam}, d = e^{gam_L};
    // the register-resident spines multiply khat and qtil, which carry rk and rq
    if (tid < kC) {
      float* vec = reinterpret_cast<float*>(rec + (kPairK ? kHRecVec : 2 * kFragBytes));
      const GT gl = gam[kC - 1];
      const float rk = kPairK ? 1.0f : s_rk[tid], rq = kPairK ? 1.0f : s_rq[tid];
      vec[tid] = __expf((float)gam[tid]) * rk;
      vec[kC + tid] = rq * __expf((float)gam[tid]);
      vec[2 * kC + tid] = rk * __expf((float)(gl - gam[tid]));
      if (tid == 0) vec[3 * kC] = __expf((float)gl);
    }
    if (wave == 0 && hh + 1 < ratio) gb_store(buf ^ 1, gv_next, bv_next);
    __syncthreads();   // sA, sP and this head's decay buffer are rewritten next
  }
}

// ---------------------------------------------------------------------------
// spine: per (sequence, value head, dv tile), sequential over chunks
// ---------------------------------------------------------------------------
constexpr int kSpineThreads = 512;   // 8 waves, two per SIMD

// Register staging of one chunk's inputs: K and Q rows, the V tile, the chunk
// vectors (per-key-channel decay: rk, rq and the chunk's log decays g).  Issued
// while the previous chunk computes, committed to LDS at the top of the chunk.
// The Tt / Pt fragments do not pass through here: each wave loads its own row
// tile of them straight into registers.
template <bool F32, bool kPC> struct Stage {
  u32x4_t k[F32 ? 4 : 2], q[F32 ? 4 : 2], v;
  float vec, gv[kPC && F32 ? 16 : 1];
};

// Loads are issued in parts (kParts: bit 0 K and Q, bit 1 V and the vectors,
// bit 2 the per-key-channel log decays), at different points of the chunk:
// the texture units take in about 64 bytes per clock per CU, and a wave
// stalls at a load while they are full.
template <int kParts, bool F32, bool kPC, typename Tin>
__device__ __forceinline__ void stage_issue(Stage<F32, kPC>& sg, const Tin* k, const Tin* q, int64_t qk_stride,
                                            const Tin* v, int64_t v_stride, const float* g, int hv,
                                            const uint8_t* rec, int L) {
  const int tid = threadIdx.x;
  const u32x4_t z = {0u, 0u, 0u, 0u};
  auto row16 = [&](const Tin* base, int64_t stride, int t, int col) -> u32x4_t {
    return t < L ? *reinterpret_cast<const u32x4_t*>(base + (int64_t)t * stride + col) : z;
  };
  if constexpr ((kParts & 1) && F32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = tid + i * kSpineThreads;            // 64 rows x 32 pieces of 4 floats
      sg.k[i] = row16(k, qk_stride, p / 32, 4 * (p % 32));
      sg.q[i] = row16(q, qk_stride, p / 32, 4 * (p % 32));
    }
  } else if constexpr (kParts & 1) {
    const int t = 2 * (tid % (kC / 2)), j0 = 8 * (tid / (kC / 2));   // row pair x 8 columns
    sg.k[0] = row16(k, qk_stride, t, j0);
    sg.k[1] = row16(k, qk_stride, t + 1, j0);
    if constexpr (kPC) {
      sg.q[0] = row16(q, qk_stride, t, j0);
      sg.q[1] = row16(q, qk_stride, t + 1, j0);
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int p = tid + i * kSpineThreads;            // 64 rows x 16 pieces of 8
        sg.q[i] = row16(q, qk_stride, p / 16, 8 * (p % 16));
      }
    }
  }
  if constexpr (kParts & 2) {
    if constexpr (F32) sg.v = row16(v, v_stride, tid / 8, 4 * (tid % 8));  // 64 rows x 8 pieces
    else sg.v = tid < kC * 4 ? row16(v, v_stride, tid / 4, 8 * (tid % 4)) : z;
    if constexpr (kPC) sg.vec = tid < 2 * kC ? reinterpret_cast<const float*>(rec + 2 * kFragBytes)[tid] : 0.0f;
    else sg.vec = tid < 3 * kC + 1 ? reinterpret_cast<const float*>(rec + 2 * kFragBytes)[tid] : 0.0f;
  }
  if constexpr ((kParts & 4) && kPC) {
    // channel tid/4, rows 16 (tid%4) .. +15 of the chunk
    const int ch = tid / 4, r0 = 16 * (tid % 4);
#pragma unroll
    for (int r = 0; r < 16; ++r) sg.gv[r] = r0 + r < L ? g[((int64_t)(r0 + r) * hv) * kD + ch] : 0.0f;
  }
}

template <bool F32, bool kPC>
__device__ __forceinline__ void stage_commit(const Stage<F32, kPC>& sg, typename Ops<F32>::E* sK,
                                             typename Ops<F32>::E* sKt, typename Ops<F32>::E* sQ, int pitch,
                                             int tpitch, float* sV, int vpitch, float* sGam,
                                             int gpitch, float* s_vec, float2* sGLP = nullptr) {
  const int tid = threadIdx.x;
  if constexpr (F32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = tid + i * kSpineThreads;
      *reinterpret_cast<u32x4_t*>(sK + (p / 32) * pitch + 4 * (p % 32)) = sg.k[i];
      *reinterpret_cast<u32x4_t*>(sQ + (p / 32) * pitch + 4 * (p % 32)) = sg.q[i];
    }
    const int t = tid / 8, i0 = 4 * (tid % 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) sV[t * vpitch + i0 + e] = __uint_as_float(sg.v[e]);
  } else {
    {
      const int t = 2 * (tid % (kC / 2)), j0 = 8 * (tid / (kC / 2));
      *reinterpret_cast<u32x4_t*>(sK + t * pitch + j0) = sg.k[0];
      *reinterpret_cast<u32x4_t*>(sK + (t + 1) * pitch + j0) = sg.k[1];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // columns j0+2e (low halves) and j0+2e+1 (high halves) of rows t, t+1
        *reinterpret_cast<uint32_t*>(sKt + (j0 + 2 * e) * tpitch + t) =
            __builtin_amdgcn_perm(sg.k[1][e], sg.k[0][e], 0x05040100u);
        *reinterpret_cast<uint32_t*>(sKt + (j0 + 2 * e + 1) * tpitch + t) =
            __builtin_amdgcn_perm(sg.k[1][e], sg.k[0][e], 0x07060302u);
      }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int p = tid + i * kSpineThreads;
      *reinterpret_cast<u32x4_t*>(sQ + (p / 16) * pitch + 8 * (p % 16)) = sg.q[i];
    }
    if (tid < kC * 4) {
      const int t = tid / 4, i0 = 8 * (tid % 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sV[t * vpitch + i0 + 2 * e] = __uint_as_float(sg.v[e] << 16);
        sV[t * vpitch + i0 + 2 * e + 1] = __uint_as_float(sg.v[e] & 0xffff0000u);
      }
    }
  }
  if constexpr (kPC) {
    // cumulative log decay per channel.  The products need both gam_t (Y, Z)
    // and gam_L - gam_t (the update), and one of the two is a difference of
    // large sums after a strong decay.  Both are therefore summed directly,
    // each over terms of one sign (the part totals come by shuffle, so nothing
    // is subtracted), and with p_c the number of rows where |gam_t| <= |gam_L| / 2,
    // rows t < p_c keep gam_t and the others gam_L - gam_t: the value not kept
    // is then gam_L minus one of at most half its size, accurate to fp32
    // rounding.
    static_assert(F32, "per-key-channel decay on the LDS spine is the fp32 path");
    const int ch = tid / 4, part = tid % 4;
    float own = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) own += sg.gv[r];
    float excl = 0.0f, later = 0.0f;
#pragma unroll
    for (int o = 0; o < 4; ++o) {
      const float t_o = __shfl(own, o, 4);
      if (o < part) excl += t_o;
      if (o > part) later += t_o;
    }
    const float tot = (excl + own) + later;
    int cnt = 0;
    {
      float run = excl;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        run += sg.gv[r];
        cnt += fabsf(run) <= 0.5f * fabsf(tot);
      }
    }
    cnt += __shfl_xor(cnt, 1, 4);
    cnt += __shfl_xor(cnt, 2, 4);
    {
      float run = excl;   // gam_t of row 16 part + r
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        run += sg.gv[r];
        if (16 * part + r < cnt) sGam[(16 * part + r) * gpitch + ch] = run;
      }
      float suf = later;  // gam_L - gam_t: the log decays after row 16 part + r
#pragma unroll
      for (int r = 15; r >= 0; --r) {
        if (16 * part + r >= cnt) sGam[(16 * part + r) * gpitch + ch] = suf;
        suf += sg.gv[r];
      }
    }
    if (part == 0) sGLP[ch] = make_float2(tot, (float)cnt);
    if (tid < 2 * kC) s_vec[tid] = sg.vec;
  } else {
    if (tid < 3 * kC + 1) s_vec[tid] = sg.vec;
  }
}

template <bool F32, bool kPC, typename Tin, typename To>
__global__ __launch_bounds__(kSpineThreads) void chunk_spine_kernel(
    const Tin* __restrict__ q, const Tin* __restrict__ k, int64_t qk_stride,
    const Tin* __restrict__ v, int64_t v_stride, const float* __restrict__ g,
    const float* __restrict__ init_state, const int32_t* __restrict__ cu, int n_seq, int hk, int hv,
    const uint8_t* __restrict__ ws, To* __restrict__ out, float* final_state) {
  using O = Ops<F32>;
  using E = typename O::E;
  using F = typename O::F;
  // bf16 inputs (scalar or per-key-channel decay) take the register-resident
  // spines; this one serves the fp32 path
  static_assert(F32 || !kPC, "bf16 per-key-channel decay runs on the register-resident spine");
  constexpr int kPad = O::kPadK;
  constexpr int kPitch = kD + kPad;              // K, Q and state rows
  constexpr int kTP = kC + kPad;                 // transposed [i][t] tiles
  constexpr int kVP = kTile + 1;                 // fp32 V tile pitch
  constexpr int kGP = kD + 4;                    // per-channel log decay pitch
  __shared__ __attribute__((aligned(16))) E sK[kC * kPitch];
  __shared__ __attribute__((aligned(16))) E sQ[kC * kPitch];
  __shared__ __attribute__((aligned(16))) E sKt[F32 ? 1 : kD * kTP];
  // The fp32 state tile lives in the waves' MFMA accumulators across chunks;
  // LDS holds it as the B operand of product 1, split into bf16 hi / lo
  // (fp32 on the fp32 path), row-major [i][j].
  __shared__ __attribute__((aligned(16))) E sSh[kTile * kPitch], sSl[F32 ? 1 : kTile * kPitch];
  __shared__ float sV[kC * kVP];
  __shared__ __attribute__((aligned(16))) E sRh[kTile * kTP], sRl[F32 ? 1 : kTile * kTP];
  __shared__ __attribute__((aligned(16))) E sNh[kTile * kTP], sNl[F32 ? 1 : kTile * kTP];
  __shared__ __attribute__((aligned(16))) E sWh[kTile * kTP], sWl[F32 ? 1 : kTile * kTP];
  __shared__ __attribute__((aligned(16))) float sGam[kPC ? kC * kGP : 1];
  // fp32 per-key-channel path: (gam_L, p_c) per channel, p_c the prefix / suffix
  // switch row (sGam holds gam_t for rows t < p_c, gam_L - gam_t from p_c on)
  __shared__ float2 sGLP[kPC && F32 ? kD : 1];
  __shared__ __attribute__((aligned(16))) float s_vec[3 * kC + 4];

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
  const int n = plan_order(order, n_seq, grp / hk);
  const int kh = grp % hk;
  const int h = kh * ratio + member / (kD / kTile);
  const int tile = member % (kD / kTile);
  const int i0 = tile * kTile;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const uint8_t* recs = ws + records_offset(n_seq);
  const int seq_beg = cu[n], seq_end = cu[n + 1];
  const int chunk0 = plan_first(first, n_seq, n);
  auto rec_of = [&](int cidx) { return recs + ((size_t)cidx * hv + h) * kRecBytes; };

  // Roles.  Wave w owns token row tile mt = w % 4 and dv half hf = w / 4 of
  // Y, Z, R, Vnew and O.  For the state update it owns the transposed state
  // tiles S^T[16 nj ..][si ..], nj = 2 (w / 2) + {0, 1}, si = 16 (w % 2): a lane
  // holds S[si + l%16][16 nj + 4 (l/16) .. +3], four consecutive key columns.
  const int mt = wave & 3, hf = wave >> 2;
  const int si = 16 * (wave & 1);
  const int nj0 = 2 * (wave >> 1);
  const int nks = F32 ? 4 * (mt + 1) : 1 + (mt >> 1);   // k steps up to the diagonal
  constexpr int kMaxKs = F32 ? 16 : 2;

  // Each wave keeps its row tile of Tt / Pt in registers, loaded from the
  // record one chunk ahead (right after its use in this chunk), so the record
  // never passes through LDS and its loads drain behind the compute.
  [[maybe_unused]] F th[kMaxKs], tl[kMaxKs], ph[kMaxKs], pl[kMaxKs];
  auto load_row_frags = [&](const uint8_t* src, F* fh, F* fl) {
    // every k step is loaded (those past the diagonal are in the record and
    // unused) so that the count of loads in flight is the same on every wave
    // and the compiler's waits for them stay exact
#pragma unroll
    for (int ks = 0; ks < kMaxKs; ++ks) {
      if constexpr (F32) {
        fh[ks] = reinterpret_cast<const float*>(src)[(mt * 16 + ks) * kWave + lane];
      } else {
        const int f = mt * 2 + ks;
        fh[ks] = *reinterpret_cast<const bf16x8_t*>(src + ((size_t)(f * 2 + 0) * kWave + lane) * 16);
        fl[ks] = *reinterpret_cast<const bf16x8_t*>(src + ((size_t)(f * 2 + 1) * kWave + lane) * 16);
      }
    }
  };
  // fragment of Tt (which = 0) or Pt (1), row tile mt, k step ks
  auto tri_frag = [&](int which, int ks, F& fh, F& fl) {
    fh = which == 0 ? th[ks] : ph[ks];
    if constexpr (F32) fl = 0.0f;
    else fl = which == 0 ? tl[ks] : pl[ks];
  };

  f32x4_t sacc[2];
  auto store_state_lds = [&]() {
#pragma unroll
    for (int q2 = 0; q2 < 2; ++q2) {
      const int off = (si + (lane & 15)) * kPitch + 16 * (nj0 + q2) + 4 * (lane >> 4);
      if constexpr (F32) {
        *reinterpret_cast<f32x4_t*>(sSh + off) = sacc[q2];
      } else {
        uint32_t hp[2], lp[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          __bf16 h0, l0, h1, l1;
          split_bf16(sacc[q2][2 * e], h0, l0);
          split_bf16(sacc[q2][2 * e + 1], h1, l1);
          hp[e] = __builtin_bit_cast(uint16_t, h0) | (uint32_t(__builtin_bit_cast(uint16_t, h1)) << 16);
          lp[e] = __builtin_bit_cast(uint16_t, l0) | (uint32_t(__builtin_bit_cast(uint16_t, l1)) << 16);
        }
        *reinterpret_cast<uint2*>(sSh + off) = make_uint2(hp[0], hp[1]);
        *reinterpret_cast<uint2*>(sSl + off) = make_uint2(lp[0], lp[1]);
      }
    }
  };
  {
    const float* s_in = init_state ? init_state + (((int64_t)n * hv + h) * kD + i0) * kD : nullptr;
#pragma unroll
    for (int q2 = 0; q2 < 2; ++q2) {
      sacc[q2] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if (s_in)
        sacc[q2] = *reinterpret_cast<const f32x4_t*>(s_in + (si + (lane & 15)) * kD + 16 * (nj0 + q2) + 4 * (lane >> 4));
    }
    store_state_lds();
  }

  Stage<F32, kPC> stage;
  auto issue = [&](auto parts, int t0c, int cidx) {
    stage_issue<decltype(parts)::value, F32, kPC>(
        stage, k + (int64_t)t0c * qk_stride + kh * kD, q + (int64_t)t0c * qk_stride + kh * kD, qk_stride,
        v + (int64_t)t0c * v_stride + h * kD + i0, v_stride, kPC ? g + ((int64_t)t0c * hv + h) * kD : nullptr,
        hv, rec_of(cidx), min(kC, seq_end - t0c));
  };
  if (seq_beg < seq_end) {
    issue(std::integral_constant<int, 7>{}, seq_beg, chunk0);
    load_row_frags(rec_of(chunk0), th, tl);
    load_row_frags(rec_of(chunk0) + kFragBytes, ph, pl);
  }

  for (int t0 = seq_beg, c = chunk0; t0 < seq_end; t0 += kC, ++c) {
    const int L = min(kC, seq_end - t0);
    const bool more = t0 + kC < seq_end;
    __syncthreads();   // the previous chunk is done with every LDS tile
    stage_commit<F32, kPC>(stage, sK, sKt, sQ, kPitch, kTP, sV, kVP, sGam, kGP, s_vec, sGLP);
    if (more) issue(std::integral_constant<int, 3>{}, t0 + kC, c + 1);   // K, Q, V, vectors
    __syncthreads();

    // ---- Y = K S0^T and Z = Q S0^T: rows of tile mt, columns of half hf ----
    // (per-key-channel decay: Y = (khat e^gam) S0^T, Z = (qtil e^gam) S0^T)
    f32x4_t accY = {0.f, 0.f, 0.f, 0.f}, accZ = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int ks = 0; ks < kD; ks += O::kKs) {
      const F bh = frag<F32>(sSh, kPitch, 16 * hf, ks);
      F bl{};
      if constexpr (!F32) bl = frag<F32>(sSl, kPitch, 16 * hf, ks);
      if constexpr (kPC) {
        // fp32: A = K rk e^{gam_t}, Q rq e^{gam_t}, gam_t recovered from the split store
        const int r = 16 * mt + (lane & 15), c0 = ks + (lane >> 4);
        const float gv = sGam[r * kGP + c0];
        const float2 lp = sGLP[c0];
        const float ex = __expf((float)r < lp.y ? gv : lp.x - gv);
        accY = mma<F32>(sK[r * kPitch + c0] * s_vec[r] * ex, bh, accY);
        accZ = mma<F32>(sQ[r * kPitch + c0] * s_vec[kC + r] * ex, bh, accZ);
      } else {
        const F ak = frag<F32>(sK, kPitch, 16 * mt, ks);
        const F aq = frag<F32>(sQ, kPitch, 16 * mt, ks);
        accY = mma<F32>(ak, bh, accY);
        accZ = mma<F32>(aq, bh, accZ);
        if constexpr (!F32) {
          accY = mma<F32>(ak, bl, accY);
          accZ = mma<F32>(aq, bl, accZ);
        }
      }
    }
    if constexpr (kPC) {
      if (more) issue(std::integral_constant<int, 4>{}, t0 + kC, c + 1);   // the next chunk's log decays
    }
    // R = V - a_t Y (per-key-channel decay: R = V - Y), stored transposed [i][t] as hi/lo
    {
      f32x4_t rv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * mt + 4 * (lane >> 4) + e;
        rv[e] = sV[t * kVP + 16 * hf + (lane & 15)] - (kPC ? 1.0f : s_vec[t]) * accY[e];
      }
      store_acc_transposed<F32>(sRh, sRl, kTP, 16 * hf, 16 * mt, rv);
    }
    __syncthreads();

    // ---- Vnew = Tt R (row tile mt, half hf); W = c_t Vnew (per-key-channel: W = Vnew) ----
    {
      f32x4_t vn = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < kMaxKs; ++ks) {
        if (ks < nks) {
          F th_, tl_, bl{};
          tri_frag(0, ks, th_, tl_);
          const F bh = frag<F32>(sRh, kTP, 16 * hf, ks * O::kKs);
          if constexpr (!F32) bl = frag<F32>(sRl, kTP, 16 * hf, ks * O::kKs);
          vn = mma3<F32>(th_, tl_, bh, bl, vn);
        }
      }
      store_acc_transposed<F32>(sNh, sNl, kTP, 16 * hf, 16 * mt, vn);
      load_row_frags(rec_of(more ? c + 1 : c), th, tl);   // next chunk's Tt rows (unconditional: exact waits)
      if constexpr (kPC) {
        store_acc_transposed<F32>(sWh, sWl, kTP, 16 * hf, 16 * mt, vn);
      } else {
        f32x4_t w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = s_vec[2 * kC + 16 * mt + 4 * (lane >> 4) + e] * vn[e];
        store_acc_transposed<F32>(sWh, sWl, kTP, 16 * hf, 16 * mt, w);
      }
    }
    __syncthreads();

    // ---- O = b_t Z + Pt Vnew (row tile mt, half hf) ----
    {
      if constexpr (!kPC) {
#pragma unroll
        for (int e = 0; e < 4; ++e) accZ[e] *= s_vec[kC + 16 * mt + 4 * (lane >> 4) + e];
      }
#pragma unroll
      for (int ks = 0; ks < kMaxKs; ++ks) {
        if (ks < nks) {
          F ph_, pl_, bl{};
          tri_frag(1, ks, ph_, pl_);
          const F bh = frag<F32>(sNh, kTP, 16 * hf, ks * O::kKs);
          if constexpr (!F32) bl = frag<F32>(sNl, kTP, 16 * hf, ks * O::kKs);
          accZ = mma3<F32>(ph_, pl_, bh, bl, accZ);
        }
      }
      load_row_frags(rec_of(more ? c + 1 : c) + kFragBytes, ph, pl);   // next chunk's Pt rows
      To* orow = out + ((int64_t)t0 * hv + h) * kD + i0 + 16 * hf + (lane & 15);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * mt + 4 * (lane >> 4) + e;
        if (t < L) st(orow + (int64_t)t * hv * kD, accZ[e]);
      }
    }

    // ---- S^T <- d S^T + K^T W on this wave's two tiles, then its LDS copy ----
    // (per-key-channel decay: column j decays by e^{gam_L[j]} and the key rows
    //  enter as khat_t e^{gam_L - gam_t})
    {
      if constexpr (kPC) {
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
          for (int e = 0; e < 4; ++e) sacc[q2][e] *= __expf(sGLP[16 * (nj0 + q2) + 4 * (lane >> 4) + e].x);
      } else {
        const float d = s_vec[3 * kC];
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
          for (int e = 0; e < 4; ++e) sacc[q2][e] *= d;
      }
#pragma unroll 2
      for (int ks = 0; ks < kC; ks += O::kKs) {
        const F bh = frag<F32>(sWh, kTP, si, ks);
        F bl{};
        if constexpr (!F32) bl = frag<F32>(sWl, kTP, si, ks);
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2) {
          const int j = 16 * (nj0 + q2) + (lane & 15);
          if constexpr (kPC) {
            // A[j][t] = K[t][j] rk[t] e^{gam_L[j] - gam_t[j]}, t = ks + l/16 (fp32: the
            // suffix gam_L - gam_t from the split store)
            static_assert(F32, "the bf16 per-channel update reads the committed K^T operand");
            F ah, al;
            const int tb = ks + (lane >> 4);
            const float gv = sGam[tb * kGP + j];
            const float2 lp = sGLP[j];
            ah = sK[tb * kPitch + j] * s_vec[tb] * __expf((float)tb < lp.y ? lp.x - gv : gv);
            al = 0.0f;
            sacc[q2] = mma3<F32>(ah, al, bh, bl, sacc[q2]);
          } else {
            F a;
            if constexpr (F32) a = sK[(ks + (lane >> 4)) * kPitch + j];
            else a = frag<F32>(sKt, kTP, 16 * (nj0 + q2), ks);
            sacc[q2] = mma<F32>(a, bh, sacc[q2]);
            if constexpr (!F32) sacc[q2] = mma<F32>(a, bl, sacc[q2]);
          }
        }
      }
      // every wave's product 1 read the old copy before the Vnew barrier
      store_state_lds();
    }
  }
  if (final_state) {
    float* s_out = final_state + (((int64_t)n * hv + h) * kD + i0) * kD;
#pragma unroll
    for (int q2 = 0; q2 < 2; ++q2)
      *reinterpret_cast<f32x4_t*>(s_out + (si + (lane & 15)) * kD + 16 * (nj0 + q2) + 4 * (lane >> 4)) = sacc[q2];
  }
}

// ---------------------------------------------------------------------------
// spine, register-resident form (bf16 inputs, scalar decay).
//
// One wave owns 16 value rows i of a head's state, for all 128 key columns and
// all 64 tokens of a chunk, so every product of the chunk step is wave-local
// (khat = rk K, qtil = rq Q, the normalised fp16 rows the intra kernel wrote):
//   Y, Z   = khat S0^T, qtil S0^T    (A: khat / qtil rows from LDS, B: the state)
//   R      = V - a Y
//   Vnew   = Tt R                     (A: Tt from the record, B: R)
//   O      = b Z + Pt Vnew            (A: Pt, B: Vnew)
//   S^T   <- d S^T + khat^T (c Vnew)  (A: khat^T by transposing LDS reads, B: c Vnew)
// with a = b = e^gam, c = e^{gam_L - gam}, d = e^{gam_L}.  The state is held as
// eight 16x16 fp32 accumulator tiles of S^T (key rows j, value columns i).  In
// the paired-tile k order every B operand above is a pair of accumulator tiles
// of the previous product, rounded to fp16 in registers: nothing but the
// chunk's shared inputs passes through LDS.  khat and qtil are stored in LDS
// with each 32-column block in paired-tile order, so an A fragment is one
// 16-byte read.  A workgroup is kNW waves (16 kNW value rows of one head)
// sharing the chunk's khat, qtil, V, vectors and the record's Tt / Pt
// fragments, double-buffered in LDS and staged through registers one chunk
// ahead; each wave reads the Tt / Pt fragments from LDS as A operands.  One
// barrier per chunk.
// ---------------------------------------------------------------------------
constexpr int kWP = kD + 16;   // khat / qtil row pitch in LDS (fp16 elements): 288 bytes

// LDS column of logical column j of a K / Q row (paired-tile order per 32 columns)
__device__ __forceinline__ int wave_col(int j) {
  return (j & ~31) + 8 * ((j >> 2) & 3) + 4 * ((j >> 4) & 1) + (j & 3);
}

// two accumulator tiles -> one fp16 operand in paired-tile k order
__device__ __forceinline__ f16x8_t f16_pair(const f32x4_t& a, const f32x4_t& b) {
  return as_f16x8(u32x4_t{pack_f16x2(a[0], a[1]), pack_f16x2(a[2], a[3]), pack_f16x2(b[0], b[1]),
                          pack_f16x2(b[2], b[3])});
}

// 4 bf16 of a transposing LDS read: within each 16-lane group, lane 4r + q
// supplies the address of row r, columns 4q .. 4q+3 of a 4 x 16 block, and
// lane j receives column j, rows 0..3.
typedef short v4s_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ v4s_t lds_read_tr4(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s_t*)(p));
}
__device__ __forceinline__ bf16x8_t lds_read_tr8(const uint16_t* p, int second) {
  const v4s_t a = lds_read_tr4(p), b = lds_read_tr4(p + second);
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Raw buffer access: a descriptor with a uniform base and a byte range, and
// 32-bit per-lane offsets.  Loads past the range return zero and stores past
// it are dropped, which is how the spine handles a chunk's rows past the end
// of its sequence.  Offsets that the range check must see are always in the
// per-lane offset (the scalar offset is used only for accesses known to be in
// range).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4_t buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

__device__ __forceinline__ void buf_store4(__amdgpu_buffer_rsrc_t r, uint32_t voff, f32x4_t v, float*) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, voff, 0, 0);
}
__device__ __forceinline__ void buf_store4(__amdgpu_buffer_rsrc_t r, uint32_t voff, f32x4_t v, _Float16*) {
  typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
  __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3])}, r, voff, 0, 0);
}
__device__ __forceinline__ void buf_store4(__amdgpu_buffer_rsrc_t r, uint32_t voff, f32x4_t v, uint16_t*) {
  const uint32_t lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{v[0], v[1]}, bf16x2_t));
  const uint32_t hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{v[2], v[3]}, bf16x2_t));
  typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
  __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{lo, hi}, r, voff, 0, 0);
}

// Workgroup shape of the register-resident spines: kThreadsT threads sharing
// one chunk's inputs for kRowsT value rows of one head; kPCT: per-key-channel
// decay, whose state update multiplies a third row tile (Kb) instead of khat.
template <int kThreadsT, int kRowsT, bool kPCT = false>
struct SpineCfg {
  static constexpr int kThreadsW = kThreadsT;
  static constexpr int kRows = kRowsT;                    // value rows per workgroup
  static constexpr int kVP = kRows + 8;                   // V row pitch (bf16)
  static constexpr int kTiles = kPCT ? 3 : 2;             // fp16 row tiles of 64 x 128
  // one LDS slot (bytes): khat | qtil [| Kb] | V (fp16 tiles, bf16 V) | Tt, Pt fragments | chunk vectors
  // (per-key-channel decay: Kt | Qt | Kb)
  static constexpr int kOffQ = kC * kWP * 2;
  static constexpr int kOffKb = 2 * kOffQ;
  static constexpr int kOffV = kTiles * kOffQ;
  static constexpr int kOffTri = kOffV + kC * kVP * 2;
  static constexpr int kTriFrags = 2 * kNF;               // (Tt, Pt) x 6 fp16 fragments, 1 KB each
  static constexpr int kOffVec = kOffTri + kTriFrags * (int)kHFrag;
  static constexpr int kSlotBytes = kOffVec + 1024;
  static constexpr int kPiecesKQ = kC * kD / 8 / kThreadsW;    // 16-byte pieces of khat (and qtil) per thread
  static constexpr int kPiecesV = kC * kRows / 8 / kThreadsW;  // ... of V
  // ... of the fragments: the last round may cover only some of the waves
  static constexpr int kPiecesTri = (kTriFrags * kWave + kThreadsW - 1) / kThreadsW;
  static constexpr int kLoads = kTiles * kPiecesKQ + kPiecesV + kPiecesTri + 1;   // + the vectors
  static_assert(kPiecesKQ * kThreadsW == kC * kD / 8 && kPiecesV * kThreadsW == kC * kRows / 8 &&
                kThreadsW % kWave == 0, "pieces must divide evenly over the threads");
};

// One chunk's inputs (khat and qtil rows, the workgroup's V columns, the Tt / Pt
// fragments and the chunk vectors of its record) staged through registers into
// an LDS slot, one 16-byte piece per call so the loads and the LDS writes can
// be spread between MFMAs.  Per chunk a buffer descriptor covers its rows:
// rows past the end of the sequence load as zeros, and a chunk past the end of
// the sequence has an empty range (no access at all).
template <typename Cf>
struct ChunkStage {
  static constexpr int kKQ = Cf::kPiecesKQ, kT3 = Cf::kTiles * kKQ;   // pieces of the row tiles
  u32x4_t k[kKQ], q[kKQ], kb[Cf::kTiles == 3 ? kKQ : 1], v[Cf::kPiecesV], tri[Cf::kPiecesTri], vec;
  struct Rsrc { __amdgpu_buffer_rsrc_t k, q, kb, v, r; };
  const uint16_t *kp, *qp, *kbp, *vp;   // row tiles' head / value head / value row base of row 0
  int64_t qk_stride, v_stride;
  const uint8_t* rec0;               // the sequence's first record of this value head
  size_t rec_step;                   // bytes between the records of consecutive chunks
  int seq_beg, seq_end, n_chunks, tid;
  uint32_t qk_row, v_row, off_kq, off_v;

  __device__ void init() {
    qk_row = (uint32_t)qk_stride * 2;
    v_row = (uint32_t)v_stride * 2;
    off_kq = (uint32_t)(tid >> 4) * qk_row + 16 * (tid & 15);
    off_v = (uint32_t)(tid / (Cf::kRows / 8)) * v_row + 16 * (tid % (Cf::kRows / 8));
  }
  __device__ Rsrc rsrc(int cl) const {   // local chunk index cl (may be past the end)
    const int t0 = seq_beg + cl * kC;
    const bool in = cl < n_chunks;
    const uint32_t L = in ? (uint32_t)min(kC, seq_end - t0) : 0u;
    Rsrc r;
    r.k = make_rsrc(kp + (int64_t)t0 * qk_stride, L * qk_row);
    r.q = make_rsrc(qp + (int64_t)t0 * qk_stride, L * qk_row);
    r.kb = make_rsrc(kbp + (int64_t)t0 * qk_stride, L * qk_row);
    r.v = make_rsrc(vp + (int64_t)t0 * v_stride, L * v_row);
    r.r = make_rsrc(rec0 + (in ? cl : 0) * rec_step, in ? (uint32_t)kHRecBytes : 0u);
    return r;
  }
  __device__ void load(const Rsrc& r, int i) {   // i < kLoads, a compile-time constant after unrolling
    constexpr int kT = Cf::kThreadsW;
    if (i < kKQ) {
      k[i] = buf_load16(r.k, off_kq + (uint32_t)i * (kT / 16) * qk_row, 0);
    } else if (i < 2 * kKQ) {
      const int j = i - kKQ;
      q[j] = buf_load16(r.q, off_kq + (uint32_t)j * (kT / 16) * qk_row, 0);
    } else if (i < kT3) {
      const int j = i - 2 * kKQ;
      kb[j] = buf_load16(r.kb, off_kq + (uint32_t)j * (kT / 16) * qk_row, 0);
    } else if (i < kT3 + Cf::kPiecesV) {
      const int j = i - kT3;
      v[j] = buf_load16(r.v, off_v + (uint32_t)j * (kT / (Cf::kRows / 8)) * v_row, 0);
    } else if (i < Cf::kLoads - 1) {
      // the record's twelve fragments are the slot's, in the same order
      const int j = i - kT3 - Cf::kPiecesV;
      const int p = tid + j * kT;
      if (p < Cf::kTriFrags * kWave) tri[j] = buf_load16(r.r, 16 * (uint32_t)p, 0);   // uniform per wave
    } else {
      vec = buf_load16(r.r, 16 * (tid % kC) + (uint32_t)kHRecVec, 0);
    }
  }
  // every piece, with each index a compile-time constant (so the staging
  // registers are never indexed at run time)
  template <int... I>
  __device__ void load_seq(const Rsrc& r, std::integer_sequence<int, I...>) { (load(r, I), ...); }
  template <int... I>
  __device__ void commit_seq(uint8_t* base, std::integer_sequence<int, I...>) const { (commit(base, I), ...); }
  __device__ void load_all(const Rsrc& r) { load_seq(r, std::make_integer_sequence<int, Cf::kLoads>{}); }
  __device__ void commit_all(uint8_t* base) const { commit_seq(base, std::make_integer_sequence<int, Cf::kLoads>{}); }

  __device__ void commit(uint8_t* base, int i) const {
    constexpr int kT = Cf::kThreadsW;
    if (i < kT3) {
      const int tile = i / kKQ, j = i % kKQ;
      uint16_t* dst = reinterpret_cast<uint16_t*>(base + tile * Cf::kOffQ);
      const u32x4_t& val = tile == 0 ? k[j] : tile == 1 ? q[j] : kb[Cf::kTiles == 3 ? j : 0];
      const int p = tid + j * kT, r = p >> 4, c8 = 8 * (p & 15);
      // logical columns c8 .. c8+3 and c8+4 .. c8+7 land as two 8-byte runs
      *reinterpret_cast<uint2*>(dst + r * kWP + wave_col(c8)) = make_uint2(val[0], val[1]);
      *reinterpret_cast<uint2*>(dst + r * kWP + wave_col(c8 + 4)) = make_uint2(val[2], val[3]);
    } else if (i < kT3 + Cf::kPiecesV) {
      const int j = i - kT3;
      const int p = tid + j * kT, r = p / (Cf::kRows / 8), c8 = 8 * (p % (Cf::kRows / 8));
      *reinterpret_cast<u32x4_t*>(base + Cf::kOffV + 2 * (r * Cf::kVP + c8)) = v[j];
    } else if (i < Cf::kLoads - 1) {
      const int j = i - kT3 - Cf::kPiecesV;
      const int p = tid + j * kT;
      if (p < Cf::kTriFrags * kWave) *reinterpret_cast<u32x4_t*>(base + Cf::kOffTri + 16 * p) = tri[j];
    } else {
      // every thread loaded piece tid % kC and writes it (duplicates carry the same
      // bytes): a write under tid < kC would let the compiler sink the load into
      // that branch and wait for it there, a full memory round trip per chunk
      reinterpret_cast<u32x4_t*>(base + Cf::kOffVec)[tid % kC] = vec;
    }
  }
};

// Register-resident spine.  kNW waves per workgroup, each holding all 128 key
// columns of its 16 value rows, so every product of the chunk step is
// wave-local.
// kLoaders > 0 adds that many loader waves: they stage chunk cl+1 into the other
// LDS slot while the kNW compute waves work on chunk cl, so the compute waves
// never wait at the texture path; without them the compute waves stage in
// pieces between their MFMAs.
// kNorm (a whole value head per workgroup) applies the sigmoid-gated RMSNorm
// to each chunk's output before it is stored: per token, each wave's partial
// sum of squares over its 16 value columns meets the others' in LDS at the
// chunk's barrier, so the pre-norm output never goes to memory.
struct FusedNorm {
  const uint16_t* z;   // bf16 gate [T][Hv][dv], or null when the norm is not fused
  const float* w;      // [dv]
  float eps;
};

template <int kNW, int kLoaders, typename To, bool kNorm = false, bool kPC = false>
__global__ __launch_bounds__((kNW + kLoaders) * kWave) void chunk_spine_wave_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ kb,
    int64_t qk_stride, const uint16_t* __restrict__ v, int64_t v_stride, const float* __restrict__ init_state,
    const int32_t* __restrict__ cu, int n_seq, int hk, int hv, const uint8_t* __restrict__ ws,
    To* __restrict__ out, float* final_state, FusedNorm nrm) {
  using Cf = SpineCfg<kNW * kWave, 16 * kNW, kPC>;
  using StageCf = SpineCfg<(kLoaders > 0 ? kLoaders : kNW) * kWave, Cf::kRows, kPC>;   // same LDS layout
  static_assert(!kNorm || kNW * 16 == kD, "the fused norm needs a whole value head per workgroup");
  constexpr int kKS = 4;                          // 32-key steps of a wave's state
  constexpr int kJT = 8;                          // 16-key tiles of a wave's state
  // kNorm: per chunk parity, token and wave a partial sum of squares
  constexpr int kExch = kNorm ? 2 * kC * kNW * 4 : 16;
  __shared__ __attribute__((aligned(1024))) uint8_t s_in[2][Cf::kSlotBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_ex[kExch];

  // block -> (sequence, key head) group and member (value head, row block);
  // the members of a group get block ids congruent mod kXcds (one XCD, one L2)
  const int ratio = hv / hk;
  const int blocks_per_head = kD / Cf::kRows;
  const int members = ratio * blocks_per_head;
  const int xcd = blockIdx.x % kXcds;
  const int rest = blockIdx.x / kXcds;
  const int grp = (rest / members) * kXcds + xcd;
  if (grp >= n_seq * hk) return;
  const int member = rest % members;
  const int32_t* first = reinterpret_cast<const int32_t*>(ws);
  const int32_t* order = first + n_seq + 1;
  const int n = plan_order(order, n_seq, grp / hk);
  const int kh = grp % hk;
  const int h = kh * ratio + member / blocks_per_head;
  const int i0 = (member % blocks_per_head) * Cf::kRows;     // first value row of the workgroup
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int iw = 16 * wave;                                  // the wave's rows within the block
  const int g = lane >> 4, m = lane & 15;
  const int seq_beg = cu[n], seq_end = cu[n + 1];
  const int n_chunks = (seq_end - seq_beg + kC - 1) / kC;

  const bool loader = kLoaders > 0 && wave >= kNW;
  ChunkStage<StageCf> stage;
  // scalar decay: khat, qtil of the key head; per-key-channel decay: Kt, Qt, Kb of the value head
  const int rh = kPC ? h : kh;
  stage.kp = k + rh * kD;
  stage.qp = q + rh * kD;
  stage.kbp = kb + rh * kD;
  stage.vp = v + h * kD + i0;
  stage.qk_stride = qk_stride;
  stage.v_stride = v_stride;
  stage.rec0 = ws + records_offset(n_seq) + ((size_t)plan_first(first, n_seq, n) * hv + h) * kHRecBytes;
  stage.rec_step = (size_t)hv * kHRecBytes;
  stage.seq_beg = seq_beg;
  stage.seq_end = seq_end;
  stage.n_chunks = n_chunks;
  stage.tid = kLoaders > 0 ? tid - kNW * kWave : tid;
  stage.init();
  constexpr int kLoads = StageCf::kLoads;


  // ---- the state: S^T tiles, lane holds S[i0 + iw + m][16 jt + 4 g + e], jt < kJT ----
  f32x4_t sst[kJT];
  f32x4_t nw = {0.f, 0.f, 0.f, 0.f};   // norm weights of the lane's output columns iw + 4 g .. +3
  if constexpr (kNorm) nw = *reinterpret_cast<const f32x4_t*>(nrm.w + iw + 4 * g);
  if (!loader) {
    const float* s0 = init_state ? init_state + (((int64_t)n * hv + h) * kD + i0 + iw + m) * kD : nullptr;
#pragma unroll
    for (int jt = 0; jt < kJT; ++jt)
      sst[jt] = s0 ? *reinterpret_cast<const f32x4_t*>(s0 + 16 * jt + 4 * g) : f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // gate inputs of a chunk's outputs (tokens 16 mt + m, columns iw + 4 g .. +3), bf16
  // bits; a chunk past the end of the sequence has an empty range
  typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
  u32x2_t zr[4], zn[4];
  auto load_z = [&](int cl, u32x2_t* dst) {
    const int t0 = seq_beg + cl * kC;
    const uint32_t L = cl < n_chunks ? (uint32_t)min(kC, seq_end - t0) : 0u;
    const __amdgpu_buffer_rsrc_t rz = make_rsrc(nrm.z + ((int64_t)min(t0, seq_end) * hv + h) * kD + iw, L * hv * kD * 2);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
      dst[mt] = __builtin_amdgcn_raw_buffer_load_b64(rz, (16 * mt + m) * (uint32_t)(hv * kD * 2) + 8 * g, 0, 0);
  };
  if constexpr (kNorm) load_z(0, zr);

  // Per-key-channel decay: the loader waves hold the chunk after next in
  // registers (its row tiles are the value head's own, read from HBM, not
  // shared through L2 by a key head's value heads, so their latency shows;
  // with scalar decay the deeper prefetch measured no gain)
  constexpr bool kAhead2 = kPC && kLoaders > 0;
  if (n_chunks > 0 && (kLoaders == 0 || loader)) {
    stage.load_all(stage.rsrc(0));
    stage.commit_all(s_in[0]);
    if constexpr (kAhead2) stage.load_all(stage.rsrc(1));
  }
  // Let every load issued so far land here, once: otherwise the compiler's
  // wait for the initial state (first used at the top of the chunk loop) is
  // placed inside the loop and drains all prefetches on every chunk.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
  const uint32_t orow = (uint32_t)(hv * kD * sizeof(To));
  for (int cl = 0; cl < n_chunks; ++cl) {
    const int slot = cl & 1;
    if (loader) {
      // stage chunk cl+1 into the other slot (free since the last barrier),
      // meeting the compute waves at each of their barriers
      if constexpr (kAhead2) {
        stage.commit_all(s_in[slot ^ 1]);   // loaded during chunk cl-1
        stage.load_all(stage.rsrc(cl + 2));
      } else {
        stage.load_all(stage.rsrc(cl + 1));
        stage.commit_all(s_in[slot ^ 1]);
      }
      __syncthreads();
      continue;
    }
    const int t0 = seq_beg + cl * kC;
    const int L = min(kC, seq_end - t0);
    const uint8_t* base = s_in[slot];
    const uint16_t* sk = reinterpret_cast<const uint16_t*>(base);
    const uint16_t* sq = reinterpret_cast<const uint16_t*>(base + Cf::kOffQ);
    // the state update's row tile: khat itself, or Kb with per-key-channel decay
    const uint16_t* skb = reinterpret_cast<const uint16_t*>(base + (kPC ? Cf::kOffKb : 0));
    const uint16_t* sv = reinterpret_cast<const uint16_t*>(base + Cf::kOffV);
    const uint8_t* tri = base + Cf::kOffTri;
    const float* vec = reinterpret_cast<const float*>(base + Cf::kOffVec);
    auto tri_frag = [&](int which, int x) {
      return load_f16x8(reinterpret_cast<const uint16_t*>(tri + (which * kNF + x) * kHFrag + 16 * lane));
    };
    // LDS operands of the first k step of Y / Z, the V tile, the vectors
    f16x8_t fk[4], fq[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int off = (16 * mt + m) * kWP + 8 * g;
      fk[mt] = load_f16x8(sk + off);
      fq[mt] = load_f16x8(sq + off);
    }
    v4s_t vv[4];
    f32x4_t va[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      vv[mt] = lds_read_tr4(sv + (16 * mt + 4 * g + (m >> 2)) * Cf::kVP + iw + 4 * (m & 3));
      // per-key-channel decay: the decay is in Kt, Qt and Kb, a = b = c = 1
      va[mt] = kPC ? f32x4_t{1.f, 1.f, 1.f, 1.f} : *reinterpret_cast<const f32x4_t*>(vec + 16 * mt + 4 * g);
    }

    // state as B operands (and, for Z^T = S Q^T, as A operands): k step ks = key tiles 2ks, 2ks+1
    f16x8_t sb[kKS];
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) sb[ks] = f16_pair(sst[2 * ks], sst[2 * ks + 1]);
    // Whole-head shape (no loader waves): the state's decay is applied here, off the
    // chain's end, and the update U accumulates into the state tiles themselves
    // (varlen one-call prefill 1.092 -> 1.082 ms; no gain with the 32-row shape)
    constexpr bool kDecayFirst = kLoaders == 0 && !kPC;
    if constexpr (kDecayFirst) {
      const float d = vec[3 * kC];
#pragma unroll
      for (int jt = 0; jt < kJT; ++jt)
#pragma unroll
        for (int e = 0; e < 4; ++e) sst[jt][e] *= d;
    }

    // ---- Y = khat S0^T (rows t, columns i) and Z^T = S0 qtil^T (rows i, columns t), over this wave's keys ----
    f32x4_t y[4], zt[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) y[mt] = zt[mt] = zero4;
    // without loader waves the next chunk's loads go out between these MFMAs
    const auto rn = stage.rsrc(cl + 1);
    constexpr int kLPer = (kLoads + 4 * kKS - 1) / (4 * kKS);
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
      f16x8_t nk[4], nq[4];
      if (ks + 1 < kKS) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const int off = (16 * mt + m) * kWP + 32 * (ks + 1) + 8 * g;
          nk[mt] = load_f16x8(sk + off);
          nq[mt] = load_f16x8(sq + off);
        }
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        if constexpr (kLoaders == 0) {
#pragma unroll
          for (int u = 0; u < kLPer; ++u) {
            const int i = (4 * ks + mt) * kLPer + u;
            if (i < kLoads) stage.load(rn, i);
          }
        }
        y[mt] = mfma_f16(fk[mt], sb[ks], y[mt]);
        zt[mt] = mfma_f16(sb[ks], fq[mt], zt[mt]);
        if constexpr (kLoaders == 0) __builtin_amdgcn_sched_barrier(0);   // keep the staging interleaved
      }
      if (ks + 1 < kKS) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) { fk[mt] = nk[mt]; fq[mt] = nq[mt]; }
      }
    }

    // gate inputs of the next chunk's outputs, issued after the staging loads of
    // the next chunk: loads complete in issue order, so z issued before them
    // would hold up their commits; a chunk ahead, z has a whole chunk to land
    if constexpr (kNorm) load_z(cl + 1, zn);

    // LDS operands of the later products: Tt, Pt (this wave's token tiles) and
    // khat^T for the state update (transposing reads: A[j][slot (g, e)] =
    // khat[k0 + pair_k(0, g, e)][16 jt + j])
    f16x8_t th[kNF], ph[kNF], kt[kJT];
    auto read_tt = [&]() {
#pragma unroll
      for (int x = 0; x < kNF; ++x) th[x] = tri_frag(0, x);
    };
    auto read_pt = [&]() {
#pragma unroll
      for (int x = 0; x < kNF; ++x) ph[x] = tri_frag(1, x);
    };
    auto read_kt = [&](int k0, f16x8_t* dst) {
#pragma unroll
      for (int jt = 0; jt < kJT; ++jt)
        dst[jt] = __builtin_bit_cast(f16x8_t, lds_read_tr8(skb + (k0 + 4 * g + (m >> 2)) * kWP + wave_col(16 * jt + 4 * (m & 3)), 16 * kWP));
    };

    // ---- R = V - a Y (accumulator layout: rows 16 mt + 4 g + e, column iw + m) ----
    f16x8_t rb[2];
    {
      f32x4_t r[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) r[mt][e] = bf16_bits_to_f32((uint16_t)vv[mt][e]) - va[mt][e] * y[mt][e];
      rb[0] = f16_pair(r[0], r[1]);
      rb[1] = f16_pair(r[2], r[3]);
    }

    read_kt(0, kt);
    read_tt();

    // ---- Vnew = Tt R ----
    f32x4_t vn[4];
    {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) vn[mt] = zero4;
#pragma unroll
      for (int x = 0; x < kNF; ++x) vn[frag_mt(x)] = mfma_f16(th[x], rb[frag_ks(x)], vn[frag_mt(x)]);
    }

    f16x8_t nb[2], wb[2];
    nb[0] = f16_pair(vn[0], vn[1]);
    nb[1] = f16_pair(vn[2], vn[3]);
    {
      f32x4_t w[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const f32x4_t c = kPC ? f32x4_t{1.f, 1.f, 1.f, 1.f} : *reinterpret_cast<const f32x4_t*>(vec + 2 * kC + 16 * mt + 4 * g);
#pragma unroll
        for (int e = 0; e < 4; ++e) w[mt][e] = c[e] * vn[mt][e];
      }
      wb[0] = f16_pair(w[0], w[1]);
      wb[1] = f16_pair(w[2], w[3]);
    }

    // The next chunk's inputs go to the other LDS slot in pieces between the
    // remaining MFMAs (groups: U first half, U second half, O^T).
    constexpr int kCGroups = 2 * kJT + kNF;
    constexpr int kCPer = (kLoads + kCGroups - 1) / kCGroups;
    auto commit_group = [&](int grp_idx) {
      if constexpr (kLoaders == 0) {
#pragma unroll
        for (int uu = 0; uu < kCPer; ++uu) {
          const int i = grp_idx * kCPer + uu;
          if (i < kLoads) stage.commit(s_in[slot ^ 1], i);
        }
      }
    };

    // ---- U = K^T W on this wave's key tiles (the state update without the decay) ----
    f32x4_t u_own[kDecayFirst ? 1 : kJT];
    f32x4_t* u = kDecayFirst ? sst : u_own;
#pragma unroll
    for (int jt = 0; jt < kJT; ++jt) {
      commit_group(jt);
      u[jt] = mfma_f16(kt[jt], wb[0], kDecayFirst ? u[jt] : zero4);
      if constexpr (kLoaders == 0) __builtin_amdgcn_sched_barrier(0);
    }
    read_kt(32, kt);   // the second k step reuses kt
    read_pt();

    // the second half of U and the state update before O^T: the update is the
    // chain into the next chunk, O^T only feeds this chunk's output
#pragma unroll
    for (int jt = 0; jt < kJT; ++jt) {
      commit_group(kJT + kNF + jt);
      u[jt] = mfma_f16(kt[jt], wb[1], u[jt]);
      if constexpr (kLoaders == 0) __builtin_amdgcn_sched_barrier(0);
    }

    // ---- S <- d S + U (per-key-channel decay: d per key, S^T's rows) ----
    if constexpr (kDecayFirst) {
      // done: S was decayed before the update accumulated into it
    } else if constexpr (kPC) {
#pragma unroll
      for (int jt = 0; jt < kJT; ++jt) {
        const f32x4_t d = *reinterpret_cast<const f32x4_t*>(vec + 16 * jt + 4 * g);
#pragma unroll
        for (int e = 0; e < 4; ++e) sst[jt][e] = fmaf(d[e], sst[jt][e], u[jt][e]);
      }
    } else {
      const float d = vec[3 * kC];
#pragma unroll
      for (int jt = 0; jt < kJT; ++jt)
#pragma unroll
        for (int e = 0; e < 4; ++e) sst[jt][e] = fmaf(d, sst[jt][e], u[jt][e]);
    }

    // ---- O^T = Z^T diag(b) + Vnew^T Pt^T on this wave's token tiles ----
    // (rows i, columns t: A = Vnew pairs, B = Pt fragments)
    if constexpr (!kPC) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const float b = vec[kC + 16 * mt + m];
#pragma unroll
        for (int e = 0; e < 4; ++e) zt[mt][e] *= b;
      }
    }
    {
#pragma unroll
      for (int x = 0; x < kNF; ++x) {
        commit_group(kJT + x);
        zt[frag_mt(x)] = mfma_f16(nb[frag_ks(x)], ph[x], zt[frag_mt(x)]);
        if constexpr (kLoaders == 0) __builtin_amdgcn_sched_barrier(0);   // keep the staging interleaved
      }
    }

    // ---- the output: lane (g, m) of tile mt holds O[16 mt + m][iw + 4 g .. +3] ----
    // (rows past the end of the sequence fall outside the descriptor)
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(out + ((int64_t)t0 * hv + h) * kD + i0 + iw, (uint32_t)L * orow);
    float* s_ss = reinterpret_cast<float*>(s_ex) + slot * kC * kNW;   // [token][wave]
    if constexpr (kNorm) {
      // this wave's sum of squares per token: the lane's four columns, then the
      // four lane groups holding the same token
      float ss[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        ss[mt] = zt[mt][0] * zt[mt][0] + zt[mt][1] * zt[mt][1] + zt[mt][2] * zt[mt][2] + zt[mt][3] * zt[mt][3];
        ss[mt] += __shfl_xor(ss[mt], 16, kWave);
        ss[mt] += __shfl_xor(ss[mt], 32, kWave);
      }
      s_ss[(16 * g + m) * kNW + wave] = g == 0 ? ss[0] : g == 1 ? ss[1] : g == 2 ? ss[2] : ss[3];
      // w * sigmoid(z), folded into the output tiles
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const float zf[4] = {__uint_as_float(zr[mt][0] << 16), __uint_as_float(zr[mt][0] & 0xffff0000u),
                             __uint_as_float(zr[mt][1] << 16), __uint_as_float(zr[mt][1] & 0xffff0000u)};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          zt[mt][e] *= nw[e] * sigmoidf_(zf[e]);
      }
    } else {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        buf_store4(ro, (16 * mt + m) * orow + 4 * g * (uint32_t)sizeof(To), zt[mt], (To*)nullptr);
    }
    __syncthreads();
    if constexpr (kNorm) {
      // every wave's partial sums are in: scale by rsqrt(mean o^2 + eps) and store
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const f32x4_t* p = reinterpret_cast<const f32x4_t*>(s_ss + (16 * mt + m) * kNW);
        const f32x4_t a = p[0], b = p[1];
        const float tot = ((a[0] + a[1]) + (a[2] + a[3])) + ((b[0] + b[1]) + (b[2] + b[3]));
        const float r = rsqrtf(tot * (1.0f / kD) + nrm.eps);
#pragma unroll
        for (int e = 0; e < 4; ++e) zt[mt][e] *= r;
        buf_store4(ro, (16 * mt + m) * orow + 4 * g * (uint32_t)sizeof(To), zt[mt], (To*)nullptr);
      }
      // (a copy that waits for z of the next chunk here; unrolling two chunks to
      // alternate the register sets instead spills at this register budget)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) zr[mt] = zn[mt];
    }
  }

  if (final_state && !loader) {
    float* s_out = final_state + (((int64_t)n * hv + h) * kD + i0 + iw + m) * kD;
#pragma unroll
    for (int jt = 0; jt < kJT; ++jt) *reinterpret_cast<f32x4_t*>(s_out + 16 * jt + 4 * g) = sst[jt];
  }
}

int chunk_spine_kind(const Dims& d, bool in_bf16, int n) {
  if (!in_bf16) return kSpineLds;
  // per-key-channel decay stages three row tiles: only the 32-row shape's two
  // slots of them fit LDS
  if (d.per_channel) return kSpineRows;
  return n * d.hv >= kWaveSpineMinBlocks ? kSpineWave : kSpineRows;
}

template <bool F32, bool kPC, typename Tin, typename To>
hipError_t chunk_impl(const Dims& d, const void* q, const void* k, int64_t qk_stride, const void* v,
                      int64_t v_stride, const Gates& gt, const float* init_state,
                      const int32_t* cu_dev, int n, int t, int total_chunks, void* out,
                      float* final_state, void* ws, const FusedNorm& nrm, hipStream_t s) {
  uint8_t* w = static_cast<uint8_t*>(ws);
  // register-resident spines: the fp16 row tiles the intra kernel writes after
  // its records -- scalar decay: khat, qtil [T][Hk][dk] (khat also the state
  // update's tile); per-key-channel decay: Kt, Qt, Kb [T][Hv][dk]
  uint16_t* khat = F32 ? nullptr : reinterpret_cast<uint16_t*>(w + hat_offset(n, t, d.hv));
  const int hat_heads = kPC ? d.hv : d.hk;
  uint16_t* qhat = khat ? khat + (size_t)t * hat_heads * kD : nullptr;
  uint16_t* kbar = khat ? (kPC ? qhat + (size_t)t * hat_heads * kD : khat) : nullptr;
  const int64_t hat_stride = (int64_t)hat_heads * kD;
  // bf16 inputs with scalar decay run a register-resident spine: a whole
  // value head per workgroup (eight waves, two per SIMD, so one wave's VALU
  // work overlaps the other's MFMAs, and the gated norm can be fused) once
  // there is a workgroup for every CU; for fewer sequences 32 value rows per
  // workgroup (two compute waves, one per SIMD, and four loader waves) spread
  // them over four times as many workgroups.
  const int spine = chunk_spine_kind(d, !F32, n);
  hipError_t e = hipSuccess;
  if (n > 1) {   // one sequence: the kernels know its plan (plan_first, plan_order)
    hipLaunchKernelGGL(chunk_plan_kernel, dim3(1), dim3(kThreads), 0, s, cu_dev, n,
                       reinterpret_cast<int32_t*>(w), reinterpret_cast<int32_t*>(w) + n + 1);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (total_chunks > 0) {
    if constexpr (kPC)
      hipLaunchKernelGGL((chunk_intra_pc_kernel<F32, Tin>), dim3(total_chunks, d.hv), dim3(kThreads), 0, s,
                         static_cast<const Tin*>(q), static_cast<const Tin*>(k), qk_stride, gt.g, gt.beta,
                         cu_dev, n, d.hk, d.hv, d.l2norm, d.l2_eps, d.q_scale, w, khat);
    else   // bf16: records in the paired-tile k order of the register-resident spines
      hipLaunchKernelGGL((chunk_intra_kernel<F32, Tin, !F32>), dim3(total_chunks, d.hk), dim3(kThreads), 0, s,
                         static_cast<const Tin*>(q), static_cast<const Tin*>(k), qk_stride, gt,
                         cu_dev, n, d.hk, d.hv, d.l2norm, d.l2_eps, d.q_scale, w, khat);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int groups = n * d.hk;
  if (!F32 && spine == kSpineWave) {
    const int members = d.hv / d.hk;
    const int blocks = (groups + kXcds - 1) / kXcds * kXcds * members;
    // (per-key-channel decay and an fp16 output always take the 32-row shape)
    if constexpr (kPC || std::is_same_v<To, _Float16>) return hipErrorInvalidValue;
    else if (nrm.z)
      hipLaunchKernelGGL((chunk_spine_wave_kernel<8, 0, To, true>), dim3(blocks), dim3(8 * kWave), 0, s,
                         qhat, khat, kbar, hat_stride,
                         static_cast<const uint16_t*>(v), v_stride, init_state, cu_dev, n, d.hk, d.hv, w,
                         static_cast<To*>(out), final_state, nrm);
    else
      hipLaunchKernelGGL((chunk_spine_wave_kernel<8, 0, To>), dim3(blocks), dim3(8 * kWave), 0, s,
                         qhat, khat, kbar, hat_stride,
                         static_cast<const uint16_t*>(v), v_stride, init_state, cu_dev, n, d.hk, d.hv, w,
                         static_cast<To*>(out), final_state, nrm);
  } else if (!F32 && spine == kSpineRows) {
    const int members = (d.hv / d.hk) * (kD / (16 * kRowsNW));
    const int blocks = (groups + kXcds - 1) / kXcds * kXcds * members;
    hipLaunchKernelGGL((chunk_spine_wave_kernel<kRowsNW, kRowsLoaders, To, false, kPC>), dim3(blocks),
                       dim3((kRowsNW + kRowsLoaders) * kWave), 0, s,
                       qhat, khat, kbar, hat_stride,
                       static_cast<const uint16_t*>(v), v_stride, init_state, cu_dev, n, d.hk, d.hv, w,
                       static_cast<To*>(out), final_state, nrm);
  } else if constexpr (F32) {
    const int members = (d.hv / d.hk) * (kD / kTile);
    const int blocks = (groups + kXcds - 1) / kXcds * kXcds * members;
    hipLaunchKernelGGL((chunk_spine_kernel<F32, kPC, Tin, To>), dim3(blocks), dim3(kSpineThreads), 0, s,
                       static_cast<const Tin*>(q), static_cast<const Tin*>(k), qk_stride,
                       static_cast<const Tin*>(v), v_stride, gt.g, init_state, cu_dev, n, d.hk, d.hv, w,
                       static_cast<To*>(out), final_state);
  }
  return hipGetLastError();
}

template <bool kPC>
hipError_t chunk_dispatch(const Dims& d, bool in_bf16, bool out_bf16, bool out_f16, const void* q, const void* k,
                          int64_t qk_stride, const void* v, int64_t v_stride, const Gates& gt,
                          const float* init_state, const int32_t* cu_dev, int n, int t,
                          int total, void* out, float* final_state, void* ws, const FusedNorm& nrm,
                          hipStream_t s) {
  if (in_bf16 && out_f16)
    return chunk_impl<false, kPC, uint16_t, _Float16>(d, q, k, qk_stride, v, v_stride, gt, init_state, cu_dev, n, t, total, out, final_state, ws, nrm, s);
  if (in_bf16)
    return out_bf16 ? chunk_impl<false, kPC, uint16_t, uint16_t>(d, q, k, qk_stride, v, v_stride, gt, init_state, cu_dev, n, t, total, out, final_state, ws, nrm, s)
                    : chunk_impl<false, kPC, uint16_t, float>(d, q, k, qk_stride, v, v_stride, gt, init_state, cu_dev, n, t, total, out, final_state, ws, nrm, s);
  return out_bf16 ? chunk_impl<true, kPC, float, uint16_t>(d, q, k, qk_stride, v, v_stride, gt, init_state, cu_dev, n, t, total, out, final_state, ws, nrm, s)
                  : chunk_impl<true, kPC, float, float>(d, q, k, qk_stride, v, v_stride, gt, init_state, cu_dev, n, t, total, out, final_state, ws, nrm, s);
}

}  // namespace

bool chunk_fuses_norm(const Dims& d, bool in_bf16, int n) {
  return chunk_spine_kind(d, in_bf16, n) == kSpineWave;
}

bool chunk_out_f16(const Dims& d, bool in_bf16, int n) {
  return chunk_spine_kind(d, in_bf16, n) == kSpineRows;
}

size_t chunk_workspace_bytes(const Dims& d, int n, int t) {
  const size_t max_chunks = (size_t)t / kC + (size_t)n;
  // the larger of the two layouts: hi/lo or fp32 records (fp32 inputs, per-key-channel
  // decay), or fp16 records and the normalised rows (the register-resident spines)
  const size_t split = records_offset(n) + max_chunks * d.hv * kRecBytes;
  const size_t half = hat_offset(n, t, d.hv) +
                      (d.per_channel ? 3 * (size_t)d.hv : 2 * (size_t)d.hk) * t * kD * sizeof(uint16_t);
  return std::max(split, half);
}

hipError_t launch_chunk_prefill(const Dims& d, bool in_bf16, bool out_bf16, const void* q,
                                const void* k, int64_t qk_stride, const void* v,
                                int64_t v_stride, const Gates& gt, const float* init_state,
                                const int32_t* cu_dev,
                                const int32_t* cu_host, int n, int t, void* out,
                                float* final_state, void* ws, size_t ws_bytes,
                                const uint16_t* norm_z, const float* norm_w, hipStream_t s, bool out_f16) {
  (void)ws_bytes;
  if (n == 0) return hipSuccess;
  if (norm_z && !chunk_fuses_norm(d, in_bf16, n)) return hipErrorInvalidValue;
  if (out_f16 && !chunk_out_f16(d, in_bf16, n)) return hipErrorInvalidValue;
  int total = 0;
  for (int i = 0; i < n; ++i) total += (cu_host[i + 1] - cu_host[i] + kC - 1) / kC;
  const FusedNorm nrm{norm_z, norm_w, d.rms_eps};
  return d.per_channel
             ? chunk_dispatch<true>(d, in_bf16, out_bf16, out_f16, q, k, qk_stride, v, v_stride, gt, init_state, cu_dev, n, t, total, out, final_state, ws, nrm, s)
             : chunk_dispatch<false>(d, in_bf16, out_bf16, out_f16, q, k, qk_stride, v, v_stride, gt, init_state, cu_dev, n, t, total, out, final_state, ws, nrm, s);
}

}  // namespace gdn
