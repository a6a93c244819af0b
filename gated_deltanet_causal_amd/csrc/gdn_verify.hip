// gdn_verify.hip -- the speculative verify transaction: K rows per sequence
// decoded from the prior logical state, which only the commit changes.
//
// Follows the Qwen3.8 kernel TDD ledger's transaction rules (the verified
// rows are computed from the prior state; a commit publishes the state after
// the accepted prefix; abort, error or an unresolved drop leaves the prior
// state; rejected rows must never be read) and the Qwen3SsmLayer field notes
// on the WY verify kernels (one kernel for all K rows of a window, the h-state
// read once, with either per-token rollback snapshots or a write-on-accept
// twin whose post-verdict fold applies only the accepted rows).  This is the
// write-on-accept form:
//
//   verify  per (sequence, value head) workgroup, the head's state is read
//           once into registers and carried through the K rows; row
//           t is exactly the fused decode step (conv from register windows,
//           L2 / q scale, decay, predict, write, output, gated norm), with the
//           state-free parts (conv, gates, norms) of four rows at a time done
//           before those rows' state work, so a group of rows costs four
//           barriers rather than four per row.  Besides
//           the outputs it records, per row, the update's two vectors: u
//           ([Hv][dv]) and the normalised key ([Hk][dk]).  The state and the
//           conv state in memory are not written.
//   commit  per (sequence, value head): with c = accepted rows, the state is
//           read, the c rank-one updates S <- S diag(a_t) + u_t khat_t^T are
//           replayed in the verify's own operation order (so the result is the
//           state the verify carried after row c, bit for bit) and written;
//           c = 0 touches nothing.  The conv state takes the last three inputs
//           of (its rows, x rows 0 .. c-1).
//
// HBM per transaction: the state is read twice and written once (2R + 1W),
// against 1R + KW for per-row snapshots plus a copy at commit.
#include <type_traits>

#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

constexpr int kGroup = 256;             // threads per value head
constexpr int kD = 128;                 // head_k_dim == head_v_dim
constexpr int kCThreads = 512;          // commit: threads per value head
constexpr int kCRowGroups = kCThreads / 32;
constexpr int kCRows = kD / kCRowGroups;  // commit: state rows per thread, rows rg + kCRowGroups m
constexpr int kVRows = 4;               // verify: state rows per thread, rows rb + 32 m
constexpr int kVGroup = 4;              // verify: rows of the window prepared together

// Sum over the 8 lanes holding one state row in the verify (lanes 8r .. 8r+7):
// quad permutes for lane distance 1 and 2, then the half-row mirror (lane i of
// the eight with lane 7 - i, in the other quad).
__device__ __forceinline__ float row8_sum(float v) {
  v = dpp_add<0xB1>(v);    // quad_perm [1,0,3,2]
  v = dpp_add<0x4E>(v);    // quad_perm [2,3,0,1]
  return dpp_add<0x141>(v);  // row_half_mirror
}

// One conv window of a channel, carried in registers across the rows (the
// taps are read again for each row: they stay in cache and keep registers free).
struct ConvWindow {
  float s0, s1, s2;
  // y = act(w . (s0, s1, s2, x)); the window becomes (s1, s2, x).  Same
  // arithmetic as the decode step's conv.
  __device__ float step(const float* conv_w, int c, float xv, int act) {
    const f32x4_t w = *reinterpret_cast<const f32x4_t*>(conv_w + (int64_t)c * 4);
    float y = w[0] * s0;
    y = fmaf(w[1], s1, y);
    y = fmaf(w[2], s2, y);
    y = fmaf(w[3], xv, y);
    s0 = s1;
    s1 = s2;
    s2 = xv;
    return act ? silu_conv(y) : y;
  }
};

// A stored value as loaded (bf16: its 16 bits, zero-extended; fp32: the value),
// widened to fp32 at its use.  pin() marks the register as written at that point,
// so that neither the widening nor anything else that uses the load can be
// moved above it: placed after the state loads, the wait for an early load then
// comes after the state loads are issued.
template <typename T>
struct Raw {
  typename std::conditional<sizeof(T) == 2, uint32_t, float>::type r;
  __device__ __forceinline__ void load(const T* p) { r = *p; }
  __device__ __forceinline__ float widen() const {
    if constexpr (sizeof(T) == 2) return __uint_as_float(r << 16); else return r;
  }
  __device__ __forceinline__ void pin() { asm volatile("" : "+v"(r)); }
};

// The window's three stored values, loaded early and widened after the pin.
template <typename T>
struct RawWindow {
  Raw<T> s0, s1, s2;
  __device__ __forceinline__ void pin() { s0.pin(); s1.pin(); s2.pin(); }
  __device__ __forceinline__ ConvWindow widen() const { return ConvWindow{s0.widen(), s1.widen(), s2.widen()}; }
};
template <typename T>
__device__ __forceinline__ RawWindow<T> load_window(const T* cs_row, int c, int cc) {
  RawWindow<T> w;
  w.s0.load(cs_row + c);
  w.s1.load(cs_row + cc + c);
  w.s2.load(cs_row + 2 * cc + c);
  return w;
}

template <typename T, typename To, bool kPerChannel>
__global__ __launch_bounds__(kGroup) void verify_kernel(
    const T* __restrict__ x, const float* __restrict__ conv_w, const T* __restrict__ conv_state,
    const float* __restrict__ g, const float* __restrict__ beta, const T* __restrict__ z,
    const float* __restrict__ norm_w, const float* __restrict__ state, To* __restrict__ out,
    float* __restrict__ rec_u, float* __restrict__ rec_k, int K, int hk, int hv, int cc, int act,
    int l2norm, float l2_eps, float q_scale, float rms_eps) {
  const int b = blockIdx.x / hv;
  const int h = blockIdx.x % hv;
  const int kh = h / (hv / hk);           // the key head it reads (repeat-interleave)
  const int tid = threadIdx.x;
  const int gt = tid;
  const int gwave = gt / kWave;
  const int lane = tid % kWave;
  // Each thread holds 16 columns of 4 state rows: rows rb + 32 m, columns
  // 32 i + 4 cb + e (i, e < 4).  A row's dot products then reduce over its 8
  // lanes (three DPP steps), and each 16-byte access of 8 lanes is one full
  // 128-byte line of a row.
  const int cb = gt % 8;
  const int rb = gt / 8;

  // per row of the current group: conv outputs, decay factors (per channel, or
  // one), beta, the q / k norm factors, the outputs and their sums of squares
  __shared__ float s_q[kVGroup][kD], s_k[kVGroup][kD], s_v[kVGroup][kD], s_o[kVGroup][kD];
  __shared__ float s_a[kVGroup][kPerChannel ? kD : 1], s_bt[kVGroup];
  __shared__ float s_scal[kVGroup][2], s_nrm[kVGroup][2];

  // conv windows: thread i owns q channel i (i < kD) or k channel i - kD of the
  // key head, and threads below kD also v channel i of the value head.  The
  // conv state is only read, so the value heads of a key head each redo the
  // key head's q / k conv (a workgroup per value head).
  const T* cs_row = conv_state + (int64_t)b * 3 * cc;
  const int c_qk = tid < kD ? kh * kD + tid : hk * kD + kh * kD + (tid - kD);
  const int c_v = 2 * hk * kD + h * kD + gt % kD;
  // loaded by every thread (threads past kD repeat a channel, unused): a load
  // under a branch is waited for inside it, before the state loads are issued
  RawWindow<T> raw_qk = load_window(cs_row, c_qk, cc);
  RawWindow<T> raw_v = load_window(cs_row, c_v, cc);

  // A group's row inputs, fetched for all its rows at once (the first group's
  // before the state loads, each later one at the end of the group before it).
  // Thread i < kD also loads the per-channel log decay of channel i; the
  // scalar gates are loaded by every thread.
  Raw<T> xqk_n[kVGroup], xv_n[kVGroup], z_n[kVGroup];
  float g_n[kVGroup], bt_n[kVGroup];
  auto fetch = [&](int t0, int nb) {
#pragma unroll
    for (int j = 0; j < kVGroup; ++j) {
      const int t = t0 + min(j, nb - 1);   // rows past the group repeat its last (unused)
      const int64_t row_t = (int64_t)b * K + t;
      const T* x_row = x + row_t * cc;
      xqk_n[j].load(x_row + c_qk);
      xv_n[j].load(x_row + c_v);
      z_n[j].load(z + (row_t * hv + h) * kD + gt % kD);
      g_n[j] = kPerChannel ? g[(row_t * hv + h) * kD + gt % kD] : g[row_t * hv + h];
      bt_n[j] = beta[row_t * hv + h];
    }
  };
  fetch(0, min(K, kVGroup));

  // the head's state, read once and carried through the K rows.  Its loads are
  // issued after the conv windows and the first group's inputs: loads complete
  // in issue order, so the first group's conv and norms wait only for their own
  // inputs while the 64 KiB of state is still in flight
  // (buffer loads, streamed: a plain load would be sunk to its first use)
  const float* S = state + ((int64_t)b * hv + h) * kD * kD;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(S), (short)0,
                                                                     kD * kD * (int)sizeof(float), 0x00020000);
  const uint32_t voff = (uint32_t)(rb * kD + 4 * cb) * sizeof(float);
  f32x4_t sreg[kVRows][4];
#pragma unroll
  for (int m = 0; m < kVRows; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      sreg[m][i] = __builtin_bit_cast(
          f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, (uint32_t)((32 * m * kD + 32 * i) * sizeof(float)), 2));
  // nothing that uses the window or row loads may move above the state loads
  __builtin_amdgcn_sched_barrier(0);
  raw_qk.pin();
  raw_v.pin();
#pragma unroll
  for (int j = 0; j < kVGroup; ++j) {
    xqk_n[j].pin();
    xv_n[j].pin();
    z_n[j].pin();
  }
  ConvWindow wqk = raw_qk.widen(), wv = raw_v.widen();

  // Rows in groups of kVGroup.  Per group: the conv, gates and q / k norms of
  // all its rows first (they do not depend on the state), then the state rows
  // through all of them without a barrier, then the rows' gated norms.  Each
  // row's arithmetic is the decode step's, in the same order.
  // K >= 1 (checked before the launch): a do-while has no entry test, which
  // would let the compiler sink the state loads behind it
  int t0 = 0;
  do {
    const int nb = min(K - t0, kVGroup);
    float zv[kVGroup];
#pragma unroll
    for (int j = 0; j < kVGroup; ++j) {
      if (j < nb) {
        const float y = wqk.step(conv_w, c_qk, xqk_n[j].widen(), act);
        if (tid < kD) s_q[j][tid] = y; else s_k[j][tid - kD] = y;
        if (gt < kD) {
          s_v[j][gt] = wv.step(conv_w, c_v, xv_n[j].widen(), act);
          if constexpr (kPerChannel) s_a[j][gt] = __expf(g_n[j]);
        }
        if (tid == 0) {
          if constexpr (!kPerChannel) s_a[j][0] = __expf(g_n[j]);
          s_bt[j] = bt_n[j];
        }
      }
      zv[j] = z_n[j].widen();
    }
    __syncthreads();
    // q / k norm factors: (row, q or k) tasks over the waves
    for (int task = gwave; task < 2 * nb; task += kGroup / kWave) {
      const int j = task >> 1, w = task & 1;
      const float* src = w == 0 ? s_q[j] : s_k[j];
      const float a0 = src[2 * lane], a1 = src[2 * lane + 1];
      const float ss = wave_sum(a0 * a0 + a1 * a1);
      if (lane == 0) s_scal[j][w] = l2norm ? 1.0f / sqrtf(ss + l2_eps) : 1.0f;
    }
    __syncthreads();
    // the next group's inputs, in flight during this group's state work
    if (t0 + kVGroup < K) fetch(t0 + kVGroup, min(K - t0 - kVGroup, kVGroup));

#pragma unroll
    for (int j = 0; j < kVGroup; ++j) {
      if (j < nb) {
        const int64_t row_t = (int64_t)b * K + t0 + j;   // (sequence, verified row)
        const float rq = s_scal[j][0] * q_scale, rk = s_scal[j][1];
        const float kq = wave_sum(s_k[j][2 * lane] * s_q[j][2 * lane] + s_k[j][2 * lane + 1] * s_q[j][2 * lane + 1]) * rq * rk;
        f32x4_t kcol[4], qcol[4], a[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x4_t kv = *reinterpret_cast<const f32x4_t*>(&s_k[j][32 * i + 4 * cb]);
          const f32x4_t qv = *reinterpret_cast<const f32x4_t*>(&s_q[j][32 * i + 4 * cb]);
#pragma unroll
          for (int e = 0; e < 4; ++e) { kcol[i][e] = kv[e] * rk; qcol[i][e] = qv[e] * rq; }
          if constexpr (kPerChannel) {
            a[i] = *reinterpret_cast<const f32x4_t*>(&s_a[j][32 * i + 4 * cb]);
          } else {
            const float av = s_a[j][0];
            a[i] = f32x4_t{av, av, av, av};
          }
        }
        const float bt = s_bt[j];
        // the normalised key of this row, for the commit's replay
        if (h % (hv / hk) == 0 && gt < kD) rec_k[(row_t * hk + kh) * kD + gt] = s_k[j][gt] * rk;

        // per state row: decay, the two dot products, u = beta (v - p),
        // o = r + u (khat . qtil), S' = Sd + u khat^T (as the decode step)
        float* u_out = rec_u + (row_t * hv + h) * kD;
#pragma unroll
        for (int m = 0; m < kVRows; ++m) {
          const int row = rb + 32 * m;
          float pk = 0.0f, pq = 0.0f;
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              sreg[m][i][e] *= a[i][e];
              pk = fmaf(sreg[m][i][e], kcol[i][e], pk);
              pq = fmaf(sreg[m][i][e], qcol[i][e], pq);
            }
          pk = row8_sum(pk);
          pq = row8_sum(pq);
          const float u = bt * (s_v[j][row] - pk);
          if (cb == 0) {
            s_o[j][row] = fmaf(u, kq, pq);
            u_out[row] = u;
          }
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) sreg[m][i][e] = fmaf(u, kcol[i][e], sreg[m][i][e]);
        }
      }
    }
    __syncthreads();

    // the sigmoid gated RMSNorm of each row's 128 outputs: the sums of squares
    // of the two 64-output halves, (row, half) tasks over the waves
    for (int task = gwave; task < 2 * nb; task += kGroup / kWave) {
      const int j = task >> 1, half = task & 1;
      const float o = s_o[j][64 * half + lane];
      const float ss = wave_sum(o * o);
      if (lane == 0) s_nrm[j][half] = ss;
    }
    __syncthreads();
    if (gt < kD) {
#pragma unroll
      for (int j = 0; j < kVGroup; ++j) {
        if (j < nb) {
          const int64_t row_t = (int64_t)b * K + t0 + j;
          const float o = s_o[j][gt];
          const float r = rsqrtf((s_nrm[j][0] + s_nrm[j][1]) * (1.0f / kD) + rms_eps);
          st(out + (row_t * hv + h) * kD + gt, o * r * norm_w[gt] * sigmoidf_(zv[j]));
        }
      }
    }
    t0 += kVGroup;
  } while (t0 < K);
}

// Commit of the recurrent state: sequence b keeps its first clamp(accepted[b],
// 0, K) verified rows.  One 512-thread workgroup per (sequence, value head),
// eight state rows per thread: four share a CU at eight waves per SIMD, so the
// 3072 heads of a 64-sequence batch run as three full rounds (256-thread
// workgroups, 96 VGPRs, ran 2.4 rounds).
template <bool kPerChannel>
__global__ __launch_bounds__(kCThreads, kCThreads / 64) void verify_commit_state_kernel(
    const int32_t* __restrict__ accepted, const float* __restrict__ g, const float* __restrict__ rec_u,
    const float* __restrict__ rec_k, float* __restrict__ state, int K, int hk, int hv) {
  const int b = blockIdx.x / hv;
  const int h = blockIdx.x % hv;
  const int kh = h / (hv / hk);
  const int c = min(max(accepted[b], 0), K);
  if (c == 0) return;   // abort: the prior state stays
  const int gt = threadIdx.x;
  const int cg = gt % 32, rg = gt / 32;
  float* S = state + ((int64_t)b * hv + h) * kD * kD;
  f32x4_t sreg[kCRows];
#pragma unroll
  for (int m = 0; m < kCRows; ++m)
    sreg[m] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(S + (rg + kCRowGroups * m) * kD + 4 * cg));
  for (int t = 0; t < c; ++t) {
    const int64_t row_t = (int64_t)b * K + t;
    float a[4];
    if constexpr (kPerChannel) {
      const f32x4_t gv = *reinterpret_cast<const f32x4_t*>(g + (row_t * hv + h) * kD + 4 * cg);
#pragma unroll
      for (int e = 0; e < 4; ++e) a[e] = __expf(gv[e]);
    } else {
      const float av = __expf(g[row_t * hv + h]);
#pragma unroll
      for (int e = 0; e < 4; ++e) a[e] = av;
    }
    const f32x4_t kcol = *reinterpret_cast<const f32x4_t*>(rec_k + (row_t * hk + kh) * kD + 4 * cg);
    const float* u_in = rec_u + (row_t * hv + h) * kD;
#pragma unroll
    for (int m = 0; m < kCRows; ++m) {
      const float u = u_in[rg + kCRowGroups * m];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sreg[m][e] *= a[e];
        sreg[m][e] = fmaf(u, kcol[e], sreg[m][e]);
      }
    }
  }
#pragma unroll
  for (int m = 0; m < kCRows; ++m)
    __builtin_nontemporal_store(sreg[m], reinterpret_cast<f32x4_t*>(S + (rg + kCRowGroups * m) * kD + 4 * cg));
}

// Commit of the conv state: the last three inputs of (the state's rows, x rows
// 0 .. c-1).  One thread per (sequence, channel).
template <typename T>
__global__ __launch_bounds__(kGroup) void verify_commit_conv_kernel(const int32_t* __restrict__ accepted,
                                                                    const T* __restrict__ x,
                                                                    T* __restrict__ conv_state, int K,
                                                                    int cc) {
  const int b = blockIdx.y;
  const int ch = blockIdx.x * kGroup + threadIdx.x;
  if (ch >= cc) return;
  const int c = min(max(accepted[b], 0), K);
  if (c == 0) return;
  T* cs = conv_state + (int64_t)b * 3 * cc + ch;
  float win[3] = {ld(cs), ld(cs + cc), ld(cs + 2 * cc)};
  for (int t = 0; t < c; ++t) {
    win[0] = win[1];
    win[1] = win[2];
    win[2] = ld(x + ((int64_t)b * K + t) * cc + ch);
  }
  st(cs, win[0]);
  st(cs + cc, win[1]);
  st(cs + 2 * cc, win[2]);
}

template <typename T, typename To, bool kPC>
hipError_t verify_launch(const Dims& d, const void* x, const float* conv_w, const void* conv_state,
                         const float* g, const float* beta, const void* z, const float* norm_w,
                         const float* state, void* out, float* rec_u, float* rec_k, int b, int k,
                         hipStream_t s) {
  hipLaunchKernelGGL((verify_kernel<T, To, kPC>), dim3(b * d.hv), dim3(kGroup), 0, s, static_cast<const T*>(x),
                     conv_w, static_cast<const T*>(conv_state), g, beta, static_cast<const T*>(z), norm_w, state,
                     static_cast<To*>(out), rec_u, rec_k, k, d.hk, d.hv, d.cc, d.act, d.l2norm, d.l2_eps, d.q_scale,
                     d.rms_eps);
  return hipGetLastError();
}

}  // namespace

size_t verify_workspace_bytes(const Dims& d, int b, int k) {
  return (size_t)b * k * ((size_t)d.hv * d.dv + (size_t)d.hk * d.dk) * sizeof(float);
}

hipError_t launch_verify(const Dims& d, bool bf16, bool out_bf16, const void* x, const float* conv_w,
                         const void* conv_state, const float* g, const float* beta, const void* z,
                         const float* norm_w, const float* state, void* out, int b, int k, void* ws,
                         hipStream_t s) {
  if (b == 0) return hipSuccess;
  float* rec_u = static_cast<float*>(ws);
  float* rec_k = rec_u + (size_t)b * k * d.hv * d.dv;
#define GDN_VERIFY_TYPES(T, To)                                                                         \
  return d.per_channel                                                                                  \
             ? verify_launch<T, To, true>(d, x, conv_w, conv_state, g, beta, z, norm_w, state, out,    \
                                          rec_u, rec_k, b, k, s)                                      \
             : verify_launch<T, To, false>(d, x, conv_w, conv_state, g, beta, z, norm_w, state, out,   \
                                           rec_u, rec_k, b, k, s)
  if (bf16) {
    if (out_bf16) { GDN_VERIFY_TYPES(uint16_t, uint16_t); }
    GDN_VERIFY_TYPES(uint16_t, float);
  }
  if (out_bf16) { GDN_VERIFY_TYPES(float, uint16_t); }
  GDN_VERIFY_TYPES(float, float);
#undef GDN_VERIFY_TYPES
}

hipError_t launch_verify_commit(const Dims& d, bool bf16, const int32_t* accepted, const void* x,
                                const float* g, void* conv_state, float* state, int b, int k,
                                const void* ws, hipStream_t s) {
  if (b == 0) return hipSuccess;
  const float* rec_u = static_cast<const float*>(ws);
  const float* rec_k = rec_u + (size_t)b * k * d.hv * d.dv;
  if (d.per_channel)
    hipLaunchKernelGGL(verify_commit_state_kernel<true>, dim3(b * d.hv), dim3(kCThreads), 0, s, accepted, g, rec_u,
                       rec_k, state, k, d.hk, d.hv);
  else
    hipLaunchKernelGGL(verify_commit_state_kernel<false>, dim3(b * d.hv), dim3(kCThreads), 0, s, accepted, g, rec_u,
                       rec_k, state, k, d.hk, d.hv);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 cgrid((d.cc + kGroup - 1) / kGroup, b);
  if (bf16)
    hipLaunchKernelGGL(verify_commit_conv_kernel<uint16_t>, cgrid, dim3(kGroup), 0, s, accepted,
                       static_cast<const uint16_t*>(x), static_cast<uint16_t*>(conv_state), k, d.cc);
  else
    hipLaunchKernelGGL(verify_commit_conv_kernel<float>, cgrid, dim3(kGroup), 0, s, accepted,
                       static_cast<const float*>(x), static_cast<float*>(conv_state), k, d.cc);
  return hipGetLastError();
}

}  // namespace gdn
