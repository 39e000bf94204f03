// libmhc: gfx950 (MI355X, CDNA4) kernels and C ABI of the Single-Pass mHC step.
//
// Pages followed (by title and section):
//   [SW] "DeepSeek V4.1 · Stream weights for the feed-forward": "Why" (one fused
//        pass over the streams, (2n+2)*d traffic), "All 5 steps" and the Code
//        excerpts hc_mixes / hc_pre / hc_post and the split/Sinkhorn kernel.
//   [RN] "DeepSeek V4.1 · MoE RMSNorm": RMSNorm formula and Code (RMSNorm,
//        Block.forward).
//
// Design (one pass per token; every HBM byte of the streams is touched once):
//   * A workgroup owns a tile of 16 tokens and all d features of them. Its 8
//     waves split the features: wave w takes the 32-feature steps w, w+8, ...
//     Lane l works on token l%16 and on 8 consecutive features (one 16-byte
//     bf16 load per stream), so the four lanes of a token read 64 contiguous
//     bytes per stream and step.
//   * That lane layout IS the A-operand layout of v_mfma_f32_16x16x32_bf16
//     (row = token, 8 K values per lane), so the freshly rounded new streams
//     feed the 24-wide projection without any reshuffle. The projection
//     weights are pre-split into three exact bf16 terms (mhc_pack_wmix) and
//     packed in B-operand order; 72 columns (3 x 24) padded to 5 tiles of 16.
//   * The rounded hc_pre result h (bf16, 8 values per lane and step) stays in
//     registers until the token's sum of squares is complete, then the
//     normalised y is written: streams are read once and written once.
//   * The per-token tail (RMS, split, 4x4 Sinkhorn) runs after one LDS
//     reduction of the per-wave partials.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "mhc.h"

namespace {

constexpr int kStreams = 4;
constexpr int kMix = 24;
constexpr int kTok = 16;              // tokens per workgroup = rows of one MFMA tile
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kStep = 32;             // features per wave step (4 lane groups x 8)
constexpr int kMaxSpw = 20;           // steps per wave with h held in registers
constexpr int kTilesBf = 5;           // bf16 path: 80 packed columns (hi/mid/lo x 24 + pad)
constexpr int kTilesF = 2;            // f32 path: 32 packed columns (24 + pad)
constexpr int kColsMax = 16 * kTilesBf;

enum Mode { kFused = 0, kMixesOnly = 1 };

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats -> two bf16 (round to nearest even), `a` in the low half: the
// packed hardware conversion (v_cvt_pk_bf16_f32, round to nearest even in the
// default mode).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Every vector store of more than 64 bits is followed by this guard. On gfx950
// the compiler may overwrite a store's data registers with the very next VALU
// instruction (no wait state), and such stores have written wrong data for
// some lanes (lanes 12-15 of each 16-lane row, the words rewritten first,
// intermittently). A few wait states right after the store, with the
// scheduler kept from moving anything across, avoid it. The store's data is an
// input of the wait-state asm, so its registers stay allocated to it until the
// wait states have passed: no copy inserted after scheduling can land between
// the store and the guard and overwrite them (a CPU test checks the compiled
// code: every store wider than 64 bits is followed at once by s_nop 4).
template <class T>
__device__ __forceinline__ void store_guard(const T& data) {
  __builtin_amdgcn_sched_barrier(0);
  __asm__ volatile("s_nop 4" ::"v"(data));
  __builtin_amdgcn_sched_barrier(0);
}
// pins the store that follows in place (nothing is scheduled across it)
__device__ __forceinline__ void store_pin() { __builtin_amdgcn_sched_barrier(0); }

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) {
  store_pin();
  *reinterpret_cast<u32x4*>(p) = v;
  store_guard(v);
}
__device__ __forceinline__ void st4f(float* p, f32x4 v) {
  store_pin();
  *reinterpret_cast<f32x4*>(p) = v;
  store_guard(v);
}

// Stream tensors are touched once: load/store them non-temporally so they do
// not push the packed projection out of L2.
__device__ __forceinline__ u32x4 lds16(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void sts16(void* p, u32x4 v) {
  store_pin();
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
  store_guard(v);
}

__device__ __forceinline__ float sigmoidf(float z) { return 1.0f / (1.0f + expf(-z)); }

// Split one token's mixes into (pre, post, comb): [SW] Code, the split/Sinkhorn
// kernel, and "All 5 steps" (p, u, C). The 4x4 lives in registers; the first row
// normalisation is the max-subtracted softmax, every later division is by
// (sum + hc_eps); the schedule ends with a column division.
__device__ void split_sinkhorn_token(const float* m, const float* base, const float* scale,
                                     int iters, float eps, float* pre, float* post,
                                     float* comb) {
  const float s0 = scale[0], s1 = scale[1], s2 = scale[2];
#pragma unroll
  for (int j = 0; j < 4; ++j) pre[j] = sigmoidf(m[j] * s0 + base[j]) + eps;
#pragma unroll
  for (int k = 0; k < 4; ++k) post[k] = 2.0f * sigmoidf(m[4 + k] * s1 + base[4 + k]);
  float c[4][4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int k = 0; k < 4; ++k) c[j][k] = m[8 + 4 * j + k] * s2 + base[8 + 4 * j + k];
    const float mx = fmaxf(fmaxf(c[j][0], c[j][1]), fmaxf(c[j][2], c[j][3]));
#pragma unroll
    for (int k = 0; k < 4; ++k) c[j][k] = expf(c[j][k] - mx);
    const float rs = (c[j][0] + c[j][1]) + (c[j][2] + c[j][3]);
#pragma unroll
    for (int k = 0; k < 4; ++k) c[j][k] = c[j][k] / rs + eps;
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float cs = ((c[0][k] + c[1][k]) + (c[2][k] + c[3][k])) + eps;
#pragma unroll
    for (int j = 0; j < 4; ++j) c[j][k] = c[j][k] / cs;
  }
  for (int it = 1; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float rs = ((c[j][0] + c[j][1]) + (c[j][2] + c[j][3])) + eps;
#pragma unroll
      for (int k = 0; k < 4; ++k) c[j][k] = c[j][k] / rs;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float cs = ((c[0][k] + c[1][k]) + (c[2][k] + c[3][k])) + eps;
#pragma unroll
      for (int j = 0; j < 4; ++j) c[j][k] = c[j][k] / cs;
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int k = 0; k < 4; ++k) comb[4 * j + k] = c[j][k];
}

struct StepArgs {
  const void* x;
  const void* f;
  const float* pre_in;
  const float* post_in;
  const float* comb_in;
  const void* wpk;
  const float* base;
  const float* scale;
  const float* gamma;
  void* x_out;
  void* y_out;
  float* pre_out;
  float* post_out;
  float* comb_out;
  float* mix_out;
  int64_t tokens;
  int d;
  int iters;
  float norm_eps;
  float hc_eps;
};

// Per-lane state carried through a tile.
template <int kTiles>
struct LaneState {
  float C[4][4];   // comb_in of the lane's token, [j][k]
  float U[4];      // post_in
  float P[4];      // pre_in
  f32x4 acc[kTiles];
  float ss;        // partial sum of squares of the new streams
  float hs;        // partial sum of squares of h
};

// ----- bf16 streams ---------------------------------------------------------------------

struct InBf {
  u32x4 x[4];
  u32x4 f;
};

template <int MODE>
__device__ __forceinline__ void load_bf(InBf& in, const uint16_t* xrow, const uint16_t* frow,
                                        int d, int f0, bool valid) {
  if (valid) {
#pragma unroll
    for (int j = 0; j < 4; ++j) in.x[j] = lds16(xrow + (size_t)j * d + f0);
    in.f = MODE == kFused ? lds16(frow + f0) : u32x4{0, 0, 0, 0};
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) in.x[j] = u32x4{0, 0, 0, 0};
    in.f = u32x4{0, 0, 0, 0};
  }
}

// One 32-feature step of one wave for 16 tokens: hc_post, the running sums,
// hc_pre, the store of the new streams and 20 MFMAs of the projection.
// Returns the packed bf16 h of the lane's 8 features.
template <int MODE>
__device__ __forceinline__ u32x4 step_bf(const InBf& in, LaneState<kTilesBf>& st,
                                         const u32x4* __restrict__ wstep, int lane,
                                         uint16_t* xorow, int d, int f0, bool valid) {
  u32x4 xo[4];
  if (MODE == kFused) {
    // hc_post ([SW] Code): new stream k = sum_j comb[j][k] * x_j + post[k] * f, fp32,
    // then rounded to bf16.
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      float a0[4], a1[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        a0[j] = bf_lo(in.x[j][w]);
        a1[j] = bf_hi(in.x[j][w]);
      }
      const float f0v = bf_lo(in.f[w]), f1v = bf_hi(in.f[w]);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float v0 = a0[0] * st.C[0][k];
        float v1 = a1[0] * st.C[0][k];
#pragma unroll
        for (int j = 1; j < 4; ++j) {
          v0 = fmaf(a0[j], st.C[j][k], v0);
          v1 = fmaf(a1[j], st.C[j][k], v1);
        }
        v0 = fmaf(f0v, st.U[k], v0);
        v1 = fmaf(f1v, st.U[k], v1);
        xo[k][w] = pack_bf16x2(v0, v1);
      }
    }
    if (valid) {
#pragma unroll
      for (int k = 0; k < 4; ++k) sts16(xorow + (size_t)k * d + f0, xo[k]);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) xo[k] = in.x[k];
  }

  // projection partials: A = new stream k (8 features of the lane's token),
  // B = packed weight terms for the same features.
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const bf16x8 A = __builtin_bit_cast(bf16x8, xo[k]);
#pragma unroll
    for (int q = 0; q < kTilesBf; ++q) {
      // the last tile holds columns 64..79 of which 72..79 are padding
      const bool pad = q == kTilesBf - 1 && (lane & 15) >= 3 * kMix - 64;
      const u32x4 B = pad ? u32x4{0, 0, 0, 0} : wstep[(k * kTilesBf + q) * 64 + lane];
      st.acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, __builtin_bit_cast(bf16x8, B),
                                                          st.acc[q], 0, 0, 0);
    }
  }

  // sums of squares of the rounded new streams, and hc_pre
  u32x4 hpk = {0, 0, 0, 0};
  float ssa = 0.f, ssb = 0.f, hsa = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    float r0[4], r1[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      r0[k] = bf_lo(xo[k][w]);
      r1[k] = bf_hi(xo[k][w]);
      ssa = fmaf(r0[k], r0[k], ssa);
      ssb = fmaf(r1[k], r1[k], ssb);
    }
    if (MODE == kFused) {
      float h0 = st.P[0] * r0[0], h1 = st.P[0] * r1[0];
#pragma unroll
      for (int k = 1; k < 4; ++k) {
        h0 = fmaf(st.P[k], r0[k], h0);
        h1 = fmaf(st.P[k], r1[k], h1);
      }
      const uint32_t hp = pack_bf16x2(h0, h1);
      hpk[w] = hp;
      const float q0 = bf_lo(hp), q1 = bf_hi(hp);
      hsa = fmaf(q0, q0, hsa);
      hsa = fmaf(q1, q1, hsa);
    }
  }
  st.ss += ssa + ssb;
  st.hs += hsa;
  return hpk;
}

// y = bf16(gamma * (h * rh)) for the lane's 8 features ([RN] RMSNorm: the
// normalised value first, then the gain).
__device__ __forceinline__ u32x4 norm_bf(u32x4 hpk, const float* gamma, int f0, float rh) {
  const f32x4 g0 = *reinterpret_cast<const f32x4*>(gamma + f0);
  const f32x4 g1 = *reinterpret_cast<const f32x4*>(gamma + f0 + 4);
  const float gv[8] = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};
  u32x4 y;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float a = gv[2 * w] * (bf_lo(hpk[w]) * rh);
    const float b = gv[2 * w + 1] * (bf_hi(hpk[w]) * rh);
    y[w] = pack_bf16x2(a, b);
  }
  return y;
}

// ----- f32 streams ----------------------------------------------------------------------

struct InF {
  u32x4 x[4][2];
  u32x4 f[2];
};

template <int MODE>
__device__ __forceinline__ void load_f(InF& in, const float* xrow, const float* frow, int d,
                                       int f0, bool valid) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if (valid) {
#pragma unroll
      for (int j = 0; j < 4; ++j) in.x[j][h] = ld16(xrow + (size_t)j * d + f0 + 4 * h);
      in.f[h] = MODE == kFused ? ld16(frow + f0 + 4 * h) : u32x4{0, 0, 0, 0};
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) in.x[j][h] = u32x4{0, 0, 0, 0};
      in.f[h] = u32x4{0, 0, 0, 0};
    }
  }
}

// f32 variant of step_bf: the projection uses v_mfma_f32_16x16x4_f32 (one K
// value per lane per instruction, eight instructions per stream and tile) on
// the float32 weights; h goes to the y buffer as scratch.
template <int MODE>
__device__ __forceinline__ void step_f(const InF& in, LaneState<kTilesF>& st,
                                       const u32x4* __restrict__ wstep, int lane, float* xorow,
                                       float* hrow, int d, int f0, bool valid) {
  float xr[4][8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float a[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] = __uint_as_float(in.x[j][e >> 2][e & 3]);
    if (MODE == kFused) {
      const float fv = __uint_as_float(in.f[e >> 2][e & 3]);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float v = a[0] * st.C[0][k];
#pragma unroll
        for (int j = 1; j < 4; ++j) v = fmaf(a[j], st.C[j][k], v);
        xr[k][e] = fmaf(fv, st.U[k], v);
      }
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) xr[k][e] = a[k];
    }
  }
  if (MODE == kFused && valid) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        st16(xorow + (size_t)k * d + f0 + 4 * h,
             u32x4{__float_as_uint(xr[k][4 * h]), __float_as_uint(xr[k][4 * h + 1]),
                   __float_as_uint(xr[k][4 * h + 2]), __float_as_uint(xr[k][4 * h + 3])});
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
#pragma unroll
    for (int q = 0; q < kTilesF; ++q) {
      const u32x4* wp = wstep + ((k * kTilesF + q) * 64 + lane) * 2;
      const u32x4 b0 = wp[0], b1 = wp[1];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float B = __uint_as_float(e < 4 ? b0[e] : b1[e - 4]);
        st.acc[q] = __builtin_amdgcn_mfma_f32_16x16x4f32(xr[k][e], B, st.acc[q], 0, 0, 0);
      }
    }
  }
  float ss = 0.f, hs = 0.f;
  float hv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
#pragma unroll
    for (int k = 0; k < 4; ++k) ss = fmaf(xr[k][e], xr[k][e], ss);
    if (MODE == kFused) {
      float h = st.P[0] * xr[0][e];
#pragma unroll
      for (int k = 1; k < 4; ++k) h = fmaf(st.P[k], xr[k][e], h);
      hv[e] = h;
      hs = fmaf(h, h, hs);
    }
  }
  if (MODE == kFused && valid) {
    st16(hrow + f0, u32x4{__float_as_uint(hv[0]), __float_as_uint(hv[1]), __float_as_uint(hv[2]),
                          __float_as_uint(hv[3])});
    st16(hrow + f0 + 4, u32x4{__float_as_uint(hv[4]), __float_as_uint(hv[5]),
                              __float_as_uint(hv[6]), __float_as_uint(hv[7])});
  }
  st.ss += ss;
  st.hs += hs;
}

// ----- the step kernel ------------------------------------------------------------------

template <int DT, int MODE, bool HREG>
__global__ __launch_bounds__(kThreads) void step_kernel(StepArgs a) {
  constexpr bool kBf = (DT == MHC_BF16);
  constexpr int kTiles = kBf ? kTilesBf : kTilesF;

  __shared__ float red_acc[kWaves][kTok][kColsMax];
  __shared__ float red_ss[kWaves][kTok];
  __shared__ float red_hs[kWaves][kTok];
  __shared__ float m_lds[kTok][kMix];
  __shared__ float rh_lds[kTok];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int tr = lane & 15;
  const int g = lane >> 4;
  const int64_t t0 = (int64_t)blockIdx.x * kTok;
  const int64_t t = t0 + tr;
  const bool valid = t < a.tokens;
  const int d = a.d;
  const int nsteps = d / kStep;
  const int cnt = wave < nsteps ? (nsteps - wave + kWaves - 1) / kWaves : 0;

  LaneState<kTiles> st;
#pragma unroll
  for (int q = 0; q < kTiles; ++q) st.acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.ss = 0.f;
  st.hs = 0.f;
  if (MODE == kFused) {
    if (valid) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 c = *reinterpret_cast<const f32x4*>(a.comb_in + t * 16 + 4 * j);
#pragma unroll
        for (int k = 0; k < 4; ++k) st.C[j][k] = c[k];
      }
      const f32x4 u = *reinterpret_cast<const f32x4*>(a.post_in + t * 4);
      const f32x4 p = *reinterpret_cast<const f32x4*>(a.pre_in + t * 4);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        st.U[k] = u[k];
        st.P[k] = p[k];
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int k = 0; k < 4; ++k) st.C[j][k] = 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) st.U[k] = st.P[k] = 0.f;
    }
  }

  const float rh_unused = 0.f;
  (void)rh_unused;

  if constexpr (kBf) {
    const uint16_t* xrow = static_cast<const uint16_t*>(a.x) + t * kStreams * (int64_t)d;
    const uint16_t* frow = static_cast<const uint16_t*>(a.f) + t * (int64_t)d;
    uint16_t* xorow = static_cast<uint16_t*>(a.x_out) + t * kStreams * (int64_t)d;
    uint16_t* yrow = static_cast<uint16_t*>(a.y_out) + t * (int64_t)d;
    const u32x4* wpk = static_cast<const u32x4*>(a.wpk);
    const size_t wstride = (size_t)kStreams * kTilesBf * 64;   // u32x4 per step

    InBf cur, nxt;
    if (cnt > 0) load_bf<MODE>(cur, xrow, frow, d, wave * kStep + g * 8, valid);
    if constexpr (HREG) {
      u32x4 hb[kMaxSpw];
#pragma unroll
      for (int i = 0; i < kMaxSpw; ++i) {
        if (i < cnt) {
          const int s = wave + kWaves * i;
          const int f0 = s * kStep + g * 8;
          if (i + 1 < cnt) load_bf<MODE>(nxt, xrow, frow, d, f0 + kWaves * kStep, valid);
          hb[i] = step_bf<MODE>(cur, st, wpk + (size_t)s * wstride, lane, xorow, d, f0, valid);
          cur = nxt;
        }
      }
      // ---- reduction + tail (shared code below via lambda-free duplication) ----
      float ss = st.ss, hs = st.hs;
      ss += __shfl_xor(ss, 16);
      ss += __shfl_xor(ss, 32);
      hs += __shfl_xor(hs, 16);
      hs += __shfl_xor(hs, 32);
      if (g == 0) {
        red_ss[wave][tr] = ss;
        red_hs[wave][tr] = hs;
      }
#pragma unroll
      for (int q = 0; q < kTiles; ++q)
#pragma unroll
        for (int r = 0; r < 4; ++r) red_acc[wave][4 * g + r][16 * q + tr] = st.acc[q][r];
      __syncthreads();
      if (tid < kTok) {
        float hsum = 0.f;
        for (int w = 0; w < kWaves; ++w) hsum += red_hs[w][tid];
        rh_lds[tid] = rsqrtf(hsum / (float)d + a.norm_eps);
      }
      __syncthreads();
      if (MODE == kFused) {
        const float rh = rh_lds[tr];
#pragma unroll
        for (int i = 0; i < kMaxSpw; ++i) {
          if (i < cnt && valid) {
            const int f0 = (wave + kWaves * i) * kStep + g * 8;
            sts16(yrow + f0, norm_bf(hb[i], a.gamma, f0, rh));
          }
        }
      }
    } else {
      for (int i = 0; i < cnt; ++i) {
        const int s = wave + kWaves * i;
        const int f0 = s * kStep + g * 8;
        if (i + 1 < cnt) load_bf<MODE>(nxt, xrow, frow, d, f0 + kWaves * kStep, valid);
        const u32x4 h = step_bf<MODE>(cur, st, wpk + (size_t)s * wstride, lane, xorow, d, f0, valid);
        if (MODE == kFused && valid) st16(yrow + f0, h);   // h parked in y until rh is known
        cur = nxt;
      }
      float ss = st.ss, hs = st.hs;
      ss += __shfl_xor(ss, 16);
      ss += __shfl_xor(ss, 32);
      hs += __shfl_xor(hs, 16);
      hs += __shfl_xor(hs, 32);
      if (g == 0) {
        red_ss[wave][tr] = ss;
        red_hs[wave][tr] = hs;
      }
#pragma unroll
      for (int q = 0; q < kTiles; ++q)
#pragma unroll
        for (int r = 0; r < 4; ++r) red_acc[wave][4 * g + r][16 * q + tr] = st.acc[q][r];
      __syncthreads();
      if (tid < kTok) {
        float hsum = 0.f;
        for (int w = 0; w < kWaves; ++w) hsum += red_hs[w][tid];
        rh_lds[tid] = rsqrtf(hsum / (float)d + a.norm_eps);
      }
      __syncthreads();
      if (MODE == kFused) {
        const float rh = rh_lds[tr];
        for (int i = 0; i < cnt; ++i) {
          if (valid) {
            const int f0 = (wave + kWaves * i) * kStep + g * 8;
            st16(yrow + f0, norm_bf(ld16(yrow + f0), a.gamma, f0, rh));
          }
        }
      }
    }
  } else {
    const float* xrow = static_cast<const float*>(a.x) + t * kStreams * (int64_t)d;
    const float* frow = static_cast<const float*>(a.f) + t * (int64_t)d;
    float* xorow = static_cast<float*>(a.x_out) + t * kStreams * (int64_t)d;
    float* yrow = static_cast<float*>(a.y_out) + t * (int64_t)d;
    const u32x4* wpk = static_cast<const u32x4*>(a.wpk);
    const size_t wstride = (size_t)kStreams * kTilesF * 64 * 2;   // u32x4 per step

    InF cur, nxt;
    if (cnt > 0) load_f<MODE>(cur, xrow, frow, d, wave * kStep + g * 8, valid);
    for (int i = 0; i < cnt; ++i) {
      const int s = wave + kWaves * i;
      const int f0 = s * kStep + g * 8;
      if (i + 1 < cnt) load_f<MODE>(nxt, xrow, frow, d, f0 + kWaves * kStep, valid);
      step_f<MODE>(cur, st, wpk + (size_t)s * wstride, lane, xorow, yrow, d, f0, valid);
      cur = nxt;
    }
    float ss = st.ss, hs = st.hs;
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    hs += __shfl_xor(hs, 16);
    hs += __shfl_xor(hs, 32);
    if (g == 0) {
      red_ss[wave][tr] = ss;
      red_hs[wave][tr] = hs;
    }
#pragma unroll
    for (int q = 0; q < kTiles; ++q)
#pragma unroll
      for (int r = 0; r < 4; ++r) red_acc[wave][4 * g + r][16 * q + tr] = st.acc[q][r];
    __syncthreads();
    if (tid < kTok) {
      float hsum = 0.f;
      for (int w = 0; w < kWaves; ++w) hsum += red_hs[w][tid];
      rh_lds[tid] = rsqrtf(hsum / (float)d + a.norm_eps);
    }
    __syncthreads();
    if (MODE == kFused) {
      const float rh = rh_lds[tr];
      for (int i = 0; i < cnt; ++i) {
        if (valid) {
          const int f0 = (wave + kWaves * i) * kStep + g * 8;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const u32x4 hv = ld16(yrow + f0 + 4 * h);
            const f32x4 gv = *reinterpret_cast<const f32x4*>(a.gamma + f0 + 4 * h);
            u32x4 y;
#pragma unroll
            for (int e = 0; e < 4; ++e) y[e] = __float_as_uint(gv[e] * (__uint_as_float(hv[e]) * rh));
            st16(yrow + f0 + 4 * h, y);
          }
        }
      }
    }
  }

  // ---- mixes: total over waves, the three weight terms, times the RMS factor ----
  if (tid < kTok * kMix) {
    const int tt = tid / kMix;
    const int j = tid - tt * kMix;
    float ssum = 0.f;
    for (int w = 0; w < kWaves; ++w) ssum += red_ss[w][tt];
    const float r = rsqrtf(ssum / (float)(kStreams * d) + a.norm_eps);
    float mv;
    if (kBf) {
      float hi = 0.f, mid = 0.f, lo = 0.f;
      for (int w = 0; w < kWaves; ++w) {
        hi += red_acc[w][tt][j];
        mid += red_acc[w][tt][kMix + j];
        lo += red_acc[w][tt][2 * kMix + j];
      }
      mv = ((hi + mid) + lo) * r;
    } else {
      float s = 0.f;
      for (int w = 0; w < kWaves; ++w) s += red_acc[w][tt][j];
      mv = s * r;
    }
    m_lds[tt][j] = mv;
    if (a.mix_out != nullptr && t0 + tt < a.tokens) a.mix_out[(t0 + tt) * kMix + j] = mv;
  }
  __syncthreads();
  if (tid < kTok && t0 + tid < a.tokens) {
    const int64_t tt = t0 + tid;
    float pre[4], post[4], comb[16];
    split_sinkhorn_token(m_lds[tid], a.base, a.scale, a.iters, a.hc_eps, pre, post, comb);
    st4f(a.pre_out + tt * 4, f32x4{pre[0], pre[1], pre[2], pre[3]});
    st4f(a.post_out + tt * 4, f32x4{post[0], post[1], post[2], post[3]});
#pragma unroll
    for (int j = 0; j < 4; ++j)
      st4f(a.comb_out + tt * 16 + 4 * j,
           f32x4{comb[4 * j], comb[4 * j + 1], comb[4 * j + 2], comb[4 * j + 3]});
  }
}

// ----- pipelined bf16 kernel (d <= 5120) ------------------------------------------------
//
// Persistent workgroups of 8 waves (two per SIMD; one workgroup per CU because
// h fills the LDS) walk over 16-token tiles. The unit of work of a wave is a
// PAIR of adjacent 32-feature steps (64 features = one 128-byte line of every
// token row): wave w takes the pairs w, w+8, ... of the tile, so both halves of
// each line are loaded and stored by the same wave, back to back. The memory
// streams are software-pipelined by hand, because the vector-memory counter
// retires in issue order and a wait on a late-issued load would otherwise drain
// every earlier prefetch. Per pair (steps A and B):
//   1. projection operands of A (20 loads, L2)
//   2. [wait streams of A] hc_post, sums of squares, hc_pre for A; h to LDS
//   3. stream loads of the NEXT pair's A into the freed registers
//   4. [wait operands of A] 20 MFMAs
//   5. projection operands of B
//   6. [wait streams of B] VALU work of B
//   7. stream loads of the next pair's B; stores of A and B interleaved, so
//      every 128-byte line of the new streams is written by two adjacent
//      instructions
//   8. [wait operands of B] 20 MFMAs
// Stream tensors use buffer instructions whose range check drops the lanes of
// tokens past the end of the tensor (no branches), and the padding half of the
// last operand tile is read from outside the range, which returns zeros without
// memory traffic. h is kept in LDS (one 1 KB slot per step; the steps beyond the
// LDS capacity stay in registers) until the token's sum of squares is known.

namespace pipe {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kMaxSteps = 160;              // d <= 5120
constexpr int kSlots = kMaxSteps - kWaves;  // LDS slots for h
constexpr int kCols = 3 * kMix;             // real packed columns (hi/mid/lo x 24)
constexpr int kTiles = kTilesBf;            // column tiles per (step, stream) in the packing
// Tiles a chunked-kernel instance reads (the tile kernel reads all five):
// all of them (three terms, hi + mid + lo = w exactly) or the first three
// (hi + mid, |w - hi - mid| <= 2^-16 |w|, 40% fewer operand bytes from L2
// and MFMAs). Calls with a single Sinkhorn round take three terms: the comb's
// row sums are then not normalised and would carry the two-term error.
constexpr int kTilesHiMid = 3;
constexpr int used_cols(int T) { return T == kTiles ? 3 * kMix : 2 * kMix; }
constexpr uint32_t kRsrcWord3 = 0x00020000u;   // raw buffer, 32-bit data format (gfx9)
constexpr int kNT = 2;                         // cache-policy bit: non-temporal
constexpr uint32_t kOutOfRange = 0x80000000u;

constexpr int kStoreAux = 0;                   // cache policy of the tile kernels' stream stores

struct __align__(16) Smem {
  union {
    u32x4 h[kSlots][64];
    float acc[kWaves][kTok][kCols];
  } u;
  float ss[kWaves][kTok];
  float hs[kWaves][kTok];
};

typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, (int)kRsrcWord3);
}
template <int AUX>
__device__ __forceinline__ u32x4 bload(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, AUX));
}
template <int AUX>
__device__ __forceinline__ void bstore(rsrc_t r, uint32_t voff, uint32_t soff, u32x4 v) {
  store_pin();
  __builtin_amdgcn_raw_buffer_store_b128(
      __builtin_bit_cast(decltype(__builtin_amdgcn_raw_buffer_load_b128(r, 0, 0, 0)), v), r,
      (int)voff, (int)soff, AUX);
  store_guard(v);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// DPP controls: quad permutations and rotations inside a 16-lane row
constexpr int kQuadSwap1 = 0xB1;   // [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;   // [2,3,0,1]
constexpr int kRowRor4 = 0x124;
constexpr int kRowRor8 = 0x128;

__device__ __forceinline__ float quad_sum(float v) {
  v += dpp<kQuadSwap1>(v);
  return v + dpp<kQuadSwap2>(v);
}
__device__ __forceinline__ float quad_max(float v) {
  v = fmaxf(v, dpp<kQuadSwap1>(v));
  return fmaxf(v, dpp<kQuadSwap2>(v));
}
// sum over lanes e, e+4, e+8, e+12 of a 16-lane row
__device__ __forceinline__ float col_sum(float v) {
  v += dpp<kRowRor8>(v);
  return v + dpp<kRowRor4>(v);
}

struct Half {   // stream inputs of one 32-feature step
  u32x4 x[4];
  u32x4 f;
};

struct Ctx {
  rsrc_t xr, fr, xor_, yr, wr;
  uint32_t xoff, foff;   // lane byte offsets inside the tile's stream rows
  uint32_t woff, woff_last;
  int d2;                // d * 2 bytes (stream stride)
  float C[4][4], U[4], P[4];
  f32x4 acc[kTiles];
  float ss, hs;
  u32x4 hlast[2];
};

template <int MODE>
__device__ __forceinline__ void load_half(Half& hf, const Ctx& c, int s) {
  const uint32_t col = (uint32_t)s * 64;   // 32 features x 2 bytes
#pragma unroll
  for (int j = 0; j < 4; ++j) hf.x[j] = bload<kNT>(c.xr, c.xoff, col + (uint32_t)j * c.d2);
  hf.f = MODE == kFused ? bload<kNT>(c.fr, c.foff, col) : u32x4{0, 0, 0, 0};
}

template <int T>
__device__ __forceinline__ void load_w(u32x4 (&w)[4][T], const Ctx& c, int s) {
  const uint32_t base = (uint32_t)s * (kStreams * kTiles * 1024);
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int q = 0; q < T; ++q)
      w[k][q] = bload<0>(c.wr, q == T - 1 ? c.woff_last : c.woff,
                         base + (uint32_t)(k * kTiles + q) * 1024);
}

// hc_post, the sums of squares and hc_pre of one step (the arithmetic per
// element is that of step_bf); returns the lane's 8 values of h.
template <int MODE>
__device__ __forceinline__ u32x4 valu_core(const Half& in, u32x4 (&xo)[4], Ctx& c) {
  if (MODE == kFused) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float a0[4], a1[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        a0[j] = bf_lo(in.x[j][q]);
        a1[j] = bf_hi(in.x[j][q]);
      }
      const float f0v = bf_lo(in.f[q]), f1v = bf_hi(in.f[q]);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float v0 = a0[0] * c.C[0][k];
        float v1 = a1[0] * c.C[0][k];
#pragma unroll
        for (int j = 1; j < 4; ++j) {
          v0 = fmaf(a0[j], c.C[j][k], v0);
          v1 = fmaf(a1[j], c.C[j][k], v1);
        }
        v0 = fmaf(f0v, c.U[k], v0);
        v1 = fmaf(f1v, c.U[k], v1);
        xo[k][q] = pack_bf16x2(v0, v1);
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) xo[k] = in.x[k];
  }

  u32x4 hpk = {0, 0, 0, 0};
  float ssa = 0.f, ssb = 0.f, hsa = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float r0[4], r1[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      r0[k] = bf_lo(xo[k][q]);
      r1[k] = bf_hi(xo[k][q]);
      ssa = fmaf(r0[k], r0[k], ssa);
      ssb = fmaf(r1[k], r1[k], ssb);
    }
    if (MODE == kFused) {
      float h0 = c.P[0] * r0[0], h1 = c.P[0] * r1[0];
#pragma unroll
      for (int k = 1; k < 4; ++k) {
        h0 = fmaf(c.P[k], r0[k], h0);
        h1 = fmaf(c.P[k], r1[k], h1);
      }
      const uint32_t hp = pack_bf16x2(h0, h1);
      hpk[q] = hp;
      const float q0 = bf_lo(hp), q1 = bf_hi(hp);
      hsa = fmaf(q0, q0, hsa);
      hsa = fmaf(q1, q1, hsa);
    }
  }
  c.ss += ssa + ssb;
  c.hs += hsa;
  return hpk;
}

// valu_core, with h going to LDS slot s (or a register).
template <int MODE>
__device__ __forceinline__ void valu_step(const Half& in, u32x4 (&xo)[4], Ctx& c, Smem& sm, int s,
                                          int lane, int half) {
  const u32x4 hpk = valu_core<MODE>(in, xo, c);
  if (MODE == kFused) {
    if (s < kSlots) sm.u.h[s][lane] = hpk;
    else c.hlast[half] = hpk;
  }
}

template <int T>
__device__ __forceinline__ void mfma_step(const u32x4 (&xo)[4], const u32x4 (&w)[4][T],
                                          Ctx& c) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const bf16x8 A = __builtin_bit_cast(bf16x8, xo[k]);
#pragma unroll
    for (int q = 0; q < T; ++q)
      c.acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, __builtin_bit_cast(bf16x8, w[k][q]),
                                                         c.acc[q], 0, 0, 0);
  }
}

// One pair of steps (A = 2P, B = 2P + 1), prefetching the next pair's streams
// when the wave has one in this tile (the branch is uniform across the wave;
// the next tile's first pair is loaded by the tile set-up).
template <int MODE, int T>
__device__ __forceinline__ void pair_body(int p, int cnt, int wave, Ctx& c, Smem& sm, int lane,
                                          Half& ha, Half& hb) {
  const int sa = 2 * (wave + kWaves * p);
  const bool more = p + 1 < cnt;
  const int sn = sa + 2 * kWaves;   // the next pair
  u32x4 w[4][T];
  u32x4 xa[4], xb[4];

  load_w(w, c, sa);
  __builtin_amdgcn_sched_barrier(0);
  valu_step<MODE>(ha, xa, c, sm, sa, lane, 0);
  __builtin_amdgcn_sched_barrier(0);
  if (more) load_half<MODE>(ha, c, sn);
  __builtin_amdgcn_sched_barrier(0);
  mfma_step(xa, w, c);
  __builtin_amdgcn_sched_barrier(0);

  load_w(w, c, sa + 1);
  __builtin_amdgcn_sched_barrier(0);
  valu_step<MODE>(hb, xb, c, sm, sa + 1, lane, 1);
  __builtin_amdgcn_sched_barrier(0);
  if (more) load_half<MODE>(hb, c, sn + 1);
  if (MODE == kFused) {
    const uint32_t col = (uint32_t)sa * 64;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      bstore<kStoreAux>(c.xor_, c.xoff, col + (uint32_t)k * c.d2, xa[k]);
      bstore<kStoreAux>(c.xor_, c.xoff, col + 64 + (uint32_t)k * c.d2, xb[k]);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  mfma_step(xb, w, c);
  __builtin_amdgcn_sched_barrier(0);
}

template <int MODE>
__global__ __launch_bounds__(kThreads) void fused_bf16_kernel(StepArgs a, int ntiles) {
  constexpr int T = kTiles;   // all three terms of W
  __shared__ Smem sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tr = lane & 15;
  const int g = lane >> 4;
  const int d = a.d;
  const int nsteps = d / kStep;
  const int npairs = nsteps / 2;
  const int cnt = wave < npairs ? (npairs - wave + kWaves - 1) / kWaves : 0;

  Ctx c;
  c.d2 = d * 2;
  c.wr = make_rsrc(a.wpk, (uint32_t)nsteps * kStreams * kTiles * 1024);
  c.woff = (uint32_t)lane * 16;
  c.woff_last = (tr < kCols - 16 * (T - 1)) ? (uint32_t)lane * 16 : kOutOfRange;

  Half ha, hb;

  auto setup = [&](int tile) {
    const int64_t t0 = (int64_t)tile * kTok;
    const int ntok = (int)min((int64_t)kTok, a.tokens - t0);
    const uint32_t rowx = (uint32_t)(kStreams * d * 2), rowf = (uint32_t)(d * 2);
    c.xr = make_rsrc(static_cast<const char*>(a.x) + t0 * rowx, ntok * rowx);
    if (MODE == kFused) {
      c.fr = make_rsrc(static_cast<const char*>(a.f) + t0 * rowf, ntok * rowf);
      c.xor_ = make_rsrc(static_cast<char*>(a.x_out) + t0 * rowx, ntok * rowx);
      c.yr = make_rsrc(static_cast<char*>(a.y_out) + t0 * rowf, ntok * rowf);
    }
    c.xoff = (uint32_t)tr * rowx + (uint32_t)g * 16;
    c.foff = (uint32_t)tr * rowf + (uint32_t)g * 16;
    if (MODE == kFused) {
      const int64_t tc = t0 + min(tr, ntok - 1);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 cv = *reinterpret_cast<const f32x4*>(a.comb_in + tc * 16 + 4 * j);
#pragma unroll
        for (int k = 0; k < 4; ++k) c.C[j][k] = cv[k];
      }
      const f32x4 u = *reinterpret_cast<const f32x4*>(a.post_in + tc * 4);
      const f32x4 p = *reinterpret_cast<const f32x4*>(a.pre_in + tc * 4);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        c.U[k] = u[k];
        c.P[k] = p[k];
      }
    }
    if (cnt > 0) {
      load_half<MODE>(ha, c, 2 * wave);
      load_half<MODE>(hb, c, 2 * wave + 1);
    }
  };

  int tile = blockIdx.x;
  if (tile < ntiles) setup(tile);
  for (; tile < ntiles; tile += gridDim.x) {
    const int64_t t0 = (int64_t)tile * kTok;
    const int ntok = (int)min((int64_t)kTok, a.tokens - t0);
#pragma unroll
    for (int q = 0; q < T; ++q) c.acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
    c.ss = 0.f;
    c.hs = 0.f;
    c.hlast[0] = c.hlast[1] = u32x4{0, 0, 0, 0};

    for (int p = 0; p < cnt; ++p) pair_body<MODE, T>(p, cnt, wave, c, sm, lane, ha, hb);

    // keep what the tail needs; start the next tile's loads so they fly while
    // this tile's y, reductions and Sinkhorn run
    const rsrc_t yr = c.yr;
    const float hsum_part = c.hs, ssum_part = c.ss;
    f32x4 acc[T];
#pragma unroll
    for (int q = 0; q < T; ++q) acc[q] = c.acc[q];
    const u32x4 hlast0 = c.hlast[0], hlast1 = c.hlast[1];
    const uint32_t foff = c.foff;
    if (tile + (int)gridDim.x < ntiles) setup(tile + gridDim.x);

    // ---- sums of squares: over the four lane groups, then across waves ----
    float ss = ssum_part, hs = hsum_part;
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    hs += __shfl_xor(hs, 16);
    hs += __shfl_xor(hs, 32);
    if (g == 0) {
      sm.ss[wave][tr] = ss;
      sm.hs[wave][tr] = hs;
    }
    __syncthreads();

    // ---- y = bf16(gamma * (h * rh)) ([RN] RMSNorm), both halves of each line together ----
    if (MODE == kFused) {
      float hsum = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) hsum += sm.hs[w][tr];
      const float rh = rsqrtf(hsum / (float)d + a.norm_eps);
      for (int pp = 0; pp < cnt; ++pp) {
        const int sa = 2 * (wave + kWaves * pp);
        const u32x4 h0 = sa < kSlots ? sm.u.h[sa][lane] : hlast0;
        const u32x4 h1 = sa + 1 < kSlots ? sm.u.h[sa + 1][lane] : hlast1;
        const int f0 = sa * kStep + g * 8;
        const u32x4 y0 = norm_bf(h0, a.gamma, f0, rh);
        const u32x4 y1 = norm_bf(h1, a.gamma, f0 + kStep, rh);
        bstore<kNT>(yr, foff, (uint32_t)sa * 64, y0);
        bstore<kNT>(yr, foff, (uint32_t)sa * 64 + 64, y1);
      }
      __syncthreads();
    }

    // ---- projection partials across waves ----
#pragma unroll
    for (int q = 0; q < T; ++q) {
      const int col = 16 * q + tr;
      if (col < kCols) {
#pragma unroll
        for (int r = 0; r < 4; ++r) sm.u.acc[wave][4 * g + r][col] = acc[q][r];
      }
    }
    __syncthreads();

    // ---- per-token tail: one token per 16-lane row, one comb entry per lane ----
    if (tid < kTok * 16) {
      const int tt = tid >> 4;
      const int e = tid & 15;
      float ssum = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) ssum += sm.ss[w][tt];
      const float r = rsqrtf(ssum / (float)(kStreams * d) + a.norm_eps);
      auto mix_at = [&](int j) {
        float hi = 0.f, mid = 0.f, lo = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          hi += sm.u.acc[w][tt][j];
          mid += sm.u.acc[w][tt][kMix + j];
          lo += sm.u.acc[w][tt][2 * kMix + j];
        }
        return ((hi + mid) + lo) * r;
      };
      const float mc = mix_at(8 + e);                 // comb logit slot of (j, k) = (e/4, e%4)
      const float mp = mix_at(e < 8 ? e : 0);         // pre / post slot for e < 8
      const bool tok_ok = tt < ntok;
      const int64_t t = t0 + tt;
      if (tok_ok && a.mix_out != nullptr) {
        a.mix_out[t * kMix + 8 + e] = mc;
        if (e < 8) a.mix_out[t * kMix + e] = mp;
      }
      const float s0 = a.scale[0], s1 = a.scale[1], s2 = a.scale[2];
      const float eps = a.hc_eps;
      if (tok_ok && e < 4) a.pre_out[t * 4 + e] = sigmoidf(mp * s0 + a.base[e]) + eps;
      if (tok_ok && e >= 4 && e < 8)
        a.post_out[t * 4 + (e - 4)] = 2.0f * sigmoidf(mp * s1 + a.base[e]);
      float cv = mc * s2 + a.base[8 + e];
      cv = expf(cv - quad_max(cv));
      cv = cv / quad_sum(cv) + eps;
      cv = cv * __builtin_amdgcn_rcpf(col_sum(cv) + eps);
      for (int it = 1; it < a.iters; ++it) {
        cv = cv * __builtin_amdgcn_rcpf(quad_sum(cv) + eps);
        cv = cv * __builtin_amdgcn_rcpf(col_sum(cv) + eps);
      }
      if (tok_ok) a.comb_out[t * 16 + e] = cv;
    }
    __syncthreads();
  }
}

}  // namespace pipe

#include "split_kernel.h"
#include "chunk_kernel.h"
#include "unfused.h"
#include "general_n.h"
#include "split_n.h"
#include "backward.h"

// ----- packing of the projection --------------------------------------------------------

// bf16: one thread per (step s, stream k, tile q, lane) writes the lane's 8
// B-operand values: column n = 16q + lane%16 is term n/24 (hi, mid, lo) of
// projection row n%24; K slots are features 32s + 8(lane/16) + 0..7 of stream k.
// hi = bf16(w), mid = bf16(w - hi), lo = bf16(w - hi - mid); both differences
// are exact in float32 and hi + mid + lo == w.
__global__ __launch_bounds__(256) void pack_bf16_kernel(const float* __restrict__ w, int d,
                                                        int64_t total, u32x4* __restrict__ out) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  const int lane = (int)(idx & 63);
  int64_t r = idx >> 6;
  const int q = (int)(r % kTilesBf);
  r /= kTilesBf;
  const int k = (int)(r % kStreams);
  const int64_t s = r / kStreams;
  const int n = 16 * q + (lane & 15);
  const int g = lane >> 4;
  const int64_t c0 = (int64_t)k * d + s * kStep + 8 * g;
  float v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = 0.f;
  if (n < 3 * kMix) {
    const int row = n % kMix;
    const int part = n / kMix;
    const float* src = w + (int64_t)row * kStreams * d + c0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = src[e];
      const float hi = __uint_as_float(pack_bf16x2(x, 0.f) << 16);
      const float r1 = x - hi;
      const float mid = __uint_as_float(pack_bf16x2(r1, 0.f) << 16);
      const float r2 = r1 - mid;
      v[e] = part == 0 ? hi : (part == 1 ? mid : r2);
    }
  }
  st16(out + idx, u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                        pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])});
}

// f32: one thread per (s, k, q, lane) copies the lane's 8 float32 weights
// (row n = 16q + lane%16, zero for n >= 24).
__global__ __launch_bounds__(256) void pack_f32_kernel(const float* __restrict__ w, int d,
                                                       int64_t total, u32x4* __restrict__ out) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  const int lane = (int)(idx & 63);
  int64_t r = idx >> 6;
  const int q = (int)(r % kTilesF);
  r /= kTilesF;
  const int k = (int)(r % kStreams);
  const int64_t s = r / kStreams;
  const int n = 16 * q + (lane & 15);
  const int g = lane >> 4;
  const int64_t c0 = (int64_t)k * d + s * kStep + 8 * g;
  u32x4 o0 = {0, 0, 0, 0}, o1 = {0, 0, 0, 0};
  if (n < kMix) {
    const float* src = w + (int64_t)n * kStreams * d + c0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      o0[e] = __float_as_uint(src[e]);
      o1[e] = __float_as_uint(src[4 + e]);
    }
  }
  st16(out + 2 * idx, o0);
  st16(out + 2 * idx + 1, o1);
}

// ----- host side ------------------------------------------------------------------------

thread_local char g_last_error[512] = "";

mhc_status fail(mhc_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return s;
}

mhc_status ok() {
  g_last_error[0] = '\0';
  return MHC_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Span {
  const char* name;
  const void* p;
  uint64_t bytes;
};

bool overlaps(const Span& a, const Span& b) {
  if (a.p == nullptr || b.p == nullptr || a.bytes == 0 || b.bytes == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

int elem_size(int32_t dtype) { return dtype == MHC_BF16 ? 2 : (dtype == MHC_F32 ? 4 : 0); }

mhc_status check_common(int32_t dtype, int64_t tokens, int32_t d, int32_t iters, float norm_eps,
                        float hc_eps) {
  if (dtype != MHC_BF16 && dtype != MHC_F32) return fail(MHC_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (tokens < 0) return fail(MHC_ERR_INVALID_ARG, "tokens must be >= 0 (got %lld)", (long long)tokens);
  if (d <= 0 || d % kStep != 0)
    return fail(MHC_ERR_INVALID_ARG, "d must be a positive multiple of %d (got %d)", kStep, d);
  if (iters < 1) return fail(MHC_ERR_INVALID_ARG, "sinkhorn_iters must be >= 1 (got %d)", iters);
  if (!(norm_eps >= 0.f) || !isfinite(norm_eps))
    return fail(MHC_ERR_INVALID_ARG, "norm_eps must be finite and >= 0");
  if (!(hc_eps >= 0.f) || !isfinite(hc_eps))
    return fail(MHC_ERR_INVALID_ARG, "hc_eps must be finite and >= 0");
  // element offsets of the stream tensors are computed in 64 bits; the grid
  // has one workgroup per 16 tokens
  if (tokens > ((int64_t)1 << 35))
    return fail(MHC_ERR_UNSUPPORTED, "tokens beyond 2^35 are not supported");
  return MHC_OK;
}

mhc_status check_spans(const Span* in, int nin, const Span* out, int nout, const void* inplace_a,
                       const void* inplace_b) {
  for (int i = 0; i < nin; ++i)
    if (in[i].p == nullptr) return fail(MHC_ERR_INVALID_ARG, "%s is NULL", in[i].name);
  for (int i = 0; i < nout; ++i)
    if (out[i].p == nullptr) return fail(MHC_ERR_INVALID_ARG, "%s is NULL", out[i].name);
  for (int i = 0; i < nin; ++i)
    if (!aligned16(in[i].p)) return fail(MHC_ERR_INVALID_ARG, "%s is not 16-byte aligned", in[i].name);
  for (int i = 0; i < nout; ++i)
    if (!aligned16(out[i].p))
      return fail(MHC_ERR_INVALID_ARG, "%s is not 16-byte aligned", out[i].name);
  for (int i = 0; i < nout; ++i) {
    for (int j = i + 1; j < nout; ++j)
      if (overlaps(out[i], out[j]))
        return fail(MHC_ERR_INVALID_ARG, "outputs %s and %s overlap", out[i].name, out[j].name);
    for (int j = 0; j < nin; ++j) {
      if (out[i].p == inplace_a && in[j].p == inplace_b && out[i].bytes == in[j].bytes) continue;
      if (overlaps(out[i], in[j]))
        return fail(MHC_ERR_INVALID_ARG, "output %s overlaps input %s", out[i].name, in[j].name);
    }
  }
  return MHC_OK;
}

// A workspace of `given` bytes for a route that needs `need`: large enough,
// 256-byte aligned and overlapping none of the call's other buffers.
mhc_status check_workspace(const void* ws, int64_t given, int64_t need, const Span* others,
                           int nothers) {
  if (given < need)
    return fail(MHC_ERR_INVALID_ARG, "workspace holds %lld bytes, %lld needed", (long long)given,
                (long long)need);
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
    return fail(MHC_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
  const Span wsp[] = {{"workspace", ws, (uint64_t)need}};
  return check_spans(others, nothers, wsp, 1, nullptr, nullptr);
}

mhc_status launch_status(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MHC_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

int64_t packed_bytes(int32_t d, int32_t dtype) {
  if (d <= 0 || d % kStep != 0) return -1;
  const int64_t steps = d / kStep;
  if (dtype == MHC_BF16) return steps * kStreams * kTilesBf * 64 * 16;
  if (dtype == MHC_F32) return steps * kStreams * kTilesF * 64 * 32;
  return -1;
}

typedef void (*StepKernel)(StepArgs);

StepKernel pick_step_kernel(int32_t dtype, int mode, int32_t d) {
  const int nsteps = d / kStep;
  const bool hreg = (nsteps + kWaves - 1) / kWaves <= kMaxSpw;
  if (dtype == MHC_BF16) {
    if (mode == kMixesOnly) return step_kernel<MHC_BF16, kMixesOnly, false>;
    return hreg ? step_kernel<MHC_BF16, kFused, true> : step_kernel<MHC_BF16, kFused, false>;
  }
  if (mode == kMixesOnly) return step_kernel<MHC_F32, kMixesOnly, false>;
  return step_kernel<MHC_F32, kFused, false>;
}

// Compute units of the current device (cached per device ordinal; threads
// that race here store the same value).
mhc_status device_cu_count(int* out) {
  static std::atomic<int> cache[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MHC_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev >= 0 && dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *out = c;
      return MHC_OK;
    }
  }
  int n = 0;
  e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess || n <= 0)
    return fail(MHC_ERR_HIP, "hipDeviceGetAttribute(multiprocessor count): %s", hipGetErrorString(e));
  if (dev >= 0 && dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  *out = n;
  return MHC_OK;
}

// Feature-split kernel geometry: `ns` workgroups per group, each owning S = d/ns
// features, and `groups` groups (one workgroup per compute unit). For large
// calls, slices of a multiple of 64 features (128-byte aligned rows, no
// 32-feature tail) are preferred, then the most compute units in use, then
// fewer slices (less exchange traffic). Calls of at most kSplitCostBatches
// 128-token batches take the geometry with the least estimated time
// (split_cost_us), which may be another one. groups = 0 when the kernel does
// not apply: bf16 streams, S in {64, 96, 128, 160}, at least `ns` compute
// units and cooperative launch support are required.

struct SplitCfg {
  int groups = 0;
  int ns = 0;
  int S = 0;      // 256: the two-term projection (hi + mid of W), else three terms
};

// Cooperative-launch support of the current device, cached per device
// ordinal (1 = no, 2 = yes).
mhc_status coop_supported(bool* ok) {
  static std::atomic<int> coop_cache[64];
  int dev = 0, coop = 0;
  hipError_t e = hipGetDevice(&dev);
  const int cached = (e == hipSuccess && dev >= 0 && dev < 64)
                         ? coop_cache[dev].load(std::memory_order_relaxed)
                         : 0;
  if (cached != 0) {
    coop = cached - 1;
  } else {
    if (e == hipSuccess)
      e = hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev);
    if (e != hipSuccess)
      return fail(MHC_ERR_HIP, "cooperative-launch attribute: %s", hipGetErrorString(e));
    if (dev >= 0 && dev < 64) coop_cache[dev].store(coop ? 2 : 1, std::memory_order_relaxed);
  }
  *ok = coop != 0;
  return MHC_OK;
}

// Estimated time of a feature-split call of `tokens` tokens, in microseconds:
// a fixed part plus a round time per round of the call's batches (whole
// rounds plus the last round's share of 128 tokens, see fsplit::BatchSpans),
// the round time proportional to the slice width (plus 4% for the 32-feature
// tail's 64-byte row pieces). Fitted to calls issued back to back (ordinary
// launch) at d = 5120 on the MI355X, 256 to 5,120 tokens: 15.9 us per round
// per 128 features; fixed 22.4 us, 25.5 us on 256-feature slices. For
// example, at 4,096 tokens 20 x 256 (12 groups: 2 whole rounds + 96 tokens),
// 32 x 160 (8 groups: 4 rounds) and 40 x 128 (6 groups: 5 rounds + 48)
// measured 108.9, 104.7 and 109.2 us, estimated 113.0, 105.1 and 107.9. At
// more tokens the rounds cost more as the device saturates, and the 256-
// feature slices are the fastest at every size measured from 6,144 tokens
// (8,192: 198.2 against 206.0 and 224.4 us).
constexpr int64_t kSplitCostBatches = 40;

double split_cost_us(const SplitCfg& c, int64_t tokens) {
  const fsplit::BatchSpans sp = fsplit::BatchSpans::make(tokens, c.groups);
  const double rounds = sp.full + sp.share / (double)fsplit::kBatch;
  const bool tail = c.S % 64 != 0;
  return (c.S == fsplit::kMaxSW ? 25.5 : 22.4) + 15.9 * c.S / 128.0 * (tail ? 1.04 : 1.0) * rounds;
}

// Every geometry the kernel can run for (dtype, d) on this device, the
// preferred one for large calls first: the 256-feature slices where d allows,
// then the best-scored narrow geometry, then the other narrow ones; none
// without cooperative launch support.
mhc_status split_candidates(int32_t dtype, int32_t d, SplitCfg (&out)[5], int* count) {
  *count = 0;
  if (dtype != MHC_BF16) return MHC_OK;
  int cus = 0;
  mhc_status s = device_cu_count(&cus);
  if (s != MHC_OK) return s;
  // 256-feature slices on the two-term projection: 512-byte row segments per
  // workgroup, half the exchange rows of 128-feature slices
  if (d % fsplit::kMaxSW == 0) {
    const int ns = d / fsplit::kMaxSW;
    if (ns >= 16 && ns <= fsplit::kMaxSlicesW && ns <= cus)
      out[(*count)++] = SplitCfg{cus / ns, ns, fsplit::kMaxSW};
  }
  const int first_narrow = *count;
  int best_score = -1;
  for (int ns : {32, 40, 48, 64}) {
    if (d % ns != 0 || ns > cus) continue;
    const int S = d / ns;
    if (S % 32 != 0 || S < 64 || S > fsplit::kMaxS) continue;
    const int used = (cus / ns) * ns;
    const int score = (S % 64 == 0 ? 1 << 20 : 0) + used * 64 + (64 - ns);
    out[*count] = SplitCfg{cus / ns, ns, S};
    if (score > best_score) {
      best_score = score;
      std::swap(out[first_narrow], out[*count]);
    }
    ++*count;
  }
  if (*count == 0) return MHC_OK;
  bool coop = false;
  if ((s = coop_supported(&coop)) != MHC_OK) return s;
  if (!coop) *count = 0;
  return MHC_OK;
}

// The geometry of a call of `tokens` tokens, and the workspace bytes that
// cover every candidate geometry at that size (so a workspace sized for T
// tokens serves every call of at most T tokens, whichever geometry it takes).
// one_round: the call runs a single Sinkhorn round. After one round nothing
// divides the comb's row sums back to 1, so the error of the two-term
// projection (|w - hi - mid| <= 2^-16 |w|, within the mixes' tolerance)
// reaches them undivided and put some of them just past the 1e-5 comb-sum
// tolerance (up to 1.1e-5 at 6,000 tokens); such calls take a geometry on the
// exact three-term projection where d has one. From two rounds on the row
// normalisations absorb it.
mhc_status split_config(int32_t dtype, int32_t d, int64_t tokens, SplitCfg* cfg,
                        int64_t* bytes, bool one_round = false) {
  *cfg = SplitCfg{};
  *bytes = 0;
  SplitCfg cand[5];
  int count = 0;
  const mhc_status s = split_candidates(dtype, d, cand, &count);
  if (s != MHC_OK || count == 0) return s;
  const int first = one_round && count > 1 && cand[0].S == fsplit::kMaxSW ? 1 : 0;
  *cfg = cand[first];
  const int64_t nbatch = (tokens + fsplit::kBatch - 1) / fsplit::kBatch;
  for (int i = 0; i < count; ++i) {
    *bytes = std::max(*bytes, fsplit::workspace_bytes(cand[i].groups, cand[i].ns, tokens));
    if (i >= first && nbatch <= kSplitCostBatches &&
        split_cost_us(cand[i], tokens) < split_cost_us(*cfg, tokens))
      *cfg = cand[i];
  }
  return MHC_OK;
}

// Launch of a feature-split kernel, whose workgroups wait for the others of
// their group: as an ordinary kernel (the default: the groups are filled in
// start order, so the kernel finishes whenever the device can eventually hold
// one group at once), or, with MHC_PATH_COOPERATIVE, cooperatively (the
// runtime runs it alone on the device, all workgroups resident, at the price
// of about 11 us of device idle before and after it).
hipError_t launch_resident(const void* fn, unsigned grid, void** params, bool plain,
                           hipStream_t stream) {
  if (plain) return hipLaunchKernel(fn, dim3(grid), dim3(fsplit::kThreads), params, 0, stream);
  return hipLaunchCooperativeKernel(fn, dim3(grid), dim3(fsplit::kThreads), params, 0, stream);
}

// The feature-split kernel (it leaves the workspace header as it found it, see
// split_kernel.h), then the split/Sinkhorn of its mixes rows.
mhc_status launch_split(const StepArgs& a, void* ws, const SplitCfg& cfg, int mode, bool plain,
                        hipStream_t stream) {
  if (fsplit::ctr_off(cfg.groups, 0) > fsplit::kWsHeader)
    return fail(MHC_ERR_UNSUPPORTED, "feature-split kernel: %d groups exceed the header", cfg.groups);
  mhc_status s = MHC_OK;
  float* mix = a.mix_out != nullptr
                   ? a.mix_out
                   : reinterpret_cast<float*>(static_cast<char*>(ws) + fsplit::mix_off(cfg.groups, cfg.ns));
  fsplit::Args fs{static_cast<char*>(ws), mix, cfg.groups, cfg.ns,
                  fsplit::BatchSpans::make(a.tokens, cfg.groups)};
  StepArgs args = a;
  void* params[] = {&args, &fs};
  const void* fn = nullptr;
  const bool full = mode == kFused;
  switch (cfg.S) {
    case 64:
      fn = full ? reinterpret_cast<const void*>(fsplit::split_kernel<1, false, kFused, 3>)
                : reinterpret_cast<const void*>(fsplit::split_kernel<1, false, kMixesOnly, 3>);
      break;
    case 96:
      fn = full ? reinterpret_cast<const void*>(fsplit::split_kernel<1, true, kFused, 3>)
                : reinterpret_cast<const void*>(fsplit::split_kernel<1, true, kMixesOnly, 3>);
      break;
    case 128:
      fn = full ? reinterpret_cast<const void*>(fsplit::split_kernel<2, false, kFused, 3>)
                : reinterpret_cast<const void*>(fsplit::split_kernel<2, false, kMixesOnly, 3>);
      break;
    case 160:
      fn = full ? reinterpret_cast<const void*>(fsplit::split_kernel<2, true, kFused, 3>)
                : reinterpret_cast<const void*>(fsplit::split_kernel<2, true, kMixesOnly, 3>);
      break;
    case fsplit::kMaxSW:
      fn = full ? reinterpret_cast<const void*>(fsplit::split_kernel<4, false, kFused, 2>)
                : reinterpret_cast<const void*>(fsplit::split_kernel<4, false, kMixesOnly, 2>);
      break;
    default: return fail(MHC_ERR_UNSUPPORTED, "feature-split kernel: slice of %d features", cfg.S);
  }
  const hipError_t e = launch_resident(fn, (unsigned)(cfg.groups * cfg.ns), params, plain, stream);
  if (e != hipSuccess)
    return fail(MHC_ERR_HIP, "feature-split kernel launch: %s", hipGetErrorString(e));
  s = launch_status("feature-split kernel launch");
  if (s != MHC_OK) return s;
  hipLaunchKernelGGL(fsplit::tail_kernel,
                     dim3((unsigned)((a.tokens + fsplit::kTailThreads - 1) / fsplit::kTailThreads)),
                     dim3(fsplit::kTailThreads), 0, stream, mix, a.tokens, a.base, a.scale, a.iters, a.hc_eps, a.pre_out,
                     a.post_out, a.comb_out);
  return launch_status("split/Sinkhorn tail kernel launch");
}

// Chunked small-batch path, at most kChunkMaxTokens tokens (the partial rows
// take 128 bytes per token and chunk): bf16 streams with an even number of
// 32-feature steps, at most the pipelined kernel's 160, in chunks of
// kChunkPairs pairs of steps (one pair per wave); f32 streams with any
// number of steps, in chunks of kChunkStepsF steps (one per wave; 16 steps,
// two per wave, took 37.3 against 29.2 us on 64 tokens at d = 5120).
constexpr int kChunkPairs = 8;
// Largest call that path "auto" runs on the chunked kernels (when a workspace
// is given); larger calls take the feature-split kernel. At d = 5120 the
// two routes' call time (cache-flushed medians; the split route with its
// cooperative-launch gaps) is about 16.5 + 0.0355 T and 45.6 + 0.0243 T
// microseconds: equal near 2,600 tokens. Launched as an ordinary kernel (the
// default) the split route loses about 20 us per call; back to back the
// chunks then win up to 768 tokens (37.3 against 39.8 us) and the split
// kernel from 1,024 (46.0 against 48.2): equal near 900 tokens.
constexpr int64_t kChunkAutoTokensCoop = 2048;
constexpr int64_t kChunkAutoTokensPlain = 896;
constexpr int64_t kChunkMaxTokens = 8192;

constexpr int kChunkStepsF = 8;

struct ChunkCfg {
  int nchunks = 0;
  int per = 0;     // pairs of steps (bf16) or steps (f32) per chunk
  int32_t dtype = MHC_BF16;
};

ChunkCfg chunk_config(int32_t dtype, int32_t d, int64_t tokens) {
  const int nsteps = d / kStep;
  if (d <= 0 || d % kStep != 0 || tokens > kChunkMaxTokens) return ChunkCfg{};
  if (dtype == MHC_BF16) {
    if (nsteps % 2 != 0 || nsteps > pipe::kMaxSteps) return ChunkCfg{};
    const int npairs = nsteps / 2;
    const int cp = std::min(kChunkPairs, npairs);
    return ChunkCfg{(npairs + cp - 1) / cp, cp, dtype};
  }
  if (dtype == MHC_F32) {
    const int cs = std::min(kChunkStepsF, nsteps);
    return ChunkCfg{(nsteps + cs - 1) / cs, cs, dtype};
  }
  return ChunkCfg{};
}

mhc_status launch_chunk(const StepArgs& a, void* ws, const ChunkCfg& cc, int mode,
                        hipStream_t stream) {
  const unsigned grid = (unsigned)pipe::chunk_grid((a.tokens + kTok - 1) / kTok, cc.nchunks);
  const dim3 blk(pipe::kThreads), tok((unsigned)a.tokens);
  char* w = static_cast<char*>(ws);
  const bool bf = cc.dtype == MHC_BF16, full = mode == kFused;
  // three projection terms for a single Sinkhorn round, else hi + mid (pipe::used_cols)
  const bool exact = a.iters == 1;
  constexpr int T3 = pipe::kTiles, T2 = pipe::kTilesHiMid;
  if (bf && full && exact)
    hipLaunchKernelGGL((pipe::chunk_kernel<kFused, T3>), dim3(grid), blk, 0, stream, a,
                       cc.nchunks, cc.per, w);
  else if (bf && full)
    hipLaunchKernelGGL((pipe::chunk_kernel<kFused, T2>), dim3(grid), blk, 0, stream, a,
                       cc.nchunks, cc.per, w);
  else if (bf && exact)
    hipLaunchKernelGGL((pipe::chunk_kernel<kMixesOnly, T3>), dim3(grid), blk, 0, stream, a,
                       cc.nchunks, cc.per, w);
  else if (bf)
    hipLaunchKernelGGL((pipe::chunk_kernel<kMixesOnly, T2>), dim3(grid), blk, 0, stream, a,
                       cc.nchunks, cc.per, w);
  else if (full)
    hipLaunchKernelGGL(pipe::chunk_f32_kernel<kFused>, dim3(grid), blk, 0, stream, a, cc.nchunks,
                       cc.per, w);
  else
    hipLaunchKernelGGL(pipe::chunk_f32_kernel<kMixesOnly>, dim3(grid), blk, 0, stream, a,
                       cc.nchunks, cc.per, w);
  mhc_status s = launch_status("chunk kernel launch");
  if (s != MHC_OK) return s;
  if (bf && full)
    hipLaunchKernelGGL((pipe::chunk_finish_kernel<kFused, MHC_BF16>), tok, dim3(256), 0, stream, a,
                       cc.nchunks, w);
  else if (full)
    hipLaunchKernelGGL((pipe::chunk_finish_kernel<kFused, MHC_F32>), tok, dim3(256), 0, stream, a,
                       cc.nchunks, w);
  else
    hipLaunchKernelGGL((pipe::chunk_finish_kernel<kMixesOnly, MHC_BF16>), tok, dim3(256), 0,
                       stream, a, cc.nchunks, w);
  return launch_status("chunk finish kernel launch");
}

// Which kernel family runs a fused step or mixes call: the tile kernel (no
// workspace), the feature-split kernel or the chunked kernels (workspace).
enum class Route { kTile, kSplit, kChunk };

// Workspace bytes each workspace route needs (0: the route does not apply).
struct RouteNeeds {
  SplitCfg split;
  ChunkCfg chunk;
  int64_t split_bytes = 0;
  int64_t chunk_bytes = 0;
};

mhc_status route_needs(int32_t dtype, int32_t d, int64_t tokens, RouteNeeds* rn,
                       bool one_round = false) {
  *rn = RouteNeeds{};
  mhc_status s = split_config(dtype, d, tokens, &rn->split, &rn->split_bytes, one_round);
  if (s != MHC_OK) return s;
  rn->chunk = chunk_config(dtype, d, tokens);
  if (rn->chunk.nchunks > 0) rn->chunk_bytes = pipe::chunk_workspace_bytes(rn->chunk.nchunks, tokens);
  return MHC_OK;
}

// The route of a call with `path` and a workspace (or none), or an error for
// a path that cannot run these arguments.
mhc_status pick_route(int32_t path, const void* workspace, int64_t tokens, int64_t split_bytes,
                      int64_t chunk_bytes, Route* r, int64_t chunk_auto = kChunkAutoTokensCoop) {
  switch (path) {
    case MHC_PATH_TILE:
      *r = Route::kTile;
      return MHC_OK;
    case MHC_PATH_AUTO:
      if (workspace == nullptr) *r = Route::kTile;
      else if (chunk_bytes > 0 && tokens <= chunk_auto) *r = Route::kChunk;
      else if (split_bytes > 0) *r = Route::kSplit;
      else *r = Route::kTile;
      return MHC_OK;
    case MHC_PATH_SPLIT:
    case MHC_PATH_CHUNK: {
      const bool split = path == MHC_PATH_SPLIT;
      if ((split ? split_bytes : chunk_bytes) == 0)
        return fail(MHC_ERR_UNSUPPORTED, "the %s kernel does not apply to these arguments",
                    split ? "feature-split" : "chunked");
      if (workspace == nullptr)
        return fail(MHC_ERR_INVALID_ARG, "path %s needs a workspace", split ? "SPLIT" : "CHUNK");
      *r = split ? Route::kSplit : Route::kChunk;
      return MHC_OK;
    }
    default: return fail(MHC_ERR_INVALID_ARG, "unknown path %d", path);
  }
}

// The kernel family of `path` (the launch flags taken out) and whether the
// feature-split kernel is launched as an ordinary kernel (no
// MHC_PATH_COOPERATIVE). Both launch flags at once: -1, an unknown path.
int32_t path_family(int32_t path, bool* plain) {
  *plain = (path & MHC_PATH_COOPERATIVE) == 0;
  if ((path & MHC_PATH_COOPERATIVE) != 0 && (path & MHC_PATH_PLAIN_LAUNCH) != 0) return -1;
  return path & ~(MHC_PATH_PLAIN_LAUNCH | MHC_PATH_COOPERATIVE);
}

// pick_route, querying the device only when a workspace route is possible.
// `path` may carry MHC_PATH_COOPERATIVE, which raises auto's switch to the
// feature-split kernel (*plain reports the launch). iters: the call's Sinkhorn
// rounds (a single round picks a three-term slice geometry, see split_config).
mhc_status choose_route(int32_t path, const void* workspace, int32_t dtype, int32_t d,
                        int64_t tokens, RouteNeeds* rn, Route* r, bool* plain,
                        int32_t iters = 0) {
  path = path_family(path, plain);
  *rn = RouteNeeds{};
  if (path == MHC_PATH_TILE || (path == MHC_PATH_AUTO && workspace == nullptr)) {
    *r = Route::kTile;
    return MHC_OK;
  }
  if (path == MHC_PATH_AUTO || path == MHC_PATH_SPLIT || path == MHC_PATH_CHUNK) {
    const mhc_status s = route_needs(dtype, d, tokens, rn, iters == 1);
    if (s != MHC_OK) return s;
  }
  const bool lower = *plain && rn->split_bytes > 0;   // only where the split kernel runs
  return pick_route(path, workspace, tokens, rn->split_bytes, rn->chunk_bytes, r,
                    lower ? kChunkAutoTokensPlain : kChunkAutoTokensCoop);
}

mhc_status launch_step(const StepArgs& a, int32_t dtype, int mode, hipStream_t stream,
                       const char* what) {
  const int nsteps = a.d / kStep;
  const int64_t ntiles = (a.tokens + kTok - 1) / kTok;
  if (dtype == MHC_BF16 && nsteps <= pipe::kMaxSteps && nsteps % 2 == 0) {
    int cus = 0;
    const mhc_status s = device_cu_count(&cus);
    if (s != MHC_OK) return s;
    const unsigned grid = (unsigned)std::min<int64_t>(ntiles, cus);
    if (mode == kFused)
      hipLaunchKernelGGL(pipe::fused_bf16_kernel<kFused>, dim3(grid), dim3(pipe::kThreads), 0,
                         stream, a, (int)ntiles);
    else
      hipLaunchKernelGGL(pipe::fused_bf16_kernel<kMixesOnly>, dim3(grid), dim3(pipe::kThreads), 0,
                         stream, a, (int)ntiles);
    return launch_status(what);
  }
  hipLaunchKernelGGL(pick_step_kernel(dtype, mode, a.d), dim3((unsigned)ntiles), dim3(kThreads), 0,
                     stream, a);
  return launch_status(what);
}

// ----- the general-n family ------------------------------------------------------------

bool n_supported(int32_t n) { return n == 2 || n == 4 || n == 8; }

int n_mix(int32_t n) { return (2 + n) * n; }

int64_t packed_bytes_n(int32_t n, int32_t d, int32_t dtype) {
  if (!n_supported(n) || d <= 0 || d % kStep != 0) return -1;
  const int64_t steps = d / kStep;
  auto vecs = [&](auto tag) -> int64_t {
    constexpr int N = decltype(tag)::value;
    return dtype == MHC_BF16 ? gen::Slice<N, MHC_BF16>::kVecs : gen::Slice<N, MHC_F32>::kVecs;
  };
  if (dtype != MHC_BF16 && dtype != MHC_F32) return -1;
  int64_t v = 0;
  switch (n) {
    case 2: v = vecs(std::integral_constant<int, 2>{}); break;
    case 4: v = vecs(std::integral_constant<int, 4>{}); break;
    default: v = vecs(std::integral_constant<int, 8>{}); break;
  }
  return steps * v * 16;
}

template <int N>
void launch_pack_n(const float* w, int d, int32_t dtype, int64_t total, void* out, hipStream_t st) {
  const unsigned blocks = (unsigned)((total + 255) / 256);
  if (dtype == MHC_BF16)
    hipLaunchKernelGGL((gen::pack_kernel<N, MHC_BF16>), dim3(blocks), dim3(256), 0, st, w, d, total,
                       static_cast<u32x4*>(out));
  else
    hipLaunchKernelGGL((gen::pack_kernel<N, MHC_F32>), dim3(blocks), dim3(256), 0, st, w, d, total,
                       static_cast<u32x4*>(out));
}

template <int N, int DT, int SPI>
void launch_block(const StepArgs& a, int mode, hipStream_t st) {
  const unsigned grid = (unsigned)((a.tokens + gen::kBlock - 1) / gen::kBlock);
  const gen::ChunkN none{nullptr, 0, 1};
  if (mode == kFused)
    hipLaunchKernelGGL((gen::block_kernel<N, DT, kFused, SPI>), dim3(grid), dim3(gen::kThreads), 0,
                       st, a, none);
  else
    hipLaunchKernelGGL((gen::block_kernel<N, DT, kMixesOnly, SPI>), dim3(grid),
                       dim3(gen::kThreads), 0, st, a, none);
}

// bf16 streams with n <= 4 and an even step count run two steps per unit
// (both halves of each 128-byte line of a token row loaded back to back)
template <int N>
void launch_block_n(const StepArgs& a, int32_t dtype, int mode, hipStream_t st) {
  if (dtype == MHC_F32) {
    launch_block<N, MHC_F32, 1>(a, mode, st);
    return;
  }
  if constexpr (N <= 4) {
    if ((a.d / kStep) % 2 == 0) {
      launch_block<N, MHC_BF16, 2>(a, mode, st);
      return;
    }
  }
  launch_block<N, MHC_BF16, 1>(a, mode, st);
}

template <int N>
void launch_sinkhorn_n(const float* mix, int64_t tokens, const float* base, const float* scale,
                       int iters, float eps, float* pre, float* post, float* comb, hipStream_t st) {
  constexpr int kTok = gen::kSinkTokens<N>;
  hipLaunchKernelGGL(gen::sinkhorn_kernel<N>, dim3((unsigned)((tokens + kTok - 1) / kTok)),
                     dim3(256), 0, st, mix, tokens, base, scale, iters, eps, pre, post, comb);
}

// The two kernels of the general step: one pass over the streams, then the
// split/Sinkhorn of the mixes it wrote.
mhc_status run_n(int32_t n, const StepArgs& a, int32_t dtype, int mode, hipStream_t st) {
  switch (n) {
    case 2: launch_block_n<2>(a, dtype, mode, st); break;
    case 4: launch_block_n<4>(a, dtype, mode, st); break;
    default: launch_block_n<8>(a, dtype, mode, st); break;
  }
  mhc_status s = launch_status("general-n step kernel launch");
  if (s != MHC_OK) return s;
  switch (n) {
    case 2: launch_sinkhorn_n<2>(a.mix_out, a.tokens, a.base, a.scale, a.iters, a.hc_eps,
                                 a.pre_out, a.post_out, a.comb_out, st); break;
    case 4: launch_sinkhorn_n<4>(a.mix_out, a.tokens, a.base, a.scale, a.iters, a.hc_eps,
                                 a.pre_out, a.post_out, a.comb_out, st); break;
    default: launch_sinkhorn_n<8>(a.mix_out, a.tokens, a.base, a.scale, a.iters, a.hc_eps,
                                  a.pre_out, a.post_out, a.comb_out, st); break;
  }
  return launch_status("general-n split/Sinkhorn kernel launch");
}

// ----- the feature-split kernel of the n-family (n in {2, 4}, bf16) ---------------------

struct SplitCfgN {
  int groups = 0;
  int ns = 0;
  int nr = 0;   // slice = 64 * nr features
};

// The slice shape for (n, d) on this device: S = 64 * nr features per slice,
// ns = d / S slices (16 <= ns <= 64 and at most one per CU); the most CUs in
// use wins, then the widest slice. groups == 0: the kernel does not apply.
mhc_status split_config_n(int32_t n, int32_t dtype, int32_t d, SplitCfgN* cfg) {
  *cfg = SplitCfgN{};
  if (dtype != MHC_BF16 || (n != 2 && n != 4) || d <= 0) return MHC_OK;
  int cus = 0;
  mhc_status s = device_cu_count(&cus);
  if (s != MHC_OK) return s;
  const int maxr = n == 2 ? fsn::max_rounds<2>() : fsn::max_rounds<4>();
  int best = -1;
  for (int nr = maxr; nr >= 1; --nr) {
    const int S = 64 * nr;
    if (d % S != 0) continue;
    const int ns = d / S;
    if (ns < 16 || ns > fsplit::kMaxSlices || ns > cus) continue;
    const int score = (cus / ns) * ns * 8 + nr;
    if (score > best) {
      best = score;
      *cfg = SplitCfgN{cus / ns, ns, nr};
    }
  }
  if (cfg->groups == 0) return MHC_OK;
  bool coop = false;
  if ((s = coop_supported(&coop)) != MHC_OK) return s;
  if (!coop) *cfg = SplitCfgN{};
  return MHC_OK;
}

int64_t split_n_workspace_bytes(int32_t n, const SplitCfgN& c, int64_t tokens) {
  if (c.groups == 0) return 0;
  return n == 2 ? fsn::workspace_bytes<2>(c.groups, c.ns, tokens)
                : fsn::workspace_bytes<4>(c.groups, c.ns, tokens);
}

// the split kernel (it leaves the workspace header as it found it), then the
// split/Sinkhorn of the mixes rows it wrote
template <int N>
mhc_status launch_split_n(const StepArgs& a, void* ws, const SplitCfgN& cfg, int mode, bool plain,
                          hipStream_t stream) {
  if (fsn::ctr_off<N>(cfg.groups, 0) > fsplit::kWsHeader)
    return fail(MHC_ERR_UNSUPPORTED, "feature-split kernel: %d groups exceed the header", cfg.groups);
  mhc_status s = MHC_OK;
  float* mix = a.mix_out != nullptr
                   ? a.mix_out
                   : reinterpret_cast<float*>(static_cast<char*>(ws) +
                                              fsn::mix_off<N>(cfg.groups, cfg.ns));
  fsn::Args fs{static_cast<char*>(ws), mix, cfg.groups, cfg.ns,
               fsplit::BatchSpans::make(a.tokens, cfg.groups)};
  StepArgs args = a;
  void* params[] = {&args, &fs};
  const bool full = mode == kFused;
  const void* fn = nullptr;
  switch (cfg.nr) {
    case 1:
      fn = full ? reinterpret_cast<const void*>(fsn::split_kernel<N, 1, kFused>)
                : reinterpret_cast<const void*>(fsn::split_kernel<N, 1, kMixesOnly>);
      break;
    case 2:
      fn = full ? reinterpret_cast<const void*>(fsn::split_kernel<N, 2, kFused>)
                : reinterpret_cast<const void*>(fsn::split_kernel<N, 2, kMixesOnly>);
      break;
    case 4:
      if constexpr (fsn::max_rounds<N>() >= 4)
        fn = full ? reinterpret_cast<const void*>(fsn::split_kernel<N, 4, kFused>)
                  : reinterpret_cast<const void*>(fsn::split_kernel<N, 4, kMixesOnly>);
      break;
    default: break;
  }
  if (fn == nullptr)
    return fail(MHC_ERR_UNSUPPORTED, "feature-split kernel: n = %d, %d rounds", N, cfg.nr);
  const hipError_t e = launch_resident(fn, (unsigned)(cfg.groups * cfg.ns), params, plain, stream);
  if (e != hipSuccess)
    return fail(MHC_ERR_HIP, "feature-split kernel launch: %s", hipGetErrorString(e));
  if ((s = launch_status("feature-split kernel launch")) != MHC_OK) return s;
  launch_sinkhorn_n<N>(mix, a.tokens, a.base, a.scale, a.iters, a.hc_eps, a.pre_out, a.post_out,
                       a.comb_out, stream);
  return launch_status("general-n split/Sinkhorn kernel launch");
}

// Workspace argument of the n-family: (NULL or 0 bytes: the block kernel);
// otherwise the feature-split kernel when it applies, after the checks of
// mhc_fused_step.
// Chunked launches of the general-n block kernel (at most kChunkMaxTokens
// tokens): up to kChunksN chunks of whole units per row.
constexpr int kChunksN = 80;

struct ChunkCfgN {
  int nchunks = 0;
  int per = 0;   // units per chunk
  int spi = 1;   // steps per unit
};

ChunkCfgN chunk_config_n(int32_t n, int32_t dtype, int32_t d, int64_t tokens) {
  const int nsteps = d / kStep;
  if (d <= 0 || d % kStep != 0 || tokens > kChunkMaxTokens || elem_size(dtype) == 0)
    return ChunkCfgN{};
  const int spi = (dtype == MHC_BF16 && n <= 4 && nsteps % 2 == 0) ? 2 : 1;
  const int nunits = nsteps / spi;
  const int per = (nunits + kChunksN - 1) / kChunksN;
  return ChunkCfgN{(nunits + per - 1) / per, per, spi};
}

int64_t chunk_n_workspace_bytes(int32_t n, const ChunkCfgN& c, int64_t tokens) {
  const int row = n == 2 ? gen::row_n<2>() : (n == 4 ? gen::row_n<4>() : gen::row_n<8>());
  return gen::kChunkHeaderN + (int64_t)c.nchunks * tokens * row * 4;
}

template <int N, int DT, int SPI>
void launch_chunk_block(const StepArgs& a, const gen::ChunkN& cn, int mode, hipStream_t st) {
  const unsigned grid =
      (unsigned)pipe::chunk_grid((a.tokens + gen::kBlock - 1) / gen::kBlock, cn.nchunks);
  if (mode == kFused)
    hipLaunchKernelGGL((gen::block_kernel<N, DT, kFused, SPI, true>), dim3(grid),
                       dim3(gen::kThreads), 0, st, a, cn);
  else
    hipLaunchKernelGGL((gen::block_kernel<N, DT, kMixesOnly, SPI, true>), dim3(grid),
                       dim3(gen::kThreads), 0, st, a, cn);
}

template <int N>
mhc_status launch_chunk_n(const StepArgs& a, void* ws, const ChunkCfgN& c, int32_t dtype,
                          int mode, hipStream_t st) {
  const gen::ChunkN cn{static_cast<char*>(ws), c.per, c.nchunks};
  if (dtype == MHC_F32) {
    launch_chunk_block<N, MHC_F32, 1>(a, cn, mode, st);
  } else {
    if constexpr (N <= 4) {
      if (c.spi == 2) launch_chunk_block<N, MHC_BF16, 2>(a, cn, mode, st);
      else launch_chunk_block<N, MHC_BF16, 1>(a, cn, mode, st);
    } else {
      launch_chunk_block<N, MHC_BF16, 1>(a, cn, mode, st);
    }
  }
  mhc_status s = launch_status("general-n chunk kernel launch");
  if (s != MHC_OK) return s;
  const dim3 tok((unsigned)a.tokens);
  if (mode == kFused && dtype == MHC_BF16)
    hipLaunchKernelGGL((gen::chunk_finish_kernel<N, MHC_BF16, kFused>), tok, dim3(256), 0, st, a,
                       cn);
  else if (mode == kFused)
    hipLaunchKernelGGL((gen::chunk_finish_kernel<N, MHC_F32, kFused>), tok, dim3(256), 0, st, a,
                       cn);
  else
    hipLaunchKernelGGL((gen::chunk_finish_kernel<N, MHC_BF16, kMixesOnly>), tok, dim3(256), 0, st,
                       a, cn);
  if ((s = launch_status("general-n chunk finish kernel launch")) != MHC_OK) return s;
  launch_sinkhorn_n<N>(a.mix_out, a.tokens, a.base, a.scale, a.iters, a.hc_eps, a.pre_out,
                       a.post_out, a.comb_out, st);
  return launch_status("general-n split/Sinkhorn kernel launch");
}

// Workspace routes of the n-family and what each needs (0: does not apply).
struct RouteNeedsN {
  SplitCfgN split;
  ChunkCfgN chunk;
  int64_t split_bytes = 0;
  int64_t chunk_bytes = 0;
};

mhc_status route_needs_n(int32_t n, int32_t dtype, int32_t d, int64_t tokens, RouteNeedsN* rn) {
  *rn = RouteNeedsN{};
  mhc_status s = split_config_n(n, dtype, d, &rn->split);
  if (s != MHC_OK) return s;
  if (rn->split.groups > 0) rn->split_bytes = split_n_workspace_bytes(n, rn->split, tokens);
  rn->chunk = chunk_config_n(n, dtype, d, tokens);
  if (rn->chunk.nchunks > 0) rn->chunk_bytes = chunk_n_workspace_bytes(n, rn->chunk, tokens);
  return MHC_OK;
}

// The route of an n-family call (MHC_PATH_TILE names the block kernel here).
mhc_status choose_route_n(int32_t path, const void* workspace, int32_t n, int32_t dtype,
                          int32_t d, int64_t tokens, RouteNeedsN* rn, Route* r) {
  *rn = RouteNeedsN{};
  if (path == MHC_PATH_TILE || (path == MHC_PATH_AUTO && workspace == nullptr)) {
    *r = Route::kTile;
    return MHC_OK;
  }
  if (path == MHC_PATH_AUTO || path == MHC_PATH_SPLIT || path == MHC_PATH_CHUNK) {
    const mhc_status s = route_needs_n(n, dtype, d, tokens, rn);
    if (s != MHC_OK) return s;
  }
  const mhc_status s = pick_route(path, workspace, tokens, rn->split_bytes, rn->chunk_bytes, r);
  // without a feature-split kernel the chunks beat the block kernel at every
  // size they cover (a call of T tokens has only T / 128 blocks)
  if (s == MHC_OK && path == MHC_PATH_AUTO && *r == Route::kTile && workspace != nullptr &&
      rn->chunk_bytes > 0)
    *r = Route::kChunk;
  return s;
}

mhc_status launch_route_n(int32_t n, Route route, const RouteNeedsN& rn, const StepArgs& a,
                          void* workspace, int32_t dtype, int mode, bool plain, hipStream_t st) {
  if (route == Route::kSplit)
    return n == 2 ? launch_split_n<2>(a, workspace, rn.split, mode, plain, st)
                  : launch_split_n<4>(a, workspace, rn.split, mode, plain, st);
  if (route == Route::kChunk) {
    switch (n) {
      case 2: return launch_chunk_n<2>(a, workspace, rn.chunk, dtype, mode, st);
      case 4: return launch_chunk_n<4>(a, workspace, rn.chunk, dtype, mode, st);
      default: return launch_chunk_n<8>(a, workspace, rn.chunk, dtype, mode, st);
    }
  }
  return run_n(n, a, dtype, mode, st);
}

// ----- backward ------------------------------------------------------------------------

bool bwd_supported(int32_t n) { return n == 2 || n == 4; }

int64_t bwd_workspace_floats(int32_t n, int64_t tokens, int32_t d) {
  if (n == 2) return bwd::Ws<2>{tokens, d}.floats();
  return bwd::Ws<4>{tokens, d}.floats();
}

// The backward's regions start after the header the forward kernels keep at
// the start of every workspace, so one workspace serves both directions.
int64_t bwd_workspace_bytes(int32_t n, int64_t tokens, int32_t d) {
  return fsplit::kWsHeader + bwd_workspace_floats(n, tokens, d) * 4;
}


template <int N, int DT>
mhc_status run_backward(const bwd::Args& args, hipStream_t st) {
  // bf16 streams with d % 64 == 0 take the row kernel (64-token workgroups),
  // the rest the MFMA-layout stream kernel (128-token workgroups)
  const bool rows = DT == MHC_BF16 && args.d % bwd::kUnit == 0;
  bwd::Args a = args;
  const int64_t block = rows ? bwd::kRowBlock : bwd::kBlock;
  a.dg_groups = (a.tokens + block - 1) / block;
  const unsigned tok_blocks = (unsigned)((a.tokens + 256 / (N * N) - 1) / (256 / (N * N)));
  hipLaunchKernelGGL((bwd::split_kernel<N>), dim3(tok_blocks), dim3(256), 0, st, a);
  mhc_status s = launch_status("backward split/Sinkhorn kernel launch");
  if (s != MHC_OK) return s;
  hipLaunchKernelGGL((bwd::stats_kernel<N, DT>), dim3((unsigned)((a.tokens + 3) / 4)), dim3(256),
                     0, st, a);
  if ((s = launch_status("backward statistics kernel launch")) != MHC_OK) return s;
  if (rows) {
    const bwd::Ws<N> wsl{a.tokens, a.d};
    const int64_t vecs = (int64_t)(a.d / bwd::kUnit) * bwd::RowDims<N>::kWtVecs;
    hipLaunchKernelGGL((bwd::wt_pack_kernel<N>), dim3((unsigned)((vecs + 255) / 256)), dim3(256),
                       0, st, a.w, a.d, vecs, reinterpret_cast<u32x4*>(a.ws + wsl.wt_off()));
    if ((s = launch_status("backward W^T packing kernel launch")) != MHC_OK) return s;
    hipLaunchKernelGGL((bwd::row_kernel<N>), dim3((unsigned)a.dg_groups), dim3(bwd::kThreads), 0,
                       st, a);
  } else {
    hipLaunchKernelGGL((bwd::stream_kernel<N, DT>), dim3((unsigned)a.dg_groups),
                       dim3(bwd::kThreads), 0, st, a);
  }
  if ((s = launch_status("backward stream kernel launch")) != MHC_OK) return s;
  if (DT == MHC_BF16 && a.d % 64 == 0)
    hipLaunchKernelGGL((bwd::param_mfma_kernel<N>),
                       dim3((unsigned)((a.d / 64 + 3) / 4), N, bwd::kParamChunks), dim3(256), 0, st,
                       a);
  else
    hipLaunchKernelGGL((bwd::param_kernel<N, DT>),
                       dim3((unsigned)((a.d + 255) / 256), N, bwd::kParamChunks), dim3(256), 0, st,
                       a);
  if ((s = launch_status("backward parameter kernel launch")) != MHC_OK) return s;
  const int64_t nw = (int64_t)bwd::Dims<N>::kMix * N * a.d;
  hipLaunchKernelGGL((bwd::param_reduce_kernel<N>), dim3((unsigned)((nw + 255) / 256)),
                     dim3(256), 0, st, a);
  if ((s = launch_status("backward parameter reduction launch")) != MHC_OK) return s;
  hipLaunchKernelGGL((bwd::gamma_reduce_kernel<N>), dim3((unsigned)((a.d + 63) / 64)), dim3(256),
                     0, st, a);
  if ((s = launch_status("backward gain reduction launch")) != MHC_OK) return s;
  hipLaunchKernelGGL((bwd::slot_kernel<N>), dim3(bwd::kSlotChunks), dim3(256), 0, st, a);
  if ((s = launch_status("backward slot reduction launch")) != MHC_OK) return s;
  hipLaunchKernelGGL((bwd::scale_kernel<N>), dim3(1), dim3(64), 0, st, a);
  return launch_status("backward scale reduction launch");
}


// ----- scratch of the allocation-free entry point -------------------------------------
//
// mhc_fused_step_noalloc's workspace is `scratch`, a file-scope device array:
// every GPU the library runs on holds one copy (at its own address) until the
// process ends. On the host the array's name is only a stand-in symbol, never
// a device address: the address is looked up once per device, with that
// device current, and kept; kernels get that address.

constexpr int64_t kScratchBytes = int64_t(32) << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

__global__ void zero_header_kernel(uint32_t* p, int words) {
  for (int i = threadIdx.x; i < words; i += blockDim.x) p[i] = 0u;
}

// Device address of the current device's scratch. The first call on a device
// also zeroes the workspace header on `stream` with a plain kernel (static
// device memory starts zeroed when the code object is loaded; this makes the
// header rule explicit for one launch per device); every call leaves it zero.
mhc_status device_scratch(hipStream_t stream, void** out) {
  static std::atomic<void*> ptrs[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MHC_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(MHC_ERR_UNSUPPORTED, "device ordinal %d", dev);
  void* p = ptrs[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(MHC_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    hipLaunchKernelGGL(zero_header_kernel, dim3(1), dim3(256), 0, stream,
                       static_cast<uint32_t*>(p), (int)(fsplit::kWsHeader / 4));
    const mhc_status s = launch_status("scratch header clear launch");
    if (s != MHC_OK) return s;
    ptrs[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return MHC_OK;
}

}  // namespace

extern "C" {

int32_t mhc_abi_version(void) { return MHC_ABI_VERSION; }

const char* mhc_status_string(int32_t status) {
  switch (status) {
    case MHC_OK: return "MHC_OK";
    case MHC_ERR_INVALID_ARG: return "MHC_ERR_INVALID_ARG";
    case MHC_ERR_UNSUPPORTED: return "MHC_ERR_UNSUPPORTED";
    case MHC_ERR_HIP: return "MHC_ERR_HIP";
    default: return "unknown status";
  }
}

const char* mhc_last_error(void) { return g_last_error; }

int32_t mhc_d_granule(void) { return kStep; }

int64_t mhc_wmix_packed_bytes(int32_t d, int32_t dtype) { return packed_bytes(d, dtype); }

int64_t mhc_fused_step_workspace_bytes(int64_t tokens, int32_t d, int32_t dtype) {
  if (tokens < 0 || d <= 0 || d % kStep != 0 || elem_size(dtype) == 0) {
    fail(MHC_ERR_INVALID_ARG, "bad tokens (%lld), d (%d) or dtype (%d)", (long long)tokens, d, dtype);
    return -1;
  }
  RouteNeeds rn;
  if (route_needs(dtype, d, tokens, &rn) != MHC_OK) return -1;
  return std::max(rn.split_bytes, rn.chunk_bytes);
}

int32_t mhc_fused_step_route(int32_t path, int64_t tokens, int32_t d, int32_t dtype,
                             int32_t with_workspace) {
  if (tokens < 0 || d <= 0 || d % kStep != 0 || elem_size(dtype) == 0) {
    fail(MHC_ERR_INVALID_ARG, "bad tokens (%lld), d (%d) or dtype (%d)", (long long)tokens, d, dtype);
    return -1;
  }
  RouteNeeds rn;
  Route r;
  bool plain = false;
  static const char kDummy = 0;   // stands for a workspace; never dereferenced
  if (choose_route(path, with_workspace ? &kDummy : nullptr, dtype, d, tokens, &rn, &r,
                   &plain) != MHC_OK)
    return -1;
  return r == Route::kTile ? MHC_PATH_TILE : (r == Route::kSplit ? MHC_PATH_SPLIT : MHC_PATH_CHUNK);
}

mhc_status mhc_pack_wmix(const float* w_mix, int32_t d, int32_t dtype, void* w_packed,
                         int64_t packed_bytes_given, mhc_stream_t stream) {
  const int64_t need = packed_bytes(d, dtype);
  if (need < 0) return fail(MHC_ERR_INVALID_ARG, "bad d (%d) or dtype (%d)", d, dtype);
  if (packed_bytes_given < need)
    return fail(MHC_ERR_INVALID_ARG, "w_packed holds %lld bytes, %lld needed",
                (long long)packed_bytes_given, (long long)need);
  const Span in[] = {{"w_mix", w_mix, (uint64_t)kMix * kStreams * d * 4}};
  const Span out[] = {{"w_packed", w_packed, (uint64_t)need}};
  mhc_status s = check_spans(in, 1, out, 1, nullptr, nullptr);
  if (s != MHC_OK) return s;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t total = (dtype == MHC_BF16 ? need / 16 : need / 32);
  const unsigned blocks = (unsigned)((total + 255) / 256);
  if (dtype == MHC_BF16)
    hipLaunchKernelGGL(pack_bf16_kernel, dim3(blocks), dim3(256), 0, st, w_mix, d, total,
                       static_cast<u32x4*>(w_packed));
  else
    hipLaunchKernelGGL(pack_f32_kernel, dim3(blocks), dim3(256), 0, st, w_mix, d, total,
                       static_cast<u32x4*>(w_packed));
  return launch_status("pack kernel launch");
}

mhc_status mhc_fused_step(const void* x, const void* f, int32_t dtype, int64_t tokens, int32_t d,
                          const float* pre_in, const float* post_in, const float* comb_in,
                          const void* w_packed, const float* base, const float* scale,
                          const float* gamma, int32_t sinkhorn_iters, float norm_eps,
                          float hc_eps, void* x_out, void* y_out, float* pre_out,
                          float* post_out, float* comb_out, float* mix_out, int32_t path,
                          void* workspace, int64_t workspace_bytes, mhc_stream_t stream) {
  mhc_status s = check_common(dtype, tokens, d, sinkhorn_iters, norm_eps, hc_eps);
  if (s != MHC_OK) return s;
  if (tokens == 0) return ok();
  const uint64_t es = elem_size(dtype), T = (uint64_t)tokens;
  const Span in[] = {
      {"x", x, T * kStreams * d * es},     {"f", f, T * d * es},
      {"pre_in", pre_in, T * 16},          {"post_in", post_in, T * 16},
      {"comb_in", comb_in, T * 64},        {"w_packed", w_packed, (uint64_t)packed_bytes(d, dtype)},
      {"base", base, kMix * 4},            {"scale", scale, 12},
      {"gamma", gamma, (uint64_t)d * 4},
  };
  const Span out[] = {
      {"x_out", x_out, T * kStreams * d * es}, {"y_out", y_out, T * d * es},
      {"pre_out", pre_out, T * 16},            {"post_out", post_out, T * 16},
      {"comb_out", comb_out, T * 64},
  };
  s = check_spans(in, 9, out, 5, x_out, x);
  if (s != MHC_OK) return s;
  if (mix_out != nullptr) {
    const Span mo[] = {{"mix_out", mix_out, T * kMix * 4}};
    Span all[14];
    for (int i = 0; i < 9; ++i) all[i] = in[i];
    for (int i = 0; i < 5; ++i) all[9 + i] = out[i];
    s = check_spans(all, 14, mo, 1, nullptr, nullptr);
    if (s != MHC_OK) return s;
  }
  RouteNeeds rn;
  Route route;
  bool plain = false;
  if ((s = choose_route(path, workspace, dtype, d, tokens, &rn, &route, &plain,
                        sinkhorn_iters)) != MHC_OK)
    return s;
  if (route != Route::kTile) {
    const int64_t need = route == Route::kSplit ? rn.split_bytes : rn.chunk_bytes;
    Span all[15];
    for (int i = 0; i < 9; ++i) all[i] = in[i];
    for (int i = 0; i < 5; ++i) all[9 + i] = out[i];
    int nall = 14;
    if (mix_out != nullptr) all[nall++] = {"mix_out", mix_out, T * kMix * 4};
    if ((s = check_workspace(workspace, workspace_bytes, need, all, nall)) != MHC_OK) return s;
  }
  StepArgs a{x, f, pre_in, post_in, comb_in, w_packed, base, scale, gamma, x_out, y_out,
             pre_out, post_out, comb_out, mix_out, tokens, d, sinkhorn_iters, norm_eps, hc_eps};
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (route == Route::kSplit) return launch_split(a, workspace, rn.split, kFused, plain, st);
  if (route == Route::kChunk) return launch_chunk(a, workspace, rn.chunk, kFused, st);
  return launch_step(a, dtype, kFused, st, "fused step kernel launch");
}

mhc_status mhc_fused_step_noalloc(const void* x, const void* f, int32_t dtype, int64_t tokens,
                                  int32_t d, const float* pre_in, const float* post_in,
                                  const float* comb_in, const void* w_packed, const float* base,
                                  const float* scale, const float* gamma, int32_t sinkhorn_iters,
                                  float norm_eps, float hc_eps, void* x_out, void* y_out,
                                  float* pre_out, float* post_out, float* comb_out,
                                  float* mix_out, int32_t path, mhc_stream_t stream) {
  mhc_status s = check_common(dtype, tokens, d, sinkhorn_iters, norm_eps, hc_eps);
  if (s != MHC_OK) return s;
  if (tokens == 0) return ok();
  bool plain = false;
  if (path_family(path, &plain) != MHC_PATH_TILE) {
    RouteNeeds rn;
    Route r;
    static const char kDummy = 0;   // stands for a workspace; never dereferenced
    if ((s = choose_route(path, &kDummy, dtype, d, tokens, &rn, &r, &plain, sinkhorn_iters)) !=
        MHC_OK)
      return s;
    const int64_t need =
        r == Route::kSplit ? rn.split_bytes : (r == Route::kChunk ? rn.chunk_bytes : 0);
    if (need > kScratchBytes)
      return fail(MHC_ERR_INVALID_ARG,
                  "%lld tokens at d = %d need %lld bytes of scratch; the static scratch holds "
                  "%lld (use mhc_fused_step with a workspace)",
                  (long long)tokens, d, (long long)need, (long long)kScratchBytes);
  }
  void* ws = nullptr;
  if ((s = device_scratch(static_cast<hipStream_t>(stream), &ws)) != MHC_OK) return s;
  return mhc_fused_step(x, f, dtype, tokens, d, pre_in, post_in, comb_in, w_packed, base, scale,
                        gamma, sinkhorn_iters, norm_eps, hc_eps, x_out, y_out, pre_out, post_out,
                        comb_out, mix_out, path, ws, kScratchBytes, stream);
}

mhc_status mhc_mixes(const void* x, int32_t dtype, int64_t tokens, int32_t d,
                     const void* w_packed, const float* base, const float* scale,
                     int32_t sinkhorn_iters, float norm_eps, float hc_eps, float* pre_out,
                     float* post_out, float* comb_out, float* mix_out, int32_t path,
                     void* workspace, int64_t workspace_bytes, mhc_stream_t stream) {
  mhc_status s = check_common(dtype, tokens, d, sinkhorn_iters, norm_eps, hc_eps);
  if (s != MHC_OK) return s;
  if (tokens == 0) return ok();
  const uint64_t es = elem_size(dtype), T = (uint64_t)tokens;
  const Span in[] = {
      {"x", x, T * kStreams * d * es},
      {"w_packed", w_packed, (uint64_t)packed_bytes(d, dtype)},
      {"base", base, kMix * 4},
      {"scale", scale, 12},
  };
  const Span out[] = {
      {"pre_out", pre_out, T * 16}, {"post_out", post_out, T * 16},
      {"comb_out", comb_out, T * 64}, {"mix_out", mix_out, T * kMix * 4},
  };
  s = check_spans(in, 4, out, mix_out ? 4 : 3, nullptr, nullptr);
  if (s != MHC_OK) return s;
  RouteNeeds rn;
  Route route;
  bool plain = false;
  if ((s = choose_route(path, workspace, dtype, d, tokens, &rn, &route, &plain,
                        sinkhorn_iters)) != MHC_OK)
    return s;
  if (route != Route::kTile) {
    const int64_t need = route == Route::kSplit ? rn.split_bytes : rn.chunk_bytes;
    Span all[8];
    for (int i = 0; i < 4; ++i) all[i] = in[i];
    for (int i = 0; i < (mix_out ? 4 : 3); ++i) all[4 + i] = out[i];
    if ((s = check_workspace(workspace, workspace_bytes, need, all, mix_out ? 8 : 7)) != MHC_OK)
      return s;
  }
  StepArgs a{x, nullptr, nullptr, nullptr, nullptr, w_packed, base, scale, nullptr, nullptr,
             nullptr, pre_out, post_out, comb_out, mix_out, tokens, d, sinkhorn_iters, norm_eps,
             hc_eps};
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (route == Route::kSplit)
    return launch_split(a, workspace, rn.split, kMixesOnly, plain, st);
  if (route == Route::kChunk) return launch_chunk(a, workspace, rn.chunk, kMixesOnly, st);
  return launch_step(a, dtype, kMixesOnly, st, "mixes kernel launch");
}

mhc_status mhc_hc_post(const void* x, const void* f, int32_t dtype, int64_t tokens, int32_t d,
                       const float* post_in, const float* comb_in, void* x_out,
                       mhc_stream_t stream) {
  mhc_status s = check_common(dtype, tokens, d, 1, 0.f, 0.f);
  if (s != MHC_OK) return s;
  if (tokens == 0) return ok();
  const uint64_t es = elem_size(dtype), T = (uint64_t)tokens;
  const Span in[] = {{"x", x, T * kStreams * d * es}, {"f", f, T * d * es},
                     {"post_in", post_in, T * 16}, {"comb_in", comb_in, T * 64}};
  const Span out[] = {{"x_out", x_out, T * kStreams * d * es}};
  s = check_spans(in, 4, out, 1, x_out, x);
  if (s != MHC_OK) return s;
  const unsigned blocks = (unsigned)((tokens * (d / 8) + unfused::kThreads - 1) / unfused::kThreads);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (dtype == MHC_BF16)
    hipLaunchKernelGGL(unfused::hc_post_kernel<MHC_BF16>, dim3(blocks), dim3(unfused::kThreads), 0,
                       st, x, f, post_in, comb_in, tokens, d, x_out);
  else
    hipLaunchKernelGGL(unfused::hc_post_kernel<MHC_F32>, dim3(blocks), dim3(unfused::kThreads), 0,
                       st, x, f, post_in, comb_in, tokens, d, x_out);
  return launch_status("hc_post kernel launch");
}

mhc_status mhc_hc_pre(const void* x, int32_t dtype, int64_t tokens, int32_t d,
                      const float* pre_in, void* h_out, mhc_stream_t stream) {
  mhc_status s = check_common(dtype, tokens, d, 1, 0.f, 0.f);
  if (s != MHC_OK) return s;
  if (tokens == 0) return ok();
  const uint64_t es = elem_size(dtype), T = (uint64_t)tokens;
  const Span in[] = {{"x", x, T * kStreams * d * es}, {"pre_in", pre_in, T * 16}};
  const Span out[] = {{"h_out", h_out, T * d * es}};
  s = check_spans(in, 2, out, 1, nullptr, nullptr);
  if (s != MHC_OK) return s;
  const unsigned blocks = (unsigned)((tokens * (d / 8) + unfused::kThreads - 1) / unfused::kThreads);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (dtype == MHC_BF16)
    hipLaunchKernelGGL(unfused::hc_pre_kernel<MHC_BF16>, dim3(blocks), dim3(unfused::kThreads), 0,
                       st, x, pre_in, tokens, d, h_out);
  else
    hipLaunchKernelGGL(unfused::hc_pre_kernel<MHC_F32>, dim3(blocks), dim3(unfused::kThreads), 0,
                       st, x, pre_in, tokens, d, h_out);
  return launch_status("hc_pre kernel launch");
}

mhc_status mhc_rmsnorm(const void* h, int32_t dtype, int64_t tokens, int32_t d,
                       const float* gamma, float norm_eps, void* y_out, mhc_stream_t stream) {
  mhc_status s = check_common(dtype, tokens, d, 1, norm_eps, 0.f);
  if (s != MHC_OK) return s;
  if (tokens == 0) return ok();
  const uint64_t es = elem_size(dtype), T = (uint64_t)tokens;
  const Span in[] = {{"h", h, T * d * es}, {"gamma", gamma, (uint64_t)d * 4}};
  const Span out[] = {{"y_out", y_out, T * d * es}};
  s = check_spans(in, 2, out, 1, y_out, h);
  if (s != MHC_OK) return s;
  const unsigned blocks = (unsigned)((tokens + 3) / 4);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (dtype == MHC_BF16)
    hipLaunchKernelGGL(unfused::rmsnorm_kernel<MHC_BF16>, dim3(blocks), dim3(unfused::kThreads), 0,
                       st, h, gamma, tokens, d, norm_eps, y_out);
  else
    hipLaunchKernelGGL(unfused::rmsnorm_kernel<MHC_F32>, dim3(blocks), dim3(unfused::kThreads), 0,
                       st, h, gamma, tokens, d, norm_eps, y_out);
  return launch_status("rmsnorm kernel launch");
}

mhc_status mhc_sinkhorn4(const float* mixes, int64_t tokens, const float* base,
                         const float* scale, int32_t sinkhorn_iters, float hc_eps,
                         float* pre_out, float* post_out, float* comb_out,
                         mhc_stream_t stream) {
  if (tokens < 0) return fail(MHC_ERR_INVALID_ARG, "tokens must be >= 0");
  if (sinkhorn_iters < 1) return fail(MHC_ERR_INVALID_ARG, "sinkhorn_iters must be >= 1");
  if (!(hc_eps >= 0.f) || !isfinite(hc_eps))
    return fail(MHC_ERR_INVALID_ARG, "hc_eps must be finite and >= 0");
  if (tokens > ((int64_t)1 << 35)) return fail(MHC_ERR_UNSUPPORTED, "too many tokens");
  if (tokens == 0) return ok();
  const uint64_t T = (uint64_t)tokens;
  const Span in[] = {{"mixes", mixes, T * kMix * 4}, {"base", base, kMix * 4}, {"scale", scale, 12}};
  const Span out[] = {{"pre_out", pre_out, T * 16}, {"post_out", post_out, T * 16},
                      {"comb_out", comb_out, T * 64}};
  mhc_status s = check_spans(in, 3, out, 3, nullptr, nullptr);
  if (s != MHC_OK) return s;
  hipLaunchKernelGGL(fsplit::tail_kernel,
                     dim3((unsigned)((tokens + fsplit::kTailThreads - 1) / fsplit::kTailThreads)),
                     dim3(fsplit::kTailThreads), 0, static_cast<hipStream_t>(stream), mixes, tokens, base, scale, sinkhorn_iters,
                     hc_eps, pre_out, post_out, comb_out);
  return launch_status("split/Sinkhorn kernel launch");
}

int64_t mhc_wmix_packed_bytes_n(int32_t n, int32_t d, int32_t dtype) {
  const int64_t b = packed_bytes_n(n, d, dtype);
  if (b < 0) fail(MHC_ERR_INVALID_ARG, "bad n (%d), d (%d) or dtype (%d)", n, d, dtype);
  return b;
}

mhc_status mhc_pack_wmix_n(int32_t n, const float* w_mix, int32_t d, int32_t dtype,
                           void* w_packed, int64_t packed_bytes_given, mhc_stream_t stream) {
  if (!n_supported(n)) return fail(MHC_ERR_UNSUPPORTED, "n = %d streams (2, 4 or 8 supported)", n);
  const int64_t need = packed_bytes_n(n, d, dtype);
  if (need < 0) return fail(MHC_ERR_INVALID_ARG, "bad d (%d) or dtype (%d)", d, dtype);
  if (packed_bytes_given < need)
    return fail(MHC_ERR_INVALID_ARG, "w_packed holds %lld bytes, %lld needed",
                (long long)packed_bytes_given, (long long)need);
  const Span in[] = {{"w_mix", w_mix, (uint64_t)n_mix(n) * n * d * 4}};
  const Span out[] = {{"w_packed", w_packed, (uint64_t)need}};
  mhc_status s = check_spans(in, 1, out, 1, nullptr, nullptr);
  if (s != MHC_OK) return s;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t total = need / (dtype == MHC_BF16 ? 16 : 32);
  switch (n) {
    case 2: launch_pack_n<2>(w_mix, d, dtype, total, w_packed, st); break;
    case 4: launch_pack_n<4>(w_mix, d, dtype, total, w_packed, st); break;
    default: launch_pack_n<8>(w_mix, d, dtype, total, w_packed, st); break;
  }
  return launch_status("general-n pack kernel launch");
}

int64_t mhc_fused_step_n_workspace_bytes(int32_t n, int64_t tokens, int32_t d, int32_t dtype) {
  if (!n_supported(n) || tokens < 0 || d <= 0 || d % kStep != 0 || elem_size(dtype) == 0) {
    fail(MHC_ERR_INVALID_ARG, "bad n (%d), tokens (%lld), d (%d) or dtype (%d)", n,
         (long long)tokens, d, dtype);
    return -1;
  }
  RouteNeedsN rn;
  if (route_needs_n(n, dtype, d, tokens, &rn) != MHC_OK) return -1;
  return std::max(rn.split_bytes, rn.chunk_bytes);
}

int32_t mhc_fused_step_route_n(int32_t n, int32_t path, int64_t tokens, int32_t d, int32_t dtype,
                               int32_t with_workspace) {
  if (!n_supported(n) || tokens < 0 || d <= 0 || d % kStep != 0 || elem_size(dtype) == 0) {
    fail(MHC_ERR_INVALID_ARG, "bad n (%d), tokens (%lld), d (%d) or dtype (%d)", n,
         (long long)tokens, d, dtype);
    return -1;
  }
  RouteNeedsN rn;
  Route r;
  bool plain = false;
  static const char kDummy = 0;   // stands for a workspace; never dereferenced
  if (choose_route_n(path_family(path, &plain), with_workspace ? &kDummy : nullptr, n, dtype, d,
                     tokens, &rn, &r) != MHC_OK)
    return -1;
  return r == Route::kTile ? MHC_PATH_TILE : (r == Route::kSplit ? MHC_PATH_SPLIT : MHC_PATH_CHUNK);
}

mhc_status mhc_fused_step_n(int32_t n, const void* x, const void* f, int32_t dtype,
                            int64_t tokens, int32_t d, const float* pre_in,
                            const float* post_in, const float* comb_in, const void* w_packed,
                            const float* base, const float* scale, const float* gamma,
                            int32_t sinkhorn_iters, float norm_eps, float hc_eps, void* x_out,
                            void* y_out, float* pre_out, float* post_out, float* comb_out,
                            float* mix_out, int32_t path, void* workspace,
                            int64_t workspace_bytes, mhc_stream_t stream) {
  if (!n_supported(n)) return fail(MHC_ERR_UNSUPPORTED, "n = %d streams (2, 4 or 8 supported)", n);
  mhc_status s = check_common(dtype, tokens, d, sinkhorn_iters, norm_eps, hc_eps);
  if (s != MHC_OK) return s;
  if (tokens == 0) return ok();
  const uint64_t es = elem_size(dtype), T = (uint64_t)tokens, nn = (uint64_t)n, nm = n_mix(n);
  const Span in[] = {
      {"x", x, T * nn * d * es},           {"f", f, T * d * es},
      {"pre_in", pre_in, T * nn * 4},      {"post_in", post_in, T * nn * 4},
      {"comb_in", comb_in, T * nn * nn * 4},
      {"w_packed", w_packed, (uint64_t)packed_bytes_n(n, d, dtype)},
      {"base", base, nm * 4},              {"scale", scale, 12},
      {"gamma", gamma, (uint64_t)d * 4},
  };
  const Span out[] = {
      {"x_out", x_out, T * nn * d * es},   {"y_out", y_out, T * d * es},
      {"pre_out", pre_out, T * nn * 4},    {"post_out", post_out, T * nn * 4},
      {"comb_out", comb_out, T * nn * nn * 4}, {"mix_out", mix_out, T * nm * 4},
  };
  s = check_spans(in, 9, out, 6, x_out, x);
  if (s != MHC_OK) return s;
  RouteNeedsN rn;
  Route route;
  bool plain = false;
  if ((s = choose_route_n(path_family(path, &plain), workspace, n, dtype, d, tokens, &rn,
                          &route)) != MHC_OK)
    return s;
  if (route != Route::kTile) {
    const int64_t need = route == Route::kSplit ? rn.split_bytes : rn.chunk_bytes;
    Span all[15];
    for (int i = 0; i < 9; ++i) all[i] = in[i];
    for (int i = 0; i < 6; ++i) all[9 + i] = out[i];
    if ((s = check_workspace(workspace, workspace_bytes, need, all, 15)) != MHC_OK) return s;
  }
  StepArgs a{x, f, pre_in, post_in, comb_in, w_packed, base, scale, gamma, x_out, y_out,
             pre_out, post_out, comb_out, mix_out, tokens, d, sinkhorn_iters, norm_eps, hc_eps};
  const hipStream_t st = static_cast<hipStream_t>(stream);
  return launch_route_n(n, route, rn, a, workspace, dtype, kFused, plain, st);
}

mhc_status mhc_mixes_n(int32_t n, const void* x, int32_t dtype, int64_t tokens, int32_t d,
                       const void* w_packed, const float* base, const float* scale,
                       int32_t sinkhorn_iters, float norm_eps, float hc_eps, float* pre_out,
                       float* post_out, float* comb_out, float* mix_out, int32_t path,
                       void* workspace, int64_t workspace_bytes, mhc_stream_t stream) {
  if (!n_supported(n)) return fail(MHC_ERR_UNSUPPORTED, "n = %d streams (2, 4 or 8 supported)", n);
  mhc_status s = check_common(dtype, tokens, d, sinkhorn_iters, norm_eps, hc_eps);
  if (s != MHC_OK) return s;
  if (tokens == 0) return ok();
  const uint64_t es = elem_size(dtype), T = (uint64_t)tokens, nn = (uint64_t)n, nm = n_mix(n);
  const Span in[] = {
      {"x", x, T * nn * d * es},
      {"w_packed", w_packed, (uint64_t)packed_bytes_n(n, d, dtype)},
      {"base", base, nm * 4},
      {"scale", scale, 12},
  };
  const Span out[] = {
      {"pre_out", pre_out, T * nn * 4}, {"post_out", post_out, T * nn * 4},
      {"comb_out", comb_out, T * nn * nn * 4}, {"mix_out", mix_out, T * nm * 4},
  };
  s = check_spans(in, 4, out, 4, nullptr, nullptr);
  if (s != MHC_OK) return s;
  RouteNeedsN rn;
  Route route;
  bool plain = false;
  if ((s = choose_route_n(path_family(path, &plain), workspace, n, dtype, d, tokens, &rn,
                          &route)) != MHC_OK)
    return s;
  if (route != Route::kTile) {
    const int64_t need = route == Route::kSplit ? rn.split_bytes : rn.chunk_bytes;
    Span all[8];
    for (int i = 0; i < 4; ++i) all[i] = in[i];
    for (int i = 0; i < 4; ++i) all[4 + i] = out[i];
    if ((s = check_workspace(workspace, workspace_bytes, need, all, 8)) != MHC_OK) return s;
  }
  StepArgs a{x, nullptr, nullptr, nullptr, nullptr, w_packed, base, scale, nullptr, nullptr,
             nullptr, pre_out, post_out, comb_out, mix_out, tokens, d, sinkhorn_iters, norm_eps,
             hc_eps};
  const hipStream_t st = static_cast<hipStream_t>(stream);
  return launch_route_n(n, route, rn, a, workspace, dtype, kMixesOnly, plain, st);
}

mhc_status mhc_sinkhorn_n(int32_t n, const float* mixes, int64_t tokens, const float* base,
                          const float* scale, int32_t sinkhorn_iters, float hc_eps,
                          float* pre_out, float* post_out, float* comb_out,
                          mhc_stream_t stream) {
  if (!n_supported(n)) return fail(MHC_ERR_UNSUPPORTED, "n = %d streams (2, 4 or 8 supported)", n);
  if (tokens < 0) return fail(MHC_ERR_INVALID_ARG, "tokens must be >= 0");
  if (sinkhorn_iters < 1) return fail(MHC_ERR_INVALID_ARG, "sinkhorn_iters must be >= 1");
  if (!(hc_eps >= 0.f) || !isfinite(hc_eps))
    return fail(MHC_ERR_INVALID_ARG, "hc_eps must be finite and >= 0");
  if (tokens > ((int64_t)1 << 35)) return fail(MHC_ERR_UNSUPPORTED, "too many tokens");
  if (tokens == 0) return ok();
  const uint64_t T = (uint64_t)tokens, nn = (uint64_t)n, nm = n_mix(n);
  const Span in[] = {{"mixes", mixes, T * nm * 4}, {"base", base, nm * 4}, {"scale", scale, 12}};
  const Span out[] = {{"pre_out", pre_out, T * nn * 4}, {"post_out", post_out, T * nn * 4},
                      {"comb_out", comb_out, T * nn * nn * 4}};
  mhc_status s = check_spans(in, 3, out, 3, nullptr, nullptr);
  if (s != MHC_OK) return s;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  switch (n) {
    case 2: launch_sinkhorn_n<2>(mixes, tokens, base, scale, sinkhorn_iters, hc_eps, pre_out,
                                 post_out, comb_out, st); break;
    case 4: launch_sinkhorn_n<4>(mixes, tokens, base, scale, sinkhorn_iters, hc_eps, pre_out,
                                 post_out, comb_out, st); break;
    default: launch_sinkhorn_n<8>(mixes, tokens, base, scale, sinkhorn_iters, hc_eps, pre_out,
                                  post_out, comb_out, st); break;
  }
  return launch_status("general-n split/Sinkhorn kernel launch");
}

int64_t mhc_fused_step_backward_workspace_bytes_n(int32_t n, int64_t tokens, int32_t d) {
  if (!bwd_supported(n) || tokens < 0 || d <= 0 || d % kStep != 0) {
    fail(MHC_ERR_INVALID_ARG, "bad n (%d), tokens (%lld) or d (%d)", n, (long long)tokens, d);
    return -1;
  }
  return bwd_workspace_bytes(n, tokens, d);
}

mhc_status mhc_fused_step_backward_n(
    int32_t n, const void* x, const void* f, int32_t dtype, int64_t tokens, int32_t d,
    const float* pre_in, const float* post_in, const float* comb_in, const void* x_out,
    const float* mix, const float* w_mix, const float* base, const float* scale,
    const float* gamma, int32_t sinkhorn_iters, float norm_eps, float hc_eps, const void* d_x_out,
    const void* d_y, const float* d_pre, const float* d_post, const float* d_comb, void* d_x,
    void* d_f, float* d_pre_in, float* d_post_in, float* d_comb_in, float* d_w_mix,
    float* d_base, float* d_scale, float* d_gamma, void* workspace, int64_t workspace_bytes,
    mhc_stream_t stream) {
  if (!bwd_supported(n))
    return fail(MHC_ERR_UNSUPPORTED, "backward: n = %d streams (2 or 4 supported)", n);
  mhc_status s = check_common(dtype, tokens, d, sinkhorn_iters, norm_eps, hc_eps);
  if (s != MHC_OK) return s;
  if (tokens == 0) return ok();
  const uint64_t es = elem_size(dtype), T = (uint64_t)tokens, nn = (uint64_t)n, nm = n_mix(n);
  const int64_t need = bwd_workspace_bytes(n, tokens, d);
  if (workspace_bytes < need)
    return fail(MHC_ERR_INVALID_ARG, "workspace holds %lld bytes, %lld needed",
                (long long)workspace_bytes, (long long)need);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(MHC_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
  const Span in[] = {
      {"x", x, T * nn * d * es},            {"f", f, T * d * es},
      {"pre_in", pre_in, T * nn * 4},       {"post_in", post_in, T * nn * 4},
      {"comb_in", comb_in, T * nn * nn * 4}, {"x_out", x_out, T * nn * d * es},
      {"mix", mix, T * nm * 4},             {"w_mix", w_mix, nm * nn * d * 4},
      {"base", base, nm * 4},               {"scale", scale, 12},
      {"gamma", gamma, (uint64_t)d * 4},    {"d_x_out", d_x_out, T * nn * d * es},
      {"d_y", d_y, T * d * es},             {"d_pre", d_pre, T * nn * 4},
      {"d_post", d_post, T * nn * 4},       {"d_comb", d_comb, T * nn * nn * 4},
  };
  const Span out[] = {
      {"d_x", d_x, T * nn * d * es},        {"d_f", d_f, T * d * es},
      {"d_pre_in", d_pre_in, T * nn * 4},   {"d_post_in", d_post_in, T * nn * 4},
      {"d_comb_in", d_comb_in, T * nn * nn * 4}, {"d_w_mix", d_w_mix, nm * nn * d * 4},
      {"d_base", d_base, nm * 4},           {"d_scale", d_scale, 12},
      {"d_gamma", d_gamma, (uint64_t)d * 4}, {"workspace", workspace, (uint64_t)need},
  };
  s = check_spans(in, 16, out, 10, nullptr, nullptr);
  if (s != MHC_OK) return s;
  // the backward's regions begin after the forward kernels' header
  float* const bws = reinterpret_cast<float*>(static_cast<char*>(workspace) + fsplit::kWsHeader);
  bwd::Args a{x, f, pre_in, post_in, comb_in, x_out, mix, w_mix, base, scale, gamma, d_x_out,
              d_y, d_pre, d_post, d_comb, d_x, d_f, d_pre_in, d_post_in, d_comb_in, d_w_mix,
              d_base, d_scale, d_gamma, bws, tokens, 0, d,
              sinkhorn_iters, norm_eps, hc_eps};
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (n == 2)
    return dtype == MHC_BF16 ? run_backward<2, MHC_BF16>(a, st) : run_backward<2, MHC_F32>(a, st);
  return dtype == MHC_BF16 ? run_backward<4, MHC_BF16>(a, st) : run_backward<4, MHC_F32>(a, st);
}

}  // extern "C"
