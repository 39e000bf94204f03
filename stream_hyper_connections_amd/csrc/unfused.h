// The step as separate kernels, in the order the pages run them ([RN] Code,
// Block.forward): hc_post, hc_mixes (mhc_mixes), hc_pre, RMSNorm. Every kernel
// reads its inputs from HBM and writes its outputs back, so the streams move
// (4n+4)*d elements per token instead of the fused step's (2n+2)*d ([SW] "Why").
// These are the comparison the fused kernels are measured against; their
// per-element arithmetic is the fused kernels' (same operation order and
// rounding points), so the new streams and h agree bit for bit.
//
// Included by mhc.hip (one translation unit).

namespace unfused {

constexpr int kThreads = 256;

// lanes of a chunk: 8 consecutive features of one token
template <int DT>
struct Chunk;
template <>
struct Chunk<MHC_BF16> {
  u32x4 v;
  __device__ __forceinline__ void load(const void* base, int64_t elem) {
    v = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + elem);
  }
  __device__ __forceinline__ float get(int i) const { return (i & 1) ? bf_hi(v[i >> 1]) : bf_lo(v[i >> 1]); }
};
template <>
struct Chunk<MHC_F32> {
  f32x4 a, b;
  __device__ __forceinline__ void load(const void* base, int64_t elem) {
    const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + elem);
    a = p[0];
    b = p[1];
  }
  __device__ __forceinline__ float get(int i) const { return i < 4 ? a[i] : b[i - 4]; }
};

// Round 8 floats to the stream dtype and store them at element `elem`.
template <int DT>
__device__ __forceinline__ void put8(void* base, int64_t elem, const float (&v)[8]) {
  if constexpr (DT == MHC_BF16) {
    st16(static_cast<uint16_t*>(base) + elem,
         u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
               pack_bf16x2(v[6], v[7])});
  } else {
    float* p = static_cast<float*>(base) + elem;
    st4f(p, f32x4{v[0], v[1], v[2], v[3]});
    st4f(p + 4, f32x4{v[4], v[5], v[6], v[7]});
  }
}

// hc_post ([SW] Code, hc_post): x_out[t][k] = S(sum_j comb[t][j][k] x[t][j] +
// post[t][k] f[t]). One thread per (token, 8-feature chunk); a wave covers a
// contiguous 1 KB (bf16) of one stream row per load.
template <int DT>
__global__ __launch_bounds__(kThreads) void hc_post_kernel(const void* __restrict__ x,
                                                           const void* __restrict__ f,
                                                           const float* __restrict__ post_in,
                                                           const float* __restrict__ comb_in,
                                                           int64_t tokens, int d,
                                                           void* __restrict__ x_out) {
  const int cpr = d / 8;   // chunks per row
  const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (gid >= tokens * cpr) return;
  const int64_t t = gid / cpr;
  const int f0 = (int)(gid % cpr) * 8;
  float C[4][4], U[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f32x4 cv = *reinterpret_cast<const f32x4*>(comb_in + t * 16 + 4 * j);
#pragma unroll
    for (int k = 0; k < 4; ++k) C[j][k] = cv[k];
  }
  const f32x4 u = *reinterpret_cast<const f32x4*>(post_in + t * 4);
#pragma unroll
  for (int k = 0; k < 4; ++k) U[k] = u[k];
  Chunk<DT> xs[4], fs;
#pragma unroll
  for (int j = 0; j < 4; ++j) xs[j].load(x, (t * 4 + j) * d + f0);
  fs.load(f, t * d + f0);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float v = xs[0].get(i) * C[0][k];
#pragma unroll
      for (int j = 1; j < 4; ++j) v = fmaf(xs[j].get(i), C[j][k], v);
      o[i] = fmaf(fs.get(i), U[k], v);
    }
    put8<DT>(x_out, (t * 4 + k) * d + f0, o);
  }
}

// hc_pre ([SW] Code, hc_pre): h[t] = S(sum_k pre[t][k] x[t][k]).
template <int DT>
__global__ __launch_bounds__(kThreads) void hc_pre_kernel(const void* __restrict__ x,
                                                          const float* __restrict__ pre_in,
                                                          int64_t tokens, int d,
                                                          void* __restrict__ h_out) {
  const int cpr = d / 8;
  const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (gid >= tokens * cpr) return;
  const int64_t t = gid / cpr;
  const int f0 = (int)(gid % cpr) * 8;
  const f32x4 p = *reinterpret_cast<const f32x4*>(pre_in + t * 4);
  Chunk<DT> xs[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) xs[k].load(x, (t * 4 + k) * d + f0);
  float o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float h = p[0] * xs[0].get(i);
#pragma unroll
    for (int k = 1; k < 4; ++k) h = fmaf(p[k], xs[k].get(i), h);
    o[i] = h;
  }
  put8<DT>(h_out, t * d + f0, o);
}

// RMSNorm ([RN] formula and Code, RMSNorm): y[t] = S(gamma * (h[t] * rh)),
// rh = 1/sqrt(mean(h[t]^2) + eps). One wave per token: pass 1 sums h^2 over the
// row (lane chunks l, l+64, ...), pass 2 rereads the row (cache-resident) and
// scales it.
template <int DT>
__global__ __launch_bounds__(kThreads) void rmsnorm_kernel(const void* __restrict__ h,
                                                           const float* __restrict__ gamma,
                                                           int64_t tokens, int d, float eps,
                                                           void* __restrict__ y_out) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (t >= tokens) return;
  const int cpr = d / 8;
  float ss = 0.f;
  for (int c = lane; c < cpr; c += 64) {
    Chunk<DT> hc;
    hc.load(h, t * d + 8 * c);
#pragma unroll
    for (int i = 0; i < 8; ++i) ss = fmaf(hc.get(i), hc.get(i), ss);
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) ss += __shfl_xor(ss, m);
  const float rh = rsqrtf(ss / (float)d + eps);
  for (int c = lane; c < cpr; c += 64) {
    Chunk<DT> hc;
    hc.load(h, t * d + 8 * c);
    const f32x4 g0 = *reinterpret_cast<const f32x4*>(gamma + 8 * c);
    const f32x4 g1 = *reinterpret_cast<const f32x4*>(gamma + 8 * c + 4);
    const float gv[8] = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};
    float o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = gv[i] * (hc.get(i) * rh);
    put8<DT>(y_out, t * d + 8 * c, o);
  }
}

}  // namespace unfused
