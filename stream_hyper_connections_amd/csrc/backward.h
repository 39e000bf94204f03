// Backward of the fused step, for n in {2, 4} streams. The pages define the
// forward only ([SW] "All 5 steps" and Code; [RN] formula and Code); the
// gradient follows from those definitions by the chain rule, with the casts to
// the stream dtype passing gradients through unchanged. Per token, with
// forward values X' (the stored new streams), h = S(sum_k p_k X'_k),
// r = (mean X'^2 + eps)^-1/2, rho = (mean h^2 + eps)^-1/2 and m (the mixes):
//
//   g      = gradient at the split's pre-activations a = scale * m + base
//            (sigmoid derivatives; the unrolled Sinkhorn in reverse; the
//            row softmax)                                  split_kernel
//   r, rho, S = sum_f dy gamma h                             stats_kernel
//   V = r * scale * g, dr = (scale * g) . m / r, c = dr r^3 / (n d),
//   kappa = rho^3 S / d
//   dh     = rho gamma dy - kappa h
//   dA_k   = dX'_k + (W^T V)_k - c X'_k + p_k dh
//   dX_j   = S(sum_k C[j][k] dA_k), dF = S(sum_k u_k dA_k)
//   d comb_in[j][k] = sum_f X_j dA_k, d post_in_k = sum_f F dA_k,
//   d pre_in_k = sum_f dh X'_k                    row_kernel / stream_kernel
//   d gamma[f] = sum_t dy h rho (per-workgroup partials)    the same
//   dW[i][k d + f] = sum_t V_i X'_k[f]                       param_kernel
//   d base_i = sum_t g_i, d scale = sums of g_i m_i per group
//                                                slot_kernel, scale_kernel
//
// Two stream kernels compute the same arithmetic. row_kernel (bf16 streams,
// d % 64 == 0) gives each wave 8 tokens and each lane 8 features of one
// token, so that every load and store moves whole 128-byte row segments;
// stream_kernel (the other cases) follows the general-n block kernel: a
// workgroup owns 128 tokens, each wave 16 of them over all features. In both
// W^T V is a product over the (2+n)n slots, computed with
// v_mfma_f32_16x16x32_bf16 on exact three-term bf16 splits of W and of V, with
// the weights as the A operand (rows = features) and V as the B operand
// (columns = tokens). Reductions over
// tokens (dW, d gamma, d base, d scale) are written as per-chunk partial sums
// and added in a fixed order: the results are deterministic.
//
// Included by mhc.hip after general_n.h.

namespace bwd {

// Per-token coefficient gradients (M floats, M even), written in 16-byte
// pieces through the guarded store where M fills whole pieces, else as 8-byte
// stores (a store of up to 64 bits needs no guard).
template <int M>
__device__ __forceinline__ void put_coef(float* p, const float (&v)[M]) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  if constexpr (M % 4 == 0) {
#pragma unroll
    for (int i = 0; i < M; i += 4) st4f(p + i, f32x4{v[i], v[i + 1], v[i + 2], v[i + 3]});
  } else {
#pragma unroll
    for (int i = 0; i < M; i += 2) *reinterpret_cast<f32x2_t*>(p + i) = f32x2_t{v[i], v[i + 1]};
  }
}

constexpr int kTok = gen::kTok;
constexpr int kWaves = gen::kWaves;
constexpr int kThreads = gen::kThreads;
constexpr int kBlock = gen::kBlock;
constexpr int kStep = gen::kStep;
constexpr int kParamChunks = 16;   // token chunks of the parameter kernel
constexpr int kRowTok = 8;                      // tokens per wave of the row kernel
constexpr int kRowBlock = kWaves * kRowTok;     // tokens per workgroup of the row kernel
constexpr int kUnit = 64;                       // features per unit of the row kernel
constexpr int kSlotChunks = 256;   // token chunks of the slot sums

template <int N>
struct Dims {
  static constexpr int kMix = (2 + N) * N;
  static constexpr int kSlots = 32;   // the K of one bf16 MFMA, (2+n)n padded
  static_assert(kMix <= kSlots, "the backward covers n <= 4");
  static constexpr int kVecs = N * 2 * 3 * 64;    // u32x4 of one step's W^T (3 terms)
  static constexpr int kItems = N * kSlots * 8;   // f32x4 loads staging one step
  static constexpr int kStage = (kItems + kThreads - 1) / kThreads;
};

// Workspace (floats, each region 256-byte aligned).
__host__ __device__ constexpr int64_t al64(int64_t v) { return (v + 63) / 64 * 64; }
template <int N>
struct Ws {
  int64_t tokens;
  int d;
  __host__ __device__ int64_t g_off() const { return 0; }
  __host__ __device__ int64_t v_off() const { return g_off() + al64(tokens * Dims<N>::kMix); }
  __host__ __device__ int64_t st_off() const {
    return v_off() + al64((tokens + 31) / 32 * 32 * Dims<N>::kSlots);
  }
  __host__ __device__ int64_t pw_off() const { return st_off() + al64(tokens * 4); }
  // d gamma partials: one row per workgroup of the stream kernel (64 or 128
  // tokens); sized for the smaller blocks
  __host__ __device__ int64_t groups() const { return (tokens + kRowBlock - 1) / kRowBlock; }
  __host__ __device__ int64_t pg_off() const {
    return pw_off() + al64((int64_t)kParamChunks * Dims<N>::kMix * N * d);
  }
  __host__ __device__ int64_t e_off() const { return pg_off() + al64(groups() * d); }
  __host__ __device__ int64_t wt_off() const {
    return e_off() + al64((int64_t)kSlotChunks * 2 * Dims<N>::kMix);
  }
  // packed W^T of the row kernel: 32 floats per feature and stream
  __host__ __device__ int64_t floats() const { return wt_off() + al64((int64_t)d * N * 32); }
};

// V[t][slot] in the workspace: blocks of 32 tokens, slot-major inside a block,
// so that 8 consecutive tokens of one slot are 32 contiguous bytes.
template <int N>
__host__ __device__ __forceinline__ int64_t vidx(int64_t t, int slot) {
  return ((t >> 5) * Dims<N>::kSlots + slot) * 32 + (t & 31);
}

// Tokens per chunk of the parameter kernels: a multiple of 32.
__host__ __device__ __forceinline__ int64_t param_per(int64_t tokens) {
  return ((tokens + kParamChunks - 1) / kParamChunks + 31) / 32 * 32;
}

struct Args {
  const void* x;
  const void* f;
  const float* pre_in;
  const float* post_in;
  const float* comb_in;
  const void* x_out;
  const float* mix;
  const float* w;
  const float* base;
  const float* scale;
  const float* gamma;
  const void* dxo;
  const void* dy;
  const float* d_pre;
  const float* d_post;
  const float* d_comb;
  void* dx;
  void* df;
  float* d_pre_in;
  float* d_post_in;
  float* d_comb_in;
  float* d_w;
  float* d_base;
  float* d_scale;
  float* d_gamma;
  float* ws;
  int64_t tokens;
  int64_t dg_groups;   // d gamma partial rows written by the stream kernel
  int d;
  int iters;
  float norm_eps;
  float hc_eps;
};

// ----- split / Sinkhorn backward, n^2 lanes per token --------------------------------------

// Sums and maximum over the n lanes of an entry's row (lanes e with the same
// e / n) and over the n lanes of its column (same e % n), within one DPP row
// (n = 4: a token is one 16-lane row; n = 2: one quad).
template <int N>
__device__ __forceinline__ float row_sum(float v) {
  if constexpr (N == 4) return pipe::quad_sum(v);
  else return v + pipe::dpp<pipe::kQuadSwap1>(v);
}
template <int N>
__device__ __forceinline__ float row_max(float v) {
  if constexpr (N == 4) return pipe::quad_max(v);
  else return fmaxf(v, pipe::dpp<pipe::kQuadSwap1>(v));
}
template <int N>
__device__ __forceinline__ float col_sum(float v) {
  if constexpr (N == 4) return pipe::col_sum(v);
  else return v + pipe::dpp<pipe::kQuadSwap2>(v);
}

// Gradient g at the split's pre-activations of (pre, post, comb) =
// split_sinkhorn(m): lane e of a token's n^2 lanes holds comb entry
// (e / n, e % n), and lanes e < 2n also the pre (e < n) or post slot.
// Step k of the comb's normalisations divides the columns (k = 0 and even k)
// or the rows (odd k) by (sum + eps), here as a product with the hardware
// reciprocal, as the forward kernels do. The reverse pass recomputes each step's
// output from the nearest of kCp checkpoints (the matrices entering every
// seg-th step). For Y = X / (sum + eps) along an axis, dX = (dY - sum_axis(dY
// * Y)) / (sum + eps); for P = softmax(L) along rows, dL = P * (dP -
// sum_row(dP * P)). Every lane stays active (the sums are DPP lane
// exchanges); lanes of tokens past the end compute on token 0 and store
// nothing.
template <int N>
__global__ __launch_bounds__(256) void split_kernel(Args a) {
  constexpr int kMix = Dims<N>::kMix;
  constexpr int kE = N * N;
  constexpr int kCp = 8;
  static_assert(N == 2 || N == 4, "one DPP row or quad per token");
  const int e = threadIdx.x % kE;
  const int64_t t = (int64_t)blockIdx.x * (256 / kE) + threadIdx.x / kE;
  const bool ok = t < a.tokens;
  const int64_t tc = ok ? t : 0;
  const float* m = a.mix + tc * kMix;
  float* g = a.ws + tc * kMix;   // region g at offset 0
  if (e < N) {
    const float sp = sigmoidf(m[e] * a.scale[0] + a.base[e]);
    if (ok) g[e] = a.d_pre[tc * N + e] * sp * (1.0f - sp);
  } else if (e < 2 * N) {
    const float sq = sigmoidf(m[e] * a.scale[1] + a.base[e]);
    if (ok) g[e] = a.d_post[tc * N + (e - N)] * 2.0f * sq * (1.0f - sq);
  }
  // the row softmax of the comb logits
  const float lg = m[2 * N + e] * a.scale[2] + a.base[2 * N + e];
  const float ex = expf(lg - row_max<N>(lg));
  const float p = ex / row_sum<N>(ex);
  float dc = a.d_comb[tc * kE + e];
  const float eps = a.hc_eps;
  auto axis_sum = [&](int q, float v) {
    return (q == 0 || (q & 1) == 0) ? col_sum<N>(v) : row_sum<N>(v);
  };
  const int nsteps = 2 * a.iters - 1;
  const int seg = (nsteps + kCp - 1) / kCp;
  float ck[kCp];
  {
    float c = p + eps;
#pragma unroll
    for (int cp = 0; cp < kCp; ++cp) {
      ck[cp] = c;
      const int hi = (cp + 1) * seg < nsteps ? (cp + 1) * seg : nsteps;
      for (int q = cp * seg; q < hi; ++q) c = c * __builtin_amdgcn_rcpf(axis_sum(q, c) + eps);
    }
  }
#pragma unroll
  for (int cp = kCp - 1; cp >= 0; --cp) {
    const int lo = cp * seg;
    const int hi = lo + seg < nsteps ? lo + seg : nsteps;
    for (int step = hi - 1; step >= lo; --step) {
      float c = ck[cp], r = 1.f;
      for (int q = lo; q <= step; ++q) {   // c = output of `step`, r = 1 / its divisor
        r = __builtin_amdgcn_rcpf(axis_sum(q, c) + eps);
        c = c * r;
      }
      const float dot = axis_sum(step, dc * c);
      dc = (dc - dot) * r;
    }
  }
  // dc is now the gradient of softmax + eps, i.e. of p
  const float dot = row_sum<N>(dc * p);
  if (ok) g[2 * N + e] = p * (dc - dot);
}

// ----- per-token statistics, one wave per token ----------------------------------------

// 8 consecutive stream elements as floats.
template <int DT>
__device__ __forceinline__ void load8(const void* base, int64_t elem, float (&v)[8]) {
  if constexpr (DT == MHC_BF16) {
    // non-temporal: the statistics pass reads X' and dy once (with the dW
    // kernel's loads also non-temporal: 3.411 -> 3.317 ms per backward call)
    const u32x4 w = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + elem));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf_lo(w[i]);
      v[2 * i + 1] = bf_hi(w[i]);
    }
  } else {
    const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + elem);
    const f32x4 lo = p[0], hi = p[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = lo[i];
      v[4 + i] = hi[i];
    }
  }
}

// Round to the stream dtype (RNE), as the forward does.
template <int DT>
__device__ __forceinline__ void round8(float (&v)[8]) {
  if constexpr (DT == MHC_BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w = pack_bf16x2(v[2 * i], v[2 * i + 1]);
      v[2 * i] = bf_lo(w);
      v[2 * i + 1] = bf_hi(w);
    }
  }
}

// r, rho and S = sum_f dy gamma h of each token, from the stored new streams
// (h is recomputed with the forward's operation order and rounding).
template <int N, int DT>
__global__ __launch_bounds__(256) void stats_kernel(Args a) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.tokens) return;
  const int d = a.d;
  float P[N];
#pragma unroll
  for (int k = 0; k < N; ++k) P[k] = a.pre_in[t * N + k];
  float sx = 0.f, sh = 0.f, sd = 0.f;
  for (int f0 = 8 * lane; f0 < d; f0 += 512) {
    float xp[N][8], dy[8];
#pragma unroll
    for (int k = 0; k < N; ++k) load8<DT>(a.x_out, (t * N + k) * (int64_t)d + f0, xp[k]);
    load8<DT>(a.dy, t * (int64_t)d + f0, dy);
    float h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = P[0] * xp[0][e];
#pragma unroll
      for (int k = 1; k < N; ++k) v = fmaf(P[k], xp[k][e], v);
      h[e] = v;
#pragma unroll
      for (int k = 0; k < N; ++k) sx = fmaf(xp[k][e], xp[k][e], sx);
    }
    round8<DT>(h);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sh = fmaf(h[e], h[e], sh);
      sd = fmaf(dy[e] * a.gamma[f0 + e], h[e], sd);
    }
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    sx += __shfl_xor(sx, o);
    sh += __shfl_xor(sh, o);
    sd += __shfl_xor(sd, o);
  }
  if (lane == 0) {
    Ws<N> w{a.tokens, d};
    st4f(a.ws + w.st_off() + t * 4,
         f32x4{rsqrtf(sx / (float)(N * d) + a.norm_eps), rsqrtf(sh / (float)d + a.norm_eps), sd,
               0.f});
  }
}

// ----- the stream kernel ----------------------------------------------------------------

// One step's W^T in the A-operand order of v_mfma_f32_16x16x32_bf16, as
// three exact bf16 terms (hi, mid, lo): u32x4 index ((k * 2 + q) * 3 + term)
// * 64 + lane holds, in bf16 element e, the term of
// W[8 (lane / 16) + e][k d + 32 s + feat(q, lane % 16)] with
// feat(q, rho) = 8 (rho / 4) + 4 q + rho % 4, so that the product's rows
// 4g..4g+3 are features 8g + 4q + 0..3 (the lane's own features).
// Staging item i = ((k * kSlots) + slot) * 8 + c8 covers features 4 c8..4 c8+3.
template <int N>
__device__ __forceinline__ void stage_load(f32x4 (&st)[Dims<N>::kStage], const float* w, int d,
                                           int s, int tid) {
  using D = Dims<N>;
#pragma unroll
  for (int r = 0; r < D::kStage; ++r) {
    const int i = tid + r * kThreads;
    const int c8 = i & 7;
    const int slot = (i >> 3) % D::kSlots;
    const int k = (i >> 3) / D::kSlots;
    st[r] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (i < D::kItems && slot < D::kMix)
      st[r] = *reinterpret_cast<const f32x4*>(w + (int64_t)slot * N * d + (int64_t)k * d +
                                              s * kStep + 4 * c8);
  }
}

// The three bf16 terms of x: hi = bf16(x), mid = bf16(x - hi), lo = x - hi - mid
// (both differences exact in float32; hi + mid + lo == x), as bits.
__device__ __forceinline__ void split3(float x, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  const float h = __uint_as_float(pack_bf16x2(x, 0.f) << 16);
  const float r1 = x - h;
  const float m = __uint_as_float(pack_bf16x2(r1, 0.f) << 16);
  hi = pack_bf16x2(x, 0.f) & 0xffffu;
  mid = pack_bf16x2(r1, 0.f) & 0xffffu;
  lo = pack_bf16x2(r1 - m, 0.f) & 0xffffu;
}

template <int N>
__device__ __forceinline__ void stage_store(uint16_t* wl, const f32x4 (&st)[Dims<N>::kStage],
                                            int tid) {
  using D = Dims<N>;
#pragma unroll
  for (int r = 0; r < D::kStage; ++r) {
    const int i = tid + r * kThreads;
    if (i >= D::kItems) continue;
    const int c8 = i & 7;
    const int slot = (i >> 3) % D::kSlots;
    const int k = (i >> 3) / D::kSlots;
    const int q = c8 & 1;                 // features 4 c8 .. 4 c8 + 3: 8 (c8 / 2) + 4 q + 0..3
    const int rho0 = 4 * (c8 >> 1);       // rows rho0 .. rho0 + 3
    const int e = slot & 7, gq = slot >> 3;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int lane = rho0 + u + 16 * gq;
      uint32_t t3[3];
      split3(st[r][u], t3[0], t3[1], t3[2]);
#pragma unroll
      for (int term = 0; term < 3; ++term)
        wl[((((k * 2 + q) * 3 + term) * 64 + lane) << 3) + e] = (uint16_t)t3[term];
    }
  }
}

template <int N, int DT>
__global__ __launch_bounds__(kThreads) void stream_kernel(Args a) {
  using D = Dims<N>;
  constexpr int kMix = D::kMix;
  constexpr int es = DT == MHC_BF16 ? 2 : 4;
  __shared__ __align__(16) uint16_t wl[2][D::kVecs * 8];
  __shared__ float red[2][kWaves][kStep];   // per-wave d gamma sums of one step

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tr = lane & 15;
  const int g = lane >> 4;
  const int64_t tw = (int64_t)blockIdx.x * kBlock + wave * kTok;
  const int64_t t = tw + tr;
  const bool valid = t < a.tokens;
  const int64_t tc = valid ? t : 0;   // a valid row for the per-token loads
  const int d = a.d;
  const int nsteps = d / kStep;
  Ws<N> wsl{a.tokens, d};

  f32x4 st[D::kStage];
  stage_load<N>(st, a.w, d, 0, tid);

  // per-token constants
  float C[N][N], U[N], P[N];
#pragma unroll
  for (int j = 0; j < N; ++j)
#pragma unroll
    for (int k = 0; k < N; ++k) C[j][k] = a.comb_in[(tc * N + j) * N + k];
#pragma unroll
  for (int k = 0; k < N; ++k) {
    U[k] = a.post_in[tc * N + k];
    P[k] = a.pre_in[tc * N + k];
  }
  const float* stt = a.ws + wsl.st_off() + tc * 4;
  const float r = stt[0], rho = stt[1], ssum = stt[2];
  const float* gr = a.ws + wsl.g_off() + tc * kMix;
  const float* mr = a.mix + tc * kMix;
  float dmm = 0.f;   // (scale * g) . m
#pragma unroll
  for (int i = 0; i < kMix; ++i) {
    const float sc = i < N ? a.scale[0] : (i < 2 * N ? a.scale[1] : a.scale[2]);
    dmm = fmaf(sc * gr[i], mr[i], dmm);
  }
  const float cr = dmm * r * r / (float)(N * d);       // dr r^3 / (n d), dr = dmm / r
  const float kappa = rho * rho * rho * ssum / (float)d;
  // B operand: V[slot 8g + e] of the lane's token, as three bf16 terms
  typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
  bf16x8_t vb[3];
  {
    u32x4 w3[3];
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      uint32_t tt[2][3];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int i = 8 * g + 2 * e2 + u;
        const float sc = i < N ? a.scale[0] : (i < 2 * N ? a.scale[1] : a.scale[2]);
        const float vi = i < kMix ? r * sc * gr[i < kMix ? i : 0] : 0.f;
        split3(vi, tt[u][0], tt[u][1], tt[u][2]);
        // V for the parameter kernel: lane g writes the slots it holds
        if (valid) a.ws[wsl.v_off() + vidx<N>(t, i)] = vi;
      }
#pragma unroll
      for (int term = 0; term < 3; ++term) w3[term][e2] = tt[0][term] | (tt[1][term] << 16);
    }
#pragma unroll
    for (int term = 0; term < 3; ++term) vb[term] = __builtin_bit_cast(bf16x8_t, w3[term]);
  }

  stage_store<N>(wl[0], st, tid);
  __syncthreads();

  float dC[N][N], du[N], dp[N];
#pragma unroll
  for (int k = 0; k < N; ++k) {
    du[k] = dp[k] = 0.f;
#pragma unroll
    for (int j = 0; j < N; ++j) dC[j][k] = 0.f;
  }

  const int64_t xrow = (int64_t)N * d, frow = d;
  for (int s = 0; s < nsteps; ++s) {
    const int f0 = s * kStep + 8 * g;
    if (s + 1 < nsteps) stage_load<N>(st, a.w, d, s + 1, tid);
    // lane inputs (8 features of the token)
    float xv[N][8], dxo[N][8], fv[8], dyv[8];
#pragma unroll
    for (int j = 0; j < N; ++j) {
      load8<DT>(a.x, tc * xrow + j * (int64_t)d + f0, xv[j]);
      load8<DT>(a.dxo, tc * xrow + j * (int64_t)d + f0, dxo[j]);
    }
    load8<DT>(a.f, tc * frow + f0, fv);
    load8<DT>(a.dy, tc * frow + f0, dyv);
    const f32x4 g0 = *reinterpret_cast<const f32x4*>(a.gamma + f0);
    const f32x4 g1 = *reinterpret_cast<const f32x4*>(a.gamma + f0 + 4);
    const float gv[8] = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};

    // W^T V for the lane's features: tile q gives features 8g + 4q + 0..3.
    // Six of the nine term products (the three dropped ones are below 2^-24
    // of the product).
    const u32x4* wb = reinterpret_cast<const u32x4*>(wl[s & 1]);
    float dxm[N][8];
#pragma unroll
    for (int k = 0; k < N; ++k) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const bf16x8_t w0 = __builtin_bit_cast(bf16x8_t, wb[((k * 2 + q) * 3 + 0) * 64 + lane]);
        const bf16x8_t w1 = __builtin_bit_cast(bf16x8_t, wb[((k * 2 + q) * 3 + 1) * 64 + lane]);
        const bf16x8_t w2 = __builtin_bit_cast(bf16x8_t, wb[((k * 2 + q) * 3 + 2) * 64 + lane]);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w2, vb[0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w0, vb[2], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w1, vb[1], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w1, vb[0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w0, vb[1], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w0, vb[0], acc, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) dxm[k][4 * q + i] = acc[i];
      }
    }

    // recompute X' and h exactly as the forward did
    float xp[N][8], h[8];
#pragma unroll
    for (int k = 0; k < N; ++k) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float v = xv[0][e] * C[0][k];
#pragma unroll
        for (int j = 1; j < N; ++j) v = fmaf(xv[j][e], C[j][k], v);
        xp[k][e] = fmaf(fv[e], U[k], v);
      }
      round8<DT>(xp[k]);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = P[0] * xp[0][e];
#pragma unroll
      for (int k = 1; k < N; ++k) v = fmaf(P[k], xp[k][e], v);
      h[e] = v;
    }
    round8<DT>(h);

    float dxj[N][8], dfv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // d gamma: sum over the wave's 16 tokens (lanes of one 16-lane row)
      float dg = valid ? dyv[e] * h[e] * rho : 0.f;
      dg += __shfl_xor(dg, 1);
      dg += __shfl_xor(dg, 2);
      dg += __shfl_xor(dg, 4);
      dg += __shfl_xor(dg, 8);
      if (tr == 0) red[s & 1][wave][8 * g + e] = dg;
      const float dh = rho * (gv[e] * dyv[e]) - kappa * h[e];
      float da[N];
#pragma unroll
      for (int k = 0; k < N; ++k) {
        da[k] = dxo[k][e] + (dxm[k][e] - cr * xp[k][e]) + P[k] * dh;
        dp[k] = fmaf(dh, xp[k][e], dp[k]);
        du[k] = fmaf(fv[e], da[k], du[k]);
#pragma unroll
        for (int j = 0; j < N; ++j) dC[j][k] = fmaf(xv[j][e], da[k], dC[j][k]);
      }
#pragma unroll
      for (int j = 0; j < N; ++j) {
        float v = C[j][0] * da[0];
#pragma unroll
        for (int k = 1; k < N; ++k) v = fmaf(C[j][k], da[k], v);
        dxj[j][e] = v;
      }
      float v = U[0] * da[0];
#pragma unroll
      for (int k = 1; k < N; ++k) v = fmaf(U[k], da[k], v);
      dfv[e] = v;
    }
    if (valid) {
#pragma unroll
      for (int j = 0; j < N; ++j)
        unfused::put8<DT>(a.dx, tc * xrow + j * (int64_t)d + f0, dxj[j]);
      unfused::put8<DT>(a.df, tc * frow + f0, dfv);
    }

    // next step's W^T into the other buffer (read two steps ago; every wave
    // passed the barrier at the end of the previous step since)
    if (s + 1 < nsteps) stage_store<N>(wl[(s + 1) & 1], st, tid);
    __syncthreads();
    // the workgroup's d gamma partial of this step's features (red[s & 1] is
    // rewritten two steps later, after the next barrier)
    if (wave == 0 && lane < kStep) {
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) v += red[s & 1][w][lane];
      a.ws[wsl.pg_off() + (int64_t)blockIdx.x * d + s * kStep + lane] = v;
    }
  }

  // per-token sums over the 4 lanes of a token
#pragma unroll
  for (int k = 0; k < N; ++k) {
    dp[k] += __shfl_xor(dp[k], 16);
    dp[k] += __shfl_xor(dp[k], 32);
    du[k] += __shfl_xor(du[k], 16);
    du[k] += __shfl_xor(du[k], 32);
#pragma unroll
    for (int j = 0; j < N; ++j) {
      dC[j][k] += __shfl_xor(dC[j][k], 16);
      dC[j][k] += __shfl_xor(dC[j][k], 32);
    }
  }
  if (valid && g == 0) {
    put_coef<N>(a.d_pre_in + t * N, dp);
    put_coef<N>(a.d_post_in + t * N, du);
    float dcr[N * N];
#pragma unroll
    for (int j = 0; j < N; ++j)
#pragma unroll
      for (int k = 0; k < N; ++k) dcr[j * N + k] = dC[j][k];
    put_coef<N * N>(a.d_comb_in + t * N * N, dcr);
  }
}

// ----- the stream kernel on whole 128-byte rows (bf16, d % 64 == 0) -------------------
//
// Same arithmetic as stream_kernel, another layout. A workgroup owns 64
// tokens, each wave 8 of them; features go in units of 64 (128 bytes of every
// row). Lane l holds token l / 8 of the wave and features 8 (l % 8) .. +7 of
// the unit, so that one load or store instruction moves 8 whole 128-byte row
// segments (as a plain copy on the MI355X: 5.0 TB/s, against 2.8 TB/s for 16
// rows x 64 bytes, the MFMA result order).
//
// W^T V runs on v_mfma_f32_16x16x32_bf16 with W^T as A (rows = 16 features of
// one stream, K = the 32 slots; two bf16 terms w0, w1, packed once per call in
// operand order by wt_pack_kernel) and V as B: columns 0-7 are the wave's
// tokens with V's terms (v0 | v2), columns 8-15 the same tokens with (v1 | 0).
// The products (w0 w1) x (v0 | v1) and w0 x (v2 | 0) leave out term pairs
// below 2^-18 of each product (W's third term, w1 v2): a relative error far
// below the float32-level tolerance of the gradients (1e-4 of the magnitude
// of their terms), at two thirds of the W^T staging traffic of three terms.
// The two column halves are added (DPP), and a 2 KB per-wave LDS buffer turns
// the result (4 features of one token per lane) into the lane layout above. Each unit's packed W^T and
// gamma are staged in LDS (double-buffered) one unit ahead, with the next
// unit's stream loads issued after the product phase, ahead of the current
// unit's elementwise arithmetic; the one barrier per unit waits for LDS
// traffic only, so loads and stores stay in flight across it. Register
// budget (n = 4: 256 VGPRs, none spilled): the coefficients are re-read from
// LDS each unit, and empty asm statements keep the compiler from widening all
// packed inputs at once or sinking the token sums to the end of the unit.

using pipe::bload;
using pipe::bstore;
using pipe::kNT;
using pipe::make_rsrc;
using pipe::rsrc_t;

template <int N>
struct RowDims {
  static constexpr int kWtVecs = N * 4 * 2 * 64;       // u32x4 of one unit's W^T
  static constexpr int kWtPer = kWtVecs / kThreads;    // staged per thread
  static_assert(kWtPer * kThreads == kWtVecs, "whole staging rounds");
};

// Packed W^T: u32x4 index (((u N + k) 4 + q) 2 + term) 64 + lane holds, in bf16
// element e, term `term` (hi = bf16(w), mid = bf16(w - hi)) of
// W[8 (lane / 16) + e][k d + 64 u + 16 q + lane % 16] (zero for slots >=
// (2+n)n). |w - hi - mid| <= 2^-18 |w|.
template <int N>
__global__ __launch_bounds__(256) void wt_pack_kernel(const float* __restrict__ w, int d,
                                                      int64_t total, u32x4* __restrict__ out) {
  constexpr int kMix = Dims<N>::kMix;
  const int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (v >= total) return;
  const int lane = (int)(v & 63);
  const int term = (int)((v >> 6) & 1);
  const int64_t uq = (v >> 6) >> 1;   // (u N + k) 4 + q
  const int q = (int)(uq & 3);
  const int64_t uk = uq >> 2;
  const int k = (int)(uk % N);
  const int64_t u = uk / N;
  const int64_t col = (int64_t)k * d + 64 * u + 16 * q + (lane & 15);
  uint32_t h[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int slot = 8 * (lane >> 4) + e;
    uint32_t t3[3] = {0u, 0u, 0u};
    if (slot < kMix) split3(w[(int64_t)slot * N * d + col], t3[0], t3[1], t3[2]);
    h[e] = term == 0 ? t3[0] : t3[1];
  }
  st16(out + v, u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                      h[6] | (h[7] << 16)});
}

// Barrier for LDS traffic only: waits for the wave's LDS operations, not for
// its outstanding global loads and stores.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int N>
__global__ __launch_bounds__(kThreads) void row_kernel(Args a) {
  using D = Dims<N>;
  using R = RowDims<N>;
  constexpr int kMix = D::kMix;
  typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
  __shared__ __align__(16) u32x4 wt[2][R::kWtVecs];
  __shared__ __align__(16) float gm[2][kUnit];
  __shared__ __align__(16) float tr[kWaves][kRowTok][kUnit + 4];
  __shared__ float red[2][kWaves][kUnit];
  constexpr int kCoef = N * N + 2 * N;   // comb_in, post_in, pre_in of a token
  __shared__ __align__(16) float cst[kWaves][kRowTok][kCoef];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m8 = lane >> 3, x8 = lane & 7;     // stream layout: token, 16-byte chunk
  const int col = lane & 15, rg = lane >> 4;   // MFMA layout: column, row group
  const int d = a.d;
  const int nu = d / kUnit;
  const int64_t tw = (int64_t)blockIdx.x * kRowBlock + wave * kRowTok;
  const int64_t t = tw + m8;
  const bool valid = t < a.tokens;
  const int64_t tc = valid ? t : 0;
  Ws<N> wsl{a.tokens, d};
  const u32x4* wpk = reinterpret_cast<const u32x4*>(a.ws + wsl.wt_off());

  // buffer resources over the wave's rows (rows past the end read zeros,
  // stores to them are dropped)
  const int ntok = (int)max<int64_t>(0, min<int64_t>(kRowTok, a.tokens - tw));
  const uint32_t rowx = (uint32_t)(N * d * 2), rowf = (uint32_t)(d * 2), d2 = (uint32_t)(d * 2);
  const int64_t tws = ntok > 0 ? tw : 0;
  const rsrc_t rx = make_rsrc(static_cast<const char*>(a.x) + tws * rowx, ntok * rowx);
  const rsrc_t rdxo = make_rsrc(static_cast<const char*>(a.dxo) + tws * rowx, ntok * rowx);
  const rsrc_t rf = make_rsrc(static_cast<const char*>(a.f) + tws * rowf, ntok * rowf);
  const rsrc_t rdy = make_rsrc(static_cast<const char*>(a.dy) + tws * rowf, ntok * rowf);
  const rsrc_t rdx = make_rsrc(static_cast<char*>(a.dx) + tws * rowx, ntok * rowx);
  const rsrc_t rdf = make_rsrc(static_cast<char*>(a.df) + tws * rowf, ntok * rowf);
  const uint32_t vx = (uint32_t)m8 * rowx + 16u * x8;
  const uint32_t vf = (uint32_t)m8 * rowf + 16u * x8;

  struct Raw {
    u32x4 x[N], dxo[N], f, dy;
  };
  auto load_raw = [&](Raw& r, int u) {
    const uint32_t cu = 128u * u;
#pragma unroll
    for (int k = 0; k < N; ++k) r.x[k] = bload<kNT>(rx, vx + k * d2, cu);
#pragma unroll
    for (int k = 0; k < N; ++k) r.dxo[k] = bload<kNT>(rdxo, vx + k * d2, cu);
    r.f = bload<kNT>(rf, vf, cu);
    r.dy = bload<kNT>(rdy, vf, cu);
  };
  u32x4 wst[R::kWtPer];
  f32x4 gst = {0.f, 0.f, 0.f, 0.f};
  auto stage_load_w = [&](int u) {
#pragma unroll
    for (int r = 0; r < R::kWtPer; ++r) wst[r] = wpk[(int64_t)u * R::kWtVecs + tid + r * kThreads];
    if (tid < kUnit / 4) gst = *reinterpret_cast<const f32x4*>(a.gamma + kUnit * u + 4 * tid);
  };
  auto stage_store_w = [&](int b) {
#pragma unroll
    for (int r = 0; r < R::kWtPer; ++r) wt[b][tid + r * kThreads] = wst[r];
    if (tid < kUnit / 4) *reinterpret_cast<f32x4*>(&gm[b][4 * tid]) = gst;
  };

  Raw ra, rb;
  stage_load_w(0);
  load_raw(ra, 0);

  // the coefficients of the wave's tokens go to LDS (re-read per unit, so
  // that they hold no registers through the product phase)
  if (x8 == 0) {
#pragma unroll
    for (int i = 0; i < N * N; ++i) cst[wave][m8][i] = a.comb_in[tc * N * N + i];
#pragma unroll
    for (int k = 0; k < N; ++k) {
      cst[wave][m8][N * N + k] = a.post_in[tc * N + k];
      cst[wave][m8][N * N + N + k] = a.pre_in[tc * N + k];
    }
  }
  float cr, kappa, rho;
  {
    const float* stt = a.ws + wsl.st_off() + tc * 4;
    const float r = stt[0];
    rho = stt[1];
    const float ssum = stt[2];
    const float* gr = a.ws + wsl.g_off() + tc * kMix;
    const float* mr = a.mix + tc * kMix;
    float dmm = 0.f;   // (scale * g) . m
#pragma unroll
    for (int i = 0; i < kMix; ++i) {
      const float sc = i < N ? a.scale[0] : (i < 2 * N ? a.scale[1] : a.scale[2]);
      dmm = fmaf(sc * gr[i], mr[i], dmm);
    }
    cr = dmm * r * r / (float)(N * d);   // dr r^3 / (n d), dr = dmm / r
    kappa = rho * rho * rho * ssum / (float)d;
  }
  // B operands (MFMA layout): V[slot 8 rg + e] of token col % 8, as bf16 terms;
  // the lanes of columns 0-7 also write V for the parameter kernel
  bf16x8_t ba, bb;
  {
    const int64_t tv = tw + (col & 7);
    const bool vvalid = tv < a.tokens;
    const int64_t tvc = vvalid ? tv : 0;
    const float rv = a.ws[wsl.st_off() + tvc * 4];
    const float* gr = a.ws + wsl.g_off() + tvc * kMix;
    u32x4 wa, wb;
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      uint32_t tt[2][3];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int i = 8 * rg + 2 * e2 + u;
        const float sc = i < N ? a.scale[0] : (i < 2 * N ? a.scale[1] : a.scale[2]);
        const float vi = i < kMix ? rv * sc * gr[i < kMix ? i : 0] : 0.f;
        split3(vi, tt[u][0], tt[u][1], tt[u][2]);
        if (vvalid && col < 8) a.ws[wsl.v_off() + vidx<N>(tv, i)] = vi;
      }
      const uint32_t v0 = tt[0][0] | (tt[1][0] << 16), v1 = tt[0][1] | (tt[1][1] << 16);
      const uint32_t v2 = tt[0][2] | (tt[1][2] << 16);
      wa[e2] = col < 8 ? v0 : v1;
      wb[e2] = col < 8 ? v2 : 0u;
    }
    ba = __builtin_bit_cast(bf16x8_t, wa);
    bb = __builtin_bit_cast(bf16x8_t, wb);
  }

  stage_store_w(0);
  lds_barrier();

  float dC[N][N], du[N], dp[N];
#pragma unroll
  for (int k = 0; k < N; ++k) {
    du[k] = dp[k] = 0.f;
#pragma unroll
    for (int j = 0; j < N; ++j) dC[j][k] = 0.f;
  }

  Raw& cur = ra;
  Raw& nxt = rb;
  for (int u = 0; u < nu; ++u) {
    const int b = u & 1;
    const bool more = u + 1 < nu;
    // the next unit's W^T and gamma, then its stream rows (vector memory
    // retires in order: the staging loads complete first)
    __builtin_amdgcn_sched_barrier(0);
    if (more) stage_load_w(u + 1);
    __builtin_amdgcn_sched_barrier(0);

    // W^T V of the unit, one stream at a time, through the wave's LDS buffer
    float dxm[N][8];
    const u32x4* wb = wt[b];
#pragma unroll
    for (int k = 0; k < N; ++k) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int base = ((k * 4 + q) * 2) * 64 + lane;
        const bf16x8_t w0 = __builtin_bit_cast(bf16x8_t, wb[base]);
        const bf16x8_t w1 = __builtin_bit_cast(bf16x8_t, wb[base + 64]);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w0, bb, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w1, ba, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w0, ba, acc, 0, 0, 0);
        f32x4 tot;
#pragma unroll
        for (int i = 0; i < 4; ++i) tot[i] = acc[i] + pipe::dpp<pipe::kRowRor8>(acc[i]);
        if (col < 8) *reinterpret_cast<f32x4*>(&tr[wave][col][16 * q + 4 * rg]) = tot;
        __builtin_amdgcn_sched_barrier(0);   // one tile's operands in flight at a time
      }
      __builtin_amdgcn_wave_barrier();
      const f32x4 lo = *reinterpret_cast<const f32x4*>(&tr[wave][m8][8 * x8]);
      const f32x4 hi = *reinterpret_cast<const f32x4*>(&tr[wave][m8][8 * x8 + 4]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dxm[k][i] = lo[i];
        dxm[k][4 + i] = hi[i];
      }
      __builtin_amdgcn_wave_barrier();
    }

    // the next unit's W^T and gamma into the other buffers (last read in the
    // previous unit, before the barrier that ended it), then the next unit's
    // stream rows, in flight through this unit's arithmetic
    if (more) stage_store_w(b ^ 1);
    __builtin_amdgcn_sched_barrier(0);
    if (more) load_raw(nxt, u + 1);

    __builtin_amdgcn_sched_barrier(0);
    const f32x4 g0 = *reinterpret_cast<const f32x4*>(&gm[b][8 * x8]);
    const f32x4 g1 = *reinterpret_cast<const f32x4*>(&gm[b][8 * x8 + 4]);
    const float gv[8] = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};
    float C[N][N], U[N], P[N];
    {
      int ci = m8;
      asm volatile("" : "+v"(ci));   // re-read every unit
      const float* cp = cst[wave][ci];
#pragma unroll
      for (int j = 0; j < N; ++j)
#pragma unroll
        for (int k = 0; k < N; ++k) C[j][k] = cp[j * N + k];
#pragma unroll
      for (int k = 0; k < N; ++k) {
        U[k] = cp[N * N + k];
        P[k] = cp[N * N + N + k];
      }
    }

    // dA (in place of W^T V), the token sums and the d gamma sums, two
    // features at a time (the empty asm keeps the packed words from being
    // widened to floats all at once ahead of their use)
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      uint32_t wx[N], wd[N], wf = cur.f[e2], wy = cur.dy[e2];
#pragma unroll
      for (int j = 0; j < N; ++j) {
        wx[j] = cur.x[j][e2];
        wd[j] = cur.dxo[j][e2];
        asm volatile("" : "+v"(wx[j]), "+v"(wd[j]));
      }
      asm volatile("" : "+v"(wf), "+v"(wy));
#pragma unroll
      for (int hi = 0; hi < 2; ++hi) {
        const int e = 2 * e2 + hi;
        float xv[N];
#pragma unroll
        for (int j = 0; j < N; ++j) xv[j] = hi ? bf_hi(wx[j]) : bf_lo(wx[j]);
        const float fv = hi ? bf_hi(wf) : bf_lo(wf);
        const float dyv = hi ? bf_hi(wy) : bf_lo(wy);
        // recompute X' and h exactly as the forward did
        float xp[N];
#pragma unroll
        for (int k = 0; k < N; ++k) {
          float v = xv[0] * C[0][k];
#pragma unroll
          for (int j = 1; j < N; ++j) v = fmaf(xv[j], C[j][k], v);
          xp[k] = __uint_as_float(pack_bf16x2(fmaf(fv, U[k], v), 0.f) << 16);
        }
        float hv = P[0] * xp[0];
#pragma unroll
        for (int k = 1; k < N; ++k) hv = fmaf(P[k], xp[k], hv);
        hv = __uint_as_float(pack_bf16x2(hv, 0.f) << 16);
        // d gamma: sum over the wave's 8 tokens (lanes l ^ 8, ^ 16, ^ 32)
        float dg = valid ? dyv * hv * rho : 0.f;
        dg += pipe::dpp<pipe::kRowRor8>(dg);
        dg += __shfl_xor(dg, 16);
        dg += __shfl_xor(dg, 32);
        if (m8 == 0) red[b][wave][8 * x8 + e] = dg;
        const float dh = rho * (gv[e] * dyv) - kappa * hv;
#pragma unroll
        for (int k = 0; k < N; ++k) {
          const float dxo = hi ? bf_hi(wd[k]) : bf_lo(wd[k]);
          const float da = dxo + (dxm[k][e] - cr * xp[k]) + P[k] * dh;
          dxm[k][e] = da;
          dp[k] = fmaf(dh, xp[k], dp[k]);
          du[k] = fmaf(fv, da, du[k]);
#pragma unroll
          for (int j = 0; j < N; ++j) dC[j][k] = fmaf(xv[j], da, dC[j][k]);
        }
      }
      // the token sums are updated here, not sunk to the end of the unit
#pragma unroll
      for (int k = 0; k < N; ++k) {
        asm volatile("" : "+v"(dp[k]), "+v"(du[k]));
#pragma unroll
        for (int j = 0; j < N; ++j) asm volatile("" : "+v"(dC[j][k]));
      }
      __builtin_amdgcn_sched_barrier(0);   // one pair's temporaries at a time
    }
    // dX_j = sum_k C[j][k] dA_k, dF = sum_k u_k dA_k, one row segment at a time
    {
      const uint32_t cu = 128u * u;
#pragma unroll
      for (int j = 0; j <= N; ++j) {
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float* cj = j < N ? C[j] : U;
          float v = cj[0] * dxm[0][e];
#pragma unroll
          for (int k = 1; k < N; ++k) v = fmaf(cj[k], dxm[k][e], v);
          o[e] = v;
        }
        const u32x4 ov = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]),
                          pack_bf16x2(o[4], o[5]), pack_bf16x2(o[6], o[7])};
        // non-temporal, like the loads (3.525 -> 3.484 ms per backward call
        // at 65,536 x 5120 against the default policy)
        if (j < N)
          bstore<kNT>(rdx, vx + j * d2, cu, ov);
        else
          bstore<kNT>(rdf, vf, cu, ov);
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    lds_barrier();
    // the workgroup's d gamma partial of the unit's features (red[b] is
    // rewritten two units later, after the next barrier)
    if (wave == 0) {
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) v += red[b][w][lane];
      a.ws[wsl.pg_off() + (int64_t)blockIdx.x * d + kUnit * u + lane] = v;
    }
    cur = nxt;
  }

  // per-token sums over the 8 lanes of a token
#pragma unroll
  for (int k = 0; k < N; ++k) {
    dp[k] = pipe::quad_sum(dp[k]);
    dp[k] += __shfl_xor(dp[k], 4);
    du[k] = pipe::quad_sum(du[k]);
    du[k] += __shfl_xor(du[k], 4);
#pragma unroll
    for (int j = 0; j < N; ++j) {
      dC[j][k] = pipe::quad_sum(dC[j][k]);
      dC[j][k] += __shfl_xor(dC[j][k], 4);
    }
  }
  if (valid && x8 == 0) {
    put_coef<N>(a.d_pre_in + t * N, dp);
    put_coef<N>(a.d_post_in + t * N, du);
    float dcr[N * N];
#pragma unroll
    for (int j = 0; j < N; ++j)
#pragma unroll
      for (int k = 0; k < N; ++k) dcr[j * N + k] = dC[j][k];
    put_coef<N * N>(a.d_comb_in + t * N * N, dcr);
  }
}

// ----- parameter gradients: features across threads, tokens in chunks ----------------

// Thread (feature f, stream k, chunk c) accumulates
// dW[i][k d + f] = sum_t V_t[i] X'_t[k][f] over the chunk's tokens (V_t from
// the stream kernel; X' the stored new streams). Tokens are taken kBatch at a
// time so that their loads are in flight together. Partial sums per chunk go
// to the workspace.
template <int N, int DT>
__global__ __launch_bounds__(256) void param_kernel(Args a) {
  constexpr int kMix = Dims<N>::kMix;
  constexpr int kBatch = 8;
  const int d = a.d;
  const int64_t f = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int k = blockIdx.y;
  const int chunk = blockIdx.z;
  if (f >= d) return;
  Ws<N> wsl{a.tokens, d};
  const int64_t per = param_per(a.tokens);
  const int64_t t0 = chunk * per;
  const int64_t t1 = t0 + per < a.tokens ? t0 + per : a.tokens;
  const float* v = a.ws + wsl.v_off();
  float acc[kMix];
#pragma unroll
  for (int i = 0; i < kMix; ++i) acc[i] = 0.f;
  for (int64_t tb = t0; tb < t1; tb += kBatch) {
    float xp[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int64_t t = tb + b < t1 ? tb + b : t1 - 1;
      const int64_t idx = (t * N + k) * d + f;
      if constexpr (DT == MHC_BF16)
        xp[b] = __uint_as_float((uint32_t) static_cast<const uint16_t*>(a.x_out)[idx] << 16);
      else
        xp[b] = static_cast<const float*>(a.x_out)[idx];
      if (tb + b >= t1) xp[b] = 0.f;
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int64_t t = tb + b < t1 ? tb + b : t1 - 1;
#pragma unroll
      for (int i = 0; i < kMix; ++i) acc[i] = fmaf(v[vidx<N>(t, i)], xp[b], acc[i]);
    }
  }
  float* pw = a.ws + wsl.pw_off() + (int64_t)chunk * kMix * N * d;
#pragma unroll
  for (int i = 0; i < kMix; ++i) pw[(int64_t)i * N * d + (int64_t)k * d + f] = acc[i];
}

// bf16 streams: the same partial sums on v_mfma_f32_16x16x32_bf16. A wave
// owns 64 features of one stream and the chunk's tokens, 32 at a time:
//   D[slot][feature] += V^T[slot][token] X'[token][feature]
// with A = V^T (slots 16 st + lane % 16, tokens 8 (lane / 16) + 0..7) split
// into three exact bf16 terms (hi, mid, lo) accumulated into the same tile,
// and B = X' (exact in bf16), where column c of feature tile tau is feature
// 4c + tau, so that a lane loads 4 adjacent features of a token row (8 bytes)
// and the 16 lanes of a row group cover 128 contiguous bytes. The four waves
// of a workgroup share the chunk's tokens: V of each 32-token step is staged
// once in LDS (one 16-byte load per thread), and the next step's X' and V
// loads are issued before the current step's products. Five waves per SIMD:
// the d = 5120, n = 4 grid (5,120 waves) then runs in a single round.
template <int N>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(5, 5))) void param_mfma_kernel(Args a) {
  constexpr int kMix = Dims<N>::kMix;
  constexpr int kST = Dims<N>::kSlots / 16;   // slot tiles
  typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
  const int d = a.d;
  const int lane = threadIdx.x & 63;
  const int c = lane & 15, g = lane >> 4;
  // a wave past the last feature still stages V and meets every barrier; it
  // reads features 0.. and writes nothing
  const int64_t fw = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 64;   // 64 features
  const bool active = fw < d;
  const int64_t f0 = active ? fw : 0;
  const int k = blockIdx.y;
  const int chunk = blockIdx.z;
  Ws<N> wsl{a.tokens, d};
  const int64_t per = param_per(a.tokens);
  const int64_t t0 = chunk * per;
  const int64_t t1 = t0 + per < a.tokens ? t0 + per : a.tokens;
  const float* v = a.ws + wsl.v_off();
  const uint16_t* xo = static_cast<const uint16_t*>(a.x_out);
  f32x4 acc[kST][4];
#pragma unroll
  for (int st = 0; st < kST; ++st)
#pragma unroll
    for (int tau = 0; tau < 4; ++tau) acc[st][tau] = f32x4{0.f, 0.f, 0.f, 0.f};
  // one step's X' rows: X'[tb + 8g + e][k][f0 + 4c .. +3] (e = 0..7); rows
  // past the chunk are read clamped and zeroed before use
  auto load = [&](uint2 (&xw)[8], int64_t tb) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int64_t t = tb + 8 * g + e;
      const int64_t tc = t < t1 ? t : t1 - 1;
      typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
      const u32x2_t v2 = __builtin_nontemporal_load(
          reinterpret_cast<const u32x2_t*>(xo + (tc * N + k) * (int64_t)d + f0 + 4 * c));
      xw[e] = make_uint2(v2[0], v2[1]);
    }
  };
  // V of one step (32 tokens x 32 slots, the workspace block) staged in LDS
  // by the workgroup, rows of 36 floats: slot row, token column
  __shared__ __align__(16) float vs[2][Dims<N>::kSlots * 36];
  const int vi = threadIdx.x;   // f32x4 of the block: slot vi / 8, tokens 4 (vi % 8) ..
  auto vload = [&](int64_t tb) {
    return *reinterpret_cast<const f32x4*>(v + vidx<N>(tb, 0) + 4 * vi);
  };
  auto vstore = [&](int b, f32x4 x) {
    *reinterpret_cast<f32x4*>(&vs[b][(vi >> 3) * 36 + 4 * (vi & 7)]) = x;
  };
  static_assert(Dims<N>::kSlots * 8 == 256, "one f32x4 per thread");
  uint2 cur[8], nxt[8];
  if (t0 < t1) {
    load(cur, t0);
    vstore(0, vload(t0));
  }
  __syncthreads();
  int buf = 0;
  for (int64_t tb = t0; tb < t1; tb += 32) {
    const bool more = tb + 32 < t1;
    f32x4 vn = {0.f, 0.f, 0.f, 0.f};
    if (more) {
      load(nxt, tb + 32);
      vn = vload(tb + 32);
    }
    uint32_t xw[8][2];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const bool ok = tb + 8 * g + e < t1;
      xw[e][0] = ok ? cur[e].x : 0u;
      xw[e][1] = ok ? cur[e].y : 0u;
    }
    bf16x8_t B[4];   // feature tile tau: feature 4c + tau of the 8 tokens
#pragma unroll
    for (int tau = 0; tau < 4; ++tau) {
      u32x4 w;
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const uint32_t a0 = xw[2 * e2][tau >> 1], a1 = xw[2 * e2 + 1][tau >> 1];
        const uint32_t lo = (tau & 1) ? (a0 >> 16) : (a0 & 0xffffu);
        const uint32_t hi = (tau & 1) ? (a1 & 0xffff0000u) : (a1 << 16);
        w[e2] = lo | hi;
      }
      B[tau] = __builtin_bit_cast(bf16x8_t, w);
    }
#pragma unroll
    for (int st = 0; st < kST; ++st) {
      // A: V[tb + 8g + e][16 st + c], split into three bf16 terms
      float vv[8];
      const f32x4 v0 = *reinterpret_cast<const f32x4*>(&vs[buf][(16 * st + c) * 36 + 8 * g]);
      const f32x4 v1 = *reinterpret_cast<const f32x4*>(&vs[buf][(16 * st + c) * 36 + 8 * g + 4]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = e < 4 ? v0[e] : v1[e - 4];
        vv[e] = tb + 8 * g + e < t1 ? x : 0.f;
      }
      u32x4 th, tm, tl;
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        float h2[2], m2[2], l2[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const float x = vv[2 * e2 + u];
          h2[u] = __uint_as_float(pack_bf16x2(x, 0.f) << 16);
          const float r1 = x - h2[u];
          m2[u] = __uint_as_float(pack_bf16x2(r1, 0.f) << 16);
          l2[u] = r1 - m2[u];
        }
        th[e2] = pack_bf16x2(h2[0], h2[1]);
        tm[e2] = pack_bf16x2(m2[0], m2[1]);
        tl[e2] = pack_bf16x2(l2[0], l2[1]);
      }
      const bf16x8_t Ah = __builtin_bit_cast(bf16x8_t, th);
      const bf16x8_t Am = __builtin_bit_cast(bf16x8_t, tm);
      const bf16x8_t Al = __builtin_bit_cast(bf16x8_t, tl);
#pragma unroll
      for (int tau = 0; tau < 4; ++tau) {
        acc[st][tau] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Ah, B[tau], acc[st][tau], 0, 0, 0);
        acc[st][tau] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Am, B[tau], acc[st][tau], 0, 0, 0);
        acc[st][tau] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Al, B[tau], acc[st][tau], 0, 0, 0);
      }
    }
    if (more) vstore(buf ^ 1, vn);
#pragma unroll
    for (int e = 0; e < 8; ++e) cur[e] = nxt[e];
    buf ^= 1;
    __syncthreads();
  }
  // D[slot 16 st + 4g + i][feature 4c + tau] = acc[st][tau][i]
  if (!active) return;
  float* pw = a.ws + wsl.pw_off() + (int64_t)chunk * kMix * N * d;
#pragma unroll
  for (int st = 0; st < kST; ++st)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int slot = 16 * st + 4 * g + i;
      if (slot < kMix)
        st4f(pw + (int64_t)slot * N * d + (int64_t)k * d + f0 + 4 * c,
             f32x4{acc[st][0][i], acc[st][1][i], acc[st][2][i], acc[st][3][i]});
    }
}

// dW: sum of the per-chunk partials, in chunk order.
template <int N>
__global__ __launch_bounds__(256) void param_reduce_kernel(Args a) {
  const int d = a.d;
  const int64_t nw = (int64_t)Dims<N>::kMix * N * d;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= nw) return;
  Ws<N> wsl{a.tokens, d};
  const float* pw = a.ws + wsl.pw_off();
  float s = 0.f;
  for (int c = 0; c < kParamChunks; ++c) s += pw[(int64_t)c * nw + i];
  a.d_w[i] = s;
}

// d gamma: the per-workgroup partials summed in a fixed order. A block owns
// 64 features; its 4 waves sum the workgroups w = slice, slice + 4, ... (8 at
// a time, so that their loads are in flight together), then the 4 slice sums
// are added in slice order.
template <int N>
__global__ __launch_bounds__(256) void gamma_reduce_kernel(Args a) {
  __shared__ float part[4][64];
  const int d = a.d;
  const int lane = threadIdx.x & 63, slice = threadIdx.x >> 6;
  const int64_t f = (int64_t)blockIdx.x * 64 + lane;
  Ws<N> wsl{a.tokens, d};
  const int64_t groups = a.dg_groups;
  const float* pg = a.ws + wsl.pg_off();
  float s = 0.f;
  if (f < d) {
    for (int64_t w0 = slice; w0 < groups; w0 += 128) {
      float v[32];
#pragma unroll
      for (int u = 0; u < 32; ++u) {
        const int64_t w = w0 + 4 * u;
        v[u] = w < groups ? pg[w * d + f] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 32; ++u) s += v[u];
    }
  }
  part[slice][lane] = s;
  __syncthreads();
  if (slice == 0 && f < d)
    a.d_gamma[f] = ((part[0][lane] + part[1][lane]) + part[2][lane]) + part[3][lane];
}

// d base and the per-slot sums of g * m, stage 1: each block sums a chunk of
// consecutive tokens (contiguous rows of g and of the mixes) per slot, with a
// fixed-order tree.
template <int N>
__global__ __launch_bounds__(256) void slot_kernel(Args a) {
  constexpr int kMix = Dims<N>::kMix;
  constexpr int kRows = 256 / kMix;   // token rows per pass of the block
  __shared__ float sg[256], sm[256];
  Ws<N> wsl{a.tokens, a.d};
  const float* g = a.ws + wsl.g_off();
  const int64_t per = (a.tokens + kSlotChunks - 1) / kSlotChunks;
  const int64_t t0 = blockIdx.x * per;
  const int64_t t1 = t0 + per < a.tokens ? t0 + per : a.tokens;
  const int i = threadIdx.x % kMix, r = threadIdx.x / kMix;
  float s1 = 0.f, s2 = 0.f;
  if (r < kRows) {
    // eight rows in flight, added in row order
    for (int64_t tb = t0 + r; tb < t1; tb += 8 * kRows) {
      float gv[8], mv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t t = tb + (int64_t)u * kRows;
        gv[u] = t < t1 ? g[t * kMix + i] : 0.f;
        mv[u] = t < t1 ? a.mix[t * kMix + i] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (tb + (int64_t)u * kRows < t1) {
          s1 += gv[u];
          s2 = fmaf(gv[u], mv[u], s2);
        }
      }
    }
  }
  sg[threadIdx.x] = s1;
  sm[threadIdx.x] = s2;
  __syncthreads();
  if (threadIdx.x < kMix) {
    float a1 = 0.f, a2 = 0.f;
    for (int rr = 0; rr < kRows; ++rr) {
      a1 += sg[rr * kMix + threadIdx.x];
      a2 += sm[rr * kMix + threadIdx.x];
    }
    float* e = a.ws + wsl.e_off() + (int64_t)blockIdx.x * 2 * kMix;
    e[threadIdx.x] = a1;
    e[kMix + threadIdx.x] = a2;
  }
}

// Stage 2: chunk sums in chunk order; d scale folds the slot sums of g * m
// per group.
template <int N>
__global__ __launch_bounds__(64) void scale_kernel(Args a) {
  constexpr int kMix = Dims<N>::kMix;
  __shared__ float em[kMix];
  Ws<N> wsl{a.tokens, a.d};
  const float* e = a.ws + wsl.e_off();
  const int i = threadIdx.x;
  if (i < kMix) {
    float s1 = 0.f, s2 = 0.f;
    static_assert(kSlotChunks % 64 == 0, "whole batches of chunks");
    for (int c0 = 0; c0 < kSlotChunks; c0 += 64) {   // 64 chunks in flight, added in order
      float v1[64], v2[64];
#pragma unroll
      for (int c = 0; c < 64; ++c) {
        v1[c] = e[(int64_t)(c0 + c) * 2 * kMix + i];
        v2[c] = e[(int64_t)(c0 + c) * 2 * kMix + kMix + i];
      }
#pragma unroll
      for (int c = 0; c < 64; ++c) {
        s1 += v1[c];
        s2 += v2[c];
      }
    }
    a.d_base[i] = s1;
    em[i] = s2;
  }
  __syncthreads();
  if (i < 3) {   // d scale[i]: the slots of pre (i = 0), post (1) or comb (2), in order
    const int j0 = i == 0 ? 0 : (i == 1 ? N : 2 * N), j1 = i == 0 ? N : (i == 1 ? 2 * N : kMix);
    float v = 0.f;
    for (int j = j0; j < j1; ++j) v += em[j];
    a.d_scale[i] = v;
  }
}

}  // namespace bwd
