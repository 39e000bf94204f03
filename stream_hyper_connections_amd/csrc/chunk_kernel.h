// Chunked small-batch path: the fused step, or the mixes alone, as two plain
// kernel launches (bf16 streams with d a multiple of 64 up to 5120, on the
// pipelined tile kernel's steps; f32 streams with any d, on the generic
// kernel's steps).
//
// Included by mhc.hip (one translation unit) after the pipelined tile kernel,
// whose per-step pieces (stream and operand loads, hc_post / hc_pre / sums of
// squares, the MFMA projection) it reuses.
//
// Why. For a few hundred tokens the feature-split kernel occupies only a few
// of its 128-token batches, and the device-side cost of its cooperative launch
// (about 11 us before and after it, against none between plain launches)
// outweighs the kernel itself; the tile kernel, one workgroup per 16 tokens,
// leaves most compute units idle. Here the features are cut into chunks as
// well, and the per-token reduction moves to a second kernel:
//
//   * chunk_kernel: workgroup (tile, chunk) = 16 tokens x `cpairs` pairs of
//     32-feature steps (64 * cpairs features of every row). Its 8 waves run the
//     pipelined tile kernel's steps on them (wave w takes the pairs w, w + 8,
//     ... of the chunk; W read from L2), store the new streams, store h into
//     y_out (normalised in place later), and write one partial row of 32 floats
//     per token: the 24 projection sums of the chunk (from the hi + mid + lo
//     terms of W for a single Sinkhorn round, as the tile kernel always does,
//     and from hi + mid from two rounds on), sum x'^2 and sum h^2.
//   * chunk_finish_kernel: one workgroup per token sums the token's partial
//     rows over the chunks (in chunk order), forms the mixes
//     (r * projection, [SW] Code, hc_mixes), runs the split and the Sinkhorn on
//     16 lanes of wave 0 ([SW] Code, hc_split_sinkhorn), and rewrites y_out
//     = S(gamma * (h * rh)) ([RN] RMSNorm).
// No workgroup ever waits for another: the launch boundary orders the partial
// rows. Workspace: the step kernels' shared header (fsplit::kWsHeader bytes,
// which this path leaves untouched: nothing in it can fail after launch) and
// then the partial rows, [chunk][token][32] float32.

namespace pipe {

constexpr int kPart = 32;                  // floats per partial row
constexpr int64_t kChunkHeader = fsplit::kWsHeader;   // bytes before the partial rows

inline int64_t chunk_workspace_bytes(int nchunks, int64_t tokens) {
  return kChunkHeader + (int64_t)nchunks * tokens * kPart * 4;
}

// XCD-aware work list of the chunked kernels. The hardware hands workgroup b
// to XCD b % 8, and each XCD has its own L2. The (chunk, tile) work items are
// listed chunk-major (every tile of chunk 0, then chunk 1, ...) and cut into
// 8 contiguous ranges, one per XCD, so each XCD's L2 fetches the packed
// weights of about nchunks / 8 chunks instead of all of them; workgroups past
// the end of the list (grid padded to 8 ranges) do nothing.
constexpr int kXcds = 8;
inline int64_t chunk_grid(int64_t ntiles, int nchunks) {
  return kXcds * ((ntiles * nchunks + kXcds - 1) / kXcds);
}
struct ChunkItem {
  int tile, chunk;
  bool live;
};
__device__ __forceinline__ ChunkItem chunk_item(int64_t ntiles, int nchunks) {
  const int64_t total = ntiles * nchunks;
  const int64_t per = (total + kXcds - 1) / kXcds;
  const int64_t w = (int64_t)(blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
  ChunkItem it;
  it.live = w < total;
  it.chunk = it.live ? (int)(w / ntiles) : 0;
  it.tile = it.live ? (int)(w - (int64_t)it.chunk * ntiles) : 0;
  return it;
}

// One pair of steps (A = sa, B = sa + 1) of a chunk: the order of pair_body,
// with h stored to y_out instead of LDS, and the next pair's streams (pair
// sn) loaded only when there is one (`more`, uniform across the wave: with
// one pair per wave, as at d = 5120, a reload would only delay the in-order
// wait on step B's operands).
template <int MODE, int T>
__device__ __forceinline__ void chunk_pair(int sa, int sn, bool more, Ctx& c, Half& ha,
                                           Half& hb) {
  u32x4 w[4][T];
  u32x4 xa[4], xb[4];

  load_w(w, c, sa);
  __builtin_amdgcn_sched_barrier(0);
  const u32x4 h_a = valu_core<MODE>(ha, xa, c);
  __builtin_amdgcn_sched_barrier(0);
  if (more) load_half<MODE>(ha, c, sn);
  __builtin_amdgcn_sched_barrier(0);
  mfma_step(xa, w, c);
  __builtin_amdgcn_sched_barrier(0);

  load_w(w, c, sa + 1);
  __builtin_amdgcn_sched_barrier(0);
  const u32x4 h_b = valu_core<MODE>(hb, xb, c);
  __builtin_amdgcn_sched_barrier(0);
  if (more) load_half<MODE>(hb, c, sn + 1);
  if (MODE == kFused) {
    const uint32_t col = (uint32_t)sa * 64;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      bstore<kStoreAux>(c.xor_, c.xoff, col + (uint32_t)k * c.d2, xa[k]);
      bstore<kStoreAux>(c.xor_, c.xoff, col + 64 + (uint32_t)k * c.d2, xb[k]);
    }
    bstore<0>(c.yr, c.foff, col, h_a);
    bstore<0>(c.yr, c.foff, col + 64, h_b);
  }
  __builtin_amdgcn_sched_barrier(0);
  mfma_step(xb, w, c);
  __builtin_amdgcn_sched_barrier(0);
}

// Grid: ceil(tokens / 16) * nchunks workgroups of kThreads; nchunks * cpairs
// covers the d / 64 pairs of the row. T: the packed column tiles read (all
// three terms of W, or hi + mid; see used_cols).
template <int MODE, int T>
__global__ __launch_bounds__(kThreads) void chunk_kernel(StepArgs a, int nchunks, int cpairs,
                                                         char* __restrict__ ws) {
  constexpr int kC = used_cols(T);
  __shared__ float acc_s[kWaves][kTok][kCols];
  __shared__ float ss_s[kWaves][kTok];
  __shared__ float hs_s[kWaves][kTok];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tr = lane & 15;
  const int g = lane >> 4;
  const int d = a.d;
  const int nsteps = d / kStep;
  const int npairs = nsteps / 2;
  const ChunkItem item = chunk_item((a.tokens + kTok - 1) / kTok, nchunks);
  if (!item.live) return;
  const int tile = item.tile;
  const int chunk = item.chunk;
  const int pair0 = chunk * cpairs;
  const int np = min(cpairs, npairs - pair0);
  const int cnt = wave < np ? (np - wave + kWaves - 1) / kWaves : 0;

  const int64_t t0 = (int64_t)tile * kTok;
  const int ntok = (int)min((int64_t)kTok, a.tokens - t0);
  const uint32_t rowx = (uint32_t)(kStreams * d * 2), rowf = (uint32_t)(d * 2);
  Ctx c;
  c.d2 = d * 2;
  c.wr = make_rsrc(a.wpk, (uint32_t)nsteps * kStreams * kTiles * 1024);
  c.woff = (uint32_t)lane * 16;
  c.woff_last = (tr < kC - 16 * (T - 1)) ? (uint32_t)lane * 16 : kOutOfRange;
  c.xr = make_rsrc(static_cast<const char*>(a.x) + t0 * rowx, ntok * rowx);
  c.xoff = (uint32_t)tr * rowx + (uint32_t)g * 16;
  c.foff = (uint32_t)tr * rowf + (uint32_t)g * 16;
  if (MODE == kFused) {
    c.fr = make_rsrc(static_cast<const char*>(a.f) + t0 * rowf, ntok * rowf);
    c.xor_ = make_rsrc(static_cast<char*>(a.x_out) + t0 * rowx, ntok * rowx);
    c.yr = make_rsrc(static_cast<char*>(a.y_out) + t0 * rowf, ntok * rowf);
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
#pragma unroll
  for (int q = 0; q < T; ++q) c.acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
  c.ss = 0.f;
  c.hs = 0.f;

  Half ha, hb;
  if (cnt > 0) {
    load_half<MODE>(ha, c, 2 * (pair0 + wave));
    load_half<MODE>(hb, c, 2 * (pair0 + wave) + 1);
  }
  for (int p = 0; p < cnt; ++p) {
    const int sa = 2 * (pair0 + wave + kWaves * p);
    chunk_pair<MODE, T>(sa, sa + 2 * kWaves, p + 1 < cnt, c, ha, hb);
  }

  // sums of squares over the four lane groups, then the waves' partials to LDS
  float ss = c.ss, hs = c.hs;
  ss += __shfl_xor(ss, 16);
  ss += __shfl_xor(ss, 32);
  hs += __shfl_xor(hs, 16);
  hs += __shfl_xor(hs, 32);
  if (g == 0) {
    ss_s[wave][tr] = ss;
    hs_s[wave][tr] = hs;
  }
#pragma unroll
  for (int q = 0; q < T; ++q) {
    const int col = 16 * q + tr;
    if (col < kC) {
#pragma unroll
      for (int r = 0; r < 4; ++r) acc_s[wave][4 * g + r][col] = c.acc[q][r];
    }
  }
  __syncthreads();

  // one partial row per token: thread (token tt, column j), 16 x 32 threads
  const int tt = tid >> 5, j = tid & 31;
  float v = 0.f;
  if (j < kMix) {
    float hi = 0.f, mid = 0.f, lo = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      hi += acc_s[w][tt][j];
      mid += acc_s[w][tt][kMix + j];
      if constexpr (T == kTiles) lo += acc_s[w][tt][2 * kMix + j];
    }
    v = T == kTiles ? (hi + mid) + lo : hi + mid;
  } else if (j == kMix || j == kMix + 1) {
#pragma unroll
    for (int w = 0; w < kWaves; ++w) v += j == kMix ? ss_s[w][tt] : hs_s[w][tt];
  }
  if (tt < ntok) {
    float* part = reinterpret_cast<float*>(ws + kChunkHeader);
    part[((int64_t)chunk * a.tokens + t0 + tt) * kPart + j] = v;
  }
}

// f32 streams: workgroup (tile, chunk) = 16 tokens x `csteps` 32-feature steps
// (8 by default), wave w taking the chunk's steps w, w + 8, ... with the
// generic kernel's step (step_f: hc_post, the projection on
// v_mfma_f32_16x16x4_f32 from the float32 weights, sums of squares, hc_pre; h
// parked in y_out as float32), then the same partial rows as chunk_kernel (one
// projection term).
// Grid: ceil(tokens / 16) * nchunks workgroups of kThreads; nchunks * csteps
// covers the d / 32 steps of the row.
template <int MODE>
__global__ __launch_bounds__(kThreads) void chunk_f32_kernel(StepArgs a, int nchunks, int csteps,
                                                             char* __restrict__ ws) {
  constexpr int kColsF = 16 * kTilesF;
  __shared__ float acc_s[kWaves][kTok][kColsF];
  __shared__ float ss_s[kWaves][kTok];
  __shared__ float hs_s[kWaves][kTok];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tr = lane & 15;
  const int g = lane >> 4;
  const int d = a.d;
  const int nsteps = d / kStep;
  const ChunkItem item = chunk_item((a.tokens + kTok - 1) / kTok, nchunks);
  if (!item.live) return;
  const int tile = item.tile;
  const int chunk = item.chunk;
  const int s0 = chunk * csteps;
  const int ns = min(csteps, nsteps - s0);
  const int cnt = wave < ns ? (ns - wave + kWaves - 1) / kWaves : 0;

  const int64_t t0 = (int64_t)tile * kTok;
  const int64_t t = t0 + tr;
  const bool valid = t < a.tokens;
  const int64_t tc = valid ? t : 0;   // rows of tokens past the end are never read
  LaneState<kTilesF> st;
#pragma unroll
  for (int q = 0; q < kTilesF; ++q) st.acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.ss = 0.f;
  st.hs = 0.f;
  if (MODE == kFused) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 c = *reinterpret_cast<const f32x4*>(a.comb_in + tc * 16 + 4 * j);
#pragma unroll
      for (int k = 0; k < 4; ++k) st.C[j][k] = valid ? c[k] : 0.f;
    }
    const f32x4 u = *reinterpret_cast<const f32x4*>(a.post_in + tc * 4);
    const f32x4 p = *reinterpret_cast<const f32x4*>(a.pre_in + tc * 4);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      st.U[k] = valid ? u[k] : 0.f;
      st.P[k] = valid ? p[k] : 0.f;
    }
  }
  const float* xrow = static_cast<const float*>(a.x) + tc * kStreams * (int64_t)d;
  const float* frow = MODE == kFused ? static_cast<const float*>(a.f) + tc * (int64_t)d : nullptr;
  float* xorow = MODE == kFused ? static_cast<float*>(a.x_out) + tc * kStreams * (int64_t)d : nullptr;
  float* yrow = MODE == kFused ? static_cast<float*>(a.y_out) + tc * (int64_t)d : nullptr;
  const u32x4* wpk = static_cast<const u32x4*>(a.wpk);
  const size_t wstride = (size_t)kStreams * kTilesF * 64 * 2;   // u32x4 per step

  InF cur, nxt;
  if (cnt > 0) load_f<MODE>(cur, xrow, frow, d, (s0 + wave) * kStep + g * 8, valid);
  for (int i = 0; i < cnt; ++i) {
    const int s = s0 + wave + kWaves * i;
    const int f0 = s * kStep + g * 8;
    if (i + 1 < cnt) load_f<MODE>(nxt, xrow, frow, d, f0 + kWaves * kStep, valid);
    step_f<MODE>(cur, st, wpk + (size_t)s * wstride, lane, xorow, yrow, d, f0, valid);
    if (i + 1 < cnt) cur = nxt;
  }

  float ss = st.ss, hs = st.hs;
  ss += __shfl_xor(ss, 16);
  ss += __shfl_xor(ss, 32);
  hs += __shfl_xor(hs, 16);
  hs += __shfl_xor(hs, 32);
  if (g == 0) {
    ss_s[wave][tr] = ss;
    hs_s[wave][tr] = hs;
  }
#pragma unroll
  for (int q = 0; q < kTilesF; ++q)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc_s[wave][4 * g + r][16 * q + tr] = st.acc[q][r];
  __syncthreads();

  const int tt = tid >> 5, j = tid & 31;
  float v = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w)
    v += j < kMix ? acc_s[w][tt][j] : (j == kMix ? ss_s[w][tt] : (j == kMix + 1 ? hs_s[w][tt] : 0.f));
  if (t0 + tt < a.tokens) {
    float* part = reinterpret_cast<float*>(ws + kChunkHeader);
    part[((int64_t)chunk * a.tokens + t0 + tt) * kPart + j] = v;
  }
}

// Grid: tokens workgroups of 256 threads. DT: the stream dtype of h / y.
template <int MODE, int DT>
__global__ __launch_bounds__(256) void chunk_finish_kernel(StepArgs a, int nchunks,
                                                           const char* __restrict__ ws) {
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const float* part = reinterpret_cast<const float*>(ws + kChunkHeader);
  float v = 0.f;   // lane j < 32: column j of the token's partial rows, summed
  if (lane < kPart) {
    // in chunk order, eight loads in flight at a time (one at a time, each
    // waited for before the next, the loop cost a full memory latency per chunk)
    const float* p = part + t * kPart + lane;
    const int64_t stride = a.tokens * kPart;
    for (int ch = 0; ch < nchunks; ch += 8) {
      float x[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = ch + i < nchunks ? p[(ch + i) * stride] : 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (ch + i < nchunks) v += x[i];
    }
  }
  const float ssum = __shfl(v, kMix);
  const float hsum = __shfl(v, kMix + 1);
  if (tid < 64) {
    const float r = rsqrtf(ssum / (float)(kStreams * a.d) + a.norm_eps);
    const int e = lane & 15;
    const float mc = __shfl(v, 8 + e) * r;   // comb logit slot of (j, k) = (e/4, e%4)
    const float mp = __shfl(v, e & 7) * r;   // pre / post slot for e < 8
    if (lane < 16) {
      if (a.mix_out != nullptr) {
        a.mix_out[t * kMix + 8 + e] = mc;
        if (e < 8) a.mix_out[t * kMix + e] = mp;
      }
      const float eps = a.hc_eps;
      if (e < 4) a.pre_out[t * 4 + e] = sigmoidf(mp * a.scale[0] + a.base[e]) + eps;
      if (e >= 4 && e < 8) a.post_out[t * 4 + (e - 4)] = 2.0f * sigmoidf(mp * a.scale[1] + a.base[e]);
      float cv = mc * a.scale[2] + a.base[8 + e];
      cv = expf(cv - quad_max(cv));
      cv = cv / quad_sum(cv) + eps;
      cv = cv * __builtin_amdgcn_rcpf(col_sum(cv) + eps);
      for (int it = 1; it < a.iters; ++it) {
        cv = cv * __builtin_amdgcn_rcpf(quad_sum(cv) + eps);
        cv = cv * __builtin_amdgcn_rcpf(col_sum(cv) + eps);
      }
      a.comb_out[t * 16 + e] = cv;
    }
  }
  if (MODE == kFused) {
    const float rh = rsqrtf(hsum / (float)a.d + a.norm_eps);
    // 128-bit stores through st16 / st4f (followed by the store guard)
    if (DT == MHC_BF16) {
      u32x4* y = reinterpret_cast<u32x4*>(static_cast<char*>(a.y_out) + t * a.d * 2);
      for (int u = tid; u < a.d / 8; u += 256) st16(y + u, norm_bf(ld16(y + u), a.gamma, 8 * u, rh));
    } else {   // y = gamma * (h * rh), as the generic kernel
      float* y = static_cast<float*>(a.y_out) + t * a.d;
      for (int u = tid; u < a.d / 4; u += 256) {
        const f32x4 h = *reinterpret_cast<const f32x4*>(y + 4 * u);
        const f32x4 gv = *reinterpret_cast<const f32x4*>(a.gamma + 4 * u);
        f32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = gv[e] * (h[e] * rh);
        st4f(y + 4 * u, o);
      }
    }
  }
}

}  // namespace pipe
