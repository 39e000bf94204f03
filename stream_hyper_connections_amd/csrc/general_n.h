// The step for any stream count n in {2, 4, 8} ([SW] Code: the Block
// constructor sizes the projection as (2+n)*n rows over n*d columns, and
// hc_pre / hc_post / the split kernel take hc_mult as a parameter).
//
// The projection weights grow as n^2 (2+n) d (19.7 MB of exact bf16 terms at
// n = 8, d = 5120), so a kernel that re-reads them per 16-token tile moves
// several times the stream bytes through the caches. Here a workgroup owns a
// block of 128 tokens; each of its 8 waves owns 16 of them (one MFMA row tile)
// over ALL features, and the packed weights of one 32-feature step are staged
// in LDS once per workgroup and read by all 8 waves. Consequences:
//   * every wave has complete per-token sums at the end: no cross-wave
//     reduction of the projection;
//   * h cannot stay on chip for a whole row (16 tokens x d per wave), so it is
//     parked in y and normalised in a second pass over y by the same wave
//     (2d extra stream elements per token);
//   * the split/Sinkhorn runs as a separate kernel, one thread per token,
//     reading the mixes from mix_out.
// Per-element arithmetic (operation order, rounding points) is that of the
// n = 4 kernels, so at n = 4 the new streams agree bit for bit with them.
//
// Packed weights (mhc_pack_wmix_n): the three exact bf16 terms of W (hi, mid,
// lo) are laid out term-major, each term padded to T1 = ceil((2+n)n / 16)
// column tiles, so the three terms of mix j sit in tiles q, T1+q, 2*T1+q at
// the same lane and are summed without a shuffle. Order [step][stream][tile]
// [lane] (u32x4 = 8 bf16 B-operand values of v_mfma_f32_16x16x32_bf16); the
// f32 form has one term and 8 floats (2 x u32x4) per lane.
//
// Included by mhc.hip (one translation unit).

namespace gen {

constexpr int kTok = 16;                 // tokens per wave (rows of one MFMA tile)
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kBlock = kTok * kWaves;    // tokens per workgroup
constexpr int kStep = 32;                // features per step (4 lane groups x 8)

template <int N>
struct Dims {
  static constexpr int kMix = (2 + N) * N;
  static constexpr int kT1 = (kMix + 15) / 16;   // column tiles of one weight term
  // an 8x8 comb per lane would not fit in registers beside the accumulators
  static constexpr bool kCoefLds = N > 4;
};

// Packed weights of one unit of SPI consecutive steps (SPI = 2 lets a lane
// load both 64-byte halves of a 128-byte line of each token row back to back;
// it needs two steps' weights in LDS, which fits for n <= 4).
template <int N, int DT, int SPI = 1>
struct Slice {
  static constexpr int kTiles = DT == MHC_BF16 ? 3 * Dims<N>::kT1 : Dims<N>::kT1;
  static constexpr int kPerLane = DT == MHC_BF16 ? 1 : 2;   // u32x4 per lane and tile
  static constexpr int kStepVecs = N * kTiles * 64 * kPerLane;   // u32x4 per step
  static constexpr int kVecs = SPI * kStepVecs;                  // u32x4 per unit
  // a unit's slice is staged in parts of (SPI * N) / kParts stream-steps each,
  // so that the registers holding the next unit's weights in flight stay few
  static constexpr int kParts = N == 8 ? 4 : 1;
  static constexpr int kPartVecs = kVecs / kParts;
  static constexpr int kStage = (kPartVecs + kThreads - 1) / kThreads;
};

// ----- packing --------------------------------------------------------------------------

// One thread per (step s, stream k, tile q, lane): column n = 16q + lane%16 of
// the padded term-major layout is term n / (16 T1) of mix row n % (16 T1)
// (zero past the (2+n)n rows); K slots are features 32s + 8(lane/16) + 0..7 of
// stream k. hi = bf16(w), mid = bf16(w - hi), lo = w - hi - mid (exact).
template <int N, int DT>
__global__ __launch_bounds__(256) void pack_kernel(const float* __restrict__ w, int d,
                                                   int64_t total, u32x4* __restrict__ out) {
  using S = Slice<N, DT>;
  constexpr int kMix = Dims<N>::kMix;
  constexpr int kPad = 16 * Dims<N>::kT1;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  const int lane = (int)(idx & 63);
  int64_t r = idx >> 6;
  const int q = (int)(r % S::kTiles);
  r /= S::kTiles;
  const int k = (int)(r % N);
  const int64_t s = r / N;
  const int n = 16 * q + (lane & 15);
  const int part = n / kPad;
  const int row = n % kPad;
  const int64_t c0 = (int64_t)k * d + s * kStep + 8 * (lane >> 4);
  float v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = 0.f;
  if (row < kMix) {
    const float* src = w + (int64_t)row * N * d + c0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = src[e];
      if (DT == MHC_BF16) {
        const float hi = __uint_as_float(pack_bf16x2(x, 0.f) << 16);
        const float r1 = x - hi;
        const float mid = __uint_as_float(pack_bf16x2(r1, 0.f) << 16);
        v[e] = part == 0 ? hi : (part == 1 ? mid : r1 - mid);
      } else {
        v[e] = x;
      }
    }
  }
  if (DT == MHC_BF16) {
    st16(out + idx, u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                          pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])});
  } else {
    st16(out + 2 * idx, u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]),
                              __float_as_uint(v[2]), __float_as_uint(v[3])});
    st16(out + 2 * idx + 1, u32x4{__float_as_uint(v[4]), __float_as_uint(v[5]),
                                  __float_as_uint(v[6]), __float_as_uint(v[7])});
  }
}

// ----- per-lane coefficients ------------------------------------------------------------

template <int N>
__device__ __forceinline__ void load_row(const float* p, float (&v)[N]) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      const f32x4 q = *reinterpret_cast<const f32x4*>(p + 4 * i);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * i + e] = q[e];
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = p[i];
  }
}

// comb / post / pre of the lane's token; comb in registers ...
template <int N, bool LDS>
struct Coef {
  float C[N][N];
  float U[N];
  float P[N];
  __device__ __forceinline__ void col(int k, float (&c)[N]) const {
#pragma unroll
    for (int j = 0; j < N; ++j) c[j] = C[j][k];
  }
};
// ... or, for n = 8, transposed in LDS: ct[k * N + j] = comb[j][k]
template <int N>
struct Coef<N, true> {
  const float* ct;
  float U[N];
  float P[N];
  __device__ __forceinline__ void col(int k, float (&c)[N]) const {
    load_row<N>(ct + k * N, c);
  }
};

// ----- bf16 streams ---------------------------------------------------------------------

template <int N>
struct InBf {
  u32x4 x[N];
  u32x4 f;
};

// Buffer views of one wave's 16 token rows. The range of each view ends at
// the last token, so the lanes of tokens past the end read zeros and their
// stores are dropped, without branches. Byte offsets: the lane's token row and
// 8-feature group go in the vector offset, the step and the stream in the
// scalar offset.
struct Rows {
  pipe::rsrc_t x, f, xo, y;
  uint32_t xoff, foff;
  uint32_t xstride;   // bytes between the streams of a token (d elements)
};

template <int N>
__device__ __forceinline__ Rows make_rows(const StepArgs& a, int64_t tw, int tr, int g, int es,
                                          bool full) {
  const int d = a.d;
  const int64_t left = a.tokens - tw;
  const uint32_t rows = (uint32_t)(left <= 0 ? 0 : (left < kTok ? left : kTok));
  const uint64_t xrow = (uint64_t)N * d * es, frow = (uint64_t)d * es;
  Rows r;
  r.x = pipe::make_rsrc(static_cast<const char*>(a.x) + tw * xrow, (uint32_t)(rows * xrow));
  if (full) {
    r.f = pipe::make_rsrc(static_cast<const char*>(a.f) + tw * frow, (uint32_t)(rows * frow));
    r.xo = pipe::make_rsrc(static_cast<char*>(a.x_out) + tw * xrow, (uint32_t)(rows * xrow));
    r.y = pipe::make_rsrc(static_cast<char*>(a.y_out) + tw * frow, (uint32_t)(rows * frow));
  } else {
    r.f = r.xo = r.y = r.x;
  }
  r.xoff = (uint32_t)(tr * xrow + (uint64_t)g * 8 * es);
  r.foff = (uint32_t)(tr * frow + (uint64_t)g * 8 * es);
  r.xstride = (uint32_t)frow;
  return r;
}

template <int N, int MODE>
__device__ __forceinline__ void load_bf(InBf<N>& in, const Rows& r, uint32_t col) {
#pragma unroll
  for (int j = 0; j < N; ++j) in.x[j] = pipe::bload<pipe::kNT>(r.x, r.xoff, col + j * r.xstride);
  if (MODE == kFused) in.f = pipe::bload<pipe::kNT>(r.f, r.foff, col);
}

// hc_post ([SW] Code): new stream k = sum_j comb[j][k] x_j + post[k] f in fp32,
// rounded to bf16 (the n = 4 kernels' operation order).
template <int N, class CF>
__device__ __forceinline__ void post_bf(const InBf<N>& in, const CF& cf, u32x4 (&xo)[N]) {
#pragma unroll
  for (int k = 0; k < N; ++k) {
    float c[N];
    cf.col(k, c);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      float v0 = bf_lo(in.x[0][w]) * c[0];
      float v1 = bf_hi(in.x[0][w]) * c[0];
#pragma unroll
      for (int j = 1; j < N; ++j) {
        v0 = fmaf(bf_lo(in.x[j][w]), c[j], v0);
        v1 = fmaf(bf_hi(in.x[j][w]), c[j], v1);
      }
      v0 = fmaf(bf_lo(in.f[w]), cf.U[k], v0);
      v1 = fmaf(bf_hi(in.f[w]), cf.U[k], v1);
      xo[k][w] = pack_bf16x2(v0, v1);
    }
    if (N > 4) __builtin_amdgcn_sched_barrier(0);   // one comb column live at a time
  }
}

// Sums of squares of the rounded new streams and, in the full step, hc_pre
// (h = bf16(sum_k pre[k] x'_k)) with the sum of squares of the rounded h.
template <int N, int MODE>
__device__ __forceinline__ u32x4 sums_bf(const u32x4 (&xo)[N], const float (&P)[N], float& ss,
                                         float& hs) {
  u32x4 hpk = {0, 0, 0, 0};
  float ssa = 0.f, ssb = 0.f, hsa = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    float r0[N], r1[N];
#pragma unroll
    for (int k = 0; k < N; ++k) {
      r0[k] = bf_lo(xo[k][w]);
      r1[k] = bf_hi(xo[k][w]);
      ssa = fmaf(r0[k], r0[k], ssa);
      ssb = fmaf(r1[k], r1[k], ssb);
    }
    if (MODE == kFused) {
      float h0 = P[0] * r0[0], h1 = P[0] * r1[0];
#pragma unroll
      for (int k = 1; k < N; ++k) {
        h0 = fmaf(P[k], r0[k], h0);
        h1 = fmaf(P[k], r1[k], h1);
      }
      const uint32_t hp = pack_bf16x2(h0, h1);
      hpk[w] = hp;
      const float q0 = bf_lo(hp), q1 = bf_hi(hp);
      hsa = fmaf(q0, q0, hsa);
      hsa = fmaf(q1, q1, hsa);
    }
  }
  ss += ssa + ssb;
  hs += hsa;
  return hpk;
}

// ----- f32 streams ----------------------------------------------------------------------

template <int N>
struct InF {
  u32x4 x[N][2];
  u32x4 f[2];
};

template <int N, int MODE>
__device__ __forceinline__ void load_f(InF<N>& in, const Rows& r, uint32_t col) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int j = 0; j < N; ++j)
      in.x[j][h] = pipe::bload<pipe::kNT>(r.x, r.xoff, col + 16 * h + j * r.xstride);
    if (MODE == kFused) in.f[h] = pipe::bload<pipe::kNT>(r.f, r.foff, col + 16 * h);
  }
}

// ----- the block kernel -----------------------------------------------------------------

// Issue the loads of one part of a step's packed weights (thread tid stages
// vectors tid, tid + 512, ... of the part). Past the end of the part a thread
// repeats the last vector, so that it writes the same value to the same LDS
// slot as the thread that owns it (no branch).
template <int N, int DT, int SPI>
__device__ __forceinline__ int stage_index(int tid, int i) {
  using S = Slice<N, DT, SPI>;
  const int v = tid + i * kThreads;
  return S::kPartVecs % kThreads == 0 ? v : (v < S::kPartVecs ? v : S::kPartVecs - 1);
}

template <int N, int DT, int SPI>
__device__ __forceinline__ void stage_load(u32x4* st, const u32x4* __restrict__ src, int tid) {
#pragma unroll
  for (int i = 0; i < Slice<N, DT, SPI>::kStage; ++i) st[i] = src[stage_index<N, DT, SPI>(tid, i)];
}

template <int N, int DT, int SPI>
__device__ __forceinline__ void stage_store(u32x4* wl, const u32x4* st, int tid) {
#pragma unroll
  for (int i = 0; i < Slice<N, DT, SPI>::kStage; ++i) wl[stage_index<N, DT, SPI>(tid, i)] = st[i];
}

// After part p of a step has been consumed by every wave: overwrite it with
// the same part of the next unit (held in `st`; on the last unit, the unit
// itself again) and issue the loads of the next part. A part is rewritten only
// after a barrier that follows all reads of it, and read again only after the
// barrier that follows the next part's reads (with a single part, after an
// extra barrier at the end of the step).
template <int N, int DT, int SPI>
__device__ __forceinline__ void next_part(u32x4* wl, u32x4* st, const u32x4* wnext, int p,
                                          int tid) {
  using S = Slice<N, DT, SPI>;
  __syncthreads();
  stage_store<N, DT, SPI>(wl + p * S::kPartVecs, st, tid);
  if (p + 1 < S::kParts) stage_load<N, DT, SPI>(st, wnext + (p + 1) * S::kPartVecs, tid);
}

// Chunked launches (small calls): workgroup (block, chunk) covers the units
// [chunk * per, (chunk + 1) * per) of its 128-token block and writes, per
// token, a partial row of kRowN floats to the workspace (after a 256-byte
// header): the (2+n)n projection sums of its units (the three terms added),
// sum x'^2 and sum h^2. h stays parked in y; chunk_finish_kernel completes the
// tokens.
struct ChunkN {
  char* ws;       // workspace (nullptr: not chunked)
  int per;        // units per chunk
  int nchunks;    // chunks per row
};
constexpr int64_t kChunkHeaderN = fsplit::kWsHeader;
template <int N>
__host__ __device__ constexpr int row_n() { return ((Dims<N>::kMix + 2 + 3) / 4) * 4; }

// One pass over a 128-token block: hc_post (stored), the RMS statistic and the
// (2+n)n-wide projection of the new streams (written to mix_out), hc_pre (h
// parked in y) and, after the token's sum of h^2 is complete, RMSNorm over y.
// MODE kMixesOnly reads x as the streams and writes mix_out only. CH: one
// chunk of the units, partial rows instead of the mixes and RMSNorm.
template <int N, int DT, int MODE, int SPI, bool CH = false>
__global__ __launch_bounds__(kThreads) void block_kernel(StepArgs a, ChunkN cn) {
  using Dm = Dims<N>;
  using S = Slice<N, DT, SPI>;
  constexpr bool kBf = DT == MHC_BF16;
  constexpr bool kFull = MODE == kFused;
  constexpr int kMix = Dm::kMix;
  constexpr int kT1 = Dm::kT1;
  constexpr bool kCL = kFull && Dm::kCoefLds;
  static_assert(SPI == 1 || (kBf && N <= 4), "two-step units are for bf16 streams, n <= 4");

  __shared__ u32x4 wl[S::kVecs];
  __shared__ float ct[kCL ? kBlock * N * N : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tr = lane & 15;
  const int g = lane >> 4;
  // chunks: the XCD-aware work list of the chunked kernels (pipe::chunk_item)
  pipe::ChunkItem item{(int)blockIdx.x, 0, true};
  if constexpr (CH) item = pipe::chunk_item((a.tokens + kBlock - 1) / kBlock, cn.nchunks);
  if (!item.live) return;
  const int blk = item.tile;
  const int chunk = item.chunk;
  const int64_t tb = (int64_t)blk * kBlock;
  const int64_t tw = tb + wave * kTok;
  const int64_t t = tw + tr;
  const bool valid = t < a.tokens;
  const int d = a.d;
  const int nsteps = d / kStep;
  const int nunits_all = nsteps / SPI;
  const int u0 = CH ? chunk * cn.per : 0;                       // this launch's units
  const int u1 = CH ? min(u0 + cn.per, nunits_all) : nunits_all;
  const u32x4* wpk = static_cast<const u32x4*>(a.wpk);
  const u32x4* wpk0 = wpk + (size_t)u0 * S::kVecs;

  // packed weights of the first unit, part 0 (the other parts follow below)
  u32x4 wst[S::kStage];
  stage_load<N, DT, SPI>(wst, wpk0, tid);

  Coef<N, kCL> cf;
  if (kFull) {
    if constexpr (kCL) {
      for (int i = tid; i < kBlock * N * N; i += kThreads) {
        const int tt = i / (N * N), jk = i - tt * (N * N);
        const int j = jk / N, k = jk - j * N;
        ct[tt * N * N + k * N + j] = tb + tt < a.tokens ? a.comb_in[(tb + tt) * N * N + jk] : 0.f;
      }
      cf.ct = ct + (wave * kTok + tr) * N * N;
    } else {
#pragma unroll
      for (int j = 0; j < N; ++j) {
        if (valid) {
          load_row<N>(a.comb_in + t * N * N + j * N, cf.C[j]);
        } else {
#pragma unroll
          for (int k = 0; k < N; ++k) cf.C[j][k] = 0.f;
        }
      }
    }
    if (valid) {
      load_row<N>(a.post_in + t * N, cf.U);
      load_row<N>(a.pre_in + t * N, cf.P);
    } else {
#pragma unroll
      for (int k = 0; k < N; ++k) cf.U[k] = cf.P[k] = 0.f;
    }
  }
  stage_store<N, DT, SPI>(wl, wst, tid);
#pragma unroll
  for (int p = 1; p < S::kParts; ++p) {
    stage_load<N, DT, SPI>(wst, wpk0 + p * S::kPartVecs, tid);
    stage_store<N, DT, SPI>(wl + p * S::kPartVecs, wst, tid);
  }
  __syncthreads();

  f32x4 acc[S::kTiles];
#pragma unroll
  for (int q = 0; q < S::kTiles; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
  float ss = 0.f, hs = 0.f;
  constexpr int es = kBf ? 2 : 4;
  const Rows rw = make_rows<N>(a, tw, tr, g, es, kFull);

  if constexpr (kBf) {
    // a unit of SPI steps; lane loads and stores of the SPI halves of a line
    // are issued back to back
    constexpr int kE = SPI * N;                 // stream-steps per unit
    InBf<N> cur[SPI];
#pragma unroll
    for (int h = 0; h < SPI; ++h)
      load_bf<N, MODE>(cur[h], rw, (uint32_t)u0 * (SPI * kStep * 2) + h * (kStep * 2));
    for (int u = u0; u < u1; ++u) {
      const uint32_t col = (uint32_t)u * (SPI * kStep * 2);
      // the last unit reloads its own data instead of reading past the rows
      // (no branch around the loads, which the compiler would hoist)
      const int un = u + 1 < u1 ? u + 1 : u;
      const u32x4* wnext = wpk + (size_t)un * S::kVecs;
      // Loads retire in issue order: the next unit's weights are issued before
      // its streams, so that the wait for the weights at the end of this unit
      // does not also wait for the stream prefetch.
      stage_load<N, DT, SPI>(wst, wnext, tid);
      __builtin_amdgcn_sched_barrier(0);
      u32x4 xo[SPI][N];
#pragma unroll
      for (int h = 0; h < SPI; ++h) {
        if (kFull) {
          post_bf<N>(cur[h], cf, xo[h]);
        } else {
#pragma unroll
          for (int k = 0; k < N; ++k) xo[h][k] = cur[h].x[k];
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      const uint32_t ncol = (uint32_t)un * (SPI * kStep * 2);
#pragma unroll
      for (int j = 0; j < N; ++j)
#pragma unroll
        for (int h = 0; h < SPI; ++h)
          cur[h].x[j] = pipe::bload<pipe::kNT>(rw.x, rw.xoff, ncol + h * (kStep * 2) + j * rw.xstride);
      if (kFull) {
#pragma unroll
        for (int h = 0; h < SPI; ++h)
          cur[h].f = pipe::bload<pipe::kNT>(rw.f, rw.foff, ncol + h * (kStep * 2));
      }
      __builtin_amdgcn_sched_barrier(0);
      if (kFull) {
#pragma unroll
        for (int k = 0; k < N; ++k)
#pragma unroll
          for (int h = 0; h < SPI; ++h)
            pipe::bstore<pipe::kNT>(rw.xo, rw.xoff, col + h * (kStep * 2) + k * rw.xstride,
                                    xo[h][k]);
      }
      float pz[N];
#pragma unroll
      for (int k = 0; k < N; ++k) pz[k] = kFull ? cf.P[k] : 0.f;
      u32x4 hp[SPI];
#pragma unroll
      for (int h = 0; h < SPI; ++h) hp[h] = sums_bf<N, MODE>(xo[h], pz, ss, hs);
      if (kFull) {
#pragma unroll
        for (int h = 0; h < SPI; ++h)   // h parked in y until rh is known
          pipe::bstore<0>(rw.y, rw.foff, col + h * (kStep * 2), hp[h]);
      }
#pragma unroll
      for (int p = 0; p < S::kParts; ++p) {
#pragma unroll
        for (int e = p * (kE / S::kParts); e < (p + 1) * (kE / S::kParts); ++e) {
          const bf16x8 A = __builtin_bit_cast(bf16x8, xo[e / N][e % N]);
#pragma unroll
          for (int q = 0; q < S::kTiles; ++q)
            acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                A, __builtin_bit_cast(bf16x8, wl[(e * S::kTiles + q) * 64 + lane]), acc[q], 0, 0,
                0);
          if (Dm::kCoefLds) __builtin_amdgcn_sched_barrier(0);   // one stream's operands live
        }
        next_part<N, DT, SPI>(wl, wst, wnext, p, tid);
      }
      if (S::kParts == 1) __syncthreads();
    }
  } else {
    for (int s = u0; s < u1; ++s) {
      const uint32_t col = (uint32_t)s * (kStep * 4);
      const int sn = s + 1 < u1 ? s + 1 : s;
      const u32x4* wnext = wpk + (size_t)sn * S::kVecs;
      InF<N> in;
      load_f<N, MODE>(in, rw, col);
      stage_load<N, DT, SPI>(wst, wnext, tid);
      float xr[N][8];
#pragma unroll
      for (int k = 0; k < N; ++k) {
        float c[N];
        if (kFull) cf.col(k, c);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if (kFull) {
            float v = __uint_as_float(in.x[0][e >> 2][e & 3]) * c[0];
#pragma unroll
            for (int j = 1; j < N; ++j) v = fmaf(__uint_as_float(in.x[j][e >> 2][e & 3]), c[j], v);
            xr[k][e] = fmaf(__uint_as_float(in.f[e >> 2][e & 3]), cf.U[k], v);
          } else {
            xr[k][e] = __uint_as_float(in.x[k][e >> 2][e & 3]);
          }
        }
      }
      if (kFull) {
#pragma unroll
        for (int k = 0; k < N; ++k)
#pragma unroll
          for (int hf = 0; hf < 2; ++hf)
            pipe::bstore<0>(rw.xo, rw.xoff, col + 16 * hf + k * rw.xstride,
                            u32x4{__float_as_uint(xr[k][4 * hf]), __float_as_uint(xr[k][4 * hf + 1]),
                                  __float_as_uint(xr[k][4 * hf + 2]),
                                  __float_as_uint(xr[k][4 * hf + 3])});
      }
      float hv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
#pragma unroll
        for (int k = 0; k < N; ++k) ss = fmaf(xr[k][e], xr[k][e], ss);
        if (kFull) {
          float h = cf.P[0] * xr[0][e];
#pragma unroll
          for (int k = 1; k < N; ++k) h = fmaf(cf.P[k], xr[k][e], h);
          hv[e] = h;
          hs = fmaf(h, h, hs);
        }
      }
      if (kFull) {
        pipe::bstore<0>(rw.y, rw.foff, col, u32x4{__float_as_uint(hv[0]), __float_as_uint(hv[1]),
                                                  __float_as_uint(hv[2]), __float_as_uint(hv[3])});
        pipe::bstore<0>(rw.y, rw.foff, col + 16,
                        u32x4{__float_as_uint(hv[4]), __float_as_uint(hv[5]),
                              __float_as_uint(hv[6]), __float_as_uint(hv[7])});
      }
#pragma unroll
      for (int p = 0; p < S::kParts; ++p) {
#pragma unroll
        for (int k = p * (N / S::kParts); k < (p + 1) * (N / S::kParts); ++k) {
#pragma unroll
          for (int q = 0; q < S::kTiles; ++q) {
            const u32x4 b0 = wl[((k * S::kTiles + q) * 64 + lane) * 2];
            const u32x4 b1 = wl[((k * S::kTiles + q) * 64 + lane) * 2 + 1];
#pragma unroll
            for (int e = 0; e < 8; ++e)
              acc[q] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                  xr[k][e], __uint_as_float(e < 4 ? b0[e] : b1[e - 4]), acc[q], 0, 0, 0);
          }
          if (Dm::kCoefLds) __builtin_amdgcn_sched_barrier(0);
        }
        next_part<N, DT, SPI>(wl, wst, wnext, p, tid);
      }
      if (S::kParts == 1) __syncthreads();
    }
  }

  // per-token totals over the 4 lanes of a token
  ss += __shfl_xor(ss, 16);
  ss += __shfl_xor(ss, 32);
  hs += __shfl_xor(hs, 16);
  hs += __shfl_xor(hs, 32);

  if constexpr (CH) {
    // partial row of this chunk: lane (c, g) holds rows 4g + i, column 16q + c
    constexpr int kR = row_n<N>();
    float* part = reinterpret_cast<float*>(cn.ws + kChunkHeaderN);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t tt = tw + 4 * g + i;
      if (tt >= a.tokens) continue;
      float* row = part + ((int64_t)chunk * a.tokens + tt) * kR;
#pragma unroll
      for (int q = 0; q < kT1; ++q) {
        const int j = 16 * q + tr;
        if (j < kMix)
          row[j] = kBf ? (acc[q][i] + acc[kT1 + q][i]) + acc[2 * kT1 + q][i] : acc[q][i];
      }
    }
    if (g == 0 && valid) {
      float* row = part + ((int64_t)chunk * a.tokens + t) * kR;
      row[kMix] = ss;
      row[kMix + 1] = hs;
    }
    return;
  }
  const float r = rsqrtf(ss / (float)(N * d) + a.norm_eps);

  // mixes: lane (c, g) holds rows 4g + i of the tile, column 16q + c of every
  // tile; the three weight terms of mix j = 16q + c are tiles q, T1+q, 2T1+q
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 4 * g + i;
    const float rr = __shfl(r, row);
    const int64_t tt = tw + row;
#pragma unroll
    for (int q = 0; q < kT1; ++q) {
      const int j = 16 * q + tr;
      float mv;
      if (kBf)
        mv = ((acc[q][i] + acc[kT1 + q][i]) + acc[2 * kT1 + q][i]) * rr;
      else
        mv = acc[q][i] * rr;
      if (j < kMix && tt < a.tokens) a.mix_out[tt * kMix + j] = mv;
    }
  }

  // RMSNorm over the parked h ([RN] RMSNorm: the normalised value, then the
  // gain), kYBatch steps at a time so that their loads are in flight together
  if (kFull) {
    constexpr int kYBatch = 8;
    constexpr int kVec = kBf ? 1 : 2;   // u32x4 per lane and step
    const float rh = rsqrtf(hs / (float)d + a.norm_eps);
    for (int s0 = 0; s0 < nsteps; s0 += kYBatch) {
      u32x4 hv[kYBatch][kVec];
#pragma unroll
      for (int i = 0; i < kYBatch; ++i) {
        const int s = s0 + i < nsteps ? s0 + i : nsteps - 1;
#pragma unroll
        for (int v = 0; v < kVec; ++v)
          hv[i][v] = pipe::bload<0>(rw.y, rw.foff, (uint32_t)s * (kStep * es) + 16 * v);
      }
#pragma unroll
      for (int i = 0; i < kYBatch; ++i) {
        if (s0 + i >= nsteps) break;
        const int s = s0 + i;
        const int f0 = s * kStep + g * 8;
        const uint32_t col = (uint32_t)s * (kStep * es);
        const f32x4 g0 = *reinterpret_cast<const f32x4*>(a.gamma + f0);
        const f32x4 g1 = *reinterpret_cast<const f32x4*>(a.gamma + f0 + 4);
        if constexpr (kBf) {
          const float gv[8] = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};
          u32x4 y;
#pragma unroll
          for (int w = 0; w < 4; ++w)
            y[w] = pack_bf16x2(gv[2 * w] * (bf_lo(hv[i][0][w]) * rh),
                               gv[2 * w + 1] * (bf_hi(hv[i][0][w]) * rh));
          pipe::bstore<pipe::kNT>(rw.y, rw.foff, col, y);
        } else {
#pragma unroll
          for (int v = 0; v < 2; ++v) {
            const f32x4 gv = v ? g1 : g0;
            u32x4 y;
#pragma unroll
            for (int e = 0; e < 4; ++e)
              y[e] = __float_as_uint(gv[e] * (__uint_as_float(hv[i][v][e]) * rh));
            pipe::bstore<0>(rw.y, rw.foff, col + 16 * v, y);
          }
        }
      }
    }
  }
}

// Completes the tokens of a chunked launch: sums each token's partial rows,
// writes the mixes (r * projection, [SW] Code, hc_mixes) to mix_out and
// rewrites y = S(gamma * (h * rh)) over the parked h ([RN] RMSNorm), with the
// block kernel's arithmetic per element. One workgroup of 256 threads per
// token; sinkhorn_kernel then splits the mixes. The sums are split over kG
// groups of kR threads, each adding a contiguous run of chunks eight loads at
// a time, then added in group order (a fixed order: results repeat bit for
// bit).
template <int N, int DT, int MODE>
__global__ __launch_bounds__(256) void chunk_finish_kernel(StepArgs a, ChunkN cn) {
  constexpr int kMix = Dims<N>::kMix;
  constexpr int kR = row_n<N>();
  constexpr int kG = 256 / kR;
  __shared__ float grp_sum[kG][kR];
  __shared__ float sum[kR];
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x;
  const float* part = reinterpret_cast<const float*>(cn.ws + kChunkHeaderN);
  const int grp = tid / kR;
  const int col = tid - grp * kR;
  if (grp < kG) {
    const int cper = (cn.nchunks + kG - 1) / kG;
    const int c1 = min((grp + 1) * cper, cn.nchunks);
    float v = 0.f;
    int c = grp * cper;
    for (; c + 8 <= c1; c += 8) {
      float b[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) b[e] = part[((int64_t)(c + e) * a.tokens + t) * kR + col];
#pragma unroll
      for (int e = 0; e < 8; ++e) v += b[e];
    }
    for (; c < c1; ++c) v += part[((int64_t)c * a.tokens + t) * kR + col];
    grp_sum[grp][col] = v;
  }
  __syncthreads();
  if (tid < kR) {
    float v = 0.f;
#pragma unroll
    for (int g = 0; g < kG; ++g) v += grp_sum[g][tid];
    sum[tid] = v;
  }
  __syncthreads();
  const float r = rsqrtf(sum[kMix] / (float)(N * a.d) + a.norm_eps);
  if (tid < kMix) a.mix_out[t * kMix + tid] = sum[tid] * r;
  if (MODE == kFused) {
    const float rh = rsqrtf(sum[kMix + 1] / (float)a.d + a.norm_eps);
    if (DT == MHC_BF16) {
      u32x4* y = reinterpret_cast<u32x4*>(static_cast<char*>(a.y_out) + t * a.d * 2);
      for (int u = tid; u < a.d / 8; u += 256) {
        const u32x4 h = ld16(y + u);
        const f32x4 g0 = *reinterpret_cast<const f32x4*>(a.gamma + 8 * u);
        const f32x4 g1 = *reinterpret_cast<const f32x4*>(a.gamma + 8 * u + 4);
        const float gv[8] = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};
        u32x4 o;
#pragma unroll
        for (int w = 0; w < 4; ++w)
          o[w] = pack_bf16x2(gv[2 * w] * (bf_lo(h[w]) * rh), gv[2 * w + 1] * (bf_hi(h[w]) * rh));
        st16(y + u, o);
      }
    } else {
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

// ----- split and Sinkhorn, one lane per comb entry -------------------------------------

// [SW] Code, the split/Sinkhorn kernel, for hc_mult = N: pre = sigmoid(s0 m +
// b) + eps, post = 2 sigmoid(s1 m + b), comb = row softmax of s2 m + b plus eps,
// a column division, then iters - 1 rounds of (row, column) divisions, every
// divisor being (sum + eps). Each division is a multiplication by the
// correctly rounded reciprocal of the divisor.
//
// A token owns kLanes = N*N consecutive lanes, lane e holding entry (j, k) =
// (e / N, e % N); row j is N consecutive lanes and column k the lanes e with
// e % N = k. Row and column sums (and the row maximum) are xor butterflies over
// those lanes, so every lane of a row or column gets the same bits. Lanes
// e < N also give pre[e], lanes N <= e < 2N post[e - N]. kSinkTokens tokens
// per 256-thread workgroup.
template <int N>
constexpr int kSinkTokens = 256 / (N * N);

template <int N>
__global__ __launch_bounds__(256) void sinkhorn_kernel(const float* __restrict__ mix,
                                                       int64_t tokens,
                                                       const float* __restrict__ base,
                                                       const float* __restrict__ scale, int iters,
                                                       float eps, float* __restrict__ pre_out,
                                                       float* __restrict__ post_out,
                                                       float* __restrict__ comb_out) {
  constexpr int kMix = Dims<N>::kMix;
  constexpr int kLanes = N * N;
  const int e = threadIdx.x % kLanes;
  const int64_t t = (int64_t)blockIdx.x * kSinkTokens<N> + threadIdx.x / kLanes;
  if (t >= tokens) return;   // whole tokens: the butterflies never reach a lane that left
  const float* m = mix + t * kMix;
  if (e < N) pre_out[t * N + e] = sigmoidf(m[e] * scale[0] + base[e]) + eps;
  else if (e < 2 * N) post_out[t * N + e - N] = 2.0f * sigmoidf(m[e] * scale[1] + base[e]);
  const auto row_sum = [](float v) {
#pragma unroll
    for (int o = 1; o < N; o <<= 1) v += __shfl_xor(v, o);
    return v;
  };
  const auto col_sum = [](float v) {
#pragma unroll
    for (int o = N; o < kLanes; o <<= 1) v += __shfl_xor(v, o);
    return v;
  };
  float c = m[2 * N + e] * scale[2] + base[2 * N + e];
  float mx = c;
#pragma unroll
  for (int o = 1; o < N; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  c = expf(c - mx);
  c = c * (1.0f / row_sum(c)) + eps;
  c *= 1.0f / (col_sum(c) + eps);
  for (int it = 1; it < iters; ++it) {
    c *= 1.0f / (row_sum(c) + eps);
    c *= 1.0f / (col_sum(c) + eps);
  }
  comb_out[t * kLanes + e] = c;
}

}  // namespace gen
