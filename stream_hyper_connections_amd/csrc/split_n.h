// Feature-split fused step for n in {2, 4} streams on the general packed
// layout (mhc_pack_wmix_n): the kernel behind mhc_fused_step_n / mhc_mixes_n
// when a workspace is given. bf16 streams, d = ns * S with S = 64 * NR
// features per slice and ns <= 64 slices.
//
// Included by mhc.hip after split_kernel.h and general_n.h; the design is
// that of the n = 4 feature-split kernel (fsplit), written for any n:
//   * Workgroup (group g, slice c) = (ticket / ns, ticket % ns) keeps slice c of the features of every
//     stream row and its part of the packed projection (S / 32 steps of n
//     streams x 3 T1 tiles, T1 = ceil((2+n)n / 16); term-major hi | mid | lo)
//     in LDS for the whole call, and takes 128-token batches b = g, g + G, ...
//     Wave w owns tokens 16w .. 16w + 15 of a batch.
//   * Loads and stores move 8 token rows x 128 bytes per instruction ("half
//     rounds" of 64 features, NR rounds per batch).
//   * Per token the slice yields (2+n)n projection partials, sum x'^2 and sum
//     h^2; they go to a workspace ring (kRing slots per group) as rows of
//     kRow floats, counted per group and slot as in fsplit.
//   * One batch later each wave waits for all ns slices, sums the h^2
//     partials of its tokens and writes y of its slice from h kept in
//     registers; waves 0 .. ceil(128 / ns) - 1 (ns >= 16) each sum the ns
//     partial rows of one token of the batch (token c + ns * wave) and write
//     its mixes row.
//     gen::sinkhorn_kernel then runs the split and Sinkhorn on every token.
// The cross-workgroup protocol, the bounded waits, the status and abort
// words, the start-order tickets that assign the groups and the end-of-call
// reset of the header are those of fsplit (see split_kernel.h); the host
// launches one workgroup per CU, as an ordinary kernel or, on request,
// cooperatively.

namespace fsn {

using pipe::bload;
using pipe::bstore;
using pipe::dpp;
using pipe::kOutOfRange;
using pipe::make_rsrc;
using pipe::rsrc_t;
using fsplit::kBatch;
using fsplit::kCtrStride;
using fsplit::kHdr;
using fsplit::kMaxSlices;
using fsplit::kRing;
using fsplit::kSC1;
using fsplit::kThreads;
using fsplit::kWaves;
using fsplit::wait_count;
using fsplit::waitcnt_vm;

template <int N>
struct Dims {
  static constexpr int kMix = (2 + N) * N;
  static constexpr int kT1 = (kMix + 15) / 16;        // tiles of one weight term
  static constexpr int kTiles = 3 * kT1;              // packed tiles per stream and step
  static constexpr int kCols = 16 * kTiles;           // packed columns
  static constexpr int kStepBytes = N * kTiles * 1024;
  static constexpr int kRow = 16 * ((kMix + 2 + 15) / 16);   // floats per token and slice
  static constexpr int kChunks = kRow / 4;            // 16-byte chunks of a row
  static constexpr int kCoef = N * N + 2 * N;         // comb_in, post_in, pre_in
};

// slice shapes: S = 64 * NR features; the packed projection slice and the
// per-wave buffers must fit the 160 KB of LDS
template <int N>
__host__ __device__ constexpr int max_rounds() { return N == 2 ? 4 : 2; }

// workspace layout for `groups` groups of `ns` slices (as fsplit, with rows
// of kRow floats): status word, one counter per (group, slot), then from the
// end of the 16 KB header the partial rows [group][slot][slice][token][kRow],
// the h^2 partials [group][slot][slice][token], then the mixes rows
// [T][(2+n)n]
template <int N>
__host__ __device__ constexpr int64_t ctr_off(int g, int slot) {
  return kHdr + ((int64_t)g * kRing + slot) * kCtrStride;
}
template <int N>
__host__ __device__ constexpr int64_t mp_off(int) { return fsplit::kWsHeader; }
template <int N>
__host__ __device__ constexpr int64_t mp_slot_bytes(int ns) {
  return (int64_t)ns * kBatch * Dims<N>::kRow * 4;
}
template <int N>
__host__ __device__ constexpr int64_t hs_off(int groups, int ns) {
  return mp_off<N>(groups) + (int64_t)groups * kRing * mp_slot_bytes<N>(ns);
}
template <int N>
__host__ __device__ constexpr int64_t hs_slot_bytes(int ns) { return (int64_t)ns * kBatch * 4; }
template <int N>
__host__ __device__ constexpr int64_t mix_off(int groups, int ns) {
  return hs_off<N>(groups, ns) + (int64_t)groups * kRing * hs_slot_bytes<N>(ns);
}
template <int N>
__host__ __device__ constexpr int64_t workspace_bytes(int groups, int ns, int64_t tokens) {
  return mix_off<N>(groups, ns) + ((tokens * Dims<N>::kMix * 4 + 255) / 256) * 256;
}

template <int N>
struct __align__(16) WaveSmem {
  union {
    struct {
      u32x4 xs[2][kTok * 8];            // A-operand staging: [token][8 chunks of 16 B], swizzled
      float coef[kTok][Dims<N>::kCoef];
    } e;
    float cst[kTok][Dims<N>::kCols];    // projection partials before the hi/mid/lo sums
  } u;
  float rh[kTok];
};

template <int N, int NR>
struct __align__(16) Smem {
  u32x4 w[2 * NR * Dims<N>::kStepBytes / 16];   // projection slice, packed B-operand order
  WaveSmem<N> wv[kWaves];
  float gamma[64 * NR];
  uint32_t lcount[kRing];
  uint32_t ticket;
};

struct Args {
  char* ws;      // workspace
  float* mix;    // [T][(2+n)n] mixes rows (mix_out, or a workspace region)
  int groups;    // G
  int ns;        // slices per group (d = ns * S)
  fsplit::BatchSpans spans;
};

template <int N>
struct Items {   // one load group: n stream rows + the F row, 16 B per lane each
  u32x4 x[N];
  u32x4 f;
};

struct Rs {      // buffer resources of one wave's 16 tokens of one batch
  rsrc_t x, f, xo, y, cb, po, pr;
};

struct Cf {      // raw coefficient loads of one batch (16-byte chunks)
  u32x4 cb, po, pr;
};

__device__ __forceinline__ f32x4 bload_sc1(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(f32x4, bload<kSC1>(r, voff, soff));
}

// hc_post, sums of squares and hc_pre for the 8 features of one lane, in the
// operation order of the n = 4 kernels: xo[k] = bf16(sum_j C[j][k] x_j + U[k]
// f), h = bf16(sum_k P[k] xo[k]).
template <int N>
__device__ __forceinline__ void elementwise(const Items<N>& in, const float (&C)[N][N],
                                            const float (&U)[N], const float (&P)[N],
                                            u32x4 (&xo)[N], u32x4& hp, float& ss, float& hs) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float a0[N], a1[N];
#pragma unroll
    for (int j = 0; j < N; ++j) {
      a0[j] = bf_lo(in.x[j][q]);
      a1[j] = bf_hi(in.x[j][q]);
    }
    const float f0v = bf_lo(in.f[q]), f1v = bf_hi(in.f[q]);
#pragma unroll
    for (int k = 0; k < N; ++k) {
      float v0 = a0[0] * C[0][k];
      float v1 = a1[0] * C[0][k];
#pragma unroll
      for (int j = 1; j < N; ++j) {
        v0 = fmaf(a0[j], C[j][k], v0);
        v1 = fmaf(a1[j], C[j][k], v1);
      }
      v0 = fmaf(f0v, U[k], v0);
      v1 = fmaf(f1v, U[k], v1);
      xo[k][q] = pack_bf16x2(v0, v1);
    }
  }
  float ssa = 0.f, ssb = 0.f, hsa = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float r0[N], r1[N];
#pragma unroll
    for (int k = 0; k < N; ++k) {
      r0[k] = bf_lo(xo[k][q]);
      r1[k] = bf_hi(xo[k][q]);
      ssa = fmaf(r0[k], r0[k], ssa);
      ssb = fmaf(r1[k], r1[k], ssb);
    }
    float h0 = P[0] * r0[0], h1 = P[0] * r1[0];
#pragma unroll
    for (int k = 1; k < N; ++k) {
      h0 = fmaf(P[k], r0[k], h0);
      h1 = fmaf(P[k], r1[k], h1);
    }
    const uint32_t w = pack_bf16x2(h0, h1);
    hp[q] = w;
    const float q0 = bf_lo(w), q1 = bf_hi(w);
    hsa = fmaf(q0, q0, hsa);
    hsa = fmaf(q1, q1, hsa);
  }
  ss += ssa + ssb;
  hs += hsa;
}

// hc_mixes alone: the input streams are the new streams.
template <int N>
__device__ __forceinline__ void streams_only(const Items<N>& in, u32x4 (&xo)[N], float& ss) {
  float ssa = 0.f, ssb = 0.f;
#pragma unroll
  for (int k = 0; k < N; ++k) {
    xo[k] = in.x[k];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float r0 = bf_lo(in.x[k][q]), r1 = bf_hi(in.x[k][q]);
      ssa = fmaf(r0, r0, ssa);
      ssb = fmaf(r1, r1, ssb);
    }
  }
  ss += ssa + ssb;
}

template <int N, int NR, int MODE>
__global__ __launch_bounds__(kThreads) void split_kernel(StepArgs a, Args fs) {
  using D = Dims<N>;
  constexpr bool kFull = MODE == kFused;
  constexpr int kMix = D::kMix;
  constexpr int kTiles = D::kTiles;
  constexpr int kT1 = D::kT1;
  constexpr int kRow = D::kRow;
  constexpr int kCH = D::kChunks;           // lanes per row of the exchange
  constexpr int kGroupsPerWave = 64 / kCH;  // slice groups of the row sum
  constexpr int S = 64 * NR;                // features per slice
  constexpr int KS = S / 32;                // packed steps per slice
  constexpr int NI = 2 * NR;                // load groups per wave and batch
  static_assert(NR >= 1 && NR <= max_rounds<N>(), "slice shape");
  __shared__ Smem<N, NR> sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = fs.groups;
  const int ticket = fsplit::take_ticket(fs.ws, &sm.ticket);
  const int g = ticket / fs.ns;
  const int c = ticket % fs.ns;
  const fsplit::BatchSpans spans = fs.spans.uniform();
  const int d = a.d;
  const uint32_t d2 = (uint32_t)d * 2;
  const uint32_t rowx = N * d2, rowf = d2;
  const int f0 = c * S;                     // first feature of the slice
  WaveSmem<N>& wsm = sm.wv[wave];
  char* const ws = fs.ws;
  const int ns = fs.ns;
  const rsrc_t wsr = make_rsrc(ws, (uint32_t)mix_off<N>(G, ns));

  {
    const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const char*>(a.wpk) +
                                                      (size_t)c * KS * D::kStepBytes);
    fsplit::stage_lds<KS * D::kStepBytes / 16>(sm.w, src, [](int i) { return i; });
    if constexpr (kFull)
      for (int i = tid; i < S; i += kThreads) sm.gamma[i] = a.gamma[f0 + i];
    if (tid < kRing) sm.lcount[tid] = 0;
  }
  __syncthreads();

  // lane map of the half rounds: token 8h + m8, 16-byte chunk x8 of 64 features
  const int m8 = lane >> 3, x8 = lane & 7;
  const int t16 = lane & 15, g16 = lane >> 4;
  uint32_t vxh[2], vfh[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    vxh[h] = (uint32_t)(8 * h + m8) * rowx + (uint32_t)f0 * 2 + 16u * x8;
    vfh[h] = (uint32_t)(8 * h + m8) * rowf + (uint32_t)f0 * 2 + 16u * x8;
  }

  auto batch_rs = [&](int i) {
    int64_t bt0;
    int blen;
    spans.span(g, i, G, bt0, blen);
    // wave-uniform by construction; said so explicitly, or the compiler keeps
    // the buffer resources in vector registers and loops over lanes
    const int64_t t0 = fsplit::uniform64(bt0 + (int64_t)wave * kTok);
    const int ntok = __builtin_amdgcn_readfirstlane(max(0, min(kTok, blen - wave * kTok)));
    const int64_t tb = ntok > 0 ? t0 : 0;
    Rs r;
    r.x = make_rsrc(static_cast<const char*>(a.x) + tb * rowx, ntok * rowx);
    if constexpr (kFull) {
      r.f = make_rsrc(static_cast<const char*>(a.f) + tb * rowf, ntok * rowf);
      r.xo = make_rsrc(static_cast<char*>(a.x_out) + tb * rowx, ntok * rowx);
      r.y = make_rsrc(static_cast<char*>(a.y_out) + tb * rowf, ntok * rowf);
      r.cb = make_rsrc(a.comb_in + tb * N * N, ntok * N * N * 4);
      r.po = make_rsrc(a.post_in + tb * N, ntok * N * 4);
      r.pr = make_rsrc(a.pre_in + tb * N, ntok * N * 4);
    } else {
      r.f = r.xo = r.y = r.cb = r.po = r.pr = r.x;   // unused
    }
    return r;
  };
  auto load_half = [&](Items<N>& it, const Rs& r, int rr, int h) {
    const uint32_t col = 128u * rr;
#pragma unroll
    for (int k = 0; k < N; ++k) it.x[k] = bload<fsplit::kLoadAux>(r.x, vxh[h], col + k * d2);
    if constexpr (kFull) it.f = bload<fsplit::kLoadAux>(r.f, vfh[h], col);
    else it.f = u32x4{0, 0, 0, 0};
  };
  // coefficients of the wave's 16 tokens as 16-byte chunks: lane l loads
  // chunk l of the comb block [16][n][n] (4 n^2 chunks) and of the post and
  // pre blocks [16][n] (4 n chunks); a chunk may span two tokens (n = 2)
  constexpr int kCbChunks = kTok * N * N / 4;
  constexpr int kPChunks = kTok * N / 4;
  static_assert(kCbChunks <= 64, "one comb chunk per lane");
  auto load_coef = [&](Cf& cf, const Rs& r) {
    if constexpr (!kFull) return;
    cf.cb = bload<0>(r.cb, lane < kCbChunks ? 16u * lane : kOutOfRange, 0);
    cf.po = bload<0>(r.po, lane < kPChunks ? 16u * lane : kOutOfRange, 0);
    cf.pr = bload<0>(r.pr, lane < kPChunks ? 16u * lane : kOutOfRange, 0);
  };
  auto store_coef = [&](const Cf& cf) {
    if constexpr (!kFull) return;
    float* co = &wsm.u.e.coef[0][0];
    if (lane < kCbChunks) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int idx = 4 * lane + e;
        co[(idx / (N * N)) * D::kCoef + idx % (N * N)] = __uint_as_float(cf.cb[e]);
      }
    }
    if (lane < kPChunks) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int idx = 4 * lane + e;
        co[(idx / N) * D::kCoef + N * N + idx % N] = __uint_as_float(cf.po[e]);
        co[(idx / N) * D::kCoef + N * N + N + idx % N] = __uint_as_float(cf.pr[e]);
      }
    }
  };
  auto get_coef = [&](int tau, float (&C)[N][N], float (&U)[N], float (&P)[N]) {
    const float* row = wsm.u.e.coef[tau];
#pragma unroll
    for (int j = 0; j < N; ++j)
#pragma unroll
      for (int k = 0; k < N; ++k) C[j][k] = row[j * N + k];
#pragma unroll
    for (int k = 0; k < N; ++k) {
      U[k] = row[N * N + k];
      P[k] = row[N * N + N + k];
    }
  };
  auto wlds = [&](int step, int k, int q) -> bf16x8 {
    return __builtin_bit_cast(bf16x8, sm.w[((step * N + k) * kTiles + q) * 64 + lane]);
  };
  auto sidx = [](int tok, int chunk) { return tok * 8 + (chunk ^ ((tok >> 1) & 7)); };

  const int nbg = spans.count(g);

  auto count_batch = [&](int i) {
    const int slot = i % kRing;
    uint32_t old = 0;
    if (lane == 0)
      old = __hip_atomic_fetch_add(&sm.lcount[slot], 1u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_WORKGROUP);
    old = __builtin_amdgcn_readfirstlane(old);
    if (old % kWaves == kWaves - 1 && lane == 0)
      __hip_atomic_fetch_add(reinterpret_cast<uint32_t*>(ws + ctr_off<N>(g, slot)), 1u,
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };

  // finish batch i: y of the wave's tokens; the mixes row of token c + ns*wave
  auto finish = [&](int i, const Rs& r, const u32x4 (&hk)[NI]) {
    const int slot = i % kRing;
    const uint32_t target = (uint32_t)ns * (uint32_t)(i / kRing + 1);
    wait_count(ws, ctr_off<N>(g, slot), target);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_sched_barrier(0);
    const int64_t slot_id = (int64_t)g * kRing + slot;
    // sum of h^2 over the ns slices for the wave's 16 tokens: lane l reads
    // slices l/2 and l/2 + 32, tokens 8(l&1) .. 8(l&1)+7
    f32x4 p0 = {0.f, 0.f, 0.f, 0.f}, p1 = p0;
    if constexpr (kFull) {
      const uint32_t hbase = (uint32_t)(hs_off<N>(G, ns) + slot_id * hs_slot_bytes<N>(ns)) +
                             (uint32_t)((wave * kTok + 8 * (lane & 1)) * 4);
      const int s0 = lane >> 1, s1 = 32 + (lane >> 1);
      const uint32_t o0 = hbase + (uint32_t)(s0 * kBatch * 4);
      const uint32_t o1 = s1 < ns ? hbase + (uint32_t)(s1 * kBatch * 4) : kOutOfRange;
      p0 = bload_sc1(wsr, s0 < ns ? o0 : kOutOfRange, 0);
      p1 = bload_sc1(wsr, s0 < ns ? o0 : kOutOfRange, 16);
      p0 += bload_sc1(wsr, o1, 0);
      p1 += bload_sc1(wsr, o1, 16);
    }
    // the mixes row of token tb = c + ns * wave of the batch: lane l reads
    // 16-byte chunk l % kCH of the row of slices l / kCH + kGroupsPerWave * j
    const int tb = c + ns * wave;
    int64_t bt0;
    int blen;
    spans.span(g, i, G, bt0, blen);
    const bool sk = tb < blen;
    constexpr int kSk = (kMaxSlices + kGroupsPerWave - 1) / kGroupsPerWave;
    f32x4 sk_part[kSk];
    {
      const uint32_t base = (uint32_t)(mp_off<N>(G) + slot_id * mp_slot_bytes<N>(ns)) +
                            (uint32_t)((tb * kRow + 4 * (lane % kCH)) * 4);
#pragma unroll
      for (int j = 0; j < kSk; ++j) {
        const int sl = lane / kCH + kGroupsPerWave * j;
        sk_part[j] = bload_sc1(
            wsr, sk && sl < ns ? base + (uint32_t)(sl * kBatch * kRow * 4) : kOutOfRange, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kFull) {
      float rh[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        rh[e] = rsqrtf(fsplit::sum_same_parity(p0[e]) / (float)d + a.norm_eps);
        rh[4 + e] = rsqrtf(fsplit::sum_same_parity(p1[e]) / (float)d + a.norm_eps);
      }
      if (lane < 2) {
        *reinterpret_cast<f32x4*>(&wsm.rh[8 * lane]) = f32x4{rh[0], rh[1], rh[2], rh[3]};
        *reinterpret_cast<f32x4*>(&wsm.rh[8 * lane + 4]) = f32x4{rh[4], rh[5], rh[6], rh[7]};
      }
      __builtin_amdgcn_wave_barrier();
      // y = bf16(gamma * (h * rh)) ([RN] RMSNorm) for the slice
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const int rr = j >> 1, h = j & 1;
        const float rhv = wsm.rh[8 * h + m8];
        const u32x4 y = norm_bf(hk[j], sm.gamma, 64 * rr + 8 * x8, rhv);
        bstore<fsplit::kYAux>(r.y, vfh[h], 128u * rr, y);
      }
    }
    if (sk) {
      f32x4 acc = sk_part[0];
#pragma unroll
      for (int j = 1; j < kSk; ++j) acc += sk_part[j];
      // sum over the slice groups: lanes l ^ kCH, ..., ^ 32
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float x = acc[e];
        if constexpr (kCH == 4) x = pipe::col_sum(x);   // lanes l, l^4, l^8, l^12 of a row
        else x += dpp<pipe::kRowRor8>(x);                // kCH == 8: lanes l, l^8 of a row
        x += __shfl_xor(x, 16);
        v[e] = x + __shfl_xor(x, 32);
      }
      // every lane holds floats 4(l % kCH) .. +3 of the token's row; float kMix
      // is the sum of x'^2
      const float ssum = __shfl(v[kMix % 4], kMix / 4);
      const float rr = rsqrtf(ssum / (float)(N * d) + a.norm_eps);
      const int64_t t = bt0 + tb;
      if (lane < kCH && 4 * lane < kMix) {
        st4f(&fs.mix[t * kMix + 4 * lane], f32x4{v[0] * rr, v[1] * rr, v[2] * rr, v[3] * rr});
      }
    }
  };

  Rs rcur = batch_rs(0), rprev = rcur;
  Cf cf;
  Items<N> bufA, bufB;
  u32x4 hcur[NI], hprev[NI];
  if (nbg > 0) {
    load_coef(cf, rcur);
    load_half(bufA, rcur, 0, 0);
    load_half(bufB, rcur, 0, 1);
  }

  for (int i = 0; i < nbg; ++i) {
    store_coef(cf);
    __builtin_amdgcn_wave_barrier();
    f32x4 acc[kTiles];
#pragma unroll
    for (int q = 0; q < kTiles; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
    float ssA[2] = {0.f, 0.f}, hsA[2] = {0.f, 0.f};

#pragma unroll
    for (int rr = 0; rr < NR; ++rr) {
      // streaming phase at high wave priority, the MFMA phase at the base one
      // (as in fsplit::split_kernel)
      __builtin_amdgcn_s_setprio(3);
      u32x4 xo0[N], xo1[N];
      float C[N][N], U[N], P[N];
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (kFull) get_coef(m8, C, U, P);
      if constexpr (kFull) elementwise<N>(bufA, C, U, P, xo0, hcur[2 * rr], ssA[0], hsA[0]);
      else streams_only<N>(bufA, xo0, ssA[0]);
#pragma unroll
      for (int k = 0; k < N; ++k)
        // new streams non-temporal, as in fsplit's 256-feature slices (n = 2 at
        // 65,536 x 5120, 256 features: 0.838 -> 0.830 ms per call)
        if constexpr (kFull) bstore<fsplit::kXoAuxWide>(rcur.xo, vxh[0], 128u * rr + k * d2, xo0[k]);
      __builtin_amdgcn_sched_barrier(0);
      if (rr + 1 < NR) load_half(bufA, rcur, rr + 1, 0);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (kFull) get_coef(8 + m8, C, U, P);
      if constexpr (kFull) elementwise<N>(bufB, C, U, P, xo1, hcur[2 * rr + 1], ssA[1], hsA[1]);
      else streams_only<N>(bufB, xo1, ssA[1]);
#pragma unroll
      for (int k = 0; k < N; ++k)
        if constexpr (kFull) bstore<fsplit::kXoAuxWide>(rcur.xo, vxh[1], 128u * rr + k * d2, xo1[k]);
      __builtin_amdgcn_sched_barrier(0);
      if (rr + 1 < NR) load_half(bufB, rcur, rr + 1, 1);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(0);
      // new streams of the two halves -> A operands, 2 K-steps per stream
#pragma unroll
      for (int k = 0; k < N; ++k) {
        u32x4* buf = wsm.u.e.xs[k & 1];
        buf[sidx(m8, x8)] = xo0[k];
        buf[sidx(8 + m8, x8)] = xo1[k];
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2) {
          const bf16x8 A = __builtin_bit_cast(bf16x8, buf[sidx(t16, 4 * q2 + g16)]);
          const int step = 2 * rr + q2;
#pragma unroll
          for (int q = 0; q < kTiles; ++q)
            acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, wlds(step, k, q), acc[q], 0, 0, 0);
        }
        __builtin_amdgcn_wave_barrier();
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- publish the slice's per-token partials of batch i ----
    {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        ssA[h] = pipe::quad_sum(ssA[h]);
        ssA[h] += __shfl_xor(ssA[h], 4);
        hsA[h] = pipe::quad_sum(hsA[h]);
        hsA[h] += __shfl_xor(hsA[h], 4);
      }
      const int u = lane >> 2;   // token this lane publishes
      const int src = 8 * (u & 7);
      const float s0 = __shfl(ssA[0], src), s1 = __shfl(ssA[1], src);
      const float h0 = __shfl(hsA[0], src), h1 = __shfl(hsA[1], src);
      const float ssu = u < 8 ? s0 : s1, hsu = u < 8 ? h0 : h1;
      // projection partials -> per-token rows, hi + mid + lo (term-major tiles)
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int q = 0; q < kTiles; ++q) {
#pragma unroll
        for (int e = 0; e < 4; ++e) wsm.u.cst[4 * g16 + e][16 * q + t16] = acc[q][e];
      }
      __builtin_amdgcn_wave_barrier();
      constexpr int kPer = kMix / 4;   // mixes per lane (4 lanes per token)
      float mv[kPer];
#pragma unroll
      for (int jj = 0; jj < kPer; ++jj) {
        const int row = kPer * (lane & 3) + jj;
        mv[jj] = (wsm.u.cst[u][row] + wsm.u.cst[u][16 * kT1 + row]) + wsm.u.cst[u][32 * kT1 + row];
      }
      __builtin_amdgcn_wave_barrier();
      // the 16 token rows (mixes, x'^2, h^2, zero pad) in LDS, then written as
      // kCH lanes x 16 bytes per row
      float(*rows)[kRow] = reinterpret_cast<float(*)[kRow]>(&wsm.u.cst[0][0]);
#pragma unroll
      for (int jj = 0; jj < kPer; ++jj) rows[u][kPer * (lane & 3) + jj] = mv[jj];
      if ((lane & 3) == 0) {
        rows[u][kMix] = ssu;
        rows[u][kMix + 1] = hsu;
#pragma unroll
        for (int e = kMix + 2; e < kRow; ++e) rows[u][e] = 0.f;
      }
      __builtin_amdgcn_wave_barrier();
      const int slot = i % kRing;
      const int64_t slot_id = (int64_t)g * kRing + slot;
      const uint32_t rows_off = (uint32_t)(mp_off<N>(G) + slot_id * mp_slot_bytes<N>(ns)) +
                                (uint32_t)((c * kBatch + wave * kTok) * kRow * 4);
      constexpr int kRowsPerInst = 64 / kCH;
#pragma unroll
      for (int hh = 0; hh < kTok / kRowsPerInst; ++hh) {
        const int tk = kRowsPerInst * hh + lane / kCH;
        const u32x4 v = *reinterpret_cast<const u32x4*>(&rows[tk][4 * (lane % kCH)]);
        bstore<kSC1>(wsr, rows_off + (uint32_t)(tk * kRow * 4 + 16 * (lane % kCH)), 0, v);
      }
      {
        // sum of h^2 of the 16 tokens: 4 lanes x 4 tokens
        const int t0 = 4 * (lane & 3);
        const u32x4 v = {__float_as_uint(rows[t0][kMix + 1]), __float_as_uint(rows[t0 + 1][kMix + 1]),
                         __float_as_uint(rows[t0 + 2][kMix + 1]),
                         __float_as_uint(rows[t0 + 3][kMix + 1])};
        const uint32_t hoff = (uint32_t)(hs_off<N>(G, ns) + slot_id * hs_slot_bytes<N>(ns)) +
                              (uint32_t)((c * kBatch + wave * kTok + t0) * 4);
        if constexpr (kFull) bstore<kSC1>(wsr, lane < 4 ? hoff : kOutOfRange, 0, v);
      }
      __builtin_amdgcn_wave_barrier();
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_sched_barrier(0);

      // next batch's first round and coefficients (empty ranges past the end)
      const Rs rnext = batch_rs(i + 1);
      load_coef(cf, rnext);
      load_half(bufA, rnext, 0, 0);
      load_half(bufB, rnext, 0, 1);
      __builtin_amdgcn_sched_barrier(0);
      // wait for the exchange stores (the loads above were issued after them)
      // and count the batch
      constexpr int kAfter = kFull ? 2 * (N + 1) + 3 : 2 * N;
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(kAfter));
      __builtin_amdgcn_sched_barrier(0);
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      count_batch(i);
      if (i > 0) finish(i - 1, rprev, hprev);
      rprev = rcur;
      rcur = rnext;
#pragma unroll
      for (int j = 0; j < NI; ++j) hprev[j] = hcur[j];
    }
  }
  if (nbg > 0) finish(nbg - 1, rprev, hprev);
  fsplit::release_workspace(ws, ctr_off<N>(0, 0), G * kRing);
}

}  // namespace fsn
