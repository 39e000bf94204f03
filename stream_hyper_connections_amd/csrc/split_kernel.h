// Feature-split fused step (bf16 streams, d = ns * S with S = 64 * NR + 32 * TAIL,
// NR >= 1; three-term projection: S <= 160, ns <= 64 slices; two-term
// projection: S = 256, 16 <= ns <= 24): the kernel behind mhc_fused_step when
// a workspace is given.
//
// Included by mhc.hip (one translation unit); uses its helpers and the pipe::
// buffer-instruction wrappers.
//
// Why a second kernel. The tile kernel re-reads the packed projection (three
// bf16 terms of W, 20 KB per 32 features) from L2 for every 16-token tile:
// twice the stream bytes through each CU's vector-memory path. Its lane layout
// (16 token rows x 64 bytes per load instruction, the MFMA operand order) also
// moves at most ~3 TB/s even as a plain copy, against 4.3-4.8 TB/s for 4-8 rows
// x 128-256 bytes. Here every CU owns one slice of the features for good:
//
//   * Workgroup (group g, slice c): g = ticket / ns, c = ticket % ns, where the
//     ticket is the workgroup's place in start order (take_ticket), with G
//     groups of ns workgroups (the host picks ns; d = 5120 runs 20 slices of
//     256 features). Slice c is features [c*S, (c+1)*S) of every stream row,
//     F row, new-stream row and y row; its W slice (S/32 packed steps: 96 KB
//     for S = 256 with two terms, 80 KB for S = 128 with three) is loaded
//     into LDS once and used for every token the group processes. Groups
//     take 128-token batches b = g, g+G, ... while every group has one; the
//     tokens after the last such round are shared out evenly (BatchSpans).
//     Wave w of a workgroup owns tokens 16w .. 16w+15 of each batch.
//   * Loads and stores move 8 token rows x 128 bytes per instruction ("half
//     rounds" of 64 features); an S % 64 = 32 remainder ("tail", 16 rows x 64
//     bytes) sits at the 128-byte-aligned end of the slice (first for odd c).
//     New streams pass through a 2 KB per-wave LDS buffer per stream to reach
//     the MFMA A-operand order (row = token, 8 consecutive features per lane).
//   * Per token the slice yields 24 projection partials, sum x'^2 and sum h^2.
//     They go to a workspace ring (kRing slots per group) as whole 128-byte
//     rows with device-scope (sc1) stores; the last wave of a workgroup to
//     finish a batch bumps the group's counter for that slot (one device-scope
//     atomic per workgroup and batch).
//   * One batch later each wave waits for all ns slices of the batch, sums the
//     ns partial sums of h^2 of its 16 tokens and writes y for its slice from h
//     kept in registers; waves 0 .. ceil(128 / ns) - 1 each sum the ns partial
//     rows of one token of the batch (token c + ns * wave), apply the RMS
//     scaling and write its 24 mixes (alternating the wave halves from batch
//     to batch was 0.6% slower); tail_kernel then runs the split and the 4x4
//     Sinkhorn on all tokens (one thread per token).
//
// Cross-workgroup protocol (correct wherever the workgroups run; the group ->
// XCD mapping only matters for speed). In the GFX942 memory model of the LLVM
// AMDGPU backend (also applied to gfx950) an agent-scope relaxed atomic load
// or store is a load or store with the sc1 bit, so every exchange access
// below is, per dword, such an atomic: coherent across the XCDs' L2 caches.
//   * writer: exchange stores carry sc1; s_waitcnt makes them complete (vmcnt
//     counts loads and stores together and decrements in issue order on this
//     architecture family, so waiting until only the loads issued after them
//     remain outstanding suffices) before the wave's LDS increment; the wave
//     that completes the workgroup's count issues an agent-scope atomic add
//     on the counter. That is an agent-scope release minus the L2 write-back,
//     which only stores without sc1 would need.
//   * reader: polls the counter with agent-scope atomic loads until it
//     reaches ns * (generation + 1); the value decides the loop exit, so the
//     exchange loads (sc1, never served from a stale cache line) issue only
//     after it: an agent-scope acquire minus the cache invalidation, which
//     only loads without sc1 would need.
//   * slots: a workgroup writes batch i's slot only after it has seen every
//     workgroup of the group finish batch i-2, whose waves had all finished
//     reading batch i-4 before that; four slots are therefore never read and
//     written at once.
//   * every wait is bounded: after kSpinLimit polls the wave sets the status
//     word (workspace offset 0) and the call's abort word (offset 4) and stops
//     waiting (outputs are then invalid); later waits of the same call return
//     at once once the abort word is set. The library never clears the status
//     word: it reports every give-up since the caller last cleared it.
//   * the workspace cleans up after itself: each workgroup, once all of its
//     waves are done with the exchange, adds one to the done word (offset 8)
//     with an acquire-release atomic; the workgroup that brings it to the
//     grid size resets the counters, the abort word, the start-order ticket
//     count (offset 12) and the done word. The
//     next call therefore finds the header as the caller first provided it
//     (zero-filled), without a clearing launch.
// Residency: groups are filled in start order (take_ticket), so the kernel
// completes whenever the device can eventually hold ns of its workgroups at
// once. The host launches one workgroup per CU (at most), as an ordinary
// kernel or, on request, cooperatively.

namespace fsplit {

using pipe::bload;
using pipe::bstore;
using pipe::col_sum;
using pipe::dpp;
using pipe::kNT;
using pipe::kOutOfRange;
using pipe::make_rsrc;
using pipe::quad_max;
using pipe::quad_sum;
using pipe::rsrc_t;

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kMaxSlices = 64;                 // workgroups per group = feature slices (at most)
constexpr int kBatch = kWaves * kTok;          // 128 tokens per batch
constexpr int kRing = 4;                       // exchange slots per group
constexpr int kRow = 32;                       // floats per token and slice: 24 mixes, x'^2, h^2, pad
constexpr int kTiles = kTilesBf;
constexpr int kCols = 3 * kMix;                // 72 packed columns in use
constexpr int kMaxS = 160;                     // features per slice (d <= 5120)
constexpr int kMaxSW = 256;                    // features per slice, two-term projection
constexpr int kMaxSlicesW = 24;                // slices per group, two-term projection
constexpr int kStepBytes = kStreams * kTiles * 1024;   // packed bytes per 32 features
constexpr int kSC1 = 16;                       // cache-policy bit: device scope
constexpr uint32_t kSpinLimit = 1u << 20;
constexpr int kCtrStride = 128;                // bytes between counters
constexpr int64_t kHdr = 256;                  // status, abort and done words + padding
constexpr int64_t kAbortOff = 4;               // byte offset of the call's abort word
constexpr int64_t kDoneOff = 8;                // byte offset of the done count
constexpr int64_t kTicketOff = 12;             // byte offset of the start-order count
// Bytes reserved at the start of every workspace of the step's kernels: the
// counters of the largest group count (16 groups x kRing slots) fit, and the
// chunked kernels' partial rows start here, so they never overwrite them.
constexpr int64_t kWsHeader = 16384;

constexpr int kRowRor2 = 0x122;                // DPP row rotate right by 2

// cache policies: stream loads and y stores non-temporal; new-stream stores
// non-temporal on 256-feature slices, default on the narrower ones (each the
// fastest combination measured for its geometry: at 65,536 x 5120 on 256
// features, non-temporal new streams 1.360 against 1.384 ms per call, default
// loads 1.375, default y stores 1.386)
constexpr int kLoadAux = kNT;
constexpr int kXoAuxNarrow = 0;
constexpr int kXoAuxWide = kNT;
constexpr int kYAux = kNT;

// workspace layout for `groups` groups of `ns` slices: status word, one
// counter per (group, slot), then from the end of the 16 KB header per
// (group, slot) the mixes rows [slice][token][kRow] and the h^2 partials
// [slice][token]
__host__ __device__ constexpr int64_t ctr_off(int g, int slot) {
  return kHdr + ((int64_t)g * kRing + slot) * kCtrStride;
}
// (the exchange rows begin after the whole header, whatever the group count,
// so no call's data lands where another call's counters live)
__host__ __device__ constexpr int64_t mp_off(int) { return kWsHeader; }
__host__ __device__ constexpr int64_t mp_slot_bytes(int ns) { return (int64_t)ns * kBatch * kRow * 4; }
__host__ __device__ constexpr int64_t hs_off(int groups, int ns) {
  return mp_off(groups) + (int64_t)groups * kRing * mp_slot_bytes(ns);
}
__host__ __device__ constexpr int64_t hs_slot_bytes(int ns) { return (int64_t)ns * kBatch * 4; }
__host__ __device__ constexpr int64_t mix_off(int groups, int ns) {
  return hs_off(groups, ns) + (int64_t)groups * kRing * hs_slot_bytes(ns);
}
// the mixes region [T][24] follows (used when the caller passes no mix_out)
__host__ __device__ constexpr int64_t workspace_bytes(int groups, int ns, int64_t tokens) {
  return mix_off(groups, ns) + ((tokens * kMix * 4 + 255) / 256) * 256;
}

// s_waitcnt with only vmcnt limited (gfx9 encoding: vmcnt[3:0], expcnt[6:4],
// lgkmcnt[11:8], vmcnt[5:4] in [15:14]).
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

struct __align__(16) WaveSmem {
  union {
    struct {
      u32x4 xs[2][kTok * 8];      // A-operand staging: [token][8 chunks of 16 B], swizzled
      float coef[kTok][24];       // comb_in (16), post_in (4), pre_in (4) of the wave's tokens
    } e;
    float cst[kTok][kCols];       // projection partials before the hi/mid/lo sums
  } u;
  float rh[kTok];                 // 1/rms(h) of the wave's tokens
};

struct __align__(16) Smem {
  u32x4 w[kMaxS / 32 * kStepBytes / 16];   // W slice, packed B-operand order
  WaveSmem wv[kWaves];
  float gamma[kMaxSW];
  float base[kMix];
  float scale[4];
  uint32_t lcount[kRing];
  uint32_t ticket;
};

// A wave-uniform 64-bit value moved to scalar registers.
__device__ __forceinline__ int64_t uniform64(int64_t v) {
  return (int64_t)(((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32)) << 32) |
                   (uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)v));
}

// Token spans of a group's batches. While every group has a whole 128-token
// batch left, group g takes batches b = g + i*G (tokens [128b, 128b + 128));
// the tokens after the last such round (`full` rounds) are split over the
// groups in equal shares of `share` tokens, rounded up to a multiple of 16
// (one wave's rows). So the last round, and the only round of a call of fewer
// than G batches, keeps every group busy on a shorter batch instead of
// leaving groups idle.
struct BatchSpans {
  int64_t rest0;  // first token after the full rounds
  int full;       // rounds of whole 128-token batches
  int rest;       // tokens after them (< G * 128)
  int share;      // tokens per group in the last round (0: none)

  __host__ __device__ static BatchSpans make(int64_t tokens, int groups) {
    const int64_t full = tokens / ((int64_t)groups * kBatch);
    const int64_t rest0 = full * groups * kBatch;
    const int rest = (int)(tokens - rest0);
    return BatchSpans{rest0, (int)full, rest, ((rest + groups - 1) / groups + kTok - 1) / kTok * kTok};
  }
  // the fields as wave-uniform values (the kernel reads them from its
  // argument struct through lambdas; without this the compiler cannot prove
  // the buffer resources built from them uniform and loops over lanes)
  __device__ BatchSpans uniform() const {
    BatchSpans u;
    u.rest0 = (int64_t)__builtin_amdgcn_readfirstlane((uint32_t)rest0) |
              ((int64_t)__builtin_amdgcn_readfirstlane((uint32_t)(rest0 >> 32)) << 32);
    u.full = __builtin_amdgcn_readfirstlane(full);
    u.rest = __builtin_amdgcn_readfirstlane(rest);
    u.share = __builtin_amdgcn_readfirstlane(share);
    return u;
  }
  // batches of group g (32-bit comparisons: every quantity stays scalar)
  __device__ int count(int g) const { return full + (g * share < rest ? 1 : 0); }
  // first token and length of batch i of group g of G (length 0 past the last)
  __device__ void span(int g, int i, int G, int64_t& t0, int& len) const {
    if (i < full) {
      t0 = (int64_t)(g + i * G) * kBatch;
      len = kBatch;
    } else {
      const int off = i == full ? g * share : rest;
      t0 = rest0 + off;
      len = max(0, min(share, rest - off));
    }
  }
};

struct Args {
  char* ws;      // workspace (mhc_fused_step_workspace_bytes)
  float* mix;    // [T][24] mixes (mix_out, or a workspace region)
  int groups;    // G
  int ns;        // slices per group (d = ns * S)
  BatchSpans spans;
};

struct Items {   // one load group: 4 stream rows + the F row, 16 B per lane each
  u32x4 x[4];
  u32x4 f;
};

struct Rs {      // buffer resources of one wave's 16 tokens of one batch
  rsrc_t x, f, xo, y, cb, po, pr;
};

struct Cf {      // raw coefficient loads of one batch (see store_coef)
  u32x4 cb, po, pr;
};

__device__ __forceinline__ f32x4 bload_sc1(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(f32x4, bload<kSC1>(r, voff, soff));
}

// Sum over the lanes l' == l (mod 2) of the wave (32 lanes).
__device__ __forceinline__ float sum_same_parity(float v) {
  v += dpp<pipe::kRowRor8>(v);
  v += dpp<pipe::kRowRor4>(v);
  v += dpp<kRowRor2>(v);
  v += __shfl_xor(v, 16);
  return v + __shfl_xor(v, 32);
}

// hc_post, sums of squares and hc_pre for the 8 features of one lane (the
// arithmetic of the tile kernels): xo[k] = bf16(sum_j C[j][k] x_j + U[k] f),
// h = bf16(sum_k P[k] xo[k]).
__device__ __forceinline__ void elementwise(const Items& in, const float (&C)[4][4],
                                            const float (&U)[4], const float (&P)[4],
                                            u32x4 (&xo)[4], u32x4& hp, float& ss, float& hs) {
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
      float v0 = a0[0] * C[0][k];
      float v1 = a1[0] * C[0][k];
#pragma unroll
      for (int j = 1; j < 4; ++j) {
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
    float r0[4], r1[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      r0[k] = bf_lo(xo[k][q]);
      r1[k] = bf_hi(xo[k][q]);
      ssa = fmaf(r0[k], r0[k], ssa);
      ssb = fmaf(r1[k], r1[k], ssb);
    }
    float h0 = P[0] * r0[0], h1 = P[0] * r1[0];
#pragma unroll
    for (int k = 1; k < 4; ++k) {
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

// hc_mixes alone: the input streams are the new streams; only their sum of
// squares is needed here.
__device__ __forceinline__ void streams_only(const Items& in, u32x4 (&xo)[4], float& ss) {
  float ssa = 0.f, ssb = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
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

// Bounded wait until the counter reaches `target`; false after a time-out or
// when another wave of the call has already timed out.
__device__ __forceinline__ bool wait_count(char* ws, int64_t off, uint32_t target) {
  uint32_t* status = reinterpret_cast<uint32_t*>(ws);
  uint32_t* abort_w = reinterpret_cast<uint32_t*>(ws + kAbortOff);
  const uint32_t* ctr = reinterpret_cast<const uint32_t*>(ws + off);
  for (uint32_t n = 0;; ++n) {
    const uint32_t v = __builtin_amdgcn_readfirstlane(
        __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    if (v >= target) return true;
    if ((n & 31) == 31) {
      const uint32_t ab = __builtin_amdgcn_readfirstlane(
          __hip_atomic_load(abort_w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
      if (ab != 0) return false;
    }
    if (n >= kSpinLimit) {
      __hip_atomic_store(status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(abort_w, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return false;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

// Copy kItems 16-byte items into LDS, item i from src[map(i)], with all of a
// thread's loads issued before its first LDS write. (A plain strided loop
// waits for each load before the next: 10 to 12 dependent global loads per
// thread at kernel start.)
template <int kItems, typename Map>
__device__ __forceinline__ void stage_lds(u32x4* dst, const u32x4* src, Map map) {
  constexpr int kPer = (kItems + kThreads - 1) / kThreads;
  u32x4 v[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int i = (int)threadIdx.x + j * kThreads;
    if (i < kItems) v[j] = src[map(i)];
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int i = (int)threadIdx.x + j * kThreads;
    if (i < kItems) dst[i] = v[j];
  }
}

// The workgroup's place in the order in which the workgroups started (thread
// 0 takes it with one agent-scope atomic; `slot` is LDS). Groups are filled in
// that order: group = ticket / ns, slice = ticket % ns. A workgroup waits only
// for workgroups of its own group, so at any time the only workgroups that
// can be waiting are those of the one group still being filled; all others
// belong to complete groups, which run to the end and free their compute
// units. The kernel therefore finishes whenever the device can eventually
// hold ns of its workgroups at once, launched cooperatively or not.
__device__ __forceinline__ int take_ticket(char* ws, uint32_t* slot) {
  if (threadIdx.x == 0)
    *slot = __hip_atomic_fetch_add(reinterpret_cast<uint32_t*>(ws + kTicketOff), 1u,
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  return (int)__builtin_amdgcn_readfirstlane(*slot);
}

// End of a split kernel: called by every thread of every workgroup after its
// last exchange access. The workgroup that completes the done count resets
// the `nctr` counters at `ctr0` (kCtrStride apart), the abort word, the
// start-order count and the done word, leaving the header zero for the next
// call (every workgroup took its ticket before it counted itself done).
__device__ __forceinline__ void release_workspace(char* ws, int64_t ctr0, int nctr) {
  __syncthreads();
  if (threadIdx.x >= 64) return;
  uint32_t old = 0;
  if (threadIdx.x == 0)
    old = __hip_atomic_fetch_add(reinterpret_cast<uint32_t*>(ws + kDoneOff), 1u,
                                 __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
  old = __builtin_amdgcn_readfirstlane(old);
  if (old != gridDim.x - 1) return;
  for (int i = threadIdx.x; i < nctr; i += 64)
    __hip_atomic_store(reinterpret_cast<uint32_t*>(ws + ctr0 + (int64_t)i * kCtrStride), 0u,
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (threadIdx.x == 0) {
    __hip_atomic_store(reinterpret_cast<uint32_t*>(ws + kAbortOff), 0u, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(reinterpret_cast<uint32_t*>(ws + kTicketOff), 0u, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(reinterpret_cast<uint32_t*>(ws + kDoneOff), 0u, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
}

// TERMS: bf16 terms of W in the projection. 3: hi + mid + lo = w exactly
// (packed tiles 0..4 in LDS). 2: hi + mid (tiles 0..2 of the same packing),
// |w - hi - mid| <= 2^-16 |w|, which leaves LDS room for 256-feature slices.
template <int NR, bool TAIL, int MODE, int TERMS>
__global__ __launch_bounds__(kThreads) void split_kernel(StepArgs a, Args fs) {
  constexpr bool kFull = MODE == kFused;   // else mixes only (hc_mixes)
  __shared__ Smem sm;
  constexpr int S = 64 * NR + (TAIL ? 32 : 0);   // features per slice
  constexpr int KS = S / 32;                      // packed steps per slice
  constexpr int NI = 2 * NR + (TAIL ? 1 : 0);     // load groups per wave and batch
  constexpr int kT = TERMS == 3 ? kTiles : 3;     // packed tiles in LDS per (step, stream)
  constexpr int kC = TERMS * kMix;                // projection columns in use
  constexpr int kSk = (TERMS == 3 ? kMaxSlices : kMaxSlicesW) / 8;   // slice loads per mixes row
  static_assert(TERMS == 2 || TERMS == 3, "terms");
  static_assert(NR >= 1 && S <= (TERMS == 3 ? kMaxS : kMaxSW), "slice shape");
  static_assert(KS * kStreams * kT * 1024 <= (int)sizeof(sm.w), "W slice fits");
  constexpr int kXoAux = TERMS == 2 ? kXoAuxWide : kXoAuxNarrow;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = fs.groups;
  const int ticket = take_ticket(fs.ws, &sm.ticket);
  const int g = ticket / fs.ns;
  const int c = ticket % fs.ns;
  const BatchSpans spans = fs.spans.uniform();
  const int d = a.d;
  const uint32_t d2 = (uint32_t)d * 2;
  const uint32_t rowx = kStreams * d2, rowf = d2;
  const bool odd = (c & 1) != 0;
  const int fr0 = (TAIL && odd) ? 32 : 0;        // slice feature where the rounds start
  const int ftl = odd ? 0 : S - 32;              // slice feature of the tail
  const int f0 = c * S;                          // first feature of the slice
  WaveSmem& wsm = sm.wv[wave];
  char* const ws = fs.ws;
  const int ns = fs.ns;
  const rsrc_t wsr = make_rsrc(ws, (uint32_t)mix_off(G, ns));

  {
    const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const char*>(a.wpk) +
                                                      (size_t)c * KS * kStepBytes);
    if constexpr (TERMS == 3) {
      stage_lds<KS * kStepBytes / 16>(sm.w, src, [](int i) { return i; });
    } else {
      // tiles 0 .. kT-1 of every (step, stream): the hi and mid columns
      stage_lds<KS * kStreams * kT * 64>(sm.w, src, [](int i) {
        const int sk = i / (kT * 64), q = (i / 64) % kT;
        return (sk * kTiles + q) * 64 + (i & 63);
      });
    }
    if constexpr (kFull)
      for (int i = tid; i < S; i += kThreads) sm.gamma[i] = a.gamma[f0 + i];
    if (tid < kMix) sm.base[tid] = a.base[tid];
    if (tid < 3) sm.scale[tid] = a.scale[tid];
    if (tid < kRing) sm.lcount[tid] = 0;
  }
  __syncthreads();

  // lane maps: half rounds (token 8h + m8, 16 B chunk x8 of 64 features) and
  // tail (token t16, chunk g16 of 32 features: the MFMA A-operand order)
  const int m8 = lane >> 3, x8 = lane & 7;
  const int t16 = lane & 15, g16 = lane >> 4;
  uint32_t vxh[2], vfh[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    vxh[h] = (uint32_t)(8 * h + m8) * rowx + (uint32_t)(f0 + fr0) * 2 + 16u * x8;
    vfh[h] = (uint32_t)(8 * h + m8) * rowf + (uint32_t)(f0 + fr0) * 2 + 16u * x8;
  }
  const uint32_t vxt = (uint32_t)t16 * rowx + (uint32_t)(f0 + ftl) * 2 + 16u * g16;
  const uint32_t vft = (uint32_t)t16 * rowf + (uint32_t)(f0 + ftl) * 2 + 16u * g16;

  auto batch_rs = [&](int i) {
    int64_t bt0;
    int blen;
    spans.span(g, i, G, bt0, blen);
    // wave-uniform by construction; said so explicitly, or the compiler keeps
    // the buffer resources in vector registers and loops over lanes
    const int64_t t0 = uniform64(bt0 + (int64_t)wave * kTok);
    const int ntok = __builtin_amdgcn_readfirstlane(max(0, min(kTok, blen - wave * kTok)));
    const int64_t tw = ntok > 0 ? t0 : 0;   // no base pointer past the arrays
    Rs r;
    r.x = make_rsrc(static_cast<const char*>(a.x) + tw * rowx, ntok * rowx);
    if constexpr (kFull) {
      r.f = make_rsrc(static_cast<const char*>(a.f) + tw * rowf, ntok * rowf);
      r.xo = make_rsrc(static_cast<char*>(a.x_out) + tw * rowx, ntok * rowx);
      r.y = make_rsrc(static_cast<char*>(a.y_out) + tw * rowf, ntok * rowf);
      r.cb = make_rsrc(a.comb_in + tw * 16, ntok * 64);
      r.po = make_rsrc(a.post_in + tw * 4, ntok * 16);
      r.pr = make_rsrc(a.pre_in + tw * 4, ntok * 16);
    } else {
      r.f = r.xo = r.y = r.cb = r.po = r.pr = r.x;   // unused
    }
    return r;
  };
  auto load_half = [&](Items& it, const Rs& r, int rr, int h) {
    const uint32_t col = 128u * rr;
#pragma unroll
    for (int k = 0; k < 4; ++k) it.x[k] = bload<kLoadAux>(r.x, vxh[h], col + k * d2);
    if constexpr (kFull) it.f = bload<kLoadAux>(r.f, vfh[h], col);
    else it.f = u32x4{0, 0, 0, 0};
  };
  auto load_tail = [&](Items& it, const Rs& r) {
#pragma unroll
    for (int k = 0; k < 4; ++k) it.x[k] = bload<kLoadAux>(r.x, vxt, k * d2);
    if constexpr (kFull) it.f = bload<kLoadAux>(r.f, vft, 0);
    else it.f = u32x4{0, 0, 0, 0};
  };
  auto load_coef = [&](Cf& cf, const Rs& r) {
    if constexpr (!kFull) return;
    cf.cb = bload<0>(r.cb, 16u * lane, 0);
    cf.po = bload<0>(r.po, lane < kTok ? 16u * lane : kOutOfRange, 0);
    cf.pr = bload<0>(r.pr, lane < kTok ? 16u * lane : kOutOfRange, 0);
  };
  auto store_coef = [&](const Cf& cf) {
    if constexpr (!kFull) return;
    *reinterpret_cast<u32x4*>(&wsm.u.e.coef[lane >> 2][4 * (lane & 3)]) = cf.cb;
    if (lane < kTok) {
      *reinterpret_cast<u32x4*>(&wsm.u.e.coef[lane][16]) = cf.po;
      *reinterpret_cast<u32x4*>(&wsm.u.e.coef[lane][20]) = cf.pr;
    }
  };
  auto get_coef = [&](int tau, float (&C)[4][4], float (&U)[4], float (&P)[4]) {
    const f32x4* row = reinterpret_cast<const f32x4*>(wsm.u.e.coef[tau]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 v = row[j];
#pragma unroll
      for (int k = 0; k < 4; ++k) C[j][k] = v[k];
    }
    const f32x4 u = row[4], p = row[5];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      U[k] = u[k];
      P[k] = p[k];
    }
  };
  auto wlds = [&](int step, int k, int q) -> bf16x8 {
    return __builtin_bit_cast(bf16x8, sm.w[((step * kStreams + k) * kT + q) * 64 + lane]);
  };
  // staging index of (token, 16-byte chunk) with the XOR swizzle that keeps
  // both the row writes and the operand reads free of bank conflicts
  auto sidx = [](int tok, int chunk) { return tok * 8 + (chunk ^ ((tok >> 1) & 7)); };

  const int nbg = spans.count(g);

  // ---- finish batch i: y of the wave's tokens, Sinkhorn of 4 tokens ----
  // The wave's exchange stores of batch i are complete: count them in LDS; the
  // workgroup's eighth count raises the group counter of the slot.
  auto count_batch = [&](int i) {
    const int slot = i % kRing;
    uint32_t old = 0;
    if (lane == 0)
      old = __hip_atomic_fetch_add(&sm.lcount[slot], 1u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_WORKGROUP);
    old = __builtin_amdgcn_readfirstlane(old);
    if (old % kWaves == kWaves - 1 && lane == 0)
      __hip_atomic_fetch_add(reinterpret_cast<uint32_t*>(ws + ctr_off(g, slot)), 1u,
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };

  auto finish = [&](int i, const Rs& r, const u32x4 (&hk)[NI]) {
    const int slot = i % kRing;
    const uint32_t target = (uint32_t)ns * (uint32_t)(i / kRing + 1);
    wait_count(ws, ctr_off(g, slot), target);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);   // exchange loads stay behind the wait
    __builtin_amdgcn_sched_barrier(0);
    const int64_t slot_id = (int64_t)g * kRing + slot;
    // sum of h^2 over the ns slices for the wave's 16 tokens: lane l reads
    // slices l/2 and l/2 + 32, tokens 8(l&1) .. 8(l&1)+7
    f32x4 p0 = {0.f, 0.f, 0.f, 0.f}, p1 = p0;
    if constexpr (kFull) {
      const uint32_t hbase = (uint32_t)(hs_off(G, ns) + slot_id * hs_slot_bytes(ns)) +
                             (uint32_t)((wave * kTok + 8 * (lane & 1)) * 4);
      const int s0 = lane >> 1, s1 = 32 + (lane >> 1);
      const uint32_t o0 = hbase + (uint32_t)(s0 * kBatch * 4);
      const uint32_t o1 = s1 < ns ? hbase + (uint32_t)(s1 * kBatch * 4) : kOutOfRange;
      p0 = bload_sc1(wsr, s0 < ns ? o0 : kOutOfRange, 0);
      p1 = bload_sc1(wsr, s0 < ns ? o0 : kOutOfRange, 16);
      p0 += bload_sc1(wsr, o1, 0);
      p1 += bload_sc1(wsr, o1, 16);
    }
    // wave w takes the batch's token c + ns*w (when it exists) for the mixes
    // row; its partial loads (lane: 16-byte chunk l&7 of the token row, slices
    // l>>3 + 8k) follow at once so their latency hides behind the y work
    const int tb = c + ns * wave;
    int64_t bt0;
    int blen;
    spans.span(g, i, G, bt0, blen);
    const bool sk = tb < blen;
    f32x4 sk_part[kSk];
    {
      const uint32_t base = (uint32_t)(mp_off(G) + slot_id * mp_slot_bytes(ns)) +
                            (uint32_t)((tb * kRow + 4 * (lane & 7)) * 4);
#pragma unroll
      for (int j = 0; j < kSk; ++j) {
        const int sl = (lane >> 3) + 8 * j;
        sk_part[j] = bload_sc1(
            wsr, sk && sl < ns ? base + (uint32_t)(sl * kBatch * kRow * 4) : kOutOfRange, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kFull) {
      float rh[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        rh[e] = rsqrtf(sum_same_parity(p0[e]) / (float)d + a.norm_eps);
        rh[4 + e] = rsqrtf(sum_same_parity(p1[e]) / (float)d + a.norm_eps);
      }
      if (lane < 2) {
        *reinterpret_cast<f32x4*>(&wsm.rh[8 * lane]) = f32x4{rh[0], rh[1], rh[2], rh[3]};
        *reinterpret_cast<f32x4*>(&wsm.rh[8 * lane + 4]) = f32x4{rh[4], rh[5], rh[6], rh[7]};
      }
      __builtin_amdgcn_wave_barrier();
      // y = bf16(gamma * (h * rh)) ([RN] RMSNorm) for the slice
#pragma unroll
      for (int j = 0; j < 2 * NR; ++j) {
        const int rr = j >> 1, h = j & 1;
        const float rhv = wsm.rh[8 * h + m8];
        const u32x4 y = norm_bf(hk[j], sm.gamma, fr0 + 64 * rr + 8 * x8, rhv);
        bstore<kYAux>(r.y, vfh[h], 128u * rr, y);
      }
      if (TAIL) {
        const u32x4 y = norm_bf(hk[NI - 1], sm.gamma, ftl + 8 * g16, wsm.rh[t16]);
        bstore<kYAux>(r.y, vft, 0, y);
      }
    }
    // split + Sinkhorn of token tb of the batch
    if (sk) {
      f32x4 acc = sk_part[0];
#pragma unroll
      for (int j = 1; j < kSk; ++j) acc += sk_part[j];
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {   // sum over the 8 slice groups (lanes l ^ 8, 16, 32)
        float x = acc[e] + dpp<pipe::kRowRor8>(acc[e]);
        x += __shfl_xor(x, 16);
        v[e] = x + __shfl_xor(x, 32);
      }
      // every lane now holds floats 4(l&7) .. 4(l&7)+3 of the token's row:
      // lanes 0..5 write mixes 4l .. 4l+3; float 24 (lane 6) is sum x'^2
      const float ssum = __shfl(v[0], 6);
      const float rr = rsqrtf(ssum / (float)(kStreams * d) + a.norm_eps);
      const int64_t t = bt0 + tb;
      // the mixes row; split and Sinkhorn run in tail_kernel
      if (lane < kMix / 4) {
        st4f(&fs.mix[t * kMix + 4 * lane], f32x4{v[0] * rr, v[1] * rr, v[2] * rr, v[3] * rr});
      }
    }
  };

  Rs rcur = batch_rs(0), rprev = rcur;
  Cf cf;
  Items bufA, bufB, bufT;
  u32x4 hcur[NI], hprev[NI];
  if (nbg > 0) {
    load_coef(cf, rcur);
    load_half(bufA, rcur, 0, 0);
    load_half(bufB, rcur, 0, 1);
  }

  for (int i = 0; i < nbg; ++i) {
    store_coef(cf);
    __builtin_amdgcn_wave_barrier();
    f32x4 acc[kT];
#pragma unroll
    for (int q = 0; q < kT; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
    float ssA[2] = {0.f, 0.f}, hsA[2] = {0.f, 0.f}, ssT = 0.f, hsT = 0.f;

    // both halves of round rr are in flight on entry; each half's buffer is
    // refilled with the next round's half (or the tail) once consumed. Phases
    // are fenced so every wait stays at its consumer (vmcnt retires in order).
#pragma unroll
    for (int rr = 0; rr < NR; ++rr) {
      // Wave priority: the two waves of a SIMD alternate between streaming
      // phases (hc_post, stores, the refill loads) and the MFMA phase below.
      // Giving the streaming phase the higher priority lets the other wave's
      // loads and stores issue ahead of this wave's MFMAs: 1.514 -> 1.480 ms
      // at 65,536 tokens.
      __builtin_amdgcn_s_setprio(3);
      u32x4 xo0[4], xo1[4];
      float C[4][4], U[4], P[4];
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (kFull) get_coef(m8, C, U, P);
      if constexpr (kFull) elementwise(bufA, C, U, P, xo0, hcur[2 * rr], ssA[0], hsA[0]);
      else streams_only(bufA, xo0, ssA[0]);
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if constexpr (kFull) bstore<kXoAux>(rcur.xo, vxh[0], 128u * rr + k * d2, xo0[k]);
      __builtin_amdgcn_sched_barrier(0);
      if (rr + 1 < NR) load_half(bufA, rcur, rr + 1, 0);
      else if (TAIL) load_tail(bufT, rcur);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (kFull) get_coef(8 + m8, C, U, P);
      if constexpr (kFull) elementwise(bufB, C, U, P, xo1, hcur[2 * rr + 1], ssA[1], hsA[1]);
      else streams_only(bufB, xo1, ssA[1]);
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if constexpr (kFull) bstore<kXoAux>(rcur.xo, vxh[1], 128u * rr + k * d2, xo1[k]);
      __builtin_amdgcn_sched_barrier(0);
      if (rr + 1 < NR) load_half(bufB, rcur, rr + 1, 1);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(0);
      // new streams of the two halves -> A operands, 2 K-steps x 4 streams
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        u32x4* buf = wsm.u.e.xs[k & 1];
        buf[sidx(m8, x8)] = xo0[k];
        buf[sidx(8 + m8, x8)] = xo1[k];
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2) {
          const bf16x8 A = __builtin_bit_cast(bf16x8, buf[sidx(t16, 4 * q2 + g16)]);
          const int step = fr0 / 32 + 2 * rr + q2;
#pragma unroll
          for (int q = 0; q < kT; ++q)
            acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, wlds(step, k, q), acc[q], 0, 0, 0);
        }
        __builtin_amdgcn_wave_barrier();
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (TAIL) {
      u32x4 xot[4];
      float C[4][4], U[4], P[4];
      if constexpr (kFull) get_coef(t16, C, U, P);
      if constexpr (kFull) elementwise(bufT, C, U, P, xot, hcur[NI - 1], ssT, hsT);
      else streams_only(bufT, xot, ssT);
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if constexpr (kFull) bstore<kXoAux>(rcur.xo, vxt, k * d2, xot[k]);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const bf16x8 A = __builtin_bit_cast(bf16x8, xot[k]);
#pragma unroll
        for (int q = 0; q < kT; ++q)
          acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, wlds(ftl / 32, k, q), acc[q], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- publish the slice's per-token partials of batch i ----
    {
      // sums of squares: half rounds over the 8 lanes of a token, tail over
      // the 4 lanes of a token
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        ssA[h] = quad_sum(ssA[h]);
        ssA[h] += __shfl_xor(ssA[h], 4);
        hsA[h] = quad_sum(hsA[h]);
        hsA[h] += __shfl_xor(hsA[h], 4);
      }
      if (TAIL) {
        ssT += __shfl_xor(ssT, 16);
        ssT += __shfl_xor(ssT, 32);
        hsT += __shfl_xor(hsT, 16);
        hsT += __shfl_xor(hsT, 32);
      }
      const int u = lane >> 2;   // token this lane publishes
      const int src = 8 * (u & 7);
      const float s0 = __shfl(ssA[0], src), s1 = __shfl(ssA[1], src);
      const float h0 = __shfl(hsA[0], src), h1 = __shfl(hsA[1], src);
      float ssu = u < 8 ? s0 : s1, hsu = u < 8 ? h0 : h1;
      if (TAIL) {
        ssu += __shfl(ssT, u);
        hsu += __shfl(hsT, u);
      }
      // projection partials -> per-token rows, hi + mid + lo
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int q = 0; q < kT; ++q) {
        const int col = 16 * q + t16;
        if (col < kC) {
#pragma unroll
          for (int e = 0; e < 4; ++e) wsm.u.cst[4 * g16 + e][col] = acc[q][e];
        }
      }
      __builtin_amdgcn_wave_barrier();
      float mv[6];
#pragma unroll
      for (int jj = 0; jj < 6; ++jj) {
        const int row = 6 * (lane & 3) + jj;
        mv[jj] = wsm.u.cst[u][row] + wsm.u.cst[u][kMix + row];
        if constexpr (TERMS == 3) mv[jj] += wsm.u.cst[u][2 * kMix + row];
      }
      __builtin_amdgcn_wave_barrier();
      // assemble the 16 token rows (24 mixes, x'^2, h^2, zero pad) in LDS, then
      // write each row as 8 lanes x 16 bytes: whole 128-byte lines
      float(*rows)[kRow] = reinterpret_cast<float(*)[kRow]>(&wsm.u.cst[0][0]);
#pragma unroll
      for (int jj = 0; jj < 6; ++jj) rows[u][6 * (lane & 3) + jj] = mv[jj];
      if ((lane & 3) == 0) {
        *reinterpret_cast<f32x4*>(&rows[u][24]) = f32x4{ssu, hsu, 0.f, 0.f};
        *reinterpret_cast<f32x4*>(&rows[u][28]) = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      __builtin_amdgcn_wave_barrier();
      const int slot = i % kRing;
      const int64_t slot_id = (int64_t)g * kRing + slot;
      const uint32_t rows_off = (uint32_t)(mp_off(G) + slot_id * mp_slot_bytes(ns)) +
                                (uint32_t)((c * kBatch + wave * kTok) * kRow * 4);
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int tk = 8 * hh + (lane >> 3);
        const u32x4 v = *reinterpret_cast<const u32x4*>(&rows[tk][4 * (lane & 7)]);
        bstore<kSC1>(wsr, rows_off + (uint32_t)(tk * kRow * 4 + 16 * (lane & 7)), 0, v);
      }
      {
        // sum of h^2 of the 16 tokens: 4 lanes x 4 tokens
        const int t0 = 4 * (lane & 3);
        const u32x4 v = {__float_as_uint(rows[t0][25]), __float_as_uint(rows[t0 + 1][25]),
                         __float_as_uint(rows[t0 + 2][25]), __float_as_uint(rows[t0 + 3][25])};
        const uint32_t hoff = (uint32_t)(hs_off(G, ns) + slot_id * hs_slot_bytes(ns)) +
                              (uint32_t)((c * kBatch + wave * kTok + t0) * 4);
        if constexpr (kFull) bstore<kSC1>(wsr, lane < 4 ? hoff : kOutOfRange, 0, v);
      }
      __builtin_amdgcn_wave_barrier();
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_sched_barrier(0);

      // next batch's first round (both halves) and coefficients, empty ranges
      // past the end: they fly while batch i-1 is finished
      const Rs rnext = batch_rs(i + 1);
      load_coef(cf, rnext);
      load_half(bufA, rnext, 0, 0);
      load_half(bufB, rnext, 0, 1);
      __builtin_amdgcn_sched_barrier(0);
      {
        // wait for the exchange stores directly (13 loads were issued after
        // them) and count the batch now
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(kFull ? 13 : 8));
        __builtin_amdgcn_sched_barrier(0);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        count_batch(i);
      }
      if (i > 0) finish(i - 1, rprev, hprev);
      rprev = rcur;
      rcur = rnext;
#pragma unroll
      for (int j = 0; j < NI; ++j) hprev[j] = hcur[j];
    }
  }
  if (nbg > 0) finish(nbg - 1, rprev, hprev);
  release_workspace(ws, ctr_off(0, 0), G * kRing);
}

// Split and Sinkhorn of the mixes rows [T][24] the feature-split kernel wrote,
// one thread per token with the 4x4 in registers ([SW] Code, the
// split/Sinkhorn kernel; "All 5 steps"). The sums are associated as the
// 16-lane form's quad and column sums (DPP, in the tile and chunked kernels)
// are (row: (c0 + c1) + (c2 + c3); column: (r0 + r2) + (r1 + r3)), and the
// divisions after the softmax are multiplications by the hardware
// reciprocal, as there; a token takes half the 16-lane form's arithmetic.
constexpr int kTailThreads = 64;

__global__ __launch_bounds__(kTailThreads) void tail_kernel(const float* __restrict__ mix,
                                                           int64_t tokens,
                                                           const float* __restrict__ base,
                                                           const float* __restrict__ scale,
                                                           int iters, float eps,
                                                           float* __restrict__ pre_out,
                                                           float* __restrict__ post_out,
                                                           float* __restrict__ comb_out) {
  const int64_t t = (int64_t)blockIdx.x * kTailThreads + threadIdx.x;
  if (t >= tokens) return;
  float m[kMix];
  const f32x4* row = reinterpret_cast<const f32x4*>(mix + t * kMix);
#pragma unroll
  for (int q = 0; q < kMix / 4; ++q) {
    const f32x4 v = row[q];
#pragma unroll
    for (int e = 0; e < 4; ++e) m[4 * q + e] = v[e];
  }
  const float s0 = scale[0], s1 = scale[1], s2 = scale[2];
  f32x4 pre, post;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    pre[k] = sigmoidf(m[k] * s0 + base[k]) + eps;
    post[k] = 2.0f * sigmoidf(m[4 + k] * s1 + base[4 + k]);
  }
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
  auto columns = [&]() {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float r = __builtin_amdgcn_rcpf(((c[0][k] + c[2][k]) + (c[1][k] + c[3][k])) + eps);
#pragma unroll
      for (int j = 0; j < 4; ++j) c[j][k] = c[j][k] * r;
    }
  };
  columns();
  for (int it = 1; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float r = __builtin_amdgcn_rcpf(((c[j][0] + c[j][1]) + (c[j][2] + c[j][3])) + eps);
#pragma unroll
      for (int k = 0; k < 4; ++k) c[j][k] = c[j][k] * r;
    }
    columns();
  }
  st4f(pre_out + t * 4, pre);
  st4f(post_out + t * 4, post);
#pragma unroll
  for (int j = 0; j < 4; ++j) st4f(comb_out + t * 16 + 4 * j, f32x4{c[j][0], c[j][1], c[j][2], c[j][3]});
}

}  // namespace fsplit
