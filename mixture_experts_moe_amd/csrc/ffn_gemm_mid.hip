// Grouped GEMM for blocks of 128 tokens with e4m3fn weights: the expert
// kernels of fine-grained experts at large T (a few dozen to a few hundred
// tokens per expert).
//
// Sources: the Hungarian news page "Az AWS új MoE-optimalizációkkal
// gyorsítja a SageMaker AI-t", section "FP8 esetén a Triton backend
// bizonyult gyorsabbnak" (FP8 scaling fused with the matrix product over
// variable-size token groups, data read once from HBM), and section "A fused
// MoE a számítási folyamat több lépését egyesíti" (the experts' computation
// as one batched operation).
//
// A workgroup computes 256 weight rows x the block's 128 tokens: eight waves
// of 128 rows x 32 tokens.  Both operands move HBM/L2 -> LDS by gfx950's
// direct-to-LDS 16-byte buffer loads (no VGPR staging), in K stages of 64
// through a ring of four buffers, so that two stages are in flight while
// one is multiplied: a stage holds 256 weight rows x 64 bytes
// (64 e4m3fn values) and 128 token rows x 128 bytes (64 bf16 values), 32 KB.
// 16-byte slots are XOR-swizzled by row ((row >> 1) & 3 for the 4-slot
// weight rows, & 7 for the 8-slot token rows), so that the 16 rows one
// 16-lane group reads at the same k spread over the banks.  Weight fragments
// are read 8 bytes at a time and widened to bf16 in registers
// (v_cvt_scalef32_pk_bf16_fp8, exact); the product runs on
// v_mfma_f32_16x16x32_bf16 with fp32 accumulation.
//
// A block of a few dozen tokens is mostly padding: the waves whose 32
// token rows hold no real slot only load weights and meet the barriers, and
// token rows past the block's last real slot are not loaded.  Waves 2m and
// 2m+1 take token rows 32m .. 32m+31 and wave w runs on SIMD w % 4, so the
// live waves of a half-full block sit on four different SIMDs.
//
// W13: the tile's rows are 128 gate rows then the matching 128 up rows
// (128 channels of h); the epilogue applies the per-channel (or per-tensor)
// scales and writes h = SiLU(gate) * up for the live waves' rows.  W2: 256
// output channels; the epilogue scales by the channel scale and the slot's
// gate and writes the slot's fp32 row for the combine.  The grid is
// rasterised per XCD like the big tile's.

#include "ffn_big_common.h"

namespace moe {

constexpr int kMidTokens = 128;  // block size B of this path
constexpr int kMidRows = 256;    // weight rows per tile
constexpr int kMidK = 64;        // K per stage
constexpr int kMidWaves = 8;
constexpr int kMidThreads = 64 * kMidWaves;
constexpr int kMidTA = 8;                                // 16-row weight tiles per wave
constexpr int kMidNB = 2;                                // 16-token tiles per wave
constexpr int kMidARowBytes = kMidK;                     // e4m3fn weight row per stage
constexpr int kMidBRowBytes = 2 * kMidK;                 // bf16 token row per stage
constexpr int kMidABytes = kMidRows * kMidARowBytes;     // 16 KB
constexpr int kMidStageBytes = kMidABytes + kMidTokens * kMidBRowBytes;  // 32 KB
constexpr int kMidLoadsA = kMidABytes / 1024 / kMidWaves;                // 1 KB loads per wave
constexpr int kMidLoadsB = kMidTokens * kMidBRowBytes / 1024 / kMidWaves;
constexpr int kMidStages = 4;  // ring depth: two stages in flight while one is multiplied
static_assert(kMidStages * kMidStageBytes <= 160 * 1024, "stages fit in LDS");
static_assert(kMidLoadsA == 2 && kMidLoadsB == 2, "two weight and two token loads per wave");
static_assert((kMidStages - 2) * (kMidLoadsA + kMidLoadsB) <= 63, "wait counts fit vmcnt");

typedef f32x4 MidAcc[kMidTA][kMidNB];

// Channel groups per super-row of the XCD raster (big_tile_of): the
// workgroups an XCD runs together cover this many channel groups of
// consecutive row blocks (at ~64 tokens per expert, about one expert per
// block).  Measured at e4m3fn T = 2048 (d = 7168, I = 2048, 256 experts):
// W13 1.86 / 1.81 / 2.45 / 2.31 / 2.29 ms with 1 / 2 / 3 / 4 / 8 groups;
// W2 1.18 / 1.25 / 1.18 / 1.41 / 1.42 ms with 2 / 3 / 4 / 5 / 8 (W2 also
// moves with W13's order, which decides which h rows are still cached).
#ifndef MOE_MID13_GROUP_COLS
#define MOE_MID13_GROUP_COLS 2
#endif
#ifndef MOE_MID2_GROUP_COLS
#define MOE_MID2_GROUP_COLS 4
#endif

// Per-lane sources of one stage's loads.  Weight load i of wave w fills LDS
// rows 32w + 16i .. +15 (16 rows x 64 bytes): lane l writes row l/4,
// physical slot l%4, which holds logical slot (l%4) ^ ((row >> 1) & 3).
// Token load i fills rows 16w + 8i .. +7 (8 rows x 128 bytes): lane l
// writes row l/8, physical slot l%8 = logical (l%8) ^ ((row >> 1) & 7).
struct MidLoader {
  __amdgpu_buffer_rsrc_t ra;   // the expert's weight matrix
  __amdgpu_buffer_rsrc_t rb;   // token rows (x, or the block's h rows)
  uint32_t a[kMidLoadsA];      // byte offset of this lane's weight source, k = 0
  uint32_t b[kMidLoadsB];      // byte offset of this lane's token source, k = 0
  bool b_live;                 // this wave's 16 token rows hold a real slot
};

// Stage s into `stage`: weights at byte 64 s along K, tokens at byte 128 s.
__device__ __forceinline__ void mid_issue(const MidLoader& ld, uint8_t* stage, int s, int wave) {
#pragma unroll
  for (int i = 0; i < kMidLoadsA; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        ld.ra,
        (__attribute__((address_space(3))) void*)(stage + (wave * kMidLoadsA + i) * 1024), 16,
        ld.a[i] + static_cast<uint32_t>(s) * kMidARowBytes, 0, 0, 0);
  if (!ld.b_live) return;
#pragma unroll
  for (int i = 0; i < kMidLoadsB; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        ld.rb,
        (__attribute__((address_space(3))) void*)(stage + kMidABytes +
                                                   (wave * kMidLoadsB + i) * 1024),
        16, ld.b[i] + static_cast<uint32_t>(s) * kMidBRowBytes, 0, 0, 0);
}

// A lane's byte offsets inside a stage buffer for the two 32-K steps j of a
// stage: weight fragment of row r16 (logical slot 2j + g/2, half g&1), token
// fragment of row r16 of the token region (logical slot 4j + g).  Tiles
// start at multiples of 16 rows, so the swizzles depend on r16 only and a
// tile adds a constant.
struct MidLane {
  uint32_t a[2], b[2];
};

__device__ __forceinline__ MidLane mid_lane() {
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int swa = (r16 >> 1) & 3;
  const int swb = (r16 >> 1) & 7;
  MidLane ln;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    ln.a[j] = r16 * kMidARowBytes + (((2 * j + (g >> 1)) ^ swa) << 4) + 8 * (g & 1);
    ln.b[j] = kMidABytes + r16 * kMidBRowBytes + (((4 * j + g) ^ swb) << 4);
  }
  return ln;
}

// The two 32-K steps of one stage: acc[t][u] += W(rows of tile t) .
// X(tokens of tile u)^T.  Weight tile t: rows arow0 + 16t (t < 4) and
// arow_up + 16(t - 4); token tile u: rows brow0 + 16u.
__device__ __forceinline__ void mid_stage(const uint8_t* cur, const MidLane& lane_off, int arow0,
                                          int arow_up, int brow0, MidAcc& acc) {
  // Opaque copies of the lane offsets: otherwise the compiler forms every
  // fragment address of every buffer outside the stage loop, keeps them in
  // registers and spills; this way each stage forms its bases and a tile's
  // offset is a read's immediate.
  uint32_t a0 = lane_off.a[0], a1 = lane_off.a[1], b0 = lane_off.b[0], b1 = lane_off.b[1];
  asm volatile("" : "+v"(a0), "+v"(a1), "+v"(b0), "+v"(b1));
  const uint32_t la[2] = {a0, a1}, lb[2] = {b0, b1};
#pragma unroll
  for (int j = 0; j < kMidK / 32; ++j) {
    bf16x8 b[kMidNB];
#pragma unroll
    for (int u = 0; u < kMidNB; ++u)
      b[u] = as_frag(*reinterpret_cast<const uint4*>(cur + lb[j] + (brow0 + 16 * u) * kMidBRowBytes));
#pragma unroll
    for (int t = 0; t < kMidTA; ++t) {
      const int row = t < 4 ? arow0 + 16 * t : arow_up + 16 * (t - 4);
      const uint2 q = *reinterpret_cast<const uint2*>(cur + la[j] + row * kMidARowBytes);
      const bf16x8 a = as_frag(e4m3x8_to_frag_bits(q.x, q.y));
#pragma unroll
      for (int u = 0; u < kMidNB; ++u) acc[t][u] = mfma16x16x32(a, b[u], acc[t][u]);
    }
  }
}

// The ring's buffers are separate LDS arrays: with one array the compiler
// cannot tell that reads of one stage do not depend on the loads into
// another, and waits for every load before every read.
#define MID_RING(name)                                                       \
  __shared__ __attribute__((aligned(1024))) uint8_t name##0[kMidStageBytes]; \
  __shared__ __attribute__((aligned(1024))) uint8_t name##1[kMidStageBytes]; \
  __shared__ __attribute__((aligned(1024))) uint8_t name##2[kMidStageBytes]; \
  __shared__ __attribute__((aligned(1024))) uint8_t name##3[kMidStageBytes]; \
  uint8_t* const name[kMidStages] = {name##0, name##1, name##2, name##3}

// The ring: stage s in buffer s % 4.  Stages 0 .. 2 are issued up front.
// At stage s a wave waits until its loads of s have landed (loads complete
// in issue order: only its loads of the later stages already issued may
// stay outstanding, kL per stage), meets the other waves (after which all
// of stage s is in LDS and nobody reads buffer (s - 1) % 4 any more),
// issues stage s + 3 into that buffer while there is one, and runs stage
// s's MFMAs.  The stage count is a multiple of 4 (d and I multiples of
// 256), so the loop goes four stages at a time with the same waits and the
// last four run as one fixed sequence: every wait count and buffer index is
// a compile-time constant, and the accumulators flow through one path.
// kL: loads per stage of this wave (weights, plus tokens when b_live);
// kLive: the wave's token rows hold a real slot (else it only loads and
// meets the barriers).  Both are chosen once, outside the loop, so that the
// loop body has no branch around the MFMAs (a branch there makes the
// compiler keep copies of the accumulators at the join and spill).
template <int kL, bool kLive>
struct MidRing {
  const MidLoader& ld;
  uint8_t* const (&buf)[kMidStages];
  const MidLane& lane_off;
  int wave, arow0, arow_up, brow0;

  // stage s in buffer p with W later stages issued; issues stage s + 3
  // into buffer (p + 3) % 4 when kIssue
  template <int p, int W, bool kIssue>
  __device__ __forceinline__ void step(int s, MidAcc& acc) const {
    static_assert(kL * W <= 63, "wait count exceeds the 6-bit vmcnt field");
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(kL * W));
    big_barrier();
    if constexpr (kIssue) mid_issue(ld, buf[(p + 3) % 4], s + 3, wave);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kLive) mid_stage(buf[p], lane_off, arow0, arow_up, brow0, acc);
    // keep each stage's fragment reads and MFMAs inside its step: moved
    // across steps they hold several stages' fragments in registers
    __builtin_amdgcn_sched_barrier(0);
  }

  __device__ __forceinline__ void run(int nst, MidAcc& acc) const {
    mid_issue(ld, buf[0], 0, wave);
    mid_issue(ld, buf[1], 1, wave);
    mid_issue(ld, buf[2], 2, wave);
    int s = 0;
    for (; s + 4 < nst; s += 4) {  // stages that each issue the one three ahead
      step<0, 2, true>(s, acc);
      step<1, 2, true>(s + 1, acc);
      step<2, 2, true>(s + 2, acc);
      step<3, 2, true>(s + 3, acc);
    }
    // the last four: the first issues the last stage, then 2, 1, 0 issued after
    step<0, 2, true>(s, acc);
    step<1, 2, false>(s + 1, acc);
    step<2, 1, false>(s + 2, acc);
    step<3, 0, false>(s + 3, acc);
  }
};

__device__ __forceinline__ void mid_run(const MidLoader& ld, uint8_t* const (&buf)[kMidStages], int nst,
                                        int wave, int arow0, int arow_up, int brow0, bool live,
                                        MidAcc& acc) {
  const MidLane lane_off = mid_lane();
  constexpr int kLB = kMidLoadsA + kMidLoadsB;
  if (ld.b_live) {
    if (live)
      MidRing<kLB, true>{ld, buf, lane_off, wave, arow0, arow_up, brow0}.run(nst, acc);
    else
      MidRing<kLB, false>{ld, buf, lane_off, wave, arow0, arow_up, brow0}.run(nst, acc);
  } else {
    if (live)
      MidRing<kMidLoadsA, true>{ld, buf, lane_off, wave, arow0, arow_up, brow0}.run(nst, acc);
    else
      MidRing<kMidLoadsA, false>{ld, buf, lane_off, wave, arow0, arow_up, brow0}.run(nst, acc);
  }
}

// Weight load i's LDS row (of the tile) and the logical slot this lane
// loads; the same for the token loads.
__device__ __forceinline__ int mid_a_row(int wave, int i, int lane) {
  return 32 * wave + 16 * i + lane / 4;
}
__device__ __forceinline__ int mid_a_slot(int lane) {
  return (lane % 4) ^ (((lane / 4) >> 1) & 3);  // (row >> 1) & 3: 32w + 16i adds a multiple of 4
}
__device__ __forceinline__ int mid_b_row(int wave, int i, int lane) {
  return 16 * wave + 8 * i + lane / 8;
}
__device__ __forceinline__ int mid_b_slot(int i, int lane) {
  return (lane % 8) ^ (((8 * i + lane / 8) >> 1) & 7);  // the row's swizzle, (row >> 1) & 7
}

// ------------------------------------------------------------ W13 + SiLU*mul
// Tile (b, y): channels n0 = 128y .. +127 (rows: 128 gate, then 128 up) x
// the 128 tokens of row block b.

__global__ __launch_bounds__(kMidThreads) void ffn13_mid_kernel(
    const bf16_t* __restrict__ x, const fp8_t* __restrict__ w13, const float* __restrict__ s13,
    int scale_mode, const int32_t* __restrict__ sorted_ids,
    const int32_t* __restrict__ block_expert, const int32_t* __restrict__ num_padded,
    bf16_t* __restrict__ h, int d, int I, int k, int A, int T, int gx, int gy) {
  MID_RING(buf);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const BigTile tl = big_tile_live<MOE_MID13_GROUP_COLS>(blockIdx.x, gx, gy, num_padded, kMidTokens);
  if (!tl.live) return;  // uniform
  const int b = tl.b;
  const int32_t* blk = sorted_ids + static_cast<size_t>(b) * kMidTokens;
  if (blk[0] >= A) return;  // real slots come first: this block holds none
  const int e = block_expert[b];
  const int n0 = tl.y * 128;
  const size_t two_i = 2 * static_cast<size_t>(I);

  MidLoader ld;
  ld.ra = big_rsrc(w13 + static_cast<size_t>(e) * two_i * d, two_i * d);
  ld.rb = big_rsrc(x, static_cast<size_t>(T) * d * 2);
#pragma unroll
  for (int i = 0; i < kMidLoadsA; ++i) {
    const int r = mid_a_row(wave, i, lane);  // tile rows 0..127 gate, 128..255 up
    const uint32_t wrow = r < 128 ? n0 + r : I + n0 + r - 128;
    ld.a[i] = wrow * static_cast<uint32_t>(d) + 16 * mid_a_slot(lane);
  }
#pragma unroll
  for (int i = 0; i < kMidLoadsB; ++i) {
    const int f = blk[mid_b_row(wave, i, lane)];  // pad slot: any valid row (never stored)
    ld.b[i] = 2 * static_cast<uint32_t>(f < A ? f / k : 0) * d + 16 * mid_b_slot(i, lane);
  }
  ld.b_live = __builtin_amdgcn_readfirstlane(blk[16 * wave]) < A;
  const int wm = wave & 1, wn = wave >> 1;
  MidAcc acc;
#pragma unroll
  for (int t = 0; t < kMidTA; ++t)
#pragma unroll
    for (int u = 0; u < kMidNB; ++u) acc[t][u] = f32x4{0.f, 0.f, 0.f, 0.f};

  const bool live = __builtin_amdgcn_readfirstlane(blk[32 * wn]) < A;
  mid_run(ld, buf, d / kMidK, wave, 64 * wm, 128 + 64 * wm, 32 * wn, live, acc);
  if (!live) return;

  // lane: token column r16 of tile u, channels n0 + 64wm + 16t + 4g .. +3
  const int r16 = lane & 15;
  const int g = lane >> 4;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int c = n0 + 64 * wm + 16 * t + 4 * g;
    float sg[4], su[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      sg[v] = load_scale(s13, scale_mode, e, static_cast<size_t>(e) * two_i + c + v);
      su[v] = load_scale(s13, scale_mode, e, static_cast<size_t>(e) * two_i + I + c + v);
    }
#pragma unroll
    for (int u = 0; u < kMidNB; ++u) {
      const size_t row = static_cast<size_t>(b) * kMidTokens + 32 * wn + 16 * u + r16;
      uint32_t packed[2];
#pragma unroll
      for (int v = 0; v < 4; v += 2) {
        const float h0 = silu(acc[t][u][v] * sg[v]) * (acc[t + 4][u][v] * su[v]);
        const float h1 = silu(acc[t][u][v + 1] * sg[v + 1]) * (acc[t + 4][u][v + 1] * su[v + 1]);
        packed[v / 2] = static_cast<uint32_t>(f32_to_bf16(h0)) |
                        (static_cast<uint32_t>(f32_to_bf16(h1)) << 16);
      }
      *reinterpret_cast<uint2*>(h + row * I + c) = uint2{packed[0], packed[1]};
    }
  }
}

// ------------------------------------------------------------ W2 + gate scale
// Tile (b, y): output channels n0 = 256y .. +255 x the block's 128 h rows.
// Writes y[f, n] = gate_f * s(n) * (W2[e] h[row])[n] for the block's slots.

__global__ __launch_bounds__(kMidThreads) void ffn2_mid_kernel(
    const bf16_t* __restrict__ h, const fp8_t* __restrict__ w2, const float* __restrict__ s2,
    int scale_mode, const float* __restrict__ topk_w, const int32_t* __restrict__ sorted_ids,
    const int32_t* __restrict__ block_expert, const int32_t* __restrict__ num_padded,
    float* __restrict__ y, int d, int I, int A, int gx, int gy) {
  MID_RING(buf);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const BigTile tl = big_tile_live<MOE_MID2_GROUP_COLS>(blockIdx.x, gx, gy, num_padded, kMidTokens);
  if (!tl.live) return;
  const int b = tl.b;
  const int32_t* blk = sorted_ids + static_cast<size_t>(b) * kMidTokens;
  if (blk[0] >= A) return;
  const int e = block_expert[b];
  const int n0 = tl.y * kMidRows;

  MidLoader ld;
  ld.ra = big_rsrc(w2 + static_cast<size_t>(e) * d * I, static_cast<size_t>(d) * I);
  // h rows of the block; pad rows hold no token and their columns are never stored
  ld.rb = big_rsrc(h + static_cast<size_t>(b) * kMidTokens * I,
                   static_cast<size_t>(kMidTokens) * I * 2);
#pragma unroll
  for (int i = 0; i < kMidLoadsA; ++i)
    ld.a[i] = static_cast<uint32_t>(n0 + mid_a_row(wave, i, lane)) * I + 16 * mid_a_slot(lane);
#pragma unroll
  for (int i = 0; i < kMidLoadsB; ++i)
    ld.b[i] = 2 * static_cast<uint32_t>(mid_b_row(wave, i, lane)) * I + 16 * mid_b_slot(i, lane);
  ld.b_live = __builtin_amdgcn_readfirstlane(blk[16 * wave]) < A;
  const int wm = wave & 1, wn = wave >> 1;
  MidAcc acc;
#pragma unroll
  for (int t = 0; t < kMidTA; ++t)
#pragma unroll
    for (int u = 0; u < kMidNB; ++u) acc[t][u] = f32x4{0.f, 0.f, 0.f, 0.f};

  // weight rows 128wm .. +127: eight consecutive 16-row tiles
  const bool live = __builtin_amdgcn_readfirstlane(blk[32 * wn]) < A;
  mid_run(ld, buf, I / kMidK, wave, 128 * wm, 128 * wm + 64, 32 * wn, live, acc);
  if (!live) return;

  // lane: token column r16 of tile u, channels n0 + 128wm + 16t + 4g .. +3
  const int r16 = lane & 15;
  const int g = lane >> 4;
#pragma unroll
  for (int u = 0; u < kMidNB; ++u) {
    const int f = blk[32 * wn + 16 * u + r16];
    if (f < A) {
      const float gate = topk_w[f];
      float* yrow = y + static_cast<size_t>(f) * d;
#pragma unroll
      for (int t = 0; t < kMidTA; ++t) {
        const int c = n0 + 128 * wm + 16 * t + 4 * g;
        const size_t base = static_cast<size_t>(e) * d + c;
        *reinterpret_cast<float4*>(yrow + c) =
            float4{acc[t][u][0] * load_scale(s2, scale_mode, e, base) * gate,
                   acc[t][u][1] * load_scale(s2, scale_mode, e, base + 1) * gate,
                   acc[t][u][2] * load_scale(s2, scale_mode, e, base + 2) * gate,
                   acc[t][u][3] * load_scale(s2, scale_mode, e, base + 3) * gate};
      }
    }
  }
}

// ------------------------------------------------------------ launchers

// e4m3fn weights, bf16 activations, blocks of 128: W13 tiles of 128
// channels and W2 tiles of 256 output channels, K stages of 64 run four at
// a time (d and I multiples of 256); the loads
// address an expert's matrices, x and a block's h rows with 32-bit byte
// offsets.
bool mid_gemm_fits(int64_t T, int d, int I) {
#ifdef MOE_NO_MID_GEMM
  return false;
#else
  const int64_t lim = int64_t(1) << 31;
  return d % 256 == 0 && I % 256 == 0 && int64_t(2) * I * d < lim && T * d * 2 < lim &&
         int64_t(kMidTokens) * I * 2 < lim;
#endif
}

static bool mid_args_ok(const FfnArgs& a) {
  return a.B == kMidTokens && a.w_dtype == kDtypeE4M3FN && a.act_dtype == kDtypeBF16 &&
         !a.act_mx && mid_gemm_fits(a.T, a.d, a.I);
}

static int mid_grid(int gx, int gy) {
  const int total = gx * gy;
  return (total + kBigXcds - 1) / kBigXcds * kBigXcds;
}

hipError_t launch_ffn13_mid(const FfnArgs& a, hipStream_t s) {
  if (!mid_args_ok(a)) return hipErrorInvalidValue;
  const int gx = a.cap / kMidTokens, gy = a.I / 128;
  ffn13_mid_kernel<<<mid_grid(gx, gy), kMidThreads, 0, s>>>(
      static_cast<const bf16_t*>(a.x), static_cast<const fp8_t*>(a.w13), a.s13, a.scale_mode,
      a.sorted_ids, a.block_expert, a.num_padded, static_cast<bf16_t*>(a.h), a.d, a.I, a.k, a.A,
      a.T, gx, gy);
  return hipGetLastError();
}

hipError_t launch_ffn2_mid(const FfnArgs& a, hipStream_t s) {
  if (!mid_args_ok(a) || a.splits != 1) return hipErrorInvalidValue;
  const int gx = a.cap / kMidTokens, gy = a.d / kMidRows;
  ffn2_mid_kernel<<<mid_grid(gx, gy), kMidThreads, 0, s>>>(
      static_cast<const bf16_t*>(a.h), static_cast<const fp8_t*>(a.w2), a.s2, a.scale_mode,
      a.topk_w, a.sorted_ids, a.block_expert, a.num_padded, a.y_part, a.d, a.I, a.A, gx, gy);
  return hipGetLastError();
}

}  // namespace moe
