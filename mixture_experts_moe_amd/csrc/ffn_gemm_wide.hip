// Grouped GEMM for blocks of 128 tokens, bf16 or e4m3fn weights: the
// expert kernels of experts holding a few dozen to a hundred-odd tokens at
// large T, where every weight byte must be read once from HBM at close to
// the streaming rate.
//
// Sources: the Hungarian news page "Az AWS új MoE-optimalizációkkal
// gyorsítja a SageMaker AI-t", section "FP8 esetén a Triton backend
// bizonyult gyorsabbnak" (FP8 scaling fused with the matrix product over
// token groups of varying size, each weight read once from HBM), and section
// "A fused MoE a számítási folyamat több lépését egyesíti" (the experts'
// computation as one batched operation).
//
// A workgroup computes 256 weight rows x the block's 128 tokens with eight
// waves.  The weights go through LDS: direct-to-LDS 16-byte buffer loads,
// eight rows x 128 contiguous bytes per instruction (128 bytes of every row
// per stage: 64 bf16 or 128 e4m3fn values of K), through a ring of 32 KB
// stages.  Where the token rows go depends on the weights and the block:
//   - register path (bf16 weights; e4m3fn only with MOE_WID_FULL off): each
//     wave loads its own token rows of the stage's K straight into MFMA
//     fragment registers, in the same load stream (loads complete in issue
//     order, so one wait per stage covers both operands);
//   - half-full blocks (at most 64 real tokens): 64 token rows per stage
//     through LDS beside the weights, each row loaded once per workgroup;
//   - full blocks with e4m3fn weights: all 128 token rows through LDS in a
//     ring of their own (see the full-block section).
// The per-CU vector memory path (address and data units, the L1's pending
// requests) is what these kernels run into before HBM does, so the token
// bytes that path carries per weight byte are what the variants trade: the
// register path loads each e4m3fn token fragment twice (once per row
// group) as 64-byte half lines, the LDS paths once as whole rows.  The
// weight loads carry the nontemporal hint when the block is its expert's
// only one (its weights are read once); an expert with several blocks reads
// them plainly, so that its other blocks' workgroups, which run at about
// the same time, find them in L2.
//
// Weight LDS rows are 128 bytes in eight 16-byte slots, XOR-swizzled by
// (row >> 1) & 7 so that the 16 rows one 16-lane group reads at the same k
// spread over the banks.  e4m3fn fragments are read 8 bytes at a time and
// widened to bf16 in registers (exact); the product runs on
// v_mfma_f32_16x16x32_bf16 with fp32 accumulation.  Rows past the weight
// matrix (a channel tile overhanging I, or d for W2) and token rows of
// padding slots are loaded from an offset past the end of their buffer
// resource, which reads zeros without touching memory; their outputs are
// never stored.  A wave whose 32 token rows hold no real slot only loads
// weights and meets the barriers.
//
// W13: the tile's rows are 128 gate rows then the matching 128 up rows (128
// channels of h), each wave holding gate and up of the same 64 channels; the
// epilogue applies the e4m3fn scales and writes h = SiLU(gate) * up.  W2: 256
// output channels; the epilogue scales by the channel scale and the slot's
// gate and writes the slot's fp32 row.  The grid is rasterised per XCD like
// the other tiles.

#include "ffn_big_common.h"

namespace moe {

constexpr int kWidTokens = 128;  // block size B of this path
constexpr int kWidRowBytes = 128;  // weight bytes per row and stage
constexpr int kWidLoadsA = 4;      // 1 KB weight loads per wave and stage (32 rows)

// Waves per workgroup for e4m3fn weights: 8 (256 rows, two row groups), or
// 4 (128 rows, one row group, two workgroups per CU; measured slower at fp8
// T = 2048: W13 1.96 against 1.77 ms).
#ifndef MOE_WID8_WAVES
#define MOE_WID8_WAVES 8
#endif

// Wave layout and ring depth.  bf16 weights: each wave takes all 256 rows
// for 16 tokens (RG = 1 row group), so every token row is loaded once per
// workgroup.  e4m3fn weights: two row groups of 128 rows, 32 tokens per
// wave (RG = 2): each weight fragment is widened to bf16 by half as many
// waves, which there costs more than loading each token row twice.  The
// token fragments of a stage take kNB * kSteps registers of 16 bytes per
// lane, and the ring depth is what the 256 registers of a wave allow: three
// stages for e4m3fn (eight fragments a stage), four for bf16 (two).
template <typename WT>
struct WidGeom {
  static constexpr int kK = kWidRowBytes / static_cast<int>(sizeof(WT));  // K per stage
  static constexpr int kSteps = kK / 32;                    // MFMA k-steps per stage
  static constexpr int kWaves = sizeof(WT) == 1 ? MOE_WID8_WAVES : 8;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kRows = 32 * kWaves;                 // weight rows per tile
  static constexpr int kStageBytes = kRows * kWidRowBytes;
  static constexpr int kRG = kWaves == 8 && sizeof(WT) == 1 ? 2 : 1;  // row groups
  static constexpr int kTA = kRows / 16 / kRG;              // 16-row weight tiles per wave
  static constexpr int kNB = 8 * kRG / kWaves;              // 16-token tiles per wave
  static constexpr int kWaveTok = 16 * kNB;                 // tokens per wave
  static constexpr int kLoadsT = kNB * kSteps;              // token loads per wave and stage
  static constexpr int kD = kLoadsT <= 4 ? 4 : 3;           // ring depth
  static_assert(kNB * 16 * kWaves / kRG == kWidTokens, "the waves cover the block");
  static_assert(kD * kStageBytes <= 160 * 1024, "the ring fits in LDS");
};

template <typename WT>
using WidAcc = f32x4[WidGeom<WT>::kTA][WidGeom<WT>::kNB];

// Channel groups per super-row of the XCD raster (big_tile_live), W13 and
// W2, by weight type.  Measured at e4m3fn T = 2048 (raster over the
// realised blocks, LDS token paths): W13 1.61 / 1.59 / 1.60 / 1.63 ms with
// 2 / 4 / 8 / 16 groups, W2 0.99 / 0.96 / 0.97 / 0.97 ms with 2 / 4 / 8 /
// 14; bf16 (skew) W13 224 -> 218 us and W2 151 -> 147 us with 1 and 2
// groups instead of 2 and 4.
#ifndef MOE_WID13_GROUP_COLS_FP8
#define MOE_WID13_GROUP_COLS_FP8 4
#endif
#ifndef MOE_WID2_GROUP_COLS_FP8
#define MOE_WID2_GROUP_COLS_FP8 4
#endif
#ifndef MOE_WID13_GROUP_COLS_BF16
#define MOE_WID13_GROUP_COLS_BF16 1
#endif
#ifndef MOE_WID2_GROUP_COLS_BF16
#define MOE_WID2_GROUP_COLS_BF16 2
#endif
template <typename WT>
constexpr int wid13_cols() { return sizeof(WT) == 1 ? MOE_WID13_GROUP_COLS_FP8 : MOE_WID13_GROUP_COLS_BF16; }
template <typename WT>
constexpr int wid2_cols() { return sizeof(WT) == 1 ? MOE_WID2_GROUP_COLS_FP8 : MOE_WID2_GROUP_COLS_BF16; }

__device__ __forceinline__ int wid_swz(int row) { return (row >> 1) & 7; }

// Weight load i of wave w fills tile rows 8q .. 8q+7 (q = 4w + i): lane l
// writes row 8q + l/8, physical slot l%8, which holds logical slot
// (l%8) ^ swz(row).
__device__ __forceinline__ int wid_a_row(int wave, int i, int lane) {
  return 8 * (kWidLoadsA * wave + i) + lane / 8;
}
__device__ __forceinline__ int wid_a_slot(int row, int lane) { return (lane % 8) ^ wid_swz(row); }

// One 1 KB direct-to-LDS weight load (16 bytes per lane from byte `off` of
// `r` into `lds` + 16 * lane), nontemporal or plain; one 16-byte token
// fragment into registers.  (Plain functions: the builtins are only visible
// to the device pass, and the templates below call these.)
__device__ __forceinline__ void wid_load_w_nt(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, off,
                                           0, 0, 2);
}
__device__ __forceinline__ void wid_load_w(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, off,
                                           0, 0, 0);
}
__device__ __forceinline__ uint4 wid_load_t(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return uint4{v[0], v[1], v[2], v[3]};
}

// Per-lane sources (byte offsets at K = 0 of the tile's range; an offset at
// or past the resource's size reads zeros).  Token tile u, k-step j of stage
// s: lane (r16, g) loads k = 32j + 8g .. +7 of its token row, the MFMA B
// fragment layout.
struct WidLoader {
  __amdgpu_buffer_rsrc_t ra;  // the expert's weight matrix
  __amdgpu_buffer_rsrc_t rb;  // token rows (x, or the block's h rows)
  uint32_t a[kWidLoadsA];
  uint32_t b[2];              // this lane's token row of tile u, k = 8g
};

template <typename WT>
using WidTok = uint4[WidGeom<WT>::kNB][WidGeom<WT>::kSteps];

// Stage s: weights into `stage`, this wave's token fragments into `tok`
// (when kLive).
template <typename WT, bool kNT, bool kLive>
__device__ __forceinline__ void wid_issue(const WidLoader& ld, uint8_t* stage, WidTok<WT>& tok,
                                          int s, int wave) {
  using G = WidGeom<WT>;
#pragma unroll
  for (int i = 0; i < kWidLoadsA; ++i) {
    uint8_t* dst = stage + (wave * kWidLoadsA + i) * 1024;
    const uint32_t off = ld.a[i] + static_cast<uint32_t>(s) * kWidRowBytes;
    if constexpr (kNT)
      wid_load_w_nt(ld.ra, dst, off);
    else
      wid_load_w(ld.ra, dst, off);
  }
  if constexpr (kLive) {
#pragma unroll
    for (int u = 0; u < G::kNB; ++u)
#pragma unroll
      for (int j = 0; j < G::kSteps; ++j)
        tok[u][j] = wid_load_t(ld.rb, ld.b[u] + static_cast<uint32_t>(s) * (2 * G::kK) + 64 * j);
  }
}

// Part j (of kSteps) of stage s's loads: weight loads j * 4 / kSteps ..
// (j + 1) * 4 / kSteps - 1 and the token fragments of k-step j.  A live wave
// issues the next stage's loads a part at a time between the k-steps of the
// current one, so that they reach the texture units spread over the stage
// rather than as one burst at the barrier (a wave that issues them all at
// once stalls behind them before its first MFMA).
template <typename WT, bool kNT>
__device__ __forceinline__ void wid_issue_part(const WidLoader& ld, uint8_t* stage,
                                               WidTok<WT>& tok, int s, int wave, int j) {
  using G = WidGeom<WT>;
  constexpr int kPer = kWidLoadsA / G::kSteps;
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int i = j * kPer + q;
    uint8_t* dst = stage + (wave * kWidLoadsA + i) * 1024;
    const uint32_t off = ld.a[i] + static_cast<uint32_t>(s) * kWidRowBytes;
    if constexpr (kNT)
      wid_load_w_nt(ld.ra, dst, off);
    else
      wid_load_w(ld.ra, dst, off);
  }
#pragma unroll
  for (int u = 0; u < G::kNB; ++u)
    tok[u][j] = wid_load_t(ld.rb, ld.b[u] + static_cast<uint32_t>(s) * (2 * G::kK) + 64 * j);
}

// A lane's byte offset inside a weight stage for k-step j: row r16,
// e4m3fn: logical slot 2j + g/2, half g&1; bf16: slot 4j + g.  Tiles start
// at multiples of 16 rows, so the swizzle depends on r16 only.
template <typename WT>
__device__ __forceinline__ uint32_t wid_a_off(int j) {
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  if constexpr (sizeof(WT) == 1)
    return r16 * kWidRowBytes + (((2 * j + (g >> 1)) ^ wid_swz(r16)) << 4) + 8 * (g & 1);
  else
    return r16 * kWidRowBytes + (((4 * j + g) ^ wid_swz(r16)) << 4);
}

// k-step j of a stage: acc[t][u] += W(rows of tile t) . X(tokens of tile
// u)^T.  Weight tile t: rows arow0 + 16t (t < kTA/2) and arow1 + 16(t -
// kTA/2).
template <typename WT>
__device__ __forceinline__ void wid_kstep(const uint8_t* cur, const WidTok<WT>& tok, int j,
                                          int arow0, int arow1, WidAcc<WT>& acc) {
  using G = WidGeom<WT>;
  // opaque copy: the k-step forms its base, a tile's offset is an immediate
  uint32_t la = wid_a_off<WT>(j);
  asm volatile("" : "+v"(la));
#pragma unroll
  for (int t = 0; t < G::kTA; ++t) {
    const int row = t < G::kTA / 2 ? arow0 + 16 * t : arow1 + 16 * (t - G::kTA / 2);
    bf16x8 a;
    if constexpr (sizeof(WT) == 1) {
      const uint2 q = *reinterpret_cast<const uint2*>(cur + la + row * kWidRowBytes);
      a = as_frag(e4m3x8_to_frag_bits(q.x, q.y));
    } else {
      a = as_frag(*reinterpret_cast<const uint4*>(cur + la + row * kWidRowBytes));
    }
#pragma unroll
    for (int u = 0; u < G::kNB; ++u) acc[t][u] = mfma16x16x32(a, as_frag(tok[u][j]), acc[t][u]);
  }
}

#define WID_RING3(name, bytes)                                      \
  __shared__ __attribute__((aligned(1024))) uint8_t name##0[bytes]; \
  __shared__ __attribute__((aligned(1024))) uint8_t name##1[bytes]; \
  __shared__ __attribute__((aligned(1024))) uint8_t name##2[bytes]; \
  uint8_t* const name[4] = {name##0, name##1, name##2, name##2}
#define WID_RING4(name, bytes)                                      \
  __shared__ __attribute__((aligned(1024))) uint8_t name##0[bytes]; \
  __shared__ __attribute__((aligned(1024))) uint8_t name##1[bytes]; \
  __shared__ __attribute__((aligned(1024))) uint8_t name##2[bytes]; \
  __shared__ __attribute__((aligned(1024))) uint8_t name##3[bytes]; \
  uint8_t* const name[4] = {name##0, name##1, name##2, name##3}

// The ring of depth D: stage s in LDS buffer and register set s % D; stages
// 0 .. D-2 are issued up front.  At stage s a wave waits until its loads of
// s have landed (only its loads of the D-2 stages after s may stay
// outstanding, kL per stage), meets the other waves (after which all of
// stage s's weights are in LDS and nobody reads buffer (s - 1) % D any
// more), issues stage s + D - 1 into that buffer and register set while
// there is one, and runs stage s's MFMAs.  The loop goes D stages at a time;
// the last D-1 .. 2D-2 stages run as a fixed sequence chosen by the stage
// count mod D once, before the loop, so every wait count, buffer and
// register index is a compile-time constant (the LDS buffers are separate
// arrays, so the compiler sees that reads of one stage do not depend on the
// loads into another).  kLive: the wave's 32 token rows hold a real slot
// (else it only loads weights and meets the barriers); kNT: weight loads
// with the nontemporal hint.
template <typename WT, bool kNT, bool kLive>
struct WidRing {
  using G = WidGeom<WT>;
  static constexpr int D = G::kD;
  static constexpr int kL = kWidLoadsA + (kLive ? G::kLoadsT : 0);
  static_assert(kL * (D - 2) <= 63, "wait counts fit the 6-bit vmcnt field");
  const WidLoader& ld;
  uint8_t* const (&buf)[4];
  int wave, arow0, arow1;

  // stage s in buffer / register set p with W later stages issued; issues
  // stage s + D - 1 into set (p + D - 1) % D when kIssue
  template <int p, int W, bool kIssue>
  __device__ __forceinline__ void step(int s, WidTok<WT> (&tok)[G::kD], WidAcc<WT>& acc) const {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(kL * W));
    big_barrier();
    constexpr int n = (p + D - 1) % D;
    if constexpr (kLive) {
      // the next stage's loads a part at a time, each before one k-step
#pragma unroll
      for (int j = 0; j < G::kSteps; ++j) {
        if constexpr (kIssue) wid_issue_part<WT, kNT>(ld, buf[n], tok[n], s + D - 1, wave, j);
        wid_kstep<WT>(buf[p], tok[p], j, arow0, arow1, acc);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else if constexpr (kIssue) {
      wid_issue<WT, kNT, false>(ld, buf[n], tok[n], s + D - 1, wave);
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // the last N stages from s (s a multiple of D): stage s + i waits with
  // min(D - 2, N - 1 - i) later stages issued and issues while
  // i < N - (D - 1)
  template <int I, int N>
  __device__ __forceinline__ void tail(int s, WidTok<WT> (&tok)[G::kD], WidAcc<WT>& acc) const {
    if constexpr (I < N) {
      constexpr int W = (N - 1 - I) < (D - 2) ? (N - 1 - I) : (D - 2);
      step<I % D, W, (I < N - (D - 1))>(s + I, tok, acc);
      tail<I + 1, N>(s, tok, acc);
    }
  }

  // R = nst % D; nst >= D
  template <int R>
  __device__ __forceinline__ void run_r(int nst, WidAcc<WT>& acc) const {
    WidTok<WT> tok[G::kD];
#pragma unroll
    for (int i = 0; i < D - 1; ++i) wid_issue<WT, kNT, kLive>(ld, buf[i], tok[i], i, wave);
    int s = 0;
    for (; s + 2 * D - 1 <= nst; s += D) {  // D stages that each issue the one D-1 ahead
      step<0, D - 2, true>(s, tok, acc);
      step<1, D - 2, true>(s + 1, tok, acc);
      step<2, D - 2, true>(s + 2, tok, acc);
      if constexpr (D == 4) step<3, D - 2, true>(s + 3, tok, acc);
    }
    tail<0, (R == D - 1 ? D - 1 : R + D)>(s, tok, acc);
  }

  __device__ __forceinline__ void run(int nst, WidAcc<WT>& acc) const {
    const int r = nst % D;
    if (r == 0) run_r<0>(nst, acc);
    else if (r == 1) run_r<1>(nst, acc);
    else if (r == 2) run_r<2>(nst, acc);
    else if constexpr (D == 4) run_r<3>(nst, acc);
  }
};

template <typename WT>
__device__ __forceinline__ void wid_run(const WidLoader& ld, uint8_t* const (&buf)[4], int nst,
                                        int wave, int arow0, int arow1, bool nt, bool live,
                                        WidAcc<WT>& acc) {
  if (nt) {
    if (live)
      WidRing<WT, true, true>{ld, buf, wave, arow0, arow1}.run(nst, acc);
    else
      WidRing<WT, true, false>{ld, buf, wave, arow0, arow1}.run(nst, acc);
  } else {
    if (live)
      WidRing<WT, false, true>{ld, buf, wave, arow0, arow1}.run(nst, acc);
    else
      WidRing<WT, false, false>{ld, buf, wave, arow0, arow1}.run(nst, acc);
  }
}

// The block is its expert's only one (the neighbours, if any, belong to
// other experts): its weights are read once.
__device__ __forceinline__ bool wid_single_block(const int32_t* block_expert, int b, int nblocks,
                                                 int e) {
  const bool before = b > 0 && block_expert[b - 1] == e;
  const bool after = b + 1 < nblocks && block_expert[b + 1] == e;
  return !before && !after;
}

// ------------------------------------------------------------ half-full blocks
// A block whose real tokens all fit in its first 64 rows (e4m3fn weights;
// at fp8 T = 2048 about half the blocks) takes its token rows through LDS
// instead: each token row is loaded once per workgroup, as whole 256-byte
// rows per stage (four rows per 1 KB direct-to-LDS load), where the
// register path loads every token fragment twice (once per row group) as
// 64-byte half lines.  A stage holds the 32 KB of weights and 64 token rows
// (16 KB), three stages in flight-ring as above; eight waves of 64 weight
// rows x 32 tokens (wave w: rows 64 (w % 4), tokens 32 (w / 4)).  Measured
// on the tile alone (all blocks at most 64 tokens, fp8 shapes at T = 1024):
// W13 1.25 against 1.40 ms on the register path.
#ifndef MOE_WID_HALF
#define MOE_WID_HALF 1
#endif
#ifndef MOE_WID_HALF_BF16
#define MOE_WID_HALF_BF16 1
#endif
constexpr int kHalfTokens = 64;

template <typename WT>
struct HalfGeom {
  using G = WidGeom<WT>;
  static constexpr int kBRowBytes = 2 * G::kK;  // bf16 token row per stage
  static constexpr int kBSlots = kBRowBytes / 16;
  static constexpr int kBRowsPerLoad = 1024 / kBRowBytes;
  static constexpr int kBBytes = kHalfTokens * kBRowBytes;
  static constexpr int kLoadsB = kBBytes / 1024 / G::kWaves;  // token loads per wave and stage
  static constexpr int kStageBytes = G::kStageBytes + kBBytes;
  static constexpr int kTA = 4, kNB = 2;  // 16-row weight tiles, 16-token tiles per wave
  static_assert(G::kWaves == 8 && G::kRows == 256, "eight waves over 256 weight rows");
  static_assert(kLoadsB * kBRowsPerLoad == 8, "each wave loads eight token rows");
  static_assert(G::kD * kStageBytes <= 160 * 1024, "the ring's stages fit in LDS");
};

typedef f32x4 HalfAcc[4][2];

template <typename WT>
__device__ __forceinline__ int half_bswz(int row) {
  return HalfGeom<WT>::kBSlots == 16 ? (row & 15) : ((row >> 1) & 7);
}
// Token load i of wave w fills rows kBRowsPerLoad (kLoadsB w + i) + l / kBSlots
// of the token region (wave w: rows 8w .. 8w+7), lane l at physical slot
// l % kBSlots = logical slot (l % kBSlots) ^ bswz(row).
template <typename WT>
__device__ __forceinline__ int half_b_row(int wave, int i, int lane) {
  using H = HalfGeom<WT>;
  return H::kBRowsPerLoad * (H::kLoadsB * wave + i) + lane / H::kBSlots;
}
template <typename WT>
__device__ __forceinline__ int half_b_slot(int row, int lane) {
  return (lane % HalfGeom<WT>::kBSlots) ^ half_bswz<WT>(row);
}

struct HalfLoader {
  __amdgpu_buffer_rsrc_t ra, rb;
  uint32_t a[kWidLoadsA];
  uint32_t b[2];  // this lane's token source of load i, k = 0
};

__device__ __forceinline__ void wid_load_t_lds(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, off,
                                           0, 0, 0);
}

// Part j of stage s's loads (one part per k-step): weight loads
// j * 4 / kSteps .. (j + 1) * 4 / kSteps - 1, and token load j while
// j < kLoadsB (when kB).
template <typename WT, bool kNT, bool kB>
__device__ __forceinline__ void half_issue_part(const HalfLoader& ld, uint8_t* stage,
                                                uint8_t* tstage, int s, int wave, int j) {
  using G = WidGeom<WT>;
  using H = HalfGeom<WT>;
  constexpr int kPer = kWidLoadsA / G::kSteps;
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int i = j * kPer + q;
    uint8_t* dst = stage + (wave * kWidLoadsA + i) * 1024;
    const uint32_t off = ld.a[i] + static_cast<uint32_t>(s) * kWidRowBytes;
    if constexpr (kNT)
      wid_load_w_nt(ld.ra, dst, off);
    else
      wid_load_w(ld.ra, dst, off);
  }
  if constexpr (kB) {
    if (j < H::kLoadsB)
      wid_load_t_lds(ld.rb, tstage + (wave * H::kLoadsB + j) * 1024,
                     ld.b[j] + static_cast<uint32_t>(s) * H::kBRowBytes);
  }
}

template <typename WT, bool kNT, bool kB>
__device__ __forceinline__ void half_issue(const HalfLoader& ld, uint8_t* stage, uint8_t* tstage,
                                           int s, int wave) {
#pragma unroll
  for (int j = 0; j < WidGeom<WT>::kSteps; ++j)
    half_issue_part<WT, kNT, kB>(ld, stage, tstage, s, wave, j);
}

// k-step j: weight tiles t at rows arow0 + 16t (t < 2) and arow1 + 16(t - 2),
// token tiles u at rows brow0 + 16u of the token region.
template <typename WT>
__device__ __forceinline__ void half_kstep(const uint8_t* cur, const uint8_t* tcur, int j,
                                           int arow0, int arow1, int brow0, HalfAcc& acc) {
  using H = HalfGeom<WT>;
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  uint32_t la = wid_a_off<WT>(j);
  uint32_t lb = r16 * H::kBRowBytes + (((4 * j + g) ^ half_bswz<WT>(r16)) << 4);
  asm volatile("" : "+v"(la), "+v"(lb));
  bf16x8 b[2];
#pragma unroll
  for (int u = 0; u < 2; ++u)
    b[u] = as_frag(*reinterpret_cast<const uint4*>(tcur + lb + (brow0 + 16 * u) * H::kBRowBytes));
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int row = t < 2 ? arow0 + 16 * t : arow1 + 16 * (t - 2);
    bf16x8 a;
    if constexpr (sizeof(WT) == 1) {
      const uint2 q = *reinterpret_cast<const uint2*>(cur + la + row * kWidRowBytes);
      a = as_frag(e4m3x8_to_frag_bits(q.x, q.y));
    } else {
      a = as_frag(*reinterpret_cast<const uint4*>(cur + la + row * kWidRowBytes));
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) acc[t][u] = mfma16x16x32(a, b[u], acc[t][u]);
  }
}

// The ring of three stages (as WidRing at depth 3, both operands in LDS):
// kB the wave loads token rows, kLive its 32 token rows hold a real slot.
template <typename WT, bool kNT, bool kB, bool kLive>
struct HalfRing {
  using G = WidGeom<WT>;
  static constexpr int kL = kWidLoadsA + (kB ? HalfGeom<WT>::kLoadsB : 0);
  const HalfLoader& ld;
  uint8_t* const (&buf)[4];  // weights of stage p
  uint8_t* const (&tb)[4];   // token rows of stage p
  int wave, arow0, arow1, brow0;

  template <int p, int W, bool kIssue>
  __device__ __forceinline__ void step(int s, HalfAcc& acc) const {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(kL * W));
    big_barrier();
    constexpr int n = (p + 2) % 3;
    if constexpr (kLive) {
#pragma unroll
      for (int j = 0; j < G::kSteps; ++j) {
        if constexpr (kIssue) half_issue_part<WT, kNT, kB>(ld, buf[n], tb[n], s + 2, wave, j);
        half_kstep<WT>(buf[p], tb[p], j, arow0, arow1, brow0, acc);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else if constexpr (kIssue) {
      half_issue<WT, kNT, kB>(ld, buf[n], tb[n], s + 2, wave);
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  template <int R>  // R = nst % 3; nst >= 2
  __device__ __forceinline__ void run_r(int nst, HalfAcc& acc) const {
    half_issue<WT, kNT, kB>(ld, buf[0], tb[0], 0, wave);
    half_issue<WT, kNT, kB>(ld, buf[1], tb[1], 1, wave);
    int s = 0;
    for (; s + 5 <= nst; s += 3) {
      step<0, 1, true>(s, acc);
      step<1, 1, true>(s + 1, acc);
      step<2, 1, true>(s + 2, acc);
    }
    if constexpr (R == 2) {
      step<0, 1, false>(s, acc);
      step<1, 0, false>(s + 1, acc);
    } else if constexpr (R == 0) {
      step<0, 1, true>(s, acc);
      step<1, 1, false>(s + 1, acc);
      step<2, 0, false>(s + 2, acc);
    } else {
      step<0, 1, true>(s, acc);
      step<1, 1, true>(s + 1, acc);
      step<2, 1, false>(s + 2, acc);
      step<0, 0, false>(s + 3, acc);
    }
  }

  __device__ __forceinline__ void run(int nst, HalfAcc& acc) const {
    const int r = nst % 3;
    if (r == 0) run_r<0>(nst, acc);
    else if (r == 1) run_r<1>(nst, acc);
    else run_r<2>(nst, acc);
  }
};

template <typename WT>
__device__ __forceinline__ void half_run(const HalfLoader& ld, uint8_t* const (&buf)[4],
                                         uint8_t* const (&tb)[4], int nst,
                                         int wave, int arow0, int arow1, int brow0, bool nt,
                                         bool b_live, bool live, HalfAcc& acc) {
  // a live wave loads its eight token rows even when they are all padding
  // (their loads read zeros past the buffer's end), so kLive implies kB
  if (nt) {
    if (live) HalfRing<WT, true, true, true>{ld, buf, tb, wave, arow0, arow1, brow0}.run(nst, acc);
    else if (b_live) HalfRing<WT, true, true, false>{ld, buf, tb, wave, arow0, arow1, brow0}.run(nst, acc);
    else HalfRing<WT, true, false, false>{ld, buf, tb, wave, arow0, arow1, brow0}.run(nst, acc);
  } else {
    if (live) HalfRing<WT, false, true, true>{ld, buf, tb, wave, arow0, arow1, brow0}.run(nst, acc);
    else if (b_live) HalfRing<WT, false, true, false>{ld, buf, tb, wave, arow0, arow1, brow0}.run(nst, acc);
    else HalfRing<WT, false, false, false>{ld, buf, tb, wave, arow0, arow1, brow0}.run(nst, acc);
  }
}

// W13 of a half-full block: wave (wm, wn) = (w % 4, w / 4) holds gate and up
// of channels n0 + 32 wm .. +31 for tokens 32 wn .. +31.
template <typename WT>
__device__ __forceinline__ void half13_tile(const WidLoader& wl, uint8_t* const (&buf)[4],
                                            uint8_t* const (&tb)[4],
                                            const int32_t* blk, const float* s13, int scale_mode,
                                            bf16_t* h, int b, int e, int n0, int d, int I, int k,
                                            int A, uint32_t xbytes, bool nt) {
  using G = WidGeom<WT>;
  using H = HalfGeom<WT>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15;
  const int g = lane >> 4;
  HalfLoader ld;
  ld.ra = wl.ra;
  ld.rb = wl.rb;
#pragma unroll
  for (int i = 0; i < kWidLoadsA; ++i) ld.a[i] = wl.a[i];
#pragma unroll
  for (int i = 0; i < H::kLoadsB; ++i) {
    const int r = half_b_row<WT>(wave, i, lane);
    const int f = blk[r];
    ld.b[i] = f < A ? 2 * static_cast<uint32_t>(f / k) * d + 16 * half_b_slot<WT>(r, lane) : xbytes;
  }
  const bool b_live = __builtin_amdgcn_readfirstlane(blk[8 * wave]) < A;
  const int wm = wave & 3, wn = wave >> 2;
  const bool live = __builtin_amdgcn_readfirstlane(blk[32 * wn]) < A;
  HalfAcc acc;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int u = 0; u < 2; ++u) acc[t][u] = f32x4{0.f, 0.f, 0.f, 0.f};
  half_run<WT>(ld, buf, tb, d / G::kK, wave, 32 * wm, 128 + 32 * wm, 32 * wn, nt, b_live, live, acc);
  if (!live) return;

  // lane: token column r16 of tile u, channels n0 + 32wm + 16t + 4g .. +3
  // (gate in tile t, up in tile t + 2)
  const size_t two_i = 2 * static_cast<size_t>(I);
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int c = n0 + 32 * wm + 16 * t + 4 * g;
    if (c >= I) continue;
    float sg[4], su[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      sg[v] = load_scale(s13, scale_mode, e, static_cast<size_t>(e) * two_i + c + v);
      su[v] = load_scale(s13, scale_mode, e, static_cast<size_t>(e) * two_i + I + c + v);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const size_t row = static_cast<size_t>(b) * kWidTokens + 32 * wn + 16 * u + r16;
      uint32_t packed[2];
#pragma unroll
      for (int v = 0; v < 4; v += 2) {
        const float h0 = silu(acc[t][u][v] * sg[v]) * (acc[t + 2][u][v] * su[v]);
        const float h1 = silu(acc[t][u][v + 1] * sg[v + 1]) * (acc[t + 2][u][v + 1] * su[v + 1]);
        packed[v / 2] = static_cast<uint32_t>(f32_to_bf16(h0)) |
                        (static_cast<uint32_t>(f32_to_bf16(h1)) << 16);
      }
      *reinterpret_cast<uint2*>(h + row * I + c) = uint2{packed[0], packed[1]};
    }
  }
}

// W2 of a half-full block: wave (wm, wn) = (w % 4, w / 4) holds output
// channels n0 + 64 wm .. +63 for tokens 32 wn .. +31.
template <typename WT>
__device__ __forceinline__ void half2_tile(const WidLoader& wl, uint8_t* const (&buf)[4],
                                           uint8_t* const (&tb)[4],
                                           const int32_t* blk, const float* s2, int scale_mode,
                                           const float* topk_w, float* y, int e, int n0, int d,
                                           int I, int A, int k_begin, int nst, uint32_t hbytes,
                                           bool nt) {
  using H = HalfGeom<WT>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15;
  const int g = lane >> 4;
  HalfLoader ld;
  ld.ra = wl.ra;
  ld.rb = wl.rb;
#pragma unroll
  for (int i = 0; i < kWidLoadsA; ++i) ld.a[i] = wl.a[i];
  // h rows of the block; rows of padding slots read zeros
#pragma unroll
  for (int i = 0; i < H::kLoadsB; ++i) {
    const int r = half_b_row<WT>(wave, i, lane);
    ld.b[i] = blk[r] < A ? 2 * (static_cast<uint32_t>(r) * I + k_begin) + 16 * half_b_slot<WT>(r, lane)
                         : hbytes;
  }
  const bool b_live = __builtin_amdgcn_readfirstlane(blk[8 * wave]) < A;
  const int wm = wave & 3, wn = wave >> 2;
  const bool live = __builtin_amdgcn_readfirstlane(blk[32 * wn]) < A;
  HalfAcc acc;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int u = 0; u < 2; ++u) acc[t][u] = f32x4{0.f, 0.f, 0.f, 0.f};
  half_run<WT>(ld, buf, tb, nst, wave, 64 * wm, 64 * wm + 32, 32 * wn, nt, b_live, live, acc);
  if (!live) return;

  // lane: token column r16 of tile u, channels n0 + 64wm + 16t + 4g .. +3
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int f = blk[32 * wn + 16 * u + r16];
    if (f < A) {
      const float gate = topk_w[f];
      float* yrow = y + static_cast<size_t>(f) * d;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int c = n0 + 64 * wm + 16 * t + 4 * g;
        if (c >= d) continue;
        const size_t base = static_cast<size_t>(e) * d + c;
        float sc[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) sc[v] = load_scale(s2, scale_mode, e, base + v);
        store_partial4(yrow + c, acc[t][u][0] * sc[0] * gate, acc[t][u][1] * sc[1] * gate,
                       acc[t][u][2] * sc[2] * gate, acc[t][u][3] * sc[3] * gate);
      }
    }
  }
}

// ------------------------------------------------------------ full blocks (e4m3fn)
// A block with more than 64 real tokens (e4m3fn weights) also takes its
// token rows through LDS: all 128 rows of a stage (256 bytes each, 32 KB),
// loaded once per workgroup as whole rows, where the register path loads
// each token fragment twice as 64-byte half lines.  Weights and tokens
// together would take 64 KB a stage, so the two rings differ in depth: the
// weights keep three stages in flight (32 KB each) and the tokens two (the
// token rows are gathered rows of x or the block's h rows, which sit in the
// caches more often than not, so one stage ahead suffices): 96 + 64 KB.  At
// stage s a wave first issues the token rows of s + 1, then the weights of
// s + 2 a part per k-step, so that the wait at stage s + 1 lets the weights
// of s + 2 (the last four loads) stay in flight.  The token rows of a stage
// lie in two 16 KB arrays (rows 0-63 and 64-127).  Eight waves of 32 weight
// rows x all live token tiles (wave w: W13 gate rows 16w .. +15 and the
// matching up rows, W2 output rows 32w .. +31), so every weight fragment is
// widened once; a block of at most 96 tokens runs six token tiles, a
// larger one eight.
#ifndef MOE_WID_FULL
#define MOE_WID_FULL 1
#endif
constexpr int kFullRowBytes = 256;  // bf16 token row per stage (128 K)
constexpr int kFullLoadsB = 4;      // token loads per wave and stage, four rows each

struct FullLoader {
  __amdgpu_buffer_rsrc_t ra, rb;
  uint32_t a[kWidLoadsA];   // weight sources, as WidLoader
  uint32_t b[kFullLoadsB];  // token source of load i at K = 0
};

typedef f32x4 FullAcc[2][8];

// Token load i of wave w fills block rows 16w + 4i + l / 16, lane l at
// physical slot l % 16, which holds logical slot (l % 16) ^ (row & 15).
__device__ __forceinline__ int full_b_row(int wave, int i, int lane) {
  return 16 * wave + 4 * i + lane / 16;
}
__device__ __forceinline__ int full_b_slot(int row, int lane) { return (lane % 16) ^ (row & 15); }

// Weight load j of stage s (one per k-step), plain or nontemporal.
template <bool kNT>
__device__ __forceinline__ void full_issue_w(const FullLoader& ld, uint8_t* wst, int s, int wave,
                                             int j) {
  uint8_t* dst = wst + (wave * kWidLoadsA + j) * 1024;
  const uint32_t off = ld.a[j] + static_cast<uint32_t>(s) * kWidRowBytes;
  if constexpr (kNT)
    wid_load_w_nt(ld.ra, dst, off);
  else
    wid_load_w(ld.ra, dst, off);
}

// The wave's token rows of stage s (waves 0-3 rows 0-63 into xa, 4-7 rows
// 64-127 into xb).
__device__ __forceinline__ void full_issue_t(const FullLoader& ld, uint8_t* xa, uint8_t* xb, int s,
                                             int wave) {
  uint8_t* base = (wave < 4 ? xa : xb) + (wave & 3) * 16 * kFullRowBytes;
#pragma unroll
  for (int i = 0; i < kFullLoadsB; ++i)
    wid_load_t_lds(ld.rb, base + i * 1024, ld.b[i] + static_cast<uint32_t>(s) * kFullRowBytes);
}

// k-step j: weight tiles at rows arow0 and arow1 of the stage, token tiles
// u < NL at block rows 16u .. +15.
template <int NL>
__device__ __forceinline__ void full_kstep(const uint8_t* wcur, const uint8_t* xa,
                                           const uint8_t* xb, int j, int arow0, int arow1,
                                           FullAcc& acc) {
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  uint32_t la = wid_a_off<fp8_t>(j);
  uint32_t lb = r16 * kFullRowBytes + (((4 * j + g) ^ r16) << 4);
  asm volatile("" : "+v"(la), "+v"(lb));
  bf16x8 bf[NL];
#pragma unroll
  for (int u = 0; u < NL; ++u)
    bf[u] = as_frag(*reinterpret_cast<const uint4*>((u < 4 ? xa : xb) + lb +
                                                    16 * (u & 3) * kFullRowBytes));
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const uint2 q = *reinterpret_cast<const uint2*>(wcur + la + (t ? arow1 : arow0) * kWidRowBytes);
    const bf16x8 a = as_frag(e4m3x8_to_frag_bits(q.x, q.y));
#pragma unroll
    for (int u = 0; u < NL; ++u) acc[t][u] = mfma16x16x32(a, bf[u], acc[t][u]);
  }
}

// The two rings (weights depth 3, tokens depth 2) over `total` >= 2 stages;
// the loop runs six stages at a time so that both buffer indices are
// compile-time constants.
template <bool kNT, int NL>
struct FullRing {
  const FullLoader& ld;
  uint8_t* const (&wb)[4];
  uint8_t* const (&xa)[2];
  uint8_t* const (&xb)[2];
  int wave, arow0, arow1, total;

  template <int p>
  __device__ __forceinline__ void step(int s, FullAcc& acc) const {
    // stage s's loads are in; the weights of s + 1 (issued last) may not be
    if (s + 1 < total)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(kWidLoadsA));
    else
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    big_barrier();
    if (s + 1 < total) full_issue_t(ld, xa[(p + 1) % 2], xb[(p + 1) % 2], s + 1, wave);
    const bool iw = s + 2 < total;
#pragma unroll
    for (int j = 0; j < kWidLoadsA; ++j) {
      if (iw) full_issue_w<kNT>(ld, wb[(p + 2) % 3], s + 2, wave, j);
      full_kstep<NL>(wb[p % 3], xa[p % 2], xb[p % 2], j, arow0, arow1, acc);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  __device__ __forceinline__ void run(FullAcc& acc) const {
#pragma unroll
    for (int j = 0; j < kWidLoadsA; ++j) full_issue_w<kNT>(ld, wb[0], 0, wave, j);
    full_issue_t(ld, xa[0], xb[0], 0, wave);
#pragma unroll
    for (int j = 0; j < kWidLoadsA; ++j) full_issue_w<kNT>(ld, wb[1], 1, wave, j);
    for (int s = 0; s < total; s += 6) {
      step<0>(s, acc);
      if (s + 1 < total) step<1>(s + 1, acc);
      if (s + 2 < total) step<2>(s + 2, acc);
      if (s + 3 < total) step<3>(s + 3, acc);
      if (s + 4 < total) step<4>(s + 4, acc);
      if (s + 5 < total) step<5>(s + 5, acc);
    }
  }
};

template <int NL>
__device__ __forceinline__ void full_run_nl(const FullLoader& ld, uint8_t* const (&wb)[4],
                                            uint8_t* const (&xa)[2], uint8_t* const (&xb)[2],
                                            int total, int wave, int arow0, int arow1, bool nt,
                                            FullAcc& acc) {
  if (nt)
    FullRing<true, NL>{ld, wb, xa, xb, wave, arow0, arow1, total}.run(acc);
  else
    FullRing<false, NL>{ld, wb, xa, xb, wave, arow0, arow1, total}.run(acc);
}

// The token tiles a full block runs: six when its real tokens fit in 96
// rows, else eight.
__device__ __forceinline__ bool full_six(const int32_t* blk, int A) {
  return __builtin_amdgcn_readfirstlane(blk[96]) >= A;
}

// W13 of a full block: wave w holds gate and up of channels n0 + 16w + 4g
// .. +3 (lane (r16, g)) for token column r16 of every token tile u.
template <int NL>
__device__ __forceinline__ void full13_store(const FullAcc& acc, const float* s13, int scale_mode,
                                             bf16_t* h, int b, int e, int n0, int I) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int c = n0 + 16 * wave + 4 * g;
  if (c >= I) return;
  const size_t two_i = 2 * static_cast<size_t>(I);
  float sg[4], su[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    sg[v] = load_scale(s13, scale_mode, e, static_cast<size_t>(e) * two_i + c + v);
    su[v] = load_scale(s13, scale_mode, e, static_cast<size_t>(e) * two_i + I + c + v);
  }
#pragma unroll
  for (int u = 0; u < NL; ++u) {
    const size_t row = static_cast<size_t>(b) * kWidTokens + 16 * u + r16;
    uint32_t packed[2];
#pragma unroll
    for (int v = 0; v < 4; v += 2) {
      const float h0 = silu(acc[0][u][v] * sg[v]) * (acc[1][u][v] * su[v]);
      const float h1 = silu(acc[0][u][v + 1] * sg[v + 1]) * (acc[1][u][v + 1] * su[v + 1]);
      packed[v / 2] = static_cast<uint32_t>(f32_to_bf16(h0)) |
                      (static_cast<uint32_t>(f32_to_bf16(h1)) << 16);
    }
    *reinterpret_cast<uint2*>(h + row * I + c) = uint2{packed[0], packed[1]};
  }
}

template <int NL>
__device__ __forceinline__ void full13_nl(const FullLoader& ld, uint8_t* const (&wb)[4],
                                          uint8_t* const (&xa)[2], uint8_t* const (&xb)[2],
                                          const float* s13, int scale_mode, bf16_t* h, int b,
                                          int e, int n0, int d, int I, bool nt) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  FullAcc acc;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[t][u] = f32x4{0.f, 0.f, 0.f, 0.f};
  full_run_nl<NL>(ld, wb, xa, xb, d / WidGeom<fp8_t>::kK, wave, 16 * wave, 128 + 16 * wave, nt,
                  acc);
  full13_store<NL>(acc, s13, scale_mode, h, b, e, n0, I);
}

__device__ __forceinline__ void full13_tile(const WidLoader& wl, uint8_t* const (&wb)[4],
                                            uint8_t* const (&xa)[2], uint8_t* const (&xb)[2],
                                            const int32_t* blk, const float* s13, int scale_mode,
                                            bf16_t* h, int b, int e, int n0, int d, int I, int k,
                                            int A, uint32_t xbytes, bool nt) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  FullLoader ld;
  ld.ra = wl.ra;
  ld.rb = wl.rb;
#pragma unroll
  for (int i = 0; i < kWidLoadsA; ++i) ld.a[i] = wl.a[i];
#pragma unroll
  for (int i = 0; i < kFullLoadsB; ++i) {
    const int r = full_b_row(wave, i, lane);
    const int f = blk[r];
    ld.b[i] = f < A ? 2 * static_cast<uint32_t>(f / k) * d + 16 * full_b_slot(r, lane) : xbytes;
  }
  if (full_six(blk, A))
    full13_nl<6>(ld, wb, xa, xb, s13, scale_mode, h, b, e, n0, d, I, nt);
  else
    full13_nl<8>(ld, wb, xa, xb, s13, scale_mode, h, b, e, n0, d, I, nt);
}

// W2 of a full block: wave w holds output channels n0 + 32w + 16t + 4g ..
// +3 (weight tile t) for token column r16 of every token tile u.
template <int NL>
__device__ __forceinline__ void full2_nl(const FullLoader& ld, uint8_t* const (&wb)[4],
                                         uint8_t* const (&xa)[2], uint8_t* const (&xb)[2],
                                         const int32_t* blk, const float* s2, int scale_mode,
                                         const float* topk_w, float* y, int e, int n0, int d,
                                         int A, int nst, bool nt) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15;
  const int g = lane >> 4;
  FullAcc acc;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[t][u] = f32x4{0.f, 0.f, 0.f, 0.f};
  full_run_nl<NL>(ld, wb, xa, xb, nst, wave, 32 * wave, 32 * wave + 16, nt, acc);
#pragma unroll
  for (int u = 0; u < NL; ++u) {
    const int f = blk[16 * u + r16];
    if (f < A) {
      const float gate = topk_w[f];
      float* yrow = y + static_cast<size_t>(f) * d;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int c = n0 + 32 * wave + 16 * t + 4 * g;
        if (c >= d) continue;
        const size_t base = static_cast<size_t>(e) * d + c;
        float sc[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) sc[v] = load_scale(s2, scale_mode, e, base + v);
        store_partial4(yrow + c, acc[t][u][0] * sc[0] * gate, acc[t][u][1] * sc[1] * gate,
                       acc[t][u][2] * sc[2] * gate, acc[t][u][3] * sc[3] * gate);
      }
    }
  }
}

__device__ __forceinline__ void full2_tile(const WidLoader& wl, uint8_t* const (&wb)[4],
                                           uint8_t* const (&xa)[2], uint8_t* const (&xb)[2],
                                           const int32_t* blk, const float* s2, int scale_mode,
                                           const float* topk_w, float* y, int e, int n0, int d,
                                           int I, int A, int k_begin, int nst, uint32_t hbytes,
                                           bool nt) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  FullLoader ld;
  ld.ra = wl.ra;
  ld.rb = wl.rb;
#pragma unroll
  for (int i = 0; i < kWidLoadsA; ++i) ld.a[i] = wl.a[i];
  // h rows of the block; rows of padding slots read zeros
#pragma unroll
  for (int i = 0; i < kFullLoadsB; ++i) {
    const int r = full_b_row(wave, i, lane);
    ld.b[i] = blk[r] < A ? 2 * (static_cast<uint32_t>(r) * I + k_begin) + 16 * full_b_slot(r, lane)
                         : hbytes;
  }
  if (full_six(blk, A))
    full2_nl<6>(ld, wb, xa, xb, blk, s2, scale_mode, topk_w, y, e, n0, d, A, nst, nt);
  else
    full2_nl<8>(ld, wb, xa, xb, blk, s2, scale_mode, topk_w, y, e, n0, d, A, nst, nt);
}

// e4m3fn kernels' LDS: three 32 KB weight stages (`buf`, also the register
// path's ring) and four 16 KB token arrays: the half-full path's three token
// stages (`htb`), or the full path's two stages of two halves (`fxa`,
// `fxb`).  160 KB.
#define WID_FP8_LDS()                                                                    \
  __shared__ __attribute__((aligned(1024))) uint8_t wst0[WidGeom<fp8_t>::kStageBytes];  \
  __shared__ __attribute__((aligned(1024))) uint8_t wst1[WidGeom<fp8_t>::kStageBytes];  \
  __shared__ __attribute__((aligned(1024))) uint8_t wst2[WidGeom<fp8_t>::kStageBytes];  \
  __shared__ __attribute__((aligned(1024))) uint8_t xta0[64 * kFullRowBytes];           \
  __shared__ __attribute__((aligned(1024))) uint8_t xtb0[64 * kFullRowBytes];           \
  __shared__ __attribute__((aligned(1024))) uint8_t xta1[64 * kFullRowBytes];           \
  __shared__ __attribute__((aligned(1024))) uint8_t xtb1[64 * kFullRowBytes];           \
  uint8_t* const buf[4] = {wst0, wst1, wst2, wst2};                                      \
  uint8_t* const htb[4] = {xta0, xta1, xtb0, xtb0};                                      \
  uint8_t* const fxa[2] = {xta0, xta1};                                                  \
  uint8_t* const fxb[2] = {xtb0, xtb1}
static_assert(HalfGeom<fp8_t>::kBBytes == 64 * kFullRowBytes, "a half-full token stage is 64 rows");
static_assert(3 * WidGeom<fp8_t>::kStageBytes + 4 * 64 * kFullRowBytes <= 160 * 1024,
              "the e4m3fn LDS fits");

// ------------------------------------------------------------ W13 + SiLU*mul
// Tile (b, y): channels n0 = 128y .. +127 (rows: 128 gate, then 128 up;
// channels at or past I read zeros and are not stored) x the 128 tokens of
// row block b.  Wave w holds gate and up of channels n0 + 64 (w % 2) .. +63
// for tokens 32 (w / 2) .. +31.

template <typename WT>
__device__ __forceinline__ void wide13_tile(WidLoader& ld, uint8_t* const (&buf)[4],
                                            const int32_t* blk, const float* s13, int scale_mode,
                                            bf16_t* h, int b, int e, int n0, int d, int I, int k,
                                            int A, uint32_t xbytes, bool nt) {
  using G = WidGeom<WT>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int wm = wave % G::kRG, wn = wave / G::kRG;
#pragma unroll
  for (int u = 0; u < G::kNB; ++u) {
    const int f = blk[G::kWaveTok * wn + 16 * u + r16];
    ld.b[u] = f < A ? 2 * (static_cast<uint32_t>(f / k) * d + 8 * g) : xbytes;
  }
  WidAcc<WT> acc;
#pragma unroll
  for (int t = 0; t < G::kTA; ++t)
#pragma unroll
    for (int u = 0; u < G::kNB; ++u) acc[t][u] = f32x4{0.f, 0.f, 0.f, 0.f};

  const bool live = __builtin_amdgcn_readfirstlane(blk[G::kWaveTok * wn]) < A;
  const int arow0 = (G::kRows / 2 / G::kRG) * wm;
  wid_run<WT>(ld, buf, d / G::kK, wave, arow0, G::kRows / 2 + arow0, nt, live, acc);
  if (!live) return;

  // lane: token column r16 of tile u, channels n0 + arow0 + 16t + 4g .. +3
  // (gate in tile t, up in tile t + kTA/2)
  const size_t two_i = 2 * static_cast<size_t>(I);
#pragma unroll
  for (int t = 0; t < G::kTA / 2; ++t) {
    const int c = n0 + arow0 + 16 * t + 4 * g;
    if (c >= I) continue;
    float sg[4], su[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      if constexpr (sizeof(WT) == 1) {
        sg[v] = load_scale(s13, scale_mode, e, static_cast<size_t>(e) * two_i + c + v);
        su[v] = load_scale(s13, scale_mode, e, static_cast<size_t>(e) * two_i + I + c + v);
      } else {
        sg[v] = su[v] = 1.0f;
      }
    }
#pragma unroll
    for (int u = 0; u < G::kNB; ++u) {
      const size_t row = static_cast<size_t>(b) * kWidTokens + G::kWaveTok * wn + 16 * u + r16;
      uint32_t packed[2];
#pragma unroll
      for (int v = 0; v < 4; v += 2) {
        const float h0 = silu(acc[t][u][v] * sg[v]) * (acc[t + G::kTA / 2][u][v] * su[v]);
        const float h1 =
            silu(acc[t][u][v + 1] * sg[v + 1]) * (acc[t + G::kTA / 2][u][v + 1] * su[v + 1]);
        packed[v / 2] = static_cast<uint32_t>(f32_to_bf16(h0)) |
                        (static_cast<uint32_t>(f32_to_bf16(h1)) << 16);
      }
      *reinterpret_cast<uint2*>(h + row * I + c) = uint2{packed[0], packed[1]};
    }
  }
}

template <typename WT>
__global__ __launch_bounds__(WidGeom<WT>::kThreads) void ffn13_wide_kernel(
    const bf16_t* __restrict__ x, const WT* __restrict__ w13, const float* __restrict__ s13,
    int scale_mode, const int32_t* __restrict__ sorted_ids,
    const int32_t* __restrict__ block_expert, const int32_t* __restrict__ num_padded,
    bf16_t* __restrict__ h, int d, int I, int k, int A, int T, int gx, int gy) {
  using G = WidGeom<WT>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const BigTile tl = big_tile_live<wid13_cols<WT>()>(blockIdx.x, gx, gy, num_padded, kWidTokens);
  if (!tl.live) return;  // uniform
  const int b = tl.b;
  const int npad = *num_padded;
  const int32_t* blk = sorted_ids + static_cast<size_t>(b) * kWidTokens;
  if (blk[0] >= A) return;  // real slots come first: this block holds none
  const int e = block_expert[b];
  constexpr int kHalf = G::kRows / 2;  // channels per tile
  const int n0 = tl.y * kHalf;
  const size_t two_i = 2 * static_cast<size_t>(I);
  const uint32_t wbytes = static_cast<uint32_t>(two_i * d * sizeof(WT));
  const uint32_t xbytes = static_cast<uint32_t>(static_cast<size_t>(T) * d * 2);
  const uint32_t row_bytes = static_cast<uint32_t>(d) * sizeof(WT);

  WidLoader ld;
  ld.ra = big_rsrc(w13 + static_cast<size_t>(e) * two_i * d, wbytes);
  ld.rb = big_rsrc(x, xbytes);
#pragma unroll
  for (int i = 0; i < kWidLoadsA; ++i) {
    const int r = wid_a_row(wave, i, lane);  // tile rows: kHalf gate, then kHalf up
    const int c = n0 + r % kHalf;
    const uint32_t wrow = r < kHalf ? c : I + c;
    ld.a[i] = c < I ? wrow * row_bytes + 16 * wid_a_slot(r, lane) : wbytes;
  }
  const bool nt = wid_single_block(block_expert, b, npad / kWidTokens, e);
  if constexpr (sizeof(WT) == 1 && G::kWaves == 8) {
    WID_FP8_LDS();
    // real slots come first: no real slot past row 63 means a half-full block
    if (MOE_WID_HALF && __builtin_amdgcn_readfirstlane(blk[kHalfTokens]) >= A) {
      half13_tile<WT>(ld, buf, htb, blk, s13, scale_mode, h, b, e, n0, d, I, k, A, xbytes, nt);
      return;
    }
    if (MOE_WID_FULL) {
      full13_tile(ld, buf, fxa, fxb, blk, s13, scale_mode, h, b, e, n0, d, I, k, A, xbytes, nt);
      return;
    }
    wide13_tile<WT>(ld, buf, blk, s13, scale_mode, h, b, e, n0, d, I, k, A, xbytes, nt);
  } else if constexpr (G::kD == 3) {
    WID_RING3(buf, G::kStageBytes);
    wide13_tile<WT>(ld, buf, blk, s13, scale_mode, h, b, e, n0, d, I, k, A, xbytes, nt);
  } else {
    constexpr int kBytes = HalfGeom<WT>::kStageBytes > G::kStageBytes ? HalfGeom<WT>::kStageBytes
                                                                        : G::kStageBytes;
    WID_RING4(buf, MOE_WID_HALF_BF16 ? kBytes : G::kStageBytes);
    if constexpr (MOE_WID_HALF_BF16) {
      if (__builtin_amdgcn_readfirstlane(blk[kHalfTokens]) >= A) {
        uint8_t* const tb[4] = {buf[0] + G::kStageBytes, buf[1] + G::kStageBytes,
                                buf[2] + G::kStageBytes, buf[3] + G::kStageBytes};
        half13_tile<WT>(ld, buf, tb, blk, s13, scale_mode, h, b, e, n0, d, I, k, A, xbytes, nt);
        return;
      }
    }
    wide13_tile<WT>(ld, buf, blk, s13, scale_mode, h, b, e, n0, d, I, k, A, xbytes, nt);
  }
}

// ------------------------------------------------------------ W2 + gate scale
// Tile (b, y, z): output channels n0 = 256y .. +255 (those at or past d read
// zeros and are not stored) x the block's 128 h rows, over K range z.  Wave
// w holds channels n0 + 128 (w % 2) .. +127 for tokens 32 (w / 2) .. +31.

template <typename WT>
__device__ __forceinline__ void wide2_tile(WidLoader& ld, uint8_t* const (&buf)[4],
                                           const int32_t* blk, const float* s2, int scale_mode,
                                           const float* topk_w, float* y, int e, int n0, int d,
                                           int I, int A, int k_begin, int nst, uint32_t hbytes,
                                           bool nt) {
  using G = WidGeom<WT>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int wm = wave % G::kRG, wn = wave / G::kRG;
  // h rows of the block; rows of padding slots read zeros
#pragma unroll
  for (int u = 0; u < G::kNB; ++u) {
    const int r = G::kWaveTok * wn + 16 * u + r16;
    ld.b[u] = blk[r] < A ? 2 * (static_cast<uint32_t>(r) * I + k_begin + 8 * g) : hbytes;
  }
  WidAcc<WT> acc;
#pragma unroll
  for (int t = 0; t < G::kTA; ++t)
#pragma unroll
    for (int u = 0; u < G::kNB; ++u) acc[t][u] = f32x4{0.f, 0.f, 0.f, 0.f};

  // weight rows arow0 .. +16 kTA - 1: consecutive 16-row tiles
  const bool live = __builtin_amdgcn_readfirstlane(blk[G::kWaveTok * wn]) < A;
  const int arow0 = (G::kRows / G::kRG) * wm;
  wid_run<WT>(ld, buf, nst, wave, arow0, arow0 + 8 * G::kTA, nt, live, acc);
  if (!live) return;

  // lane: token column r16 of tile u, channels n0 + arow0 + 16t + 4g .. +3
#pragma unroll
  for (int u = 0; u < G::kNB; ++u) {
    const int f = blk[G::kWaveTok * wn + 16 * u + r16];
    if (f < A) {
      const float gate = topk_w[f];
      float* yrow = y + static_cast<size_t>(f) * d;
#pragma unroll
      for (int t = 0; t < G::kTA; ++t) {
        const int c = n0 + arow0 + 16 * t + 4 * g;
        if (c >= d) continue;
        float sc[4] = {1.0f, 1.0f, 1.0f, 1.0f};
        if constexpr (sizeof(WT) == 1) {
          const size_t base = static_cast<size_t>(e) * d + c;
#pragma unroll
          for (int v = 0; v < 4; ++v) sc[v] = load_scale(s2, scale_mode, e, base + v);
        }
        store_partial4(yrow + c, acc[t][u][0] * sc[0] * gate, acc[t][u][1] * sc[1] * gate,
                       acc[t][u][2] * sc[2] * gate, acc[t][u][3] * sc[3] * gate);
      }
    }
  }
}

template <typename WT>
__global__ __launch_bounds__(WidGeom<WT>::kThreads) void ffn2_wide_kernel(
    const bf16_t* __restrict__ h, const WT* __restrict__ w2, const float* __restrict__ s2,
    int scale_mode, const float* __restrict__ topk_w, const int32_t* __restrict__ sorted_ids,
    const int32_t* __restrict__ block_expert, const int32_t* __restrict__ num_padded,
    float* __restrict__ y_part, int d, int I, int A, int ksplit, int gx, int gy) {
  using G = WidGeom<WT>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const BigTile tl = big_tile_live<wid2_cols<WT>()>(blockIdx.x, gx, gy, num_padded, kWidTokens);
  if (!tl.live) return;
  const int b = tl.b;
  const int npad = *num_padded;
  const int32_t* blk = sorted_ids + static_cast<size_t>(b) * kWidTokens;
  if (blk[0] >= A) return;
  const int e = block_expert[b];
  const int n0 = tl.y * G::kRows;
  const int k_begin = blockIdx.z * ksplit;
  const int nst = (min(I, k_begin + ksplit) - k_begin) / G::kK;
  float* y = y_part + static_cast<size_t>(blockIdx.z) * A * d;
  const uint32_t wbytes = static_cast<uint32_t>(static_cast<size_t>(d) * I * sizeof(WT));
  const uint32_t hbytes = static_cast<uint32_t>(static_cast<size_t>(kWidTokens) * I * 2);

  WidLoader ld;
  ld.ra = big_rsrc(w2 + static_cast<size_t>(e) * d * I, wbytes);
  ld.rb = big_rsrc(h + static_cast<size_t>(b) * kWidTokens * I, hbytes);
#pragma unroll
  for (int i = 0; i < kWidLoadsA; ++i) {
    const int r = wid_a_row(wave, i, lane);
    const int n = n0 + r;
    ld.a[i] = n < d ? (static_cast<uint32_t>(n) * I + k_begin) * static_cast<uint32_t>(sizeof(WT)) +
                          16 * wid_a_slot(r, lane)
                    : wbytes;
  }
  const bool nt = wid_single_block(block_expert, b, npad / kWidTokens, e);
  if constexpr (sizeof(WT) == 1 && G::kWaves == 8) {
    WID_FP8_LDS();
    if (MOE_WID_HALF && __builtin_amdgcn_readfirstlane(blk[kHalfTokens]) >= A) {
      half2_tile<WT>(ld, buf, htb, blk, s2, scale_mode, topk_w, y, e, n0, d, I, A, k_begin, nst,
                     hbytes, nt);
      return;
    }
    if (MOE_WID_FULL) {
      full2_tile(ld, buf, fxa, fxb, blk, s2, scale_mode, topk_w, y, e, n0, d, I, A, k_begin, nst,
                 hbytes, nt);
      return;
    }
    wide2_tile<WT>(ld, buf, blk, s2, scale_mode, topk_w, y, e, n0, d, I, A, k_begin, nst,
                   hbytes, nt);
  } else if constexpr (G::kD == 3) {
    WID_RING3(buf, G::kStageBytes);
    wide2_tile<WT>(ld, buf, blk, s2, scale_mode, topk_w, y, e, n0, d, I, A, k_begin, nst,
                   hbytes, nt);
  } else {
    constexpr int kBytes = HalfGeom<WT>::kStageBytes > G::kStageBytes ? HalfGeom<WT>::kStageBytes
                                                                        : G::kStageBytes;
    WID_RING4(buf, MOE_WID_HALF_BF16 ? kBytes : G::kStageBytes);
    if constexpr (MOE_WID_HALF_BF16) {
      if (__builtin_amdgcn_readfirstlane(blk[kHalfTokens]) >= A) {
        uint8_t* const tb[4] = {buf[0] + G::kStageBytes, buf[1] + G::kStageBytes,
                                buf[2] + G::kStageBytes, buf[3] + G::kStageBytes};
        half2_tile<WT>(ld, buf, tb, blk, s2, scale_mode, topk_w, y, e, n0, d, I, A, k_begin, nst,
                       hbytes, nt);
        return;
      }
    }
    wide2_tile<WT>(ld, buf, blk, s2, scale_mode, topk_w, y, e, n0, d, I, A, k_begin, nst,
                   hbytes, nt);
  }
}

// ------------------------------------------------------------ launchers

int wide_kchunk(int w_dtype) {
  return w_dtype == kDtypeE4M3FN ? WidGeom<fp8_t>::kK : WidGeom<bf16_t>::kK;
}
static int wide_depth(int w_dtype) {
  return w_dtype == kDtypeE4M3FN ? WidGeom<fp8_t>::kD : WidGeom<bf16_t>::kD;
}

// K stages of 128 bytes of weight row (d and I multiples of the stage's K:
// 64 for bf16, 128 for e4m3fn; I also of 32), at least the ring depth of
// stages per K range, and 32-bit byte offsets into an expert's W13
// (2I x d), x (T x d bf16) and a block's h rows.
bool wide_gemm_fits(int64_t T, int d, int I, int w_dtype) {
#ifdef MOE_NO_WIDE_GEMM
  return false;
#else
  if (w_dtype != kDtypeBF16 && w_dtype != kDtypeE4M3FN) return false;
  const int kk = wide_kchunk(w_dtype), depth = wide_depth(w_dtype);
  const int64_t ws = w_dtype == kDtypeE4M3FN ? 1 : 2;
  const int64_t lim = int64_t(1) << 31;
  return d % kk == 0 && I % kk == 0 && I % 32 == 0 && d / kk >= depth && I / kk >= depth &&
         2 * int64_t(I) * d * ws < lim && T * d * 2 < lim && int64_t(kWidTokens) * I * 2 < lim;
#endif
}

static bool wide_args_ok(const FfnArgs& a) {
  return a.B == kWidTokens && a.act_dtype == kDtypeBF16 && !a.act_mx &&
         wide_gemm_fits(a.T, a.d, a.I, a.w_dtype);
}

static int wide_grid(int gx, int gy) {
  const int total = gx * gy;
  return (total + kBigXcds - 1) / kBigXcds * kBigXcds;
}

template <typename WT>
static void wide13_go(const FfnArgs& a, hipStream_t s) {
  constexpr int kHalf = WidGeom<WT>::kRows / 2;
  const int gx = a.cap / kWidTokens, gy = (a.I + kHalf - 1) / kHalf;
  ffn13_wide_kernel<WT><<<wide_grid(gx, gy), WidGeom<WT>::kThreads, 0, s>>>(
      static_cast<const bf16_t*>(a.x), static_cast<const WT*>(a.w13), a.s13, a.scale_mode,
      a.sorted_ids, a.block_expert, a.num_padded, static_cast<bf16_t*>(a.h), a.d, a.I, a.k, a.A,
      a.T, gx, gy);
}

template <typename WT>
static void wide2_go(const FfnArgs& a, hipStream_t s) {
  constexpr int kRows = WidGeom<WT>::kRows;
  const int gx = a.cap / kWidTokens, gy = (a.d + kRows - 1) / kRows;
  ffn2_wide_kernel<WT><<<dim3(wide_grid(gx, gy), 1, a.splits), WidGeom<WT>::kThreads, 0, s>>>(
      static_cast<const bf16_t*>(a.h), static_cast<const WT*>(a.w2), a.s2, a.scale_mode,
      a.topk_w, a.sorted_ids, a.block_expert, a.num_padded, a.y_part, a.d, a.I, a.A, a.ksplit,
      gx, gy);
}

hipError_t launch_ffn13_wide(const FfnArgs& a, hipStream_t s) {
  if (!wide_args_ok(a)) return hipErrorInvalidValue;
  if (a.w_dtype == kDtypeE4M3FN)
    wide13_go<fp8_t>(a, s);
  else
    wide13_go<bf16_t>(a, s);
  return hipGetLastError();
}

hipError_t launch_ffn2_wide(const FfnArgs& a, hipStream_t s) {
  // every K range a whole number of stages, at least the ring depth
  const int kk = wide_kchunk(a.w_dtype), depth = wide_depth(a.w_dtype);
  if (!wide_args_ok(a) || a.splits < 1 || a.ksplit < depth * kk || a.ksplit % kk != 0 ||
      static_cast<int64_t>(a.splits - 1) * a.ksplit >= a.I ||
      a.I - static_cast<int64_t>(a.splits - 1) * a.ksplit < depth * kk)
    return hipErrorInvalidValue;
  if (a.w_dtype == kDtypeE4M3FN)
    wide2_go<fp8_t>(a, s);
  else
    wide2_go<bf16_t>(a, s);
  return hipGetLastError();
}

}  // namespace moe
