// Token-tiled grouped GEMM for blocks of 128 tokens: the expert kernels of
// the large-batch regime (prefill, and fine-grained experts at large T).
//
// Sources: the Hungarian news page "Az AWS új MoE-optimalizációkkal
// gyorsítja a SageMaker AI-t", section "A fused MoE a számítási folyamat több
// lépését egyesíti" (the experts' computation as one batched operation over
// all experts), and section "FP8 esetén a Triton backend bizonyult
// gyorsabbnak" (FP8 scaling and the matrix product in one pass over data read
// once from HBM).
//
// With 128 tokens per block the product is a real dense contraction, so the
// token operand is shared: a workgroup of four waves stages the block's
// 128 x KC token tile in LDS (double buffered, rows padded by 16 bytes so the
// 16-byte reads of 16 different rows hit different banks) and every wave
// multiplies it with its own weight rows.  Weight rows still go HBM/L2 ->
// registers through the per-wave ring of the streaming kernels (each weight
// element is used by one wave only); the four waves of a workgroup cover
// 4 * 16 * RN output channels.  Operands meet on v_mfma_f32_16x16x32_bf16
// with weight rows on M and tokens on N; e4m3fn weights are widened exactly
// in registers.  The W13 epilogue applies SiLU(gate) * up, the W2 epilogue
// the per-channel scale and the slot's gate.
//
// Tiles reach workgroups by one of two schedules (same page, same section:
// dynamic scheduling of token groups of varying size): a static XCD-aware
// raster over every possible tile, or persistent workgroups that take the
// realised tiles from per-XCD work queues.  A tile's arithmetic does not
// depend on the workgroup that runs it, so both give the same bits.

#include "ffn_common.h"

namespace moe {

// Waves per workgroup (each wave owns 16 * RN output channels; the waves
// share the token tile).  Measured: W13 runs best with 4, W2 with 8.
constexpr int kWaves13 = 4;
constexpr int kWaves2 = 8;
constexpr int kGemmTokens = 128;  // block size B of this path
constexpr int kGemmNSub = kGemmTokens / 16;

#ifndef MOE_GEMM_PIPE
#define MOE_GEMM_PIPE 2
#endif
#ifndef MOE_GEMM_RN
#define MOE_GEMM_RN 1
#endif
// W2 takes two channel tiles per wave: each workgroup then covers 256
// output channels, so the block's h rows (streamed through LDS once per
// workgroup) are read half as often.  Measured side by side at the fp8
// workload's T = 2048: W2 1433 against 1444 us (W13 is much slower that way,
// 2.0 -> 2.9 ms, and keeps one).
#ifndef MOE_GEMM_RN2
#define MOE_GEMM_RN2 2
#endif

// Rows of the token tile this thread stages: KC/8 16-byte pieces per row,
// piece q = tid + 64*WAVES*i, row = q / (KC/8).  Rows that hold no token
// (pad slots, dead sub-tiles) read a valid address and are zeroed with a
// select, so staging has no branches (branching here measured slower).
template <int KC, int WAVES>
struct Stager {
  static constexpr int kPiecesPerRow = KC / 8;
  static constexpr int kRowsPerPass = 64 * WAVES / kPiecesPerRow;
  static constexpr int kPieces = kGemmTokens / kRowsPerPass;  // per thread
  static constexpr int kPitch = KC + 8;                       // elements per LDS row
  const bf16_t* src[kPieces];  // row start + piece column (a valid row if dead)
  uint32_t live;               // bit i: piece i carries a token
  int tid;                     // thread index in the workgroup
  uint4 v[kPieces];

  __device__ __forceinline__ int row(int i) const {
    return tid / kPiecesPerRow + kRowsPerPass * i;
  }
  __device__ __forceinline__ int col() const { return (tid % kPiecesPerRow) * 8; }
  __device__ __forceinline__ void load(int k0) {
#pragma unroll
    for (int i = 0; i < kPieces; ++i) {
      const uint4 q = *reinterpret_cast<const uint4*>(src[i] + k0);
      const bool on = (live >> i) & 1u;
      v[i] = uint4{on ? q.x : 0u, on ? q.y : 0u, on ? q.z : 0u, on ? q.w : 0u};
    }
  }
  __device__ __forceinline__ void store(bf16_t* buf) const {
#pragma unroll
    for (int i = 0; i < kPieces; ++i)
      *reinterpret_cast<uint4*>(buf + row(i) * kPitch + col()) = v[i];
  }
};

// Workgroup -> (row block, channel group).  The grid is 1-D.  Workgroup id p
// runs on XCD p % 8 (the dispatcher deals workgroups round-robin over the 8
// XCDs, each with its own L2), so logical tile l = (p % 8) * per_xcd + p / 8
// gives every XCD a contiguous run of the logical order.  That order walks
// super-rows of kGroupCols channel groups; inside one, the row block varies
// slowest: the workgroups an XCD runs together cover kGroupCols channel
// groups x consecutive row blocks (one expert's tokens), so their weight and
// token tiles are shared through that XCD's L2.
constexpr int kXcds = 8;
constexpr int kGroupCols = 4;

struct TileId {
  int b, y;
  bool live;
};

// Logical tile l (< gx * gy) -> (row block, channel group).
__device__ __forceinline__ TileId logical_tile(int l, int gx, int gy) {
  TileId t{0, 0, true};
  const int band = kGroupCols * gx;            // tiles per full super-row
  const int sr = l / band;
  const int rem = l - sr * band;
  const int cols = min(kGroupCols, gy - sr * kGroupCols);  // channel groups in this super-row
  t.b = rem / cols;
  t.y = sr * kGroupCols + rem % cols;
  return t;
}

__device__ __forceinline__ TileId tile_of(int p, int gx, int gy) {
  const int total = gx * gy;
  const int per_xcd = (total + kXcds - 1) / kXcds;
  const int l = (p % kXcds) * per_xcd + p / kXcds;
  if (l >= total) return TileId{0, 0, false};
  return logical_tile(l, gx, gy);
}

inline int raster_grid(int gx, int gy) {
  const int total = gx * gy;
  return (total + kXcds - 1) / kXcds * kXcds;
}

// Queue schedule (persistent workgroups).  The live tiles -- row blocks below
// num_padded, read on the device -- in the same logical order, cut into
// kXcds contiguous segments with one counter each.  Workgroup p belongs to
// segment p % kXcds, the XCD it runs on, so each XCD still walks its own
// stretch of the order and shares weight and token tiles through its L2.
// Its first tile is fixed (tile p / kXcds of the segment: no counter traffic
// while every workgroup starts at once); after that it takes tickets from
// the segment's counter, and once the segment is drained from the next
// segments in turn, so an XCD whose tiles ran faster (blocks at most half
// full skip half of the MFMA work) helps the others finish.  A workgroup
// gives up a segment after one ticket past its end and never returns to
// it, so it exits after at most kXcds empty tickets.  Device-scope atomics
// leave the XCD, so each counter sits in a 128-byte line of its own and a
// segment is read before it is added to.  The counters must be zero at
// launch.
constexpr int kQueueStride = 32;                          // int32 per counter line
constexpr int kQueueInts = 2 * kXcds * kQueueStride;      // W13's lines, then W2's

struct TileQueue {
  int32_t* cnt;  // kXcds counters, kQueueStride apart
  int total;     // live tiles
  int home;      // this workgroup's segment
  int per;       // workgroups per segment (first tiles handed out without a counter)
  int tried;     // segments given up (thread 0's copy is the one used)
  bool started;

  __device__ __forceinline__ int seg_begin(int s) const {
    return static_cast<int>(static_cast<int64_t>(total) * s / kXcds);
  }
  // Next logical tile, or -1 once every segment is drained (thread 0 only).
  __device__ __forceinline__ int take() {
    if (!started) {
      started = true;
      const int first = static_cast<int>(blockIdx.x / kXcds);
      if (first < seg_begin(home + 1) - seg_begin(home)) return seg_begin(home) + first;
    }
    while (tried < kXcds) {
      const int s = (home + tried) % kXcds;
      const int b0 = seg_begin(s), n = seg_begin(s + 1) - b0;
      int32_t* c = cnt + s * kQueueStride;
      if (per + __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < n) {
        const int t = per + atomicAdd(c, 1);
        if (t < n) return b0 + t;
      }
      ++tried;
    }
    return -1;
  }
};

// Runs body(b, y) for every tile this workgroup takes; all threads of the
// workgroup see the same tile, and the loop ends for all of them together.
// The grid is a multiple of kXcds.
template <class Body>
__device__ __forceinline__ void queue_loop(int32_t* cnt, int nblocks, int gy, Body&& body) {
  __shared__ int s_tile;
  TileQueue q{cnt, nblocks * gy, static_cast<int>(blockIdx.x % kXcds),
              static_cast<int>(gridDim.x / kXcds), 0, false};
  for (;;) {
    if (threadIdx.x == 0) s_tile = q.take();
    __syncthreads();
    const int l = s_tile;
    __syncthreads();  // every thread has read s_tile before thread 0 writes it again
    if (l < 0) break;
    const TileId t = logical_tile(l, nblocks, gy);
    body(t.b, t.y);
  }
}

// threadIdx.x through an empty asm statement: what a tile derives from it is
// then computed per tile rather than hoisted out of the persistent loop,
// where it would stay live (in registers) through every main loop.
__device__ __forceinline__ int tile_tid() {
  int t = static_cast<int>(threadIdx.x);
  asm volatile("" : "+v"(t));
  return t;
}

// Row blocks the queue hands out: the realised ones, never more than the
// capacity holds (as the static grid, whatever num_padded says).
__device__ __forceinline__ int live_blocks(const int32_t* num_padded, int gx) {
  return max(0, min(*num_padded / kGemmTokens, gx));
}

__global__ void queue_reset_kernel(int32_t* cnt) {
  for (int i = threadIdx.x; i < kQueueInts; i += blockDim.x) cnt[i] = 0;
}

// Shared main loop: acc[s][r] += W_rows[r] . tokens[s]^T over all K.  The
// block's sub-tiles are processed in two halves of four; the second half is
// skipped (one uniform branch) when it holds no token, which halves the MFMA
// work of blocks that are at most half full.  Inside a half every sub-tile
// is computed, branch-free.
template <typename WT, int KC, int P, int NROW, int WAVES>
__device__ __forceinline__ void gemm_mainloop(WeightStream<WT, KC, NROW, P>& ws,
                                              Stager<KC, WAVES>& st, bf16_t* lds, bool upper_half,
                                              f32x4 (&acc)[kGemmNSub][NROW]) {
  constexpr int NF = KC / 32;
  constexpr int kPitch = Stager<KC, WAVES>::kPitch;
  constexpr int kBuf = kGemmTokens * kPitch;
  constexpr int kHalf = kGemmNSub / 2;
  const int lane = st.tid & 63;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int last = ws.nch - 1;

  st.load(0);
  st.store(lds);
  ws.start(0);
  __syncthreads();
  for (int c0 = 0; c0 < ws.nch; c0 += P) {
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int c = c0 + p;
      if (c < ws.nch) {
        st.load(min(c + 1, last) * KC);  // the last chunk reloads itself: harmless
        bf16x8 wf[NROW][NF];
        ws.take(p, c, 0, wf);
        const bf16_t* tile = lds + (c & 1) * kBuf;
#pragma unroll
        for (int i = 0; i < NF; ++i) {
          const int off = ActChunk<WT, KC>::off(i, g);
#pragma unroll
          for (int s = 0; s < kHalf; ++s) {
            const bf16x8 bf =
                as_frag(*reinterpret_cast<const uint4*>(tile + (16 * s + r16) * kPitch + off));
#pragma unroll
            for (int r = 0; r < NROW; ++r) acc[s][r] = mfma16x16x32(wf[r][i], bf, acc[s][r]);
          }
        }
        if (upper_half) {
#pragma unroll
          for (int i = 0; i < NF; ++i) {
            const int off = ActChunk<WT, KC>::off(i, g);
#pragma unroll
            for (int s = kHalf; s < kGemmNSub; ++s) {
              const bf16x8 bf =
                  as_frag(*reinterpret_cast<const uint4*>(tile + (16 * s + r16) * kPitch + off));
#pragma unroll
              for (int r = 0; r < NROW; ++r) acc[s][r] = mfma16x16x32(wf[r][i], bf, acc[s][r]);
            }
          }
        }
        st.store(lds + ((c + 1) & 1) * kBuf);  // (after the last chunk: unread)
        __syncthreads();
      }
    }
  }
}

// ------------------------------------------------------------ W13 + SiLU*mul
//
// Tile (b, y): row block b (128 tokens of one expert) x group y of
// 4 * 16 * RN output channels of I.

template <typename WT, int KC, int P, int RN, int WAVES>
__device__ __forceinline__ void ffn13_gemm_tile(
    const bf16_t* __restrict__ x, const WT* __restrict__ w13, const float* __restrict__ s13,
    int scale_mode, const int32_t* __restrict__ sorted_ids,
    const int32_t* __restrict__ block_expert, bf16_t* __restrict__ h, int d, int I, int k, int A,
    int b, int cg, bf16_t* lds) {
  constexpr int NROW = 2 * RN;
  const int tid = tile_tid();
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int e = block_expert[b];
  const int32_t* blk = sorted_ids + static_cast<size_t>(b) * kGemmTokens;
  const int nsub = live_subtiles<kGemmNSub>(blk, A);
  const int n0 = (cg * WAVES + wave) * 16 * RN;  // the channel groups tile I exactly

  Stager<KC, WAVES> st;
  st.live = 0;
  st.tid = tid;
#pragma unroll
  for (int i = 0; i < Stager<KC, WAVES>::kPieces; ++i) {
    const int f = blk[st.row(i)];
    const bool on = f < A;
    st.live |= static_cast<uint32_t>(on) << i;
    st.src[i] = x + static_cast<size_t>(on ? f / k : 0) * d + st.col();
  }
  const size_t two_i = 2 * static_cast<size_t>(I);
  WeightStream<WT, KC, NROW, P> ws;
  ws.g = g;
  ws.nch = d / KC;
#pragma unroll
  for (int rt = 0; rt < RN; ++rt) {
    ws.row[rt] = w13 + (static_cast<size_t>(e) * two_i + n0 + rt * 16 + r16) * d;
    ws.row[RN + rt] = w13 + (static_cast<size_t>(e) * two_i + I + n0 + rt * 16 + r16) * d;
  }
  f32x4 acc[kGemmNSub][NROW];
#pragma unroll
  for (int s = 0; s < kGemmNSub; ++s)
#pragma unroll
    for (int r = 0; r < NROW; ++r) acc[s][r] = f32x4{0.f, 0.f, 0.f, 0.f};

  gemm_mainloop<WT, KC, P, NROW, WAVES>(ws, st, lds, nsub > kGemmNSub / 2, acc);

#pragma unroll
  for (int rt = 0; rt < RN; ++rt) {
    const int nb = n0 + rt * 16 + 4 * g;
    float sg[4], su[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      sg[v] = load_scale(s13, scale_mode, e, static_cast<size_t>(e) * two_i + nb + v);
      su[v] = load_scale(s13, scale_mode, e, static_cast<size_t>(e) * two_i + I + nb + v);
    }
#pragma unroll
    for (int s = 0; s < kGemmNSub; ++s) {
      if (s < nsub) {
        const size_t row = static_cast<size_t>(b) * kGemmTokens + 16 * s + r16;
        uint32_t packed[2];
#pragma unroll
        for (int v = 0; v < 4; v += 2) {
          const float h0 = silu(acc[s][rt][v] * sg[v]) * (acc[s][RN + rt][v] * su[v]);
          const float h1 = silu(acc[s][rt][v + 1] * sg[v + 1]) * (acc[s][RN + rt][v + 1] * su[v + 1]);
          packed[v / 2] = static_cast<uint32_t>(f32_to_bf16(h0)) |
                          (static_cast<uint32_t>(f32_to_bf16(h1)) << 16);
        }
        *reinterpret_cast<uint2*>(h + row * I + nb) = uint2{packed[0], packed[1]};
      }
    }
  }
}

// Static schedule: one workgroup per tile of the XCD-aware raster (dead row
// blocks exit at once).  Queue schedule: a grid of resident workgroups
// takes the live tiles from the queue.
template <typename WT, int KC, int P, int RN, int WAVES, bool kQueue>
__global__ __launch_bounds__(64 * WAVES) void ffn13_gemm_kernel(
    const bf16_t* __restrict__ x, const WT* __restrict__ w13, const float* __restrict__ s13,
    int scale_mode, const int32_t* __restrict__ sorted_ids,
    const int32_t* __restrict__ block_expert, const int32_t* __restrict__ num_padded,
    bf16_t* __restrict__ h, int d, int I, int k, int A, int gx, int gy, int32_t* queue) {
  __shared__ __attribute__((aligned(16))) bf16_t lds[2 * kGemmTokens * Stager<KC, WAVES>::kPitch];
  if constexpr (kQueue) {
    queue_loop(queue, live_blocks(num_padded, gx), gy, [&](int b, int cg) {
      ffn13_gemm_tile<WT, KC, P, RN, WAVES>(x, w13, s13, scale_mode, sorted_ids, block_expert, h,
                                            d, I, k, A, b, cg, lds);
    });
  } else {
    const TileId t = tile_of(blockIdx.x, gx, gy);
    if (!t.live || t.b * kGemmTokens >= *num_padded) return;  // uniform over the workgroup
    ffn13_gemm_tile<WT, KC, P, RN, WAVES>(x, w13, s13, scale_mode, sorted_ids, block_expert, h, d,
                                          I, k, A, t.b, t.y, lds);
  }
}

// ------------------------------------------------------------ W2 + gate scale
//
// Tile (b, cg): row block b x group cg of 4 * 16 * RN output channels of d.
// Writes y[f, n] = gate_f * s(n) * (W2[e] h[row])[n] for the block's slots.

template <typename WT, int KC, int P, int RN, int WAVES>
__device__ __forceinline__ void ffn2_gemm_tile(
    const bf16_t* __restrict__ h, const WT* __restrict__ w2, const float* __restrict__ s2,
    int scale_mode, const float* __restrict__ topk_w, const int32_t* __restrict__ sorted_ids,
    const int32_t* __restrict__ block_expert, float* __restrict__ y, int d, int I, int A, int b,
    int cg, bf16_t* lds) {
  const int tid = tile_tid();
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int e = block_expert[b];
  const int32_t* blk = sorted_ids + static_cast<size_t>(b) * kGemmTokens;
  const int nsub = live_subtiles<kGemmNSub>(blk, A);
  const int n0 = (cg * WAVES + wave) * 16 * RN;  // the channel groups tile d exactly

  Stager<KC, WAVES> st;
  st.live = 0;
  st.tid = tid;
#pragma unroll
  for (int i = 0; i < Stager<KC, WAVES>::kPieces; ++i) {
    const int r = st.row(i);
    const bool on = r < 16 * nsub && blk[r] < A;  // h rows of pads and dead sub-tiles: zero
    st.live |= static_cast<uint32_t>(on) << i;
    st.src[i] = h + (static_cast<size_t>(b) * kGemmTokens + (on ? r : 0)) * I + st.col();
  }
  WeightStream<WT, KC, RN, P> ws;
  ws.g = g;
  ws.nch = I / KC;
#pragma unroll
  for (int rt = 0; rt < RN; ++rt)
    ws.row[rt] = w2 + (static_cast<size_t>(e) * d + n0 + rt * 16 + r16) * I;
  f32x4 acc[kGemmNSub][RN];
#pragma unroll
  for (int s = 0; s < kGemmNSub; ++s)
#pragma unroll
    for (int r = 0; r < RN; ++r) acc[s][r] = f32x4{0.f, 0.f, 0.f, 0.f};

  gemm_mainloop<WT, KC, P, RN, WAVES>(ws, st, lds, nsub > kGemmNSub / 2, acc);

#pragma unroll
  for (int s = 0; s < kGemmNSub; ++s) {
    if (s < nsub) {
      const int f = blk[16 * s + r16];
      if (f < A) {
        const float gate = topk_w[f];
        float* yrow = y + static_cast<size_t>(f) * d;
#pragma unroll
        for (int rt = 0; rt < RN; ++rt) {
          const int nb = n0 + rt * 16 + 4 * g;
          float4 o;
          o.x = acc[s][rt][0] * load_scale(s2, scale_mode, e, static_cast<size_t>(e) * d + nb) * gate;
          o.y = acc[s][rt][1] * load_scale(s2, scale_mode, e, static_cast<size_t>(e) * d + nb + 1) * gate;
          o.z = acc[s][rt][2] * load_scale(s2, scale_mode, e, static_cast<size_t>(e) * d + nb + 2) * gate;
          o.w = acc[s][rt][3] * load_scale(s2, scale_mode, e, static_cast<size_t>(e) * d + nb + 3) * gate;
          *reinterpret_cast<float4*>(yrow + nb) = o;
        }
      }
    }
  }
}

template <typename WT, int KC, int P, int RN, int WAVES, bool kQueue>
__global__ __launch_bounds__(64 * WAVES) void ffn2_gemm_kernel(
    const bf16_t* __restrict__ h, const WT* __restrict__ w2, const float* __restrict__ s2,
    int scale_mode, const float* __restrict__ topk_w, const int32_t* __restrict__ sorted_ids,
    const int32_t* __restrict__ block_expert, const int32_t* __restrict__ num_padded,
    float* __restrict__ y, int d, int I, int A, int gx, int gy, int32_t* queue) {
  __shared__ __attribute__((aligned(16))) bf16_t lds[2 * kGemmTokens * Stager<KC, WAVES>::kPitch];
  if constexpr (kQueue) {
    queue_loop(queue, live_blocks(num_padded, gx), gy, [&](int b, int cg) {
      ffn2_gemm_tile<WT, KC, P, RN, WAVES>(h, w2, s2, scale_mode, topk_w, sorted_ids,
                                           block_expert, y, d, I, A, b, cg, lds);
    });
  } else {
    const TileId t = tile_of(blockIdx.x, gx, gy);
    if (!t.live || t.b * kGemmTokens >= *num_padded) return;
    ffn2_gemm_tile<WT, KC, P, RN, WAVES>(h, w2, s2, scale_mode, topk_w, sorted_ids, block_expert,
                                         y, d, I, A, t.b, t.y, lds);
  }
}

// ------------------------------------------------------------ launchers

namespace {

constexpr int kPG = MOE_GEMM_PIPE, kRNG = MOE_GEMM_RN, kRNG2 = MOE_GEMM_RN2;
static_assert(kRNG == 1 || kRNG == 2, "channel tiles per wave: 1 or 2");
static_assert(kRNG2 == 1 || kRNG2 == 2, "channel tiles per wave: 1 or 2");

// A workgroup covers 16 * RN * WAVES output channels; the launchers pick the
// widest configuration whose channel group divides the channel count (a
// multiple of 64, so 4 waves x 16 channels always fits).
// Workgroups of kernel K the chip holds at once (occupancy x compute units),
// asked of the runtime once per kernel (for the first device it runs on; a
// process is taken to drive one kind of GPU); 0 when it cannot say.
template <auto K>
int resident_workgroups(int threads) {
  static const int n = [threads] {
    int per_cu = 0, dev = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, K, threads, 0) != hipSuccess ||
        hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    return per_cu * cus;
  }();
  return n;
}

// Grid of a launch: the raster for the static schedule; for the queue, the
// resident workgroups (a multiple of kXcds so every XCD's segment has its
// own takers), at most one per possible tile.
template <auto K>
int sched_grid(bool queue, int gx, int gy, int threads) {
  const int full = raster_grid(gx, gy);
  if (!queue) return full;
  const int res = resident_workgroups<K>(threads) / kXcds * kXcds;
  return res > 0 && res < full ? res : full;
}

template <typename WT, int KC, int RN, int WAVES, bool kQueue>
void ffn13_gemm_launch(const FfnArgs& a, hipStream_t s) {
  constexpr int P = sizeof(WT) == 1 ? kPG + 1 : kPG;
  constexpr auto kern = ffn13_gemm_kernel<WT, KC, P, RN, WAVES, kQueue>;
  const int gx = a.cap / kGemmTokens, gy = a.I / (WAVES * 16 * RN);
  kern<<<sched_grid<kern>(kQueue, gx, gy, 64 * WAVES), 64 * WAVES, 0, s>>>(
      static_cast<const bf16_t*>(a.x), static_cast<const WT*>(a.w13), a.s13, a.scale_mode,
      a.sorted_ids, a.block_expert, a.num_padded, static_cast<bf16_t*>(a.h), a.d, a.I, a.k, a.A,
      gx, gy, a.queue);
}

template <typename WT, int KC, int RN, int WAVES>
void ffn13_gemm_launch(const FfnArgs& a, hipStream_t s) {
  if (a.queue_sched)
    ffn13_gemm_launch<WT, KC, RN, WAVES, true>(a, s);
  else
    ffn13_gemm_launch<WT, KC, RN, WAVES, false>(a, s);
}

template <typename WT, int KC>
void ffn13_gemm_go(const FfnArgs& a, hipStream_t s) {
  if (kRNG == 2 && a.I % (kWaves13 * 32) == 0)
    ffn13_gemm_launch<WT, KC, kRNG, kWaves13>(a, s);
  else
    ffn13_gemm_launch<WT, KC, 1, kWaves13>(a, s);
}

template <typename WT, int KC, int RN, int WAVES, bool kQueue>
void ffn2_gemm_launch(const FfnArgs& a, hipStream_t s) {
  constexpr int P = sizeof(WT) == 1 ? kPG + 1 : kPG;
  constexpr auto kern = ffn2_gemm_kernel<WT, KC, P, RN, WAVES, kQueue>;
  const int gx = a.cap / kGemmTokens, gy = a.d / (WAVES * 16 * RN);
  kern<<<sched_grid<kern>(kQueue, gx, gy, 64 * WAVES), 64 * WAVES, 0, s>>>(
      static_cast<const bf16_t*>(a.h), static_cast<const WT*>(a.w2), a.s2, a.scale_mode,
      a.topk_w, a.sorted_ids, a.block_expert, a.num_padded, a.y_part, a.d, a.I, a.A, gx, gy,
      a.queue + kXcds * kQueueStride);
}

template <typename WT, int KC, int RN, int WAVES>
void ffn2_gemm_launch(const FfnArgs& a, hipStream_t s) {
  if (a.queue_sched)
    ffn2_gemm_launch<WT, KC, RN, WAVES, true>(a, s);
  else
    ffn2_gemm_launch<WT, KC, RN, WAVES, false>(a, s);
}

template <typename WT, int KC>
void ffn2_gemm_go(const FfnArgs& a, hipStream_t s) {
  if (a.d % (kWaves2 * 16 * kRNG2) == 0)
    ffn2_gemm_launch<WT, KC, kRNG2, kWaves2>(a, s);
  else
    ffn2_gemm_launch<WT, KC, 1, 4>(a, s);
}

template <typename WT>
hipError_t ffn13_gemm_w(const FfnArgs& a, hipStream_t s) {
  if (a.d % 128 == 0)
    ffn13_gemm_go<WT, 128>(a, s);
  else
    ffn13_gemm_go<WT, 64>(a, s);
  return hipGetLastError();
}

template <typename WT>
hipError_t ffn2_gemm_w(const FfnArgs& a, hipStream_t s) {
  if (a.I % 128 == 0)
    ffn2_gemm_go<WT, 128>(a, s);
  else
    ffn2_gemm_go<WT, 64>(a, s);
  return hipGetLastError();
}

}  // namespace

int gemm_queue_ints() { return kQueueInts; }

hipError_t launch_gemm_queue_reset(const FfnArgs& a, hipStream_t s) {
  if (!a.queue) return hipErrorInvalidValue;
  queue_reset_kernel<<<1, 256, 0, s>>>(a.queue);
  return hipGetLastError();
}

hipError_t launch_ffn13_gemm(const FfnArgs& a, hipStream_t s) {
  if (a.B != kGemmTokens || (a.queue_sched && !a.queue)) return hipErrorInvalidValue;
  return a.w_dtype == kDtypeE4M3FN ? ffn13_gemm_w<fp8_t>(a, s) : ffn13_gemm_w<bf16_t>(a, s);
}

hipError_t launch_ffn2_gemm(const FfnArgs& a, hipStream_t s) {
  if (a.B != kGemmTokens || a.splits != 1 || (a.queue_sched && !a.queue))
    return hipErrorInvalidValue;
  return a.w_dtype == kDtypeE4M3FN ? ffn2_gemm_w<fp8_t>(a, s) : ffn2_gemm_w<bf16_t>(a, s);
}

}  // namespace moe
