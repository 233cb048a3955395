// Expert kernels for small token blocks (decode) with bf16 or e4m3fn
// weights, weights streamed through LDS: the HBM-bound end of the fused MoE
// layer.
//
// Sources: the Hungarian news page "Az AWS új MoE-optimalizációkkal
// gyorsítja a SageMaker AI-t", section "A fused MoE a számítási folyamat több
// lépését egyesíti" (the grouped expert computation and the gated SiLU
// product); the French summary "Ingénierie de kernels Mixture-of-Experts sur
// Amazon SageMaker AI", first paragraph (at decode the expert product has a
// tiny token dimension, so its cost is reading the weights).
//
// With at most 32 tokens per expert block every weight byte feeds at most
// 32 MACs, so the kernel's speed is the weight read rate.  Loading the
// weights straight into MFMA registers makes every load instruction cover
// 16 rows x 64 bytes, half of each row's 128-byte line; HBM serves that
// pattern well below its streaming rate.  Here every load instruction is a
// direct-to-LDS load of two rows x 512 contiguous bytes, with the
// nontemporal hint (the weights are read once), and the MFMA fragments come
// from LDS.  The token operand (x for W13, h for W2, a few L2-resident rows)
// is loaded into a register ring of the same depth, in the same stream: loads
// complete in issue order, so the wait for stage c leaves stages c+1 ..
// c+P-2 in flight, and LDS holds weights only.
//
// LDS stage: one 16-row tile per gate / up / output tile, rows of 512 bytes
// (256 bf16 or 512 e4m3fn of K; e4m3fn is widened to bf16 after the LDS
// read, exactly, and its per-channel scale applied in the epilogue).  Row r's 16-byte unit u sits in slot u ^ (r & 15), so the 16 rows one
// 16-lane group reads for the same k hit 16 different bank groups; the
// permutation is applied by choosing each lane's source address, which keeps
// every 256-byte group of a row contiguous in HBM.  One wave per workgroup,
// P stages each in an LDS array of its own (distinct arrays let the compiler
// see that reads of one stage do not depend on loads into another).

#include "ffn_common.h"

namespace moe {

constexpr int kDmaRowBytes = 512;  // bytes of one row per stage
constexpr int kDmaThreads = 64;
constexpr int kDmaAux = 2;         // cache policy of the loads: nontemporal

template <typename WT>
constexpr int dma_kc() { return kDmaRowBytes / static_cast<int>(sizeof(WT)); }  // K per stage

int dma_stream_kc(int w_dtype) { return w_dtype == kDtypeE4M3FN ? dma_kc<fp8_t>() : dma_kc<bf16_t>(); }

bool dma_stream_fits(int d, int I, int w_dtype) {
  const int kc = dma_stream_kc(w_dtype);
  return d % kc == 0 && I % kc == 0;
}

// Stage geometry for NROW weight tiles and NS live token subtiles.
template <typename WT, int NROW, int NS>
struct DmaGeom {
  static constexpr int kStageBytes = 16 * NROW * kDmaRowBytes;  // weight rows only
  static constexpr int kFrags = dma_kc<WT>() / 32;              // MFMA k-steps per stage
  static constexpr int kLoadsW = 8 * NROW;                      // direct-to-LDS loads (2 rows each)
  static constexpr int kLoadsA = kFrags * NS;                   // token loads (one per k-step)
  static constexpr int kLoads = kLoadsW + kLoadsA;
};

// s_waitcnt immediate: at most n vector-memory loads outstanding.
constexpr int dma_vmcnt(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Per-lane operand sources.
//   wlane[t]: weight tile t's row `hi` (= lane / 32) at k = 0 (bytes); the
//             stage row r of tile t is loaded by instruction 8t + (r & 15) / 2;
//   arow[s]:  the token row of this lane's MFMA column in subtile s, k = 0
//             (pad slots point at a valid row; their columns are dropped).
// The token operand uses the k layout of the weight type (ActChunk): for
// e4m3fn one 16-byte LDS read holds k = 64j + 16g .. +16 of a row, the first
// eight feeding MFMA 2j and the last eight MFMA 2j+1.
template <typename WT, int NROW, int NS>
struct DmaOperands {
  static constexpr int kF = DmaGeom<WT, NROW, NS>::kFrags;
  const uint8_t* wlane[NROW];
  const bf16_t* arow[NS];
  size_t wld;  // weight row length (bytes)
  int l31, hi, r16, g;

  __device__ __forceinline__ void issue_w(uint8_t* stage, size_t kbyte) const {
#pragma unroll
    for (int i = 0; i < 8 * NROW; ++i) {
      const int j = ((2 * i) & 15) + hi;  // row within the tile
      const uint8_t* src = wlane[i / 8] + static_cast<size_t>((2 * i) & 15) * wld + kbyte;
      __builtin_amdgcn_global_load_lds(src + 16 * (l31 ^ j), stage + 1024 * i, 16, 0, kDmaAux);
    }
  }
  template <int NSL>
  __device__ __forceinline__ void issue_a(uint4 (&a)[NS][kF], int k0) const {
#pragma unroll
    for (int s = 0; s < NSL; ++s)
#pragma unroll
      for (int i = 0; i < kF; ++i)
        a[s][i] = *reinterpret_cast<const uint4*>(arow[s] + k0 + ActChunk<WT, 64>::off(i, g));
  }

  // acc[s][t] += W_tile(t) . A_subtile(s) over the stage's K.
  template <int NSL>
  __device__ __forceinline__ void mma(const uint8_t* stage, const uint4 (&a)[NS][kF],
                                      f32x4 (&acc)[NS][NROW]) const {
    if constexpr (sizeof(WT) == 2) {
#pragma unroll
      for (int q = 0; q < kF; ++q) {
        const int slot = ((4 * q + g) ^ r16) << 4;
        bf16x8 wf[NROW];
#pragma unroll
        for (int t = 0; t < NROW; ++t)
          wf[t] = as_frag(*reinterpret_cast<const uint4*>(stage + (16 * t + r16) * kDmaRowBytes + slot));
#pragma unroll
        for (int s = 0; s < NSL; ++s)
#pragma unroll
          for (int t = 0; t < NROW; ++t)
            acc[s][t] = mfma16x16x32(wf[t], as_frag(a[s][q]), acc[s][t]);
      }
    } else {
#pragma unroll
      for (int jp = 0; jp < kF / 2; ++jp) {
        const int slot = ((4 * jp + g) ^ r16) << 4;
        bf16x8 lo[NROW], hi8[NROW];
#pragma unroll
        for (int t = 0; t < NROW; ++t) {
          const uint4 q = *reinterpret_cast<const uint4*>(stage + (16 * t + r16) * kDmaRowBytes + slot);
          lo[t] = as_frag(e4m3x8_to_frag_bits(q.x, q.y));
          hi8[t] = as_frag(e4m3x8_to_frag_bits(q.z, q.w));
        }
#pragma unroll
        for (int s = 0; s < NSL; ++s)
#pragma unroll
          for (int t = 0; t < NROW; ++t) {
            acc[s][t] = mfma16x16x32(lo[t], as_frag(a[s][2 * jp]), acc[s][t]);
            acc[s][t] = mfma16x16x32(hi8[t], as_frag(a[s][2 * jp + 1]), acc[s][t]);
          }
      }
    }
  }
};

// The ring: chunk c (K = k_begin + c*KC ..) in buffer c % P (weights in LDS,
// token fragments in registers).  Stages 0 .. P-2 are issued up front; at
// chunk c the wave waits until only the stages issued after chunk c are
// outstanding (loads complete in issue order), issues chunk c+P-1 (while
// there is one) into the buffers read at chunk c-1, then runs chunk c's
// MFMAs.  Every wait count is a compile-time immediate: the steady loop goes
// P chunks at a time, and the last P-1 chunks (which issue nothing) run from
// a switch on the buffer they start in.  NSL: live token subtiles.
template <typename WT, int NROW, int NS, int P, int NSL>
struct DmaRing {
  using Op = DmaOperands<WT, NROW, NS>;
  static constexpr int kL = DmaGeom<WT, NROW, NSL>::kLoads;
  static constexpr int kKC = dma_kc<WT>();
  static constexpr int kF = Op::kF;
  const Op& op;
  uint8_t* const (&ring)[4];
  int k_begin, nch;

  __device__ __forceinline__ void issue(uint8_t* stage, uint4 (&a)[NS][kF], int c) const {
    const int k = k_begin + c * kKC;
    op.issue_w(stage, static_cast<size_t>(k) * sizeof(WT));
    op.template issue_a<NSL>(a, k);
  }

  // chunk c in buffer p, issuing chunk c+P-1
  template <int p>
  __device__ __forceinline__ void step(int c, uint4 (&a)[P][NS][kF], f32x4 (&acc)[NS][NROW]) const {
    constexpr int pn = (p + P - 1) % P;
    __builtin_amdgcn_s_waitcnt(dma_vmcnt(kL * (P - 2)));
    issue(ring[pn], a[pn], c + P - 1);
    op.template mma<NSL>(ring[p], a[p], acc);
  }
  // chunk in buffer p with W stages issued after it, issuing nothing
  template <int p, int W>
  __device__ __forceinline__ void last(uint4 (&a)[P][NS][kF], f32x4 (&acc)[NS][NROW]) const {
    __builtin_amdgcn_s_waitcnt(dma_vmcnt(kL * W));
    op.template mma<NSL>(ring[p], a[p], acc);
  }
  // the final P-1 chunks, the first of them in buffer b
  template <int b>
  __device__ __forceinline__ void tail(uint4 (&a)[P][NS][kF], f32x4 (&acc)[NS][NROW]) const {
    last<b % P, P - 2>(a, acc);
    if constexpr (P > 2) last<(b + 1) % P, P - 3>(a, acc);
    if constexpr (P > 3) last<(b + 2) % P, P - 4>(a, acc);
  }

  __device__ __forceinline__ void run(f32x4 (&acc)[NS][NROW]) const {
    static_assert(P >= 2 && P <= 4, "ring depth");
    uint4 a[P][NS][kF];
    // prologue; a chunk past the end (only when nch < P-1) repeats the last
#pragma unroll
    for (int q = 0; q + 1 < P; ++q) issue(ring[q], a[q], min(q, nch - 1));
    if (nch >= P - 1) {
      const int M = nch - P + 1;  // chunks that issue a later one
      int c0 = 0;
      for (; c0 + P <= M; c0 += P) {
        step<0>(c0, a, acc);
        step<1>(c0 + 1, a, acc);
        if constexpr (P > 2) step<2>(c0 + 2, a, acc);
        if constexpr (P > 3) step<3>(c0 + 3, a, acc);
      }
      const int r = M - c0;  // 0 .. P-1 issuing chunks left
      if (r >= 1) step<0>(c0, a, acc);
      if constexpr (P > 2)
        if (r >= 2) step<1>(c0 + 1, a, acc);
      if constexpr (P > 3)
        if (r >= 3) step<2>(c0 + 2, a, acc);
      switch (r) {
        case 0: tail<0>(a, acc); break;
        case 1: tail<1>(a, acc); break;
        case 2: if constexpr (P > 2) tail<2>(a, acc); break;
        case 3: if constexpr (P > 3) tail<3>(a, acc); break;
      }
    } else {  // nch < P-1: the prologue issued P-1 stages for nch chunks
      last<0, P - 2>(a, acc);
      if constexpr (P > 3)
        if (nch >= 2) last<1, P - 3>(a, acc);
    }
    __builtin_amdgcn_s_waitcnt(dma_vmcnt(0));  // no load may land after the wave ends
  }
};

template <typename WT, int NROW, int NS, int P>
__device__ __forceinline__ void dma_dot(int nsub, const DmaOperands<WT, NROW, NS>& op,
                                        uint8_t* const (&ring)[4], int k_begin, int nch,
                                        f32x4 (&acc)[NS][NROW]) {
  if (nsub == 1 || NS == 1) {
    DmaRing<WT, NROW, NS, P, 1>{op, ring, k_begin, nch}.run(acc);
  } else {
    DmaRing<WT, NROW, NS, P, NS>{op, ring, k_begin, nch}.run(acc);
  }
}

#define DMA_RING(name, bytes, P)                                                   \
  __shared__ __attribute__((aligned(1024))) uint8_t name##0[bytes];                \
  __shared__ __attribute__((aligned(1024))) uint8_t name##1[(P) > 1 ? (bytes) : 16]; \
  __shared__ __attribute__((aligned(1024))) uint8_t name##2[(P) > 2 ? (bytes) : 16]; \
  __shared__ __attribute__((aligned(1024))) uint8_t name##3[(P) > 3 ? (bytes) : 16]; \
  uint8_t* const name[4] = {name##0, name##1, name##2, name##3}

template <typename WT, int NROW, int NS>
__device__ __forceinline__ void dma_lanes(DmaOperands<WT, NROW, NS>& op, size_t row_elems) {
  const int lane = threadIdx.x;
  op.l31 = lane & 31;
  op.hi = lane >> 5;
  op.r16 = lane & 15;
  op.g = lane >> 4;
  op.wld = row_elems * sizeof(WT);
}

// ------------------------------------------------------------ W13 + SiLU*mul
// Grid: x = row block b (B = 16 NS), y = 16-channel tile.  The wave computes
// gate rows n0.. and up rows I+n0.. against the block's tokens and writes
// h[row, n] = SiLU(s_g gate) * (s_u up) for the live subtiles (pad rows
// included: their columns never reach an output).

template <typename WT, int NS, int P>
__global__ __launch_bounds__(kDmaThreads) void ffn13_dma_kernel(
    const bf16_t* __restrict__ x, const WT* __restrict__ w13, const float* __restrict__ s13,
    int scale_mode, const int32_t* __restrict__ sorted_ids,
    const int32_t* __restrict__ block_expert, const int32_t* __restrict__ num_padded,
    bf16_t* __restrict__ h, int d, int I, int k, int A) {
  constexpr int B = 16 * NS;
  using G = DmaGeom<WT, 2, NS>;
  DMA_RING(ring, G::kStageBytes, P);
  const int b = blockIdx.x;
  if (b * B >= *num_padded) return;
  const int e = block_expert[b];
  const int n0 = blockIdx.y * 16;
  const int32_t* blk = sorted_ids + static_cast<size_t>(b) * B;
  const int nsub = live_subtiles<NS>(blk, A);

  DmaOperands<WT, 2, NS> op;
  dma_lanes(op, d);
  const size_t erow = static_cast<size_t>(e) * 2 * I;
  const uint8_t* wb = reinterpret_cast<const uint8_t*>(w13);
  op.wlane[0] = wb + (erow + n0 + op.hi) * op.wld;      // gate tile
  op.wlane[1] = wb + (erow + I + n0 + op.hi) * op.wld;  // up tile
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int f = blk[16 * s + op.r16];  // pad slots read token 0
    op.arow[s] = x + static_cast<size_t>(f < A ? f / k : 0) * d;
  }

  f32x4 acc[NS][2];
#pragma unroll
  for (int s = 0; s < NS; ++s) acc[s][0] = acc[s][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  dma_dot<WT, 2, NS, P>(nsub, op, ring, 0, d / dma_kc<WT>(), acc);

  // lane: token column r16, channels n0 + 4g .. +3
  const int nb = n0 + 4 * op.g;
  float sg[4], su[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    sg[v] = load_scale(s13, scale_mode, e, erow + nb + v);
    su[v] = load_scale(s13, scale_mode, e, erow + I + nb + v);
  }
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    if (s < nsub) {
      const size_t row = static_cast<size_t>(b) * B + 16 * s + op.r16;
      uint32_t packed[2];
#pragma unroll
      for (int v = 0; v < 4; v += 2) {
        const float h0 = silu(acc[s][0][v] * sg[v]) * (acc[s][1][v] * su[v]);
        const float h1 = silu(acc[s][0][v + 1] * sg[v + 1]) * (acc[s][1][v + 1] * su[v + 1]);
        packed[v / 2] = static_cast<uint32_t>(f32_to_bf16(h0)) |
                        (static_cast<uint32_t>(f32_to_bf16(h1)) << 16);
      }
      *reinterpret_cast<uint2*>(h + row * I + nb) = uint2{packed[0], packed[1]};
    }
  }
}

// ------------------------------------------------------------ W2 + gate scale
// Grid: x = row block b, y = group of 16 RN channels of d, z = split of
// K = I.  Writes y_part[z, f, n] = gate_f * s(n) * sum_{i in split} W2[e, n, i] h[row, i]
// for the block's real slots f.  RN tiles per wave: every wave reads all h
// rows of its block, so wider waves read less h per weight byte.

template <typename WT, int NS, int P, int RN>
__global__ __launch_bounds__(kDmaThreads) void ffn2_dma_kernel(
    const bf16_t* __restrict__ h, const WT* __restrict__ w2, const float* __restrict__ s2,
    int scale_mode, const float* __restrict__ topk_w, const int32_t* __restrict__ sorted_ids,
    const int32_t* __restrict__ block_expert, const int32_t* __restrict__ num_padded,
    float* __restrict__ y_part, int d, int I, int A, int ksplit) {
  constexpr int B = 16 * NS;
  using G = DmaGeom<WT, RN, NS>;
  DMA_RING(ring, G::kStageBytes, P);
  const int b = blockIdx.x;
  if (b * B >= *num_padded) return;
  const int e = block_expert[b];
  const int n0 = blockIdx.y * 16 * RN;
  const int z = blockIdx.z;
  const int k_begin = z * ksplit;
  const int nch = (min(I, k_begin + ksplit) - k_begin) / dma_kc<WT>();
  const int32_t* blk = sorted_ids + static_cast<size_t>(b) * B;
  const int nsub = live_subtiles<NS>(blk, A);

  DmaOperands<WT, RN, NS> op;
  dma_lanes(op, I);
  const uint8_t* wb = reinterpret_cast<const uint8_t*>(w2);
#pragma unroll
  for (int rt = 0; rt < RN; ++rt)
    op.wlane[rt] = wb + (static_cast<size_t>(e) * d + n0 + 16 * rt + op.hi) * op.wld;
  // h row of this lane's column; pad slots read the block's first row (a
  // real slot's) so that their loads share one address
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int slot = 16 * s + op.r16;
    const size_t row = static_cast<size_t>(b) * B + (blk[slot] < A ? slot : 0);
    op.arow[s] = h + row * I;
  }

  f32x4 acc[NS][RN];
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int rt = 0; rt < RN; ++rt) acc[s][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (nch > 0) dma_dot<WT, RN, NS, P>(nsub, op, ring, k_begin, nch, acc);

#pragma unroll
  for (int s = 0; s < NS; ++s) {
    if (s < nsub) {
      const int f = blk[16 * s + op.r16];
      if (f < A) {
        const float gate = topk_w[f];
        float* yrow = y_part + (static_cast<size_t>(z) * A + f) * d;
#pragma unroll
        for (int rt = 0; rt < RN; ++rt) {
          const int nb = n0 + 16 * rt + 4 * op.g;
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

#ifndef MOE_DMA13_P1
#define MOE_DMA13_P1 4
#endif
#ifndef MOE_DMA13_P2
#define MOE_DMA13_P2 2
#endif
#ifndef MOE_DMA2_P1
#define MOE_DMA2_P1 3
#endif
#ifndef MOE_DMA2_P2
#define MOE_DMA2_P2 3
#endif
#ifndef MOE_DMA_FP8_P13
#define MOE_DMA_FP8_P13 2
#endif
#ifndef MOE_DMA_FP8_P2
#define MOE_DMA_FP8_P2 2
#endif
#ifndef MOE_DMA2_RN
#define MOE_DMA2_RN 2
#endif
#ifndef MOE_DMA_FP8_RN2
#define MOE_DMA_FP8_RN2 2
#endif
constexpr int kDma2RN = MOE_DMA2_RN;
constexpr int kDma2RNFp8 = MOE_DMA_FP8_RN2;

// Four channel tiles per bf16 W2 wave when blocks of 16 give at most two row
// blocks (a single token of a top-2 layer): the grid is small there, and
// wider waves read the block's h rows half as often (measured at d = 4096,
// I = 14336: 50 -> 44 us with a two-stage ring); with more blocks two tiles
// per wave are faster (T = 8: 160 against 172 us).
constexpr int kDma2WideRN = 4;
constexpr int kDma2WideP = 2;
constexpr int64_t kDma2WideBlocks = 2;

static int dma_w2_rn(int w_dtype, int B, int64_t blocks_est) {
  if (w_dtype == kDtypeE4M3FN) return kDma2RNFp8;
  return B == 16 && blocks_est <= kDma2WideBlocks ? kDma2WideRN : kDma2RN;
}

int dma_w2_channels(int w_dtype, int B, int64_t blocks_est) {
  return 16 * dma_w2_rn(w_dtype, B, blocks_est);
}

namespace {

template <typename WT, int NS, int P>
hipError_t ffn13_dma_go(const FfnArgs& a, hipStream_t s) {
  const dim3 grid(a.cap / a.B, a.I / 16);
  ffn13_dma_kernel<WT, NS, P><<<grid, kDmaThreads, 0, s>>>(
      static_cast<const bf16_t*>(a.x), static_cast<const WT*>(a.w13), a.s13, a.scale_mode,
      a.sorted_ids, a.block_expert, a.num_padded, static_cast<bf16_t*>(a.h), a.d, a.I, a.k, a.A);
  return hipGetLastError();
}

template <typename WT, int NS, int P, int RN = sizeof(WT) == 1 ? kDma2RNFp8 : kDma2RN>
hipError_t ffn2_dma_go(const FfnArgs& a, hipStream_t s) {
  const dim3 grid(a.cap / a.B, a.d / (16 * RN), a.splits);
  ffn2_dma_kernel<WT, NS, P, RN><<<grid, kDmaThreads, 0, s>>>(
      static_cast<const bf16_t*>(a.h), static_cast<const WT*>(a.w2), a.s2, a.scale_mode,
      a.topk_w, a.sorted_ids, a.block_expert, a.num_padded, a.y_part, a.d, a.I, a.A, a.ksplit);
  return hipGetLastError();
}

bool dma_args_ok(const FfnArgs& a) {
  return a.act_dtype == kDtypeBF16 && dma_stream_fits(a.d, a.I, a.w_dtype) &&
         (a.w_dtype == kDtypeBF16 || a.w_dtype == kDtypeE4M3FN);
}

}  // namespace

hipError_t launch_ffn13_dma(const FfnArgs& a, hipStream_t s) {
  if (!dma_args_ok(a)) return hipErrorInvalidValue;
  if (a.w_dtype == kDtypeE4M3FN)
    return a.B == 16 ? ffn13_dma_go<fp8_t, 1, MOE_DMA_FP8_P13>(a, s) : hipErrorInvalidValue;
  switch (a.B) {
    case 16:
      // at most two row blocks (one token of a top-2 layer): a two-stage
      // ring keeps more workgroups resident for the few rounds there are
      // (d = 4096, I = 14336: 83 -> 77 us; with eight blocks it is level)
      if (ffn_blocks_estimate(a.cap, a.B, a.E, a.A) <= kDma2WideBlocks)
        return ffn13_dma_go<bf16_t, 1, 2>(a, s);
      return ffn13_dma_go<bf16_t, 1, MOE_DMA13_P1>(a, s);
    case 32: return ffn13_dma_go<bf16_t, 2, MOE_DMA13_P2>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_ffn2_dma(const FfnArgs& a, hipStream_t s) {
  if (!dma_args_ok(a) || a.ksplit % dma_stream_kc(a.w_dtype) != 0 ||
      a.d % dma_w2_channels(a.w_dtype, a.B, ffn_blocks_estimate(a.cap, a.B, a.E, a.A)) != 0)
    return hipErrorInvalidValue;
  if (a.w_dtype == kDtypeE4M3FN)
    return a.B == 16 ? ffn2_dma_go<fp8_t, 1, MOE_DMA_FP8_P2>(a, s) : hipErrorInvalidValue;
  switch (a.B) {
    case 16:
      if (dma_w2_rn(a.w_dtype, a.B, ffn_blocks_estimate(a.cap, a.B, a.E, a.A)) == kDma2WideRN)
        return ffn2_dma_go<bf16_t, 1, kDma2WideP, kDma2WideRN>(a, s);
      return ffn2_dma_go<bf16_t, 1, MOE_DMA2_P1>(a, s);
    case 32: return ffn2_dma_go<bf16_t, 2, MOE_DMA2_P2>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
