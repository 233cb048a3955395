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
#ifndef MOE_DMA_TOKEN_MASK
#define MOE_DMA_TOKEN_MASK 1
#endif
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

// s_waitcnt immediate: at most n vector-memory loads outstanding.  The
// vmcnt field is 6 bits (0..63); callers static_assert that n fits, since a
// larger count would silently encode a smaller wait.
constexpr int kDmaMaxVmcnt = 63;
constexpr int dma_vmcnt(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Per-lane operand sources.
//   wlane[t]: weight tile t's row `hi` (= lane / 32) at k = 0 (bytes); the
//             stage row r of tile t is loaded by instruction 8t + (r & 15) / 2;
//   arow[s]:  the token row of this lane's MFMA column in subtile s, k = 0
//             (pad slots point at a valid row; their columns are dropped);
//   tlive[s]: this lane's row of subtile s holds a real slot.  Only those
//             lanes load token fragments (the others keep stale registers,
//             which feed only the dropped columns): with one or a few tokens
//             in a block the token loads then cost the texture units a few
//             lanes instead of 64 per instruction.  A loaded subtile's first
//             row is always real (real slots come first), so no token load
//             instruction runs with every lane off and each still counts in
//             the stage's vmcnt.
// The token operand uses the k layout of the weight type (ActChunk): for
// e4m3fn one 16-byte LDS read holds k = 64j + 16g .. +16 of a row, the first
// eight feeding MFMA 2j and the last eight MFMA 2j+1.
template <typename WT, int NROW, int NS>
struct DmaOperands {
  static constexpr int kF = DmaGeom<WT, NROW, NS>::kFrags;
  const uint8_t* wlane[NROW];
  const bf16_t* arow[NS];
  bool tlive[NS];
  size_t wld;  // weight row length (bytes)
  int l31, hi, r16, g;

  __device__ __forceinline__ void issue_w(uint8_t* stage, size_t kbyte) const {
    // the stage as an LDS address: the low 32 bits of a generic pointer into
    // LDS are its LDS offset (taken this way rather than by an address-space
    // cast, which the backend lowered to an unencodable compare in the fused
    // kernel's tile loop)
    typedef __attribute__((address_space(3))) uint8_t lds_u8;
    lds_u8* const lds = reinterpret_cast<lds_u8*>(
        static_cast<uintptr_t>(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(stage))));
#pragma unroll
    for (int i = 0; i < 8 * NROW; ++i) {
      const int j = ((2 * i) & 15) + hi;  // row within the tile
      const uint8_t* src = wlane[i / 8] + static_cast<size_t>((2 * i) & 15) * wld + kbyte;
      __builtin_amdgcn_global_load_lds(src + 16 * (l31 ^ j), lds + 1024 * i, 16, 0, kDmaAux);
    }
  }
  // kDevA: the token rows were written in this launch by workgroups that
  // may sit on other XCDs (the fused kernel's h): each 16-byte fragment is
  // read as two 8-byte agent-scope atomic loads, which bypass this XCD's L2
  // copy, so two load instructions per fragment (kTokenLoadsPer).
  template <int NSL, bool kDevA = false>
  __device__ __forceinline__ void issue_a(uint4 (&a)[NS][kF], int k0) const {
#pragma unroll
    for (int s = 0; s < NSL; ++s)
      if (!MOE_DMA_TOKEN_MASK || tlive[s]) {
#pragma unroll
        for (int i = 0; i < kF; ++i) {
          const bf16_t* src = arow[s] + k0 + ActChunk<WT, 64>::off(i, g);
          if constexpr (kDevA) {
            const uint64_t* q = reinterpret_cast<const uint64_t*>(src);
            const uint64_t lo = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const uint64_t hi = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            a[s][i] = uint4{static_cast<uint32_t>(lo), static_cast<uint32_t>(lo >> 32),
                            static_cast<uint32_t>(hi), static_cast<uint32_t>(hi >> 32)};
          } else {
            a[s][i] = *reinterpret_cast<const uint4*>(src);
          }
        }
      }
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
template <typename WT, int NROW, int NS, int P, int NSL, bool kDevA = false>
struct DmaRing {
  using Op = DmaOperands<WT, NROW, NS>;
  // vector-memory instructions per stage: the weight loads, then one token
  // load per fragment (two with device-scope token loads)
  static constexpr int kL =
      DmaGeom<WT, NROW, NSL>::kLoadsW + DmaGeom<WT, NROW, NSL>::kLoadsA * (kDevA ? 2 : 1);
  static constexpr int kKC = dma_kc<WT>();
  static constexpr int kF = Op::kF;
  const Op& op;
  uint8_t* const (&ring)[4];
  int k_begin, nch;

  __device__ __forceinline__ void issue(uint8_t* stage, uint4 (&a)[NS][kF], int c) const {
    const int k = k_begin + c * kKC;
    op.issue_w(stage, static_cast<size_t>(k) * sizeof(WT));
    op.template issue_a<NSL, kDevA>(a, k);
  }

  // chunk c in buffer p, issuing chunk c+P-1
  static_assert(kL * (P - 2) <= kDmaMaxVmcnt,
                "loads per stage x (ring depth - 2) exceed the 6-bit vmcnt field");

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
    static_assert(kL * W <= kDmaMaxVmcnt, "wait count exceeds the 6-bit vmcnt field");
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

template <typename WT, int NROW, int NS, int P, bool kDevA = false>
__device__ __forceinline__ void dma_dot(int nsub, const DmaOperands<WT, NROW, NS>& op,
                                        uint8_t* const (&ring)[4], int k_begin, int nch,
                                        f32x4 (&acc)[NS][NROW]) {
  if (nsub == 1 || NS == 1) {
    DmaRing<WT, NROW, NS, P, 1, kDevA>{op, ring, k_begin, nch}.run(acc);
  } else {
    DmaRing<WT, NROW, NS, P, NS, kDevA>{op, ring, k_begin, nch}.run(acc);
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
// One tile: row block b (B = 16 NS), 16 channels from n0.  The wave computes
// gate rows n0.. and up rows I+n0.. against the block's tokens and writes
// h[row, n] = SiLU(s_g gate) * (s_u up) for the live subtiles (pad rows
// included: their columns never reach an output).

// kDevH: h is written with agent-scope atomic stores (write-through past
// this XCD's L2) for readers in the same launch on other XCDs.
template <typename WT, int NS, int P, int RC = 1, bool kDevH = false>
__device__ __forceinline__ void dma13_tile(
    const bf16_t* __restrict__ x, const WT* __restrict__ w13, const float* __restrict__ s13,
    int scale_mode, const int32_t* __restrict__ sorted_ids,
    const int32_t* __restrict__ block_expert, bf16_t* __restrict__ h, int d, int I, int k, int A,
    int b, int n0, uint8_t* const (&ring)[4]) {
  constexpr int B = 16 * NS;
  const int e = block_expert[b];
  const int32_t* blk = sorted_ids + static_cast<size_t>(b) * B;
  const int nsub = live_subtiles<NS>(blk, A);

  // RC channel tiles of 16: gate tiles 0 .. RC-1, then the matching up tiles
  DmaOperands<WT, 2 * RC, NS> op;
  dma_lanes(op, d);
  const size_t erow = static_cast<size_t>(e) * 2 * I;
  const uint8_t* wb = reinterpret_cast<const uint8_t*>(w13);
#pragma unroll
  for (int c = 0; c < RC; ++c) {
    op.wlane[c] = wb + (erow + n0 + 16 * c + op.hi) * op.wld;           // gate tile
    op.wlane[RC + c] = wb + (erow + I + n0 + 16 * c + op.hi) * op.wld;  // up tile
  }
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int f = blk[16 * s + op.r16];  // pad slots read token 0
    op.arow[s] = x + static_cast<size_t>(f < A ? f / k : 0) * d;
    op.tlive[s] = f < A;
  }

  f32x4 acc[NS][2 * RC];
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int t = 0; t < 2 * RC; ++t) acc[s][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  dma_dot<WT, 2 * RC, NS, P>(nsub, op, ring, 0, d / dma_kc<WT>(), acc);

#pragma unroll
  for (int c = 0; c < RC; ++c) {
    // lane: token column r16, channels n0 + 16c + 4g .. +3
    const int nb = n0 + 16 * c + 4 * op.g;
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
          const float h0 = silu(acc[s][c][v] * sg[v]) * (acc[s][RC + c][v] * su[v]);
          const float h1 =
              silu(acc[s][c][v + 1] * sg[v + 1]) * (acc[s][RC + c][v + 1] * su[v + 1]);
          packed[v / 2] = static_cast<uint32_t>(f32_to_bf16(h0)) |
                          (static_cast<uint32_t>(f32_to_bf16(h1)) << 16);
        }
        if constexpr (kDevH)
          __hip_atomic_store(reinterpret_cast<uint64_t*>(h + row * I + nb),
                             static_cast<uint64_t>(packed[0]) | (static_cast<uint64_t>(packed[1]) << 32),
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else
          *reinterpret_cast<uint2*>(h + row * I + nb) = uint2{packed[0], packed[1]};
      }
    }
  }
}

// Grid: x = row block b, y = group of 16 RC channels.
template <typename WT, int NS, int P, int RC = 1>
__global__ __launch_bounds__(kDmaThreads) void ffn13_dma_kernel(
    const bf16_t* __restrict__ x, const WT* __restrict__ w13, const float* __restrict__ s13,
    int scale_mode, const int32_t* __restrict__ sorted_ids,
    const int32_t* __restrict__ block_expert, const int32_t* __restrict__ num_padded,
    bf16_t* __restrict__ h, int d, int I, int k, int A) {
  using G = DmaGeom<WT, 2 * RC, NS>;
  DMA_RING(ring, G::kStageBytes, P);
  const int b = blockIdx.x;
  if (b * 16 * NS >= *num_padded) return;
  dma13_tile<WT, NS, P, RC>(x, w13, s13, scale_mode, sorted_ids, block_expert, h, d, I, k, A, b,
                            blockIdx.y * 16 * RC, ring);
}

// ------------------------------------------------------------ W2 + gate scale
// One tile: row block b, 16 RN channels of d from n0, split z of K = I.
// Writes y_part[z, f, n] = gate_f * s(n) * sum_{i in split} W2[e, n, i] h[row, i]
// for the block's real slots f.  RN tiles per wave: every wave reads all h
// rows of its block, so wider waves read less h per weight byte.

// Device-scope store of four floats: agent-scope atomic stores, which the
// gfx950 memory model issues with the device-coherence bit (sc1) so they
// write through this XCD's L2; readers on other XCDs use agent-scope atomic
// loads.
__device__ __forceinline__ void store_device4(float* p, const float4& o) {
  __hip_atomic_store(p + 0, o.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(p + 1, o.y, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(p + 2, o.z, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(p + 3, o.w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// kDevice: partials written with store_device4 (for a reader in the same
// launch on another XCD) instead of plain stores.
// kDevH: h rows written in this launch (device-scope token loads).
template <typename WT, int NS, int P, int RN, bool kDevice = false, bool kDevH = false>
__device__ __forceinline__ void dma2_tile(
    const bf16_t* __restrict__ h, const WT* __restrict__ w2, const float* __restrict__ s2,
    int scale_mode, const float* __restrict__ topk_w, const int32_t* __restrict__ sorted_ids,
    const int32_t* __restrict__ block_expert, float* __restrict__ y_part, int d, int I, int A,
    int ksplit, int b, int n0, int z, uint8_t* const (&ring)[4]) {
  constexpr int B = 16 * NS;
  const int e = block_expert[b];
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
    op.tlive[s] = blk[slot] < A;
  }

  f32x4 acc[NS][RN];
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int rt = 0; rt < RN; ++rt) acc[s][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (nch > 0) dma_dot<WT, RN, NS, P, kDevH>(nsub, op, ring, k_begin, nch, acc);

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
          if constexpr (kDevice)
            store_device4(yrow + nb, o);
          else
            *reinterpret_cast<float4*>(yrow + nb) = o;
        }
      }
    }
  }
}

// Grid: x = row block b, y = group of 16 RN channels of d, z = split of K = I.
template <typename WT, int NS, int P, int RN>
__global__ __launch_bounds__(kDmaThreads) void ffn2_dma_kernel(
    const bf16_t* __restrict__ h, const WT* __restrict__ w2, const float* __restrict__ s2,
    int scale_mode, const float* __restrict__ topk_w, const int32_t* __restrict__ sorted_ids,
    const int32_t* __restrict__ block_expert, const int32_t* __restrict__ num_padded,
    float* __restrict__ y_part, int d, int I, int A, int ksplit) {
  using G = DmaGeom<WT, RN, NS>;
  DMA_RING(ring, G::kStageBytes, P);
  const int b = blockIdx.x;
  if (b * 16 * NS >= *num_padded) return;
  dma2_tile<WT, NS, P, RN>(h, w2, s2, scale_mode, topk_w, sorted_ids, block_expert, y_part, d,
                           I, A, ksplit, b, blockIdx.y * 16 * RN, blockIdx.z, ring);
}

// ------------------------------------------------------------ combine in the W2 launch
// The combine's sum for one token and one group of 16 RN channels: every
// slot of the token, each slot's K splits in order (the order of
// combine_kernel, so the bits are the same), rounded to bf16 once.

__device__ __forceinline__ void store_bf16x4(bf16_t* p, float4 v) {
  const uint32_t lo = f32_to_bf16(v.x) | (static_cast<uint32_t>(f32_to_bf16(v.y)) << 16);
  const uint32_t hi = f32_to_bf16(v.z) | (static_cast<uint32_t>(f32_to_bf16(v.w)) << 16);
  *reinterpret_cast<uint2*>(p) = uint2{lo, hi};
}

// kDevice: the partials were written with store_device4 and are read with
// agent-scope atomic loads; else the caller has made them visible (an
// acquire fence after the writers' release) and plain loads read them.
template <bool kDevice>
__device__ __forceinline__ float4 load_partial4(const float* p) {
  if constexpr (kDevice)
    return float4{__hip_atomic_load(p + 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                  __hip_atomic_load(p + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                  __hip_atomic_load(p + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                  __hip_atomic_load(p + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)};
  else
    return *reinterpret_cast<const float4*>(p);
}

// After a W2 tile (row block `blk`, channel group dt of nd, 16 RN channels)
// has written its partials: one arrival per real slot on the counter of the
// slot's (token, channel group); the wave whose arrival is a counter's
// k * splits-th adds up that token's partials and writes its 16 RN outputs.
// The caller makes the tile's partials visible to other workgroups before
// this counts its arrivals.
template <int NS, int RN, bool kDevice>
__device__ __forceinline__ void arrive_and_combine(const int32_t* blk, int32_t* arrive,
                                                   const float* y_part, bf16_t* out, int A, int k,
                                                   int splits, int d, int nd, int dt) {
  const int lane = threadIdx.x & 63;
  const int total = k * splits;
  uint64_t last = 0;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    int mine = 0;
    if (lane < 16) {
      const int f = blk[16 * s + lane];
      if (f < A) {
        const int prev = __hip_atomic_fetch_add(arrive + (f / k) * nd + dt, 1, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
        mine = prev == total - 1;
      }
    }
    last |= static_cast<uint64_t>(__ballot(mine)) << (16 * s);
  }
  if (last == 0) return;
  if constexpr (kDevice)
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");  // loads stay after the counters
  else
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // the other tiles' partials
  constexpr int kGroups = 4 * RN;  // float4 groups of the 16 RN channels
  while (last) {
    const int bit = __builtin_ctzll(last);
    last &= last - 1;
    const int tok = blk[16 * (bit / 16) + bit % 16] / k;
    if (lane < kGroups) {
      const int c = dt * 16 * RN + 4 * lane;
      float4 o = {0.f, 0.f, 0.f, 0.f};
      for (int j = 0; j < k; ++j) {
        const size_t f = static_cast<size_t>(tok) * k + j;
        float4 sj = {0.f, 0.f, 0.f, 0.f};
        // kBatch splits' loads in flight before their adds (each load is a
        // round trip past the L2), added in split order
        constexpr int kBatch = 8;
        for (int z0 = 0; z0 < splits; z0 += kBatch) {
          float4 q[kBatch];
#pragma unroll
          for (int u = 0; u < kBatch; ++u)
            if (z0 + u < splits)
              q[u] = load_partial4<kDevice>(y_part + (static_cast<size_t>(z0 + u) * A + f) * d + c);
#pragma unroll
          for (int u = 0; u < kBatch; ++u) {
            if (z0 + u < splits) {
              sj.x += q[u].x;
              sj.y += q[u].y;
              sj.z += q[u].z;
              sj.w += q[u].w;
            }
          }
        }
        o.x += sj.x;
        o.y += sj.y;
        o.z += sj.z;
        o.w += sj.w;
      }
      store_bf16x4(out + static_cast<size_t>(tok) * d + c, o);
    }
  }
}

// W2 + gate scale and the combine in one launch (grid as ffn2_dma_kernel).
// Each tile writes its partials with device-scope stores, waits until they
// are acknowledged (s_waitcnt vmcnt(0): on gfx950 a store's count drops once
// it is visible at its scope), then counts its arrivals; the last tile for a
// token's channel group reads the partials with device-scope loads.  So no
// tile writes back or invalidates an L2 (the agent-scope fences would), and
// the combine launch and its re-read of the partials are gone.  The counters
// (arrive[T][d / (16 RN)]) start at zero: the routing launch clears them.
template <typename WT, int NS, int P, int RN>
__global__ __launch_bounds__(kDmaThreads) void ffn2_combine_dma_kernel(
    const bf16_t* __restrict__ h, const WT* __restrict__ w2, const float* __restrict__ s2,
    int scale_mode, const float* __restrict__ topk_w, const int32_t* __restrict__ sorted_ids,
    const int32_t* __restrict__ block_expert, const int32_t* __restrict__ num_padded,
    float* __restrict__ y_part, int d, int I, int A, int ksplit, int k, int splits,
    int32_t* __restrict__ arrive, bf16_t* __restrict__ out) {
  using G = DmaGeom<WT, RN, NS>;
  DMA_RING(ring, G::kStageBytes, P);
  const int b = blockIdx.x;
  if (b * 16 * NS >= *num_padded) return;
  dma2_tile<WT, NS, P, RN, true>(h, w2, s2, scale_mode, topk_w, sorted_ids, block_expert, y_part,
                                 d, I, A, ksplit, b, blockIdx.y * 16 * RN, blockIdx.z, ring);
  // the compiler keeps the counters after the stores; the wait makes the
  // stores complete first
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  arrive_and_combine<NS, RN, true>(sorted_ids + static_cast<size_t>(b) * 16 * NS, arrive, y_part,
                                   out, A, k, splits, d, gridDim.y, blockIdx.y);
}

// ------------------------------------------------------------ fused W13 -> W2 -> combine
// The decode path's expert computation as one persistent launch (the pages'
// "one batched GPU operation": routing, regrouping and the experts' work
// fused; Hungarian page, section "A fused MoE ...").  Workgroups take tiles
// from one monotone ticket counter: first every W13 tile (ordered channel
// tile by channel tile, so the h columns fill up in K order), then every W2
// tile (split by split).  A W2 tile waits until the W13 tiles of its block
// and K range have counted themselves done; every W13 ticket precedes every
// W2 ticket and W13 tiles wait for nothing, so a waiting workgroup only ever
// waits on work a running workgroup already holds (no deadlock, whatever
// the grid size).  The wait is bounded: after MOE_FUSED_SPIN_LIMIT polls a
// tile sets a flag in the counter words and writes NaN partials, so that a
// timeout shows in the output instead of hanging or passing unnoticed.  The
// combine is fused: after a W2 tile writes its partials it
// counts one arrival per real slot on the slot's (token, channel group); the
// tile that brings a counter to k * splits adds that token's partials, slots
// then splits in the same fixed order as the combine kernel, and writes the
// output, so the result is bit-identical to the three separate launches.
// Cross-workgroup data (h, the partials) goes out with agent-scope atomic
// stores, which write through this XCD's L2 (the GPU's L2s are per XCD),
// and is read with agent-scope atomic loads, which do not take another
// XCD's stale copy; a writer waits for its stores to complete before it
// counts, a reader reads after the count.  So no tile writes back or
// invalidates an L2, which an agent-scope fence would (once per tile).
// Counters are zeroed by the routing launch.

// Counter words: ticket, timeout flag, done13[blocks][splits], arrive[T][d / (16 RN)].
constexpr int kFusedTicket = 0;
constexpr int kFusedTimeout = 32;
constexpr int kFusedDone = 64;
#ifndef MOE_FUSED_SPIN_LIMIT
#define MOE_FUSED_SPIN_LIMIT (1 << 20)
#endif

static int fused_counter_words(int T, int cap, int B, int splits, int d, int rn) {
  return kFusedDone + (cap / B) * splits + T * (d / (16 * rn));
}

struct FusedParams {
  const bf16_t* x;
  const void* w13;
  const void* w2;
  const float* s13;
  const float* s2;
  int scale_mode;
  const float* topk_w;
  const int32_t* sorted_ids;
  const int32_t* block_expert;
  const int32_t* num_padded;
  bf16_t* h;
  float* y_part;
  bf16_t* out;
  int32_t* cnt;
  int T, d, I, k, A, cap, splits, ksplit;
};

template <typename WT, int NS, int P13, int P2, int RN>
__global__ __launch_bounds__(kDmaThreads) void ffn_fused_dma_kernel(FusedParams p) {
  constexpr int B = 16 * NS;
  constexpr int kS13 = DmaGeom<WT, 2, NS>::kStageBytes;
  constexpr int kS2 = DmaGeom<WT, RN, NS>::kStageBytes;
  constexpr int kStage = kS13 > kS2 ? kS13 : kS2;
  constexpr int P = P13 > P2 ? P13 : P2;
  DMA_RING(ring, kStage, P);
  const int lane = threadIdx.x;
  const int nblk = *p.num_padded / B;
  const int n13 = nblk * (p.I / 16);
  const int nd = p.d / (16 * RN);
  const int n2 = nblk * nd * p.splits;
  int32_t* const done13 = p.cnt + kFusedDone;
  int32_t* const arrive = done13 + (p.cap / B) * p.splits;
  const WT* w13 = static_cast<const WT*>(p.w13);
  const WT* w2 = static_cast<const WT*>(p.w2);

  // Every branch of this loop is wave-uniform (tickets and counters go
  // through readfirstlane; the one-lane atomics are issued by every lane
  // with 0 added by all but lane 0): lane-divergent branches that skip to
  // the next iteration let the compiler restructure the loop so that some
  // lanes re-entered it without lane 0 and never took a new ticket.
  for (;;) {
    const int t = __builtin_amdgcn_readfirstlane(__hip_atomic_fetch_add(
        p.cnt + kFusedTicket, lane == 0 ? 1 : 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    if (t >= n13 + n2) break;
    if (t < n13) {
      const int y = t / nblk;
      const int b = t - y * nblk;
      dma13_tile<WT, NS, P13, 1, true>(p.x, w13, p.s13, p.scale_mode, p.sorted_ids,
                                       p.block_expert, p.h, p.d, p.I, p.k, p.A, b, 16 * y, ring);
      // h went out with device-scope stores: once they have completed, the
      // count may publish them (no L2 write-back needed)
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __hip_atomic_fetch_add(done13 + b * p.splits + (16 * y) / p.ksplit, lane == 0 ? 1 : 0,
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      const int t2 = t - n13;
      const int z = t2 / (nblk * nd);
      const int r = t2 - z * (nblk * nd);
      const int dt = r / nblk;
      const int b = r - dt * nblk;
      const int kb = z * p.ksplit;
      const int need = (min(p.I, kb + p.ksplit) - kb) / 16;
      // bounded wait for the W13 tiles of this block's K range
      bool timed_out = false;  // wave-uniform: the count is broadcast from lane 0
      for (int spin = 0;; ++spin) {
        const int got = __builtin_amdgcn_readfirstlane(__hip_atomic_load(
            done13 + b * p.splits + z, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        if (got >= need) break;
        if (spin >= MOE_FUSED_SPIN_LIMIT) {
          __hip_atomic_store(p.cnt + kFusedTimeout, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          timed_out = true;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
      // h is read with device-scope loads, the partials written with
      // device-scope stores: no L2 invalidation or write-back
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");  // loads stay after the count
      dma2_tile<WT, NS, P2, RN, true, true>(p.h, w2, p.s2, p.scale_mode, p.topk_w, p.sorted_ids,
                                            p.block_expert, p.y_part, p.d, p.I, p.A, p.ksplit, b,
                                            dt * 16 * RN, z, ring);
      if (timed_out) {  // h may not be complete: make the tile's outputs NaN, not plausible
        const int32_t* blk = p.sorted_ids + static_cast<size_t>(b) * B;
        const float nan = __builtin_nanf("");
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const int f = blk[16 * s + (lane & 15)];
          if (f < p.A) {
#pragma unroll
            for (int rt = 0; rt < RN; ++rt)
              store_device4(p.y_part + (static_cast<size_t>(z) * p.A + f) * p.d + dt * 16 * RN +
                                16 * rt + 4 * (lane >> 4),
                            float4{nan, nan, nan, nan});
          }
        }
      }
      // this tile's partials have completed before it counts them
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      arrive_and_combine<NS, RN, true>(p.sorted_ids + static_cast<size_t>(b) * B, arrive,
                                       p.y_part, p.out, p.A, p.k, p.splits, p.d, nd, dt);
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
// Channel tiles per W13 wave for blocks of 32 (each tile: 16 gate + 16 up
// rows): two halve the token-fragment reads per weight byte (the block's
// two token subtiles are read once for 32 channels instead of 16).
// Measured at d = 4096, I = 14336: T = 64 313 -> 305 us, T = 32 level; with
// a three-stage ring (96 KB of LDS, one workgroup per CU) 384 us.
#ifndef MOE_DMA13_RC2
#define MOE_DMA13_RC2 2
#endif
#ifndef MOE_DMA_FP8_RN2
#define MOE_DMA_FP8_RN2 2
#endif
constexpr int kDma2RN = MOE_DMA2_RN;
constexpr int kDma2RNFp8 = MOE_DMA_FP8_RN2;

// The bf16 W2 when blocks of 16 give at most two row blocks (a single token
// of a top-2 layer; these are the blocks W2 with the combine runs on): two
// channel tiles per wave with a two-stage ring, 32 KB of LDS per workgroup,
// so that five workgroups fit on a CU and the 1024 tiles of four K splits
// are all resident at once.  Measured at d = 4096, I = 14336 (W2 with the
// combine): 40.9 us, against 42.5 with four channel tiles and a two-stage
// ring (two workgroups per CU), 50.4 with two tiles and a three-stage ring
// (three per CU, 1.3 rounds), and 50 before the combine was folded in.
#ifndef MOE_DMA2_WIDE_RN
#define MOE_DMA2_WIDE_RN 2
#endif
#ifndef MOE_DMA2_WIDE_P
#define MOE_DMA2_WIDE_P 2
#endif
constexpr int kDma2WideRN = MOE_DMA2_WIDE_RN;
constexpr int kDma2WideP = MOE_DMA2_WIDE_P;
constexpr int64_t kDma2WideBlocks = 2;

#ifndef MOE_DMA2_RN32
#define MOE_DMA2_RN32 2
#endif
constexpr int kDma2RN32 = MOE_DMA2_RN32;  // channel tiles per W2 wave, blocks of 32

static int dma_w2_rn(int w_dtype, int B, int64_t blocks_est) {
  if (w_dtype == kDtypeE4M3FN) return kDma2RNFp8;
  if (B == 32) return kDma2RN32;
  return B == 16 && blocks_est <= kDma2WideBlocks ? kDma2WideRN : kDma2RN;
}

int dma_w2_channels(int w_dtype, int B, int64_t blocks_est) {
  return 16 * dma_w2_rn(w_dtype, B, blocks_est);
}

namespace {

template <typename WT, int NS, int P, int RC = 1>
hipError_t ffn13_dma_go(const FfnArgs& a, hipStream_t s) {
  if (a.I % (16 * RC) != 0) return hipErrorInvalidValue;
  const dim3 grid(a.cap / a.B, a.I / (16 * RC));
  ffn13_dma_kernel<WT, NS, P, RC><<<grid, kDmaThreads, 0, s>>>(
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

template <typename WT, int NS, int P, int RN = sizeof(WT) == 1 ? kDma2RNFp8 : kDma2RN>
hipError_t ffn2_combine_dma_go(const FfnArgs& a, hipStream_t s) {
  const dim3 grid(a.cap / a.B, a.d / (16 * RN), a.splits);
  ffn2_combine_dma_kernel<WT, NS, P, RN><<<grid, kDmaThreads, 0, s>>>(
      static_cast<const bf16_t*>(a.h), static_cast<const WT*>(a.w2), a.s2, a.scale_mode,
      a.topk_w, a.sorted_ids, a.block_expert, a.num_padded, a.y_part, a.d, a.I, a.A, a.ksplit,
      a.k, a.splits, a.combine_cnt, static_cast<bf16_t*>(a.out));
  return hipGetLastError();
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
    case 32:
      return a.I % (16 * MOE_DMA13_RC2) == 0 ? ffn13_dma_go<bf16_t, 2, MOE_DMA13_P2, MOE_DMA13_RC2>(a, s)
                                             : ffn13_dma_go<bf16_t, 2, MOE_DMA13_P2>(a, s);
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
      if (ffn_blocks_estimate(a.cap, a.B, a.E, a.A) <= kDma2WideBlocks)
        return ffn2_dma_go<bf16_t, 1, kDma2WideP, kDma2WideRN>(a, s);
      return ffn2_dma_go<bf16_t, 1, MOE_DMA2_P1>(a, s);
    case 32: return ffn2_dma_go<bf16_t, 2, MOE_DMA2_P2, kDma2RN32>(a, s);
  }
  return hipErrorInvalidValue;
}

// Each tile of the W2 + combine kernel waits for its partials to be
// acknowledged before it counts them, and the counting and the last tile's
// combine add latency to every tile: it pays only where the W2 grid is one
// round of the chip and the combine launch is a large share of the layer,
// a single token of a top-2 bf16 layer (d = 4096, I = 14336: 137.2 ->
// 134.7 us per forward).  With more tiles it loses (T = 8: 453 against 451;
// T = 64: 556 against 504; e4m3fn weights at T = 1: 94.6 against 90.6 us;
// T = 64: 1.95 against 1.61 ms).
bool ffn2_combine_pays(int w_dtype, int B, int64_t blocks_est) {
  return w_dtype == kDtypeBF16 && B == 16 && blocks_est <= kDma2WideBlocks;
}

int ffn2_combine_ints(const FfnArgs& a) {
  return a.T * (a.d / dma_w2_channels(a.w_dtype, a.B, ffn_blocks_estimate(a.cap, a.B, a.E, a.A)));
}

hipError_t launch_ffn2_combine_dma(const FfnArgs& a, hipStream_t s) {
  const int64_t blocks = ffn_blocks_estimate(a.cap, a.B, a.E, a.A);
  // the one instantiation: blocks of 16 (one token subtile), the single-token
  // geometry (kDma2WideRN channel tiles, a kDma2WideP-stage ring)
  if (!a.combine_cnt || a.B != 16 || !dma_args_ok(a) || !dma_stream_use(a) ||
      !ffn2_combine_pays(a.w_dtype, a.B, blocks) || a.ksplit % dma_stream_kc(a.w_dtype) != 0 ||
      a.d % dma_w2_channels(a.w_dtype, a.B, blocks) != 0)
    return hipErrorInvalidValue;
  return ffn2_combine_dma_go<bf16_t, 1, kDma2WideP, kDma2WideRN>(a, s);
}

// ------------------------------------------------------------ fused launcher

// W2 channel tiles per wave in the fused kernel: two.  Its ring is sized
// for the larger of the two phases' stages, so four W2 tiles (the W2
// launch's choice for a single token) would double the W13 phase's LDS per
// workgroup and leave two workgroups per CU instead of five: measured at
// one token (d = 4096, I = 14336), the W13 phase then streamed at about
// half the W13 launch's rate.
constexpr int kFusedRN = 2;

bool fused_decode_fits(int w_dtype, int act_dtype, int B, int d, int I, int64_t blocks_est) {
#ifdef MOE_NO_FUSED_DECODE
  return false;
#else
  return w_dtype == kDtypeBF16 && act_dtype == kDtypeBF16 &&
         dma_stream_use(w_dtype, act_dtype, B, d, I, blocks_est) && d % (16 * kFusedRN) == 0;
#endif
}

int fused_counter_ints(const FfnArgs& a) {
  return fused_counter_words(a.T, a.cap, a.B, a.splits, a.d, kFusedRN);
}

namespace {

// Workgroups of kernel K the chip holds at once (occupancy x compute units),
// asked of the runtime once per kernel; 0 when it cannot say.
template <auto K>
int fused_resident(int threads) {
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

template <int NS, int P13, int P2, int RN>
hipError_t ffn_fused_go(const FfnArgs& a, hipStream_t s) {
  FusedParams p{};
  p.x = static_cast<const bf16_t*>(a.x);
  p.w13 = a.w13;
  p.w2 = a.w2;
  p.s13 = a.s13;
  p.s2 = a.s2;
  p.scale_mode = a.scale_mode;
  p.topk_w = a.topk_w;
  p.sorted_ids = a.sorted_ids;
  p.block_expert = a.block_expert;
  p.num_padded = a.num_padded;
  p.h = static_cast<bf16_t*>(a.h);
  p.y_part = a.y_part;
  p.out = static_cast<bf16_t*>(a.out);
  p.cnt = a.fused_cnt;
  p.T = a.T;
  p.d = a.d;
  p.I = a.I;
  p.k = a.k;
  p.A = a.A;
  p.cap = a.cap;
  p.splits = a.splits;
  p.ksplit = a.ksplit;
  constexpr auto kern = ffn_fused_dma_kernel<bf16_t, NS, P13, P2, RN>;
  // at most one workgroup per possible tile of the capacity's blocks
  const int64_t blocks = a.cap / a.B;
  const int64_t tiles = blocks * (a.I / 16 + (a.d / (16 * RN)) * a.splits);
  const int res = fused_resident<kern>(kDmaThreads);
  const int grid = static_cast<int>(res > 0 && res < tiles ? res : tiles);
  kern<<<grid, kDmaThreads, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ffn_fused(const FfnArgs& a, hipStream_t s) {
  const int64_t blocks = ffn_blocks_estimate(a.cap, a.B, a.E, a.A);
  if (!a.fused_cnt || !fused_decode_fits(a.w_dtype, a.act_dtype, a.B, a.d, a.I, blocks) ||
      a.ksplit % 16 != 0 || a.ksplit % dma_stream_kc(a.w_dtype) != 0)
    return hipErrorInvalidValue;
  static_assert(kDma2RN == kFusedRN && kDma2RN32 == kFusedRN,
                "the fused kernel's W2 tiles match the W2 launch's for blocks of 16 and 32");
  switch (a.B) {
    case 16:
      // at most two row blocks (one token): the W13 launch's two-stage ring
      if (blocks <= kDma2WideBlocks) return ffn_fused_go<1, 2, kDma2WideP, kFusedRN>(a, s);
      return ffn_fused_go<1, MOE_DMA13_P1, MOE_DMA2_P1, kFusedRN>(a, s);
    case 32: return ffn_fused_go<2, MOE_DMA13_P2, MOE_DMA2_P2, kFusedRN>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
