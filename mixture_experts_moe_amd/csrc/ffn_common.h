// Operand loaders shared by the expert kernels (weight streaming and the
// token-tiled grouped GEMM).
//
// K layout: within a K chunk of KC elements, one 16-byte load instruction
// covers, for each of the 16 rows of a tile, 64 contiguous bytes of that row
// (lane group g = lane/16 takes bytes 16g .. 16g+15).  For bf16 weights that
// is exactly one MFMA step (k = 32j + 8g .. +8, the operand's natural layout);
// for e4m3fn weights it is two steps (lane group g holds k = 64j + 16g .. +16
// and feeds the first eight to MFMA 2j, the last eight to MFMA 2j+1).  The
// bf16 token operand is loaded with the same k for every (lane, MFMA).
#pragma once

#include "common.h"
#include "kernels.h"

namespace moe {

// ------------------------------------------------------------ operand loads

template <typename WT, int KC>
struct RowChunk;  // one lane's part of one weight row's K chunk

template <int KC>
struct RowChunk<bf16_t, KC> {
  static constexpr int kLoads = KC / 32;  // 16-byte loads (8 bf16 each)
  uint4 v[kLoads];
  // load j: k = 32j + 8g .. +8 of the chunk (fragment j)
  __device__ __forceinline__ void load(const bf16_t* chunk, int g) {
#pragma unroll
    for (int j = 0; j < kLoads; ++j) v[j] = *reinterpret_cast<const uint4*>(chunk + 32 * j + 8 * g);
  }
  __device__ __forceinline__ bf16x8 frag(int i) const { return as_frag(v[i]); }
};

template <int KC>
struct RowChunk<fp8_t, KC> {
  static constexpr int kLoads = KC / 64;  // 16-byte loads (16 e4m3fn each)
  uint4 v[kLoads];
  // load j: k = 64j + 16g .. +16 of the chunk (fragments 2j and 2j+1)
  __device__ __forceinline__ void load(const fp8_t* chunk, int g) {
#pragma unroll
    for (int j = 0; j < kLoads; ++j) v[j] = *reinterpret_cast<const uint4*>(chunk + 64 * j + 16 * g);
  }
  __device__ __forceinline__ bf16x8 frag(int i) const {
    const uint4 q = v[i >> 1];
    const uint32_t lo = (i & 1) ? q.z : q.x;
    const uint32_t hi = (i & 1) ? q.w : q.y;
    return as_frag(e4m3x8_to_frag_bits(lo, hi));
  }
};

// The bf16 token operand of one K chunk, in the k layout of weight type WT.
template <typename WT, int KC>
struct ActChunk {
  static constexpr int kFrags = KC / 32;
  uint4 v[kFrags];
  static __device__ __forceinline__ int off(int i, int g) {
    return sizeof(WT) == 2 ? 32 * i + 8 * g : 64 * (i >> 1) + 16 * g + 8 * (i & 1);
  }
  __device__ __forceinline__ void load(const bf16_t* chunk, int g) {
#pragma unroll
    for (int i = 0; i < kFrags; ++i) v[i] = *reinterpret_cast<const uint4*>(chunk + off(i, g));
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < kFrags; ++i) v[i] = uint4{0, 0, 0, 0};
  }
  __device__ __forceinline__ bf16x8 frag(int i) const { return as_frag(v[i]); }
};

__device__ __forceinline__ float load_scale(const float* s, int mode, size_t matrix, size_t idx) {
  if (mode == kScaleChannel) return s[idx];
  if (mode == kScaleTensor) return s[matrix];
  return 1.0f;
}

// Number of leading 16-row sub-tiles of block `blk` that hold at least one
// real slot (valid slots form a prefix of every block).
template <int NSUB>
__device__ __forceinline__ int live_subtiles(const int32_t* blk, int A) {
  int n = 0;
#pragma unroll
  for (int s = 0; s < NSUB; ++s)
    if (blk[16 * s] < A) n = s + 1;
  return n;
}

// Weight rows of one wave, streamed in K chunks through a ring of P register
// buffers: chunk c is consumed from buffer c % P, which is then refilled with
// chunk c + P, so P chunks of loads stay in flight while the MFMAs run.
template <typename WT, int KC, int NROW, int P>
struct WeightStream {
  RowChunk<WT, KC> buf[P][NROW];
  const WT* row[NROW];
  int g, nch;

  __device__ __forceinline__ void start(int k_begin) {
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
      for (int r = 0; r < NROW; ++r) buf[p][r].load(row[r] + k_begin + min(p, nch - 1) * KC, g);
  }
  // fragments of chunk c (held in buffer p = c % P), then refill buffer p
  // with chunk c + P (clamped to the last chunk, which is then read twice:
  // branch-free, and the duplicate is never used).
  __device__ __forceinline__ void take(int p, int c, int k_begin, bf16x8 (&f)[NROW][KC / 32]) {
#pragma unroll
    for (int r = 0; r < NROW; ++r)
#pragma unroll
      for (int i = 0; i < KC / 32; ++i) f[r][i] = buf[p][r].frag(i);
    const int cn = min(c + P, nch - 1);
#pragma unroll
    for (int r = 0; r < NROW; ++r) buf[p][r].load(row[r] + k_begin + cn * KC, g);
  }
};

// One slot's four fp32 output channels into the W2 partials (y_part), which
// the combine reads once.  MOE_Y_NT: with the nontemporal hint.
#ifndef MOE_Y_NT
#define MOE_Y_NT 0
#endif
__device__ __forceinline__ void store_partial4(float* p, float a, float b, float c, float d) {
#if MOE_Y_NT
  __builtin_nontemporal_store(f32x4{a, b, c, d}, reinterpret_cast<f32x4*>(p));
#else
  *reinterpret_cast<float4*>(p) = float4{a, b, c, d};
#endif
}

}  // namespace moe
