// Expert-side kernels of the fused MoE layer: the grouped W13 product with
// SiLU(gate) * up fused in its epilogue, the grouped W2 product scaled by the
// slot's gate, and the combine of each token's slots.
//
// Sources: the Hungarian news page "Az AWS új MoE-optimalizációkkal
// gyorsítja a SageMaker AI-t", section "A fused MoE a számítási folyamat több
// lépését egyesíti" (expert computation as one batched operation over all
// experts) and section "FP8 esetén a Triton backend bizonyult gyorsabbnak"
// (FP8 scaling, matrix product and aggregation of the experts' results done
// in registers after one read from HBM, without intermediate round trips);
// the French page "Ingénierie de kernels Mixture-of-Experts sur Amazon
// SageMaker AI", second paragraph (decode: M = tokens is tiny, the expert
// weight block is large) and the Hungarian page's section "A mátrixok
// felcserélése jobban kihasználja a Hopper GPU-kat" (swap the operands so
// the large expert dimension fills the matrix unit's fixed M side).
//
// CDNA4 design.  Every product is computed transposed, out^T = W . X^T: the
// expert's weight rows (output channels) sit on the 16-row M side of
// v_mfma_f32_16x16x32_bf16 and the block's tokens on its N side, 16 per
// sub-tile.  Weights are read straight from HBM into registers -- each
// weight element is used by exactly one wave, so LDS staging would only add
// traffic -- and every wave reuses its weight fragments for all token
// sub-tiles of its block, so an expert's weights are streamed once per
// block.  e4m3fn weights are widened to bf16 in registers (exact) and their
// fp32 scale is applied once per output channel in the epilogue.
//
// The K layout of the operand loads is described in ffn_common.h.

#include <algorithm>

#include "ffn_common.h"

namespace moe {

constexpr int kFfnThreads = 64;  // one wave per workgroup: even spread over the CUs

// Tuning knobs (compile-time): weight chunks kept in flight per wave, and
// 16-channel tiles per wave.
#ifndef MOE_FFN13_PIPE
#define MOE_FFN13_PIPE 2
#endif
#ifndef MOE_FFN13_RN
#define MOE_FFN13_RN 2
#endif
#ifndef MOE_FFN2_PIPE
#define MOE_FFN2_PIPE 2
#endif
#ifndef MOE_FFN2_RN
#define MOE_FFN2_RN 2
#endif

// ------------------------------------------------------------ W13 + SiLU*mul
//
// Grid: x = row block b of the regrouped layout, y = group of 16 * RN output
// channels (one wave, RN 16-channel tiles).  Each wave computes, for
// its channels n, the gate rows n and the up rows I + n against every token
// of the block and writes h[row, n] = SiLU(s_g * gate) * (s_u * up) in bf16.

template <typename WT, int NSUB, int KC, int P, int RN>
__global__ __launch_bounds__(kFfnThreads) void ffn13_kernel(
    const bf16_t* __restrict__ x, const WT* __restrict__ w13, const float* __restrict__ s13,
    int scale_mode, const int32_t* __restrict__ sorted_ids,
    const int32_t* __restrict__ block_expert, const int32_t* __restrict__ num_padded,
    bf16_t* __restrict__ h, int d, int I, int k, int A, int B) {
  constexpr int NF = KC / 32;
  constexpr int NROW = 2 * RN;  // RN gate tiles then RN up tiles
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int b = blockIdx.x;
  if (b * B >= *num_padded) return;
  const int e = block_expert[b];
  const int n0 = blockIdx.y * 16 * RN;
  if (n0 >= I) return;
  const int32_t* blk = sorted_ids + static_cast<size_t>(b) * B;
  const int nsub = live_subtiles<NSUB>(blk, A);

  const bf16_t* xrow[NSUB];
  bool ok[NSUB];
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    const int f = s < nsub ? blk[16 * s + r16] : A;
    ok[s] = f < A;
    xrow[s] = x + static_cast<size_t>(ok[s] ? f / k : 0) * d;
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

  f32x4 acc[NSUB][NROW];
#pragma unroll
  for (int s = 0; s < NSUB; ++s)
#pragma unroll
    for (int r = 0; r < NROW; ++r) acc[s][r] = f32x4{0.f, 0.f, 0.f, 0.f};

  ws.start(0);
  for (int c0 = 0; c0 < ws.nch; c0 += P) {
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int c = c0 + p;
      if (c < ws.nch) {
        bf16x8 wf[NROW][NF];
        ws.take(p, c, 0, wf);
#pragma unroll
        for (int s = 0; s < NSUB; ++s) {
          if (s < nsub) {
            ActChunk<WT, KC> xs;
            if (ok[s])
              xs.load(xrow[s] + c * KC, g);
            else
              xs.zero();
#pragma unroll
            for (int i = 0; i < NF; ++i) {
              const bf16x8 xf = xs.frag(i);
#pragma unroll
              for (int r = 0; r < NROW; ++r) acc[s][r] = mfma16x16x32(wf[r][i], xf, acc[s][r]);
            }
          }
        }
      }
    }
  }

  // Epilogue: lane holds token column r16, channels n0 + rt*16 + 4g .. +3.
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
    for (int s = 0; s < NSUB; ++s) {
      if (s < nsub) {
        const size_t row = static_cast<size_t>(b) * B + 16 * s + r16;
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

// ------------------------------------------------------------ W2 + gate scale
//
// Grid: x = row block b, y = group of 16 * RN output channels of d (one
// wave), z = split of the K = I range.  Each wave owns RN tiles of 16 channels and
// writes y_part[z, f, n] = gate_f * s(n) * sum_{i in split} W2[e, n, i] h[r, i]
// for every real slot f of the block; the combine sums the splits in a
// fixed order, so the result is deterministic.

template <typename WT, int NSUB, int KC, int P, int RN>
__global__ __launch_bounds__(kFfnThreads) void ffn2_kernel(
    const bf16_t* __restrict__ h, const WT* __restrict__ w2, const float* __restrict__ s2,
    int scale_mode, const float* __restrict__ topk_w, const int32_t* __restrict__ sorted_ids,
    const int32_t* __restrict__ block_expert, const int32_t* __restrict__ num_padded,
    float* __restrict__ y_part, int d, int I, int A, int B, int ksplit) {
  constexpr int NF = KC / 32;
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int b = blockIdx.x;
  if (b * B >= *num_padded) return;
  const int e = block_expert[b];
  const int n0 = blockIdx.y * 16 * RN;
  if (n0 >= d) return;
  const int z = blockIdx.z;
  const int k_begin = z * ksplit;
  const int k_end = min(I, k_begin + ksplit);
  const int32_t* blk = sorted_ids + static_cast<size_t>(b) * B;
  const int nsub = live_subtiles<NSUB>(blk, A);

  const bf16_t* hrow[NSUB];
  bool ok[NSUB];  // pad rows hold zeros: skip their loads
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    ok[s] = s < nsub && blk[16 * s + r16] < A;
    hrow[s] = h + (static_cast<size_t>(b) * B + 16 * s + r16) * I;
  }
  WeightStream<WT, KC, RN, P> ws;
  ws.g = g;
  ws.nch = k_end > k_begin ? (k_end - k_begin) / KC : 0;
#pragma unroll
  for (int rt = 0; rt < RN; ++rt)
    ws.row[rt] = w2 + (static_cast<size_t>(e) * d + n0 + rt * 16 + r16) * I;

  f32x4 acc[NSUB][RN];
#pragma unroll
  for (int s = 0; s < NSUB; ++s)
#pragma unroll
    for (int rt = 0; rt < RN; ++rt) acc[s][rt] = f32x4{0.f, 0.f, 0.f, 0.f};

  ws.start(k_begin);
  for (int c0 = 0; c0 < ws.nch; c0 += P) {
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int c = c0 + p;
      if (c < ws.nch) {
        bf16x8 wf[RN][NF];
        ws.take(p, c, k_begin, wf);
#pragma unroll
        for (int s = 0; s < NSUB; ++s) {
          if (s < nsub) {
            ActChunk<WT, KC> hs;
            if (ok[s])
              hs.load(hrow[s] + k_begin + c * KC, g);
            else
              hs.zero();
#pragma unroll
            for (int i = 0; i < NF; ++i) {
              const bf16x8 hf = hs.frag(i);
#pragma unroll
              for (int rt = 0; rt < RN; ++rt) acc[s][rt] = mfma16x16x32(wf[rt][i], hf, acc[s][rt]);
            }
          }
        }
      }
    }
  }

#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    if (s < nsub) {
      const int f = blk[16 * s + r16];
      if (f < A) {
        const float gate = topk_w[f];
        float* yrow = y_part + (static_cast<size_t>(z) * A + f) * d;
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

// ------------------------------------------------------------ fp32 path
//
// fp32 activations and weights: one thread per (regrouped row, channel),
// fp32 fused multiply-adds.  Correctness path for fp32 models; the bf16 and
// e4m3fn paths above are the tuned ones.

__global__ __launch_bounds__(256) void ffn13_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ w13,
    const int32_t* __restrict__ sorted_ids, const int32_t* __restrict__ block_expert,
    const int32_t* __restrict__ num_padded, float* __restrict__ h, int d, int I, int k, int A,
    int B) {
  const int r = blockIdx.x;
  const int n = blockIdx.y * 256 + threadIdx.x;
  if (r >= *num_padded || n >= I) return;
  const int f = sorted_ids[r];
  float* hr = h + static_cast<size_t>(r) * I;
  if (f >= A) {
    hr[n] = 0.f;
    return;
  }
  const int e = block_expert[r / B];
  const float* xr = x + static_cast<size_t>(f / k) * d;
  const float* wgr = w13 + (static_cast<size_t>(e) * 2 * I + n) * d;
  const float* wur = w13 + (static_cast<size_t>(e) * 2 * I + I + n) * d;
  float gsum = 0.f, usum = 0.f;
  for (int i = 0; i < d; ++i) {
    gsum = fmaf(wgr[i], xr[i], gsum);
    usum = fmaf(wur[i], xr[i], usum);
  }
  hr[n] = silu(gsum) * usum;
}

__global__ __launch_bounds__(256) void ffn2_f32_kernel(
    const float* __restrict__ h, const float* __restrict__ w2, const float* __restrict__ topk_w,
    const int32_t* __restrict__ sorted_ids, const int32_t* __restrict__ block_expert,
    const int32_t* __restrict__ num_padded, float* __restrict__ y, int d, int I, int A, int B) {
  const int r = blockIdx.x;
  const int n = blockIdx.y * 256 + threadIdx.x;
  if (r >= *num_padded || n >= d) return;
  const int f = sorted_ids[r];
  if (f >= A) return;
  const int e = block_expert[r / B];
  const float* hr = h + static_cast<size_t>(r) * I;
  const float* wr = w2 + (static_cast<size_t>(e) * d + n) * I;
  float acc = 0.f;
  for (int i = 0; i < I; ++i) acc = fmaf(wr[i], hr[i], acc);
  y[static_cast<size_t>(f) * d + n] = acc * topk_w[f];
}

// ------------------------------------------------------------ combine
//
// out[t, n] = sum_j (sum_z y_part[z, t*k + j, n]) in rank order j, then
// rounded to the activation dtype (bf16: round to nearest even).

template <typename OT>
__device__ __forceinline__ void store4(OT* p, float4 v);

template <>
__device__ __forceinline__ void store4<float>(float* p, float4 v) {
  *reinterpret_cast<float4*>(p) = v;
}

template <>
__device__ __forceinline__ void store4<bf16_t>(bf16_t* p, float4 v) {
  const uint32_t lo = f32_to_bf16(v.x) | (static_cast<uint32_t>(f32_to_bf16(v.y)) << 16);
  const uint32_t hi = f32_to_bf16(v.z) | (static_cast<uint32_t>(f32_to_bf16(v.w)) << 16);
  *reinterpret_cast<uint2*>(p) = uint2{lo, hi};
}

#ifndef MOE_COMBINE_NT
#define MOE_COMBINE_NT 1
#endif

template <typename OT>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y_part,
                                                      OT* __restrict__ out, int T, int d, int k,
                                                      int splits, int A) {
  const int groups = d / 4;
  const size_t total = static_cast<size_t>(T) * groups;
  for (size_t idx = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; idx < total;
       idx += static_cast<size_t>(gridDim.x) * blockDim.x) {
    const int t = static_cast<int>(idx / groups);
    const int c = static_cast<int>(idx % groups) * 4;
    float4 o = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
      const size_t f = static_cast<size_t>(t) * k + j;
      float4 sj = {0.f, 0.f, 0.f, 0.f};
      for (int z = 0; z < splits; ++z) {
#if MOE_COMBINE_NT
        const f32x4 pv = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4*>(y_part + (static_cast<size_t>(z) * A + f) * d + c));
        const float4 p{pv[0], pv[1], pv[2], pv[3]};
#else
        const float4 p =
            *reinterpret_cast<const float4*>(y_part + (static_cast<size_t>(z) * A + f) * d + c);
#endif
        sj.x += p.x;
        sj.y += p.y;
        sj.z += p.z;
        sj.w += p.w;
      }
      o.x += sj.x;
      o.y += sj.y;
      o.z += sj.z;
      o.w += sj.w;
    }
    store4<OT>(out + static_cast<size_t>(t) * d + c, o);
  }
}

// ------------------------------------------------------------ launchers

// K chunk: 128 elements (four MFMA steps), or 64 when 128 does not divide
// the K dimension (K is a multiple of 64).  e4m3fn rows move half the bytes
// per chunk, so they keep one more chunk in flight.
template <typename WT>
int kchunk_for(int K) {
  return K % 128 == 0 ? 128 : 64;
}

int ffn2_kchunk(int d, int I, int B, int w_dtype, int act_dtype, int64_t blocks_est) {
  if (dma_stream_use(w_dtype, act_dtype, B, d, I, blocks_est)) return dma_stream_kc(w_dtype);
  return w_dtype == kDtypeE4M3FN ? kchunk_for<fp8_t>(I) : kchunk_for<bf16_t>(I);
}

namespace {

constexpr int kP13 = MOE_FFN13_PIPE, kRN13 = MOE_FFN13_RN;
constexpr int kP2 = MOE_FFN2_PIPE, kRN2 = MOE_FFN2_RN;

// Channel tiles per wave: two when that still leaves at least eight waves
// per CU (x loads are shared by twice the weight rows), else one (twice the
// waves, for small batches that touch few experts).
#ifndef MOE_RN2_MAX_NSUB
#define MOE_RN2_MAX_NSUB 4
#endif
inline int pick_rn(int blocks_est, int channels, int rn_max, int nsub) {
  return (rn_max >= 2 && nsub <= MOE_RN2_MAX_NSUB &&
          int64_t(blocks_est) * (channels / 32) >= 8 * 256) ? 2 : 1;
}

inline int blocks_estimate(const FfnArgs& a) {
  return static_cast<int>(ffn_blocks_estimate(a.cap, a.B, a.E, a.A));
}

template <typename WT, int NSUB, int KC, int RN>
void ffn13_launch(const FfnArgs& a, hipStream_t s) {
  constexpr int P = sizeof(WT) == 1 ? kP13 + 1 : kP13;
  dim3 grid(a.cap / a.B, a.I / (16 * RN));  // I is a multiple of 64: the tiles cover it
  ffn13_kernel<WT, NSUB, KC, P, RN><<<grid, kFfnThreads, 0, s>>>(
      static_cast<const bf16_t*>(a.x), static_cast<const WT*>(a.w13), a.s13, a.scale_mode,
      a.sorted_ids, a.block_expert, a.num_padded, static_cast<bf16_t*>(a.h), a.d, a.I, a.k, a.A,
      a.B);
}

template <typename WT, int NSUB, int KC>
void ffn13_go(const FfnArgs& a, hipStream_t s) {
  static_assert(kRN13 == 1 || kRN13 == 2, "channel tiles per wave: 1 or 2");
  if (pick_rn(blocks_estimate(a), a.I, kRN13, NSUB) == 2)
    ffn13_launch<WT, NSUB, KC, kRN13>(a, s);
  else
    ffn13_launch<WT, NSUB, KC, 1>(a, s);
}

template <typename WT, int NSUB>
hipError_t ffn13_nsub(const FfnArgs& a, hipStream_t s) {
  const int kc = kchunk_for<WT>(a.d);
  if (kc == 128) ffn13_go<WT, NSUB, 128>(a, s);
  else ffn13_go<WT, NSUB, 64>(a, s);
  return hipGetLastError();
}

template <typename WT>
hipError_t ffn13_w(const FfnArgs& a, hipStream_t s) {
  switch (a.B) {
    case 16: return ffn13_nsub<WT, 1>(a, s);
    case 32: return ffn13_nsub<WT, 2>(a, s);
    case 64: return ffn13_nsub<WT, 4>(a, s);
  }
  return hipErrorInvalidValue;
}

template <typename WT, int NSUB, int KC, int RN>
void ffn2_launch(const FfnArgs& a, hipStream_t s) {
  constexpr int P = sizeof(WT) == 1 ? kP2 + 1 : kP2;
  dim3 grid(a.cap / a.B, a.d / (16 * RN), a.splits);  // d is a multiple of 64
  ffn2_kernel<WT, NSUB, KC, P, RN><<<grid, kFfnThreads, 0, s>>>(
      static_cast<const bf16_t*>(a.h), static_cast<const WT*>(a.w2), a.s2, a.scale_mode,
      a.topk_w, a.sorted_ids, a.block_expert, a.num_padded, a.y_part, a.d, a.I, a.A, a.B,
      a.ksplit);
}

template <typename WT, int NSUB, int KC>
void ffn2_go(const FfnArgs& a, hipStream_t s) {
  static_assert(kRN2 == 1 || kRN2 == 2, "channel tiles per wave: 1 or 2");
  if (pick_rn(blocks_estimate(a) * a.splits, a.d, kRN2, NSUB) == 2)
    ffn2_launch<WT, NSUB, KC, kRN2>(a, s);
  else
    ffn2_launch<WT, NSUB, KC, 1>(a, s);
}

template <typename WT, int NSUB>
hipError_t ffn2_nsub(const FfnArgs& a, hipStream_t s) {
  const int kc = kchunk_for<WT>(a.I);
  if (kc == 128) ffn2_go<WT, NSUB, 128>(a, s);
  else ffn2_go<WT, NSUB, 64>(a, s);
  return hipGetLastError();
}

template <typename WT>
hipError_t ffn2_w(const FfnArgs& a, hipStream_t s) {
  switch (a.B) {
    case 16: return ffn2_nsub<WT, 1>(a, s);
    case 32: return ffn2_nsub<WT, 2>(a, s);
    case 64: return ffn2_nsub<WT, 4>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_ffn13(const FfnArgs& a, hipStream_t s) {
  if (a.w_dtype == kDtypeF32) {
    dim3 grid(a.cap, (a.I + 255) / 256);
    ffn13_f32_kernel<<<grid, 256, 0, s>>>(static_cast<const float*>(a.x),
                                          static_cast<const float*>(a.w13), a.sorted_ids,
                                          a.block_expert, a.num_padded,
                                          static_cast<float*>(a.h), a.d, a.I, a.k, a.A, a.B);
    return hipGetLastError();
  }
  if (a.act_mx) return launch_ffn13_big8(a, s);    // W8A8: block-scaled e4m3fn activations
  if (a.B == 256) return launch_ffn13_big(a, s);   // large-tile grouped GEMM
  if (wide_use(a)) return launch_ffn13_wide(a, s);  // 128-token tile, tokens in registers
  if (a.B == 128 && a.w_dtype == kDtypeE4M3FN && mid_gemm_fits(a.T, a.d, a.I))
    return launch_ffn13_mid(a, s);                 // 128-token tile, both operands via LDS
  if (a.B == 128) return launch_ffn13_gemm(a, s);  // token-tiled grouped GEMM
  if (dma_stream_use(a)) return launch_ffn13_dma(a, s);  // weights through LDS
  if (a.w_dtype == kDtypeBF16) return ffn13_w<bf16_t>(a, s);
  return ffn13_w<fp8_t>(a, s);
}

hipError_t launch_ffn2(const FfnArgs& a, hipStream_t s) {
  if (a.w_dtype == kDtypeF32) {
    dim3 grid(a.cap, (a.d + 255) / 256);
    ffn2_f32_kernel<<<grid, 256, 0, s>>>(static_cast<const float*>(a.h),
                                         static_cast<const float*>(a.w2), a.topk_w, a.sorted_ids,
                                         a.block_expert, a.num_padded, a.y_part, a.d, a.I, a.A,
                                         a.B);
    return hipGetLastError();
  }
  if (a.act_mx) return launch_ffn2_big8(a, s);
  if (a.B == 256) return launch_ffn2_big(a, s);
  if (wide_use(a)) return launch_ffn2_wide(a, s);
  if (a.B == 128 && a.w_dtype == kDtypeE4M3FN && mid_gemm_fits(a.T, a.d, a.I))
    return launch_ffn2_mid(a, s);
  if (a.B == 128) return launch_ffn2_gemm(a, s);
  if (dma_stream_use(a)) return launch_ffn2_dma(a, s);
  if (a.w_dtype == kDtypeBF16) return ffn2_w<bf16_t>(a, s);
  return ffn2_w<fp8_t>(a, s);
}

hipError_t launch_combine(const FfnArgs& a, hipStream_t s) {
  const size_t total = static_cast<size_t>(a.T) * (a.d / 4);
  const size_t want = (total + 255) / 256;
  const int blocks = static_cast<int>(want < 65536 ? want : 65536);
  if (a.act_dtype == kDtypeF32)
    combine_kernel<float><<<blocks, 256, 0, s>>>(a.y_part, static_cast<float*>(a.out), a.T, a.d,
                                                 a.k, a.splits, a.A);
  else
    combine_kernel<bf16_t><<<blocks, 256, 0, s>>>(a.y_part, static_cast<bf16_t*>(a.out), a.T,
                                                  a.d, a.k, a.splits, a.A);
  return hipGetLastError();
}

}  // namespace moe
