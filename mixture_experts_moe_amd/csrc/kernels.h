// Internal launchers of the fused MoE kernels (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Mirrors of the ABI dtype / scale codes (moe.h), for device code.
constexpr int kDtypeF32 = 0;
constexpr int kDtypeBF16 = 1;
constexpr int kDtypeE4M3FN = 2;
constexpr int kScaleNone = 0;
constexpr int kScaleTensor = 1;
constexpr int kScaleChannel = 2;

constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 64;

hipError_t launch_router_logits(const void* x, int act_dtype, const float* wg, float* logits,
                                int T, int E, int d, hipStream_t s);
hipError_t launch_router_topk(const float* logits, int32_t* ids, float* w, int T, int E, int k,
                              hipStream_t s);
// bf16 activations, T <= 64, E <= 16: logits and selection in one kernel.
bool router_fused(int act_dtype, int T, int E);
hipError_t launch_router_fused(const void* x, const float* wg, float* logits, int32_t* ids,
                               float* w, int T, int E, int d, int k, hipStream_t s);
// bf16 activations, E <= 16, any T whose logits launch_router_logits runs
// on the 16-token tiles: launch_router_fused's kernel gives the same logits
// and also selects (one launch instead of two).
bool router_selects(int act_dtype, int T, int E);
// bf16 activations, 1 <= T <= 16, E <= 16: logits, selection and the
// regrouping (same outputs as launch_align) in one single-workgroup kernel.
bool route_align_fused(int act_dtype, int T, int E);
hipError_t launch_route_align_fused(const void* x, const float* wg, float* logits, int32_t* ids,
                                    float* w, int T, int E, int d, int k, int B, int cap,
                                    int32_t* counts, int32_t* sorted_ids, int32_t* block_expert,
                                    int32_t* num_padded, hipStream_t s);
// The same two operations with K split over 16 one-wave workgroups and a
// second launch that adds their partials in the fused kernel's order (same
// results, bit for bit); `part` is router_split_bytes(T, E) of scratch.
size_t router_split_bytes(int T, int E);
// `zero`: nzero int32 words the partial launch sets to 0 (counters of the
// fused expert kernel that follows in the layer path), or none.
hipError_t launch_router_fused_split(const void* x, const float* wg, float* logits, int32_t* ids,
                                     float* w, int T, int E, int d, int k, void* part,
                                     hipStream_t s, int32_t* zero = nullptr, int nzero = 0);
hipError_t launch_route_align_fused_split(const void* x, const float* wg, float* logits,
                                          int32_t* ids, float* w, int T, int E, int d, int k,
                                          int B, int cap, int32_t* counts, int32_t* sorted_ids,
                                          int32_t* block_expert, int32_t* num_padded, void* part,
                                          hipStream_t s, int32_t* zero = nullptr, int nzero = 0);
// bf16 activations, 1 <= T <= 64, any E: the logits alone, K split the same
// way (16 one-wave workgroups per tile, then a sum in slice order: the same
// bits as launch_router_logits); `part` is router_split_bytes(T, E).
bool router_split_logits(int act_dtype, int T, int E);
hipError_t launch_router_split_logits(const void* x, const float* wg, float* logits, int T, int E,
                                      int d, void* part, hipStream_t s, int32_t* zero = nullptr,
                                      int nzero = 0);
// bf16 activations where the wide 64-token tiles would run (many tokens and
// experts), d % 256 == 0: the same logits, bit for bit, through an
// LDS-staged 128-token x 64-expert tile per K quarter, then one launch that
// adds the quarters and selects (the same ids and gates as
// launch_router_topk); `part` is router_lds_bytes(T, E) of scratch.
bool router_lds_logits(int act_dtype, int T, int E, int d);
size_t router_lds_bytes(int T, int E);
hipError_t launch_router_lds_topk(const void* x, const float* wg, float* logits, int32_t* ids,
                                  float* w, int T, int E, int d, int k, void* part, hipStream_t s);
// `zero`: nzero int32 that the launch also sets to 0 (the expert kernels'
// work-queue counters when the layer runs align right before them).
hipError_t launch_align(const int32_t* ids, int A, int E, int B, int cap, int32_t* counts,
                        int32_t* sorted_ids, int32_t* block_expert, int32_t* num_padded,
                        hipStream_t s, int32_t* zero = nullptr, int nzero = 0);

// Everything the expert-side kernels need for one call.
struct FfnArgs {
  const void* x;            // [T, d] act dtype
  const void* w13;          // [E, 2I, d]
  const void* w2;           // [E, d, I]
  const float* s13;         // scales or nullptr
  const float* s2;
  int scale_mode;
  int act_dtype;
  int w_dtype;
  const float* topk_w;      // [T, k]
  const int32_t* sorted_ids;    // [cap]
  const int32_t* block_expert;  // [cap / B]
  const int32_t* num_padded;    // [1]
  void* h;                  // [cap, I] act dtype (workspace); e4m3fn codes in the W8A8 mode
  float* y_part;            // [splits, A, d] fp32 (workspace)
  void* out;                // [T, d] act dtype
  int T, d, E, I, k, A, B, cap;
  int splits;               // split of W2's K (= I) range
  int ksplit;               // K elements per split (multiple of the K chunk)
  // W8A8 mode (block-scaled e4m3fn activations, workspace): x codes [T, d]
  // and exponents [T, d/32]; h's exponents [cap, I/32] (h holds its codes)
  bool act_mx;
  uint8_t* xq;
  uint8_t* sx;
  uint8_t* sh;
  // Tile-queue schedule of the 128-token GEMM: counters in the workspace
  // (gemm_queue_ints() int32), zeroed by launch_gemm_queue_reset unless
  // queue_zeroed says an earlier launch on the stream has done it.
  bool queue_sched;
  bool queue_zeroed;
  int32_t* queue;
  // The fused decode kernel (W13, W2 and combine in one persistent launch):
  // its counters (fused_counter_ints()), zeroed by the routing launch; null
  // when the expert kernels run as separate launches.
  int32_t* fused_cnt;
  // W2 with the combine in its launch (LDS-streaming path): arrival counters
  // (ffn2_combine_ints() int32), zeroed by the routing launch; null when the
  // combine is a launch of its own.
  int32_t* combine_cnt;
  // Blocks of 128 on the register-token tile (the plan's choice under the
  // automatic schedule) rather than the 128-token GEMM.
  bool wide;
};

hipError_t launch_ffn13(const FfnArgs& a, hipStream_t s);
hipError_t launch_ffn2(const FfnArgs& a, hipStream_t s);
hipError_t launch_combine(const FfnArgs& a, hipStream_t s);
// Token-tiled grouped GEMM (block size 128, no K split); used by the two
// launchers above when a.B == 128.
hipError_t launch_ffn13_gemm(const FfnArgs& a, hipStream_t s);
hipError_t launch_ffn2_gemm(const FfnArgs& a, hipStream_t s);
int gemm_queue_ints();
hipError_t launch_gemm_queue_reset(const FfnArgs& a, hipStream_t s);
// Large-tile grouped GEMM (block size 256, bf16 weights, d % 256 == 0 and
// I % 128 == 0); used when a.B == 256.
bool big_gemm_fits(int64_t T, int d, int I);
// W8A8 large tile (e4m3fn weights, block-scaled e4m3fn activations, blocks
// of 256): d and I multiples of 256, an expert's W13 (2I x d bytes) and xq
// (T x d bytes) under 2 GiB.
bool big8_fits(int64_t T, int d, int I);
hipError_t launch_quantize_x(const FfnArgs& a, hipStream_t s);
hipError_t launch_ffn13_big8(const FfnArgs& a, hipStream_t s);
hipError_t launch_ffn2_big8(const FfnArgs& a, hipStream_t s);
int big8_w2_kchunk();  // a split of the W8A8 W2's K range is a multiple of this
hipError_t launch_ffn13_big(const FfnArgs& a, hipStream_t s);
hipError_t launch_ffn2_big(const FfnArgs& a, hipStream_t s);
int big_w2_kchunk();  // a split of the big W2's K range is a multiple of this
// 128-token tile with e4m3fn weights and bf16 activations (d % 256 == 0,
// I % 128 == 0, 32-bit offsets); used for a.B == 128 where it fits.
bool mid_gemm_fits(int64_t T, int d, int I);
hipError_t launch_ffn13_mid(const FfnArgs& a, hipStream_t s);
hipError_t launch_ffn2_mid(const FfnArgs& a, hipStream_t s);
// 128-token tile with the token operand in registers, bf16 or e4m3fn
// weights with bf16 activations (K stages of 128 weight bytes: d and I
// multiples of 64 for bf16, 128 for e4m3fn, at least three or four stages;
// I a multiple of 32; 32-bit offsets).  A split of W2's K range is a
// multiple of wide_kchunk() elements and holds at least four of them.
bool wide_gemm_fits(int64_t T, int d, int I, int w_dtype);
int wide_kchunk(int w_dtype);
hipError_t launch_ffn13_wide(const FfnArgs& a, hipStream_t s);
hipError_t launch_ffn2_wide(const FfnArgs& a, hipStream_t s);
inline bool wide_use(int w_dtype, int act_dtype, bool act_mx, int B, int64_t T, int d, int I) {
  return B == 128 && act_dtype == kDtypeBF16 && !act_mx && wide_gemm_fits(T, d, I, w_dtype);
}
inline bool wide_use(const FfnArgs& a) {
  return a.wide && wide_use(a.w_dtype, a.act_dtype, a.act_mx, a.B, a.T, a.d, a.I);
}

// Row blocks that hold at least one slot: the realised blocks are at most
// the capacity's, and at most one partial block per used expert plus the
// full ones.
inline int64_t ffn_blocks_estimate(int64_t cap, int B, int E, int64_t A) {
  const int64_t used = E < A ? E : A;
  const int64_t est = used + A / B;
  return cap / B < est ? cap / B : est;
}

// Weight streaming through LDS: bf16 weights in blocks of 16 or 32 tokens,
// e4m3fn weights in blocks of 16 (d and I multiples of the stage's K: 256
// bf16 or 512 e4m3fn elements), bf16 activations, when the W13 grid has at
// least MOE_DMA_MIN_WORKGROUPS workgroups (about two rounds of the
// LDS-limited occupancy); smaller grids keep the register path, whose
// workgroups all fit on the chip at once.
bool dma_stream_fits(int d, int I, int w_dtype);
int dma_stream_kc(int w_dtype);  // K elements per stage
#ifndef MOE_DMA_MIN_WORKGROUPS
#define MOE_DMA_MIN_WORKGROUPS 1024
#endif
inline bool dma_stream_use(int w_dtype, int act_dtype, int B, int d, int I, int64_t blocks_est) {
#ifdef MOE_NO_DMA_STREAM
  return false;
#else
  const bool shape = (w_dtype == kDtypeBF16 && (B == 16 || B == 32)) ||
                     (w_dtype == kDtypeE4M3FN && B == 16);
  return act_dtype == kDtypeBF16 && shape && dma_stream_fits(d, I, w_dtype) &&
         blocks_est * (I / 16) >= MOE_DMA_MIN_WORKGROUPS;
#endif
}
inline bool dma_stream_use(const FfnArgs& a) {
  return dma_stream_use(a.w_dtype, a.act_dtype, a.B, a.d, a.I,
                        ffn_blocks_estimate(a.cap, a.B, a.E, a.A));
}
hipError_t launch_ffn13_dma(const FfnArgs& a, hipStream_t s);
// output channels per W2 workgroup of that path for a block size and block estimate
int dma_w2_channels(int w_dtype, int B, int64_t blocks_est);
hipError_t launch_ffn2_dma(const FfnArgs& a, hipStream_t s);
// W2 + gate scale with the combine folded in (same path, bf16 output):
// needs a.combine_cnt with ffn2_combine_ints() zeroed counters.  The layer
// uses it where ffn2_combine_pays() (measured faster than the two launches).
bool ffn2_combine_pays(int w_dtype, int B, int64_t blocks_est);
int ffn2_combine_ints(const FfnArgs& a);
hipError_t launch_ffn2_combine_dma(const FfnArgs& a, hipStream_t s);

// The fused decode kernel: bf16 activations and weights on the
// LDS-streaming path (blocks of 16 or 32).  fused_counter_ints() is the
// counter workspace it needs; launch_ffn_fused runs W13, W2 and the combine.
bool fused_decode_fits(int w_dtype, int act_dtype, int B, int d, int I, int64_t blocks_est);
int fused_counter_ints(const FfnArgs& a);
hipError_t launch_ffn_fused(const FfnArgs& a, hipStream_t s);

// K chunk the W2 kernel uses for a given shape, block size, dtypes and
// block estimate (the split length must be a multiple of it).
int ffn2_kchunk(int d, int I, int B, int w_dtype, int act_dtype, int64_t blocks_est);

}  // namespace moe
