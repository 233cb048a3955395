// Large-tile grouped GEMM for blocks of 256 tokens (prefill-sized expert
// groups, bf16 weights): the MFMA-bound end of the fused MoE layer.
//
// Sources: the Hungarian news page "Az AWS új MoE-optimalizációkkal
// gyorsítja a SageMaker AI-t", section "A fused MoE a számítási folyamat több
// lépését egyesíti" (all experts' computation as one batched operation); the
// French summary "Ingénierie de kernels Mixture-of-Experts sur Amazon
// SageMaker AI", second paragraph (the expert product A[M,K] x B[K,N], tokens
// x hidden x expert output dim).
//
// When an expert holds hundreds of tokens the product is a dense contraction
// and the limit is how many bytes each MFMA needs.  A workgroup computes a
// 256 x 256 tile (256 weight rows x 256 tokens, so every operand byte staged
// in LDS feeds 256 MACs) on v_mfma_f32_16x16x32_bf16, eight waves of
// 128 x 64 each: two waves per SIMD, so that one wave's MFMAs run while the
// other waits on its LDS reads or the stage barrier (a single wave per SIMD
// issuing this MFMA back to back keeps the matrix core only about half
// busy).  Both operands move HBM/L2 -> LDS with gfx950's direct-to-LDS
// 16-byte buffer loads (no VGPR staging), in K stages of 64 elements through
// two LDS buffers, so the loads of the next stage are in flight while the
// MFMAs of the current one run; one barrier per stage.  An LDS row holds one
// stage of one operand row in 16-byte slots, XOR-swizzled by row so that the
// 16 rows read by one 16-lane group for the same k fall in 16 different bank
// groups.  The waves of a tile whose 64 token rows are all padding (the tail
// block of an expert) only load and meet the barriers.
//
// W13: the tile's rows are 128 gate rows then the 128 matching up rows, so
// each wave holds gate and up of the same 64 channels and the epilogue writes
// h = SiLU(gate) * up.  W2: 256 output channels; the epilogue scales by the
// slot's gate.  The grid is rasterised per XCD like the 128-token GEMM.

#include "ffn_big_common.h"

namespace moe {

constexpr int kBigK = 64;  // bf16 K elements per stage (128-byte rows)

// 16-byte MFMA fragment of tile row `row`, logical slot `slot`.
__device__ __forceinline__ bf16x8 big_frag(const uint8_t* op, int row, int slot) {
  return as_frag(*reinterpret_cast<const uint4*>(op + row * kBigRowBytes +
                                                 ((slot ^ big_swz(row)) << 4)));
}

typedef f32x4 BigAcc[kBigTA][kBigNB];

// Fragments of 32 consecutive K of a stage (half h of it).
struct BigFrags {
  bf16x8 a[kBigTA], b[kBigNB];
};

// Fragments of half stage h (k = 32h .. 32h+31) for this wave's row tiles
// (rows arow0 + 16t for t < 4, arow_up + 16(t-4) after) and token tiles
// (rows brow0 + 16u); lane group l/16 holds k = 32h + 8(l/16) .. +8, logical
// slot 4h + l/16.
__device__ __forceinline__ void big_load_frags(BigFrags& f, const uint8_t* opa, const uint8_t* opb,
                                               int arow0, int arow_up, int brow0, int h) {
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15;
  const int slot = 4 * h + (lane >> 4);
#pragma unroll
  for (int t = 0; t < kBigTA; ++t)
    f.a[t] = big_frag(opa, (t < 4 ? arow0 + 16 * t : arow_up + 16 * (t - 4)) + r16, slot);
#pragma unroll
  for (int u = 0; u < kBigNB; ++u) f.b[u] = big_frag(opb, brow0 + 16 * u + r16, slot);
}

__device__ __forceinline__ void big_mma(const BigFrags& f, BigAcc& acc) {
#pragma unroll
  for (int t = 0; t < kBigTA; ++t)
#pragma unroll
    for (int u = 0; u < kBigNB; ++u) acc[t][u] = mfma16x16x32(f.a[t], f.b[u], acc[t][u]);
}

// First part of one stage: wait until this wave's loads of `cur` have
// landed (kWait of its later loads may stay outstanding), meet the other
// waves (after which nobody reads `nxt`, the buffer read one or two stages
// ago, any more), issue the stage after the in-flight ones into `nxt` (when
// kIssue), read the first half stage's fragments, run their MFMAs, and read
// the second half's (f1), whose MFMAs the caller runs.  With two waves per
// SIMD the other wave covers each wave's read latency, and one fragment set
// at a time keeps a wave within its 256 registers.  A wave whose token rows
// are all padding (kLive false) only loads and meets the barriers.
template <bool kIssue, int kWait, bool kLive>
__device__ __forceinline__ void big_half(const BigLoader& ld, const uint8_t* cur, uint8_t* nxt,
                                         int knext, int wave, int arow0, int arow_up, int brow0,
                                         BigFrags& f1, BigAcc& acc) {
  static_assert(kWait >= 0 && kWait <= 63, "wait count exceeds the 6-bit vmcnt field");
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(kWait));
  big_barrier();
  const uint8_t* opb = cur + kBigOperandBytes;
  BigFrags f0;
#if MOE_BIG_ISSUE_FIRST
  if (kIssue) big_issue(ld, nxt, 2 * knext, wave);
  if (!kLive) return;
  __builtin_amdgcn_sched_barrier(0);
  big_load_frags(f0, cur, opb, arow0, arow_up, brow0, 0);
#else
  if (!kLive) {
    if (kIssue) big_issue(ld, nxt, 2 * knext, wave);
    return;
  }
  big_load_frags(f0, cur, opb, arow0, arow_up, brow0, 0);
  __builtin_amdgcn_sched_barrier(0);
  if (kIssue) big_issue(ld, nxt, 2 * knext, wave);
#endif
  big_mma(f0, acc);
  __builtin_amdgcn_sched_barrier(0);
  big_load_frags(f1, cur, opb, arow0, arow_up, brow0, 1);
}

// acc[t][u] += A_rows(t) . B_rows(u)^T over K.  A rows: arow0 + 16t (t < 4)
// and arow_up + 16(t-4); B rows: brow0 + 16u.  Stage s (K = 64s .. 64s+63)
// lives in buffer s % S.  The buffers are separate LDS arrays: with one
// array the compiler cannot tell that reads of stage s do not depend on the
// loads of later stages in flight, and waits for those before every read.
// The loop is rotated by half a stage so that each stage's second k-step
// MFMAs can overlap the next stage's start.
struct BigRing {
  const BigLoader& ld;
  uint8_t* const (&buf)[2];
  int wave, arow0, arow_up, brow0;
  bool live;  // the wave's token rows hold at least one real slot (wave-uniform)

  // a wave whose token rows are all padding (kLive false) only loads and
  // meets the barriers; the choice is made once, outside the loops, so that
  // each loop body is branch-free
  template <bool kLive>
  __device__ __forceinline__ void mma1(const BigFrags& f1, BigAcc& acc) const {
    if constexpr (kLive) big_mma(f1, acc);
  }

  template <int b, bool kIssue, int kWait, bool kLive>
  __device__ __forceinline__ void step(int s, BigFrags& f1, BigAcc& acc) const {
    constexpr int S = kBigStages;
    big_half<kIssue, kWait, kLive>(ld, buf[b], buf[(b + S - 1) % S], (s + S - 1) * kBigK, wave,
                                   arow0, arow_up, brow0, f1, acc);
  }

  // two stages (nst even: the launchers require d % 256 == 0, I % 128 == 0)
  template <bool kLive>
  __device__ __forceinline__ void run2(int nst, BigAcc& acc) const {
    BigFrags f1;
    big_issue(ld, buf[0], 0, wave);
    step<0, true, 0, kLive>(0, f1, acc);
    for (int s = 1; s + 1 < nst; s += 2) {
      mma1<kLive>(f1, acc);
      step<1, true, 0, kLive>(s, f1, acc);
      mma1<kLive>(f1, acc);
      step<0, true, 0, kLive>(s + 1, f1, acc);
    }
    mma1<kLive>(f1, acc);
    step<1, false, 0, kLive>(nst - 1, f1, acc);
    mma1<kLive>(f1, acc);
  }

  __device__ __forceinline__ void run(int nst, BigAcc& acc) const {
    if (live)
      run2<true>(nst, acc);
    else
      run2<false>(nst, acc);
  }
};

// ------------------------------------------------------------ W13 + SiLU*mul
// Tile: channels n0 .. n0+127 (rows: 128 gate, then 128 up) x the 256
// tokens of row block b.

__global__ __launch_bounds__(kBigThreads) void ffn13_big_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ w13,
    const int32_t* __restrict__ sorted_ids, const int32_t* __restrict__ block_expert,
    const int32_t* __restrict__ num_padded, bf16_t* __restrict__ h, int d, int I, int k, int A,
    int gx, int gy) {
  BIG_BUFFERS(buf);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const BigTile tl = big_tile_live(blockIdx.x, gx, gy, num_padded, kBigTokens);
  if (!tl.live) return;  // uniform
  const int b = tl.b;
  const int32_t* blk = sorted_ids + static_cast<size_t>(b) * kBigTokens;
  if (blk[0] >= A) return;  // real slots come first: this block holds none
  const int e = block_expert[b];
  const int n0 = tl.y * 128;
  const size_t two_i = 2 * static_cast<size_t>(I);

  // tile rows: 0..127 gate rows n0.., 128..255 the matching up rows
  BigLoader ld;
  const int lrow = lane / kBigSlots;  // row within a 1 KB group
  const int c_even = ((lane % kBigSlots) ^ big_swz(lrow)) * 8;
  const int c_odd = ((lane % kBigSlots) ^ big_swz(kBigRowsPerGroup + lrow)) * 8;
  const int row0 = (kBigRows / kBigWaves) * wave + lrow;  // tile row of group 0
  const uint32_t wrow0 = row0 < 128 ? n0 + row0 : I + n0 + row0 - 128;  // row of expert e's W13
  ld.ra = big_rsrc(w13 + static_cast<size_t>(e) * two_i * d, two_i * d * 2);
  ld.rb = big_rsrc(x, static_cast<size_t>(A / k) * d * 2);
  ld.a_even = 2 * (wrow0 * d + c_even);
  ld.a_odd = 2 * ((wrow0 + kBigRowsPerGroup) * d + c_odd);
  ld.a_step = 2 * (2 * kBigRowsPerGroup * d);
  const int brow = (kBigN / kBigWaves) * wave + lrow;  // token row of B group 0
#pragma unroll
  for (int q = 0; q < kBigGroupsB; ++q) {
    const int f = blk[brow + kBigRowsPerGroup * q];  // pad slot: any valid row (never stored)
    ld.b[q] = 2 * (static_cast<uint32_t>(f < A ? f / k : 0) * d + (q & 1 ? c_odd : c_even));
  }
  const int wm = wave & 1, wn = wave >> 1;
  BigAcc acc;
#pragma unroll
  for (int t = 0; t < kBigTA; ++t)
#pragma unroll
    for (int u = 0; u < kBigNB; ++u) acc[t][u] = f32x4{0.f, 0.f, 0.f, 0.f};

  // real slots come first: the wave's token rows are all padding iff its first one is
  const bool live = __builtin_amdgcn_readfirstlane(blk[(kBigN / kBigWn) * wn]) < A;
  BigRing{ld, buf, wave, 64 * wm, 128 + 64 * wm, (kBigN / kBigWn) * wn, live}.run(d / kBigK, acc);

  // lane: token column r16 of tile u, channels n0 + 64wm + 16t + 4g .. +3
  const int r16 = lane & 15;
  const int g = lane >> 4;
#pragma unroll
  for (int u = 0; u < kBigNB; ++u) {
    const size_t row =
        static_cast<size_t>(b) * kBigTokens + (kBigN / kBigWn) * wn + 16 * u + r16;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      uint32_t packed[2];
#pragma unroll
      for (int v = 0; v < 4; v += 2) {
        const float h0 = silu(acc[t][u][v]) * acc[t + 4][u][v];
        const float h1 = silu(acc[t][u][v + 1]) * acc[t + 4][u][v + 1];
        packed[v / 2] = static_cast<uint32_t>(f32_to_bf16(h0)) |
                        (static_cast<uint32_t>(f32_to_bf16(h1)) << 16);
      }
      *reinterpret_cast<uint2*>(h + row * I + n0 + 64 * wm + 16 * t + 4 * g) =
          uint2{packed[0], packed[1]};
    }
  }
}

// ------------------------------------------------------------ W2 + gate scale
// Tile: output channels n0 .. n0+255 x kBigN tokens (h rows of the block).

__global__ __launch_bounds__(kBigThreads) void ffn2_big_kernel(
    const bf16_t* __restrict__ h, const bf16_t* __restrict__ w2,
    const float* __restrict__ topk_w, const int32_t* __restrict__ sorted_ids,
    const int32_t* __restrict__ block_expert, const int32_t* __restrict__ num_padded,
    float* __restrict__ y_part, int d, int I, int A, int ksplit, int gx, int gy) {
  BIG_BUFFERS(buf);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const BigTile tl = big_tile_live(blockIdx.x, gx, gy, num_padded, kBigTokens);
  if (!tl.live) return;
  const int b = tl.b;
  const int32_t* blk = sorted_ids + static_cast<size_t>(b) * kBigTokens;
  if (blk[0] >= A) return;
  const int e = block_expert[b];
  const int n0 = tl.y * kBigRows;
  // split z of K = I (grid z): the combine adds the splits in a fixed order
  const int k_begin = blockIdx.z * ksplit;
  const int nst = (min(I, k_begin + ksplit) - k_begin) / kBigK;
  float* y = y_part + static_cast<size_t>(blockIdx.z) * A * d;

  BigLoader ld;
  const int lrow = lane / kBigSlots;
  const int c_even = ((lane % kBigSlots) ^ big_swz(lrow)) * 8;
  const int c_odd = ((lane % kBigSlots) ^ big_swz(kBigRowsPerGroup + lrow)) * 8;
  const int row0 = (kBigRows / kBigWaves) * wave + lrow;
  ld.ra = big_rsrc(w2 + static_cast<size_t>(e) * d * I, static_cast<size_t>(d) * I * 2);
  ld.a_even = 2 * (static_cast<uint32_t>(n0 + row0) * I + k_begin + c_even);
  ld.a_odd = 2 * (static_cast<uint32_t>(n0 + row0 + kBigRowsPerGroup) * I + k_begin + c_odd);
  ld.a_step = 2 * (2 * kBigRowsPerGroup * I);
  // h rows of the tile; pad slots hold no token and their columns are never stored
  const int brow = (kBigN / kBigWaves) * wave + lrow;
  ld.rb = big_rsrc(h + (static_cast<size_t>(b) * kBigTokens) * I, static_cast<size_t>(kBigN) * I * 2);
#pragma unroll
  for (int q = 0; q < kBigGroupsB; ++q)
    ld.b[q] = 2 * (static_cast<uint32_t>(brow + kBigRowsPerGroup * q) * I + k_begin +
                   (q & 1 ? c_odd : c_even));
  const int wm = wave & 1, wn = wave >> 1;
  BigAcc acc;
#pragma unroll
  for (int t = 0; t < kBigTA; ++t)
#pragma unroll
    for (int u = 0; u < kBigNB; ++u) acc[t][u] = f32x4{0.f, 0.f, 0.f, 0.f};

  // A rows 128*wm .. +127: eight consecutive 16-row tiles
  const bool live = __builtin_amdgcn_readfirstlane(blk[(kBigN / kBigWn) * wn]) < A;
  BigRing{ld, buf, wave, 128 * wm, 128 * wm + 64, (kBigN / kBigWn) * wn, live}.run(nst, acc);

  // lane: token column r16 of tile u, channels n0 + 128wm + 16t + 4g .. +3
  const int r16 = lane & 15;
  const int g = lane >> 4;
#pragma unroll
  for (int u = 0; u < kBigNB; ++u) {
    const int f = blk[(kBigN / kBigWn) * wn + 16 * u + r16];
    if (f < A) {
      const float gate = topk_w[f];
      float* yrow = y + static_cast<size_t>(f) * d + n0 + 128 * wm + 4 * g;
#pragma unroll
      for (int t = 0; t < kBigTA; ++t)
        store_partial4(yrow + 16 * t, acc[t][u][0] * gate, acc[t][u][1] * gate,
                       acc[t][u][2] * gate, acc[t][u][3] * gate);
    }
  }
}

// ------------------------------------------------------------ launchers

// The loads address an expert's W13 (2I x d) and x (T x d) with 32-bit
// byte offsets: both must stay under 2 GiB.
bool big_gemm_fits(int64_t T, int d, int I) {
  const int64_t lim = int64_t(1) << 31;
  return d % 256 == 0 && I % 128 == 0 && int64_t(4) * I * d < lim && T * d * 2 < lim;
}

static int big_grid(int gx, int gy) {
  const int total = gx * gy;
  return (total + kBigXcds - 1) / kBigXcds * kBigXcds;
}

hipError_t launch_ffn13_big(const FfnArgs& a, hipStream_t s) {
  if (a.B != kBigTokens || a.w_dtype != kDtypeBF16 || !big_gemm_fits(a.T, a.d, a.I))
    return hipErrorInvalidValue;
  const int gx = a.cap / kBigTokens, gy = a.I / 128;
  ffn13_big_kernel<<<big_grid(gx, gy), kBigThreads, 0, s>>>(
      static_cast<const bf16_t*>(a.x), static_cast<const bf16_t*>(a.w13), a.sorted_ids,
      a.block_expert, a.num_padded, static_cast<bf16_t*>(a.h), a.d, a.I, a.k, a.A, gx, gy);
  return hipGetLastError();
}

hipError_t launch_ffn2_big(const FfnArgs& a, hipStream_t s) {
  // every split an even number (>= 2) of 64-wide K stages
  if (a.B != kBigTokens || a.w_dtype != kDtypeBF16 || !big_gemm_fits(a.T, a.d, a.I) ||
      a.ksplit % (2 * kBigK) != 0 || a.splits < 1 ||
      static_cast<int64_t>(a.splits - 1) * a.ksplit >= a.I)
    return hipErrorInvalidValue;
  const int gx = a.cap / kBigTokens, gy = a.d / kBigRows;
  ffn2_big_kernel<<<dim3(big_grid(gx, gy), 1, a.splits), kBigThreads, 0, s>>>(
      static_cast<const bf16_t*>(a.h), static_cast<const bf16_t*>(a.w2), a.topk_w, a.sorted_ids,
      a.block_expert, a.num_padded, a.y_part, a.d, a.I, a.A, a.ksplit, gx, gy);
  return hipGetLastError();
}

int big_w2_kchunk() { return 2 * kBigK; }

}  // namespace moe
