// Large-tile grouped GEMM with e4m3fn weights and block-scaled e4m3fn
// activations (the W8A8 mode), for blocks of 256 tokens.
//
// Sources: the Hungarian news page "Az AWS új MoE-optimalizációkkal
// gyorsítja a SageMaker AI-t", section "FP8 esetén a Triton backend
// bizonyult gyorsabbnak" (FP8 scaling fused with the matrix product), and
// section "A fused MoE a számítási folyamat több lépését egyesíti" (the
// experts' computation as one batched operation).
//
// Activations are quantised in blocks of 32 consecutive values of a row to
// e4m3fn with one power-of-two scale per block (an 8-bit exponent, E8M0):
// x per token by quantize_x_kernel before W13, h per routing slot in W13's
// epilogue.  gfx950's v_mfma_scale_f32_16x16x128_f8f6f4 multiplies e4m3fn
// operands and applies such exponents per 32 values of K itself, so the
// activation scales cost no instruction; the weights' fp32 per-channel (or
// per-tensor) scales are applied in the epilogues.
//
// Tile, waves, stage loader, swizzle and barrier are the bf16 big tile's
// (ffn_big_common.h); a stage holds 128 K (one 128-byte LDS row per operand
// row).  The MFMA's lane layout: lane l supplies row (A) or column (B) l%16
// and the 32 values k = 16(l/16) .. +15 and 64 + 16(l/16) .. +15 of the 128,
// i.e. logical slots l/16 and 4 + l/16 of the row; the scale of K block j
// (k = 32j .. 32j+31) of row or column r comes from lane r + 16j.  So lane
// l's B scale is its token's exponent for K block l/16 of the stage.

#include "ffn_big_common.h"

namespace moe {

constexpr int kBig8K = 128;    // e4m3fn K per stage
constexpr int kMx = 32;        // values per activation scale
constexpr int kE8M0One = 127;  // E8M0 code of 2^0

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef f32x4 Big8Acc[kBigTA][kBigNB];

// A lane's LDS byte offsets inside a stage buffer.  Lane (r16, g) reads row
// r16 of a 16-row tile, logical slots g and 4 + g.  Tiles start at multiples
// of 16 rows, so a row's swizzle big_swz(row) = (r16 >> 1) & 7 is the same
// for every tile and a tile's fragment is at these offsets plus the tile's
// first row x 128 (a constant): four registers address every read.
struct Big8Lane {
  uint32_t a_lo, a_hi;  // weight rows from the wave's first weight row
  uint32_t b_lo, b_hi;  // token rows from the wave's first token row
};

__device__ __forceinline__ Big8Lane big8_lane(int arow0, int brow0) {
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15, g = lane >> 4;
  const uint32_t lo = r16 * kBigRowBytes + ((g ^ ((r16 >> 1) & 7)) << 4);
  const uint32_t hi = lo ^ 64;  // slot 4 + g: (4 + g) ^ sw = (g ^ sw) ^ 4
  return Big8Lane{arow0 * kBigRowBytes + lo, arow0 * kBigRowBytes + hi,
                  kBigOperandBytes + brow0 * kBigRowBytes + lo,
                  kBigOperandBytes + brow0 * kBigRowBytes + hi};
}

// 32 bytes of K for the lane, `row_bytes` = the tile's first row x 128
// (relative to the wave's first row of that operand).
__device__ __forceinline__ i32x8 big8_frag(const uint8_t* buf, uint32_t lo, uint32_t hi,
                                           int row_bytes) {
  const uint4 l = *reinterpret_cast<const uint4*>(buf + lo + row_bytes);
  const uint4 h = *reinterpret_cast<const uint4*>(buf + hi + row_bytes);
  return i32x8{static_cast<int>(l.x), static_cast<int>(l.y), static_cast<int>(l.z),
               static_cast<int>(l.w), static_cast<int>(h.x), static_cast<int>(h.y),
               static_cast<int>(h.z), static_cast<int>(h.w)};
}

// acc += A . B over one stage's 128 K; B's K block l/16 scaled by 2^(sb - 127).
__device__ __forceinline__ f32x4 big8_mfma(i32x8 a, i32x8 b, f32x4 c, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, kE8M0One, 0, sb);
}

// The activation exponents of a stage travel with it: the block's 256 token
// rows x 4 bytes (K blocks 4s .. 4s + 3 of each row) go to a 1 KB LDS array
// per buffer, loaded by waves 0..3 (64 rows each, one 4-byte direct-to-LDS
// load per lane).  Kept out of registers: the loop runs at the 256-register
// limit.
constexpr int kBig8ExpBytes = kBigN * 4;

#ifndef MOE_BIG8_PREFETCH
#define MOE_BIG8_PREFETCH 1
#endif

struct Big8Scales {
  __amdgpu_buffer_rsrc_t r;
  uint32_t off;  // waves 0..3: byte offset of token row 64 * wave + lane's exponents, k = 0

  __device__ __forceinline__ void load(uint8_t* lds, int s, int wave) const {
    if (wave < kBigN / 64)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, (__attribute__((address_space(3))) void*)(lds + 256 * wave), 4, off + 4 * s, 0, 0, 0);
  }
};

// One stage: wait for this wave's loads of `cur` (and its exponents), meet
// the other waves, issue the next stage into `nxt` with its exponents (when
// kIssue), then the stage's 32 MFMAs in four groups of two weight tiles x
// the four token tiles.  The token fragments are read once; with
// MOE_BIG8_PREFETCH the weight fragments of group q + 1 are read while group
// q's MFMAs run (two register sets).  The scheduling barrier after the issue
// keeps the compiler from sinking the next stage's loads to the end of the
// stage, which would leave nothing in flight during the MFMAs.  A wave whose
// token rows are all padding (kLive false) only loads and meets the barriers.
// kUp: first tile row of the wave's second group of four weight tiles,
// relative to its first (128 for W13's up rows, 64 for W2).  ex_off: this
// lane's exponent byte in the stage's exponent array (token row
// 64 wn + r16, block g; tile u adds 64 bytes).
template <bool kIssue, bool kLive, int kUp>
__device__ __forceinline__ void big8_stage(const BigLoader& ld, const Big8Scales& sx,
                                           const uint8_t* cur, uint8_t* nxt, const uint8_t* ex,
                                           uint8_t* exn, int s, int wave, const Big8Lane& ln,
                                           uint32_t ex_off, Big8Acc& acc) {
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  big_barrier();
  if (kIssue) {
    big_issue(ld, nxt, static_cast<uint32_t>(s + 1) * kBig8K, wave);
    sx.load(exn, s + 1, wave);
  }
  __builtin_amdgcn_sched_barrier(0);
  if (!kLive) return;
  // Opaque copies of the lane offsets: otherwise the compiler hoists the
  // fragment addresses of both buffers out of the loop as separate
  // registers, runs out and spills them; this way each stage forms its bases
  // and every tile offset is a read's immediate.
  uint32_t alo = ln.a_lo, ahi = ln.a_hi, blo = ln.b_lo, bhi = ln.b_hi, eo = ex_off;
  asm volatile("" : "+v"(alo), "+v"(ahi), "+v"(blo), "+v"(bhi), "+v"(eo));
  i32x8 b[kBigNB];
  int sb[kBigNB];
#pragma unroll
  for (int u = 0; u < kBigNB; ++u) {
    b[u] = big8_frag(cur, blo, bhi, 16 * u * kBigRowBytes);
    sb[u] = ex[eo + 64 * u];
  }
  // weight tile t: rows 16t (t < 4) and kUp + 16(t - 4) past the wave's first
  constexpr auto arow = [](int t) { return (t < 4 ? 16 * t : kUp + 16 * (t - 4)) * kBigRowBytes; };
#if MOE_BIG8_PREFETCH
  i32x8 a[2][2];
  a[0][0] = big8_frag(cur, alo, ahi, arow(0));
  a[0][1] = big8_frag(cur, alo, ahi, arow(1));
#pragma unroll
  for (int q = 0; q < kBigTA / 2; ++q) {
    if (q + 1 < kBigTA / 2) {
      a[(q + 1) & 1][0] = big8_frag(cur, alo, ahi, arow(2 * q + 2));
      a[(q + 1) & 1][1] = big8_frag(cur, alo, ahi, arow(2 * q + 3));
    }
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int u = 0; u < kBigNB; ++u)
        acc[2 * q + j][u] = big8_mfma(a[q & 1][j], b[u], acc[2 * q + j][u], sb[u]);
    __builtin_amdgcn_sched_barrier(0);
  }
#else
#pragma unroll
  for (int q = 0; q < kBigTA / 2; ++q) {
    const i32x8 a0 = big8_frag(cur, alo, ahi, arow(2 * q));
    const i32x8 a1 = big8_frag(cur, alo, ahi, arow(2 * q + 1));
#pragma unroll
    for (int u = 0; u < kBigNB; ++u) {
      acc[2 * q][u] = big8_mfma(a0, b[u], acc[2 * q][u], sb[u]);
      acc[2 * q + 1][u] = big8_mfma(a1, b[u], acc[2 * q + 1][u], sb[u]);
    }
  }
#endif
}

template <bool kLive, int kUp>
__device__ __forceinline__ void big8_run(const BigLoader& ld, const Big8Scales& sx,
                                         uint8_t* const (&buf)[2], uint8_t* const (&ex)[2],
                                         int nst, int wave, const Big8Lane& ln, uint32_t ex_off,
                                         Big8Acc& acc) {
  big_issue(ld, buf[0], 0, wave);
  sx.load(ex[0], 0, wave);
  // nst is even (d % 256 == 0 for W13, splits of I in multiples of 256 for W2)
  for (int s = 0; s + 2 < nst; s += 2) {
    big8_stage<true, kLive, kUp>(ld, sx, buf[0], buf[1], ex[0], ex[1], s, wave, ln, ex_off, acc);
    big8_stage<true, kLive, kUp>(ld, sx, buf[1], buf[0], ex[1], ex[0], s + 1, wave, ln, ex_off,
                                 acc);
  }
  big8_stage<true, kLive, kUp>(ld, sx, buf[0], buf[1], ex[0], ex[1], nst - 2, wave, ln, ex_off,
                               acc);
  big8_stage<false, kLive, kUp>(ld, sx, buf[1], buf[0], ex[1], ex[0], nst - 1, wave, ln, ex_off,
                                acc);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
}

#define BIG8_EXPS(name)                                                          \
  __shared__ __attribute__((aligned(1024))) uint8_t name##0[kBig8ExpBytes];      \
  __shared__ __attribute__((aligned(1024))) uint8_t name##1[kBig8ExpBytes];      \
  uint8_t* const name[2] = {name##0, name##1}

// E8M0 exponent of a block whose largest magnitude is amax: floor(log2 amax)
// - 8 (8 = exponent of 448, e4m3fn's largest value), 0 for amax = 0, at
// least -127 (the smallest E8M0 exponent).
__device__ __forceinline__ int mx_exponent(float amax) {
  if (!(amax > 0.f)) return 0;
  int ex;
  (void)frexpf(amax, &ex);  // amax = m * 2^ex, m in [0.5, 1)
  return max(ex - 1 - 8, -127);
}

// Two values -> two e4m3fn codes (low bytes), after scaling by 2^-e and
// clamping to +-448 (the conversion rounds to nearest even; values past 448
// would become NaN, hence the clamp).
__device__ __forceinline__ uint32_t mx_encode2(float v0, float v1, int e) {
  const float y0 = fminf(fmaxf(ldexpf(v0, -e), -448.f), 448.f);
  const float y1 = fminf(fmaxf(ldexpf(v1, -e), -448.f), 448.f);
  const s16x2 p = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(s16x2{0, 0}, y0, y1, 1.f, false);
  return __builtin_bit_cast(uint32_t, p) & 0xffffu;
}

// ------------------------------------------------------------ x quantisation
// One thread per block of 32 values of a token row: xq gets the 32 codes,
// sx the block's E8M0 exponent byte.

__global__ __launch_bounds__(256) void quantize_x_kernel(const bf16_t* __restrict__ x,
                                                         uint8_t* __restrict__ xq,
                                                         uint8_t* __restrict__ sx,
                                                         int64_t nblocks) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= nblocks) return;
  const uint4* src = reinterpret_cast<const uint4*>(x + i * kMx);
  uint4 w[4];
  float amax = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    w[q] = src[q];
    const uint32_t ws[4] = {w[q].x, w[q].y, w[q].z, w[q].w};
#pragma unroll
    for (int j = 0; j < 4; ++j)
      amax = fmaxf(amax, fmaxf(fabsf(__uint_as_float(ws[j] << 16)),
                               fabsf(__uint_as_float(ws[j] & 0xffff0000u))));
  }
  const int e = mx_exponent(amax);
  uint32_t out[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t ws[4] = {w[q].x, w[q].y, w[q].z, w[q].w};
#pragma unroll
    for (int j = 0; j < 4; j += 2) {
      const uint32_t lo = mx_encode2(__uint_as_float(ws[j] << 16),
                                     __uint_as_float(ws[j] & 0xffff0000u), e);
      const uint32_t hi = mx_encode2(__uint_as_float(ws[j + 1] << 16),
                                     __uint_as_float(ws[j + 1] & 0xffff0000u), e);
      out[2 * q + j / 2] = lo | (hi << 16);
    }
  }
  uint4* dst = reinterpret_cast<uint4*>(xq + i * kMx);
  dst[0] = uint4{out[0], out[1], out[2], out[3]};
  dst[1] = uint4{out[4], out[5], out[6], out[7]};
  sx[i] = static_cast<uint8_t>(e + 127);
}

// ------------------------------------------------------------ W13 + SiLU*mul + h quantisation
// Tile: channels n0 .. n0+127 (rows: 128 gate, then 128 up) x the block's
// 256 tokens.  The epilogue scales by the weights' per-channel scale, forms
// h = SiLU(gate) * up and quantises h in blocks of 32 channels of a slot's
// row: lane (r16, g) holds channels 64wm + 16t + 4g .. +3 of token column
// r16, so block 2wm + t/2 is spread over tiles t, t+1 (t even) and the four
// lanes r16 + 16g; its maximum is reduced across those lanes.

__global__ __launch_bounds__(kBigThreads) void ffn13_big8_kernel(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ sx,
    const uint8_t* __restrict__ w13, const float* __restrict__ s13, int scale_mode,
    const int32_t* __restrict__ sorted_ids, const int32_t* __restrict__ block_expert,
    const int32_t* __restrict__ num_padded, uint8_t* __restrict__ hq, uint8_t* __restrict__ sh,
    int d, int I, int k, int A, int gx, int gy) {
  BIG_BUFFERS(buf);
  BIG8_EXPS(exb);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const BigTile tl = big_tile_live(blockIdx.x, gx, gy, num_padded, kBigTokens);
  if (!tl.live) return;
  const int b = tl.b;
  const int32_t* blk = sorted_ids + static_cast<size_t>(b) * kBigTokens;
  if (blk[0] >= A) return;
  const int e = block_expert[b];
  const int n0 = tl.y * 128;
  const size_t two_i = 2 * static_cast<size_t>(I);
  const int T = A / k;

  BigLoader ld;
  const int lrow = lane / kBigSlots;
  const uint32_t c_even = ((lane % kBigSlots) ^ big_swz(lrow)) * 16;
  const uint32_t c_odd = ((lane % kBigSlots) ^ big_swz(kBigRowsPerGroup + lrow)) * 16;
  const int row0 = (kBigRows / kBigWaves) * wave + lrow;
  const uint32_t wrow0 = row0 < 128 ? n0 + row0 : I + n0 + row0 - 128;
  ld.ra = big_rsrc(w13 + static_cast<size_t>(e) * two_i * d, two_i * d);
  ld.rb = big_rsrc(xq, static_cast<size_t>(T) * d);
  ld.a_even = wrow0 * d + c_even;
  ld.a_odd = (wrow0 + kBigRowsPerGroup) * d + c_odd;
  ld.a_step = 2 * kBigRowsPerGroup * d;
  const int brow = (kBigN / kBigWaves) * wave + lrow;
#pragma unroll
  for (int q = 0; q < kBigGroupsB; ++q) {
    const int f = blk[brow + kBigRowsPerGroup * q];  // pad slot: any valid row (never stored)
    ld.b[q] = static_cast<uint32_t>(f < A ? f / k : 0) * d + (q & 1 ? c_odd : c_even);
  }
  const int wm = wave & 1, wn = wave >> 1;
  const int r16 = lane & 15, g = lane >> 4;
  const int kb = d / kMx;  // exponent bytes per token row
  Big8Scales sc;
  sc.r = big_rsrc(sx, static_cast<size_t>(T) * kb);
  {
    const int f = blk[64 * (wave & 3) + lane];  // waves 0..3 load rows 64 wave + lane
    sc.off = static_cast<uint32_t>(f < A ? f / k : 0) * kb;
  }
  Big8Acc acc;
#pragma unroll
  for (int t = 0; t < kBigTA; ++t)
#pragma unroll
    for (int u = 0; u < kBigNB; ++u) acc[t][u] = f32x4{0.f, 0.f, 0.f, 0.f};

  const bool live = __builtin_amdgcn_readfirstlane(blk[(kBigN / kBigWn) * wn]) < A;
  const int nst = d / kBig8K;
  // weight rows: gate 64wm .. +63 and up 128 + 64wm .. +63 of the tile
  const Big8Lane ln = big8_lane(64 * wm, (kBigN / kBigWn) * wn);
  const uint32_t ex_off = ((kBigN / kBigWn) * wn + r16) * 4 + g;
  if (live)
    big8_run<true, 128>(ld, sc, buf, exb, nst, wave, ln, ex_off, acc);
  else
    big8_run<false, 128>(ld, sc, buf, exb, nst, wave, ln, ex_off, acc);

  // weight scales of this lane's channels n0 + 64wm + 16t + 4g + v
  float sg[4][4], su[4][4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const size_t ch = n0 + 64 * wm + 16 * t + 4 * g + v;
      sg[t][v] = load_scale(s13, scale_mode, e, static_cast<size_t>(e) * two_i + ch);
      su[t][v] = load_scale(s13, scale_mode, e, static_cast<size_t>(e) * two_i + I + ch);
    }
  const int ib = I / kMx;  // exponent bytes per h row
#pragma unroll
  for (int u = 0; u < kBigNB; ++u) {
    const size_t row = static_cast<size_t>(b) * kBigTokens + (kBigN / kBigWn) * wn + 16 * u + r16;
#pragma unroll
    for (int tp = 0; tp < 4; tp += 2) {  // one 32-channel block: tiles tp, tp + 1
      float hv[2][4];
      float amax = 0.f;
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int t = tp + dt;
          hv[dt][v] = silu(acc[t][u][v] * sg[t][v]) * (acc[t + 4][u][v] * su[t][v]);
          amax = fmaxf(amax, fabsf(hv[dt][v]));
        }
      amax = fmaxf(amax, __shfl_xor(amax, 16, kWave));
      amax = fmaxf(amax, __shfl_xor(amax, 32, kWave));
      const int ex = mx_exponent(amax);
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        const uint32_t q = mx_encode2(hv[dt][0], hv[dt][1], ex) |
                           (mx_encode2(hv[dt][2], hv[dt][3], ex) << 16);
        *reinterpret_cast<uint32_t*>(hq + row * I + n0 + 64 * wm + 16 * (tp + dt) + 4 * g) = q;
      }
      if (g == 0) sh[row * ib + (n0 + 64 * wm + 16 * tp) / kMx] = static_cast<uint8_t>(ex + 127);
    }
  }
}

// ------------------------------------------------------------ W2 + gate scale
// Tile: output channels n0 .. n0+255 x the block's 256 h rows (e4m3fn with
// their block exponents); split z of K = I.

__global__ __launch_bounds__(kBigThreads) void ffn2_big8_kernel(
    const uint8_t* __restrict__ hq, const uint8_t* __restrict__ sh,
    const uint8_t* __restrict__ w2, const float* __restrict__ s2, int scale_mode,
    const float* __restrict__ topk_w, const int32_t* __restrict__ sorted_ids,
    const int32_t* __restrict__ block_expert, const int32_t* __restrict__ num_padded,
    float* __restrict__ y_part, int d, int I, int A, int ksplit, int gx, int gy) {
  BIG_BUFFERS(buf);
  BIG8_EXPS(exb);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const BigTile tl = big_tile_live(blockIdx.x, gx, gy, num_padded, kBigTokens);
  if (!tl.live) return;
  const int b = tl.b;
  const int32_t* blk = sorted_ids + static_cast<size_t>(b) * kBigTokens;
  if (blk[0] >= A) return;
  const int e = block_expert[b];
  const int n0 = tl.y * kBigRows;
  const int k_begin = blockIdx.z * ksplit;
  const int nst = (min(I, k_begin + ksplit) - k_begin) / kBig8K;
  float* y = y_part + static_cast<size_t>(blockIdx.z) * A * d;

  BigLoader ld;
  const int lrow = lane / kBigSlots;
  const uint32_t c_even = ((lane % kBigSlots) ^ big_swz(lrow)) * 16;
  const uint32_t c_odd = ((lane % kBigSlots) ^ big_swz(kBigRowsPerGroup + lrow)) * 16;
  const int row0 = (kBigRows / kBigWaves) * wave + lrow;
  ld.ra = big_rsrc(w2 + static_cast<size_t>(e) * d * I, static_cast<size_t>(d) * I);
  ld.a_even = static_cast<uint32_t>(n0 + row0) * I + k_begin + c_even;
  ld.a_odd = static_cast<uint32_t>(n0 + row0 + kBigRowsPerGroup) * I + k_begin + c_odd;
  ld.a_step = 2 * kBigRowsPerGroup * I;
  const int brow = (kBigN / kBigWaves) * wave + lrow;
  const size_t hrow0 = static_cast<size_t>(b) * kBigTokens;  // the block's first h row
  ld.rb = big_rsrc(hq + hrow0 * I, static_cast<size_t>(kBigN) * I);
#pragma unroll
  for (int q = 0; q < kBigGroupsB; ++q)
    ld.b[q] = static_cast<uint32_t>(brow + kBigRowsPerGroup * q) * I + k_begin +
              (q & 1 ? c_odd : c_even);
  const int wm = wave & 1, wn = wave >> 1;
  const int r16 = lane & 15, g = lane >> 4;
  const int ib = I / kMx;
  Big8Scales sc;
  sc.r = big_rsrc(sh + hrow0 * ib, static_cast<size_t>(kBigN) * ib);
  sc.off = static_cast<uint32_t>(64 * (wave & 3) + lane) * ib + k_begin / kMx;
  Big8Acc acc;
#pragma unroll
  for (int t = 0; t < kBigTA; ++t)
#pragma unroll
    for (int u = 0; u < kBigNB; ++u) acc[t][u] = f32x4{0.f, 0.f, 0.f, 0.f};

  const bool live = __builtin_amdgcn_readfirstlane(blk[(kBigN / kBigWn) * wn]) < A;
  // weight rows 128wm .. +127 of the tile
  const Big8Lane ln = big8_lane(128 * wm, (kBigN / kBigWn) * wn);
  const uint32_t ex_off = ((kBigN / kBigWn) * wn + r16) * 4 + g;
  if (live)
    big8_run<true, 64>(ld, sc, buf, exb, nst, wave, ln, ex_off, acc);
  else
    big8_run<false, 64>(ld, sc, buf, exb, nst, wave, ln, ex_off, acc);

  // lane: token column r16 of tile u, channels n0 + 128wm + 16t + 4g .. +3
#pragma unroll
  for (int u = 0; u < kBigNB; ++u) {
    const int f = blk[(kBigN / kBigWn) * wn + 16 * u + r16];
    if (f < A) {
      const float gate = topk_w[f];
      float* yrow = y + static_cast<size_t>(f) * d;
#pragma unroll
      for (int t = 0; t < kBigTA; ++t) {
        const int nb = n0 + 128 * wm + 16 * t + 4 * g;
        const size_t base = static_cast<size_t>(e) * d + nb;
        store_partial4(yrow + nb, acc[t][u][0] * load_scale(s2, scale_mode, e, base) * gate,
                       acc[t][u][1] * load_scale(s2, scale_mode, e, base + 1) * gate,
                       acc[t][u][2] * load_scale(s2, scale_mode, e, base + 2) * gate,
                       acc[t][u][3] * load_scale(s2, scale_mode, e, base + 3) * gate);
      }
    }
  }
}

// ------------------------------------------------------------ launchers

bool big8_fits(int64_t T, int d, int I) {
  const int64_t lim = int64_t(1) << 31;
  return d % 256 == 0 && I % 256 == 0 && int64_t(2) * I * d < lim && T * d < lim;
}

static int big8_grid(int gx, int gy) {
  const int total = gx * gy;
  return (total + kBigXcds - 1) / kBigXcds * kBigXcds;
}

hipError_t launch_quantize_x(const FfnArgs& a, hipStream_t s) {
  if (!a.xq || !a.sx || a.d % kMx != 0) return hipErrorInvalidValue;
  const int64_t nblocks = static_cast<int64_t>(a.T) * (a.d / kMx);
  if (nblocks == 0) return hipSuccess;
  quantize_x_kernel<<<static_cast<unsigned>((nblocks + 255) / 256), 256, 0, s>>>(
      static_cast<const bf16_t*>(a.x), a.xq, a.sx, nblocks);
  return hipGetLastError();
}

hipError_t launch_ffn13_big8(const FfnArgs& a, hipStream_t s) {
  if (a.B != kBigTokens || a.w_dtype != kDtypeE4M3FN || !a.act_mx || !big8_fits(a.T, a.d, a.I))
    return hipErrorInvalidValue;
  const int gx = a.cap / kBigTokens, gy = a.I / 128;
  ffn13_big8_kernel<<<big8_grid(gx, gy), kBigThreads, 0, s>>>(
      a.xq, a.sx, static_cast<const uint8_t*>(a.w13), a.s13, a.scale_mode, a.sorted_ids,
      a.block_expert, a.num_padded, static_cast<uint8_t*>(a.h), a.sh, a.d, a.I, a.k, a.A, gx, gy);
  return hipGetLastError();
}

hipError_t launch_ffn2_big8(const FfnArgs& a, hipStream_t s) {
  // every split an even number (>= 2) of 128-wide K stages
  if (a.B != kBigTokens || a.w_dtype != kDtypeE4M3FN || !a.act_mx || !big8_fits(a.T, a.d, a.I) ||
      a.ksplit % (2 * kBig8K) != 0 || a.splits < 1 ||
      static_cast<int64_t>(a.splits - 1) * a.ksplit >= a.I)
    return hipErrorInvalidValue;
  const int gx = a.cap / kBigTokens, gy = a.d / kBigRows;
  ffn2_big8_kernel<<<dim3(big8_grid(gx, gy), 1, a.splits), kBigThreads, 0, s>>>(
      static_cast<const uint8_t*>(a.h), a.sh, static_cast<const uint8_t*>(a.w2), a.s2,
      a.scale_mode, a.topk_w, a.sorted_ids, a.block_expert, a.num_padded, a.y_part, a.d, a.I,
      a.A, a.ksplit, gx, gy);
  return hipGetLastError();
}

int big8_w2_kchunk() { return 2 * kBig8K; }

}  // namespace moe
