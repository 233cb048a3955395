// Router kernels: logits = x . W_gate^T in fp32, then per-token top-k
// selection and softmax gates over the selection.
//
// Sources: the Hungarian news page "Az AWS új MoE-optimalizációkkal
// gyorsítja a SageMaker AI-t", section "A fused MoE a számítási folyamat
// több lépését egyesíti" (token routing is the first fused step).  The pages
// do not give the routing rule; the reading taken is: top-k on the logits,
// ties to the lower expert index, gates = softmax over the selected logits.

#include "common.h"
#include "kernels.h"

namespace moe {

// ---------------------------------------------------------------- top-k + gates
//
// One wavefront per token.  Lane l holds the logits of experts l, l+64, ...
// Each of the k rounds takes the wave-wide best untaken expert, ordering by
// (logit descending, index ascending); NaN counts as -inf.  Lane j keeps the
// j-th pick, then the gates are exp(l_j - l_0) / sum, with l_0 the largest
// selected logit.

constexpr int kMaxExpertsPerLane = 16;  // E <= 1024

__device__ __forceinline__ bool better(float av, int ae, float bv, int be) {
  return av > bv || (av == bv && ae < be);
}

// The whole wave selects for one token: `row` holds its E logits (global or
// LDS); writes k ids and gates.
__device__ __forceinline__ void topk_wave(const float* row, int E, int k, int32_t* ids,
                                          float* gates, int* lds_ids = nullptr) {
  const int lane = threadIdx.x & 63;
  float v[kMaxExpertsPerLane];
  const int per_lane = (E + 63) >> 6;
#pragma unroll
  for (int i = 0; i < kMaxExpertsPerLane; ++i) {
    const int e = lane + 64 * i;
    float val = -INFINITY;
    if (i < per_lane && e < E) {
      val = row[e];
      if (val != val) val = -INFINITY;  // NaN ranks below every number
    }
    v[i] = val;
  }
  uint32_t taken = 0;  // bit i: expert lane + 64*i already selected
  float my_v = -INFINITY;
  int my_e = 0;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < kMaxExpertsPerLane; ++i) {
      const int e = lane + 64 * i;
      if (i < per_lane && e < E && !((taken >> i) & 1u) && better(v[i], e, bv, be)) {
        bv = v[i];
        be = e;
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const float ov = __shfl_xor(bv, off, kWave);
      const int oe = __shfl_xor(be, off, kWave);
      if (better(ov, oe, bv, be)) {
        bv = ov;
        be = oe;
      }
    }
    if (be < E && (be & 63) == lane) taken |= 1u << (be >> 6);
    if (lane == j) {
      my_v = bv;
      my_e = be;
    }
  }
  const float l0 = __shfl(my_v, 0, kWave);
  const float p = lane < k ? expf(my_v - l0) : 0.f;
  const float s = wave_sum(p);
  if (lane < k) {
    ids[lane] = my_e;
    gates[lane] = p / s;
    if (lds_ids) lds_ids[lane] = my_e;
  }
}

__global__ __launch_bounds__(256) void router_topk_kernel(const float* __restrict__ logits,
                                                          int32_t* __restrict__ topk_ids,
                                                          float* __restrict__ topk_w, int T,
                                                          int E, int k) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  topk_wave(logits + static_cast<size_t>(t) * E, E, k, topk_ids + static_cast<size_t>(t) * k,
            topk_w + static_cast<size_t>(t) * k);
}

// ---------------------------------------------------------------- regrouping in the router
//
// For a batch routed by a single workgroup (at most 16 tokens, so at most
// 16 * 16 slots) the same workgroup also regroups the slots by expert, which
// saves the separate regrouping launch on the small-batch (decode) path.  It
// writes what the regrouping kernel writes, by the same definition: slot f
// of expert e lands at off[e] + (number of slots f' < f routed to e), where
// off[e] = sum over e' < e of counts rounded up to the block size; pads and
// the tail hold the sentinel A, block owners -1 past the padded total.  Each
// wave ranks its 64 slots per expert with a ballot; a wave's base is the sum
// over lower waves.

struct AlignOut {
  int B, cap;
  int32_t* counts;
  int32_t* sorted_ids;
  int32_t* block_expert;
  int32_t* num_padded;
  // int32 words the split router's partial launch sets to 0 (the next
  // kernels' counters), or none
  int32_t* zero = nullptr;
  int nzero = 0;
};

constexpr int kRaWaves = 16;  // the fused router's workgroup

__device__ __forceinline__ void align_in_block(const int* s_ids, int A, int E, const AlignOut& o) {
  __shared__ int s_wc[kRaWaves][16];  // [wave][expert]: this wave's slots routed to the expert
  __shared__ int s_off[17], s_cnt[16];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int id = tid < A ? s_ids[tid] : -1;  // slot f = tid
  int rank = 0;
  for (int e = 0; e < E; ++e) {
    const uint64_t m = __ballot(id == e);
    if (id == e) rank = __popcll(m & ((1ull << lane) - 1ull));
    if (lane == 0) s_wc[wave][e] = __popcll(m);
  }
  __syncthreads();
  if (tid == 0) {
    int off = 0;
    for (int e = 0; e < E; ++e) {
      int c = 0;
      for (int w = 0; w < kRaWaves; ++w) c += s_wc[w][e];
      s_cnt[e] = c;
      s_off[e] = off;
      off += (c + o.B - 1) / o.B * o.B;
    }
    s_off[E] = off;
  }
  __syncthreads();
  if (static_cast<unsigned>(id) < static_cast<unsigned>(E)) {
    int base = 0;
    for (int w = 0; w < wave; ++w) base += s_wc[w][id];
    o.sorted_ids[s_off[id] + base + rank] = tid;
  }
  const int total = s_off[E];
  for (int r = tid; r < o.cap; r += 64 * kRaWaves) {  // pads and the tail
    int e = 0;
    while (e + 1 < E && s_off[e + 1] <= r) ++e;
    if (r >= total || r - s_off[e] >= s_cnt[e]) o.sorted_ids[r] = A;
  }
  for (int b = tid; b < o.cap / o.B; b += 64 * kRaWaves) {
    const int r = b * o.B;
    int e = 0;
    while (e + 1 < E && s_off[e + 1] <= r) ++e;
    o.block_expert[b] = r < total ? e : -1;
  }
  if (tid < E) o.counts[tid] = s_cnt[tid];
  if (tid == 0) *o.num_padded = total;
}

// ---------------------------------------------------------------- logits
//
// fp32 matrix-core product, experts on the MFMA M side and tokens on N
// (16 x 16 output tile per wave, 4 waves per workgroup along experts;
// grid x runs over token tiles, grid y over groups of 64 experts).
// Each lane loads four consecutive k of its W_gate row and of its token row
// and feeds them to four 16x16x4 fp32 MFMAs: MFMA q takes k = kc + 4*g + q
// for lane group g = lane/16, so A and B use the same k for every lane.
// Products and sums are fp32; bf16 activations are widened exactly.

template <typename XT>
__device__ __forceinline__ void load4(const XT* p, float* v);

template <>
__device__ __forceinline__ void load4<float>(const float* p, float* v) {
  float4 q = *reinterpret_cast<const float4*>(p);
  v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
}

template <>
__device__ __forceinline__ void load4<bf16_t>(const bf16_t* p, float* v) {
  uint2 q = *reinterpret_cast<const uint2*>(p);
  v[0] = __uint_as_float(q.x << 16);
  v[1] = __uint_as_float(q.x & 0xffff0000u);
  v[2] = __uint_as_float(q.y << 16);
  v[3] = __uint_as_float(q.y & 0xffff0000u);
}

template <typename XT>
__global__ __launch_bounds__(256) void router_logits_kernel(const XT* __restrict__ x,
                                                            const float* __restrict__ wg,
                                                            float* __restrict__ logits, int T,
                                                            int E, int d) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int e_tile = blockIdx.y * 4 + wave;
  const int e = e_tile * 16 + r16;
  const int t = blockIdx.x * 16 + r16;
  if (e_tile * 16 >= E) return;  // whole wave past the last expert
  const bool e_ok = e < E;
  const bool t_ok = t < T;
  const float* wrow = wg + static_cast<size_t>(e_ok ? e : 0) * d;
  const XT* xrow = x + static_cast<size_t>(t_ok ? t : 0) * d;

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int kc = 0; kc < d; kc += 16) {
    float a[4] = {0.f, 0.f, 0.f, 0.f};
    float b[4] = {0.f, 0.f, 0.f, 0.f};
    if (e_ok) load4<float>(wrow + kc + 4 * g, a);
    if (t_ok) load4<XT>(xrow + kc + 4 * g, b);
#pragma unroll
    for (int q = 0; q < 4; ++q) acc = mfma16x16x4f32(a[q], b[q], acc);
  }
  // D: lane holds token column r16, expert rows 4*g .. 4*g+3 of the tile.
  if (t_ok) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int ee = e_tile * 16 + 4 * g + v;
      if (ee < E) logits[static_cast<size_t>(t) * E + ee] = acc[v];
    }
  }
}

// bf16 activations: the same product on bf16 matrix cores.  Each fp32
// W_gate value is split exactly into three bf16 parts, w = hi + mid + lo, by
// truncation: hi keeps the top 8 significand bits, mid the next 8 of the
// remainder, lo the last 8 (an fp32 significand has 24), so each part is a
// bf16 value and both subtractions are exact.  A bf16 x bf16 product is
// exact in fp32, so x.w = x.hi + x.mid + x.lo is an fp32 dot product of
// exact products, at three 16x16x32 bf16 MFMAs per 32 k instead of eight
// 16x16x4 fp32 ones.  K is split over the waves of a workgroup (each wave
// takes a contiguous range of 32-wide steps) and the partial tiles are added
// in wave order through LDS, so the result is deterministic.  A workgroup
// covers 16 experts x 16*NT tokens.  NaN weights stay NaN in hi.

__device__ __forceinline__ uint32_t trunc_bf16_bits(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t t = u & 0xffff0000u;
  return (u & 0x7fffffffu) > 0x7f800000u ? (t | 0x00400000u) : t;  // keep NaN a NaN
}

__device__ __forceinline__ void split3_bf16(const float (&w)[8], uint4& hi, uint4& mid, uint4& lo) {
  uint32_t h[4], m[4], l[4];
#pragma unroll
  for (int i = 0; i < 8; i += 2) {
    uint32_t hb[2], mb[2], lb[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float v = w[i + j];
      hb[j] = trunc_bf16_bits(v);
      const float r = v - __uint_as_float(hb[j]);
      mb[j] = __float_as_uint(r) & 0xffff0000u;
      lb[j] = __float_as_uint(r - __uint_as_float(mb[j])) & 0xffff0000u;
    }
    h[i / 2] = (hb[0] >> 16) | hb[1];
    m[i / 2] = (mb[0] >> 16) | mb[1];
    l[i / 2] = (lb[0] >> 16) | lb[1];
  }
  hi = uint4{h[0], h[1], h[2], h[3]};
  mid = uint4{m[0], m[1], m[2], m[3]};
  lo = uint4{l[0], l[1], l[2], l[3]};
}

// kTopk (NT = 1, NW = 16, E <= 16: one workgroup holds every expert of its
// 16 tokens): the workgroup also selects, one wave per token.
// K split over several workgroups (kPart): the 16-wave workgroup's work cut
// in two launches with the same arithmetic.  kPart = 1: a one-wave workgroup
// per (token tile, expert tile, slice z) computes what wave z of the 16-wave
// workgroup computes and stores that partial tile; kPart = 2: the 16-wave
// workgroup takes wave w's partial tile from that store instead of computing
// it, then adds, selects and regroups exactly as kPart = 0 does.  A few
// tokens' W_gate (128 KB at d = 4096, E = 8) then streams through 16 CUs'
// miss queues instead of one.
constexpr int kRouterSlices = 16;

template <int NT, int NW, bool kTopk, bool kAlign = false, int kPart = 0>
__global__ __launch_bounds__(64 * NW) void router_logits_bf16_kernel(
    const bf16_t* __restrict__ x, const float* __restrict__ wg, float* __restrict__ logits,
    int32_t* __restrict__ topk_ids, float* __restrict__ topk_w, int T, int E, int d, int k,
    AlignOut ao, f32x4* __restrict__ part) {
  static_assert(!kTopk || (NT == 1 && NW == 16), "fused selection: 16 tokens, 16 waves");
  static_assert(!kAlign || kTopk, "regrouping follows the selection");
  static_assert(kPart == 0 || (NT == 1 && NW == (kPart == 1 ? 1 : kRouterSlices)),
                "split K: one-wave slices, then the 16-wave workgroup");
  // 32-wide steps whose loads are issued together: the few-token kernel is
  // latency-bound, so it takes a whole wave's K range (d = 4096) in one round
  constexpr int U = NT == 1 ? 8 : 4;
  __shared__ f32x4 red[NW][NT][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int t0 = blockIdx.x * 16 * NT;
  const int e = blockIdx.y * 16 + r16;
  const bool e_ok = e < E;
  const float* wrow = wg + static_cast<size_t>(e_ok ? e : 0) * d + 8 * g;
  const bf16_t* xrow[NT];
  bool t_ok[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int t = t0 + nt * 16 + r16;
    t_ok[nt] = t < T;
    xrow[nt] = x + static_cast<size_t>(t_ok[nt] ? t : 0) * d + 8 * g;
  }
  const int steps = d / 32;
  constexpr int kSlices = kPart == 0 ? NW : kRouterSlices;
  const int slice = kPart == 1 ? static_cast<int>(blockIdx.z) : wave;
  const int s_begin = slice * steps / kSlices;
  const int s_end = kPart == 2 ? s_begin : (slice + 1) * steps / kSlices;  // 2: nothing to compute
  f32x4 acc_h[NT], acc_m[NT], acc_l[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc_h[nt] = acc_m[nt] = acc_l[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int s0 = s_begin; s0 < s_end; s0 += U) {
    float4 wa[U], wb[U];
    uint4 xb[U][NT];
#pragma unroll
    for (int u = 0; u < U; ++u) {  // issue every load of U steps first
      const int k = (s0 + u) * 32;
      const bool live = s0 + u < s_end;
      wa[u] = (live && e_ok) ? *reinterpret_cast<const float4*>(wrow + k) : float4{0.f, 0.f, 0.f, 0.f};
      wb[u] = (live && e_ok) ? *reinterpret_cast<const float4*>(wrow + k + 4) : float4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        xb[u][nt] = (live && t_ok[nt]) ? *reinterpret_cast<const uint4*>(xrow[nt] + k) : uint4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float w[8] = {wa[u].x, wa[u].y, wa[u].z, wa[u].w, wb[u].x, wb[u].y, wb[u].z, wb[u].w};
      uint4 hi, mid, lo;
      split3_bf16(w, hi, mid, lo);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const bf16x8 xf = as_frag(xb[u][nt]);
        acc_h[nt] = mfma16x16x32(as_frag(hi), xf, acc_h[nt]);
        acc_m[nt] = mfma16x16x32(as_frag(mid), xf, acc_m[nt]);
        acc_l[nt] = mfma16x16x32(as_frag(lo), xf, acc_l[nt]);
      }
    }
  }
  // partial tile of slice z for this (token tile, expert tile)
  const size_t part_at =
      ((static_cast<size_t>(slice) * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x) * 64 + lane;
  if constexpr (kPart == 1) {
    part[part_at] = acc_h[0] + (acc_m[0] + acc_l[0]);
    if (ao.nzero > 0) {  // every workgroup clears its share of the counters
      const int nwg = gridDim.x * gridDim.y * gridDim.z;
      const int wg = (blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x;
      for (int i = wg * 64 + lane; i < ao.nzero; i += nwg * 64) ao.zero[i] = 0;
    }
    return;
  } else {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      red[wave][nt][lane] = kPart == 2 ? part[part_at] : acc_h[nt] + (acc_m[nt] + acc_l[nt]);
  }
  __syncthreads();
  // D layout: lane holds token column r16, expert rows 4g .. 4g+3.  The wave
  // partials are added in wave order.
  __shared__ float lg[kTopk ? 16 : 1][16];
  for (int nt = wave; nt < NT; nt += NW) {
    f32x4 v = red[0][nt][lane];
#pragma unroll
    for (int w = 1; w < NW; ++w) v += red[w][nt][lane];
    const int t = t0 + nt * 16 + r16;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int ee = blockIdx.y * 16 + 4 * g + q;
      if (t < T && ee < E) logits[static_cast<size_t>(t) * E + ee] = v[q];
      if constexpr (kTopk) lg[r16][4 * g + q] = v[q];
    }
  }
  if constexpr (kTopk) {
    __shared__ int s_ids[kAlign ? 16 * 16 : 1];  // [token][rank] expert ids (grid of one)
    __syncthreads();
    const int t = t0 + wave;
    if (t < T)
      topk_wave(lg[wave], E, k, topk_ids + static_cast<size_t>(t) * k,
                topk_w + static_cast<size_t>(t) * k, kAlign ? s_ids + wave * k : nullptr);
    if constexpr (kAlign) {
      __syncthreads();
      align_in_block(s_ids, T * k, E, ao);
    }
  }
}

// ---------------------------------------------------------------- many tokens, many experts
// The 64-token x 16-expert tiles above read each token row once per 16
// experts: at T = 2048, E = 256, d = 7168 that is 470 MB of x and 235 MB of
// W_gate pulled from L2 and the last-level cache for 36 MB of data.  Here a
// wave covers 64 tokens x 16 NE experts (NE expert tiles share each x
// fragment), four waves split K as above and the tiles are added in wave
// order, so every logit is computed with the same operations in the same
// order as by router_logits_bf16_kernel<4, 4> (bit-identical); only the
// reuse changes.

constexpr int kRouterWideWaves = 4;  // waves splitting K in the wide tiles

template <int NE>
__global__ __launch_bounds__(64 * kRouterWideWaves) void router_logits_wide_kernel(
    const bf16_t* __restrict__ x, const float* __restrict__ wg, float* __restrict__ logits, int T,
    int E, int d) {
  constexpr int NT = 4, NW = kRouterWideWaves, U = 2;
  __shared__ f32x4 red[NW][NT][NE][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int t0 = blockIdx.x * 16 * NT;
  const int e0 = blockIdx.y * 16 * NE;
  const float* wrow[NE];
  bool e_ok[NE];
#pragma unroll
  for (int ne = 0; ne < NE; ++ne) {
    const int e = e0 + 16 * ne + r16;
    e_ok[ne] = e < E;
    wrow[ne] = wg + static_cast<size_t>(e_ok[ne] ? e : 0) * d + 8 * g;
  }
  const bf16_t* xrow[NT];
  bool t_ok[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int t = t0 + nt * 16 + r16;
    t_ok[nt] = t < T;
    xrow[nt] = x + static_cast<size_t>(t_ok[nt] ? t : 0) * d + 8 * g;
  }
  const int steps = d / 32;
  const int s_begin = wave * steps / NW;
  const int s_end = (wave + 1) * steps / NW;
  f32x4 acc_h[NT][NE], acc_m[NT][NE], acc_l[NT][NE];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int ne = 0; ne < NE; ++ne)
      acc_h[nt][ne] = acc_m[nt][ne] = acc_l[nt][ne] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int s0 = s_begin; s0 < s_end; s0 += U) {
    float4 wa[U][NE], wb[U][NE];
    uint4 xb[U][NT];
#pragma unroll
    for (int u = 0; u < U; ++u) {  // issue every load of U steps first
      const int k = (s0 + u) * 32;
      const bool live = s0 + u < s_end;
#pragma unroll
      for (int ne = 0; ne < NE; ++ne) {
        const bool on = live && e_ok[ne];
        wa[u][ne] = on ? *reinterpret_cast<const float4*>(wrow[ne] + k) : float4{0.f, 0.f, 0.f, 0.f};
        wb[u][ne] = on ? *reinterpret_cast<const float4*>(wrow[ne] + k + 4) : float4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        xb[u][nt] = (live && t_ok[nt]) ? *reinterpret_cast<const uint4*>(xrow[nt] + k) : uint4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int ne = 0; ne < NE; ++ne) {
        const float w[8] = {wa[u][ne].x, wa[u][ne].y, wa[u][ne].z, wa[u][ne].w,
                            wb[u][ne].x, wb[u][ne].y, wb[u][ne].z, wb[u][ne].w};
        uint4 hi, mid, lo;
        split3_bf16(w, hi, mid, lo);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const bf16x8 xf = as_frag(xb[u][nt]);
          acc_h[nt][ne] = mfma16x16x32(as_frag(hi), xf, acc_h[nt][ne]);
          acc_m[nt][ne] = mfma16x16x32(as_frag(mid), xf, acc_m[nt][ne]);
          acc_l[nt][ne] = mfma16x16x32(as_frag(lo), xf, acc_l[nt][ne]);
        }
      }
    }
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int ne = 0; ne < NE; ++ne) red[wave][nt][ne][lane] = acc_h[nt][ne] + (acc_m[nt][ne] + acc_l[nt][ne]);
  __syncthreads();
  // D layout: lane holds token column r16, expert rows 4g .. 4g+3 of a tile
  for (int i = wave; i < NT * NE; i += NW) {
    const int nt = i / NE, ne = i % NE;
    f32x4 v = red[0][nt][ne][lane];
#pragma unroll
    for (int w = 1; w < NW; ++w) v += red[w][nt][ne][lane];
    const int t = t0 + nt * 16 + r16;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int ee = e0 + 16 * ne + 4 * g + q;
      if (t < T && ee < E) logits[static_cast<size_t>(t) * E + ee] = v[q];
    }
  }
}

// ---------------------------------------------------------------- many tokens, many experts, through LDS
// The wide tiles above load their operands straight into fragment
// registers: each load instruction covers 16 rows x 64 bytes (half of each
// row's 128-byte line), and a 64-token x 32-expert tile re-reads its x rows
// once per 32 experts and its W_gate rows once per 64 tokens.  At T = 2048,
// E = 256, d = 7168 that is about 470 MB through L2 and the last-level cache
// for 36 MB of data, and the per-CU load path, not the arithmetic, sets the
// time.  Here a workgroup of eight waves computes 128 tokens x 64 experts
// over one quarter of K: each 64-wide K stage of the 128 x rows (128 bytes
// each) and 64 W_gate rows (256 bytes each) moves into LDS once, with
// consecutive lanes on consecutive 16 bytes (whole lines), two stages ahead
// in registers, and wave w multiplies tokens 64 (w / 4) .. +63 by experts
// 16 (w % 4) .. +15 out of LDS.  Per 16-token x 16-expert tile the MFMA
// sequence is the wide kernel's, over the same K quarter (the quarters are
// its four waves' ranges), and the quarters' partial tiles are added in the
// same order by router_quarter_topk_kernel: the logits are bit-identical to
// router_logits_wide_kernel's.
//
// LDS rows: x rows of 128 bytes in eight 16-byte slots, slot s of row r at
// s ^ ((r >> 1) & 7); W_gate rows of 256 bytes in sixteen slots, slot s of
// row r at s ^ (r & 15).  So the 16 rows one 16-lane group reads at one k
// fall in 16 different 16-byte bank groups.
constexpr int kRlTok = 128;  // tokens per workgroup tile
constexpr int kRlExp = 64;   // experts per workgroup tile
constexpr int kRlK = 64;     // K per stage
constexpr int kRlQuarters = kRouterWideWaves;  // the wide tiles' K ranges
constexpr int kRlWaves = 8;  // wave w: experts 16 (w % 4) .., tokens 64 (w / 4) ..
constexpr int kRlThreads = 64 * kRlWaves;
constexpr int kRlXBytes = kRlTok * kRlK * 2;  // 16 KB
constexpr int kRlWBytes = kRlExp * kRlK * 4;  // 16 KB
// two 16-byte slots of each operand per thread and stage
static_assert(2 * 16 * kRlThreads == kRlXBytes && 2 * 16 * kRlThreads == kRlWBytes,
              "every slot has one thread");

// A stage's share of one thread, in registers: x slots 0 and 1, W_gate
// slots 0 and 1 (plain members, so that they stay in registers).
struct RlRegs {
  uint4 x0, x1, w0, w1;
};

__global__ __launch_bounds__(kRlThreads) void router_logits_lds_kernel(
    const bf16_t* __restrict__ x, const float* __restrict__ wg, float* __restrict__ part, int T,
    int E, int d) {
  __shared__ __attribute__((aligned(16))) uint8_t sx[2][kRlXBytes];
  __shared__ __attribute__((aligned(16))) uint8_t sw[2][kRlWBytes];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int t0 = blockIdx.x * kRlTok;
  const int e0 = blockIdx.y * kRlExp;
  const int z = blockIdx.z;
  const int steps = d / 32;
  const int k_begin = (z * steps / kRlQuarters) * 32;
  const int nst = ((z + 1) * steps / kRlQuarters - z * steps / kRlQuarters) / 2;  // 64-wide stages

  // this thread's slots: x slot u = tid + kRlThreads i (row u >> 3, slot
  // u & 7), W_gate slot u (row u >> 4, slot u & 15), i = 0, 1.  Rows past T
  // or E read row 0: every load is issued (so the compiler's wait counts
  // stay exact and the later stages' loads stay in flight), and those rows
  // feed only output rows and columns that are never stored.
  const bf16_t* xs[2];
  const float* ws[2];
  uint32_t xo[2], wo[2];  // LDS byte offsets
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int u = tid + kRlThreads * i;
    const int xr = u >> 3, xsl = u & 7;
    const int t = t0 + xr;
    xs[i] = x + static_cast<size_t>(t < T ? t : 0) * d + k_begin + 8 * xsl;
    xo[i] = xr * 128 + ((xsl ^ ((xr >> 1) & 7)) << 4);
    const int wr = u >> 4, wsl = u & 15;
    const int e = e0 + wr;
    ws[i] = wg + static_cast<size_t>(e < E ? e : 0) * d + k_begin + 4 * wsl;
    wo[i] = wr * 256 + ((wsl ^ (wr & 15)) << 4);
  }
  auto load = [&](int st) {
    const int o = st * kRlK;
    return RlRegs{*reinterpret_cast<const uint4*>(xs[0] + o), *reinterpret_cast<const uint4*>(xs[1] + o),
                  *reinterpret_cast<const uint4*>(ws[0] + o), *reinterpret_cast<const uint4*>(ws[1] + o)};
  };
  auto store = [&](const RlRegs r, int b) {
    *reinterpret_cast<uint4*>(sx[b] + xo[0]) = r.x0;
    *reinterpret_cast<uint4*>(sx[b] + xo[1]) = r.x1;
    *reinterpret_cast<uint4*>(sw[b] + wo[0]) = r.w0;
    *reinterpret_cast<uint4*>(sw[b] + wo[1]) = r.w1;
  };

  const int er = 16 * (wave & 3) + r16;  // this lane's W_gate row in the tile
  const int tr0 = 64 * (wave >> 2);      // the wave's first token row
  f32x4 acc_h[4], acc_m[4], acc_l[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) acc_h[u] = acc_m[u] = acc_l[u] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int b) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {  // the stage's two 32-wide steps, in K order
      const int sl = 8 * h + 2 * g;  // W_gate slots of k = 32 h + 8 g .. +8
      const float4 wa = *reinterpret_cast<const float4*>(sw[b] + er * 256 + ((sl ^ r16) << 4));
      const float4 wb =
          *reinterpret_cast<const float4*>(sw[b] + er * 256 + (((sl + 1) ^ r16) << 4));
      const float w[8] = {wa.x, wa.y, wa.z, wa.w, wb.x, wb.y, wb.z, wb.w};
      uint4 hi, mid, lo;
      split3_bf16(w, hi, mid, lo);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int tr = tr0 + 16 * u + r16;
        const bf16x8 xf = as_frag(*reinterpret_cast<const uint4*>(
            sx[b] + tr * 128 + (((4 * h + g) ^ ((tr >> 1) & 7)) << 4)));
        acc_h[u] = mfma16x16x32(as_frag(hi), xf, acc_h[u]);
        acc_m[u] = mfma16x16x32(as_frag(mid), xf, acc_m[u]);
        acc_l[u] = mfma16x16x32(as_frag(lo), xf, acc_l[u]);
      }
    }
  };

  // stages s + 1 and s + 2 are in flight in registers while stage s is
  // multiplied out of LDS buffer s % 2.  Every load is issued (past the
  // last stage it repeats the last one, unused), so that the two register
  // sets stay in registers and the compiler's wait counts leave the later
  // set in flight.
  RlRegs ra = load(0);
  RlRegs rb = load(min(1, nst - 1));
  store(ra, 0);
  __syncthreads();
  for (int s = 0; s < nst; s += 2) {
    // stage s in buffer 0 (registers rb: stage s + 1)
    ra = load(min(s + 2, nst - 1));
    compute(0);
    if (s + 1 < nst) store(rb, 1);
    __syncthreads();
    if (s + 1 >= nst) break;
    // stage s + 1 in buffer 1 (registers ra: stage s + 2)
    rb = load(min(s + 3, nst - 1));
    compute(1);
    if (s + 2 < nst) store(ra, 0);
    __syncthreads();
  }
  // D layout: lane holds token column r16, expert rows 4g .. 4g+3
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const f32x4 v = acc_h[u] + (acc_m[u] + acc_l[u]);
    const int t = t0 + tr0 + 16 * u + r16;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = e0 + 16 * (wave & 3) + 4 * g + q;
      if (t < T && e < E) part[(static_cast<size_t>(z) * T + t) * E + e] = v[q];
    }
  }
}

// The quarter sum and the top-k in one launch: one wave per token adds its
// E logits' quarters (the order above), writes them, keeps them in LDS and
// selects from there (topk_wave, as router_topk_kernel does).
__global__ __launch_bounds__(256) void router_quarter_topk_kernel(const float* __restrict__ part,
                                                                  float* __restrict__ logits,
                                                                  int32_t* __restrict__ topk_ids,
                                                                  float* __restrict__ topk_w,
                                                                  int T, int E, int k) {
  __shared__ float row[4][kMaxExpertsPerLane * 64];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;  // whole wave
  const int64_t n = static_cast<int64_t>(T) * E;
  for (int e = lane; e < E; e += 64) {
    const int64_t i = static_cast<int64_t>(t) * E + e;
    float v = part[i];
#pragma unroll
    for (int q = 1; q < kRlQuarters; ++q) v += part[q * n + i];
    logits[i] = v;
    row[wave][e] = v;
  }
  // the wave's own LDS row: its writes are visible to its later reads
  topk_wave(row[wave], E, k, topk_ids + static_cast<size_t>(t) * k,
            topk_w + static_cast<size_t>(t) * k);
}

// ---------------------------------------------------------------- launchers

// Below this many (64-token x 16-expert) tiles the logits kernel runs
// 16-token tiles with K split over 16 waves instead: at prefill with 8
// experts the 64-token tiling leaves most CUs idle (64 workgroups); measured
// 35 -> 18 us at T = 4096, E = 8 and 27 -> 15 us at T = 512, E = 32.
#ifndef MOE_ROUTER_WIDE_WGS
#define MOE_ROUTER_WIDE_WGS 512
#endif
// Expert tiles per wave of router_logits_wide_kernel, and the workgroups its
// grid needs before it is used.
#ifndef MOE_ROUTER_WIDE_NE
#define MOE_ROUTER_WIDE_NE 2
#endif
// (128: at E = 256 the 16-token tiles re-read W_gate's 7.3 MB once per 16
// tokens, 93 us at T = 1024 and 139 at T = 1536 on them.)
// Logits of the wide-tile shapes through LDS when the layer has scratch
// for the quarters (0: the wide tiles).
#ifndef MOE_ROUTER_LDS
#define MOE_ROUTER_LDS 1
#endif
#ifndef MOE_ROUTER_WIDE_NE_WGS
#define MOE_ROUTER_WIDE_NE_WGS 128
#endif
constexpr int kRouterWideNE = MOE_ROUTER_WIDE_NE;

// enough 64-token x (16 NE)-expert tiles to fill half the GPU or more
static bool router_wide(int T, int E) {
  return T > 64 &&
         int64_t((T + 63) / 64) * ((E + 16 * kRouterWideNE - 1) / (16 * kRouterWideNE)) >=
             MOE_ROUTER_WIDE_NE_WGS;
}

// few tokens, or too few 64-token tiles to fill the GPU: 16-token tiles
// with K split 16 ways (router_logits_bf16_kernel<1, 16>)
static bool router_tile16(int T, int E) {
  return !router_wide(T, E) &&
         (T <= 64 || int64_t((T + 63) / 64) * ((E + 15) / 16) < MOE_ROUTER_WIDE_WGS);
}

hipError_t launch_router_logits(const void* x, int act_dtype, const float* wg, float* logits,
                                int T, int E, int d, hipStream_t s) {
  if (act_dtype == kDtypeF32) {
    dim3 grid((T + 15) / 16, (E + 63) / 64);
    router_logits_kernel<float><<<grid, 256, 0, s>>>(static_cast<const float*>(x), wg, logits,
                                                     T, E, d);
  } else if (router_wide(T, E)) {
    // each x fragment feeds NE expert tiles
    dim3 grid((T + 63) / 64, (E + 16 * kRouterWideNE - 1) / (16 * kRouterWideNE));
    router_logits_wide_kernel<kRouterWideNE><<<grid, 64 * kRouterWideWaves, 0, s>>>(static_cast<const bf16_t*>(x), wg,
                                                                  logits, T, E, d);
  } else if (router_tile16(T, E)) {
    dim3 grid((T + 15) / 16, (E + 15) / 16);
    router_logits_bf16_kernel<1, 16, false><<<grid, 1024, 0, s>>>(
        static_cast<const bf16_t*>(x), wg, logits, nullptr, nullptr, T, E, d, 0, AlignOut{}, nullptr);
  } else {
    dim3 grid((T + 63) / 64, (E + 15) / 16);
    router_logits_bf16_kernel<4, 4, false><<<grid, 256, 0, s>>>(
        static_cast<const bf16_t*>(x), wg, logits, nullptr, nullptr, T, E, d, 0, AlignOut{}, nullptr);
  }
  return hipGetLastError();
}

// The logits through LDS (router_logits_lds_kernel) where the wide tiles
// would run and K splits into quarters of whole 64-wide stages, then the
// quarters' sum and the selection: the same bits as launch_router_logits
// and launch_router_topk, in two launches, with `part` of
// router_lds_bytes(T, E) scratch.
bool router_lds_logits(int act_dtype, int T, int E, int d) {
  static_assert(kRouterWideNE == 2, "the LDS tile reproduces the wide kernel's two expert tiles");
  return MOE_ROUTER_LDS && act_dtype == kDtypeBF16 && router_wide(T, E) && d % 256 == 0;
}

size_t router_lds_bytes(int T, int E) {
  return static_cast<size_t>(kRlQuarters) * T * E * sizeof(float);
}

hipError_t launch_router_lds_topk(const void* x, const float* wg, float* logits, int32_t* ids,
                                  float* w, int T, int E, int d, int k, void* part, hipStream_t s) {
  if (!router_lds_logits(kDtypeBF16, T, E, d) || !part || E > kMaxExpertsPerLane * 64)
    return hipErrorInvalidValue;
  float* pt = static_cast<float*>(part);
  const dim3 grid((T + kRlTok - 1) / kRlTok, (E + kRlExp - 1) / kRlExp, kRlQuarters);
  router_logits_lds_kernel<<<grid, kRlThreads, 0, s>>>(static_cast<const bf16_t*>(x), wg, pt, T,
                                                       E, d);
  router_quarter_topk_kernel<<<(T + 3) / 4, 256, 0, s>>>(pt, logits, ids, w, T, E, k);
  return hipGetLastError();
}

bool router_fused(int act_dtype, int T, int E) {
  return act_dtype == kDtypeBF16 && T <= 64 && E <= 16;
}

bool router_selects(int act_dtype, int T, int E) {
  return act_dtype == kDtypeBF16 && E <= 16 && router_tile16(T, E);
}

hipError_t launch_router_fused(const void* x, const float* wg, float* logits, int32_t* ids,
                               float* w, int T, int E, int d, int k, hipStream_t s) {
  if (E > 16) return hipErrorInvalidValue;
  router_logits_bf16_kernel<1, 16, true><<<dim3((T + 15) / 16, 1), 1024, 0, s>>>(
      static_cast<const bf16_t*>(x), wg, logits, ids, w, T, E, d, k, AlignOut{}, nullptr);
  return hipGetLastError();
}

bool route_align_fused(int act_dtype, int T, int E) {
  return act_dtype == kDtypeBF16 && T >= 1 && T <= 16 && E <= 16;
}

hipError_t launch_route_align_fused(const void* x, const float* wg, float* logits, int32_t* ids,
                                    float* w, int T, int E, int d, int k, int B, int cap,
                                    int32_t* counts, int32_t* sorted_ids, int32_t* block_expert,
                                    int32_t* num_padded, hipStream_t s) {
  if (!route_align_fused(kDtypeBF16, T, E) || k > E || B < 1 || cap % B != 0)
    return hipErrorInvalidValue;
  const AlignOut ao{B, cap, counts, sorted_ids, block_expert, num_padded};
  router_logits_bf16_kernel<1, 16, true, true><<<dim3(1, 1), 1024, 0, s>>>(
      static_cast<const bf16_t*>(x), wg, logits, ids, w, T, E, d, k, ao, nullptr);
  return hipGetLastError();
}

size_t router_split_bytes(int T, int E) {
  return static_cast<size_t>(kRouterSlices) * ((T + 15) / 16) * ((E + 15) / 16) * 64 *
         sizeof(f32x4);
}

hipError_t launch_router_fused_split(const void* x, const float* wg, float* logits, int32_t* ids,
                                     float* w, int T, int E, int d, int k, void* part,
                                     hipStream_t s, int32_t* zero, int nzero) {
  if (!router_fused(kDtypeBF16, T, E) || !part || (nzero > 0 && !zero)) return hipErrorInvalidValue;
  const bf16_t* xb = static_cast<const bf16_t*>(x);
  f32x4* pt = static_cast<f32x4*>(part);
  AlignOut zo{};
  zo.zero = zero;
  zo.nzero = nzero;
  router_logits_bf16_kernel<1, 1, false, false, 1><<<dim3((T + 15) / 16, 1, kRouterSlices), 64, 0, s>>>(
      xb, wg, nullptr, nullptr, nullptr, T, E, d, 0, zo, pt);
  router_logits_bf16_kernel<1, 16, true, false, 2><<<dim3((T + 15) / 16, 1), 1024, 0, s>>>(
      xb, wg, logits, ids, w, T, E, d, k, AlignOut{}, pt);
  return hipGetLastError();
}

// Split logits for any E: slice z's partial tiles summed in slice order
// into the logits (what the 16-wave router's workgroup writes).  Grid: the
// partial launch's token and expert tiles, one wave each.
__global__ __launch_bounds__(64) void router_split_sum_kernel(const f32x4* __restrict__ part,
                                                             float* __restrict__ logits, int T,
                                                             int E) {
  const int lane = threadIdx.x;
  const size_t tile = static_cast<size_t>(blockIdx.y) * gridDim.x + blockIdx.x;
  const size_t tiles = static_cast<size_t>(gridDim.x) * gridDim.y;
  f32x4 v = part[tile * 64 + lane];
  for (int z = 1; z < kRouterSlices; ++z) v += part[(z * tiles + tile) * 64 + lane];
  const int t = blockIdx.x * 16 + (lane & 15);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int ee = blockIdx.y * 16 + 4 * (lane >> 4) + q;
    if (t < T && ee < E) logits[static_cast<size_t>(t) * E + ee] = v[q];
  }
}

bool router_split_logits(int act_dtype, int T, int E) {
  return act_dtype == kDtypeBF16 && T >= 1 && T <= 64 && E <= kMaxExperts;
}

hipError_t launch_router_split_logits(const void* x, const float* wg, float* logits, int T, int E,
                                      int d, void* part, hipStream_t s, int32_t* zero, int nzero) {
  if (!router_split_logits(kDtypeBF16, T, E) || !part || (nzero > 0 && !zero))
    return hipErrorInvalidValue;
  f32x4* pt = static_cast<f32x4*>(part);
  const int gx = (T + 15) / 16, gy = (E + 15) / 16;
  AlignOut zo{};
  zo.zero = zero;
  zo.nzero = nzero;
  router_logits_bf16_kernel<1, 1, false, false, 1><<<dim3(gx, gy, kRouterSlices), 64, 0, s>>>(
      static_cast<const bf16_t*>(x), wg, nullptr, nullptr, nullptr, T, E, d, 0, zo, pt);
  router_split_sum_kernel<<<dim3(gx, gy), 64, 0, s>>>(pt, logits, T, E);
  return hipGetLastError();
}

hipError_t launch_route_align_fused_split(const void* x, const float* wg, float* logits,
                                          int32_t* ids, float* w, int T, int E, int d, int k,
                                          int B, int cap, int32_t* counts, int32_t* sorted_ids,
                                          int32_t* block_expert, int32_t* num_padded, void* part,
                                          hipStream_t s, int32_t* zero, int nzero) {
  if (!route_align_fused(kDtypeBF16, T, E) || k > E || B < 1 || cap % B != 0 || !part ||
      (nzero > 0 && !zero))
    return hipErrorInvalidValue;
  const AlignOut ao{B, cap, counts, sorted_ids, block_expert, num_padded};
  const bf16_t* xb = static_cast<const bf16_t*>(x);
  f32x4* pt = static_cast<f32x4*>(part);
  AlignOut zo{};
  zo.zero = zero;
  zo.nzero = nzero;
  router_logits_bf16_kernel<1, 1, false, false, 1><<<dim3(1, 1, kRouterSlices), 64, 0, s>>>(
      xb, wg, nullptr, nullptr, nullptr, T, E, d, 0, zo, pt);
  router_logits_bf16_kernel<1, 16, true, true, 2><<<dim3(1, 1), 1024, 0, s>>>(
      xb, wg, logits, ids, w, T, E, d, k, ao, pt);
  return hipGetLastError();
}

hipError_t launch_router_topk(const float* logits, int32_t* ids, float* w, int T, int E, int k,
                              hipStream_t s) {
  router_topk_kernel<<<(T + 3) / 4, 256, 0, s>>>(logits, ids, w, T, E, k);
  return hipGetLastError();
}

}  // namespace moe
