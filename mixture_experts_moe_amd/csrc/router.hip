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

__global__ __launch_bounds__(256) void router_topk_kernel(const float* __restrict__ logits,
                                                          int32_t* __restrict__ topk_ids,
                                                          float* __restrict__ topk_w, int T,
                                                          int E, int k) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + static_cast<size_t>(t) * E;
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
    topk_ids[static_cast<size_t>(t) * k + lane] = my_e;
    topk_w[static_cast<size_t>(t) * k + lane] = p / s;
  }
}

// ---------------------------------------------------------------- launchers

hipError_t launch_router_logits(const void* x, int act_dtype, const float* wg, float* logits,
                                int T, int E, int d, hipStream_t s) {
  dim3 grid((T + 15) / 16, (E + 63) / 64);
  if (act_dtype == kDtypeF32)
    router_logits_kernel<float><<<grid, 256, 0, s>>>(static_cast<const float*>(x), wg, logits,
                                                     T, E, d);
  else
    router_logits_kernel<bf16_t><<<grid, 256, 0, s>>>(static_cast<const bf16_t*>(x), wg,
                                                      logits, T, E, d);
  return hipGetLastError();
}

hipError_t launch_router_topk(const float* logits, int32_t* ids, float* w, int T, int E, int k,
                              hipStream_t s) {
  router_topk_kernel<<<(T + 3) / 4, 256, 0, s>>>(logits, ids, w, T, E, k);
  return hipGetLastError();
}

}  // namespace moe
