// Regrouping of the routing slots by expert ("data rearrangement": the
// Hungarian news page "Az AWS új MoE-optimalizációkkal gyorsítja a SageMaker
// AI-t", section "A fused MoE a számítási folyamat több lépését egyesíti";
// variable-size per-expert token groups: same page, section "FP8 esetén a
// Triton backend bizonyult gyorsabbnak").
//
// Layout produced: expert e's group starts at off[e] = sum_{e'<e}
// roundup(counts[e'], B) and holds its flat slot ids f = t*k + j in
// ascending order, then the sentinel A = T*k up to the next multiple of B.
//
// One workgroup per expert, one launch, no atomics on the output order:
//   1. every workgroup builds the full expert histogram in LDS (integer
//      atomics: the counts do not depend on their order);
//   2. it sums roundup(counts, B) below its expert (its group offset) and
//      over all experts (the padded total);
//   3. it walks the slots in order and compacts those routed to its expert
//      with a wave ballot + popcount prefix and a per-wave offset in LDS,
//      so the output order is the slot order and the result is
//      deterministic;
//   4. it writes its pad entries and its block owners.
// Workgroup 0 also writes counts, the padded total and the tail past it.

#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kAlignThreads = 256;
constexpr int kAlignWaves = kAlignThreads / kWave;

__device__ __forceinline__ int block_sum(int v, int* red) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  v = wave_sum_int(v);
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  int s = 0;
#pragma unroll
  for (int w = 0; w < kAlignWaves; ++w) s += red[w];
  return s;
}

__global__ __launch_bounds__(kAlignThreads) void align_kernel(
    const int32_t* __restrict__ ids, int A, int E, int B, int cap, int32_t* __restrict__ counts,
    int32_t* __restrict__ sorted_ids, int32_t* __restrict__ block_expert,
    int32_t* __restrict__ num_padded) {
  __shared__ int cnt[kMaxExperts];
  __shared__ int red[kAlignWaves];
  __shared__ int wave_tot[kAlignWaves];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int e = blockIdx.x;

  for (int i = tid; i < E; i += kAlignThreads) cnt[i] = 0;
  __syncthreads();
  for (int f = tid; f < A; f += kAlignThreads) {
    const int id = ids[f];
    if (static_cast<unsigned>(id) < static_cast<unsigned>(E)) atomicAdd(&cnt[id], 1);
  }
  __syncthreads();

  int below = 0, all = 0;
  for (int i = tid; i < E; i += kAlignThreads) {
    const int p = (cnt[i] + B - 1) / B * B;
    all += p;
    if (i < e) below += p;
  }
  const int off = block_sum(below, red);
  const int total = block_sum(all, red);
  const int mine = cnt[e];
  const int padded = (mine + B - 1) / B * B;

  // 3. ordered compaction of this expert's slots
  int running = 0;
  for (int base = 0; base < A; base += kAlignThreads) {
    const int f = base + tid;
    const bool hit = f < A && ids[f] == e;
    const uint64_t mask = __ballot(hit);
    const int before = __popcll(mask & ((1ull << lane) - 1ull));
    __syncthreads();  // wave_tot reuse
    if (lane == 0) wave_tot[wave] = __popcll(mask);
    __syncthreads();
    int wave_off = 0, chunk = 0;
#pragma unroll
    for (int w = 0; w < kAlignWaves; ++w) {
      wave_off += (w < wave) ? wave_tot[w] : 0;
      chunk += wave_tot[w];
    }
    if (hit) sorted_ids[off + running + wave_off + before] = f;
    running += chunk;
  }
  // 4. pads and block owners of this expert
  for (int r = mine + tid; r < padded; r += kAlignThreads) sorted_ids[off + r] = A;
  for (int b = tid; b < padded / B; b += kAlignThreads) block_expert[off / B + b] = e;

  if (e == 0) {
    for (int i = tid; i < E; i += kAlignThreads) counts[i] = cnt[i];
    if (tid == 0) *num_padded = total;
    for (int r = total + tid; r < cap; r += kAlignThreads) sorted_ids[r] = A;
    for (int b = total / B + tid; b < cap / B; b += kAlignThreads) block_expert[b] = -1;
  }
}

hipError_t launch_align(const int32_t* ids, int A, int E, int B, int cap, int32_t* counts,
                        int32_t* sorted_ids, int32_t* block_expert, int32_t* num_padded,
                        hipStream_t s) {
  align_kernel<<<E, kAlignThreads, 0, s>>>(ids, A, E, B, cap, counts, sorted_ids, block_expert,
                                           num_padded);
  return hipGetLastError();
}

}  // namespace moe
