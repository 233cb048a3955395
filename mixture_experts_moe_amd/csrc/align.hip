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
//   3. it walks the slots in order, four consecutive slots per thread, and
//      compacts those routed to its expert: each thread's hit count goes
//      through a wave prefix sum and per-wave offsets in LDS, so a hit's
//      position is its rank in slot order and the result is deterministic;
//   4. it writes its pad entries and its block owners.
// A workgroup is 1024 threads when there are more than 2048 slots, so a pass
// covers 4096 slots and T = 4096, k = 2 takes two passes (with one slot per
// thread and 256 threads it took 32); small batches keep 256 threads, which
// start sooner.
// Workgroup 0 also writes counts, the padded total and the tail past it.

#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kAlignSlots = 4;  // consecutive slots per thread in the compaction

// Inclusive prefix sum over the wave's lanes (lane order).
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int u = __shfl_up(v, d, kWave);
    if (lane >= d) v += u;
  }
  return v;
}

template <int kAlignWaves>
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

template <int kAlignThreads>
__global__ __launch_bounds__(kAlignThreads) void align_kernel(
    const int32_t* __restrict__ ids, int A, int E, int B, int cap, int32_t* __restrict__ counts,
    int32_t* __restrict__ sorted_ids, int32_t* __restrict__ block_expert,
    int32_t* __restrict__ num_padded, int32_t* __restrict__ zero, int nzero) {
  constexpr int kAlignWaves = kAlignThreads / kWave;
  __shared__ int cnt[kMaxExperts];
  __shared__ int red[kAlignWaves];
  __shared__ int wave_tot[kAlignWaves];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int e = blockIdx.x;

  if (e == 0)  // the next kernels' work-queue counters (none: nzero = 0)
    for (int i = tid; i < nzero; i += kAlignThreads) zero[i] = 0;
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
  const int off = block_sum<kAlignWaves>(below, red);
  const int total = block_sum<kAlignWaves>(all, red);
  const int mine = cnt[e];
  const int padded = (mine + B - 1) / B * B;

  // 3. ordered compaction of this expert's slots: thread tid of a pass owns
  // slots f0 .. f0 + 3, f0 = base + 4 tid, so thread order is slot order
  int running = 0;
  for (int base = 0; base < A; base += kAlignThreads * kAlignSlots) {
    const int f0 = base + kAlignSlots * tid;
    int id[kAlignSlots];
    if (f0 + kAlignSlots <= A) {
      const int4 v = *reinterpret_cast<const int4*>(ids + f0);  // f0 % 4 == 0, ids 16-byte aligned
      id[0] = v.x;
      id[1] = v.y;
      id[2] = v.z;
      id[3] = v.w;
    } else {
#pragma unroll
      for (int j = 0; j < kAlignSlots; ++j) id[j] = f0 + j < A ? ids[f0 + j] : -1;
    }
    int hits = 0;
#pragma unroll
    for (int j = 0; j < kAlignSlots; ++j) hits += id[j] == e;
    const int incl = wave_incl_scan(hits);
    __syncthreads();  // wave_tot reuse
    if (lane == kWave - 1) wave_tot[wave] = incl;
    __syncthreads();
    int wave_off = 0, chunk = 0;
#pragma unroll
    for (int w = 0; w < kAlignWaves; ++w) {
      wave_off += (w < wave) ? wave_tot[w] : 0;
      chunk += wave_tot[w];
    }
    int pos = off + running + wave_off + incl - hits;
#pragma unroll
    for (int j = 0; j < kAlignSlots; ++j)
      if (id[j] == e) sorted_ids[pos++] = f0 + j;
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
                        hipStream_t s, int32_t* zero, int nzero) {
  if (nzero > 0 && !zero) return hipErrorInvalidValue;
  if (A > 2048)
    align_kernel<1024><<<E, 1024, 0, s>>>(ids, A, E, B, cap, counts, sorted_ids, block_expert,
                                          num_padded, zero, nzero);
  else
    align_kernel<256><<<E, 256, 0, s>>>(ids, A, E, B, cap, counts, sorted_ids, block_expert,
                                        num_padded, zero, nzero);
  return hipGetLastError();
}

}  // namespace moe
