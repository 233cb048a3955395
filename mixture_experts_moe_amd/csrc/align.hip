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
//
// That costs E passes over the slots.  For large E * A a counting
// sort over slot tiles takes over (align_tiles_kernel): one workgroup per
// tile of consecutive slots; each builds the histogram of all slots and of
// the slots before its tile (a pass over the ids, which are 4 bytes a slot),
// so that it knows every expert's group offset and where its tile's slots of
// each expert start, then places its tile's slots 1024 at a time: a slot's
// rank among its wave's lanes routed to the same expert (a shuffle loop),
// plus the earlier waves' counts for that expert (LDS), plus the earlier
// chunks' counts.  Each workgroup then writes the pads and block owners of
// every gridDim.x-th expert.  The output is the same, slot for slot.

#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kAlignSlots = 4;  // consecutive slots per thread in the compaction
constexpr int kRegPasses = 4;   // passes whose slots stay in registers between the steps

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
  // this thread's slots of pass p: f0 .. f0 + 3, f0 = p * kPassSlots + 4 tid
  // (thread order is slot order inside a pass); with at most kRegPasses
  // passes they are read once, here, and kept in registers for step 3
  constexpr int kPassSlots = kAlignThreads * kAlignSlots;
  const int passes = (A + kPassSlots - 1) / kPassSlots;
  const bool in_regs = passes <= kRegPasses;
  auto read4 = [&](int f0, int (&id)[kAlignSlots]) {
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
  };
  int held[kRegPasses][kAlignSlots];
  if (in_regs) {
#pragma unroll
    for (int p = 0; p < kRegPasses; ++p) {
      if (p < passes) {
        read4(p * kPassSlots + kAlignSlots * tid, held[p]);
      } else {
#pragma unroll
        for (int j = 0; j < kAlignSlots; ++j) held[p][j] = -1;
      }
    }
  }
  __syncthreads();
  if (in_regs) {
#pragma unroll
    for (int p = 0; p < kRegPasses; ++p)
#pragma unroll
      for (int j = 0; j < kAlignSlots; ++j)
        if (static_cast<unsigned>(held[p][j]) < static_cast<unsigned>(E)) atomicAdd(&cnt[held[p][j]], 1);
  } else {
    for (int f = tid; f < A; f += kAlignThreads) {
      const int id = ids[f];
      if (static_cast<unsigned>(id) < static_cast<unsigned>(E)) atomicAdd(&cnt[id], 1);
    }
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
  auto compact = [&](const int (&id)[kAlignSlots], int f0) {
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
  };
  if (in_regs) {
#pragma unroll
    for (int p = 0; p < kRegPasses; ++p)
      if (p < passes) compact(held[p], p * kPassSlots + kAlignSlots * tid);
  } else {
    for (int base = 0; base < A; base += kPassSlots) {
      int id[kAlignSlots];
      read4(base + kAlignSlots * tid, id);
      compact(id, base + kAlignSlots * tid);
    }
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

// ---------------------------------------------------------------- counting sort over slot tiles

constexpr int kTileThreads = 1024;
constexpr int kTileWaves = kTileThreads / kWave;
// The per-expert kernel's cost grows with E * A, the counting sort's with A
// (measured at E = 256: 13 against 27 us at 16384 slots, 105 against 71 us at
// 262144; at E = 1024 and 16384 slots 39 against 57 us): the counting sort
// runs above this many expert-slot pairs.
#ifndef MOE_ALIGN_TILES_FROM
#define MOE_ALIGN_TILES_FROM (24ll << 20)
#endif
constexpr int64_t kAlignTilesFrom = MOE_ALIGN_TILES_FROM;
constexpr int kAlignTileSlots = 2048;                  // slots per tile (about)
constexpr int kAlignMaxTiles = 64;

// Exclusive prefix sum over the workgroup (v: one value per thread); *total
// gets the sum.  `red` holds kTileWaves ints.
__device__ __forceinline__ int tile_excl_scan(int v, int* red, int* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int incl = wave_incl_scan(v);
  __syncthreads();
  if (lane == kWave - 1) red[wave] = incl;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kTileWaves; ++w) {
    before += w < wave ? red[w] : 0;
    all += red[w];
  }
  *total = all;
  return before + incl - v;
}

__global__ __launch_bounds__(kTileThreads) void align_tiles_kernel(
    const int32_t* __restrict__ ids, int A, int E, int B, int cap, int tile,
    int32_t* __restrict__ counts, int32_t* __restrict__ sorted_ids,
    int32_t* __restrict__ block_expert, int32_t* __restrict__ num_padded,
    int32_t* __restrict__ zero, int nzero) {
  __shared__ int all[kMaxExperts];     // slots per expert
  __shared__ int base[kMaxExperts];    // next position of the tile's slots of each expert
  __shared__ int off[kMaxExperts];     // group offset of each expert
  __shared__ int chunk[kMaxExperts];   // the current chunk's slots per expert
  __shared__ int wc[kTileWaves][kMaxExperts];  // per chunk: wave's slots per expert, then their prefix
  __shared__ int red[kTileWaves];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int t0 = blockIdx.x * tile;
  const int t1 = min(A, t0 + tile);

  if (blockIdx.x == 0)  // the next kernels' work-queue counters
    for (int i = tid; i < nzero; i += kTileThreads) zero[i] = 0;
  for (int i = tid; i < E; i += kTileThreads) all[i] = base[i] = 0;
  __syncthreads();
  // 1. histograms of every slot (all) and of the slots before the tile (base)
  for (int f = tid; f < A; f += kTileThreads) {
    const int id = ids[f];
    if (static_cast<unsigned>(id) < static_cast<unsigned>(E)) {
      atomicAdd(&all[id], 1);
      if (f < t0) atomicAdd(&base[id], 1);
    }
  }
  __syncthreads();
  // 2. group offsets: exclusive scan of the block-rounded counts (E <= 1024:
  // one expert per thread)
  const int mine = tid < E ? (all[tid] + B - 1) / B * B : 0;
  int total = 0;
  const int o = tile_excl_scan(mine, red, &total);
  if (tid < E) {
    off[tid] = o;
    base[tid] += o;
    if (blockIdx.x == 0) counts[tid] = all[tid];
  }
  __syncthreads();
  // 3. the tile's slots in order, one chunk of kTileThreads at a time
  for (int c0 = t0; c0 < t1; c0 += kTileThreads) {
    const int f = c0 + tid;
    int id = f < t1 ? ids[f] : -1;
    if (static_cast<unsigned>(id) >= static_cast<unsigned>(E)) id = -1;
    // rank: lanes below this one routed to the same expert; n: all of the
    // wave's lanes routed to it
    int rank = 0, n = 0;
    for (int j = 0; j < kWave; ++j) {
      const int v = __shfl(id, j, kWave);
      rank += (j < lane && v == id) ? 1 : 0;
      n += v == id ? 1 : 0;
    }
    for (int i = tid; i < kTileWaves * E; i += kTileThreads) wc[i / E][i % E] = 0;
    __syncthreads();
    if (id >= 0 && rank == 0) wc[wave][id] = n;  // the wave's first slot of the expert
    __syncthreads();
    for (int e = tid; e < E; e += kTileThreads) {  // prefix over the waves, in place
      int run = 0;
#pragma unroll
      for (int w = 0; w < kTileWaves; ++w) {
        const int c = wc[w][e];
        wc[w][e] = run;
        run += c;
      }
      chunk[e] = run;
    }
    __syncthreads();
    if (id >= 0) sorted_ids[base[id] + wc[wave][id] + rank] = f;
    __syncthreads();
    for (int e = tid; e < E; e += kTileThreads) base[e] += chunk[e];
    __syncthreads();
  }
  // 4. pads and block owners of experts blockIdx.x, blockIdx.x + gridDim.x, ...
  for (int e = blockIdx.x; e < E; e += gridDim.x) {
    const int begin = off[e];
    const int padded = (all[e] + B - 1) / B * B;
    for (int r = all[e] + tid; r < padded; r += kTileThreads) sorted_ids[begin + r] = A;
    for (int b = tid; b < padded / B; b += kTileThreads) block_expert[begin / B + b] = e;
  }
  if (blockIdx.x == 0) {
    if (tid == 0) *num_padded = total;
    for (int r = total + tid; r < cap; r += kTileThreads) sorted_ids[r] = A;
    for (int b = total / B + tid; b < cap / B; b += kTileThreads) block_expert[b] = -1;
  }
}

hipError_t launch_align(const int32_t* ids, int A, int E, int B, int cap, int32_t* counts,
                        int32_t* sorted_ids, int32_t* block_expert, int32_t* num_padded,
                        hipStream_t s, int32_t* zero, int nzero) {
  if (nzero > 0 && !zero) return hipErrorInvalidValue;
  if (static_cast<int64_t>(A) * E > kAlignTilesFrom) {
    // tiles of whole chunks; about kAlignTileSlots slots each, at most kAlignMaxTiles
    const int want = (A + kAlignTileSlots - 1) / kAlignTileSlots;
    const int tiles = want < kAlignMaxTiles ? want : kAlignMaxTiles;
    const int per = (A + tiles - 1) / tiles;
    const int tile = (per + kTileThreads - 1) / kTileThreads * kTileThreads;
    align_tiles_kernel<<<(A + tile - 1) / tile, kTileThreads, 0, s>>>(
        ids, A, E, B, cap, tile, counts, sorted_ids, block_expert, num_padded, zero, nzero);
    return hipGetLastError();
  }
  if (A > 2048)
    align_kernel<1024><<<E, 1024, 0, s>>>(ids, A, E, B, cap, counts, sorted_ids, block_expert,
                                          num_padded, zero, nzero);
  else
    align_kernel<256><<<E, 256, 0, s>>>(ids, A, E, B, cap, counts, sorted_ids, block_expert,
                                        num_padded, zero, nzero);
  return hipGetLastError();
}

}  // namespace moe
