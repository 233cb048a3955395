// Pieces shared by the large-tile grouped GEMMs (bf16 in ffn_gemm_big.hip,
// e4m3fn weights with block-scaled e4m3fn activations in
// ffn_gemm_big8.hip): tile shape, grid rasterisation, the direct-to-LDS
// stage loader, the LDS slot swizzle and the stage barrier.
#pragma once

#include "ffn_common.h"

namespace moe {

// Stage shape: 2 buffers x 2 operands x 256 rows x 128 bytes of K = 128 KB
// LDS (64 K of bf16, or 128 K of e4m3fn, per stage).
constexpr int kBigWaves = 8;              // 128 x 64 per wave, two waves per SIMD
constexpr int kBigWn = kBigWaves / 2;     // waves along the tokens (two along the rows)
constexpr int kBigThreads = 64 * kBigWaves;
constexpr int kBigTokens = 256;  // block size B of this path
constexpr int kBigRows = 256;    // weight rows per tile
constexpr int kBigN = kBigTokens;  // tokens per workgroup tile: the whole block
constexpr int kBigTA = 8;                      // 16-row weight tiles per wave (128 rows)
constexpr int kBigNB = kBigN / (16 * kBigWn);  // 16-token tiles per wave
constexpr int kBigRowBytes = 128;                    // bytes of K per LDS row and stage
constexpr int kBigSlots = kBigRowBytes / 16;         // 16-byte slots per LDS row
constexpr int kBigRowsPerGroup = 1024 / kBigRowBytes;  // rows filled by one 1 KB load
constexpr int kBigGroups = kBigRows / kBigRowsPerGroup / kBigWaves;  // A loads per wave and stage
constexpr int kBigGroupsB = kBigN / kBigRowsPerGroup / kBigWaves;   // B loads per wave and stage
constexpr int kBigLoads = kBigGroups + kBigGroupsB;
constexpr int kBigOperandBytes = kBigRows * kBigRowBytes;
constexpr int kBigStageBytes = kBigOperandBytes + kBigN * kBigRowBytes;
constexpr int kBigStages = 2;  // 2 x 64 KB of the 160 KB LDS
static_assert(kBigStages * kBigStageBytes <= 160 * 1024, "stages fit in LDS");
#ifndef MOE_BIG_ISSUE_FIRST
#define MOE_BIG_ISSUE_FIRST 1
#endif
#ifndef MOE_BIG_RASTER
#define MOE_BIG_RASTER 1
#endif
#ifndef MOE_BIG_GROUP_COLS
#define MOE_BIG_GROUP_COLS 4
#endif
constexpr int kBigXcds = MOE_BIG_RASTER ? 8 : 1;  // 1: plain order, no XCD remap
constexpr int kBigGroupCols = MOE_BIG_GROUP_COLS;

// Slot swizzle: 8 slots per row, rows pair up per bank line, so the 16 rows
// one 16-lane group reads for the same k land in 16 different 16-byte bank
// groups.
__device__ __forceinline__ int big_swz(int row) { return (row >> 1) & 7; }

struct BigTile {
  int b, y;
  bool live;
};

// Same rasterisation as the 128-token GEMM: contiguous runs of the logical
// order per XCD, super-rows of kBigGroupCols channel groups, row block
// slowest inside a super-row.
// kCols channel groups per super-row.
template <int kCols = kBigGroupCols>
__device__ __forceinline__ BigTile big_tile_of(int p, int gx, int gy) {
  const int total = gx * gy;
  const int per_xcd = (total + kBigXcds - 1) / kBigXcds;
  // (a grid larger than 8 per_xcd, sized for more tiles than `total`:
  // workgroups past per_xcd on their XCD have no tile)
  const int l = (p % kBigXcds) * per_xcd + p / kBigXcds;
  BigTile t{0, 0, p / kBigXcds < per_xcd && l < total};
  if (!t.live) return t;
  const int band = kCols * gx;
  const int sr = l / band;
  const int rem = l - sr * band;
  const int cols = min(kCols, gy - sr * kCols);
  t.b = rem / cols;
  t.y = sr * kCols + rem % cols;
  return t;
}

// The raster over the realised row blocks only.  The grid is sized from the
// capacity (gx blocks of bm slots), which also counts blocks that stay
// empty; rasterising over gx would leave the XCDs whose share lies past the
// realised blocks with less work.  Over the count read on the device every
// XCD gets the same number of live tiles, and the workgroups left over
// return.
template <int kCols = kBigGroupCols>
__device__ __forceinline__ BigTile big_tile_live(int p, int gx, int gy,
                                                 const int32_t* num_padded, int bm) {
  return big_tile_of<kCols>(p, min(gx, *num_padded / bm), gy);
}

// Each wave fills kBigGroups consecutive 1 KB groups (kBigRowsPerGroup rows
// each) of an operand per stage: in group q, lane l writes tile row
// 64*wave + kBigRowsPerGroup*q + l/kBigSlots, physical slot l%kBigSlots,
// which holds logical slot (l%kBigSlots) ^ swz(row).  swz(row) depends on q
// only through q's parity, so a lane's weight sources are two bases plus a
// stride; token sources (gathered x rows, or h rows) are one pointer per
// group.
struct BigLoader {
  __amdgpu_buffer_rsrc_t ra;  // weight rows of the tile's expert
  __amdgpu_buffer_rsrc_t rb;  // token rows (x, or the block's h rows)
  uint32_t a_even;            // byte offset of this lane's group-0 source (q even), k = 0
  uint32_t a_odd;             // group 1 (q odd)
  uint32_t a_step;            // bytes between groups q and q + 2
  uint32_t b[kBigGroupsB];    // byte offset of this lane's token source of group q, k = 0

  __device__ __forceinline__ uint32_t a_off(int q, uint32_t kbyte) const {
    return (q & 1 ? a_odd : a_even) + (q >> 1) * a_step + kbyte;
  }
};

// Buffer resource over `bytes` bytes at `base` (raw: stride 0, byte
// offsets; flags word as gfx9-family kernels use for plain dword data).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t big_rsrc(const void* base, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                           0x00020000);
}

// The stage's direct-to-LDS loads go through buffer resources
// (buffer_load ... lds) rather than global_load_lds: with the latter in
// flight the compiler waits for every outstanding LDS read (lgkmcnt(0)) before
// each MFMA group, which undoes the fragment pipelining; the buffer form
// keeps those waits partial.
// kbyte: byte offset along K of the stage (2 * k for bf16, k for e4m3fn).
__device__ __forceinline__ void big_issue(const BigLoader& ld, uint8_t* stage, uint32_t kbyte,
                                          int wave) {
#pragma unroll
  for (int q = 0; q < kBigGroups; ++q)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        ld.ra, (__attribute__((address_space(3))) void*)(stage + (wave * kBigGroups + q) * 1024), 16,
        ld.a_off(q, kbyte), 0, 0, 0);
#pragma unroll
  for (int q = 0; q < kBigGroupsB; ++q)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        ld.rb,
        (__attribute__((address_space(3))) void*)(stage + kBigOperandBytes +
                                                   (wave * kBigGroupsB + q) * 1024),
        16, ld.b[q] + kbyte, 0, 0, 0);
}

// s_waitcnt immediate that waits until at most n vector-memory loads are
// outstanding (lgkm and exp counters not waited on).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Wait for this wave's LDS reads, then meet the other waves.  No memory
// fence: a workgroup-scope fence would also wait for every direct-to-LDS
// load this wave has in flight, later stages' included.  Each wave waits
// explicitly for its own loads of the stage about to be read before it
// arrives; the memory clobber keeps the compiler from moving LDS accesses
// across.
__device__ __forceinline__ void big_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

#define BIG_BUFFERS(name)                                                                 \
  __shared__ __attribute__((aligned(1024))) uint8_t name##0[kBigStageBytes];              \
  __shared__ __attribute__((aligned(1024))) uint8_t name##1[kBigStageBytes];              \
  uint8_t* const name[2] = {name##0, name##1}

}  // namespace moe
