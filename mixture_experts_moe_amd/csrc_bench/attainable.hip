// Attainable-rate kernels behind include/moe_bench.h: a streaming HBM read in
// the layer's best weight-streaming pattern, and the large-tile GEMMs'
// LDS-fed MFMA loops (bf16, and e4m3fn with block scales) on random data.
// Measurement support only.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"
#include "moe_bench.h"

// Sinks the kernels store to (device code only; never read back).  External
// linkage: with internal linkage the compiler may drop stores nobody reads,
// and the work feeding them with the stores.
__device__ __attribute__((used)) uint32_t moe_bench_sink_word[64];
__device__ __attribute__((used)) float moe_bench_sink_float[64];

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// ------------------------------------------------------------ HBM read
// One wave per workgroup reads one 32 KB chunk: 32 direct-to-LDS loads of
// 1 KB contiguous each (nontemporal), then waits.  The LDS contents are
// folded into one word so that nothing is dead; the word is stored only if it
// equals a value the fill never makes.
constexpr int kChunk = 32 * 1024;

__global__ __launch_bounds__(64) void hbm_read_kernel(const uint8_t* __restrict__ base) {
  __shared__ __attribute__((aligned(1024))) uint8_t buf[kChunk];
  const int l = threadIdx.x;
  const uint8_t* src = base + static_cast<size_t>(blockIdx.x) * kChunk + 16 * l;
#pragma unroll
  for (int i = 0; i < 32; ++i) __builtin_amdgcn_global_load_lds(src + 1024 * i, buf + 1024 * i, 16, 0, 2);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const uint32_t v = reinterpret_cast<const uint32_t*>(buf)[l * 7];
  if (v == 0x9e3779b9u) moe_bench_sink_word[l] = v;
}

// ------------------------------------------------------------ MFMA loop
// LDS: 512 rows of 128 bytes (64 bf16 of K), 16-byte slots XOR-swizzled by
// row as in the large-tile GEMM.  Wave w of 8: rows of A from 128 (w & 1),
// of B from 256 + 64 (w >> 1); per iteration two k-steps of 32, fragments of
// the next k-step read before the current one's 32 MFMAs, one barrier.
constexpr int kMmaWaves = 8;

__device__ __forceinline__ bf16x8 frag(const uint8_t* buf, int row, int slot) {
  row &= 511;
  return __builtin_bit_cast(
      bf16x8, *reinterpret_cast<const uint4*>(buf + row * 128 + ((slot ^ ((row >> 1) & 7)) << 4)));
}

__global__ __launch_bounds__(64 * kMmaWaves) void mfma_loop_kernel(int iters) {
  __shared__ __attribute__((aligned(1024))) uint8_t buf[64 * 1024];
  const int tid = threadIdx.x, lane = tid & 63, r16 = lane & 15, g = lane >> 4, wave = tid >> 6;
  // random bf16 of magnitude 2^-7 .. 2^-6, both signs (a multiplicative hash)
  for (int i = tid; i < 4096; i += 64 * kMmaWaves) {
    uint32_t h = static_cast<uint32_t>(i) * 2654435761u + 12345u;
    uint32_t w[4];
    for (int q = 0; q < 4; ++q) {
      w[q] = ((h ^ (h >> 13)) & 0x807f807fu) | 0x3c003c00u;
      h = h * 1664525u + 1013904223u;
    }
    reinterpret_cast<uint4*>(buf)[i] = uint4{w[0], w[1], w[2], w[3]};
  }
  __syncthreads();
  const int abase = 128 * (wave & 1), bbase = 256 + 64 * (wave >> 1);
  f32x4 acc[8][4];
  for (int t = 0; t < 8; ++t)
    for (int u = 0; u < 4; ++u) acc[t][u] = f32x4{0.f, 0.f, 0.f, 0.f};
  bf16x8 a[2][8], b[2][4];
  for (int t = 0; t < 8; ++t) a[0][t] = frag(buf, abase + 16 * t + r16, g);
  for (int u = 0; u < 4; ++u) b[0][u] = frag(buf, bbase + 16 * u + r16, g);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int slot = g + 4 * (p ^ 1);
      const int rot = (it * 32 + 16 * p) & 127;  // walk the rows so reads are not loop-invariant
#pragma unroll
      for (int t = 0; t < 8; ++t) a[p ^ 1][t] = frag(buf, abase + ((16 * t + rot) & 127) + r16, slot);
#pragma unroll
      for (int u = 0; u < 4; ++u) b[p ^ 1][u] = frag(buf, bbase + ((16 * u + rot) & 63) + r16, slot);
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int u = 0; u < 4; ++u)
          acc[t][u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[p][t], b[p][u], acc[t][u], 0, 0, 0);
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }
  float s = 0.f;
  for (int t = 0; t < 8; ++t)
    for (int u = 0; u < 4; ++u) s += acc[t][u][0] + acc[t][u][3];
  if (s == 1234.5f) moe_bench_sink_float[lane] = s;
}

// ------------------------------------------------------------ fp8 MFMA loop
// The W8A8 large tile's inner loop: LDS as above (rows of 128 e4m3fn bytes
// of K), per iteration one k-step of 128: each wave reads its four token
// fragments, then its eight weight fragments in two halves of four, each
// half followed by 16 v_mfma_scale_f32_16x16x128_f8f6f4 (unit E8M0 scales);
// one barrier per iteration.  Random e4m3fn codes of magnitude 0.5 .. 1.875,
// both signs (no NaN code).

__device__ __forceinline__ i32x8 frag8(const uint8_t* buf, int row, int g) {
  row &= 511;
  const uint8_t* r = buf + row * 128;
  const int sw = (row >> 1) & 7;
  const uint4 lo = *reinterpret_cast<const uint4*>(r + ((g ^ sw) << 4));
  const uint4 hi = *reinterpret_cast<const uint4*>(r + (((4 + g) ^ sw) << 4));
  return i32x8{static_cast<int>(lo.x), static_cast<int>(lo.y), static_cast<int>(lo.z),
               static_cast<int>(lo.w), static_cast<int>(hi.x), static_cast<int>(hi.y),
               static_cast<int>(hi.z), static_cast<int>(hi.w)};
}

__global__ __launch_bounds__(64 * kMmaWaves) void mfma_fp8_loop_kernel(int iters) {
  __shared__ __attribute__((aligned(1024))) uint8_t buf[64 * 1024];
  const int tid = threadIdx.x, lane = tid & 63, r16 = lane & 15, g = lane >> 4, wave = tid >> 6;
  for (int i = tid; i < 4096; i += 64 * kMmaWaves) {
    uint32_t h = static_cast<uint32_t>(i) * 2654435761u + 777u;
    uint32_t w[4];
    for (int q = 0; q < 4; ++q) {
      // per byte: sign, mantissa and the exponent field's low bit random (field 6 or 7)
      w[q] = ((h ^ (h >> 11)) & 0x8f8f8f8fu) | 0x30303030u;
      h = h * 1664525u + 1013904223u;
    }
    reinterpret_cast<uint4*>(buf)[i] = uint4{w[0], w[1], w[2], w[3]};
  }
  __syncthreads();
  const int abase = 128 * (wave & 1), bbase = 256 + 64 * (wave >> 1);
  f32x4 acc[8][4];
  for (int t = 0; t < 8; ++t)
    for (int u = 0; u < 4; ++u) acc[t][u] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
    const int rot = (it * 16) & 127;  // walk the rows so reads are not loop-invariant
    i32x8 a[4], b[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) b[u] = frag8(buf, bbase + ((16 * u + rot) & 63) + r16, g);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
        a[t] = frag8(buf, abase + ((64 * half + 16 * t + rot) & 127) + r16, g);
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int u = 0; u < 4; ++u)
          acc[4 * half + t][u] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              a[t], b[u], acc[4 * half + t][u], 0, 0, 0, 127, 0, 127);
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }
  float s = 0.f;
  for (int t = 0; t < 8; ++t)
    for (int u = 0; u < 4; ++u) s += acc[t][u][0] + acc[t][u][3];
  if (s == 1234.5f) moe_bench_sink_float[lane] = s;
}

template <class F>
int best_ms(hipStream_t s, int reps, F&& launch, float* best) {
  hipEvent_t a, b;
  if (hipEventCreate(&a) != hipSuccess) return MOE_ERR_HIP;
  if (hipEventCreate(&b) != hipSuccess) {
    (void)hipEventDestroy(a);
    return MOE_ERR_HIP;
  }
  int st = MOE_OK;
  *best = 0.f;
  for (int r = 0; r < reps && st == MOE_OK; ++r) {
    float ms = 0.f;
    if (hipEventRecord(a, s) != hipSuccess || (launch(), hipGetLastError()) != hipSuccess ||
        hipEventRecord(b, s) != hipSuccess || hipEventSynchronize(b) != hipSuccess ||
        hipEventElapsedTime(&ms, a, b) != hipSuccess)
      st = MOE_ERR_HIP;
    else if (r > 0 && (*best == 0.f || ms < *best))
      *best = ms;
  }
  (void)hipEventDestroy(a);
  (void)hipEventDestroy(b);
  if (st == MOE_OK && *best <= 0.f) st = MOE_ERR_HIP;
  return st;
}

// ------------------------------------------------------------ fp8 dot probe
// One wave per trial: the trial's 128-byte A row and B column (e4m3fn codes,
// K in byte order) are given to every row and column of one
// v_mfma_scale_f32_16x16x128_f8f6f4 with unit block scales and accumulator
// input c[t], so all 256 outputs are the same dot product.  Lane l supplies
// K bytes 16(l/16)..+15 and 64 + 16(l/16)..+15 of both operands; every load
// lies inside the trial's 128 bytes.  Every lane stores its four outputs
// (out[t, 4l .. 4l + 3]): with a store by lane 0 alone the compiler moved the
// MFMA under that lane's branch, where it ran with one lane enabled.
__global__ __launch_bounds__(64) void fp8_dot_kernel(const uint8_t* __restrict__ a,
                                                     const uint8_t* __restrict__ b,
                                                     const float* __restrict__ c,
                                                     float* __restrict__ out, int n) {
  const int t = blockIdx.x;
  if (t >= n) return;
  const int kg = threadIdx.x / 16;
  const uint8_t* ar = a + static_cast<size_t>(t) * 128;
  const uint8_t* br = b + static_cast<size_t>(t) * 128;
  i32x8 av, bv;
  for (int i = 0; i < 4; ++i) {
    av[i] = *reinterpret_cast<const int*>(ar + 16 * kg + 4 * i);
    av[4 + i] = *reinterpret_cast<const int*>(ar + 64 + 16 * kg + 4 * i);
    bv[i] = *reinterpret_cast<const int*>(br + 16 * kg + 4 * i);
    bv[4 + i] = *reinterpret_cast<const int*>(br + 64 + 16 * kg + 4 * i);
  }
  const float c0 = c[t];
  f32x4 acc = {c0, c0, c0, c0};
  acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc, 0, 0, 0, 127, 0, 127);
  float4* o = reinterpret_cast<float4*>(out + static_cast<size_t>(t) * 256) + threadIdx.x;
  *o = float4{acc[0], acc[1], acc[2], acc[3]};
}

}  // namespace

extern "C" {

MOE_BENCH_API int moe_bench_fp8_dot(const void* a, const void* b, const float* c, float* out,
                                    int n, void* stream) {
  if (!a || !b || !c || !out) return MOE_ERR_NULL_PTR;
  if (n < 1 || reinterpret_cast<uintptr_t>(a) % 16 || reinterpret_cast<uintptr_t>(b) % 16 ||
      reinterpret_cast<uintptr_t>(out) % 16)
    return MOE_ERR_BAD_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  fp8_dot_kernel<<<n, 64, 0, s>>>(static_cast<const uint8_t*>(a), static_cast<const uint8_t*>(b),
                                  c, out, n);
  if (hipGetLastError() != hipSuccess || hipStreamSynchronize(s) != hipSuccess) return MOE_ERR_HIP;
  return MOE_OK;
}

MOE_BENCH_API int moe_bench_hbm_read(const void* buf, size_t bytes, int reps, double* gbps,
                                     void* stream) {
  if (!buf || !gbps) return MOE_ERR_NULL_PTR;
  if (reps < 2 || bytes == 0 || bytes % kChunk != 0 || bytes / kChunk > 0x7fffffffull ||
      reinterpret_cast<uintptr_t>(buf) % 16)
    return MOE_ERR_BAD_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const unsigned grid = static_cast<unsigned>(bytes / kChunk);
  float ms;
  const int st = best_ms(s, reps, [&] {
    hbm_read_kernel<<<grid, 64, 0, s>>>(static_cast<const uint8_t*>(buf));
  }, &ms);
  if (st) return st;
  *gbps = static_cast<double>(bytes) / (ms * 1e-3) / 1e9;
  return MOE_OK;
}

MOE_BENCH_API int moe_bench_mfma_bf16(int iters, int reps, double* tflops, void* stream) {
  if (!tflops) return MOE_ERR_NULL_PTR;
  if (iters < 2 || reps < 2) return MOE_ERR_BAD_ARG;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return MOE_ERR_HIP;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float ms;
  const int st = best_ms(s, reps, [&] {
    mfma_loop_kernel<<<cus, 64 * kMmaWaves, 0, s>>>(iters);
  }, &ms);
  if (st) return st;
  // per workgroup and iteration: 8 waves x 2 k-steps x 32 MFMAs of 16 x 16 x 32
  const double flop = 2.0 * 16 * 16 * 32 * 32 * 2 * kMmaWaves * static_cast<double>(iters) * cus;
  *tflops = flop / (ms * 1e-3) / 1e12;
  return MOE_OK;
}

MOE_BENCH_API int moe_bench_mfma_fp8(int iters, int reps, double* tflops, void* stream) {
  if (!tflops) return MOE_ERR_NULL_PTR;
  if (iters < 2 || reps < 2) return MOE_ERR_BAD_ARG;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return MOE_ERR_HIP;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float ms;
  const int st = best_ms(s, reps, [&] {
    mfma_fp8_loop_kernel<<<cus, 64 * kMmaWaves, 0, s>>>(iters);
  }, &ms);
  if (st) return st;
  // per workgroup and iteration: 8 waves x 32 MFMAs of 16 x 16 x 128
  const double flop = 2.0 * 16 * 16 * 128 * 32 * kMmaWaves * static_cast<double>(iters) * cus;
  *tflops = flop / (ms * 1e-3) / 1e12;
  return MOE_OK;
}

}  // extern "C"
