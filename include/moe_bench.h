/*
 * moe_bench.h -- attainable rates of the GPU for the bounds the fused
 * MoE layer's kernels meet, measured on the device itself, so that a
 * kernel's roofline fraction can be read against what the chip delivers as
 * well as against its published peaks.  Measurement support, not part of the
 * layer: each call launches its own kernels, times them with HIP events on
 * `stream` and synchronises that stream before returning.
 *
 * Statuses are those of moe.h (0 = OK, MOE_ERR_NULL_PTR, MOE_ERR_BAD_ARG,
 * MOE_ERR_HIP); arguments are checked before any HIP call.
 */
#ifndef MOE_BENCH_H_
#define MOE_BENCH_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define MOE_BENCH_API __attribute__((visibility("default")))
#else
#define MOE_BENCH_API
#endif

/* Streaming HBM read: reads `bytes` bytes of the device buffer `buf` (a
 * caller-owned device allocation, 16-byte aligned, bytes a positive multiple
 * of 32 KiB and larger than the 256 MB last-level cache for a meaningful
 * figure) with the access pattern the layer's weight streaming uses at best:
 * direct-to-LDS 16-byte loads, 1 KB contiguous per instruction, nontemporal.
 * Runs `reps` >= 2 times and writes the best rate after the first, in GB/s
 * (1e9 bytes), to *gbps.  The buffer is only read; nothing is allocated. */
MOE_BENCH_API int moe_bench_hbm_read(const void* buf, size_t bytes, int reps, double* gbps,
                                     void* stream);

/* bf16 matrix-core rate of an LDS-fed register-tiled loop, the inner loop of
 * the layer's large-tile GEMM: eight waves per CU, 128 x 64 accumulator tile
 * per wave on v_mfma_f32_16x16x32_bf16, operands read from XOR-swizzled LDS
 * rows, one barrier per 64 of K, operand data random bf16 (the rate depends
 * on how many bits toggle).  `iters` >= 2 loop iterations (of 64 K) per
 * workgroup, one workgroup per CU; best of `reps` >= 2 runs after the first,
 * in TFLOP/s (1e12), to *tflops.  Allocates nothing. */
MOE_BENCH_API int moe_bench_mfma_bf16(int iters, int reps, double* tflops, void* stream);

/* The same for the W8A8 large tile's loop: e4m3fn operands (random codes,
 * no NaN) on v_mfma_scale_f32_16x16x128_f8f6f4 with unit block scales, one
 * k-step of 128 and one barrier per iteration; `iters` >= 2 iterations per
 * workgroup.  TFLOP/s to *tflops.  Allocates nothing. */
MOE_BENCH_API int moe_bench_mfma_fp8(int iters, int reps, double* tflops, void* stream);

/* Numerics probe of the scaled fp8 matrix-core instruction the W8A8 tile
 * uses (v_mfma_scale_f32_16x16x128_f8f6f4, unit block scales): for each of
 * `n` trials, c[t] + sum_k A[t,k] * B[t,k] as the instruction computes
 * it, A and B [n, 128] e4m3fn codes (device buffers, 16-byte aligned), c
 * [n] fp32; out [n, 256] fp32 (16-byte aligned) receives all 256 outputs of
 * the trial's 16 x 16 tile, which all hold that one dot product.  Lets a test pin how the
 * instruction accumulates (the parity bounds of the W8A8 mode rest on it).
 * Synchronises `stream` before returning.  Allocates nothing. */
MOE_BENCH_API int moe_bench_fp8_dot(const void* a, const void* b, const float* c, float* out,
                                    int n, void* stream);

#ifdef __cplusplus
}
#endif

#endif  // MOE_BENCH_H_
