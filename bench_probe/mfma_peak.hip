// Matrix-core ceiling of the part, for the projection's roofline: the
// projection's MFMA (v_mfma_f32_32x32x16_bf16) issued back to back from
// registers, with no memory traffic inside the timed loop, 8 waves per CU as
// the projection runs them.  Two operand modes:
//   * changing: bf16 values in +-[1, 2) whose sign and mantissa bits are
//     re-drawn every step (a GEMM's fragments change every k-step; the
//     part's power draw, and so its clock, depends on the toggling bits);
//   * zero: all-zero operands (the spec clock is reachable here).
// Each workgroup also reads the shader clock and the constant-rate wall
// clock at its start and end, so the host can report the clock the loop ran
// at.  A third loop feeds the same MFMA from LDS as the projection does
// (below).  Measurement support for the bench; not part of the Engram path.
#include <hip/hip_runtime.h>

#include <cstdint>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

namespace {

constexpr int kThreads = 512;  // 8 waves, two per SIMD
constexpr int kAcc = 8;        // independent accumulators per wave

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__global__ void __launch_bounds__(kThreads, 1)
mfma_loop(const uint4* __restrict__ seed, float* __restrict__ sums, uint64_t* __restrict__ clocks,
          int iters, int zero) {
    const int tid = blockIdx.x * kThreads + threadIdx.x;
    // operand bit patterns: sign and mantissa from the seed, exponent 127
    uint4 a = seed[2 * tid], b = seed[2 * tid + 1];
    const uint32_t keep = zero ? 0u : 0x807F807Fu, one = zero ? 0u : 0x3F803F80u;
    a = make_uint4((a.x & keep) | one, (a.y & keep) | one, (a.z & keep) | one, (a.w & keep) | one);
    b = make_uint4((b.x & keep) | one, (b.y & keep) | one, (b.z & keep) | one, (b.w & keep) | one);
    uint32_t m = seed[2 * tid].x | 1u;
    f32x16 acc[kAcc];
#pragma unroll
    for (int j = 0; j < kAcc; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[j][v] = 0.0f;
    __syncthreads();
    const uint64_t c0 = clock64(), w0 = wall_clock64();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < kAcc; ++j)
            acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), acc[j],
                                                              0, 0, 0);
        // next step's operands: flip a fresh draw of sign and mantissa bits
        m = m * 1664525u + 1013904223u;
        const uint32_t f = m & keep;
        a = make_uint4(a.x ^ f, a.y ^ (f >> 1 & keep), a.z ^ (f << 1 & keep), a.w ^ ~f & keep);
        b = make_uint4(b.x ^ (f >> 2 & keep), b.y ^ f, b.z ^ (f << 2 & keep), b.w ^ (f >> 3 & keep));
    }
    __syncthreads();
    const uint64_t c1 = clock64(), w1 = wall_clock64();
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < kAcc; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) s += acc[j][v];
    sums[tid] = s;  // keeps the loop's results live
    if (threadIdx.x == 0) {
        clocks[2 * blockIdx.x] = c1 - c0;
        clocks[2 * blockIdx.x + 1] = w1 - w0;
    }
}

// The same MFMA fed the way the projection's k-loop feeds it, with no global
// traffic: 128 KiB of the projection's own W values are staged in LDS once,
// then per k-step of 8 MFMAs every wave reads the next k-step's 4 W and
// (every other k-step) 2 A fragments, 16 bytes per lane, from LDS into
// double-buffered operand registers.  This prices the fragment traffic
// (LDS bandwidth and its power) that any LDS-staged GEMM tile of this shape
// pays on top of the bare matrix-core work.
constexpr int kLdsChunks = 8192;  // 16-byte chunks, 128 KiB

__global__ void __launch_bounds__(kThreads, 1)
mfma_lds_loop(const uint4* __restrict__ src, long src_chunks, float* __restrict__ sums,
              uint64_t* __restrict__ clocks, int iters) {
    __shared__ uint4 lds[kLdsChunks];
    for (int i = threadIdx.x; i < kLdsChunks; i += kThreads)
        lds[i] = src[((long)blockIdx.x * kLdsChunks + i) % src_chunks];
    __syncthreads();
    const int tid = blockIdx.x * kThreads + threadIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int base = (wave * 1024 + lane) & (kLdsChunks - 1);  // distinct 16-byte slots per lane
    uint4 fw[2][4], fa[2][2];
#pragma unroll
    for (int j = 0; j < 4; ++j) fw[0][j] = lds[(base + 64 * j) & (kLdsChunks - 1)];
#pragma unroll
    for (int i = 0; i < 2; ++i) fa[0][i] = lds[(base + 512 + 64 * i) & (kLdsChunks - 1)];
    f32x16 acc[4][2];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[j][i][v] = 0.0f;
    __syncthreads();
    const uint64_t c0 = clock64(), w0 = wall_clock64();
    int off = 0;
    for (int it = 0; it < iters; it += 2) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            off = (off + 256) & 4095;
#pragma unroll
            for (int j = 0; j < 4; ++j) fw[u ^ 1][j] = lds[(base + off + 64 * j) & (kLdsChunks - 1)];
            if (u == 0)
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    fa[1][i] = lds[(base + off + 4096 + 64 * i) & (kLdsChunks - 1)];
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        as_bf16x8(fw[u][j]), as_bf16x8(fa[u][i]), acc[j][i], 0, 0, 0);
            if (u == 1) {
                fa[0][0] = fa[1][0];
                fa[0][1] = fa[1][1];
            }
        }
    }
    __syncthreads();
    const uint64_t c1 = clock64(), w1 = wall_clock64();
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) s += acc[j][i][v];
    sums[tid] = s;
    if (threadIdx.x == 0) {
        clocks[2 * blockIdx.x] = c1 - c0;
        clocks[2 * blockIdx.x + 1] = w1 - w0;
    }
}

}  // namespace

extern "C" {

// Flops of one call: blocks * 8 waves * iters * kAcc MFMAs of 32x32x16.
double engram_probe_mfma_flops(int blocks, int iters) {
    return (double)blocks * (kThreads / 64) * (double)iters * kAcc * 2.0 * 32 * 32 * 16;
}

// seed: device, blocks * 512 * 2 uint4 (32 bytes per thread); sums: device,
// blocks * 512 floats; clocks: device, blocks * 2 uint64 (shader-clock and
// wall-clock ticks of each workgroup's loop).  Returns 0, or a hipError_t.
int engram_probe_mfma(const void* seed, float* sums, uint64_t* clocks, int blocks, int iters,
                      int zero, hipStream_t stream) {
    if (!seed || !sums || !clocks || blocks < 1 || iters < 1) return (int)hipErrorInvalidValue;
    mfma_loop<<<dim3(blocks), dim3(kThreads), 0, stream>>>(
        reinterpret_cast<const uint4*>(seed), sums, clocks, iters, zero);
    return (int)hipGetLastError();
}

// Flops of one mfma_lds_loop call: blocks * 8 waves * iters k-steps of 8
// MFMAs of 32x32x16 (iters even).
double engram_probe_mfma_lds_flops(int blocks, int iters) {
    return (double)blocks * (kThreads / 64) * (double)iters * 8 * 2.0 * 32 * 32 * 16;
}

// src: device, src_bytes of bf16 operand values (at least 16 bytes, a
// multiple of 16); sums and clocks as for engram_probe_mfma.
int engram_probe_mfma_lds(const void* src, size_t src_bytes, float* sums, uint64_t* clocks,
                          int blocks, int iters, hipStream_t stream) {
    if (!src || src_bytes < 16 || src_bytes % 16 || !sums || !clocks || blocks < 1 || iters < 2 ||
        iters % 2)
        return (int)hipErrorInvalidValue;
    mfma_lds_loop<<<dim3(blocks), dim3(kThreads), 0, stream>>>(
        reinterpret_cast<const uint4*>(src), (long)(src_bytes / 16), sums, clocks, iters);
    return (int)hipGetLastError();
}

// Ticks per second of the wall clock read by the probe.
int engram_probe_wall_clock_hz(int64_t* hz) {
    int dev = 0, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess)
        return 1;
    *hz = (int64_t)khz * 1000;
    return 0;
}

}  // extern "C"
