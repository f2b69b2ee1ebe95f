// MFMA ceiling probe (libtdg_probe.so): the per-wave MFMA streams of the
// 256 x 256 GEMM kernels (16x16x32 bf16; scaled 32x32x64 E4M3) with the
// operands held in registers, timed to give the rate the matrix cores sustain
// on a given operand distribution at the clock the chip holds under that load.  Interface and buffer layout are
// described in tdg_probe.h beside this file.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tdg_probe.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kLanes = 512;       // threads per workgroup: 8 waves, 2 per SIMD
constexpr int kFragments = 24;    // 2 K sub-steps x (8 A + 4 B)
constexpr int kWaveRows = 8;      // 16-row accumulator tiles per wave (128 rows)
constexpr int kWaveCols = 4;      // 16-column accumulator tiles per wave (64 columns)

__global__ __launch_bounds__(kLanes) void mfma_stream_kernel(const bf16x8 *__restrict__ ops, int64_t iters,
                                                             float *__restrict__ sink,
                                                             uint64_t *__restrict__ clocks) {
    const int t = threadIdx.x;
    bf16x8 a[2][kWaveRows], b[2][kWaveCols];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int i = 0; i < kWaveRows; ++i) a[s][i] = ops[(s * 12 + i) * kLanes + t];
#pragma unroll
        for (int j = 0; j < kWaveCols; ++j) b[s][j] = ops[(s * 12 + kWaveRows + j) * kLanes + t];
    }
    f32x4 acc[kWaveRows][kWaveCols];
#pragma unroll
    for (int i = 0; i < kWaveRows; ++i)
#pragma unroll
        for (int j = 0; j < kWaveCols; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const uint64_t c0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int i = 0; i < kWaveRows; ++i)
#pragma unroll
                for (int j = 0; j < kWaveCols; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[s][i], b[s][j], acc[i][j], 0, 0, 0);
    }
    const uint64_t c1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();

    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < kWaveRows; ++i)
#pragma unroll
        for (int j = 0; j < kWaveCols; ++j) sum += (acc[i][j][0] + acc[i][j][1]) + (acc[i][j][2] + acc[i][j][3]);
    sink[(int64_t)blockIdx.x * kLanes + t] = sum;
    if (clocks != nullptr && t == 0) {
        clocks[2 * (int64_t)blockIdx.x] = c1 - c0;
        clocks[2 * (int64_t)blockIdx.x + 1] = r1 - r0;
    }
}

// The 8-bit kernel's per-wave stream: a 128 x 64 wave tile as 4 x 2 tiles of
// 32 x 32 fp32, two K sub-steps of 64 per K tile of 128, each sub-step taking
// 4 A and 2 B fragments of 32 bytes (E4M3 both, unit block scales).
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
constexpr int kF8Fragments = 12;  // 2 K sub-steps x (4 A + 2 B)

__global__ __launch_bounds__(kLanes) void mfma_stream_f8_kernel(const i32x8 *__restrict__ ops, int64_t iters,
                                                                float *__restrict__ sink,
                                                                uint64_t *__restrict__ clocks) {
    const int t = threadIdx.x;
    i32x8 a[2][4], b[2][2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int i = 0; i < 4; ++i) a[s][i] = ops[(s * 6 + i) * kLanes + t];
#pragma unroll
        for (int j = 0; j < 2; ++j) b[s][j] = ops[(s * 6 + 4 + j) * kLanes + t];
    }
    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
    const uint64_t c0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b[s][j], a[s][i], acc[i][j], 0, 0, 0,
                                                                               127, 0, 127);
    }
    const uint64_t c1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; e += 2) sum += acc[i][j][e] + acc[i][j][e + 1];
    sink[(int64_t)blockIdx.x * kLanes + t] = sum;
    if (clocks != nullptr && t == 0) {
        clocks[2 * (int64_t)blockIdx.x] = c1 - c0;
        clocks[2 * (int64_t)blockIdx.x + 1] = r1 - r0;
    }
}

// One MFMA of each kind the kernels use, on one wave, for pinning the lane
// maps: lane l passes its 32-byte X and Y operand slots (the first 16 bytes
// for the 16-bit kinds) and, for the scaled kind, its scale bytes; every
// accumulator register starts at zero and is written to d[l * 16 + r].
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x8 __attribute__((ext_vector_type(8)));

template <int KIND>
__global__ __launch_bounds__(64) void mfma_lanes_kernel(const u32x8 *__restrict__ x, const u32x8 *__restrict__ y,
                                                        const uint8_t *__restrict__ sx,
                                                        const uint8_t *__restrict__ sy, float *__restrict__ d) {
    const int l = threadIdx.x;
    const u32x8 xv = x[l], yv = y[l];
    typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
    const u32x4v x4 = {xv[0], xv[1], xv[2], xv[3]}, y4 = {yv[0], yv[1], yv[2], yv[3]};
    if constexpr (KIND <= 1) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if constexpr (KIND == 0)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, x4), __builtin_bit_cast(f16x8, y4),
                                                         acc, 0, 0, 0);
        else
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, x4),
                                                          __builtin_bit_cast(bf16x8, y4), acc, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) d[l * 16 + r] = acc[r];
    } else {
        f32x16 acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.f;
        if constexpr (KIND == 2)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, x4), __builtin_bit_cast(f16x8, y4),
                                                         acc, 0, 0, 0);
        else if constexpr (KIND == 3)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, x4),
                                                          __builtin_bit_cast(bf16x8, y4), acc, 0, 0, 0);
        else
            acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(__builtin_bit_cast(i32x8, xv),
                                                                 __builtin_bit_cast(i32x8, yv), acc, 0, 0, 0,
                                                                 (int)sx[l], 0, (int)sy[l]);
#pragma unroll
        for (int r = 0; r < 16; ++r) d[l * 16 + r] = acc[r];
    }
}

}  // namespace

extern "C" {

int tdgp_mfma_lanes(int kind, const void *x, const void *y, const void *scale_x, const void *scale_y, float *d,
                    void *stream) {
    if (x == nullptr || y == nullptr || d == nullptr) return 1;
    if ((((uintptr_t)x | (uintptr_t)y) & 31) != 0 || ((uintptr_t)d & 3) != 0) return 1;
    if (kind == 4 && (scale_x == nullptr || scale_y == nullptr)) return 1;
    const u32x8 *xv = static_cast<const u32x8 *>(x), *yv = static_cast<const u32x8 *>(y);
    const uint8_t *sx = static_cast<const uint8_t *>(scale_x), *sy = static_cast<const uint8_t *>(scale_y);
    hipStream_t s = static_cast<hipStream_t>(stream);
    switch (kind) {
    case 0: hipLaunchKernelGGL(mfma_lanes_kernel<0>, dim3(1), dim3(64), 0, s, xv, yv, sx, sy, d); break;
    case 1: hipLaunchKernelGGL(mfma_lanes_kernel<1>, dim3(1), dim3(64), 0, s, xv, yv, sx, sy, d); break;
    case 2: hipLaunchKernelGGL(mfma_lanes_kernel<2>, dim3(1), dim3(64), 0, s, xv, yv, sx, sy, d); break;
    case 3: hipLaunchKernelGGL(mfma_lanes_kernel<3>, dim3(1), dim3(64), 0, s, xv, yv, sx, sy, d); break;
    case 4: hipLaunchKernelGGL(mfma_lanes_kernel<4>, dim3(1), dim3(64), 0, s, xv, yv, sx, sy, d); break;
    default: return 1;
    }
    return hipGetLastError() == hipSuccess ? 0 : 3;
}

size_t tdgp_operand_bytes_f8(void) { return (size_t)kF8Fragments * kLanes * 32; }

double tdgp_flops_f8(int64_t iters, int blocks) {
    return 2.0 * 32 * 32 * 64 * 16 * (kLanes / 64) * (double)blocks * (double)iters;
}

int tdgp_mfma_stream_f8(const void *operands, int64_t iters, int blocks, float *sink, uint64_t *clocks,
                        void *stream) {
    if (operands == nullptr || sink == nullptr) return 1;
    if (((uintptr_t)operands & 31) != 0) return 1;
    if (iters < 1 || iters > ((int64_t)1 << 31) || blocks < 1 || blocks > 65536) return 1;
    hipLaunchKernelGGL(mfma_stream_f8_kernel, dim3((unsigned)blocks), dim3(kLanes), 0, (hipStream_t)stream,
                       static_cast<const i32x8 *>(operands), iters, sink, clocks);
    return hipGetLastError() == hipSuccess ? 0 : 3;
}


size_t tdgp_operand_elems(void) { return (size_t)kFragments * kLanes * 8; }

double tdgp_flops(int64_t iters, int blocks) {
    return 2.0 * 16 * 16 * 32 * (2 * kWaveRows * kWaveCols) * (kLanes / 64) * (double)blocks * (double)iters;
}

int tdgp_mfma_stream(const void *operands, int64_t iters, int blocks, float *sink, uint64_t *clocks, void *stream) {
    if (operands == nullptr || sink == nullptr) return 1;
    if (((uintptr_t)operands & 15) != 0) return 1;
    if (iters < 1 || iters > ((int64_t)1 << 31) || blocks < 1 || blocks > 65536) return 1;
    hipLaunchKernelGGL(mfma_stream_kernel, dim3((unsigned)blocks), dim3(kLanes), 0, (hipStream_t)stream,
                       static_cast<const bf16x8 *>(operands), iters, sink, clocks);
    return hipGetLastError() == hipSuccess ? 0 : 3;
}

}  // extern "C"
