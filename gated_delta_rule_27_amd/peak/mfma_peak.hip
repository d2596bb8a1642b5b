// mfma_peak.hip — achievable dense bf16 matrix-core throughput on gfx950, the
// measured ceiling beside the datasheet peak for the chunk kernels' matrix-core
// fraction.  Not part of the linear-attention library: bench.py loads it
// (libmfmapeak.so) on its own.
//
// Every wave runs `iters` rounds of NCH independent accumulation chains of one
// MFMA shape, operands held in registers (no memory traffic inside the loop),
// and writes one float per lane at the end so nothing is dead code.  FLOP per
// launch = grid * waves per workgroup * iters * NCH * (2 M N K of the shape).
#include <hip/hip_runtime.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

namespace {

constexpr int kThreads = 256;   // 4 waves: one per SIMD

// v_mfma_f32_16x16x32_bf16: 16 * 16 * 32 * 2 = 16384 FLOP per instruction
template <int NCH>
__global__ __launch_bounds__(kThreads) void peak_16x16x32(int iters, float* out)
{
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = static_cast<__bf16>(0.001f * (lane + i));
        b[i] = static_cast<__bf16>(0.002f * (63 - lane + i));
    }
    floatx4 acc[NCH];
#pragma unroll
    for (int j = 0; j < NCH; ++j) acc[j] = floatx4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < NCH; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < NCH; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    out[blockIdx.x * kThreads + threadIdx.x] = s;
}

// v_mfma_f32_32x32x16_bf16: 32 * 32 * 16 * 2 = 32768 FLOP per instruction
template <int NCH>
__global__ __launch_bounds__(kThreads) void peak_32x32x16(int iters, float* out)
{
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = static_cast<__bf16>(0.001f * (lane + i));
        b[i] = static_cast<__bf16>(0.002f * (63 - lane + i));
    }
    floatx16 acc[NCH];
#pragma unroll
    for (int j = 0; j < NCH; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < NCH; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < NCH; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += acc[j][e];
    out[blockIdx.x * kThreads + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Threads per workgroup of both kernels (out needs grid * this floats).
int mfma_peak_threads(void) { return kThreads; }

// FLOP one launch performs: grid workgroups of 4 waves, `iters` rounds of 8
// chains; shape 0 = 16x16x32, 1 = 32x32x16 (both bf16, fp32 accumulate).
double mfma_peak_flops(int shape, int grid, int iters)
{
    const double per = shape == 0 ? 16.0 * 16 * 32 * 2 : 32.0 * 32 * 16 * 2;
    return per * 8 * iters * (double)grid * (kThreads / 64);
}

// Enqueue one launch on `stream`; returns 0 on success, else the HIP error.
int mfma_peak_launch(int shape, int grid, int iters, float* out, void* stream)
{
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (grid <= 0 || iters <= 0 || !out) return (int)hipErrorInvalidValue;
    if (shape == 0)
        hipLaunchKernelGGL(peak_16x16x32<8>, dim3(grid), dim3(kThreads), 0, s, iters, out);
    else
        hipLaunchKernelGGL(peak_32x32x16<8>, dim3(grid), dim3(kThreads), 0, s, iters, out);
    return (int)hipGetLastError();
}

}  // extern "C"
