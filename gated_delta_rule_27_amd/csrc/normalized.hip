// normalized.hip — normalised linear attention ("All sorts of famous Attention
// Layers", "Linear Magic": the feature-map attention divided by its
// normaliser): o_t = (q_t S_t) / (q_t . z_t) with z_t = a_t z_{t-1} + k_t.
//
// z evolves exactly like one value column of S whose values are all 1, so the
// denominator is the add-rule output for a value block of ones, with the state
// columns of that block started at z_0.  The library runs the chunk kernels
// twice (values, then ones) and these kernels supply the block of ones and its
// initial state, divide the numerator by the denominator, and return z_T.
#include "device_common.h"
#include "launch.h"

namespace linattn {

namespace {

constexpr int kOnes = 64;   // columns of the value block of ones (the narrowest the chunk kernels take)

unsigned grid_for(int64_t n)
{
    const int64_t b = (n + 255) / 256;
    return (unsigned)(b < 4096 ? (b > 0 ? b : 1) : 4096);
}

template <typename T>
__global__ __launch_bounds__(256) void fill_ones_kernel(T* __restrict__ x, int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        x[i] = from_f32<T>(1.f);
}

// s[bh][i][c] = z0 ? z0[bh][i] : 0 for the kOnes columns c
__global__ __launch_bounds__(256) void broadcast_z_kernel(const float* __restrict__ z0, float* __restrict__ s,
                                                          int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        s[i] = z0 ? z0[i / kOnes] : 0.f;
}

// o[row][c] = o[row][c] / den[row][0]
template <typename T>
__global__ __launch_bounds__(256) void divide_kernel(T* __restrict__ o, const T* __restrict__ den, int64_t rows,
                                                     int dv)
{
    const int64_t n = rows * dv;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        o[i] = from_f32<T>(to_f32(o[i]) / to_f32(den[(i / dv) * kOnes]));
}

// z[bh][i] = s[bh][i][0]
__global__ __launch_bounds__(256) void column0_kernel(const float* __restrict__ s, float* __restrict__ z, int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) z[i] = s[i * kOnes];
}

}  // namespace

int normalized_ones_columns() { return kOnes; }

hipError_t launch_norm_prepare(const NormalizedProblem& p, hipStream_t s)
{
    const int64_t nones = p.rows * kOnes;
    if (p.dtype == kBF16)
        hipLaunchKernelGGL(fill_ones_kernel<bf16>, dim3(grid_for(nones)), dim3(256), 0, s,
                           static_cast<bf16*>(p.ones), nones);
    else
        hipLaunchKernelGGL(fill_ones_kernel<float>, dim3(grid_for(nones)), dim3(256), 0, s,
                           static_cast<float*>(p.ones), nones);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t ns = p.heads * p.dk * kOnes;
    hipLaunchKernelGGL(broadcast_z_kernel, dim3(grid_for(ns)), dim3(256), 0, s, p.z0, p.s0_den, ns);
    return hipGetLastError();
}

hipError_t launch_norm_finish(const NormalizedProblem& p, hipStream_t s)
{
    const int64_t n = p.rows * p.dv;
    if (p.rows > 0) {
        if (p.dtype == kBF16)
            hipLaunchKernelGGL(divide_kernel<bf16>, dim3(grid_for(n)), dim3(256), 0, s, static_cast<bf16*>(p.o),
                               static_cast<const bf16*>(p.den), p.rows, p.dv);
        else
            hipLaunchKernelGGL(divide_kernel<float>, dim3(grid_for(n)), dim3(256), 0, s,
                               static_cast<float*>(p.o), static_cast<const float*>(p.den), p.rows, p.dv);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (p.z_final) {
        const int64_t nz = p.heads * p.dk;
        hipLaunchKernelGGL(column0_kernel, dim3(grid_for(nz)), dim3(256), 0, s, p.sf_den, p.z_final, nz);
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace linattn
