// deltaproduct.hip — Gated DeltaProduct as Gated DeltaNet over a virtual
// sequence ("Linear Attention, Visualized", "Gated Delta Product (GDP)" and
// "GDP as GDN over a virtual sequence").
//
// Each real token t carries n_h substeps (keys k_{t,j}, values v_{t,j},
// correction gates beta_{t,j}); flattened in order they form a GDN sequence of
// n_h T virtual steps in which step (t, j) takes the decay a_t when j is the
// first substep and 1 otherwise, and the query q_t when j is the last substep
// and 0 otherwise; every n_h-th output is kept.  The inputs already store k, v
// and beta as [B,H,T,n_h,...], which is the virtual sequence's own layout, so
// only the query and the log-gate need expanding; the chunk kernels then run
// unchanged, and a gather keeps the outputs of the last substeps.
#include "device_common.h"
#include "launch.h"

namespace linattn {

namespace {

typedef __attribute__((__vector_size__(16))) int i4;

// qv[bh, t nh + j, :] = q[bh, t, :] for j = nh-1, else 0   (16-byte vectors)
// gv[bh, t nh + j]    = g[bh, t] for j = 0, else 0           (one per virtual step)
template <typename T>
__global__ __launch_bounds__(256) void dp_expand_kernel(const T* __restrict__ q, const T* __restrict__ g,
                                                        T* __restrict__ qv, T* __restrict__ gv,
                                                        int64_t rows, int nh, int dk)
{
    constexpr int E = 16 / sizeof(T);
    const int vpr = dk / E;                                  // vectors per row
    const int64_t nvec = rows * nh * vpr;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nvec; i += stride) {
        const int64_t vrow = i / vpr;                        // virtual step (all heads)
        const int c = (int)(i % vpr);
        const int64_t row = vrow / nh;                       // real token (all heads)
        const int j = (int)(vrow % nh);
        i4 x = {0, 0, 0, 0};
        if (j == nh - 1) x = reinterpret_cast<const i4*>(q)[row * vpr + c];
        reinterpret_cast<i4*>(qv)[i] = x;
        if (g && c == 0) gv[vrow] = j == 0 ? g[row] : from_f32<T>(0.f);
    }
}

// o[bh, t, :] = ov[bh, t nh + nh - 1, :]   (16-byte vectors)
template <typename T>
__global__ __launch_bounds__(256) void dp_gather_kernel(const T* __restrict__ ov, T* __restrict__ o,
                                                        int64_t rows, int nh, int dv)
{
    constexpr int E = 16 / sizeof(T);
    const int vpr = dv / E;
    const int64_t nvec = rows * vpr;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nvec; i += stride) {
        const int64_t row = i / vpr;
        const int c = (int)(i % vpr);
        reinterpret_cast<i4*>(o)[i] = reinterpret_cast<const i4*>(ov)[(row * nh + nh - 1) * vpr + c];
    }
}

// dov[bh, t nh + j, :] = do[bh, t, :] for j = nh-1, else 0 (the gradient of
// the virtual outputs: only the last substep's output is the token's)
template <typename T>
__global__ __launch_bounds__(256) void dp_scatter_kernel(const T* __restrict__ d, T* __restrict__ dv_,
                                                         int64_t rows, int nh, int dv)
{
    constexpr int E = 16 / sizeof(T);
    const int vpr = dv / E;
    const int64_t nvec = rows * nh * vpr;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nvec; i += stride) {
        const int64_t vrow = i / vpr;
        const int c = (int)(i % vpr);
        const int64_t row = vrow / nh;
        const int j = (int)(vrow % nh);
        i4 x = {0, 0, 0, 0};
        if (j == nh - 1) x = reinterpret_cast<const i4*>(d)[row * vpr + c];
        reinterpret_cast<i4*>(dv_)[i] = x;
    }
}

// dst[row, :] = src[row nh + j, :] (width w, 16-byte vectors), and the same
// for one value per row (w == 1)
template <typename T>
__global__ __launch_bounds__(256) void dp_pick_kernel(const T* __restrict__ src, T* __restrict__ dst, int64_t rows,
                                                      int nh, int j, int w)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    if (w == 1) {
        for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < rows; i += stride)
            dst[i] = src[i * nh + j];
        return;
    }
    constexpr int E = 16 / sizeof(T);
    const int vpr = w / E;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < rows * vpr; i += stride) {
        const int64_t row = i / vpr;
        const int c = (int)(i % vpr);
        reinterpret_cast<i4*>(dst)[i] = reinterpret_cast<const i4*>(src)[(row * nh + j) * vpr + c];
    }
}

unsigned grid_for(int64_t n)
{
    const int64_t b = (n + 255) / 256;
    return (unsigned)(b < 4096 ? (b > 0 ? b : 1) : 4096);
}

}  // namespace

hipError_t launch_dp_expand(const DeltaProductProblem& p, hipStream_t s)
{
    const int64_t rows = p.B * p.H * p.T;
    const int64_t nvec = rows * p.nh * p.dk / (p.dtype == kBF16 ? 8 : 4);
    if (p.dtype == kBF16)
        hipLaunchKernelGGL(dp_expand_kernel<bf16>, dim3(grid_for(nvec)), dim3(256), 0, s,
                           static_cast<const bf16*>(p.q), static_cast<const bf16*>(p.g),
                           static_cast<bf16*>(p.qv), static_cast<bf16*>(p.gv), rows, p.nh, p.dk);
    else
        hipLaunchKernelGGL(dp_expand_kernel<float>, dim3(grid_for(nvec)), dim3(256), 0, s,
                           static_cast<const float*>(p.q), static_cast<const float*>(p.g),
                           static_cast<float*>(p.qv), static_cast<float*>(p.gv), rows, p.nh, p.dk);
    return hipGetLastError();
}

hipError_t launch_dp_gather(const DeltaProductProblem& p, hipStream_t s)
{
    const int64_t rows = p.B * p.H * p.T;
    const int64_t nvec = rows * p.dv / (p.dtype == kBF16 ? 8 : 4);
    if (p.dtype == kBF16)
        hipLaunchKernelGGL(dp_gather_kernel<bf16>, dim3(grid_for(nvec)), dim3(256), 0, s,
                           static_cast<const bf16*>(p.ov), static_cast<bf16*>(p.o), rows, p.nh, p.dv);
    else
        hipLaunchKernelGGL(dp_gather_kernel<float>, dim3(grid_for(nvec)), dim3(256), 0, s,
                           static_cast<const float*>(p.ov), static_cast<float*>(p.o), rows, p.nh, p.dv);
    return hipGetLastError();
}

}  // namespace linattn

namespace linattn {

hipError_t launch_dp_scatter(const DeltaProductProblem& p, const void* dout, void* dov, hipStream_t s)
{
    const int64_t rows = p.B * p.H * p.T;
    const int64_t nvec = rows * p.nh * p.dv / (p.dtype == kBF16 ? 8 : 4);
    if (p.dtype == kBF16)
        hipLaunchKernelGGL(dp_scatter_kernel<bf16>, dim3(grid_for(nvec)), dim3(256), 0, s,
                           static_cast<const bf16*>(dout), static_cast<bf16*>(dov), rows, p.nh, p.dv);
    else
        hipLaunchKernelGGL(dp_scatter_kernel<float>, dim3(grid_for(nvec)), dim3(256), 0, s,
                           static_cast<const float*>(dout), static_cast<float*>(dov), rows, p.nh, p.dv);
    return hipGetLastError();
}

hipError_t launch_dp_pick(const void* src, void* dst, int64_t rows, int nh, int j, int w, int dtype, hipStream_t s)
{
    const int64_t n = w == 1 ? rows : rows * w / (dtype == kBF16 ? 8 : 4);
    if (dtype == kBF16)
        hipLaunchKernelGGL(dp_pick_kernel<bf16>, dim3(grid_for(n)), dim3(256), 0, s, static_cast<const bf16*>(src),
                           static_cast<bf16*>(dst), rows, nh, j, w);
    else
        hipLaunchKernelGGL(dp_pick_kernel<float>, dim3(grid_for(n)), dim3(256), 0, s,
                           static_cast<const float*>(src), static_cast<float*>(dst), rows, nh, j, w);
    return hipGetLastError();
}

}  // namespace linattn
