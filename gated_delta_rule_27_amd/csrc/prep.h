// prep.h — input preparation from raw projections, applied by the chunk
// kernels while they stage tokens, so that the prepared q, k, log-gate and
// beta never make a round trip through HBM:
//   q, k  per token: L2-normalised, x / max(|x|, 1e-6)  ("All sorts of famous
//         Attention Layers", "DeltaNet"), or the positive feature map elu + 1
//         (same page, "Linear Magic")
//   g     log-gate = -softplus(x), i.e. forget gate exp(-softplus(x)) in (0, 1)
//         ("Linear Attention, Visualized", "Mamba-2", "Gated DeltaNet (GDN)")
//   beta  sigmoid(x)  ("All sorts of famous Attention Layers", "DeltaNet")
// Arithmetic in fp32; the prepared values are rounded to the token type once,
// where the kernels store them as matrix-core operands.
#pragma once

#include "device_common.h"

namespace linattn {

// packed preparation flags: bits 0-1 q/k map, bit 2 gate map, bit 3 beta map
enum { kQkAsIs = 0, kQkL2 = 1, kQkElu1 = 2 };
__device__ __forceinline__ int prep_qk_map(int prep) { return prep & 3; }
__device__ __forceinline__ bool prep_gate_map(int prep) { return (prep >> 2) & 1; }
__device__ __forceinline__ bool prep_beta_map(int prep) { return (prep >> 3) & 1; }

// softplus(x) = max(x, 0) + log(1 + exp(-|x|)); the hardware exp and log
// (v_exp_f32, v_log_f32) keep the map to a few instructions
__device__ __forceinline__ float prep_gate(float x, int prep)
{
    return prep_gate_map(prep) ? -(fmaxf(x, 0.f) + __logf(1.f + __expf(-fabsf(x)))) : x;
}

__device__ __forceinline__ float prep_beta(float x, int prep)
{
    return prep_beta_map(prep) ? 1.f / (1.f + __expf(-x)) : x;
}

// Sum over groups of LANES (4, 8 or 16) consecutive lanes, every lane getting
// its group's sum, in DPP (no LDS): quad exchanges, then the half-row and row
// mirrors.
template <int LANES>
__device__ __forceinline__ float group_sum(float x)
{
    x += dpp_move<0xB1, 0xf>(x);                 // quad_perm 1,0,3,2
    x += dpp_move<0x4E, 0xf>(x);                 // quad_perm 2,3,0,1
    if constexpr (LANES >= 8) x += dpp_move<0x141, 0xf>(x);   // row_half_mirror
    if constexpr (LANES >= 16) x += dpp_move<0x140, 0xf>(x);  // row_mirror
    static_assert(LANES == 4 || LANES == 8 || LANES == 16, "group size");
    return x;
}

typedef __attribute__((__vector_size__(16))) int prep_vec;

// The q/k map on one 16-byte vector of a token row (8 bf16 or 4 fp32 values).
// LANES consecutive lanes hold one row together (the L2 norm is reduced over
// them); every lane of the wave must call this with the same map.
template <typename T, int LANES>
__device__ __forceinline__ prep_vec prep_qk(prep_vec raw, int qk_map)
{
    if (qk_map == kQkAsIs) return raw;
    constexpr int E = 16 / sizeof(T);
    T e[E];
    __builtin_memcpy(e, &raw, 16);
    float x[E];
#pragma unroll
    for (int i = 0; i < E; ++i) x[i] = to_f32(e[i]);
    if (qk_map == kQkElu1) {
#pragma unroll
        for (int i = 0; i < E; ++i) x[i] = x[i] > 0.f ? x[i] + 1.f : __expf(x[i]);
    } else {
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < E; ++i) ss += x[i] * x[i];
        ss = group_sum<LANES>(ss);
        // 1 / max(|x|, 1e-6)
        const float sc = rsqrtf(fmaxf(ss, 1e-12f));
#pragma unroll
        for (int i = 0; i < E; ++i) x[i] *= sc;
    }
#pragma unroll
    for (int i = 0; i < E; ++i) e[i] = from_f32<T>(x[i]);
    prep_vec out;
    __builtin_memcpy(&out, e, 16);
    return out;
}

}  // namespace linattn
