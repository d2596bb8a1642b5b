// device_common.h — small device-side helpers shared by the gfx950 kernels:
// vector types for MFMA operands, bf16 <-> fp32 conversion, wave shuffles.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace linattn {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return static_cast<float>(x); }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
// float -> bf16 conversion of the compiler lowers to the gfx950 hardware
// convert, which rounds to nearest even.
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return static_cast<bf16>(x); }

// 2^x through the hardware transcendental unit (v_exp_f32)
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Wait for every outstanding vector-memory access (gfx9 s_waitcnt: vmcnt 0,
// expcnt and lgkmcnt left at their maxima).  After registers were filled by
// global loads before a loop, this tells the compiler's wait-count tracking
// that they are ready; otherwise it keeps them "pending" at the loop head and
// places a full wait inside the loop, which also waits for the loads the loop
// issues to prefetch its next iteration.
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// An opaque copy of a value: the compiler cannot see through it, so lane
// arithmetic derived from it inside a loop is recomputed there instead of
// being hoisted out and held in registers for the whole loop.
__device__ __forceinline__ int opaque(int x)
{
    asm volatile("" : "+v"(x));
    return x;
}

// A float the compiler must compute where it stands: used for a value that
// feeds a per-lane select, which the compiler would otherwise turn into a
// branch around the value's load and arithmetic.
__device__ __forceinline__ float opaquef(float x)
{
    asm volatile("" : "+v"(x));
    return x;
}

// DPP move of a float (lanes whose source is outside the row, or whose row is
// masked off, read 0)
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_move(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, true));
}

// Inclusive prefix sum over the 64 lanes of a wave, all in DPP (no LDS):
// Hillis-Steele steps of 1, 2, 4, 8 inside each row of 16 lanes, then the row
// totals carried by the row broadcasts of lane 15 (to rows 1 and 3) and of
// lane 31 (to rows 2 and 3).
__device__ __forceinline__ float wave_prefix_sum(float x)
{
    x += dpp_move<0x111, 0xf>(x);   // row_shr:1
    x += dpp_move<0x112, 0xf>(x);   // row_shr:2
    x += dpp_move<0x114, 0xf>(x);   // row_shr:4
    x += dpp_move<0x118, 0xf>(x);   // row_shr:8
    x += dpp_move<0x142, 0xa>(x);   // row_bcast:15
    x += dpp_move<0x143, 0xc>(x);   // row_bcast:31
    return x;
}

// value of lane 63 in every lane
__device__ __forceinline__ float wave_last(float x)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}

__device__ __forceinline__ float shfl_xor(float v, int mask) { return __shfl_xor(v, mask, kWave); }

}  // namespace linattn
