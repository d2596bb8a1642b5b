// tile_rows.h — row-wise store of a 16x16 matrix-core result tile, for the
// chain kernels that hand a state tile to their helper waves through LDS.
#pragma once

#include "device_common.h"

namespace linattn {

// Row store of a 16x16 result tile in the token type: lane l holds rows
// 4(l/16)..+3 of column l%16; a 4x4 transpose inside each quad of lanes (two
// DPP exchanges) leaves lane l with row 4(l/16) + l%4 over columns
// 4(l%16 / 4)..+3, stored as one 8-byte (bf16) or 16-byte (fp32) write.
template <typename T>
__device__ __forceinline__ void store_tile_rows(T* P, int64_t ld, floatx4 v, int lane)
{
    const int s = lane & 3;
    float v0 = v[0], v1 = v[1], v2 = v[2], v3 = v[3];
    {
        // lanes s, s^1: afterwards lane s holds rows (s&1, s&1 + 2), columns (s&2, s&2 + 1)
        const bool odd = s & 1;
        const float a = dpp_move<0xB1, 0xf>(odd ? v0 : v1), b = dpp_move<0xB1, 0xf>(odd ? v2 : v3);
        if (odd) { v0 = a; v2 = b; } else { v1 = a; v3 = b; }
    }
    {
        // lanes s, s^2: afterwards lane s holds row s, columns 0..3
        const bool hi = s & 2;
        const float a = dpp_move<0x4E, 0xf>(hi ? v0 : v2), b = dpp_move<0x4E, 0xf>(hi ? v1 : v3);
        if (hi) { v0 = a; v1 = b; } else { v2 = a; v3 = b; }
    }
    T* p = P + (int64_t)(4 * (lane >> 4) + s) * ld + 4 * ((lane & 15) >> 2);
    if constexpr (sizeof(T) == 2) {
        bf16x4 w = {from_f32<bf16>(v0), from_f32<bf16>(v1), from_f32<bf16>(v2), from_f32<bf16>(v3)};
        *reinterpret_cast<bf16x4*>(p) = w;
    } else {
        *reinterpret_cast<floatx4*>(p) = floatx4{v0, v1, v2, v3};
    }
}

}  // namespace linattn
