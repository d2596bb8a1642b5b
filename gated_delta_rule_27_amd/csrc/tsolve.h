// tsolve.h — the per-chunk triangular transform of the delta rule, run by one
// wave.
//
// "Linear Attention, Visualized", "The triangular correction system" and
// "Optional: Use UT to share the triangular transform": with the strictly
// lower-triangular N = diag(beta) L of a chunk, the corrections solve
// (I + N) U = diag(beta) V; the chunk kernels need T = (I + N)^-1 once and
// apply Tb = T diag(beta) by matrix products.
//
// For C = 64 the inverse is built in 16x16 blocks:
//   * the four diagonal blocks X_bb = (I + N_bb)^-1 by forward substitution,
//     one lane group of 16 per block and one lane per column, sweeping columns
//     so that each step's updates are independent;
//   * level 1: T10 = -X11 N10 X00 and T32 = -X33 N32 X22;
//   * level 2: the lower-left 32x32 block -T_B (N_BA T_A) (block inverse of a
//     2x2 lower-triangular block matrix), 16 columns at a time.
// Diagonal blocks are fp32; the block products use the operand type T (bf16
// MFMA with fp32 accumulation, or fp32 MFMA).  No workgroup barrier is needed:
// the wave only reads what it wrote itself.
#pragma once

#include "mfma.h"

namespace linattn {

// Nf: fp32 [64][ldn]; on entry its strictly lower part holds N (the diagonal
// and upper part are ignored), on exit its block-lower part holds pieces of T.
// Tb: operand type [64][ldt], receives T diag(beta) on and below the diagonal
// (the strictly upper blocks are never written).  bet: beta of the 64 rows.
template <typename T>
__device__ __forceinline__ void tsolve64_wave(float* Nf, int ldn, T* Tb, int ldt, const float* bet,
                                              int lane)
{
    // the off-diagonal N blocks used by the block products, read up front so
    // their LDS latency hides behind the diagonal substitution
    const int ra = lane & 15, ca = 4 * (lane >> 4);
    auto rowfrag = [&](int bi, int bj) {
        return *reinterpret_cast<const floatx4*>(&Nf[(bi * 16 + ra) * ldn + bj * 16 + ca]);
    };
    const floatx4 n10 = rowfrag(1, 0), n32 = rowfrag(3, 2);
    const floatx4 n20 = rowfrag(2, 0), n21 = rowfrag(2, 1), n30 = rowfrag(3, 0), n31 = rowfrag(3, 1);
    {
        // an opaque copy of the lane index keeps the compiler from hoisting the
        // identity below out of the caller's chunk loop (it would stay live,
        // and spill, across the whole loop)
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int b = ln >> 4, c = ln & 15;
        float* Nb = &Nf[(b * 16) * ldn + b * 16];
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = (i == c) ? 1.f : 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j)
#pragma unroll
            for (int i = j + 1; i < 16; ++i) x[i] = fmaf(-Nb[i * ldn + j], x[j], x[i]);
        const float bc = bet[b * 16 + c];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            Nb[i * ldn + c] = x[i];
            Tb[(b * 16 + i) * ldt + b * 16 + c] = from_f32<T>(x[i] * bc);
        }
    }
    {
        const floatx4 x00 = load_tile_rl(&Nf[0 * 16 * ldn + 0 * 16], ldn, lane);
        const floatx4 x22 = load_tile_rl(&Nf[2 * 16 * ldn + 2 * 16], ldn, lane);
        const floatx4 y1 = mm16r<T>(n10, x00, zero4());
        const floatx4 y3 = mm16r<T>(n32, x22, zero4());
        floatx4 t10 = mm16<T>(&Nf[1 * 16 * ldn + 1 * 16], ldn, y1, zero4(), lane);
        floatx4 t32 = mm16<T>(&Nf[3 * 16 * ldn + 3 * 16], ldn, y3, zero4(), lane);
        const int rw = 4 * (lane >> 4), cl = lane & 15;
        const float b0 = bet[cl], b2 = bet[32 + cl];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            t10[rr] = -t10[rr];
            t32[rr] = -t32[rr];
            Nf[(16 + rw + rr) * ldn + cl] = t10[rr];
            Nf[(48 + rw + rr) * ldn + 32 + cl] = t32[rr];
            Tb[(16 + rw + rr) * ldt + cl] = from_f32<T>(t10[rr] * b0);
            Tb[(48 + rw + rr) * ldt + 32 + cl] = from_f32<T>(t32[rr] * b2);
        }
    }
#pragma unroll
    for (int qc = 0; qc < 2; ++qc) {
        // Y_p = sum_{s >= qc} N[2+p][s] T_A[s][qc]
        floatx4 y[2];
        const floatx4 ta1 = load_tile_rl(&Nf[1 * 16 * ldn + qc * 16], ldn, lane);
        y[0] = mm16r<T>(n21, ta1, zero4());
        y[1] = mm16r<T>(n31, ta1, zero4());
        if (qc == 0) {
            const floatx4 ta0 = load_tile_rl(&Nf[0], ldn, lane);
            y[0] = mm16r<T>(n20, ta0, y[0]);
            y[1] = mm16r<T>(n30, ta0, y[1]);
        }
        const floatx4 t2 = mm16<T>(&Nf[2 * 16 * ldn + 2 * 16], ldn, y[0], zero4(), lane);
        floatx4 t3 = mm16<T>(&Nf[3 * 16 * ldn + 2 * 16], ldn, y[0], zero4(), lane);
        t3 = mm16<T>(&Nf[3 * 16 * ldn + 3 * 16], ldn, y[1], t3, lane);
        const int col = qc * 16 + (lane & 15);
        const float bc = bet[col];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int row = 4 * (lane >> 4) + rr;
            Tb[(32 + row) * ldt + col] = from_f32<T>(-t2[rr] * bc);
            Tb[(48 + row) * ldt + col] = from_f32<T>(-t3[rr] * bc);
        }
    }
}

}  // namespace linattn
