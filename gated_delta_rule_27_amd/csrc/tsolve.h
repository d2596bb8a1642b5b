// tsolve.h — the per-chunk triangular transform of the delta rule, run by one
// wave.
//
// "Linear Attention, Visualized", "The triangular correction system" and
// "Optional: Use UT to share the triangular transform": with the strictly
// lower-triangular N = diag(beta) L of a chunk, the corrections solve
// (I + N) U = diag(beta) V; the chunk kernels need T = (I + N)^-1 once and
// apply Tb = T diag(beta) by matrix products.
//
// For C = 64 the inverse is built in 16x16 blocks (X_bb = (I + N_bb)^-1):
//   * the four diagonal blocks on the matrix core as the finite product
//     (I - N)(I + N^2)(I + N^4)(I + N^8) (N_bb is nilpotent, N^16 = 0);
//   * the off-diagonal blocks from the block inverse of a 2x2 lower-triangular
//     block matrix, [[A,0],[C,D]]^-1 = [[A^-1,0],[-D^-1 C A^-1, D^-1]]:
//       T10 = -X11 N10 X00,   T32 = -X33 N32 X22            (level 1)
//       for each 16-column block q of the lower-left 32x32 block:
//         Y0 = N20 T_A[0][q] + N21 T_A[1][q],  Y1 = N30 T_A[0][q] + N31 T_A[1][q]
//         T2q = -X22 Y0,  T3q = -(T32 Y0 + X33 Y1) = -X33 (N32 T2q + Y1)
//     The last form (T32 = -X33 N32 X22, T2q = -X22 Y0) needs every left
//     factor only as a row fragment and every right factor only as a tile.
// All products use the operand type T (bf16 MFMA with fp32 accumulation, or
// fp32 MFMA) on register tiles; only Tb is written, and no barrier is needed.
#pragma once

#include "mfma.h"

namespace linattn {

// The ten 16x16 blocks of N on and below the diagonal come in registers, in the
// MFMA result-tile layout (lane l holds rows 4(l/16)..+3 of column l%16):
//   nd[b]  = tile(N_bb)       nt[b] = tile(N_bb^T)        (diagonal blocks)
//   n10, n20, n21, n30, n31, n32 = tile(N_ij^T)           (below the diagonal)
// A tile of X^T is, lane by lane, the row fragment of X (lane holds
// X[l%16][4(l/16)..+3]), i.e. the left operand that makes an MFMA product X B.
// Tb: operand type [64][ldt], receives T diag(beta) on and below the diagonal
// (the strictly upper blocks are never written).  beta in registers:
// brow[b][r] = beta[16 b + 4(l/16) + r] and bcol[b] = beta[16 b + l%16].
template <typename T>
__device__ __forceinline__ void tsolve64_regs(const floatx4 (&nd)[4], const floatx4 (&nt)[4],
                                              floatx4 n10, floatx4 n20, floatx4 n21, floatx4 n30,
                                              floatx4 n31, floatx4 n32, T* Tb, int ldt,
                                              const floatx4 (&brow)[4], const float (&bcol)[4],
                                              int lane)
{
    // an opaque copy of the lane index keeps the compiler from hoisting the
    // identity below out of the caller's chunk loop (it would stay live, and
    // spill, across the whole loop)
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int ra = ln & 15, ca = 4 * (ln >> 4);

    // ---- diagonal blocks on the matrix core ------------------------------------
    // X_bb = (I + N_bb)^-1 = (I + M)(I + M^2)(I + M^4)(I + M^8), M = -N_bb
    // (N_bb is strictly lower, so M^16 = 0).  A K = 16 product of register tiles
    // gives A^T B (mfma.h), so every matrix is carried together with its
    // transpose; the four blocks are four independent chains of depth four.
    floatx4 X[4], Xt[4];           // X_bb as right factor, and as left factor (row fragment)
    {
        floatx4 id;
#pragma unroll
        for (int r = 0; r < 4; ++r) id[r] = (ca + r == ra) ? 1.f : 0.f;
        floatx4 M[4], Mt[4], P[4], Pt[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                M[b][r] = -nd[b][r];
                Mt[b][r] = -nt[b][r];
                P[b][r] = id[r] + M[b][r];
                Pt[b][r] = id[r] + Mt[b][r];
            }
        }
#pragma unroll
        for (int step = 0; step < 3; ++step) {
            floatx4 M2[4], M2t[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                M2[b] = mm16r<T>(Mt[b], M[b], zero4());      // M M
                M2t[b] = mm16r<T>(M[b], Mt[b], zero4());     // M^T M^T
            }
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const floatx4 p = P[b];
                P[b] = mm16r<T>(Pt[b], M2[b], p);            // P + P M2
                Pt[b] = mm16r<T>(M2[b], Pt[b], Pt[b]);       // P^T + M2^T P^T
                M[b] = M2[b];
                Mt[b] = M2t[b];
            }
        }
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            X[b] = P[b];
            Xt[b] = Pt[b];
            // Tb diagonal block: X diag(beta), stored from the row fragment
            floatx4 w = Xt[b];
#pragma unroll
            for (int r = 0; r < 4; ++r) w[r] *= brow[b][r];
            store_tile_t(&Tb[(b * 16) * ldt + b * 16], ldt, w, lane);
        }
    }
    const floatx4 x00 = X[0], x11 = X[1], x22 = X[2];
    const floatx4 x11r = Xt[1], x22r = Xt[2], x33r = Xt[3];

    // ---- level 1 ----------------------------------------------------------------
    floatx4 t10 = mm16r<T>(x11r, mm16r<T>(n10, x00, zero4()), zero4());
    floatx4 t32 = mm16r<T>(x33r, mm16r<T>(n32, x22, zero4()), zero4());
    const int rw = 4 * (lane >> 4), cl = lane & 15;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
        t10[rr] = -t10[rr];
        t32[rr] = -t32[rr];
        Tb[(16 + rw + rr) * ldt + cl] = from_f32<T>(t10[rr] * bcol[0]);
        Tb[(48 + rw + rr) * ldt + 32 + cl] = from_f32<T>(t32[rr] * bcol[2]);
    }

    // ---- level 2: lower-left 32x32 block, 16 columns at a time ------------------
#pragma unroll
    for (int qc = 0; qc < 2; ++qc) {
        const floatx4 ta1 = qc == 0 ? t10 : x11;          // T_A[1][qc]
        floatx4 y0 = mm16r<T>(n21, ta1, zero4());
        floatx4 y1 = mm16r<T>(n31, ta1, zero4());
        if (qc == 0) {                                    // T_A[0][0] = X00, T_A[0][1] = 0
            y0 = mm16r<T>(n20, x00, y0);
            y1 = mm16r<T>(n30, x00, y1);
        }
        floatx4 t2 = mm16r<T>(x22r, y0, zero4());
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) t2[rr] = -t2[rr];
        const floatx4 u = mm16r<T>(n32, t2, y1);
        const floatx4 t3 = mm16r<T>(x33r, u, zero4());
        const int col = qc * 16 + cl;
        const float bc = bcol[qc];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            Tb[(32 + rw + rr) * ldt + col] = from_f32<T>(t2[rr] * bc);
            Tb[(48 + rw + rr) * ldt + col] = from_f32<T>(-t3[rr] * bc);
        }
    }
}

// The same transform with N and beta read from LDS.  Nf: fp32 [64][ldn]; its
// block-lower part holds N with zeros on and above the diagonal of the diagonal
// blocks.  bet: beta of the 64 rows, 16-byte aligned.
template <typename T>
__device__ __forceinline__ void tsolve64_wave(const float* Nf, int ldn, T* Tb, int ldt,
                                              const float* bet, int lane)
{
    const int ra = lane & 15, ca = 4 * (lane >> 4);
    // tile of the transpose of block (bi, bj) = its row fragment
    auto tile_t = [&](int bi, int bj) {
        return *reinterpret_cast<const floatx4*>(&Nf[(bi * 16 + ra) * ldn + bj * 16 + ca]);
    };
    floatx4 nd[4], nt[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        nd[b] = load_tile_rl(&Nf[(b * 16) * ldn + b * 16], ldn, lane);
        nt[b] = tile_t(b, b);
    }
    floatx4 brow[4];
    float bcol[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        brow[b] = *reinterpret_cast<const floatx4*>(&bet[16 * b + ca]);
        bcol[b] = bet[16 * b + ra];
    }
    tsolve64_regs<T>(nd, nt, tile_t(1, 0), tile_t(2, 0), tile_t(2, 1), tile_t(3, 0), tile_t(3, 1),
                     tile_t(3, 2), Tb, ldt, brow, bcol, lane);
}

}  // namespace linattn
