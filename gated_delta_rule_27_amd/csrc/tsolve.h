// tsolve.h — the per-chunk triangular transform of the delta rule, on the
// matrix core of one wave.
//
// "Linear Attention, Visualized", "The triangular correction system" and
// "Optional: Use UT to share the triangular transform": with the strictly
// lower-triangular N = diag(beta) L of a chunk, the corrections solve
// (I + N) U = diag(beta) V; the chunk kernels need T = (I + N)^-1 once and
// apply Tb = T diag(beta) by matrix products.
//
// For C = 64 the inverse is built in 16x16 blocks (X_bb = (I + N_bb)^-1):
//   * the four diagonal blocks as the finite product
//     (I - N)(I + N^2)(I + N^4)(I + N^8) (N_bb is nilpotent, N^16 = 0);
//   * the off-diagonal blocks from the block inverse of a 2x2 lower-triangular
//     block matrix, [[A,0],[C,D]]^-1 = [[A^-1,0],[-D^-1 C A^-1, D^-1]]:
//       T10 = -X11 N10 X00,   T32 = -X33 N32 X22            (level 1)
//       for each 16-column block q of the lower-left 32x32 block:
//         Y0 = N20 T_A[0][q] + N21 T_A[1][q],  Y1 = N30 T_A[0][q] + N31 T_A[1][q]
//         T2q = -X22 Y0,  T3q = -(T32 Y0 + X33 Y1) = -X33 (N32 T2q + Y1)
//     The last form (T32 = -X33 N32 X22, T2q = -X22 Y0) needs every left
//     factor only as a row fragment and every right factor only as a tile.
//
// Register forms (mfma.h): a result tile of X (lane l holds X[4(l/16)+r][l%16])
// is X as a K = 16 right factor and X^T as a left factor; the row fragment of X
// (lane holds X[l%16][4(l/16)+r]) is the tile of X^T.  mma16(a, b) with a the
// row fragment of A and b the tile of B gives the tile of A B; with the two
// swapped it gives the tile of (A B)^T, whose transposed store (store_tile_t)
// writes A B row by row.  Every fp32 tile is rounded to the operand type once.
#pragma once

#include "mfma.h"

namespace linattn {

// Tb block (rb, qb) from -tile(C^T)-style data: with PC = 1 the columns of Tb
// are stored in pcol order, with PC = 2 in swizzled pcol order (mfma.h).
template <typename T, int PC>
__device__ __forceinline__ void store_tb(T* Tb, int ldt, int rb, int qb, floatx4 v, int lane)
{
    if constexpr (PC == 2) store_tile_t_pc_sw(&Tb[(rb * 16) * ldt], ldt, qb, v, lane);
    else if constexpr (PC == 1) store_tile_t_pc(&Tb[(rb * 16) * ldt], ldt, qb, v, lane);
    else store_tile_t(&Tb[(rb * 16) * ldt + qb * 16], ldt, v, lane);
}

// Diagonal blocks b0 .. b0+NB-1 (index i of the arrays is block b0 + i; b0
// defaults to B0).
// nd[i] = tile(N_bb), nt[i] = tile(N_bb^T).  Returns X[i] = tile(X_bb) and
// Xt[i] = tile(X_bb^T) (fp32) and stores those diagonal blocks of
// Tb = T diag(beta); brow[i][r] = beta[16 b + 4(l/16) + r].
template <typename T, int PC = 0, int NB = 4, int B0 = 0>
__device__ __forceinline__ void tsolve_diag(const floatx4 (&nd)[NB], const floatx4 (&nt)[NB],
                                            floatx4 (&X)[NB], floatx4 (&Xt)[NB], T* Tb, int ldt,
                                            const floatx4 (&brow)[NB], int lane, int b0 = B0)
{
    using F = typename Frag16<T>::type;
    // an opaque copy of the lane index keeps the compiler from hoisting the
    // identity out of the caller's chunk loop (it would stay live across it)
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int ra = ln & 15, ca = 4 * (ln >> 4);
    floatx4 id;
#pragma unroll
    for (int r = 0; r < 4; ++r) id[r] = (ca + r == ra) ? 1.f : 0.f;

    // P = I + M with M = -N_bb, then P <- P (I + M^2), P (I + M^4), P (I + M^8);
    // the four blocks are independent chains, interleaved
    F fM[NB], fMt[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        floatx4 M, Mt;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            M[r] = -nd[b][r];
            Mt[r] = -nt[b][r];
            X[b][r] = id[r] + M[r];
            Xt[b][r] = id[r] + Mt[r];
        }
        fM[b] = frag16_acc<T>(M);
        fMt[b] = frag16_acc<T>(Mt);
    }
#pragma unroll
    for (int step = 0; step < 3; ++step) {
        floatx4 M2[NB], M2t[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            M2[b] = mma16<T>(fMt[b], fM[b], zero4());                    // M M
            if (step < 2) M2t[b] = mma16<T>(fM[b], fMt[b], zero4());     // M^T M^T
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const F fM2 = frag16_acc<T>(M2[b]);
            const F fPt = frag16_acc<T>(Xt[b]);
            X[b] = mma16<T>(fPt, fM2, X[b]);                             // P + P M2
            Xt[b] = mma16<T>(fM2, fPt, Xt[b]);                           // P^T + M2^T P^T
            if (step < 2) {
                fM[b] = fM2;
                fMt[b] = frag16_acc<T>(M2t[b]);
            }
        }
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        floatx4 w = Xt[b];
#pragma unroll
        for (int r = 0; r < 4; ++r) w[r] *= brow[b][r];
        store_tb<T, PC>(Tb, ldt, b0 + b, b0 + b, w, lane);
    }
}

// Off-diagonal blocks of T, in two independent halves (each one wave's work):
//   half A: T10 = -X11 N10 X00, then column block 0 of the lower-left quarter,
//           Y0 = N20 X00 + N21 T10, Y1 = N30 X00 + N31 T10, T20 = -X22 Y0,
//           T30 = -X33 (N32 T20 + Y1)
//   half B: T32 = -X33 N32 X22, then column block 1,
//           Y0 = N21 X11, Y1 = N31 X11, T21 = -X22 Y0, T31 = -X33 (N32 T21 + Y1)
// Arguments are fp32 tiles: x_bb = tile(X_bb), xt_bb = tile(X_bb^T) and
// n_ij = tile(N_ij^T); brow as for tsolve_diag (all four blocks).
template <typename T, int PC>
__device__ __forceinline__ void tb_store_neg(T* Tb, int ldt, floatx4 ct, int rb, int qb,
                                             const floatx4 (&brow)[4], int lane)
{
    // store -tile(C^T) scaled by beta of C's columns (block qb) as block (rb, qb)
#pragma unroll
    for (int r = 0; r < 4; ++r) ct[r] = -ct[r] * brow[qb][r];
    store_tb<T, PC>(Tb, ldt, rb, qb, ct, lane);
}

template <typename T, int PC = 0>
__device__ __forceinline__ void tsolve_offdiag_a(floatx4 x00, floatx4 xt11, floatx4 xt22, floatx4 xt33,
                                                 floatx4 n10, floatx4 n20, floatx4 n21, floatx4 n30,
                                                 floatx4 n31, floatx4 n32, T* Tb, int ldt,
                                                 const floatx4 (&brow)[4], int lane)
{
    using F = typename Frag16<T>::type;
    const F fx00 = frag16_acc<T>(x00), fx11r = frag16_acc<T>(xt11);
    const F fx22r = frag16_acc<T>(xt22), fx33r = frag16_acc<T>(xt33);
    const F fu10 = frag16_acc<T>(mma16<T>(frag16_acc<T>(n10), fx00, zero4()));   // N10 X00
    floatx4 t10 = mma16<T>(fx11r, fu10, zero4());                                 // -T10
#pragma unroll
    for (int r = 0; r < 4; ++r) t10[r] = -t10[r];
    tb_store_neg<T, PC>(Tb, ldt, mma16<T>(fu10, fx11r, zero4()), 1, 0, brow, lane);
    const F ft10 = frag16_acc<T>(t10);
    floatx4 y0 = mma16<T>(frag16_acc<T>(n20), fx00, mma16<T>(frag16_acc<T>(n21), ft10, zero4()));
    floatx4 y1 = mma16<T>(frag16_acc<T>(n30), fx00, mma16<T>(frag16_acc<T>(n31), ft10, zero4()));
    const F fy0 = frag16_acc<T>(y0);
    floatx4 t2 = mma16<T>(fx22r, fy0, zero4());                                   // -T20
#pragma unroll
    for (int r = 0; r < 4; ++r) t2[r] = -t2[r];
    tb_store_neg<T, PC>(Tb, ldt, mma16<T>(fy0, fx22r, zero4()), 2, 0, brow, lane);
    const F fu = frag16_acc<T>(mma16<T>(frag16_acc<T>(n32), frag16_acc<T>(t2), y1));
    tb_store_neg<T, PC>(Tb, ldt, mma16<T>(fu, fx33r, zero4()), 3, 0, brow, lane);
}

template <typename T, int PC = 0>
__device__ __forceinline__ void tsolve_offdiag_b(floatx4 x11, floatx4 x22, floatx4 xt22, floatx4 xt33,
                                                 floatx4 n21, floatx4 n31, floatx4 n32, T* Tb, int ldt,
                                                 const floatx4 (&brow)[4], int lane)
{
    using F = typename Frag16<T>::type;
    const F fx11 = frag16_acc<T>(x11), fx22 = frag16_acc<T>(x22);
    const F fx22r = frag16_acc<T>(xt22), fx33r = frag16_acc<T>(xt33);
    const F fn32 = frag16_acc<T>(n32);
    const F fu32 = frag16_acc<T>(mma16<T>(fn32, fx22, zero4()));                 // N32 X22
    tb_store_neg<T, PC>(Tb, ldt, mma16<T>(fu32, fx33r, zero4()), 3, 2, brow, lane);
    const floatx4 y0 = mma16<T>(frag16_acc<T>(n21), fx11, zero4());
    const floatx4 y1 = mma16<T>(frag16_acc<T>(n31), fx11, zero4());
    const F fy0 = frag16_acc<T>(y0);
    floatx4 t2 = mma16<T>(fx22r, fy0, zero4());                                   // -T21
#pragma unroll
    for (int r = 0; r < 4; ++r) t2[r] = -t2[r];
    tb_store_neg<T, PC>(Tb, ldt, mma16<T>(fy0, fx22r, zero4()), 2, 1, brow, lane);
    const F fu = frag16_acc<T>(mma16<T>(fn32, frag16_acc<T>(t2), y1));
    tb_store_neg<T, PC>(Tb, ldt, mma16<T>(fu, fx33r, zero4()), 3, 1, brow, lane);
}

// Half B without T32 (tsolve_t32), so the two can run on different waves:
// T21 = -X22 N21 X11, T31 = -X33 (N32 T21 + N31 X11).
template <typename T, int PC = 0>
__device__ __forceinline__ void tsolve_offdiag_b1(floatx4 x11, floatx4 xt22, floatx4 xt33, floatx4 n21,
                                                  floatx4 n31, floatx4 n32, T* Tb, int ldt,
                                                  const floatx4 (&brow)[4], int lane)
{
    using F = typename Frag16<T>::type;
    const F fx11 = frag16_acc<T>(x11);
    const F fx22r = frag16_acc<T>(xt22), fx33r = frag16_acc<T>(xt33);
    const F fn32 = frag16_acc<T>(n32);
    const floatx4 y0 = mma16<T>(frag16_acc<T>(n21), fx11, zero4());
    const floatx4 y1 = mma16<T>(frag16_acc<T>(n31), fx11, zero4());
    const F fy0 = frag16_acc<T>(y0);
    floatx4 t2 = mma16<T>(fx22r, fy0, zero4());                                   // -T21
#pragma unroll
    for (int r = 0; r < 4; ++r) t2[r] = -t2[r];
    tb_store_neg<T, PC>(Tb, ldt, mma16<T>(fy0, fx22r, zero4()), 2, 1, brow, lane);
    const F fu = frag16_acc<T>(mma16<T>(fn32, frag16_acc<T>(t2), y1));
    tb_store_neg<T, PC>(Tb, ldt, mma16<T>(fu, fx33r, zero4()), 3, 1, brow, lane);
}

// T32 = -X33 N32 X22 alone.
template <typename T, int PC = 0>
__device__ __forceinline__ void tsolve_t32(floatx4 x22, floatx4 xt33, floatx4 n32, T* Tb, int ldt,
                                           const floatx4 (&brow)[4], int lane)
{
    using F = typename Frag16<T>::type;
    const F fu32 = frag16_acc<T>(mma16<T>(frag16_acc<T>(n32), frag16_acc<T>(x22), zero4()));   // N32 X22
    tb_store_neg<T, PC>(Tb, ldt, mma16<T>(fu32, frag16_acc<T>(xt33), zero4()), 3, 2, brow, lane);
}

// Both halves on one wave, from X, Xt of tsolve_diag.
template <typename T, int PC = 0>
__device__ __forceinline__ void tsolve_offdiag(const floatx4 (&X)[4], const floatx4 (&Xt)[4],
                                               floatx4 n10, floatx4 n20, floatx4 n21, floatx4 n30,
                                               floatx4 n31, floatx4 n32, T* Tb, int ldt,
                                               const floatx4 (&brow)[4], int lane)
{
    tsolve_offdiag_a<T, PC>(X[0], Xt[1], Xt[2], Xt[3], n10, n20, n21, n30, n31, n32, Tb, ldt, brow, lane);
    tsolve_offdiag_b<T, PC>(X[1], X[2], Xt[2], Xt[3], n21, n31, n32, Tb, ldt, brow, lane);
}

// Both steps with every N block in registers: nd, nt as for tsolve_diag and
// n_ij = tile(N_ij^T) below the diagonal.
template <typename T>
__device__ __forceinline__ void tsolve64_regs(const floatx4 (&nd)[4], const floatx4 (&nt)[4],
                                              floatx4 n10, floatx4 n20, floatx4 n21, floatx4 n30,
                                              floatx4 n31, floatx4 n32, T* Tb, int ldt,
                                              const floatx4 (&brow)[4], int lane)
{
    floatx4 X[4], Xt[4];
    tsolve_diag<T>(nd, nt, X, Xt, Tb, ldt, brow, lane);
    tsolve_offdiag<T>(X, Xt, n10, n20, n21, n30, n31, n32, Tb, ldt, brow, lane);
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
    floatx4 nd[4], nt[4], brow[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        nd[b] = load_tile_rl(&Nf[(b * 16) * ldn + b * 16], ldn, lane);
        nt[b] = tile_t(b, b);
        brow[b] = *reinterpret_cast<const floatx4*>(&bet[16 * b + ca]);
    }
    tsolve64_regs<T>(nd, nt, tile_t(1, 0), tile_t(2, 0), tile_t(2, 1), tile_t(3, 0), tile_t(3, 1),
                     tile_t(3, 2), Tb, ldt, brow, lane);
}

}  // namespace linattn
