// mfma.h — 16x16 matrix-core tile helpers for gfx950 (CDNA4, wave64).
//
// Every product here is written as D = A * B^T with both operands stored
// row-major with the contraction index contiguous ("NT" form), so each lane's
// operand fragment is one contiguous LDS read.  Fragment layouts:
//   bf16 v_mfma_f32_16x16x32_bf16: lane l holds A[l%16][k0+8(l/16) .. +7]
//   fp32 v_mfma_f32_16x16x4_f32:   lane l holds A[l%16][k0+(l/16)]
// (B the same with its own rows), and the 16x16 fp32 result is spread as
//   lane l, register r  <->  D[4(l/16)+r][l%16].
// Writing a result tile "transposed" (dst[col][row..row+3]) is therefore a
// single 4-element contiguous store per lane; the kernels use that to produce
// whichever orientation the next product needs.
#pragma once

#include "device_common.h"

namespace linattn {

template <typename T> struct Mfma;

template <> struct Mfma<bf16> {
    static constexpr int kStep = 32;
    typedef bf16x8 frag;
    __device__ static __forceinline__ floatx4 mma(frag a, frag b, floatx4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    __device__ static __forceinline__ frag load(const bf16* row0, int ld, int k0, int lane)
    {
        return *reinterpret_cast<const frag*>(row0 + (lane & 15) * ld + k0 + 8 * (lane >> 4));
    }
};

template <> struct Mfma<float> {
    static constexpr int kStep = 4;
    typedef float frag;
    __device__ static __forceinline__ floatx4 mma(frag a, frag b, floatx4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
    __device__ static __forceinline__ frag load(const float* row0, int ld, int k0, int lane)
    {
        return row0[(lane & 15) * ld + k0 + (lane >> 4)];
    }
};

// acc += A[0:16][kb:ke] * B[0:16][kb:ke]^T, A and B pointing at their first row.
template <typename T>
__device__ __forceinline__ floatx4 mma_nt(floatx4 acc, const T* A, int lda, const T* B, int ldb,
                                          int kb, int ke, int lane)
{
    for (int k = kb; k < ke; k += Mfma<T>::kStep)
        acc = Mfma<T>::mma(Mfma<T>::load(A, lda, k, lane), Mfma<T>::load(B, ldb, k, lane), acc);
    return acc;
}

__device__ __forceinline__ floatx4 zero4() { return floatx4{0.f, 0.f, 0.f, 0.f}; }

// acc += A[0:16][0:K] * B[0:16][0:K]^T with every fragment loaded before the
// first MFMA issues, so the LDS reads overlap instead of each MFMA waiting on
// its own pair.  Only the first `nk` steps are accumulated (nk <= K / step);
// the later fragments are read but unused (they must be in bounds).
template <typename T, int K>
__device__ __forceinline__ floatx4 mma_nt_k(floatx4 acc, const T* A, int lda, const T* B, int ldb,
                                            int lane, int nk = K / Mfma<T>::kStep)
{
    constexpr int NK = K / Mfma<T>::kStep;
    typename Mfma<T>::frag a[NK], b[NK];
#pragma unroll
    for (int i = 0; i < NK; ++i) {
        a[i] = Mfma<T>::load(A, lda, i * Mfma<T>::kStep, lane);
        b[i] = Mfma<T>::load(B, ldb, i * Mfma<T>::kStep, lane);
    }
#pragma unroll
    for (int i = 0; i < NK; ++i)
        if (i < nk) acc = Mfma<T>::mma(a[i], b[i], acc);
    return acc;
}

// Twenty wait states, with nothing scheduled across them: placed after a chain
// of matrix-core ops whose results are next read past a branch (a loop exit,
// a skipped block).  Measured on gfx950: with the wait states the compiler
// inserted on the branch-taken path alone (a branch and s_nop 3), the last
// result register of a v_mfma_f32_16x16x4_f32 chain read its value from
// before the last op.  Twenty cover the longest (16-pass) op.
__device__ __forceinline__ void mfma_settle()
{
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// Workgroup barrier that orders LDS only: waits for this wave's LDS traffic,
// then s_barrier.  Global loads in flight (prefetch of the next chunk) stay in
// flight across it; no kernel here communicates through global memory inside
// a workgroup.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Store the 4 values a lane holds of a result tile D (rows 4(l/16)+r, column
// l%16) into dst as D^T: dst[(l%16)*ld + 4(l/16) + r], r = 0..3.
template <typename T>
__device__ __forceinline__ void store_tile_t(T* dst, int ld, floatx4 v, int lane)
{
    T* p = dst + (lane & 15) * ld + 4 * (lane >> 4);
    if constexpr (sizeof(T) == 2) {
        bf16x4 w;
        w[0] = from_f32<bf16>(v[0]); w[1] = from_f32<bf16>(v[1]);
        w[2] = from_f32<bf16>(v[2]); w[3] = from_f32<bf16>(v[3]);
        *reinterpret_cast<bf16x4*>(p) = w;
    } else {
        *reinterpret_cast<floatx4*>(p) = v;
    }
}

// 16x16x16 product with fp32 operands held in fp32: A from LDS (row-major,
// lane reads A[l%16][4(l/16)..+3]), B given in the result layout (lane holds
// B[4(l/16)+r][l%16]).  The contraction index is assigned to (lane group,
// register) as k = 4(l/16)+r on both sides, so a previous result tile can be
// fed straight back as B.  T selects the arithmetic: bf16 operands through
// v_mfma_f32_16x16x16_bf16, or fp32 through four v_mfma_f32_16x16x4_f32.
template <typename T>
__device__ __forceinline__ floatx4 mm16(const float* A, int lda, floatx4 b, floatx4 acc, int lane)
{
    const floatx4 a = *reinterpret_cast<const floatx4*>(A + (lane & 15) * lda + 4 * (lane >> 4));
    if constexpr (sizeof(T) == 2) {
        bf16x4 ab, bb;
#pragma unroll
        for (int r = 0; r < 4; ++r) { ab[r] = from_f32<bf16>(a[r]); bb[r] = from_f32<bf16>(b[r]); }
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ab, bb, acc, 0, 0, 0);
    } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[r], b[r], acc, 0, 0, 0);
        return acc;
    }
}

// The same product with A already in registers as a row fragment (lane holds
// A[l%16][4(l/16)..+3]).
template <typename T>
__device__ __forceinline__ floatx4 mm16r(floatx4 a, floatx4 b, floatx4 acc)
{
    if constexpr (sizeof(T) == 2) {
        bf16x4 ab, bb;
#pragma unroll
        for (int r = 0; r < 4; ++r) { ab[r] = from_f32<bf16>(a[r]); bb[r] = from_f32<bf16>(b[r]); }
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ab, bb, acc, 0, 0, 0);
    } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[r], b[r], acc, 0, 0, 0);
        return acc;
    }
}

// Transpose through the matrix core: D = A * I for a 16x16 block of A
// (row-major in LDS), returned in the result layout (lane holds
// A[4(l/16)+r][l%16]); store_tile_t then writes A^T with contiguous stores.
// Exact: every product is by 1 or 0 and every sum has one nonzero term.
template <typename T>
__device__ __forceinline__ floatx4 ident_tile(const T* A, int lda, int lane)
{
    int ln = lane;
    asm volatile("" : "+v"(ln));   // rebuild the identity here, not once per kernel
    const int c = ln & 15, g4 = 4 * (ln >> 4);
    if constexpr (sizeof(T) == 2) {
        const bf16x4 a = *reinterpret_cast<const bf16x4*>(A + c * lda + g4);
        bf16x4 b;
#pragma unroll
        for (int r = 0; r < 4; ++r) b[r] = from_f32<bf16>(g4 + r == c ? 1.f : 0.f);
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, zero4(), 0, 0, 0);
    } else {
        const floatx4 a = *reinterpret_cast<const floatx4*>(A + c * lda + g4);
        floatx4 acc = zero4();
#pragma unroll
        for (int r = 0; r < 4; ++r)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[r], g4 + r == c ? 1.f : 0.f, acc, 0, 0, 0);
        return acc;
    }
}

// ---------------------------------------------------------------------------
// K = 16 products with register-resident operands.
//
// For v_mfma_f32_16x16x16_bf16 lane l supplies A[l%16][4(l/16)+r] and
// B[4(l/16)+r][l%16] (r = 0..3), exactly the positions a lane holds of a
// 16x16 result tile X (X[4(l/16)+r][l%16]).  Hence a result tile can be fed
// back without any data movement: as B it is X, as A it is X^T.  From a
// row-major block M in LDS a lane reads M[l%16][4(l/16)..+3] (one 8-byte read
// for bf16): as A that is M, as B it is M^T.  With fp32 operands the same
// bookkeeping runs through four v_mfma_f32_16x16x4_f32 (register r in the
// r-th instruction).
// ---------------------------------------------------------------------------
template <typename T> struct Frag16;
template <> struct Frag16<bf16> { typedef bf16x4 type; };
template <> struct Frag16<float> { typedef floatx4 type; };

template <typename T>
__device__ __forceinline__ typename Frag16<T>::type frag16_lds(const T* M, int ld, int lane)
{
    return *reinterpret_cast<const typename Frag16<T>::type*>(M + (lane & 15) * ld + 4 * (lane >> 4));
}

template <typename T>
__device__ __forceinline__ typename Frag16<T>::type frag16_acc(floatx4 x)
{
    if constexpr (sizeof(T) == 2) {
        bf16x4 f;
#pragma unroll
        for (int r = 0; r < 4; ++r) f[r] = from_f32<bf16>(x[r]);
        return f;
    } else {
        return x;
    }
}

template <typename T>
__device__ __forceinline__ floatx4 mma16(typename Frag16<T>::type a, typename Frag16<T>::type b,
                                         floatx4 acc)
{
    if constexpr (sizeof(T) == 2) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, acc, 0, 0, 0);
    } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[r], b[r], acc, 0, 0, 0);
        return acc;
    }
}

// Two K = 16 products summed, D = A0 B0 + A1 B1 + acc, as one K = 32 matrix-core
// op in bf16 (the 16x16x16 bf16 form takes as long as the 16x16x32 one).  The
// K = 32 op sums over its 32 k slots, and lane group g holds slots 8g..8g+7;
// filling them with k-block 0's k = 4g..4g+3 and then k-block 1's (the same
// k in both operands) keeps every K = 16 register tile usable as is.
// Do not feed the accumulator of a 16x16x32 bf16 op straight into a 16x16x16
// bf16 op (or back): on gfx950 that chain read stale accumulator values with
// the wait states the compiler inserted, so every chain here keeps one shape.
template <typename T>
__device__ __forceinline__ floatx4 mma16x2(typename Frag16<T>::type a0, typename Frag16<T>::type a1,
                                           typename Frag16<T>::type b0, typename Frag16<T>::type b1,
                                           floatx4 acc)
{
    if constexpr (sizeof(T) == 2) {
        const bf16x8 a = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
        const bf16x8 b = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
    } else {
        return mma16<T>(a1, b1, mma16<T>(a0, b0, acc));
    }
}

// ---- paired (K = 32) operands from LDS ---------------------------------------
// Column order of LDS tiles that feed paired products: inside every group of 32
// columns, column 16h + 4g + j is stored at 8g + 4h + j.  The eight values lane
// group g needs for a paired operand (k-block 0's 4g..4g+3, then k-block 1's,
// the slot order of mma16x2) are then one 16-byte read, and every aligned run of
// four columns stays contiguous (so K = 16 fragments and transposed tile stores
// keep 8-byte accesses).  A 16x16x32 fragment read straight from such a tile is
// the same k permutation, which any product of two tiles stored alike allows.
__host__ __device__ constexpr int pcol(int c)
{
    return (c & ~31) | ((c & 12) << 1) | ((c & 16) >> 2) | (c & 3);
}

// first logical column of the 8 stored at position P (a multiple of 8) in pcol
// order: they are columns c0..c0+3 and c0+16..c0+19
__host__ __device__ constexpr int pcol_first(int P) { return (P & ~31) | ((P & 24) >> 1); }

template <typename T> struct Pair;
template <> struct Pair<bf16> { typedef bf16x8 type; };
template <> struct Pair<float> { struct type { floatx4 lo, hi; }; };

// paired operand of the row block at M (columns 32p..32p+31 of the block start
// at M, stored in pcol order): lane holds row l%16, k-blocks 2p and 2p+1
template <typename T>
__device__ __forceinline__ typename Pair<T>::type pair_lds(const T* M, int ld, int lane)
{
    const T* p = M + (lane & 15) * ld + 8 * (lane >> 4);
    if constexpr (sizeof(T) == 2) {
        return *reinterpret_cast<const bf16x8*>(p);
    } else {
        return {*reinterpret_cast<const floatx4*>(p), *reinterpret_cast<const floatx4*>(p + 4)};
    }
}

// paired operand from two result tiles (k-block 0 = x0, k-block 1 = x1)
template <typename T>
__device__ __forceinline__ typename Pair<T>::type pair_regs(floatx4 x0, floatx4 x1)
{
    if constexpr (sizeof(T) == 2) {
        return __builtin_shufflevector(frag16_acc<bf16>(x0), frag16_acc<bf16>(x1), 0, 1, 2, 3, 4, 5, 6, 7);
    } else {
        return {x0, x1};
    }
}

template <typename T>
__device__ __forceinline__ floatx4 mma_pair(typename Pair<T>::type a, typename Pair<T>::type b, floatx4 acc)
{
    if constexpr (sizeof(T) == 2) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
    } else {
        return mma16<float>(a.hi, b.hi, mma16<float>(a.lo, b.lo, acc));
    }
}

// K = 16 fragment (as frag16_lds) of k-block kb of a row block stored in pcol order
template <typename T>
__device__ __forceinline__ typename Frag16<T>::type frag16_lds_pc(const T* M, int ld, int kb, int lane)
{
    return *reinterpret_cast<const typename Frag16<T>::type*>(
        M + (lane & 15) * ld + 32 * (kb >> 1) + 4 * (kb & 1) + 8 * (lane >> 4));
}

// store_tile_t into column block kb of a row block stored in pcol order
template <typename T>
__device__ __forceinline__ void store_tile_t_pc(T* M, int ld, int kb, floatx4 v, int lane)
{
    store_tile_t(M + 32 * (kb >> 1) + 4 * (kb & 1) + 4 * (lane >> 4), ld, v, lane);
}

// ---- swizzled pcol tiles ----------------------------------------------------
// The same column order with, in rows 4..11 of every 16-row block, the
// 16-byte units 2u and 2u + 1 of the row trading places (element offset XOR 8
// for 2-byte types; swz_x gives the XOR of row r).  Measured on gfx950: a
// ds_read_b128 serves 16 lanes per clock over 64 four-byte banks, lane 0
// together with lanes 1-3, 12-15 and 20-27 (the quads of equal bit parity),
// and a paired-operand read (16 rows, four 16-byte units each, at row strides
// of 17 or 9 units) puts two lanes on one bank in every group: 8 clocks
// instead of 4.  With the swap every group covers 64 distinct banks.  Every
// access to such a tile (reads, transposed stores, staging writes) applies
// the XOR of its row; base pointers sit at a 16-row block and at a multiple
// of 16 columns, so the XOR touches only the in-block offset.
__host__ __device__ constexpr int swz_x(int r) { return ((((r & 15) + 4) >> 3) & 1) << 3; }

template <typename T>
__device__ __forceinline__ typename Pair<T>::type pair_lds_sw(const T* M, int ld, int lane)
{
    static_assert(sizeof(T) == 2, "16-byte units of 2-byte elements");
    return *reinterpret_cast<const bf16x8*>(M + (lane & 15) * ld + ((8 * (lane >> 4)) ^ swz_x(lane & 15)));
}

// Mfma<T>::load of a swizzled tile (k0 a multiple of 32)
template <typename T>
__device__ __forceinline__ typename Mfma<T>::frag mfma_load_sw(const T* row0, int ld, int k0, int lane)
{
    static_assert(sizeof(T) == 2, "16-byte units of 2-byte elements");
    return *reinterpret_cast<const typename Mfma<T>::frag*>(
        row0 + (lane & 15) * ld + ((k0 + 8 * (lane >> 4)) ^ swz_x(lane & 15)));
}

template <typename T>
__device__ __forceinline__ typename Frag16<T>::type frag16_lds_pc_sw(const T* M, int ld, int kb, int lane)
{
    static_assert(sizeof(T) == 2, "16-byte units of 2-byte elements");
    return *reinterpret_cast<const typename Frag16<T>::type*>(
        M + (lane & 15) * ld + ((32 * (kb >> 1) + 4 * (kb & 1) + 8 * (lane >> 4)) ^ swz_x(lane & 15)));
}

template <typename T>
__device__ __forceinline__ void store_tile_t_pc_sw(T* M, int ld, int kb, floatx4 v, int lane)
{
    static_assert(sizeof(T) == 2, "16-byte units of 2-byte elements");
    T* p = M + (lane & 15) * ld + ((32 * (kb >> 1) + 4 * (kb & 1) + 8 * (lane >> 4)) ^ swz_x(lane & 15));
    bf16x4 w;
    w[0] = from_f32<bf16>(v[0]); w[1] = from_f32<bf16>(v[1]);
    w[2] = from_f32<bf16>(v[2]); w[3] = from_f32<bf16>(v[3]);
    *reinterpret_cast<bf16x4*>(p) = w;
}

// Identity as a K = 16 right factor (lane holds I[4(l/16)+r][l%16]): mma16
// with it returns the left factor's block in the result layout, i.e. an exact
// transpose when stored with store_tile_t.
template <typename T>
__device__ __forceinline__ typename Frag16<T>::type ident_frag(int lane)
{
    int ln = lane;
    asm volatile("" : "+v"(ln));   // rebuild here, not once per kernel
    const int c = ln & 15, g4 = 4 * (ln >> 4);
    floatx4 b;
#pragma unroll
    for (int r = 0; r < 4; ++r) b[r] = (g4 + r == c) ? 1.f : 0.f;
    return frag16_acc<T>(b);
}

// Load a 16x16 fp32 block from LDS in the result layout (lane holds
// B[4(l/16)+r][l%16]).
__device__ __forceinline__ floatx4 load_tile_rl(const float* B, int ldb, int lane)
{
    floatx4 b;
#pragma unroll
    for (int r = 0; r < 4; ++r) b[r] = B[(4 * (lane >> 4) + r) * ldb + (lane & 15)];
    return b;
}

}  // namespace linattn
