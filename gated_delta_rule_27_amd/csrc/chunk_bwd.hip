// chunk_bwd.hip — backward pass of the chunkwise forward, gates none and
// scalar, add and delta rules ("Linear Attention, Visualized", "Update the
// state": the chunk form trains with one saved state per chunk; the per-chunk
// quantities of "Chunkwise algorithm", the GDN table and "The triangular
// correction system", differentiated; "Beyond attention", "Chunkwise parallel
// training").
//
// Per chunk r (C = 64 local positions, G the in-chunk prefix of the log-gate,
// D[l,m] = exp(G_l - G_m), <-Q = exp(G) Q, <-K = exp(G) K, ->K = exp(G_C - G) K,
// A the causal decayed scores, L the strict decayed key scores,
// T = (I + diag(beta) L)^-1, Tb = T diag(beta); forward R = V - <-K S_r,
// Z = Tb R (add rule: Z = V)):
//
//   reverse state pass, newest chunk first (dS = gradient w.r.t. S_{r+1}):
//     dZ = A^T dO + ->K dS ;  dR = Tb^T dZ ;  dS_r = exp(G_C) dS + <-Q^T dO - <-K^T dR
//   per-chunk gradients, from S_r and dS_{r+1} alone:
//     dv = dR ; d<-Q = dO S_r^T ; d<-K = -dR S_r^T ; d->K = Z dS^T
//     dA = dO Z^T (causal) ; dTb = dZ R^T (causal)
//     dbeta_m = sum_l T[l,m] dTb[l,m] + sum_k dM[m,k] L[m,k],  dM = -T^T dTb Tb^T
//     dL = diag(beta) dM (strict) ; P = dA . D ; P2 = dL . D
//     dq = exp(G) d<-Q + P K
//     dk = exp(G) d<-K + exp(G_C - G) d->K + P^T Q + (P2 + P2^T) K
//     dG_l = q_l.(exp(G_l) d<-Q_l) + k_l.(exp(G_l) d<-K_l) - k_l.(exp(G_C-G_l) d->K_l)
//            + rowsum_l(dA.A) - colsum_l(dA.A) + rowsum_l(dL.L) - colsum_l(dL.L)
//     dG_C += sum_l k_l.(exp(G_C-G_l) d->K_l) + exp(G_C) <S_r, dS>
//     dg = reverse prefix sum of dG within the chunk.
//
// Three kernels: bwd_ops_kernel (per chunk, parallel) prepares the operands of
// the reverse state pass; bwd_chain_kernel runs that pass per (head, 64 value
// columns) and stores dS_{r+1} of every chunk; bwd_grad_kernel (per chunk,
// parallel) forms every gradient of its chunk.  The incoming states S_r come
// from the forward (chunk_fused_kernel with SAVE).  Padding rows of a ragged
// last chunk are zero (q = k = v = dO = 0, g = 0, beta = 0), as in the forward.
//
// The 16x16 products read their operands from LDS in either orientation
// (tile<>): a product of this pass has several operand orientations, and every
// matrix is kept once.
#include <cstdlib>

#include "device_common.h"
#include "launch.h"
#include "mfma.h"
#include "prep.h"
#include "tile_rows.h"

namespace linattn {

namespace {

constexpr int kC = 64;
constexpr int kNT = 512;                 // 8 waves
constexpr float kLog2eB = 1.4426950408889634f;   // log2(e): channel gates are kept in base 2
// A diagonal 16x16 block of a per-channel decay splits at its middle row m7,
// 2^(G_l - G_m) = 2^(G_l - G_m7) 2^(G_m7 - G_m), each factor within 2^(+-kSpanMax)
// when every |G_l - G_m7| of the block is: then the block is one matrix-core
// product like the others; past that it is summed element by element.
constexpr float kSpanMax = 120.f;
typedef __attribute__((__vector_size__(16))) int i4;

template <typename T> using F16 = typename Frag16<T>::type;

// K = 16 operand fragment of lane l at contraction offset k0: element
// (x0 + l%16, k0 + 4(l/16) + r), r = 0..3, of a matrix whose element (x, k) is
// stored at P[x*ld + k] (frag_xk, one vector read) or at P[k*ld + x] (frag_kx).
// x is the output row for an A operand and the output column for a B operand.
// frag_xk reads through a volatile pointer of the LDS address space so that
// each read stays one ds_read_b64: the compiler would otherwise merge two reads
// from one base into a ds_read2_b64, which on gfx950 serves 16 lanes per clock
// over 32 banks and takes four times the LDS cycles of one ds_read_b64.
template <typename T>
__device__ __forceinline__ F16<T> frag_xk(const T* P, int ld, int x0, int k0, int lane)
{
    typedef const volatile __attribute__((address_space(3))) F16<T>* LP;
    return *(LP)(P + (x0 + (lane & 15)) * ld + k0 + 4 * (lane >> 4));
}

template <typename T>
__device__ __forceinline__ F16<T> frag_kx(const T* P, int ld, int x0, int k0, int lane)
{
    if constexpr (sizeof(T) == 2) {
        // gfx950's LDS transpose read: each 16-lane group g reads the 4 x 16
        // block at rows k0 + 4g .. k0 + 4g + 3, columns x0 .. x0 + 15, lane
        // 4j + c of the group supplying the address of row j, columns 4c ..
        // 4c + 3 (8 bytes), and lane i of the group receives column i of the
        // four rows: the fragment in one read instead of four 2-byte reads
        // (each lane's 8 bytes must be aligned: ld and x0 are multiples of 4
        // at every call)
        typedef short v4s __attribute__((ext_vector_type(4)));
        typedef __attribute__((address_space(3))) v4s* LP;
        const int w = lane & 15;
        const T* p = P + (k0 + 4 * (lane >> 4) + (w >> 2)) * ld + x0 + 4 * (w & 3);
        const v4s x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LP)(T*)p);
        F16<T> f;
        __builtin_memcpy(&f, &x, 8);
        return f;
    } else {
        const T* p = P + (k0 + 4 * (lane >> 4)) * ld + x0 + (lane & 15);
        F16<T> f;
        f[0] = p[0];
        f[1] = p[ld];
        f[2] = p[2 * ld];
        f[3] = p[3 * ld];
        return f;
    }
}

// acc += sum_{k in [kb, ke)} A(m0 + ., k) B(k, n0 + .) as a 16x16 result tile
// (lane l holds D[4(l/16) + r][l%16]); AXK / BXK: operand stored as (x, k)
// rows, else as (k, x) rows.
template <typename T, bool AXK, bool BXK>
__device__ __forceinline__ floatx4 tile(floatx4 acc, const T* A, int lda, int m0, const T* B, int ldb,
                                        int n0, int kb, int ke, int lane)
{
    for (int k0 = kb; k0 < ke; k0 += 16) {
        F16<T> a, b;
        if constexpr (AXK) a = frag_xk(A, lda, m0, k0, lane);
        else a = frag_kx(A, lda, m0, k0, lane);
        if constexpr (BXK) b = frag_xk(B, ldb, n0, k0, lane);
        else b = frag_kx(B, ldb, n0, k0, lane);
        acc = mma16<T>(a, b, acc);
    }
    return acc;
}

// The same product over a fixed range [k0, k0 + K), every fragment read before
// the first matrix-core op and pairs of K = 16 steps issued as one K = 32 op.
// Causal operands are zero outside their triangle, so a product over the full
// range equals the one over the causal part.
template <typename T, bool AXK, bool BXK, int K>
__device__ __forceinline__ floatx4 tilek(floatx4 acc, const T* A, int lda, int m0, const T* B, int ldb,
                                         int n0, int k0, int lane)
{
    constexpr int NS = K / 16;
    static_assert(NS % 2 == 0 || sizeof(T) == 4 || NS == 1, "one matrix-core shape per chain");
    F16<T> a[NS], b[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        if constexpr (AXK) a[s] = frag_xk(A, lda, m0, k0 + 16 * s, lane);
        else a[s] = frag_kx(A, lda, m0, k0 + 16 * s, lane);
        if constexpr (BXK) b[s] = frag_xk(B, ldb, n0, k0 + 16 * s, lane);
        else b[s] = frag_kx(B, ldb, n0, k0 + 16 * s, lane);
    }
    if constexpr (NS == 1) {
        acc = mma16<T>(a[0], b[0], acc);
    } else {
#pragma unroll
        for (int s = 0; s < NS; s += 2) acc = mma16x2<T>(a[s], a[s + 1], b[s], b[s + 1], acc);
    }
    return acc;
}

// result tile into P[m*ld + n] (row-major)
template <typename T>
__device__ __forceinline__ void put(T* P, int ld, int m0, int n0, floatx4 v, int lane)
{
    T* p = P + (m0 + 4 * (lane >> 4)) * ld + n0 + (lane & 15);
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r * ld] = from_f32<T>(v[r]);
}

// (lj, mi) of the p-th causal 16x16 tile (mi <= lj), row-major over lj
__device__ __forceinline__ void causal_tile(int p, int& lj, int& mi)
{
    lj = 0;
    while (p > lj) { p -= lj + 1; ++lj; }
    mi = p;
}

template <typename T, int DK>
struct BwdCfg {
    static constexpr int PAD = 16 / sizeof(T);       // 16-byte row padding
    static constexpr int E = 16 / sizeof(T);         // elements per 16-byte vector
    static constexpr int LDQ = DK + PAD;             // rows of length dk
    static constexpr int LDC = kC + PAD;             // rows of length C
    static constexpr int J = sizeof(T) == 2 ? 32 : 16;   // value columns per step of the gradient kernel
    static constexpr int LDJ = J + PAD;
    static constexpr int LDF = kC + 4;               // fp32 scratch rows
    // per-chunk operands (token type, dense): of the reverse state pass A^T,
    // Tb^T [C][C], ->K [C][dk], <-Q^T, -<-K^T [dk][C]; and Tb [C][C] for the
    // gradient pass
    static constexpr int OPS = 3 * kC * kC + 3 * kC * DK;
    static constexpr int O_AQT = 0, O_TBT = kC * kC, O_TB = 2 * kC * kC, O_KR = 3 * kC * kC,
                         O_QDT = O_KR + kC * DK, O_NKDT = O_QDT + DK * kC;
};

// 16 consecutive rows of one column of a [rows][ld] bf16 matrix, rows from
// row0; rows at or past nvalid read as 0.  The addresses are clamped instead
// of branched around, so the 16 loads issue back to back.
__device__ __forceinline__ void load_col16(float* x, const bf16* base, int ld, int row0, int nvalid)
{
    bf16 raw[16];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
        const int row = row0 + rr < nvalid ? row0 + rr : nvalid - 1;
        raw[rr] = base[(int64_t)row * ld];
    }
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) x[rr] = row0 + rr < nvalid ? to_f32(raw[rr]) : 0.f;
}

// T = (I + diag(beta) L)^-1 and Tb = T diag(beta) from the strict lower
// triangular L in LDS (Tm must hold zeros above its diagonal blocks); every
// thread of the workgroup calls this, the results are in LDS on return.
template <typename T>
__device__ __forceinline__ void tri_inverse(const T* Lm, T* Tm, T* Tb, const float* bet, int tid)
{
    using C = BwdCfg<T, 64>;
    constexpr int LDC = C::LDC;
    const int lane = tid & 63, wave = tid >> 6;
    // diagonal 16x16 blocks of T by forward substitution, fp32: lane = (block
    // b, column j); x_i = [i == j] - beta_i sum_{s < i} L_is x_s
    if (wave == 0) {
        const int b = lane >> 4, j = lane & 15;
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float acc = i == j ? 1.f : 0.f;
            const T* lrow = Lm + (16 * b + i) * LDC + 16 * b;
            float s = 0.f;
#pragma unroll
            for (int s2 = 0; s2 < i; ++s2) s += to_f32(lrow[s2]) * x[s2];
            x[i] = acc - bet[16 * b + i] * s;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) Tm[(16 * b + i) * LDC + 16 * b + j] = from_f32<T>(x[i]);
    }
    __syncthreads();
    // blocks below the diagonal, one diagonal of blocks at a time:
    // T_ij = -T_ii diag(beta_i) sum_{s=j}^{i-1} L_is T_sj
    for (int d = 1; d < 4; ++d) {
        if (wave < 4 - d) {
            const int i = wave + d, j = wave;
            floatx4 y = tile<T, true, false>(zero4(), Lm, LDC, 16 * i, Tm, LDC, 16 * j, 16 * j, 16 * i, lane);
#pragma unroll
            for (int r = 0; r < 4; ++r) y[r] *= -bet[16 * i + 4 * (lane >> 4) + r];
            const floatx4 t = mma16<T>(frag_xk(Tm, LDC, 16 * i, 16 * i, lane), frag16_acc<T>(y), zero4());
            put(Tm, LDC, 16 * i, 16 * j, t, lane);
        }
        __syncthreads();
    }
    for (int i = tid; i < kC * kC; i += kNT) {
        const int l = i / kC, m = i % kC;
        Tb[l * LDC + m] = from_f32<T>(to_f32(Tm[l * LDC + m]) * bet[m]);
    }
    __syncthreads();
}

// Shared front of the two per-chunk kernels: chunk r's q and k (zero rows past
// the end), the in-chunk gate prefix G, exp(G), beta, the causal decayed
// scores A, the strict decayed key scores L and, for the delta rule,
// T = (I + diag(beta) L)^-1 and Tb = T diag(beta), all in LDS.
template <typename T, int DK>
struct IntraLds {
    T *Qs, *Ks, *Aq, *Lm, *Tm, *Tb;
    float *G, *gam, *bet;
};

template <typename T, int DK, int RULE, int GATE>
__device__ void intra_chunk(const IntraLds<T, DK>& L, const T* __restrict__ q, const T* __restrict__ k,
                            const T* __restrict__ g, const T* __restrict__ beta, int64_t bh, int64_t Tlen,
                            int64_t t0, int tvalid, int tid)
{
    using C = BwdCfg<T, DK>;
    constexpr int LDQ = C::LDQ, LDC = C::LDC, E = C::E;
    constexpr bool DELTA = RULE == kRuleDelta, GATED = GATE == kGateScalar;
    const int lane = tid & 63, wave = tid >> 6;

    // A, L and T are written on their causal part only: clear them
    {
        constexpr int NZ = 3 * kC * LDC * (int)sizeof(T) / 16;
        i4* z = reinterpret_cast<i4*>(L.Aq);   // Aq, Lm, Tm are contiguous
        for (int i = tid; i < NZ; i += kNT) z[i] = i4{0, 0, 0, 0};
    }
    {
        constexpr int VR = DK / E;
        for (int i = tid; i < kC * VR; i += kNT) {
            const int row = i / VR, c = (i % VR) * E;
            i4 a = {0, 0, 0, 0}, b = {0, 0, 0, 0};
            if (row < tvalid) {
                a = *reinterpret_cast<const i4*>(q + (bh * Tlen + t0 + row) * DK + c);
                b = *reinterpret_cast<const i4*>(k + (bh * Tlen + t0 + row) * DK + c);
            }
            *reinterpret_cast<i4*>(L.Qs + row * LDQ + c) = a;
            *reinterpret_cast<i4*>(L.Ks + row * LDQ + c) = b;
        }
    }
    if (wave == 0) {
        float gl = 0.f, bl = 0.f;
        if (lane < tvalid) {
            if constexpr (GATED) gl = to_f32(g[bh * Tlen + t0 + lane]);
            if constexpr (DELTA) bl = to_f32(beta[bh * Tlen + t0 + lane]);
        }
        const float G = wave_prefix_sum(gl);
        L.G[lane] = G;
        L.gam[lane] = GATED ? expf(G) : 1.f;
        L.bet[lane] = bl;
    }
    __syncthreads();

    // A (causal) and L (strict): 10 causal tiles each
    {
        constexpr int NJOB = DELTA ? 20 : 10;
        for (int j = wave; j < NJOB; j += 8) {
            const bool isL = j >= 10;
            int lb, mb;
            causal_tile(isL ? j - 10 : j, lb, mb);
            floatx4 acc = tilek<T, true, true, DK>(zero4(), isL ? L.Ks : L.Qs, LDQ, 16 * lb, L.Ks, LDQ,
                                                   16 * mb, 0, lane);
            const int m = 16 * mb + (lane & 15);
            floatx4 val;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int l = 16 * lb + 4 * (lane >> 4) + r;
                const float d = GATED ? expf(fminf(L.G[l] - L.G[m], 0.f)) : 1.f;
                val[r] = (isL ? m < l : m <= l) ? acc[r] * d : 0.f;
            }
            put(isL ? L.Lm : L.Aq, LDC, 16 * lb, 16 * mb, val, lane);
        }
    }
    __syncthreads();
    if constexpr (DELTA) tri_inverse<T>(L.Lm, L.Tm, L.Tb, L.bet, tid);
}

// ============================================================================
// bwd_ops_kernel: per chunk, the operands of the reverse state pass.
// ============================================================================
template <typename T, int DK, int RULE, int GATE>
__global__ __launch_bounds__(kNT, 1) void bwd_ops_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                         const T* __restrict__ g, const T* __restrict__ beta,
                                                         T* __restrict__ ops, float* __restrict__ gC,
                                                         int64_t Tlen, int64_t nchunks)
{
    using C = BwdCfg<T, DK>;
    constexpr int LDQ = C::LDQ, LDC = C::LDC, E = C::E;
    constexpr bool DELTA = RULE == kRuleDelta, GATED = GATE == kGateScalar;
    __shared__ __align__(16) T Qs[kC * LDQ], Ks[kC * LDQ];
    __shared__ __align__(16) T CC[4 * kC * LDC];    // Aq, Lm, Tm, Tb
    __shared__ __align__(16) float G[kC], gam[kC], bet[kC];

    const int tid = threadIdx.x;
    const int64_t bh = blockIdx.x / nchunks, r = blockIdx.x % nchunks;
    const int64_t t0 = r * kC;
    const int tvalid = (int)(Tlen - t0 < kC ? Tlen - t0 : kC);
    IntraLds<T, DK> L{Qs, Ks, CC, CC + kC * LDC, CC + 2 * kC * LDC, CC + 3 * kC * LDC, G, gam, bet};
    intra_chunk<T, DK, RULE, GATE>(L, q, k, g, beta, bh, Tlen, t0, tvalid, tid);

    T* out = ops + (bh * nchunks + r) * (int64_t)C::OPS;
    auto store = [&](T* dst, const float* x) {
        T e[E];
#pragma unroll
        for (int i = 0; i < E; ++i) e[i] = from_f32<T>(x[i]);
        i4 w;
        __builtin_memcpy(&w, e, 16);
        *reinterpret_cast<i4*>(dst) = w;
    };
    if constexpr (sizeof(T) == 2) {
        // 2-byte tokens: every transposed operand goes out in 8x8 blocks, one
        // per thread: eight 16-byte rows read from LDS, transposed (and scaled)
        // in registers, eight 16-byte rows written.  Within a wave, lane =
        // column block + 8 x row block of the source, so each 16-lane group of
        // a row read covers 64 distinct banks and the eight lanes of a row
        // block write 128 contiguous bytes.
        // Blocks: A^T (64), Tb^T (64, delta), <-Q^T and -<-K^T (delta), 8 dk/8
        // each; every part is a whole number of waves.
        constexpr int NQB = 8 * (DK / 8);
        constexpr int NB = 64 + (DELTA ? 64 : 0) + NQB + (DELTA ? NQB : 0);
        for (int job = tid; job < NB; job += kNT) {
            const T* M;
            T* dst;
            int ldm, b = job;
            bool scaled = false;
            float sgn = 1.f;
            if (b < 64) {
                M = L.Aq; ldm = LDC; dst = out + C::O_AQT;
            } else if (DELTA && b < 128) {
                M = L.Tb; ldm = LDC; dst = out + C::O_TBT; b -= 64;
            } else {
                b -= DELTA ? 128 : 64;
                ldm = LDQ; scaled = GATED;
                if (b < NQB) {
                    M = Qs; dst = out + C::O_QDT;
                } else {
                    M = Ks; dst = out + C::O_NKDT; b -= NQB; sgn = -1.f; scaled = true;
                }
            }
            const int bc = 8 * (b >> 6) + (b & 7), br = (b & 63) >> 3;
            bf16x8 rw[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) rw[i] = *reinterpret_cast<const bf16x8*>(M + (8 * br + i) * ldm + 8 * bc);
            float sc[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) sc[i] = sgn * gam[8 * br + i];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                bf16x8 w;
#pragma unroll
                for (int i = 0; i < 8; ++i) w[i] = scaled ? from_f32<T>(to_f32(rw[i][j]) * sc[i]) : rw[i][j];
                *reinterpret_cast<bf16x8*>(dst + (8 * bc + j) * kC + 8 * br) = w;
            }
        }
        if constexpr (DELTA) {
            for (int v = tid; v < kC * kC / E; v += kNT) {
                const int l = v / (kC / E), m0 = (v % (kC / E)) * E;
                *reinterpret_cast<i4*>(out + C::O_TB + l * kC + m0) = *reinterpret_cast<const i4*>(L.Tb + l * LDC + m0);
            }
        }
        // ->K = exp(G_C - G) K
        for (int v = tid; v < kC * DK / E; v += kNT) {
            const int l = v / (DK / E), i0 = (v % (DK / E)) * E;
            const float sv = GATED ? expf(G[kC - 1] - G[l]) : 1.f;
            const bf16x8 kr = *reinterpret_cast<const bf16x8*>(Ks + l * LDQ + i0);
            bf16x8 w;
#pragma unroll
            for (int i = 0; i < E; ++i) w[i] = from_f32<T>(to_f32(kr[i]) * sv);
            *reinterpret_cast<bf16x8*>(out + C::O_KR + l * DK + i0) = w;
        }
    } else {
        float x[E];
        // A^T and Tb^T: row l holds column l of A / Tb
        for (int v = tid; v < kC * kC / E; v += kNT) {
            const int l = v / (kC / E), m0 = (v % (kC / E)) * E;
    #pragma unroll
            for (int i = 0; i < E; ++i) x[i] = to_f32(L.Aq[(m0 + i) * LDC + l]);
            store(out + C::O_AQT + l * kC + m0, x);
            if constexpr (DELTA) {
    #pragma unroll
                for (int i = 0; i < E; ++i) x[i] = to_f32(L.Tb[(m0 + i) * LDC + l]);
                store(out + C::O_TBT + l * kC + m0, x);
            }
        }
        if constexpr (DELTA) {
            for (int v = tid; v < kC * kC / E; v += kNT) {
                const int l = v / (kC / E), m0 = (v % (kC / E)) * E;
                *reinterpret_cast<i4*>(out + C::O_TB + l * kC + m0) = *reinterpret_cast<const i4*>(L.Tb + l * LDC + m0);
            }
        }
        // ->K = exp(G_C - G) K
        for (int v = tid; v < kC * DK / E; v += kNT) {
            const int l = v / (DK / E), i0 = (v % (DK / E)) * E;
            const float s = GATED ? expf(G[kC - 1] - G[l]) : 1.f;
    #pragma unroll
            for (int i = 0; i < E; ++i) x[i] = to_f32(Ks[l * LDQ + i0 + i]) * s;
            store(out + C::O_KR + l * DK + i0, x);
        }
        // <-Q^T and -<-K^T: row i holds key channel i over the chunk
        for (int v = tid; v < DK * kC / E; v += kNT) {
            const int i = v / (kC / E), m0 = (v % (kC / E)) * E;
    #pragma unroll
            for (int e = 0; e < E; ++e) x[e] = to_f32(Qs[(m0 + e) * LDQ + i]) * gam[m0 + e];
            store(out + C::O_QDT + i * kC + m0, x);
            if constexpr (DELTA) {
    #pragma unroll
                for (int e = 0; e < E; ++e) x[e] = -to_f32(Ks[(m0 + e) * LDQ + i]) * gam[m0 + e];
                store(out + C::O_NKDT + i * kC + m0, x);
            }
        }
    }
    if (tid == 0) gC[bh * nchunks + r] = gam[kC - 1];
}

// ============================================================================
// bwd_ops_channel_kernel: per chunk, the operands of the reverse state pass and
// of the gradient pass for the per-key-channel gate (bf16 tokens; "Linear
// Attention, Visualized", "Gated Linear Attention (GLA)" and "Kimi Delta
// Attention (KDA)": the decay is a diagonal matrix, so every score keeps the
// decay inside its sum over key channels).  With G[l][c] the in-chunk prefix
// of channel c's log-gate (kept in base 2: log2(e) g, so each factor is one
// hardware exp2):
//   A[l][m] = sum_c q_lc 2^(G_lc - G_mc) k_mc (m <= l),  L[l][m] the same with
//   k_l in place of q_l (m < l).
// Off the diagonal 16x16 blocks (row l in block i, key m in block j < i) the
// factor splits at row s = 16 i - 1 into 2^(G_l - G_s) 2^(G_s - G_m), both at
// most 1 for decays, applied to the operands of one matrix-core product; a
// diagonal block splits at its middle row when both factors stay within
// 2^(+-kSpanMax), else it is summed element by element with the exact factor.
// Stored per chunk: A^T, Tb^T, Tb, ->K, <-Q^T, -<-K^T (the reverse state pass,
// as bwd_ops_kernel), T and L (the gradient pass), and 2^(G_C) per channel.
// ============================================================================
template <int DK, int RULE>
__global__ __launch_bounds__(kNT, 1) void bwd_ops_channel_kernel(const bf16* __restrict__ q,
                                                                 const bf16* __restrict__ k,
                                                                 const bf16* __restrict__ g,
                                                                 const bf16* __restrict__ beta,
                                                                 bf16* __restrict__ ops, float* __restrict__ gC,
                                                                 int64_t Tlen, int64_t nchunks)
{
    using C = BwdCfg<bf16, DK>;
    constexpr int LDQ = C::LDQ, LDC = C::LDC, E = C::E, LDG = DK + 4;
    constexpr bool DELTA = RULE == kRuleDelta;
    constexpr int OSTRIDE = C::OPS + 2 * kC * kC;
    __shared__ __align__(16) bf16 Qs[kC * LDQ], Ks[kC * LDQ];
    __shared__ __align__(16) bf16 CC[4 * kC * LDC];    // Aq, Lm, Tm, Tb
    __shared__ __align__(16) float Gf[kC * LDG];        // G, base 2
    __shared__ __align__(16) float tot[4][DK];
    __shared__ float bet[kC], spanw[8];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t bh = blockIdx.x / nchunks, r = blockIdx.x % nchunks;
    const int64_t t0 = r * kC;
    const int tvalid = (int)(Tlen - t0 < kC ? Tlen - t0 : kC);
    bf16* const Aq = CC;
    bf16* const Lm = CC + kC * LDC;
    bf16* const Tm = CC + 2 * kC * LDC;
    bf16* const Tb = CC + 3 * kC * LDC;

    {
        constexpr int NZ = 3 * kC * LDC * 2 / 16;      // Aq, Lm, Tm
        i4* z = reinterpret_cast<i4*>(CC);
        for (int i = tid; i < NZ; i += kNT) z[i] = i4{0, 0, 0, 0};
    }
    {
        constexpr int VR = DK / E;
        for (int i = tid; i < kC * VR; i += kNT) {
            const int row = i / VR, c = (i % VR) * E;
            i4 a = {0, 0, 0, 0}, b = {0, 0, 0, 0};
            if (row < tvalid) {
                a = *reinterpret_cast<const i4*>(q + (bh * Tlen + t0 + row) * DK + c);
                b = *reinterpret_cast<const i4*>(k + (bh * Tlen + t0 + row) * DK + c);
            }
            *reinterpret_cast<i4*>(Qs + row * LDQ + c) = a;
            *reinterpret_cast<i4*>(Ks + row * LDQ + c) = b;
        }
    }
    if (tid < kC) bet[tid] = (DELTA && tid < tvalid) ? to_f32(beta[bh * Tlen + t0 + tid]) : 0.f;
    // prefix: thread (block pb, channel pc) walks its block's 16 rows
    const int pc = tid % DK, pb = tid / DK;
    const bool pre = tid < 4 * DK;
    float Gl[16];
    if (pre) {
        load_col16(Gl, g + (bh * Tlen + t0) * DK + pc, DK, 16 * pb, tvalid);
        float acc = 0.f;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            acc += Gl[rr] * kLog2eB;
            Gl[rr] = acc;
        }
        tot[pb][pc] = acc;
    }
    __syncthreads();
    float span = 0.f;
    if (pre) {
        float off = 0.f;
#pragma unroll
        for (int b = 0; b < 3; ++b)
            if (b < pb) off += tot[b][pc];
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            Gf[(16 * pb + rr) * LDG + pc] = off + Gl[rr];
            span = fmaxf(span, fabsf(Gl[rr] - Gl[7]));
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) span = fmaxf(span, shfl_xor(span, o));
    if (lane == 0) spanw[wave] = span;
    __syncthreads();
    bool safe[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        float sp = spanw[b * (DK / 64)];
        if constexpr (DK == 128) sp = fmaxf(sp, spanw[2 * b + 1]);
        safe[b] = sp <= kSpanMax;
    }

    // score tiles, A and L together (their query-side factors are the same):
    // jobs 0-5 the off-diagonal pairs (1,0)(2,0)(2,1)(3,0)(3,1)(3,2), split at
    // the row before the query block; jobs 6-9 the diagonal blocks, split at
    // their middle row
    for (int job = wave; job < 10; job += 8) {
        const bool diag = job >= 6;
        const int i = diag ? job - 6 : (job < 1 ? 1 : (job < 3 ? 2 : 3));
        const int j = diag ? i : job - i * (i - 1) / 2;
        if (diag && !safe[i]) continue;
        const int s = diag ? 16 * i + 7 : 16 * i - 1;
        const int xa = 16 * i + (lane & 15), xb = 16 * j + (lane & 15);
        floatx4 accA = zero4(), accL = zero4();
#pragma unroll
        for (int k0 = 0; k0 < DK; k0 += 16) {
            const int c0 = k0 + 4 * (lane >> 4);
            const floatx4 gs = *reinterpret_cast<const floatx4*>(&Gf[s * LDG + c0]);
            const floatx4 ga = *reinterpret_cast<const floatx4*>(&Gf[xa * LDG + c0]);
            const floatx4 gb = *reinterpret_cast<const floatx4*>(&Gf[xb * LDG + c0]);
            const bf16x4 qa = *reinterpret_cast<const bf16x4*>(&Qs[xa * LDQ + c0]);
            const bf16x4 ka = *reinterpret_cast<const bf16x4*>(&Ks[xa * LDQ + c0]);
            const bf16x4 kb = *reinterpret_cast<const bf16x4*>(&Ks[xb * LDQ + c0]);
            bf16x4 fq, fk, fb;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float ua = fast_exp2(ga[e] - gs[e]), wb = fast_exp2(gs[e] - gb[e]);
                fq[e] = from_f32<bf16>(to_f32(qa[e]) * ua);
                fk[e] = from_f32<bf16>(to_f32(ka[e]) * ua);
                fb[e] = from_f32<bf16>(to_f32(kb[e]) * wb);
            }
            accA = mma16<bf16>(fq, fb, accA);
            if constexpr (DELTA) accL = mma16<bf16>(fk, fb, accL);
        }
        if (diag) {
            // result (l = 16 i + 4(lane/16) + rr, m = 16 i + lane%16): causal / strict
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int lo = 4 * (lane >> 4) + rr, mo = lane & 15;
                accA[rr] = mo <= lo ? accA[rr] : 0.f;
                accL[rr] = mo < lo ? accL[rr] : 0.f;
            }
        }
        put(Aq, LDC, 16 * i, 16 * j, accA, lane);
        if constexpr (DELTA) put(Lm, LDC, 16 * i, 16 * j, accL, lane);
    }
    // diagonal blocks past the split's range, element by element with the
    // exact factor: item = (block b, l >= m inside it)
    for (int it = tid; it < 4 * 136; it += kNT) {
        const int b = it / 136;
        if (safe[b]) continue;
        int li = 0, p = it % 136;
        while (p > li) { p -= li + 1; ++li; }
        const int l = 16 * b + li, m = 16 * b + p;
        float a = 0.f, n = 0.f;
        for (int c0 = 0; c0 < DK; c0 += 4) {
            const floatx4 gl = *reinterpret_cast<const floatx4*>(&Gf[l * LDG + c0]);
            const floatx4 gm = *reinterpret_cast<const floatx4*>(&Gf[m * LDG + c0]);
            const bf16x4 ql = *reinterpret_cast<const bf16x4*>(&Qs[l * LDQ + c0]);
            const bf16x4 kl = *reinterpret_cast<const bf16x4*>(&Ks[l * LDQ + c0]);
            const bf16x4 km = *reinterpret_cast<const bf16x4*>(&Ks[m * LDQ + c0]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float dk_ = to_f32(km[e]) * fast_exp2(gl[e] - gm[e]);
                a = fmaf(to_f32(ql[e]), dk_, a);
                n = fmaf(to_f32(kl[e]), dk_, n);
            }
        }
        Aq[l * LDC + m] = from_f32<bf16>(a);
        if constexpr (DELTA) Lm[l * LDC + m] = from_f32<bf16>(m < l ? n : 0.f);
    }
    __syncthreads();
    if constexpr (DELTA) tri_inverse<bf16>(Lm, Tm, Tb, bet, tid);

    bf16* out = ops + (bh * nchunks + r) * (int64_t)OSTRIDE;
    auto copy_rows = [&](bf16* dst, const bf16* src) {
        for (int v = tid; v < kC * kC / E; v += kNT) {
            const int l = v / (kC / E), m0 = (v % (kC / E)) * E;
            *reinterpret_cast<i4*>(dst + l * kC + m0) = *reinterpret_cast<const i4*>(src + l * LDC + m0);
        }
    };
    // The transposed operands go out in 8x8 blocks, one per thread: eight
    // 16-byte rows read from LDS, transposed (and scaled) in registers, eight
    // 16-byte rows written.  Within a wave, lane = column block + 8 x row
    // block of the source, so each 16-lane group of a row read covers 64
    // distinct banks.  Blocks: A^T (64), Tb^T (64, delta), then <-Q^T with
    // -<-K^T (8 dk/8; the two share their factors 2^(G[m][c])).
    {
        constexpr int NQB = 8 * (DK / 8);
        constexpr int NB = 64 + (DELTA ? 64 : 0) + NQB;
        for (int job = tid; job < NB; job += kNT) {
            int b = job;
            const bool qk = b >= (DELTA ? 128 : 64);
            const bf16* M = Aq;
            int ldm = LDC;
            if (qk) {
                b -= DELTA ? 128 : 64;
                M = Qs;
                ldm = LDQ;
            } else if (b >= 64) {
                b -= 64;
                M = Tb;
            }
            const int bc = 8 * (b >> 6) + (b & 7), br = (b & 63) >> 3;
            bf16x8 rw[8], kw[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) rw[i] = *reinterpret_cast<const bf16x8*>(M + (8 * br + i) * ldm + 8 * bc);
            if (!qk) {
                bf16* dst = out + (M == Aq ? C::O_AQT : C::O_TBT);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    bf16x8 w;
#pragma unroll
                    for (int i = 0; i < 8; ++i) w[i] = rw[i][j];
                    *reinterpret_cast<bf16x8*>(dst + (8 * bc + j) * kC + 8 * br) = w;
                }
            } else {
                float ef[8][8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float* gr = &Gf[(8 * br + i) * LDG + 8 * bc];
                    const floatx4 a = *reinterpret_cast<const floatx4*>(gr);
                    const floatx4 c = *reinterpret_cast<const floatx4*>(gr + 4);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        ef[i][j] = fast_exp2(a[j]);
                        ef[i][j + 4] = fast_exp2(c[j]);
                    }
                    if constexpr (DELTA) kw[i] = *reinterpret_cast<const bf16x8*>(Ks + (8 * br + i) * LDQ + 8 * bc);
                }
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    bf16x8 w, wk;
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        w[i] = from_f32<bf16>(to_f32(rw[i][j]) * ef[i][j]);
                        if constexpr (DELTA) wk[i] = from_f32<bf16>(-to_f32(kw[i][j]) * ef[i][j]);
                    }
                    *reinterpret_cast<bf16x8*>(out + C::O_QDT + (8 * bc + j) * kC + 8 * br) = w;
                    if constexpr (DELTA)
                        *reinterpret_cast<bf16x8*>(out + C::O_NKDT + (8 * bc + j) * kC + 8 * br) = wk;
                }
            }
        }
    }
    if constexpr (DELTA) {
        copy_rows(out + C::O_TB, Tb);
        copy_rows(out + C::OPS, Tm);
        copy_rows(out + C::OPS + kC * kC, Lm);
    }
    // ->K = 2^(G_C - G) . K, per channel
    for (int v = tid; v < kC * DK / E; v += kNT) {
        const int l = v / (DK / E), i0 = (v % (DK / E)) * E;
        const bf16x8 kr = *reinterpret_cast<const bf16x8*>(Ks + l * LDQ + i0);
        const float* gl = &Gf[l * LDG + i0];
        const float* gc = &Gf[(kC - 1) * LDG + i0];
        float gv[8], cv[8];
        *reinterpret_cast<floatx4*>(gv) = *reinterpret_cast<const floatx4*>(gl);
        *reinterpret_cast<floatx4*>(gv + 4) = *reinterpret_cast<const floatx4*>(gl + 4);
        *reinterpret_cast<floatx4*>(cv) = *reinterpret_cast<const floatx4*>(gc);
        *reinterpret_cast<floatx4*>(cv + 4) = *reinterpret_cast<const floatx4*>(gc + 4);
        bf16x8 w;
#pragma unroll
        for (int i = 0; i < E; ++i) w[i] = from_f32<bf16>(to_f32(kr[i]) * fast_exp2(cv[i] - gv[i]));
        *reinterpret_cast<bf16x8*>(out + C::O_KR + l * DK + i0) = w;
    }
    if (tid < DK) gC[(bh * nchunks + r) * DK + tid] = fast_exp2(Gf[(kC - 1) * LDG + tid]);
}

// The gradients of the chunk-leaving states (dstates) are kept in blocks of
// 16 value columns, [B,H,N][dv/16][dk][16], so that the reverse state pass
// writes each wave's 16 columns as one contiguous block: offset of element
// (key row i, value column j) inside one chunk's [dk][dv] state.
__device__ __forceinline__ int dstate_offset(int i, int j, int dk)
{
    return ((j >> 4) * dk + i) * 16 + (j & 15);
}

// ============================================================================
// bwd_chain_kernel: the reverse state pass.  One workgroup per (b, h, 64 value
// columns): waves 0-3 own 16 columns of dS each (dk/16 result tiles, kept in
// registers for the whole sequence; with CHAN the chunk decay is a vector over
// the key rows) and touch no global memory inside the loop; waves 4-7 move the
// chunk operands from HBM to LDS, two chunks ahead (bf16), and dS to HBM.
// Per chunk, newest first: dS (= dS_{r+1}) to LDS; phase 1 dZ = A^T dO + ->K dS,
// dR = Tb^T dZ while the helpers stage <-Q^T, -<-K^T; phase 2
// dS = exp(G_C) dS + <-Q^T dO - <-K^T dR while they stage the previous chunk's
// A^T, Tb^T, ->K and dO^T (dO^T double-buffered, phase 2 reads it) and copy
// the dS of phase 1 to dstates.
// ============================================================================
template <typename T, int DK, int RULE, bool CHAN, int VB = 64>
__global__ __launch_bounds__(kNT, 1) void bwd_chain_kernel(const T* __restrict__ dout, const T* __restrict__ ops,
                                                           int64_t ostride, const float* __restrict__ gC,
                                                           const float* dsT, T* __restrict__ dstates, float* ds0,
                                                           int64_t Tlen, int64_t nchunks, int DV)
{
    using C = BwdCfg<T, DK>;
    constexpr int LDQ = C::LDQ, LDC = C::LDC, E = C::E, ND = DK / 16;
    constexpr bool DELTA = RULE == kRuleDelta;
    constexpr int NH = 256;                            // helper threads
    constexpr int NA = kC * kC / E / NH;               // [C][C] vectors per helper thread
    constexpr int NK = kC * DK / E / NH;               // [C][dk] / [dk][C]
    constexpr int NO = kC * VB / E / NH;               // dO block
    static_assert(VB == 64 || VB == 32, "value block of 64 or 32 columns");
    static_assert(NA >= 1 && NK >= 1 && NO >= 1, "staging split");

    __shared__ __align__(16) T AqT[kC * LDC];
    __shared__ __align__(16) T TbT[DELTA ? kC * LDC : 8];
    __shared__ __align__(16) T Kr[kC * LDQ];
    __shared__ __align__(16) T QdT[DK * LDC];
    __shared__ __align__(16) T NKdT[DELTA ? DK * LDC : 8];
    __shared__ __align__(16) T dOT[2][64 * LDC];       // dO^T of the block: row j, column m
    __shared__ __align__(16) T dSs[DK * LDC];          // dS of the block, handed to the helpers
    __shared__ __align__(16) float gCs[2][CHAN ? DK : 1];   // exp(G_C), per key channel with CHAN

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nvb = DV / VB;
    // the value blocks of one head read the same chunk operands: dispatch puts
    // workgroup i on XCD i mod 8, so consecutive logical blocks are spread to
    // land on one XCD (and its L2)
    int blk = blockIdx.x;
    if ((gridDim.x & 7) == 0) blk = (blk & 7) * (gridDim.x >> 3) + (blk >> 3);
    const int64_t bh = blk / nvb;
    const int vb = blk % nvb;

    if (wave < VB / 16) {
        const int n0 = 16 * wave;
        const int cl = lane & 15, g4 = 4 * (lane >> 4);
        const int64_t col = (int64_t)vb * VB + n0 + cl;
        floatx4 dS[ND];
#pragma unroll
        for (int db = 0; db < ND; ++db)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
                dS[db][rr] = dsT ? dsT[(bh * DK + 16 * db + g4 + rr) * DV + col] : 0.f;
        wait_vmem_all();
        __syncthreads();
        for (int64_t c = nchunks - 1; c >= 0; --c) {
            const int ln = opaque(lane);
            const int buf = (int)(c & 1);
            // Fragments are read from LDS two row blocks ahead of the products
            // that use them; the scheduling barriers keep the compiler from
            // sinking each read down to its product, which would make every
            // matrix-core op wait for one LDS round trip.
            // ---- phase 1: dZ = A^T dO + ->K dS ; dR = Tb^T dZ ----
            // every product as K = 32 pairs of K = 16 steps; the blocks of A^T and
            // Tb^T left of the diagonal are zero, so the full range is exact
            constexpr int NF1 = 4 + ND;                // A^T and ->K fragments of one row block
            floatx4 X[4], dR[4];
            F16<T> dof[4], fa[NF1], fb[NF1], tb[DELTA ? 16 : 1];
            auto load1 = [&](int li, F16<T>* f) {
#pragma unroll
                for (int mb = 0; mb < 4; ++mb) f[mb] = frag_xk(AqT, LDC, 16 * li, 16 * mb, ln);
#pragma unroll
                for (int db = 0; db < ND; ++db) f[4 + db] = frag_xk(Kr, LDQ, 16 * li, 16 * db, ln);
            };
            auto prod1x2 = [&](const F16<T>* f, const F16<T>* h, floatx4& xf, floatx4& xh) {
                floatx4 a = zero4(), b = zero4();
#pragma unroll
                for (int mb = 0; mb < 4; mb += 2) {
                    a = mma16x2<T>(f[mb], f[mb + 1], dof[mb], dof[mb + 1], a);
                    b = mma16x2<T>(h[mb], h[mb + 1], dof[mb], dof[mb + 1], b);
                }
#pragma unroll
                for (int db = 0; db < ND; db += 2) {
                    const F16<T> s0 = frag16_acc<T>(dS[db]), s1 = frag16_acc<T>(dS[db + 1]);
                    a = mma16x2<T>(f[4 + db], f[5 + db], s0, s1, a);
                    b = mma16x2<T>(h[4 + db], h[5 + db], s0, s1, b);
                }
                xf = a;
                xh = b;
            };
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) dof[mb] = frag_xk(dOT[buf], LDC, n0, 16 * mb, ln);
            load1(0, fa);
            load1(1, fb);
            __builtin_amdgcn_sched_barrier(0);
            // dS_{r+1} of this chunk to LDS while the reads are in flight; the
            // helper waves write it to HBM in phase 2
#pragma unroll
            for (int db = 0; db < ND; ++db) store_tile_rows(dSs + 16 * db * LDC + n0, LDC, dS[db], ln);
            // two row blocks at a time, their products interleaved (two
            // independent accumulation chains for the matrix cores)
            prod1x2(fa, fb, X[0], X[1]);
            load1(2, fa);
            load1(3, fb);
            if constexpr (DELTA) {
#pragma unroll
                for (int li = 0; li < 4; ++li)
#pragma unroll
                    for (int kb = 0; kb < 4; ++kb) tb[4 * li + kb] = frag_xk(TbT, LDC, 16 * li, 16 * kb, ln);
            }
            __builtin_amdgcn_sched_barrier(0);
            prod1x2(fa, fb, X[2], X[3]);
            if constexpr (DELTA) {
                const F16<T> x0 = frag16_acc<T>(X[0]), x1 = frag16_acc<T>(X[1]), x2 = frag16_acc<T>(X[2]),
                             x3 = frag16_acc<T>(X[3]);
#pragma unroll
                for (int li = 0; li < 4; ++li)
                    dR[li] = mma16x2<T>(tb[4 * li + 2], tb[4 * li + 3], x2, x3,
                                        mma16x2<T>(tb[4 * li], tb[4 * li + 1], x0, x1, zero4()));
            }
            lds_barrier();
            // ---- phase 2: dS = exp(G_C) dS + <-Q^T dO - <-K^T dR ----
            F16<T> drf[4];
            if constexpr (DELTA) {
#pragma unroll
                for (int mb = 0; mb < 4; ++mb) drf[mb] = frag16_acc<T>(dR[mb]);
            }
            constexpr int NF2 = DELTA ? 8 : 4;         // <-Q^T and -<-K^T fragments of one row block
            F16<T> fq[2][NF2];
            auto load2 = [&](int db, F16<T>* f) {
#pragma unroll
                for (int mb = 0; mb < 4; ++mb) {
                    f[mb] = frag_xk(QdT, LDC, 16 * db, 16 * mb, ln);
                    if constexpr (DELTA) f[4 + mb] = frag_xk(NKdT, LDC, 16 * db, 16 * mb, ln);
                }
            };
            load2(0, fq[0]);
            load2(1, fq[1]);
            __builtin_amdgcn_sched_barrier(0);
            // two row blocks of dS at a time, their products interleaved; the
            // next pair's fragments are read meanwhile
#pragma unroll
            for (int db = 0; db < ND; db += 2) {
                floatx4 a, b;
                if constexpr (CHAN) {
                    a = dS[db] * *reinterpret_cast<const floatx4*>(&gCs[buf][16 * db + g4]);
                    b = dS[db + 1] * *reinterpret_cast<const floatx4*>(&gCs[buf][16 * db + 16 + g4]);
                } else {
                    a = dS[db] * gCs[buf][0];
                    b = dS[db + 1] * gCs[buf][0];
                }
                const F16<T>* f = fq[0];
                const F16<T>* h = fq[1];
#pragma unroll
                for (int mb = 0; mb < 4; mb += 2) {
                    a = mma16x2<T>(f[mb], f[mb + 1], dof[mb], dof[mb + 1], a);
                    b = mma16x2<T>(h[mb], h[mb + 1], dof[mb], dof[mb + 1], b);
                }
                if constexpr (DELTA) {
#pragma unroll
                    for (int mb = 0; mb < 4; mb += 2) {
                        a = mma16x2<T>(f[4 + mb], f[5 + mb], drf[mb], drf[mb + 1], a);
                        b = mma16x2<T>(h[4 + mb], h[5 + mb], drf[mb], drf[mb + 1], b);
                    }
                }
                dS[db] = a;
                dS[db + 1] = b;
                if (db + 2 < ND) {
                    load2(db + 2, fq[0]);
                    load2(db + 3, fq[1]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            lds_barrier();
        }
        if (ds0) {
#pragma unroll
            for (int db = 0; db < ND; ++db)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) ds0[(bh * DK + 16 * db + g4 + rr) * DV + col] = dS[db][rr];
        }
    } else if (wave < 4) {
        // a 32-column block has two state waves: waves 2 and 3 keep the
        // barrier schedule of the state waves' loop (two per chunk) and idle
        __syncthreads();
        for (int64_t c = nchunks - 1; c >= 0; --c) {
            lds_barrier();
            lds_barrier();
        }
    } else {
        const int ht = tid - 256;
        // The operands of one chunk in registers: group 1 (A^T, Tb^T, ->K, dO
        // and the chunk decay, read in phase 1) and group 2 (<-Q^T, -<-K^T, read
        // in phase 2).  Two sets, the chunk being staged and the next one, so
        // each load is issued about one chunk period before it is staged: the
        // HBM round trip, not the products, would otherwise set the pace.
        struct Regs {
            i4 ra[NA], rt[NA], rk[NK], ro[NO], rq[NK], rn[NK], rgv;
            float rg;
        };
        Regs A, B;
        auto load_g1 = [&](int64_t c, Regs& R) {
            const T* base = ops + (bh * nchunks + c) * ostride;
#pragma unroll
            for (int p = 0; p < NA; ++p) {
                const int e = (p * NH + ht) * E;
                R.ra[p] = *reinterpret_cast<const i4*>(base + C::O_AQT + e);
                if constexpr (DELTA) R.rt[p] = *reinterpret_cast<const i4*>(base + C::O_TBT + e);
            }
#pragma unroll
            for (int p = 0; p < NK; ++p) {
                const int e = (p * NH + ht) * E;
                R.rk[p] = *reinterpret_cast<const i4*>(base + C::O_KR + e);
            }
#pragma unroll
            for (int p = 0; p < NO; ++p) {
                // lane-consecutive rows; rows past the end read the last row and
                // are zeroed, so every chunk issues the same loads
                const int e = p * NH + ht;
                const int row = e % kC, cc = (e / kC) * E;
                const int64_t t = c * kC + row;
                const int64_t tr = t < Tlen ? t : Tlen - 1;
                const i4 x = *reinterpret_cast<const i4*>(dout + (bh * Tlen + tr) * DV + vb * VB + cc);
                R.ro[p] = t < Tlen ? x : i4{0, 0, 0, 0};
            }
            if constexpr (CHAN) {
                if (ht < DK / 4) R.rgv = *reinterpret_cast<const i4*>(gC + (bh * nchunks + c) * DK + 4 * ht);
            } else {
                R.rg = gC[bh * nchunks + c];
            }
        };
        auto load_g2 = [&](int64_t c, Regs& R) {
            const T* base = ops + (bh * nchunks + c) * ostride;
#pragma unroll
            for (int p = 0; p < NK; ++p) {
                const int e = (p * NH + ht) * E;
                R.rq[p] = *reinterpret_cast<const i4*>(base + C::O_QDT + e);
                if constexpr (DELTA) R.rn[p] = *reinterpret_cast<const i4*>(base + C::O_NKDT + e);
            }
        };
        auto load = [&](int64_t c, Regs& R) {
            load_g1(c, R);
            load_g2(c, R);
        };
        auto stage1 = [&](int64_t c, const Regs& R) {
            const int buf = (int)(c & 1);
#pragma unroll
            for (int p = 0; p < NA; ++p) {
                const int e = (p * NH + ht) * E;
                *reinterpret_cast<i4*>(AqT + (e / kC) * LDC + e % kC) = R.ra[p];
                if constexpr (DELTA) *reinterpret_cast<i4*>(TbT + (e / kC) * LDC + e % kC) = R.rt[p];
            }
#pragma unroll
            for (int p = 0; p < NK; ++p) {
                const int e = (p * NH + ht) * E;
                *reinterpret_cast<i4*>(Kr + (e / DK) * LDQ + e % DK) = R.rk[p];
            }
#pragma unroll
            for (int p = 0; p < NO; ++p) {
                const int e = p * NH + ht;
                const int row = e % kC, cc = (e / kC) * E;
                T x[E];
                __builtin_memcpy(x, &R.ro[p], 16);
#pragma unroll
                for (int i = 0; i < E; ++i) dOT[buf][(cc + i) * LDC + row] = x[i];
            }
            if constexpr (CHAN) {
                if (ht < DK / 4) *reinterpret_cast<i4*>(&gCs[buf][4 * ht]) = R.rgv;
            } else {
                if (ht == 0) gCs[buf][0] = R.rg;
            }
        };
        auto stage2 = [&](const Regs& R) {
#pragma unroll
            for (int p = 0; p < NK; ++p) {
                const int e = (p * NH + ht) * E;
                *reinterpret_cast<i4*>(QdT + (e / kC) * LDC + e % kC) = R.rq[p];
                if constexpr (DELTA) *reinterpret_cast<i4*>(NKdT + (e / kC) * LDC + e % kC) = R.rn[p];
            }
        };
        // dS of chunk c from LDS to HBM, in the 16-column blocked layout
        auto copy_ds = [&](int64_t c) {
            constexpr int VR = VB / E, ND2 = DK * VR / NH;
            static_assert(ND2 * NH == DK * VR, "dS copy split");
            T* base = dstates + (bh * nchunks + c) * DK * DV;
#pragma unroll
            for (int p = 0; p < ND2; ++p) {
                const int e = p * NH + ht;
                const int row = e / VR, col = (e % VR) * E;
                *reinterpret_cast<i4*>(base + dstate_offset(row, vb * VB + col, DK)) =
                    *reinterpret_cast<const i4*>(dSs + row * LDC + col);
            }
        };
        // one chunk of the state waves' loop: X holds chunk c (its group 1
        // already staged), Y chunk c - 1; X is refilled with chunk c - 2 (the
        // last chunk again past the start, never staged)
        auto step = [&](int64_t c, Regs& X, Regs& Y) {
            stage2(X);                      // <-Q^T, -<-K^T of chunk c (read in phase 2)
            load(c >= 2 ? c - 2 : 0, X);
            lds_barrier();
            if (c > 0) stage1(c - 1, Y);    // the buffers phase 1 read are free now
            copy_ds(c);                     // written by the state waves in phase 1
            lds_barrier();
        };
        if constexpr (sizeof(T) == 2) {
            if (nchunks > 0) {
                load(nchunks - 1, A);
                stage1(nchunks - 1, A);
                load(nchunks >= 2 ? nchunks - 2 : 0, B);
            }
            __syncthreads();
            int64_t c = nchunks - 1;
            for (; c >= 1; c -= 2) {
                step(c, A, B);
                step(c - 1, B, A);
            }
            if (c == 0) step(0, A, B);
        } else {
            // fp32 operands take twice the registers: one set, each group
            // loaded one phase ahead of its staging
            if (nchunks > 0) {
                load_g1(nchunks - 1, A);
                stage1(nchunks - 1, A);
                load_g2(nchunks - 1, A);
            }
            __syncthreads();
            for (int64_t c = nchunks - 1; c >= 0; --c) {
                const int64_t cn = c > 0 ? c - 1 : 0;
                stage2(A);
                load_g1(cn, A);
                lds_barrier();
                if (c > 0) stage1(cn, A);
                copy_ds(c);
                load_g2(cn, A);
                lds_barrier();
            }
        }
        wait_vmem_all();
    }
}

// ============================================================================
// bwd_grad_kernel: every gradient of one chunk from S_r and dS_{r+1}.
// ============================================================================
template <typename T, int DK, int RULE, int GATE>
__global__ __launch_bounds__(kNT, 1) void bwd_grad_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ g,
    const T* __restrict__ beta, const T* __restrict__ dout, const T* __restrict__ states,
    const T* __restrict__ dstates, T* __restrict__ dq, T* __restrict__ dk, T* __restrict__ dv,
    T* __restrict__ dg, T* __restrict__ dbeta, int64_t Tlen, int64_t nchunks, int DV)
{
    using C = BwdCfg<T, DK>;
    constexpr int LDQ = C::LDQ, LDC = C::LDC, LDJ = C::LDJ, LDF = C::LDF, J = C::J, E = C::E;
    constexpr bool DELTA = RULE == kRuleDelta, GATED = GATE == kGateScalar;
    constexpr int NI = DK / 32;            // key-column tiles per wave (of dq, dk)
    constexpr int NJT = J / 16;            // value-column tiles per step
    // the value-block arrays of the loop, and the scratch of the final phase in
    // the same bytes
    constexpr int SZ = (int)sizeof(T);
    constexpr int LOOP_BYTES = (5 * kC * LDJ + 2 * DK * LDJ) * SZ;
    constexpr int FIN_BYTES = 2 * kC * LDF * 4;
    constexpr int REGION = LOOP_BYTES > FIN_BYTES ? LOOP_BYTES : FIN_BYTES;
    static_assert(kC * LDC * SZ <= kC * LDF * 4, "scratch sizes");

    __shared__ __align__(16) T Qs[kC * LDQ], Ks[kC * LDQ];
    __shared__ __align__(16) T CC[4 * kC * LDC];    // Aq (then P), Lm (then P2), Tm, Tb
    __shared__ __align__(16) unsigned char region[REGION];
    __shared__ __align__(16) float G[kC], gam[kC], bet[kC];
    __shared__ float dGs[kC], dBs[kC], rowp[2][kC], rowp2[2][kC], krp[2][kC], sdp[8];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t bh = blockIdx.x / nchunks, r = blockIdx.x % nchunks;
    const int64_t t0 = r * kC;
    const int tvalid = (int)(Tlen - t0 < kC ? Tlen - t0 : kC);
    T* const Aq = CC;
    T* const Lm = CC + kC * LDC;
    T* const Tm = CC + 2 * kC * LDC;
    T* const Tb = CC + 3 * kC * LDC;
    IntraLds<T, DK> L{Qs, Ks, Aq, Lm, Tm, Tb, G, gam, bet};
    const T* Sr = states + (bh * nchunks + r) * (int64_t)DK * DV;
    const T* dSr = dstates + (bh * nchunks + r) * (int64_t)DK * DV;

    // the value block's dO and V rows and its S_r and dS_{r+1} columns go
    // through registers: the next block's loads are issued before this block's
    // products (the first block's before the intra-chunk work)
    constexpr int VR = J / E, NVJ = (kC * VR + kNT - 1) / kNT;
    constexpr int SR = J / E, NSJ = (DK * SR + kNT - 1) / kNT;
    i4 pdo[NVJ], pv[NVJ], ps[NSJ], pds[NSJ];
    auto fetch = [&](int j0) {
#pragma unroll
        for (int u = 0; u < NVJ; ++u) {
            const int i = tid + u * kNT, row = i / VR, c = (i % VR) * E;
            pdo[u] = pv[u] = i4{0, 0, 0, 0};
            if (i < kC * VR && row < tvalid) {
                pdo[u] = *reinterpret_cast<const i4*>(dout + (bh * Tlen + t0 + row) * DV + j0 + c);
                pv[u] = *reinterpret_cast<const i4*>(v + (bh * Tlen + t0 + row) * DV + j0 + c);
            }
        }
#pragma unroll
        for (int u = 0; u < NSJ; ++u) {
            const int i = tid + u * kNT, row = i / SR, c = (i % SR) * E;
            ps[u] = pds[u] = i4{0, 0, 0, 0};
            if (i < DK * SR) {
                ps[u] = *reinterpret_cast<const i4*>(Sr + row * DV + j0 + c);
                pds[u] = *reinterpret_cast<const i4*>(dSr + dstate_offset(row, j0 + c, DK));
            }
        }
    };
    fetch(0);
    intra_chunk<T, DK, RULE, GATE>(L, q, k, g, beta, bh, Tlen, t0, tvalid, tid);

    T* const dOs = reinterpret_cast<T*>(region);
    T* const Rs = dOs + kC * LDJ;
    T* const Zs = Rs + kC * LDJ;
    T* const dZs = Zs + kC * LDJ;
    T* const dRs = dZs + kC * LDJ;
    T* const Ss = dRs + kC * LDJ;
    T* const dSs = Ss + DK * LDJ;

    const int cl = lane & 15, g4 = 4 * (lane >> 4);
    const int lbq = wave >> 1;                       // row block of this wave's dq/dk tiles
    const int lbt = wave >> 1;                       // row block of its dA/dTb tiles
    floatx4 dQd[NI], dKd[NI], dKr[NI], dAq[2], dTb[2];
#pragma unroll
    for (int u = 0; u < NI; ++u) dQd[u] = dKd[u] = dKr[u] = zero4();
    dAq[0] = dAq[1] = dTb[0] = dTb[1] = zero4();
    float sdot = 0.f;

    for (int j0 = 0; j0 < DV; j0 += J) {
        // ---- stage dO and V (token rows), S_r and dS_{r+1} (value columns j0..j0+J) ----
#pragma unroll
        for (int u = 0; u < NVJ; ++u) {
            const int i = tid + u * kNT, row = i / VR, c = (i % VR) * E;
            if (i < kC * VR) {
                *reinterpret_cast<i4*>(dOs + row * LDJ + c) = pdo[u];
                *reinterpret_cast<i4*>(Zs + row * LDJ + c) = pv[u];
            }
        }
#pragma unroll
        for (int u = 0; u < NSJ; ++u) {
            const int i = tid + u * kNT, row = i / SR, c = (i % SR) * E;
            if (i < DK * SR) {
                T a[E], b[E];
                __builtin_memcpy(a, &ps[u], 16);
                __builtin_memcpy(b, &pds[u], 16);
#pragma unroll
                for (int x = 0; x < E; ++x) sdot += to_f32(a[x]) * to_f32(b[x]);
                *reinterpret_cast<i4*>(Ss + row * LDJ + c) = ps[u];
                *reinterpret_cast<i4*>(dSs + row * LDJ + c) = pds[u];
            }
        }
        __syncthreads();
        if (j0 + J < DV) fetch(j0 + J);
        // ---- step A: R = V - <-K S_r ; dZ = A^T dO + ->K dS ; d<-Q += dO S_r^T ----
        if (wave < 4 * NJT) {
            const int lb = wave / NJT, jc = wave % NJT;
            floatx4 a1 = tilek<T, false, false, kC>(zero4(), Aq, LDC, 16 * lb, dOs, LDJ, 16 * jc, 0, lane);
            floatx4 a2 = tilek<T, true, false, DK>(zero4(), Ks, LDQ, 16 * lb, dSs, LDJ, 16 * jc, 0, lane);
            floatx4 dz;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int l = 16 * lb + g4 + rr;
                dz[rr] = a1[rr] + (GATED ? expf(G[kC - 1] - G[l]) : 1.f) * a2[rr];
            }
            put(dZs, LDJ, 16 * lb, 16 * jc, dz, lane);
            if constexpr (DELTA) {
                const floatx4 ks = tilek<T, true, false, DK>(zero4(), Ks, LDQ, 16 * lb, Ss, LDJ, 16 * jc, 0, lane);
                floatx4 rv;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int l = 16 * lb + g4 + rr;
                    rv[rr] = to_f32(Zs[l * LDJ + 16 * jc + cl]) - gam[l] * ks[rr];
                }
                put(Rs, LDJ, 16 * lb, 16 * jc, rv, lane);
            } else {
                // add rule: dv = dZ
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int l = 16 * lb + g4 + rr;
                    if (l < tvalid) dv[(bh * Tlen + t0 + l) * DV + j0 + 16 * jc + cl] = from_f32<T>(dz[rr]);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < NI; ++u)
            dQd[u] = tilek<T, true, true, J>(dQd[u], dOs, LDJ, 16 * lbq, Ss, LDJ, 16 * (NI * (wave & 1) + u), 0, lane);
        __syncthreads();
        // ---- step B (delta): Z = Tb R ; dR = Tb^T dZ (= dv) ; dTb += dZ R^T ----
        if constexpr (DELTA) {
            if (wave < 4 * NJT) {
                const int lb = wave / NJT, jc = wave % NJT;
                const floatx4 z = tilek<T, true, false, kC>(zero4(), Tb, LDC, 16 * lb, Rs, LDJ, 16 * jc, 0, lane);
                const floatx4 dr = tilek<T, false, false, kC>(zero4(), Tb, LDC, 16 * lb, dZs, LDJ, 16 * jc, 0, lane);
                put(Zs, LDJ, 16 * lb, 16 * jc, z, lane);
                put(dRs, LDJ, 16 * lb, 16 * jc, dr, lane);
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int l = 16 * lb + g4 + rr;
                    if (l < tvalid) dv[(bh * Tlen + t0 + l) * DV + j0 + 16 * jc + cl] = from_f32<T>(dr[rr]);
                }
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int mb = 2 * (wave & 1) + u;
                if (mb <= lbt) dTb[u] = tilek<T, true, true, J>(dTb[u], dZs, LDJ, 16 * lbt, Rs, LDJ, 16 * mb, 0, lane);
            }
            __syncthreads();
        }
        // ---- step C: d<-K += dR S_r^T (negated later) ; d->K += Z dS^T ; dA += dO Z^T ----
#pragma unroll
        for (int u = 0; u < NI; ++u) {
            const int ib = NI * (wave & 1) + u;
            if constexpr (DELTA) dKd[u] = tilek<T, true, true, J>(dKd[u], dRs, LDJ, 16 * lbq, Ss, LDJ, 16 * ib, 0, lane);
            dKr[u] = tilek<T, true, true, J>(dKr[u], Zs, LDJ, 16 * lbq, dSs, LDJ, 16 * ib, 0, lane);
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int mb = 2 * (wave & 1) + u;
            if (mb <= lbt) dAq[u] = tilek<T, true, true, J>(dAq[u], dOs, LDJ, 16 * lbt, Zs, LDJ, 16 * mb, 0, lane);
        }
        __syncthreads();
    }

    // ============ final phase ============
    float* const sc = reinterpret_cast<float*>(region);               // fp32 [C][LDF]
    unsigned char* const second = region + kC * LDF * 4;
    T* const dTbs = reinterpret_cast<T*>(second);                     // [C][LDC]
    T* const X1s = reinterpret_cast<T*>(region);                      // [C][LDC], after sc is read
    float* const E2 = reinterpret_cast<float*>(second);               // [C][LDF], after dTbs is read
    {
        const float tot = wave_last(wave_prefix_sum(sdot));
        if (lane == 0) sdp[wave] = tot;
    }
    // F0: dA . A to the scratch, P = dA . D over A in place; dTb to LDS
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int mb = 2 * (wave & 1) + u;
        const int m = 16 * mb + cl;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int l = 16 * lbt + g4 + rr;
            const bool on = mb <= lbt && m <= l;
            const float da = on ? dAq[u][rr] : 0.f;
            const float a = to_f32(Aq[l * LDC + m]);
            sc[l * LDF + m] = da * a;
            const float d = GATED ? expf(fminf(G[l] - G[m], 0.f)) : 1.f;
            Aq[l * LDC + m] = from_f32<T>(da * d);
            if constexpr (DELTA) dTbs[l * LDC + m] = from_f32<T>(on ? dTb[u][rr] : 0.f);
        }
    }
    __syncthreads();
    // F1: dG from dA . A; dbeta from T . dTb; X1 = T^T dTb; the row dots of the
    // dq/dk accumulators
    // row and column sums of the 64x64 matrices: thread t takes index t/8 and
    // eight of its elements, then the 8 lanes of the index add up in DPP
    const int sx = tid >> 3, sp = tid & 7;
    {
        float s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int m = 8 * sp + u;
            s1 += sc[sx * LDF + m];
            s2 += sc[m * LDF + sx];
            if constexpr (DELTA) s3 += to_f32(Tm[m * LDC + sx]) * to_f32(dTbs[m * LDC + sx]);
        }
        s1 = group_sum<8>(s1);
        s2 = group_sum<8>(s2);
        s3 = group_sum<8>(s3);
        if (sp == 0) {
            dGs[sx] = s1 - s2;
            dBs[sx] = s3;
        }
    }
    floatx4 X1[2];
    if constexpr (DELTA) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int sb = 2 * (wave & 1) + u;
            X1[u] = tilek<T, false, false, kC>(zero4(), Tm, LDC, 16 * lbt, dTbs, LDC, 16 * sb, 0, lane);
        }
    }
    {
        float rd[4] = {0.f, 0.f, 0.f, 0.f}, kr[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < NI; ++u) {
            const int i = 16 * (NI * (wave & 1) + u) + cl;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int l = 16 * lbq + g4 + rr;
                const float qv = to_f32(Qs[l * LDQ + i]), kv = to_f32(Ks[l * LDQ + i]);
                const float er = GATED ? expf(G[kC - 1] - G[l]) : 1.f;
                const float t3 = kv * er * dKr[u][rr];
                rd[rr] += qv * gam[l] * dQd[u][rr] - kv * gam[l] * dKd[u][rr] - t3;
                kr[rr] += t3;
            }
        }
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const float a = group_sum<16>(rd[rr]), b = group_sum<16>(kr[rr]);
            if (cl == 0) {
                rowp[wave & 1][16 * lbq + g4 + rr] = a;
                krp[wave & 1][16 * lbq + g4 + rr] = b;
            }
        }
    }
    __syncthreads();
    if constexpr (DELTA) {
        // F2: X1 to LDS (over the first scratch)
#pragma unroll
        for (int u = 0; u < 2; ++u) put(X1s, LDC, 16 * lbt, 16 * (2 * (wave & 1) + u), X1[u], lane);
        __syncthreads();
        // F3: dM = -X1 Tb^T (causal tiles); dL = diag(beta) dM (strict);
        // dbeta += rowsum(dM . L); dL . L to the scratch; P2 = dL . D over L
        float rb[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int mb = 2 * (wave & 1) + u;
            const int m = 16 * mb + cl;
            floatx4 dm = zero4();
            if (mb <= lbt) dm = tilek<T, true, true, kC>(zero4(), X1s, LDC, 16 * lbt, Tb, LDC, 16 * mb, 0, lane);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int l = 16 * lbt + g4 + rr;
                const bool strict = mb <= lbt && m < l;
                const float dM = -dm[rr];
                const float lv = to_f32(Lm[l * LDC + m]);
                rb[rr] += strict ? dM * lv : 0.f;
                const float dl = strict ? bet[l] * dM : 0.f;
                E2[l * LDF + m] = dl * lv;
                if (strict) Lm[l * LDC + m] = from_f32<T>(dl * (GATED ? expf(G[l] - G[m]) : 1.f));
            }
        }
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const float a = group_sum<16>(rb[rr]);
            if (cl == 0) rowp2[wave & 1][16 * lbt + g4 + rr] = a;
        }
        __syncthreads();
    }
    // F4: dG and dbeta totals per row; dq = exp(G) d<-Q + P K;
    // dk = -exp(G) (dR S^T) + exp(G_C - G) d->K + P^T Q + (P2 + P2^T) K
    {
        float s1 = 0.f, s2 = 0.f;
        if constexpr (DELTA) {
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int m = 8 * sp + u;
                s1 += E2[sx * LDF + m];
                s2 += E2[m * LDF + sx];
            }
            s1 = group_sum<8>(s1);
            s2 = group_sum<8>(s2);
        }
        if (sp == 0) {
            dGs[sx] += rowp[0][sx] + rowp[1][sx] + (s1 - s2);
            if constexpr (DELTA) dBs[sx] += rowp2[0][sx] + rowp2[1][sx];
        }
    }
#pragma unroll
    for (int u = 0; u < NI; ++u) {
        const int ib = NI * (wave & 1) + u;
        floatx4 aq, ak;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int l = 16 * lbq + g4 + rr;
            aq[rr] = gam[l] * dQd[u][rr];
            ak[rr] = -gam[l] * dKd[u][rr] + (GATED ? expf(G[kC - 1] - G[l]) : 1.f) * dKr[u][rr];
        }
        aq = tilek<T, true, false, kC>(aq, Aq, LDC, 16 * lbq, Ks, LDQ, 16 * ib, 0, lane);
        ak = tilek<T, false, false, kC>(ak, Aq, LDC, 16 * lbq, Qs, LDQ, 16 * ib, 0, lane);
        if constexpr (DELTA) {
            ak = tilek<T, true, false, kC>(ak, Lm, LDC, 16 * lbq, Ks, LDQ, 16 * ib, 0, lane);
            ak = tilek<T, false, false, kC>(ak, Lm, LDC, 16 * lbq, Ks, LDQ, 16 * ib, 0, lane);
        }
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int l = 16 * lbq + g4 + rr;
            if (l < tvalid) {
                dq[(bh * Tlen + t0 + l) * DK + 16 * ib + cl] = from_f32<T>(aq[rr]);
                dk[(bh * Tlen + t0 + l) * DK + 16 * ib + cl] = from_f32<T>(ak[rr]);
            }
        }
    }
    __syncthreads();
    // F5: dG_C extras, then dg = reverse prefix sum of dG
    if (wave == 0) {
        if constexpr (GATED) {
            const float krs = wave_last(wave_prefix_sum(krp[0][lane] + krp[1][lane]));
            float sd = 0.f;
#pragma unroll
            for (int w = 0; w < 8; ++w) sd += sdp[w];
            float x = dGs[kC - 1 - lane];
            if (lane == 0) x += krs + gam[kC - 1] * sd;
            const float dgs = wave_prefix_sum(x);      // lane L: dg at position 63 - L
            const int s = kC - 1 - lane;
            if (s < tvalid) dg[bh * Tlen + t0 + s] = from_f32<T>(dgs);
        }
    }
    if constexpr (DELTA) {
        if (wave == 1 && lane < tvalid) dbeta[bh * Tlen + t0 + lane] = from_f32<T>(dBs[lane]);
    }
}

// ============================================================================
// bwd_grad_bf16_kernel: the gradient pass for bf16 tokens.  Same equations as
// bwd_grad_kernel; every matrix-core operand is one contiguous vector read:
// each matrix is kept in LDS in the orientation its products contract over
// (transposed copies are written while staging or from result tiles), A^T, Tb
// and Tb^T come from the operand pass, and the row and column sums of the
// final phase are reduced in registers (DPP rows, lane shuffles).
// ============================================================================
// result tile transposed into P[n*ld + m] (four contiguous values per lane)
__device__ __forceinline__ void put_t(bf16* P, int ld, int m0, int n0, floatx4 v, int lane)
{
    store_tile_t(P + n0 * ld + m0, ld, v, lane);
}

// column sums of a result tile: every lane gets the sum over the 16 rows of its
// column l%16
__device__ __forceinline__ float tile_colsum(floatx4 x)
{
    float s = x[0] + x[1] + x[2] + x[3];
    s += __shfl_xor(s, 16, kWave);
    s += __shfl_xor(s, 32, kWave);
    return s;
}

template <int DK, int RULE, int GATE>
__global__ __launch_bounds__(kNT, 1) void bwd_grad_bf16_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ g, const bf16* __restrict__ beta, const bf16* __restrict__ dout,
    const bf16* __restrict__ ops, const bf16* __restrict__ states, const bf16* __restrict__ dstates,
    bf16* __restrict__ dq, bf16* __restrict__ dk, bf16* __restrict__ dv, bf16* __restrict__ dg,
    bf16* __restrict__ dbeta, int64_t Tlen, int64_t nchunks, int DV)
{
    using T = bf16;
    using C = BwdCfg<T, DK>;
    constexpr int LDQ = C::LDQ, LDC = C::LDC, E = 8, J = 32, LDJ = J + 8;
    constexpr bool DELTA = RULE == kRuleDelta, GATED = GATE == kGateScalar;
    constexpr int NI = DK / 32;            // key-column tiles per wave (of dq, dk)
    // value-block arrays of the loop (row-major: products that need them
    // transposed read them with the LDS transpose read), and the matrices of
    // the final phase, in the same bytes
    constexpr int LOOP_ELEMS = 5 * kC * LDJ + 2 * DK * LDJ;
    constexpr int FIN_ELEMS = 5 * kC * LDC + 2 * DK * LDC;
    constexpr int REGION = 2 * (LOOP_ELEMS > FIN_ELEMS ? LOOP_ELEMS : FIN_ELEMS);

    __shared__ __align__(16) T Ks[kC * LDQ];
    __shared__ __align__(16) T AqT[kC * LDC];
    __shared__ __align__(16) T Tb[DELTA ? kC * LDC : 8];
    __shared__ __align__(16) T TbT[DELTA ? kC * LDC : 8];
    __shared__ __align__(16) unsigned char region[REGION];
    __shared__ float G[kC], gam[kC], bet[kC];
    __shared__ float rowE[2][kC], colE[4][kC], rowB[2][kC], colB[4][kC], rdp[2][kC], krp[2][kC], sdp[8];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t bh = blockIdx.x / nchunks, r = blockIdx.x % nchunks;
    const int64_t t0 = r * kC;
    const int tvalid = (int)(Tlen - t0 < kC ? Tlen - t0 : kC);
    const int cl = lane & 15, g4 = 4 * (lane >> 4);
    const int lbq = wave >> 1, lbt = wave >> 1;    // row block of this wave's tiles

    // loop arrays
    T* const dOs = reinterpret_cast<T*>(region);   // [C][LDJ]
    T* const Rs = dOs + kC * LDJ;
    T* const Zs = Rs + kC * LDJ;
    T* const dZs = Zs + kC * LDJ;
    T* const dRs = dZs + kC * LDJ;
    T* const Ss = dRs + kC * LDJ;                   // [DK][LDJ]
    T* const dSs = Ss + DK * LDJ;
    // final-phase arrays
    T* const Pm = reinterpret_cast<T*>(region);    // [C][LDC]
    T* const PT = Pm + kC * LDC;
    T* const dTbT = PT + kC * LDC;                  // then P2
    T* const LT = dTbT + kC * LDC;                  // then P2^T
    T* const TT = LT + kC * LDC;                    // then X1
    T* const KT = TT + kC * LDC;                    // [DK][LDC]
    T* const QT = KT + DK * LDC;

    // ---- prologue: k, A^T, Tb, Tb^T to LDS; q to registers; gate prefix ----
    constexpr int NKV = kC * DK / E / kNT;          // k / q vectors per thread
    i4 rq[NKV];
    {
        const T* base = ops + (bh * nchunks + r) * (int64_t)C::OPS;
        i4 rk[NKV], ra, rt = {0, 0, 0, 0}, rb = {0, 0, 0, 0};
#pragma unroll
        for (int u = 0; u < NKV; ++u) {
            const int i = tid + u * kNT, row = i / (DK / E), c = (i % (DK / E)) * E;
            // q: lane-consecutive rows (its transposed copy is written from these)
            const int qrow = i % kC, qc = (i / kC) * E;
            rk[u] = rq[u] = i4{0, 0, 0, 0};
            if (row < tvalid) rk[u] = *reinterpret_cast<const i4*>(k + (bh * Tlen + t0 + row) * DK + c);
            if (qrow < tvalid) rq[u] = *reinterpret_cast<const i4*>(q + (bh * Tlen + t0 + qrow) * DK + qc);
        }
        ra = *reinterpret_cast<const i4*>(base + C::O_AQT + tid * E);
        if constexpr (DELTA) {
            rt = *reinterpret_cast<const i4*>(base + C::O_TBT + tid * E);
            rb = *reinterpret_cast<const i4*>(base + C::O_TB + tid * E);
        }
#pragma unroll
        for (int u = 0; u < NKV; ++u) {
            const int i = tid + u * kNT, row = i / (DK / E), c = (i % (DK / E)) * E;
            *reinterpret_cast<i4*>(Ks + row * LDQ + c) = rk[u];
        }
        const int row = tid / (kC / E), c = (tid % (kC / E)) * E;
        *reinterpret_cast<i4*>(AqT + row * LDC + c) = ra;
        if constexpr (DELTA) {
            *reinterpret_cast<i4*>(TbT + row * LDC + c) = rt;
            *reinterpret_cast<i4*>(Tb + row * LDC + c) = rb;
        }
    }
    if (wave == 0) {
        float gl = 0.f, bl = 0.f;
        if (lane < tvalid) {
            if constexpr (GATED) gl = to_f32(g[bh * Tlen + t0 + lane]);
            if constexpr (DELTA) bl = to_f32(beta[bh * Tlen + t0 + lane]);
        }
        const float Gl = wave_prefix_sum(gl);
        G[lane] = Gl;
        gam[lane] = GATED ? expf(Gl) : 1.f;
        bet[lane] = bl;
    }

    // ---- value blocks: dO, V, S_r, dS_{r+1} through registers, next block prefetched ----
    const T* Sr = states + (bh * nchunks + r) * (int64_t)DK * DV;
    const T* dSr = dstates + (bh * nchunks + r) * (int64_t)DK * DV;
    constexpr int VR = J / E, NVJ = (kC * VR + kNT - 1) / kNT;
    constexpr int SR = J / E, NSJ = (DK * SR + kNT - 1) / kNT;
    i4 pdo[NVJ], pv[NVJ], ps[NSJ], pds[NSJ];
    // lane i holds row i % rows of its vector: the transposed copies written from
    // these registers then go to consecutive LDS addresses
    auto fetch = [&](int j0) {
#pragma unroll
        for (int u = 0; u < NVJ; ++u) {
            const int i = tid + u * kNT, row = i % kC, c = (i / kC) * E;
            pdo[u] = pv[u] = i4{0, 0, 0, 0};
            if (i < kC * VR && row < tvalid) {
                pdo[u] = *reinterpret_cast<const i4*>(dout + (bh * Tlen + t0 + row) * DV + j0 + c);
                pv[u] = *reinterpret_cast<const i4*>(v + (bh * Tlen + t0 + row) * DV + j0 + c);
            }
        }
#pragma unroll
        for (int u = 0; u < NSJ; ++u) {
            const int i = tid + u * kNT, row = i % DK, c = (i / DK) * E;
            ps[u] = pds[u] = i4{0, 0, 0, 0};
            if (i < DK * SR) {
                ps[u] = *reinterpret_cast<const i4*>(Sr + row * DV + j0 + c);
                pds[u] = *reinterpret_cast<const i4*>(dSr + dstate_offset(row, j0 + c, DK));
            }
        }
    };
    fetch(0);

    floatx4 dQd[NI], dKd[NI], dKr[NI], dAq[2], dTb[2];
#pragma unroll
    for (int u = 0; u < NI; ++u) dQd[u] = dKd[u] = dKr[u] = zero4();
    dAq[0] = dAq[1] = dTb[0] = dTb[1] = zero4();
    float sdot = 0.f;

    for (int j0 = 0; j0 < DV; j0 += J) {
        __syncthreads();       // the previous block's arrays are free (and the prologue's LDS is written)
#pragma unroll
        for (int u = 0; u < NVJ; ++u) {
            const int i = tid + u * kNT, row = i % kC, c = (i / kC) * E;
            if (i < kC * VR) {
                *reinterpret_cast<i4*>(dOs + row * LDJ + c) = pdo[u];
                *reinterpret_cast<i4*>(Zs + row * LDJ + c) = pv[u];
            }
        }
#pragma unroll
        for (int u = 0; u < NSJ; ++u) {
            const int i = tid + u * kNT, row = i % DK, c = (i / DK) * E;
            if (i < DK * SR) {
                T a[E], b[E];
                __builtin_memcpy(a, &ps[u], 16);
                __builtin_memcpy(b, &pds[u], 16);
#pragma unroll
                for (int x = 0; x < E; ++x) sdot += to_f32(a[x]) * to_f32(b[x]);
                *reinterpret_cast<i4*>(Ss + row * LDJ + c) = ps[u];
                *reinterpret_cast<i4*>(dSs + row * LDJ + c) = pds[u];
            }
        }
        __syncthreads();
        if (j0 + J < DV) fetch(j0 + J);
        // ---- step A: dZ = A^T dO + ->K dS ; R = V - <-K S_r ; d<-Q += dO S_r^T ----
        {
            const int lb = wave >> 1, jc = wave & 1;
            const floatx4 a1 = tilek<T, true, false, kC>(zero4(), AqT, LDC, 16 * lb, dOs, LDJ, 16 * jc, 0, lane);
            // K dS and K S_r share their K fragments
            floatx4 a2 = zero4(), ks = zero4();
#pragma unroll
            for (int k0 = 0; k0 < DK; k0 += 32) {
                const F16<T> a0 = frag_xk(Ks, LDQ, 16 * lb, k0, lane), a1f = frag_xk(Ks, LDQ, 16 * lb, k0 + 16, lane);
                a2 = mma16x2<T>(a0, a1f, frag_kx(dSs, LDJ, 16 * jc, k0, lane),
                                frag_kx(dSs, LDJ, 16 * jc, k0 + 16, lane), a2);
                if constexpr (DELTA)
                    ks = mma16x2<T>(a0, a1f, frag_kx(Ss, LDJ, 16 * jc, k0, lane),
                                    frag_kx(Ss, LDJ, 16 * jc, k0 + 16, lane), ks);
            }
            floatx4 dz;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int l = 16 * lb + g4 + rr;
                dz[rr] = a1[rr] + (GATED ? expf(G[kC - 1] - G[l]) : 1.f) * a2[rr];
            }
            put(dZs, LDJ, 16 * lb, 16 * jc, dz, lane);
            if constexpr (DELTA) {
                floatx4 rv;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int l = 16 * lb + g4 + rr;
                    rv[rr] = to_f32(Zs[l * LDJ + 16 * jc + cl]) - gam[l] * ks[rr];
                }
                put(Rs, LDJ, 16 * lb, 16 * jc, rv, lane);
            } else {
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int l = 16 * lb + g4 + rr;
                    if (l < tvalid) dv[(bh * Tlen + t0 + l) * DV + j0 + 16 * jc + cl] = from_f32<T>(dz[rr]);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < NI; ++u)
            dQd[u] = tilek<T, true, true, J>(dQd[u], dOs, LDJ, 16 * lbq, Ss, LDJ, 16 * (NI * (wave & 1) + u), 0, lane);
        __syncthreads();
        // ---- step B (delta): Z = Tb R ; dR = Tb^T dZ (= dv) ; dTb += dZ R^T ----
        if constexpr (DELTA) {
            const int lb = wave >> 1, jc = wave & 1;
            const floatx4 z = tilek<T, true, false, kC>(zero4(), Tb, LDC, 16 * lb, Rs, LDJ, 16 * jc, 0, lane);
            const floatx4 dr = tilek<T, true, false, kC>(zero4(), TbT, LDC, 16 * lb, dZs, LDJ, 16 * jc, 0, lane);
            put(Zs, LDJ, 16 * lb, 16 * jc, z, lane);
            put(dRs, LDJ, 16 * lb, 16 * jc, dr, lane);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int l = 16 * lb + g4 + rr;
                if (l < tvalid) dv[(bh * Tlen + t0 + l) * DV + j0 + 16 * jc + cl] = from_f32<T>(dr[rr]);
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int mb = 2 * (wave & 1) + u;
                if (mb <= lbt) dTb[u] = tilek<T, true, true, J>(dTb[u], dZs, LDJ, 16 * lbt, Rs, LDJ, 16 * mb, 0, lane);
            }
            __syncthreads();
        }
        // ---- step C: d<-K += dR S_r^T (negated later) ; d->K += Z dS^T ; dA += dO Z^T ----
        // every fragment of the step is read before its first product (the
        // scheduling barrier keeps the reads together), so the products do not
        // wait for LDS one tile at a time; the row-side fragments are shared
        {
            F16<T> aR[2], aZ[2], aO[2], bS[NI][2], bD[NI][2], bZ[2][2];
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                if constexpr (DELTA) aR[s2] = frag_xk(dRs, LDJ, 16 * lbq, 16 * s2, lane);
                aZ[s2] = frag_xk(Zs, LDJ, 16 * lbq, 16 * s2, lane);
                aO[s2] = frag_xk(dOs, LDJ, 16 * lbt, 16 * s2, lane);
#pragma unroll
                for (int u = 0; u < NI; ++u) {
                    const int ib = NI * (wave & 1) + u;
                    if constexpr (DELTA) bS[u][s2] = frag_xk(Ss, LDJ, 16 * ib, 16 * s2, lane);
                    bD[u][s2] = frag_xk(dSs, LDJ, 16 * ib, 16 * s2, lane);
                }
#pragma unroll
                for (int u = 0; u < 2; ++u) bZ[u][s2] = frag_xk(Zs, LDJ, 16 * (2 * (wave & 1) + u), 16 * s2, lane);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < NI; ++u) {
                if constexpr (DELTA) dKd[u] = mma16x2<T>(aR[0], aR[1], bS[u][0], bS[u][1], dKd[u]);
                dKr[u] = mma16x2<T>(aZ[0], aZ[1], bD[u][0], bD[u][1], dKr[u]);
            }
#pragma unroll
            for (int u = 0; u < 2; ++u)
                if (2 * (wave & 1) + u <= lbt) dAq[u] = mma16x2<T>(aO[0], aO[1], bZ[u][0], bZ[u][1], dAq[u]);
        }
    }
    __syncthreads();

    // ============ final phase ============
    {
        const float tot = wave_last(wave_prefix_sum(sdot));
        if (lane == 0) sdp[wave] = tot;
    }
    // F0: P = dA . D (and P^T), dA . A kept in registers; dTb^T; L in registers
    // and L^T; K^T and Q^T
    floatx4 Ev[2], Lr[2], Bt[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int mb = 2 * (wave & 1) + u;
        const int m = 16 * mb + cl;
        floatx4 pv2, dt, lv = zero4();
        if constexpr (DELTA) {
            if (mb <= lbt) {
                lv = tilek<T, true, true, 64>(zero4(), Ks, LDQ, 16 * lbt, Ks, LDQ, 16 * mb, 0, lane);
                if constexpr (DK > 64) lv = tilek<T, true, true, 64>(lv, Ks, LDQ, 16 * lbt, Ks, LDQ, 16 * mb, 64, lane);
            }
        }
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int l = 16 * lbt + g4 + rr;
            const bool on = mb <= lbt && m <= l;
            const float d = GATED ? expf(fminf(G[l] - G[m], 0.f)) : 1.f;
            const float da = on ? dAq[u][rr] : 0.f;
            Ev[u][rr] = da * to_f32(AqT[m * LDC + l]);
            pv2[rr] = da * d;
            dt[rr] = on ? dTb[u][rr] : 0.f;
            Lr[u][rr] = (mb <= lbt && m < l) ? lv[rr] * d : 0.f;
        }
        put(Pm, LDC, 16 * lbt, 16 * mb, pv2, lane);
        put_t(PT, LDC, 16 * lbt, 16 * mb, pv2, lane);
        if constexpr (DELTA) {
            Bt[u] = dt;
            put_t(dTbT, LDC, 16 * lbt, 16 * mb, dt, lane);
            put_t(LT, LDC, 16 * lbt, 16 * mb, Lr[u], lane);
        }
    }
    {
        // K^T from LDS, Q^T from the registers loaded in the prologue
        for (int i = tid; i < kC * DK / 4; i += kNT) {
            const int m = i % kC, c = (i / kC) * 4;
            const bf16x4 x = *reinterpret_cast<const bf16x4*>(Ks + m * LDQ + c);
#pragma unroll
            for (int e = 0; e < 4; ++e) KT[(c + e) * LDC + m] = x[e];
        }
#pragma unroll
        for (int u = 0; u < NKV; ++u) {
            const int i = tid + u * kNT, row = i % kC, c = (i / kC) * E;
            T x[E];
            __builtin_memcpy(x, &rq[u], 16);
#pragma unroll
            for (int e = 0; e < E; ++e) QT[(c + e) * LDC + row] = x[e];
        }
    }
    __syncthreads();
    // F1: T^T = I - L^T Tb^T (upper tiles); the row dots of the dq/dk accumulators
    floatx4 X1[2];
    if constexpr (DELTA) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int kb = 2 * (wave & 1) + u;
            floatx4 tt = zero4();
            if (kb >= lbt) tt = tilek<T, true, true, kC>(zero4(), LT, LDC, 16 * lbt, Tb, LDC, 16 * kb, 0, lane);
            X1[u] = tt;                             // held until T^T is stored
        }
    }
    {
        float rd[4] = {0.f, 0.f, 0.f, 0.f}, kr[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < NI; ++u) {
            const int i = 16 * (NI * (wave & 1) + u) + cl;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int l = 16 * lbq + g4 + rr;
                const float qv = to_f32(QT[i * LDC + l]), kv = to_f32(Ks[l * LDQ + i]);
                const float er = GATED ? expf(G[kC - 1] - G[l]) : 1.f;
                const float t3 = kv * er * dKr[u][rr];
                rd[rr] += qv * gam[l] * dQd[u][rr] - kv * gam[l] * dKd[u][rr] - t3;
                kr[rr] += t3;
            }
        }
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const float a = group_sum<16>(rd[rr]), b = group_sum<16>(kr[rr]);
            if (cl == 0) {
                rdp[wave & 1][16 * lbq + g4 + rr] = a;
                krp[wave & 1][16 * lbq + g4 + rr] = b;
            }
        }
    }
    if constexpr (DELTA) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int kb = 2 * (wave & 1) + u;
            floatx4 t;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int l = 16 * lbt + g4 + rr, kk = 16 * kb + cl;
                t[rr] = kb < lbt ? 0.f : (kk == l ? 1.f : 0.f) - (kk > l ? X1[u][rr] : 0.f);
            }
            put(TT, LDC, 16 * lbt, 16 * kb, t, lane);
        }
        __syncthreads();
        // F2: dbeta (part 1) = column sums of T . dTb; X1 = T^T dTb
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int mb = 2 * (wave & 1) + u;
            const int m = 16 * mb + cl;
            floatx4 f;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int l = 16 * lbt + g4 + rr;
                f[rr] = Bt[u][rr] * to_f32(TT[m * LDC + l]);
            }
            const float cs = tile_colsum(f);
            if (g4 == 0) colB[lbt][m] = cs;
            X1[u] = tilek<T, true, true, kC>(zero4(), TT, LDC, 16 * lbt, dTbT, LDC, 16 * mb, 0, lane);
        }
        __syncthreads();
        // F3: X1 over T^T; then dM = -X1 Tb^T, dL = diag(beta) dM (strict),
        // P2 = dL . D and its transpose, dbeta part 2, dL . L into the sums
#pragma unroll
        for (int u = 0; u < 2; ++u) put(TT, LDC, 16 * lbt, 16 * (2 * (wave & 1) + u), X1[u], lane);
        __syncthreads();
        float rb[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int mb = 2 * (wave & 1) + u;
            const int m = 16 * mb + cl;
            floatx4 dm = zero4(), p2;
            if (mb <= lbt) dm = tilek<T, true, true, kC>(zero4(), TT, LDC, 16 * lbt, Tb, LDC, 16 * mb, 0, lane);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int l = 16 * lbt + g4 + rr;
                const bool strict = mb <= lbt && m < l;
                const float dM = -dm[rr];
                rb[rr] += strict ? dM * Lr[u][rr] : 0.f;
                const float dl = strict ? bet[l] * dM : 0.f;
                Ev[u][rr] += dl * Lr[u][rr];
                p2[rr] = dl * (GATED ? expf(fminf(G[l] - G[m], 0.f)) : 1.f);
            }
            put(dTbT, LDC, 16 * lbt, 16 * mb, p2, lane);    // P2
            put_t(LT, LDC, 16 * lbt, 16 * mb, p2, lane);    // P2^T
        }
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const float a = group_sum<16>(rb[rr]);
            if (cl == 0) rowB[wave & 1][16 * lbt + g4 + rr] = a;
        }
    }
    // row and column sums of dA . A + dL . L
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int mb = 2 * (wave & 1) + u;
        const float cs = tile_colsum(Ev[u]);
        if (g4 == 0) colE[lbt][16 * mb + cl] = cs;
    }
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
        const float a = group_sum<16>(Ev[0][rr] + Ev[1][rr]);
        if (cl == 0) rowE[wave & 1][16 * lbt + g4 + rr] = a;
    }
    __syncthreads();
    // F4: dq = exp(G) d<-Q + P K;  dk = -exp(G) (dR S^T) + exp(G_C - G) d->K + P^T Q + P2 K + P2^T K
#pragma unroll
    for (int u = 0; u < NI; ++u) {
        const int ib = NI * (wave & 1) + u;
        floatx4 aq, ak;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int l = 16 * lbq + g4 + rr;
            aq[rr] = gam[l] * dQd[u][rr];
            ak[rr] = -gam[l] * dKd[u][rr] + (GATED ? expf(G[kC - 1] - G[l]) : 1.f) * dKr[u][rr];
        }
        aq = tilek<T, true, true, kC>(aq, Pm, LDC, 16 * lbq, KT, LDC, 16 * ib, 0, lane);
        ak = tilek<T, true, true, kC>(ak, PT, LDC, 16 * lbq, QT, LDC, 16 * ib, 0, lane);
        if constexpr (DELTA) {
            ak = tilek<T, true, true, kC>(ak, dTbT, LDC, 16 * lbq, KT, LDC, 16 * ib, 0, lane);
            ak = tilek<T, true, true, kC>(ak, LT, LDC, 16 * lbq, KT, LDC, 16 * ib, 0, lane);
        }
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int l = 16 * lbq + g4 + rr;
            if (l < tvalid) {
                dq[(bh * Tlen + t0 + l) * DK + 16 * ib + cl] = from_f32<T>(aq[rr]);
                dk[(bh * Tlen + t0 + l) * DK + 16 * ib + cl] = from_f32<T>(ak[rr]);
            }
        }
    }
    // F5: dG per row, its chunk-end extras, dg = reverse prefix sum; dbeta
    if (wave == 0) {
        const int l = kC - 1 - lane;                 // reversed: lane 0 holds the last row
        float x = rowE[0][l] + rowE[1][l] - (colE[0][l] + colE[1][l] + colE[2][l] + colE[3][l]) + rdp[0][l] +
                  rdp[1][l];
        if constexpr (GATED) {
            const float krs = wave_last(wave_prefix_sum(krp[0][lane] + krp[1][lane]));
            float sd = 0.f;
#pragma unroll
            for (int w = 0; w < 8; ++w) sd += sdp[w];
            if (lane == 0) x += krs + gam[kC - 1] * sd;
            const float dgs = wave_prefix_sum(x);
            if (l < tvalid) dg[bh * Tlen + t0 + l] = from_f32<T>(dgs);
        }
    }
    if constexpr (DELTA) {
        if (wave == 1 && lane < tvalid) {
            const float b = colB[0][lane] + colB[1][lane] + colB[2][lane] + colB[3][lane] + rowB[0][lane] +
                            rowB[1][lane];
            dbeta[bh * Tlen + t0 + lane] = from_f32<T>(b);
        }
    }
}

// ============================================================================
// bwd_grad_channel_kernel: every gradient of one chunk for the per-key-channel
// gate (bf16 tokens).  The value loop is that of bwd_grad_kernel with the
// decayed keys as explicit operands (<-K = 2^G . K and ->K = 2^(G_C - G) . K
// per channel, built in LDS).  The score gradients then keep the decay per
// channel c, D_c[l][m] = 2^(G_lc - G_mc):
//   dq_A[l][c] = sum_m dA[l][m] D_c[l][m] k_mc        dk_L1[l][c] likewise with dL
//   dk_A[m][c] = sum_l dA[l][m] D_c[l][m] q_lc        dk_L2[m][c] = sum_l dL[l][m] D_c[l][m] k_lc
// Off the diagonal 16x16 blocks each is one matrix-core product over the other
// block's rows, the decay split at a block boundary into two factors of at most
// 1 for decays (one on the operand, one on the result); the diagonal blocks
// are summed element by element by thread (block, channel) with the exact
// factors and handed to the result tiles through LDS.  Per element then
//   dq = 2^G d<-Q + dq_A ; dk = 2^G d<-K + 2^(G_C - G) d->K + dk_A + dk_L1 + dk_L2
//   dG = q 2^G d<-Q + k 2^G d<-K - k 2^(G_C-G) d->K + q dq_A - k dk_A + k dk_L1 - k dk_L2
//   dG_C += sum_l k_l 2^(G_C-G_l) d->K_l + 2^(G_C) sum_j S_r[c][j] dS[c][j]
// and dg is the reverse prefix sum of dG over the chunk, per channel.
// ============================================================================
template <int DK, int RULE>
__global__ __launch_bounds__(kNT, 1) void bwd_grad_channel_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ g, const bf16* __restrict__ beta, const bf16* __restrict__ dout,
    const bf16* __restrict__ ops, const bf16* __restrict__ states, const bf16* __restrict__ dstates,
    bf16* __restrict__ dq, bf16* __restrict__ dk, bf16* __restrict__ dv, bf16* __restrict__ dg,
    bf16* __restrict__ dbeta, int64_t Tlen, int64_t nchunks, int DV)
{
    using C = BwdCfg<bf16, DK>;
    constexpr int LDQ = C::LDQ, LDC = C::LDC, LDJ = C::LDJ, J = C::J, E = C::E, LDG = DK + 4;
    constexpr bool DELTA = RULE == kRuleDelta;
    constexpr int NI = DK / 32;            // key-channel tiles per wave (of dq, dk)
    constexpr int NJT = J / 16;            // value-column tiles per step
    constexpr int OSTRIDE = C::OPS + 2 * kC * kC;
    static_assert(4 * NJT == 8, "one step-A tile per wave");
    // the value loop's arrays, and in the same bytes the final phase's
    // X (fp32 [C][LDG]: dTb and X1 first, then the hand-over buffer), G (fp32
    // [C][LDG], base 2), dA and dL (bf16 [C][LDC])
    constexpr int LOOP_BYTES = (5 * kC * LDJ + 2 * DK * LDJ) * 2;
    constexpr int XB = kC * LDG * 4, CB = kC * LDC * 2;
    constexpr int XS = XB > 2 * CB ? XB : 2 * CB;                 // X holds dTb and X1 first
    constexpr int FIN_BYTES = XS + XB + 2 * CB;
    constexpr int REGION = LOOP_BYTES > FIN_BYTES ? LOOP_BYTES : FIN_BYTES;

    __shared__ __align__(16) bf16 KA[kC * LDQ];                // <-K in the loop, then q
    __shared__ __align__(16) bf16 KB[kC * LDQ];                // ->K in the loop, then k
    __shared__ __align__(16) bf16 AqT[kC * LDC];               // A^T in the loop, then T
    __shared__ __align__(16) bf16 TbT[DELTA ? kC * LDC : 8];   // Tb^T in the loop, then L
    __shared__ __align__(16) bf16 Tb[DELTA ? kC * LDC : 8];
    __shared__ __align__(16) unsigned char region[REGION];
    __shared__ __align__(16) float tot[4][DK], tsum[4][DK];
    __shared__ float sdc[DK], bet[kC], colB[kC], rowB[2][kC];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t bh = blockIdx.x / nchunks, r = blockIdx.x % nchunks;
    const int64_t t0 = r * kC;
    const int tvalid = (int)(Tlen - t0 < kC ? Tlen - t0 : kC);
    const bf16* Sr = states + (bh * nchunks + r) * (int64_t)DK * DV;
    const bf16* dSr = dstates + (bh * nchunks + r) * (int64_t)DK * DV;
    const bf16* opc = ops + (bh * nchunks + r) * (int64_t)OSTRIDE;
    const int pc = tid % DK, pb = tid / DK;
    const bool pre = tid < 4 * DK;          // thread (block pb, channel pc)

    // in-chunk prefix of the gate, thread (pb, pc): G of its 16 rows (base 2);
    // every thread calls this (it holds a barrier)
    auto prefix = [&](float* Gl) {
        if (pre) {
            load_col16(Gl, g + (bh * Tlen + t0) * DK + pc, DK, 16 * pb, tvalid);
            float acc = 0.f;
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                acc += Gl[rr] * kLog2eB;
                Gl[rr] = acc;
            }
            tot[pb][pc] = acc;
        }
        __syncthreads();
        if (pre) {
            float off = 0.f;
#pragma unroll
            for (int b = 0; b < 3; ++b)
                if (b < pb) off += tot[b][pc];
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) Gl[rr] += off;
        }
    };

    // ---- front: A^T, Tb, Tb^T and the decayed keys ----
    for (int vv = tid; vv < kC * kC / E; vv += kNT) {
        const int l = vv / (kC / E), m0 = (vv % (kC / E)) * E;
        *reinterpret_cast<i4*>(AqT + l * LDC + m0) = *reinterpret_cast<const i4*>(opc + C::O_AQT + l * kC + m0);
        if constexpr (DELTA) {
            *reinterpret_cast<i4*>(Tb + l * LDC + m0) = *reinterpret_cast<const i4*>(opc + C::O_TB + l * kC + m0);
            *reinterpret_cast<i4*>(TbT + l * LDC + m0) = *reinterpret_cast<const i4*>(opc + C::O_TBT + l * kC + m0);
        }
    }
    if (tid < kC) bet[tid] = (DELTA && tid < tvalid) ? to_f32(beta[bh * Tlen + t0 + tid]) : 0.f;
    {
        float Gl[16], kv[16];
        if (pre) load_col16(kv, k + (bh * Tlen + t0) * DK + pc, DK, 16 * pb, tvalid);
        prefix(Gl);
        if (pre) {
            // 2^(G_C) of this channel: the last row's prefix, read back from the
            // block totals
            const float gl = tot[0][pc] + tot[1][pc] + tot[2][pc] + tot[3][pc];
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                const int row = 16 * pb + rr;
                KA[row * LDQ + pc] = from_f32<bf16>(kv[rr] * fast_exp2(Gl[rr]));
                KB[row * LDQ + pc] = from_f32<bf16>(kv[rr] * fast_exp2(gl - Gl[rr]));
            }
        }
    }

    // the value block's dO and V rows and its S_r and dS_{r+1} columns go
    // through registers, the next block's loads issued before this block's products
    constexpr int VR = J / E, NVJ = (kC * VR + kNT - 1) / kNT;
    constexpr int SR = J / E, NSJ = (DK * SR + kNT - 1) / kNT;
    static_assert(NSJ == 1, "one state row piece per thread");
    i4 pdo[NVJ], pv[NVJ], ps, pds;
    auto fetch = [&](int j0) {
#pragma unroll
        for (int u = 0; u < NVJ; ++u) {
            const int i = tid + u * kNT, row = i / VR, c = (i % VR) * E;
            pdo[u] = pv[u] = i4{0, 0, 0, 0};
            if (i < kC * VR && row < tvalid) {
                pdo[u] = *reinterpret_cast<const i4*>(dout + (bh * Tlen + t0 + row) * DV + j0 + c);
                pv[u] = *reinterpret_cast<const i4*>(v + (bh * Tlen + t0 + row) * DV + j0 + c);
            }
        }
        const int row = tid / SR, c = (tid % SR) * E;
        ps = pds = i4{0, 0, 0, 0};
        if (tid < DK * SR) {
            ps = *reinterpret_cast<const i4*>(Sr + row * DV + j0 + c);
            pds = *reinterpret_cast<const i4*>(dSr + dstate_offset(row, j0 + c, DK));
        }
    };
    fetch(0);

    bf16* const dOs = reinterpret_cast<bf16*>(region);
    bf16* const Rs = dOs + kC * LDJ;
    bf16* const Zs = Rs + kC * LDJ;
    bf16* const dZs = Zs + kC * LDJ;
    bf16* const dRs = dZs + kC * LDJ;
    bf16* const Ss = dRs + kC * LDJ;
    bf16* const dSs = Ss + DK * LDJ;

    const int cl = lane & 15, g4 = 4 * (lane >> 4);
    const int lbq = wave >> 1;                       // row block of this wave's dq/dk tiles
    const int lbt = wave >> 1;                       // row block of its dA/dTb tiles
    floatx4 dQd[NI], dKd[NI], dKr[NI], dAq[2], dTb[2];
#pragma unroll
    for (int u = 0; u < NI; ++u) dQd[u] = dKd[u] = dKr[u] = zero4();
    dAq[0] = dAq[1] = dTb[0] = dTb[1] = zero4();
    float sdot = 0.f;

    for (int j0 = 0; j0 < DV; j0 += J) {
        __syncthreads();
#pragma unroll
        for (int u = 0; u < NVJ; ++u) {
            const int i = tid + u * kNT, row = i / VR, c = (i % VR) * E;
            if (i < kC * VR) {
                *reinterpret_cast<i4*>(dOs + row * LDJ + c) = pdo[u];
                *reinterpret_cast<i4*>(Zs + row * LDJ + c) = pv[u];
            }
        }
        if (tid < DK * SR) {
            const int row = tid / SR, c = (tid % SR) * E;
            bf16 a[E], b[E];
            __builtin_memcpy(a, &ps, 16);
            __builtin_memcpy(b, &pds, 16);
#pragma unroll
            for (int x = 0; x < E; ++x) sdot += to_f32(a[x]) * to_f32(b[x]);
            *reinterpret_cast<i4*>(Ss + row * LDJ + c) = ps;
            *reinterpret_cast<i4*>(dSs + row * LDJ + c) = pds;
        }
        __syncthreads();
        if (j0 + J < DV) fetch(j0 + J);
        // ---- step A: R = V - <-K S_r ; dZ = A^T dO + ->K dS ; d<-Q += dO S_r^T ----
        {
            const int lb = wave / NJT, jc = wave % NJT;
            floatx4 dz = tilek<bf16, true, false, kC>(zero4(), AqT, LDC, 16 * lb, dOs, LDJ, 16 * jc, 0, lane);
            dz = tilek<bf16, true, false, DK>(dz, KB, LDQ, 16 * lb, dSs, LDJ, 16 * jc, 0, lane);
            put(dZs, LDJ, 16 * lb, 16 * jc, dz, lane);
            if constexpr (DELTA) {
                const floatx4 ks = tilek<bf16, true, false, DK>(zero4(), KA, LDQ, 16 * lb, Ss, LDJ, 16 * jc, 0, lane);
                floatx4 rv;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) rv[rr] = to_f32(Zs[(16 * lb + g4 + rr) * LDJ + 16 * jc + cl]) - ks[rr];
                put(Rs, LDJ, 16 * lb, 16 * jc, rv, lane);
            } else {
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int l = 16 * lb + g4 + rr;
                    if (l < tvalid) dv[(bh * Tlen + t0 + l) * DV + j0 + 16 * jc + cl] = from_f32<bf16>(dz[rr]);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < NI; ++u)
            dQd[u] = tilek<bf16, true, true, J>(dQd[u], dOs, LDJ, 16 * lbq, Ss, LDJ, 16 * (NI * (wave & 1) + u), 0, lane);
        __syncthreads();
        // ---- step B (delta): Z = Tb R ; dR = Tb^T dZ (= dv) ; dTb += dZ R^T ----
        if constexpr (DELTA) {
            {
                const int lb = wave / NJT, jc = wave % NJT;
                const floatx4 z = tilek<bf16, true, false, kC>(zero4(), Tb, LDC, 16 * lb, Rs, LDJ, 16 * jc, 0, lane);
                const floatx4 dr = tilek<bf16, true, false, kC>(zero4(), TbT, LDC, 16 * lb, dZs, LDJ, 16 * jc, 0, lane);
                put(Zs, LDJ, 16 * lb, 16 * jc, z, lane);
                put(dRs, LDJ, 16 * lb, 16 * jc, dr, lane);
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int l = 16 * lb + g4 + rr;
                    if (l < tvalid) dv[(bh * Tlen + t0 + l) * DV + j0 + 16 * jc + cl] = from_f32<bf16>(dr[rr]);
                }
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int mb = 2 * (wave & 1) + u;
                if (mb <= lbt) dTb[u] = tilek<bf16, true, true, J>(dTb[u], dZs, LDJ, 16 * lbt, Rs, LDJ, 16 * mb, 0, lane);
            }
            __syncthreads();
        }
        // ---- step C: d<-K += dR S_r^T (negated later) ; d->K += Z dS^T ; dA += dO Z^T ----
#pragma unroll
        for (int u = 0; u < NI; ++u) {
            const int ib = NI * (wave & 1) + u;
            if constexpr (DELTA) dKd[u] = tilek<bf16, true, true, J>(dKd[u], dRs, LDJ, 16 * lbq, Ss, LDJ, 16 * ib, 0, lane);
            dKr[u] = tilek<bf16, true, true, J>(dKr[u], Zs, LDJ, 16 * lbq, dSs, LDJ, 16 * ib, 0, lane);
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int mb = 2 * (wave & 1) + u;
            if (mb <= lbt) dAq[u] = tilek<bf16, true, true, J>(dAq[u], dOs, LDJ, 16 * lbt, Zs, LDJ, 16 * mb, 0, lane);
        }
    }
    __syncthreads();

    // ============ final phase ============
    float* const X = reinterpret_cast<float*>(region);
    float* const Gf = reinterpret_cast<float*>(region + XS);
    bf16* const dAs = reinterpret_cast<bf16*>(region + XS + XB);
    bf16* const dLs = reinterpret_cast<bf16*>(region + XS + XB + CB);
    bf16* const dTbs = reinterpret_cast<bf16*>(region);           // in X
    bf16* const X1s = reinterpret_cast<bf16*>(region + CB);       // in X
    bf16* const Tm = AqT;
    bf16* const Lm = TbT;
    {
        const float s = group_sum<4>(sdot);
        if (tid < DK * SR && tid % SR == 0) sdc[tid / SR] = s;
    }
    // F0: dA and dTb (causal) to LDS; T, L over A^T, Tb^T; raw q, k over the
    // decayed keys; G to LDS
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int mb = 2 * (wave & 1) + u;
        floatx4 a = dAq[u], t = dTb[u];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const bool on = mb < lbt || (mb == lbt && cl <= g4 + rr);
            a[rr] = on ? a[rr] : 0.f;
            t[rr] = on ? t[rr] : 0.f;
        }
        put(dAs, LDC, 16 * lbt, 16 * mb, a, lane);
        if constexpr (DELTA) put(dTbs, LDC, 16 * lbt, 16 * mb, t, lane);
    }
    for (int vv = tid; vv < kC * kC / E; vv += kNT) {
        const int l = vv / (kC / E), m0 = (vv % (kC / E)) * E;
        if constexpr (DELTA) {
            *reinterpret_cast<i4*>(Tm + l * LDC + m0) = *reinterpret_cast<const i4*>(opc + C::OPS + l * kC + m0);
            *reinterpret_cast<i4*>(Lm + l * LDC + m0) =
                *reinterpret_cast<const i4*>(opc + C::OPS + kC * kC + l * kC + m0);
        }
    }
    {
        constexpr int VQ = DK / E;
        for (int i = tid; i < kC * VQ; i += kNT) {
            const int row = i / VQ, c = (i % VQ) * E;
            i4 a = {0, 0, 0, 0}, b = {0, 0, 0, 0};
            if (row < tvalid) {
                a = *reinterpret_cast<const i4*>(q + (bh * Tlen + t0 + row) * DK + c);
                b = *reinterpret_cast<const i4*>(k + (bh * Tlen + t0 + row) * DK + c);
            }
            *reinterpret_cast<i4*>(KA + row * LDQ + c) = a;
            *reinterpret_cast<i4*>(KB + row * LDQ + c) = b;
        }
    }
    {
        float Gl[16];
        prefix(Gl);
        if (pre) {
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) Gf[(16 * pb + rr) * LDG + pc] = Gl[rr];
        }
    }
    __syncthreads();
    bf16* const Qr = KA;
    bf16* const Kr = KB;

    if constexpr (DELTA) {
        // F1: dbeta from T . dTb (column sums); X1 = T^T dTb
        const int sx = tid >> 3, sp = tid & 7;
        {
            float s3 = 0.f;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int m = 8 * sp + u;
                s3 += to_f32(Tm[m * LDC + sx]) * to_f32(dTbs[m * LDC + sx]);
            }
            s3 = group_sum<8>(s3);
            if (sp == 0) colB[sx] = s3;
        }
        floatx4 X1[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int sb = 2 * (wave & 1) + u;
            X1[u] = tilek<bf16, false, false, kC>(zero4(), Tm, LDC, 16 * lbt, dTbs, LDC, 16 * sb, 0, lane);
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) put(X1s, LDC, 16 * lbt, 16 * (2 * (wave & 1) + u), X1[u], lane);
        __syncthreads();
        // F3: dM = -X1 Tb^T ; dL = diag(beta) dM (strict) ; dbeta += rowsum(dM . L)
        float rb[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int mb = 2 * (wave & 1) + u;
            const int m = 16 * mb + cl;
            floatx4 dm = zero4();
            if (mb <= lbt) dm = tilek<bf16, true, true, kC>(zero4(), X1s, LDC, 16 * lbt, Tb, LDC, 16 * mb, 0, lane);
            floatx4 dl;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int l = 16 * lbt + g4 + rr;
                const bool strict = mb <= lbt && m < l;
                const float dM = -dm[rr];
                rb[rr] += strict ? dM * to_f32(Lm[l * LDC + m]) : 0.f;
                dl[rr] = strict ? bet[l] * dM : 0.f;
            }
            put(dLs, LDC, 16 * lbt, 16 * mb, dl, lane);
        }
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const float a = group_sum<16>(rb[rr]);
            if (cl == 0) rowB[wave & 1][16 * lbt + g4 + rr] = a;
        }
        __syncthreads();
    }

    // F4: the off-diagonal blocks of dq_A, dk_L1 (rows of block lbq against
    // keys of earlier blocks, decay split at s = 16 lbq - 1) and of
    // dk_A + dk_L2 (keys of block lbq against rows of later blocks, split at
    // e = 16 lbq + 15)
    floatx4 DQ[NI], KP[NI], KM[NI];
#pragma unroll
    for (int u = 0; u < NI; ++u) {
        DQ[u] = KP[u] = KM[u] = zero4();
        const int c = 16 * (NI * (wave & 1) + u) + cl;   // this lane's channel in the tiles
        if (lbq > 0) {
            const int s = 16 * lbq - 1;
            const float gs = Gf[s * LDG + c];
            floatx4 dq_ = zero4(), kp_ = zero4();
            for (int j = 0; j < lbq; ++j) {
                const int m0 = 16 * j + g4;
                bf16x4 b;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    b[e] = from_f32<bf16>(to_f32(Kr[(m0 + e) * LDQ + c]) * fast_exp2(gs - Gf[(m0 + e) * LDG + c]));
                dq_ = mma16<bf16>(frag_xk(dAs, LDC, 16 * lbq, 16 * j, lane), b, dq_);
                if constexpr (DELTA) kp_ = mma16<bf16>(frag_xk(dLs, LDC, 16 * lbq, 16 * j, lane), b, kp_);
            }
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const float f = fast_exp2(Gf[(16 * lbq + g4 + rr) * LDG + c] - gs);
                DQ[u][rr] += dq_[rr] * f;
                KP[u][rr] += kp_[rr] * f;
            }
        }
        if (lbq < 3) {
            const int e = 16 * lbq + 15;
            const float ge = Gf[e * LDG + c];
            floatx4 km_ = zero4();
            for (int i = lbq + 1; i < 4; ++i) {
                const int l0 = 16 * i + g4;
                bf16x4 bq, bk;
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const float f = fast_exp2(Gf[(l0 + x) * LDG + c] - ge);
                    bq[x] = from_f32<bf16>(to_f32(Qr[(l0 + x) * LDQ + c]) * f);
                    bk[x] = from_f32<bf16>(to_f32(Kr[(l0 + x) * LDQ + c]) * f);
                }
                km_ = mma16<bf16>(frag_kx(dAs, LDC, 16 * lbq, 16 * i, lane), bq, km_);
                if constexpr (DELTA) km_ = mma16<bf16>(frag_kx(dLs, LDC, 16 * lbq, 16 * i, lane), bk, km_);
            }
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) KM[u][rr] += km_[rr] * fast_exp2(ge - Gf[(16 * lbq + g4 + rr) * LDG + c]);
        }
    }
    // F5: the diagonal blocks, thread (pb, pc) over its block's 16 rows with
    // the exact factors, handed to the tiles through X in three rounds.  The
    // terms of a pair (l, m) enter row l of q dq_A and row m of k dk_A with one
    // and the same fp32 product, so they cancel in the suffix sums of dg as
    // they do in the exact gradient (a rounded split of the decay would not).
    // 2^(G_l - G_m) = prod_{s=m+1..l} 2^(G_s - G_{s-1}): one exp per row.
    float aq[16], ap[16], am[16];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) aq[rr] = ap[rr] = am[rr] = 0.f;
    if (pre) {
        float es[16], qd[16], kd[16];
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            const int row = 16 * pb + rr;
            es[rr] = rr > 0 ? fast_exp2(Gf[row * LDG + pc] - Gf[(row - 1) * LDG + pc]) : 1.f;
            qd[rr] = to_f32(Qr[row * LDQ + pc]);
            kd[rr] = to_f32(Kr[row * LDQ + pc]);
        }
#pragma unroll
        for (int li = 0; li < 16; ++li) {
            const int l = 16 * pb + li;
            bf16 ra[16], rl[16];
            {
                const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(dAs + l * LDC + 16 * pb);
                const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(dAs + l * LDC + 16 * pb + 8);
                __builtin_memcpy(ra, &a0, 16);
                __builtin_memcpy(ra + 8, &a1, 16);
            }
            if constexpr (DELTA) {
                const bf16x8 b0 = *reinterpret_cast<const bf16x8*>(dLs + l * LDC + 16 * pb);
                const bf16x8 b1 = *reinterpret_cast<const bf16x8*>(dLs + l * LDC + 16 * pb + 8);
                __builtin_memcpy(rl, &b0, 16);
                __builtin_memcpy(rl + 8, &b1, 16);
            }
            float d = 1.f;                       // 2^(G_l - G_m), m from l down
#pragma unroll
            for (int mi = li; mi >= 0; --mi) {
                if (mi < li) d *= es[mi + 1];
                const float a = to_f32(ra[mi]) * d;
                aq[li] = fmaf(a, kd[mi], aq[li]);
                am[mi] = fmaf(a, qd[li], am[mi]);
                if constexpr (DELTA) {
                    if (mi < li) {
                        const float b = to_f32(rl[mi]) * d;
                        ap[li] = fmaf(b, kd[mi], ap[li]);
                        am[mi] = fmaf(b, kd[li], am[mi]);
                    }
                }
            }
        }
    }
    auto hand_over = [&](const float* part, floatx4* acc) {
        if (pre) {
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) X[(16 * pb + rr) * LDG + pc] = part[rr];
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < NI; ++u) {
            const int c = 16 * (NI * (wave & 1) + u) + cl;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) acc[u][rr] += X[(16 * lbq + g4 + rr) * LDG + c];
        }
        __syncthreads();
    };
    hand_over(aq, DQ);
    if constexpr (DELTA) hand_over(ap, KP);
    hand_over(am, KM);

    // F6: dq, dk; dG per element to X; column sums of k 2^(G_C - G) d->K
#pragma unroll
    for (int u = 0; u < NI; ++u) {
        const int c = 16 * (NI * (wave & 1) + u) + cl;
        const float gC_ = Gf[(kC - 1) * LDG + c];
        floatx4 tk;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int l = 16 * lbq + g4 + rr;
            const float G = Gf[l * LDG + c];
            const float eG = fast_exp2(G), eR = fast_exp2(gC_ - G);
            const float qv = to_f32(Qr[l * LDQ + c]), kv = to_f32(Kr[l * LDQ + c]);
            const float a = eG * dQd[u][rr], b = eG * dKd[u][rr], t = eR * dKr[u][rr];
            const float dqv = a + DQ[u][rr];
            const float dkv = t - b + KP[u][rr] + KM[u][rr];
            X[l * LDG + c] = qv * (a + DQ[u][rr]) - kv * (b + t - KP[u][rr] + KM[u][rr]);
            tk[rr] = kv * t;
            if (l < tvalid) {
                dq[(bh * Tlen + t0 + l) * DK + c] = from_f32<bf16>(dqv);
                dk[(bh * Tlen + t0 + l) * DK + c] = from_f32<bf16>(dkv);
            }
        }
        const float ts = tile_colsum(tk);
        if (lane < 16) tsum[lbq][c] = ts;
    }
    __syncthreads();
    // F7: dg = reverse prefix sum of dG per channel, plus the chunk-end terms
    {
        float suf[16], acc = 0.f;
        if (pre) {
#pragma unroll
            for (int rr = 15; rr >= 0; --rr) {
                acc += X[(16 * pb + rr) * LDG + pc];
                suf[rr] = acc;
            }
            tot[pb][pc] = acc;
        }
        __syncthreads();
        if (pre) {
        float later = tsum[0][pc] + tsum[1][pc] + tsum[2][pc] + tsum[3][pc] +
                      fast_exp2(Gf[(kC - 1) * LDG + pc]) * sdc[pc];
#pragma unroll
        for (int b = 1; b < 4; ++b)
            if (b > pb) later += tot[b][pc];
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            const int row = 16 * pb + rr;
            if (row < tvalid) dg[(bh * Tlen + t0 + row) * DK + pc] = from_f32<bf16>(suf[rr] + later);
        }
        }
    }
    if constexpr (DELTA) {
        if (wave == 7 && lane < tvalid)
            dbeta[bh * Tlen + t0 + lane] = from_f32<bf16>(colB[lane] + rowB[0][lane] + rowB[1][lane]);
    }
}

// The reverse state pass runs one workgroup per (b, h, value block); blocks of
// 32 value columns (two state waves) instead of 64 when the 64-column blocks
// would leave compute units idle (bf16 tokens; LINATTN_CHAIN_VB=32 or 64 fixes
// the width for tests).
inline bool chain_vb32(int64_t bh, int dv)
{
    if (const char* e = getenv("LINATTN_CHAIN_VB")) return atoi(e) == 32;
    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return false;
    return bh * (dv / 64) < ncu;
}

template <typename T, int DK, int RULE, int GATE>
hipError_t launch_bwd_t(const ChunkBwdProblem& p, hipStream_t s)
{
    const int64_t bh = p.B * p.H;
    const int64_t nchunks = (p.T + kC - 1) / kC;
    const T* q = static_cast<const T*>(p.q);
    const T* k = static_cast<const T*>(p.k);
    const T* g = static_cast<const T*>(p.g);
    const T* beta = static_cast<const T*>(p.beta);
    if (bh * nchunks > 0) {
        hipLaunchKernelGGL((bwd_ops_kernel<T, DK, RULE, GATE>), dim3((unsigned)(bh * nchunks)), dim3(kNT), 0, s,
                           q, k, g, beta, static_cast<T*>(p.ops), p.gC, p.T, nchunks);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    bool vb32 = false;
    if constexpr (sizeof(T) == 2) {
        vb32 = chain_vb32(bh, p.dv);
        if (vb32)
            hipLaunchKernelGGL((bwd_chain_kernel<T, DK, RULE, false, 32>), dim3((unsigned)(bh * (p.dv / 32))),
                               dim3(kNT), 0, s, static_cast<const T*>(p.dout), static_cast<const T*>(p.ops),
                               (int64_t)BwdCfg<T, DK>::OPS, p.gC, p.dsT, static_cast<T*>(p.dstates), p.ds0, p.T,
                               nchunks, p.dv);
    }
    if (!vb32)
        hipLaunchKernelGGL((bwd_chain_kernel<T, DK, RULE, false>), dim3((unsigned)(bh * (p.dv / 64))), dim3(kNT), 0,
                           s, static_cast<const T*>(p.dout), static_cast<const T*>(p.ops),
                           (int64_t)BwdCfg<T, DK>::OPS, p.gC, p.dsT, static_cast<T*>(p.dstates), p.ds0, p.T,
                           nchunks, p.dv);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || bh * nchunks == 0) return e;
    if constexpr (sizeof(T) == 2)
        hipLaunchKernelGGL((bwd_grad_bf16_kernel<DK, RULE, GATE>), dim3((unsigned)(bh * nchunks)), dim3(kNT), 0,
                           s, q, k, static_cast<const T*>(p.v), g, beta, static_cast<const T*>(p.dout),
                           static_cast<const T*>(p.ops), static_cast<const T*>(p.states),
                           static_cast<const T*>(p.dstates), static_cast<T*>(p.dq),
                           static_cast<T*>(p.dk_out), static_cast<T*>(p.dv_out), static_cast<T*>(p.dg),
                           static_cast<T*>(p.dbeta), p.T, nchunks, p.dv);
    else
        hipLaunchKernelGGL((bwd_grad_kernel<T, DK, RULE, GATE>), dim3((unsigned)(bh * nchunks)), dim3(kNT), 0, s,
                           q, k, static_cast<const T*>(p.v), g, beta, static_cast<const T*>(p.dout),
                           static_cast<const T*>(p.states), static_cast<const T*>(p.dstates),
                           static_cast<T*>(p.dq), static_cast<T*>(p.dk_out),
                           static_cast<T*>(p.dv_out), static_cast<T*>(p.dg), static_cast<T*>(p.dbeta), p.T,
                           nchunks, p.dv);
    return hipGetLastError();
}

template <int DK, int RULE>
hipError_t launch_bwd_channel(const ChunkBwdProblem& p, hipStream_t s)
{
    using C = BwdCfg<bf16, DK>;
    const int64_t bh = p.B * p.H;
    const int64_t nchunks = (p.T + kC - 1) / kC;
    const bf16* q = static_cast<const bf16*>(p.q);
    const bf16* k = static_cast<const bf16*>(p.k);
    const bf16* g = static_cast<const bf16*>(p.g);
    const bf16* beta = static_cast<const bf16*>(p.beta);
    if (bh * nchunks > 0) {
        hipLaunchKernelGGL((bwd_ops_channel_kernel<DK, RULE>), dim3((unsigned)(bh * nchunks)), dim3(kNT), 0, s,
                           q, k, g, beta, static_cast<bf16*>(p.ops), p.gC, p.T, nchunks);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (chain_vb32(bh, p.dv))
        hipLaunchKernelGGL((bwd_chain_kernel<bf16, DK, RULE, true, 32>), dim3((unsigned)(bh * (p.dv / 32))),
                           dim3(kNT), 0, s, static_cast<const bf16*>(p.dout), static_cast<const bf16*>(p.ops),
                           (int64_t)(C::OPS + 2 * kC * kC), p.gC, p.dsT, static_cast<bf16*>(p.dstates), p.ds0,
                           p.T, nchunks, p.dv);
    else
        hipLaunchKernelGGL((bwd_chain_kernel<bf16, DK, RULE, true>), dim3((unsigned)(bh * (p.dv / 64))), dim3(kNT),
                           0, s, static_cast<const bf16*>(p.dout), static_cast<const bf16*>(p.ops),
                           (int64_t)(C::OPS + 2 * kC * kC), p.gC, p.dsT, static_cast<bf16*>(p.dstates), p.ds0,
                           p.T, nchunks, p.dv);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || bh * nchunks == 0) return e;
    hipLaunchKernelGGL((bwd_grad_channel_kernel<DK, RULE>), dim3((unsigned)(bh * nchunks)), dim3(kNT), 0, s, q, k,
                       static_cast<const bf16*>(p.v), g, beta, static_cast<const bf16*>(p.dout),
                       static_cast<const bf16*>(p.ops), static_cast<const bf16*>(p.states),
                       static_cast<const bf16*>(p.dstates), static_cast<bf16*>(p.dq), static_cast<bf16*>(p.dk_out),
                       static_cast<bf16*>(p.dv_out), static_cast<bf16*>(p.dg), static_cast<bf16*>(p.dbeta), p.T,
                       nchunks, p.dv);
    return hipGetLastError();
}

template <typename T, int DK>
hipError_t bwd_by_rule_gate(const ChunkBwdProblem& p, hipStream_t s)
{
    if constexpr (sizeof(T) == 2) {
        if (p.gate == kGateChannel)
            return p.rule == kRuleAdd ? launch_bwd_channel<DK, kRuleAdd>(p, s) : launch_bwd_channel<DK, kRuleDelta>(p, s);
    }
    if (p.rule == kRuleAdd)
        return p.gate == kGateNone ? launch_bwd_t<T, DK, kRuleAdd, kGateNone>(p, s)
                                   : launch_bwd_t<T, DK, kRuleAdd, kGateScalar>(p, s);
    return p.gate == kGateNone ? launch_bwd_t<T, DK, kRuleDelta, kGateNone>(p, s)
                               : launch_bwd_t<T, DK, kRuleDelta, kGateScalar>(p, s);
}

}  // namespace

bool chunk_bwd_supported(int dk, int dv, int rule, int gate, int dtype)
{
    (void)rule;
    if (dtype == kBF16) return (dk == 64 || dk == 128) && (dv == 64 || dv == 128);
    return gate != kGateChannel && dk == 64 && (dv == 64 || dv == 128);
}

size_t chunk_bwd_ops_bytes(int dk, int gate, int dtype)
{
    const size_t esz = dtype == kBF16 ? 2 : 4;
    return (size_t)(3 * kC * kC + 3 * kC * dk + (gate == kGateChannel ? 2 * kC * kC : 0)) * esz;
}

hipError_t launch_chunk_bwd(const ChunkBwdProblem& p, hipStream_t s)
{
    if (p.dtype == kBF16)
        return p.dk == 64 ? bwd_by_rule_gate<bf16, 64>(p, s) : bwd_by_rule_gate<bf16, 128>(p, s);
    return bwd_by_rule_gate<float, 64>(p, s);
}

}  // namespace linattn
