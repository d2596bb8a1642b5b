// chunk_pipe.hip — single-pass chunkwise forward for bf16 tokens (add rule and
// delta rule, no gate or a scalar per-token gate), software-pipelined over
// chunks: the intra-chunk work of chunk r+1 runs beside the state pass of
// chunk r.
//
// Sources: "Linear Attention, Visualized" — "Chunkwise algorithm" (parallel
// form inside a chunk, state recurrence between chunks), "Mamba-2: input-
// dependent scalar decay" (chunkwise form: decayed query <-q, right-boundary
// key ->k, local decay matrix Gamma), "DeltaNet" (triangular correction system,
// "Optional: Use UT to share the triangular transform", "Correct the incoming
// state") and the GDN row of the chunkwise table.
//
// What is computed per chunk r (positions l, m = 0..C-1, G = prefix sum of the
// log-gate, gamma_l = exp(G_l), rho_l = exp(G_{C-1} - G_l)):
//   a1  G, gamma, rho (one wave, DPP scan)
//   a2  Aq[l][m] = (q_l . k_m) exp(G_l - G_m)            (m <= l)
//       N [l][m] = beta_l (k_l . k_m) exp(G_l - G_m)     (m <  l)   [delta]
//   a3  T = (I + N)^-1 (tsolve.h)                                [delta]
//   a4  Tb = T diag(beta)                                        [delta]
//   b1  R = V - diag(gamma) K S_r ;  Z = Tb R                   [delta]
//       (Z = U - W S_r of the UT form, with U = Tb V and W = Tb <-K applied
//        to V - <-K S_r in one product; add rule: Z = V)
//       S_{r+1} = gamma_{C-1} S_r + K^T diag(rho) Z
//   c1  O = diag(gamma) Q S_r + Aq Z
//
// One workgroup owns one (batch, head, 64 value columns) and walks its chunks
// in order with eight waves in two roles, each role running its own copy of
// the loop; all waves meet at the same two LDS barriers per step.  Step r:
//
//            state waves 0..3 (chunk r)          waves 4..7 (chunk r+1, r+2)
//   phase 1  R = V - gamma K S_r,                 delta: diagonal N blocks, their
//            gamma Q S_r, K^T (matrix-core        inverses, N blocks below the
//            transposes); delta: Aq of chunk      diagonal (chunk r+1); add: Aq
//            r+1                                  of chunk r+1
//   ---- barrier
//   phase 2  Z = Tb R, O = gamma Q S_r + Aq Z     chunk r+2's Q, K and chunk r+1's
//            (straight to HBM), S_{r+1}; delta,   V from registers to LDS, chunk
//            waves 0, 1, 2: off-diagonal blocks   r+2's gate scan; loads for the
//            of T (chunk r+1)                     step after next
//   ---- barrier
//
// Q and K are double-buffered in LDS (chunk parity), and so are Aq and Tb; the
// gate arrays rotate through three slots (chunk mod 3).  The state waves own
// 16 value columns each and keep S[:, those columns] (fp32) as dk/16 MFMA
// result tiles for the whole sequence; S, R and Z never leave registers.
// Inside the loop their only global accesses are the output stores.  Operands
// are bf16, accumulation is fp32; the state is rounded to bf16 only as an
// operand.
#include "device_common.h"
#include "launch.h"
#include "mfma.h"
#include "prep.h"
#include "tsolve.h"

namespace linattn {

namespace {

constexpr int kC = 64;                 // chunk length
constexpr int kNW = 8;                 // waves per workgroup
constexpr int kNT = kNW * kWave;
constexpr int kNS = 4 * kWave;         // threads of waves 4..7 (loads and staging)
constexpr int kDVB = 64;               // value columns per workgroup (4 state waves x 16)
constexpr float kLog2e = 1.4426950408889634f;

template <int DK, int RULE, int GATE>
struct PipeCfg {
    using T = bf16;
    static constexpr int PADE = 16 / sizeof(T);   // 16-byte row padding
    static constexpr int LDQ = DK + PADE;         // rows of length dk: Qs, Ks
    static constexpr int LDC = kC + PADE;         // rows of length C: KsT, Aq, Tb
    static constexpr int LDV = kDVB + PADE;       // rows of V and O
    static constexpr bool DELTA = RULE == kRuleDelta;
    static constexpr bool GATED = GATE == kGateScalar;
    static constexpr int ND = DK / 16, NL = kC / 16;
    static constexpr int E = 16 / sizeof(T);                 // elements per 16-byte load
    static constexpr int NQ = kC * DK / (E * kNS);           // Q/K vectors per loading thread
    static constexpr int NV = kC * kDVB / (E * kNS);         // V vectors per loading thread
    static constexpr int NPAIR = NL * (NL + 1) / 2;          // causal 16x16 tiles
    static_assert(NQ >= 1 && NV >= 1 && E == 8, "load split");
};

// (lj, mi) of the p-th causal tile, mi <= lj, row-major over lj
__device__ __forceinline__ void causal_pair(int p, int& lj, int& mi)
{
    lj = 0;
    while (p > lj) { p -= lj + 1; ++lj; }
    mi = p;
}

// VIRT: Gated DeltaProduct read in place ("Linear Attention, Visualized",
// "GDP as GDN over a virtual sequence"): the chunks walk the virtual sequence
// of Tlen = T nh substeps (k, v, beta already in that layout), the query of
// real token t sits on its last substep and its log-gate on its first, both
// read from the real [B,H,T] layout, and only the last substep's output of each
// token is written, to the real o [B,H,T,dv].
// NHC > 0 fixes n_h at compile time (its divisions become shifts for 2).
template <int DK, int RULE, int GATE, bool VIRT, int NHC = 0>
__global__ __launch_bounds__(kNT, 1) void chunk_pipe_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ g, const bf16* __restrict__ beta, const float* s0, bf16* __restrict__ o,
    float* s_final, int64_t Tlen, int DV, int nblocks, int prep, int nh_arg)
{
    const int nh = NHC > 0 ? NHC : nh_arg;
    using T = bf16;
    using Cfg = PipeCfg<DK, RULE, GATE>;
    using F = typename Frag16<T>::type;
    using Fr = typename Mfma<T>::frag;
    constexpr int LDQ = Cfg::LDQ, LDC = Cfg::LDC, LDV = Cfg::LDV;
    constexpr bool DELTA = Cfg::DELTA, GATED = Cfg::GATED;
    constexpr int ND = Cfg::ND, NL = Cfg::NL, E = Cfg::E, NQ = Cfg::NQ, NV = Cfg::NV;
    constexpr int NK = DK / Mfma<T>::kStep;          // MFMA steps over the key dimension

    __shared__ __align__(16) T Qs[2][kC * LDQ];
    __shared__ __align__(16) T Ks[2][kC * LDQ];
    __shared__ __align__(16) T KsT[DK * LDC];
    __shared__ __align__(16) T Vs[kC * LDV];
    __shared__ __align__(16) T Aq[2][kC * LDC];
    __shared__ __align__(16) T Tb[DELTA ? 2 : 1][DELTA ? kC * LDC : 8];
    // the six N blocks below the diagonal as row fragments, lane by lane, and the
    // X tiles (diagonal-block inverses) the two halves of the off-diagonal
    // transform need: X11^T, X22, X22^T, X33^T, X00, X11 in slots 0..5
    __shared__ __align__(16) floatx4 Nlo[DELTA ? 6 * kWave : 1];
    __shared__ __align__(16) floatx4 Xx[DELTA ? 6 * kWave : 1];
    // gate values of chunk c in slot c mod 3: the state waves read chunk r's
    // while waves 4..7 read chunk r+1's and wave 4 writes chunk r+2's
    __shared__ __align__(16) float Gsb[3][kC], gamb[3][kC], rhob[3][kC], betb[3][kC];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int nvb = DV / kDVB;

    // Workgroups of one head land on the same XCD (dispatch is round-robin
    // over the 8 XCDs), so its value blocks share q/k reads in that XCD's L2.
    int blk = blockIdx.x;
    if ((nblocks & 7) == 0) blk = (blk & 7) * (nblocks >> 3) + (blk >> 3);
    const int64_t bh = blk / nvb;
    const int vb = blk % nvb;
    const int64_t Treal = VIRT ? Tlen / nh : Tlen;   // rows of q, g and o
    const T* qh = q + bh * Treal * DK;
    const T* kh = k + bh * Tlen * DK;
    const T* vh = v + bh * Tlen * DV + vb * kDVB;
    const int64_t nchunks = (Tlen + kC - 1) / kC;
    const int64_t tlast = (nchunks - 1) * kC;     // start of the last chunk
    auto clampc = [&](int64_t t0) { return t0 < tlast ? t0 : tlast; };

    // causal blocks above the diagonal of Aq and Tb stay zero for the whole run
    for (int i = tid; i < 2 * kC * LDC; i += kNT) (&Aq[0][0])[i] = from_f32<T>(0.f);
    if constexpr (DELTA)
        for (int i = tid; i < 2 * kC * LDC; i += kNT) (&Tb[0][0])[i] = from_f32<T>(0.f);

    typedef __attribute__((__vector_size__(16))) int i4;

    // ---- loads and staging (waves 4..7, thread st of kNS).  Loads never wait
    // where they are issued: rows past the end read the last row (in bounds) and
    // are zeroed when staged, so every load is unconditional.  Two register sets
    // alternate between steps, so a load has about two steps to arrive.
    struct Pref {
        i4 q[NQ], k[NQ], v[NV];
        T g, b;
    };
    const int st = tid - (kNT - kNS);
    auto fetch_qk = [&](Pref& P, int64_t t0) {
#pragma unroll
        for (int p = 0; p < NQ; ++p) {
            const int idx = (p * kNS + st) * E;
            const int row = idx / DK, col = idx % DK;
            const int64_t tr = t0 + row < Tlen ? t0 + row : Tlen - 1;
            P.q[p] = *reinterpret_cast<const i4*>(qh + (VIRT ? (int64_t)((int)tr / nh) : tr) * DK + col);
            P.k[p] = *reinterpret_cast<const i4*>(kh + tr * DK + col);
        }
    };
    auto fetch_v = [&](Pref& P, int64_t t0) {
#pragma unroll
        for (int p = 0; p < NV; ++p) {
            const int idx = (p * kNS + st) * E;
            const int row = idx / kDVB, col = idx % kDVB;
            const int64_t tr = t0 + row < Tlen ? t0 + row : Tlen - 1;
            P.v[p] = *reinterpret_cast<const i4*>(vh + tr * DV + col);
        }
    };
    // gate and beta of one chunk, one token per lane (every wave of the group
    // loads them so that all its global accesses are unconditional)
    auto fetch_gate = [&](Pref& P, int64_t t0) {
        const int64_t tr = t0 + lane < Tlen ? t0 + lane : Tlen - 1;
        P.g = GATED ? g[bh * Treal + (VIRT ? (int64_t)((int)tr / nh) : tr)] : from_f32<T>(0.f);
        P.b = DELTA ? beta[bh * Tlen + tr] : from_f32<T>(0.f);
    };
    // Q and K rows go to LDS with their columns in swizzled pcol order
    // (mfma.h), four columns (8 bytes) at a time.  At dk = 128 the threads of
    // the second 64 columns of a row write their upper four columns first, so
    // each 16-lane group of a write instruction covers 32 distinct banks.
    // (raw projections first go through the q/k map of prep.h; rows past the
    // end are zeroed after it)
    auto stage_qk = [&](const Pref& P, int64_t t0, T* Qb, T* Kb) {
        typedef __attribute__((__vector_size__(8))) int i2;
        const int qk_map = prep_qk_map(prep);
#pragma unroll
        for (int p = 0; p < NQ; ++p) {
            const int idx = (p * kNS + st) * E;
            const int row = idx / DK, col = idx % DK;
            const bool ok = t0 + row < Tlen;
            // (virtual sequence: the query only on a token's last substep)
            const bool okq = ok && (!VIRT || (int)(t0 + row) % nh == nh - 1);
            // every lane maps its vector (the L2 norm is reduced across lanes)
            const i4 qp = prep_qk<T, DK / E>(P.q[p], qk_map);
            const i4 kp = prep_qk<T, DK / E>(P.k[p], qk_map);
            const i4 qv = okq ? qp : i4{0, 0, 0, 0};
            const i4 kv = ok ? kp : i4{0, 0, 0, 0};
            const int sw = swz_x(row);
            const bool hi = DK == 128 && (col & 64);
            const int c0 = row * LDQ + (pcol(col + (hi ? 4 : 0)) ^ sw);
            const int c1 = row * LDQ + (pcol(col + (hi ? 0 : 4)) ^ sw);
            *reinterpret_cast<i2*>(&Qb[c0]) = hi ? i2{qv[2], qv[3]} : i2{qv[0], qv[1]};
            *reinterpret_cast<i2*>(&Kb[c0]) = hi ? i2{kv[2], kv[3]} : i2{kv[0], kv[1]};
            *reinterpret_cast<i2*>(&Qb[c1]) = hi ? i2{qv[0], qv[1]} : i2{qv[2], qv[3]};
            *reinterpret_cast<i2*>(&Kb[c1]) = hi ? i2{kv[0], kv[1]} : i2{kv[2], kv[3]};
        }
    };
    auto stage_v = [&](const Pref& P, int64_t t0) {
#pragma unroll
        for (int p = 0; p < NV; ++p) {
            const int idx = (p * kNS + st) * E;
            const int row = idx / kDVB, col = idx % kDVB;
            const bool ok = t0 + row < Tlen;
            *reinterpret_cast<i4*>(&Vs[row * LDV + col]) = ok ? P.v[p] : i4{0, 0, 0, 0};
        }
    };
    // wave 7's gate scan of one chunk into slot sl.  G is kept in base 2
    // (log2 e * prefix sum) so every decay factor is one hardware exp2.
    auto scan = [&](const Pref& P, int64_t t0, int sl) {
        const bool ok = t0 + lane < Tlen;
        // (virtual sequence: the log-gate only on a token's first substep)
        const bool okg = ok && (!VIRT || (int)(t0 + lane) % nh == 0);
        const float G = wave_prefix_sum((GATED && okg) ? prep_gate(to_f32(P.g), prep) * kLog2e : 0.f);
        const float Glast = wave_last(G);
        Gsb[sl][lane] = G;
        gamb[sl][lane] = GATED ? fast_exp2(G) : 1.f;
        rhob[sl][lane] = GATED ? fast_exp2(Glast - G) : 1.f;
        betb[sl][lane] = (DELTA && ok) ? prep_beta(to_f32(P.b), prep) : 0.f;
    };

    // The state waves store their output tiles straight to HBM, through a buffer
    // resource over this head's rows: rows past the end (and, on the virtual
    // sequence, the substeps that are not a token's last) fall outside it and
    // the hardware drops them.  The state waves issue no global loads inside
    // the loop, so the stores never enter a wait count there.
    const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
        o + bh * Treal * DV, (short)0, (int)(Treal * DV * (int64_t)sizeof(T)), 0x00020000);

    // ---- matrix-core helpers over LDS tiles
    // All fragments (every k step) of the 16-row block b of a [C][DK] tile (Qs or
    // Ks); a wave loads each block it needs once per chunk.
    auto block_frags = [&](const T* A, int b, int ln, Fr (&f)[NK]) {
#pragma unroll
        for (int i = 0; i < NK; ++i) f[i] = mfma_load_sw(&A[b * 16 * LDQ], LDQ, i * Mfma<T>::kStep, ln);
    };
    // x[rr] = sum_c A[16 mi + g4 + rr][c] B[16 lj + cl][c] from the blocks' fragments
    auto tile_dot = [&](const Fr (&fa)[NK], const Fr (&fb)[NK]) {
        floatx4 x = zero4();
#pragma unroll
        for (int i = 0; i < NK; ++i) x = Mfma<T>::mma(fa[i], fb[i], x);
        return x;
    };
    // a2 Aq tile (lj, mi), mi <= lj, from xa[rr] = k_m . q_l:
    // Aq[l][m] = (q_l . k_m) exp(G_l - G_m), m <= l
    auto aq_store = [&](const float* Gs, T* Aqb, int lj, int mi, floatx4 xa, int ln) {
        const int cl = ln & 15, g4 = 4 * (ln >> 4);
        const float Gl = Gs[lj * 16 + cl];
        const floatx4 Gm = *reinterpret_cast<const floatx4*>(&Gs[mi * 16 + g4]);
        floatx4 va;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const float dec = GATED ? fast_exp2(Gl - Gm[rr]) : 1.f;
            va[rr] = (mi < lj || g4 + rr <= cl) ? xa[rr] * dec : 0.f;
        }
        store_tile_t_pc_sw(&Aqb[lj * 16 * LDC], LDC, mi, va, ln);
    };
    // a2 diagonal N block b in registers.  x = K_b K_b^T is symmetric, so one
    // product gives N_bb both as tile(N_bb^T) (lane value N[l][m], l = 16 b + cl)
    // and as tile(N_bb); at most one of the two is nonzero at each position, so
    // one exp2 serves both.  br[rr] = beta[16 b + g4 + rr]; kb returns K_b's
    // fragments for the wave's other tiles.
    auto diag_block = [&](const T* Kb, const float* Gs, const float* bet, int b, int ln, floatx4& nd,
                          floatx4& nt, floatx4& br, Fr (&kb)[NK]) {
        const int cl = ln & 15, g4 = 4 * (ln >> 4);
        block_frags(Kb, b, ln, kb);
        const floatx4 Grow = *reinterpret_cast<const floatx4*>(&Gs[16 * b + g4]);
        br = *reinterpret_cast<const floatx4*>(&bet[16 * b + g4]);
        const float Gcol = Gs[16 * b + cl], bcol = bet[16 * b + cl];
        const floatx4 x = tile_dot(kb, kb);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const bool up = g4 + rr < cl;                       // N[l][m] with m < l
            const float d = GATED ? fast_exp2(up ? Gcol - Grow[rr] : Grow[rr] - Gcol) : 1.f;
            nt[rr] = up ? bcol * x[rr] * d : 0.f;
            nd[rr] = (cl < g4 + rr) ? br[rr] * x[rr] * d : 0.f;
        }
    };
    // a2 N block (lj, mi), mi < lj, from K_mi and K_lj fragments, as a row
    // fragment into slot lj (lj - 1) / 2 + mi of Nlo
    auto n_block = [&](const float* Gs, const float* bet, int lj, int mi, const Fr (&fm)[NK],
                       const Fr (&fl)[NK], int ln) {
        const int cl = ln & 15, g4 = 4 * (ln >> 4);
        const floatx4 x = tile_dot(fm, fl);
        const floatx4 Grow = *reinterpret_cast<const floatx4*>(&Gs[16 * mi + g4]);
        const float Gcol = Gs[16 * lj + cl], bcol = bet[16 * lj + cl];
        floatx4 t;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) t[rr] = bcol * x[rr] * (GATED ? fast_exp2(Gcol - Grow[rr]) : 1.f);
        Nlo[(lj * (lj - 1) / 2 + mi) * kWave + ln] = t;
    };
    // delta rule, phase 1 of wave 4 + b: diagonal block b and its inverse (the
    // diagonal block of Tb), the N blocks below the diagonal that share K_b
    // (wave 4: N10, N20; wave 5: N21, N31; wave 6: N32; wave 7: N30), and the X
    // tiles the off-diagonal transform needs.
    auto intra_p1 = [&](const T* Kb, const float* Gs, const float* bet, T* Tbb, int b, int ln) {
        floatx4 nd[1], nt[1], br[1], Xa[1], Xta[1];
        Fr kb[NK], k2[NK];
        diag_block(Kb, Gs, bet, b, ln, nd[0], nt[0], br[0], kb);
        tsolve_diag<T, 2, 1>(nd, nt, Xa, Xta, Tbb, LDC, br, ln, b);
        const floatx4 X = Xa[0], Xt = Xta[0];
        // the six blocks below the diagonal, 1-2 per wave: blocks 0 and 1 also
        // hold the off-diagonal transform's longest inputs (X00, X11), so the
        // waves of blocks 2 and 3 take two N blocks each
        if (b == 0) {
            block_frags(Kb, 1, ln, k2);
            n_block(Gs, bet, 1, 0, kb, k2, ln);
            Xx[4 * kWave + ln] = X;
        } else if (b == 1) {
            block_frags(Kb, 2, ln, k2);
            n_block(Gs, bet, 2, 1, kb, k2, ln);
            Xx[0 * kWave + ln] = Xt;
            Xx[5 * kWave + ln] = X;
        } else if (b == 2) {
            block_frags(Kb, 3, ln, k2);
            n_block(Gs, bet, 3, 2, kb, k2, ln);
            block_frags(Kb, 0, ln, k2);
            n_block(Gs, bet, 2, 0, k2, kb, ln);
            Xx[1 * kWave + ln] = X;
            Xx[2 * kWave + ln] = Xt;
        } else {
            block_frags(Kb, 0, ln, k2);
            n_block(Gs, bet, 3, 0, k2, kb, ln);
            block_frags(Kb, 1, ln, k2);
            n_block(Gs, bet, 3, 1, k2, kb, ln);
            Xx[3 * kWave + ln] = Xt;
        }
    };
    // delta rule: half h of the off-diagonal blocks of T (tsolve.h) for the chunk
    // whose beta is bet, from the N blocks and X tiles in LDS, into Tbb
    auto offdiag = [&](int h, const float* bet, T* Tbb, int ln) {
        const int g4 = 4 * (ln >> 4);
        floatx4 brow[NL];
#pragma unroll
        for (int b = 0; b < NL; ++b) brow[b] = *reinterpret_cast<const floatx4*>(&bet[16 * b + g4]);
        const floatx4* nl = Nlo + ln;
        const floatx4* xx = Xx + ln;
        if (h == 0)
            tsolve_offdiag_a<T, 2>(xx[4 * kWave], xx[0 * kWave], xx[2 * kWave], xx[3 * kWave], nl[0 * kWave],
                                      nl[1 * kWave], nl[2 * kWave], nl[3 * kWave], nl[4 * kWave], nl[5 * kWave],
                                      Tbb, LDC, brow, ln);
        else if (h == 1)
            tsolve_offdiag_b1<T, 2>(xx[5 * kWave], xx[2 * kWave], xx[3 * kWave], nl[2 * kWave], nl[4 * kWave],
                                    nl[5 * kWave], Tbb, LDC, brow, ln);
        else
            tsolve_t32<T, 2>(xx[1 * kWave], xx[3 * kWave], nl[5 * kWave], Tbb, LDC, brow, ln);
    };

    if (wave < 4) {
        // ======== state waves: wave w owns value columns n0..n0+15 of the block and
        // keeps S[:, those columns] as ND result tiles S[db][rr] = S[16 db + g4 + rr][n0 + cl]
        const int n0 = 16 * wave;
        floatx4 S[ND];
        {
            const int cl = lane & 15, g4 = 4 * (lane >> 4);
#pragma unroll
            for (int db = 0; db < ND; ++db) {
                S[db] = zero4();
                if (s0) {
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr)
                        S[db][rr] = s0[(bh * DK + 16 * db + g4 + rr) * DV + vb * kDVB + n0 + cl];
                }
            }
        }
        wait_vmem_all();
        // delta rule: a2 Aq tiles of chunk c, grouped so each wave loads few
        // blocks: wave 0 the query blocks 0-1, wave 1 block 2, waves 2-3 block 3
        auto aq_state = [&](int64_t c, int ln) {
            const float* const Gs = Gsb[c % 3];
            const T* const Qb = Qs[c & 1];
            const T* const Kb = Ks[c & 1];
            T* const Aqb = Aq[c & 1];
            Fr fq[NK], fa[NK], fb[NK];
            if (wave == 0) {
                block_frags(Kb, 0, ln, fa);
                block_frags(Qb, 0, ln, fq);
                aq_store(Gs, Aqb, 0, 0, tile_dot(fa, fq), ln);
                block_frags(Qb, 1, ln, fq);
                aq_store(Gs, Aqb, 1, 0, tile_dot(fa, fq), ln);
                block_frags(Kb, 1, ln, fb);
                aq_store(Gs, Aqb, 1, 1, tile_dot(fb, fq), ln);
            } else if (wave == 1) {
                block_frags(Qb, 2, ln, fq);
                block_frags(Kb, 0, ln, fa);
                aq_store(Gs, Aqb, 2, 0, tile_dot(fa, fq), ln);
                block_frags(Kb, 1, ln, fb);
                aq_store(Gs, Aqb, 2, 1, tile_dot(fb, fq), ln);
                block_frags(Kb, 2, ln, fa);
                aq_store(Gs, Aqb, 2, 2, tile_dot(fa, fq), ln);
            } else {
                const int m0 = wave == 2 ? 0 : 2;
                block_frags(Qb, 3, ln, fq);
                block_frags(Kb, m0, ln, fa);
                aq_store(Gs, Aqb, 3, m0, tile_dot(fa, fq), ln);
                block_frags(Kb, m0 + 1, ln, fb);
                aq_store(Gs, Aqb, 3, m0 + 1, tile_dot(fb, fq), ln);
            }
        };
        if (nchunks > 0) {
            // step -1: chunk 0's Aq tiles and (waves 0, 1) off-diagonal T blocks
            lds_barrier();
            if constexpr (DELTA) aq_state(0, opaque(lane));
            lds_barrier();
            if constexpr (DELTA)
                if (wave < 3) offdiag(wave, betb[0], Tb[0], opaque(lane));
            lds_barrier();
        }
        for (int64_t r = 0; r < nchunks; ++r) {
            const int ln = lane;
            const int cl = ln & 15, g4 = 4 * (ln >> 4);
            const int sl = (int)(r % 3);
            const float* const gam = gamb[sl];
            const float* const rho = rhob[sl];
            const T* const Qc = Qs[r & 1];
            const T* const Kc = Ks[r & 1];

            // ---- phase 1: R = V - gamma K S_r (delta; V for add) ---------------------
            floatx4 R[NL], Ot[NL];
#pragma unroll
            for (int li = 0; li < NL; ++li)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) R[li][rr] = to_f32(Vs[(16 * li + g4 + rr) * LDV + n0 + cl]);
            if constexpr (DELTA) {
                floatx4 P[NL];
#pragma unroll
                for (int li = 0; li < NL; ++li) P[li] = zero4();
#pragma unroll
                for (int db = 0; db < ND; db += 2) {
                    const auto sp = pair_regs<T>(S[db], S[db + 1]);
#pragma unroll
                    for (int li = 0; li < NL; ++li)
                        P[li] = mma_pair<T>(pair_lds_sw(&Kc[16 * li * LDQ + 16 * db], LDQ, ln), sp, P[li]);
                }
#pragma unroll
                for (int li = 0; li < NL; ++li) {
                    const floatx4 gr = *reinterpret_cast<const floatx4*>(&gam[16 * li + g4]);
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) R[li][rr] -= gr[rr] * P[li][rr];
                }
            }
            // O^T = (S_r^T Q^T) gamma
#pragma unroll
            for (int li = 0; li < NL; ++li) Ot[li] = zero4();
#pragma unroll
            for (int db = 0; db < ND; db += 2) {
                const auto sp = pair_regs<T>(S[db], S[db + 1]);
#pragma unroll
                for (int li = 0; li < NL; ++li)
                    Ot[li] = mma_pair<T>(sp, pair_lds_sw(&Qc[16 * li * LDQ + 16 * db], LDQ, ln), Ot[li]);
            }
#pragma unroll
            for (int li = 0; li < NL; ++li) {
                const float gl = gam[16 * li + cl];
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) Ot[li][rr] *= gl;
            }
            // K^T through the matrix core (this wave's quarter of the tiles)
            {
                constexpr int NKT = NL * ND / 4;
                F af[NKT];
#pragma unroll
                for (int i = 0; i < NKT; ++i) {
                    const int t = wave + 4 * i;
                    af[i] = frag16_lds_pc_sw(&Kc[(t / ND) * 16 * LDQ], LDQ, t % ND, ln);
                }
                const F id = ident_frag<T>(ln);
                floatx4 d[NKT];
#pragma unroll
                for (int i = 0; i < NKT; ++i) d[i] = mma16<T>(af[i], id, zero4());
#pragma unroll
                for (int i = 0; i < NKT; ++i) {
                    const int t = wave + 4 * i;
                    store_tile_t_pc_sw(&KsT[(t % ND) * 16 * LDC], LDC, t / ND, d[i], ln);
                }
            }
            if constexpr (DELTA)
                if (r + 1 < nchunks) aq_state(r + 1, ln);
            lds_barrier();

            // ---- phase 2: b1 Z = Tb R ; c1 O^T += Z^T Aq^T ; S_{r+1} ------------------
            // Products over token blocks run in pairs (blocks 0,1 and 2,3); the
            // causal blocks above the diagonal of Tb and Aq are zero, so block rows
            // 0 and 2 take them as partners and every accumulation chain keeps one
            // MFMA shape (mfma.h).
            const T* const Aqc = Aq[r & 1];
            floatx4 Z[NL];
            if constexpr (DELTA) {
                const T* const Tbc = Tb[r & 1];
                // Z[li] = sum_{mj <= li} Tb(li, mj) R[mj]
                const auto r01 = pair_regs<T>(R[0], R[1]), r23 = pair_regs<T>(R[2], R[3]);
#pragma unroll
                for (int li = 0; li < NL; ++li) {
                    Z[li] = mma_pair<T>(pair_lds_sw(&Tbc[16 * li * LDC], LDC, ln), r01, zero4());
                    if (li >= 2) Z[li] = mma_pair<T>(pair_lds_sw(&Tbc[16 * li * LDC + 32], LDC, ln), r23, Z[li]);
                }
            } else {
#pragma unroll
                for (int li = 0; li < NL; ++li) Z[li] = R[li];
            }
            {
                // Ot[lj] += sum_{mj <= lj} Z[mj]^T Aq(lj, mj)^T
                const auto z01 = pair_regs<T>(Z[0], Z[1]), z23 = pair_regs<T>(Z[2], Z[3]);
#pragma unroll
                for (int lj = 0; lj < NL; ++lj) {
                    Ot[lj] = mma_pair<T>(z01, pair_lds_sw(&Aqc[16 * lj * LDC], LDC, ln), Ot[lj]);
                    if (lj >= 2) Ot[lj] = mma_pair<T>(z23, pair_lds_sw(&Aqc[16 * lj * LDC + 32], LDC, ln), Ot[lj]);
                }
            }
            // O^T tiles to HBM: lane (cl, g4) holds token 16 lj + cl of the chunk and
            // value columns n0 + g4 .. n0 + g4 + 3, one 8-byte store
#pragma unroll
            for (int lj = 0; lj < NL; ++lj) {
                const int64_t vr = r * kC + 16 * lj + cl;
                const bool keep = !VIRT || (int)vr % nh == nh - 1;
                const int off = keep ? (int)(((VIRT ? (int64_t)((int)vr / nh) : vr) * DV + vb * kDVB + n0 + g4) *
                                             (int64_t)sizeof(T))
                                     : 0x7fffffff;
                typedef __attribute__((__vector_size__(8))) int i2;
                T e[4];
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) e[rr] = from_f32<T>(Ot[lj][rr]);
                i2 x;
                __builtin_memcpy(&x, e, 8);
                __builtin_amdgcn_raw_buffer_store_b64(x, orsrc, off, 0, 0);
            }
            // S_{r+1} = gamma_{C-1} S_r + K^T diag(rho) Z
            const float gC = gam[kC - 1];
            floatx4 zr[NL];
#pragma unroll
            for (int lj = 0; lj < NL; ++lj) {
                zr[lj] = Z[lj];
                if constexpr (GATED) {
                    const floatx4 rh = *reinterpret_cast<const floatx4*>(&rho[16 * lj + g4]);
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) zr[lj][rr] *= rh[rr];
                }
            }
            const auto zr01 = pair_regs<T>(zr[0], zr[1]), zr23 = pair_regs<T>(zr[2], zr[3]);
#pragma unroll
            for (int db = 0; db < ND; ++db) {
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) S[db][rr] *= gC;
                S[db] = mma_pair<T>(pair_lds_sw(&KsT[16 * db * LDC + 32], LDC, ln), zr23,
                                    mma_pair<T>(pair_lds_sw(&KsT[16 * db * LDC], LDC, ln), zr01, S[db]));
            }
            if constexpr (DELTA)
                if (wave < 3 && r + 1 < nchunks) offdiag(wave, betb[(r + 1) % 3], Tb[(r + 1) & 1], ln);
            lds_barrier();
        }
        // waves 4..7 run an even number of steps; the spare one has no work here
        if (nchunks > 0 && (nchunks & 1) == 0) {
            lds_barrier();
            lds_barrier();
        }
        if (s_final) {
            const int cl = lane & 15, g4 = 4 * (lane >> 4);
#pragma unroll
            for (int db = 0; db < ND; ++db)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr)
                    s_final[(bh * DK + 16 * db + g4 + rr) * DV + vb * kDVB + n0 + cl] = S[db][rr];
        }
        return;
    }

    // ======== waves 4..7 ===========================================================
    if (nchunks == 0) return;
    // chunk 0's Q, K and gates into LDS; register set 1 gets what step -1 stages
    // (chunk 1's Q, K and gates, chunk 0's V), set 0 what step 0 stages
    Pref P0, P1;
    fetch_qk(P0, 0);
    fetch_gate(P0, 0);
    stage_qk(P0, 0, Qs[0], Ks[0]);
    if (wave == 7) scan(P0, 0, 0);
    fetch_qk(P1, clampc(kC));
    fetch_v(P1, 0);
    fetch_gate(P1, clampc(kC));
    fetch_qk(P0, clampc(2 * kC));
    fetch_v(P0, clampc(kC));
    fetch_gate(P0, clampc(2 * kC));
    lds_barrier();

    // end of phase 2 of step r: chunk r+2's Q, K and gates and chunk r+1's V
    // from register set P into LDS, then the loads for step r+2 into P
    auto stage_and_fetch = [&](Pref& P, int64_t r) {
        stage_qk(P, (r + 2) * kC, Qs[r & 1], Ks[r & 1]);
        stage_v(P, (r + 1) * kC);
        if (wave == 7) scan(P, (r + 2) * kC, (int)((r + 2) % 3));
        fetch_qk(P, clampc((r + 4) * kC));
        fetch_v(P, clampc((r + 3) * kC));
        fetch_gate(P, clampc((r + 4) * kC));
    };

    // one step r (chunk r+1 prepared; a step past the last chunk does no work
    // but keeps the loop's accesses unconditional)
    auto step = [&](int64_t r, Pref& P) {
        const int ln = lane;
        const int64_t c = r + 1;
        const bool go = c < nchunks;
        const int iw = wave - 4;
        if constexpr (DELTA) {
            const int sl = (int)(c % 3);
            const float* const Gs = Gsb[sl];
            const float* const bet = betb[sl];
            T* const Tbn = Tb[c & 1];
            // ---- phase 1: diagonal block iw, its inverse, lower N blocks
            if (go) intra_p1(Ks[c & 1], Gs, bet, Tbn, iw, ln);
            lds_barrier();
        } else {
            // ---- phase 1: this wave's share of chunk c's Aq tiles
            if (go) {
                const float* const Gs = Gsb[c % 3];
                const T* const Qb = Qs[c & 1];
                const T* const Kb = Ks[c & 1];
#pragma unroll
                for (int p = 0; p < Cfg::NPAIR; ++p) {
                    if (p % 4 == iw) {
                        int lj, mi;
                        causal_pair(p, lj, mi);
                        Fr fa[NK], fb[NK];
                        block_frags(Kb, mi, ln, fa);
                        block_frags(Qb, lj, ln, fb);
                        aq_store(Gs, Aq[c & 1], lj, mi, tile_dot(fa, fb), ln);
                    }
                }
            }
            lds_barrier();
        }
        stage_and_fetch(P, r);
        lds_barrier();
    };
    // steps -1 .. nchunks-1, rounded up to an even count
    for (int64_t r = -1; r < nchunks; r += 2) {
        step(r, P1);
        step(r + 1, P0);
    }
}

template <int DK, int RULE, int GATE, bool VIRT, int NHC = 0>
hipError_t launch_t(const ChunkProblem& p, int nh, hipStream_t s)
{
    const int nvb = p.dv / kDVB;
    const int64_t nblocks = p.B * p.H * nvb;
    hipLaunchKernelGGL((chunk_pipe_kernel<DK, RULE, GATE, VIRT, NHC>), dim3((unsigned)nblocks), dim3(kNT), 0, s,
                       static_cast<const bf16*>(p.q), static_cast<const bf16*>(p.k),
                       static_cast<const bf16*>(p.v), static_cast<const bf16*>(p.g),
                       static_cast<const bf16*>(p.beta), p.s0, static_cast<bf16*>(p.o), p.s_final, p.T,
                       p.dv, (int)nblocks, p.prep, nh);
    return hipGetLastError();
}

template <int DK>
hipError_t by_rule_gate(const ChunkProblem& p, hipStream_t s)
{
    if (p.rule == kRuleAdd)
        return p.gate == kGateNone ? launch_t<DK, kRuleAdd, kGateNone, false>(p, 1, s)
                                   : launch_t<DK, kRuleAdd, kGateScalar, false>(p, 1, s);
    return p.gate == kGateNone ? launch_t<DK, kRuleDelta, kGateNone, false>(p, 1, s)
                               : launch_t<DK, kRuleDelta, kGateScalar, false>(p, 1, s);
}

// the virtual sequence with n_h fixed at compile time for 2, 3 and 4
template <int DK, int GATE>
hipError_t virtual_by_nh(const ChunkProblem& p, int nh, hipStream_t s)
{
    switch (nh) {
    case 2: return launch_t<DK, kRuleDelta, GATE, true, 2>(p, nh, s);
    case 3: return launch_t<DK, kRuleDelta, GATE, true, 3>(p, nh, s);
    case 4: return launch_t<DK, kRuleDelta, GATE, true, 4>(p, nh, s);
    default: return launch_t<DK, kRuleDelta, GATE, true>(p, nh, s);
    }
}

}  // namespace

bool chunk_pipe_supported(const ChunkProblem& p)
{
    return p.dtype == kBF16 && p.gate != kGateChannel && p.chunk == kC && (p.dk == 64 || p.dk == 128) &&
           (p.dv == 64 || p.dv == 128);
}

hipError_t launch_chunk_pipe(const ChunkProblem& p, hipStream_t s)
{
    return p.dk == 64 ? by_rule_gate<64>(p, s) : by_rule_gate<128>(p, s);
}

hipError_t launch_chunk_pipe_virtual(const ChunkProblem& p, int nh, hipStream_t s)
{
    if (p.dk == 64)
        return p.gate == kGateNone ? virtual_by_nh<64, kGateNone>(p, nh, s) : virtual_by_nh<64, kGateScalar>(p, nh, s);
    return p.gate == kGateNone ? virtual_by_nh<128, kGateNone>(p, nh, s) : virtual_by_nh<128, kGateScalar>(p, nh, s);
}

}  // namespace linattn
