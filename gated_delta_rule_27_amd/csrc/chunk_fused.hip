// chunk_fused.hip — single-pass chunkwise forward for the add rule and the
// delta rule with no gate or a scalar (per token) gate.
//
// Sources: "Linear Attention, Visualized" — "Chunkwise algorithm" (parallel
// form inside a chunk, state recurrence between chunks), "Mamba-2: input-
// dependent scalar decay" (chunkwise form: decayed query <-q, right-boundary
// key ->k, local decay matrix Gamma), "DeltaNet" (triangular correction system,
// "Optional: Use UT to share the triangular transform", "Correct the incoming
// state") and the GDN row of the chunkwise table.
//
// One workgroup owns one (batch, head, 64 value columns) and walks its chunks
// in order.  Per chunk r (positions l, m = 0..C-1, G = prefix sum of the
// log-gate, gamma_l = exp(G_l), rho_l = exp(G_{C-1} - G_l)):
//   a1  G, gamma, rho (one wave, shuffle scan)
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
// Eight waves in three roles, each running its own copy of the chunk loop (so
// the register allocation of one role does not burden another); all of them
// meet at the same two LDS barriers per chunk:
//   * state waves 0..3: wave w owns value columns 16w..16w+15 and keeps
//     S[:, those columns] (fp32) as dk/16 MFMA result tiles for the whole
//     sequence.  S, R and Z never leave registers: a result tile is directly a
//     K = 16 MFMA operand (mfma.h), so LDS only supplies Q, K, K^T, V, Aq, Tb.
//   * wave 4: the gate scan; for the delta rule the N blocks (kept in
//     registers) and the triangular transform.
//   * waves 5..7 (4..7 for the add rule): the Aq tiles, K^T (matrix-core
//     transpose) and the copy of the previous chunk's output to HBM.
// Schedule of one chunk (the next chunk's tokens are loaded into registers
// during the whole chunk):
//   P1  all: registers -> LDS; issue next chunk's loads; wave 4: gate scan
//   --- barrier
//   P2  state waves: R = V - gamma K S_r and the inter-chunk output gamma Q S_r
//       wave 4: N, then T and Tb                                    [delta]
//       waves 5..7: previous output to HBM, Aq tiles, K^T
//   --- barrier
//   P4  state waves: Z = Tb R, O = gamma Q S_r + Aq Z (to LDS), S_{r+1}
//       (the other waves go on with the next chunk's P1)
// Operands are bf16 (fp32 for fp32 tokens), accumulation is fp32; the state
// stays fp32 and is rounded to the operand type only as an operand.
#include "device_common.h"
#include "launch.h"
#include "mfma.h"
#include "tsolve.h"

namespace linattn {

namespace {

constexpr int kC = 64;      // chunk length
constexpr int kNW = 8;      // waves per workgroup
constexpr int kNT = kNW * kWave;
constexpr int kDVB = 64;    // value columns per workgroup (4 state waves x 16)
constexpr float kLog2e = 1.4426950408889634f;

template <typename T, int DK, int RULE, int GATE>
struct FusedCfg {
    static constexpr int PADE = 16 / sizeof(T);   // 16-byte row padding
    static constexpr int LDQ = DK + PADE;         // rows of length dk: Qs, Ks
    static constexpr int LDC = kC + PADE;         // rows of length C: KsT, Aq, Tb
    static constexpr int LDV = kDVB + PADE;       // rows of V
    static constexpr int LDN = kC + 4;            // fp32 rows of N / T
    static constexpr bool DELTA = RULE == kRuleDelta;
    static constexpr bool GATED = GATE == kGateScalar;
    static constexpr int ND = DK / 16, NL = kC / 16;
    static constexpr int E = 16 / sizeof(T);                 // elements per 16-byte load
    static constexpr int NQ = kC * DK / (E * kNT);           // Q/K vectors per thread
    static constexpr int NV = kC * kDVB / (E * kNT);         // V vectors per thread
    static constexpr int NPAIR = NL * (NL + 1) / 2;          // causal 16x16 tiles
    static_assert(NQ >= 1 && NV >= 1, "load split");
};

// (lj, mi) of the p-th causal tile, mi <= lj, row-major over lj
__device__ __forceinline__ void causal_pair(int p, int& lj, int& mi)
{
    lj = 0;
    while (p > lj) { p -= lj + 1; ++lj; }
    mi = p;
}

template <typename T, int DK, int RULE, int GATE>
__global__ __launch_bounds__(kNT, 1) void chunk_fused_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ g, const T* __restrict__ beta, const float* s0, T* __restrict__ o,
    float* s_final, int64_t Tlen, int DV, int nblocks)
{
    using Cfg = FusedCfg<T, DK, RULE, GATE>;
    constexpr int LDQ = Cfg::LDQ, LDC = Cfg::LDC, LDV = Cfg::LDV;
    constexpr bool DELTA = Cfg::DELTA, GATED = Cfg::GATED;
    constexpr int ND = Cfg::ND, NL = Cfg::NL, E = Cfg::E, NQ = Cfg::NQ, NV = Cfg::NV;
    constexpr int NK = DK / Mfma<T>::kStep;          // MFMA steps over the key dimension
    // waves kW0..7 share the Aq tiles, K^T and the output copy
    constexpr int kW0 = DELTA ? 5 : 4, kNIW = kNW - kW0;

    __shared__ __align__(16) T Qs[kC * LDQ];
    __shared__ __align__(16) T Ks[kC * LDQ];
    __shared__ __align__(16) T KsT[DK * LDC];
    __shared__ __align__(16) T Vs[kC * LDV];
    __shared__ __align__(16) T Aq[kC * LDC];
    __shared__ __align__(16) T Os[kC * LDV];
    __shared__ __align__(16) T Tb[DELTA ? kC * LDC : 8];
    // gate values alternate between two buffers: the state waves still read the
    // previous chunk's while wave 4 writes this chunk's
    __shared__ __align__(16) float Gsb[2][kC], gamb[2][kC], rhob[2][kC], betb[2][kC];

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

    const T* qh = q + bh * Tlen * DK;
    const T* kh = k + bh * Tlen * DK;
    const T* vh = v + bh * Tlen * DV + vb * kDVB;

    // causal blocks above the diagonal of Aq and Tb stay zero for the whole run
    for (int i = tid; i < kC * LDC; i += kNT) Aq[i] = from_f32<T>(0.f);
    if constexpr (DELTA)
        for (int i = tid; i < kC * LDC; i += kNT) Tb[i] = from_f32<T>(0.f);

    typedef __attribute__((__vector_size__(16))) int i4;
    const int64_t nchunks = (Tlen + kC - 1) / kC;

    // ---- P1 of every role: this thread's share of the chunk from registers
    // into LDS, then the next chunk's loads into the same registers.  Loads never
    // wait here: rows past the end read the last row (in bounds) and are zeroed
    // when staged.
    i4 qreg[NQ], kreg[NQ], vreg[NV];
    auto fetch = [&](int64_t t0) {
#pragma unroll
        for (int p = 0; p < NQ; ++p) {
            const int idx = (p * kNT + tid) * E;
            const int row = idx / DK, col = idx % DK;
            const int64_t tr = t0 + row < Tlen ? t0 + row : Tlen - 1;
            qreg[p] = *reinterpret_cast<const i4*>(qh + tr * DK + col);
            kreg[p] = *reinterpret_cast<const i4*>(kh + tr * DK + col);
        }
#pragma unroll
        for (int p = 0; p < NV; ++p) {
            const int idx = (p * kNT + tid) * E;
            const int row = idx / kDVB, col = idx % kDVB;
            const int64_t tr = t0 + row < Tlen ? t0 + row : Tlen - 1;
            vreg[p] = *reinterpret_cast<const i4*>(vh + tr * DV + col);
        }
    };
    auto stage = [&](int64_t t0) {
#pragma unroll
        for (int p = 0; p < NQ; ++p) {
            const int idx = (p * kNT + tid) * E;
            const int row = idx / DK, col = idx % DK;
            const bool ok = t0 + row < Tlen;
            *reinterpret_cast<i4*>(&Qs[row * LDQ + col]) = ok ? qreg[p] : i4{0, 0, 0, 0};
            *reinterpret_cast<i4*>(&Ks[row * LDQ + col]) = ok ? kreg[p] : i4{0, 0, 0, 0};
        }
#pragma unroll
        for (int p = 0; p < NV; ++p) {
            const int idx = (p * kNT + tid) * E;
            const int row = idx / kDVB, col = idx % kDVB;
            const bool ok = t0 + row < Tlen;
            *reinterpret_cast<i4*>(&Vs[row * LDV + col]) = ok ? vreg[p] : i4{0, 0, 0, 0};
        }
    };
    if (nchunks > 0) fetch(0);

    // The output of a chunk is staged in LDS (Os) by the state waves and written
    // to HBM by waves kW0..7 during the next chunk's P2, after that chunk's loads
    // were issued: loads and stores share one vector-memory counter, so a store
    // issued between a load and its wait would make the wait include the store.
    // Rows of 64 columns go out as full 16-byte vectors.
    auto copy_out = [&](int64_t tb, int cw, int ln) {
        constexpr int NCOPY = kC * kDVB / E, NROUND = (NCOPY + kNIW * kWave - 1) / (kNIW * kWave);
        T* oh = o + bh * Tlen * DV + vb * kDVB;
#pragma unroll
        for (int p = 0; p < NROUND; ++p) {
            const int idx = (p * kNIW + cw) * kWave + ln;
            if (idx < NCOPY) {
                const int row = idx / (kDVB / E), col = (idx % (kDVB / E)) * E;
                const int64_t l = tb + row;
                if (l < Tlen)
                    *reinterpret_cast<i4*>(oh + l * DV + col) = *reinterpret_cast<const i4*>(&Os[row * LDV + col]);
            }
        }
    };

    // a2 Aq tiles and K^T through the matrix core, shared by kNIW waves (iw-th)
    auto aq_kt = [&](const float* Gs, int iw, int ln) {
        const int cl = ln & 15, g4 = 4 * (ln >> 4);
        for (int p = iw; p < Cfg::NPAIR; p += kNIW) {
            int lj, mi;
            causal_pair(p, lj, mi);
            floatx4 xa = zero4();    // xa[rr] = k_m . q_l, m = 16 mi + g4 + rr, l = 16 lj + cl
            typename Mfma<T>::frag fa[NK], fq[NK];
#pragma unroll
            for (int i = 0; i < NK; ++i) {
                fa[i] = Mfma<T>::load(&Ks[mi * 16 * LDQ], LDQ, i * Mfma<T>::kStep, ln);
                fq[i] = Mfma<T>::load(&Qs[lj * 16 * LDQ], LDQ, i * Mfma<T>::kStep, ln);
            }
#pragma unroll
            for (int i = 0; i < NK; ++i) xa = Mfma<T>::mma(fa[i], fq[i], xa);
            const int l = lj * 16 + cl;
            const float Gl = Gs[l];
            floatx4 va;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int m = mi * 16 + g4 + rr;
                const float dec = GATED ? opaquef(fast_exp2(Gl - Gs[m])) : 1.f;
                va[rr] = (m <= l) ? xa[rr] * dec : 0.f;
            }
            store_tile_t(&Aq[lj * 16 * LDC + mi * 16], LDC, va, ln);
        }
        // all of this wave's transposes in flight, with separate accumulators
        constexpr int NKTT = NL * ND, NKT = (NKTT + kNIW - 1) / kNIW;
        typename Frag16<T>::type af[NKT];
#pragma unroll
        for (int i = 0; i < NKT; ++i) {
            const int t = iw + kNIW * i;
            if (t < NKTT) af[i] = frag16_lds(&Ks[(t / ND) * 16 * LDQ + (t % ND) * 16], LDQ, ln);
        }
        const auto id = ident_frag<T>(ln);
        floatx4 d[NKT];
#pragma unroll
        for (int i = 0; i < NKT; ++i)
            if (iw + kNIW * i < NKTT) d[i] = mma16<T>(af[i], id, zero4());
#pragma unroll
        for (int i = 0; i < NKT; ++i) {
            const int t = iw + kNIW * i;
            if (t < NKTT) store_tile_t(&KsT[(t % ND) * 16 * LDC + (t / ND) * 16], LDC, d[i], ln);
        }
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
        for (int64_t r = 0; r < nchunks; ++r) {
            const int64_t t0 = r * kC;
            // lane indices recomputed per chunk so the LDS addresses derived from
            // them are not held in registers across the loop
            const int ln = opaque(lane);
            const int cl = ln & 15, g4 = 4 * (ln >> 4);
            const float* const gam = gamb[r & 1];
            const float* const rho = rhob[r & 1];

            stage(t0);
            if (r + 1 < nchunks) fetch(t0 + kC);
            lds_barrier();

            // ---- P2: R = V - gamma K S_r (delta; V for add) ; O^T = (S_r^T Q^T) gamma
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
                for (int db = 0; db < ND; ++db) {
                    const auto sf = frag16_acc<T>(S[db]);
#pragma unroll
                    for (int li = 0; li < NL; ++li)
                        P[li] = mma16<T>(frag16_lds(&Ks[16 * li * LDQ + 16 * db], LDQ, ln), sf, P[li]);
                }
#pragma unroll
                for (int li = 0; li < NL; ++li)
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) R[li][rr] -= gam[16 * li + g4 + rr] * P[li][rr];
            }
#pragma unroll
            for (int li = 0; li < NL; ++li) Ot[li] = zero4();
#pragma unroll
            for (int db = 0; db < ND; ++db) {
                const auto sf = frag16_acc<T>(S[db]);
#pragma unroll
                for (int li = 0; li < NL; ++li)
                    Ot[li] = mma16<T>(sf, frag16_lds(&Qs[16 * li * LDQ + 16 * db], LDQ, ln), Ot[li]);
            }
#pragma unroll
            for (int li = 0; li < NL; ++li) {
                const float gl = gam[16 * li + cl];
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) Ot[li][rr] *= gl;
            }
            lds_barrier();

            // ---- P4: b1 Z = Tb R ; c1 O^T += Z^T Aq^T ; S_{r+1} -----------------------
            floatx4 Z[NL];
            if constexpr (DELTA) {
#pragma unroll
                for (int li = 0; li < NL; ++li) Z[li] = zero4();
#pragma unroll
                for (int mj = 0; mj < NL; ++mj) {
                    const auto rb = frag16_acc<T>(R[mj]);
#pragma unroll
                    for (int li = mj; li < NL; ++li)
                        Z[li] = mma16<T>(frag16_lds(&Tb[16 * li * LDC + 16 * mj], LDC, ln), rb, Z[li]);
                }
            } else {
#pragma unroll
                for (int li = 0; li < NL; ++li) Z[li] = R[li];
            }
#pragma unroll
            for (int mj = 0; mj < NL; ++mj) {
                const auto za = frag16_acc<T>(Z[mj]);
#pragma unroll
                for (int lj = mj; lj < NL; ++lj)
                    Ot[lj] = mma16<T>(za, frag16_lds(&Aq[16 * lj * LDC + 16 * mj], LDC, ln), Ot[lj]);
            }
            // O^T tile -> Os[token][column]
#pragma unroll
            for (int lj = 0; lj < NL; ++lj) store_tile_t(&Os[16 * lj * LDV + n0], LDV, Ot[lj], ln);
            // S_{r+1} = gamma_{C-1} S_r + K^T diag(rho) Z
            const float gC = gam[kC - 1];
#pragma unroll
            for (int db = 0; db < ND; ++db)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) S[db][rr] *= gC;
#pragma unroll
            for (int lj = 0; lj < NL; ++lj) {
                floatx4 zr = Z[lj];
                if constexpr (GATED) {
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) zr[rr] *= rho[16 * lj + g4 + rr];
                }
                const auto zb = frag16_acc<T>(zr);
#pragma unroll
                for (int db = 0; db < ND; ++db)
                    S[db] = mma16<T>(frag16_lds(&KsT[16 * db * LDC + 16 * lj], LDC, ln), zb, S[db]);
            }
        }
        if (s_final) {
            const int cl = lane & 15, g4 = 4 * (lane >> 4);
#pragma unroll
            for (int db = 0; db < ND; ++db)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr)
                    s_final[(bh * DK + 16 * db + g4 + rr) * DV + vb * kDVB + n0 + cl] = S[db][rr];
        }
    } else if (wave == 4) {
        // ======== wave 4: a1 gate scan; delta rule: a2 N blocks and a3/a4 T -------
        T greg = from_f32<T>(0.f), breg = from_f32<T>(0.f);
        auto fetch_gate = [&](int64_t t0) {
            const int64_t tr = t0 + lane < Tlen ? t0 + lane : Tlen - 1;
            if constexpr (GATED) greg = g[bh * Tlen + tr];
            if constexpr (DELTA) breg = beta[bh * Tlen + tr];
        };
        if (nchunks > 0) fetch_gate(0);
        for (int64_t r = 0; r < nchunks; ++r) {
            const int64_t t0 = r * kC;
            const int ln = opaque(lane);
            const int cl = ln & 15, g4 = 4 * (ln >> 4);
            float* const Gs = Gsb[r & 1];
            float* const bet = betb[r & 1];

            stage(t0);
            {
                // G is kept in base 2 (log2 e * prefix sum) so every decay factor
                // is one hardware exp2
                const bool ok = t0 + lane < Tlen;
                const float G = wave_prefix_sum((GATED && ok) ? to_f32(greg) * kLog2e : 0.f);
                const float Glast = wave_last(G);
                Gs[lane] = G;
                gamb[r & 1][lane] = GATED ? fast_exp2(G) : 1.f;
                rhob[r & 1][lane] = GATED ? fast_exp2(Glast - G) : 1.f;
                bet[lane] = (DELTA && ok) ? to_f32(breg) : 0.f;
            }
            if (r + 1 < nchunks) {
                fetch(t0 + kC);
                fetch_gate(t0 + kC);
            }
            lds_barrier();

            if constexpr (DELTA) {
                // ---- P2: N blocks in registers, then the triangular transform.
                // x = K_mi K_lj^T; as k_m . k_l is symmetric, one product gives a
                // diagonal block both as tile(N_bb^T) and as tile(N_bb).
                typename Mfma<T>::frag kf[NL][NK];
#pragma unroll
                for (int b = 0; b < NL; ++b)
#pragma unroll
                    for (int i = 0; i < NK; ++i) kf[b][i] = Mfma<T>::load(&Ks[16 * b * LDQ], LDQ, i * Mfma<T>::kStep, ln);
                // gate and beta of this lane's rows (16 b + g4 + rr) and column (16 b + cl)
                floatx4 Grow[NL], brow[NL];
                float Gcol[NL], bcol[NL];
#pragma unroll
                for (int b = 0; b < NL; ++b) {
                    Grow[b] = *reinterpret_cast<const floatx4*>(&Gs[16 * b + g4]);
                    brow[b] = *reinterpret_cast<const floatx4*>(&bet[16 * b + g4]);
                    Gcol[b] = Gs[16 * b + cl];
                    bcol[b] = bet[16 * b + cl];
                }
                floatx4 nd[NL], nt[NL], no[NL * (NL - 1) / 2];
#pragma unroll
                for (int lj = 0; lj < NL; ++lj) {
#pragma unroll
                    for (int mi = 0; mi <= lj; ++mi) {
                        floatx4 x = zero4();     // x[rr] = k_m . k_l, m = 16 mi + g4 + rr, l = 16 lj + cl
#pragma unroll
                        for (int i = 0; i < NK; ++i) x = Mfma<T>::mma(kf[mi][i], kf[lj][i], x);
                        floatx4 t;               // N[l][m]
#pragma unroll
                        for (int rr = 0; rr < 4; ++rr) {
                            const float dec = GATED ? fast_exp2(Gcol[lj] - Grow[mi][rr]) : 1.f;
                            t[rr] = (mi < lj || g4 + rr < cl) ? bcol[lj] * x[rr] * dec : 0.f;
                        }
                        if (mi == lj) {
                            floatx4 u;           // N[m][l]
#pragma unroll
                            for (int rr = 0; rr < 4; ++rr) {
                                const float dec = GATED ? fast_exp2(Grow[mi][rr] - Gcol[lj]) : 1.f;
                                u[rr] = (cl < g4 + rr) ? brow[mi][rr] * x[rr] * dec : 0.f;
                            }
                            nt[lj] = t;
                            nd[lj] = u;
                        } else {
                            no[lj * (lj - 1) / 2 + mi] = t;
                        }
                    }
                }
                tsolve64_regs<T>(nd, nt, no[0], no[1], no[2], no[3], no[4], no[5], Tb, LDC, brow, bcol, ln);
            } else {
                if (r > 0) copy_out(t0 - kC, 0, ln);
                aq_kt(Gs, 0, ln);
            }
            lds_barrier();
        }
    } else {
        // ======== waves kW0..7: output copy, a2 Aq tiles, K^T -----------------------
        const int iw = wave - kW0;
        for (int64_t r = 0; r < nchunks; ++r) {
            const int64_t t0 = r * kC;
            const int ln = opaque(lane);
            stage(t0);
            if (r + 1 < nchunks) fetch(t0 + kC);
            lds_barrier();
            if (r > 0) copy_out(t0 - kC, iw, ln);
            aq_kt(Gsb[r & 1], iw, ln);
            lds_barrier();
        }
    }

    // the last chunk's output, once every state wave has staged it
    __syncthreads();
    if (wave >= kW0 && nchunks > 0) copy_out((nchunks - 1) * kC, wave - kW0, lane);
}

template <typename T, int DK, int RULE, int GATE>
hipError_t launch_t(const ChunkProblem& p, hipStream_t s)
{
    const int nvb = p.dv / kDVB;
    const int64_t nblocks = p.B * p.H * nvb;
    hipLaunchKernelGGL((chunk_fused_kernel<T, DK, RULE, GATE>), dim3((unsigned)nblocks), dim3(kNT), 0,
                       s, static_cast<const T*>(p.q), static_cast<const T*>(p.k),
                       static_cast<const T*>(p.v), static_cast<const T*>(p.g),
                       static_cast<const T*>(p.beta), p.s0, static_cast<T*>(p.o), p.s_final, p.T,
                       p.dv, (int)nblocks);
    return hipGetLastError();
}

template <typename T, int DK>
hipError_t by_rule_gate(const ChunkProblem& p, hipStream_t s)
{
    if (p.rule == kRuleAdd)
        return p.gate == kGateNone ? launch_t<T, DK, kRuleAdd, kGateNone>(p, s)
                                   : launch_t<T, DK, kRuleAdd, kGateScalar>(p, s);
    return p.gate == kGateNone ? launch_t<T, DK, kRuleDelta, kGateNone>(p, s)
                               : launch_t<T, DK, kRuleDelta, kGateScalar>(p, s);
}

}  // namespace

bool chunk_fused_supported(const ChunkProblem& p)
{
    if (p.gate == kGateChannel || p.chunk != kC) return false;
    if (p.dtype == kBF16) return (p.dk == 64 || p.dk == 128) && (p.dv == 64 || p.dv == 128);
    return p.dk == 64 && (p.dv == 64 || p.dv == 128);
}

hipError_t launch_chunk_fused(const ChunkProblem& p, hipStream_t s)
{
    if (p.dtype == kBF16)
        return p.dk == 64 ? by_rule_gate<bf16, 64>(p, s) : by_rule_gate<bf16, 128>(p, s);
    return by_rule_gate<float, 64>(p, s);
}

}  // namespace linattn
