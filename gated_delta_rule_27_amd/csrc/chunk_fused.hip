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
// Eight waves in two roles:
//   * state waves 0..3: wave w owns value columns 16w..16w+15 and keeps
//     S[:, those columns] (fp32) as dk/16 MFMA result tiles for the whole
//     sequence.  S, R and Z never leave registers: a result tile is directly a
//     K = 16 MFMA operand (mfma.h), so LDS only supplies Q, K, K^T, V, Aq, Tb.
//   * intra waves 4..7: the gate scan (wave 4), K^T (matrix-core transpose),
//     the Aq and N tiles, and the triangular solve (wave 4).
// Schedule of one chunk (4 LDS barriers, 3 for the add rule; the next chunk's
// tokens are loaded into registers during the whole chunk):
//   P1  all: registers -> LDS; wave 4: gate scan; issue next chunk's loads
//   P2  state waves: R = V - gamma K S_r
//       intra waves: Aq and N tiles (sharing K fragments), K^T
//   P3  wave 4: the triangular solve                               [delta]
//   P4  state waves: Z = Tb R, O = gamma Q S_r + Aq Z (to HBM), S_{r+1}
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
    constexpr int LDQ = Cfg::LDQ, LDC = Cfg::LDC, LDV = Cfg::LDV, LDN = Cfg::LDN;
    constexpr bool DELTA = Cfg::DELTA, GATED = Cfg::GATED;
    constexpr int ND = Cfg::ND, NL = Cfg::NL, E = Cfg::E, NQ = Cfg::NQ, NV = Cfg::NV;

    __shared__ __align__(16) T Qs[kC * LDQ];
    __shared__ __align__(16) T Ks[kC * LDQ];
    __shared__ __align__(16) T KsT[DK * LDC];
    __shared__ __align__(16) T Vs[kC * LDV];
    __shared__ __align__(16) T Aq[kC * LDC];
    __shared__ __align__(16) float Nf[DELTA ? kC * LDN : 4];
    __shared__ __align__(16) T Tb[DELTA ? kC * LDC : 8];
    __shared__ float Gs[kC], gam[kC], rho[kC], bet[kC];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int cl = lane & 15, g4 = 4 * (lane >> 4);
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
    const bool state_wave = wave < 4;
    const int n0 = 16 * (state_wave ? wave : 0);        // this state wave's first column in the block

    // ---- state tiles S[16 db + g4 + rr][n0 + cl] (state waves only) ---------
    floatx4 S[ND];
#pragma unroll
    for (int db = 0; db < ND; ++db) {
        S[db] = zero4();
        if (state_wave && s0) {
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
                S[db][rr] = s0[(bh * DK + 16 * db + g4 + rr) * DV + vb * kDVB + n0 + cl];
        }
    }
    // causal blocks above the diagonal of Aq and Tb stay zero for the whole run
    for (int i = tid; i < kC * LDC; i += kNT) Aq[i] = from_f32<T>(0.f);
    if constexpr (DELTA)
        for (int i = tid; i < kC * LDC; i += kNT) Tb[i] = from_f32<T>(0.f);

    typedef __attribute__((__vector_size__(16))) int i4;
    const int64_t nchunks = (Tlen + kC - 1) / kC;

    // Next chunk's tokens travel in registers while the current chunk computes.
    // Loads never wait here: rows past the end read the last row (in bounds)
    // and are zeroed when stored, and the gate values stay raw until used.
    i4 qreg[NQ], kreg[NQ], vreg[NV];
    T greg = from_f32<T>(0.f), breg = from_f32<T>(0.f);
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
        if (wave == 4) {
            const int64_t tr = t0 + lane < Tlen ? t0 + lane : Tlen - 1;
            if constexpr (GATED) greg = g[bh * Tlen + tr];
            if constexpr (DELTA) breg = beta[bh * Tlen + tr];
        }
    };
    if (nchunks > 0) fetch(0);

    for (int64_t r = 0; r < nchunks; ++r) {
        const int64_t t0 = r * kC;
        lds_barrier();

        // ---- P1: the chunk into LDS; a1 gate scan; next chunk's loads --------
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
        if (wave == 4) {
            // G is kept in base 2 (log2 e * prefix sum) so every decay factor is
            // one hardware exp2
            const bool ok = t0 + lane < Tlen;
            float G = (GATED && ok) ? to_f32(greg) * kLog2e : 0.f;
#pragma unroll
            for (int off = 1; off < kWave; off <<= 1) {
                const float up = __shfl_up(G, off, kWave);
                if (lane >= off) G += up;
            }
            const float Glast = __shfl(G, kWave - 1, kWave);
            Gs[lane] = G;
            gam[lane] = GATED ? fast_exp2(G) : 1.f;
            rho[lane] = GATED ? fast_exp2(Glast - G) : 1.f;
            bet[lane] = (DELTA && ok) ? to_f32(breg) : 0.f;
        }
        if (r + 1 < nchunks) fetch(t0 + kC);
        lds_barrier();

        floatx4 R[NL];      // state waves: R (delta) or V (add)
        if (state_wave) {
            // ---- P2 (state waves): R = V - gamma K S_r ---------------------------
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
                    const auto sb = frag16_acc<T>(S[db]);
#pragma unroll
                    for (int li = 0; li < NL; ++li)
                        P[li] = mma16<T>(frag16_lds(&Ks[16 * li * LDQ + 16 * db], LDQ, lane), sb, P[li]);
                }
#pragma unroll
                for (int li = 0; li < NL; ++li)
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) R[li][rr] -= gam[16 * li + g4 + rr] * P[li][rr];
            }
        } else {
            // ---- P2 (intra waves): a2 for every causal (l-block, m-block) pair,
            // N and Aq together so the K fragments are read once; K^T --------------
            const int iw = wave - 4;
            for (int p = iw; p < Cfg::NPAIR; p += 4) {
                int lj, mi;
                causal_pair(p, lj, mi);
                // X[m][l] = k_m . q_l and k_m . k_l
                constexpr int NK = DK / Mfma<T>::kStep;
                floatx4 xa = zero4(), xn = zero4();
                typename Mfma<T>::frag fa[NK], fq[NK], fk[NK];
#pragma unroll
                for (int i = 0; i < NK; ++i) {
                    fa[i] = Mfma<T>::load(&Ks[mi * 16 * LDQ], LDQ, i * Mfma<T>::kStep, lane);
                    fq[i] = Mfma<T>::load(&Qs[lj * 16 * LDQ], LDQ, i * Mfma<T>::kStep, lane);
                    if constexpr (DELTA) fk[i] = Mfma<T>::load(&Ks[lj * 16 * LDQ], LDQ, i * Mfma<T>::kStep, lane);
                }
#pragma unroll
                for (int i = 0; i < NK; ++i) {
                    xa = Mfma<T>::mma(fa[i], fq[i], xa);
                    if constexpr (DELTA) xn = Mfma<T>::mma(fa[i], fk[i], xn);
                }
                const int l = lj * 16 + cl;
                const int m0 = mi * 16 + g4;
                const float Gl = Gs[l], bl = bet[l];
                floatx4 va, vn;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int m = m0 + rr;
                    const float dec = GATED ? fast_exp2(Gl - Gs[m]) : 1.f;
                    va[rr] = (m <= l) ? xa[rr] * dec : 0.f;
                    vn[rr] = (m < l) ? bl * xn[rr] * dec : 0.f;
                }
                store_tile_t(&Aq[lj * 16 * LDC + mi * 16], LDC, va, lane);
                if constexpr (DELTA) store_tile_t(&Nf[lj * 16 * LDN + mi * 16], LDN, vn, lane);
            }
            {
                // K^T through the matrix core, all of this wave's tiles in flight
                constexpr int NKT = NL * ND / 4;
                typename Frag16<T>::type af[NKT];
#pragma unroll
                for (int i = 0; i < NKT; ++i) {
                    const int t = iw + 4 * i;
                    af[i] = frag16_lds(&Ks[(t / ND) * 16 * LDQ + (t % ND) * 16], LDQ, lane);
                }
                const auto id = ident_frag<T>(lane);
                floatx4 d[NKT];     // separate accumulators, so the products overlap
#pragma unroll
                for (int i = 0; i < NKT; ++i) d[i] = mma16<T>(af[i], id, zero4());
#pragma unroll
                for (int i = 0; i < NKT; ++i) {
                    const int t = iw + 4 * i;
                    store_tile_t(&KsT[(t % ND) * 16 * LDC + (t / ND) * 16], LDC, d[i], lane);
                }
            }
        }
        lds_barrier();

        if constexpr (DELTA) {
            // ---- P3: a3/a4 triangular transform (wave 4) --------------------------
            if (wave == 4) tsolve64_wave<T>(Nf, LDN, Tb, LDC, bet, lane);
            lds_barrier();
        }

        if (state_wave) {
            // ---- P4: b1 Z = Tb R ; c1 O^T = (S_r^T Q^T) gamma + Z^T Aq^T ; S_{r+1} ----
            floatx4 Ot[NL];     // O^T tiles: rows = this wave's columns, columns = tokens
#pragma unroll
            for (int lj = 0; lj < NL; ++lj) Ot[lj] = zero4();
#pragma unroll
            for (int db = 0; db < ND; ++db) {
                const auto sa = frag16_acc<T>(S[db]);
#pragma unroll
                for (int lj = 0; lj < NL; ++lj)
                    Ot[lj] = mma16<T>(sa, frag16_lds(&Qs[16 * lj * LDQ + 16 * db], LDQ, lane), Ot[lj]);
            }
#pragma unroll
            for (int lj = 0; lj < NL; ++lj) {
                const float gl = gam[16 * lj + cl];
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) Ot[lj][rr] *= gl;
            }
            floatx4 Z[NL];
            if constexpr (DELTA) {
#pragma unroll
                for (int li = 0; li < NL; ++li) Z[li] = zero4();
#pragma unroll
                for (int mj = 0; mj < NL; ++mj) {
                    const auto rb = frag16_acc<T>(R[mj]);
#pragma unroll
                    for (int li = mj; li < NL; ++li)
                        Z[li] = mma16<T>(frag16_lds(&Tb[16 * li * LDC + 16 * mj], LDC, lane), rb, Z[li]);
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
                    Ot[lj] = mma16<T>(za, frag16_lds(&Aq[16 * lj * LDC + 16 * mj], LDC, lane), Ot[lj]);
            }
            T* oh = o + bh * Tlen * DV + vb * kDVB + n0 + g4;
#pragma unroll
            for (int lj = 0; lj < NL; ++lj) {
                const int64_t l = t0 + 16 * lj + cl;
                if (l < Tlen) {
                    if constexpr (sizeof(T) == 2) {
                        bf16x4 w;
#pragma unroll
                        for (int rr = 0; rr < 4; ++rr) w[rr] = from_f32<bf16>(Ot[lj][rr]);
                        *reinterpret_cast<bf16x4*>(oh + l * DV) = w;
                    } else {
                        *reinterpret_cast<floatx4*>(oh + l * DV) = Ot[lj];
                    }
                }
            }
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
                    S[db] = mma16<T>(frag16_lds(&KsT[16 * db * LDC + 16 * lj], LDC, lane), zb, S[db]);
            }
        }
    }

    // ---- final state -----------------------------------------------------------
    if (state_wave && s_final) {
#pragma unroll
        for (int db = 0; db < ND; ++db)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
                s_final[(bh * DK + 16 * db + g4 + rr) * DV + vb * kDVB + n0 + cl] = S[db][rr];
    }
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
