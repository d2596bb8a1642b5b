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
// One workgroup owns one (batch, head, dv-block) and walks its chunks in
// order, keeping the fp32 state block S (dk x DVB) in MFMA accumulators for the
// whole sequence.  Per chunk r (positions l, m = 0..C-1, G = prefix sum of the
// log-gate, gamma_l = exp(G_l), rho_l = exp(G_{C-1} - G_l)):
//   a1  G, gamma, rho (one wave, shuffle scan)
//   a2  Aq[l][m] = (q_l . k_m) exp(G_l - G_m)            (m <= l)
//       N [l][m] = beta_l (k_l . k_m) exp(G_l - G_m)     (m <  l)   [delta]
//   a3  T = (I + N)^-1 in fp32: 16x16 diagonal blocks by forward substitution,
//       off-diagonal blocks by two levels of block products     [delta]
//   a4  Tb = T diag(beta)                                       [delta]
//   b1  R = V - diag(gamma) K S_r ;  Z = Tb R                  [delta]
//       (Z = U - W S_r of the UT form, with U = Tb V and W = Tb <-K applied
//        to V - <-K S_r in one product; add rule: Z = V)
//       S_{r+1} = gamma_{C-1} S_r + K^T diag(rho) Z
//   c1  O = diag(gamma) Q S_r + Aq Z
// Operands are bf16 (fp32 for fp32 tokens) in LDS, accumulation is fp32; the
// state stays fp32 and is rounded to the operand type only as an operand.
//
// Schedule of one chunk (5 LDS barriers; the next chunk's tokens are loaded
// into registers during the whole chunk):
//   P1  registers -> LDS (Q, K, V), gate scan, issue next chunk's loads
//   P2  K^T, V^T (matrix-core transposes), Aq and N tiles
//   P3  wave 0: the whole triangular solve (no barrier inside);
//       waves 1..: R = V - gamma K S_r and the history part gamma Q S_r of O
//   P4  Z = Tb R
//   P5  O += Aq Z (to HBM), S_{r+1}
#include "device_common.h"
#include "launch.h"
#include "mfma.h"
#include "tsolve.h"

namespace linattn {

namespace {

constexpr int kC = 64;      // chunk length
constexpr int kNW = 8;      // waves per workgroup
constexpr int kNT = kNW * kWave;

template <typename T, int DK, int DVB, int RULE, int GATE>
struct FusedCfg {
    static constexpr int PADE = 16 / sizeof(T);   // 16-byte row padding
    static constexpr int LDQ = DK + PADE;         // rows of length dk: Qs, Ks, ST
    static constexpr int LDC = kC + PADE;         // rows of length C: KsT, VsT, Aq, Tb, RT, ZT
    static constexpr int LDN = kC + 4;            // fp32 rows of N / T
    static constexpr int LDV = DVB + PADE;        // row-major V staging
    static constexpr bool DELTA = RULE == kRuleDelta;
    static constexpr bool GATED = GATE == kGateScalar;
    static constexpr int NTS = (DK / 16) * (DVB / 16);       // state tiles
    static constexpr int NS = (NTS + kNW - 1) / kNW;         // state tiles per wave (max)
    static constexpr int NTO = (DVB / 16) * (kC / 16);       // output / R / Z tiles
    static constexpr int NOW = DELTA ? kNW - 1 : kNW;        // waves holding O tiles
    static constexpr int NO = (NTO + NOW - 1) / NOW;         // O tiles per wave (max)
    static constexpr int E = 16 / sizeof(T);                 // elements per 16-byte load
    static constexpr int NQ = kC * DK / (E * kNT);           // Q/K vectors per thread
    static constexpr int NV = (kC * DVB + E * kNT - 1) / (E * kNT);
    static constexpr int ZSZ = (DVB * LDC > kC * LDV) ? DVB * LDC : kC * LDV;
    static constexpr int NPAIR = (kC / 16) * (kC / 16 + 1) / 2;   // causal 16x16 tiles
    static_assert(NQ >= 1 && (kC * DK) % (E * kNT) == 0, "Q/K load split");
};

// (lj, mi) of the p-th causal tile, mi <= lj, row-major over lj
__device__ __forceinline__ void causal_pair(int p, int& lj, int& mi)
{
    lj = 0;
    while (p > lj) { p -= lj + 1; ++lj; }
    mi = p;
}

template <typename T, int DK, int DVB, int RULE, int GATE>
__global__ __launch_bounds__(kNT, 1) void chunk_fused_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ g, const T* __restrict__ beta, const float* s0, T* __restrict__ o,
    float* s_final, int64_t Tlen, int DV, int nblocks)
{
    using Cfg = FusedCfg<T, DK, DVB, RULE, GATE>;
    constexpr int LDQ = Cfg::LDQ, LDC = Cfg::LDC, LDN = Cfg::LDN, LDV = Cfg::LDV;
    constexpr bool DELTA = Cfg::DELTA, GATED = Cfg::GATED;
    constexpr int NS = Cfg::NS, NTS = Cfg::NTS, NTO = Cfg::NTO, NOW = Cfg::NOW, NO = Cfg::NO;
    constexpr int E = Cfg::E, NQ = Cfg::NQ, NV = Cfg::NV;
    constexpr int KS = Mfma<T>::kStep;

    __shared__ __align__(16) T Qs[kC * LDQ];
    __shared__ __align__(16) T Ks[kC * LDQ];
    __shared__ __align__(16) T KsT[DK * LDC];
    __shared__ __align__(16) T VsT[DVB * LDC];
    __shared__ __align__(16) T Aq[kC * LDC];
    __shared__ __align__(16) T ST[2][DVB * LDQ];
    __shared__ __align__(16) T ZT[Cfg::ZSZ];        // also stages V row-major
    __shared__ __align__(16) T ZrT[GATED ? DVB * LDC : 1];
    __shared__ __align__(16) float Nf[DELTA ? kC * LDN : 4];
    __shared__ __align__(16) T Tb[DELTA ? kC * LDC : 1];
    __shared__ __align__(16) T RT[DELTA ? DVB * LDC : 1];
    __shared__ float Gs[kC], gam[kC], rho[kC], bet[kC];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int nvb = DV / DVB;

    // Workgroups of one head land on the same XCD (dispatch is round-robin
    // over the 8 XCDs), so its dv-blocks share q/k reads in that XCD's L2.
    int blk = blockIdx.x;
    if ((nblocks & 7) == 0) blk = (blk & 7) * (nblocks >> 3) + (blk >> 3);
    const int64_t bh = blk / nvb;
    const int vb = blk % nvb;

    const T* qh = q + bh * Tlen * DK;
    const T* kh = k + bh * Tlen * DK;
    const T* vh = v + bh * Tlen * DV + vb * DVB;
    T* oh = o + bh * Tlen * DV + vb * DVB;

    // ---- initial state into accumulators and its operand copy --------------
    floatx4 sacc[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        const int t = wave + i * kNW;
        sacc[i] = zero4();
        if (NTS % kNW != 0 && t >= NTS) continue;
        const int di = t / (DVB / 16), nj = t % (DVB / 16);
        const int d = di * 16 + 4 * (lane >> 4), n = nj * 16 + (lane & 15);
#pragma unroll
        for (int r = 0; r < 4; ++r)
            sacc[i][r] = s0 ? s0[(bh * DK + d + r) * DV + vb * DVB + n] : 0.f;
        store_tile_t(&ST[0][nj * 16 * LDQ + di * 16], LDQ, sacc[i], lane);
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
            const int row = (idx / DVB) % kC, col = idx % DVB;
            const int64_t tr = t0 + row < Tlen ? t0 + row : Tlen - 1;
            vreg[p] = *reinterpret_cast<const i4*>(vh + tr * DV + col);
        }
        if (wave == 0) {
            const int64_t tr = t0 + lane < Tlen ? t0 + lane : Tlen - 1;
            if constexpr (GATED) greg = g[bh * Tlen + tr];
            if constexpr (DELTA) breg = beta[bh * Tlen + tr];
        }
    };
    if (nchunks > 0) fetch(0);

    for (int64_t r = 0; r < nchunks; ++r) {
        const int64_t t0 = r * kC;
        const int cur = (int)(r & 1);
        const T* STc = ST[cur];
        T* STn = ST[cur ^ 1];
        T* Vs = ZT;
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
            if (idx < kC * DVB) {
                const int row = idx / DVB, col = idx % DVB;
                const bool ok = t0 + row < Tlen;
                *reinterpret_cast<i4*>(&Vs[row * LDV + col]) = ok ? vreg[p] : i4{0, 0, 0, 0};
            }
        }
        if (wave == 0) {
            const bool ok = t0 + lane < Tlen;
            float G = ok ? to_f32(greg) : 0.f;
#pragma unroll
            for (int off = 1; off < kWave; off <<= 1) {
                const float up = __shfl_up(G, off, kWave);
                if (lane >= off) G += up;
            }
            const float Glast = __shfl(G, kWave - 1, kWave);
            Gs[lane] = G;
            gam[lane] = GATED ? expf(G) : 1.f;
            rho[lane] = GATED ? expf(Glast - G) : 1.f;
            bet[lane] = ok ? to_f32(breg) : 0.f;
        }
        if (r + 1 < nchunks) fetch(t0 + kC);
        lds_barrier();

        // ---- P2: K^T, V^T through the matrix core; a2 Aq and N tiles ---------
#pragma unroll
        for (int i = 0; i < (kC / 16) * (DK / 16) / kNW; ++i) {
            const int t = wave + i * kNW;
            const int li = t / (DK / 16), dj = t % (DK / 16);
            const floatx4 d = ident_tile(&Ks[li * 16 * LDQ + dj * 16], LDQ, lane);
            store_tile_t(&KsT[dj * 16 * LDC + li * 16], LDC, d, lane);
        }
#pragma unroll
        for (int i = 0; i < ((kC / 16) * (DVB / 16) + kNW - 1) / kNW; ++i) {
            const int t = wave + i * kNW;
            if (t < (kC / 16) * (DVB / 16)) {
                const int li = t / (DVB / 16), nj = t % (DVB / 16);
                const floatx4 d = ident_tile(&Vs[li * 16 * LDV + nj * 16], LDV, lane);
                store_tile_t(&VsT[nj * 16 * LDC + li * 16], LDC, d, lane);
            }
        }
        {
            constexpr int NPROD = Cfg::NPAIR * (DELTA ? 2 : 1);
            constexpr int NPW = (NPROD + kNW - 1) / kNW;
            floatx4 acc[NPW];
            int plj[NPW], pmi[NPW];
#pragma unroll
            for (int i = 0; i < NPW; ++i) {
                const int c = wave + i * kNW;
                const int which = c % (DELTA ? 2 : 1);
                causal_pair(c / (DELTA ? 2 : 1), plj[i], pmi[i]);
                acc[i] = zero4();
                if (c < NPROD) {
                    // X[m][l] = k_m . (q_l | k_l)
                    const T* Bop = which == 0 ? &Qs[plj[i] * 16 * LDQ] : &Ks[plj[i] * 16 * LDQ];
                    acc[i] = mma_nt_k<T, DK>(zero4(), &Ks[pmi[i] * 16 * LDQ], LDQ, Bop, LDQ, lane);
                }
            }
#pragma unroll
            for (int i = 0; i < NPW; ++i) {
                const int c = wave + i * kNW;
                if (c >= NPROD) continue;
                const int which = c % (DELTA ? 2 : 1);
                const int l = plj[i] * 16 + (lane & 15);
                const int m0 = pmi[i] * 16 + 4 * (lane >> 4);
                const float Gl = Gs[l];
                floatx4 val;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int m = m0 + rr;
                    const float dec = GATED ? expf(Gl - Gs[m]) : 1.f;
                    if (which == 0) val[rr] = (m <= l) ? acc[i][rr] * dec : 0.f;
                    else val[rr] = (m < l) ? bet[l] * acc[i][rr] * dec : 0.f;
                }
                if (which == 0) store_tile_t(&Aq[plj[i] * 16 * LDC + pmi[i] * 16], LDC, val, lane);
                else store_tile_t(&Nf[plj[i] * 16 * LDN + pmi[i] * 16], LDN, val, lane);
            }
        }
        lds_barrier();

        // ---- P3: triangular solve (wave 0) || R and gamma Q S_r (others) ------
        floatx4 oacc[NO];
#pragma unroll
        for (int i = 0; i < NO; ++i) oacc[i] = zero4();
        const int ow = DELTA ? wave - 1 : wave;     // index among the O-tile waves
        if (DELTA && wave == 0) {
            // a3/a4 (see tsolve.h)
            tsolve64_wave<T>(Nf, LDN, Tb, LDC, bet, lane);
        } else {
            if constexpr (DELTA) {
                // b1: R = V - diag(gamma) K S_r  ->  R^T  (tiles spread over waves 1..)
                constexpr int NR = (NTO + kNW - 2) / (kNW - 1);
                floatx4 racc[NR];
#pragma unroll
                for (int i = 0; i < NR; ++i) {
                    const int t = (wave - 1) + i * (kNW - 1);
                    racc[i] = zero4();
                    if (t < NTO) {
                        const int li = t / (DVB / 16), nj = t % (DVB / 16);
                        racc[i] = mma_nt_k<T, DK>(zero4(), &Ks[li * 16 * LDQ], LDQ,
                                                  &STc[nj * 16 * LDQ], LDQ, lane);
                    }
                }
#pragma unroll
                for (int i = 0; i < NR; ++i) {
                    const int t = (wave - 1) + i * (kNW - 1);
                    if (t >= NTO) continue;
                    const int li = t / (DVB / 16), nj = t % (DVB / 16);
                    const int l0 = li * 16 + 4 * (lane >> 4), n = nj * 16 + (lane & 15);
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr)
                        racc[i][rr] = to_f32(VsT[n * LDC + l0 + rr]) - gam[l0 + rr] * racc[i][rr];
                    store_tile_t(&RT[nj * 16 * LDC + li * 16], LDC, racc[i], lane);
                }
            }
            // c1 (history part): O^T tile = (S_r^T Q^T) diag(gamma), kept in registers
#pragma unroll
            for (int i = 0; i < NO; ++i) {
                const int t = ow + i * NOW;
                if (t < NTO) {
                    const int nj = t / (kC / 16), lj = t % (kC / 16);
                    oacc[i] = mma_nt_k<T, DK>(zero4(), &STc[nj * 16 * LDQ], LDQ,
                                              &Qs[lj * 16 * LDQ], LDQ, lane);
                    const float gl = gam[lj * 16 + (lane & 15)];
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) oacc[i][rr] *= gl;
                }
            }
        }
        if constexpr (!DELTA && GATED) {
            // add rule: Z = V, the state update takes (rho V)^T
            for (int i = tid; i < DVB * kC; i += kNT) {
                const int n = i / kC, l = i % kC;
                ZrT[n * LDC + l] = from_f32<T>(to_f32(VsT[n * LDC + l]) * rho[l]);
            }
        }
        lds_barrier();

        if constexpr (DELTA) {
            // ---- P4: Z = Tb R  ->  Z^T and (rho Z)^T ------------------------------
            constexpr int NZ = (NTO + kNW - 1) / kNW;
            floatx4 zacc[NZ];
#pragma unroll
            for (int i = 0; i < NZ; ++i) {
                const int t = wave + i * kNW;
                zacc[i] = zero4();
                if (t < NTO) {
                    const int li = t / (DVB / 16), nj = t % (DVB / 16);
                    const int nk = (li * 16 + 16 + KS - 1) / KS;
                    zacc[i] = mma_nt_k<T, kC>(zero4(), &Tb[li * 16 * LDC], LDC, &RT[nj * 16 * LDC],
                                              LDC, lane, nk);
                }
            }
#pragma unroll
            for (int i = 0; i < NZ; ++i) {
                const int t = wave + i * kNW;
                if (t >= NTO) continue;
                const int li = t / (DVB / 16), nj = t % (DVB / 16);
                store_tile_t(&ZT[nj * 16 * LDC + li * 16], LDC, zacc[i], lane);
                if constexpr (GATED) {
                    const int l0 = li * 16 + 4 * (lane >> 4);
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) zacc[i][rr] *= rho[l0 + rr];
                    store_tile_t(&ZrT[nj * 16 * LDC + li * 16], LDC, zacc[i], lane);
                }
            }
            lds_barrier();
        }
        const T* ZTs = DELTA ? ZT : VsT;
        const T* ZrTs = GATED ? ZrT : ZTs;

        // ---- P5: c1 O^T += Z^T Aq^T, written to HBM; b1 S_{r+1} ---------------
        if (!DELTA || wave > 0) {
#pragma unroll
            for (int i = 0; i < NO; ++i) {
                const int t = ow + i * NOW;
                if (t >= NTO) continue;
                const int nj = t / (kC / 16), lj = t % (kC / 16);
                const int nk = (lj * 16 + 16 + KS - 1) / KS;
                oacc[i] = mma_nt_k<T, kC>(oacc[i], &ZTs[nj * 16 * LDC], LDC, &Aq[lj * 16 * LDC], LDC,
                                          lane, nk);
                const int l = lj * 16 + (lane & 15);
                if (t0 + l < Tlen) {
                    T* dst = oh + (t0 + l) * DV + nj * 16 + 4 * (lane >> 4);
                    if constexpr (sizeof(T) == 2) {
                        bf16x4 w;
#pragma unroll
                        for (int rr = 0; rr < 4; ++rr) w[rr] = from_f32<bf16>(oacc[i][rr]);
                        *reinterpret_cast<bf16x4*>(dst) = w;
                    } else {
                        *reinterpret_cast<floatx4*>(dst) = oacc[i];
                    }
                }
            }
        }
        const float gC = gam[kC - 1];
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            const int t = wave + i * kNW;
            if (NTS % kNW != 0 && t >= NTS) continue;
            const int di = t / (DVB / 16), nj = t % (DVB / 16);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) sacc[i][rr] *= gC;
            sacc[i] = mma_nt_k<T, kC>(sacc[i], &KsT[di * 16 * LDC], LDC, &ZrTs[nj * 16 * LDC], LDC, lane);
        }
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            const int t = wave + i * kNW;
            if (NTS % kNW != 0 && t >= NTS) continue;
            const int di = t / (DVB / 16), nj = t % (DVB / 16);
            store_tile_t(&STn[nj * 16 * LDQ + di * 16], LDQ, sacc[i], lane);
        }
    }

    // ---- final state -----------------------------------------------------------
    if (s_final) {
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            const int t = wave + i * kNW;
            if (NTS % kNW != 0 && t >= NTS) continue;
            const int di = t / (DVB / 16), nj = t % (DVB / 16);
            const int d = di * 16 + 4 * (lane >> 4), n = nj * 16 + (lane & 15);
#pragma unroll
            for (int r = 0; r < 4; ++r) s_final[(bh * DK + d + r) * DV + vb * DVB + n] = sacc[i][r];
        }
    }
}

template <typename T> constexpr int dv_block() { return sizeof(T) == 2 ? 64 : 16; }

template <typename T, int DK, int RULE, int GATE>
hipError_t launch_t(const ChunkProblem& p, hipStream_t s)
{
    constexpr int DVB = dv_block<T>();
    const int nvb = p.dv / DVB;
    const int64_t nblocks = p.B * p.H * nvb;
    hipLaunchKernelGGL((chunk_fused_kernel<T, DK, DVB, RULE, GATE>), dim3((unsigned)nblocks),
                       dim3(kNT), 0, s, static_cast<const T*>(p.q), static_cast<const T*>(p.k),
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
