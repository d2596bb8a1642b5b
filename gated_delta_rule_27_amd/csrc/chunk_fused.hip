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
#include "device_common.h"
#include "launch.h"
#include "mfma.h"

namespace linattn {

namespace {

constexpr int kC = 64;      // chunk length
constexpr int kNW = 4;      // waves per workgroup
constexpr int kNT = kNW * kWave;

template <typename T, int DK, int DVB, int RULE, int GATE>
struct FusedCfg {
    static constexpr int PADE = 16 / sizeof(T);   // 16-byte row padding
    static constexpr int LDQ = DK + PADE;         // rows of length dk: Qs, Ks, ST
    static constexpr int LDC = kC + PADE;         // rows of length C: KsT, VsT, Aq, Tb, RT, ZT
    static constexpr int LDN = kC + 4;            // fp32 rows of N / T
    static constexpr bool DELTA = RULE == kRuleDelta;
    static constexpr bool GATED = GATE == kGateScalar;
    static constexpr int NS = (DK / 16) * (DVB / 16) / kNW;   // state tiles per wave
    static_assert((DK / 16) * (DVB / 16) % kNW == 0, "state tiles per wave");
};

template <typename T, int DK, int DVB, int RULE, int GATE>
__global__ __launch_bounds__(kNT, 1) void chunk_fused_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ g, const T* __restrict__ beta, const float* s0, T* __restrict__ o,
    float* s_final, int64_t Tlen, int DV, int nblocks)
{
    using Cfg = FusedCfg<T, DK, DVB, RULE, GATE>;
    constexpr int LDQ = Cfg::LDQ, LDC = Cfg::LDC, LDN = Cfg::LDN;
    constexpr bool DELTA = Cfg::DELTA, GATED = Cfg::GATED;
    constexpr int NS = Cfg::NS;
    constexpr int E = 16 / sizeof(T);            // elements per 16-byte load

    __shared__ __align__(16) T Qs[kC * LDQ];
    __shared__ __align__(16) T Ks[kC * LDQ];
    __shared__ __align__(16) T KsT[DK * LDC];
    __shared__ __align__(16) T VsT[DVB * LDC];
    __shared__ __align__(16) T Aq[kC * LDC];
    __shared__ __align__(16) T ST[2][DVB * LDQ];
    __shared__ __align__(16) T ZT[DVB * LDC];
    __shared__ __align__(16) T ZrT[GATED ? DVB * LDC : 1];
    __shared__ __align__(16) float Nf[DELTA ? kC * LDN : 4];
    __shared__ __align__(16) T Tb[DELTA ? kC * LDC : 1];
    __shared__ float Gs[kC], gam[kC], rho[kC], bet[kC];

    T* RT = reinterpret_cast<T*>(Nf);            // R^T reuses N's space after the solve
    T* ZrTp = GATED ? ZrT : ZT;                  // no gate: rho == 1

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
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

    const int64_t nchunks = (Tlen + kC - 1) / kC;
    for (int64_t r = 0; r < nchunks; ++r) {
        const int64_t t0 = r * kC;
        const int cur = (int)(r & 1);
        const T* STc = ST[cur];
        T* STn = ST[cur ^ 1];
        __syncthreads();

        // ---- load the chunk: Q, K row-major and K^T, V^T (zero past the end)
#pragma unroll
        for (int p = 0; p < kC * DK / (E * kNT); ++p) {
            const int idx = (p * kNT + tid) * E;
            const int row = idx / DK, col = idx % DK;
            typedef __attribute__((__vector_size__(16))) int i4;
            i4 qv = {0, 0, 0, 0}, kv = {0, 0, 0, 0};
            if (t0 + row < Tlen) {
                qv = *reinterpret_cast<const i4*>(qh + (t0 + row) * DK + col);
                kv = *reinterpret_cast<const i4*>(kh + (t0 + row) * DK + col);
            }
            *reinterpret_cast<i4*>(&Qs[row * LDQ + col]) = qv;
            *reinterpret_cast<i4*>(&Ks[row * LDQ + col]) = kv;
            const T* ke = reinterpret_cast<const T*>(&kv);
#pragma unroll
            for (int e = 0; e < E; ++e) KsT[(col + e) * LDC + row] = ke[e];
        }
#pragma unroll
        for (int p = 0; p < kC * DVB / (E * kNT); ++p) {
            const int idx = (p * kNT + tid) * E;
            const int row = idx / DVB, col = idx % DVB;
            typedef __attribute__((__vector_size__(16))) int i4;
            i4 vv = {0, 0, 0, 0};
            if (t0 + row < Tlen) vv = *reinterpret_cast<const i4*>(vh + (t0 + row) * DV + col);
            const T* ve = reinterpret_cast<const T*>(&vv);
#pragma unroll
            for (int e = 0; e < E; ++e) VsT[(col + e) * LDC + row] = ve[e];
        }
        // ---- a1: gate prefix sums and boundary factors (wave 0) -------------
        if (wave == 0) {
            const bool valid = t0 + lane < Tlen;
            float gl = 0.f, bl = 0.f;
            if constexpr (GATED) gl = valid ? to_f32(g[bh * Tlen + t0 + lane]) : 0.f;
            if constexpr (DELTA) bl = valid ? to_f32(beta[bh * Tlen + t0 + lane]) : 0.f;
            float G = gl;
#pragma unroll
            for (int off = 1; off < kWave; off <<= 1) {
                const float up = __shfl_up(G, off, kWave);
                if (lane >= off) G += up;
            }
            const float Glast = __shfl(G, kWave - 1, kWave);
            Gs[lane] = G;
            gam[lane] = GATED ? expf(G) : 1.f;
            rho[lane] = GATED ? expf(Glast - G) : 1.f;
            bet[lane] = bl;
        }
        __syncthreads();

        // ---- a2: Aq (and N) tiles on the causal lower half -------------------
        {
            int cnt = 0;
#pragma unroll
            for (int lj = 0; lj < kC / 16; ++lj) {
#pragma unroll
                for (int mi = 0; mi <= lj; ++mi) {
#pragma unroll
                    for (int which = 0; which < (DELTA ? 2 : 1); ++which, ++cnt) {
                        if (cnt % kNW != wave) continue;
                        // X[m][l] = k_m . (q_l | k_l)
                        const T* Bop = which == 0 ? &Qs[lj * 16 * LDQ] : &Ks[lj * 16 * LDQ];
                        floatx4 acc = mma_nt(zero4(), &Ks[mi * 16 * LDQ], LDQ, Bop, LDQ, 0, DK, lane);
                        const int l = lj * 16 + (lane & 15);
                        const int m0 = mi * 16 + 4 * (lane >> 4);
                        const float Gl = Gs[l];
                        floatx4 val;
#pragma unroll
                        for (int rr = 0; rr < 4; ++rr) {
                            const int m = m0 + rr;
                            const float dec = GATED ? expf(Gl - Gs[m]) : 1.f;
                            if (which == 0) val[rr] = (m <= l) ? acc[rr] * dec : 0.f;
                            else val[rr] = (m < l) ? bet[l] * acc[rr] * dec : 0.f;
                        }
                        if (which == 0) store_tile_t(&Aq[lj * 16 * LDC + mi * 16], LDC, val, lane);
                        else store_tile_t(&Nf[lj * 16 * LDN + mi * 16], LDN, val, lane);
                    }
                }
            }
        }
        __syncthreads();

        if constexpr (DELTA) {
            // ---- a3/a4: T = (I + N)^-1, Tb = T diag(beta) -----------------------
            // diagonal 16x16 blocks: wave w inverts block w, lane c < 16 owns column c
            {
                const int w = wave;
                float* Nb = &Nf[(w * 16) * LDN + w * 16];
                if (lane < 16) {
                    const int c = lane;
                    float x[16];
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        float acc = (i == c) ? 1.f : 0.f;
#pragma unroll
                        for (int j = 0; j < i; ++j) acc = fmaf(-Nb[i * LDN + j], x[j], acc);
                        x[i] = acc;
                    }
                    const float bc = bet[w * 16 + c];
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        Nb[i * LDN + c] = x[i];
                        Tb[(w * 16 + i) * LDC + w * 16 + c] = from_f32<T>(x[i] * bc);
                    }
                }
            }
            __syncthreads();
            // level 1: T10 = -X11 N10 X00 (wave 0), T32 = -X33 N32 X22 (wave 1)
            if (wave < 2) {
                const int i = 2 * wave + 1, j = 2 * wave;
                const floatx4 xjj = load_tile_rl(&Nf[j * 16 * LDN + j * 16], LDN, lane);
                const floatx4 y = mm16<T>(&Nf[i * 16 * LDN + j * 16], LDN, xjj, zero4(), lane);
                floatx4 t = mm16<T>(&Nf[i * 16 * LDN + i * 16], LDN, y, zero4(), lane);
                const int row = i * 16 + 4 * (lane >> 4), col = j * 16 + (lane & 15);
                const float bc = bet[col];
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    t[rr] = -t[rr];
                    Nf[(row + rr) * LDN + col] = t[rr];
                    Tb[(row + rr) * LDC + col] = from_f32<T>(t[rr] * bc);
                }
            }
            __syncthreads();
            // level 2: the lower-left 32x32 block, T_BA = -T_B N_BA T_A.
            // wave qc handles column block qc of it (qc = 0, 1).
            if (wave < 2) {
                const int qc = wave;
                // Y_p = sum_s N[2+p][s] T_A[s][qc], s = qc..1   (p = 0, 1)
                floatx4 y[2];
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    y[p] = zero4();
#pragma unroll
                    for (int s = 0; s < 2; ++s) {
                        if (s < qc) continue;
                        const floatx4 tb = load_tile_rl(&Nf[s * 16 * LDN + qc * 16], LDN, lane);
                        y[p] = mm16<T>(&Nf[(2 + p) * 16 * LDN + s * 16], LDN, tb, y[p], lane);
                    }
                }
                // T[2][qc] = -X22 Y_0 ; T[3][qc] = -(T32 Y_0 + X33 Y_1)
                floatx4 t2 = mm16<T>(&Nf[2 * 16 * LDN + 2 * 16], LDN, y[0], zero4(), lane);
                floatx4 t3 = mm16<T>(&Nf[3 * 16 * LDN + 2 * 16], LDN, y[0], zero4(), lane);
                t3 = mm16<T>(&Nf[3 * 16 * LDN + 3 * 16], LDN, y[1], t3, lane);
                const int col = qc * 16 + (lane & 15);
                const float bc = bet[col];
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int row = 4 * (lane >> 4) + rr;
                    Tb[(32 + row) * LDC + col] = from_f32<T>(-t2[rr] * bc);
                    Tb[(48 + row) * LDC + col] = from_f32<T>(-t3[rr] * bc);
                }
            }
            __syncthreads();

            // ---- b1: R = V - diag(gamma) K S_r  ->  R^T ---------------------------
#pragma unroll
            for (int t = wave; t < (kC / 16) * (DVB / 16); t += kNW) {
                const int li = t / (DVB / 16), nj = t % (DVB / 16);
                floatx4 acc = mma_nt(zero4(), &Ks[li * 16 * LDQ], LDQ, &STc[nj * 16 * LDQ], LDQ, 0, DK, lane);
                const int l0 = li * 16 + 4 * (lane >> 4), n = nj * 16 + (lane & 15);
#pragma unroll
                for (int rr = 0; rr < 4; ++rr)
                    acc[rr] = to_f32(VsT[n * LDC + l0 + rr]) - gam[l0 + rr] * acc[rr];
                store_tile_t(&RT[nj * 16 * LDC + li * 16], LDC, acc, lane);
            }
            __syncthreads();
            // ---- b1: Z = Tb R  ->  Z^T and (rho Z)^T -------------------------------
#pragma unroll
            for (int t = wave; t < (kC / 16) * (DVB / 16); t += kNW) {
                const int li = t / (DVB / 16), nj = t % (DVB / 16);
                const int ke = ((li * 16 + 16 + Mfma<T>::kStep - 1) / Mfma<T>::kStep) * Mfma<T>::kStep;
                floatx4 acc = mma_nt(zero4(), &Tb[li * 16 * LDC], LDC, &RT[nj * 16 * LDC], LDC, 0,
                                     ke < kC ? ke : kC, lane);
                store_tile_t(&ZT[nj * 16 * LDC + li * 16], LDC, acc, lane);
                if constexpr (GATED) {
                    const int l0 = li * 16 + 4 * (lane >> 4);
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) acc[rr] *= rho[l0 + rr];
                    store_tile_t(&ZrT[nj * 16 * LDC + li * 16], LDC, acc, lane);
                }
            }
            __syncthreads();
        } else {
            // add rule: Z = V (Z^T is V^T); the gated copy carries rho
            if constexpr (GATED) {
                for (int i = tid; i < DVB * kC; i += kNT) {
                    const int n = i / kC, l = i % kC;
                    ZrT[n * LDC + l] = from_f32<T>(to_f32(VsT[n * LDC + l]) * rho[l]);
                }
            }
            __syncthreads();
        }
        const T* ZTs = DELTA ? ZT : VsT;
        const T* ZrTs = DELTA ? ZrTp : (GATED ? ZrT : VsT);

        // ---- c1: O^T = (S_r^T Q^T) diag(gamma) + Z^T Aq^T, written to HBM -------
#pragma unroll
        for (int t = wave; t < (DVB / 16) * (kC / 16); t += kNW) {
            const int nj = t / (kC / 16), lj = t % (kC / 16);
            floatx4 acc = mma_nt(zero4(), &STc[nj * 16 * LDQ], LDQ, &Qs[lj * 16 * LDQ], LDQ, 0, DK, lane);
            const int l = lj * 16 + (lane & 15);
            const float gl = gam[l];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) acc[rr] *= gl;
            const int ke = ((lj * 16 + 16 + Mfma<T>::kStep - 1) / Mfma<T>::kStep) * Mfma<T>::kStep;
            acc = mma_nt(acc, &ZTs[nj * 16 * LDC], LDC, &Aq[lj * 16 * LDC], LDC, 0, ke < kC ? ke : kC, lane);
            if (t0 + l < Tlen) {
                T* dst = oh + (t0 + l) * DV + nj * 16 + 4 * (lane >> 4);
                if constexpr (sizeof(T) == 2) {
                    bf16x4 w;
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) w[rr] = from_f32<bf16>(acc[rr]);
                    *reinterpret_cast<bf16x4*>(dst) = w;
                } else {
                    *reinterpret_cast<floatx4*>(dst) = acc;
                }
            }
        }
        // ---- b1: S_{r+1} = gamma_{C-1} S_r + K^T diag(rho) Z ----------------------
        const float gC = gam[kC - 1];
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            const int t = wave + i * kNW;
            const int di = t / (DVB / 16), nj = t % (DVB / 16);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) sacc[i][rr] *= gC;
            sacc[i] = mma_nt(sacc[i], &KsT[di * 16 * LDC], LDC, &ZrTs[nj * 16 * LDC], LDC, 0, kC, lane);
            store_tile_t(&STn[nj * 16 * LDQ + di * 16], LDQ, sacc[i], lane);
        }
    }

    // ---- final state -----------------------------------------------------------
    if (s_final) {
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            const int t = wave + i * kNW;
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
