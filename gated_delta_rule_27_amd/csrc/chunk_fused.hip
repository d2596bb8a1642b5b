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
// in order (add rule with fewer such workgroups than compute units: one
// segment of the chunks, see seg_split).  Per chunk r (positions l, m = 0..C-1, G = prefix sum of the
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
// meet at the same LDS barriers, three per chunk for the delta rule and two for
// the add rule:
//   * state waves 0..3: wave w owns value columns 16w..16w+15 and keeps
//     S[:, those columns] (fp32) as dk/16 MFMA result tiles for the whole
//     sequence.  S, R and Z never leave registers: a result tile is directly a
//     K = 16 MFMA operand (mfma.h), and two of them make one K = 32 operand, so
//     LDS only supplies Q, K, K^T, V, Aq, Tb.
//   * wave 4: the gate scan; for the delta rule the diagonal N blocks (in
//     registers) and the triangular transform.
//   * waves 5..7, delta rule: the N blocks below the diagonal and the copy of
//     the previous chunk's output to HBM; waves 4..7, add rule: the Aq tiles
//     and that copy.
// Schedule of one chunk, delta rule (the next chunk's tokens are loaded into
// registers during the whole chunk):
//   P1   all: registers -> LDS; issue next chunk's loads; wave 4: gate scan
//   ---  barrier
//   P2a  state waves: R = V - gamma K S_r, Aq tiles, K^T by matrix-core
//        transposes; wave 4: diagonal N blocks, their inverses, diagonal
//        blocks of Tb; waves 5..7: N blocks below the diagonal (to LDS)
//   ---  barrier
//   P2b  state waves: gamma Q S_r; wave 4: off-diagonal blocks of Tb;
//        waves 6, 7: previous chunk's output to HBM
//   ---  barrier
//   P4   state waves: Z = Tb R, O = gamma Q S_r + Aq Z (to LDS), S_{r+1}
//        (the other waves go on with the next chunk's P1)
// Add rule, two barriers:
//   P1   all: registers -> LDS; issue next chunk's loads; wave 4: gate scan
//   ---  barrier
//   P2   state waves: R = V, gamma Q S_r, K^T; waves 4..7: Aq tiles
//   ---  barrier
//   P4   state waves: O = gamma Q S_r + Aq V (to one of two LDS buffers),
//        S_{r+1}; waves 4..7: previous chunk's output to HBM, then the next
//        chunk's P1
// Operands are bf16 (fp32 for fp32 tokens), accumulation is fp32; the state
// stays fp32 and is rounded to the operand type only as an operand.
#include "device_common.h"
#include "launch.h"
#include "mfma.h"
#include "prep.h"
#include "segments.h"
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
    static_assert(NQ >= 1 && NV >= 1, "load split");
};

// the E = 16 / sizeof(T) elements of a 16-byte vector, as floats and back
template <typename T, typename V>
__device__ __forceinline__ void vec_f32(V x, float (&f)[16 / sizeof(T)])
{
    T e[16 / sizeof(T)];
    __builtin_memcpy(e, &x, 16);
#pragma unroll
    for (int j = 0; j < 16 / (int)sizeof(T); ++j) f[j] = to_f32(e[j]);
}
template <typename T, typename V>
__device__ __forceinline__ V f32_vec(const float (&f)[16 / sizeof(T)])
{
    T e[16 / sizeof(T)];
#pragma unroll
    for (int j = 0; j < 16 / (int)sizeof(T); ++j) e[j] = from_f32<T>(f[j]);
    V x;
    __builtin_memcpy(&x, e, 16);
    return x;
}

// Qs, Ks, KsT, Aq and Tb hold their columns in swizzled pcol order (mfma.h)
// for 2-byte tokens and in plain pcol order for fp32; every access goes
// through these, which pick the matching form.
template <typename T>
constexpr int kTilePc = sizeof(T) == 2 ? 2 : 1;
template <typename T>
__device__ __forceinline__ int tile_sw(int row)
{
    return sizeof(T) == 2 ? swz_x(row) : 0;
}
template <typename T>
__device__ __forceinline__ typename Pair<T>::type tile_pair(const T* M, int ld, int lane)
{
    if constexpr (sizeof(T) == 2) return pair_lds_sw(M, ld, lane);
    else return pair_lds(M, ld, lane);
}
template <typename T>
__device__ __forceinline__ typename Mfma<T>::frag tile_load(const T* row0, int ld, int k0, int lane)
{
    if constexpr (sizeof(T) == 2) return mfma_load_sw(row0, ld, k0, lane);
    else return Mfma<T>::load(row0, ld, k0, lane);
}
template <typename T>
__device__ __forceinline__ typename Frag16<T>::type tile_frag16(const T* M, int ld, int kb, int lane)
{
    if constexpr (sizeof(T) == 2) return frag16_lds_pc_sw(M, ld, kb, lane);
    else return frag16_lds_pc(M, ld, kb, lane);
}
template <typename T>
__device__ __forceinline__ void tile_store_t(T* M, int ld, int kb, floatx4 v, int lane)
{
    if constexpr (sizeof(T) == 2) store_tile_t_pc_sw(M, ld, kb, v, lane);
    else store_tile_t_pc(M, ld, kb, v, lane);
}

// SAVE: also write the state entering every chunk, states[b,h,r] = S_r
// ([dk][dv] per chunk, rounded to the token type once), for the backward pass.
// NORM (add rule): normalised linear attention ("All sorts of famous Attention
// Layers", "Linear Magic" and its normaliser) in the same pass.  The key sum
// z_t = a_t z_{t-1} + k_t is one more state, a d_k vector; per chunk, with the
// notation below,
//   den_l   = gamma_l (q_l . z_r) + sum_m Aq[l][m]
//   z_{r+1} = gamma_{C-1} z_r + sum_m rho_m k_m
// and each output row leaves multiplied by 1 / den_l.  The state waves carry
// z as one more value column: gamma_l (q_l . z_r) beside their Q S_r products
// (phase P2a), z_{r+1} beside their state update (P4), each wave a quarter of
// z's key blocks, with rho as that column of Z; in the next chunk's P1, while
// the state waves finish this chunk, waves 4..7 each add the Aq row sums of
// one 16-row block.
template <typename T, int DK, int RULE, int GATE, bool SAVE = false, bool NORM = false>
__global__ __launch_bounds__(kNT, 1) void chunk_fused_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ g, const T* __restrict__ beta, const float* s0, T* __restrict__ o,
    float* s_final, T* __restrict__ states, int64_t Tlen, int DV, int nblocks, int prep,
    const float* z0, float* z_final, SegSplit seg)
{
    static_assert(!NORM || RULE == kRuleAdd, "the normaliser belongs to the add rule");
    using Cfg = FusedCfg<T, DK, RULE, GATE>;
    using F = typename Frag16<T>::type;
    constexpr int LDQ = Cfg::LDQ, LDC = Cfg::LDC, LDV = Cfg::LDV;
    constexpr bool DELTA = Cfg::DELTA, GATED = Cfg::GATED;
    constexpr int ND = Cfg::ND, NL = Cfg::NL, E = Cfg::E, NQ = Cfg::NQ, NV = Cfg::NV;
    constexpr int NK = DK / Mfma<T>::kStep;          // MFMA steps over the key dimension
    // waves kW0..7 share the output copy (add rule: also the Aq tiles)
    constexpr int kW0 = DELTA ? 6 : 4, kNIW = kNW - kW0;

    __shared__ __align__(16) T Qs[kC * LDQ];
    __shared__ __align__(16) T Ks[kC * LDQ];
    __shared__ __align__(16) T KsT[DK * LDC];
    __shared__ __align__(16) T Vs[kC * LDV];
    __shared__ __align__(16) T Aq[kC * LDC];
    // output of a chunk, staged for the copy to HBM; the add rule alternates two
    // buffers (its copy runs beside the next chunk's staging)
    __shared__ __align__(16) T Os[DELTA ? 1 : 2][kC * LDV];
    __shared__ __align__(16) T Tb[DELTA ? kC * LDC : 8];
    // the six N blocks below the diagonal as row fragments, lane by lane, and the
    // X tiles the two halves of the off-diagonal transform need from the other
    // waves: X11^T (wave 5), X22 and X22^T (wave 6), X33^T (wave 7)
    __shared__ __align__(16) floatx4 Nlo[DELTA ? 6 * kWave : 1];
    __shared__ __align__(16) floatx4 Xx[DELTA ? 4 * kWave : 1];
    // gate values alternate between two buffers: the state waves still read the
    // previous chunk's while wave 4 writes this chunk's
    __shared__ __align__(16) float Gsb[2][kC], gamb[2][kC], rhob[2][kC], betb[2][kC];
    // NORM: z_r and z_{r+1}, gamma_l (q_l . z_r), and the reciprocal
    // denominators of two chunks (the one formed, the one copied out)
    __shared__ __align__(16) float zSb[2][NORM ? DK : 4], denb[2][NORM ? kC : 4], qzs[2][NORM ? kC : 4];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int nvb = DV / kDVB;

    // Workgroups of one head land on the same XCD (dispatch is round-robin
    // over the 8 XCDs), so its value blocks share q/k reads in that XCD's L2.
    int blk = blockIdx.x;
    if ((nblocks & 7) == 0) blk = (blk & 7) * (nblocks >> 3) + (blk >> 3);
    const int nunit = nvb * seg.n;
    const int64_t bh = blk / nunit;
    const int vb = (blk % nunit) % nvb;
    const int sg = (blk % nunit) / nvb;
    // this workgroup's chunks [rb, re); the add rule's later segments first form
    // the state entering chunk rb from the chunks before it (prefix pass below)
    const int64_t rb = DELTA ? 0 : seg.c[sg], re = DELTA ? (Tlen + kC - 1) / kC : seg.c[sg + 1];
    const bool last_seg = DELTA || sg == seg.n - 1;

    const T* qh = q + bh * Tlen * DK;
    const T* kh = k + bh * Tlen * DK;
    const T* vh = v + bh * Tlen * DV + vb * kDVB;

    // causal blocks above the diagonal of Aq and Tb stay zero for the whole run
    for (int i = tid; i < kC * LDC; i += kNT) Aq[i] = from_f32<T>(0.f);
    if constexpr (DELTA)
        for (int i = tid; i < kC * LDC; i += kNT) Tb[i] = from_f32<T>(0.f);

    typedef __attribute__((__vector_size__(16))) int i4;
    const int64_t nchunks = (Tlen + kC - 1) / kC;
    if constexpr (NORM)
        for (int i = tid; i < DK; i += kNT) zSb[0][i] = z0 ? z0[bh * DK + i] : 0.f;

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
    // Q and K rows go to LDS with their columns in (swizzled) pcol order, 8
    // bytes (four columns) at a time for bf16; at dk = 128 the threads of the
    // second 64 columns of a row write their upper four columns first, so each
    // 16-lane group of a write covers 32 distinct banks.  Raw projections first
    // go through the q/k map of prep.h, and rows past the end are zeroed after it
    auto stage = [&](int64_t t0) {
        const int qk_map = prep_qk_map(prep);
#pragma unroll
        for (int p = 0; p < NQ; ++p) {
            const int idx = (p * kNT + tid) * E;
            const int row = idx / DK, col = idx % DK;
            const bool ok = t0 + row < Tlen;
            // every lane maps its vector (the L2 norm is reduced across lanes)
            const i4 qp = prep_qk<T, DK / E>(qreg[p], qk_map);
            const i4 kp = prep_qk<T, DK / E>(kreg[p], qk_map);
            const i4 qv = ok ? qp : i4{0, 0, 0, 0};
            const i4 kv = ok ? kp : i4{0, 0, 0, 0};
            if constexpr (E == 8) {
                typedef __attribute__((__vector_size__(8))) int i2;
                const int sw = tile_sw<T>(row);
                const bool hi = DK == 128 && (col & 64);
                const int c0 = row * LDQ + (pcol(col + (hi ? 4 : 0)) ^ sw);
                const int c1 = row * LDQ + (pcol(col + (hi ? 0 : 4)) ^ sw);
                *reinterpret_cast<i2*>(&Qs[c0]) = hi ? i2{qv[2], qv[3]} : i2{qv[0], qv[1]};
                *reinterpret_cast<i2*>(&Ks[c0]) = hi ? i2{kv[2], kv[3]} : i2{kv[0], kv[1]};
                *reinterpret_cast<i2*>(&Qs[c1]) = hi ? i2{qv[0], qv[1]} : i2{qv[2], qv[3]};
                *reinterpret_cast<i2*>(&Ks[c1]) = hi ? i2{kv[0], kv[1]} : i2{kv[2], kv[3]};
            } else {
                *reinterpret_cast<i4*>(&Qs[row * LDQ + pcol(col)]) = qv;
                *reinterpret_cast<i4*>(&Ks[row * LDQ + pcol(col)]) = kv;
            }
        }
#pragma unroll
        for (int p = 0; p < NV; ++p) {
            const int idx = (p * kNT + tid) * E;
            const int row = idx / kDVB, col = idx % kDVB;
            const bool ok = t0 + row < Tlen;
            *reinterpret_cast<i4*>(&Vs[row * LDV + col]) = ok ? vreg[p] : i4{0, 0, 0, 0};
        }
    };
    // Prefix pass (later segments of the add rule): K and V only, loaded two
    // chunks ahead into two register sets (kreg, vreg and qreg, vreg2), since
    // its chunks take far less time than one load's latency.  Loads are
    // unconditional (chunk index clamped), as in the main loop.
    i4 vreg2[NV];
    auto fetch_kv = [&](int64_t t0, i4 (&kr)[NQ], i4 (&vr)[NV]) {
#pragma unroll
        for (int p = 0; p < NQ; ++p) {
            const int idx = (p * kNT + tid) * E;
            const int row = idx / DK, col = idx % DK;
            const int64_t tr = t0 + row < Tlen ? t0 + row : Tlen - 1;
            kr[p] = *reinterpret_cast<const i4*>(kh + tr * DK + col);
        }
#pragma unroll
        for (int p = 0; p < NV; ++p) {
            const int idx = (p * kNT + tid) * E;
            const int row = idx / kDVB, col = idx % kDVB;
            const int64_t tr = t0 + row < Tlen ? t0 + row : Tlen - 1;
            vr[p] = *reinterpret_cast<const i4*>(vh + tr * DV + col);
        }
    };
    auto stage_kv = [&](int64_t t0, const i4 (&kr)[NQ], const i4 (&vr)[NV]) {
        const int qk_map = prep_qk_map(prep);
#pragma unroll
        for (int p = 0; p < NQ; ++p) {
            const int idx = (p * kNT + tid) * E;
            const int row = idx / DK, col = idx % DK;
            const bool ok = t0 + row < Tlen;
            const i4 kp = prep_qk<T, DK / E>(kr[p], qk_map);
            const i4 kv = ok ? kp : i4{0, 0, 0, 0};
            if constexpr (E == 8) {
                typedef __attribute__((__vector_size__(8))) int i2;
                const int sw = tile_sw<T>(row);
                const bool hi = DK == 128 && (col & 64);
                const int c0 = row * LDQ + (pcol(col + (hi ? 4 : 0)) ^ sw);
                const int c1 = row * LDQ + (pcol(col + (hi ? 0 : 4)) ^ sw);
                *reinterpret_cast<i2*>(&Ks[c0]) = hi ? i2{kv[2], kv[3]} : i2{kv[0], kv[1]};
                *reinterpret_cast<i2*>(&Ks[c1]) = hi ? i2{kv[0], kv[1]} : i2{kv[2], kv[3]};
            } else {
                *reinterpret_cast<i4*>(&Ks[row * LDQ + pcol(col)]) = kv;
            }
        }
#pragma unroll
        for (int p = 0; p < NV; ++p) {
            const int idx = (p * kNT + tid) * E;
            const int row = idx / kDVB, col = idx % kDVB;
            const bool ok = t0 + row < Tlen;
            *reinterpret_cast<i4*>(&Vs[row * LDV + col]) = ok ? vr[p] : i4{0, 0, 0, 0};
        }
    };
    // prefix chunk r: stage it from its register set and refill the set with
    // chunk r + 2 (clamped to the last prefix chunk)
    auto prefix_stage = [&](int64_t r, i4 (&kr)[NQ], i4 (&vr)[NV]) {
        stage_kv(r * kC, kr, vr);
        fetch_kv((r + 2 < rb ? r + 2 : rb - 1) * kC, kr, vr);
    };
    if (rb > 0) {
        fetch_kv(0, kreg, vreg);
        fetch_kv(rb > 1 ? kC : 0, qreg, vreg2);
    } else if (re > 0) {
        fetch(0);
    }

    // The output of a chunk is staged in LDS (Os) by the state waves and written
    // to HBM by waves kW0..7 during the next chunk, after that chunk's loads were
    // issued: loads and stores share one vector-memory counter, so a store issued
    // between a load and its wait would make the wait include the store.  Rows of
    // 64 columns go out as full 16-byte vectors.
    // The stores go through a buffer resource over this head's rows: rows past
    // the end (and the spare lanes of the last round) fall outside it and the
    // hardware drops them, so no branch hides a store from the compiler's wait
    // counts (the next chunk's loads are likewise issued unconditionally).
    const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
        o + bh * Tlen * DV, (short)0, (int)(Tlen * DV * (int64_t)sizeof(T)), 0x00020000);
    auto copy_out = [&](int64_t tb, int cw, int ln) {
        constexpr int NCOPY = kC * kDVB / E, NROUND = (NCOPY + kNIW * kWave - 1) / (kNIW * kWave);
#pragma unroll
        for (int p = 0; p < NROUND; ++p) {
            const int idx = (p * kNIW + cw) * kWave + ln;
            const int row = idx / (kDVB / E), col = (idx % (kDVB / E)) * E;
            const int off = idx < NCOPY ? (int)(((tb + row) * DV + vb * kDVB + col) * (int64_t)sizeof(T))
                                        : 0x7fffffff;
            const int ro = idx < NCOPY ? row : 0;
            i4 x = *reinterpret_cast<const i4*>(&Os[DELTA ? 0 : (int)(tb / kC) & 1][ro * LDV + col]);
            if constexpr (NORM) {
                const float rd = denb[(int)(tb / kC) & 1][ro];   // 1 / den
                float f[E];
                vec_f32<T>(x, f);
#pragma unroll
                for (int j = 0; j < E; ++j) f[j] *= rd;
                x = f32_vec<T, i4>(f);
            }
            __builtin_amdgcn_raw_buffer_store_b128(x, orsrc, off, 0, 0);
        }
    };
    const int64_t tlast = (re - 1) * kC;          // start of the segment's last chunk
    // All matrix-core fragments (every k step) of the 16-row block b of a [C][DK]
    // tile (Qs or Ks); a wave loads each block it needs once per chunk and forms
    // its tiles from the registers.
    using Fr = typename Mfma<T>::frag;
    auto block_frags = [&](const T* A, int b, int ln, Fr (&f)[NK]) {
#pragma unroll
        for (int i = 0; i < NK; ++i) f[i] = tile_load(&A[b * 16 * LDQ], LDQ, i * Mfma<T>::kStep, ln);
    };
    // x[rr] = sum_c A[16 mi + g4 + rr][c] B[16 lj + cl][c] from the blocks' fragments
    auto tile_dot = [&](const Fr (&fa)[NK], const Fr (&fb)[NK]) {
        floatx4 x = zero4();
#pragma unroll
        for (int i = 0; i < NK; ++i) x = Mfma<T>::mma(fa[i], fb[i], x);
        return x;
    };
    // ---- NORM.  z is kept in natural key order; Qs columns, and the token
    // columns of KsT and Aq, are stored in pcol order (swizzled for 2-byte
    // tokens, which the fragment loads undo), so position s of a fragment holds
    // logical column pcol_first(s & ~7) + (s & 4 ? 16 : 0) + (s & 3).
    // Matrix-core right factor: a 16-row block whose row 0 is x (logical
    // order, at the fragment's stored positions; x == nullptr: all ones) and
    // whose other rows are zero, so lanes 0, 16, 32, 48 (result column 0)
    // receive the products with x.  The loads are unconditional (in bounds for
    // every lane) and the selection follows, so no lane mask guards them.
    auto row0_frag = [&](const float* x, int k0, int ln) {
        const bool r0 = (ln & 15) == 0;
        if constexpr (sizeof(T) == 4) {
            const int sp = k0 + (ln >> 4);
            const float xv = x ? x[pcol_first(sp & ~7) + ((sp & 4) ? 16 : 0) + (sp & 3)] : 1.f;
            return r0 ? xv : 0.f;
        } else {
            float f[E];
            if (x) {
                const int c0 = pcol_first(k0 + E * (ln >> 4));
                const floatx4 a = *reinterpret_cast<const floatx4*>(&x[c0]);
                const floatx4 b = *reinterpret_cast<const floatx4*>(&x[c0 + 16]);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    f[j] = r0 ? a[j] : 0.f;
                    f[j + 4] = r0 ? b[j] : 0.f;
                }
            } else {
#pragma unroll
                for (int j = 0; j < E; ++j) f[j] = r0 ? 1.f : 0.f;
            }
            return f32_vec<T, Fr>(f);
        }
    };
    // Waves 4..7 (part = wave - 4) once chunk rp's state pass is under way
    // (Aq and qz of chunk rp stay in place until the next chunk's P2a):
    // 1 / den for row block part.
    auto norm_tail = [&](int64_t rp, int part, int ln) {
        constexpr int kS = Mfma<T>::kStep, NA = kC / kS;
        const int cl = ln & 15, g4 = 4 * (ln >> 4);
        const Fr f1 = row0_frag(nullptr, 0, ln);
        floatx4 xa = zero4();
#pragma unroll
        for (int i = 0; i < NA; ++i) xa = Mfma<T>::mma(tile_load(&Aq[part * 16 * LDC], LDC, i * kS, ln), f1, xa);
        if (cl == 0) {
            const floatx4 qz = *reinterpret_cast<const floatx4*>(&qzs[rp & 1][16 * part + g4]);
            floatx4 d;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) d[rr] = 1.f / (qz[rr] + xa[rr]);
            *reinterpret_cast<floatx4*>(&denb[rp & 1][16 * part + g4]) = d;
        }
    };
    // a2 Aq tile (lj, mi), mi <= lj, from xa[rr] = k_m . q_l:
    // Aq[l][m] = (q_l . k_m) exp(G_l - G_m), m <= l
    auto aq_store = [&](const float* Gs, int lj, int mi, floatx4 xa, int ln) {
        const int cl = ln & 15, g4 = 4 * (ln >> 4);
        const float Gl = Gs[lj * 16 + cl];
        const floatx4 Gm = *reinterpret_cast<const floatx4*>(&Gs[mi * 16 + g4]);
        floatx4 va;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const float dec = GATED ? fast_exp2(Gl - Gm[rr]) : 1.f;
            va[rr] = (mi < lj || g4 + rr <= cl) ? xa[rr] * dec : 0.f;
        }
        tile_store_t(&Aq[lj * 16 * LDC], LDC, mi, va, ln);
    };
    // add rule: the ten causal Aq tiles (lj, mi) on waves 4..7, grouped by query
    // block so each wave loads three or four blocks once:
    // (3,0) (3,1) | (3,2) (3,3) | (2,0) (2,1) (2,2) | (0,0) (1,0) (1,1)
    auto aq_add = [&](const float* Gs, int iw, int ln) {
        Fr fq[NK], fk[NK];
        if (iw < 2) {
            block_frags(Qs, 3, ln, fq);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                block_frags(Ks, 2 * iw + j, ln, fk);
                aq_store(Gs, 3, 2 * iw + j, tile_dot(fk, fq), ln);
            }
        } else if (iw == 2) {
            block_frags(Qs, 2, ln, fq);
#pragma unroll
            for (int mi = 0; mi < 3; ++mi) {
                block_frags(Ks, mi, ln, fk);
                aq_store(Gs, 2, mi, tile_dot(fk, fq), ln);
            }
        } else {
            block_frags(Ks, 0, ln, fk);
            block_frags(Qs, 0, ln, fq);
            aq_store(Gs, 0, 0, tile_dot(fk, fq), ln);
            block_frags(Qs, 1, ln, fq);
            aq_store(Gs, 1, 0, tile_dot(fk, fq), ln);
            block_frags(Ks, 1, ln, fk);
            aq_store(Gs, 1, 1, tile_dot(fk, fq), ln);
        }
    };

    // a2 diagonal N block b in registers.  x = K_b K_b^T is symmetric, so one
    // product gives N_bb both as tile(N_bb^T) (lane value N[l][m], l = 16 b + cl)
    // and as tile(N_bb); at most one of the two is nonzero at each position, so
    // one exp2 serves both.  br[rr] = beta[16 b + g4 + rr]; kb returns K_b's
    // fragments for the wave's other tiles.
    auto diag_block = [&](const float* Gs, const float* bet, int b, int ln, floatx4& nd, floatx4& nt,
                          floatx4& br, Fr (&kb)[NK]) {
        const int cl = ln & 15, g4 = 4 * (ln >> 4);
        block_frags(Ks, b, ln, kb);
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
    // delta rule, P2a of intra wave b = wave - 4: diagonal block b and its
    // inverse, the wave's N blocks below the diagonal, and the X tiles the two
    // off-diagonal halves need from it.  Returns X_bb and X_bb^T.
    auto intra_p2a = [&](const float* Gs, const float* bet, int b, int ln, floatx4& X, floatx4& Xt) {
        floatx4 nd[1], nt[1], br[1], Xa[1], Xta[1];
        Fr kb[NK], k2[NK];
        diag_block(Gs, bet, b, ln, nd[0], nt[0], br[0], kb);
        tsolve_diag<T, kTilePc<T>, 1>(nd, nt, Xa, Xta, Tb, LDC, br, ln, b);
        X = Xa[0];
        Xt = Xta[0];
        if (b == 0) {                                  // N(1,0)
            block_frags(Ks, 1, ln, k2);
            n_block(Gs, bet, 1, 0, kb, k2, ln);
        } else if (b == 1) {                           // N(2,1); X11^T
            block_frags(Ks, 2, ln, k2);
            n_block(Gs, bet, 2, 1, kb, k2, ln);
            Xx[0 * kWave + ln] = Xt;
        } else if (b == 2) {                           // N(3,2), N(2,0); X22, X22^T
            block_frags(Ks, 3, ln, k2);
            n_block(Gs, bet, 3, 2, kb, k2, ln);
            block_frags(Ks, 0, ln, k2);
            n_block(Gs, bet, 2, 0, k2, kb, ln);
            Xx[1 * kWave + ln] = X;
            Xx[2 * kWave + ln] = Xt;
        } else {                                       // N(3,0), N(3,1); X33^T
            block_frags(Ks, 0, ln, k2);
            n_block(Gs, bet, 3, 0, k2, kb, ln);
            block_frags(Ks, 1, ln, k2);
            n_block(Gs, bet, 3, 1, k2, kb, ln);
            Xx[3 * kWave + ln] = Xt;
        }
    };

    // K^T through the matrix core: tiles iw, iw + NW, ... of the NL x ND tiles
    // of Ks (transposed into KsT) for wave iw of NW
    auto kt_share = [&](auto nwc, int iw, int ln) {
        constexpr int NW = decltype(nwc)::value, NKT = NL * ND / NW;
        F af[NKT];
#pragma unroll
        for (int i = 0; i < NKT; ++i) {
            const int t = iw + NW * i;
            af[i] = tile_frag16(&Ks[(t / ND) * 16 * LDQ], LDQ, t % ND, ln);
        }
        const F id = ident_frag<T>(ln);
        floatx4 d[NKT];
#pragma unroll
        for (int i = 0; i < NKT; ++i) d[i] = mma16<T>(af[i], id, zero4());
#pragma unroll
        for (int i = 0; i < NKT; ++i) {
            const int t = iw + NW * i;
            tile_store_t(&KsT[(t % ND) * 16 * LDC], LDC, t / ND, d[i], ln);
        }
    };
    // b1 of state wave w: S_{r+1} = gamma_{C-1} S_r + K^T diag(rho) Z (NORM: and
    // z_{r+1} for the wave's quarter of the key blocks)
    auto state_update = [&](floatx4 (&S)[ND], const floatx4 (&Z)[NL], const float* gam, const float* rho,
                            int64_t r, int ln) {
        const int cl = ln & 15, g4 = 4 * (ln >> 4);
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
            S[db] = mma_pair<T>(tile_pair(&KsT[16 * db * LDC + 32], LDC, ln), zr23,
                                mma_pair<T>(tile_pair(&KsT[16 * db * LDC], LDC, ln), zr01, S[db]));
        }
        if constexpr (NORM) {
            // z_{r+1} = gamma_{C-1} z_r + K^T rho for this wave's key blocks: rho
            // as value column 0 of Z, z as value column 0 of the state (lanes
            // with cl = 0 hold and store it)
            floatx4 rz[NL];
#pragma unroll
            for (int lj = 0; lj < NL; ++lj) {
                const floatx4 rh = *reinterpret_cast<const floatx4*>(&rho[16 * lj + g4]);
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) rz[lj][rr] = cl == 0 ? rh[rr] : 0.f;
            }
            const auto rz01 = pair_regs<T>(rz[0], rz[1]), rz23 = pair_regs<T>(rz[2], rz[3]);
#pragma unroll
            for (int d2 = 0; d2 < ND / 4; ++d2) {
                const int db = (ND / 4) * wave + d2;
                floatx4 zt = *reinterpret_cast<const floatx4*>(&zSb[r & 1][16 * db + g4]);
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) zt[rr] *= gC;
                zt = mma_pair<T>(tile_pair(&KsT[16 * db * LDC + 32], LDC, ln), rz23,
                                 mma_pair<T>(tile_pair(&KsT[16 * db * LDC], LDC, ln), rz01, zt));
                if (cl == 0) *reinterpret_cast<floatx4*>(&zSb[(r + 1) & 1][16 * db + g4]) = zt;
            }
        }
    };
    // Prefix pass, per chunk r < rb: K and V to LDS (wave 4: the gate scan) and
    // the next loads; K^T on all eight waves, the state waves also take their V
    // columns into registers; then the state waves update S while the others
    // stage the next chunk.  Two barriers per chunk; the other waves' part:
    auto prefix_other = [&](int ln) {
        lds_barrier();
        kt_share(IntC<kNW>{}, wave, ln);
        lds_barrier();
    };

    // The lane index each role's chunk loop derives its LDS addresses from:
    // the addresses stay in registers across chunks, except with the delta
    // rule's state saving at dk = 128, whose registers are full (an opaque copy
    // per chunk makes the compiler recompute them instead of spilling).
    auto lane_id = [&]() {
        if constexpr (DELTA && SAVE && DK == 128) return opaque(lane);
        else return lane;
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
        if constexpr (!DELTA) {
            auto pchunk = [&](int64_t r, i4 (&kr)[NQ], i4 (&vr)[NV]) {
                const int ln = lane_id();
                const int cl = ln & 15, g4 = 4 * (ln >> 4);
                prefix_stage(r, kr, vr);
                lds_barrier();
                kt_share(IntC<kNW>{}, wave, ln);
                floatx4 Zv[NL];
#pragma unroll
                for (int li = 0; li < NL; ++li)
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) Zv[li][rr] = to_f32(Vs[(16 * li + g4 + rr) * LDV + n0 + cl]);
                lds_barrier();
                state_update(S, Zv, gamb[r & 1], rhob[r & 1], r, ln);
            };
            for (int64_t r = 0; r < rb; r += 2) {
                pchunk(r, kreg, vreg);
                if (r + 1 < rb) pchunk(r + 1, qreg, vreg2);
            }
            if (rb > 0) fetch(rb * kC);
        }
        for (int64_t r = rb; r < re; ++r) {
            const int64_t t0 = r * kC;
            const int ln = lane_id();
            const int cl = ln & 15, g4 = 4 * (ln >> 4);
            const float* const gam = gamb[r & 1];
            const float* const rho = rhob[r & 1];

            stage(t0);
            fetch(t0 + kC < tlast ? t0 + kC : tlast);
            if constexpr (SAVE) {
                T* sr = states + ((bh * nchunks + r) * DK) * DV + vb * kDVB + n0 + cl;
#pragma unroll
                for (int db = 0; db < ND; ++db)
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) sr[(16 * db + g4 + rr) * DV] = from_f32<T>(S[db][rr]);
            }
            lds_barrier();

            // ---- P2a: R = V - gamma K S_r (delta; V for add) --------------------------
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
                        P[li] = mma_pair<T>(tile_pair(&Ks[16 * li * LDQ + 16 * db], LDQ, ln), sp, P[li]);
                }
#pragma unroll
                for (int li = 0; li < NL; ++li) {
                    const floatx4 gr = *reinterpret_cast<const floatx4*>(&gam[16 * li + g4]);
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) R[li][rr] -= gr[rr] * P[li][rr];
                }
            }
            // O^T = (S_r^T Q^T) gamma: here for the add rule, after the barrier for
            // the delta rule (whose P2a is longer elsewhere)
            auto ohist = [&]() {
#pragma unroll
                for (int li = 0; li < NL; ++li) Ot[li] = zero4();
#pragma unroll
                for (int db = 0; db < ND; db += 2) {
                    const auto sp = pair_regs<T>(S[db], S[db + 1]);
#pragma unroll
                    for (int li = 0; li < NL; ++li)
                        Ot[li] = mma_pair<T>(sp, tile_pair(&Qs[16 * li * LDQ + 16 * db], LDQ, ln), Ot[li]);
                }
#pragma unroll
                for (int li = 0; li < NL; ++li) {
                    const float gl = gam[16 * li + cl];
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) Ot[li][rr] *= gl;
                }
                if constexpr (NORM) {
                    // qz[l] = gamma_l (q_l . z_r) for this wave's row block l = 16 wave + cl:
                    // z_r as value column 0 of a state-shaped tile (zero elsewhere)
                    floatx4 oz = zero4();
#pragma unroll
                    for (int db = 0; db < ND; db += 2) {
                        const floatx4 z0v = *reinterpret_cast<const floatx4*>(&zSb[r & 1][16 * db + g4]);
                        const floatx4 z1v = *reinterpret_cast<const floatx4*>(&zSb[r & 1][16 * db + 16 + g4]);
                        floatx4 za, zb;
#pragma unroll
                        for (int rr = 0; rr < 4; ++rr) {
                            za[rr] = cl == 0 ? z0v[rr] : 0.f;
                            zb[rr] = cl == 0 ? z1v[rr] : 0.f;
                        }
                        oz = mma_pair<T>(pair_regs<T>(za, zb), tile_pair(&Qs[16 * wave * LDQ + 16 * db], LDQ, ln), oz);
                    }
                    if (g4 == 0) qzs[r & 1][16 * wave + cl] = gam[16 * wave + cl] * oz[0];
                }
            };
            auto ksT = [&]() { kt_share(IntC<4>{}, wave, ln); };
            if constexpr (!DELTA) {
                ohist();
                ksT();
            } else {
                // a2 Aq tiles, grouped so each wave loads few blocks: wave 0 the
                // query blocks 0-1, wave 1 block 2, waves 2-3 block 3
                const float* const Gs = Gsb[r & 1];
                Fr fq[NK], fa[NK], fb[NK];
                if (wave == 0) {
                    block_frags(Ks, 0, ln, fa);
                    block_frags(Qs, 0, ln, fq);
                    aq_store(Gs, 0, 0, tile_dot(fa, fq), ln);
                    block_frags(Qs, 1, ln, fq);
                    aq_store(Gs, 1, 0, tile_dot(fa, fq), ln);
                    block_frags(Ks, 1, ln, fb);
                    aq_store(Gs, 1, 1, tile_dot(fb, fq), ln);
                } else if (wave == 1) {
                    block_frags(Qs, 2, ln, fq);
                    block_frags(Ks, 0, ln, fa);
                    aq_store(Gs, 2, 0, tile_dot(fa, fq), ln);
                    block_frags(Ks, 1, ln, fb);
                    aq_store(Gs, 2, 1, tile_dot(fb, fq), ln);
                    block_frags(Ks, 2, ln, fa);
                    aq_store(Gs, 2, 2, tile_dot(fa, fq), ln);
                } else {
                    const int m0 = wave == 2 ? 0 : 2;
                    block_frags(Qs, 3, ln, fq);
                    block_frags(Ks, m0, ln, fa);
                    aq_store(Gs, 3, m0, tile_dot(fa, fq), ln);
                    block_frags(Ks, m0 + 1, ln, fb);
                    aq_store(Gs, 3, m0 + 1, tile_dot(fb, fq), ln);
                }
                ksT();
            }
            lds_barrier();

            // ---- P2b (delta): O^T history ---------------------------------------------
            if constexpr (DELTA) {
                ohist();
                lds_barrier();
            }

            // ---- P4: b1 Z = Tb R ; c1 O^T += Z^T Aq^T ; S_{r+1} -----------------------
            // Products over token blocks run in pairs (blocks 0,1 and 2,3); the
            // causal blocks above the diagonal of Tb and Aq are zero, so block rows
            // 0 and 2 take them as partners and every accumulation chain keeps one
            // MFMA shape (mfma.h).
            floatx4 Z[NL];
            if constexpr (DELTA) {
                // Z[li] = sum_{mj <= li} Tb(li, mj) R[mj]
                const auto r01 = pair_regs<T>(R[0], R[1]), r23 = pair_regs<T>(R[2], R[3]);
#pragma unroll
                for (int li = 0; li < NL; ++li) {
                    Z[li] = mma_pair<T>(tile_pair(&Tb[16 * li * LDC], LDC, ln), r01, zero4());
                    if (li >= 2) Z[li] = mma_pair<T>(tile_pair(&Tb[16 * li * LDC + 32], LDC, ln), r23, Z[li]);
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
                    Ot[lj] = mma_pair<T>(z01, tile_pair(&Aq[16 * lj * LDC], LDC, ln), Ot[lj]);
                    if (lj >= 2) Ot[lj] = mma_pair<T>(z23, tile_pair(&Aq[16 * lj * LDC + 32], LDC, ln), Ot[lj]);
                }
            }
            // O^T tile -> Os[token][column]
#pragma unroll
            for (int lj = 0; lj < NL; ++lj) store_tile_t(&Os[DELTA ? 0 : r & 1][16 * lj * LDV + n0], LDV, Ot[lj], ln);
            state_update(S, Z, gam, rho, r, ln);
        }
        if (s_final && last_seg) {
            const int cl = lane & 15, g4 = 4 * (lane >> 4);
#pragma unroll
            for (int db = 0; db < ND; ++db)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr)
                    s_final[(bh * DK + 16 * db + g4 + rr) * DV + vb * kDVB + n0 + cl] = S[db][rr];
        }
    } else if (wave == 4) {
        // ======== wave 4: a1 gate scan; delta rule: a2 diagonal N blocks, a3/a4 T --
        T greg = from_f32<T>(0.f), breg = from_f32<T>(0.f);
        auto fetch_gate = [&](int64_t t0) {
            const int64_t tr = t0 + lane < Tlen ? t0 + lane : Tlen - 1;
            if constexpr (GATED) greg = g[bh * Tlen + tr];
            if constexpr (DELTA) breg = beta[bh * Tlen + tr];
        };
        // a1 of chunk r: G is kept in base 2 (log2 e * prefix sum) so every decay
        // factor is one hardware exp2
        auto gate_scan = [&](int64_t r, T gv) {
            const bool ok = r * kC + lane < Tlen;
            const float G = wave_prefix_sum((GATED && ok) ? prep_gate(to_f32(gv), prep) * kLog2e : 0.f);
            const float Glast = wave_last(G);
            Gsb[r & 1][lane] = G;
            gamb[r & 1][lane] = GATED ? fast_exp2(G) : 1.f;
            rhob[r & 1][lane] = GATED ? fast_exp2(Glast - G) : 1.f;
            betb[r & 1][lane] = (DELTA && ok) ? prep_beta(to_f32(breg), prep) : 0.f;
        };
        if constexpr (!DELTA) {
            // the prefix's gate values, two chunks ahead like its tokens
            T ga = from_f32<T>(0.f), gb = from_f32<T>(0.f);
            auto load_gate = [&](int64_t r, T& gv) {
                const int64_t t = (r < rb ? r : rb - 1) * kC + lane;
                if constexpr (GATED) gv = g[bh * Tlen + (t < Tlen ? t : Tlen - 1)];
            };
            auto pchunk = [&](int64_t r, i4 (&kr)[NQ], i4 (&vr)[NV], T& gv) {
                const int ln = lane_id();
                prefix_stage(r, kr, vr);
                gate_scan(r, gv);
                load_gate(r + 2, gv);
                prefix_other(ln);
            };
            if (rb > 0) {
                load_gate(0, ga);
                load_gate(1, gb);
            }
            for (int64_t r = 0; r < rb; r += 2) {
                pchunk(r, kreg, vreg, ga);
                if (r + 1 < rb) pchunk(r + 1, qreg, vreg2, gb);
            }
            if (rb > 0) fetch(rb * kC);
        }
        if (re > rb) fetch_gate(rb * kC);
        for (int64_t r = rb; r < re; ++r) {
            const int64_t t0 = r * kC;
            const int ln = lane_id();
            const int g4 = 4 * (ln >> 4);
            float* const Gs = Gsb[r & 1];
            float* const bet = betb[r & 1];

            stage(t0);
            gate_scan(r, greg);
            fetch(t0 + kC < tlast ? t0 + kC : tlast);
            fetch_gate(t0 + kC < tlast ? t0 + kC : tlast);
            if constexpr (NORM)
                if (r > rb) norm_tail(r - 1, 0, ln);
            lds_barrier();

            if constexpr (DELTA) {
                // ---- P2a: diagonal block 0, its inverse, N(1,0) ----
                floatx4 X0, Xt0;
                intra_p2a(Gs, bet, 0, ln, X0, Xt0);
                lds_barrier();
                // ---- P2b: half A of the off-diagonal blocks (column block 0, T10)
                floatx4 brow[NL];
#pragma unroll
                for (int b = 0; b < NL; ++b) brow[b] = *reinterpret_cast<const floatx4*>(&bet[16 * b + g4]);
                const floatx4* nl = Nlo + ln;
                tsolve_offdiag_a<T, kTilePc<T>>(X0, Xx[0 * kWave + ln], Xx[2 * kWave + ln], Xx[3 * kWave + ln],
                                          nl[0 * kWave], nl[1 * kWave], nl[2 * kWave], nl[3 * kWave],
                                          nl[4 * kWave], nl[5 * kWave], Tb, LDC, brow, ln);
                lds_barrier();
            } else {
                // the previous chunk's output goes out while the state waves
                // finish this chunk
                aq_add(Gs, 0, ln);
                lds_barrier();
                if (r > rb) copy_out(t0 - kC, 0, ln);
            }
        }
    } else if (DELTA && wave == 5) {
        // ======== wave 5 (delta): a2 diagonal block 1, its inverse, N(2,1); half B
        // of the off-diagonal blocks -------------------------------------------------
        for (int64_t r = rb; r < re; ++r) {
            const int64_t t0 = r * kC;
            const int ln = lane_id();
            const int g4 = 4 * (ln >> 4);
            const float* const Gs = Gsb[r & 1];
            const float* const bet = betb[r & 1];
            stage(t0);
            fetch(t0 + kC < tlast ? t0 + kC : tlast);
            lds_barrier();
            // ---- P2a ----
            floatx4 X1, Xt1;
            intra_p2a(Gs, bet, 1, ln, X1, Xt1);
            lds_barrier();
            // ---- P2b: column block 1 and T32 ----
            floatx4 brow[NL];
#pragma unroll
            for (int b = 0; b < NL; ++b) brow[b] = *reinterpret_cast<const floatx4*>(&bet[16 * b + g4]);
            const floatx4* nl = Nlo + ln;
            tsolve_offdiag_b<T, kTilePc<T>>(X1, Xx[1 * kWave + ln], Xx[2 * kWave + ln], Xx[3 * kWave + ln],
                                      nl[2 * kWave], nl[4 * kWave], nl[5 * kWave], Tb, LDC, brow, ln);
            lds_barrier();
        }
    } else {
        // ======== waves 6, 7 (delta): N blocks below the diagonal; waves 4..7
        // (add): Aq tiles.  Both: output copy ----------------------------------------
        const int iw = wave - kW0;
        if constexpr (!DELTA) {
            for (int64_t r = 0; r < rb; r += 2) {
                prefix_stage(r, kreg, vreg);
                prefix_other(lane_id());
                if (r + 1 < rb) {
                    prefix_stage(r + 1, qreg, vreg2);
                    prefix_other(lane_id());
                }
            }
            if (rb > 0) fetch(rb * kC);
        }
        for (int64_t r = rb; r < re; ++r) {
            const int64_t t0 = r * kC;
            const int ln = lane_id();
            const float* const Gs = Gsb[r & 1];
            const float* const bet = betb[r & 1];
            stage(t0);
            fetch(t0 + kC < tlast ? t0 + kC : tlast);
            if constexpr (NORM)
                if (r > rb) norm_tail(r - 1, iw, ln);
            lds_barrier();
            // ---- P2a ----
            if constexpr (DELTA) {
                floatx4 X, Xt;
                intra_p2a(Gs, bet, wave - 4, ln, X, Xt);
                lds_barrier();
                // ---- P2b ----
                if (r > rb) copy_out(t0 - kC, iw, ln);
                lds_barrier();
            } else {
                aq_add(Gs, iw, ln);
                lds_barrier();
                if (r > rb) copy_out(t0 - kC, iw, ln);
            }
        }
    }

    // the last chunk's output, once every state wave has staged it
    __syncthreads();
    if constexpr (NORM) {
        if (wave >= 4 && re > rb) norm_tail(re - 1, wave - 4, lane);
        __syncthreads();
    }
    if (wave >= kW0 && re > rb) copy_out((re - 1) * kC, wave - kW0, lane);
    if constexpr (NORM)
        if (z_final && vb == 0 && last_seg)
            for (int i = tid; i < DK; i += kNT) z_final[bh * DK + i] = zSb[re & 1][i];
}

// A prefix chunk (state update only) costs about this fraction of a full chunk
// step of the add rule (cycle probe at d_k = d_v = 128: 2.3 K against 5.0 K
// cycles; a sweep of the split at B4 H16 T4096 has its minimum near 0.45).
constexpr double kPrefixCost = 0.45;

template <typename T, int DK, int RULE, int GATE, bool SAVE, bool NORM = false>
hipError_t launch_t(const ChunkProblem& p, void* states, hipStream_t s, const float* z0 = nullptr,
                    float* z_final = nullptr)
{
    const int nvb = p.dv / kDVB;
    // add rule: segments of a head's chunks when the grid leaves compute units idle
    // (segments.h); the state-keeping forward keeps one
    const SegSplit sp = seg_split((p.T + kC - 1) / kC, p.B * p.H * nvb, RULE == kRuleAdd && !SAVE, p.s0,
                                  p.s_final, (size_t)(p.B * p.H) * p.dk * p.dv * sizeof(float), kPrefixCost);
    const int64_t nblocks = p.B * p.H * nvb * sp.n;
    hipLaunchKernelGGL((chunk_fused_kernel<T, DK, RULE, GATE, SAVE, NORM>), dim3((unsigned)nblocks), dim3(kNT),
                       0, s, static_cast<const T*>(p.q), static_cast<const T*>(p.k),
                       static_cast<const T*>(p.v), static_cast<const T*>(p.g),
                       static_cast<const T*>(p.beta), p.s0, static_cast<T*>(p.o), p.s_final, static_cast<T*>(states),
                       p.T, p.dv, (int)nblocks, p.prep, z0, z_final, sp);
    return hipGetLastError();
}

template <typename T, int DK>
hipError_t norm_by_gate(const ChunkProblem& p, const float* z0, float* z_final, hipStream_t s)
{
    return p.gate == kGateNone ? launch_t<T, DK, kRuleAdd, kGateNone, false, true>(p, nullptr, s, z0, z_final)
                               : launch_t<T, DK, kRuleAdd, kGateScalar, false, true>(p, nullptr, s, z0, z_final);
}

template <typename T, int DK, bool SAVE>
hipError_t by_rule_gate(const ChunkProblem& p, void* states, hipStream_t s)
{
    if (p.rule == kRuleAdd)
        return p.gate == kGateNone ? launch_t<T, DK, kRuleAdd, kGateNone, SAVE>(p, states, s)
                                   : launch_t<T, DK, kRuleAdd, kGateScalar, SAVE>(p, states, s);
    return p.gate == kGateNone ? launch_t<T, DK, kRuleDelta, kGateNone, SAVE>(p, states, s)
                               : launch_t<T, DK, kRuleDelta, kGateScalar, SAVE>(p, states, s);
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
        return p.dk == 64 ? by_rule_gate<bf16, 64, false>(p, nullptr, s)
                          : by_rule_gate<bf16, 128, false>(p, nullptr, s);
    return by_rule_gate<float, 64, false>(p, nullptr, s);
}

hipError_t launch_chunk_fused_normalized(const ChunkProblem& p, const float* z0, float* z_final, hipStream_t s)
{
    if (p.rule != kRuleAdd) return hipErrorInvalidValue;
    if (p.dtype == kBF16)
        return p.dk == 64 ? norm_by_gate<bf16, 64>(p, z0, z_final, s) : norm_by_gate<bf16, 128>(p, z0, z_final, s);
    return norm_by_gate<float, 64>(p, z0, z_final, s);
}

hipError_t launch_chunk_fused_save(const ChunkProblem& p, void* states, hipStream_t s)
{
    if (p.dtype == kBF16)
        return p.dk == 64 ? by_rule_gate<bf16, 64, true>(p, states, s)
                          : by_rule_gate<bf16, 128, true>(p, states, s);
    return by_rule_gate<float, 64, true>(p, states, s);
}

}  // namespace linattn
