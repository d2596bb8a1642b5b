// chunk_split.hip — two-kernel chunkwise forward for the per-key-channel
// gate (GLA-style decay with the add rule, Kimi Delta Attention with the delta
// rule); it also takes a scalar gate (every channel equal) when selected.
//
// Sources: "Linear Attention, Visualized" — "Gated Linear Attention (GLA)"
// (channelwise prefix products, decayed query <-Q and right-boundary key ->K,
// local scores), "Kimi Delta Attention (KDA)" (table of channelwise
// quantities: incoming prediction key <-k, L[l][m] for m < l; reuse of GDN's
// triangular transform), "Correct the incoming state" and the GDN chunkwise
// table with Diag(lambda[1:C]) as the state decay.
//
// Kernel A (intra-chunk, one workgroup per (b, h, chunk), all chunks in
// parallel) computes what does not depend on the incoming state and stages it
// in the workspace:
//   a1  G[l][c] = sum_{s<=l} g[s][c]  (per key channel)
//       Qd = exp(G) . Q, Kd = exp(G) . K, Kr = exp(G_{C-1} - G) . K, gC = exp(G_{C-1})
//   a2  Aq[l][m] = sum_c q_lc exp(G_lc - G_mc) k_mc   (m <= l)
//       N [l][m] = beta_l sum_c k_lc exp(G_lc - G_mc) k_mc   (m < l)
//   a3/a4  Tb = (I + N)^-1 diag(beta)                  [delta]
// Kernel B (state pass + output, one workgroup per (b, h, 64 value columns),
// chunks in order, state in registers):
//   b1  Z = Tb (V - Kd S_r)  [delta]  |  Z = V  [add]
//       S_{r+1} = Diag(gC) S_r + Kr^T Z
//   c1  O = Qd S_r + Aq Z
//
// The channelwise scores need exp(G_lc - G_mc) inside a sum over channels.  For
// a 16x16 tile it is split as exp(G_l - G_p) exp(G_p - G_m) with a reference
// row p, so the tile is one matrix-core product of two decayed operands.  Off
// the diagonal p is the row just before the query block: both factors are at
// most 1 and nothing can overflow.  On a diagonal block p is its middle row;
// each factor then stays within exp(span) where span is the block's largest
// per-channel decay, and a block whose span exceeds kSpanMax is computed
// element by element in fp32 instead.
#include "device_common.h"
#include "launch.h"
#include "mfma.h"
#include "tsolve.h"

namespace linattn {

namespace {

constexpr int kC = 64;
constexpr float kSpanMax = 80.f;   // exp(80) ~ 5.5e34 < bf16 / fp32 max

// Workspace of one chunk of one head (bf16 operands, fp32 channel factors).
template <int DK>
struct SplitWs {
    static constexpr size_t QD = 0;                                 // [C][DK]
    static constexpr size_t KD = QD + size_t(kC) * DK * 2;          // [C][DK]
    static constexpr size_t KRT = KD + size_t(kC) * DK * 2;         // [DK][C]
    static constexpr size_t AQ = KRT + size_t(DK) * kC * 2;         // [C][C]
    static constexpr size_t TB = AQ + size_t(kC) * kC * 2;          // [C][C]
    static constexpr size_t GC = TB + size_t(kC) * kC * 2;          // [DK] fp32
    static constexpr size_t BYTES = ((GC + size_t(DK) * 4) + 255) / 256 * 256;
};

typedef __attribute__((__vector_size__(16))) int i4;

// ===========================================================================
// Kernel A
// ===========================================================================
template <int DK, int RULE, int GATE>
__global__ __launch_bounds__(512, 1) void chunk_intra_channel_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ g,
    const bf16* __restrict__ beta, unsigned char* __restrict__ ws, int64_t Tlen, int64_t nchunks)
{
    using W = SplitWs<DK>;
    constexpr int NT = 512;
    constexpr bool DELTA = RULE == kRuleDelta;
    constexpr int LDQ = DK + 8, LDG = DK + 4, LDN = kC + 4, LDC = kC + 8;

    __shared__ __align__(16) bf16 qs[kC * LDQ];
    __shared__ __align__(16) bf16 ks[kC * LDQ];
    __shared__ __align__(16) float Gf[kC * LDG];
    __shared__ __align__(16) bf16 scr[4][3][16 * LDQ];
    __shared__ __align__(16) float Nf[DELTA ? kC * LDN : 4];
    __shared__ __align__(16) bf16 Aq[kC * LDC];
    __shared__ __align__(16) bf16 Tb[DELTA ? kC * LDC : 8];
    __shared__ __align__(16) float bet[kC];
    __shared__ float tot[NT / DK][DK];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int64_t bh = blockIdx.x / nchunks;
    const int64_t r = blockIdx.x % nchunks;
    const int64_t t0 = r * kC;
    unsigned char* wc = ws + (bh * nchunks + r) * W::BYTES;

    // ---- load q, k, g (fp32), beta; zero past the end ---------------------
#pragma unroll
    for (int p = 0; p < kC * DK / (8 * NT); ++p) {
        const int idx = (p * NT + tid) * 8;
        const int row = idx / DK, col = idx % DK;
        const bool ok = t0 + row < Tlen;
        const int64_t off = (bh * Tlen + t0 + row) * DK + col;
        const i4 z = {0, 0, 0, 0};
        const i4 qv = ok ? *reinterpret_cast<const i4*>(q + off) : z;
        const i4 kv = ok ? *reinterpret_cast<const i4*>(k + off) : z;
        *reinterpret_cast<i4*>(&qs[row * LDQ + col]) = qv;
        *reinterpret_cast<i4*>(&ks[row * LDQ + col]) = kv;
        floatx4 lo, hi;
        if constexpr (GATE == kGateChannel) {
            const i4 gv = ok ? *reinterpret_cast<const i4*>(g + off) : z;
            const bf16* ge = reinterpret_cast<const bf16*>(&gv);
#pragma unroll
            for (int e = 0; e < 4; ++e) { lo[e] = to_f32(ge[e]); hi[e] = to_f32(ge[4 + e]); }
        } else {
            // a scalar gate is the channel gate with every channel equal
            const float gs = ok ? to_f32(g[bh * Tlen + t0 + row]) : 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) { lo[e] = gs; hi[e] = gs; }
        }
        *reinterpret_cast<floatx4*>(&Gf[row * LDG + col]) = lo;
        *reinterpret_cast<floatx4*>(&Gf[row * LDG + col + 4]) = hi;
    }
    if (tid < kC) bet[tid] = (DELTA && t0 + tid < Tlen) ? to_f32(beta[bh * Tlen + t0 + tid]) : 0.f;
    for (int i = tid; i < kC * LDC; i += NT) Aq[i] = from_f32<bf16>(0.f);
    if constexpr (DELTA)
        for (int i = tid; i < kC * LDC; i += NT) Tb[i] = from_f32<bf16>(0.f);
    __syncthreads();

    // ---- a1: prefix sums over the chunk, per channel -------------------------
    {
        constexpr int NSEG = NT / DK, SEG = kC / NSEG;
        const int c = tid % DK, seg = tid / DK;
        float x[SEG];
#pragma unroll
        for (int i = 0; i < SEG; ++i) x[i] = Gf[(seg * SEG + i) * LDG + c];
#pragma unroll
        for (int i = 1; i < SEG; ++i) x[i] += x[i - 1];
        tot[seg][c] = x[SEG - 1];
        __syncthreads();
        float off = 0.f;
        for (int s2 = 0; s2 < seg; ++s2) off += tot[s2][c];
#pragma unroll
        for (int i = 0; i < SEG; ++i) Gf[(seg * SEG + i) * LDG + c] = x[i] + off;
    }
    __syncthreads();

    // ---- decayed operands straight to the workspace ---------------------------
    {
        bf16* Qd = reinterpret_cast<bf16*>(wc + W::QD);
        bf16* Kd = reinterpret_cast<bf16*>(wc + W::KD);
        bf16* KrT = reinterpret_cast<bf16*>(wc + W::KRT);
        float* gC = reinterpret_cast<float*>(wc + W::GC);
#pragma unroll
        for (int p = 0; p < kC * DK / (8 * NT); ++p) {
            const int idx = (p * NT + tid) * 8;
            const int row = idx / DK, col = idx % DK;
            bf16x8 qo, ko;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float d = expf(Gf[row * LDG + col + e]);
                qo[e] = from_f32<bf16>(to_f32(qs[row * LDQ + col + e]) * d);
                ko[e] = from_f32<bf16>(to_f32(ks[row * LDQ + col + e]) * d);
            }
            *reinterpret_cast<bf16x8*>(Qd + row * DK + col) = qo;
            if constexpr (DELTA) *reinterpret_cast<bf16x8*>(Kd + row * DK + col) = ko;
        }
#pragma unroll
        for (int p = 0; p < kC * DK / (8 * NT); ++p) {
            const int idx = (p * NT + tid) * 8;         // over [DK][C]
            const int c = idx / kC, l0 = idx % kC;
            const float Gend = Gf[(kC - 1) * LDG + c];
            bf16x8 kr;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                kr[e] = from_f32<bf16>(to_f32(ks[(l0 + e) * LDQ + c]) * expf(Gend - Gf[(l0 + e) * LDG + c]));
            *reinterpret_cast<bf16x8*>(KrT + c * kC + l0) = kr;
        }
        if (tid < DK) gC[tid] = expf(Gf[(kC - 1) * LDG + tid]);
    }

    // ---- a2: Aq and N tiles (waves 0..3) ------------------------------------------
    if (wave < 4) {
        bf16* Xq = scr[wave][0];
        bf16* Xk = scr[wave][1];
        bf16* Km = scr[wave][2];
        for (int task = wave; task < 10; task += 4) {
            int i, j;
            if (task < 4) { i = task; j = task; }
            else { const int pi[6] = {1, 2, 2, 3, 3, 3}, pj[6] = {0, 0, 1, 0, 1, 2};
                   i = pi[task - 4]; j = pj[task - 4]; }
            const bool diag = i == j;
            // reference row: before the query block (off-diagonal) or its middle row
            const int p = diag ? 16 * i + 7 : 16 * i - 1;
            bool safe = true;
            if (diag) {
                float span = 0.f;
                for (int c = lane; c < DK; c += 64) {
                    const float gs = i > 0 ? Gf[(16 * i - 1) * LDG + c] : 0.f;
                    span = fmaxf(span, gs - Gf[(16 * i + 15) * LDG + c]);
                }
#pragma unroll
                for (int off = 32; off > 0; off >>= 1) span = fmaxf(span, __shfl_xor(span, off, 64));
                safe = span <= kSpanMax;
            }
            if (safe) {
                for (int e = lane; e < 16 * DK; e += 64) {
                    const int rr = e / DK, c = e % DK;
                    const float Gp = Gf[p * LDG + c];
                    const float fl = expf(Gf[(16 * i + rr) * LDG + c] - Gp);
                    const float fm = expf(Gp - Gf[(16 * j + rr) * LDG + c]);
                    Xq[rr * LDQ + c] = from_f32<bf16>(to_f32(qs[(16 * i + rr) * LDQ + c]) * fl);
                    if constexpr (DELTA)
                        Xk[rr * LDQ + c] = from_f32<bf16>(to_f32(ks[(16 * i + rr) * LDQ + c]) * fl);
                    Km[rr * LDQ + c] = from_f32<bf16>(to_f32(ks[(16 * j + rr) * LDQ + c]) * fm);
                }
                // D[m][l] = sum_c Km[m][c] X[l][c]; stored transposed as [l][m]
                const floatx4 da = mma_nt_k<bf16, DK>(zero4(), Km, LDQ, Xq, LDQ, lane);
                floatx4 dn = zero4();
                if constexpr (DELTA) dn = mma_nt_k<bf16, DK>(zero4(), Km, LDQ, Xk, LDQ, lane);
                const int l = 16 * i + (lane & 15);
                const int m0 = 16 * j + 4 * (lane >> 4);
                floatx4 va, vn;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int m = m0 + rr;
                    va[rr] = (m <= l) ? da[rr] : 0.f;
                    vn[rr] = (m < l) ? bet[l] * dn[rr] : 0.f;
                }
                store_tile_t(&Aq[16 * i * LDC + 16 * j], LDC, va, lane);
                if constexpr (DELTA) store_tile_t(&Nf[16 * i * LDN + 16 * j], LDN, vn, lane);
            } else {
                // exact element-wise fallback for a diagonal block with extreme decay
                for (int e = lane; e < 256; e += 64) {
                    const int l = 16 * i + e / 16, m = 16 * i + e % 16;
                    float a = 0.f, n = 0.f;
                    if (m <= l) {
                        for (int c = 0; c < DK; ++c) {
                            const float d = expf(Gf[l * LDG + c] - Gf[m * LDG + c]);
                            const float km = to_f32(ks[m * LDQ + c]) * d;
                            a = fmaf(to_f32(qs[l * LDQ + c]), km, a);
                            n = fmaf(to_f32(ks[l * LDQ + c]), km, n);
                        }
                    }
                    Aq[l * LDC + m] = from_f32<bf16>(a);
                    if constexpr (DELTA) Nf[l * LDN + m] = (m < l) ? bet[l] * n : 0.f;
                }
            }
        }
    }
    __syncthreads();

    // ---- a3/a4: triangular transform (wave 0) -----------------------------------
    if constexpr (DELTA) {
        if (wave == 0) tsolve64_wave<bf16>(Nf, LDN, Tb, LDC, bet, lane);
        __syncthreads();
    }

    // ---- Aq and Tb to the workspace --------------------------------------------------
    {
        bf16* Aqw = reinterpret_cast<bf16*>(wc + W::AQ);
        bf16* Tbw = reinterpret_cast<bf16*>(wc + W::TB);
        const int row = tid / (kC / 8), col = (tid % (kC / 8)) * 8;
        *reinterpret_cast<i4*>(Aqw + row * kC + col) = *reinterpret_cast<const i4*>(&Aq[row * LDC + col]);
        if constexpr (DELTA)
            *reinterpret_cast<i4*>(Tbw + row * kC + col) = *reinterpret_cast<const i4*>(&Tb[row * LDC + col]);
    }
}

// ===========================================================================
// Kernel B: state pass + output.  Wave w owns value columns 16w..16w+15 of the
// workgroup's 64-column block and keeps S[:, those columns] as dk/16 result
// tiles; every product takes S, R or Z straight from registers (see mfma.h,
// K = 16 products), so LDS only supplies the per-chunk operand tiles.
// ===========================================================================
template <int DK, int RULE>
__global__ __launch_bounds__(256, 1) void chunk_chain_kernel(
    const bf16* __restrict__ v, const unsigned char* __restrict__ ws, const float* s0,
    bf16* __restrict__ o, float* s_final, int64_t Tlen, int64_t nchunks, int DV, int nblocks)
{
    using W = SplitWs<DK>;
    constexpr int NT = 256, DVB = 64, ND = DK / 16, NL = kC / 16;
    constexpr bool DELTA = RULE == kRuleDelta;
    constexpr int LDQ = DK + 8, LDC = kC + 8, LDV = DVB + 8;
    constexpr int VQ = kC * DK / (8 * NT);       // 16-byte vectors per thread, [C][DK] tile
    constexpr int VA = kC * kC / (8 * NT);       // [C][C] tile
    constexpr int VV = kC * DVB / (8 * NT);      // V block
    static_assert(VQ >= 1 && VA >= 1 && VV >= 1, "tile split");

    __shared__ __align__(16) bf16 Qd[kC * LDQ];
    __shared__ __align__(16) bf16 Kd[DELTA ? kC * LDQ : 8];
    __shared__ __align__(16) bf16 KrT[DK * LDC];
    __shared__ __align__(16) bf16 Aq[kC * LDC];
    __shared__ __align__(16) bf16 Tb[DELTA ? kC * LDC : 8];
    __shared__ __align__(16) bf16 Vs[kC * LDV];
    __shared__ __align__(16) float gC[DK];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int nvb = DV / DVB;
    int blk = blockIdx.x;
    if ((nblocks & 7) == 0) blk = (blk & 7) * (nblocks >> 3) + (blk >> 3);
    const int64_t bh = blk / nvb;
    const int vb = blk % nvb;
    const int n0 = vb * DVB + 16 * wave;          // first value column of this wave
    const int cl = lane & 15, g4 = 4 * (lane >> 4);

    // S[16 db + g4 + rr][n0 + cl]
    floatx4 S[ND];
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
            S[db][rr] = s0 ? s0[(bh * DK + 16 * db + g4 + rr) * DV + n0 + cl] : 0.f;
    wait_vmem_all();

    i4 rq[VQ], rk[VQ], rkr[VQ], ra[VA], rt[VA], rv[VV];
    i4 rg = {0, 0, 0, 0};
    auto fetch = [&](int64_t c) {
        const unsigned char* wc = ws + (bh * nchunks + c) * W::BYTES;
#pragma unroll
        for (int p = 0; p < VQ; ++p) {
            const int e = (p * NT + tid) * 8;
            rq[p] = *reinterpret_cast<const i4*>(wc + W::QD + 2 * e);
            if constexpr (DELTA) rk[p] = *reinterpret_cast<const i4*>(wc + W::KD + 2 * e);
            rkr[p] = *reinterpret_cast<const i4*>(wc + W::KRT + 2 * e);
        }
#pragma unroll
        for (int p = 0; p < VA; ++p) {
            const int e = (p * NT + tid) * 8;
            ra[p] = *reinterpret_cast<const i4*>(wc + W::AQ + 2 * e);
            if constexpr (DELTA) rt[p] = *reinterpret_cast<const i4*>(wc + W::TB + 2 * e);
        }
#pragma unroll
        for (int p = 0; p < VV; ++p) {
            const int e = (p * NT + tid) * 8;
            const int row = e / DVB, col = e % DVB;
            const int64_t tr = c * kC + row < Tlen ? c * kC + row : Tlen - 1;
            rv[p] = *reinterpret_cast<const i4*>(v + (bh * Tlen + tr) * DV + vb * DVB + col);
        }
        if (tid < DK / 4) rg = *reinterpret_cast<const i4*>(wc + W::GC + 16 * tid);
    };
    if (nchunks > 0) fetch(0);

    for (int64_t c = 0; c < nchunks; ++c) {
        const int64_t t0 = c * kC;
        lds_barrier();
#pragma unroll
        for (int p = 0; p < VQ; ++p) {
            const int e = (p * NT + tid) * 8;
            const int row = e / DK, col = e % DK;
            *reinterpret_cast<i4*>(&Qd[row * LDQ + col]) = rq[p];
            if constexpr (DELTA) *reinterpret_cast<i4*>(&Kd[row * LDQ + col]) = rk[p];
            const int rt_ = e / kC, ct = e % kC;
            *reinterpret_cast<i4*>(&KrT[rt_ * LDC + ct]) = rkr[p];
        }
#pragma unroll
        for (int p = 0; p < VA; ++p) {
            const int e = (p * NT + tid) * 8;
            const int row = e / kC, col = e % kC;
            *reinterpret_cast<i4*>(&Aq[row * LDC + col]) = ra[p];
            if constexpr (DELTA) *reinterpret_cast<i4*>(&Tb[row * LDC + col]) = rt[p];
        }
#pragma unroll
        for (int p = 0; p < VV; ++p) {
            const int e = (p * NT + tid) * 8;
            const int row = e / DVB, col = e % DVB;
            const i4 z = {0, 0, 0, 0};
            *reinterpret_cast<i4*>(&Vs[row * LDV + col]) = (t0 + row < Tlen) ? rv[p] : z;
        }
        if (tid < DK / 4) *reinterpret_cast<i4*>(&gC[4 * tid]) = rg;
        if (c + 1 < nchunks) fetch(c + 1);
        lds_barrier();

        // ---- b1: Z = Tb (V - Kd S_r)  (add rule: Z = V) ----------------------
        floatx4 Z[NL];
#pragma unroll
        for (int li = 0; li < NL; ++li) {
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) Z[li][rr] = to_f32(Vs[(16 * li + g4 + rr) * LDV + 16 * wave + cl]);
        }
        if constexpr (DELTA) {
            floatx4 R[NL];
#pragma unroll
            for (int li = 0; li < NL; ++li) {
                floatx4 acc = zero4();
#pragma unroll
                for (int db = 0; db < ND; ++db)
                    acc = mma16<bf16>(frag16_lds(&Kd[16 * li * LDQ + 16 * db], LDQ, lane),
                                      frag16_acc<bf16>(S[db]), acc);
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) R[li][rr] = Z[li][rr] - acc[rr];
            }
#pragma unroll
            for (int li = 0; li < NL; ++li) {
                floatx4 acc = zero4();
#pragma unroll
                for (int mj = 0; mj <= li; ++mj)
                    acc = mma16<bf16>(frag16_lds(&Tb[16 * li * LDC + 16 * mj], LDC, lane),
                                      frag16_acc<bf16>(R[mj]), acc);
                Z[li] = acc;
            }
        }
        // ---- c1: O^T = S_r^T Qd^T + Z^T Aq^T, straight to HBM ----------------------
#pragma unroll
        for (int lj = 0; lj < NL; ++lj) {
            floatx4 acc = zero4();
#pragma unroll
            for (int db = 0; db < ND; ++db)
                acc = mma16<bf16>(frag16_acc<bf16>(S[db]), frag16_lds(&Qd[16 * lj * LDQ + 16 * db], LDQ, lane),
                                  acc);
#pragma unroll
            for (int mj = 0; mj <= lj; ++mj)
                acc = mma16<bf16>(frag16_acc<bf16>(Z[mj]), frag16_lds(&Aq[16 * lj * LDC + 16 * mj], LDC, lane),
                                  acc);
            const int64_t l = t0 + 16 * lj + cl;
            if (l < Tlen) {
                bf16x4 w;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) w[rr] = from_f32<bf16>(acc[rr]);
                *reinterpret_cast<bf16x4*>(o + (bh * Tlen + l) * DV + n0 + g4) = w;
            }
        }
        // ---- b1: S_{r+1} = Diag(gC) S_r + Kr^T Z ----------------------------------
#pragma unroll
        for (int db = 0; db < ND; ++db) {
            floatx4 acc = S[db];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) acc[rr] *= gC[16 * db + g4 + rr];
#pragma unroll
            for (int lj = 0; lj < NL; ++lj)
                acc = mma16<bf16>(frag16_lds(&KrT[16 * db * LDC + 16 * lj], LDC, lane),
                                  frag16_acc<bf16>(Z[lj]), acc);
            S[db] = acc;
        }
    }

    if (s_final) {
#pragma unroll
        for (int db = 0; db < ND; ++db)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
                s_final[(bh * DK + 16 * db + g4 + rr) * DV + n0 + cl] = S[db][rr];
    }
}

template <int DK, int RULE, int GATE>
hipError_t launch_split(const ChunkProblem& p, hipStream_t s)
{
    const int64_t nchunks = (p.T + kC - 1) / kC;
    const int64_t bh = p.B * p.H;
    unsigned char* ws = static_cast<unsigned char*>(p.workspace);
    if (nchunks > 0) {
        hipLaunchKernelGGL((chunk_intra_channel_kernel<DK, RULE, GATE>), dim3((unsigned)(bh * nchunks)),
                           dim3(512), 0, s, static_cast<const bf16*>(p.q),
                           static_cast<const bf16*>(p.k), static_cast<const bf16*>(p.g),
                           static_cast<const bf16*>(p.beta), ws, p.T, nchunks);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int nblocks = (int)(bh * (p.dv / 64));
    hipLaunchKernelGGL((chunk_chain_kernel<DK, RULE>), dim3((unsigned)nblocks), dim3(256), 0, s,
                       static_cast<const bf16*>(p.v), ws, p.s0, static_cast<bf16*>(p.o), p.s_final,
                       p.T, nchunks, p.dv, nblocks);
    return hipGetLastError();
}

}  // namespace

bool chunk_split_supported(const ChunkProblem& p)
{
    return p.gate != kGateNone && p.chunk == kC && p.dtype == kBF16 &&
           (p.dk == 64 || p.dk == 128) && (p.dv == 64 || p.dv == 128);
}

size_t chunk_split_workspace_bytes(const ChunkProblem& p)
{
    const size_t nchunks = (size_t)((p.T + kC - 1) / kC);
    const size_t per = p.dk == 64 ? SplitWs<64>::BYTES : SplitWs<128>::BYTES;
    return (size_t)(p.B * p.H) * nchunks * per;
}

template <int DK>
hipError_t split_by_rule_gate(const ChunkProblem& p, hipStream_t s)
{
    if (p.gate == kGateChannel)
        return p.rule == kRuleDelta ? launch_split<DK, kRuleDelta, kGateChannel>(p, s)
                                    : launch_split<DK, kRuleAdd, kGateChannel>(p, s);
    return p.rule == kRuleDelta ? launch_split<DK, kRuleDelta, kGateScalar>(p, s)
                                : launch_split<DK, kRuleAdd, kGateScalar>(p, s);
}

hipError_t launch_chunk_split(const ChunkProblem& p, hipStream_t s)
{
    return p.dk == 64 ? split_by_rule_gate<64>(p, s) : split_by_rule_gate<128>(p, s);
}

}  // namespace linattn
