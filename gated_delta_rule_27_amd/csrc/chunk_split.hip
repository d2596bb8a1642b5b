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
// Kernel A (intra-chunk, persistent workgroups walking the (b, h, chunk)
// tasks, all chunks in parallel) computes what does not depend on the incoming
// state and stages it in the workspace:
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
// The channelwise scores need exp(G_lc - G_mc) inside a sum over channels.
// Kernel A splits it into per-row factors local to each 16-row block, so every
// 16x16 score tile is one matrix-core product of two decayed operands (the
// factorisation and its overflow guard are described at kernel A).
#include "device_common.h"
#include "launch.h"
#include "mfma.h"
#include "prep.h"
#include "segments.h"
#include "tsolve.h"
#include "tile_rows.h"

namespace linattn {

namespace {

constexpr int kC = 64;

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
// Kernel A: persistent.  Workgroup w walks the chunk-heads w, w + grid, ...;
// the next one's q, k, g and beta are loaded into registers while the current
// one is processed.  Gates are kept in base 2 (log2 e . g) so every decay
// factor is one hardware exp2.
//
// With G the per-channel prefix inside the chunk, block b = rows 16b..16b+15,
// s(b) the row before it (G_{-1} = 0) and e(b) its last row, every row l of
// block b gets two block-local factors per channel, both at most 1 for decays:
//   u_l = 2^(G_l - G_s(b)),   w_l = 2^(G_e(b) - G_l)
// and the staged operands Qu = u.q, Ku = u.k, Kw = w.k.  Then, per channel,
//   off the diagonal (i > j):  2^(G_l - G_m) = u_l . 2^(G_s(i) - G_e(j)) . w_m
//   on the diagonal  (i = j):  2^(G_l - G_m) = (u_l 2^(G_s - G_mid)) . (w_m 2^(G_mid - G_e))
// so every 16x16 score tile is one matrix-core product of Kw scaled by a
// channel vector and Qu (or Ku), scaled by a channel vector on the diagonal.
// The diagonal factors stay within 2^(span/2) (span = the block's largest
// per-channel decay); a block whose span exceeds kSpan2Max is computed element
// by element instead, from the raw tokens, before they are overwritten.  The
// decayed operands of kernel B follow from the same factors:
//   Qd = Qu . 2^G_s(b),  Kd = Ku . 2^G_s(b),  Kr = Kw . 2^(G_63 - G_e(b)).
// ===========================================================================
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kSpan2Max = 120.f;   // 2^60 per factor, far inside bf16 / fp32 range

// PREP: the input maps of prep.h (flags in prep) applied while staging; a
// separate instantiation, so the kernel without maps is the plain one.
template <int DK, int RULE, int GATE, bool PREP>
__global__ __launch_bounds__(512, 1) void chunk_intra_channel_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ g,
    const bf16* __restrict__ beta, unsigned char* __restrict__ ws, int64_t Tlen, int64_t nchunks,
    int64_t ntasks, int prep)
{
    using W = SplitWs<DK>;
    constexpr int NT = 512;
    constexpr bool DELTA = RULE == kRuleDelta;
    constexpr int LDQ = DK + 8, LDN = kC + 4, LDC = kC + 8;
    constexpr int NK = DK / 32;                       // 16x16x32 steps over the channels
    constexpr int NV = kC * DK / (8 * NT);            // 16-byte vectors per thread of a [C][DK] tile
    static_assert(NV >= 1, "tile split");

    __shared__ __align__(16) bf16 qs[kC * LDQ];       // q, then Qu
    __shared__ __align__(16) bf16 ks[kC * LDQ];       // k, then Ku
    __shared__ __align__(16) bf16 kw[kC * LDQ];       // Kw
    __shared__ __align__(16) bf16 gs[kC * LDQ];       // raw gate (channel gate)
    __shared__ __align__(16) float tot[4][DK];        // block sums of the base-2 gate
    __shared__ __align__(16) float Es[4][DK];         // 2^G_s(b)
    __shared__ __align__(16) float Fe[4][DK];         // 2^(G_63 - G_e(b))
    __shared__ __align__(16) float Pv[4][DK];         // 2^(G_s(b) - G_mid(b))
    __shared__ __align__(16) float Rv[4][DK];         // 2^(G_mid(b) - G_e(b))
    __shared__ __align__(16) float Dt[6][DK];         // 2^(G_s(i) - G_e(j)), pairs (1,0)(2,0)(2,1)(3,0)(3,1)(3,2)
    __shared__ __align__(16) float Nf[DELTA ? kC * LDN : 4];
    __shared__ __align__(16) bf16 Aq[kC * LDC];
    __shared__ __align__(16) bf16 Tb[DELTA ? kC * LDC : 8];
    __shared__ __align__(16) float bet[kC];
    __shared__ float gsc[kC];                         // scalar gate, base 2
    __shared__ float spanw[8];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int cl = lane & 15, g4 = 4 * (lane >> 4);

    // the causal blocks above the diagonal stay zero
    for (int i = tid; i < kC * LDC; i += NT) Aq[i] = from_f32<bf16>(0.f);
    if constexpr (DELTA)
        for (int i = tid; i < kC * LDC; i += NT) Tb[i] = from_f32<bf16>(0.f);

    i4 qreg[NV], kreg[NV], greg[NV];
    bf16 gsreg = from_f32<bf16>(0.f), breg = from_f32<bf16>(0.f);
    auto fetch = [&](int64_t task) {
        const int64_t bh = task / nchunks, t0 = (task % nchunks) * kC;
#pragma unroll
        for (int p = 0; p < NV; ++p) {
            const int idx = (p * NT + tid) * 8;
            const int row = idx / DK, col = idx % DK;
            const int64_t tr = t0 + row < Tlen ? t0 + row : Tlen - 1;
            const int64_t off = (bh * Tlen + tr) * DK + col;
            qreg[p] = *reinterpret_cast<const i4*>(q + off);
            kreg[p] = *reinterpret_cast<const i4*>(k + off);
            if constexpr (GATE == kGateChannel) greg[p] = *reinterpret_cast<const i4*>(g + off);
        }
        if (tid < kC) {
            const int64_t tr = t0 + tid < Tlen ? t0 + tid : Tlen - 1;
            if constexpr (GATE != kGateChannel) gsreg = g[bh * Tlen + tr];
            if constexpr (DELTA) breg = beta[bh * Tlen + tr];
        }
    };
    if (blockIdx.x < ntasks) fetch(blockIdx.x);

    for (int64_t task = blockIdx.x; task < ntasks; task += gridDim.x) {
        const int64_t t0 = (task % nchunks) * kC;
        unsigned char* wc = ws + task * W::BYTES;     // task = (b, h) * nchunks + chunk

        // ---- stage the chunk; issue the next chunk-head's loads ---------------------
        // (raw projections first go through the maps of prep.h: q/k here, the
        // DK / 8 lanes holding a row reducing its L2 norm; the log-gate map where
        // the gate is read in fp32; beta below)
        __syncthreads();
        const int qk_map = PREP ? prep_qk_map(prep) : 0;
#pragma unroll
        for (int p = 0; p < NV; ++p) {
            const int idx = (p * NT + tid) * 8;
            const int row = idx / DK, col = idx % DK;
            const bool ok = t0 + row < Tlen;
            const i4 z = {0, 0, 0, 0};
            const i4 qp = PREP ? prep_qk<bf16, DK / 8>(qreg[p], qk_map) : qreg[p];
            const i4 kp = PREP ? prep_qk<bf16, DK / 8>(kreg[p], qk_map) : kreg[p];
            *reinterpret_cast<i4*>(&qs[row * LDQ + col]) = ok ? qp : z;
            *reinterpret_cast<i4*>(&ks[row * LDQ + col]) = ok ? kp : z;
            if constexpr (GATE == kGateChannel) *reinterpret_cast<i4*>(&gs[row * LDQ + col]) = ok ? greg[p] : z;
        }
        if (tid < kC) {
            // a scalar gate is the channel gate with every channel equal
            if constexpr (GATE != kGateChannel)
                gsc[tid] = (t0 + tid < Tlen) ? (PREP ? prep_gate(to_f32(gsreg), prep) : to_f32(gsreg)) * kLog2e : 0.f;
            bet[tid] = (DELTA && t0 + tid < Tlen) ? (PREP ? prep_beta(to_f32(breg), prep) : to_f32(breg)) : 0.f;
        }
        if (task + gridDim.x < ntasks) fetch(task + gridDim.x);
        __syncthreads();

        // ---- a1: per-channel prefix, block factors, tables ------------------------------
        // thread (c, b): channel c, block b (the first 4 DK threads)
        float Gl[16];
        const int pc = tid % DK, pb = tid / DK;
        const bool pre = tid < 4 * DK;
        if (pre) {
            float acc = 0.f;
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                float gv;
                if constexpr (GATE == kGateChannel)
                    gv = !PREP ? to_f32(gs[(16 * pb + rr) * LDQ + pc]) * kLog2e
                       : t0 + 16 * pb + rr < Tlen ? prep_gate(to_f32(gs[(16 * pb + rr) * LDQ + pc]), prep) * kLog2e
                                                   : 0.f;
                else gv = gsc[16 * pb + rr];
                acc += gv;
                Gl[rr] = acc;                          // G_l - G_s(b)
            }
            tot[pb][pc] = acc;
        }
        __syncthreads();
        float span = 0.f;
        if (pre) {
            float off = 0.f, all = 0.f, ends[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                all += tot[b][pc];
                ends[b] = all;                         // G_e(b)
                if (b < pb) off += tot[b][pc];
            }
            const float Gst = off;
            Es[pb][pc] = fast_exp2(Gst);
            Fe[pb][pc] = fast_exp2(all - ends[pb]);
            Pv[pb][pc] = fast_exp2(-Gl[7]);
            Rv[pb][pc] = fast_exp2(Gl[7] - Gl[15]);
            // pair (pb, j) for j < pb: slot pb (pb - 1) / 2 + j
#pragma unroll
            for (int j = 0; j < 3; ++j)
                if (j < pb) Dt[pb * (pb - 1) / 2 + j][pc] = fast_exp2(Gst - ends[j]);
            if (pb == 0) reinterpret_cast<float*>(wc + W::GC)[pc] = fast_exp2(all);
            span = -Gl[15];
        }
        // largest decay span of each diagonal block (waves of one block combine)
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) span = fmaxf(span, shfl_xor(span, off));
        if (lane == 0) spanw[wave] = span;
        __syncthreads();
        constexpr int WPB = DK / 64;                   // waves per block in the prefix mapping
        bool safe[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            float sp = spanw[b * WPB];
            if constexpr (WPB == 2) sp = fmaxf(sp, spanw[b * WPB + 1]);
            safe[b] = sp <= kSpan2Max;
        }

        // ---- exact element-wise diagonal blocks where the span is too large ----------
        // (raw q, k and g still in LDS; wave b takes block b)
        if (wave < 4 && !safe[wave]) {
            const int b = wave;
            for (int e = lane; e < 256; e += 64) {
                const int l = 16 * b + e / 16, m = 16 * b + e % 16;
                float a = 0.f, n = 0.f;
                if (m <= l) {
                    for (int c = 0; c < DK; ++c) {
                        float dG = 0.f;                // G_l - G_m, base 2
                        for (int s2 = m + 1; s2 <= l; ++s2) {
                            if constexpr (GATE == kGateChannel)
                                dG += !PREP ? to_f32(gs[s2 * LDQ + c]) * kLog2e
                                    : t0 + s2 < Tlen ? prep_gate(to_f32(gs[s2 * LDQ + c]), prep) * kLog2e : 0.f;
                            else dG += gsc[s2];
                        }
                        const float km = to_f32(ks[m * LDQ + c]) * fast_exp2(dG);
                        a = fmaf(to_f32(qs[l * LDQ + c]), km, a);
                        n = fmaf(to_f32(ks[l * LDQ + c]), km, n);
                    }
                }
                Aq[l * LDC + m] = from_f32<bf16>(a);
                if constexpr (DELTA) Nf[l * LDN + m] = (m < l) ? bet[l] * n : 0.f;
            }
        }
        __syncthreads();

        // ---- staged operands Qu, Ku, Kw ---------------------------------------------
        if (pre) {
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                const int row = 16 * pb + rr;
                const float u = fast_exp2(Gl[rr]), w = fast_exp2(Gl[15] - Gl[rr]);
                const float qv = to_f32(qs[row * LDQ + pc]), kv = to_f32(ks[row * LDQ + pc]);
                qs[row * LDQ + pc] = from_f32<bf16>(qv * u);
                ks[row * LDQ + pc] = from_f32<bf16>(kv * u);
                kw[row * LDQ + pc] = from_f32<bf16>(kv * w);
            }
        }
        __syncthreads();

        // ---- a2: score and N tiles (10 causal pairs over the 8 waves) ------------------
        for (int p = wave; p < 10; p += 8) {
            // p < 4: diagonal block p; else pair slot p - 4 of (1,0)(2,0)(2,1)(3,0)(3,1)(3,2)
            const int qn = p - 4;
            const int i = p < 4 ? p : (qn < 1 ? 1 : (qn < 3 ? 2 : 3));
            const int j = p < 4 ? p : qn - i * (i - 1) / 2;
            const bool diag = i == j;
            if (diag && !safe[i]) continue;
            const float* dk_ = diag ? Rv[j] : Dt[p - 4];   // channel scale of the key side
            floatx4 xa = zero4(), xn = zero4();
#pragma unroll
            for (int kk = 0; kk < NK; ++kk) {
                const int c0 = 32 * kk + 8 * (lane >> 4);
                // key side: Kw rows of block j, scaled per channel
                const bf16x8 kv = *reinterpret_cast<const bf16x8*>(&kw[(16 * j + cl) * LDQ + c0]);
                const floatx4 s0 = *reinterpret_cast<const floatx4*>(&dk_[c0]);
                const floatx4 s1 = *reinterpret_cast<const floatx4*>(&dk_[c0 + 4]);
                bf16x8 ka;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    ka[e] = from_f32<bf16>(to_f32(kv[e]) * s0[e]);
                    ka[4 + e] = from_f32<bf16>(to_f32(kv[4 + e]) * s1[e]);
                }
                // query side: Qu (and Ku) rows of block i, scaled on the diagonal
                bf16x8 qb = *reinterpret_cast<const bf16x8*>(&qs[(16 * i + cl) * LDQ + c0]);
                bf16x8 kb = *reinterpret_cast<const bf16x8*>(&ks[(16 * i + cl) * LDQ + c0]);
                if (diag) {
                    const floatx4 p0 = *reinterpret_cast<const floatx4*>(&Pv[i][c0]);
                    const floatx4 p1 = *reinterpret_cast<const floatx4*>(&Pv[i][c0 + 4]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        qb[e] = from_f32<bf16>(to_f32(qb[e]) * p0[e]);
                        qb[4 + e] = from_f32<bf16>(to_f32(qb[4 + e]) * p1[e]);
                        kb[e] = from_f32<bf16>(to_f32(kb[e]) * p0[e]);
                        kb[4 + e] = from_f32<bf16>(to_f32(kb[4 + e]) * p1[e]);
                    }
                }
                xa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qb, xa, 0, 0, 0);
                if constexpr (DELTA) xn = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, kb, xn, 0, 0, 0);
            }
            // D[m][l]: m = 16 j + g4 + rr (key), l = 16 i + cl (query); stored as [l][m]
            const int l = 16 * i + cl;
            floatx4 va, vn;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int m = 16 * j + g4 + rr;
                va[rr] = (m <= l) ? xa[rr] : 0.f;
                vn[rr] = (m < l) ? bet[l] * xn[rr] : 0.f;
            }
            store_tile_t(&Aq[16 * i * LDC + 16 * j], LDC, va, lane);
            if constexpr (DELTA) store_tile_t(&Nf[16 * i * LDN + 16 * j], LDN, vn, lane);
        }

        __syncthreads();

        // ---- wave 0: a3/a4 triangular transform; waves 1..7 meanwhile write the
        // decayed operands of kernel B and Aq to the workspace, columns in pcol
        // order (mfma.h): the 8 values stored at position P are the logical
        // columns c0..c0+3 and c0+16..c0+19, c0 = pcol_first(P) ---------------------
        if (wave == 0) {
            if constexpr (DELTA) tsolve64_wave<bf16>(Nf, LDN, Tb, LDC, bet, lane);
        } else {
            constexpr int NW1 = NT - 64;              // threads of waves 1..7
            const int wt = tid - 64;
            bf16* Qd = reinterpret_cast<bf16*>(wc + W::QD);
            bf16* Kd = reinterpret_cast<bf16*>(wc + W::KD);
            bf16* KrT = reinterpret_cast<bf16*>(wc + W::KRT);
            bf16* Aqw = reinterpret_cast<bf16*>(wc + W::AQ);
            for (int v8 = wt; v8 < kC * DK / 8; v8 += NW1) {
                const int idx = v8 * 8;
                const int row = idx / DK, P = idx % DK, b = row / 16;
                const int c0 = pcol_first(P), c1 = c0 + 16;
                const bf16x4 qa = *reinterpret_cast<const bf16x4*>(&qs[row * LDQ + c0]);
                const bf16x4 qb = *reinterpret_cast<const bf16x4*>(&qs[row * LDQ + c1]);
                const bf16x4 ka = *reinterpret_cast<const bf16x4*>(&ks[row * LDQ + c0]);
                const bf16x4 kb = *reinterpret_cast<const bf16x4*>(&ks[row * LDQ + c1]);
                const floatx4 e0 = *reinterpret_cast<const floatx4*>(&Es[b][c0]);
                const floatx4 e1 = *reinterpret_cast<const floatx4*>(&Es[b][c1]);
                bf16x8 qo, ko;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    qo[e] = from_f32<bf16>(to_f32(qa[e]) * e0[e]);
                    qo[4 + e] = from_f32<bf16>(to_f32(qb[e]) * e1[e]);
                    ko[e] = from_f32<bf16>(to_f32(ka[e]) * e0[e]);
                    ko[4 + e] = from_f32<bf16>(to_f32(kb[e]) * e1[e]);
                }
                *reinterpret_cast<bf16x8*>(Qd + row * DK + P) = qo;
                if constexpr (DELTA) *reinterpret_cast<bf16x8*>(Kd + row * DK + P) = ko;
            }
            for (int v8 = wt; v8 < DK * kC / 8; v8 += NW1) {
                const int idx = v8 * 8;                 // over [DK][C]
                const int c = idx / kC, P = idx % kC;
                const int l0 = pcol_first(P), l1 = l0 + 16;
                const float f0 = Fe[l0 / 16][c], f1 = Fe[l1 / 16][c];
                bf16x8 kr;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    kr[e] = from_f32<bf16>(to_f32(kw[(l0 + e) * LDQ + c]) * f0);
                    kr[4 + e] = from_f32<bf16>(to_f32(kw[(l1 + e) * LDQ + c]) * f1);
                }
                *reinterpret_cast<bf16x8*>(KrT + c * kC + P) = kr;
            }
            for (int v8 = wt; v8 < kC * kC / 8; v8 += NW1) {
                const int row = v8 / (kC / 8), P = (v8 % (kC / 8)) * 8;
                const int c0 = pcol_first(P), c1 = c0 + 16;
                *reinterpret_cast<bf16x8*>(Aqw + row * kC + P) =
                    __builtin_shufflevector(*reinterpret_cast<const bf16x4*>(&Aq[row * LDC + c0]),
                                            *reinterpret_cast<const bf16x4*>(&Aq[row * LDC + c1]), 0, 1, 2, 3, 4, 5, 6, 7);
            }
        }
        if constexpr (DELTA) {
            __syncthreads();
            // ---- Tb to the workspace, columns in pcol order --------------------------------
            bf16* Tbw = reinterpret_cast<bf16*>(wc + W::TB);
            const int row = tid / (kC / 8), P = (tid % (kC / 8)) * 8;
            const int c0 = pcol_first(P), c1 = c0 + 16;
            *reinterpret_cast<bf16x8*>(Tbw + row * kC + P) =
                __builtin_shufflevector(*reinterpret_cast<const bf16x4*>(&Tb[row * LDC + c0]),
                                        *reinterpret_cast<const bf16x4*>(&Tb[row * LDC + c1]), 0, 1, 2, 3, 4, 5, 6, 7);
        }
    }
}

// ===========================================================================
// Kernel B: state pass + output.  One workgroup per (b, h, DVB = 64 or 32 value
// columns), chunks in order, DVB/16 + 4 waves:
//   * state waves 0..DVB/16-1: wave w owns value columns 16w..16w+15 and keeps
//     S[:, those columns] (fp32) as dk/16 MFMA result tiles; every product
//     takes S, R or Z straight from registers (mfma.h), paired into K = 32
//     products whose LDS operands are single 16-byte reads (pcol order, as
//     kernel A stores them, with the conflict-free swizzle of mfma.h applied
//     when the helpers stage the rows into LDS).
//   * the four helper waves after them move everything between HBM and LDS: the chunk's
//     staged operands, loaded into registers one chunk ahead, and the output.
//     The state waves touch no global memory inside the loop.
// Two LDS barriers per chunk split it into
//   phase 1: R = V - Kd S_r, Z = Tb R (delta; add rule: Z = V), O^T = S_r^T Qd^T
//            (needs Kd, V, Tb, Qd: group 1);  helpers stage group 2 of this
//            chunk and copy the previous chunk's output to HBM
//   phase 2: O^T += Z^T Aq^T (to LDS), S_{r+1} = Diag(gC) S_r + Kr^T Z
//            (needs Aq, Kr^T, gC: group 2);  helpers stage group 1 of the next
//            chunk
// so each LDS region is refilled while the other phase runs.
// ===========================================================================
//
// With SAVE the state waves also write S_r, the state entering chunk r, to an
// LDS tile at the top of every chunk, and the helper waves copy it to
// states[b, h, r] ([dk][dv], bf16) during phase 2 with 16-byte stores.
//
// Segments (segments.h): a workgroup may own chunks [rb, re) of its head; it
// first runs the state update alone over chunks [0, rb) (phase 1 without O,
// phase 2 without O; the helpers stage neither Qd nor Aq), then its own chunks
// as usual.  With SAVE each segment writes the states of its own chunks; the
// prefix pass runs the same update code, so they equal one segment's bit for bit.
template <int DK, int RULE, int DVB, bool SAVE>
__global__ __launch_bounds__((DVB / 16 + 4) * 64, 1) void chunk_chain_kernel(
    const bf16* __restrict__ v, const unsigned char* __restrict__ ws, const float* s0,
    bf16* __restrict__ o, float* s_final, bf16* __restrict__ states, int64_t Tlen, int64_t nchunks, int DV,
    int nblocks, SegSplit seg)
{
    using W = SplitWs<DK>;
    constexpr int NSW = DVB / 16;                // state waves, 16 value columns each
    constexpr int NH = 256, ND = DK / 16, NL = kC / 16;
    constexpr bool DELTA = RULE == kRuleDelta;
    constexpr int LDQ = DK + 8, LDC = kC + 8, LDV = DVB + 8;
    constexpr int VQ = kC * DK / (8 * NH);       // 16-byte vectors per helper thread, [C][DK] tile
    constexpr int VA = kC * kC / (8 * NH);       // [C][C] tile
    constexpr int VV = kC * DVB / (8 * NH);      // V block
    constexpr int VK = DK * kC / (8 * NH);       // Kr^T [DK][C]
    static_assert(VQ >= 1 && VA >= 1 && VV >= 1 && VK >= 1, "tile split");

    __shared__ __align__(16) bf16 Qd[kC * LDQ];
    __shared__ __align__(16) bf16 Kd[DELTA ? kC * LDQ : 8];
    __shared__ __align__(16) bf16 KrT[DK * LDC];
    __shared__ __align__(16) bf16 Aq[kC * LDC];
    __shared__ __align__(16) bf16 Tb[DELTA ? kC * LDC : 8];
    __shared__ __align__(16) bf16 Vs[kC * LDV];
    __shared__ __align__(16) bf16 Os[kC * LDV];
    __shared__ __align__(16) bf16 Sst[SAVE ? DK * LDV : 8];
    __shared__ __align__(16) float gC[DK];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int nvb = DV / DVB;
    int blk = blockIdx.x;
    if ((nblocks & 7) == 0) blk = (blk & 7) * (nblocks >> 3) + (blk >> 3);
    const int nunit = nvb * seg.n;
    const int64_t bh = blk / nunit;
    const int vb = (blk % nunit) % nvb;
    const int sg = (blk % nunit) / nvb;
    const int64_t rb = seg.c[sg], re = seg.c[sg + 1];
    const bool last_seg = sg == seg.n - 1;

    if (wave < NSW) {
        // ======== state waves ============================================================
        const int n0 = 16 * wave;                 // first column of this wave in the block
        floatx4 S[ND];
        {
            const int cl = lane & 15, g4 = 4 * (lane >> 4);
#pragma unroll
            for (int db = 0; db < ND; ++db)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr)
                    S[db][rr] = s0 ? s0[(bh * DK + 16 * db + g4 + rr) * DV + vb * DVB + n0 + cl] : 0.f;
        }
        wait_vmem_all();
        __syncthreads();                          // group 1 of the first chunk staged
        {
            // prefix pass: S_{r+1} = Diag(gC) S_r + Kr^T Tb (V - Kd S_r) over chunks [0, rb)
            for (int64_t c = 0; c < rb; ++c) {
                const int ln = opaque(lane);
                const int cl = ln & 15, g4 = 4 * (ln >> 4);
                floatx4 R[NL], Z[NL];
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
                        const auto sp = pair_regs<bf16>(S[db], S[db + 1]);
#pragma unroll
                        for (int li = 0; li < NL; ++li)
                            P[li] = mma_pair<bf16>(pair_lds_sw(&Kd[16 * li * LDQ + 16 * db], LDQ, ln), sp, P[li]);
                    }
#pragma unroll
                    for (int li = 0; li < NL; ++li)
#pragma unroll
                        for (int rr = 0; rr < 4; ++rr) R[li][rr] -= P[li][rr];
                    const auto r01 = pair_regs<bf16>(R[0], R[1]), r23 = pair_regs<bf16>(R[2], R[3]);
#pragma unroll
                    for (int li = 0; li < NL; ++li) {
                        Z[li] = mma_pair<bf16>(pair_lds_sw(&Tb[16 * li * LDC], LDC, ln), r01, zero4());
                        if (li >= 2) Z[li] = mma_pair<bf16>(pair_lds_sw(&Tb[16 * li * LDC + 32], LDC, ln), r23, Z[li]);
                    }
                } else {
#pragma unroll
                    for (int li = 0; li < NL; ++li) Z[li] = R[li];
                }
                lds_barrier();
                const auto z01 = pair_regs<bf16>(Z[0], Z[1]), z23 = pair_regs<bf16>(Z[2], Z[3]);
#pragma unroll
                for (int db = 0; db < ND; ++db) {
                    const floatx4 gd = *reinterpret_cast<const floatx4*>(&gC[16 * db + g4]);
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) S[db][rr] *= gd[rr];
                    S[db] = mma_pair<bf16>(pair_lds_sw(&KrT[16 * db * LDC + 32], LDC, ln), z23,
                                           mma_pair<bf16>(pair_lds_sw(&KrT[16 * db * LDC], LDC, ln), z01, S[db]));
                }
                lds_barrier();
            }
            if (rb > 0) __syncthreads();          // group 1 of chunk rb staged
        }
        for (int64_t c = rb; c < re; ++c) {
            const int ln = opaque(lane);
            const int cl = ln & 15, g4 = 4 * (ln >> 4);
            if constexpr (SAVE) {
#pragma unroll
                for (int db = 0; db < ND; ++db) store_tile_rows(Sst + 16 * db * LDV + n0, LDV, S[db], ln);
            }
            // ---- phase 1: R = V - Kd S_r ; Z = Tb R ; O^T = S_r^T Qd^T ----------------
            floatx4 R[NL], Z[NL], Ot[NL];
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
                    const auto sp = pair_regs<bf16>(S[db], S[db + 1]);
#pragma unroll
                    for (int li = 0; li < NL; ++li)
                        P[li] = mma_pair<bf16>(pair_lds_sw(&Kd[16 * li * LDQ + 16 * db], LDQ, ln), sp, P[li]);
                }
#pragma unroll
                for (int li = 0; li < NL; ++li)
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) R[li][rr] -= P[li][rr];
                // Z[li] = sum_{mj <= li} Tb(li, mj) R[mj]; block rows 0 and 2 take the
                // zero causal block as a partner (one MFMA shape per chain)
                const auto r01 = pair_regs<bf16>(R[0], R[1]), r23 = pair_regs<bf16>(R[2], R[3]);
#pragma unroll
                for (int li = 0; li < NL; ++li) {
                    Z[li] = mma_pair<bf16>(pair_lds_sw(&Tb[16 * li * LDC], LDC, ln), r01, zero4());
                    if (li >= 2) Z[li] = mma_pair<bf16>(pair_lds_sw(&Tb[16 * li * LDC + 32], LDC, ln), r23, Z[li]);
                }
            } else {
#pragma unroll
                for (int li = 0; li < NL; ++li) Z[li] = R[li];
            }
#pragma unroll
            for (int li = 0; li < NL; ++li) Ot[li] = zero4();
#pragma unroll
            for (int db = 0; db < ND; db += 2) {
                const auto sp = pair_regs<bf16>(S[db], S[db + 1]);
#pragma unroll
                for (int li = 0; li < NL; ++li)
                    Ot[li] = mma_pair<bf16>(sp, pair_lds_sw(&Qd[16 * li * LDQ + 16 * db], LDQ, ln), Ot[li]);
            }
            lds_barrier();
            // ---- phase 2: O^T += Z^T Aq^T ; S_{r+1} = Diag(gC) S_r + Kr^T Z ------------
            const auto z01 = pair_regs<bf16>(Z[0], Z[1]), z23 = pair_regs<bf16>(Z[2], Z[3]);
#pragma unroll
            for (int lj = 0; lj < NL; ++lj) {
                Ot[lj] = mma_pair<bf16>(z01, pair_lds_sw(&Aq[16 * lj * LDC], LDC, ln), Ot[lj]);
                if (lj >= 2) Ot[lj] = mma_pair<bf16>(z23, pair_lds_sw(&Aq[16 * lj * LDC + 32], LDC, ln), Ot[lj]);
            }
#pragma unroll
            for (int lj = 0; lj < NL; ++lj) store_tile_t(&Os[16 * lj * LDV + n0], LDV, Ot[lj], ln);
#pragma unroll
            for (int db = 0; db < ND; ++db) {
                const floatx4 gd = *reinterpret_cast<const floatx4*>(&gC[16 * db + g4]);
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) S[db][rr] *= gd[rr];
                S[db] = mma_pair<bf16>(pair_lds_sw(&KrT[16 * db * LDC + 32], LDC, ln), z23,
                                       mma_pair<bf16>(pair_lds_sw(&KrT[16 * db * LDC], LDC, ln), z01, S[db]));
            }
            lds_barrier();
        }
        if (s_final && last_seg) {
            const int cl = lane & 15, g4 = 4 * (lane >> 4);
#pragma unroll
            for (int db = 0; db < ND; ++db)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr)
                    s_final[(bh * DK + 16 * db + g4 + rr) * DV + vb * DVB + n0 + cl] = S[db][rr];
        }
        __syncthreads();                          // the last output is in Os
    } else {
        // ======== helper waves =============================================================
        const int ht = tid - NSW * 64;
        // group 1: Kd, Qd, V, Tb ; group 2: Aq, Kr^T, gC
        i4 rkd[VQ], rqd[VQ], rv[VV], rtb[VA];
        i4 raq[VA], rkr[VK], rg = {0, 0, 0, 0};
        // the loads and staging of the two groups; with full = IntC<false> (prefix
        // pass) without Qd and Aq
        auto load1 = [&](int64_t c, auto full) {
            constexpr bool FULL = decltype(full)::value;
            const unsigned char* wc = ws + (bh * nchunks + c) * W::BYTES;
#pragma unroll
            for (int p = 0; p < VQ; ++p) {
                const int e = (p * NH + ht) * 8;
                if constexpr (FULL) rqd[p] = *reinterpret_cast<const i4*>(wc + W::QD + 2 * e);
                if constexpr (DELTA) rkd[p] = *reinterpret_cast<const i4*>(wc + W::KD + 2 * e);
            }
#pragma unroll
            for (int p = 0; p < VA; ++p) {
                const int e = (p * NH + ht) * 8;
                if constexpr (DELTA) rtb[p] = *reinterpret_cast<const i4*>(wc + W::TB + 2 * e);
            }
#pragma unroll
            for (int p = 0; p < VV; ++p) {
                const int e = (p * NH + ht) * 8;
                const int row = e / DVB, col = e % DVB;
                const int64_t tr = c * kC + row < Tlen ? c * kC + row : Tlen - 1;
                rv[p] = *reinterpret_cast<const i4*>(v + (bh * Tlen + tr) * DV + vb * DVB + col);
            }
        };
        auto stage1 = [&](int64_t c, auto full) {
            constexpr bool FULL = decltype(full)::value;
#pragma unroll
            for (int p = 0; p < VQ; ++p) {
                const int e = (p * NH + ht) * 8;
                const int row = e / DK, col = e % DK;
                const int cs = col ^ swz_x(row);
                if constexpr (FULL) *reinterpret_cast<i4*>(&Qd[row * LDQ + cs]) = rqd[p];
                if constexpr (DELTA) *reinterpret_cast<i4*>(&Kd[row * LDQ + cs]) = rkd[p];
            }
#pragma unroll
            for (int p = 0; p < VA; ++p) {
                const int e = (p * NH + ht) * 8;
                const int row = e / kC, col = e % kC;
                if constexpr (DELTA) *reinterpret_cast<i4*>(&Tb[row * LDC + (col ^ swz_x(row))]) = rtb[p];
            }
#pragma unroll
            for (int p = 0; p < VV; ++p) {
                const int e = (p * NH + ht) * 8;
                const int row = e / DVB, col = e % DVB;
                const i4 z = {0, 0, 0, 0};
                *reinterpret_cast<i4*>(&Vs[row * LDV + col]) = (c * kC + row < Tlen) ? rv[p] : z;
            }
        };
        auto load2 = [&](int64_t c, auto full) {
            constexpr bool FULL = decltype(full)::value;
            const unsigned char* wc = ws + (bh * nchunks + c) * W::BYTES;
#pragma unroll
            for (int p = 0; p < VA; ++p) {
                const int e = (p * NH + ht) * 8;
                if constexpr (FULL) raq[p] = *reinterpret_cast<const i4*>(wc + W::AQ + 2 * e);
            }
#pragma unroll
            for (int p = 0; p < VK; ++p) {
                const int e = (p * NH + ht) * 8;
                rkr[p] = *reinterpret_cast<const i4*>(wc + W::KRT + 2 * e);
            }
            if (ht < DK / 4) rg = *reinterpret_cast<const i4*>(wc + W::GC + 16 * ht);
        };
        auto stage2 = [&](auto full) {
            constexpr bool FULL = decltype(full)::value;
#pragma unroll
            for (int p = 0; p < VA; ++p) {
                const int e = (p * NH + ht) * 8;
                const int row = e / kC, col = e % kC;
                if constexpr (FULL) *reinterpret_cast<i4*>(&Aq[row * LDC + (col ^ swz_x(row))]) = raq[p];
            }
#pragma unroll
            for (int p = 0; p < VK; ++p) {
                const int e = (p * NH + ht) * 8;
                const int row = e / kC, col = e % kC;
                *reinterpret_cast<i4*>(&KrT[row * LDC + (col ^ swz_x(row))]) = rkr[p];
            }
            if (ht < DK / 4) *reinterpret_cast<i4*>(&gC[4 * ht]) = rg;
        };
        // Output block of chunk c from Os, 16-byte rows, through a buffer resource
        // over this head's rows: rows past the end fall outside it and the
        // hardware drops them, so no branch hides a store from the compiler's
        // wait counts.  Likewise every chunk issues the same loads (the chunk
        // index clamped to the last one), so a wait for one group never includes
        // the group loaded after it.
        const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
            o + bh * Tlen * DV, (short)0, (int)(Tlen * DV * 2), 0x00020000);
        auto copy_out = [&](int64_t c) {
#pragma unroll
            for (int p = 0; p < VV; ++p) {
                const int e = (p * NH + ht) * 8;
                const int row = e / DVB, col = e % DVB;
                const int off = (int)(((c * kC + row) * DV + vb * DVB + col) * 2);
                __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const i4*>(&Os[row * LDV + col]), orsrc,
                                                       off, 0, 0);
            }
        };
        // S_r of chunk c from LDS to HBM (written by the state waves at the top
        // of the chunk, stable until its second barrier)
        auto copy_state = [&](int64_t c) {
            constexpr int VR = DVB / 8, NS = DK * VR / NH;
            static_assert(NS * NH == DK * VR, "state copy split");
#pragma unroll
            for (int p = 0; p < NS; ++p) {
                const int e = p * NH + ht;
                const int row = e / VR, col = (e % VR) * 8;
                *reinterpret_cast<i4*>(states + ((bh * nchunks + c) * DK + row) * DV + vb * DVB + col) =
                    *reinterpret_cast<const i4*>(&Sst[row * LDV + col]);
            }
        };
        constexpr IntC<true> kFull{};
        constexpr IntC<false> kPrefix{};
        const int64_t last = re - 1, plast = rb - 1;
        if (rb > 0) {
            load1(0, kPrefix);
            load2(0, kPrefix);
            stage1(0, kPrefix);
            load1(1 < plast ? 1 : plast, kPrefix);
        } else if (re > rb) {
            load1(rb, kFull);
            load2(rb, kFull);
            stage1(rb, kFull);
            load1(rb + 1 < last ? rb + 1 : last, kFull);
        }
        __syncthreads();                          // group 1 of the first chunk staged
        {
            for (int64_t c = 0; c < rb; ++c) {
                stage2(kPrefix);
                load2(c + 1 < plast ? c + 1 : plast, kPrefix);
                lds_barrier();
                if (c + 1 < rb) stage1(c + 1, kPrefix);
                load1(c + 2 < plast ? c + 2 : plast, kPrefix);
                lds_barrier();
            }
            if (rb > 0) {
                load1(rb, kFull);
                load2(rb, kFull);
                stage1(rb, kFull);
                load1(rb + 1 < last ? rb + 1 : last, kFull);
                __syncthreads();                  // group 1 of chunk rb staged
            }
        }
        for (int64_t c = rb; c < re; ++c) {
            // ---- phase 1 ----
            stage2(kFull);
            load2(c + 1 < last ? c + 1 : last, kFull);
            if (c > rb) copy_out(c - 1);
            lds_barrier();
            // ---- phase 2 ----
            if (c + 1 < re) stage1(c + 1, kFull);
            load1(c + 2 < last ? c + 2 : last, kFull);
            if constexpr (SAVE) copy_state(c);
            lds_barrier();
        }
        __syncthreads();                          // the last output is in Os
        if (re > rb) copy_out(re - 1);
    }
}

// A prefix chunk of the state pass (no Qd, Aq, output) costs about this
// fraction of a full chunk: it moves 65 % of the bytes, and the pass is bound
// by the memory system rather than by its own latency (KDA B1 H32 T262144,
// two segments: 0.5, 0.65, 0.8 gave 9.24, 9.23, 9.20 ms per forward).
constexpr double kChainPrefixCost = 0.8;

template <int DK, int RULE, int GATE>
hipError_t launch_split(const ChunkProblem& p, bf16* states, hipStream_t s)
{
    const int64_t nchunks = (p.T + kC - 1) / kC;
    const int64_t bh = p.B * p.H;
    unsigned char* ws = static_cast<unsigned char*>(p.workspace);
    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu <= 0)
        ncu = 256;
    if (nchunks > 0) {
        // persistent: one workgroup per CU (its LDS use allows no second one)
        const int64_t ntasks = bh * nchunks;
        const int64_t grid = ntasks < ncu ? ntasks : ncu;
        if (p.prep != 0)
            hipLaunchKernelGGL((chunk_intra_channel_kernel<DK, RULE, GATE, true>), dim3((unsigned)grid), dim3(512), 0,
                               s, static_cast<const bf16*>(p.q), static_cast<const bf16*>(p.k),
                               static_cast<const bf16*>(p.g), static_cast<const bf16*>(p.beta), ws, p.T,
                               nchunks, ntasks, p.prep);
        else
            hipLaunchKernelGGL((chunk_intra_channel_kernel<DK, RULE, GATE, false>), dim3((unsigned)grid), dim3(512), 0,
                               s, static_cast<const bf16*>(p.q), static_cast<const bf16*>(p.k),
                               static_cast<const bf16*>(p.g), static_cast<const bf16*>(p.beta), ws, p.T,
                               nchunks, ntasks, 0);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // The state pass runs one workgroup per (b, h, value block).  With few heads
    // (fewer 64-column blocks than CUs) the blocks are 32 columns wide, which
    // doubles the number of independent chains; each staged tile is then read
    // by twice as many workgroups (mostly from L2).
    // A grid that still leaves CUs idle splits each head's chunks into
    // segments (segments.h).
    const bool narrow = bh * (p.dv / 64) < ncu;
    const int64_t nblocks1 = bh * (p.dv / (narrow ? 32 : 64));
    const SegSplit sp = seg_split(nchunks, nblocks1, true, p.s0, p.s_final,
                                  (size_t)bh * p.dk * p.dv * sizeof(float), kChainPrefixCost);
    const int nblocks = (int)(nblocks1 * sp.n);
    const dim3 grid((unsigned)nblocks);
    const bf16* v = static_cast<const bf16*>(p.v);
    bf16* o = static_cast<bf16*>(p.o);
    if (narrow && states)
        hipLaunchKernelGGL((chunk_chain_kernel<DK, RULE, 32, true>), grid, dim3(6 * 64), 0, s, v, ws, p.s0, o,
                           p.s_final, states, p.T, nchunks, p.dv, nblocks, sp);
    else if (narrow)
        hipLaunchKernelGGL((chunk_chain_kernel<DK, RULE, 32, false>), grid, dim3(6 * 64), 0, s, v, ws, p.s0, o,
                           p.s_final, states, p.T, nchunks, p.dv, nblocks, sp);
    else if (states)
        hipLaunchKernelGGL((chunk_chain_kernel<DK, RULE, 64, true>), grid, dim3(8 * 64), 0, s, v, ws, p.s0, o,
                           p.s_final, states, p.T, nchunks, p.dv, nblocks, sp);
    else
        hipLaunchKernelGGL((chunk_chain_kernel<DK, RULE, 64, false>), grid, dim3(8 * 64), 0, s, v, ws, p.s0, o,
                           p.s_final, states, p.T, nchunks, p.dv, nblocks, sp);
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
hipError_t split_by_rule_gate(const ChunkProblem& p, bf16* states, hipStream_t s)
{
    if (p.gate == kGateChannel)
        return p.rule == kRuleDelta ? launch_split<DK, kRuleDelta, kGateChannel>(p, states, s)
                                    : launch_split<DK, kRuleAdd, kGateChannel>(p, states, s);
    return p.rule == kRuleDelta ? launch_split<DK, kRuleDelta, kGateScalar>(p, states, s)
                                : launch_split<DK, kRuleAdd, kGateScalar>(p, states, s);
}

hipError_t launch_chunk_split(const ChunkProblem& p, hipStream_t s)
{
    return p.dk == 64 ? split_by_rule_gate<64>(p, nullptr, s) : split_by_rule_gate<128>(p, nullptr, s);
}

hipError_t launch_chunk_split_save(const ChunkProblem& p, void* states, hipStream_t s)
{
    bf16* st = static_cast<bf16*>(states);
    return p.dk == 64 ? split_by_rule_gate<64>(p, st, s) : split_by_rule_gate<128>(p, st, s);
}

}  // namespace linattn
