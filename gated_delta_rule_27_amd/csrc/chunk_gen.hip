// chunk_gen.hip — chunkwise forward for every supported chunk size
// C in {16, 32, 64, 128}, fp32 or bf16 tokens, dk, dv in {64, 128}, the add
// or delta rule and no / scalar / per-key-channel gate.  It serves what the
// tuned single-pass and two-kernel paths (chunk 64) do not: other chunk sizes,
// fp32 tokens at dk = 128 and fp32 tokens with the per-channel gate.
//
// Sources: "Linear Attention, Visualized" — "Chunkwise algorithm" and "Cost"
// (any chunk size gives the exact result; the size only trades the C x C
// intra-chunk work against the n / C state steps), "Gated Linear Attention
// (GLA)" and "Kimi Delta Attention (KDA)" (channelwise decay inside the
// scores, decayed query <-Q and right-boundary key ->K), "The triangular
// correction system", "Optional: Use UT to share the triangular transform"
// (W = T B <-K, U = T B V) and "Correct the incoming state" (Z = U - W S_r),
// and the GDN row of the chunkwise table.
//
// Two kernels, the first over all chunks in parallel, the second walking each
// head's chunks in order:
//
//   gen_intra_kernel   one workgroup per (b, h, chunk), 4 waves (8 at chunk
//     128); chunks of 16 or 32 tokens without the per-channel gate run four or
//     two to a workgroup as the diagonal blocks of a 64-row tile.  It stages
//     q, k (and the per-channel gate) 32 key channels at a time in fp32 LDS
//     and writes each chunk's operands to the workspace, in the token type:
//       a1  G = prefix of the log-gate (base 2; per channel or scalar)
//       a2  Aq[l][m] = sum_c q_lc 2^(G_lc - G_mc) k_mc   (m <= l)
//           scalar gate / no gate: a matrix-core product, decay applied after;
//           per-channel gate: element-wise fp32 sums with the decay of every
//           (l, m, c) formed from the difference G_lc - G_mc <= 0, so no
//           factor can overflow whatever the gate
//       a3  T = (I + diag(beta) L)^-1, L[l][m] = as Aq with k for q, m < l
//           (fp32: 16 x 16 diagonal blocks by forward substitution, one lane
//           per column; the blocks below by block substitution on the fp32
//           matrix cores)
//       a4  W = T diag(beta) <-K,  U = T diag(beta) V   (matrix cores with
//           operands of the token type: T rounded once, like every operand)
//       and the operands of the state pass: <-Q = 2^G . Q, ->K^T with
//       ->k_l = 2^(G_{C-1} - G_l) . k_l, and 2^(G_{C-1})
//   gen_chain_kernel   one workgroup per (b, h, 64 value columns): 4 state
//     waves of 16 columns each, S (fp32) in matrix-core result registers, and
//     4 helper waves staging each 16-row block's operands in LDS; per chunk and
//     per 16-row block li of the chunk:
//       b1  Z_li = U_li - W_li S_r   (add rule: Z = V)
//       c1  O_li = <-Q_li S_r + sum_{mj <= li} Aq(li, mj) Z_mj
//           dS  += ->K_li^T Z_li
//     then S_{r+1} = Diag(2^(G_{C-1})) S_r + dS.
//
// Rows past the end of the sequence are staged as zeros (k = v = 0, g = 0,
// beta = 0), which leaves the state unchanged; their outputs are not written.
#include "device_common.h"
#include "launch.h"
#include "mfma.h"
#include "prep.h"
#include "segments.h"

namespace linattn {

namespace {

// A K = 16 fragment read as frag16_lds (mfma.h), through a volatile pointer of
// the LDS address space, so that every 8-byte read stays one ds_read_b64: two
// reads from one base register would otherwise be merged into a ds_read2_b64,
// which on gfx950 serves 16 lanes per clock over 32 banks and takes 8 LDS
// cycles, against 2 cycles (32 lanes per clock over 64 banks) for each
// ds_read_b64 (lane-group probe, peak/lds_banks.hip).
template <typename T>
__device__ __forceinline__ typename Frag16<T>::type frag16_lds_sep(const T* M, int ld, int lane)
{
    typedef const volatile __attribute__((address_space(3))) typename Frag16<T>::type* LP;
    return *(LP)(M + (lane & 15) * ld + 4 * (lane >> 4));
}

constexpr float kLog2e = 1.4426950408889634f;
// waves of the intra-chunk kernel: 8 at C = 128, else 4
__host__ __device__ constexpr int gen_waves(int C) { return C == 128 ? 8 : 4; }

// Workspace of one chunk of one head: byte offsets of its pieces (256-byte
// aligned), operands in the token type (element size esz), 2^(G_{C-1}) fp32.
struct GenWs {
    size_t qd, krt, aq, gc, w, u, bytes;
};
__host__ __device__ inline GenWs gen_ws(int C, int DK, int DV, int esz, bool delta)
{
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    GenWs l{};
    l.qd = 0;                                           // <-Q   [C][DK]
    l.krt = l.qd + up((size_t)C * DK * esz);            // ->K^T [DK][C]
    l.aq = l.krt + up((size_t)DK * C * esz);            // Aq    [C][C] (causal blocks)
    l.gc = l.aq + up((size_t)C * C * esz);              // 2^(G_{C-1}) [DK] fp32
    l.w = l.gc + up((size_t)DK * 4);                    // W     [C][DK]  (delta)
    l.u = l.w + (delta ? up((size_t)C * DK * esz) : 0); // U     [C][DV]  (delta)
    l.bytes = l.u + (delta ? up((size_t)C * DV * esz) : 0);
    return l;
}

// four consecutive token values as fp32
__device__ __forceinline__ floatx4 load4(const float* p) { return *reinterpret_cast<const floatx4*>(p); }
__device__ __forceinline__ floatx4 load4(const bf16* p)
{
    const bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
    return floatx4{to_f32(v[0]), to_f32(v[1]), to_f32(v[2]), to_f32(v[3])};
}

// (i, j) of the p-th causal 16 x 16 tile, j <= i, row-major over i
__device__ __forceinline__ void tile_ij(int p, int& i, int& j)
{
    i = 0;
    while (p > i) { p -= i + 1; ++i; }
    j = p;
}

// ===========================================================================
// Intra-chunk kernel
// ===========================================================================
// Rows per workgroup of the intra kernel for chunk size CH: chunks of 16 or 32
// tokens (gate none or scalar) run two or four to a workgroup as the diagonal
// blocks of a 64-row tile, so all four waves have tiles and the per-workgroup
// steps (gate scan, slice staging, barriers) are shared; else one chunk.
__host__ __device__ constexpr int gen_tile(int CH, int gate) { return CH < 64 && gate != kGateChannel ? 64 : CH; }

// At chunk 128 (under 80 KB of LDS) two 8-wave workgroups share a CU when the
// kernel keeps to 128 VGPRs, which it does without spills except for fp32
// tokens with the per-channel gate.
template <typename T, int CH, int GATE>
constexpr int gen_intra_waves_per_simd()
{
    return gen_tile(CH, GATE) == 128 && !(sizeof(T) == 4 && GATE == kGateChannel) ? 4 : 1;
}

template <typename T, int CH, int DK, int RULE, int GATE>
__global__ __launch_bounds__(64 * gen_waves(gen_tile(CH, GATE)))
__attribute__((amdgpu_waves_per_eu(gen_intra_waves_per_simd<T, CH, GATE>(), 8))) void gen_intra_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ g,
    const T* __restrict__ beta, unsigned char* __restrict__ ws, int64_t Tlen, int64_t nchunks, int DV,
    int prep)
{
    constexpr int C = gen_tile(CH, GATE);       // rows of the tile
    constexpr int SUB = C / CH;                 // chunks in the tile
    constexpr int BC = CH / 16;                 // 16-row blocks per chunk
    constexpr int NB = C / 16;
    constexpr bool DELTA = RULE == kRuleDelta;
    constexpr bool CHAN = GATE == kGateChannel;
    constexpr bool GATED = GATE != kGateNone;
    constexpr int NW = gen_waves(C), kGT = 64 * NW;
    constexpr int NTILE = SUB * BC * (BC + 1) / 2;   // causal 16x16 tiles inside the chunks
    static_assert(SUB == 1 || (C == 64 && !CHAN), "several chunks per workgroup: 64-row tiles, no per-channel gate");
    constexpr int MS = (NTILE + NW - 1) / NW;    // causal tiles per wave
    // key / value channels per staged slice (16 at C = 128, which with the
    // packed blocks of T keeps the workgroup under 80 KB of LDS: two per CU)
    constexpr int kKS = C == 128 ? 16 : 32;
    constexpr int kLDS = kKS + 4;                // row stride of a staged fp32 slice
    constexpr int LDB = 16 + 4;                  // row stride of a packed 16x16 block of L / T
    constexpr int NLB = NB * (NB + 1) / 2;       // blocks on and below the diagonal
    constexpr int NSL = DK / kKS;                // key-channel slices
    static_assert(NB >= 1 && NB <= 8 && DK % kKS == 0, "chunk and head sizes");

    __shared__ __align__(16) float xs[C * kLDS];                  // q slice, later beta <-K or beta V
    __shared__ __align__(16) float ys[C * kLDS];                  // k slice
    __shared__ __align__(16) float gs[CHAN ? C * kLDS : 4];       // per-channel prefix (base 2)
    __shared__ __align__(16) float Lm[DELTA ? NLB * 16 * LDB : 4]; // beta L, then T: blocks (i, j <= i) packed
    __shared__ __align__(16) float Gsc[C];                        // scalar prefix (base 2)
    __shared__ __align__(16) float bet[C];
    __shared__ __align__(16) float rq[C], rk[C];                  // 1 / |q_l|, 1 / |k_l| (L2 map)
    __shared__ __align__(16) float gtot[CHAN ? NB * kKS : 4];     // block totals of a channel slice

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t ntile = (nchunks + SUB - 1) / SUB;          // workgroups per head
    const int64_t task = blockIdx.x;
    const int64_t bh = task / ntile, c0i = (task % ntile) * SUB, t0 = c0i * CH;
    const int nrow = (int)(Tlen - t0 < C ? Tlen - t0 : C);      // rows of this tile in the sequence
    const int qkm = prep_qk_map(prep);
    // workspace piece at byte offset off of the tile's chunk sc (chunk rows
    // sc CH .. of the tile); chunks past the head's last one are not written
    const GenWs L = gen_ws(CH, DK, DV, (int)sizeof(T), DELTA);
    unsigned char* const wc0 = ws + (bh * nchunks + c0i) * L.bytes;
    auto wsp = [&](int sc, size_t off) { return wc0 + (size_t)sc * L.bytes + off; };
    auto has = [&](int sc) { return SUB == 1 || c0i + sc < nchunks; };
    const int64_t rowbase = bh * Tlen + t0;
    auto lmb = [&](int i, int j) { return &Lm[(i * (i + 1) / 2 + j) * 16 * LDB]; };   // block (i, j), j <= i
    // (i, j) of the p-th causal 16x16 tile inside the tile's chunks
    auto tile_of = [&](int p, int& i, int& j) {
        if constexpr (SUB == 1) {
            tile_ij(p, i, j);
        } else {
            constexpr int TPC = BC * (BC + 1) / 2;         // tiles per chunk
            tile_ij(p % TPC, i, j);
            i += (p / TPC) * BC;
            j += (p / TPC) * BC;
        }
    };
    // chunk of tile row r and its row inside that chunk
    auto chunk_of = [](int r) { return SUB == 1 ? 0 : r / CH; };
    auto row_in = [](int r) { return SUB == 1 ? r : r % CH; };

    // ---- token loads.  Thread tid owns the 4-element groups tid + j kGT of
    // every staged [C][kKS] slice (row e / (kKS / 4), columns 4 (e % (kKS / 4))
    // onwards).  Two register sets, A and B, hold the groups of q and k (and of
    // the per-channel log-gate, or of v) of the next two slices: a set is
    // refilled with the slice after next as soon as it has been staged, so each
    // load has two slices' work to arrive (the first two the gate scan, those of
    // the second pass over the key channels and of v the triangular solve).
    constexpr int PE = C * kKS / 4;                  // 4-element groups of a slice
    constexpr int PP = (PE + kGT - 1) / kGT;         // groups per thread
    using R4 = typename Frag16<T>::type;             // four token values
    struct Slice {
        R4 q[PP], k[PP], g[CHAN ? PP : 1];
    };
    auto grp = [&](int j, int& row, int& cq) {
        const int e = tid + j * kGT;
        row = e / (kKS / 4);
        cq = 4 * (e % (kKS / 4));
        return PE % kGT == 0 || e < PE;
    };
    auto ld4 = [](const T* p) { return *reinterpret_cast<const R4*>(p); };
    auto cvt4 = [](R4 x) { return floatx4{to_f32(x[0]), to_f32(x[1]), to_f32(x[2]), to_f32(x[3])}; };
    // key channels sl kKS .. of q and k (and the log-gate); rows past the end
    // read row 0 and are zeroed when staged
    auto load_qk = [&](Slice& S, int sl) {
#pragma unroll
        for (int j = 0; j < PP; ++j) {
            int row, cq;
            if (grp(j, row, cq)) {
                const int64_t off = (rowbase + (row < nrow ? row : 0)) * DK + sl * kKS + cq;
                S.q[j] = ld4(q + off);
                S.k[j] = ld4(k + off);
                if constexpr (CHAN) S.g[j] = ld4(g + off);
            }
        }
    };
    // value columns vs kKS .. of v, into S.q
    auto load_v = [&](Slice& S, int vs) {
#pragma unroll
        for (int j = 0; j < PP; ++j) {
            int row, cq;
            if (grp(j, row, cq)) S.q[j] = ld4(v + (rowbase + (row < nrow ? row : 0)) * DV + vs * kKS + cq);
        }
    };
    Slice SA, SB;
    load_qk(SA, 0);
    load_qk(SB, 1);

    // ---- a1 (scalar gate) and beta: one wave, 64 rows at a time ------------------
    if (wave == 0) {
        // every row's gate and beta loaded (rows past the end read row 0) before
        // the first is used
        constexpr int NH = (C + 63) / 64;
        float gr[NH], br[NH];
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            const int l = 64 * h + lane;
            const int lc = l < nrow ? l : 0;
            gr[h] = (GATED && !CHAN) ? to_f32(g[rowbase + lc]) : 0.f;
            br[h] = DELTA ? to_f32(beta[rowbase + lc]) : 0.f;
        }
        float carry = 0.f;
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            const int l = 64 * h + lane;
            const bool ok = l < nrow;
            const float gv = (GATED && !CHAN && ok) ? prep_gate(gr[h], prep) * kLog2e : 0.f;
            float G = wave_prefix_sum(gv) + carry;
            carry = wave_last(G);
            if constexpr (SUB > 1) {
                // (one pass: C = 64) the prefix restarts at each chunk of the tile
                const int st = (lane / CH) * CH;
                const float base = __shfl(G, st > 0 ? st - 1 : 0, 64);
                if (st > 0) G -= base;
            }
            if (l < C) {
                Gsc[l] = G;
                bet[l] = (DELTA && ok) ? prep_beta(br[h], prep) : 0.f;
            }
        }
    }
    // ---- inverse L2 norms of the raw rows (q/k map L2): one thread per row -------
    if (qkm == kQkL2 && tid < 2 * C) {
        const int l = tid % C;
        const T* src = (tid < C ? q : k) + (rowbase + (l < nrow ? l : 0)) * DK;
        float ss = 0.f;
        for (int c = 0; c < DK; c += 4) {
            const floatx4 x = load4(src + c);
            ss += x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
        }
        (tid < C ? rq : rk)[l] = rsqrtf(fmaxf(ss, 1e-12f));
    }
    __syncthreads();

    // prepared q / k value (the map, then one rounding to the token type)
    auto mapqk = [&](float x, float rn) {
        float y = x;
        if (qkm == kQkL2) y = x * rn;
        else if (qkm == kQkElu1) y = x > 0.f ? x + 1.f : __expf(x);
        return to_f32(from_f32<T>(y));
    };

    // Stage the slice held in register set S (kKS key channels of q and k, and
    // the per-channel log-gate as its prefix within the chunk) into xs, ys
    // (gs), fp32.
    auto stage_qk = [&](const Slice& S) {
        __syncthreads();
#pragma unroll
        for (int j = 0; j < PP; ++j) {
            int row, cq;
            if (!grp(j, row, cq)) continue;
            const bool ok = row < nrow;
            // (the map branches are uniform and taken once per group; values of
            // the token type pass through unmapped exactly)
            floatx4 xq = cvt4(S.q[j]), xk = cvt4(S.k[j]);
            if (qkm != kQkAsIs) {
                const float rnq = rq[row], rnk = rk[row];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    xq[i] = mapqk(xq[i], rnq);
                    xk[i] = mapqk(xk[i], rnk);
                }
            }
            if (!ok) xq = xk = zero4();
            *reinterpret_cast<floatx4*>(&xs[row * kLDS + cq]) = xq;
            *reinterpret_cast<floatx4*>(&ys[row * kLDS + cq]) = xk;
            if constexpr (CHAN) {
                floatx4 xg = cvt4(S.g[j]);
                if (prep_gate_map(prep)) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) xg[i] = prep_gate(xg[i], prep);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) xg[i] *= kLog2e;
                if (!ok) xg = zero4();
                *reinterpret_cast<floatx4*>(&gs[row * kLDS + cq]) = xg;
            }
        }
        if constexpr (CHAN) {
            // prefix along the rows of each channel: 16-row blocks in parallel,
            // then the block totals carried
            __syncthreads();
            const int c = tid % kKS, b = tid / kKS;
            float acc = 0.f;
            if (b < NB) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    acc += gs[(16 * b + r) * kLDS + c];
                    gs[(16 * b + r) * kLDS + c] = acc;
                }
                gtot[b * kKS + c] = acc;
            }
            __syncthreads();
            if (b < NB && b > 0) {
                float off = 0.f;
                for (int bb = 0; bb < b; ++bb) off += gtot[bb * kKS + c];
#pragma unroll
                for (int r = 0; r < 16; ++r) gs[(16 * b + r) * kLDS + c] += off;
            }
        }
        __syncthreads();
    };

    // ---- a2: score tiles, accumulated over the key-channel slices ---------------
    floatx4 xa[MS], xn[MS];
#pragma unroll
    for (int s = 0; s < MS; ++s) { xa[s] = zero4(); xn[s] = zero4(); }
    // the score tiles of the staged slice
    auto score_slice = [&]() {
#pragma unroll
        for (int s = 0; s < MS; ++s) {
            const int p = wave + NW * s;
            if (p >= NTILE) continue;
            int i, j;
            tile_of(p, i, j);
            if constexpr (!CHAN) {
                // x[rr] = q_l . k_m (and k_l . k_m), l = 16 i + g4 + rr, m = 16 j + cl
#pragma unroll
                for (int kk = 0; kk < kKS / 16; ++kk) {
                    const floatx4 bk = load4(&ys[(16 * j + (lane & 15)) * kLDS + 16 * kk + 4 * (lane >> 4)]);
                    xa[s] = mm16<T>(&xs[16 * i * kLDS + 16 * kk], kLDS, bk, xa[s], lane);
                    if constexpr (DELTA) xn[s] = mm16<T>(&ys[16 * i * kLDS + 16 * kk], kLDS, bk, xn[s], lane);
                }
            } else {
                // exact per-channel decay of every pair: 2^(G_lc - G_mc), m <= l
                const int m = 16 * j + (lane & 15), lb = 16 * i + 4 * (lane >> 4);
#pragma unroll 2
                for (int c4 = 0; c4 < kKS; c4 += 4) {
                    const floatx4 km = load4(&ys[m * kLDS + c4]);
                    const floatx4 Gm = load4(&gs[m * kLDS + c4]);
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) {
                        const int l = lb + rr;
                        const floatx4 qv = load4(&xs[l * kLDS + c4]);
                        const floatx4 Gl = load4(&gs[l * kLDS + c4]);
                        floatx4 kv = zero4();
                        if constexpr (DELTA) kv = load4(&ys[l * kLDS + c4]);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float t = m <= l ? km[e] * fast_exp2(Gl[e] - Gm[e]) : 0.f;
                            xa[s][rr] = fmaf(qv[e], t, xa[s][rr]);
                            if constexpr (DELTA) xn[s][rr] = fmaf(kv[e], t, xn[s][rr]);
                        }
                    }
                }
            }
        }
    };
    // slices in pairs through the register sets A, B; the last two refill them
    // with the first two slices again for the second pass
#pragma unroll 1
    for (int sl = 0; sl < NSL; sl += 2) {
        stage_qk(SA);
        load_qk(SA, sl + 2 < NSL ? sl + 2 : 0);
        score_slice();
        stage_qk(SB);
        load_qk(SB, sl + 3 < NSL ? sl + 3 : 1);
        score_slice();
    }
    mfma_settle();
    // Aq to the workspace, beta L to LDS (rows l = 16 i + g4 + rr, column m)
#pragma unroll
    for (int s = 0; s < MS; ++s) {
        const int p = wave + NW * s;
        if (p >= NTILE) continue;
        int i, j;
        tile_of(p, i, j);
        const int m = 16 * j + (lane & 15), l0 = 16 * i + 4 * (lane >> 4);
        // branch-free: the row values read once as vectors, the decay of every
        // position formed (its exponent clamped at 0 above the diagonal) and
        // masked by selects
        const float Gm = Gsc[m];
        const floatx4 Gl = *reinterpret_cast<const floatx4*>(&Gsc[l0]);
        const floatx4 bl = *reinterpret_cast<const floatx4*>(&bet[l0]);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int l = l0 + rr;
            const float dec = (GATED && !CHAN) ? fast_exp2(fminf(Gl[rr] - Gm, 0.f)) : 1.f;
            if (has(chunk_of(l)))
                reinterpret_cast<T*>(wsp(chunk_of(l), L.aq))[row_in(l) * CH + row_in(m)] =
                    from_f32<T>(m <= l ? xa[s][rr] * dec : 0.f);
            if constexpr (DELTA) lmb(l >> 4, m >> 4)[(l & 15) * LDB + (m & 15)] = m < l ? bl[rr] * xn[s][rr] * dec : 0.f;
        }
    }
    __syncthreads();

    if constexpr (DELTA) {
        // ---- a3: T = (I + beta L)^-1.  Diagonal block i: wave i % NW, lane group
        // i / NW, lane column jj; rows by forward substitution -------------------
        {
            const int jj = lane & 15, i = wave + NW * (lane >> 4);
            if (i < NB) {
                float x[16];
#pragma unroll
                for (int t = 0; t < 16; ++t) {
                    float acc = t == jj ? 1.f : 0.f;
#pragma unroll
                    for (int s2 = 0; s2 < t; ++s2) acc = fmaf(-lmb(i, i)[t * LDB + s2], x[s2], acc);
                    x[t] = acc;
                }
#pragma unroll
                for (int t = 0; t < 16; ++t) lmb(i, i)[t * LDB + jj] = x[t];
            }
        }
        __syncthreads();
        // blocks below the diagonal, column by column:
        // T(i, j) = -T(i, i) sum_{kb = j}^{i - 1} L(i, kb) T(kb, j).
        // Column j needs only its own blocks above row i, so wave j walks it down
        // the rows with no barrier, holding the column in registers; L(i, j) is
        // still read by the columns left of j, so the column goes to LDS (over
        // L) after one barrier.  (Same products in the same order as row by row.)
        // With several chunks per tile only the blocks inside a chunk are solved.
        static_assert(NW >= NB - 1, "one column block per wave");
        {
            floatx4 Tc[NB];
            const int j = wave;
            const bool col = j < NB - 1 && (SUB == 1 || j % BC < BC - 1);   // column with blocks below it in its chunk
            if (col) {
                Tc[0] = zero4();
#pragma unroll
                for (int b = 0; b < NB; ++b)
                    if (b == j) Tc[b] = load_tile_rl(lmb(b, b), LDB, lane);   // T(j, j)
#pragma unroll
                for (int i = 1; i < NB; ++i) {
                    if (i <= j || (SUB > 1 && i / BC != j / BC)) continue;
                    floatx4 X = zero4();
#pragma unroll
                    for (int kb = 0; kb < NB - 1; ++kb)
                        if (kb >= j && kb < i) X = mm16<float>(lmb(i, kb), LDB, Tc[kb], X, lane);
                    const floatx4 t = mm16<float>(lmb(i, i), LDB, X, zero4(), lane);
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) Tc[i][rr] = -t[rr];
                }
            }
            mfma_settle();
            __syncthreads();
            if (col) {
#pragma unroll
                for (int i = 1; i < NB; ++i) {
                    if (i <= j || (SUB > 1 && i / BC != j / BC)) continue;
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr)
                        lmb(i, j)[(4 * (lane >> 4) + rr) * LDB + (lane & 15)] = Tc[i][rr];
                }
            }
            __syncthreads();
        }
    }

    // ---- products T (beta X) for the staged slice in xs: tiles (lb, cb) of a
    // [C][kKS] block, written to dst (row stride ld) at column c0 --------------
    auto tb_product = [&](size_t off, int ld, int c0) {
        for (int p = wave; p < NB * (kKS / 16); p += NW) {
            const int lb = p / (kKS / 16), cb = p % (kKS / 16);
            floatx4 acc = zero4();
            for (int mb = SUB == 1 ? 0 : (lb / BC) * BC; mb <= lb; ++mb)
                acc = mm16<T>(lmb(lb, mb), LDB, load_tile_rl(&xs[16 * mb * kLDS + 16 * cb], kLDS, lane),
                              acc, lane);
            mfma_settle();
            const int sc = chunk_of(16 * lb);              // the chunk of block row lb
            if (has(sc)) {
                T* const dst = reinterpret_cast<T*>(wsp(sc, off));
#pragma unroll
                for (int rr = 0; rr < 4; ++rr)
                    dst[(row_in(16 * lb) + 4 * (lane >> 4) + rr) * ld + c0 + 16 * cb + (lane & 15)] =
                        from_f32<T>(acc[rr]);
            }
        }
    };

    // four values as the token type, one 8- or 16-byte store
    auto st4 = [](T* dst, floatx4 y) {
        R4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = from_f32<T>(y[i]);
        *reinterpret_cast<R4*>(dst) = w;
    };
    // ---- operands of the state pass for the staged slice sl ----------------------
    auto operands = [&](int sl) {
        const int c0 = sl * kKS;
        // <-Q: four channels of a row per thread
#pragma unroll
        for (int j = 0; j < PP; ++j) {
            int row, cq;
            if (!grp(j, row, cq)) continue;
            const floatx4 x = *reinterpret_cast<const floatx4*>(&xs[row * kLDS + cq]);
            floatx4 y;
            if constexpr (CHAN) {
                const floatx4 G = *reinterpret_cast<const floatx4*>(&gs[row * kLDS + cq]);
#pragma unroll
                for (int i = 0; i < 4; ++i) y[i] = x[i] * fast_exp2(G[i]);
            } else {
                const float d = GATED ? fast_exp2(Gsc[row]) : 1.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) y[i] = x[i] * d;
            }
            if (has(chunk_of(row))) st4(&reinterpret_cast<T*>(wsp(chunk_of(row), L.qd))[row_in(row) * DK + c0 + cq], y);
        }
        // ->K^T: four channels of a row per thread, rows fastest across lanes
        // (one vector LDS read; each of the four stores is contiguous across lanes)
#pragma unroll
        for (int j = 0; j < PP; ++j) {
            const int e = tid + j * kGT;
            if (PE % kGT != 0 && e >= PE) continue;
            const int r = e % C, c4 = 4 * (e / C);
            const floatx4 x = *reinterpret_cast<const floatx4*>(&ys[r * kLDS + c4]);
            floatx4 y;
            if constexpr (CHAN) {
                const floatx4 G = *reinterpret_cast<const floatx4*>(&gs[r * kLDS + c4]);
                const floatx4 Ge = *reinterpret_cast<const floatx4*>(&gs[(C - 1) * kLDS + c4]);
#pragma unroll
                for (int i = 0; i < 4; ++i) y[i] = x[i] * fast_exp2(Ge[i] - G[i]);
            } else {
                const float d = GATED ? fast_exp2(Gsc[chunk_of(r) * CH + CH - 1] - Gsc[r]) : 1.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) y[i] = x[i] * d;
            }
            if (has(chunk_of(r))) {
                T* const krt = reinterpret_cast<T*>(wsp(chunk_of(r), L.krt));
#pragma unroll
                for (int i = 0; i < 4; ++i) krt[(c0 + c4 + i) * CH + row_in(r)] = from_f32<T>(y[i]);
            }
        }
        if (tid < SUB * kKS && has(tid / kKS)) {
            const int sc = tid / kKS, c = tid % kKS;
            reinterpret_cast<float*>(wsp(sc, L.gc))[c0 + c] =
                GATED ? fast_exp2(CHAN ? gs[(C - 1) * kLDS + c] : Gsc[sc * CH + CH - 1]) : 1.f;
        }
        if constexpr (DELTA) {
            // W = T (beta <-K): xs <- beta_m 2^(G_m) k_m
            __syncthreads();
#pragma unroll
            for (int j = 0; j < PP; ++j) {
                int row, cq;
                if (!grp(j, row, cq)) continue;
                const floatx4 x = *reinterpret_cast<const floatx4*>(&ys[row * kLDS + cq]);
                floatx4 y;
                if constexpr (CHAN) {
                    const floatx4 G = *reinterpret_cast<const floatx4*>(&gs[row * kLDS + cq]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) y[i] = bet[row] * fast_exp2(G[i]) * x[i];
                } else {
                    const float d = bet[row] * (GATED ? fast_exp2(Gsc[row]) : 1.f);
#pragma unroll
                    for (int i = 0; i < 4; ++i) y[i] = d * x[i];
                }
                *reinterpret_cast<floatx4*>(&xs[row * kLDS + cq]) = y;
            }
            __syncthreads();
            tb_product(L.w, DK, c0);
        }
    };
    // the last two slices refill A, B with the first two value slices
#pragma unroll 1
    for (int sl = 0; sl < NSL; sl += 2) {
        stage_qk(SA);
        if (sl + 2 < NSL) load_qk(SA, sl + 2);
        else if (DELTA) load_v(SA, 0);
        operands(sl);
        stage_qk(SB);
        if (sl + 3 < NSL) load_qk(SB, sl + 3);
        else if (DELTA) load_v(SB, 1);
        operands(sl + 1);
    }
    if constexpr (DELTA) {
        // U = T (beta V), kKS value columns at a time
        auto u_slice = [&](const Slice& S, int vs) {
            __syncthreads();
#pragma unroll
            for (int j = 0; j < PP; ++j) {
                int row, cq;
                if (!grp(j, row, cq)) continue;
                const bool ok = row < nrow;
                const floatx4 vv = cvt4(S.q[j]);
                floatx4 y;
#pragma unroll
                for (int i = 0; i < 4; ++i) y[i] = ok ? bet[row] * vv[i] : 0.f;
                *reinterpret_cast<floatx4*>(&xs[row * kLDS + cq]) = y;
            }
            __syncthreads();
            tb_product(L.u, DV, vs * kKS);
        };
        const int nvs = DV / kKS;
#pragma unroll 1
        for (int vs = 0; vs < nvs; vs += 2) {
            u_slice(SA, vs);
            if (vs + 2 < nvs) load_v(SA, vs + 2);
            u_slice(SB, vs + 1);
            if (vs + 3 < nvs) load_v(SB, vs + 3);
        }
    }
}

// ===========================================================================
// State pass + output
// ===========================================================================
// One workgroup per (b, h, 64 value columns), 8 waves.  Waves 0..3 each own 16
// value columns of S (fp32 result tiles, for the whole sequence); waves 4..7
// copy each 16-row block's operands from the workspace into LDS: W and <-Q
// rows, the block's 16 columns of ->K^T, the block's row of Aq, U (the values
// for the add rule) at the workgroup's columns, and 2^(G_{C-1}) of its chunk.
// A block's operands are loaded into registers three blocks ahead (three
// register sets, so a load has two blocks' time to arrive) and written into
// one of two LDS buffers while the state waves compute from the other; one
// barrier per block.  Every load is issued unconditionally (indices clamped),
// and the helpers run a multiple of three blocks (spare ones copy nothing), so
// the compiler's wait counts stay exact.
template <typename T, int C, int DK>
struct GenStage {
    static constexpr int PAD = 16 / (int)sizeof(T);
    static constexpr int E = 16 / (int)sizeof(T);  // elements per 16-byte vector
    static constexpr int LDK = DK + PAD;            // W, <-Q rows: [16][DK]
    static constexpr int LDT = 16 + PAD;            // ->K^T block: [DK][16]
    static constexpr int LDA = C + PAD;             // Aq row block: [16][C]
    static constexpr int LDU = 64 + PAD;            // U / V: [16][64]
    static constexpr int W = 0, Q = W + 16 * LDK, KR = Q + 16 * LDK, A = KR + DK * LDT, U = A + 16 * LDA;
    static constexpr int ELEMS = U + 16 * LDU;
    // 16-byte vectors of each piece, and per helper thread (256 threads)
    static constexpr int VW = 16 * DK / E, VKR = DK * 16 / E, VA = 16 * C / E, VU = 16 * 64 / E, VG = DK / 4;
    static constexpr int NW = (VW + 255) / 256, NKR = (VKR + 255) / 256, NA = (VA + 255) / 256,
                         NU = (VU + 255) / 256;
};

template <typename T, int C, int DK>
struct GenRegs {
    using G = GenStage<T, C, DK>;
    typedef __attribute__((__vector_size__(16))) int i4;
    i4 w[G::NW], q[G::NW], kr[G::NKR], a[G::NA], u[G::NU], g;
};

template <typename T, int C, int DK, int RULE>
__global__ __launch_bounds__(512, 1) void gen_chain_kernel(
    const T* __restrict__ v, const unsigned char* __restrict__ ws, const float* s0, T* __restrict__ o,
    float* s_final, int64_t Tlen, int64_t nchunks, int DV, int nblocks, SegSplit seg)
{
    using F = typename Frag16<T>::type;
    using G = GenStage<T, C, DK>;
    using Regs = GenRegs<T, C, DK>;
    typedef __attribute__((__vector_size__(16))) int i4;
    constexpr int NB = C / 16, ND = DK / 16, E = G::E;
    constexpr bool DELTA = RULE == kRuleDelta;

    __shared__ __align__(16) T stage[2][G::ELEMS];
    __shared__ __align__(16) float gcs[2][DK];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nvb = DV / 64;
    // the value blocks of a head on one XCD (dispatch is round-robin over 8)
    int blk = blockIdx.x;
    if ((nblocks & 7) == 0) blk = (blk & 7) * (nblocks >> 3) + (blk >> 3);
    const int nunit = nvb * seg.n;
    const int64_t bh = blk / nunit;
    const int vb = (blk % nunit) % nvb;
    const int sg = (blk % nunit) / nvb;
    // this workgroup's chunks [rb, re) (segments.h); chunks [0, rb) run the state
    // update alone first
    const int64_t rb = seg.c[sg], re = seg.c[sg + 1];
    const GenWs L = gen_ws(C, DK, DV, (int)sizeof(T), DELTA);
    const int64_t nsteps = re * NB;                // 16-row blocks staged, prefix included
    const int64_t nspad = (nsteps + 2) / 3 * 3;     // the helpers' count, a multiple of 3

    if (wave < 4) {
        // ======== state waves: columns n0..n0+15 of the block ==========================
        const int n0 = vb * 64 + 16 * wave;
        const int cl = lane & 15, g4 = 4 * (lane >> 4);
        floatx4 S[ND];
#pragma unroll
        for (int db = 0; db < ND; ++db)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
                S[db][rr] = s0 ? s0[(bh * DK + 16 * db + g4 + rr) * DV + n0 + cl] : 0.f;
        lds_barrier();                               // block 0 staged
        // prefix pass over chunks [0, rb): Z and the state update, no output
        for (int64_t c = 0; c < rb; ++c) {
            F Sf[ND];
#pragma unroll
            for (int db = 0; db < ND; ++db) Sf[db] = frag16_acc<T>(S[db]);
            floatx4 dS[ND];
#pragma unroll
            for (int db = 0; db < ND; ++db) dS[db] = zero4();
#pragma unroll
            for (int li = 0; li < NB; ++li) {
                const int ln = opaque(lane);
                const int b = (int)((c * NB + li) & 1);
                const T* const st = stage[b];
                floatx4 Z;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) Z[rr] = to_f32(st[G::U + (g4 + rr) * G::LDU + 16 * wave + cl]);
                if constexpr (DELTA) {
                    floatx4 P = zero4();
#pragma unroll
                    for (int db = 0; db < ND; ++db) P = mma16<T>(frag16_lds_sep(st + G::W + 16 * db, G::LDK, ln), Sf[db], P);
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) Z[rr] -= P[rr];
                }
                const F zf = frag16_acc<T>(Z);
#pragma unroll
                for (int db = 0; db < ND; ++db)
                    dS[db] = mma16<T>(frag16_lds_sep(st + G::KR + 16 * db * G::LDT, G::LDT, ln), zf, dS[db]);
                if (li == NB - 1) {
#pragma unroll
                    for (int db = 0; db < ND; ++db) {
                        const floatx4 gd = *reinterpret_cast<const floatx4*>(&gcs[b][16 * db + g4]);
#pragma unroll
                        for (int rr = 0; rr < 4; ++rr) S[db][rr] = gd[rr] * S[db][rr] + dS[db][rr];
                    }
                }
                mfma_settle();
                lds_barrier();
            }
        }
        for (int64_t c = rb; c < re; ++c) {
            const int64_t t0 = c * C;
            F Sf[ND];
#pragma unroll
            for (int db = 0; db < ND; ++db) Sf[db] = frag16_acc<T>(S[db]);
            floatx4 dS[ND];
#pragma unroll
            for (int db = 0; db < ND; ++db) dS[db] = zero4();
            F Zf[NB];
#pragma unroll
            for (int li = 0; li < NB; ++li) {
                const int ln = opaque(lane);
                const int b = (int)((c * NB + li) & 1);
                const T* const st = stage[b];
                // b1: Z = U - W S_r (delta) | V (add; rows past the end staged as zeros)
                floatx4 Z;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) Z[rr] = to_f32(st[G::U + (g4 + rr) * G::LDU + 16 * wave + cl]);
                if constexpr (DELTA) {
                    floatx4 P = zero4();
#pragma unroll
                    for (int db = 0; db < ND; ++db) P = mma16<T>(frag16_lds_sep(st + G::W + 16 * db, G::LDK, ln), Sf[db], P);
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) Z[rr] -= P[rr];
                }
                Zf[li] = frag16_acc<T>(Z);
                // c1: O = <-Q S_r + sum_{mj <= li} Aq(li, mj) Z_mj
                floatx4 O = zero4();
#pragma unroll
                for (int db = 0; db < ND; ++db) O = mma16<T>(frag16_lds_sep(st + G::Q + 16 * db, G::LDK, ln), Sf[db], O);
#pragma unroll
                for (int mj = 0; mj <= li; ++mj) O = mma16<T>(frag16_lds_sep(st + G::A + 16 * mj, G::LDA, ln), Zf[mj], O);
                // ->K_li^T Z_li
#pragma unroll
                for (int db = 0; db < ND; ++db)
                    dS[db] = mma16<T>(frag16_lds_sep(st + G::KR + 16 * db * G::LDT, G::LDT, ln), Zf[li], dS[db]);
                if (li == NB - 1) {
                    // S_{r+1} = Diag(2^(G_{C-1})) S_r + ->K^T Z
#pragma unroll
                    for (int db = 0; db < ND; ++db) {
                        const floatx4 gd = *reinterpret_cast<const floatx4*>(&gcs[b][16 * db + g4]);
#pragma unroll
                        for (int rr = 0; rr < 4; ++rr) S[db][rr] = gd[rr] * S[db][rr] + dS[db][rr];
                    }
                }
                mfma_settle();   // O is read inside the row-bounds branches below
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int64_t row = t0 + 16 * li + g4 + rr;
                    if (row < Tlen) o[(bh * Tlen + row) * DV + n0 + cl] = from_f32<T>(O[rr]);
                }
                lds_barrier();
            }
        }
        for (int64_t s = nsteps; s < nspad; ++s) lds_barrier();
        if (s_final && sg == seg.n - 1) {
#pragma unroll
            for (int db = 0; db < ND; ++db)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) s_final[(bh * DK + 16 * db + g4 + rr) * DV + n0 + cl] = S[db][rr];
        }
        return;
    }

    // ======== helper waves: thread ht of 256 ==========================================
    const int ht = threadIdx.x - 256;
    const int64_t lastb = nsteps > 0 ? nsteps - 1 : 0;
    // the operands of block s into R (s clamped to the last block)
    auto hload = [&](Regs& R, int64_t s) {
        s = s < lastb ? s : lastb;
        const int64_t c = s / NB;
        const int li = (int)(s % NB);
        const unsigned char* wc = ws + (bh * nchunks + c) * L.bytes;
#pragma unroll
        for (int p = 0; p < G::NW; ++p) {
            int i = p * 256 + ht;
            i = i < G::VW ? i : G::VW - 1;
            const int row = i / (DK / E), col = (i % (DK / E)) * E;
            const size_t off = ((size_t)(16 * li + row) * DK + col) * sizeof(T);
            if constexpr (DELTA) R.w[p] = *reinterpret_cast<const i4*>(wc + L.w + off);
            R.q[p] = *reinterpret_cast<const i4*>(wc + L.qd + off);
        }
#pragma unroll
        for (int p = 0; p < G::NKR; ++p) {
            int i = p * 256 + ht;
            i = i < G::VKR ? i : G::VKR - 1;
            const int row = i / (16 / E), col = (i % (16 / E)) * E;
            R.kr[p] = *reinterpret_cast<const i4*>(wc + L.krt + ((size_t)row * C + 16 * li + col) * sizeof(T));
        }
#pragma unroll
        for (int p = 0; p < G::NA; ++p) {
            int i = p * 256 + ht;
            i = i < G::VA ? i : G::VA - 1;
            const int row = i / (C / E), col = (i % (C / E)) * E;
            R.a[p] = *reinterpret_cast<const i4*>(wc + L.aq + ((size_t)(16 * li + row) * C + col) * sizeof(T));
        }
#pragma unroll
        for (int p = 0; p < G::NU; ++p) {
            int i = p * 256 + ht;
            i = i < G::VU ? i : G::VU - 1;
            const int row = i / (64 / E), col = vb * 64 + (i % (64 / E)) * E;
            if constexpr (DELTA) {
                R.u[p] = *reinterpret_cast<const i4*>(wc + L.u + ((size_t)(16 * li + row) * DV + col) * sizeof(T));
            } else {
                const int64_t t = c * C + 16 * li + row;
                R.u[p] = *reinterpret_cast<const i4*>(v + (bh * Tlen + (t < Tlen ? t : Tlen - 1)) * DV + col);
            }
        }
        {
            const int i = ht < G::VG ? ht : G::VG - 1;
            R.g = *reinterpret_cast<const i4*>(wc + L.gc + 16 * i);
        }
    };
    // R (the operands of block s) into LDS buffer s & 1
    auto hstore = [&](const Regs& R, int64_t s) {
        const int64_t c = s / NB;
        const int li = (int)(s % NB);
        T* const st = stage[s & 1];
#pragma unroll
        for (int p = 0; p < G::NW; ++p) {
            const int i = p * 256 + ht;
            if (i < G::VW) {
                const int row = i / (DK / E), col = (i % (DK / E)) * E;
                if constexpr (DELTA) *reinterpret_cast<i4*>(st + G::W + row * G::LDK + col) = R.w[p];
                *reinterpret_cast<i4*>(st + G::Q + row * G::LDK + col) = R.q[p];
            }
        }
#pragma unroll
        for (int p = 0; p < G::NKR; ++p) {
            const int i = p * 256 + ht;
            if (i < G::VKR) {
                const int row = i / (16 / E), col = (i % (16 / E)) * E;
                *reinterpret_cast<i4*>(st + G::KR + row * G::LDT + col) = R.kr[p];
            }
        }
#pragma unroll
        for (int p = 0; p < G::NA; ++p) {
            const int i = p * 256 + ht;
            if (i < G::VA) {
                const int row = i / (C / E), col = (i % (C / E)) * E;
                *reinterpret_cast<i4*>(st + G::A + row * G::LDA + col) = R.a[p];
            }
        }
#pragma unroll
        for (int p = 0; p < G::NU; ++p) {
            const int i = p * 256 + ht;
            if (i < G::VU) {
                const int row = i / (64 / E), col = (i % (64 / E)) * E;
                const bool past = !DELTA && c * C + 16 * li + row >= Tlen;
                *reinterpret_cast<i4*>(st + G::U + row * G::LDU + col) = past ? i4{0, 0, 0, 0} : R.u[p];
            }
        }
        if (ht < G::VG) *reinterpret_cast<i4*>(&gcs[s & 1][4 * ht]) = R.g;
    };
    // block s: stage block s + 1 (held in Rw), load block s + 3 into Rl
    auto hstep = [&](int64_t s, const Regs& Rw, Regs& Rl) {
        if (s + 1 < nsteps) hstore(Rw, s + 1);
        hload(Rl, s + 3);
        lds_barrier();
    };
    Regs R0, R1, R2;
    if (nsteps > 0) {
        hload(R0, 0);
        hload(R1, 1);
        hload(R2, 2);
        hstore(R0, 0);
    }
    lds_barrier();
    for (int64_t s = 0; s < nspad; s += 3) {
        hstep(s, R1, R0);
        hstep(s + 1, R2, R1);
        hstep(s + 2, R0, R2);
    }
}

// A prefix block of the state pass (Z and the state update, no output) costs
// about this fraction of a full block.
constexpr double kGenPrefixCost = 0.6;

template <typename T, int C, int DK, int RULE, int GATE>
hipError_t launch_gen_t(const ChunkProblem& p, hipStream_t s)
{
    const int64_t nchunks = (p.T + C - 1) / C;
    const int64_t bh = p.B * p.H;
    unsigned char* ws = static_cast<unsigned char*>(p.workspace);
    if (nchunks > 0) {
        constexpr int SUB = gen_tile(C, GATE) / C;         // chunks per workgroup
        hipLaunchKernelGGL((gen_intra_kernel<T, C, DK, RULE, GATE>), dim3((unsigned)(bh * ((nchunks + SUB - 1) / SUB))),
                           dim3(64 * gen_waves(gen_tile(C, GATE))), 0, s,
                           static_cast<const T*>(p.q), static_cast<const T*>(p.k), static_cast<const T*>(p.v),
                           static_cast<const T*>(p.g), static_cast<const T*>(p.beta), ws, p.T, nchunks, p.dv,
                           p.prep);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // segments of each head's chunks when the grid leaves CUs idle (segments.h)
    const int64_t nblocks1 = bh * (p.dv / 64);
    const SegSplit sp = seg_split(nchunks, nblocks1, true, p.s0, p.s_final,
                                  (size_t)bh * p.dk * p.dv * sizeof(float), kGenPrefixCost);
    const int nblocks = (int)(nblocks1 * sp.n);
    hipLaunchKernelGGL((gen_chain_kernel<T, C, DK, RULE>), dim3((unsigned)nblocks), dim3(512), 0, s,
                       static_cast<const T*>(p.v), ws, p.s0, static_cast<T*>(p.o), p.s_final, p.T, nchunks, p.dv,
                       nblocks, sp);
    return hipGetLastError();
}

template <typename T, int C, int DK>
hipError_t gen_by_rule_gate(const ChunkProblem& p, hipStream_t s)
{
    if (p.rule == kRuleDelta) {
        if (p.gate == kGateNone) return launch_gen_t<T, C, DK, kRuleDelta, kGateNone>(p, s);
        if (p.gate == kGateScalar) return launch_gen_t<T, C, DK, kRuleDelta, kGateScalar>(p, s);
        return launch_gen_t<T, C, DK, kRuleDelta, kGateChannel>(p, s);
    }
    if (p.gate == kGateNone) return launch_gen_t<T, C, DK, kRuleAdd, kGateNone>(p, s);
    if (p.gate == kGateScalar) return launch_gen_t<T, C, DK, kRuleAdd, kGateScalar>(p, s);
    return launch_gen_t<T, C, DK, kRuleAdd, kGateChannel>(p, s);
}

template <typename T, int C>
hipError_t gen_by_dk(const ChunkProblem& p, hipStream_t s)
{
    return p.dk == 64 ? gen_by_rule_gate<T, C, 64>(p, s) : gen_by_rule_gate<T, C, 128>(p, s);
}

template <typename T>
hipError_t gen_by_chunk(const ChunkProblem& p, hipStream_t s)
{
    switch (p.chunk) {
    case 16: return gen_by_dk<T, 16>(p, s);
    case 32: return gen_by_dk<T, 32>(p, s);
    case 64: return gen_by_dk<T, 64>(p, s);
    default: return gen_by_dk<T, 128>(p, s);
    }
}

}  // namespace

bool chunk_gen_supported(const ChunkProblem& p)
{
    return (p.chunk == 16 || p.chunk == 32 || p.chunk == 64 || p.chunk == 128) && (p.dk == 64 || p.dk == 128) &&
           (p.dv == 64 || p.dv == 128) && (p.dtype == kF32 || p.dtype == kBF16);
}

size_t chunk_gen_workspace_bytes(const ChunkProblem& p)
{
    const size_t nchunks = (size_t)((p.T + p.chunk - 1) / p.chunk);
    const GenWs l = gen_ws(p.chunk, p.dk, p.dv, p.dtype == kBF16 ? 2 : 4, p.rule == kRuleDelta);
    return (size_t)(p.B * p.H) * nchunks * l.bytes;
}

hipError_t launch_chunk_gen(const ChunkProblem& p, hipStream_t s)
{
    return p.dtype == kBF16 ? gen_by_chunk<bf16>(p, s) : gen_by_chunk<float>(p, s);
}

}  // namespace linattn
