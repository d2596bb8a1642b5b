// decode_step.hip — one recurrent token per (sequence, head), state in place.
//
// "Linear Attention, Visualized", "DeltaNet: correcting memory collisions"
// (predict v_hat = k S', write beta (v - v_hat) at k) with the scalar gate of
// "Mamba-2: input-dependent scalar decay" or the per-key-channel gate of
// "Gated Linear Attention (GLA)", decayed first as in "Kimi Delta Attention
// (KDA)"; read-out o = q S_t after the write ("Naive linear attention").
//
// With S' = D S (D = I, a I or Diag(a)) everything the step needs from the old
// state is two reductions over the key channels (rows of S):
//     kS' = sum_r k_r d_r S_r        qS' = sum_r q_r d_r S_r
// after which the update S_t = D S + k^T u, u = beta (v - kS') (add rule:
// u = v), and the output o = qS' + (q . k) u are element-wise.  So one
// workgroup streams its head's dk x dv fp32 state through registers once: read
// (coalesced 16-byte loads), reduce (wave shuffles + one LDS exchange between
// the four waves), write back in place.  The kernel is HBM-bound: 8 dk dv
// bytes of state traffic per head against about 7 dk dv flops.
#include "device_common.h"
#include "launch.h"

namespace linattn {

template <typename T, int DK, int DV, int RULE, int GATE>
__global__ __launch_bounds__(256) void decode_step_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ g, const T* __restrict__ beta, float* __restrict__ state,
    T* __restrict__ o)
{
    constexpr int NT = 256;
    constexpr int CG = DV / 4;           // threads across a row, 4 columns each
    constexpr int RG = NT / CG;          // row groups
    constexpr int ROWS = DK / RG;        // contiguous rows per thread
    constexpr int WAVES = NT / kWave;
    constexpr int RG_PER_WAVE = kWave / CG;
    static_assert(DV % 4 == 0 && NT % CG == 0 && DK % RG == 0, "tile shape");
    static_assert(RG_PER_WAVE >= 1 && (RG_PER_WAVE & (RG_PER_WAVE - 1)) == 0, "shape");

    __shared__ float red[WAVES][2 * DV + 1];

    const int64_t head = blockIdx.x;
    const int tid = threadIdx.x;
    const int cg = tid % CG;
    const int rg = tid / CG;
    const int r0 = rg * ROWS;
    const int lane = tid % kWave;
    const int wave = tid / kWave;

    float* S = state + head * (int64_t)(DK * DV) + cg * 4;

    // 1. the state rows of this thread, issued first so the loads overlap
    floatx4 s[ROWS];
#pragma unroll
    for (int m = 0; m < ROWS; ++m)
        s[m] = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(S + (r0 + m) * DV));

    // 2. token values for the rows and columns this thread touches
    const T* qh = q + head * DK + r0;
    const T* kh = k + head * DK + r0;
    float qr[ROWS], kr[ROWS], dr[ROWS];
#pragma unroll
    for (int m = 0; m < ROWS; ++m) {
        qr[m] = to_f32(qh[m]);
        kr[m] = to_f32(kh[m]);
    }
    float a = 1.f;
    if constexpr (GATE == kGateScalar) a = expf(to_f32(g[head]));
#pragma unroll
    for (int m = 0; m < ROWS; ++m) {
        if constexpr (GATE == kGateChannel) dr[m] = expf(to_f32(g[head * DK + r0 + m]));
        else dr[m] = a;
    }
    float vv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) vv[j] = to_f32(v[head * DV + cg * 4 + j]);
    const float b = (RULE == kRuleDelta) ? to_f32(beta[head]) : 0.f;

    // 3. partial reductions over this thread's rows: kS', qS', q.k
    float kp[4] = {0.f, 0.f, 0.f, 0.f}, qp[4] = {0.f, 0.f, 0.f, 0.f}, qk = 0.f;
#pragma unroll
    for (int m = 0; m < ROWS; ++m) {
        const float kd = kr[m] * (GATE == kGateChannel ? dr[m] : 1.f);
        const float qd = qr[m] * (GATE == kGateChannel ? dr[m] : 1.f);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if constexpr (RULE == kRuleDelta) kp[j] = fmaf(kd, s[m][j], kp[j]);
            qp[j] = fmaf(qd, s[m][j], qp[j]);
        }
        qk = fmaf(qr[m], kr[m], qk);
    }
    // across the row groups inside the wave (lanes CG apart share columns)
#pragma unroll
    for (int off = CG; off < kWave; off <<= 1) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if constexpr (RULE == kRuleDelta) kp[j] += shfl_xor(kp[j], off);
            qp[j] += shfl_xor(qp[j], off);
        }
        qk += shfl_xor(qk, off);
    }
    // across the waves through LDS
    if (lane < CG) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            red[wave][cg * 4 + j] = kp[j];
            red[wave][DV + cg * 4 + j] = qp[j];
        }
        if (lane == 0) red[wave][2 * DV] = qk;
    }
    __syncthreads();
    float kS[4], qS[4];
    qk = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) { kS[j] = 0.f; qS[j] = 0.f; }
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            kS[j] += red[w][cg * 4 + j];
            qS[j] += red[w][DV + cg * 4 + j];
        }
        qk += red[w][2 * DV];
    }
    if constexpr (GATE == kGateScalar) {
#pragma unroll
        for (int j = 0; j < 4; ++j) { kS[j] *= a; qS[j] *= a; }
    }

    // 4. correction u, state write-back, read-out
    float u[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) u[j] = (RULE == kRuleDelta) ? b * (vv[j] - kS[j]) : vv[j];
#pragma unroll
    for (int m = 0; m < ROWS; ++m) {
        floatx4 n;
#pragma unroll
        for (int j = 0; j < 4; ++j) n[j] = fmaf(kr[m], u[j], dr[m] * s[m][j]);
        __builtin_nontemporal_store(n, reinterpret_cast<floatx4*>(S + (r0 + m) * DV));
    }
    if (rg == 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) o[head * DV + cg * 4 + j] = from_f32<T>(fmaf(qk, u[j], qS[j]));
    }
}

template <typename T, int DK, int DV, int RULE, int GATE>
static hipError_t launch_one(const DecodeProblem& p, hipStream_t stream)
{
    const int64_t heads = p.N * p.H;
    hipLaunchKernelGGL((decode_step_kernel<T, DK, DV, RULE, GATE>), dim3((unsigned)heads), dim3(256),
                       0, stream, static_cast<const T*>(p.q), static_cast<const T*>(p.k),
                       static_cast<const T*>(p.v), static_cast<const T*>(p.g),
                       static_cast<const T*>(p.beta), p.state, static_cast<T*>(p.o));
    return hipGetLastError();
}

template <typename T, int DK, int DV>
static hipError_t by_rule_gate(const DecodeProblem& p, hipStream_t s)
{
    if (p.rule == kRuleAdd) {
        if (p.gate == kGateNone) return launch_one<T, DK, DV, kRuleAdd, kGateNone>(p, s);
        if (p.gate == kGateScalar) return launch_one<T, DK, DV, kRuleAdd, kGateScalar>(p, s);
        return launch_one<T, DK, DV, kRuleAdd, kGateChannel>(p, s);
    }
    if (p.gate == kGateNone) return launch_one<T, DK, DV, kRuleDelta, kGateNone>(p, s);
    if (p.gate == kGateScalar) return launch_one<T, DK, DV, kRuleDelta, kGateScalar>(p, s);
    return launch_one<T, DK, DV, kRuleDelta, kGateChannel>(p, s);
}

template <typename T>
static hipError_t by_dims(const DecodeProblem& p, hipStream_t s)
{
    if (p.dk == 64 && p.dv == 64) return by_rule_gate<T, 64, 64>(p, s);
    if (p.dk == 64 && p.dv == 128) return by_rule_gate<T, 64, 128>(p, s);
    if (p.dk == 128 && p.dv == 64) return by_rule_gate<T, 128, 64>(p, s);
    return by_rule_gate<T, 128, 128>(p, s);
}

hipError_t launch_decode_step(const DecodeProblem& p, hipStream_t stream)
{
    if (p.dtype == kBF16) return by_dims<bf16>(p, stream);
    return by_dims<float>(p, stream);
}

}  // namespace linattn
