// launch.h — internal interface between the C-ABI layer (linattn_api.hip) and
// the kernel files.  Problems arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace linattn {

enum { kRuleAdd = 0, kRuleDelta = 1 };
enum { kGateNone = 0, kGateScalar = 1, kGateChannel = 2 };
enum { kF32 = 0, kBF16 = 1 };

struct DecodeProblem {
    int64_t N, H;
    int dk, dv, rule, gate, dtype;
    const void *q, *k, *v, *g, *beta;
    float* state;
    void* o;
};

struct ChunkProblem {
    int64_t B, H, T;
    int dk, dv, chunk, rule, gate, dtype;
    const void *q, *k, *v, *g, *beta;
    const float* s0;
    void* o;
    float* s_final;
    void* workspace;
    size_t workspace_bytes;
    int prep;          // input preparation flags (prep.h); the single-pass kernels only
};

hipError_t launch_decode_step(const DecodeProblem& p, hipStream_t stream);

// Gated DeltaProduct over its virtual sequence: the expanded query and
// log-gate (qv [B,H,T*nh,dk], gv [B,H,T*nh] or NULL), and the gather of every
// nh-th output of the virtual sequence (ov [B,H,T*nh,dv]) into o [B,H,T,dv].
struct DeltaProductProblem {
    int64_t B, H, T;
    int nh, dk, dv, dtype;
    const void *q, *g;
    void *qv, *gv;
    const void* ov;
    void* o;
};
hipError_t launch_dp_expand(const DeltaProductProblem& p, hipStream_t stream);
hipError_t launch_dp_gather(const DeltaProductProblem& p, hipStream_t stream);
// backward: dO of the virtual outputs (do at every nh-th step, zero between),
// and the pick of row j of every group of nh virtual rows (width w; w = 1 for
// one value per row)
hipError_t launch_dp_scatter(const DeltaProductProblem& p, const void* dout, void* dov, hipStream_t stream);
hipError_t launch_dp_pick(const void* src, void* dst, int64_t rows, int nh, int j, int w, int dtype,
                          hipStream_t stream);

// Normalised linear attention as two add-rule passes (values, then a block of
// ones started at z0): the block of ones and its initial state before them;
// o /= den (column 0 of the second pass's output) and z_T = column 0 of its
// final state after them.
struct NormalizedProblem {
    int64_t rows, heads;          // B*H*T token rows, B*H heads
    int dk, dv, dtype;
    void* ones;                   // [rows][normalized_ones_columns()] token dtype
    const float* z0;              // [heads][dk] or NULL
    float* s0_den;                // [heads][dk][normalized_ones_columns()]
    void* o;                      // [rows][dv] numerator in, output out
    const void* den;              // [rows][normalized_ones_columns()]
    const float* sf_den;          // [heads][dk][normalized_ones_columns()]
    float* z_final;               // [heads][dk] or NULL
};
int normalized_ones_columns();
hipError_t launch_norm_prepare(const NormalizedProblem& p, hipStream_t stream);
hipError_t launch_norm_finish(const NormalizedProblem& p, hipStream_t stream);

// Single-pass chunk kernel (gate NONE or SCALAR), three phases per chunk.
bool chunk_fused_supported(const ChunkProblem& p);
hipError_t launch_chunk_fused(const ChunkProblem& p, hipStream_t stream);
// The same kernel also writing the state entering every chunk,
// states [B,H,nchunks,dk,dv] in the token type (for the backward pass).
hipError_t launch_chunk_fused_save(const ChunkProblem& p, void* states, hipStream_t stream);
// The same kernel for normalised linear attention (add rule, gate NONE or
// SCALAR): it also carries the key sum z (z0, z_final [B,H,dk] fp32, either
// may be NULL for zero / not wanted) and writes o_t = (q_t S_t) / (q_t . z_t).
hipError_t launch_chunk_fused_normalized(const ChunkProblem& p, const float* z0, float* z_final,
                                         hipStream_t stream);
// Single-pass chunk kernel for bf16 tokens (gate NONE or SCALAR), pipelined:
// chunk r+1's intra-chunk work beside chunk r's state pass.
bool chunk_pipe_supported(const ChunkProblem& p);
hipError_t launch_chunk_pipe(const ChunkProblem& p, hipStream_t stream);
// The same kernel over the virtual sequence of Gated DeltaProduct (delta rule,
// p.T = T nh substeps): q, g and o in the real [B,H,T] layout, k, v and beta in
// the virtual one; no expand or gather pass.
hipError_t launch_chunk_pipe_virtual(const ChunkProblem& p, int nh, hipStream_t stream);

// Two-kernel chunk path (intra-chunk precompute, then the state pass with the
// output); used for the per-channel gate.
bool chunk_split_supported(const ChunkProblem& p);
size_t chunk_split_workspace_bytes(const ChunkProblem& p);
hipError_t launch_chunk_split(const ChunkProblem& p, hipStream_t stream);
// The same, also writing the state entering every chunk, states
// [B,H,nchunks,dk,dv] bf16 (for the backward pass).
hipError_t launch_chunk_split_save(const ChunkProblem& p, void* states, hipStream_t stream);

// Generic two-kernel chunk path (intra-chunk operands to the workspace, then
// the state pass): every chunk size 16, 32, 64, 128, fp32 or bf16 tokens,
// every rule and gate, input maps of prep.h.
bool chunk_gen_supported(const ChunkProblem& p);
size_t chunk_gen_workspace_bytes(const ChunkProblem& p);
hipError_t launch_chunk_gen(const ChunkProblem& p, hipStream_t stream);

// Backward pass of the chunk form (chunk 64; the per-channel gate with bf16
// tokens): given the incoming state of every chunk (states), the per-chunk
// operands of the reverse state pass are prepared, the gradients of the
// outgoing states are carried newest chunk first (dstates, ds0), and every
// chunk's gradients are then formed independently.
struct ChunkBwdProblem {
    int64_t B, H, T;
    int dk, dv, rule, gate, dtype;
    const void *q, *k, *v, *g, *beta, *dout;
    const void* states;           // [B,H,N,dk,dv] token type, S entering chunk r
    const float* dsT;             // [B,H,dk,dv] or NULL
    void *dq, *dk_out, *dv_out, *dg, *dbeta;
    float* ds0;                   // [B,H,dk,dv] or NULL
    void* ops;                    // [B,H,N] chunk operand blocks (chunk_bwd_ops_bytes each)
    float* gC;                    // [B,H,N] exp of the chunk's total log-gate ([B,H,N,dk] per channel)
    void* dstates;                // [B,H,N,dv/16,dk,16] token type, gradient w.r.t. S leaving chunk r
};
bool chunk_bwd_supported(int dk, int dv, int rule, int gate, int dtype);
size_t chunk_bwd_ops_bytes(int dk, int gate, int dtype);
hipError_t launch_chunk_bwd(const ChunkBwdProblem& p, hipStream_t stream);

}  // namespace linattn
