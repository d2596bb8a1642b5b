// linattn_api.hip — the C ABI declared in include/linattn.h: argument
// validation (before anything is enqueued) and dispatch to the kernels.
#include "../../include/linattn.h"
#include "launch.h"

#include <hip/hip_runtime.h>

#include <cstdlib>
#include <cstring>
#include <mutex>

using namespace linattn;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool mul_ok(int64_t a, int64_t b, int64_t* out) { return !__builtin_mul_overflow(a, b, out); }

bool head_dim_ok(int d) { return d == 64 || d == 128; }

// Which chunk path serves a problem.  Chunk 64 (the default) with bf16 tokens,
// or fp32 tokens at dk = 64 with gate NONE or SCALAR, takes a tuned path: the
// per-channel gate the two-kernel path, the delta rule with bf16 tokens the
// pipelined single-pass kernel (its intra-chunk work is large enough to pay
// for the pipelining), everything else the three-phase one.  Every other
// chunk size, fp32 tokens at dk = 128 and fp32 tokens with the per-channel
// gate take the generic two-kernel path.  LINATTN_CHUNK_PATH=split, =fused,
// =pipe or =gen selects that path instead (for A/B measurement) where it
// supports the problem.
enum ChunkPath { kPathSplit, kPathFused, kPathPipe, kPathGen };
ChunkPath chunk_path(const ChunkProblem& p)
{
    const char* e = getenv("LINATTN_CHUNK_PATH");
    if (e && strcmp(e, "gen") == 0 && chunk_gen_supported(p)) return kPathGen;
    if (p.chunk != 64 || (p.dtype == kF32 && (p.dk != 64 || p.gate == kGateChannel))) return kPathGen;
    if (p.gate == kGateChannel) return kPathSplit;
    if (e && strcmp(e, "split") == 0 && chunk_split_supported(p)) return kPathSplit;
    if (e && strcmp(e, "fused") == 0 && chunk_fused_supported(p)) return kPathFused;
    if (e && strcmp(e, "pipe") == 0 && chunk_pipe_supported(p)) return kPathPipe;
    return p.dtype == kBF16 && p.rule == kRuleDelta ? kPathPipe : kPathFused;
}

// Workspace the chosen path needs (the two-kernel paths stage per-chunk
// operands in it; the single-pass kernels need none).
size_t path_workspace_bytes(const ChunkProblem& p)
{
    switch (chunk_path(p)) {
    case kPathSplit: return chunk_split_workspace_bytes(p);
    case kPathGen: return chunk_gen_workspace_bytes(p);
    default: return 0;
    }
}

linattn_status check_enums(int rule, int gate, int dtype)
{
    if (rule != LINATTN_RULE_ADD && rule != LINATTN_RULE_DELTA) return LINATTN_ERR_ARG;
    if (gate != LINATTN_GATE_NONE && gate != LINATTN_GATE_SCALAR && gate != LINATTN_GATE_CHANNEL)
        return LINATTN_ERR_ARG;
    if (dtype != LINATTN_F32 && dtype != LINATTN_BF16) return LINATTN_ERR_ARG;
    return LINATTN_OK;
}

// Shared pointer checks: required tensors present, gate/beta present exactly
// when the rule/gate need them, everything 16-byte aligned.
linattn_status check_pointers(int rule, int gate, const void* q, const void* k, const void* v,
                              const void* g, const void* beta, const void* st, const void* o)
{
    if (!q || !k || !v || !o || !st) return LINATTN_ERR_NULL;
    if ((gate == LINATTN_GATE_NONE) != (g == nullptr)) return g ? LINATTN_ERR_ARG : LINATTN_ERR_NULL;
    if ((rule == LINATTN_RULE_DELTA) != (beta != nullptr))
        return beta ? LINATTN_ERR_ARG : LINATTN_ERR_NULL;
    const void* ptrs[] = {q, k, v, g, beta, st, o};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return LINATTN_ERR_UNSUPPORTED;
    return LINATTN_OK;
}

// Input-preparation maps as the kernels' packed flags (prep.h): bits 0-1 the
// q/k map, bit 2 the gate map, bit 3 the beta map.
linattn_status prep_flags(const linattn_prep_args* pa, int rule, int gate, int* out)
{
    *out = 0;
    if (!pa) return LINATTN_OK;
    if (pa->qk_map < LINATTN_QK_AS_IS || pa->qk_map > LINATTN_QK_ELU1 ||
        (pa->gate_map != LINATTN_GMAP_AS_IS && pa->gate_map != LINATTN_GMAP_NEG_SOFTPLUS) ||
        (pa->beta_map != LINATTN_BMAP_AS_IS && pa->beta_map != LINATTN_BMAP_SIGMOID))
        return LINATTN_ERR_ARG;
    if (pa->gate_map != LINATTN_GMAP_AS_IS && gate == LINATTN_GATE_NONE) return LINATTN_ERR_ARG;
    if (pa->beta_map != LINATTN_BMAP_AS_IS && rule == LINATTN_RULE_ADD) return LINATTN_ERR_ARG;
    *out = pa->qk_map | (pa->gate_map << 2) | (pa->beta_map << 3);
    return LINATTN_OK;
}

linattn_status validate_chunk(const linattn_chunk_args* a, ChunkProblem* p,
                              const linattn_prep_args* prep = nullptr)
{
    if (!a) return LINATTN_ERR_NULL;
    if (a->B < 0 || a->H < 0 || a->T < 0 || a->dk <= 0 || a->dv <= 0 || a->chunk < 0)
        return LINATTN_ERR_SHAPE;
    linattn_status st = check_enums(a->rule, a->gate, a->dtype);
    if (st != LINATTN_OK) return st;
    int64_t bh, bht, tot;
    if (!mul_ok(a->B, a->H, &bh) || !mul_ok(bh, a->T, &bht) ||
        !mul_ok(bht, (int64_t)(a->dk > a->dv ? a->dk : a->dv), &tot) || bh > (int64_t)INT32_MAX)
        return LINATTN_ERR_SHAPE;
    if (!head_dim_ok(a->dk) || !head_dim_ok(a->dv)) return LINATTN_ERR_UNSUPPORTED;
    p->B = a->B; p->H = a->H; p->T = a->T;
    p->dk = a->dk; p->dv = a->dv;
    p->chunk = a->chunk == 0 ? 64 : a->chunk;
    p->rule = a->rule; p->gate = a->gate; p->dtype = a->dtype;
    st = prep_flags(prep, a->rule, a->gate, &p->prep);
    if (st != LINATTN_OK) return st;
    if (p->chunk != 16 && p->chunk != 32 && p->chunk != 64 && p->chunk != 128) return LINATTN_ERR_UNSUPPORTED;
    const ChunkPath path = chunk_path(*p);
    const bool ok = path == kPathSplit ? chunk_split_supported(*p)
                  : path == kPathPipe  ? chunk_pipe_supported(*p)
                  : path == kPathGen   ? chunk_gen_supported(*p)
                                       : chunk_fused_supported(*p);
    if (!ok) return LINATTN_ERR_UNSUPPORTED;
    // the generic path launches one workgroup per chunk of every head
    if (path == kPathGen && bh * ((a->T + p->chunk - 1) / p->chunk) >= ((int64_t)1 << 31)) return LINATTN_ERR_SHAPE;
    // every chunk kernel addresses one head's output through a buffer resource
    // with a 31-bit byte range
    const int64_t esz = a->dtype == LINATTN_BF16 ? 2 : 4;
    if (a->T * a->dv * esz >= ((int64_t)1 << 31)) return LINATTN_ERR_UNSUPPORTED;
    return LINATTN_OK;
}

// Initial and final state: 16-byte aligned; s_final may alias s0 exactly, but
// must not partially overlap it.
linattn_status check_states(const ChunkProblem& p, const float* s0, const float* s_final)
{
    if ((s0 && !aligned16(s0)) || (s_final && !aligned16(s_final))) return LINATTN_ERR_UNSUPPORTED;
    if (s0 && s_final && s0 != s_final) {
        const char* a0 = reinterpret_cast<const char*>(s0);
        const char* a1 = reinterpret_cast<const char*>(s_final);
        const size_t n = (size_t)(p.B * p.H) * p.dk * p.dv * sizeof(float);
        if (a0 < a1 + n && a1 < a0 + n) return LINATTN_ERR_ARG;
    }
    return LINATTN_OK;
}

// Gated DeltaProduct: the virtual GDN problem (n_h T steps) it runs as.
linattn_status validate_dp(const linattn_deltaproduct_args* a, linattn_chunk_args* va, ChunkProblem* vp)
{
    if (!a) return LINATTN_ERR_NULL;
    if (a->nh < 1 || a->T < 0) return LINATTN_ERR_SHAPE;
    if (a->gate == LINATTN_GATE_CHANNEL) return LINATTN_ERR_UNSUPPORTED;
    int64_t tv;
    if (!mul_ok(a->T, (int64_t)a->nh, &tv)) return LINATTN_ERR_SHAPE;
    *va = linattn_chunk_args{a->B, a->H, tv, a->dk, a->dv, a->chunk, LINATTN_RULE_DELTA, a->gate, a->dtype};
    return validate_chunk(va, vp);
}

// Workspace of an n_h > 1 problem, 256-byte aligned pieces: expanded queries
// [B,H,T*nh,dk], expanded log-gates [B,H,T*nh] (scalar gate), virtual outputs
// [B,H,T*nh,dv], then whatever the chunk path needs.
struct DpLayout {
    size_t qv, gv, ov, cws, total;
};
DpLayout dp_layout(const linattn_chunk_args& va, const ChunkProblem& vp)
{
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t esz = va.dtype == LINATTN_BF16 ? 2 : 4;
    const size_t steps = (size_t)(va.B * va.H) * (size_t)va.T;
    DpLayout l{};
    l.qv = 0;
    l.gv = up(steps * va.dk * esz);
    l.ov = l.gv + (va.gate == LINATTN_GATE_SCALAR ? up(steps * esz) : 0);
    l.cws = l.ov + up(steps * va.dv * esz);
    l.total = l.cws + path_workspace_bytes(vp);
    return l;
}

// Normalised linear attention: the second (denominator) pass's problem and the
// workspace pieces, 256-byte aligned: ones [B,H,T,64], den [B,H,T,64], its
// initial and final states [B,H,dk,64] fp32, then the two-kernel path's
// workspace (shared by both passes, sized for the wider one).
struct NormLayout {
    size_t ones, den, s0d, sfd, cws, total;
};
NormLayout norm_layout(const ChunkProblem& p, const ChunkProblem& pd)
{
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t esz = p.dtype == kBF16 ? 2 : 4;
    const size_t rows = (size_t)(p.B * p.H) * (size_t)p.T;
    const size_t nc = (size_t)normalized_ones_columns();
    NormLayout l{};
    l.ones = 0;
    l.den = up(rows * nc * esz);
    l.s0d = l.den + up(rows * nc * esz);
    l.sfd = l.s0d + up((size_t)(p.B * p.H) * p.dk * nc * 4);
    l.cws = l.sfd + up((size_t)(p.B * p.H) * p.dk * nc * 4);
    const size_t w = path_workspace_bytes(p);
    const size_t wd = path_workspace_bytes(pd);
    l.total = l.cws + (w > wd ? w : wd);
    return l;
}

linattn_status validate_norm(const linattn_chunk_args* a, const linattn_prep_args* prep,
                             linattn_chunk_args* ad, ChunkProblem* p, ChunkProblem* pd)
{
    if (!a) return LINATTN_ERR_NULL;
    if (a->rule != LINATTN_RULE_ADD) return LINATTN_ERR_ARG;
    linattn_status st = validate_chunk(a, p, prep);
    if (st != LINATTN_OK) return st;
    *ad = *a;
    ad->dv = normalized_ones_columns();
    return validate_chunk(ad, pd, prep);
}

// Backward pass and the forward that keeps the chunk states: the problem (gate
// NONE or SCALAR, chunk 64) and its sizes.
linattn_status validate_train(const linattn_chunk_args* a, ChunkProblem* p)
{
    if (!a) return LINATTN_ERR_NULL;
    if (a->B < 0 || a->H < 0 || a->T < 0 || a->dk <= 0 || a->dv <= 0 || a->chunk < 0)
        return LINATTN_ERR_SHAPE;
    linattn_status st = check_enums(a->rule, a->gate, a->dtype);
    if (st != LINATTN_OK) return st;
    int64_t bh, bht, tot;
    if (!mul_ok(a->B, a->H, &bh) || !mul_ok(bh, a->T, &bht) ||
        !mul_ok(bht, (int64_t)(a->dk > a->dv ? a->dk : a->dv), &tot) || bh > (int64_t)INT32_MAX)
        return LINATTN_ERR_SHAPE;
    if (a->chunk != 0 && a->chunk != 64) return LINATTN_ERR_UNSUPPORTED;
    if (!chunk_bwd_supported(a->dk, a->dv, a->rule, a->gate, a->dtype)) return LINATTN_ERR_UNSUPPORTED;
    const int64_t esz = a->dtype == LINATTN_BF16 ? 2 : 4;
    if (a->T * a->dv * esz >= ((int64_t)1 << 31)) return LINATTN_ERR_UNSUPPORTED;
    // every chunk-indexed launch grid stays within 2^31 workgroups
    if (bh * ((a->T + 63) / 64) >= ((int64_t)1 << 31)) return LINATTN_ERR_SHAPE;
    *p = ChunkProblem{};
    p->B = a->B; p->H = a->H; p->T = a->T;
    p->dk = a->dk; p->dv = a->dv; p->chunk = 64;
    p->rule = a->rule; p->gate = a->gate; p->dtype = a->dtype;
    if (p->gate == kGateChannel) return chunk_split_supported(*p) ? LINATTN_OK : LINATTN_ERR_UNSUPPORTED;
    return chunk_fused_supported(*p) ? LINATTN_OK : LINATTN_ERR_UNSUPPORTED;
}

// The state-saving forward: the two-kernel path for the per-channel gate (its
// staged operands in the workspace), the single-pass kernel otherwise.
size_t fwd_save_workspace_bytes(const ChunkProblem& p)
{
    return p.gate == kGateChannel ? chunk_split_workspace_bytes(p) : 0;
}
hipError_t launch_fwd_save(ChunkProblem p, void* states, void* ws, size_t wsb, hipStream_t s)
{
    if (p.gate != kGateChannel) return launch_chunk_fused_save(p, states, s);
    p.workspace = ws;
    p.workspace_bytes = wsb;
    return launch_chunk_split_save(p, states, s);
}

// Backward workspace, 256-byte aligned pieces: chunk operands [B,H,N] blocks,
// exp(G_C) [B,H,N] (per channel: [B,H,N,dk]), dstates [B,H,N,dv/16,dk,16], then
// (states not given) the recomputed states [B,H,N,dk,dv], a forward output
// [B,H,T,dv] and the forward's own workspace, all in the token type except
// exp(G_C).
struct BwdLayout {
    size_t ops, gc, dst, st, o, fws, total;
};
BwdLayout bwd_layout(const ChunkProblem& p, bool states_given)
{
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t bh = (size_t)(p.B * p.H), nch = (size_t)((p.T + 63) / 64);
    const size_t esz = p.dtype == kBF16 ? 2 : 4;
    BwdLayout l{};
    l.ops = 0;
    l.gc = up(bh * nch * chunk_bwd_ops_bytes(p.dk, p.gate, p.dtype));
    l.dst = l.gc + up(bh * nch * (p.gate == kGateChannel ? (size_t)p.dk : 1) * 4);
    l.st = l.dst + up(bh * nch * p.dk * p.dv * esz);
    l.o = l.st + (states_given ? 0 : up(bh * nch * p.dk * p.dv * esz));
    l.fws = l.o + (states_given ? 0 : up(bh * (size_t)p.T * p.dv * esz));
    l.total = l.fws + (states_given ? 0 : up(fwd_save_workspace_bytes(p)));
    return l;
}

// Gated DeltaProduct backward workspace, 256-byte aligned pieces: expanded
// queries and log-gates, the virtual dO, dq and dg, then the chunk backward's
// own workspace for the virtual problem (its states recomputed).
struct DpBwdLayout {
    size_t qv, gv, dov, dqv, dgv, cws, total;
};
DpBwdLayout dp_bwd_layout(const linattn_chunk_args& va, const ChunkProblem& vp)
{
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t esz = va.dtype == LINATTN_BF16 ? 2 : 4;
    const size_t steps = (size_t)(va.B * va.H) * (size_t)va.T;
    const bool gated = va.gate == LINATTN_GATE_SCALAR;
    DpBwdLayout l{};
    l.qv = 0;
    l.gv = up(steps * va.dk * esz);
    l.dov = l.gv + (gated ? up(steps * esz) : 0);
    l.dqv = l.dov + up(steps * va.dv * esz);
    l.dgv = l.dqv + up(steps * va.dk * esz);
    l.cws = l.dgv + (gated ? up(steps * esz) : 0);
    l.total = l.cws + bwd_layout(vp, false).total;
    return l;
}

}  // namespace

extern "C" {

int linattn_abi_version(void) { return LINATTN_ABI_VERSION; }

const char* linattn_status_string(int s)
{
    switch (s) {
    case LINATTN_OK: return "ok";
    case LINATTN_ERR_NULL: return "a required pointer is NULL";
    case LINATTN_ERR_SHAPE: return "invalid or overflowing sizes";
    case LINATTN_ERR_UNSUPPORTED: return "unsupported head size, chunk size, dtype or alignment";
    case LINATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case LINATTN_ERR_LAUNCH: return "kernel launch failed";
    case LINATTN_ERR_ARG: return "inconsistent arguments";
    default: return "unknown status";
    }
}

size_t linattn_chunk_workspace_bytes(const linattn_chunk_args* a)
{
    ChunkProblem p{};
    if (validate_chunk(a, &p) != LINATTN_OK) return 0;
    return path_workspace_bytes(p);
}

linattn_status linattn_chunk_fwd(const linattn_chunk_args* a, const void* q, const void* k,
                                 const void* v, const void* g, const void* beta, const float* s0,
                                 void* o, float* s_final, void* workspace, size_t workspace_bytes,
                                 void* stream)
{
    return linattn_chunk_fwd_prep(a, nullptr, q, k, v, g, beta, s0, o, s_final, workspace,
                                  workspace_bytes, stream);
}

linattn_status linattn_chunk_fwd_prep(const linattn_chunk_args* a, const linattn_prep_args* prep,
                                      const void* q, const void* k, const void* v, const void* g,
                                      const void* beta, const float* s0, void* o, float* s_final,
                                      void* workspace, size_t workspace_bytes, void* stream)
{
    ChunkProblem p{};
    linattn_status st = validate_chunk(a, &p, prep);
    if (st != LINATTN_OK) return st;
    if (p.B * p.H == 0) return LINATTN_OK;
    // q,k,v,o may be absent only when there are no tokens; pass q as the
    // stand-in for the state pointer check in that case.
    if (p.T > 0) {
        st = check_pointers(p.rule, p.gate, q, k, v, g, beta, q, o);
        if (st != LINATTN_OK) return st;
    }
    st = check_states(p, s0, s_final);
    if (st != LINATTN_OK) return st;
    p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta;
    p.s0 = s0; p.o = o; p.s_final = s_final;
    p.workspace = workspace; p.workspace_bytes = workspace_bytes;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t err;
    const ChunkPath path = chunk_path(p);
    if (path == kPathPipe) {
        err = launch_chunk_pipe(p, s);
    } else if (path == kPathFused) {
        err = launch_chunk_fused(p, s);
    } else {
        const size_t need = path_workspace_bytes(p);
        if (need > 0 && (!workspace || workspace_bytes < need)) return LINATTN_ERR_WORKSPACE;
        if (workspace && !aligned16(workspace)) return LINATTN_ERR_UNSUPPORTED;
        err = path == kPathSplit ? launch_chunk_split(p, s) : launch_chunk_gen(p, s);
    }
    return err == hipSuccess ? LINATTN_OK : LINATTN_ERR_LAUNCH;
}

linattn_status linattn_decode_step(const linattn_decode_args* a, const void* q, const void* k,
                                   const void* v, const void* g, const void* beta, float* state,
                                   void* o, void* stream)
{
    if (!a) return LINATTN_ERR_NULL;
    if (a->N < 0 || a->H < 0 || a->dk <= 0 || a->dv <= 0) return LINATTN_ERR_SHAPE;
    linattn_status st = check_enums(a->rule, a->gate, a->dtype);
    if (st != LINATTN_OK) return st;
    int64_t heads, tot;
    if (!mul_ok(a->N, a->H, &heads) || !mul_ok(heads, (int64_t)a->dk * a->dv, &tot) ||
        heads > (int64_t)INT32_MAX)
        return LINATTN_ERR_SHAPE;
    if (!head_dim_ok(a->dk) || !head_dim_ok(a->dv)) return LINATTN_ERR_UNSUPPORTED;
    if (heads == 0) return LINATTN_OK;
    st = check_pointers(a->rule, a->gate, q, k, v, g, beta, state, o);
    if (st != LINATTN_OK) return st;
    DecodeProblem p{a->N, a->H, a->dk, a->dv, a->rule, a->gate, a->dtype,
                    q, k, v, g, beta, state, o};
    hipError_t err = launch_decode_step(p, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? LINATTN_OK : LINATTN_ERR_LAUNCH;
}

size_t linattn_deltaproduct_workspace_bytes(const linattn_deltaproduct_args* a)
{
    linattn_chunk_args va{};
    ChunkProblem vp{};
    if (validate_dp(a, &va, &vp) != LINATTN_OK) return 0;
    if (a->nh == 1) return linattn_chunk_workspace_bytes(&va);
    return dp_layout(va, vp).total;
}

linattn_status linattn_deltaproduct_fwd(const linattn_deltaproduct_args* a, const void* q, const void* k,
                                        const void* v, const void* g, const void* beta, const float* s0,
                                        void* o, float* s_final, void* workspace, size_t workspace_bytes,
                                        void* stream)
{
    linattn_chunk_args va{};
    ChunkProblem vp{};
    linattn_status st = validate_dp(a, &va, &vp);
    if (st != LINATTN_OK) return st;
    // one substep per token: the virtual sequence is the sequence itself
    if (a->nh == 1)
        return linattn_chunk_fwd(&va, q, k, v, g, beta, s0, o, s_final, workspace, workspace_bytes, stream);
    if (vp.B * vp.H == 0) return LINATTN_OK;
    const DpLayout l = dp_layout(va, vp);
    st = check_states(vp, s0, s_final);
    if (st != LINATTN_OK) return st;
    if (a->T > 0) {
        st = check_pointers(LINATTN_RULE_DELTA, a->gate, q, k, v, g, beta, q, o);
        if (st != LINATTN_OK) return st;
        if (!workspace || workspace_bytes < l.total) return LINATTN_ERR_WORKSPACE;
        if (!aligned16(workspace)) return LINATTN_ERR_UNSUPPORTED;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    // the pipelined kernel reads q and g and writes o in the real token layout
    // itself; the workspace stays part of the contract for the other paths
    if (chunk_path(vp) == kPathPipe) {
        vp.q = q; vp.k = k; vp.v = v; vp.g = g; vp.beta = beta;
        vp.s0 = s0; vp.o = o; vp.s_final = s_final;
        return launch_chunk_pipe_virtual(vp, a->nh, s) == hipSuccess ? LINATTN_OK : LINATTN_ERR_LAUNCH;
    }
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    DeltaProductProblem p{a->B, a->H, a->T, a->nh, a->dk, a->dv, a->dtype, q, g,
                          a->T > 0 ? ws + l.qv : nullptr,
                          a->T > 0 && a->gate == LINATTN_GATE_SCALAR ? ws + l.gv : nullptr,
                          a->T > 0 ? ws + l.ov : nullptr, o};
    if (a->T > 0 && launch_dp_expand(p, s) != hipSuccess) return LINATTN_ERR_LAUNCH;
    st = linattn_chunk_fwd(&va, p.qv, k, v, p.gv, beta, s0, a->T > 0 ? ws + l.ov : nullptr, s_final,
                           a->T > 0 ? ws + l.cws : nullptr, a->T > 0 ? workspace_bytes - l.cws : 0, stream);
    if (st != LINATTN_OK) return st;
    if (a->T > 0 && launch_dp_gather(p, s) != hipSuccess) return LINATTN_ERR_LAUNCH;
    return LINATTN_OK;
}

size_t linattn_normalized_workspace_bytes(const linattn_chunk_args* a)
{
    linattn_chunk_args ad{};
    ChunkProblem p{}, pd{};
    if (validate_norm(a, nullptr, &ad, &p, &pd) != LINATTN_OK) return 0;
    return norm_layout(p, pd).total;
}

linattn_status linattn_chunk_fwd_normalized(const linattn_chunk_args* a, const linattn_prep_args* prep,
                                            const void* q, const void* k, const void* v, const void* g,
                                            const float* s0, const float* z0, void* o, float* s_final,
                                            float* z_final, void* workspace, size_t workspace_bytes,
                                            void* stream)
{
    linattn_chunk_args ad{};
    ChunkProblem p{}, pd{};
    linattn_status st = validate_norm(a, prep, &ad, &p, &pd);
    if (st != LINATTN_OK) return st;
    if (p.B * p.H == 0) return LINATTN_OK;
    if (p.T > 0) {
        st = check_pointers(LINATTN_RULE_ADD, a->gate, q, k, v, g, nullptr, q, o);
        if (st != LINATTN_OK) return st;
    }
    st = check_states(p, s0, s_final);
    if (st != LINATTN_OK) return st;
    if ((z0 && !aligned16(z0)) || (z_final && !aligned16(z_final))) return LINATTN_ERR_UNSUPPORTED;
    // z_final may alias z0 exactly (the key sum carried in place), but must not
    // partially overlap it
    const size_t zbytes = (size_t)(p.B * p.H) * p.dk * sizeof(float);
    if (z0 && z_final && z0 != z_final) {
        const char* a0 = reinterpret_cast<const char*>(z0);
        const char* a1 = reinterpret_cast<const char*>(z_final);
        if (a0 < a1 + zbytes && a1 < a0 + zbytes) return LINATTN_ERR_ARG;
    }
    const NormLayout l = norm_layout(p, pd);
    if (!workspace || workspace_bytes < l.total) return LINATTN_ERR_WORKSPACE;
    if (!aligned16(workspace)) return LINATTN_ERR_UNSUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(stream);
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    // gate NONE or SCALAR on the fused path: one pass carries z beside S.
    // Every value block of a head reads z0 when it starts, but only the first
    // writes z_final, so an in-place z0 is read from a copy in the workspace
    // (the denominator pass's state region, unused on this route)
    if (chunk_path(p) == kPathFused) {
        const float* zin = z0;
        if (z0 && z0 == z_final) {
            if (hipMemcpyAsync(ws + l.s0d, z0, zbytes, hipMemcpyDeviceToDevice, s) != hipSuccess)
                return LINATTN_ERR_LAUNCH;
            zin = reinterpret_cast<const float*>(ws + l.s0d);
        }
        p.q = q; p.k = k; p.v = v; p.g = g; p.beta = nullptr;
        p.s0 = s0; p.o = o; p.s_final = s_final;
        return launch_chunk_fused_normalized(p, zin, z_final, s) == hipSuccess ? LINATTN_OK : LINATTN_ERR_LAUNCH;
    }
    NormalizedProblem np{p.B * p.H * p.T, p.B * p.H, p.dk, p.dv, p.dtype, ws + l.ones, z0,
                         reinterpret_cast<float*>(ws + l.s0d), o, ws + l.den,
                         reinterpret_cast<const float*>(ws + l.sfd), z_final};
    if (launch_norm_prepare(np, s) != hipSuccess) return LINATTN_ERR_LAUNCH;
    // numerator: the add rule on the values; denominator: on the block of ones
    st = linattn_chunk_fwd_prep(a, prep, q, k, v, g, nullptr, s0, o, s_final, ws + l.cws,
                                workspace_bytes - l.cws, stream);
    if (st != LINATTN_OK) return st;
    st = linattn_chunk_fwd_prep(&ad, prep, q, k, ws + l.ones, g, nullptr, reinterpret_cast<float*>(ws + l.s0d),
                                ws + l.den, reinterpret_cast<float*>(ws + l.sfd), ws + l.cws,
                                workspace_bytes - l.cws, stream);
    if (st != LINATTN_OK) return st;
    return launch_norm_finish(np, s) == hipSuccess ? LINATTN_OK : LINATTN_ERR_LAUNCH;
}

}  // extern "C"

extern "C" {

linattn_status linattn_chunk_fwd_save(const linattn_chunk_args* a, const void* q, const void* k,
                                      const void* v, const void* g, const void* beta, const float* s0,
                                      void* o, float* s_final, void* states, void* workspace,
                                      size_t workspace_bytes, void* stream)
{
    ChunkProblem p{};
    linattn_status st = validate_train(a, &p);
    if (st != LINATTN_OK) return st;
    if (p.B * p.H == 0) return LINATTN_OK;
    if (p.T > 0) {
        st = check_pointers(p.rule, p.gate, q, k, v, g, beta, q, o);
        if (st != LINATTN_OK) return st;
        if (!states) return LINATTN_ERR_NULL;
        if (!aligned16(states)) return LINATTN_ERR_UNSUPPORTED;
    }
    st = check_states(p, s0, s_final);
    if (st != LINATTN_OK) return st;
    const size_t need = fwd_save_workspace_bytes(p);
    if (p.T > 0 && need > 0) {
        if (!workspace || workspace_bytes < need) return LINATTN_ERR_WORKSPACE;
        if (!aligned16(workspace)) return LINATTN_ERR_UNSUPPORTED;
    }
    p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta;
    p.s0 = s0; p.o = o; p.s_final = s_final;
    return launch_fwd_save(p, states, workspace, workspace_bytes, static_cast<hipStream_t>(stream)) == hipSuccess
               ? LINATTN_OK : LINATTN_ERR_LAUNCH;
}

size_t linattn_chunk_bwd_workspace_bytes(const linattn_chunk_args* a, int states_given)
{
    ChunkProblem p{};
    if (validate_train(a, &p) != LINATTN_OK) return 0;
    return bwd_layout(p, states_given != 0).total;
}

linattn_status linattn_chunk_bwd(const linattn_chunk_args* a, const void* q, const void* k, const void* v,
                                 const void* g, const void* beta, const float* s0, const void* states,
                                 const void* dout, const float* dsT, void* dq, void* dk, void* dv, void* dg,
                                 void* dbeta, float* ds0, void* workspace, size_t workspace_bytes,
                                 void* stream)
{
    ChunkProblem p{};
    linattn_status st = validate_train(a, &p);
    if (st != LINATTN_OK) return st;
    if (p.B * p.H == 0) return LINATTN_OK;
    if (p.T > 0) {
        st = check_pointers(p.rule, p.gate, q, k, v, g, beta, q, dout);
        if (st != LINATTN_OK) return st;
        // gradient outputs: dg exactly for a gate, dbeta for the delta rule
        if (!dq || !dk || !dv) return LINATTN_ERR_NULL;
        if ((p.gate != kGateNone) != (dg != nullptr)) return dg ? LINATTN_ERR_ARG : LINATTN_ERR_NULL;
        if ((p.rule == kRuleDelta) != (dbeta != nullptr)) return dbeta ? LINATTN_ERR_ARG : LINATTN_ERR_NULL;
        const void* outs[] = {dq, dk, dv, dg, dbeta, states};
        for (const void* x : outs)
            if (x && !aligned16(x)) return LINATTN_ERR_UNSUPPORTED;
    }
    const void* st_ptrs[] = {s0, dsT, ds0};
    for (const void* x : st_ptrs)
        if (x && !aligned16(x)) return LINATTN_ERR_UNSUPPORTED;
    const bool given = states != nullptr;
    const BwdLayout l = bwd_layout(p, given);
    if (p.T > 0) {
        if (!workspace || workspace_bytes < l.total) return LINATTN_ERR_WORKSPACE;
        if (!aligned16(workspace)) return LINATTN_ERR_UNSUPPORTED;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    const void* sts = states;
    if (p.T > 0 && !given) {
        ChunkProblem fp = p;
        fp.q = q; fp.k = k; fp.v = v; fp.g = g; fp.beta = beta;
        fp.s0 = s0; fp.o = ws + l.o; fp.s_final = nullptr;
        if (launch_fwd_save(fp, ws + l.st, ws + l.fws, l.total - l.fws, s) != hipSuccess) return LINATTN_ERR_LAUNCH;
        sts = ws + l.st;
    }
    ChunkBwdProblem b{p.B, p.H, p.T, p.dk, p.dv, p.rule, p.gate, p.dtype,
                      q, k, v, g, beta, dout, sts, dsT, dq, dk, dv, dg, dbeta, ds0,
                      p.T > 0 ? ws + l.ops : nullptr,
                      p.T > 0 ? reinterpret_cast<float*>(ws + l.gc) : nullptr,
                      p.T > 0 ? ws + l.dst : nullptr};
    return launch_chunk_bwd(b, s) == hipSuccess ? LINATTN_OK : LINATTN_ERR_LAUNCH;
}

}  // extern "C"

extern "C" {

size_t linattn_deltaproduct_bwd_workspace_bytes(const linattn_deltaproduct_args* a)
{
    linattn_chunk_args va{};
    ChunkProblem vp{};
    if (validate_dp(a, &va, &vp) != LINATTN_OK || validate_train(&va, &vp) != LINATTN_OK) return 0;
    if (a->nh == 1) return bwd_layout(vp, false).total;
    return dp_bwd_layout(va, vp).total;
}

linattn_status linattn_deltaproduct_bwd(const linattn_deltaproduct_args* a, const void* q, const void* k,
                                        const void* v, const void* g, const void* beta, const float* s0,
                                        const void* dout, const float* dsT, void* dq, void* dk, void* dv,
                                        void* dg, void* dbeta, float* ds0, void* workspace,
                                        size_t workspace_bytes, void* stream)
{
    linattn_chunk_args va{};
    ChunkProblem vp{};
    linattn_status st = validate_dp(a, &va, &vp);
    if (st != LINATTN_OK) return st;
    st = validate_train(&va, &vp);
    if (st != LINATTN_OK) return st;
    // one substep per token: the virtual sequence is the sequence itself
    if (a->nh == 1)
        return linattn_chunk_bwd(&va, q, k, v, g, beta, s0, nullptr, dout, dsT, dq, dk, dv, dg, dbeta, ds0,
                                 workspace, workspace_bytes, stream);
    if (vp.B * vp.H == 0) return LINATTN_OK;
    if (a->T == 0)
        return linattn_chunk_bwd(&va, q, k, v, g, beta, s0, nullptr, dout, dsT, dq, dk, dv, dg, dbeta, ds0,
                                 workspace, workspace_bytes, stream);
    st = check_pointers(LINATTN_RULE_DELTA, a->gate, q, k, v, g, beta, q, dout);
    if (st != LINATTN_OK) return st;
    if (!dq || !dk || !dv || !dbeta) return LINATTN_ERR_NULL;
    if ((a->gate == LINATTN_GATE_SCALAR) != (dg != nullptr)) return dg ? LINATTN_ERR_ARG : LINATTN_ERR_NULL;
    const void* outs[] = {dq, dk, dv, dg, dbeta, s0, dsT, ds0};
    for (const void* x : outs)
        if (x && !aligned16(x)) return LINATTN_ERR_UNSUPPORTED;
    const DpBwdLayout l = dp_bwd_layout(va, vp);
    if (!workspace || workspace_bytes < l.total) return LINATTN_ERR_WORKSPACE;
    if (!aligned16(workspace)) return LINATTN_ERR_UNSUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(stream);
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    const bool gated = a->gate == LINATTN_GATE_SCALAR;
    DeltaProductProblem p{a->B, a->H, a->T, a->nh, a->dk, a->dv, a->dtype, q, g, ws + l.qv,
                          gated ? ws + l.gv : nullptr, nullptr, nullptr};
    if (launch_dp_expand(p, s) != hipSuccess) return LINATTN_ERR_LAUNCH;
    if (launch_dp_scatter(p, dout, ws + l.dov, s) != hipSuccess) return LINATTN_ERR_LAUNCH;
    st = linattn_chunk_bwd(&va, ws + l.qv, k, v, gated ? ws + l.gv : nullptr, beta, s0, nullptr, ws + l.dov, dsT,
                           ws + l.dqv, dk, dv, gated ? ws + l.dgv : nullptr, dbeta, ds0, ws + l.cws,
                           workspace_bytes - l.cws, stream);
    if (st != LINATTN_OK) return st;
    const int64_t rows = a->B * a->H * a->T;
    // the query sits on the last substep, the gate on the first
    if (launch_dp_pick(ws + l.dqv, dq, rows, a->nh, a->nh - 1, a->dk, a->dtype, s) != hipSuccess)
        return LINATTN_ERR_LAUNCH;
    if (gated && launch_dp_pick(ws + l.dgv, dg, rows, a->nh, 0, 1, a->dtype, s) != hipSuccess)
        return LINATTN_ERR_LAUNCH;
    return LINATTN_OK;
}

}  // extern "C"

// ---- the chunk forward that allocates nothing ------------------------------
// Scratch of linattn_chunk_fwd_noalloc: a static device array, one per GPU.  In
// host code `scratch` names a host-side stand-in; kernels get the device
// address that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[LINATTN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];

// This device's scratch address, looked up once per device with it current.
hipError_t device_scratch(void** out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch[dev] = ptr;
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

}  // namespace

extern "C" linattn_status linattn_chunk_fwd_noalloc(const linattn_chunk_args* a, const linattn_prep_args* prep,
                                                    const void* q, const void* k, const void* v, const void* g,
                                                    const void* beta, const float* s0, void* o, float* s_final,
                                                    void* stream)
{
    ChunkProblem p{};
    const linattn_status st = validate_chunk(a, &p, prep);
    if (st != LINATTN_OK) return st;
    const size_t need = path_workspace_bytes(p);
    if (need > LINATTN_NOALLOC_SCRATCH_BYTES) return LINATTN_ERR_WORKSPACE;
    void* ws = nullptr;
    if (need > 0 && p.B * p.H > 0 && p.T > 0 && device_scratch(&ws) != hipSuccess) return LINATTN_ERR_LAUNCH;
    return linattn_chunk_fwd_prep(a, prep, q, k, v, g, beta, s0, o, s_final, ws, ws ? need : 0, stream);
}
