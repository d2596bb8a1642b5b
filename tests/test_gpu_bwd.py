"""Parity of the chunkwise backward pass (HIP, through the C ABI) with the
fp64 oracle's reverse-mode recurrence: every rule and gate (the per-channel
gate with bf16 tokens), both dtypes and head sizes, ragged lengths, initial
state and final-state gradient, the forward that keeps the chunk states, and
sampled full-size workloads (GDN and KDA)."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from gpu_util import TOL, dev, dev_state, host, note, rel_l2

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

NAMES = ("dq", "dk", "dv", "dg", "dbeta", "ds0")


def run_bwd(case, x, gr, use_states=False):
    import gated_delta_rule_27_amd as la
    d = lambda a: dev(a, case.dtype)
    args = (d(x["q"]), d(x["k"]), d(x["v"]), d(x["g"]), d(x["beta"]))
    states = None
    if use_states:
        _, _, states = la.chunk_fwd_save(*args, dev_state(x["s0"]), rule=case.rule, gate=case.gate)
    out = la.chunk_bwd(*args, d(gr["do"]), dev_state(x["s0"]), dev_state(gr["dsT"]), states=states,
                       rule=case.rule, gate=case.gate)
    torch.cuda.synchronize()
    return out


def check_bwd(case, use_states=False, tol=None):
    tol = TOL[case.dtype] if tol is None else tol
    note(f"[bwd] {case.name} rule={case.rule} gate={case.gate} dtype={case.dtype} B={case.B} H={case.H} "
         f"T={case.T} dk={case.dk} dv={case.dv} states={'saved' if use_states else 'recomputed'}")
    x, gr = syn.chunk_inputs(case), syn.grad_inputs(case)
    out = run_bwd(case, x, gr, use_states)
    ref = oracle.recurrence_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], gr["do"], gr["dsT"],
                                rule=case.rule, gate=case.gate)
    errs = {}
    for n in NAMES:
        if ref[n] is None:
            assert out[n] is None
            continue
        a = host(out[n])
        assert np.all(np.isfinite(a)), f"non-finite {n}"
        errs[n] = rel_l2(a, ref[n])
    note("    rel L2 " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    bad = {n: e for n, e in errs.items() if e > tol}
    assert not bad, f"above {tol}: {bad}"
    return out


SMALL = []
for dtype, dims in (("bf16", ((128, 128), (64, 64), (64, 128), (128, 64))), ("fp32", ((64, 64), (64, 128)))):
    for (dk, dv) in dims:
        for rule in ("add", "delta"):
            for gate in ("none", "scalar"):
                SMALL.append((dtype, dk, dv, rule, gate))


@pytest.mark.parametrize("dtype,dk,dv,rule,gate", SMALL)
def test_small_ragged(dtype, dk, dv, rule, gate):
    # T = 200: three full chunks and a ragged tail of 8; s0 and dS_T nonzero;
    # gates weak enough that the carried state matters
    case = syn.Case("bwd_small", 2, 2, 200, dk, dv, rule, gate, dtype, gate_scale=0.1, s0_std=0.3,
                    case_id=140)
    check_bwd(case)


@pytest.mark.parametrize("T", [1, 17, 63, 64, 65, 128, 130])
def test_lengths(T):
    case = syn.Case("bwd_len", 1, 2, T, 128, 128, "delta", "scalar", "bf16", gate_scale=0.2, s0_std=0.2,
                    case_id=141)
    check_bwd(case)


@pytest.mark.parametrize("beta_mode", ["zero", "one"])
def test_beta_extremes(beta_mode):
    case = syn.Case("bwd_beta", 1, 2, 150, 128, 128, "delta", "scalar", "bf16", gate_scale=0.1,
                    beta_mode=beta_mode, s0_std=0.2, case_id=142)
    check_bwd(case)


def test_strong_decay():
    # the workloads' own gate law (a chunk decays by ~e^-40): the carried
    # state barely reaches the next chunk, the in-chunk decays dominate dg
    case = syn.Case("bwd_strong", 2, 2, 192, 128, 128, "delta", "scalar", "bf16", s0_std=0.3,
                    case_id=143)
    check_bwd(case)


@pytest.mark.parametrize("rule", ["add", "delta"])
@pytest.mark.parametrize("dtype,dk", [("bf16", 128), ("fp32", 64)])
@pytest.mark.parametrize("scale", [12.0, 30.0])
def test_scalar_gate_underflow(rule, dtype, dk, scale):
    # log-gates ~ -10 and ~ -24 per token: every in-chunk decay product below
    # the diagonal underflows within a few tokens; the gradients must stay
    # finite and match (decay factors formed from differences of G only)
    case = syn.Case("bwd_underflow", 2, 2, 200, dk, 128, rule, "scalar", dtype, gate_scale=scale,
                    s0_std=0.3, case_id=147)
    check_bwd(case)


def test_saved_states_equal_recomputed():
    import gated_delta_rule_27_amd as la
    case = syn.Case("bwd_saved", 2, 3, 333, 128, 128, "delta", "scalar", "bf16", gate_scale=0.1,
                    s0_std=0.3, case_id=144)
    a = check_bwd(case, use_states=True)
    x, gr = syn.chunk_inputs(case), syn.grad_inputs(case)
    b = run_bwd(case, x, gr, use_states=False)
    for n in NAMES:
        if a[n] is not None:
            assert torch.equal(a[n], b[n]), f"{n}: saved and recomputed states differ"
    # the states themselves: chunk r starts from the oracle's state after 64 r tokens
    d = lambda t: dev(t, case.dtype)
    _, _, states = la.chunk_fwd_save(d(x["q"]), d(x["k"]), d(x["v"]), d(x["g"]), d(x["beta"]),
                                     dev_state(x["s0"]), rule=case.rule, gate=case.gate)
    torch.cuda.synchronize()
    st = host(states)
    assert np.array_equal(st[:, :, 0], syn.to_dtype(x["s0"], case.dtype).astype(np.float64))
    for r in (1, 3, 5):
        cut = 64 * r
        sub = {k2: (None if v2 is None else np.ascontiguousarray(v2[:, :, :cut])) for k2, v2 in x.items()
               if k2 != "s0"}
        _, sref = oracle.recurrence(sub["q"], sub["k"], sub["v"], sub["g"], sub["beta"], x["s0"],
                                    rule=case.rule, gate=case.gate)
        assert rel_l2(st[:, :, r], sref) <= TOL["bf16"], f"state entering chunk {r}"


def test_zero_tokens():
    import gated_delta_rule_27_amd as la
    e = lambda *s: torch.empty(s, dtype=torch.bfloat16, device="cuda")
    dsT = torch.randn(1, 2, 64, 64, device="cuda")
    out = la.chunk_bwd(e(1, 2, 0, 64), e(1, 2, 0, 64), e(1, 2, 0, 64), e(1, 2, 0), e(1, 2, 0),
                       e(1, 2, 0, 64), None, dsT, rule="delta", gate="scalar")
    torch.cuda.synchronize()
    assert torch.equal(out["ds0"], dsT)
    out = la.chunk_bwd(e(1, 2, 0, 64), e(1, 2, 0, 64), e(1, 2, 0, 64), None, None, e(1, 2, 0, 64),
                       rule="add", gate="none")
    torch.cuda.synchronize()
    assert torch.count_nonzero(out["ds0"]) == 0


def test_deterministic():
    case = syn.Case("bwd_det", 1, 4, 300, 128, 128, "delta", "scalar", "bf16", gate_scale=0.2,
                    s0_std=0.2, case_id=145)
    x, gr = syn.chunk_inputs(case), syn.grad_inputs(case)
    a, b = run_bwd(case, x, gr), run_bwd(case, x, gr)
    for n in NAMES:
        if a[n] is not None:
            assert torch.equal(a[n], b[n]), f"{n} differs between runs"


def test_gdn_full_size_sampled():
    # the GDN workload's shape (B8 H16 T8192 d128), every head on the GPU;
    # the oracle checks two heads
    import gated_delta_rule_27_amd as la
    case = syn.CFG3
    heads = [(0, 0), (7, 15)]
    xs = syn.chunk_inputs(case, heads=heads)
    gs = syn.grad_inputs(case, heads=heads)
    full = syn.chunk_inputs_torch(case, "cuda")
    gfull = syn.grad_inputs_torch(case, "cuda")
    for i, (b, h) in enumerate(heads):
        for key in ("q", "k", "v", "g", "beta"):
            full[key][b, h] = dev(xs[key][i], case.dtype)
        gfull["do"][b, h] = dev(gs["do"][i], case.dtype)
    out = la.chunk_bwd(full["q"], full["k"], full["v"], full["g"], full["beta"], gfull["do"],
                       rule=case.rule, gate=case.gate)
    torch.cuda.synchronize()
    sub = lambda a: None if a is None else a[:, None]
    ref = oracle.recurrence_bwd(sub(xs["q"]), sub(xs["k"]), sub(xs["v"]), sub(xs["g"]), sub(xs["beta"]),
                                None, sub(gs["do"]), None, rule=case.rule, gate=case.gate)
    for i, (b, h) in enumerate(heads):
        errs = {n: rel_l2(host(out[n][b, h]), ref[n][i, 0]) for n in NAMES}
        note(f"    head ({b},{h}): " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
        assert all(e <= TOL["bf16"] for e in errs.values()), errs


# ---- per-key-channel gate (GLA decay with the add rule, KDA with the delta rule) ----
CHANNEL = [(dk, dv, rule) for (dk, dv) in ((128, 128), (64, 64), (64, 128), (128, 64))
           for rule in ("add", "delta")]


@pytest.mark.parametrize("dk,dv,rule", CHANNEL)
def test_channel_small_ragged(dk, dv, rule):
    case = syn.Case("bwd_chan", 2, 2, 200, dk, dv, rule, "channel", "bf16", gate_scale=1 / 16, s0_std=0.3,
                    case_id=146)
    check_bwd(case)


@pytest.mark.parametrize("T", [1, 16, 63, 65, 130])
def test_channel_lengths(T):
    case = syn.Case("bwd_chan_len", 1, 2, T, 128, 128, "delta", "channel", "bf16", gate_scale=0.25,
                    s0_std=0.2, case_id=147)
    check_bwd(case)


@pytest.mark.parametrize("gate_scale", [1.0, 12.0, 30.0])
def test_channel_decay_laws(gate_scale):
    # gate_scale 1: the workloads' law per channel; 12: per-token log-decays
    # near -10, so whole 16-row blocks decay past the fp32 range and some of
    # them past the split of the diagonal blocks; 30: every diagonal block is
    # summed element by element
    case = syn.Case("bwd_chan_law", 1, 2, 192, 128, 128, "delta", "channel", "bf16", gate_scale=gate_scale,
                    s0_std=0.3, case_id=148)
    check_bwd(case)


def test_channel_saved_states_equal_recomputed():
    case = syn.Case("bwd_chan_saved", 1, 3, 150, 128, 128, "delta", "channel", "bf16", gate_scale=0.25,
                    s0_std=0.3, case_id=149)
    a = check_bwd(case, use_states=True)
    x, gr = syn.chunk_inputs(case), syn.grad_inputs(case)
    b = run_bwd(case, x, gr, use_states=False)
    for n in NAMES:
        if a[n] is not None:
            assert torch.equal(a[n], b[n]), f"{n}: saved and recomputed states differ"


def test_channel_equal_channels_match_scalar_gate():
    # every channel with the same log-gate is the scalar gate: the same dq, dk,
    # dv, dbeta, ds0, and the channel gradients of dg sum to the scalar one
    import gated_delta_rule_27_amd as la
    case = syn.Case("bwd_chan_eq", 1, 2, 140, 128, 128, "delta", "scalar", "bf16", gate_scale=0.3, s0_std=0.3,
                    case_id=150)
    x, gr = syn.chunk_inputs(case), syn.grad_inputs(case)
    d = lambda a: dev(a, case.dtype)
    gs = d(x["g"])
    gc = gs[..., None].expand(*gs.shape, case.dk).contiguous()
    common = (d(x["q"]), d(x["k"]), d(x["v"]))
    a = la.chunk_bwd(*common, gs, d(x["beta"]), d(gr["do"]), dev_state(x["s0"]), dev_state(gr["dsT"]),
                     rule="delta", gate="scalar")
    b = la.chunk_bwd(*common, gc, d(x["beta"]), d(gr["do"]), dev_state(x["s0"]), dev_state(gr["dsT"]),
                     rule="delta", gate="channel")
    torch.cuda.synchronize()
    for n in ("dq", "dk", "dv", "dbeta", "ds0"):
        e = rel_l2(host(b[n]), host(a[n]))
        note(f"    {n} rel L2 {e:.2e}")
        assert e <= TOL["bf16"], n
    e = rel_l2(host(b["dg"]).sum(axis=-1), host(a["dg"]))
    note(f"    dg (summed over channels) rel L2 {e:.2e}")
    assert e <= TOL["bf16"]


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64)])
def test_channel_many_heads_wide_blocks(dk, dv):
    # 256 heads (512 with d_v = 64 counted in 64-column blocks): the forward's
    # state pass takes 64-column value blocks (the narrow 32-column blocks
    # serve fewer blocks than CUs), so its saved states go through the wide
    # copy path; saved and recomputed states agree and the gradients match the
    # oracle on every head
    case = syn.Case("bwd_chan_wide", 2, 128, 130, dk, dv, "delta", "channel", "bf16", gate_scale=0.25,
                    s0_std=0.2, case_id=152)
    a = check_bwd(case, use_states=True)
    x, gr = syn.chunk_inputs(case), syn.grad_inputs(case)
    b = run_bwd(case, x, gr, use_states=False)
    for n in NAMES:
        if a[n] is not None:
            assert torch.equal(a[n], b[n]), f"{n}: saved and recomputed states differ"


@pytest.mark.parametrize("gate,dk,dv,rule", [("scalar", 128, 128, "delta"), ("none", 64, 128, "add"),
                                             ("channel", 128, 128, "delta"), ("channel", 64, 64, "add")])
def test_chain_value_block_widths_agree(monkeypatch, gate, dk, dv, rule):
    # the reverse state pass in 32-column value blocks (two state waves; chosen
    # when 64-column blocks leave CUs idle) gives the same bits as in 64-column
    # blocks, and both match the oracle
    case = syn.Case("bwd_vb", 1, 3, 200, dk, dv, rule, gate, "bf16", gate_scale=0.25, s0_std=0.2,
                    case_id=160)
    monkeypatch.setenv("LINATTN_CHAIN_VB", "64")
    a = check_bwd(case)
    monkeypatch.setenv("LINATTN_CHAIN_VB", "32")
    b = check_bwd(case)
    for n in NAMES:
        if a[n] is not None:
            assert torch.equal(a[n], b[n]), f"{n}: 32- and 64-column value blocks differ"


def test_channel_deterministic():
    case = syn.Case("bwd_chan_det", 1, 4, 300, 128, 128, "delta", "channel", "bf16", gate_scale=0.2,
                    s0_std=0.2, case_id=151)
    x, gr = syn.chunk_inputs(case), syn.grad_inputs(case)
    a, b = run_bwd(case, x, gr), run_bwd(case, x, gr)
    for n in NAMES:
        if a[n] is not None:
            assert torch.equal(a[n], b[n]), f"{n} differs between runs"


@pytest.mark.timeout(900)
def test_kda_full_size_sampled():
    # the KDA workload's shape (B1 H32 T262144 d128), every head on the GPU.
    # The gradients of the last n tokens depend on the earlier ones only
    # through the state entering them, so the oracle checks them exactly: its
    # forward over the first T - n tokens gives that state, its backward over
    # the last n tokens the gradients (the loss has no dS_T term).
    import gated_delta_rule_27_amd as la
    case = syn.CFG4
    n = 300
    heads = [(0, 0), (0, 31)]
    note(f"[bwd full] {case.name}: inputs on the GPU, heads {heads} from the host generator")
    xs = syn.chunk_inputs(case, heads=heads)
    gs = syn.grad_inputs(case, heads=heads)
    full = syn.chunk_inputs_torch(case, "cuda")
    gfull = syn.grad_inputs_torch(case, "cuda")
    for i, (b, h) in enumerate(heads):
        for key in ("q", "k", "v", "g", "beta"):
            full[key][b, h] = dev(xs[key][i], case.dtype)
        gfull["do"][b, h] = dev(gs["do"][i], case.dtype)
    note(f"[bwd full] {case.name}: GPU backward (states recomputed)")
    out = la.chunk_bwd(full["q"], full["k"], full["v"], full["g"], full["beta"], gfull["do"],
                       rule=case.rule, gate=case.gate)
    torch.cuda.synchronize()
    for nm in NAMES:
        if out[nm] is not None:
            assert torch.isfinite(out[nm]).all(), nm
    cut = case.T - n
    head = lambda a, sl: None if a is None else np.ascontiguousarray(a[:, None, sl])
    note(f"[bwd full] {case.name}: oracle forward over {cut} tokens, backward over the last {n}")
    _, s_cut = oracle.recurrence(head(xs["q"], slice(0, cut)), head(xs["k"], slice(0, cut)),
                                 head(xs["v"], slice(0, cut)), head(xs["g"], slice(0, cut)),
                                 head(xs["beta"], slice(0, cut)), None, rule=case.rule, gate=case.gate)
    tail = slice(cut, None)
    ref = oracle.recurrence_bwd(head(xs["q"], tail), head(xs["k"], tail), head(xs["v"], tail),
                                head(xs["g"], tail), head(xs["beta"], tail), s_cut, head(gs["do"], tail), None,
                                rule=case.rule, gate=case.gate)
    for i, (b, h) in enumerate(heads):
        errs = {nm: rel_l2(host(out[nm][b, h, cut:]), ref[nm][i, 0]) for nm in NAMES if nm != "ds0"}
        note(f"    head ({b},{h}) last {n} tokens: " + " ".join(f"{nm}={e:.2e}" for nm, e in errs.items()))
        assert all(e <= TOL["bf16"] for e in errs.values()), errs
