"""Parity of the segmented chunk forwards (the add rule's single-pass kernel
and the two-kernel path's state pass) with the fp64 oracle and with the
unsegmented run.

The two-kernel path's state pass (per-channel gate, or any gate on request)
splits the same way for every rule: its prefix pass runs the main loop's state
update, S <- Diag(gamma_C) S + Kr^T Tb (V - Kd S), without the output.

For the add rule (no gate or a scalar gate) the chunk transition is a scalar
times the identity ("Linear Attention, Visualized", "Chunkwise algorithm":
"Update the state"), so the state entering any chunk is the decayed sum of
the keys times values before it.  When a launch has fewer workgroups than
compute units, the single-pass kernel splits each head's chunks into
segments; a later segment first forms its incoming state in a state-only pass
over the chunks before it.  That pass runs the same state update on the same
operands as the main loop, so the result is bit for bit the one-segment
result; LINATTN_SEGMENTS fixes the segment count for these comparisons."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from gpu_util import TOL, check_chunk, dev, dev_state, host, note, oracle_chunk, rel_l2, run_chunk, worst_block

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DIMS = [("bf16", 128, 128), ("bf16", 64, 64), ("bf16", 128, 64), ("fp32", 64, 64), ("fp32", 64, 128)]


def worst_block_all(case, o, oref):
    oh = host(o)
    return max(worst_block(oh[b, h], oref[b, h])[0] for b in range(case.B) for h in range(case.H))


@pytest.mark.parametrize("T", [1000, 4097])
@pytest.mark.parametrize("gate", ["none", "scalar"])
@pytest.mark.parametrize("dtype,dk,dv", DIMS)
def test_segments_parity(dtype, dk, dv, gate, T):
    # one batch of two heads: few workgroups, so the launch takes the most
    # segments; ragged tails; weak decay so early chunks matter at the end
    case = syn.Case("seg", 1, 2, T, dk, dv, "add", gate, dtype, gate_scale=1 / 16, s0_std=0.3,
                    case_id=160)
    x = syn.chunk_inputs(case)
    check_chunk(case, x, s0=x["s0"])
    o, _ = run_chunk(case, x, x["s0"])
    oref, _ = oracle_chunk(case, x, x["s0"])
    wb = worst_block_all(case, o, oref)
    note(f"    worst 64-token block {wb:.3e}")
    assert wb <= TOL[dtype]


@pytest.mark.parametrize("nseg", [2, 3, 4])
@pytest.mark.parametrize("gate", ["none", "scalar"])
@pytest.mark.parametrize("dtype,dk,dv", [("bf16", 128, 128), ("fp32", 64, 64)])
def test_segments_bitwise_one_segment(monkeypatch, dtype, dk, dv, gate, nseg):
    case = syn.Case("segbits", 2, 2, 777, dk, dv, "add", gate, dtype, gate_scale=1 / 8, s0_std=0.3,
                    case_id=161)
    x = syn.chunk_inputs(case)
    monkeypatch.setenv("LINATTN_SEGMENTS", "1")
    o1, s1 = run_chunk(case, x, x["s0"])
    monkeypatch.setenv("LINATTN_SEGMENTS", str(nseg))
    on, sn = run_chunk(case, x, x["s0"])
    note(f"[segments] {nseg} vs 1: max |do| {(on.float() - o1.float()).abs().max().item():.3e} "
         f"max |dS| {(sn - s1).abs().max().item():.3e}")
    assert torch.equal(on, o1) and torch.equal(sn, s1)


@pytest.mark.parametrize("T", [2, 65, 129, 200])
def test_segments_short(monkeypatch, T):
    # forced segments down to one chunk each (the last one ragged)
    monkeypatch.setenv("LINATTN_SEGMENTS", "4")
    case = syn.Case("segshort", 1, 3, T, 128, 128, "add", "scalar", "bf16", gate_scale=0.25, s0_std=0.3,
                    case_id=162)
    x = syn.chunk_inputs(case)
    check_chunk(case, x, s0=x["s0"])


@pytest.mark.parametrize("scale", [12.0, 30.0])
def test_segments_strong_scalar_gate(monkeypatch, scale):
    # log-gates ~ -10 and ~ -24 per token: the state carried into a segment
    # is negligible, the decay products underflow inside every chunk
    monkeypatch.setenv("LINATTN_SEGMENTS", "4")
    case = syn.Case("segstrong", 1, 2, 900, 128, 128, "add", "scalar", "bf16", gate_scale=scale,
                    s0_std=0.3, case_id=163)
    x = syn.chunk_inputs(case)
    check_chunk(case, x, s0=x["s0"])
    o, _ = run_chunk(case, x, x["s0"])
    oref, _ = oracle_chunk(case, x, x["s0"])
    assert worst_block_all(case, o, oref) <= TOL["bf16"]


def test_segments_no_initial_state():
    case = syn.Case("segnos0", 1, 2, 3000, 128, 128, "add", "none", "bf16", case_id=164)
    x = syn.chunk_inputs(case)
    check_chunk(case, x, s0=None)


def test_segments_state_in_place():
    # s_final aliasing s0: every segment would read s0 while the last writes
    # s_final, so the launch keeps one segment; same result as out of place
    import gated_delta_rule_27_amd as la
    case = syn.Case("seginplace", 1, 2, 2000, 128, 128, "add", "scalar", "bf16", gate_scale=1 / 16,
                    s0_std=0.3, case_id=165)
    x = syn.chunk_inputs(case)
    d = lambda a: dev(a, case.dtype)
    o_ref, s_ref = la.chunk_fwd(d(x["q"]), d(x["k"]), d(x["v"]), d(x["g"]), None, dev_state(x["s0"]),
                                rule="add", gate="scalar")
    s_io = dev_state(x["s0"])
    o, s = la.chunk_fwd(d(x["q"]), d(x["k"]), d(x["v"]), d(x["g"]), None, s_io, rule="add", gate="scalar",
                        s_final=s_io)
    torch.cuda.synchronize()
    assert s.data_ptr() == s_io.data_ptr()
    assert torch.equal(o, o_ref) and torch.equal(s, s_ref)


def test_segments_normalized(monkeypatch):
    # normalised attention carries the key sum z beside S through the prefix
    import gated_delta_rule_27_amd as la
    case = syn.Case("segnorm", 1, 2, 1500, 128, 128, "add", "scalar", "bf16", qk="elu1", gate_scale=0.05,
                    s0_std=0.3, case_id=166)
    x = syn.chunk_inputs(case)
    rng = np.random.default_rng([syn.SEED, 166])
    z0 = np.abs(rng.standard_normal((case.B, case.H, case.dk))).astype(np.float32)
    s0 = np.abs(x["s0"]).astype(np.float32)
    d = lambda a: dev(a, case.dtype)
    outs = {}
    for n in ("1", "4"):
        monkeypatch.setenv("LINATTN_SEGMENTS", n)
        outs[n] = la.chunk_fwd_normalized(d(x["q"]), d(x["k"]), d(x["v"]), d(x["g"]), dev_state(s0),
                                          dev_state(z0), gate="scalar")
    torch.cuda.synchronize()
    for a, b in zip(outs["1"], outs["4"]):
        assert torch.equal(a, b)
    o, s, z = outs["4"]
    oref, sref, zref = oracle.normalized(x["q"], x["k"], x["v"], x["g"], s0, z0, gate="scalar")
    eo, es, ez = rel_l2(host(o), oref), rel_l2(host(s), sref), rel_l2(host(z), zref)
    note(f"[segments norm] rel L2 o={eo:.3e} S={es:.3e} z={ez:.3e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"] and ez <= TOL["bf16"]


def test_segments_raw_projections(monkeypatch):
    # elu+1 feature map and -softplus gate applied inside the kernel, also in
    # the prefix pass
    import gated_delta_rule_27_amd as la
    monkeypatch.setenv("LINATTN_SEGMENTS", "3")
    case = syn.Case("segprep", 1, 2, 1111, 128, 128, "add", "scalar", "bf16", gate_scale=1.0, s0_std=0.3,
                    case_id=167)
    x = syn.raw_inputs(case)
    d = lambda a: dev(a, case.dtype)
    o, s = la.chunk_fwd(d(x["q"]), d(x["k"]), d(x["v"]), d(x["g"]), None, dev_state(x["s0"]), rule="add",
                        gate="scalar", qk_map="elu1", gate_map="neg_softplus")
    torch.cuda.synchronize()
    q, k = oracle.prepare_qk(x["q"], "elu1"), oracle.prepare_qk(x["k"], "elu1")
    g = oracle.prepare_gate(x["g"], "neg_softplus")
    oref, sref = oracle.recurrence(q, k, x["v"], g, None, x["s0"], rule="add", gate="scalar")
    eo, es = rel_l2(host(o), oref), rel_l2(host(s), sref)
    note(f"[segments prep] rel L2 o={eo:.3e} S={es:.3e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


# ---- the two-kernel path's state pass (per-channel gate; any gate on request) ----

@pytest.mark.parametrize("dk", [64, 128])
@pytest.mark.parametrize("rule", ["add", "delta"])
def test_chain_segments_channel_gate(monkeypatch, rule, dk):
    # one batch of two heads at d_v = 128: the state pass runs 32-column blocks,
    # 16 workgroups, and splits every head into four segments
    case = syn.Case("segchan", 1, 2, 1500, dk, 128, rule, "channel", "bf16", gate_scale=1 / 16, s0_std=0.3,
                    case_id=168)
    x = syn.chunk_inputs(case)
    check_chunk(case, x, s0=x["s0"])
    o, s = run_chunk(case, x, x["s0"])
    oref, _ = oracle_chunk(case, x, x["s0"])
    wb = worst_block_all(case, o, oref)
    note(f"    worst 64-token block {wb:.3e}")
    assert wb <= TOL["bf16"]
    monkeypatch.setenv("LINATTN_SEGMENTS", "1")
    o1, s1 = run_chunk(case, x, x["s0"])
    assert torch.equal(o, o1) and torch.equal(s, s1)


@pytest.mark.parametrize("nseg", [2, 3])
@pytest.mark.parametrize("gate", ["none", "scalar"])
def test_chain_segments_split_path(monkeypatch, gate, nseg):
    monkeypatch.setenv("LINATTN_CHUNK_PATH", "split")
    case = syn.Case("segsplit", 2, 1, 1300, 128, 128, "delta", gate, "bf16", gate_scale=1 / 16, s0_std=0.3,
                    case_id=169)
    x = syn.chunk_inputs(case)
    monkeypatch.setenv("LINATTN_SEGMENTS", str(nseg))
    check_chunk(case, x, s0=x["s0"])
    on, sn = run_chunk(case, x, x["s0"])
    monkeypatch.setenv("LINATTN_SEGMENTS", "1")
    o1, s1 = run_chunk(case, x, x["s0"])
    assert torch.equal(on, o1) and torch.equal(sn, s1)


def test_chain_segments_short(monkeypatch):
    # forced segments of one or two chunks, a ragged last chunk
    monkeypatch.setenv("LINATTN_SEGMENTS", "4")
    case = syn.Case("segchshort", 1, 3, 250, 128, 128, "delta", "channel", "bf16", gate_scale=0.25, s0_std=0.3,
                    case_id=170)
    x = syn.chunk_inputs(case)
    check_chunk(case, x, s0=x["s0"])


def test_chain_segments_raw_projections(monkeypatch):
    # KDA from raw projections: L2 q/k, -softplus per key channel, sigmoid beta
    import gated_delta_rule_27_amd as la
    monkeypatch.setenv("LINATTN_SEGMENTS", "3")
    case = syn.Case("segchprep", 1, 2, 1100, 128, 128, "delta", "channel", "bf16", gate_scale=1.0, s0_std=0.3,
                    case_id=171)
    x = syn.raw_inputs(case)
    d = lambda a: dev(a, case.dtype)
    o, s = la.chunk_fwd(d(x["q"]), d(x["k"]), d(x["v"]), d(x["g"]), d(x["beta"]), dev_state(x["s0"]),
                        rule="delta", gate="channel", qk_map="l2", gate_map="neg_softplus", beta_map="sigmoid")
    torch.cuda.synchronize()
    q, k = oracle.prepare_qk(x["q"], "l2"), oracle.prepare_qk(x["k"], "l2")
    g = oracle.prepare_gate(x["g"], "neg_softplus")
    b = oracle.prepare_beta(x["beta"], "sigmoid")
    oref, sref = oracle.recurrence(q, k, x["v"], g, b, x["s0"], rule="delta", gate="channel")
    eo, es = rel_l2(host(o), oref), rel_l2(host(s), sref)
    note(f"[chain segments prep] rel L2 o={eo:.3e} S={es:.3e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


@pytest.mark.parametrize("nseg", [2, 4])
@pytest.mark.parametrize("rule", ["add", "delta"])
def test_chain_segments_saved_states(monkeypatch, rule, nseg):
    # the state-keeping forward of the training path: every segment saves the
    # states of its own chunks, so output, final state and all saved states
    # equal the one-segment run bit for bit (ragged last chunk, s0 given)
    import gated_delta_rule_27_amd as la
    case = syn.Case("segchsave", 1, 2, 1250, 128, 128, rule, "channel", "bf16", gate_scale=1 / 16, s0_std=0.3,
                    case_id=173)
    x = syn.chunk_inputs(case)
    d = lambda a: dev(a, case.dtype)
    args = (d(x["q"]), d(x["k"]), d(x["v"]), d(x["g"]), d(x["beta"]), dev_state(x["s0"]))
    monkeypatch.setenv("LINATTN_SEGMENTS", str(nseg))
    on, sn, stn = la.chunk_fwd_save(*args, rule=rule, gate="channel")
    monkeypatch.setenv("LINATTN_SEGMENTS", "1")
    o1, s1, st1 = la.chunk_fwd_save(*args, rule=rule, gate="channel")
    torch.cuda.synchronize()
    note(f"[chain segments save] rule={rule} nseg={nseg}")
    assert torch.equal(on, o1) and torch.equal(sn, s1) and torch.equal(stn, st1)
    oref, sref = oracle_chunk(case, x, x["s0"])
    assert rel_l2(host(on), oref) <= TOL["bf16"] and rel_l2(host(sn), sref) <= TOL["bf16"]


def test_chain_segments_state_in_place():
    import gated_delta_rule_27_amd as la
    case = syn.Case("segchinplace", 1, 2, 1200, 128, 128, "delta", "channel", "bf16", gate_scale=1 / 16,
                    s0_std=0.3, case_id=172)
    x = syn.chunk_inputs(case)
    d = lambda a: dev(a, case.dtype)
    o_ref, s_ref = la.chunk_fwd(d(x["q"]), d(x["k"]), d(x["v"]), d(x["g"]), d(x["beta"]), dev_state(x["s0"]),
                                rule="delta", gate="channel")
    s_io = dev_state(x["s0"])
    o, s = la.chunk_fwd(d(x["q"]), d(x["k"]), d(x["v"]), d(x["g"]), d(x["beta"]), s_io, rule="delta",
                        gate="channel", s_final=s_io)
    torch.cuda.synchronize()
    assert s.data_ptr() == s_io.data_ptr()
    assert torch.equal(o, o_ref) and torch.equal(s, s_ref)


# ---- the generic path's state pass (chunk 16, 32, 128; fp32 at d_k = 128) ----

@pytest.mark.parametrize("chunk", [16, 32, 128])
@pytest.mark.parametrize("rule,gate", [("delta", "scalar"), ("delta", "channel"), ("add", "none"), ("add", "channel")])
def test_gen_segments(monkeypatch, rule, gate, chunk):
    # one head at d_v = 128: two state-pass workgroups, split into the most
    # segments; compared with the oracle and bit for bit with one segment
    case = syn.Case("seggen", 1, 1, 1300, 128, 128, rule, gate, "bf16", chunk=chunk, gate_scale=1 / 16,
                    s0_std=0.3, case_id=173)
    x = syn.chunk_inputs(case)
    check_chunk(case, x, s0=x["s0"])
    o, s = run_chunk(case, x, x["s0"])
    monkeypatch.setenv("LINATTN_SEGMENTS", "1")
    o1, s1 = run_chunk(case, x, x["s0"])
    assert torch.equal(o, o1) and torch.equal(s, s1)


def test_gen_segments_fp32(monkeypatch):
    monkeypatch.setenv("LINATTN_SEGMENTS", "3")
    case = syn.Case("seggen32", 1, 2, 700, 128, 64, "delta", "scalar", "fp32", gate_scale=1 / 16, s0_std=0.3,
                    case_id=174)
    x = syn.chunk_inputs(case)
    check_chunk(case, x, s0=x["s0"])
