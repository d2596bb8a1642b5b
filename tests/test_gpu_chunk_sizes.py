"""Parity of the chunk forward at every supported chunk size and dtype with
the fp64 oracle (through the C ABI): chunk sizes 16, 32 and 128 (the generic
two-kernel path) for every rule x gate x dtype with ragged lengths and an
initial state, fp32 tokens at d_k = 128 and with the per-channel gate (chunk
64, generic path), chunk 64 through the generic path beside the tuned ones,
lengths around the chunk boundaries, strong gates, input maps from raw
projections (generic path and the per-channel gate's two-kernel path), and
the entry points built on the chunk forward (Gated DeltaProduct, normalised
attention) at other chunk sizes.  The result does not depend on the chunk
size ("Linear Attention, Visualized", "Cost"): every case is checked against
the same token recurrence."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from gpu_util import TOL, check_chunk, dev, dev_state, host, note, oracle_chunk, rel_l2, worst_block

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

RULE_GATE = [(r, g) for r in ("add", "delta") for g in ("none", "scalar", "channel")]


@pytest.mark.parametrize("chunk", [16, 32, 128])
@pytest.mark.parametrize("dtype,dk,dv", [("bf16", 128, 128), ("bf16", 64, 128), ("fp32", 64, 64),
                                         ("fp32", 128, 64)])
@pytest.mark.parametrize("rule,gate", RULE_GATE)
def test_chunk_sizes_ragged(chunk, dtype, dk, dv, rule, gate):
    # T = 300: several chunks of every size and a ragged tail; weak decay so
    # the carried state matters; nonzero initial state
    case = syn.Case("csize", 2, 2, 300, dk, dv, rule, gate, dtype, chunk=chunk, gate_scale=1 / 16,
                    s0_std=0.3, case_id=150)
    x = syn.chunk_inputs(case)
    check_chunk(case, x, s0=x["s0"])


@pytest.mark.parametrize("dv", [64, 128])
@pytest.mark.parametrize("rule,gate", RULE_GATE)
def test_fp32_dk128_and_channel(dv, rule, gate):
    # fp32 tokens at d_k = 128 (every gate) at the default chunk 64
    case = syn.Case("fp32wide", 2, 2, 200, 128, dv, rule, gate, "fp32", gate_scale=1 / 16, s0_std=0.3,
                    case_id=151)
    x = syn.chunk_inputs(case)
    check_chunk(case, x, s0=x["s0"])


@pytest.mark.parametrize("rule", ["add", "delta"])
@pytest.mark.parametrize("dv", [64, 128])
def test_fp32_channel_gate_dk64(rule, dv):
    case = syn.Case("fp32chan", 2, 3, 200, 64, dv, rule, "channel", "fp32", gate_scale=1 / 16,
                    s0_std=0.3, case_id=152)
    x = syn.chunk_inputs(case)
    check_chunk(case, x, s0=x["s0"])


@pytest.mark.parametrize("rule,gate", RULE_GATE)
def test_chunk64_generic_path(monkeypatch, rule, gate):
    # the generic path at chunk 64 (bf16), where the tuned kernels also serve
    monkeypatch.setenv("LINATTN_CHUNK_PATH", "gen")
    case = syn.Case("gen64", 2, 2, 260, 128, 128, rule, gate, "bf16", gate_scale=1 / 16, s0_std=0.3,
                    case_id=153)
    x = syn.chunk_inputs(case)
    check_chunk(case, x, s0=x["s0"])


@pytest.mark.parametrize("T", [1, 15, 16, 17, 127, 128, 129, 255, 257])
@pytest.mark.parametrize("chunk", [16, 32, 128])
def test_lengths_around_chunk_boundaries(chunk, T):
    # chunks of 16 and 32 tokens share a workgroup four or two at a time: these
    # lengths leave the last workgroup of a head with fewer chunks than that
    case = syn.Case("csize_len", 1, 2, T, 128, 128, "delta", "scalar", "bf16", chunk=chunk, gate_scale=0.1,
                    s0_std=0.2, case_id=154)
    x = syn.chunk_inputs(case)
    check_chunk(case, x, s0=x["s0"])


@pytest.mark.parametrize("chunk", [16, 32])
@pytest.mark.parametrize("rule,gate", [("add", "none"), ("delta", "none"), ("add", "scalar")])
def test_shared_workgroup_rules(chunk, rule, gate):
    # several heads, an odd number of chunks per head (the last workgroup of each
    # head holds fewer chunks), both rules and gate kinds, fp32 and bf16 tokens
    for dtype in ("bf16", "fp32"):
        case = syn.Case("csize_shared", 2, 3, 4 * chunk + 7, 64, 128, rule, gate, dtype, chunk=chunk,
                        gate_scale=0.1, s0_std=0.2, case_id=157)
        x = syn.chunk_inputs(case)
        check_chunk(case, x, s0=x["s0"])


@pytest.mark.parametrize("chunk", [32, 128])
@pytest.mark.parametrize("gate", ["scalar", "channel"])
@pytest.mark.parametrize("scale", [1.0, 12.0, 30.0])
def test_strong_gates(chunk, gate, scale):
    # the workloads' gate law and log-gates of ~ -10 and ~ -24 per token: the
    # decay of a 128-token chunk is far below fp32's range
    case = syn.Case("csize_law", 1, 2, 300, 128, 128, "delta", gate, "bf16", chunk=chunk, gate_scale=scale,
                    s0_std=0.2, case_id=155)
    x = syn.chunk_inputs(case)
    check_chunk(case, x, s0=x["s0"])


@pytest.mark.parametrize("rule,gate,dtype,chunk,qk_map,gate_map,beta_map", [
    ("delta", "scalar", "bf16", 32, "l2", "neg_softplus", "sigmoid"),
    ("delta", "channel", "bf16", 128, "l2", "neg_softplus", "sigmoid"),
    ("add", "none", "fp32", 16, "elu1", "as_is", "as_is"),
    ("delta", "channel", "fp32", 64, "l2", "neg_softplus", "sigmoid"),
    ("add", "channel", "bf16", 64, "elu1", "neg_softplus", "as_is"),     # two-kernel path
    ("delta", "channel", "bf16", 64, "l2", "neg_softplus", "sigmoid"),   # two-kernel path (KDA)
])
def test_prep_maps(rule, gate, dtype, chunk, qk_map, gate_map, beta_map):
    import gated_delta_rule_27_amd as la
    dk = 128 if dtype == "bf16" else 64
    case = syn.Case("csize_prep", 2, 2, 200, dk, 128, rule, gate, dtype, chunk=chunk, s0_std=0.3,
                    case_id=156)
    x = syn.raw_inputs(case)
    note(f"[prep] {rule}/{gate} {dtype} chunk={chunk} qk={qk_map} g={gate_map} beta={beta_map}")
    d = lambda a: dev(a, dtype)
    o, s = la.chunk_fwd(d(x["q"]), d(x["k"]), d(x["v"]), d(x["g"]), d(x["beta"]), dev_state(x["s0"]),
                        rule=rule, gate=gate, chunk=chunk, qk_map=qk_map, gate_map=gate_map,
                        beta_map=beta_map)
    torch.cuda.synchronize()
    om = {"as_is": "identity"}.get(qk_map, qk_map)
    q, k = oracle.prepare_qk(x["q"], om), oracle.prepare_qk(x["k"], om)
    g = oracle.prepare_gate(x["g"], "log" if gate_map == "as_is" else gate_map)
    b = None if x["beta"] is None else oracle.prepare_beta(x["beta"], "identity" if beta_map == "as_is"
                                                           else beta_map)
    oref, sref = oracle.recurrence(q, k, x["v"], g, b, x["s0"], rule=rule, gate=gate)
    eo, es = rel_l2(host(o), oref), rel_l2(host(s), sref)
    note(f"    rel L2 o={eo:.3e} S={es:.3e}")
    assert np.all(np.isfinite(host(o)))
    assert eo <= TOL[dtype] and es <= TOL[dtype]


@pytest.mark.parametrize("chunk", [16, 32, 128])
def test_gdn_workload_sampled_heads(chunk):
    # the B8 H16 T8192 GDN workload at every other chunk size, sampled heads
    # against the oracle, each 64-token block within the bound
    import gated_delta_rule_27_amd as la
    case = syn.CFG3.with_(chunk=chunk)
    x = syn.chunk_inputs(case)
    d = {kk: dev(vv, case.dtype) for kk, vv in x.items() if kk != "s0"}
    note(f"[full] GDN B8 H16 T8192 chunk={chunk}")
    o, s = la.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], None, rule="delta", gate="scalar",
                        chunk=chunk)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all()
    for (b, h) in [(0, 0), (7, 15)]:
        xs = {kk: (None if vv is None else vv[b:b + 1, h:h + 1]) for kk, vv in x.items()}
        oref, sref = oracle_chunk(case, xs)
        oh = host(o[b, h])
        eo, es = rel_l2(oh, oref[0, 0]), rel_l2(host(s[b, h]), sref[0, 0])
        wb, at = worst_block(oh, oref[0, 0])
        note(f"    head ({b},{h}): rel L2 o={eo:.3e} S={es:.3e}; worst 64-token block {wb:.3e} at t={at}")
        assert eo <= TOL["bf16"] and es <= TOL["bf16"] and wb <= TOL["bf16"]


def test_chunk_size_independence():
    # one problem at every chunk size: the outputs agree with each other to
    # rounding (bf16 tokens, weak decay so the state carries across chunks)
    import gated_delta_rule_27_amd as la
    case = syn.Case("csize_all", 2, 3, 500, 128, 128, "delta", "scalar", "bf16", gate_scale=1 / 32,
                    s0_std=0.3, case_id=157)
    x = syn.chunk_inputs(case)
    d = {kk: dev(vv, case.dtype) for kk, vv in x.items() if kk != "s0"}
    oref, sref = oracle_chunk(case, x, x["s0"])
    outs = {}
    for c in (16, 32, 64, 128):
        o, s = la.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], dev_state(x["s0"]), chunk=c)
        torch.cuda.synchronize()
        outs[c] = (host(o), host(s))
        note(f"    chunk {c}: rel L2 o={rel_l2(outs[c][0], oref):.3e} S={rel_l2(outs[c][1], sref):.3e}")
        assert rel_l2(outs[c][0], oref) <= TOL["bf16"] and rel_l2(outs[c][1], sref) <= TOL["bf16"]
    for c in (16, 32, 128):
        assert rel_l2(outs[c][0], outs[64][0]) <= 2 * TOL["bf16"]


@pytest.mark.parametrize("chunk", [32, 128])
def test_deltaproduct_other_chunk(chunk):
    import gated_delta_rule_27_amd as la
    case = syn.DeltaProductCase("dp_csize", 1, 2, 90, 2, 128, 128, "scalar", "bf16", gate_scale=0.2,
                                s0_std=0.2, case_id=158)
    x = syn.deltaproduct_inputs(case)
    d = lambda a: dev(a, case.dtype)
    o, s = la.deltaproduct_fwd(d(x["q"]), d(x["k"]), d(x["v"]), d(x["g"]), d(x["beta"]), dev_state(x["s0"]),
                               gate="scalar", chunk=chunk)
    torch.cuda.synchronize()
    oref, sref = oracle.deltaproduct(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], gate="scalar")
    eo, es = rel_l2(host(o), oref), rel_l2(host(s), sref)
    note(f"[dp chunk={chunk}] rel L2 o={eo:.3e} S={es:.3e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


@pytest.mark.parametrize("chunk", [16, 128])
def test_normalized_other_chunk(chunk):
    import gated_delta_rule_27_amd as la
    case = syn.Case("norm_csize", 1, 2, 170, 128, 128, "add", "scalar", "bf16", qk="elu1", chunk=chunk,
                    gate_scale=0.25, case_id=159)
    x = syn.chunk_inputs(case)
    rng = np.random.default_rng([syn.SEED, 159])
    z0 = np.abs(rng.standard_normal((1, 2, 128))).astype(np.float32)
    d = lambda a: dev(a, case.dtype)
    o, s, z = la.chunk_fwd_normalized(d(x["q"]), d(x["k"]), d(x["v"]), d(x["g"]), None, dev_state(z0),
                                      gate="scalar", chunk=chunk)
    torch.cuda.synchronize()
    oref, sref, zref = oracle.normalized(x["q"], x["k"], x["v"], x["g"], None, z0, gate="scalar")
    eo, ez = rel_l2(host(o), oref), rel_l2(host(z), zref)
    note(f"[norm chunk={chunk}] rel L2 o={eo:.3e} z={ez:.3e}")
    assert eo <= TOL["bf16"] and ez <= TOL["bf16"]
