"""Parity of normalised linear attention (HIP, through the C ABI: one fused pass
carrying the key sum for no gate and the scalar gate, two add-rule passes and a
division for the per-channel gate or when another chunk path is selected) with
the fp64 oracle's normalised recurrence: positive
features (elu + 1), every head size and dtype, no gate / scalar gate /
per-channel gate, carried S_0 and z_0, the feature map fused from raw
projections, empty sequences and resume."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from gpu_util import TOL, dev, dev_state, host, note, rel_l2

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def inputs(case, rng_id):
    x = syn.chunk_inputs(case)
    rng = np.random.default_rng([syn.SEED, rng_id])
    z0 = np.abs(rng.standard_normal((case.B, case.H, case.dk))).astype(np.float32)
    s0 = None if x["s0"] is None else np.abs(x["s0"]).astype(np.float32)
    return x, s0, z0


def check(case, x, s0, z0, **maps):
    import gated_delta_rule_27_amd as la
    note(f"[norm] {case.gate} {case.dtype} dk={case.dk} dv={case.dv} T={case.T} {maps}")
    d = lambda a: dev(a, case.dtype)
    o, s, z = la.chunk_fwd_normalized(d(x["q"]), d(x["k"]), d(x["v"]), d(x["g"]), dev_state(s0),
                                      dev_state(z0), gate=case.gate, **maps)
    torch.cuda.synchronize()
    q, k = x["q"], x["k"]
    if maps.get("qk_map") == "elu1":
        q, k = oracle.prepare_qk(q, "elu1"), oracle.prepare_qk(k, "elu1")
    oref, sref, zref = oracle.normalized(q, k, x["v"], x["g"], s0, z0, gate=case.gate)
    eo, es, ez = rel_l2(host(o), oref), rel_l2(host(s), sref), rel_l2(host(z), zref)
    note(f"    rel L2 o={eo:.3e} S={es:.3e} z={ez:.3e}")
    tol = TOL[case.dtype]
    assert np.all(np.isfinite(host(o)))
    assert eo <= tol and es <= tol and ez <= tol
    return o, s, z


CASES = []
for dtype, dims in (("bf16", ((64, 64), (128, 128), (64, 128), (128, 64))), ("fp32", ((64, 64),))):
    for (dk, dv) in dims:
        for gate in ("none", "scalar"):
            CASES.append((dtype, dk, dv, gate))


@pytest.mark.parametrize("dtype,dk,dv,gate", CASES)
def test_small_ragged(dtype, dk, dv, gate):
    case = syn.Case("norm", 2, 2, 200, dk, dv, "add", gate, dtype, qk="elu1", gate_scale=0.25,
                    s0_std=0.3, case_id=140)
    x, s0, z0 = inputs(case, 140)
    check(case, x, s0, z0)


@pytest.mark.parametrize("path,gate", [("pipe", "none"), ("split", "scalar"), ("pipe", "scalar")])
def test_two_pass_route(monkeypatch, path, gate):
    # another chunk path selected: the two add-rule passes and the division
    monkeypatch.setenv("LINATTN_CHUNK_PATH", path)
    case = syn.Case("norm_route", 1, 3, 170, 128, 128, "add", gate, "bf16", qk="elu1", gate_scale=0.25,
                    s0_std=0.3, case_id=145)
    x, s0, z0 = inputs(case, 145)
    check(case, x, s0, z0)


@pytest.mark.parametrize("gate", ["none", "scalar"])
def test_long_sequence(gate):
    # 63 chunks and a ragged tail through the one-pass kernel, no initial states
    case = syn.Case("norm_long", 1, 2, 4001, 128, 128, "add", gate, "bf16", qk="elu1", gate_scale=0.05,
                    case_id=146)
    x, _, _ = inputs(case, 146)
    check(case, x, None, None)


def test_channel_gate():
    case = syn.Case("norm_chan", 1, 2, 150, 128, 128, "add", "channel", "bf16", qk="elu1",
                    gate_scale=0.1, s0_std=0.3, case_id=141)
    x, s0, z0 = inputs(case, 141)
    check(case, x, s0, z0)


def test_feature_map_from_raw_projections():
    # q, k raw Gaussian; elu + 1 applied inside the kernel
    case = syn.Case("norm_raw", 2, 2, 130, 128, 128, "add", "scalar", "bf16", qk="gauss",
                    gate_scale=0.25, case_id=142)
    x, _, z0 = inputs(case, 142)
    check(case, x, None, None, qk_map="elu1")


def test_zero_tokens_returns_states():
    import gated_delta_rule_27_amd as la
    rng = np.random.default_rng(143)
    s0 = rng.random((1, 2, 64, 64)).astype(np.float32)
    z0 = rng.random((1, 2, 64)).astype(np.float32)
    e = lambda *shape: torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    o, s, z = la.chunk_fwd_normalized(e(1, 2, 0, 64), e(1, 2, 0, 64), e(1, 2, 0, 64), None,
                                      dev_state(s0), dev_state(z0))
    torch.cuda.synchronize()
    assert o.numel() == 0
    assert np.array_equal(host(s), s0.astype(np.float64)) and np.array_equal(host(z), z0.astype(np.float64))


def test_resume_equals_one_pass():
    case = syn.Case("norm_resume", 1, 2, 300, 128, 128, "add", "scalar", "bf16", qk="elu1",
                    gate_scale=0.1, case_id=144)
    import gated_delta_rule_27_amd as la
    x, _, _ = inputs(case, 144)
    d = lambda a: dev(a, case.dtype)
    o, s, z = la.chunk_fwd_normalized(d(x["q"]), d(x["k"]), d(x["v"]), d(x["g"]), gate="scalar")
    cut = 131
    part = lambda a, sl: d(np.ascontiguousarray(a[:, :, sl]))
    o1, s1, z1 = la.chunk_fwd_normalized(part(x["q"], slice(0, cut)), part(x["k"], slice(0, cut)),
                                         part(x["v"], slice(0, cut)), part(x["g"], slice(0, cut)),
                                         gate="scalar")
    o2, s2, z2 = la.chunk_fwd_normalized(part(x["q"], slice(cut, None)), part(x["k"], slice(cut, None)),
                                         part(x["v"], slice(cut, None)), part(x["g"], slice(cut, None)),
                                         s1, z1, gate="scalar")
    torch.cuda.synchronize()
    assert rel_l2(host(torch.cat([o1, o2], dim=2)), host(o)) < 1e-2
    assert rel_l2(host(s2), host(s)) < 1e-2 and rel_l2(host(z2), host(z)) < 1e-2


@pytest.mark.parametrize("gate", ["none", "scalar"])
def test_key_sum_in_place(gate):
    # z_final aliasing z0 (and s_final aliasing s0): the key sum carried in
    # place.  d_v = 128 gives every head two value-block workgroups that read
    # z0, and 256 heads put them in more than one wave of workgroups, so a
    # block that started after its partner finished would read the advanced
    # key sum if the entry point did not read z0 from a copy.
    import gated_delta_rule_27_amd as la
    case = syn.Case("norm_inplace", 4, 64, 150, 128, 128, "add", gate, "bf16", qk="elu1",
                    gate_scale=0.25, s0_std=0.3, case_id=147)
    x, s0, z0 = inputs(case, 147)
    d = lambda a: dev(a, case.dtype)
    ref_o, ref_s, ref_z = la.chunk_fwd_normalized(d(x["q"]), d(x["k"]), d(x["v"]), d(x["g"]), dev_state(s0),
                                                  dev_state(z0), gate=gate)
    s_io, z_io = dev_state(s0), dev_state(z0)
    o, s, z = la.chunk_fwd_normalized(d(x["q"]), d(x["k"]), d(x["v"]), d(x["g"]), s_io, z_io, gate=gate,
                                      s_final=s_io, z_final=z_io)
    torch.cuda.synchronize()
    assert z.data_ptr() == z_io.data_ptr() and s.data_ptr() == s_io.data_ptr()
    assert torch.equal(o, ref_o), "in-place key sum changed the output"
    assert torch.equal(s, ref_s) and torch.equal(z, ref_z)
    oref, sref, zref = oracle.normalized(x["q"], x["k"], x["v"], x["g"], s0, z0, gate=gate)
    eo, ez = rel_l2(host(o), oref), rel_l2(host(z), zref)
    note(f"[norm in place] {gate}: rel L2 o={eo:.3e} z={ez:.3e}")
    assert eo <= TOL["bf16"] and ez <= TOL["bf16"]


def test_key_sum_partial_overlap_rejected():
    import gated_delta_rule_27_amd as la
    e = lambda *shape: torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
    zbuf = torch.zeros(2 * 2 * 64 + 4, dtype=torch.float32, device="cuda")
    z0 = zbuf[:256].view(1, 2, 128)
    zf = zbuf[4:260].view(1, 2, 128)
    with pytest.raises(la.LinattnError) as ei:
        la.chunk_fwd_normalized(e(1, 2, 10, 128), e(1, 2, 10, 128), e(1, 2, 10, 64), None, None, z0,
                                z_final=zf)
    assert ei.value.status == 6
