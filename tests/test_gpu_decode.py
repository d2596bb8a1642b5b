"""Parity of the decode step (HIP, through the C ABI) with the fp64 oracle:
every rule x gate x dtype x head size over several steps, the 256 x 32 x 128
workload over all 1000 steps on sampled sequences, and decode == chunk
forward."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from gpu_util import TOL, dev, dev_state, host, note, rel_l2

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def run_steps(case, steps, sample=None):
    """Run `steps` decode steps on all sequences; compare sampled sequences
    (all when sample is None) with the oracle at every step."""
    import gated_delta_rule_27_amd as la
    note(f"[decode] {case.name} rule={case.rule} gate={case.gate} dtype={case.dtype} "
         f"N={case.N} H={case.H} dk={case.dk} dv={case.dv} steps={steps}")
    s0 = syn.decode_state(case)
    st = dev_state(s0)
    idx = np.arange(case.N) if sample is None else np.asarray(sample)
    ref = s0[idx].astype(np.float64)
    worst = 0.0
    for t in range(steps):
        x = syn.decode_tokens(case, t)
        o = la.decode_step(dev(x["q"], case.dtype), dev(x["k"], case.dtype),
                           dev(x["v"], case.dtype), dev(x["g"], case.dtype),
                           dev(x["beta"], case.dtype), st, rule=case.rule, gate=case.gate)
        sub = {kk: (None if vv is None else vv[idx]) for kk, vv in x.items()}
        oref, ref = oracle.decode_step(sub["q"], sub["k"], sub["v"], sub["g"], sub["beta"], ref,
                                       rule=case.rule, gate=case.gate)
        e = rel_l2(host(o)[idx], oref)
        worst = max(worst, e)
        assert e <= TOL[case.dtype], f"step {t}: o rel L2 {e:.3e}"
    torch.cuda.synchronize()
    es = rel_l2(host(st)[idx], ref)
    note(f"    worst step o rel L2 {worst:.3e}; final state rel L2 {es:.3e}")
    assert es <= TOL[case.dtype]


CASES = []
for dtype in ("bf16", "fp32"):
    for (dk, dv) in ((64, 64), (64, 128), (128, 64), (128, 128)):
        for rule in ("add", "delta"):
            for gate in ("none", "scalar", "channel"):
                CASES.append((dtype, dk, dv, rule, gate))


@pytest.mark.parametrize("dtype,dk,dv,rule,gate", CASES)
def test_decode_variants(dtype, dk, dv, rule, gate):
    case = syn.DecodeCase("dec", 3, 5, dk, dv, 6, rule, gate, dtype, state_std=0.5,
                          gate_scale=0.2, case_id=200)
    run_steps(case, 6)


@pytest.mark.timeout(600)
def test_cfg5_decode_1000_steps_sampled():
    run_steps(syn.CFG5, syn.CFG5.steps, sample=[0, 77, 255])


def test_decode_steps_equal_chunk_forward():
    import gated_delta_rule_27_amd as la
    case = syn.Case("x", 2, 4, 150, 128, 128, "delta", "scalar", "bf16", gate_scale=1 / 16,
                    s0_std=0.2, case_id=201)
    x = syn.chunk_inputs(case)
    d = {kk: dev(vv, case.dtype) for kk, vv in x.items() if kk != "s0"}
    o, s = la.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], dev_state(x["s0"]))
    st = dev_state(x["s0"])
    outs = []
    for t in range(case.T):
        sl = lambda n: d[n][:, :, t].contiguous()
        outs.append(la.decode_step(sl("q"), sl("k"), sl("v"), sl("g"), sl("beta"), st))
    torch.cuda.synchronize()
    od = torch.stack(outs, dim=2)
    assert rel_l2(host(od), host(o)) < 1e-2
    assert rel_l2(host(st), host(s)) < 1e-2
