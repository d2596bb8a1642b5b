"""Parity of the chunk forward with input preparation fused into the kernel
(linattn_chunk_fwd_prep: raw q/k mapped by L2 or elu+1, raw gate logits by
-softplus, raw beta logits by sigmoid) with the fp64 oracle applying the same
maps to the same raw values and then running the recurrence."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from gpu_util import TOL, dev, dev_state, host, note, rel_l2

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def check_prep(case, qk_map, gate_map, beta_map):
    import gated_delta_rule_27_amd as la
    x = syn.raw_inputs(case)
    note(f"[prep] {case.rule}/{case.gate} {case.dtype} dk={case.dk} dv={case.dv} T={case.T} "
         f"qk={qk_map} g={gate_map} beta={beta_map}")
    d = lambda a: dev(a, case.dtype)
    o, s = la.chunk_fwd(d(x["q"]), d(x["k"]), d(x["v"]), d(x["g"]), d(x["beta"]),
                        dev_state(x["s0"]), rule=case.rule, gate=case.gate, qk_map=qk_map,
                        gate_map=gate_map, beta_map=beta_map)
    torch.cuda.synchronize()
    om = {"as_is": "identity"}.get(qk_map, qk_map)
    q, k = oracle.prepare_qk(x["q"], om), oracle.prepare_qk(x["k"], om)
    g = oracle.prepare_gate(x["g"], "log" if gate_map == "as_is" else gate_map)
    b = oracle.prepare_beta(x["beta"], "identity" if beta_map == "as_is" else beta_map)
    oref, sref = oracle.recurrence(q, k, x["v"], g, b, x["s0"], rule=case.rule, gate=case.gate)
    eo, es = rel_l2(host(o), oref), rel_l2(host(s), sref)
    note(f"    rel L2 o={eo:.3e} S={es:.3e}")
    assert np.all(np.isfinite(host(o)))
    assert eo <= TOL[case.dtype] and es <= TOL[case.dtype]


CASES = [
    # (rule, gate, dtype, dk, dv, qk_map, gate_map, beta_map)
    ("delta", "scalar", "bf16", 128, 128, "l2", "neg_softplus", "sigmoid"),   # GDN from projections
    ("delta", "scalar", "bf16", 64, 128, "l2", "neg_softplus", "sigmoid"),
    ("delta", "none", "bf16", 128, 64, "l2", "as_is", "sigmoid"),             # DeltaNet
    ("add", "none", "bf16", 128, 128, "elu1", "as_is", "as_is"),              # feature-map LA
    ("add", "scalar", "bf16", 64, 64, "elu1", "neg_softplus", "as_is"),
    ("delta", "scalar", "fp32", 64, 64, "l2", "neg_softplus", "sigmoid"),
    ("add", "none", "fp32", 64, 128, "elu1", "as_is", "as_is"),
]


@pytest.mark.parametrize("rule,gate,dtype,dk,dv,qk_map,gate_map,beta_map", CASES)
def test_prep_small(rule, gate, dtype, dk, dv, qk_map, gate_map, beta_map):
    # T = 200: several chunks and a ragged tail (the maps must leave padded rows zero)
    case = syn.Case("prep", 2, 2, 200, dk, dv, rule, gate, dtype, gate_scale=1.0, s0_std=0.3,
                    case_id=130)
    check_prep(case, qk_map, gate_map, beta_map)


@pytest.mark.parametrize("path", ["pipe", "fused"])
def test_prep_both_single_pass_kernels(monkeypatch, path):
    monkeypatch.setenv("LINATTN_CHUNK_PATH", path)
    case = syn.Case("prep_path", 1, 3, 333, 128, 128, "delta", "scalar", "bf16", s0_std=0.2,
                    case_id=131)
    check_prep(case, "l2", "neg_softplus", "sigmoid")


def test_prep_longer_gdn():
    case = syn.Case("prep_long", 2, 4, 2048, 128, 128, "delta", "scalar", "bf16", case_id=132)
    check_prep(case, "l2", "neg_softplus", "sigmoid")
