"""The chunk forward that allocates nothing (linattn_chunk_fwd_noalloc, through
the C ABI): its staged per-chunk operands live in the library's static device
array instead of a caller workspace.  Two calls in a row, the second smaller,
must give the same outputs as linattn_chunk_fwd with a workspace (same
kernels: bit for bit) and match the oracle; a problem whose workspace exceeds
the array is refused before anything runs."""
import ctypes

import numpy as np
import pytest
import torch

import synthetic as syn
from gpu_util import TOL, dev, dev_state, host, note, oracle_chunk, rel_l2

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def run_both(case):
    import gated_delta_rule_27_amd as la
    x = syn.chunk_inputs(case)
    d = lambda a: dev(a, case.dtype)
    args = (d(x["q"]), d(x["k"]), d(x["v"]), d(x["g"]), d(x["beta"]), dev_state(x["s0"]))
    kw = dict(rule=case.rule, gate=case.gate, chunk=case.chunk)
    need = la.chunk_workspace_bytes(case.B, case.H, case.T, case.dk, case.dv, rule=case.rule, gate=case.gate,
                                    dtype=case.dtype, chunk=case.chunk)
    assert 0 < need <= (64 << 20), "the case must use the scratch and fit it"
    out = torch.empty(case.B, case.H, case.T, case.dv, dtype=args[0].dtype, device="cuda")
    sfin = torch.empty(case.B, case.H, case.dk, case.dv, dtype=torch.float32, device="cuda")
    o1, s1 = la.chunk_fwd(*args, **kw, out=out, s_final=sfin, no_alloc=True)
    o2, s2 = la.chunk_fwd(*args, **kw)
    torch.cuda.synchronize()
    oref, sref = oracle_chunk(case, x, x["s0"])
    eo, es = rel_l2(host(o1), oref), rel_l2(host(s1), sref)
    note(f"[noalloc] {case.name} {case.rule}/{case.gate} chunk={case.chunk} workspace {need} B: "
         f"rel L2 o={eo:.3e} S={es:.3e}")
    assert torch.equal(o1, o2) and torch.equal(s1, s2), "scratch run differs from the workspace run"
    assert eo <= TOL[case.dtype] and es <= TOL[case.dtype]


def test_two_calls_second_smaller():
    # KDA-style per-channel gate (two-kernel path), then a smaller problem on
    # the generic path at chunk 32: the second call reuses the array the first
    # filled
    run_both(syn.Case("noalloc_big", 2, 4, 1000, 128, 128, "delta", "channel", "bf16", gate_scale=0.1,
                      s0_std=0.2, case_id=160))
    run_both(syn.Case("noalloc_small", 1, 2, 300, 128, 128, "delta", "scalar", "bf16", chunk=32,
                      gate_scale=0.1, s0_std=0.2, case_id=161))


def test_too_large_is_refused():
    import gated_delta_rule_27_amd as la
    from gated_delta_rule_27_amd import _binding as bd
    lib = la.load()
    a = bd.chunk_args(1, 32, 262144, 128, 128, rule="delta", gate="channel", dtype="bf16")
    assert lib.linattn_chunk_workspace_bytes(ctypes.byref(a)) > (64 << 20)
    F = ctypes.c_void_p(0x10000)
    st = lib.linattn_chunk_fwd_noalloc(ctypes.byref(a), None, F, F, F, F, F, None, F, None, None)
    assert st == 4
