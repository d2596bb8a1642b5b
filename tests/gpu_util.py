"""Helpers for the GPU parity tests: upload seeded inputs, run the HIP path,
compare with the fp64 oracle by relative L2 error."""
import sys

import numpy as np
import torch

import oracle
import synthetic as syn

# Relative L2 bounds on o and on the final state: 1e-3 for fp32 tokens,
# 2e-2 for bf16 tokens (fp32 state and accumulation in both cases).
TOL = {"fp32": 1e-3, "bf16": 2e-2}


def note(msg):
    print(msg, file=sys.stderr, flush=True)


def tdtype(dtype):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def dev(x, dtype):
    if x is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(tdtype(dtype))


def dev_state(x):
    if x is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda")


def host(t):
    return t.detach().to("cpu", torch.float64).numpy()


def rel_l2(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / (den if den > 0 else 1.0))


def worst_head(x, ref):
    """Largest per-head relative L2 error over the leading (head) axis."""
    return max(rel_l2(a, b) for a, b in zip(x.reshape(-1, *x.shape[-2:]),
                                           ref.reshape(-1, *ref.shape[-2:])))


def worst_block(x, ref, block=64):
    """Largest relative L2 error over consecutive blocks of ``block`` tokens
    (axis 0 = tokens) and the first token of that block: one wrong token moves
    a whole head's relative L2 by only ~1/sqrt(T), a block's by ~1/sqrt(block)."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    worst, at = 0.0, 0
    for t0 in range(0, ref.shape[0], block):
        e = rel_l2(x[t0:t0 + block], ref[t0:t0 + block])
        if e > worst:
            worst, at = e, t0
    return worst, at


def run_chunk(case, x, s0=None):
    import gated_delta_rule_27_amd as la
    o, s = la.chunk_fwd(dev(x["q"], case.dtype), dev(x["k"], case.dtype), dev(x["v"], case.dtype),
                        dev(x["g"], case.dtype), dev(x["beta"], case.dtype), dev_state(s0),
                        rule=case.rule, gate=case.gate, chunk=case.chunk)
    torch.cuda.synchronize()
    return o, s


def oracle_chunk(case, x, s0=None):
    return oracle.recurrence(x["q"], x["k"], x["v"], x["g"], x["beta"], s0,
                             rule=case.rule, gate=case.gate)


def check_chunk(case, x, s0=None, tol=None):
    """Full-tensor parity of one small case; returns (err_o, err_s)."""
    tol = TOL[case.dtype] if tol is None else tol
    note(f"[chunk] {case.name} rule={case.rule} gate={case.gate} dtype={case.dtype} "
         f"B={case.B} H={case.H} T={case.T} dk={case.dk} dv={case.dv}")
    o, s = run_chunk(case, x, s0)
    oref, sref = oracle_chunk(case, x, s0)
    eo, es = rel_l2(host(o), oref), rel_l2(host(s), sref)
    note(f"    rel L2 o={eo:.3e} S={es:.3e}")
    assert np.all(np.isfinite(host(o))), "non-finite output"
    assert eo <= tol, f"o rel L2 {eo:.3e} > {tol}"
    assert es <= tol, f"S rel L2 {es:.3e} > {tol}"
    return eo, es
