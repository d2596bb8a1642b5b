"""Benchmark: chunkwise forward (gated delta rule, B=8, H=16, T=8192,
dk=dv=128, bf16 tokens, fp32 state, chunk 64) and the decode step (256
sequences x 32 heads, dk=dv=128, fp32 state, bf16 tokens, 1000 steps) on one
MI355X.

One step = one chunkwise forward over the whole batch; ``value`` is its
throughput in tokens/s (B*T per step).  The decode step is timed separately
over its own step count and reported under ``decode`` as state GB/s against
the HBM peak.  Inputs are seeded synthetic tensors already resident in HBM
when timing starts.  Kernel times come from HIP events recorded on the stream
the kernels are launched on (torch's current stream).

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "tokens/s chunk fwd (H=16,d=128,T=8192) + decode state GB/s vs peak"
SETTLE_STEPS = 100    # untimed headline steps before timing, warm-up included
CSRC = os.path.join(ROOT, "gated_delta_rule_27_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")
# the sources each measured kernel is built from: counter figures in profiles/
# are valid only while these hash to the value recorded with them
CHUNK_SOURCES = ("chunk_pipe.hip", "mfma.h", "tsolve.h", "device_common.h", "prep.h")
DECODE_SOURCES = ("decode_step.hip", "device_common.h")
CHUNK_PROFILE = "chunk_pipe_gdn_B8_H16_T8192_d128.md"
DECODE_PROFILE = "decode_step_gdn_N256_H32_d128.md"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
MFMA_FP32_PEAK_TFLOPS = 157.3   # MI355X dense fp32 matrix peak (fp32 tokens: fp32 operands)


def chunk_alg_bytes(B, H, T, dk, dv, s, rule, gate, with_state=True):
    """Bytes the chunk forward must move at minimum: q, k, v in, o out, the
    gate and beta, the fp32 final state."""
    per_tok = (2 * dk + 2 * dv) * s
    if gate == "scalar":
        per_tok += s
    elif gate == "channel":
        per_tok += dk * s
    if rule == "delta":
        per_tok += s
    return B * H * T * per_tok + (B * H * dk * dv * 4 if with_state else 0)


def chunk_nominal_flops(B, H, T, dk, dv, rule, C=64):
    """Nominal FLOPs per head-token at chunk size C (dense C x C tiles, the
    O(C^2) triangular solve excluded)."""
    if rule == "delta":
        f = 2 * (3 * C * dk + 2 * C * dv + 3 * dk * dv)
    else:
        f = 2 * (C * dk + C * dv + 2 * dk * dv)
    return B * H * T * f


def decode_alg_bytes(N, H, dk, dv, s, rule, gate):
    per_head = 2 * dk * dv * 4 + (2 * dk + 2 * dv) * s
    if gate == "scalar":
        per_head += s
    elif gate == "channel":
        per_head += dk * s
    if rule == "delta":
        per_head += s
    return N * H * per_head


def sources_sha256(names):
    import hashlib
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def counter_traffic(profile, sources):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when it is missing or was taken on different kernel sources."""
    path = os.path.join(PROFILES, profile)
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line:
            key, _, val = line.partition(":")
            vals[key.strip()] = val.strip()
    if vals.get("kernel_sources_sha256") != sources_sha256(sources):
        return None
    try:
        return int(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def time_chunk(la, syn, case, dev, steps, warmup=20):
    """Event-timed chunk forward of one workload (inputs resident in HBM); the
    figures of a secondary line beside the headline one."""
    import torch
    B, H, T, dk, dv = case.B, case.H, case.T, case.dk, case.dv
    x = syn.chunk_inputs_torch(case, dev)
    tdt = torch.bfloat16 if case.dtype == "bf16" else torch.float32
    out = torch.empty((B, H, T, dv), dtype=tdt, device=dev)
    s_fin = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    wsb = la.chunk_workspace_bytes(B, H, T, dk, dv, rule=case.rule, gate=case.gate, dtype=case.dtype,
                                   chunk=case.chunk)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev) if wsb else None

    def step():
        la.chunk_fwd(x["q"], x["k"], x["v"], x.get("g"), x.get("beta"), None, rule=case.rule,
                     gate=case.gate, chunk=case.chunk, out=out, s_final=s_fin, workspace=ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    s = 2 if case.dtype == "bf16" else 4
    abytes = chunk_alg_bytes(B, H, T, dk, dv, s, case.rule, case.gate)
    aflops = chunk_nominal_flops(B, H, T, dk, dv, case.rule, case.chunk)
    return {"workload": f"{case.rule}/{case.gate} chunk_fwd B={B} H={H} T={T} dk={dk} dv={dv} "
                        f"chunk={case.chunk} {case.dtype} tokens fp32 state",
            "ms_per_step": round(ms, 4), "tokens_per_s": round(B * T / (ms * 1e-3), 1),
            "hbm_frac": round(abytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "mfma_frac": round(aflops / (ms * 1e-3) / 1e12 / (MFMA_BF16_PEAK_TFLOPS if case.dtype == "bf16"
                                                             else MFMA_FP32_PEAK_TFLOPS), 4),
            "mfma_peak_TFLOPs": MFMA_BF16_PEAK_TFLOPS if case.dtype == "bf16" else MFMA_FP32_PEAK_TFLOPS,
            "path": chunk_path(case, wsb), "steps": steps}


def time_prep(la, case, dev, steps, warmup=20):
    """Event-timed chunk forward from raw projections with the input
    preparation fused into the kernel (q, k L2-normalised, log-gate
    -softplus per token or per key channel, beta sigmoid), at the shape and
    gate of ``case``; raw inputs drawn on the device (q, k N(0,1) * 2, gate and
    beta logits N(0,1))."""
    import torch
    B, H, T, dk, dv = case.B, case.H, case.T, case.dk, case.dv
    gen = torch.Generator(device=dev)
    gen.manual_seed(27 * 1000 + 77)
    rn = lambda *sh: torch.randn(*sh, generator=gen, device=dev, dtype=torch.float32)
    q, k = (rn(B, H, T, dk) * 2).bfloat16(), (rn(B, H, T, dk) * 2).bfloat16()
    gshape = (B, H, T, dk) if case.gate == "channel" else (B, H, T)
    v, g, beta = rn(B, H, T, dv).bfloat16(), rn(*gshape).bfloat16(), rn(B, H, T).bfloat16()
    out = torch.empty((B, H, T, dv), dtype=torch.bfloat16, device=dev)
    s_fin = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    wsb = la.chunk_workspace_bytes(B, H, T, dk, dv, rule="delta", gate=case.gate)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev) if wsb else None

    def step():
        la.chunk_fwd(q, k, v, g, beta, None, rule="delta", gate=case.gate, out=out, s_final=s_fin,
                     workspace=ws, qk_map="l2", gate_map="neg_softplus", beta_map="sigmoid")

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    abytes = chunk_alg_bytes(B, H, T, dk, dv, 2, "delta", case.gate)
    aflops = chunk_nominal_flops(B, H, T, dk, dv, "delta")
    kind = "kda" if case.gate == "channel" else "gdn"
    return {"workload": f"{kind} chunk_fwd from raw projections (fused L2 q/k, -softplus gate, "
                        f"sigmoid beta) B={B} H={H} T={T} dk={dk} dv={dv} bf16",
            "ms_per_step": round(ms, 4), "tokens_per_s": round(B * T / (ms * 1e-3), 1),
            "hbm_frac": round(abytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "mfma_frac": round(aflops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "path": ("split" if case.gate == "channel" else "pipe") + " with input preparation", "steps": steps}


def time_normalized(la, syn, case, dev, steps, warmup=20):
    """Event-timed normalised linear attention (no gate or a scalar gate: one
    fused pass that carries the key sum beside the state) at the shape and input
    laws of ``case``; minimal bytes as for the add rule plus the fp32 key sum."""
    import torch
    B, H, T, dk, dv = case.B, case.H, case.T, case.dk, case.dv
    x = syn.chunk_inputs_torch(case, dev)
    out = torch.empty((B, H, T, dv), dtype=torch.bfloat16, device=dev)
    s_fin = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    z_fin = torch.empty((B, H, dk), dtype=torch.float32, device=dev)
    wsb = la.normalized_workspace_bytes(B, H, T, dk, dv, gate=case.gate)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)

    def step():
        la.chunk_fwd_normalized(x["q"], x["k"], x["v"], x["g"], None, None, gate=case.gate, out=out,
                                s_final=s_fin, z_final=z_fin, workspace=ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    abytes = chunk_alg_bytes(B, H, T, dk, dv, 2, "add", case.gate) + B * H * dk * 4
    aflops = chunk_nominal_flops(B, H, T, dk, dv, "add")
    return {"workload": f"normalised {case.gate}-gate linear attention (elu+1 features) "
                        f"B={B} H={H} T={T} dk={dk} dv={dv} bf16",
            "ms_per_step": round(ms, 4), "tokens_per_s": round(B * T / (ms * 1e-3), 1),
            "hbm_frac": round(abytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "mfma_frac": round(aflops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "path": "fused, one pass with the key sum", "steps": steps}


def time_deltaproduct(la, syn, case, dev, steps, warmup=20):
    """Event-timed Gated DeltaProduct forward (inputs resident in HBM).  Minimal
    bytes: q and o once, k, v and beta per substep, the gate and the final
    state; nominal FLOPs: the GDN count over the n_h T virtual steps."""
    import torch
    B, H, T, nh, dk, dv = case.B, case.H, case.T, case.nh, case.dk, case.dv
    x = syn.deltaproduct_inputs_torch(case, dev)
    out = torch.empty((B, H, T, dv), dtype=torch.bfloat16, device=dev)
    s_fin = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    wsb = la.deltaproduct_workspace_bytes(B, H, T, nh, dk, dv, gate=case.gate)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev) if wsb else None

    def step():
        la.deltaproduct_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], None, gate=case.gate,
                            out=out, s_final=s_fin, workspace=ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    s = 2
    abytes = B * H * T * ((dk + dv) * s + nh * (dk + dv + 1) * s + (s if case.gate == "scalar" else 0)) \
        + B * H * dk * dv * 4
    aflops = chunk_nominal_flops(B, H, T * nh, dk, dv, "delta")
    return {"workload": f"gated deltaproduct n_h={nh} B={B} H={H} T={T} dk={dk} dv={dv} "
                        f"bf16 tokens fp32 state (virtual length {T * nh})",
            "ms_per_step": round(ms, 4), "tokens_per_s": round(B * T / (ms * 1e-3), 1),
            "hbm_frac": round(abytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "mfma_frac": round(aflops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "path": "pipe over the virtual sequence in place (no expand or gather)", "steps": steps}


def bwd_alg_bytes(B, H, T, dk, dv, s, rule, gate, states):
    """Bytes the backward pass must move at minimum: q, k, v, dO (and g, beta)
    in, dq, dk, dv (and dg, dbeta) out, plus the saved chunk states when they
    are read (one per chunk, token dtype)."""
    per_tok = (2 * dk + 2 * dv) * s + (2 * dk + dv) * s
    if gate == "scalar":
        per_tok += 2 * s
    elif gate == "channel":
        per_tok += 2 * dk * s
    if rule == "delta":
        per_tok += 2 * s
    nch = (T + 63) // 64
    return B * H * T * per_tok + (B * H * nch * dk * dv * s if states else 0)


def bwd_nominal_flops(B, H, T, dk, dv, C=64):
    """Nominal FLOPs per head-token of the delta-rule backward as built: the
    operand pass (A, L), the reverse state pass (A^T dO, ->K dS, Tb^T dZ,
    <-Q^T dO, <-K^T dR) and the gradient pass (A, L, R, Z, dZ, dR, d<-Q, d<-K,
    d->K, dA, dTb, T^T dTb, dM, P K, P^T Q, P2 K, P2^T K)."""
    macs = 8 * C * dk + 7 * C * dv + 8 * dk * dv + 2 * C * C
    return B * H * T * 2 * macs


def rmw_ceiling(dev, mib=1024, reps=20):
    """Read-modify-write bandwidth a plain streaming kernel reaches on this
    device: torch's in-place scale of a ``mib`` MiB fp32 buffer (every byte
    read once and written once, like the decode step's state), HIP events; 23
    halvings of ones stay normal fp32."""
    import torch
    x = torch.ones(mib * (1 << 20) // 4, dtype=torch.float32, device=dev)
    for _ in range(3):
        x.mul_(0.5)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        x.mul_(0.5)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del x
    return {"kernel": f"torch in-place scale of {mib} MiB fp32", "GBps": round(2 * mib * (1 << 20) / (ms * 1e-3) / 1e9, 1)}


def mfma_achievable(dev, grid=2048, iters=20000, reps=5):
    """Dense bf16 matrix-core throughput a register-only MFMA loop reaches on
    this device (``peak/mfma_peak.hip``: 8 independent accumulation chains per
    wave, 4 waves per workgroup, no memory traffic in the loop), for the two
    bf16 shapes; the best of ``reps`` event-timed launches of each."""
    import ctypes

    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "gated_delta_rule_27_amd", "libmfmapeak.so"))
    lib.mfma_peak_threads.restype = ctypes.c_int
    lib.mfma_peak_flops.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.mfma_peak_flops.restype = ctypes.c_double
    lib.mfma_peak_launch.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.mfma_peak_launch.restype = ctypes.c_int
    out = torch.empty(grid * lib.mfma_peak_threads(), dtype=torch.float32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    res = {"kernel": f"register-only MFMA loop, {grid} workgroups x 4 waves x {iters} rounds of 8 chains"}
    for shape, name in ((0, "16x16x32_bf16"), (1, "32x32x16_bf16")):
        best = None
        for r in range(reps + 1):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            rc = lib.mfma_peak_launch(shape, grid, iters, ctypes.c_void_p(out.data_ptr()), stream)
            e1.record()
            torch.cuda.synchronize()
            if rc != 0:
                raise RuntimeError(f"mfma_peak_launch failed ({rc})")
            ms = e0.elapsed_time(e1)
            if r > 0 and (best is None or ms < best):
                best = ms
        res[f"TFLOPs_{name}"] = round(lib.mfma_peak_flops(shape, grid, iters) / (best * 1e-3) / 1e12, 1)
    del out
    return res


def time_backward(la, syn, case, dev, steps, warmup=2):
    """Event-timed training passes at the shape and laws of ``case``: the
    forward that keeps the chunk states, the backward from those states, and
    the backward that recomputes them."""
    import torch
    B, H, T, dk, dv = case.B, case.H, case.T, case.dk, case.dv
    x = syn.chunk_inputs_torch(case, dev)
    do = syn.grad_inputs_torch(case, dev)["do"]
    out = torch.empty((B, H, T, dv), dtype=torch.bfloat16, device=dev)
    states = torch.empty(la.chunk_states_shape(B, H, T, dk, dv), dtype=torch.bfloat16, device=dev)
    grads = {"dq": torch.empty_like(x["q"]), "dk": torch.empty_like(x["k"]), "dv": torch.empty_like(x["v"]),
             "dg": torch.empty_like(x["g"]), "dbeta": torch.empty_like(x["beta"]),
             "ds0": torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)}
    ws = torch.empty(la.chunk_bwd_workspace_bytes(B, H, T, dk, dv, rule=case.rule, gate=case.gate,
                                                  states_given=False), dtype=torch.uint8, device=dev)
    fws = None
    if case.gate == "channel":
        fws = torch.empty(la.chunk_workspace_bytes(B, H, T, dk, dv, rule=case.rule, gate=case.gate),
                          dtype=torch.uint8, device=dev)
    args = (x["q"], x["k"], x["v"], x["g"], x["beta"])

    def fwd():
        la.chunk_fwd_save(*args, rule=case.rule, gate=case.gate, out=out, states=states, return_state=False,
                          workspace=fws)

    def bwd_saved():
        la.chunk_bwd(*args, do, states=states, rule=case.rule, gate=case.gate, workspace=ws, grads=grads)

    def bwd_recompute():
        la.chunk_bwd(*args, do, rule=case.rule, gate=case.gate, workspace=ws, grads=grads)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    ms_f, ms_b, ms_r = timed(fwd), timed(bwd_saved), timed(bwd_recompute)
    abytes = bwd_alg_bytes(B, H, T, dk, dv, 2, case.rule, case.gate, True)
    aflops = bwd_nominal_flops(B, H, T, dk, dv)
    kind = {("delta", "scalar"): "gdn", ("delta", "channel"): "kda", ("add", "channel"): "gla"}.get(
        (case.rule, case.gate), f"{case.rule}/{case.gate}")
    path = ("split+save; bwd_ops_channel + bwd_chain + bwd_grad_channel" if case.gate == "channel"
            else "fused+save; bwd_ops + bwd_chain + bwd_grad")
    return {"workload": f"{kind} training passes B={B} H={H} T={T} dk={dk} dv={dv} bf16 (backward "
                        f"from dO, chunk states saved by the forward)",
            "fwd_save_ms": round(ms_f, 4), "bwd_ms": round(ms_b, 4), "bwd_recompute_ms": round(ms_r, 4),
            "ms_per_step": round(ms_f + ms_b, 4),
            "tokens_per_s": round(B * T / ((ms_f + ms_b) * 1e-3), 1),
            "bwd_hbm_frac": round(abytes / (ms_b * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "bwd_mfma_frac": round(aflops / (ms_b * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "bwd_alg_bytes": abytes, "bwd_nominal_flops": aflops,
            "path": path, "steps": steps}


def time_deltaproduct_bwd(la, syn, case, dev, steps, warmup=2):
    """Event-timed Gated DeltaProduct backward (GDN backward over the virtual
    sequence, its states recomputed) at the shape and laws of ``case``."""
    import torch
    B, H, T, nh, dk, dv = case.B, case.H, case.T, case.nh, case.dk, case.dv
    x = syn.deltaproduct_inputs_torch(case, dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(syn.SEED * 1000 + 600)
    do = torch.randn(B, H, T, dv, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    grads = {"dq": torch.empty_like(x["q"]), "dk": torch.empty_like(x["k"]), "dv": torch.empty_like(x["v"]),
             "dg": torch.empty_like(x["g"]), "dbeta": torch.empty_like(x["beta"]),
             "ds0": torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)}
    ws = torch.empty(la.deltaproduct_bwd_workspace_bytes(B, H, T, nh, dk, dv, gate=case.gate, dtype=case.dtype),
                     dtype=torch.uint8, device=dev)

    def step():
        la.deltaproduct_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], do, gate=case.gate, workspace=ws,
                            grads=grads)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    return {"workload": f"gated deltaproduct backward n_h={nh} B={B} H={H} T={T} dk={dk} dv={dv} bf16 "
                        f"(states recomputed)",
            "ms_per_step": round(ms, 4), "tokens_per_s": round(B * T / (ms * 1e-3), 1),
            "path": "expand + fused+save + bwd_ops + bwd_chain + bwd_grad over the virtual sequence + picks",
            "steps": steps}


def chunk_path(case, wsb):
    """Which chunk kernel the library runs for this case (its dispatch rule)."""
    if case.chunk != 64 or (case.dtype == "fp32" and (case.dk != 64 or case.gate == "channel")) \
            or os.environ.get("LINATTN_CHUNK_PATH") == "gen":
        return "gen"
    if wsb:
        return "split"
    env = os.environ.get("LINATTN_CHUNK_PATH")
    if env in ("fused", "pipe") and (env == "fused" or case.dtype == "bf16"):
        return env
    return "pipe" if case.dtype == "bf16" and case.rule == "delta" else "fused"


CHUNK_KERNELS = {"pipe": "chunk_pipe_kernel", "fused": "chunk_fused_kernel",
                 "split": "chunk_intra_channel_kernel + chunk_chain_kernel",
                 "gen": "gen_intra_kernel + gen_chain_kernel"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # 100 warm-up steps: from idle the GPU's clocks ramp for ~60 steps of this
    # workload (per-step times fall from ~580 to ~400 us); the timed steps are
    # the steady state
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peak-probe", action="store_true",
                    help="skip the register-only MFMA loop that measures the achievable matrix-core rate")
    ap.add_argument("--cpu-heads", type=int, default=128,
                    help="heads of the workload the CPU oracle runs for its baseline")
    ap.add_argument("--path", choices=["pipe", "fused", "split"], default=None,
                    help="chunk path for the scalar gate (default: the library's choice: the "
                         "pipelined single-pass kernel for the delta rule with bf16 tokens)")
    ap.add_argument("--other-configs",
                    default="cfg2,cfg3b,cfg4,gdp2,cfg3prep,cfg4prep,cfg2norm,cfg3bwd,gdp2bwd,cfg4bwd,"
                            "cfg3c16,cfg3c32,cfg3c128,cfg3fp32",
                    help="comma-separated secondary chunk workloads to time after the headline "
                         "one (cfg2, cfg3b, cfg4, gdp2, cfg3prep, cfg4prep, cfg2norm, cfg3bwd, gdp2bwd, "
                         "cfg4bwd, cfg3c16/cfg3c32/cfg3c128 (the GDN workload at other chunk sizes), "
                         "cfg3fp32 (fp32 tokens), cfg4fp32 (KDA with fp32 tokens, T = 65536)), or 'none'")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (5 times): the reference "
                         "for scaling HBM byte counters")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        n = args.copy_calibration * (1 << 20)
        a = torch.ones(n, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 5}))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}): the library has no "
              "multi-GPU path; each head's recurrence is independent, so a multi-GPU run "
              "would shard heads with no communication", file=sys.stderr)
        sys.exit(2)

    if args.path:
        os.environ["LINATTN_CHUNK_PATH"] = args.path
    import torch

    import gated_delta_rule_27_amd as la
    import synthetic as syn
    if not os.path.exists(la.LIB_PATH):
        from gated_delta_rule_27_amd import build
        build.build(verbose=False)
    la.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # ---------------- chunkwise forward -------------------------------------
    case = syn.CFG3
    B, H, T, dk, dv = case.B, case.H, case.T, case.dk, case.dv
    x = syn.chunk_inputs_torch(case, dev)
    out = torch.empty((B, H, T, dv), dtype=torch.bfloat16, device=dev)
    s_fin = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    wsb = la.chunk_workspace_bytes(B, H, T, dk, dv, rule=case.rule, gate=case.gate)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev) if wsb else None
    path = chunk_path(case, wsb)

    def step():
        la.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], None, rule=case.rule,
                     gate=case.gate, out=out, s_final=s_fin, workspace=ws)

    # at least SETTLE_STEPS untimed steps before the timed ones, whatever
    # --warmup asks for: from idle the GPU's clocks take ~60 steps of this
    # workload to settle, and the timed steps measure the steady state
    settle = max(0, SETTLE_STEPS - args.warmup)
    for _ in range(settle + args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    tokens_per_s = B * T / (ms * 1e-3)
    abytes = chunk_alg_bytes(B, H, T, dk, dv, 2, case.rule, case.gate)
    aflops = chunk_nominal_flops(B, H, T, dk, dv, case.rule)
    gbps = abytes / (ms * 1e-3) / 1e9
    tflops = aflops / (ms * 1e-3) / 1e12

    # ---------------- measured matrix-core ceiling -------------------------------
    peak = None if args.no_peak_probe else mfma_achievable(dev)

    # ---------------- secondary chunk workloads (reported beside the headline) ----
    others = []
    names = [n for n in args.other_configs.split(",") if n and n != "none"]
    del x, out, s_fin, ws
    torch.cuda.empty_cache()
    for name in names:
        if name == "gdp2":
            others.append(time_deltaproduct(la, syn, syn.GDP2, dev, steps=10))
        elif name == "cfg3prep":
            others.append(time_prep(la, syn.CFG3, dev, steps=10))
        elif name == "cfg4prep":
            others.append(time_prep(la, syn.CFG4, dev, steps=3, warmup=2))
        elif name in ("cfg3c16", "cfg3c32", "cfg3c128"):
            others.append(time_chunk(la, syn, syn.CFG3.with_(chunk=int(name[5:])), dev, steps=5, warmup=3))
        elif name == "cfg3fp32":
            others.append(time_chunk(la, syn, syn.CFG3.with_(dtype="fp32"), dev, steps=5, warmup=3))
        elif name == "cfg4fp32":
            others.append(time_chunk(la, syn, syn.CFG4.with_(dtype="fp32", T=65536), dev, steps=3, warmup=2))
        elif name == "cfg2norm":
            others.append(time_normalized(la, syn, syn.CFG2, dev, steps=50, warmup=100))
        elif name == "cfg3bwd":
            others.append(time_backward(la, syn, syn.CFG3, dev, steps=5))
        elif name == "cfg4bwd":
            others.append(time_backward(la, syn, syn.CFG4, dev, steps=3))
        elif name == "gdp2bwd":
            others.append(time_deltaproduct_bwd(la, syn, syn.GDP2, dev, steps=5))
        else:
            oc = {"cfg2": syn.CFG2, "cfg3b": syn.CFG3B, "cfg4": syn.CFG4}[name]
            # the short workloads get 100 untimed steps, so the clocks have ramped
            others.append(time_chunk(la, syn, oc, dev, steps=3 if name == "cfg4" else 50,
                                     warmup=20 if name == "cfg4" else 100))
        print(f"bench: {name} done ({others[-1]['ms_per_step']} ms per step)", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()

    # ---------------- decode step --------------------------------------------
    decode = None
    if args.decode_steps > 0:
        dc = syn.CFG5
        nsteps = args.decode_steps
        tok = syn.decode_tokens_torch(dc, nsteps, dev)
        state = syn.decode_state_torch(dc, dev)
        od = torch.empty((dc.N, dc.H, dc.dv), dtype=torch.bfloat16, device=dev)

        def dstep(i):
            la.decode_step(tok["q"][i], tok["k"][i], tok["v"][i], tok["g"][i], tok["beta"][i],
                           state, rule=dc.rule, gate=dc.gate, out=od)

        for i in range(min(10, nsteps)):
            dstep(i)
        torch.cuda.synchronize()
        d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        d0.record()
        for i in range(nsteps):
            dstep(i)
        d1.record()
        torch.cuda.synchronize()
        us = d0.elapsed_time(d1) * 1e3 / nsteps
        dbytes = decode_alg_bytes(dc.N, dc.H, dc.dk, dc.dv, 2, dc.rule, dc.gate)
        dgbps = dbytes / (us * 1e-6) / 1e9
        decode = {
            "workload": f"gdn_decode N={dc.N} H={dc.H} dk={dc.dk} dv={dc.dv} bf16 tokens, "
                        f"fp32 state, {nsteps} steps",
            "us_per_step": round(us, 3),
            "tokens_per_s": round(dc.N / (us * 1e-6), 1),
            "state_GBps": round(dgbps, 1),
            "hbm_frac": round(dgbps / HBM_PEAK_GBPS, 4),
            "alg_bytes_per_step": dbytes,
            "traffic": counter_traffic(DECODE_PROFILE, DECODE_SOURCES),
            "rmw_ceiling": rmw_ceiling(dev),
        }
        decode["frac_of_rmw_ceiling"] = round(dgbps / decode["rmw_ceiling"]["GBps"], 4)
        del tok, state

    # ---------------- CPU oracle baseline ------------------------------------
    cpu = None
    if not args.no_cpu_baseline and int(os.environ.get("RANK", "0")) == 0:
        import oracle
        nh = max(1, min(args.cpu_heads, B * H))
        sel = lambda t: t.reshape(B * H, *t.shape[2:])[:nh].unsqueeze(0).to("cpu", torch.float64).numpy()
        x = syn.chunk_inputs_torch(case, dev)
        xs = {n: sel(x[n]) for n in ("q", "k", "v", "g", "beta")}
        del x
        cores = len(os.sched_getaffinity(0))
        t0 = time.perf_counter()
        oracle.recurrence(xs["q"], xs["k"], xs["v"], xs["g"], xs["beta"], None, rule=case.rule,
                          gate=case.gate, nthreads=cores)
        wall = time.perf_counter() - t0
        # one thread on a subset of the same heads, to show how the oracle scales
        n1 = min(8, nh)
        xs1 = {n: v[:, :n1] for n, v in xs.items()}
        t1 = time.perf_counter()
        oracle.recurrence(xs1["q"], xs1["k"], xs1["v"], xs1["g"], xs1["beta"], None, rule=case.rule,
                          gate=case.gate, nthreads=1)
        wall1 = time.perf_counter() - t1
        cpu = {
            "value": round(nh * T / H / wall, 1),
            "unit": "tokens/s",
            "cores": cores,
            "kind": "oracle",
            "sample": f"{nh} of {B * H} heads x {T} tokens of the same workload (fp64 "
                      f"token recurrence, OpenMP over heads), {wall:.2f} s wall; tokens/s = "
                      f"head-tokens / {H} heads / wall",
            "cpu_model": cpu_model(),
            "one_thread": {"value": round(n1 * T / H / wall1, 1), "unit": "tokens/s", "cores": 1,
                           "sample": f"{n1} heads x {T} tokens, {wall1:.2f} s wall",
                           "speedup_all_cores": round((nh / wall) / (n1 / wall1), 2)},
        }

    line = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_steps": settle,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"gdn_chunk_fwd B={B} H={H} T={T} dk={dk} dv={dv} chunk=64 "
                               f"bf16 tokens fp32 state",
                   "B": B, "H": H, "T": T, "dk": dk, "dv": dv, "chunk": 64,
                   "rule": case.rule, "gate": case.gate, "parallelism": "single GPU",
                   "path": path},
        # the chunk forward is a dense contraction judged by its matrix-core
        # fraction; its HBM fraction (minimal bytes) stands beside it
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": counter_traffic(CHUNK_PROFILE, CHUNK_SOURCES) if path == "pipe" else None,
                     "kernel": CHUNK_KERNELS[path],
                     "nominal_flops_per_launch": aflops,
                     "frac_of_measured_peak": (round(tflops / peak["TFLOPs_16x16x32_bf16"], 4)
                                               if peak else None)},
        "roofline_hbm": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
                         "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4),
                         "alg_bytes_per_launch": abytes},
        "mfma_achievable": peak,
        "decode": decode,
        "other_chunk_workloads": others,
        "cpu_baseline": cpu,
        "gpu": torch.cuda.get_device_name(dev),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
