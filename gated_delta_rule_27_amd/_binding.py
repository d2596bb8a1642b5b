"""ctypes binding of ``liblinattn.so`` (see ``include/linattn.h``).

Argument marshalling only: tensors are checked (device, dtype, shape,
contiguity), their device pointers and torch's current HIP stream are handed
to the C ABI, and a nonzero status becomes an exception.  Every step of the
computation runs in the library's HIP kernels; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblinattn.so")

RULES = {"add": 0, "delta": 1}
GATES = {"none": 0, "scalar": 1, "channel": 2}
DTYPES = {"fp32": 0, "bf16": 1}

# Every function the header declares; a test checks the two stay in step.
EXPORTS = ("linattn_abi_version", "linattn_status_string", "linattn_chunk_workspace_bytes",
           "linattn_chunk_fwd", "linattn_decode_step", "linattn_deltaproduct_workspace_bytes",
           "linattn_deltaproduct_fwd", "linattn_chunk_fwd_prep",
           "linattn_normalized_workspace_bytes", "linattn_chunk_fwd_normalized",
           "linattn_chunk_fwd_save", "linattn_chunk_bwd_workspace_bytes", "linattn_chunk_bwd",
           "linattn_deltaproduct_bwd_workspace_bytes", "linattn_deltaproduct_bwd",
           "linattn_chunk_fwd_noalloc")
QK_MAPS = {"as_is": 0, "l2": 1, "elu1": 2}
GATE_MAPS = {"as_is": 0, "neg_softplus": 1}
BETA_MAPS = {"as_is": 0, "sigmoid": 1}


class LinattnError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} (status {status})")
        self.status = status


class ChunkArgs(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("H", ctypes.c_int64), ("T", ctypes.c_int64),
                ("dk", ctypes.c_int32), ("dv", ctypes.c_int32), ("chunk", ctypes.c_int32),
                ("rule", ctypes.c_int32), ("gate", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class PrepArgs(ctypes.Structure):
    _fields_ = [("qk_map", ctypes.c_int32), ("gate_map", ctypes.c_int32),
                ("beta_map", ctypes.c_int32)]


class DeltaProductArgs(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("H", ctypes.c_int64), ("T", ctypes.c_int64),
                ("nh", ctypes.c_int32), ("dk", ctypes.c_int32), ("dv", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("gate", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class DecodeArgs(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int64), ("H", ctypes.c_int64),
                ("dk", ctypes.c_int32), ("dv", ctypes.c_int32),
                ("rule", ctypes.c_int32), ("gate", ctypes.c_int32), ("dtype", ctypes.c_int32)]


_lock = threading.Lock()
_lib = None


def load(path: str = LIB_PATH):
    """Load the HIP library; raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is missing: build it first (python -m gated_delta_rule_27_amd.build "
                "or __graft_entry__.build()); there is no non-HIP fallback")
        lib = ctypes.CDLL(path)
        vp, sz = ctypes.c_void_p, ctypes.c_size_t
        lib.linattn_abi_version.argtypes = []
        lib.linattn_abi_version.restype = ctypes.c_int
        lib.linattn_status_string.argtypes = [ctypes.c_int]
        lib.linattn_status_string.restype = ctypes.c_char_p
        lib.linattn_chunk_workspace_bytes.argtypes = [ctypes.POINTER(ChunkArgs)]
        lib.linattn_chunk_workspace_bytes.restype = sz
        lib.linattn_chunk_fwd.argtypes = [ctypes.POINTER(ChunkArgs), vp, vp, vp, vp, vp, vp, vp,
                                          vp, vp, sz, vp]
        lib.linattn_chunk_fwd.restype = ctypes.c_int
        lib.linattn_decode_step.argtypes = [ctypes.POINTER(DecodeArgs), vp, vp, vp, vp, vp, vp,
                                            vp, vp]
        lib.linattn_decode_step.restype = ctypes.c_int
        lib.linattn_deltaproduct_workspace_bytes.argtypes = [ctypes.POINTER(DeltaProductArgs)]
        lib.linattn_deltaproduct_workspace_bytes.restype = sz
        lib.linattn_deltaproduct_fwd.argtypes = [ctypes.POINTER(DeltaProductArgs), vp, vp, vp, vp, vp,
                                                 vp, vp, vp, vp, sz, vp]
        lib.linattn_deltaproduct_fwd.restype = ctypes.c_int
        lib.linattn_chunk_fwd_prep.argtypes = [ctypes.POINTER(ChunkArgs), ctypes.POINTER(PrepArgs),
                                               vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.linattn_chunk_fwd_prep.restype = ctypes.c_int
        lib.linattn_normalized_workspace_bytes.argtypes = [ctypes.POINTER(ChunkArgs)]
        lib.linattn_normalized_workspace_bytes.restype = sz
        lib.linattn_chunk_fwd_normalized.argtypes = [ctypes.POINTER(ChunkArgs), ctypes.POINTER(PrepArgs),
                                                     vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.linattn_chunk_fwd_normalized.restype = ctypes.c_int
        lib.linattn_chunk_fwd_save.argtypes = [ctypes.POINTER(ChunkArgs), vp, vp, vp, vp, vp, vp, vp,
                                               vp, vp, vp, sz, vp]
        lib.linattn_chunk_fwd_save.restype = ctypes.c_int
        lib.linattn_chunk_bwd_workspace_bytes.argtypes = [ctypes.POINTER(ChunkArgs), ctypes.c_int]
        lib.linattn_chunk_bwd_workspace_bytes.restype = sz
        lib.linattn_chunk_bwd.argtypes = [ctypes.POINTER(ChunkArgs), vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                          vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.linattn_chunk_bwd.restype = ctypes.c_int
        lib.linattn_deltaproduct_bwd_workspace_bytes.argtypes = [ctypes.POINTER(DeltaProductArgs)]
        lib.linattn_deltaproduct_bwd_workspace_bytes.restype = sz
        lib.linattn_deltaproduct_bwd.argtypes = [ctypes.POINTER(DeltaProductArgs), vp, vp, vp, vp, vp, vp, vp,
                                                 vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.linattn_deltaproduct_bwd.restype = ctypes.c_int
        lib.linattn_chunk_fwd_noalloc.argtypes = [ctypes.POINTER(ChunkArgs), ctypes.POINTER(PrepArgs), vp, vp, vp,
                                                  vp, vp, vp, vp, vp, vp]
        lib.linattn_chunk_fwd_noalloc.restype = ctypes.c_int
        _lib = lib
    return _lib


def abi_version() -> int:
    return int(load().linattn_abi_version())


def status_string(status: int) -> str:
    return load().linattn_status_string(int(status)).decode()


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _token_dtype(t):
    import torch
    if t.dtype == torch.bfloat16:
        return "bf16"
    if t.dtype == torch.float32:
        return "fp32"
    raise TypeError(f"token tensors must be bfloat16 or float32, got {t.dtype}")


def _check(t, name, shape, dtype, device):
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def chunk_args(B, H, T, dk, dv, *, rule, gate, dtype, chunk=64) -> ChunkArgs:
    return ChunkArgs(B, H, T, dk, dv, chunk, RULES[rule], GATES[gate], DTYPES[dtype])


def chunk_workspace_bytes(B, H, T, dk, dv, *, rule, gate, dtype="bf16", chunk=64) -> int:
    a = chunk_args(B, H, T, dk, dv, rule=rule, gate=gate, dtype=dtype, chunk=chunk)
    return int(load().linattn_chunk_workspace_bytes(ctypes.byref(a)))


def chunk_fwd(q, k, v, g=None, beta=None, s0=None, *, rule="delta", gate="scalar", chunk=64,
              out=None, s_final=None, return_state=True, workspace=None, qk_map="as_is",
              gate_map="as_is", beta_map="as_is", no_alloc=False):
    """Chunkwise forward over whole sequences on the GPU.

    q, k [B,H,T,dk]; v [B,H,T,dv]; g [B,H,T] (scalar gate) or [B,H,T,dk]
    (channel gate) or None; beta [B,H,T] (delta rule) or None; s0
    [B,H,dk,dv] fp32 or None.  Returns (o [B,H,T,dv], S_T [B,H,dk,dv] fp32 or
    None).  Runs on torch's current stream of q's device, asynchronously.
    qk_map ("as_is" | "l2" | "elu1"), gate_map ("as_is" | "neg_softplus") and
    beta_map ("as_is" | "sigmoid") treat q/k, g and beta as raw projections
    mapped inside the kernel (linattn_chunk_fwd_prep).  no_alloc=True calls
    linattn_chunk_fwd_noalloc: the library's static device scratch replaces the
    workspace (pass out and s_final to allocate nothing at all).
    """
    import torch
    lib = load()
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    dtype = _token_dtype(q)
    _check(q, "q", (B, H, T, dk), dt, dev)
    _check(k, "k", (B, H, T, dk), dt, dev)
    _check(v, "v", (B, H, T, dv), dt, dev)
    if gate == "scalar":
        _check(g, "g", (B, H, T), dt, dev)
    elif gate == "channel":
        _check(g, "g", (B, H, T, dk), dt, dev)
    elif g is not None:
        raise ValueError("g must be None when gate='none'")
    if rule == "delta":
        _check(beta, "beta", (B, H, T), dt, dev)
    elif beta is not None:
        raise ValueError("beta must be None for the add rule")
    if s0 is not None:
        _check(s0, "s0", (B, H, dk, dv), torch.float32, dev)
    if out is None:
        out = torch.empty((B, H, T, dv), dtype=dt, device=dev)
    else:
        _check(out, "out", (B, H, T, dv), dt, dev)
    if s_final is None and return_state:
        s_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    elif s_final is not None:
        _check(s_final, "s_final", (B, H, dk, dv), torch.float32, dev)
    a = chunk_args(B, H, T, dk, dv, rule=rule, gate=gate, dtype=dtype, chunk=chunk)
    stream = torch.cuda.current_stream(dev).cuda_stream
    if no_alloc:
        pa = PrepArgs(QK_MAPS[qk_map], GATE_MAPS[gate_map], BETA_MAPS[beta_map])
        st = lib.linattn_chunk_fwd_noalloc(ctypes.byref(a), ctypes.byref(pa), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                           _ptr(beta), _ptr(s0), _ptr(out), _ptr(s_final), stream)
        if st != 0:
            raise LinattnError(st, "linattn_chunk_fwd_noalloc")
        return out, s_final
    need = int(lib.linattn_chunk_workspace_bytes(ctypes.byref(a)))
    if need > 0 and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if (qk_map, gate_map, beta_map) == ("as_is", "as_is", "as_is"):
        st = lib.linattn_chunk_fwd(ctypes.byref(a), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                   _ptr(s0), _ptr(out), _ptr(s_final), _ptr(workspace), ws_bytes,
                                   stream)
        what = "linattn_chunk_fwd"
    else:
        pa = PrepArgs(QK_MAPS[qk_map], GATE_MAPS[gate_map], BETA_MAPS[beta_map])
        st = lib.linattn_chunk_fwd_prep(ctypes.byref(a), ctypes.byref(pa), _ptr(q), _ptr(k), _ptr(v),
                                        _ptr(g), _ptr(beta), _ptr(s0), _ptr(out), _ptr(s_final),
                                        _ptr(workspace), ws_bytes, stream)
        what = "linattn_chunk_fwd_prep"
    if st != 0:
        raise LinattnError(st, what)
    return out, s_final


def decode_step(q, k, v, g, beta, state, *, rule="delta", gate="scalar", out=None):
    """One decode step for N sequences x H heads; ``state`` [N,H,dk,dv] fp32 is
    updated in place.  q, k [N,H,dk]; v [N,H,dv]; g [N,H] | [N,H,dk] | None;
    beta [N,H] | None.  Returns o [N,H,dv]."""
    import torch
    lib = load()
    N, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    dtype = _token_dtype(q)
    _check(k, "k", (N, H, dk), dt, dev)
    _check(v, "v", (N, H, dv), dt, dev)
    _check(q, "q", (N, H, dk), dt, dev)
    if gate == "scalar":
        _check(g, "g", (N, H), dt, dev)
    elif gate == "channel":
        _check(g, "g", (N, H, dk), dt, dev)
    elif g is not None:
        raise ValueError("g must be None when gate='none'")
    if rule == "delta":
        _check(beta, "beta", (N, H), dt, dev)
    elif beta is not None:
        raise ValueError("beta must be None for the add rule")
    _check(state, "state", (N, H, dk, dv), torch.float32, dev)
    if out is None:
        out = torch.empty((N, H, dv), dtype=dt, device=dev)
    else:
        _check(out, "out", (N, H, dv), dt, dev)
    a = DecodeArgs(N, H, dk, dv, RULES[rule], GATES[gate], DTYPES[dtype])
    stream = torch.cuda.current_stream(dev).cuda_stream
    st = lib.linattn_decode_step(ctypes.byref(a), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                 _ptr(state), _ptr(out), stream)
    if st != 0:
        raise LinattnError(st, "linattn_decode_step")
    return out


def deltaproduct_args(B, H, T, nh, dk, dv, *, gate, dtype, chunk=64) -> DeltaProductArgs:
    return DeltaProductArgs(B, H, T, nh, dk, dv, chunk, GATES[gate], DTYPES[dtype])


def deltaproduct_workspace_bytes(B, H, T, nh, dk, dv, *, gate="scalar", dtype="bf16",
                                 chunk=64) -> int:
    a = deltaproduct_args(B, H, T, nh, dk, dv, gate=gate, dtype=dtype, chunk=chunk)
    return int(load().linattn_deltaproduct_workspace_bytes(ctypes.byref(a)))


def deltaproduct_fwd(q, k, v, g=None, beta=None, s0=None, *, gate="scalar", chunk=64, out=None,
                     s_final=None, return_state=True, workspace=None):
    """Gated DeltaProduct forward on the GPU (n_h delta-rule substeps per token).

    q [B,H,T,dk]; k [B,H,T,nh,dk]; v [B,H,T,nh,dv]; g [B,H,T] (scalar gate) or
    None; beta [B,H,T,nh]; s0 [B,H,dk,dv] fp32 or None.  Returns
    (o [B,H,T,dv], S_T [B,H,dk,dv] fp32 or None).  Runs on torch's current
    stream of q's device, asynchronously.
    """
    import torch
    lib = load()
    B, H, T, dk = q.shape
    nh, dv = k.shape[3], v.shape[-1]
    dev, dt = q.device, q.dtype
    dtype = _token_dtype(q)
    _check(q, "q", (B, H, T, dk), dt, dev)
    _check(k, "k", (B, H, T, nh, dk), dt, dev)
    _check(v, "v", (B, H, T, nh, dv), dt, dev)
    _check(beta, "beta", (B, H, T, nh), dt, dev)
    if gate == "scalar":
        _check(g, "g", (B, H, T), dt, dev)
    elif gate != "none" or g is not None:
        raise ValueError("Gated DeltaProduct takes gate='scalar' with g, or gate='none'")
    if s0 is not None:
        _check(s0, "s0", (B, H, dk, dv), torch.float32, dev)
    if out is None:
        out = torch.empty((B, H, T, dv), dtype=dt, device=dev)
    else:
        _check(out, "out", (B, H, T, dv), dt, dev)
    if s_final is None and return_state:
        s_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    elif s_final is not None:
        _check(s_final, "s_final", (B, H, dk, dv), torch.float32, dev)
    a = deltaproduct_args(B, H, T, nh, dk, dv, gate=gate, dtype=dtype, chunk=chunk)
    need = int(lib.linattn_deltaproduct_workspace_bytes(ctypes.byref(a)))
    if need > 0 and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    stream = torch.cuda.current_stream(dev).cuda_stream
    st = lib.linattn_deltaproduct_fwd(ctypes.byref(a), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                      _ptr(s0), _ptr(out), _ptr(s_final), _ptr(workspace), ws_bytes,
                                      stream)
    if st != 0:
        raise LinattnError(st, "linattn_deltaproduct_fwd")
    return out, s_final


def normalized_workspace_bytes(B, H, T, dk, dv, *, gate="none", dtype="bf16", chunk=64) -> int:
    a = chunk_args(B, H, T, dk, dv, rule="add", gate=gate, dtype=dtype, chunk=chunk)
    return int(load().linattn_normalized_workspace_bytes(ctypes.byref(a)))


def chunk_fwd_normalized(q, k, v, g=None, s0=None, z0=None, *, gate="none", chunk=64, out=None,
                         s_final=None, z_final=None, return_state=True, workspace=None,
                         qk_map="as_is", gate_map="as_is"):
    """Normalised linear attention on the GPU: o_t = (q_t S_t) / (q_t . z_t), add
    rule, z_t the decayed running key sum.  q, k [B,H,T,dk]; v [B,H,T,dv];
    g [B,H,T] | [B,H,T,dk] | None; s0 [B,H,dk,dv] and z0 [B,H,dk] fp32 or None.
    Returns (o, S_T, z_T).  qk_map / gate_map as for chunk_fwd."""
    import torch
    lib = load()
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    dtype = _token_dtype(q)
    _check(q, "q", (B, H, T, dk), dt, dev)
    _check(k, "k", (B, H, T, dk), dt, dev)
    _check(v, "v", (B, H, T, dv), dt, dev)
    if gate == "scalar":
        _check(g, "g", (B, H, T), dt, dev)
    elif gate == "channel":
        _check(g, "g", (B, H, T, dk), dt, dev)
    elif g is not None:
        raise ValueError("g must be None when gate='none'")
    if s0 is not None:
        _check(s0, "s0", (B, H, dk, dv), torch.float32, dev)
    if z0 is not None:
        _check(z0, "z0", (B, H, dk), torch.float32, dev)
    if out is None:
        out = torch.empty((B, H, T, dv), dtype=dt, device=dev)
    else:
        _check(out, "out", (B, H, T, dv), dt, dev)
    if return_state:
        if s_final is None:
            s_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
        if z_final is None:
            z_final = torch.empty((B, H, dk), dtype=torch.float32, device=dev)
    for t, name, shape in ((s_final, "s_final", (B, H, dk, dv)), (z_final, "z_final", (B, H, dk))):
        if t is not None:
            _check(t, name, shape, torch.float32, dev)
    a = chunk_args(B, H, T, dk, dv, rule="add", gate=gate, dtype=dtype, chunk=chunk)
    need = int(lib.linattn_normalized_workspace_bytes(ctypes.byref(a)))
    if need > 0 and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    pa = PrepArgs(QK_MAPS[qk_map], GATE_MAPS[gate_map], 0)
    stream = torch.cuda.current_stream(dev).cuda_stream
    st = lib.linattn_chunk_fwd_normalized(ctypes.byref(a), ctypes.byref(pa), _ptr(q), _ptr(k), _ptr(v),
                                          _ptr(g), _ptr(s0), _ptr(z0), _ptr(out), _ptr(s_final),
                                          _ptr(z_final), _ptr(workspace), ws_bytes, stream)
    if st != 0:
        raise LinattnError(st, "linattn_chunk_fwd_normalized")
    return out, s_final, z_final


def _train_inputs(q, k, v, g, beta, rule, gate):
    """Shapes, dtype and device of a training-pass problem."""
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    _check(q, "q", (B, H, T, dk), dt, dev)
    _check(k, "k", (B, H, T, dk), dt, dev)
    _check(v, "v", (B, H, T, dv), dt, dev)
    if gate == "scalar":
        _check(g, "g", (B, H, T), dt, dev)
    elif gate == "channel":
        _check(g, "g", (B, H, T, dk), dt, dev)
    elif gate == "none":
        if g is not None:
            raise ValueError("g must be None when gate='none'")
    else:
        raise ValueError(f"unknown gate {gate!r}")
    if rule == "delta":
        _check(beta, "beta", (B, H, T), dt, dev)
    elif beta is not None:
        raise ValueError("beta must be None for the add rule")
    return B, H, T, dk, dv, dev, dt


def chunk_states_shape(B, H, T, dk, dv, chunk=64):
    """Shape of the per-chunk states chunk_fwd_save keeps: [B,H,ceil(T/64),dk,dv]
    (in the token dtype)."""
    return (B, H, (T + chunk - 1) // chunk, dk, dv)


def chunk_fwd_save(q, k, v, g=None, beta=None, s0=None, *, rule="delta", gate="scalar", chunk=64,
                   out=None, s_final=None, states=None, return_state=True, workspace=None):
    """Chunk forward that also returns the state entering every chunk, for
    chunk_bwd.  Returns (o, S_T or None, states [B,H,N,dk,dv] in the token
    dtype).  The per-channel gate needs a workspace (allocated here unless
    given, at least chunk_workspace_bytes)."""
    import torch
    lib = load()
    B, H, T, dk, dv, dev, dt = _train_inputs(q, k, v, g, beta, rule, gate)
    if s0 is not None:
        _check(s0, "s0", (B, H, dk, dv), torch.float32, dev)
    if out is None:
        out = torch.empty((B, H, T, dv), dtype=dt, device=dev)
    else:
        _check(out, "out", (B, H, T, dv), dt, dev)
    if s_final is None and return_state:
        s_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    elif s_final is not None:
        _check(s_final, "s_final", (B, H, dk, dv), torch.float32, dev)
    shape = chunk_states_shape(B, H, T, dk, dv, chunk)
    if states is None:
        states = torch.empty(shape, dtype=dt, device=dev)
    else:
        _check(states, "states", shape, dt, dev)
    a = chunk_args(B, H, T, dk, dv, rule=rule, gate=gate, dtype=_token_dtype(q), chunk=chunk)
    need = int(lib.linattn_chunk_workspace_bytes(ctypes.byref(a))) if gate == "channel" else 0
    if need > 0 and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    stream = torch.cuda.current_stream(dev).cuda_stream
    st = lib.linattn_chunk_fwd_save(ctypes.byref(a), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                    _ptr(s0), _ptr(out), _ptr(s_final), _ptr(states), _ptr(workspace),
                                    ws_bytes, stream)
    if st != 0:
        raise LinattnError(st, "linattn_chunk_fwd_save")
    return out, s_final, states


def chunk_bwd_workspace_bytes(B, H, T, dk, dv, *, rule, gate, dtype="bf16", states_given=False,
                              chunk=64) -> int:
    a = chunk_args(B, H, T, dk, dv, rule=rule, gate=gate, dtype=dtype, chunk=chunk)
    return int(load().linattn_chunk_bwd_workspace_bytes(ctypes.byref(a), int(bool(states_given))))


def chunk_bwd(q, k, v, g, beta, dout, s0=None, dsT=None, *, states=None, rule="delta", gate="scalar",
              chunk=64, workspace=None, grads=None):
    """Backward pass of chunk_fwd: gradients of a loss given dL/do (dout
    [B,H,T,dv], token dtype) and dL/dS_T (dsT [B,H,dk,dv] fp32 or None).
    states: the per-chunk states from chunk_fwd_save, or None to recompute
    them from q, k, v, g, beta and s0.  Returns a dict with dq, dk, dv, dg
    (None without a gate; [B,H,T,dk] for the per-channel gate), dbeta (None
    for the add rule) and ds0 (fp32).
    ``grads`` may supply preallocated outputs under the same names."""
    import torch
    lib = load()
    B, H, T, dk, dv, dev, dt = _train_inputs(q, k, v, g, beta, rule, gate)
    _check(dout, "dout", (B, H, T, dv), dt, dev)
    for t, name in ((s0, "s0"), (dsT, "dsT")):
        if t is not None:
            _check(t, name, (B, H, dk, dv), torch.float32, dev)
    if states is not None:
        _check(states, "states", chunk_states_shape(B, H, T, dk, dv, chunk), dt, dev)
    shapes = {"dq": ((B, H, T, dk), dt), "dk": ((B, H, T, dk), dt), "dv": ((B, H, T, dv), dt),
              "dg": {"scalar": ((B, H, T), dt), "channel": ((B, H, T, dk), dt)}.get(gate),
              "dbeta": ((B, H, T), dt) if rule == "delta" else None,
              "ds0": ((B, H, dk, dv), torch.float32)}
    out = dict(grads or {})
    for name, spec in shapes.items():
        if spec is None:
            out[name] = None
        elif out.get(name) is None:
            out[name] = torch.empty(spec[0], dtype=spec[1], device=dev)
        else:
            _check(out[name], name, spec[0], spec[1], dev)
    a = chunk_args(B, H, T, dk, dv, rule=rule, gate=gate, dtype=_token_dtype(q), chunk=chunk)
    need = int(lib.linattn_chunk_bwd_workspace_bytes(ctypes.byref(a), int(states is not None)))
    if need > 0 and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    stream = torch.cuda.current_stream(dev).cuda_stream
    st = lib.linattn_chunk_bwd(ctypes.byref(a), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(s0),
                               _ptr(states), _ptr(dout), _ptr(dsT), _ptr(out["dq"]), _ptr(out["dk"]),
                               _ptr(out["dv"]), _ptr(out["dg"]), _ptr(out["dbeta"]), _ptr(out["ds0"]),
                               _ptr(workspace), ws_bytes, stream)
    if st != 0:
        raise LinattnError(st, "linattn_chunk_bwd")
    return out


def deltaproduct_bwd_workspace_bytes(B, H, T, nh, dk, dv, *, gate="scalar", dtype="bf16", chunk=64) -> int:
    a = deltaproduct_args(B, H, T, nh, dk, dv, gate=gate, dtype=dtype, chunk=chunk)
    return int(load().linattn_deltaproduct_bwd_workspace_bytes(ctypes.byref(a)))


def deltaproduct_bwd(q, k, v, g, beta, dout, s0=None, dsT=None, *, gate="scalar", chunk=64, workspace=None,
                     grads=None):
    """Backward pass of deltaproduct_fwd on the GPU: gradients given dL/do
    (dout [B,H,T,dv]) and dL/dS_T (dsT [B,H,dk,dv] fp32 or None).  Returns a
    dict with dq [B,H,T,dk], dk [B,H,T,nh,dk], dv [B,H,T,nh,dv], dg [B,H,T] (None
    without a gate), dbeta [B,H,T,nh] and ds0 (fp32)."""
    import torch
    lib = load()
    B, H, T, dk = q.shape
    nh, dv = k.shape[3], v.shape[-1]
    dev, dt = q.device, q.dtype
    _check(q, "q", (B, H, T, dk), dt, dev)
    _check(k, "k", (B, H, T, nh, dk), dt, dev)
    _check(v, "v", (B, H, T, nh, dv), dt, dev)
    _check(beta, "beta", (B, H, T, nh), dt, dev)
    _check(dout, "dout", (B, H, T, dv), dt, dev)
    if gate == "scalar":
        _check(g, "g", (B, H, T), dt, dev)
    elif gate != "none" or g is not None:
        raise ValueError("Gated DeltaProduct takes gate='scalar' with g, or gate='none'")
    for t, name in ((s0, "s0"), (dsT, "dsT")):
        if t is not None:
            _check(t, name, (B, H, dk, dv), torch.float32, dev)
    shapes = {"dq": ((B, H, T, dk), dt), "dk": ((B, H, T, nh, dk), dt), "dv": ((B, H, T, nh, dv), dt),
              "dg": ((B, H, T), dt) if gate == "scalar" else None, "dbeta": ((B, H, T, nh), dt),
              "ds0": ((B, H, dk, dv), torch.float32)}
    out = dict(grads or {})
    for name, spec in shapes.items():
        if spec is None:
            out[name] = None
        elif out.get(name) is None:
            out[name] = torch.empty(spec[0], dtype=spec[1], device=dev)
        else:
            _check(out[name], name, spec[0], spec[1], dev)
    a = deltaproduct_args(B, H, T, nh, dk, dv, gate=gate, dtype=_token_dtype(q), chunk=chunk)
    need = int(lib.linattn_deltaproduct_bwd_workspace_bytes(ctypes.byref(a)))
    if need > 0 and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    stream = torch.cuda.current_stream(dev).cuda_stream
    st = lib.linattn_deltaproduct_bwd(ctypes.byref(a), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(s0),
                                      _ptr(dout), _ptr(dsT), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
                                      _ptr(out["dg"]), _ptr(out["dbeta"]), _ptr(out["ds0"]), _ptr(workspace),
                                      ws_bytes, stream)
    if st != 0:
        raise LinattnError(st, "linattn_deltaproduct_bwd")
    return out
