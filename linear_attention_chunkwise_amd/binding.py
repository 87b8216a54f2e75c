"""ctypes binding of libkda (include/kda.h): argument marshalling only.

Every step of the operator runs in the HIP kernels behind the C ABI; this module checks tensor
metadata, allocates outputs with torch (device memory is the caller's), passes raw device
pointers and the current HIP stream, and turns status codes into exceptions.  There is no
fallback: if libkda.so is missing or the GPU is absent, calls raise.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkda.so")

KDA_OK, KDA_ERR_INVALID_ARGUMENT, KDA_ERR_UNSUPPORTED, KDA_ERR_RANGE, KDA_ERR_HIP = range(5)
KDA_BF16, KDA_F32 = 0, 1

# every symbol include/kda.h declares
EXPORTS = ("kda_chunk_fwd", "kda_chunk_fwd_workspace_size", "kda_chunk_fwd_ckpt", "kda_chunk_fwd_gate", "kda_chunk_fwd_cp",
           "kda_chunk_fwd_cp_noalloc",
           "kda_chunk_fwd_cp_workspace_size", "kda_chunk_fwd_cp_segments", "kda_recurrent_step",
           "kda_recurrent_step_gate",
           "kda_recurrent_multi", "kda_recurrent_multi_fused", "kda_status_string",
           "kda_last_error", "kda_version")

_lib = None


class KdaError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(msg)
        self.status = status


def load(path: str = LIB_PATH):
    """Load libkda.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it first (python -m "
                           "linear_attention_chunkwise_amd.build)")
    lib = ctypes.CDLL(path)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.kda_chunk_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, i32,
                                  ctypes.c_int, ctypes.c_int, ctypes.c_float, vp, vp, vp,
                                  ctypes.c_size_t, vp]
    lib.kda_chunk_fwd.restype = ctypes.c_int
    lib.kda_chunk_fwd_workspace_size.argtypes = [i32, i64, i32, i32, i32, i32]
    lib.kda_chunk_fwd_workspace_size.restype = ctypes.c_size_t
    lib.kda_chunk_fwd_ckpt.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, i32,
                                       ctypes.c_int, ctypes.c_int, ctypes.c_float, vp, vp, i32, i32,
                                       vp, vp]
    lib.kda_chunk_fwd_ckpt.restype = ctypes.c_int
    lib.kda_chunk_fwd_cp.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, i32,
                                     ctypes.c_int, ctypes.c_int, ctypes.c_float, vp, vp, i32, vp,
                                     ctypes.c_size_t, vp]
    lib.kda_chunk_fwd_cp.restype = ctypes.c_int
    lib.kda_chunk_fwd_cp_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32,
                                             i32, ctypes.c_int, ctypes.c_int, ctypes.c_float, vp,
                                             vp, i32, vp]
    lib.kda_chunk_fwd_cp_noalloc.restype = ctypes.c_int
    lib.kda_chunk_fwd_cp_workspace_size.argtypes = [i32, i32, i32, i32, i32]
    lib.kda_chunk_fwd_cp_workspace_size.restype = ctypes.c_size_t
    lib.kda_chunk_fwd_cp_segments.argtypes = [i32, i32, i32, i32, i32]
    lib.kda_chunk_fwd_cp_segments.restype = i32
    lib.kda_recurrent_step.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_float, vp, vp]
    lib.kda_recurrent_step.restype = ctypes.c_int
    lib.kda_recurrent_multi.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_float, vp, vp]
    lib.kda_recurrent_multi.restype = ctypes.c_int
    lib.kda_chunk_fwd_gate.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32,
                                       i32, ctypes.c_int, ctypes.c_int, ctypes.c_float, vp, vp, vp,
                                       ctypes.c_size_t, vp]
    lib.kda_chunk_fwd_gate.restype = ctypes.c_int
    lib.kda_recurrent_step_gate.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                            ctypes.c_int, ctypes.c_int, ctypes.c_float, vp, vp]
    lib.kda_recurrent_step_gate.restype = ctypes.c_int
    lib.kda_recurrent_multi_fused.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp,
                                              i32, vp, vp, i32, i32, i32, i32, i32, ctypes.c_int,
                                              ctypes.c_int, ctypes.c_float, vp, vp]
    lib.kda_recurrent_multi_fused.restype = ctypes.c_int
    lib.kda_status_string.argtypes = [ctypes.c_int]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_last_error.argtypes = []
    lib.kda_last_error.restype = ctypes.c_char_p
    lib.kda_version.argtypes = []
    lib.kda_version.restype = ctypes.c_int32
    _lib = lib
    return lib


def _check(status):
    if status != KDA_OK:
        lib = load()
        raise KdaError(status, "%s: %s" % (lib.kda_status_string(status).decode(),
                                           lib.kda_last_error().decode()))


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float32:
        return KDA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _on(device, fn, *args):
    """Calls the library with the tensors' device current: it launches on the current HIP
    device, on the stream it is given (that device's current stream here)."""
    with torch.cuda.device(device):
        return fn(*args)


def _require(t, name, device, dtype=None, shape=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


class _Prefill:
    """The checks and output allocation every prefill entry point shares: q, k [B,T,H,dk],
    v [B,T,H,dv], beta [B,T,H] in q's dtype, the decay input (g float32, or the logits z in q's
    dtype with A_log [H] float32), S0, cu_seqlens, and o / S_T made here unless given."""

    def __init__(self, q, k, v, beta, S0, cu_seqlens, out_dtype, output_final_state, o, S_T,
                 g=None, z=None, A_log=None):
        self.dev = dev = q.device
        self.B, self.T, self.H, self.dk = B, T, H, dk = q.shape
        self.dv = dv = v.shape[-1]
        dt = q.dtype
        _require(q, "q", dev, dt)
        _require(k, "k", dev, dt, (B, T, H, dk))
        _require(v, "v", dev, dt, (B, T, H, dv))
        if z is None:
            _require(g, "g", dev, torch.float32, (B, T, H, dk))
        else:
            _require(z, "z", dev, dt, (B, T, H, dk))
            _require(A_log, "A_log", dev, torch.float32, (H,))
        _require(beta, "beta", dev, dt, (B, T, H))
        if cu_seqlens is not None:
            _require(cu_seqlens, "cu_seqlens", dev, torch.int32)
            self.N = N = cu_seqlens.numel() - 1
        else:
            self.N = N = B
        if S0 is not None:
            _require(S0, "S0", dev, torch.float32, (N, H, dk, dv))
        out_dtype = out_dtype or dt
        if o is None:
            o = torch.empty((B, T, H, dv), dtype=out_dtype, device=dev)
        else:
            _require(o, "o", dev, out_dtype, (B, T, H, dv))
        if S_T is None and output_final_state:
            S_T = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
        elif S_T is not None:
            _require(S_T, "S_T", dev, torch.float32, (N, H, dk, dv))
        self.o, self.S_T = o, S_T

    def sizes(self, q):
        """B, T, H, N, dk, dv, in_dtype, out_dtype as the C calls take them."""
        return (self.B, self.T, self.H, self.N, self.dk, self.dv, _dt(q), _dt(self.o))


def chunk_fwd_workspace_size(n_seq: int, total_tokens: int, H: int, dk: int, dv: int,
                             packed: bool, device=None) -> int:
    """Bytes of workspace kda_chunk_fwd needs to plan a split in time on ``device``."""
    dev = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
    return int(_on(dev, load().kda_chunk_fwd_workspace_size, int(n_seq), int(total_tokens), int(H),
                   int(dk), int(dv), int(bool(packed))))


def chunk_fwd(q, k, v, g, beta, S0=None, cu_seqlens=None, *, scale: float = 1.0,
              out_dtype=None, output_final_state: bool = True, o=None, S_T=None,
              workspace="auto"):
    """KDA chunkwise prefill: returns (o [B,T,H,dv], S_T [N,H,dk,dv] float32 or None).

    q, k [B,T,H,dk], v [B,T,H,dv], beta [B,T,H] share a dtype (bf16 or f32); g [B,T,H,dk]
    float32; S0 [N,H,dk,dv] float32 or None; cu_seqlens int32 [N+1] (device) with B = 1 for
    packed sequences.  ``S_T`` may be passed as S0 itself to advance the state in place.
    ``out_dtype`` defaults to q's dtype.  ``workspace``: "auto" allocates what the library asks
    for its automatic split in time (kda_chunk_fwd_workspace_size), None runs every sequence
    whole, or a uint8 device tensor."""
    lib = load()
    a = _Prefill(q, k, v, beta, S0, cu_seqlens, out_dtype, output_final_state, o, S_T, g=g)
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError("workspace must be 'auto', None or a uint8 tensor")
        need = chunk_fwd_workspace_size(a.N, a.B * a.T, a.H, a.dk, a.dv, cu_seqlens is not None,
                                        a.dev)
        workspace = torch.empty(need, dtype=torch.uint8, device=a.dev) if need else None
    if workspace is not None:
        _require(workspace, "workspace", a.dev, torch.uint8)
    nbytes = 0 if workspace is None else workspace.numel()
    st = _on(a.dev, lib.kda_chunk_fwd, _p(q), _p(k), _p(v), _p(g), _p(beta), _p(S0),
             _p(cu_seqlens), *a.sizes(q), float(scale), _p(a.o), _p(a.S_T), _p(workspace),
             nbytes, _stream(a.dev))
    _check(st)
    return a.o, a.S_T


def chunk_fwd_ckpt(q, k, v, g, beta, S0=None, cu_seqlens=None, *, interval: int, capacity: int,
                   scale: float = 1.0, out_dtype=None, output_final_state: bool = True, o=None,
                   S_T=None, ckpt=None):
    """chunk_fwd that also returns the prefix states after every ``interval`` tokens (a multiple
    of 32) of each sequence: ckpt [N,H,capacity,dk,dv] float32, slot j = state after
    (j+1)*interval tokens; slots past a sequence's last whole interval are left as allocated
    (zeros when ckpt is created here).  Returns (o, S_T, ckpt)."""
    lib = load()
    a = _Prefill(q, k, v, beta, S0, cu_seqlens, out_dtype, output_final_state, o, S_T, g=g)
    shape = (a.N, a.H, capacity, a.dk, a.dv)
    if ckpt is None:
        ckpt = torch.zeros(shape, dtype=torch.float32, device=a.dev)
    else:
        _require(ckpt, "ckpt", a.dev, torch.float32, shape)
    st = _on(a.dev, lib.kda_chunk_fwd_ckpt, _p(q), _p(k), _p(v), _p(g), _p(beta), _p(S0),
             _p(cu_seqlens), *a.sizes(q), float(scale), _p(a.o), _p(a.S_T), int(interval),
             int(capacity), _p(ckpt), _stream(a.dev))
    _check(st)
    return a.o, a.S_T, ckpt


def cp_segments(n_units: int, dk: int, dv: int, slots: int = 256) -> int:
    """The library's segment count for chunk_fwd_cp over ``n_units`` (sequence, head) units on a
    GPU with ``slots`` concurrent prefill workgroups (kda_chunk_fwd_cp_segments)."""
    return int(load().kda_chunk_fwd_cp_segments(int(n_units), 1, int(dk), int(dv), int(slots)))


def chunk_fwd_cp(q, k, v, g, beta, S0=None, cu_seqlens=None, *, segments: int, scale: float = 1.0,
                 out_dtype=None, output_final_state: bool = True, o=None, S_T=None, workspace=None):
    """chunk_fwd with each sequence split in time into ``segments`` pieces run in parallel
    (workspace allocated here unless given as a uint8 device tensor).  Returns (o, S_T)."""
    lib = load()
    a = _Prefill(q, k, v, beta, S0, cu_seqlens, out_dtype, output_final_state, o, S_T, g=g)
    need = lib.kda_chunk_fwd_cp_workspace_size(a.N, a.H, a.dk, a.dv, int(segments))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=a.dev)
    st = _on(a.dev, lib.kda_chunk_fwd_cp, _p(q), _p(k), _p(v), _p(g), _p(beta), _p(S0),
             _p(cu_seqlens), *a.sizes(q), float(scale), _p(a.o), _p(a.S_T), int(segments),
             _p(workspace), workspace.numel() * workspace.element_size(), _stream(a.dev))
    _check(st)
    return a.o, a.S_T


def recurrent_step(q, k, v, g, beta, S, *, scale: float = 1.0, out_dtype=None, o=None):
    """One KDA decode token per (sequence, head); S [N,H,dk,dv] float32 is updated IN PLACE.

    q, k [N,H,dk], v [N,H,dv], beta [N,H] share a dtype; g [N,H,dk] float32.  Returns o [N,H,dv]."""
    lib = load()
    dev = q.device
    N, H, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    _require(q, "q", dev, dt)
    _require(k, "k", dev, dt, (N, H, dk))
    _require(v, "v", dev, dt, (N, H, dv))
    _require(g, "g", dev, torch.float32, (N, H, dk))
    _require(beta, "beta", dev, dt, (N, H))
    _require(S, "S", dev, torch.float32, (N, H, dk, dv))
    out_dtype = out_dtype or dt
    if o is None:
        o = torch.empty((N, H, dv), dtype=out_dtype, device=dev)
    else:
        _require(o, "o", dev, out_dtype, (N, H, dv))
    st = _on(dev, lib.kda_recurrent_step, _p(q), _p(k), _p(v), _p(g), _p(beta), _p(S), N, H, dk, dv,
             _dt(q), _dt(o), float(scale), _p(o), _stream(dev))
    _check(st)
    return o


def recurrent_multi(q, k, v, g, beta, S, n_commit=None, *, scale: float = 1.0, out_dtype=None,
                    o=None, outputs: bool = True):
    """K decode tokens per (sequence, head) in one state pass; S [N,H,dk,dv] float32 is advanced
    IN PLACE by n_commit[n] tokens (int32 device tensor [N]; None: all K).  q, k [N,K,H,dk],
    v [N,K,H,dv], beta [N,K,H] share a dtype; g [N,K,H,dk] float32.  Returns o [N,K,H,dv]
    (None with outputs=False)."""
    lib = load()
    dev = q.device
    N, K, H, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    _require(q, "q", dev, dt)
    _require(k, "k", dev, dt, (N, K, H, dk))
    _require(v, "v", dev, dt, (N, K, H, dv))
    _require(g, "g", dev, torch.float32, (N, K, H, dk))
    _require(beta, "beta", dev, dt, (N, K, H))
    _require(S, "S", dev, torch.float32, (N, H, dk, dv))
    if n_commit is not None:
        _require(n_commit, "n_commit", dev, torch.int32, (N,))
    out_dtype = out_dtype or dt
    if outputs and o is None:
        o = torch.empty((N, K, H, dv), dtype=out_dtype, device=dev)
    elif o is not None:
        _require(o, "o", dev, out_dtype, (N, K, H, dv))
    st = _on(dev, lib.kda_recurrent_multi, _p(q), _p(k), _p(v), _p(g), _p(beta), _p(S),
             _p(n_commit), N, K, H, dk, dv, _dt(q), _dt(o) if o is not None else _dt(q),
             float(scale), _p(o), _stream(dev))
    _check(st)
    return o


def chunk_fwd_cp_noalloc(q, k, v, g, beta, S0=None, cu_seqlens=None, *, segments: int,
                         scale: float = 1.0, out_dtype=None, output_final_state: bool = True, o=None,
                         S_T=None):
    """chunk_fwd_cp with the segment summaries in the library's fixed per-device array instead of
    a workspace: the C call allocates nothing (o and S_T are made here unless given).  Calls
    that overlap in time on one device race on that array.  Returns (o, S_T)."""
    lib = load()
    a = _Prefill(q, k, v, beta, S0, cu_seqlens, out_dtype, output_final_state, o, S_T, g=g)
    st = _on(a.dev, lib.kda_chunk_fwd_cp_noalloc, _p(q), _p(k), _p(v), _p(g), _p(beta), _p(S0),
             _p(cu_seqlens), *a.sizes(q), float(scale), _p(a.o), _p(a.S_T), int(segments),
             _stream(a.dev))
    _check(st)
    return a.o, a.S_T


def chunk_fwd_gate(q, k, v, z, A_log, beta, S0=None, cu_seqlens=None, *, scale: float = 1.0,
                   out_dtype=None, output_final_state: bool = True, o=None, S_T=None,
                   workspace="auto"):
    """chunk_fwd with the decay map in the kernel: g = -5 Sigmoid(exp(A_log[h]) z) is formed from
    the logits z [B,T,H,dk] (q's dtype) and A_log [H] float32 instead of being read.  workspace as
    for chunk_fwd (its split in time when that pays)."""
    lib = load()
    a = _Prefill(q, k, v, beta, S0, cu_seqlens, out_dtype, output_final_state, o, S_T, z=z,
                 A_log=A_log)
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError("workspace must be 'auto', None or a uint8 tensor")
        need = chunk_fwd_workspace_size(a.N, a.B * a.T, a.H, a.dk, a.dv, cu_seqlens is not None,
                                        a.dev)
        workspace = torch.empty(need, dtype=torch.uint8, device=a.dev) if need else None
    if workspace is not None:
        _require(workspace, "workspace", a.dev, torch.uint8)
    nbytes = 0 if workspace is None else workspace.numel()
    st = _on(a.dev, lib.kda_chunk_fwd_gate, _p(q), _p(k), _p(v), _p(z), _p(A_log), _p(beta),
             _p(S0), _p(cu_seqlens), *a.sizes(q), float(scale), _p(a.o), _p(a.S_T),
             _p(workspace), nbytes, _stream(a.dev))
    _check(st)
    return a.o, a.S_T


def recurrent_step_gate(q, k, v, z, A_log, beta, S, *, scale: float = 1.0, out_dtype=None, o=None):
    """recurrent_step with the decay formed from the logits z [N,H,dk] (q's dtype) and A_log [H]."""
    lib = load()
    dev = q.device
    N, H, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    _require(q, "q", dev, dt)
    _require(k, "k", dev, dt, (N, H, dk))
    _require(v, "v", dev, dt, (N, H, dv))
    _require(z, "z", dev, dt, (N, H, dk))
    _require(A_log, "A_log", dev, torch.float32, (H,))
    _require(beta, "beta", dev, dt, (N, H))
    _require(S, "S", dev, torch.float32, (N, H, dk, dv))
    out_dtype = out_dtype or dt
    if o is None:
        o = torch.empty((N, H, dv), dtype=out_dtype, device=dev)
    else:
        _require(o, "o", dev, out_dtype, (N, H, dv))
    st = _on(dev, lib.kda_recurrent_step_gate, _p(q), _p(k), _p(v), _p(z), _p(A_log), _p(beta),
             _p(S), N, H, dk, dv, _dt(q), _dt(o), float(scale), _p(o), _stream(dev))
    _check(st)
    return o


def recurrent_multi_fused(q, k, v, z, A_log, beta_logit, G, S, n_commit=None, *, norm_weight=None,
                          eps: float = 1e-6, scale: float = 1.0, out_dtype=None, y=None,
                          outputs: bool = True, conv_weight=None, conv_state=None):
    """recurrent_multi with the steps around the operator fused in: optionally the short
    convolution and Swish on q, k, v (conv_weight [H, 2dk+dv, W] float32, conv_state
    [N, H, 2dk+dv, W-1] in the input dtype, oldest first, advanced in place to the committed
    token), then q, k L2-normalised, beta = Sigmoid(beta_logit), g from the logits z and A_log,
    and outputs y = Sigmoid(G) * RMSNorm(o~) (weight norm_weight [dv] float32 or None, eps).
    q, k, z [N,K,H,dk], v, G [N,K,H,dv], beta_logit [N,K,H] share a dtype; S advanced in place
    as in recurrent_multi.  Returns y [N,K,H,dv] (None with outputs=False)."""
    lib = load()
    dev = q.device
    N, K, H, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    _require(q, "q", dev, dt)
    _require(k, "k", dev, dt, (N, K, H, dk))
    _require(v, "v", dev, dt, (N, K, H, dv))
    _require(z, "z", dev, dt, (N, K, H, dk))
    _require(A_log, "A_log", dev, torch.float32, (H,))
    _require(beta_logit, "beta_logit", dev, dt, (N, K, H))
    _require(S, "S", dev, torch.float32, (N, H, dk, dv))
    if n_commit is not None:
        _require(n_commit, "n_commit", dev, torch.int32, (N,))
    if norm_weight is not None:
        _require(norm_weight, "norm_weight", dev, torch.float32, (dv,))
    width = 1
    if conv_weight is not None:
        width = conv_weight.shape[-1]
        _require(conv_weight, "conv_weight", dev, torch.float32, (H, 2 * dk + dv, width))
        if width > 1:
            _require(conv_state, "conv_state", dev, dt, (N, H, 2 * dk + dv, width - 1))
    out_dtype = out_dtype or dt
    if outputs:
        _require(G, "G", dev, dt, (N, K, H, dv))
        if y is None:
            y = torch.empty((N, K, H, dv), dtype=out_dtype, device=dev)
        else:
            _require(y, "y", dev, out_dtype, (N, K, H, dv))
    else:
        y = None
    st = _on(dev, lib.kda_recurrent_multi_fused, _p(q), _p(k), _p(v), _p(z), _p(A_log),
             _p(beta_logit), _p(G) if outputs else None, _p(norm_weight), float(eps),
             _p(conv_weight), _p(conv_state) if width > 1 else None, width, _p(S),
             _p(n_commit), N, K, H, dk, dv, _dt(q), _dt(y) if y is not None else _dt(q),
             float(scale), _p(y), _stream(dev))
    _check(st)
    return y
