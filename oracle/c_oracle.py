"""ctypes wrapper of the C reference token loop -- TEST INFRASTRUCTURE ONLY.

Builds ``oracle/libkda_oracle.so`` from ``oracle/kda_oracle.c`` with gcc (plain -O3, no fast-math; OpenMP
over independent (sequence, head) units) and evaluates the definition of eq. (1) of Kimi K3:
Open Frontier Intelligence, §2.1.1 on chosen units.  Inputs are CPU torch tensors in their
stored dtype (bfloat16 or float32), so nothing is widened to float64 in memory; results are
float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle (always when force, else only if the library is missing or older
    than its source)."""
    stale = not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)
    if force or stale:
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", "-std=c99", _SRC,
                        "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build(force=False)
        lib = ctypes.CDLL(_LIB)
        vp, i32, i64, f64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        lib.kda_oracle_units.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, i64,
                                         i32, i32, i32, f64, i32, vp, vp, vp, vp]
        lib.kda_oracle_units.restype = None
        lib.kda_oracle_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def threads() -> int:
    """OpenMP threads the C oracle uses."""
    return int(_load().kda_oracle_threads())


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return 0
    if t.dtype == torch.float32:
        return 1
    if t.dtype == torch.float64:
        return 2
    raise TypeError("stored dtype must be bfloat16 or float32, got %s" % t.dtype)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def kda_units(q, k, v, g, beta, S0=None, cu_seqlens=None, units=None, scale=1.0):
    """Evaluate eq. (1) on selected (sequence, head) units.

    Tensors are CPU torch tensors: q, k [B, T, H, dk], v [B, T, H, dv] (bf16 or f32),
    g [B, T, H, dk] f32 or f64 (torch or numpy), beta [B, T, H], S0 [N, H, dk, dv] f32 or None, cu_seqlens [N+1] or None.
    ``units``: list of (n, h); default all.
    Returns (list of o arrays [len_n, dv] float64 per unit, S_T array [n_units, dk, dv])."""
    lib = _load()
    if isinstance(g, np.ndarray):
        g = torch.from_numpy(g)
    q, k, v, g, beta = (t.detach().cpu().contiguous() for t in (q, k, v, g, beta))
    if q.dtype != k.dtype or q.dtype != v.dtype:
        raise TypeError("q, k, v must share a dtype")
    if g.dtype not in (torch.float32, torch.float64):
        raise TypeError("g must be float32 or float64")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if cu_seqlens is None:
        bounds = [(b, 0, T) for b in range(B)]
    else:
        cu = [int(c) for c in torch.as_tensor(cu_seqlens).reshape(-1).tolist()]
        bounds = [(0, cu[n], cu[n + 1]) for n in range(len(cu) - 1)]
    N = len(bounds)
    if units is None:
        units = [(n, h) for n in range(N) for h in range(H)]
    desc = np.zeros((len(units), 5), np.int64)
    off = 0
    for i, (n, h) in enumerate(units):
        b, bos, eos = bounds[n]
        desc[i] = (b, bos, eos, h, off)
        off += eos - bos
    S0u = np.zeros((len(units), dk, dv), np.float64)
    if S0 is not None:
        S0c = S0.detach().cpu().double().numpy()
        for i, (n, h) in enumerate(units):
            S0u[i] = S0c[n, h]
    o = np.zeros((max(off, 1), dv), np.float64)
    ST = np.zeros((len(units), dk, dv), np.float64)
    lib.kda_oracle_units(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _dtype_code(q),
                         _dtype_code(beta), _dtype_code(g), T, H, dk, dv, float(scale), len(units),
                         desc.ctypes.data_as(ctypes.c_void_p),
                         S0u.ctypes.data_as(ctypes.c_void_p), o.ctypes.data_as(ctypes.c_void_p),
                         ST.ctypes.data_as(ctypes.c_void_p))
    outs = [o[desc[i, 4]: desc[i, 4] + (desc[i, 2] - desc[i, 1])] for i in range(len(units))]
    return outs, ST


def kda_forward(q, k, v, g, beta, S0=None, cu_seqlens=None, scale=1.0):
    """All units, assembled like oracle.kda_oracle.kda_forward: (o [B,T,H,dv], S_T [N,H,dk,dv])."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    N = B if cu_seqlens is None else len(cu_seqlens) - 1
    units = [(n, h) for n in range(N) for h in range(H)]
    outs, ST = kda_units(q, k, v, g, beta, S0, cu_seqlens, units, scale)
    o = np.zeros((B, T, H, dv))
    if cu_seqlens is None:
        bounds = [(b, 0, T) for b in range(B)]
    else:
        cu = [int(c) for c in torch.as_tensor(cu_seqlens).reshape(-1).tolist()]
        bounds = [(0, cu[n], cu[n + 1]) for n in range(N)]
    for i, (n, h) in enumerate(units):
        b, bos, eos = bounds[n]
        o[b, bos:eos, h] = outs[i]
    return o, ST.reshape(N, H, dk, dv)
