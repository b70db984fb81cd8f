"""ctypes front end of the fp64 CPU oracle (oracle/gdn_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
CPU-baseline leg of the benchmark.  Nothing on the product path imports it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "libgdn_oracle.so")
# The mutation test points this at a deliberately broken build of the oracle.
_LIB_OVERRIDE = os.environ.get("GDN_ORACLE_LIB_OVERRIDE")

F32, BF16, F64 = 0, 1, 2
_DT = {"f32": F32, "bf16": BF16, "f64": F64}


class _Desc(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("total_tokens", ctypes.c_int64),
        ("num_k_heads", ctypes.c_int32),
        ("num_v_heads", ctypes.c_int32),
        ("head_k_dim", ctypes.c_int32),
        ("head_v_dim", ctypes.c_int32),
        ("conv_kernel", ctypes.c_int32),
        ("io_dtype", ctypes.c_int32),
        ("gate_dtype", ctypes.c_int32),
        ("state_dtype", ctypes.c_int32),
        ("use_l2", ctypes.c_int32),
        ("scale", ctypes.c_double),
        ("l2_eps", ctypes.c_double),
        ("norm_eps", ctypes.c_double),
        ("head_begin", ctypes.c_int32),
        ("head_end", ctypes.c_int32),
        ("num_threads", ctypes.c_int32),
    ]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain C, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O3", "-march=x86-64-v3", "-fopenmp", "-fPIC", "-shared",
               "-std=c11", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            l = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(_LIB):
                build()
            l = ctypes.CDLL(_LIB)
        vp = ctypes.c_void_p
        l.gdn_oracle_prefill.restype = ctypes.c_int
        l.gdn_oracle_prefill.argtypes = [ctypes.POINTER(_Desc)] + [vp] * 14
        l.gdn_oracle_conv_silu.restype = ctypes.c_int
        l.gdn_oracle_conv_silu.argtypes = [ctypes.POINTER(_Desc)] + [vp] * 7
        l.gdn_oracle_max_threads.restype = ctypes.c_int
        _lib = l
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _io_dtype_of(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.float64:
        return F64
    raise TypeError(f"unsupported dtype {a.dtype}")


def _c(a):
    return None if a is None else np.ascontiguousarray(a)


def prefill(q, k, v, g, beta, *, cu_seqlens=None, z=None, conv_w=None, norm_w=None,
            initial_state=None, conv_state_in=None, use_l2=True, scale=1.0,
            l2_eps=1e-6, norm_eps=1e-6, conv_kernel=4, heads: Optional[Tuple[int, int]] = None,
            want_conv_state=True, threads: int = 0):
    """Run the oracle.

    q, k: [T, Hk, dk]; v (and z): [T, Hv, dv] in one io dtype (uint16 = bf16 bits,
    float32 or float64); g, beta: [T, Hv] float32 or float64;
    initial_state [N, Hv, dv, dk] (uint16 bf16 bits, float32 or float64).
    Returns (out [T, nh, dv] f64, final_state [N, nh, dv, dk] f64,
    conv_state_out [N, K-1, Cch] io dtype or None), nh = heads[1] - heads[0].
    """
    q, k, v, g, beta = map(_c, (q, k, v, g, beta))
    z, conv_w, norm_w, initial_state, conv_state_in = map(
        _c, (z, conv_w, norm_w, initial_state, conv_state_in))
    T, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    if cu_seqlens is None:
        cu_seqlens = np.array([0, T], dtype=np.int32)
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    N = cu.shape[0] - 1
    h0, h1 = heads if heads is not None else (0, Hv)
    io = _io_dtype_of(q)
    d = _Desc(num_seqs=N, total_tokens=T, num_k_heads=Hk, num_v_heads=Hv, head_k_dim=dk,
              head_v_dim=dv, conv_kernel=conv_kernel, io_dtype=io,
              gate_dtype=F64 if g.dtype == np.float64 else F32,
              state_dtype=_io_dtype_of(initial_state) if initial_state is not None else F32,
              use_l2=1 if use_l2 else 0, scale=scale, l2_eps=l2_eps, norm_eps=norm_eps,
              head_begin=h0, head_end=h1, num_threads=threads)
    if g.dtype != beta.dtype:
        raise TypeError("g and beta must share a dtype")
    nh = h1 - h0
    out = np.empty((T, nh, dv), dtype=np.float64)
    fs = np.empty((N, nh, dv, dk), dtype=np.float64)
    Cch = 2 * Hk * dk + Hv * dv
    cso = None
    if want_conv_state and conv_kernel > 1:
        cso = np.empty((N, conv_kernel - 1, Cch), dtype=q.dtype)
    rc = lib().gdn_oracle_prefill(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                  _ptr(beta), _ptr(z), _ptr(conv_w), _ptr(norm_w), _ptr(cu),
                                  _ptr(initial_state), _ptr(conv_state_in), _ptr(out),
                                  _ptr(fs), _ptr(cso))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return out, fs, cso


def conv_silu(q, k, v, conv_w, *, cu_seqlens=None, conv_state_in=None, conv_kernel=4):
    """The oracle's conv + SiLU step for every channel: [T, Cch] float64."""
    q, k, v, conv_w, conv_state_in = map(_c, (q, k, v, conv_w, conv_state_in))
    T, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    if cu_seqlens is None:
        cu_seqlens = np.array([0, T], dtype=np.int32)
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    N = cu.shape[0] - 1
    d = _Desc(num_seqs=N, total_tokens=T, num_k_heads=Hk, num_v_heads=Hv, head_k_dim=dk,
              head_v_dim=dv, conv_kernel=conv_kernel, io_dtype=_io_dtype_of(q), gate_dtype=F32,
              state_dtype=F32, use_l2=0, scale=1.0, l2_eps=0.0, norm_eps=0.0, head_begin=0,
              head_end=Hv, num_threads=0)
    y = np.empty((T, 2 * Hk * dk + Hv * dv), dtype=np.float64)
    rc = lib().gdn_oracle_conv_silu(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(conv_w),
                                    _ptr(cu), _ptr(conv_state_in), _ptr(y))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return y


def max_threads() -> int:
    return int(lib().gdn_oracle_max_threads())


def run_problem(p, inputs: dict, heads=None, threads: int = 0):
    """Oracle on a gdn_synth.Problem and its generated inputs."""
    return prefill(inputs["q"], inputs["k"], inputs["v"], inputs["g"], inputs["beta"],
                   cu_seqlens=inputs["cu_seqlens"], z=inputs["z"], conv_w=inputs["conv_w"],
                   norm_w=inputs["norm_w"], initial_state=inputs["state"],
                   conv_state_in=inputs["conv_state"], use_l2=p.l2norm, scale=p.scale,
                   l2_eps=p.l2_eps, norm_eps=p.norm_eps, conv_kernel=p.K, heads=heads,
                   threads=threads)
