"""Thin ctypes binding of libgdn.so (include/gdn.h).

Argument marshalling only: every step of the layer runs in the HIP kernels of
libgdn.so.  Tensors are torch device tensors (PyTorch supplies device memory
and streams); a missing library raises instead of falling back to anything.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgdn.so")

GDN_OK = 0
GDN_F32, GDN_BF16 = 0, 1
GDN_FLAG_L2NORM_QK = 0x1
GDN_FLAG_SEPARATE_LAUNCHES = 0x2
GDN_FLAG_PREP_WRITE_BACK = 0x4
GDN_FLAG_TEST_WAITS_GIVE_UP = 0x8
GDN_FLAG_SEGMENTS = 0x10
GDN_FLAG_PIPELINED = 0x20
PREFILL_MAX_KERNELS = 64   # kernels a profiled call may record (the caller's choice)
STAGE_NAMES = {0: "chunk_table", 1: "chunk_prep", 2: "state_sweep", 3: "gated_norm",
               4: "conv_state", 5: "prep_sweep", 6: "seg_compose", 7: "seg_fixup"}

STATUS_NAMES = {0: "GDN_OK", 1: "GDN_ERR_NULL_ARG", 2: "GDN_ERR_BAD_SHAPE",
                3: "GDN_ERR_UNSUPPORTED", 4: "GDN_ERR_BAD_DTYPE", 5: "GDN_ERR_MISALIGNED",
                6: "GDN_ERR_WORKSPACE", 7: "GDN_ERR_HIP", 8: "GDN_ERR_ALIAS",
                9: "GDN_ERR_BAD_VALUE"}

EXPORTED = ["gdn_status_string", "gdn_prefill_workspace_size", "gdn_prefill",
            "gdn_prefill_profiled", "gdn_prefill_ex", "gdn_decode", "gdn_decode_verify",
            "gdn_decode_commit", "gdn_prefill_wait_status", "gdn_prefill_static"]
STATIC_SCRATCH_BYTES = 128 << 20   # GDN_STATIC_SCRATCH_BYTES


class GdnError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {gdn_status_string(code)}")
        self.code = code


class Desc(ctypes.Structure):
    """gdn_desc."""
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("total_tokens", ctypes.c_int64),
        ("num_k_heads", ctypes.c_int32),
        ("num_v_heads", ctypes.c_int32),
        ("head_k_dim", ctypes.c_int32),
        ("head_v_dim", ctypes.c_int32),
        ("conv_kernel", ctypes.c_int32),
        ("io_dtype", ctypes.c_int32),
        ("state_dtype", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("l2_eps", ctypes.c_float),
        ("norm_eps", ctypes.c_float),
        ("flags", ctypes.c_uint32),
    ]


class PrefillArgs(ctypes.Structure):
    """gdn_prefill_args (pointers as integers, NULL as None)."""
    _fields_ = [
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("g", ctypes.c_void_p), ("beta", ctypes.c_void_p),
        ("z", ctypes.c_void_p), ("conv_w", ctypes.c_void_p), ("norm_w", ctypes.c_void_p),
        ("cu_seqlens", ctypes.c_void_p),
        ("initial_state", ctypes.c_void_p), ("final_state", ctypes.c_void_p),
        ("conv_state_in", ctypes.c_void_p), ("conv_state_out", ctypes.c_void_p),
        ("state_slots", ctypes.c_void_p), ("num_state_slots", ctypes.c_int32),
        ("state_snapshots", ctypes.c_void_p), ("snapshot_base", ctypes.c_void_p),
        ("snapshot_every", ctypes.c_int32), ("num_snapshot_slots", ctypes.c_int32),
        ("out", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
    ]


def make_desc(num_seqs: int, total_tokens: int, num_k_heads: int = 16, num_v_heads: int = 32,
              io_dtype: int = GDN_BF16, state_dtype: int = GDN_F32, scale: float = 1.0,
              l2_eps: float = 1e-6, norm_eps: float = 1e-6, l2norm: bool = True,
              head_dim: int = 128, conv_kernel: int = 4, separate_launches: bool = False,
              prep_write_back: bool = False, segments: bool = False, pipelined: bool = False,
              flags: int = 0) -> Desc:
    f = (GDN_FLAG_L2NORM_QK if l2norm else 0) | (GDN_FLAG_SEPARATE_LAUNCHES if separate_launches else 0) \
        | (GDN_FLAG_PREP_WRITE_BACK if prep_write_back else 0) | (GDN_FLAG_SEGMENTS if segments else 0) \
        | (GDN_FLAG_PIPELINED if pipelined else 0) | int(flags)
    return Desc(num_seqs=num_seqs, total_tokens=total_tokens, num_k_heads=num_k_heads,
                num_v_heads=num_v_heads, head_k_dim=head_dim, head_v_dim=head_dim,
                conv_kernel=conv_kernel, io_dtype=io_dtype, state_dtype=state_dtype,
                scale=scale, l2_eps=l2_eps, norm_eps=norm_eps, flags=f)


_lib = None


def lib():
    """Load libgdn.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "gated_deltanet_layer_02_amd.build.build()")
        l = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        dp = ctypes.POINTER(Desc)
        l.gdn_status_string.restype = ctypes.c_char_p
        l.gdn_status_string.argtypes = [ctypes.c_int]
        l.gdn_prefill_workspace_size.restype = ctypes.c_int
        l.gdn_prefill_workspace_size.argtypes = [dp, ctypes.POINTER(sz)]
        l.gdn_prefill.restype = ctypes.c_int
        l.gdn_prefill.argtypes = [dp] + [vp] * 14 + [vp, sz, vp]
        l.gdn_prefill_profiled.restype = ctypes.c_int
        l.gdn_prefill_profiled.argtypes = [dp] + [vp] * 14 + [vp, sz, vp, vp, i32, vp, vp]
        l.gdn_prefill_ex.restype = ctypes.c_int
        l.gdn_prefill_ex.argtypes = [dp, ctypes.POINTER(PrefillArgs), vp]
        l.gdn_prefill_static.restype = ctypes.c_int
        l.gdn_prefill_static.argtypes = [dp, ctypes.POINTER(PrefillArgs), vp]
        l.gdn_decode_verify.restype = ctypes.c_int
        l.gdn_decode_verify.argtypes = [dp, i32] + [vp] * 11 + [i32, vp, vp, vp, vp]
        l.gdn_decode_commit.restype = ctypes.c_int
        l.gdn_decode_commit.argtypes = [dp, i32] + [vp] * 6 + [i32, vp]
        l.gdn_decode.restype = ctypes.c_int
        l.gdn_decode.argtypes = [dp] + [vp] * 11 + [i32, vp, vp]
        l.gdn_prefill_wait_status.restype = ctypes.c_int
        l.gdn_prefill_wait_status.argtypes = [vp, sz, vp, ctypes.POINTER(i32)]
        _lib = l
    return _lib


def gdn_status_string(code: int) -> str:
    try:
        return lib().gdn_status_string(int(code)).decode()
    except RuntimeError:
        return STATUS_NAMES.get(int(code), f"status {code}")


def gdn_prefill_wait_status(workspace, stream=None) -> int:
    """1 if a wait of the last prefill call on `workspace` gave up (its outputs
    are invalid), else 0.  Synchronises `stream`."""
    f = ctypes.c_int32(-1)
    rc = lib().gdn_prefill_wait_status(_ws_ptr(workspace), _ws_bytes(workspace), _stream(stream),
                                       ctypes.byref(f))
    if rc != GDN_OK:
        raise GdnError(rc, "gdn_prefill_wait_status")
    return int(f.value)


def gdn_prefill_workspace_size(desc: Desc) -> int:
    n = ctypes.c_size_t(0)
    rc = lib().gdn_prefill_workspace_size(ctypes.byref(desc), ctypes.byref(n))
    if rc != GDN_OK:
        raise GdnError(rc, "gdn_prefill_workspace_size")
    return int(n.value)


def _p(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ws_bytes(workspace) -> int:
    if workspace is None:
        return 0
    if isinstance(workspace, tuple):      # (pointer, bytes)
        return int(workspace[1])
    return workspace.numel() * workspace.element_size()


def _ws_ptr(workspace):
    if isinstance(workspace, tuple):
        return workspace[0]
    return _p(workspace)


def gdn_prefill(desc: Desc, q, k, v, g, beta, *, z=None, conv_w=None, norm_w=None,
                cu_seqlens=None, initial_state=None, conv_state_in=None, out=None,
                final_state=None, conv_state_out=None, workspace=None, stream=None,
                check: bool = True) -> int:
    rc = lib().gdn_prefill(ctypes.byref(desc), _p(q), _p(k), _p(v), _p(g), _p(beta), _p(z),
                           _p(conv_w), _p(norm_w), _p(cu_seqlens), _p(initial_state),
                           _p(conv_state_in), _p(out), _p(final_state), _p(conv_state_out),
                           _ws_ptr(workspace), _ws_bytes(workspace), _stream(stream))
    if check and rc != GDN_OK:
        raise GdnError(rc, "gdn_prefill")
    return rc


def gdn_prefill_ex(desc: Desc, q, k, v, g, beta, *, z=None, conv_w=None, norm_w=None,
                   cu_seqlens=None, initial_state=None, final_state=None, conv_state_in=None,
                   conv_state_out=None, state_slots=None, num_state_slots: int = 0,
                   state_snapshots=None, snapshot_base=None, snapshot_every: int = 0,
                   num_snapshot_slots: int = 0, out=None, workspace=None, stream=None,
                   check: bool = True) -> int:
    a = PrefillArgs(q=_p(q), k=_p(k), v=_p(v), g=_p(g), beta=_p(beta), z=_p(z),
                    conv_w=_p(conv_w), norm_w=_p(norm_w), cu_seqlens=_p(cu_seqlens),
                    initial_state=_p(initial_state), final_state=_p(final_state),
                    conv_state_in=_p(conv_state_in), conv_state_out=_p(conv_state_out),
                    state_slots=_p(state_slots), num_state_slots=int(num_state_slots),
                    state_snapshots=_p(state_snapshots), snapshot_base=_p(snapshot_base),
                    snapshot_every=int(snapshot_every), num_snapshot_slots=int(num_snapshot_slots),
                    out=_p(out), workspace=_ws_ptr(workspace), workspace_bytes=_ws_bytes(workspace))
    rc = lib().gdn_prefill_ex(ctypes.byref(desc), ctypes.byref(a), _stream(stream))
    if check and rc != GDN_OK:
        raise GdnError(rc, "gdn_prefill_ex")
    return rc


def gdn_prefill_static(desc: Desc, q, k, v, g, beta, *, z=None, conv_w=None, norm_w=None,
                       cu_seqlens=None, initial_state=None, final_state=None, conv_state_in=None,
                       conv_state_out=None, state_slots=None, num_state_slots: int = 0,
                       state_snapshots=None, snapshot_base=None, snapshot_every: int = 0,
                       num_snapshot_slots: int = 0, out=None, stream=None, check: bool = True) -> int:
    """gdn_prefill_static: gdn_prefill_ex's arguments without a workspace."""
    a = PrefillArgs(q=_p(q), k=_p(k), v=_p(v), g=_p(g), beta=_p(beta), z=_p(z),
                    conv_w=_p(conv_w), norm_w=_p(norm_w), cu_seqlens=_p(cu_seqlens),
                    initial_state=_p(initial_state), final_state=_p(final_state),
                    conv_state_in=_p(conv_state_in), conv_state_out=_p(conv_state_out),
                    state_slots=_p(state_slots), num_state_slots=int(num_state_slots),
                    state_snapshots=_p(state_snapshots), snapshot_base=_p(snapshot_base),
                    snapshot_every=int(snapshot_every), num_snapshot_slots=int(num_snapshot_slots),
                    out=_p(out), workspace=None, workspace_bytes=0)
    rc = lib().gdn_prefill_static(ctypes.byref(desc), ctypes.byref(a), _stream(stream))
    if check and rc != GDN_OK:
        raise GdnError(rc, "gdn_prefill_static")
    return rc


def gdn_prefill_profiled(desc: Desc, q, k, v, g, beta, *, events: Sequence[int], z=None,
                         conv_w=None, norm_w=None, cu_seqlens=None, initial_state=None,
                         conv_state_in=None, out=None, final_state=None, conv_state_out=None,
                         workspace=None, stream=None):
    """events: 2 + 2 m event handles.  Returns the stage id of every kernel i,
    which ran between events[2 + 2 i] and events[3 + 2 i]; events[0] and
    events[1] bracket the whole call on `stream`."""
    m = (len(events) - 2) // 2
    if m < 1:
        raise ValueError("need 2 + 2 m events, m >= 1")
    ev = (ctypes.c_void_p * len(events))(*events)
    ns = ctypes.c_int32(0)
    ids = (ctypes.c_int32 * m)()
    rc = lib().gdn_prefill_profiled(ctypes.byref(desc), _p(q), _p(k), _p(v), _p(g), _p(beta),
                                    _p(z), _p(conv_w), _p(norm_w), _p(cu_seqlens),
                                    _p(initial_state), _p(conv_state_in), _p(out),
                                    _p(final_state), _p(conv_state_out), _ws_ptr(workspace),
                                    _ws_bytes(workspace), _stream(stream), ev, m,
                                    ctypes.byref(ns), ids)
    if rc != GDN_OK:
        raise GdnError(rc, "gdn_prefill_profiled")
    return [int(ids[i]) for i in range(ns.value)]


def gdn_decode(desc: Desc, q, k, v, g, beta, *, state, out, z=None, conv_w=None, norm_w=None,
               conv_state=None, state_slots=None, num_state_slots: Optional[int] = None,
               stream=None, check: bool = True) -> int:
    if num_state_slots is None:
        num_state_slots = desc.num_seqs
    rc = lib().gdn_decode(ctypes.byref(desc), _p(q), _p(k), _p(v), _p(g), _p(beta), _p(z),
                          _p(conv_w), _p(norm_w), _p(state), _p(conv_state), _p(state_slots),
                          int(num_state_slots), _p(out), _stream(stream))
    if check and rc != GDN_OK:
        raise GdnError(rc, "gdn_decode")
    return rc


def gdn_decode_verify(desc: Desc, num_draft: int, q, k, v, g, beta, *, state, state_ckpt, out,
                      z=None, conv_w=None, norm_w=None, conv_state=None, conv_ckpt=None,
                      state_slots=None, num_state_slots: Optional[int] = None, stream=None,
                      check: bool = True) -> int:
    if num_state_slots is None:
        num_state_slots = desc.num_seqs
    rc = lib().gdn_decode_verify(ctypes.byref(desc), int(num_draft), _p(q), _p(k), _p(v), _p(g),
                                 _p(beta), _p(z), _p(conv_w), _p(norm_w), _p(state),
                                 _p(conv_state), _p(state_slots), int(num_state_slots),
                                 _p(state_ckpt), _p(conv_ckpt), _p(out), _stream(stream))
    if check and rc != GDN_OK:
        raise GdnError(rc, "gdn_decode_verify")
    return rc


def gdn_decode_commit(desc: Desc, num_draft: int, *, state_ckpt, accepted, state, conv_ckpt=None,
                      conv_state=None, state_slots=None, num_state_slots: Optional[int] = None,
                      stream=None, check: bool = True) -> int:
    if num_state_slots is None:
        num_state_slots = desc.num_seqs
    rc = lib().gdn_decode_commit(ctypes.byref(desc), int(num_draft), _p(state_ckpt), _p(conv_ckpt),
                                 _p(accepted), _p(state), _p(conv_state), _p(state_slots),
                                 int(num_state_slots), _stream(stream))
    if check and rc != GDN_OK:
        raise GdnError(rc, "gdn_decode_commit")
    return rc
