"""Device buffers for one layer call, allocated with torch and passed to
libgdn.so through the binding.  Host arrays use the io conventions of the
library: bf16 as uint16 bit patterns, fp32 as float32, indices as int32.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from . import binding as B


def to_device(a: Optional[np.ndarray], device="cuda"):
    import torch
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    if a.dtype in (np.float32, np.int32):
        return torch.from_numpy(a).to(device)
    raise TypeError(f"unsupported host dtype {a.dtype}")


def to_host(t) -> np.ndarray:
    """Device tensor -> numpy, bf16 as uint16 bit patterns."""
    import torch
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def empty_like_io(shape, io_bf16: bool, device="cuda"):
    import torch
    return torch.empty(shape, dtype=torch.bfloat16 if io_bf16 else torch.float32, device=device)


class PrefillCall:
    """All device buffers of one gdn_prefill call built from host arrays."""

    def __init__(self, x: dict, *, Hk: int, Hv: int, io_bf16: bool, l2norm: bool = True,
                 scale: float = 1.0, l2_eps: float = 1e-6, norm_eps: float = 1e-6,
                 want_final_state: bool = True, want_conv_state: bool = True,
                 pass_cu: Optional[bool] = None, state_bf16: bool = False,
                 slots: Optional[np.ndarray] = None, num_state_slots: int = 0,
                 snapshot_every: int = 0, snapshot_base: Optional[np.ndarray] = None,
                 num_snapshot_slots: int = 0, separate_launches: bool = False,
                 prep_write_back: bool = False, segments: bool = False, pipelined: bool = False,
                 device="cuda"):
        """x["state"] / x["conv_state"] hold num_state_slots rows (a pool)
        when `slots` is given, else N rows; x["state"] is float32 or, with
        state_bf16, uint16 bf16 bits.  separate_launches / prep_write_back /
        segments / pipelined set GDN_FLAG_SEPARATE_LAUNCHES /
        GDN_FLAG_PREP_WRITE_BACK / GDN_FLAG_SEGMENTS / GDN_FLAG_PIPELINED."""
        import torch
        self.cu_host = np.asarray(x["cu_seqlens"], dtype=np.int32)
        self.N = len(self.cu_host) - 1
        self.T = int(self.cu_host[-1])
        self.Hk, self.Hv, self.io_bf16 = Hk, Hv, io_bf16
        d = device
        self.q, self.k, self.v = (to_device(x[n], d) for n in ("q", "k", "v"))
        self.g, self.beta = to_device(x["g"], d), to_device(x["beta"], d)
        self.z, self.conv_w, self.norm_w = (to_device(x.get(n), d) for n in ("z", "conv_w", "norm_w"))
        self.initial_state = to_device(x.get("state"), d)
        self.conv_state_in = to_device(x.get("conv_state"), d)
        if pass_cu is None:
            pass_cu = self.N > 1
        self.cu = to_device(self.cu_host, d) if pass_cu else None
        self.state_bf16 = state_bf16
        self.slots = to_device(None if slots is None else np.asarray(slots, np.int32), d)
        self.num_state_slots = int(num_state_slots)
        rows = self.num_state_slots if self.num_state_slots > 0 else self.N
        self.snapshot_every = int(snapshot_every)
        self.snapshot_base = to_device(None if snapshot_base is None else np.asarray(snapshot_base, np.int32), d)
        self.num_snapshot_slots = int(num_snapshot_slots)
        self.extended = state_bf16 or slots is not None or self.num_state_slots > 0 or self.snapshot_every > 0
        sdt = torch.bfloat16 if state_bf16 else torch.float32
        self.desc = B.make_desc(self.N, self.T, Hk, Hv, B.GDN_BF16 if io_bf16 else B.GDN_F32,
                                B.GDN_BF16 if state_bf16 else B.GDN_F32, scale, l2_eps, norm_eps, l2norm,
                                separate_launches=separate_launches, prep_write_back=prep_write_back,
                                segments=segments, pipelined=pipelined)
        self.out = empty_like_io((max(self.T, 1), Hv, 128), io_bf16, d)
        self.final_state = (torch.empty((rows, Hv, 128, 128), dtype=sdt, device=d)
                            if want_final_state else None)
        Cch = 2 * Hk * 128 + Hv * 128
        self.conv_state_out = (empty_like_io((rows, 3, Cch), io_bf16, d)
                               if want_conv_state else None)
        self.snapshots = (torch.empty((self.num_snapshot_slots, Hv, 128, 128), dtype=sdt, device=d)
                          if self.snapshot_every > 0 else None)
        nbytes = B.gdn_prefill_workspace_size(self.desc)
        self.workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=d)

    def kwargs(self):
        return dict(z=self.z, conv_w=self.conv_w, norm_w=self.norm_w, cu_seqlens=self.cu,
                    initial_state=self.initial_state, conv_state_in=self.conv_state_in,
                    out=self.out, final_state=self.final_state,
                    conv_state_out=self.conv_state_out, workspace=self.workspace)

    def run(self, stream=None):
        if self.extended:
            B.gdn_prefill_ex(self.desc, self.q, self.k, self.v, self.g, self.beta, stream=stream,
                             state_slots=self.slots, num_state_slots=self.num_state_slots,
                             state_snapshots=self.snapshots, snapshot_base=self.snapshot_base,
                             snapshot_every=self.snapshot_every,
                             num_snapshot_slots=self.num_snapshot_slots, **self.kwargs())
            return
        B.gdn_prefill(self.desc, self.q, self.k, self.v, self.g, self.beta, stream=stream,
                      **self.kwargs())

    def set_launch(self, separate_launches: bool = False, prep_write_back: bool = False):
        """Choose the launch form of later calls (descriptor flags)."""
        f = self.desc.flags & ~(B.GDN_FLAG_SEPARATE_LAUNCHES | B.GDN_FLAG_PREP_WRITE_BACK)
        self.desc.flags = f | (B.GDN_FLAG_SEPARATE_LAUNCHES if separate_launches else 0) \
            | (B.GDN_FLAG_PREP_WRITE_BACK if prep_write_back else 0)

    def wait_status(self, stream=None) -> int:
        """1 if a wait of the last call on this workspace gave up."""
        return B.gdn_prefill_wait_status(self.workspace, stream=stream)

    def run_profiled(self, events, stream=None):
        return B.gdn_prefill_profiled(self.desc, self.q, self.k, self.v, self.g, self.beta,
                                      events=events, stream=stream, **self.kwargs())


class DecodeCall:
    """All device buffers of one gdn_decode call built from host arrays."""

    def __init__(self, x: dict, *, Hk: int, Hv: int, io_bf16: bool, state_bf16: bool,
                 l2norm: bool = True, scale: float = 1.0, l2_eps: float = 1e-6,
                 norm_eps: float = 1e-6, slots: Optional[np.ndarray] = None,
                 num_state_slots: Optional[int] = None, device="cuda"):
        d = device
        self.N = int(np.asarray(x["q"]).shape[0])
        self.q, self.k, self.v = (to_device(x[n], d) for n in ("q", "k", "v"))
        self.g, self.beta = to_device(x["g"], d), to_device(x["beta"], d)
        self.z, self.conv_w, self.norm_w = (to_device(x.get(n), d) for n in ("z", "conv_w", "norm_w"))
        self.state = to_device(x["state"], d)
        self.conv_state = to_device(x.get("conv_state"), d)
        self.slots = to_device(None if slots is None else np.asarray(slots, np.int32), d)
        self.num_state_slots = num_state_slots if num_state_slots is not None else self.state.shape[0]
        self.desc = B.make_desc(self.N, self.N, Hk, Hv, B.GDN_BF16 if io_bf16 else B.GDN_F32,
                                B.GDN_BF16 if state_bf16 else B.GDN_F32, scale, l2_eps, norm_eps,
                                l2norm)
        self.out = empty_like_io((self.N, Hv, 128), io_bf16, d)

    def run(self, stream=None):
        B.gdn_decode(self.desc, self.q, self.k, self.v, self.g, self.beta, state=self.state,
                     out=self.out, z=self.z, conv_w=self.conv_w, norm_w=self.norm_w,
                     conv_state=self.conv_state, state_slots=self.slots,
                     num_state_slots=self.num_state_slots, stream=stream)


class VerifyCall:
    """Buffers of one gdn_decode_verify call: x holds the D draft tokens of each
    of N sequences packed as a prefill of N sequences of length D (q [N*D, Hk,
    128], ...), states [N or S, ...]."""

    def __init__(self, x: dict, *, D: int, Hk: int, Hv: int, io_bf16: bool, state_bf16: bool,
                 l2norm: bool = True, scale: float = 1.0, l2_eps: float = 1e-6,
                 norm_eps: float = 1e-6, slots: Optional[np.ndarray] = None,
                 num_state_slots: Optional[int] = None, want_conv_ckpt: bool = True, device="cuda"):
        import torch
        d = device
        self.D = D
        self.N = int(np.asarray(x["q"]).shape[0]) // D
        self.q, self.k, self.v = (to_device(x[n], d) for n in ("q", "k", "v"))
        self.g, self.beta = to_device(x["g"], d), to_device(x["beta"], d)
        self.z, self.conv_w, self.norm_w = (to_device(x.get(n), d) for n in ("z", "conv_w", "norm_w"))
        self.state = to_device(x["state"], d)
        self.conv_state = to_device(x.get("conv_state"), d)
        self.slots = to_device(None if slots is None else np.asarray(slots, np.int32), d)
        self.num_state_slots = num_state_slots if num_state_slots is not None else self.state.shape[0]
        self.desc = B.make_desc(self.N, self.N * D, Hk, Hv, B.GDN_BF16 if io_bf16 else B.GDN_F32,
                                B.GDN_BF16 if state_bf16 else B.GDN_F32, scale, l2_eps, norm_eps,
                                l2norm)
        sdt = torch.bfloat16 if state_bf16 else torch.float32
        self.state_ckpt = torch.empty((self.N, D, Hv, 128, 128), dtype=sdt, device=d)
        Cch = 2 * Hk * 128 + Hv * 128
        self.conv_ckpt = empty_like_io((self.N, D, 3, Cch), io_bf16, d) if want_conv_ckpt else None
        self.out = empty_like_io((self.N * D, Hv, 128), io_bf16, d)

    def run(self, stream=None):
        B.gdn_decode_verify(self.desc, self.D, self.q, self.k, self.v, self.g, self.beta,
                            state=self.state, state_ckpt=self.state_ckpt, out=self.out, z=self.z,
                            conv_w=self.conv_w, norm_w=self.norm_w, conv_state=self.conv_state,
                            conv_ckpt=self.conv_ckpt, state_slots=self.slots,
                            num_state_slots=self.num_state_slots, stream=stream)

    def commit(self, accepted: np.ndarray, stream=None):
        acc = to_device(np.asarray(accepted, np.int32))
        B.gdn_decode_commit(self.desc, self.D, state_ckpt=self.state_ckpt, accepted=acc,
                            state=self.state, conv_ckpt=self.conv_ckpt, conv_state=self.conv_state,
                            state_slots=self.slots, num_state_slots=self.num_state_slots,
                            stream=stream)
