"""Shared helpers of the GPU tests: run the HIP library and the oracle on the
same seeded inputs and compare."""
from __future__ import annotations

import sys

import numpy as np

import gdn_synth as gs
from oracle import oracle

# Parity bars: relative L2 error on outputs and final states, 1e-4 for fp32
# inputs and 1e-2 for bf16 inputs; conv states bit-exact.
TOL_F32 = 1e-4
TOL_BF16 = 1e-2


def rel_l2(x, ref) -> float:
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / den) if den > 0 else float(np.linalg.norm(x))


def say(msg: str):
    """Name the case before each GPU step (flushed, in case the step fails)."""
    print(msg, flush=True)
    sys.stdout.flush()


def io_to_f64(a: np.ndarray) -> np.ndarray:
    return gs.to_f64(a, gs.BF16) if a.dtype == np.uint16 else a.astype(np.float64)


def gpu_prefill(p: gs.Problem, x: dict, **kw):
    import torch
    from gated_deltanet_layer_02_amd.tensors import PrefillCall, to_host
    call = PrefillCall(x, Hk=p.Hk, Hv=p.Hv, io_bf16=p.io == gs.BF16, l2norm=p.l2norm,
                       scale=p.scale, l2_eps=p.l2_eps, norm_eps=p.norm_eps, **kw)
    call.run()
    torch.cuda.synchronize()
    out = io_to_f64(to_host(call.out))[: p.T]
    fs = to_host(call.final_state) if call.final_state is not None else None
    cs = to_host(call.conv_state_out) if call.conv_state_out is not None else None
    return out, fs, cs, call


def check_prefill(p: gs.Problem, x: dict, heads=None, tol=None, **kw):
    """GPU prefill vs the oracle on value heads `heads` (default: all)."""
    say(f"prefill case: {p.name} lens={list(p.seq_lens)[:8]}{'...' if p.N > 8 else ''} "
        f"Hk={p.Hk} Hv={p.Hv} io={p.io} conv={p.conv} gate={p.gate}")
    out, fs, cs, call = gpu_prefill(p, x, **kw)
    h0, h1 = heads if heads is not None else (0, p.Hv)
    r_out, r_fs, r_cs = oracle.run_problem(p, x, heads=(h0, h1))
    tol = tol if tol is not None else (TOL_F32 if p.io == gs.F32 else TOL_BF16)
    e_out = rel_l2(out[:, h0:h1], r_out) if p.T > 0 else 0.0
    e_fs = rel_l2(fs[:, h0:h1], r_fs)
    assert np.all(np.isfinite(out[:, h0:h1]))
    assert e_out <= tol, f"{p.name}: out rel_l2 {e_out:.3e} > {tol}"
    assert e_fs <= tol, f"{p.name}: final state rel_l2 {e_fs:.3e} > {tol}"
    if cs is not None and r_cs is not None:
        assert np.array_equal(cs, r_cs), f"{p.name}: conv state not bit-exact"
    return e_out, e_fs
