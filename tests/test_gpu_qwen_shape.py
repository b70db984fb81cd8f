"""GPU robustness at the Qwen3-Next layer shape (16 key / 32 value heads):
in-place states, poisoned outputs and workspace, a non-default caller stream,
and the per-kernel events of gdn_prefill_profiled."""
import ctypes

import numpy as np
import pytest

import gdn_synth as gs
from helpers import io_to_f64, say

pytestmark = pytest.mark.gpu


def _qwen_shape(name, T, seed):
    return gs.Problem(name, [T], Hk=16, Hv=32, init_state_std=0.01, conv_state_std=0.01,
                      seed=seed)


@pytest.mark.parametrize("T", [64 * 26 + 33, 64 * 256 + 33], ids=["norm-last", "norm-first"])
def test_in_place_poisoned_side_stream(T):
    """Every output written, results equal to a fresh call, and work queued
    on the caller's stream afterwards sees them.  At 257 chunks the norm /
    conv-state workgroups run ahead of the prep ones and overwrite the conv
    state in place early: only after the first chunk's prep units read it."""
    import torch
    from gated_deltanet_layer_02_amd.tensors import PrefillCall, to_host
    p = _qwen_shape("qwen-inplace", T, seed=5)
    x = gs.generate(p)
    say(f"Qwen shape in place on a side stream: T={T}")
    ref = PrefillCall(x, Hk=16, Hv=32, io_bf16=True)
    ref.run()
    torch.cuda.synchronize()
    call = PrefillCall(x, Hk=16, Hv=32, io_bf16=True)
    call.final_state = call.initial_state
    call.conv_state_out = call.conv_state_in
    call.out.fill_(float("nan"))
    call.workspace.fill_(0xFF)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        call.run(stream=s)
        out_copy = call.out.clone()          # queued behind the call on s
        state_copy = call.initial_state.clone()
    s.synchronize()
    assert np.all(np.isfinite(io_to_f64(to_host(out_copy))))
    assert np.array_equal(to_host(out_copy), to_host(ref.out))
    assert np.array_equal(to_host(state_copy), to_host(ref.final_state))
    assert np.array_equal(to_host(call.conv_state_in), to_host(ref.conv_state_out))


@pytest.mark.parametrize("pipeline", [True, False])
def test_profiled_brackets_every_kernel(pipeline):
    import torch
    from gated_deltanet_layer_02_amd.binding import STAGE_NAMES
    from gated_deltanet_layer_02_amd.tensors import PrefillCall
    T = 64 * 40
    p = _qwen_shape("qwen-profiled", T, seed=9)
    x = gs.generate(p)
    say(f"profiled call: T={T}")
    call = PrefillCall(x, Hk=16, Hv=32, io_bf16=True, separate_launches=not pipeline)
    hip = ctypes.CDLL("libamdhip64.so.7")
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                        ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    events = []
    for _ in range(2 + 2 * 8):
        e = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
        events.append(e.value)
    ids = call.run_profiled(events, stream=torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    want = ["prep_sweep"] if pipeline else ["chunk_prep", "state_sweep", "gated_norm", "conv_state"]
    assert [STAGE_NAMES[i] for i in ids] == want

    def ms(a, b):
        f = ctypes.c_float()
        assert hip.hipEventElapsedTime(ctypes.byref(f), a, b) == 0
        return f.value
    total = ms(events[0], events[1])
    for j in range(len(ids)):
        assert 0.0 <= ms(events[2 + 2 * j], events[3 + 2 * j]) <= total
    # too few event slots: refused before anything is launched (by the
    # binding when that leaves none)
    from gated_deltanet_layer_02_amd import binding as B
    with pytest.raises(B.GdnError if len(ids) > 1 else ValueError):
        call.run_profiled(events[:2 + 2 * (len(ids) - 1)], stream=torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    for e in events:
        hip.hipEventDestroy(e)
