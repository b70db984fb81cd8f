"""Robustness of the HIP path: every output element written, bitwise
determinism, in-place state aliasing, a non-default stream."""
import numpy as np
import pytest

import gdn_synth as gs
from helpers import check_prefill, io_to_f64, rel_l2, say

pytestmark = pytest.mark.gpu


def _problem():
    return gs.Problem("robust", [70, 0, 129, 3], Hk=2, Hv=4, init_state_std=0.01,
                      conv_state_std=0.01, seed=31)


def test_every_output_written_and_deterministic():
    import torch
    from gated_deltanet_layer_02_amd.tensors import PrefillCall, to_host
    p = _problem()
    x = gs.generate(p)
    say("robustness: NaN-poisoned outputs, two runs")
    call = PrefillCall(x, Hk=2, Hv=4, io_bf16=True)
    results = []
    for _ in range(2):
        call.out.fill_(float("nan"))
        call.final_state.fill_(float("nan"))
        call.conv_state_out.fill_(float("nan"))
        call.workspace.fill_(0xFF)
        call.run()
        torch.cuda.synchronize()
        r = [to_host(call.out), to_host(call.final_state), to_host(call.conv_state_out)]
        assert np.all(np.isfinite(io_to_f64(r[0])))
        assert np.all(np.isfinite(r[1]))
        results.append(r)
    for a, b in zip(*results):
        assert np.array_equal(a, b)


def test_in_place_states_and_side_stream():
    import torch
    from gated_deltanet_layer_02_amd.tensors import PrefillCall, to_host
    p = _problem()
    x = gs.generate(p)
    say("robustness: in-place states on a side stream")
    ref = PrefillCall(x, Hk=2, Hv=4, io_bf16=True)
    ref.run()
    torch.cuda.synchronize()
    call = PrefillCall(x, Hk=2, Hv=4, io_bf16=True)
    call.final_state = call.initial_state            # in place
    call.conv_state_out = call.conv_state_in          # in place
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call.run(stream=s)
    s.synchronize()
    assert np.array_equal(to_host(call.out), to_host(ref.out))
    assert np.array_equal(to_host(call.initial_state), to_host(ref.final_state))
    assert np.array_equal(to_host(call.conv_state_in), to_host(ref.conv_state_out))


def test_decode_in_place_deterministic():
    import torch
    from gated_deltanet_layer_02_amd.tensors import DecodeCall, to_host
    p = gs.Problem("dec-det", [1] * 16, Hk=2, Hv=4, init_state_std=0.01, conv_state_std=0.01,
                   seed=32, decode=True)
    x = gs.generate(p)
    say("robustness: decode determinism")
    outs = []
    for _ in range(2):
        dc = DecodeCall(x, Hk=2, Hv=4, io_bf16=True, state_bf16=False)
        dc.out.fill_(float("nan"))
        dc.run()
        torch.cuda.synchronize()
        outs.append((to_host(dc.out), to_host(dc.state), to_host(dc.conv_state)))
        assert np.all(np.isfinite(io_to_f64(outs[-1][0])))
    for a, b in zip(*outs):
        assert np.array_equal(a, b)
