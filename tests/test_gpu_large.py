"""The largest inputs of the GPU suite: tensors past 2 GiB, so that every byte
offset the kernels form from a uniform base and a per-lane 32-bit part is
taken beyond 2^31 bytes of a buffer.  The oracle checks sampled value heads
(it runs the whole layer for them), every output is checked finite, and the
conv states bit for bit.

- prefill: one sequence of 2^18 + 37 tokens at 16 key / 32 value heads (the
  output and z are 2.15 GB each, the workspace 8.4 GB), in the pipelined and
  the separate launches, whose outputs must agree bit for bit;
- decode: 4,096 sequences with fp32 states (8.6 GB of state)."""
import numpy as np
import pytest

import gdn_synth as gs
from helpers import TOL_BF16, io_to_f64, rel_l2, say
from oracle import oracle

pytestmark = pytest.mark.gpu

SAMPLED = [(0, 4), (28, 32)]


def test_prefill_past_2gib_offsets():
    import torch
    from gated_deltanet_layer_02_amd.tensors import PrefillCall, to_host
    T = (1 << 18) + 37
    p = gs.Problem("large-prefill", [T], Hk=16, Hv=32, init_state_std=0.01, conv_state_std=0.01, seed=5151)
    say(f"large prefill: generating T={T}")
    x = gs.generate(p)
    res = {}
    for separate in (False, True):
        say(f"  gpu call, separate launches {separate}")
        call = PrefillCall(x, Hk=p.Hk, Hv=p.Hv, io_bf16=True, separate_launches=separate)
        call.run()
        torch.cuda.synchronize()
        assert call.wait_status() == 0
        res[separate] = (to_host(call.out)[:T], to_host(call.final_state), to_host(call.conv_state_out))
        del call
        torch.cuda.empty_cache()
    for a, b in zip(res[False], res[True]):
        assert np.array_equal(a, b), "pipelined and separate launches differ"
    out, fs, cs = res[False]
    del res
    assert np.all(np.isfinite(io_to_f64(out[::97]))) and np.all(np.isfinite(fs))
    for h0, h1 in SAMPLED:
        say(f"  oracle, value heads {h0}..{h1 - 1}")
        r_out, r_fs, r_cs = oracle.run_problem(p, x, heads=(h0, h1))
        e_out = rel_l2(io_to_f64(out[:, h0:h1]), r_out)
        e_fs = rel_l2(fs[:, h0:h1], r_fs)
        say(f"  heads {h0}..{h1 - 1}: rel_l2 out {e_out:.2e} state {e_fs:.2e}")
        assert e_out <= TOL_BF16 and e_fs <= TOL_BF16
        assert np.array_equal(cs, r_cs), "conv state not bit-exact"


def test_decode_past_2gib_offsets():
    import torch
    from gated_deltanet_layer_02_amd.tensors import DecodeCall, to_host
    N = 4096
    p = gs.Problem("large-decode", [1] * N, Hk=16, Hv=32, init_state_std=0.01, conv_state_std=0.01,
                   seed=5252, decode=True)
    say(f"large decode: generating N={N} (fp32 state {N * 32 * 128 * 128 * 4 / 2**30:.1f} GiB)")
    x = gs.generate(p)
    dc = DecodeCall(x, Hk=p.Hk, Hv=p.Hv, io_bf16=True, state_bf16=False)
    dc.run()
    torch.cuda.synchronize()
    out = io_to_f64(to_host(dc.out))
    st = to_host(dc.state)
    cs = to_host(dc.conv_state)
    del dc
    torch.cuda.empty_cache()
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(st[:, :, ::17]))
    for h0, h1 in SAMPLED:
        say(f"  oracle, value heads {h0}..{h1 - 1}")
        r_out, r_fs, r_cs = oracle.run_problem(p, x, heads=(h0, h1))
        e_out = rel_l2(out[:, h0:h1], r_out)
        e_st = rel_l2(st[:, h0:h1], r_fs)
        say(f"  heads {h0}..{h1 - 1}: rel_l2 out {e_out:.2e} state {e_st:.2e}")
        assert e_out <= TOL_BF16 and e_st <= TOL_BF16
        assert np.array_equal(cs, r_cs), "conv state not bit-exact"
