"""GPU parity of gdn_prefill against the fp64 oracle (through the C ABI)."""
import zlib

import numpy as np
import pytest

import gdn_synth as gs
from helpers import TOL_BF16, check_prefill, gpu_prefill, rel_l2, say

pytestmark = pytest.mark.gpu


def small(name, lens, **kw):
    base = dict(Hk=2, Hv=4, seed=zlib.crc32(name.encode()) % 10000)
    base.update(kw)
    return gs.Problem(name, lens, **base)


def test_c0_fp32_single_head():
    p = gs.configs()["C0"]
    x = gs.generate(p)
    e_out, e_fs = check_prefill(p, x)
    say(f"C0 rel_l2 out {e_out:.2e} state {e_fs:.2e}")


@pytest.mark.parametrize("T", [1, 2, 3, 63, 64, 65, 127, 200, 1000])
def test_lengths_full_layer(T):
    p = small(f"len{T}", [T], init_state_std=0.01, conv_state_std=0.01)
    check_prefill(p, gs.generate(p))


# b = 0 is pure decay; its decay is kept weak enough that the fp64 reference
# state (exp(sum g) S0) stays far above fp32 underflow.
@pytest.mark.parametrize("g_scale,beta", [(0.01, None), (0.0, None), (0.05, 0.0), (0.01, 1.0)])
def test_weak_decay_and_extreme_beta(g_scale, beta):
    p = small(f"decay{g_scale}-beta{beta}", [300], init_state_std=0.01, g_scale=g_scale,
              beta_fixed=beta)
    check_prefill(p, gs.generate(p))


def test_varlen_with_empty_and_ragged_sequences():
    p = small("varlen", [0, 1, 2, 3, 64, 65, 130, 5, 0], init_state_std=0.01,
              conv_state_std=0.01)
    check_prefill(p, gs.generate(p))


@pytest.mark.parametrize("Hk,Hv", [(4, 4), (1, 4), (3, 6)])
def test_head_groupings(Hk, Hv):
    p = small(f"heads{Hk}x{Hv}", [150, 77], Hk=Hk, Hv=Hv, init_state_std=0.01)
    check_prefill(p, gs.generate(p))


def test_no_conv_no_gate_no_l2_bf16():
    p = small("plain-bf16", [190], conv=False, gate=False, l2norm=False, prenormalize_qk=True)
    check_prefill(p, gs.generate(p))


def test_fp32_full_layer():
    p = small("f32-layer", [200, 3], io=gs.F32, init_state_std=0.01, conv_state_std=0.01)
    e_out, e_fs = check_prefill(p, gs.generate(p))
    say(f"fp32 full layer rel_l2 out {e_out:.2e} state {e_fs:.2e}")


def test_scale_argument():
    p = small("scale", [100], scale=1.0 / np.sqrt(128.0))
    check_prefill(p, gs.generate(p))


def test_zero_tokens_passes_states_through():
    p = small("empty", [0], init_state_std=0.01, conv_state_std=0.01)
    x = gs.generate(p)
    out, fs, cs, _ = gpu_prefill(p, x)
    assert np.array_equal(fs, x["state"])
    assert np.array_equal(cs, x["conv_state"])


def test_c1_full_size_sampled_heads():
    p = gs.configs()["C1"]
    x = gs.generate(p)
    for heads in ((0, 2), (30, 32)):
        e_out, e_fs = check_prefill(p, x, heads=heads)
        say(f"C1 heads {heads}: rel_l2 out {e_out:.2e} state {e_fs:.2e}")


def test_c2_long_context_sampled_heads():
    p = gs.configs()["C2"]
    x = gs.generate(p)
    e_out, e_fs = check_prefill(p, x, heads=(17, 18))
    say(f"C2 head 17: rel_l2 out {e_out:.2e} state {e_fs:.2e}")


def test_c3_varlen_sampled_heads():
    p = gs.configs()["C3"]
    x = gs.generate(p)
    e_out, e_fs = check_prefill(p, x, heads=(5, 6))
    say(f"C3 head 5: rel_l2 out {e_out:.2e} state {e_fs:.2e}")
