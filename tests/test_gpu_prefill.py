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
    say(f"C0 {check_prefill(p, x)}")


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
    say(f"fp32 full layer {check_prefill(p, gs.generate(p))}")


def test_scale_argument():
    p = small("scale", [100], scale=1.0 / np.sqrt(128.0))
    check_prefill(p, gs.generate(p))


def test_zero_tokens_passes_states_through():
    p = small("empty", [0], init_state_std=0.01, conv_state_std=0.01)
    x = gs.generate(p)
    out, fs, cs, _ = gpu_prefill(p, x)
    assert np.array_equal(fs, x["state"])
    assert np.array_equal(cs, x["conv_state"])


def test_many_short_sequences_qwen_shape():
    """Nine sequences of 0 to 6 chunks at 16 key / 32 value heads: 576 sweep
    workgroups, more than one round of CUs, so the sweep runs with split
    operand buffers; the lengths take it through its first iterations and the
    copies it repeats past a sequence's last chunk."""
    p = gs.Problem("short-seqs-qwen", [0, 1, 63, 64, 65, 130, 200, 257, 330], Hk=16, Hv=32,
                   init_state_std=0.01, conv_state_std=0.01, seed=4242)
    say(f"short sequences {check_prefill(p, gs.generate(p), batch=16)}")


@pytest.mark.parametrize("N", [1024, 1500])
def test_many_sequences_chunk_table(N):
    """1,024 packed sequences (the most the chunk table orders by length) and
    1,500 (sequence order, and a chunk-offset scan over two blocks of 1,024),
    lengths 0 to 200 tokens, 2 key / 4 value heads."""
    rng = np.random.default_rng(N)
    lens = [int(x) for x in rng.choice([0, 1, 5, 63, 64, 65, 127, 130, 200], size=N)]
    p = small(f"many-seqs-{N}", lens, init_state_std=0.01, conv_state_std=0.01)
    say(f"{N} sequences, {sum(lens)} tokens {check_prefill(p, gs.generate(p))}")


def test_serving_prefill_all_heads():
    """The serving stand-in: 93 new prompts of 250-350 tokens packed with
    cu_seqlens at 16 key / 32 value heads (separate launches: 5,952 sweep
    workgroups), every value head against the oracle."""
    p = gs.serving()["prefill"]
    say(f"serving prefill {check_prefill(p, gs.generate(p), batch=16)}")


# Full sizes, every value head against the oracle (the bench's launch
# configuration: plain calls, which take the pipelined form for C1 and C2 and
# separate launches for C3).
@pytest.mark.parametrize("separate", [False, True], ids=["default-launch", "separate-launches"])
def test_c1_full_size_all_heads(separate):
    p = gs.configs()["C1"]
    x = gs.generate(p)
    say(f"C1 ({'separate' if separate else 'default'}) {check_prefill(p, x, separate_launches=separate)}")


def test_c2_long_context_all_heads():
    p = gs.configs()["C2"]
    x = gs.generate(p)
    say(f"C2 {check_prefill(p, x, batch=16)}")


def test_c3_varlen_all_heads():
    p = gs.configs()["C3"]
    x = gs.generate(p)
    say(f"C3 {check_prefill(p, x, batch=16)}")
