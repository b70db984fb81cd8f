"""GPU parity of the segment-parallel prefill (GDN_FLAG_SEGMENTS) against the
fp64 oracle, through the C ABI.

The segment form cuts one sequence's chunks into P segments swept side by
side: every later segment from a zero state beside an identity chain, then
the start states are chained and their part added to the outputs.  Weak or
no decay keeps the start state's share of the later outputs large, so that a
wrong map or start state cannot hide behind the decay."""
import zlib

import numpy as np
import pytest

import gdn_synth as gs
from helpers import check_prefill, say

pytestmark = pytest.mark.gpu

SEG_COMPOSE, SEG_FIXUP = 6, 7   # GDN_STAGE_SEG_COMPOSE / GDN_STAGE_SEG_FIXUP


def stages(p, x, segments=True, separate_launches=False):
    """Stage ids of one profiled call (by default with the segments flag)."""
    import ctypes

    import torch
    from gated_deltanet_layer_02_amd.tensors import PrefillCall
    call = PrefillCall(x, Hk=p.Hk, Hv=p.Hv, io_bf16=p.io == gs.BF16, l2norm=p.l2norm, scale=p.scale,
                       l2_eps=p.l2_eps, norm_eps=p.norm_eps, segments=segments,
                       separate_launches=separate_launches)
    hip = ctypes.CDLL("libamdhip64.so.7")
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    ev = []
    for _ in range(2 + 2 * 16):
        e = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
        ev.append(e.value)
    ids = call.run_profiled(ev, stream=torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    for e in ev:
        hip.hipEventDestroy(e)
    return ids


def small(name, lens, **kw):
    base = dict(Hk=2, Hv=4, seed=zlib.crc32(name.encode()) % 10000)
    base.update(kw)
    return gs.Problem(name, lens, **base)


# T = 512: 8 chunks, two segments of 4; T = 1000: 16 chunks (the last of 40
# tokens), four segments of 4; T = 4096: eight segments of 8 chunks.
@pytest.mark.parametrize("T", [512, 1000, 4096])
@pytest.mark.parametrize("g_scale", [1.0, 0.01, 0.0], ids=["decay", "weak-decay", "no-decay"])
def test_segments_against_oracle(T, g_scale):
    p = small(f"seg{T}-g{g_scale}", [T], init_state_std=0.01, conv_state_std=0.01, g_scale=g_scale)
    x = gs.generate(p)
    ids = stages(p, x)
    say(f"segments T={T} g_scale={g_scale}: stages {ids}")
    assert SEG_COMPOSE in ids and SEG_FIXUP in ids
    say(f"  {check_prefill(p, x, segments=True)}")


def test_segments_no_gate_no_conv_zero_state():
    p = small("seg-plain", [1500], conv=False, gate=False, g_scale=0.01)
    x = gs.generate(p)
    assert SEG_COMPOSE in stages(p, x)
    say(f"segments, no gate / conv / initial state: {check_prefill(p, x, segments=True)}")


def test_segments_short_sequence_falls_back():
    """Fewer than 8 chunks: the flag does not apply, the call takes the usual form."""
    p = small("seg-short", [300], init_state_std=0.01, conv_state_std=0.01)
    x = gs.generate(p)
    assert SEG_COMPOSE not in stages(p, x)
    check_prefill(p, x, segments=True)


def test_segments_tp8_share():
    """One GPU's share of the 16 key / 32 value head layer under eight-way
    head parallelism: 2 key / 4 value heads, 4,096 tokens, seeded states."""
    p = gs.Problem("seg-tp8-share", [4096], Hk=2, Hv=4, init_state_std=0.01, conv_state_std=0.01,
                   seed=2024)
    x = gs.generate(p)
    assert SEG_COMPOSE in stages(p, x)
    say(f"segments, TP-8 share: {check_prefill(p, x, segments=True)}")


@pytest.mark.parametrize("Hk,Hv,T", [(4, 8, 2048), (8, 16, 4096)])
def test_segments_by_default_for_few_heads(Hk, Hv, T):
    """Without the flag, one sequence of >= 32 chunks with <= 16 value heads
    takes the segment form (2,048 tokens at 4 key / 8 value heads: seven
    segments of 5 chunks, the last of 2; 4,096 at 8 / 16: four of 16), and
    separate launches asked for alone keep the plain form."""
    p = gs.Problem(f"seg-default-{Hk}x{Hv}", [T], Hk=Hk, Hv=Hv, init_state_std=0.01,
                   conv_state_std=0.01, seed=3000 + Hv)
    x = gs.generate(p)
    assert SEG_COMPOSE in stages(p, x, segments=False)
    assert SEG_COMPOSE not in stages(p, x, segments=False, separate_launches=True)
    say(f"segments by default, {Hk}x{Hv}: {check_prefill(p, x)}")


def test_segments_tp8_share_long_context():
    """One GPU's share of the 65,536-token layer under eight-way head
    parallelism (2 key / 4 value heads, seeded states), the default call:
    sixteen segments of 64 chunks."""
    p = gs.Problem("seg-tp8-65k", [65536], Hk=2, Hv=4, init_state_std=0.01, conv_state_std=0.01,
                   seed=6553)
    x = gs.generate(p)
    assert SEG_COMPOSE in stages(p, x, segments=False)
    say(f"segments, TP-8 share, 65,536 tokens: {check_prefill(p, x)}")


def test_segments_c1_all_heads():
    p = gs.configs()["C1"]
    x = gs.generate(p)
    assert SEG_COMPOSE in stages(p, x)
    say(f"segments, C1: {check_prefill(p, x, segments=True)}")


def test_segments_c1_shape_weak_decay():
    """16 key / 32 value heads, 4,096 tokens, log-decay scaled by 0.01 and a
    seeded state: the first segment's final state still weighs on the second
    segment's outputs, so the correction is exercised at full width (with the
    workloads' decay it is negligible after a few tokens)."""
    p = gs.Problem("seg-c1-weak", [4096], init_state_std=0.01, conv_state_std=0.01, g_scale=0.01,
                   seed=4096)
    x = gs.generate(p)
    assert SEG_COMPOSE in stages(p, x)
    say(f"segments, 16 / 32 heads, weak decay: {check_prefill(p, x, batch=16, segments=True)}")


def test_segments_c2_all_heads():
    p = gs.configs()["C2"]
    x = gs.generate(p)
    assert SEG_COMPOSE in stages(p, x)
    say(f"segments, C2: {check_prefill(p, x, batch=16, segments=True)}")
