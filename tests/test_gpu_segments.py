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
from helpers import TOL_BF16, check_prefill, io_to_f64, rel_l2, say
from oracle import oracle

pytestmark = pytest.mark.gpu

SEG_COMPOSE, SEG_FIXUP = 6, 7   # GDN_STAGE_SEG_COMPOSE / GDN_STAGE_SEG_FIXUP


def stages(p, x, segments=True, separate_launches=False, **kw):
    """Stage ids of one profiled call (by default with the segments flag)."""
    import ctypes

    import torch
    from gated_deltanet_layer_02_amd.tensors import PrefillCall
    call = PrefillCall(x, Hk=p.Hk, Hv=p.Hv, io_bf16=p.io == gs.BF16, l2norm=p.l2norm, scale=p.scale,
                       l2_eps=p.l2_eps, norm_eps=p.norm_eps, segments=segments,
                       separate_launches=separate_launches, **kw)
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


def _state_f64(a):
    return gs.bf16_bits_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)


@pytest.mark.parametrize("case", ["two-sequences", "bf16-state", "snapshots", "pool"])
def test_segments_flag_falls_back(case):
    """The segment form takes one sequence with an fp32 state, no state pool
    and no snapshots.  With the flag set, a call of 2,048 tokens per sequence
    at 2 key / 4 value heads (which would otherwise qualify) that has two
    sequences, a bf16 state, snapshots every 8 chunks or a pool row gives the
    bits of the plain separate launches (the segment form's correction would
    change them) and matches the oracle."""
    import torch
    from gated_deltanet_layer_02_amd.tensors import PrefillCall, to_host
    lens = [1100, 948] if case == "two-sequences" else [2048]
    p = small(f"seg-fallback-{case}", lens, init_state_std=0.01, conv_state_std=0.01)
    x = gs.generate(p)
    kw, xo = {}, x
    if case == "bf16-state":
        x = dict(x, state=gs.f32_to_bf16_bits(x["state"]))
        xo = dict(x, state=gs.bf16_bits_to_f32(x["state"]))
        kw = dict(state_bf16=True)
    elif case == "snapshots":
        kw = dict(snapshot_every=8, snapshot_base=np.array([0], np.int32), num_snapshot_slots=3)
    elif case == "pool":
        rng = np.random.default_rng(77)
        pool = (0.01 * rng.standard_normal((3, p.Hv, 128, 128))).astype(np.float32)
        cpool = gs.f32_to_bf16_bits((0.01 * rng.standard_normal((3, 3, p.Cch))).astype(np.float32))
        x = dict(x, state=pool, conv_state=cpool)
        xo = dict(x, state=pool[[2]], conv_state=cpool[[2]])
        kw = dict(slots=np.array([2], np.int32), num_state_slots=3)
    if case == "two-sequences":   # the profiled entry point takes fp32 states without pool or snapshots
        ids = stages(p, x)
        say(f"segments flag, two sequences: stages {ids}")
        assert SEG_COMPOSE not in ids and SEG_FIXUP not in ids

    def run(**form):
        call = PrefillCall(x, Hk=p.Hk, Hv=p.Hv, io_bf16=True, **form, **kw)
        if case == "pool":   # the pool is updated in place
            call.final_state = call.initial_state
            call.conv_state_out = call.conv_state_in
        call.run()
        torch.cuda.synchronize()
        res = [to_host(call.out), to_host(call.final_state), to_host(call.conv_state_out)]
        return res + ([to_host(call.snapshots)] if case == "snapshots" else [])

    got = run(segments=True)
    plain = run(separate_launches=True)
    for name, u, w in zip(["out", "final state", "conv state", "snapshots"], got, plain):
        assert np.array_equal(u, w), f"{case}: {name} differs from the separate launches"
    out, fs, cs = io_to_f64(got[0])[: p.T], got[1], got[2]
    if case == "pool":
        assert np.array_equal(fs[:2], x["state"][:2]) and np.array_equal(cs[:2], x["conv_state"][:2])
        fs, cs = fs[[2]], cs[[2]]
    r_out, r_fs, r_cs = oracle.run_problem(p, xo)
    e_out, e_fs = rel_l2(out, r_out), rel_l2(_state_f64(fs), r_fs)
    msg = f"segments flag, {case}: rel_l2 out {e_out:.2e} state {e_fs:.2e}"
    assert np.array_equal(cs, r_cs), "conv state not bit-exact"
    if case == "snapshots":   # the states after 512, 1,024 and 1,536 tokens
        for j in range(3):
            L = 512 * (j + 1)
            sl = slice(0, L)
            _, r_s, _ = oracle.prefill(x["q"][sl], x["k"][sl], x["v"][sl], x["g"][sl], x["beta"][sl],
                                       cu_seqlens=np.array([0, L], np.int32), z=x["z"][sl],
                                       conv_w=x["conv_w"], norm_w=x["norm_w"], initial_state=x["state"],
                                       conv_state_in=x["conv_state"], use_l2=p.l2norm, scale=p.scale,
                                       l2_eps=p.l2_eps, norm_eps=p.norm_eps)
            e = rel_l2(_state_f64(got[3][j]), r_s[0])
            msg += f", snapshot {j} {e:.2e}"
            assert e <= TOL_BF16
    say(msg)
    assert e_out <= TOL_BF16 and e_fs <= TOL_BF16


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
