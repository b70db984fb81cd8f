"""The pipelined prefill launch (chunk prep and state sweep in one grid, with
per-chunk flags between them) against separate launches of the same kernels
(GDN_FLAG_SEPARATE_LAUNCHES).  Both run the same arithmetic in the same order,
so every output must match bit for bit; the pipelined result is also checked
against the fp64 oracle on every value head.  Which form ran is read from the
stage ids of a profiled call; every call's wait status must be clean."""
import ctypes
import zlib

import numpy as np
import pytest

import gdn_synth as gs
from helpers import TOL_BF16, compare_heads, io_to_f64, rel_l2, say
from oracle import oracle

pytestmark = pytest.mark.gpu


def _problem(name, lens, **kw):
    base = dict(init_state_std=0.01, conv_state_std=0.01, seed=zlib.crc32(name.encode()) % 10000)
    base.update(kw)
    return gs.Problem(name, lens, **base)


class _Events:
    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(e)) == 0
            self.ev.append(e.value)

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(e)


def _stages(call):
    import torch
    from gated_deltanet_layer_02_amd.binding import STAGE_NAMES
    ev = _Events(2 + 2 * 8)
    ids = call.run_profiled(ev.ev, stream=torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    ev.close()
    return [STAGE_NAMES[i] for i in ids]


def _outputs(call, rows=None):
    """Outputs of a call; of pool-shaped state outputs only `rows` (the slots:
    the other rows of a freshly allocated pool are never written)."""
    from gated_deltanet_layer_02_amd.tensors import to_host
    res = {"out": to_host(call.out)[: call.T]}
    for n in ("final_state", "conv_state_out", "snapshots"):
        t = getattr(call, n, None)
        if t is not None:
            a = to_host(t)
            res[n] = a[rows] if rows is not None and n != "snapshots" else a
    return res


def _run_both(p, x, expect_pipe, **kw):
    """Outputs of the pipelined and of the separate launches (two calls each,
    on the same workspace, to cover flags left by an earlier call)."""
    import torch
    from gated_deltanet_layer_02_amd.tensors import PrefillCall
    res = {}
    for pipe in (True, False):
        call = PrefillCall(x, Hk=p.Hk, Hv=p.Hv, io_bf16=True, separate_launches=not pipe, pipelined=pipe, **kw)
        if not call.extended:
            st = _stages(call)
            say(f"  pipeline={int(pipe)}: stages {st}")
            assert ("prep_sweep" in st) == (pipe and expect_pipe), st
        rows = kw.get("slots")
        call.run()
        torch.cuda.synchronize()
        first = _outputs(call, rows)
        assert call.wait_status() == 0
        call.workspace.fill_(0xA5)   # garbage in the flags must not read as published
        call.run()
        torch.cuda.synchronize()
        assert call.wait_status() == 0
        again = _outputs(call, rows)
        for n in first:
            assert np.array_equal(first[n], again[n]), (pipe, n)
        res[pipe] = (first, call)
    return res


def _assert_same(res):
    a, b = res[True][0], res[False][0]
    assert a.keys() == b.keys()
    for n in a:
        assert np.array_equal(a[n], b[n]), f"{n} differs between pipelined and separate launches"


CASES = [
    # name, seq lens, heads (Hk, Hv), extra problem options, pipelined?
    ("one-seq", [64 * 24 + 37], (16, 32), {}, True),
    ("two-seqs", [64 * 9 + 5, 64 * 7], (16, 32), {}, True),
    ("three-seqs", [64 * 3, 100, 64 * 2 + 1], (16, 32), {}, False),   # sweep > half the CUs
    ("small-heads", [64 * 10 + 3], (2, 4), {}, True),                 # Hk not a multiple of 8
    ("empty-seq", [200, 0, 130], (4, 8), {}, True),
    ("no-conv-no-gate", [64 * 5 + 9], (2, 4), dict(conv=False, gate=False), True),
    ("one-token", [1], (16, 32), {}, True),
    ("post-first", [64 * 256 + 37], (16, 32), {}, True),             # norm workgroups ahead of the prep
]


@pytest.mark.parametrize("name,lens,heads,opts,expect_pipe", CASES, ids=[c[0] for c in CASES])
def test_pipeline_matches_separate_launches(name, lens, heads, opts, expect_pipe):
    p = _problem(f"pipe-{name}", lens, Hk=heads[0], Hv=heads[1], **opts)
    x = gs.generate(p)
    say(f"pipeline case {name}: lens {lens} Hk={p.Hk} Hv={p.Hv} {opts}")
    res = _run_both(p, x, expect_pipe)
    _assert_same(res)
    # and the oracle, every value head
    r_out, r_fs, r_cs = oracle.run_problem(p, x)
    rep_ = compare_heads(p, io_to_f64(res[True][0]["out"]), res[True][0]["final_state"], r_out, r_fs,
                         TOL_BF16, chunk_check=p.gate)
    say(f"  {rep_}")
    assert np.array_equal(res[True][0]["conv_state_out"], r_cs)


@pytest.mark.parametrize("lens,heads", [([1000], (2, 4)), ([320], (16, 32)), ([1024], (16, 32)),
                                         ([1984], (8, 16))], ids=["1000x2-4", "320x16-32", "1024x16-32", "1984x8-16"])
def test_small_calls_take_separate_launches(lens, heads):
    """One sequence whose sweep takes at most an eighth of the CUs (at most
    16 value heads) or with at most 16 chunk slots: the plain call takes
    separate launches (faster there), GDN_FLAG_PIPELINED the pipelined one,
    with the same bits; every value head against the oracle."""
    from gated_deltanet_layer_02_amd.tensors import PrefillCall
    p = _problem(f"small-call-{lens[0]}-{heads[1]}", lens, Hk=heads[0], Hv=heads[1])
    x = gs.generate(p)
    assert "prep_sweep" not in _stages(PrefillCall(x, Hk=p.Hk, Hv=p.Hv, io_bf16=True))
    res = _run_both(p, x, True)
    _assert_same(res)
    r_out, r_fs, r_cs = oracle.run_problem(p, x)
    rep_ = compare_heads(p, io_to_f64(res[True][0]["out"]), res[True][0]["final_state"], r_out, r_fs,
                         TOL_BF16, chunk_check=p.gate)
    say(f"  {rep_}")


def test_pipeline_pool_bf16_state_snapshots():
    """State pool rows by slot, bf16 state storage and chunk snapshots through
    the pipelined launch (asked for: the same shape's plain call, a small one,
    takes separate launches)."""
    lens = [64 * 6 + 10, 64 * 4]
    p = _problem("pipe-pool", lens, Hk=2, Hv=4)
    x = gs.generate(p)
    rows, slots = 5, np.array([3, 0], np.int32)
    rng = np.random.default_rng(11)
    x["state"] = gs.f32_to_bf16_bits((0.01 * rng.standard_normal((rows, p.Hv, 128, 128))).astype(np.float32))
    x["conv_state"] = gs.f32_to_bf16_bits((0.01 * rng.standard_normal((rows, 3, p.Cch))).astype(np.float32))
    every = 2
    counts = [(L - 1) // (64 * every) for L in lens]
    base = np.array([0, counts[0]], np.int32)
    say(f"pipeline pool case: lens {lens}, slots {slots.tolist()}, snapshots {counts}")
    res = _run_both(p, x, True, state_bf16=True, slots=slots, num_state_slots=rows,
                    snapshot_every=every, snapshot_base=base, num_snapshot_slots=sum(counts))
    _assert_same(res)
    # the same shape as a plain call takes separate launches, and the
    # pipelined form when asked for
    from gated_deltanet_layer_02_amd.tensors import PrefillCall
    plain = x | {"state": None, "conv_state": None}
    assert "prep_sweep" not in _stages(PrefillCall(plain, Hk=p.Hk, Hv=p.Hv, io_bf16=True))
    assert "prep_sweep" in _stages(PrefillCall(plain, Hk=p.Hk, Hv=p.Hv, io_bf16=True, pipelined=True))
    xo = dict(x, state=x["state"][slots], conv_state=x["conv_state"][slots])
    r_out, r_fs, r_cs = oracle.run_problem(p, xo)
    out = io_to_f64(res[True][0]["out"])
    fs = gs.bf16_bits_to_f32(res[True][0]["final_state"]).astype(np.float64)   # slot rows
    assert rel_l2(out, r_out) <= TOL_BF16 and rel_l2(fs, r_fs) <= TOL_BF16


def test_pipeline_c1_shape():
    """The 4096-token, 16 key / 32 value head layer: pipelined and separate
    launches agree bit for bit."""
    p = gs.configs()["C1"]
    x = gs.generate(p)
    say("pipeline case C1 shape")
    res = _run_both(p, x, True)
    _assert_same(res)


def _kept_units(call):
    """Prep units of the last (bf16) call whose fragments stayed in an XCD's L2:
    their ready flag is the call's epoch + 1.  Reads the flags where the
    workspace keeps them: after the call status words, the chunk offsets, the
    sweep order (min(N, 1024) int32), KB (32 units of 1 KB per chunk slot and
    key head) and VB (40 per chunk slot and value head), each region rounded
    up to 256 bytes; chunk slots = T / 64 + N with cu_seqlens, ceil(T / 64)
    without.  The output flags that follow all hold the epoch."""
    import torch
    w = call.workspace.view(torch.int64).cpu().numpy().view(np.uint64)
    C = call.T // 64 + call.N if call.cu is not None else -(-call.T // 64)
    r256 = lambda n: (n + 255) // 256 * 256
    # the call status words (256 bytes), the chunk offsets, the sweep order, KB, VB
    off = 256 + r256(4 * (call.N + 1)) + r256(4 * min(call.N, 1024)) + r256(C * call.Hk * 32 * 1024) \
        + r256(C * call.Hv * 40 * 1024)
    ready = w[off // 8: off // 8 + C * call.Hk]
    off += r256(C * call.Hk * 8)
    published = -(-call.T // 64) * call.Hv * 8
    oready = w[off // 8: off // 8 + published]
    epoch = oready[0]
    assert epoch != 0 and epoch % 2 == 0 and np.all(oready == epoch), "workspace layout"
    return int(np.count_nonzero(ready == epoch + np.uint64(1)))


def test_pipeline_l2_hand_off_matches_write_through():
    """Prep fragments left in the L2 of the sweep's XCD and fragments written
    through to memory (GDN_FLAG_PREP_WRITE_BACK) give the same bits, in either
    order on one workspace (the flags of the other form's call are stale)."""
    import torch
    from gated_deltanet_layer_02_amd.tensors import PrefillCall
    p = gs.configs()["C1"]
    x = gs.generate(p)
    call = PrefillCall(x, Hk=p.Hk, Hv=p.Hv, io_bf16=True)
    call.workspace.zero_()
    res, kept = [], []
    for write_back in (False, True, False):
        call.set_launch(prep_write_back=write_back)
        call.run()
        torch.cuda.synchronize()
        assert call.wait_status() == 0
        res.append(_outputs(call))
        kept.append(_kept_units(call))
    say(f"pipeline L2 hand-off, C1 shape: units kept in L2 per call {kept} of {p.T // 64 * p.Hk}")
    assert kept[1] == 0
    for r in res[1:]:
        for n in res[0]:
            assert np.array_equal(res[0][n], r[n]), n


def test_pipeline_write_back_fallback():
    """Two key heads: prep units are dealt chunk-major over every XCD while the
    sweep of a key head sits on one, so most units find a reader elsewhere and
    write their L2 back before publishing; the result equals the all-write-back
    form bit for bit."""
    import torch
    from gated_deltanet_layer_02_amd.tensors import PrefillCall
    p = _problem("pipe-fallback", [64 * 20 + 11], Hk=2, Hv=4)
    x = gs.generate(p)
    call = PrefillCall(x, Hk=p.Hk, Hv=p.Hv, io_bf16=True, pipelined=True)
    assert "prep_sweep" in _stages(call)
    res, kept = [], []
    for write_back in (False, True):
        call.set_launch(prep_write_back=write_back)
        call.workspace.zero_()
        call.run()
        torch.cuda.synchronize()
        assert call.wait_status() == 0
        res.append(_outputs(call))
        kept.append(_kept_units(call))
    units = -(-p.T // 64) * p.Hk
    say(f"pipeline write-back fallback, Hk=2: units kept in L2 {kept} of {units}")
    assert 0 < kept[0] < units and kept[1] == 0
    for n in res[0]:
        assert np.array_equal(res[0][n], res[1][n]), n


def test_wait_failure_is_reported_per_call():
    """A wait that gives up marks its call as failed in the workspace, and the
    next call on the same workspace starts clean.  The failure is forced from
    the host (GDN_FLAG_TEST_WAITS_GIVE_UP: every wait gives up at its first
    check), so every kernel still ends normally."""
    import torch
    from gated_deltanet_layer_02_amd import binding as B
    from gated_deltanet_layer_02_amd.tensors import PrefillCall
    p = _problem("pipe-fail", [64 * 10 + 3], Hk=2, Hv=4)
    x = gs.generate(p)
    ref = PrefillCall(x, Hk=p.Hk, Hv=p.Hv, io_bf16=True, separate_launches=True)
    ref.run()
    torch.cuda.synchronize()
    assert ref.wait_status() == 0
    call = PrefillCall(x, Hk=p.Hk, Hv=p.Hv, io_bf16=True, pipelined=True)
    assert "prep_sweep" in _stages(call)
    assert call.wait_status() == 0
    say("pipeline: every wait gives up at once (forced), then a normal call")
    call.desc.flags |= B.GDN_FLAG_TEST_WAITS_GIVE_UP
    call.run()
    torch.cuda.synchronize()
    assert call.wait_status() == 1
    call.desc.flags &= ~B.GDN_FLAG_TEST_WAITS_GIVE_UP
    call.run()
    torch.cuda.synchronize()
    assert call.wait_status() == 0
    a, b = _outputs(call), _outputs(ref)
    for n in a:
        assert np.array_equal(a[n], b[n]), n
