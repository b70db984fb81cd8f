"""GPU parity of gdn_prefill_ex: bf16 state storage, a state pool indexed by
slots (updated in place), and chunk-boundary state snapshots, against the
fp64 oracle (a snapshot is the oracle's final state of the sequence prefix
that ends at the boundary)."""
import zlib

import numpy as np
import pytest

import gdn_synth as gs
from helpers import TOL_BF16, io_to_f64, rel_l2, say
from oracle import oracle

pytestmark = pytest.mark.gpu


def _problem(name, lens, **kw):
    base = dict(Hk=2, Hv=4, init_state_std=0.01, conv_state_std=0.01,
                seed=zlib.crc32(name.encode()) % 10000)
    base.update(kw)
    return gs.Problem(name, lens, **base)


def _state_f64(a):
    return gs.bf16_bits_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)


def _oracle_seq(p, x, n, length, state0, conv0, heads):
    """Oracle on the first `length` tokens of sequence n, from states (state0, conv0)."""
    t0 = int(x["cu_seqlens"][n])
    sl = slice(t0, t0 + length)
    return oracle.prefill(x["q"][sl], x["k"][sl], x["v"][sl], x["g"][sl], x["beta"][sl],
                          cu_seqlens=np.array([0, length], np.int32), z=x["z"][sl],
                          conv_w=x["conv_w"], norm_w=x["norm_w"], initial_state=state0[None],
                          conv_state_in=conv0[None], use_l2=p.l2norm, scale=p.scale,
                          l2_eps=p.l2_eps, norm_eps=p.norm_eps, heads=heads)


def test_bf16_state_storage():
    from gated_deltanet_layer_02_amd.tensors import PrefillCall, to_host
    import torch
    p = _problem("bf16-state", [130, 67, 1, 0])
    x = gs.generate(p)
    x["state"] = gs.f32_to_bf16_bits(x["state"])        # the stored state is bf16
    say(f"bf16 state storage: lens {p.seq_lens}")
    call = PrefillCall(x, Hk=p.Hk, Hv=p.Hv, io_bf16=True, state_bf16=True)
    call.run()
    torch.cuda.synchronize()
    r_out, r_fs, r_cs = oracle.run_problem(p, x)
    out = io_to_f64(to_host(call.out))[: p.T]
    fs = _state_f64(to_host(call.final_state))
    e_out, e_fs = rel_l2(out, r_out), rel_l2(fs, r_fs)
    say(f"  rel_l2 out {e_out:.2e} state {e_fs:.2e}")
    assert e_out <= TOL_BF16 and e_fs <= TOL_BF16
    assert np.array_equal(to_host(call.conv_state_out), r_cs)
    # the empty sequence passes its bf16 state through bit for bit
    assert np.array_equal(to_host(call.final_state)[3], x["state"][3])


@pytest.mark.parametrize("state_bf16", [False, True])
def test_state_pool_in_place(state_bf16):
    from gated_deltanet_layer_02_amd.tensors import PrefillCall, to_host
    import torch
    p = _problem(f"pool{int(state_bf16)}", [70, 0, 129])
    x = gs.generate(p)
    rows, slots = 6, np.array([4, 1, 2], np.int32)
    rng = np.random.default_rng(7)
    pool = (0.01 * rng.standard_normal((rows, p.Hv, 128, 128))).astype(np.float32)
    if state_bf16:
        pool = gs.f32_to_bf16_bits(pool)
    cpool = gs.f32_to_bf16_bits((0.01 * rng.standard_normal((rows, 3, p.Cch))).astype(np.float32))
    xs = dict(x, state=pool, conv_state=cpool)
    say(f"state pool: {rows} rows, slots {slots.tolist()}, bf16 state {state_bf16}")
    call = PrefillCall(xs, Hk=p.Hk, Hv=p.Hv, io_bf16=True, state_bf16=state_bf16, slots=slots,
                       num_state_slots=rows)
    call.final_state = call.initial_state                # the pool is updated in place
    call.conv_state_out = call.conv_state_in
    call.run()
    torch.cuda.synchronize()
    fs, cs = to_host(call.initial_state), to_host(call.conv_state_in)
    untouched = [r for r in range(rows) if r not in slots]
    assert np.array_equal(fs[untouched], pool[untouched])
    assert np.array_equal(cs[untouched], cpool[untouched])
    xo = dict(x, state=pool[slots], conv_state=cpool[slots])
    r_out, r_fs, r_cs = oracle.run_problem(p, xo)
    out = io_to_f64(to_host(call.out))[: p.T]
    e_out, e_fs = rel_l2(out, r_out), rel_l2(_state_f64(fs[slots]), r_fs)
    say(f"  rel_l2 out {e_out:.2e} state {e_fs:.2e}")
    assert e_out <= TOL_BF16 and e_fs <= TOL_BF16
    assert np.array_equal(cs[slots], r_cs)


@pytest.mark.parametrize("every,state_bf16", [(1, False), (2, False), (3, True)])
def test_snapshots(every, state_bf16):
    from gated_deltanet_layer_02_amd.tensors import PrefillCall, to_host
    import torch
    lens = [64 * 5 + 10, 64 * 2, 64 * 6, 40]
    p = _problem(f"snap{every}", lens)
    x = gs.generate(p)
    if state_bf16:
        x["state"] = gs.f32_to_bf16_bits(x["state"])
    # snapshot j (1-based) of sequence n: state after 64 * every * j tokens, j * 64 * every < L_n
    counts = [(L - 1) // (64 * every) if L > 0 else 0 for L in lens]
    base = np.concatenate([[0], np.cumsum(counts)[:-1]]).astype(np.int32)
    total = int(sum(counts))
    say(f"snapshots every {every} chunks: counts {counts}, bf16 state {state_bf16}")
    call = PrefillCall(x, Hk=p.Hk, Hv=p.Hv, io_bf16=True, state_bf16=state_bf16,
                       snapshot_every=every, snapshot_base=base, num_snapshot_slots=max(total, 1))
    call.run()
    torch.cuda.synchronize()
    snaps = _state_f64(to_host(call.snapshots))
    worst = 0.0
    for n, L in enumerate(lens):
        for j in range(1, counts[n] + 1):
            _, r_fs, _ = _oracle_seq(p, x, n, 64 * every * j, x["state"][n], x["conv_state"][n],
                                     heads=(0, p.Hv))
            e = rel_l2(snaps[base[n] + j - 1], r_fs[0])
            worst = max(worst, e)
            assert e <= TOL_BF16, (n, j, e)
    say(f"  worst snapshot rel_l2 {worst:.2e}")
    # the final state is unchanged by the snapshot option
    r_out, r_fs, _ = oracle.run_problem(p, x)
    assert rel_l2(_state_f64(to_host(call.final_state)), r_fs) <= TOL_BF16


def test_snapshots_c1_shape_all_heads():
    from gated_deltanet_layer_02_amd.tensors import PrefillCall, to_host
    import torch
    p = gs.configs()["C1"]
    x = gs.generate(p)
    every = 16                                           # every 1024 tokens: 3 snapshots
    say("C1 shape, snapshots every 16 chunks, every value head")
    call = PrefillCall(x, Hk=p.Hk, Hv=p.Hv, io_bf16=True, snapshot_every=every,
                       snapshot_base=np.array([0], np.int32), num_snapshot_slots=3)
    call.run()
    torch.cuda.synchronize()
    assert call.wait_status() == 0
    snaps = to_host(call.snapshots)
    assert np.all(np.isfinite(snaps))
    zero_state = np.zeros((p.Hv, 128, 128), np.float32)
    zero_conv = np.zeros((3, p.Cch), np.uint16)
    for j in range(1, 4):
        _, r_fs, _ = _oracle_seq(p, x, 0, 1024 * j, zero_state, zero_conv, heads=(0, p.Hv))
        got = snaps[j - 1].astype(np.float64)
        e = rel_l2(got, r_fs[0])
        per_head = [rel_l2(got[h], r_fs[0][h]) for h in range(p.Hv)]
        worst = int(np.argmax(per_head))
        say(f"  snapshot {j}: rel_l2 {e:.2e}, worst head {worst}: {per_head[worst]:.2e}")
        assert e <= TOL_BF16 and max(per_head) <= TOL_BF16


def test_short_packed_batch_pool_snapshots():
    """40 packed sequences of 0 to 300 tokens at 16 key / 32 value heads (more
    sweep workgroups than CUs, a few chunks each: the split-buffer sweep), with a
    bf16 state pool of 48 rows updated through slots and a snapshot after
    every chunk: outputs, pool rows and snapshots against the oracle, untouched
    pool rows bitwise unchanged."""
    from gated_deltanet_layer_02_amd.tensors import PrefillCall, to_host
    import torch
    rng = np.random.default_rng(4040)
    lens = [int(L) for L in rng.choice([0, 1, 63, 64, 65, 130, 200, 257, 300], size=40)]
    rows = 48
    slots = rng.permutation(rows)[:40].astype(np.int32)
    p = gs.Problem("short-pool", lens, init_state_std=0.01, conv_state_std=0.01, seed=4041)
    x = gs.generate(p)
    pool = gs.f32_to_bf16_bits((0.01 * rng.standard_normal((rows, p.Hv, 128, 128))).astype(np.float32))
    cpool = gs.f32_to_bf16_bits((0.01 * rng.standard_normal((rows, 3, p.Cch))).astype(np.float32))
    counts = [(L - 1) // 64 if L > 0 else 0 for L in lens]
    base = np.concatenate([[0], np.cumsum(counts)[:-1]]).astype(np.int32)
    total = int(sum(counts))
    say(f"short packed batch, pool and snapshots: {sum(lens)} tokens, {total} snapshots")
    xp = dict(x, state=pool, conv_state=cpool)
    call = PrefillCall(xp, Hk=p.Hk, Hv=p.Hv, io_bf16=True, state_bf16=True, slots=slots,
                       num_state_slots=rows, snapshot_every=1, snapshot_base=base,
                       num_snapshot_slots=max(total, 1))
    # the pool is updated in place: final state and conv state are the pool tensors
    call.final_state = call.initial_state
    call.conv_state_out = call.conv_state_in
    call.run()
    torch.cuda.synchronize()
    assert call.wait_status() == 0
    fs, cs = to_host(call.final_state), to_host(call.conv_state_out)
    untouched = np.setdiff1d(np.arange(rows), slots)
    assert np.array_equal(fs[untouched], pool[untouched]) and np.array_equal(cs[untouched], cpool[untouched])
    xo = dict(x, state=gs.bf16_bits_to_f32(pool[slots]), conv_state=cpool[slots])
    r_out, r_fs, r_cs = oracle.run_problem(p, xo)
    out = io_to_f64(to_host(call.out))[: p.T]
    e_out, e_fs = rel_l2(out, r_out), rel_l2(_state_f64(fs[slots]), r_fs)
    assert np.array_equal(cs[slots], r_cs), "conv states not bit-exact"
    snaps = _state_f64(to_host(call.snapshots))
    worst = 0.0
    for n, L in enumerate(lens):
        for j in range(1, counts[n] + 1):
            _, r_s, _ = _oracle_seq(p, xo, n, 64 * j, xo["state"][n], xo["conv_state"][n], heads=(0, p.Hv))
            worst = max(worst, rel_l2(snaps[base[n] + j - 1], r_s[0]))
    say(f"  rel_l2 out {e_out:.2e} state {e_fs:.2e} worst snapshot {worst:.2e}")
    assert e_out <= TOL_BF16 and e_fs <= TOL_BF16 and worst <= TOL_BF16
