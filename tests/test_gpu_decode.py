"""GPU parity of gdn_decode against the fp64 oracle (through the C ABI)."""
import numpy as np
import pytest

import gdn_synth as gs
from helpers import TOL_BF16, io_to_f64, rel_l2, say
from oracle import oracle

pytestmark = pytest.mark.gpu


def run_decode(p, x, slots=None, pool=None):
    import torch
    from gated_deltanet_layer_02_amd.tensors import DecodeCall, to_host
    xx = dict(x)
    n_slots = p.N
    if slots is not None:
        # scatter the per-sequence states into a larger pool at the given rows
        n_slots = pool
        st = x["state"]
        cs = x["conv_state"]
        big = np.zeros((pool,) + st.shape[1:], dtype=st.dtype)
        bigc = np.zeros((pool,) + cs.shape[1:], dtype=cs.dtype)
        big[slots] = st
        bigc[slots] = cs
        xx["state"], xx["conv_state"] = big, bigc
    dc = DecodeCall(xx, Hk=p.Hk, Hv=p.Hv, io_bf16=p.io == gs.BF16,
                    state_bf16=p.state_dtype == gs.BF16, l2norm=p.l2norm, scale=p.scale,
                    slots=slots, num_state_slots=n_slots)
    dc.run()
    torch.cuda.synchronize()
    out = io_to_f64(to_host(dc.out))
    st = to_host(dc.state)
    cs = to_host(dc.conv_state) if dc.conv_state is not None else None
    if slots is not None:
        st, cs = st[slots], cs[slots]
    st = io_to_f64(st) if st.dtype == np.uint16 else st
    return out, st, cs


def check_decode(p, x, **kw):
    say(f"decode case: {p.name} N={p.N} Hk={p.Hk} Hv={p.Hv} state={p.state_dtype}")
    out, st, cs = run_decode(p, x, **kw)
    r_out, r_fs, r_cs = oracle.run_problem(p, x)
    e_out, e_st = rel_l2(out, r_out), rel_l2(st, r_fs)
    assert e_out <= TOL_BF16, f"out rel_l2 {e_out:.3e}"
    assert e_st <= TOL_BF16, f"state rel_l2 {e_st:.3e}"
    if r_cs is not None:
        assert np.array_equal(cs, r_cs), "conv state not bit-exact"
    return e_out, e_st


@pytest.mark.parametrize("cfg", ["C4", "C4b"])
def test_decode_configs(cfg):
    p = gs.configs()[cfg]
    e_out, e_st = check_decode(p, gs.generate(p))
    say(f"{cfg}: rel_l2 out {e_out:.2e} state {e_st:.2e}")


def test_serving_decode():
    """The serving stand-in: one decode step of 93 sequences, fp32 state."""
    p = gs.serving()["decode"]
    e_out, e_st = check_decode(p, gs.generate(p))
    say(f"serving decode: rel_l2 out {e_out:.2e} state {e_st:.2e}")


def test_serving_decode_bf16_state():
    """The same step of 93 sequences with the state stored in bf16 (the
    cookbook's --mamba-ssm-dtype option)."""
    p = gs.Problem("serving decode, 93 sequences, bf16 state", [1] * 93, state_dtype=gs.BF16,
                   init_state_std=0.01, conv_state_std=0.01, seed=2003, decode=True)
    e_out, e_st = check_decode(p, gs.generate(p))
    say(f"serving decode, bf16 state: rel_l2 out {e_out:.2e} state {e_st:.2e}")


def test_decode_state_slots():
    p = gs.Problem("slots", [1] * 5, Hk=2, Hv=4, init_state_std=0.01, conv_state_std=0.01,
                   seed=21, decode=True)
    slots = np.array([7, 0, 3, 9, 4], dtype=np.int32)
    check_decode(p, gs.generate(p), slots=slots, pool=11)


@pytest.mark.parametrize("Hk,Hv,conv,gate", [(4, 4, True, True), (1, 4, True, True),
                                             (2, 4, False, True), (2, 4, True, False)])
def test_decode_variants(Hk, Hv, conv, gate):
    p = gs.Problem(f"dec{Hk}x{Hv}{conv}{gate}", [1] * 6, Hk=Hk, Hv=Hv, conv=conv, gate=gate,
                   init_state_std=0.01, conv_state_std=0.01, seed=22, decode=True)
    check_decode(p, gs.generate(p))


# bf16 state with bf16 io and conv: each head's inputs and rows are loaded
# while the previous head is updated; one, two and four value heads per key
# head, the gate on and off, and a state pool through slots.
@pytest.mark.parametrize("Hk,Hv,gate", [(1, 4, True), (4, 4, True), (2, 4, False)])
def test_decode_bf16_state_variants(Hk, Hv, gate):
    p = gs.Problem(f"dec-bf16state-{Hk}x{Hv}{gate}", [1] * 6, Hk=Hk, Hv=Hv, gate=gate, state_dtype=gs.BF16,
                   init_state_std=0.01, conv_state_std=0.01, seed=24, decode=True)
    check_decode(p, gs.generate(p))


def test_decode_bf16_state_slots():
    p = gs.Problem("slots-bf16state", [1] * 5, Hk=2, Hv=4, state_dtype=gs.BF16, init_state_std=0.01,
                   conv_state_std=0.01, seed=25, decode=True)
    slots = np.array([6, 1, 3, 8, 0], dtype=np.int32)
    check_decode(p, gs.generate(p), slots=slots, pool=9)


def test_decode_steps_equal_prefill_on_gpu():
    """T decode steps through gdn_decode == one gdn_prefill of T tokens."""
    import torch
    from gated_deltanet_layer_02_amd.tensors import DecodeCall, PrefillCall, to_host
    T = 9
    p = gs.Problem("chain", [T], Hk=2, Hv=4, init_state_std=0.01, conv_state_std=0.01, seed=23)
    x = gs.generate(p)
    pc = PrefillCall(x, Hk=2, Hv=4, io_bf16=True)
    pc.run()
    state = x["state"].copy()
    cs = x["conv_state"].copy()
    outs = []
    for t in range(T):
        xt = {n: x[n][t:t + 1] for n in ("q", "k", "v", "z", "g", "beta")}
        xt.update(conv_w=x["conv_w"], norm_w=x["norm_w"], state=state, conv_state=cs)
        dc = DecodeCall(xt, Hk=2, Hv=4, io_bf16=True, state_bf16=False)
        dc.run()
        torch.cuda.synchronize()
        outs.append(io_to_f64(to_host(dc.out)))
        state, cs = to_host(dc.state), to_host(dc.conv_state)
    torch.cuda.synchronize()
    dec = np.concatenate(outs)
    pre = io_to_f64(to_host(pc.out))
    assert rel_l2(dec, pre) < 5e-3
    assert rel_l2(state, to_host(pc.final_state)) < 5e-3
    assert np.array_equal(cs, to_host(pc.conv_state_out))
