"""Pins of the fp64 oracle against facts fixed by the mathematics.

The pages print no worked numbers for the layer, so the oracle is pinned by
hand-worked examples of the definitions (tests/golden/hand_worked.json),
closed forms (pure decay, exact retrieval, one-step write), an independent
chunked formulation, library routines (numpy.convolve, scipy's logistic),
bounds and structural invariants (linearity, varlen packing, state passing,
key-head sharing).  None of these compare the oracle with itself.
"""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import expit

from oracle import oracle, chunked_ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")
_EXPR_ENV = {"log": math.log, "sqrt": math.sqrt, "exp": math.exp, "__builtins__": {}}


def _ev(x):
    return float(eval(x, _EXPR_ENV)) if isinstance(x, str) else float(x)


def _arr(a):
    return np.array([[_ev(x) for x in row] for row in a], dtype=np.float64)


def run1(q, k, v, g, beta, S0=None, *, use_l2=False, z=None, norm_w=None, conv_w=None,
         conv_state=None, cu=None, l2_eps=1e-6, norm_eps=1e-6, scale=1.0, K=4,
         Hk=1, Hv=1, heads=None):
    """Oracle on float64 arrays.  q, k: [T, Hk*dk] or [T, Hk, dk]."""
    T = q.shape[0]
    q = np.asarray(q, np.float64).reshape(T, Hk, -1)
    k = np.asarray(k, np.float64).reshape(T, Hk, -1)
    v = np.asarray(v, np.float64).reshape(T, Hv, -1)
    g = np.asarray(g, np.float64).reshape(T, Hv)
    beta = np.asarray(beta, np.float64).reshape(T, Hv)
    if z is not None:
        z = np.asarray(z, np.float64).reshape(T, Hv, -1)
    if S0 is not None:
        S0 = np.asarray(S0, np.float64)
        if S0.ndim == 2:
            S0 = S0[None, None]
    return oracle.prefill(q, k, v, g, beta, cu_seqlens=cu, z=z, conv_w=conv_w,
                          norm_w=norm_w, initial_state=S0, conv_state_in=conv_state,
                          use_l2=use_l2, scale=scale, l2_eps=l2_eps, norm_eps=norm_eps,
                          conv_kernel=K, heads=heads)


def unit_rows(rng, T, d):
    x = rng.standard_normal((T, d))
    return x / np.linalg.norm(x, axis=1, keepdims=True)


def rand_gates(rng, T, weak=False):
    sp = np.log1p(np.exp(rng.standard_normal(T)))
    g = -(0.01 if weak else 1.0) * sp
    beta = expit(rng.standard_normal(T))
    return g, beta


# --------------------------------------------------------------------------
# hand-worked examples
# --------------------------------------------------------------------------
def _golden(name):
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    return next(c for c in cases if c["name"] == name)


def test_hand_worked_recurrence():
    c = _golden("two_tokens_no_conv_no_norm")
    g = np.array([_ev(x) for x in c["g"]])
    out, fs, _ = run1(_arr(c["q"]), _arr(c["k"]), _arr(c["v"]), g, np.array(c["beta"]))
    np.testing.assert_allclose(out[:, 0, :], _arr(c["expect_out"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(fs[0, 0], _arr(c["expect_state"]), rtol=0, atol=1e-14)


def test_hand_worked_l2_and_gate():
    c = _golden("one_token_l2_and_gate")
    g = np.array([_ev(x) for x in c["g"]])
    out, fs, _ = run1(_arr(c["q"]), _arr(c["k"]), _arr(c["v"]), g, np.array(c["beta"]),
                      S0=_arr(c["S0"]), use_l2=True, l2_eps=c["l2_eps"],
                      z=_arr(c["z"]), norm_w=np.array(c["norm_w"], np.float64),
                      norm_eps=c["norm_eps"])
    np.testing.assert_allclose(out[:, 0, :], _arr(c["expect_out"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(fs[0, 0], _arr(c["expect_state"]), rtol=0, atol=1e-14)


def test_hand_worked_conv_tap_order():
    c = _golden("conv_tap_order")
    x = np.array(c["x"], np.float64)            # [T, 3] channels q | k | v
    T = x.shape[0]
    q, k, v = x[:, 0].reshape(T, 1, 1), x[:, 1].reshape(T, 1, 1), x[:, 2].reshape(T, 1, 1)
    w = np.array(c["conv_w"], np.float64)
    cs = np.array(c["conv_state"], np.float64)[None]   # [1, 3, Cch]
    y = oracle.conv_silu(q, k, v, w, conv_state_in=cs)
    pre = _arr(c["expect_pre_silu"])
    np.testing.assert_allclose(y, pre / (1.0 + np.exp(-pre)), rtol=0, atol=1e-14)
    # the conv state written back by the full oracle
    _, _, cso = oracle.prefill(q, k, v, np.zeros((T, 1)), np.zeros((T, 1)), conv_w=w,
                               conv_state_in=cs, use_l2=False)
    np.testing.assert_array_equal(cso[0], np.array(c["expect_conv_state"], np.float64))


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------
@pytest.mark.parametrize("T", [1, 7, 70])
def test_b_zero_is_pure_decay(T):
    rng = np.random.default_rng(1)
    dk, dv = 16, 12
    q, k = unit_rows(rng, T, dk), unit_rows(rng, T, dk)
    v = rng.standard_normal((T, dv))
    g, _ = rand_gates(rng, T)
    S0 = rng.standard_normal((dv, dk))
    out, fs, _ = run1(q, k, v, g, np.zeros(T), S0)
    G = np.cumsum(g)
    np.testing.assert_allclose(fs[0, 0], math.exp(G[-1]) * S0, rtol=1e-13, atol=1e-300)
    expect = np.exp(G)[:, None] * (q @ S0.T)
    np.testing.assert_allclose(out[:, 0], expect, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("m", [1, 5, 16])
def test_exact_retrieval_orthonormal_keys(m):
    """a = 1, b = 1, orthonormal keys: every stored key reads back its value."""
    rng = np.random.default_rng(2)
    dk, dv = 16, 9
    keys = np.linalg.qr(rng.standard_normal((dk, dk)))[0][:m]
    v = rng.standard_normal((m, dv))
    S0 = rng.standard_normal((dv, dk))
    q = unit_rows(rng, m, dk)
    _, fs, _ = run1(q, keys, v, np.zeros(m), np.ones(m), S0)
    S = fs[0, 0]
    np.testing.assert_allclose(keys @ S.T, v, rtol=0, atol=1e-12)
    # directions orthogonal to every key keep S0's response
    if m < dk:
        perp = np.linalg.qr(rng.standard_normal((dk, dk)))[0]
        perp = perp - (perp @ keys.T) @ keys
        np.testing.assert_allclose(S @ perp.T, S0 @ perp.T, rtol=0, atol=1e-12)


def test_one_step_write():
    """b = 1, one token, any S0 and decay: S_1 k = v."""
    rng = np.random.default_rng(3)
    dk, dv = 32, 20
    k = unit_rows(rng, 1, dk)
    q = unit_rows(rng, 1, dk)
    v = rng.standard_normal((1, dv))
    S0 = rng.standard_normal((dv, dk))
    for g in (0.0, -0.3, -5.0):
        _, fs, _ = run1(q, k, v, np.array([g]), np.ones(1), S0)
        np.testing.assert_allclose(fs[0, 0] @ k[0], v[0], rtol=0, atol=1e-13)


def test_product_form_of_the_update():
    """S_t = a S_{t-1} (I - b k k^T) + b v k^T, o_t = S_t q_t, as matrix products."""
    rng = np.random.default_rng(4)
    dk, dv, T = 8, 6, 10
    q, k = unit_rows(rng, T, dk), unit_rows(rng, T, dk)
    v = rng.standard_normal((T, dv))
    g, beta = rand_gates(rng, T)
    S = rng.standard_normal((dv, dk))
    S0 = S.copy()
    outs = []
    for t in range(T):
        a, b = math.exp(g[t]), beta[t]
        S = a * S @ (np.eye(dk) - b * np.outer(k[t], k[t])) + b * np.outer(v[t], k[t])
        outs.append(S @ q[t])
    out, fs, _ = run1(q, k, v, g, beta, S0)
    np.testing.assert_allclose(out[:, 0], np.array(outs), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(fs[0, 0], S, rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------------
# independent chunked formulation
# --------------------------------------------------------------------------
@pytest.mark.parametrize("T", [1, 63, 64, 65, 203])
@pytest.mark.parametrize("weak", [False, True])
def test_chunked_equals_sequential(T, weak):
    rng = np.random.default_rng(5 + T)
    dk, dv = 32, 24
    q, k = unit_rows(rng, T, dk), unit_rows(rng, T, dk)
    v = rng.standard_normal((T, dv))
    g, beta = rand_gates(rng, T, weak)
    S0 = rng.standard_normal((dv, dk)) * 0.1
    out, fs, _ = run1(q, k, v, g, beta, S0)
    for chunk in (8, 64):
        o_c, S_c = chunked_ref.chunked_head(q, k, v, g, beta, S0, chunk=chunk)
        scale_o = np.abs(out).max()
        np.testing.assert_allclose(o_c, out[:, 0], rtol=0, atol=1e-12 * max(1.0, scale_o))
        np.testing.assert_allclose(S_c, fs[0, 0], rtol=0, atol=1e-12 * max(1.0, np.abs(fs).max()))


def test_chunk_affine_map():
    rng = np.random.default_rng(6)
    dk, dv, T = 16, 16, 64
    q, k = unit_rows(rng, T, dk), unit_rows(rng, T, dk)
    v = rng.standard_normal((T, dv))
    g, beta = rand_gates(rng, T, weak=True)
    S0 = rng.standard_normal((dv, dk))
    _, fs, _ = run1(q, k, v, g, beta, S0)
    M, B = chunked_ref.chunk_affine_map(k, v, g, beta)
    np.testing.assert_allclose(S0 @ M + B, fs[0, 0], rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# conv against a library routine
# --------------------------------------------------------------------------
def test_conv_matches_numpy_convolve():
    rng = np.random.default_rng(7)
    Hk, Hv, dk, dv, K = 2, 4, 4, 3, 4
    lens = [0, 1, 2, 3, 9, 5]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    q = rng.standard_normal((T, Hk, dk))
    k = rng.standard_normal((T, Hk, dk))
    v = rng.standard_normal((T, Hv, dv))
    Cch = 2 * Hk * dk + Hv * dv
    w = rng.standard_normal((Cch, K))
    cs = rng.standard_normal((len(lens), K - 1, Cch))
    y = oracle.conv_silu(q, k, v, w, cu_seqlens=cu, conv_state_in=cs)
    x = np.concatenate([q.reshape(T, -1), k.reshape(T, -1), v.reshape(T, -1)], axis=1)
    for n, L in enumerate(lens):
        s = cu[n]
        for c in range(Cch):
            seq = np.concatenate([cs[n, :, c], x[s:s + L, c]])
            # full convolution with the reversed taps == causal cross-correlation
            full = np.convolve(seq, w[c][::-1], mode="valid")
            pre = full[:L]
            np.testing.assert_allclose(y[s:s + L, c], pre * expit(pre), rtol=1e-13, atol=1e-15)
    # conv state out: last K-1 raw tokens of (old state ++ sequence)
    _, _, cso = oracle.prefill(q, k, v, np.zeros((T, Hv)), np.zeros((T, Hv)), cu_seqlens=cu,
                               conv_w=w, conv_state_in=cs, use_l2=False)
    for n, L in enumerate(lens):
        seq = np.concatenate([cs[n], x[cu[n]:cu[n] + L]], axis=0)
        np.testing.assert_array_equal(cso[n], seq[-(K - 1):])


def test_conv_inside_the_layer():
    """v after conv + SiLU reaches the output: one token, S0 = 0, b = 1, q = k raw."""
    rng = np.random.default_rng(8)
    dk = dv = 8
    K = 4
    x = rng.standard_normal((1, dk))
    v = rng.standard_normal((1, dv))
    Cch = 2 * dk + dv
    w = rng.standard_normal((Cch, K))
    w[dk:2 * dk] = w[:dk]                      # same taps for the q and k channels
    cs = rng.standard_normal((1, K - 1, Cch))
    cs[0, :, dk:2 * dk] = cs[0, :, :dk]
    out, _, _ = run1(x, x, v, np.zeros(1), np.ones(1), conv_w=w, conv_state=cs, use_l2=True,
                     l2_eps=0.0)
    seqv = np.concatenate([cs[0, :, 2 * dk:], v], axis=0)          # [K, dv]
    pre = (seqv * w[2 * dk:].T).sum(0)
    np.testing.assert_allclose(out[0, 0], pre * expit(pre), rtol=1e-13, atol=1e-14)


# --------------------------------------------------------------------------
# normalisations and the output gate
# --------------------------------------------------------------------------
def test_l2_normalisation_and_scale():
    """One token from S0 = 0 with b = 1 and q = k: o = v * |x|^2 / (|x|^2 + eps) * scale."""
    rng = np.random.default_rng(9)
    dk, dv = 16, 8
    x = rng.standard_normal((1, dk)) * 3.0
    v = rng.standard_normal((1, dv))
    for eps, scale in ((1e-6, 1.0), (0.5, 1.0 / math.sqrt(dk))):
        out, _, _ = run1(x, x, v, np.zeros(1), np.ones(1), use_l2=True, l2_eps=eps, scale=scale)
        n2 = float((x ** 2).sum())
        np.testing.assert_allclose(out[0, 0], v[0] * n2 / (n2 + eps) * scale, rtol=1e-13)


def test_gate_structure():
    rng = np.random.default_rng(10)
    dk, dv, T = 16, 16, 12
    q, k = unit_rows(rng, T, dk), unit_rows(rng, T, dk)
    v = rng.standard_normal((T, dv))
    g, beta = rand_gates(rng, T)
    S0 = rng.standard_normal((dv, dk))
    z = rng.standard_normal((T, dv))
    w = 1.0 + 0.02 * rng.standard_normal(dv)
    o, _, _ = run1(q, k, v, g, beta, S0)
    out, _, _ = run1(q, k, v, g, beta, S0, z=z, norm_w=w, norm_eps=1e-6)
    o, out = o[:, 0], out[:, 0]
    # per token, out / (o * w * silu(z)) is one constant: 1 / sqrt(mean(o^2) + eps)
    ratio = out / (o * w * z * expit(z))
    np.testing.assert_allclose(ratio, ratio[:, :1] * np.ones((1, dv)), rtol=1e-11)
    np.testing.assert_allclose(ratio[:, 0], 1.0 / np.sqrt((o ** 2).mean(1) + 1e-6), rtol=1e-12)
    # scale invariance of the normalised output (eps aside)
    out2, _, _ = run1(q, k, 100.0 * v, g, beta, 100.0 * S0, z=z, norm_w=w, norm_eps=0.0)
    out1, _, _ = run1(q, k, v, g, beta, S0, z=z, norm_w=w, norm_eps=0.0)
    np.testing.assert_allclose(out2, out1, rtol=1e-11, atol=1e-13)
    # a large gate input lets o / rms through: silu(z) -> z
    zbig = np.full((T, dv), 40.0)
    out3, _, _ = run1(q, k, v, g, beta, S0, z=zbig, norm_w=np.ones(dv), norm_eps=0.0)
    rms = np.sqrt((o ** 2).mean(1, keepdims=True))
    np.testing.assert_allclose(out3[:, 0], o / rms * 40.0, rtol=1e-12)


# --------------------------------------------------------------------------
# bounds and invariants
# --------------------------------------------------------------------------
def test_frobenius_bound_and_rank():
    rng = np.random.default_rng(11)
    dk, dv, T = 16, 16, 40
    q, k = unit_rows(rng, T, dk), unit_rows(rng, T, dk)
    v = rng.standard_normal((T, dv))
    g, beta = rand_gates(rng, T, weak=True)
    S = rng.standard_normal((dv, dk))
    prev = np.linalg.norm(S)
    for t in range(T):
        _, fs, _ = run1(q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1], beta[t:t + 1], S)
        S = fs[0, 0]
        now = np.linalg.norm(S)
        assert now <= math.exp(g[t]) * prev + beta[t] * np.linalg.norm(v[t]) + 1e-12
        prev = now
    # from S0 = 0 the state after t tokens has rank <= t
    for t in (1, 3, 7):
        _, fs, _ = run1(q[:t], k[:t], v[:t], g[:t], beta[:t])
        sv = np.linalg.svd(fs[0, 0], compute_uv=False)
        assert np.all(sv[t:] < 1e-12 * sv[0])


def test_linearity_in_values_and_state():
    rng = np.random.default_rng(12)
    dk, dv, T = 16, 8, 30
    q, k = unit_rows(rng, T, dk), unit_rows(rng, T, dk)
    g, beta = rand_gates(rng, T)
    v1, v2 = rng.standard_normal((T, dv)), rng.standard_normal((T, dv))
    S1, S2 = rng.standard_normal((dv, dk)), rng.standard_normal((dv, dk))
    a, b = 0.7, -1.9
    o1, f1, _ = run1(q, k, v1, g, beta, S1)
    o2, f2, _ = run1(q, k, v2, g, beta, S2)
    o3, f3, _ = run1(q, k, a * v1 + b * v2, g, beta, a * S1 + b * S2)
    np.testing.assert_allclose(o3, a * o1 + b * o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(f3, a * f1 + b * f2, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("weak", [False, True])
def test_segment_decomposition(weak):
    """One sequence cut into three segments and recomposed from per-segment
    runs: every segment from a zero state (F_s, o'_t) and from the identity
    with v = 0 (Phi_s, r_t: the rows of the state are the basis vectors e_r,
    so dv = dk), then X_0 = S0, X_{s+1} = F_s + X_s Phi_s and o_t = o'_t +
    X_s r_t give the whole run's outputs and final state.  The update is
    linear in the state (Gated DeltaNet paragraph of the hyper.ai story), and
    this is the form the segment-parallel prefill computes."""
    rng = np.random.default_rng(31 + weak)
    d, T = 16, 90
    bounds = [0, 30, 55, 90]
    q, k = unit_rows(rng, T, d), unit_rows(rng, T, d)
    g, beta = rand_gates(rng, T, weak)
    v = rng.standard_normal((T, d))
    S0 = 0.5 * rng.standard_normal((d, d))
    o_all, f_all, _ = run1(q, k, v, g, beta, S0)
    X, outs, part = S0, [], []
    for s in range(3):
        sl = slice(bounds[s], bounds[s + 1])
        n = bounds[s + 1] - bounds[s]
        o_z, F, _ = run1(q[sl], k[sl], v[sl], g[sl], beta[sl], np.zeros((d, d)))
        r, Phi, _ = run1(q[sl], k[sl], np.zeros((n, d)), g[sl], beta[sl], np.eye(d))
        corr = r.reshape(n, d) @ X.T
        part.append(np.linalg.norm(corr) / np.linalg.norm(o_z))
        outs.append(o_z.reshape(n, d) + corr)
        X = F.reshape(d, d) + X @ Phi.reshape(d, d)
    np.testing.assert_allclose(np.concatenate(outs), o_all.reshape(T, d), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(X, f_all.reshape(d, d), rtol=1e-10, atol=1e-12)
    # the start state's part is not negligible here (a dropped X_s r_t term fails)
    assert min(part) > 1e-3, part


def _rand_layer(rng, T, Hk, Hv, dk, dv, K=4):
    Cch = 2 * Hk * dk + Hv * dv
    return dict(q=rng.standard_normal((T, Hk, dk)), k=rng.standard_normal((T, Hk, dk)),
                v=rng.standard_normal((T, Hv, dv)), z=rng.standard_normal((T, Hv, dv)),
                g=-np.log1p(np.exp(rng.standard_normal((T, Hv)))) * 0.3,
                beta=expit(rng.standard_normal((T, Hv))),
                conv_w=rng.standard_normal((Cch, K)) * 0.5,
                norm_w=1.0 + 0.02 * rng.standard_normal(dv))


def _call(L, sl, cu=None, S0=None, cs=None, heads=None):
    return oracle.prefill(L["q"][sl], L["k"][sl], L["v"][sl], L["g"][sl], L["beta"][sl],
                          cu_seqlens=cu, z=L["z"][sl], conv_w=L["conv_w"], norm_w=L["norm_w"],
                          initial_state=S0, conv_state_in=cs, heads=heads)


def test_varlen_packing_equals_separate_sequences():
    rng = np.random.default_rng(13)
    Hk, Hv, dk, dv = 2, 4, 8, 8
    lens = [5, 0, 1, 70, 2]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    L = _rand_layer(rng, int(cu[-1]), Hk, Hv, dk, dv)
    N = len(lens)
    S0 = rng.standard_normal((N, Hv, dv, dk)) * 0.1
    cs = rng.standard_normal((N, 3, 2 * Hk * dk + Hv * dv))
    out, fs, cso = _call(L, slice(None), cu=cu, S0=S0, cs=cs)
    for n in range(N):
        sl = slice(int(cu[n]), int(cu[n + 1]))
        o1, f1, c1 = _call(L, sl, S0=S0[n:n + 1], cs=cs[n:n + 1])
        np.testing.assert_array_equal(out[sl], o1)
        np.testing.assert_array_equal(fs[n], f1[0])
        np.testing.assert_array_equal(cso[n], c1[0])
    # an empty sequence passes its states through
    np.testing.assert_array_equal(fs[1], S0[1])
    np.testing.assert_array_equal(cso[1], cs[1])


def test_split_prefill_and_decode_steps_equal_whole():
    rng = np.random.default_rng(14)
    Hk, Hv, dk, dv = 1, 2, 8, 8
    T = 23
    L = _rand_layer(rng, T, Hk, Hv, dk, dv)
    S0 = rng.standard_normal((1, Hv, dv, dk)) * 0.1
    cs = rng.standard_normal((1, 3, 2 * Hk * dk + Hv * dv))
    out, fs, cso = _call(L, slice(None), S0=S0, cs=cs)
    for cut in (1, 2, 10):
        oa, fa, ca = _call(L, slice(0, cut), S0=S0, cs=cs)
        ob, fb, cb = _call(L, slice(cut, T), S0=fa, cs=ca)
        np.testing.assert_allclose(np.concatenate([oa, ob]), out, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(fb, fs, rtol=1e-13, atol=1e-15)
        np.testing.assert_array_equal(cb, cso)
    S, c = S0, cs
    for t in range(T):
        ot, S, c = _call(L, slice(t, t + 1), S0=S, cs=c)
        np.testing.assert_allclose(ot[0], out[t], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(S, fs, rtol=1e-12, atol=1e-15)


def test_key_head_sharing_and_head_subset():
    """Value head h reads key head h // (Hv / Hk); a head range equals the full run's slice."""
    rng = np.random.default_rng(15)
    Hk, Hv, dk, dv, T = 2, 4, 8, 4, 19
    L = _rand_layer(rng, T, Hk, Hv, dk, dv)
    S0 = rng.standard_normal((1, Hv, dv, dk))
    out, fs, _ = _call(L, slice(None), S0=S0)
    qk = Hk * dk
    for h in range(Hv):
        hk = h // (Hv // Hk)
        w = np.concatenate([L["conv_w"][hk * dk:(hk + 1) * dk],
                            L["conv_w"][qk + hk * dk: qk + (hk + 1) * dk],
                            L["conv_w"][2 * qk + h * dv: 2 * qk + (h + 1) * dv]])
        o1, f1, _ = oracle.prefill(L["q"][:, hk:hk + 1], L["k"][:, hk:hk + 1],
                                   L["v"][:, h:h + 1], L["g"][:, h:h + 1],
                                   L["beta"][:, h:h + 1], z=L["z"][:, h:h + 1], conv_w=w,
                                   norm_w=L["norm_w"], initial_state=S0[:, h:h + 1])
        np.testing.assert_array_equal(out[:, h:h + 1], o1)
        np.testing.assert_array_equal(fs[:, h:h + 1], f1)
    o2, f2, _ = _call(L, slice(None), S0=S0, heads=(1, 3))
    np.testing.assert_array_equal(o2, out[:, 1:3])
    np.testing.assert_array_equal(f2, fs[:, 1:3])


def test_io_dtypes_widen_exactly():
    """bf16 / f32 inputs give the same result as their exact f64 widening."""
    import gdn_synth as gs
    p = gs.Problem("t", [37, 5], Hk=2, Hv=4, dk=16, dv=16, init_state_std=0.1,
                   conv_state_std=0.1, seed=3)
    x = gs.generate(p)
    out, fs, cso = oracle.run_problem(p, x)
    wide = {k: (gs.to_f64(a, gs.BF16) if isinstance(a, np.ndarray) and a.dtype == np.uint16
                else a) for k, a in x.items()}
    out2, fs2, cso2 = oracle.run_problem(p, wide)
    np.testing.assert_array_equal(out, out2)
    np.testing.assert_array_equal(fs, fs2)
    np.testing.assert_array_equal(gs.to_f64(cso, gs.BF16), cso2)
