"""Pins of the oracle's input stage (short convolution, Swish, L2 norm, sigmoid write strength,
bounded log-decay) against what the definition fixes: the impulse response of the causal width-4
convolution, exact Swish and sigmoid values, unit-norm queries and keys, the gate's bounds and
midpoint, sequence isolation and resumption from a saved convolution state.  Planted mistakes in
the oracle's source must each fail a pin."""
import inspect
import math

import numpy as np
import pytest


def _inputs(rng, T, H, dk, dv, scale=1.0):
    r = lambda *s: rng.standard_normal(s) * scale
    return dict(x_q=r(T, H, dk), x_k=r(T, H, dk), x_v=r(T, H, dv), x_z=r(T, H, dk), x_b=r(T, H),
                w_q=r(H * dk, 4), w_k=r(H * dk, 4), w_v=r(H * dv, 4), z_bias=r(H * dk), A=r(H))


def _zeros(T, H, dk, dv):
    z = lambda *s: np.zeros(s)
    return dict(x_q=z(T, H, dk), x_k=z(T, H, dk), x_v=z(T, H, dv), x_z=z(T, H, dk), x_b=z(T, H),
                w_q=z(H * dk, 4), w_k=z(H * dk, 4), w_v=z(H * dv, 4), z_bias=z(H * dk), A=z(H))


def pin_impulse_response(fe):
    """A unit input at token 5 of value channel c appears at tokens 5..8 as Swish(w[c,3]),
    Swish(w[c,2]), Swish(w[c,1]), Swish(w[c,0]) -- and nowhere else (causal, width 4)."""
    a = _zeros(12, 1, 4, 4)
    a["w_v"] = np.array([[0.5, -1.0, 2.0, 3.0]] * 4)
    a["x_v"][5, 0, 2] = 1.0
    v = fe(**a)[2]
    sw = lambda x: x / (1.0 + math.exp(-x))
    expect = np.zeros(12)
    expect[5:9] = [sw(3.0), sw(2.0), sw(-1.0), sw(0.5)]
    assert np.allclose(v[:, 0, 2], expect, rtol=0, atol=1e-15)
    assert np.abs(np.delete(v[:, 0, :], 2, axis=1)).max() == 0.0


def pin_exact_values(fe):
    """Swish(0) = 0; sigmoid(ln 3) = 3/4, so Swish(ln 3) = (3/4) ln 3, beta(ln 3) = 3/4 and the
    log-decay at A (z + bias) = ln 3 is (3/4) g_min (reached only with the bias added); at
    A (z + bias) = 0 it is g_min / 2."""
    a = _zeros(4, 2, 4, 4)
    a["w_v"][:, 3] = math.log(3.0)
    a["x_v"][2] = 1.0
    a["x_b"][1, 1] = math.log(3.0)
    a["A"][:] = [1.0, 2.0]
    a["z_bias"][4:] = 0.3                     # head 1's channels: the bias enters the logit
    a["x_z"][3, 1, :] = math.log(3.0) / 2.0 - 0.3
    q, k, v, g, beta, _ = fe(**a)
    assert np.allclose(v[2], 0.75 * math.log(3.0), rtol=0, atol=1e-15)
    assert np.abs(v[[0, 1, 3]]).max() == 0.0
    assert abs(beta[1, 1] - 0.75) < 1e-15 and abs(beta[0, 0] - 0.5) < 1e-15
    assert np.allclose(g[3, 1], 0.75 * -5.0, rtol=0, atol=1e-14)
    assert np.allclose(g[:, 0], -2.5, rtol=0, atol=1e-15)


def pin_unit_norm_and_bounds(fe):
    rng = np.random.default_rng(3)
    a = _inputs(rng, 40, 3, 16, 8, scale=2.0)
    q, k, v, g, beta, _ = fe(**a)
    for x in (q, k):
        nrm = np.linalg.norm(x, axis=-1)
        assert np.all(np.abs(nrm - 1.0) < 1e-5)
    assert np.all(g > -5.0) and np.all(g < 0.0)
    assert np.all(beta > 0.0) and np.all(beta < 1.0)
    # A_h scales the logit: doubling A equals doubling z + bias
    b = dict(a, A=2.0 * a["A"])
    c = dict(a, x_z=2.0 * a["x_z"], z_bias=2.0 * a["z_bias"])
    assert np.allclose(fe(**b)[3], fe(**c)[3], rtol=1e-14, atol=1e-14)


def pin_sequence_isolation(fe):
    """A packed batch equals each sequence run alone (the convolution restarts at each start)."""
    rng = np.random.default_rng(4)
    lens = [5, 0, 2, 9]
    cu = np.concatenate([[0], np.cumsum(lens)])
    a = _inputs(rng, int(cu[-1]), 2, 4, 4)
    out = fe(**a, cu_seqlens=cu)
    per_tok = ("x_q", "x_k", "x_v", "x_z", "x_b")
    for n, L in enumerate(lens):
        s, e = cu[n], cu[n + 1]
        b = {key: (val[s:e] if key in per_tok else val) for key, val in a.items()}
        one = fe(**b)
        for i in range(5):
            assert np.array_equal(out[i][s:e], one[i])
        assert np.array_equal(out[5][n], one[5][0])


def pin_resume_from_state(fe):
    """Splitting a sequence and passing the saved convolution state equals one run, and the saved
    state is the last three inputs of q, k and v."""
    rng = np.random.default_rng(5)
    a = _inputs(rng, 20, 2, 4, 3)
    per_tok = ("x_q", "x_k", "x_v", "x_z", "x_b")
    full = fe(**a)
    for cut in (1, 2, 7):
        first = fe(**{key: (val[:cut] if key in per_tok else val) for key, val in a.items()})
        second = fe(**{key: (val[cut:] if key in per_tok else val) for key, val in a.items()},
                    conv_in=first[5])
        for i in range(5):
            assert np.array_equal(np.concatenate([first[i], second[i]]), full[i])
        assert np.array_equal(second[5], full[5])
    last3 = np.concatenate([a["x_q"][-3:].reshape(3, -1), a["x_k"][-3:].reshape(3, -1),
                            a["x_v"][-3:].reshape(3, -1)], axis=1)
    assert np.array_equal(full[5][0], last3)


PINS = [pin_impulse_response, pin_exact_values, pin_unit_norm_and_bounds, pin_sequence_isolation,
        pin_resume_from_state]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_frontend_pin(oracle_mod, pin):
    pin(oracle_mod.frontend)


MUTANTS = {
    "taps_reversed": ("seq[t:t + 4]", "seq[t:t + 4][::-1]"),
    "conv_crosses_sequences": ("seq = np.concatenate([state[n], rows[a:e]], axis=0)",
                               "seq = np.concatenate([rows[a - 3:a] if a >= 3 else state[n], "
                               "rows[a:e]], axis=0)"),
    "no_l2_on_keys": ("k = k / np.sqrt(np.sum(k * k, axis=-1, keepdims=True) + eps)", "k = k"),
    "swish_is_sigmoid": ("return x / (1.0 + np.exp(-x))", "return 1.0 / (1.0 + np.exp(-x))"),
    "gate_sign": ("g = g_min / (1.0 + np.exp(-zz))", "g = g_min / (1.0 + np.exp(zz))"),
    "bias_dropped": ("(x_z + z_bias.reshape(H, dk)[None])", "(x_z)"),
    "state_ignored": ("state = np.zeros((N, 3, C)) if conv_in is None else",
                      "state = np.zeros((N, 3, C)) if True else"),
    "saved_state_oldest_rows": ("conv_out[n] = seq[-3:]", "conv_out[n] = seq[:3]"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(oracle_mod, name):
    mod = oracle_mod.kda_oracle
    src = inspect.getsource(mod._swish) + "\n" + inspect.getsource(mod.frontend)
    old, new = MUTANTS[name]
    assert old in src, f"mutation anchor missing: {old!r}"
    ns = {"np": np, "math": math}
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), ns)
    caught = []
    with np.errstate(all="ignore"):
        for pin in PINS:
            try:
                pin(ns["frontend"])
            except (AssertionError, ValueError):
                caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
