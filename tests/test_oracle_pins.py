"""Pins for the CPU oracle: what the pages and the mathematics fix, independent of the oracle.

Each check below is written as a function of a recurrence implementation so that the last test can
plant mistakes in copies of the oracle (on the CPU) and show that some pin catches each one.
"""
import json
import math
import os
import shutil
import subprocess
from fractions import Fraction

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand_case(rng, T, H, dk, dv, unit_keys=True, h0=True, N=1):
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    if unit_keys:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, dv))
    g = -5.0 / (1.0 + np.exp(-rng.standard_normal((T, H, dk))))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))
    S0 = rng.standard_normal((N, H, dk, dv)) if h0 else None
    return q, k, v, g, beta, S0


# --------------------------------------------------------------------------------------------
# Pin functions (each raises AssertionError on a violation)
# --------------------------------------------------------------------------------------------
def pin_unit_key_beta_one(rec):
    """Unit key and beta = 1 store v along k exactly, whatever was there and whatever the decay;
    reading with q = k returns v (decay first, then erase-and-write, then read the new state).
    Kimi K3's hybrid block -- 'From linear attention to the delta rule'."""
    rng = np.random.default_rng(11)
    T, H, dk, dv = 9, 2, 6, 5
    q, k, v, g, beta, S0 = _rand_case(rng, T, H, dk, dv)
    beta[:] = 1.0
    q = k.copy()
    o, _ = rec(q, k, v, g, beta, S0)
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-12)


def pin_unit_key_partial_beta(rec):
    """With |k| = 1 the stored value along k after one step is (1-beta) * (faded prediction) +
    beta * v: one gradient step of size beta on 1/2 |S^T k - v|^2 moves the prediction a fraction
    beta of the way to v.  Checked on the first token from a known h0 with alpha = 1 on the key's
    support so that the faded prediction is the h0 prediction.
    Kimi K3's hybrid block -- 'From linear attention to the delta rule'."""
    rng = np.random.default_rng(12)
    dk, dv = 5, 4
    S0 = rng.standard_normal((1, 1, dk, dv))
    k = np.zeros((1, 1, dk)); k[0, 0, 1] = 1.0
    v = rng.standard_normal((1, 1, dv))
    g = np.full((1, 1, dk), -0.7); g[0, 0, 1] = 0.0
    for b in (0.0, 0.25, 0.6, 1.0):
        beta = np.array([[b]])
        o, _ = rec(k.copy(), k, v, g, beta, S0)
        expect = (1 - b) * S0[0, 0, 1, :] + b * v[0, 0]
        np.testing.assert_allclose(o[0, 0], expect, rtol=0, atol=1e-13)


def pin_gradient_step(rec):
    """The write is S' - beta * grad_S' (1/2 |S'^T k - v|^2) with S' the faded state; the gradient
    is taken here by central finite differences of the loss (no closed form of the update), with
    dk != dv so a transposed state cannot pass.
    Kimi K3's hybrid block -- 'From linear attention to the delta rule'."""
    rng = np.random.default_rng(13)
    dk, dv = 4, 3
    S0 = rng.standard_normal((1, 1, dk, dv))
    k = rng.standard_normal((1, 1, dk))
    v = rng.standard_normal((1, 1, dv))
    g = -rng.uniform(0, 2, size=(1, 1, dk))
    beta = np.array([[0.37]])
    q = np.zeros((1, 1, dk))
    _, S1 = rec(q, k, v, g, beta, S0)
    # the faded state: one factor exp(g_r) per key channel, i.e. per row of S
    Sf = np.exp(g[0, 0])[:, None] * S0[0, 0]
    loss = lambda S: 0.5 * np.sum((S.T @ k[0, 0] - v[0, 0]) ** 2)
    grad = np.zeros_like(Sf)
    eps = 1e-6
    for r in range(dk):
        for c in range(dv):
            Sp, Sm = Sf.copy(), Sf.copy()
            Sp[r, c] += eps
            Sm[r, c] -= eps
            grad[r, c] = (loss(Sp) - loss(Sm)) / (2 * eps)
    np.testing.assert_allclose(S1[0, 0], Sf - 0.37 * grad, rtol=0, atol=1e-8)


def pin_pure_decay(rec):
    """beta = 0: no writes, only per-key-channel decay: S_T = Diag(exp(sum_t g_t)) h0 and every
    output reads the decayed state, o_t = S_t^T q_t.  dk != dv pins the decay to the key axis.
    Kimi K3's hybrid block -- 'From linear attention to the delta rule' (one retention factor per
    key channel)."""
    rng = np.random.default_rng(14)
    T, H, dk, dv = 13, 3, 6, 4
    q, k, v, g, beta, S0 = _rand_case(rng, T, H, dk, dv)
    beta[:] = 0.0
    o, hT = rec(q, k, v, g, beta, S0)
    G = np.cumsum(g, axis=0)  # [T, H, dk]
    for t in range(T):
        St = np.exp(G[t])[:, :, None] * S0[0]
        np.testing.assert_allclose(o[t], np.einsum("hr,hrc->hc", q[t], St), rtol=1e-12,
                                   atol=1e-12)
    np.testing.assert_allclose(hT[0], np.exp(G[-1])[:, :, None] * S0[0], rtol=1e-12, atol=0)


def pin_half_life(rec):
    """With beta = 0 and alpha = 2^(-1/m) a key channel's contents halve after exactly m tokens,
    which is the half-life n = ln 0.5 / ln alpha.
    Kimi K3's hybrid block -- 'From linear attention to the delta rule'."""
    dk, dv = 4, 2
    ms = [1, 3, 7, 69]
    T = 69
    S0 = np.ones((1, 1, dk, dv))
    g = np.zeros((T, 1, dk))
    for r, m in enumerate(ms):
        g[:, 0, r] = math.log(0.5) / m
    z = np.zeros((T, 1, dk))
    o, hT = rec(z, z, np.zeros((T, 1, dv)), g, np.zeros((T, 1)), S0)
    for r, m in enumerate(ms):
        # after m tokens the row is halved; after T tokens it is 0.5 ** (T / m)
        np.testing.assert_allclose(hT[0, 0, r], 0.5 ** (T / m), rtol=1e-12)
    # the m = 69 channel holds half of its content after 69 tokens
    np.testing.assert_allclose(hT[0, 0, 3], 0.5, rtol=1e-12)


def pin_whiteboard(rec):
    """The whiteboard worked example (golden fixture)."""
    wb = _golden("whiteboard.json")
    nrows, nlab = len(wb["rows"]), len(wb["labels"])
    for variant in ("plain", "fade"):
        toks = wb["tokens"]
        T = len(toks)
        k = np.zeros((T, 1, nrows))
        v = np.zeros((T, 1, nlab))
        alpha = np.ones((T, 1, nrows))
        beta = np.zeros((T, 1))
        for t, tok in enumerate(toks):
            k[t, 0, tok["key_row"]] = 1.0
            v[t, 0, tok["value_label"]] = 1.0
            alpha[t, 0] = tok["alpha"]
            beta[t, 0] = tok["beta"]
        expected = wb["expected_board"]
        if variant == "fade":
            alpha[-1, 0] = wb["fade_variant"]["update_alpha"]
            expected = wb["fade_variant"]["expected_board"]
        q = np.zeros((T, 1, nrows))
        q[-1, 0, wb["rows"].index("meeting_day")] = 1.0
        o, hT = rec(q, k, v, np.log(alpha), beta, None)
        np.testing.assert_allclose(hT[0, 0], np.array(expected, dtype=float), rtol=0, atol=1e-15)
        np.testing.assert_allclose(o[-1, 0], wb["expected_read_meeting_day"], rtol=0, atol=1e-15)
        # the board keeps the same number of rows: only key rows ever written are nonzero
        assert hT.shape == (1, 1, nrows, nlab)


def pin_brute_force(rec, brute):
    """General inputs (h0, two sequences, ragged) against the unrolled transition products."""
    rng = np.random.default_rng(15)
    Ttot, H, dk, dv = 11, 2, 5, 3
    q, k, v, g, beta, S0 = _rand_case(rng, Ttot, H, dk, dv, unit_keys=False, N=2)
    cu = [0, 4, 11]
    o, hT = rec(q, k, v, g, beta, S0, cu)
    ob, hb = brute(q, k, v, g, beta, S0, cu)
    np.testing.assert_allclose(o, np.array(ob, dtype=float), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(hT, np.array(hb, dtype=float), rtol=1e-11, atol=1e-11)


def pin_snapshots(rec):
    """Every saved state is the state that resumes its prefix: snapshot j of sequence n equals, bit
    for bit, the final state of a run over the first 16 j tokens of that sequence alone ("Kimi
    K3's hybrid block, from first principles", paragraph "The cache, in bytes": a prefix can be
    resumed only from a state stored at that very token).  Saving snapshots leaves o and hT
    unchanged."""
    rng = np.random.default_rng(16)
    lens = [37, 0, 32, 15, 48]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v, g, beta, _ = _rand_case(rng, int(cu[-1]), 2, 5, 4)
    S0 = rng.standard_normal((len(lens), 2, 5, 4))
    o, hT, snaps, scu = rec(q, k, v, g, beta, S0, cu, snapshot_stride=16)
    assert list(scu) == [0, 2, 2, 4, 4, 7]
    o_plain, hT_plain = rec(q, k, v, g, beta, S0, cu)
    assert np.array_equal(o, o_plain) and np.array_equal(hT, hT_plain)
    for n, L in enumerate(lens):
        for j in range(1, L // 16 + 1):
            a, e = cu[n], cu[n] + 16 * j
            _, hp = rec(q[a:e], k[a:e], v[a:e], g[a:e], beta[a:e], S0[n:n + 1])
            assert np.array_equal(snaps[scu[n] + j - 1], hp[0]), (n, j)
        if L and L % 16 == 0:
            assert np.array_equal(snaps[scu[n + 1] - 1], hT[n])


def _delta_rule_matrix_form(q, k, v, alpha, beta, S0):
    """DeltaNet / Gated DeltaNet written as explicit transition matrices, one head:
    S_t = a_t (I - b_t k_t k_t^T) S_{t-1} + b_t k_t v_t^T and o_t = S_t^T q_t, with a_t one
    scalar per token (a_t = 1 for DeltaNet).  A different formulation from the oracle's
    fade / error / write loop: the erase is an explicit dk x dk matrix and the decay multiplies
    the whole product."""
    T, dk = k.shape
    S = S0.copy()
    o = np.zeros((T, v.shape[1]))
    for t in range(T):
        E = np.eye(dk) - beta[t] * np.outer(k[t], k[t])
        S = alpha[t] * (E @ S) + beta[t] * np.outer(k[t], v[t])
        o[t] = S.T @ q[t]
    return o, S


def pin_deltanet_reduction(rec):
    """alpha = 1 (g = 0) reduces KDA to plain DeltaNet, the delta rule with no forgetting ("Kimi
    K3's hybrid block, from first principles", section "From linear attention to the delta
    rule": the delta rule alone, before any decay is added).  Compared with the matrix form
    above on general keys (not unit length) and a nonzero h0."""
    rng = np.random.default_rng(17)
    T, H, dk, dv = 12, 2, 5, 4
    q, k, v, _, beta, S0 = _rand_case(rng, T, H, dk, dv, unit_keys=False)
    g = np.zeros((T, H, dk))
    o, hT = rec(q, k, v, g, beta, S0)
    for h in range(H):
        o_ref, S_ref = _delta_rule_matrix_form(q[:, h], k[:, h], v[:, h], np.ones(T),
                                               beta[:, h], S0[0, h])
        np.testing.assert_allclose(o[:, h], o_ref, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(hT[0, h], S_ref, rtol=1e-12, atol=1e-12)


def pin_gated_deltanet_reduction(rec):
    """The same log-decay on every key channel reduces KDA to Gated DeltaNet, one decay per head
    ("Kimi K3's hybrid block, from first principles", section "From linear attention to the delta
    rule": Gated DeltaNet pairs the delta rule with a single decay per head; "Kimi K3", section
    "Forgetting different features at different rates": KDA generalises it to one factor per
    channel).  Compared with the matrix form above, where the scalar decay multiplies the
    erase-and-write product."""
    rng = np.random.default_rng(18)
    T, H, dk, dv = 12, 2, 5, 4
    q, k, v, _, beta, S0 = _rand_case(rng, T, H, dk, dv, unit_keys=False)
    gs = -rng.uniform(0.0, 3.0, size=(T, H))          # one log-decay per (token, head)
    g = np.repeat(gs[:, :, None], dk, axis=2)
    o, hT = rec(q, k, v, g, beta, S0)
    for h in range(H):
        o_ref, S_ref = _delta_rule_matrix_form(q[:, h], k[:, h], v[:, h], np.exp(gs[:, h]),
                                               beta[:, h], S0[0, h])
        np.testing.assert_allclose(o[:, h], o_ref, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(hT[0, h], S_ref, rtol=1e-12, atol=1e-12)


ALL_PINS = [pin_unit_key_beta_one, pin_unit_key_partial_beta, pin_gradient_step, pin_pure_decay,
            pin_half_life, pin_whiteboard, pin_snapshots, pin_deltanet_reduction,
            pin_gated_deltanet_reduction]


# --------------------------------------------------------------------------------------------
# Tests on the oracle itself
# --------------------------------------------------------------------------------------------
@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(oracle_mod, pin):
    pin(oracle_mod.recurrence)


def test_brute_force(oracle_mod):
    pin_brute_force(oracle_mod.recurrence, oracle_mod.brute_force)


@pytest.mark.parametrize("T,dk,dv,chunk", [(64, 32, 32, 16), (53, 32, 16, 16), (37, 8, 12, 4),
                                           (16, 16, 16, 16), (1, 8, 8, 16)])
def test_chunked_form_matches(oracle_mod, T, dk, dv, chunk):
    """The chunkwise form gives the token loop's result (the pages: handling a whole block of
    tokens together gives the same outputs as the token loop)."""
    rng = np.random.default_rng(T * 1000 + dk)
    q, k, v, g, beta, S0 = _rand_case(rng, T, 2, dk, dv)
    o, hT = oracle_mod.recurrence(q, k, v, g, beta, S0)
    oc, hc = oracle_mod.chunked(q, k, v, g, beta, S0, chunk=chunk)
    scale_o, scale_h = np.abs(o).max(), np.abs(hT).max()
    assert np.abs(o - oc).max() <= 1e-12 * scale_o
    assert np.abs(hT - hc).max() <= 1e-12 * scale_h


def test_chunk_size_invariance(oracle_mod):
    rng = np.random.default_rng(21)
    q, k, v, g, beta, S0 = _rand_case(rng, 48, 2, 8, 8)
    ref = oracle_mod.chunked(q, k, v, g, beta, S0, chunk=1)
    for C in (2, 4, 8, 16, 48):
        o, h = oracle_mod.chunked(q, k, v, g, beta, S0, chunk=C)
        assert np.abs(o - ref[0]).max() <= 1e-12 * np.abs(ref[0]).max()
        assert np.abs(h - ref[1]).max() <= 1e-12 * np.abs(ref[1]).max()


def test_varlen_isolation_bitwise(oracle_mod):
    """Packed sequences equal each sequence run alone, bit for bit; zero-length sequences give
    hT = h0."""
    rng = np.random.default_rng(22)
    lens = [5, 0, 17, 1, 9]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v, g, beta, _ = _rand_case(rng, int(cu[-1]), 3, 6, 5)
    S0 = rng.standard_normal((len(lens), 3, 6, 5))
    o, hT = oracle_mod.recurrence(q, k, v, g, beta, S0, cu)
    for n in range(len(lens)):
        a, e = cu[n], cu[n + 1]
        on, hn = oracle_mod.recurrence(q[a:e], k[a:e], v[a:e], g[a:e], beta[a:e], S0[n:n + 1])
        assert np.array_equal(on, o[a:e])
        assert np.array_equal(hn[0], hT[n])
    assert np.array_equal(hT[1], S0[1])


def test_resume_from_saved_state_bitwise(oracle_mod):
    """Running a prefix, then resuming from its final state, equals one run (a saved state is
    how a prefix is reused: What's new in Kimi K3 -- 'What it costs to serve')."""
    rng = np.random.default_rng(23)
    q, k, v, g, beta, S0 = _rand_case(rng, 40, 2, 6, 6)
    o, hT = oracle_mod.recurrence(q, k, v, g, beta, S0)
    o1, h1 = oracle_mod.recurrence(q[:17], k[:17], v[:17], g[:17], beta[:17], S0)
    o2, h2 = oracle_mod.recurrence(q[17:], k[17:], v[17:], g[17:], beta[17:], h1)
    assert np.array_equal(np.concatenate([o1, o2]), o)
    assert np.array_equal(h2, hT)


def test_affine_in_the_entering_state(oracle_mod):
    """The recurrence ("Kimi K3's hybrid block, from first principles", section "From linear
    attention to the delta rule") is affine in the state, so a run maps its entering state S to
    M S + B: a run from S_in equals its run from zero with the values (B_t, outputs B_t^T q_t)
    plus M_t S_in, where M_t is the run from the identity with v = 0 (outputs M_t^T q_t), so
    o_t = B_t^T q_t + S_in^T (M_t^T q_t).  This is what a token-range split composes."""
    rng = np.random.default_rng(29)
    T, H, dk, dv = 45, 2, 6, 5
    q, k, v, g, beta, S_in = _rand_case(rng, T, H, dk, dv)
    o, hT = oracle_mod.recurrence(q, k, v, g, beta, S_in)
    oB, B = oracle_mod.recurrence(q, k, v, g, beta, None)
    eye = np.broadcast_to(np.eye(dk), (1, H, dk, dk)).copy()
    oM, M = oracle_mod.recurrence(q, k, np.zeros((T, H, dk)), g, beta, eye)
    assert np.allclose(hT, np.einsum("nhij,nhjk->nhik", M, S_in) + B, rtol=0, atol=1e-12)
    assert np.allclose(o, oB + np.einsum("thc,hcj->thj", oM, S_in[0]), rtol=0, atol=1e-12)
    # composing two ranges: the second starts from the first's final state
    o1, h1 = oracle_mod.recurrence(q[:20], k[:20], v[:20], g[:20], beta[:20], S_in)
    oB2, B2 = oracle_mod.recurrence(q[20:], k[20:], v[20:], g[20:], beta[20:], None)
    oM2, M2 = oracle_mod.recurrence(q[20:], k[20:], np.zeros((T - 20, H, dk)), g[20:],
                                    beta[20:], eye)
    assert np.allclose(np.einsum("nhij,nhjk->nhik", M2, h1) + B2, hT, rtol=0, atol=1e-12)
    assert np.allclose(oB2 + np.einsum("thc,hcj->thj", oM2, h1[0]), o[20:], rtol=0, atol=1e-12)


def test_decode_equals_prefill_steps(oracle_mod):
    rng = np.random.default_rng(24)
    q, k, v, g, beta, S0 = _rand_case(rng, 6, 2, 5, 4)
    o, hT = oracle_mod.recurrence(q, k, v, g, beta, S0)
    S = S0
    for t in range(6):
        ot, S = oracle_mod.decode_step(q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1],
                                       beta[t:t + 1], S)
        assert np.array_equal(ot[0], o[t])
    assert np.array_equal(S, hT)


def _dyadic_case():
    """Small dyadic inputs for which every intermediate of the token loop is exact in float64."""
    rng = np.random.default_rng(31)
    T, H, dk, dv = 8, 2, 4, 3
    pick = lambda vals, shape: rng.choice(np.array(vals, dtype=float), size=shape)
    q = pick([-1, -0.5, 0, 0.5, 1], (T, H, dk))
    k = pick([-1, -0.5, 0, 0.5, 1], (T, H, dk))
    v = pick([-2, -1, 0, 1, 2], (T, H, dv))
    alpha = pick([0.25, 0.5, 1.0], (T, H, dk))
    beta = pick([0.25, 0.5, 0.75, 1.0], (T, H))
    h0 = pick([-1, 0, 1], (1, H, dk, dv))
    return q, k, v, alpha, beta, h0


def test_exact_rational_tier(oracle_mod):
    """Dyadic inputs, alpha passed directly: the float64 token loop equals the exact rational
    evaluation and the exact brute-force transition products bit for bit; the float64 chunked
    form agrees to rounding."""
    q, k, v, alpha, beta, h0 = _dyadic_case()
    o, hT = oracle_mod.recurrence(q, k, v, alpha, beta, h0, gate_is_alpha=True)
    oe, he = oracle_mod.exact(q, k, v, alpha, beta, h0)
    ob, hb = oracle_mod.brute_force(q, k, v, alpha, beta, h0, gate_is_alpha=True,
                                    exact_rational=True)
    T, H, dv = o.shape
    for t in range(T):
        for h in range(H):
            assert oe[t][h] == ob[t][h]
            for c in range(dv):
                assert Fraction(float(o[t, h, c])) == oe[t][h][c], (t, h, c)
    for h in range(H):
        assert he[0][h] == hb[0][h]
        for r in range(hT.shape[2]):
            for c in range(dv):
                assert Fraction(float(hT[0, h, r, c])) == he[0][h][r][c]
    oc, hc = oracle_mod.chunked(q, k, v, alpha, beta, h0, chunk=4, gate_is_alpha=True)
    assert np.abs(oc - o).max() <= 1e-13 * np.abs(o).max()
    assert np.abs(hc - hT).max() <= 1e-13 * np.abs(hT).max()


def test_range_facts_and_page_numbers():
    """The numbers the pages print, checked from their definitions."""
    pn = _golden("page_numbers.json")
    floor = pn["log_decay_floor"]["value"]
    assert math.exp(floor) == pytest.approx(pn["retention_floor"]["value"],
                                            rel=pn["retention_floor"]["rel_tol"])
    C = pn["tile_tokens"]["value"]
    lo, hi = pn["tile_cumulative_log_decay_open_interval"]["value"]
    # worst case over one tile: every step at the floor -> C * floor, which must be >= lo
    assert C * floor >= lo and C * floor < hi
    # and its exponentials stay finite and nonzero in float32 (the kernel's precision)
    assert np.isfinite(np.float32(np.exp(np.float32(-C * floor))))
    assert np.float32(np.exp(np.float32(C * floor))) > 0
    hl = pn["half_life_alpha_0_99"]
    assert math.log(0.5) / math.log(hl["alpha"]) == pytest.approx(hl["tokens"], abs=hl["abs_tol"])
    sp = pn["state_numbers_per_layer"]
    assert sp["head_dim"] ** 2 * sp["heads"] == sp["value"]
    ss = pn["state_numbers_per_sequence"]
    assert sp["value"] * ss["kda_layers"] == ss["value"]
    mib = ss["value"] * 4 / 2 ** 20
    assert mib == pytest.approx(pn["state_mib_fp32_per_sequence"]["value"],
                                abs=pn["state_mib_fp32_per_sequence"]["abs_tol"])
    sn = pn["snapshot_break_even_tokens"]
    assert 128 * 128 * 2 == sn["state_bytes_bf16"] and 2 * 128 * 2 == sn["kv_bytes_per_token"]
    assert sn["state_bytes_bf16"] // sn["kv_bytes_per_token"] == sn["value"]


def test_dyadic_case_is_nontrivial():
    q, k, v, alpha, beta, h0 = _dyadic_case()
    assert (alpha < 1).any() and (beta < 1).any() and np.abs(h0).sum() > 0


# --------------------------------------------------------------------------------------------
# Planted mistakes: each variant of the C oracle must fail at least one pin
# --------------------------------------------------------------------------------------------
READ_BLOCK = ("        for (int64_t c = 0; c < dv; ++c) ot[c] = 0.0;\n"
              "        for (int64_t r = 0; r < dk; ++r)\n"
              "            for (int64_t c = 0; c < dv; ++c) ot[c] += S[r * dv + c] * qt[r];\n")
WRITE_ANCHOR = "        /* erase-and-write: S <- S + k u^T */\n"


def _swap(old, new):
    def f(src):
        assert old in src, f"mutation anchor missing: {old!r}"
        return src.replace(old, new)
    return f


def _read_before_write(src):
    assert READ_BLOCK in src and WRITE_ANCHOR in src
    src = src.replace(READ_BLOCK, "")
    return src.replace(WRITE_ANCHOR, READ_BLOCK + WRITE_ANCHOR)


def _decay_after_write(src):
    """Fade the state after the erase-and-write instead of before it: S <- Diag(a) (S + k u^T)
    with u computed from the unfaded state."""
    fade = ("        for (int64_t r = 0; r < dk; ++r) {\n"
            "            a[r] = J->gate_is_alpha ? gt[r] : exp(gt[r]);\n"
            "            for (int64_t c = 0; c < dv; ++c) S[r * dv + c] *= a[r];\n"
            "        }\n")
    assert fade in src and READ_BLOCK in src
    src = src.replace(fade, "")
    return src.replace(READ_BLOCK, fade + READ_BLOCK)


MUTANTS = {
    "error_sign": _swap("u[c] = bt * (vt[c] - pred[c]);", "u[c] = bt * (vt[c] + pred[c]);"),
    "beta_dropped": _swap("u[c] = bt * (vt[c] - pred[c]);", "u[c] = (vt[c] - pred[c]);"),
    "no_decay": _swap("a[r] = J->gate_is_alpha ? gt[r] : exp(gt[r]);", "a[r] = 1.0;"),
    "decay_on_value_axis": _swap(
        "for (int64_t c = 0; c < dv; ++c) S[r * dv + c] *= a[r];",
        "for (int64_t c = 0; c < dv; ++c) S[r * dv + c] *= "
        "(J->gate_is_alpha ? gt[c % dk] : exp(gt[c % dk]));"),
    "read_with_key": _swap("ot[c] += S[r * dv + c] * qt[r];", "ot[c] += S[r * dv + c] * kt[r];"),
    "write_along_query": _swap("S[r * dv + c] += kt[r] * u[c];", "S[r * dv + c] += qt[r] * u[c];"),
    "h0_ignored": _swap("S[i] = h0 ? h0[i] : 0.0;", "S[i] = 0.0;"),
    "read_before_write": _read_before_write,
    "decay_after_write": _decay_after_write,
    # snapshot bookkeeping (in-bounds for the pin's lengths)
    "snapshot_one_token_early": _swap("const int64_t done = t - J->cu[n] + 1;",
                                      "const int64_t done = t - J->cu[n] + 2;"),
    "snapshot_wrong_sequence": _swap("(J->snap_cu[n] + done / J->stride - 1)",
                                     "(J->snap_cu[0] + done / J->stride - 1)"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(oracle_mod, tmp_path, name):
    if shutil.which("gcc") is None:
        pytest.skip("no host compiler")
    src = open(os.path.join(os.path.dirname(oracle_mod.__file__), "kda_oracle.c")).read()
    src = MUTANTS[name](src)
    cfile = tmp_path / "mut.c"
    cfile.write_text(src)
    so = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", str(cfile), "-o",
                    str(so), "-lm"], check=True)
    lib = oracle_mod.kda_oracle.load_library(str(so))
    rec = lambda *a, **kw: oracle_mod.recurrence(*a, lib=lib, **kw)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(rec)
        except AssertionError:
            caught.append(pin.__name__)
    try:
        pin_brute_force(rec, oracle_mod.brute_force)
    except AssertionError:
        caught.append("pin_brute_force")
    assert caught, f"mutant {name} passed every pin"


# Mutants each reduction pin must catch on its own (a pin that passes a wrong recurrence pins
# nothing): with alpha = 1 every mistake in the delta term shows; with one decay per head the
# decay's presence and its place before the write show as well.
REDUCTION_CATCHES = {
    "pin_deltanet_reduction": ["error_sign", "beta_dropped", "read_with_key", "write_along_query",
                               "h0_ignored", "read_before_write"],
    "pin_gated_deltanet_reduction": ["error_sign", "beta_dropped", "read_with_key",
                                     "write_along_query", "h0_ignored", "read_before_write",
                                     "no_decay", "decay_after_write"],
}


@pytest.mark.parametrize("pin_name", sorted(REDUCTION_CATCHES))
def test_reduction_pin_catches_mutants(oracle_mod, tmp_path, pin_name):
    if shutil.which("gcc") is None:
        pytest.skip("no host compiler")
    pin = globals()[pin_name]
    base = open(os.path.join(os.path.dirname(oracle_mod.__file__), "kda_oracle.c")).read()
    for name in REDUCTION_CATCHES[pin_name]:
        cfile = tmp_path / f"{name}.c"
        cfile.write_text(MUTANTS[name](base))
        so = tmp_path / f"lib{name}.so"
        subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", str(cfile),
                        "-o", str(so), "-lm"], check=True)
        lib = oracle_mod.kda_oracle.load_library(str(so))
        rec = lambda *a, **kw: oracle_mod.recurrence(*a, lib=lib, **kw)
        with pytest.raises(AssertionError):
            pin(rec)
