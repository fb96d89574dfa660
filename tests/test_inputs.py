"""The seeded workload generators: deterministic, the stated shapes, value ranges and structure."""
import numpy as np
import torch

from linear_attention_recurrence_08_amd import inputs


def test_deterministic_and_thread_independent(monkeypatch):
    a = inputs.make_inputs([100, 37], H=3, dk=32, dv=16, dtype="bf16", seed=5, h0_sigma=0.02,
                           packed=True)
    monkeypatch.setattr(inputs, "_workers", lambda: 1)
    b = inputs.make_inputs([100, 37], H=3, dk=32, dv=16, dtype="bf16", seed=5, h0_sigma=0.02,
                           packed=True)
    for x, y in ((a.q, b.q), (a.k, b.k), (a.v, b.v), (a.g, b.g), (a.beta, b.beta), (a.h0, b.h0)):
        assert torch.equal(x, y)
    assert a.cu_seqlens.tolist() == [0, 100, 137]
    c = inputs.make_inputs([100, 37], H=3, dk=32, dv=16, dtype="bf16", seed=6, packed=True)
    assert not torch.equal(a.q, c.q)


def test_tiny_workload_shapes_and_ranges():
    x = inputs.make_workload("tiny_T64_H2_d32_f32")
    assert x.q.shape == (64, 2, 32) and x.v.shape == (64, 2, 32) and x.beta.shape == (64, 2)
    assert x.q.dtype == torch.float32 and x.h0 is None and x.cu_seqlens is None
    np.testing.assert_allclose(x.q.norm(dim=-1).numpy(), 1.0, atol=1e-5)
    np.testing.assert_allclose(x.k.norm(dim=-1).numpy(), 1.0, atol=1e-5)
    assert float(x.g.min()) >= -5.0 and float(x.g.max()) <= 0.0
    assert float(x.beta.min()) > 0.0 and float(x.beta.max()) < 1.0


def test_gate_recipes():
    z = np.random.default_rng(0).standard_normal((1000, 1, 128)).astype(np.float32)
    for r in inputs.GATE_RECIPES:
        g = inputs._gate(z, r)
        assert g.min() >= -5.0 and g.max() <= 0.0
    b = inputs._gate(z, "bimodal")
    assert abs(b[..., :64].mean() + 0.005) < 0.01 and abs(b[..., 64:].mean() + 4.5) < 0.01
    assert b[..., :64].max() <= 0.0  # the jitter is clamped at alpha = 1
    s1 = inputs._gate(z, "sigmoid_shift1")
    sm1 = inputs._gate(z, "sigmoid_shiftm1")
    assert s1.mean() < inputs._gate(z, "sigmoid").mean() < sm1.mean()


def test_varlen_lengths_in_range():
    lens = inputs.varlen_lengths(2)
    assert len(lens) == 16 and min(lens) >= 1024 and max(lens) <= 16384
    assert lens == inputs.varlen_lengths(2)


def test_decode_inputs_layout():
    d = inputs.make_decode_inputs(5, 3, 32, 16, "bf16", seed=1, s_sigma=0.05)
    assert d.q.shape == (5, 3, 32) and d.v.shape == (5, 3, 16) and d.beta.shape == (5, 3)
    assert d.h0.shape == (5, 3, 32, 16) and d.h0.dtype == torch.float32
    assert 0.03 < float(d.h0.std()) < 0.07


def test_floor_and_constant_beta_recipes():
    """The edge-case recipes hold exactly the values they name, in bf16 as well, and keep the
    draw order (q, k, v are the same as with the default recipes)."""
    base = inputs.make_inputs([40], H=2, dk=128, dv=128, dtype="bf16", seed=9)
    fl = inputs.make_inputs([40], H=2, dk=128, dv=128, dtype="bf16", seed=9, gate="floor",
                            beta="one")
    assert float(fl.g.float().min()) == -5.0 and float(fl.g.float().max()) == -5.0
    assert float(fl.beta.float().min()) == 1.0 and float(fl.beta.float().max()) == 1.0
    assert torch.equal(base.q, fl.q) and torch.equal(base.k, fl.k) and torch.equal(base.v, fl.v)
    half = inputs.make_inputs([40], H=2, dk=128, dv=128, dtype="bf16", seed=9, gate="floor_half",
                              beta="zero")
    g = half.g.float()
    assert float(g[..., :64].min()) == -5.0 and float(g[..., :64].max()) == -5.0
    assert float(g[..., 64:].abs().max()) == 0.0
    assert float(half.beta.float().abs().max()) == 0.0
    # a whole 16-token tile at the floor reaches the bound's edge: cumulative log-decay -80
    assert float(fl.g.float()[:16, 0, 0].sum()) == -80.0
