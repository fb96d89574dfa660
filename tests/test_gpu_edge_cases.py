"""GPU parity at the method's edge cases, on every prefill kernel variant.

The log-decay floor: K3 bounds log alpha below by -5, so the log-decay summed over one 16-token
tile cannot fall below -80, and that bound is what keeps the chunked kernel's rescaling
factors finite ("Kimi K3's hybrid block, from first principles", section "From linear attention
to the delta rule"; "Kimi K3", section "Forgetting different features at different rates").  The
recipes "floor" (every channel at -5 for every token: whole tiles at -80) and "floor_half" (half
the key channels at -5, half at 0) drive the kernels to the largest factors they form (e^75 in
the decayed queries and keys, e^-80 on the state).

The write strength: beta = 1 with a unit key stores v along k exactly, and beta = 0 leaves pure
per-channel decay (same section).  Besides the oracle comparison, two closed forms are checked on
the GPU outputs directly: with beta = 1 and q = k every output reads back its own value, and with
beta = 0 every output is q_t^T Diag(exp(sum of g up to t)) h0.

Variants: the 64-column matrix-core kernel with stage A's and with stage
B's issue priority, the 128-column one (256 or more pairs), the float32 general kernel (bf16
forced onto it, and float32 inputs), chunk 64 on the matrix cores and in float32, and the
token-range split.
"""
import numpy as np
import pytest
import torch

from conftest import to64

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-4}


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def err(x, ref):
    return float(np.abs(x - ref).max() / max(np.abs(ref).max(), 1e-30))


# (name, seq_lens, H, dtype, packed, entry, env: {name: value})
VARIANTS = [
    ("mfma64_stageB_prio", [96, 37], 2, "bf16", True, "chunk16", None),
    ("mfma64_stageA_prio", [80], 64, "bf16", False, "chunk16", None),
    ("mfma128", [40, 37, 16, 50], 64, "bf16", True, "chunk16", None),
    ("general_bf16", [70, 33], 2, "bf16", True, "chunk16", {"KDA_FORCE_GENERAL": "1"}),
    ("general_f32", [70, 33], 2, "f32", True, "chunk16", None),
    ("chunk64_mfma", [150, 64, 21], 2, "bf16", True, "chunk64", None),
    ("chunk64_f32", [150, 64, 21], 2, "f32", True, "chunk64", None),
    ("split", [640], 2, "bf16", False, "split", None),
]


def _setenv(monkeypatch, env):
    for k, v in (env or {}).items():
        monkeypatch.setenv(k, v)


RECIPES = [("floor", "sigmoid"), ("floor_half", "sigmoid"), ("sigmoid", "one"),
           ("sigmoid", "zero"), ("floor", "one"), ("floor_half", "zero")]


def _run(entry, xd, **kw):
    from linear_attention_recurrence_08_amd import (kda_chunk_fwd, kda_chunk_fwd_chunk64,
                                                    kda_chunk_fwd_split)
    args = xd.call_views()
    if entry == "chunk16":
        return kda_chunk_fwd(*args, h0=xd.h0, cu_seqlens=xd.cu_seqlens, **kw)
    if entry == "chunk64":
        return kda_chunk_fwd_chunk64(*args, h0=xd.h0, cu_seqlens=xd.cu_seqlens, **kw)
    return kda_chunk_fwd_split(*args, h0=xd.h0, cu_seqlens=xd.cu_seqlens, segments=3, **kw)


def _inputs(lens, H, dt, packed, gate, beta, seed):
    from linear_attention_recurrence_08_amd import inputs
    return inputs.make_inputs(lens, H, 128, 128, dt, seed=seed, gate=gate, beta=beta,
                              h0_sigma=0.1, packed=packed)


def _cu(x):
    return x.cu_seqlens.tolist() if x.cu_seqlens is not None else \
        [b * x.T for b in range(x.B + 1)]


@pytest.mark.parametrize("recipe", RECIPES, ids=lambda r: f"g_{r[0]}-beta_{r[1]}")
@pytest.mark.parametrize("variant", VARIANTS, ids=lambda v: v[0])
def test_edge_against_oracle(oracle_mod, monkeypatch, variant, recipe):
    dev = _dev()
    name, lens, H, dt, packed, entry, env = variant
    _setenv(monkeypatch, env)
    x = _inputs(lens, H, dt, packed, recipe[0], recipe[1], seed=len(lens) * 7 + H)
    print(f"edge {name} g={recipe[0]} beta={recipe[1]} lens={lens} H={H} {dt}", flush=True)
    xd = x.to(dev)
    o, hT = _run(entry, xd)
    torch.cuda.synchronize()
    o = o.reshape(x.total_tokens, x.H, x.dv)
    o_ref, h_ref = oracle_mod.recurrence(to64(x.q), to64(x.k), to64(x.v), to64(x.g),
                                         to64(x.beta), to64(x.h0), _cu(x))
    eo, eh = err(to64(o), o_ref), err(to64(hT), h_ref)
    print(f"  error o={eo:.3e} hT={eh:.3e}", flush=True)
    assert np.isfinite(to64(o)).all() and np.isfinite(to64(hT)).all()
    assert eo <= TOL[dt] and eh <= TOL[dt], (eo, eh)


@pytest.mark.parametrize("gate", ["floor", "sigmoid", "zero"])
@pytest.mark.parametrize("variant", VARIANTS, ids=lambda v: v[0])
def test_unit_key_beta_one_reads_back_v(monkeypatch, variant, gate):
    """beta = 1 and a unit key replace what the state held along k with v, so reading with q = k
    returns v itself, whatever the decay and the earlier contents (closed form, no oracle).  Keys
    are unit length to bf16 rounding, so the bar is the dtype's."""
    dev = _dev()
    name, lens, H, dt, packed, entry, env = variant
    _setenv(monkeypatch, env)
    x = _inputs(lens, H, dt, packed, gate, "one", seed=11 + H)
    x.q = x.k.clone()
    xd = x.to(dev)
    o, _ = _run(entry, xd)
    torch.cuda.synchronize()
    o = to64(o.reshape(x.total_tokens, x.H, x.dv))
    e = err(o, to64(x.v))
    print(f"unit key beta=1 {name} g={gate}: max-normalised |o - v| = {e:.3e}", flush=True)
    assert e <= TOL[dt]


@pytest.mark.parametrize("gate", ["floor_half", "sigmoid_shiftm1"])
@pytest.mark.parametrize("variant", VARIANTS, ids=lambda v: v[0])
def test_beta_zero_is_pure_decay(monkeypatch, variant, gate):
    """beta = 0 writes nothing: the state only decays per key channel, S_t = Diag(exp(G_t)) h0
    with G_t the sum of g over the sequence's first t tokens, and o_t = S_t^T q_t (closed form
    in numpy, no oracle)."""
    dev = _dev()
    name, lens, H, dt, packed, entry, env = variant
    _setenv(monkeypatch, env)
    x = _inputs(lens, H, dt, packed, gate, "zero", seed=13 + H)
    xd = x.to(dev)
    o, hT = _run(entry, xd)
    torch.cuda.synchronize()
    o, hT = to64(o.reshape(x.total_tokens, x.H, x.dv)), to64(hT)
    q, g, h0 = to64(x.q), to64(x.g), to64(x.h0)
    cu = _cu(x)
    o_ref = np.zeros_like(o)
    h_ref = np.zeros_like(hT)
    for n in range(len(cu) - 1):
        a, e = cu[n], cu[n + 1]
        G = np.cumsum(g[a:e], axis=0)                              # [t, H, dk]
        o_ref[a:e] = np.einsum("thr,thr,hrc->thc", q[a:e], np.exp(G), h0[n])
        h_ref[n] = (np.exp(G[-1])[:, :, None] * h0[n]) if e > a else h0[n]
    eo, eh = err(o, o_ref), err(hT, h_ref)
    print(f"beta=0 {name} g={gate}: error o={eo:.3e} hT={eh:.3e}", flush=True)
    assert eo <= TOL[dt] and eh <= TOL[dt], (eo, eh)
