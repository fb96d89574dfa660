"""GPU parity of kda_chunk_fwd_gated: the prefill followed by the output stage y = RMSNorm(o) *
weight * sigmoid(gate) per (token, head) row ("Kimi K3's hybrid block, from first principles",
section "From linear attention to the delta rule": each head's output row is normalised by its root
mean square and, ahead of the output projection, scaled by a sigmoid gate computed from the
token).

Two references, both float64 from the oracle (bar 2e-2 max-normalised for bf16, 1e-4 for
float32):
  * the stage: the oracle's output stage applied to the o the GPU produced;
  * end to end: the oracle's recurrence, then its output stage, with every row of both results
    multiplied back by the reference row's RMS.  The stage divides each row by its own RMS, so a
    row far smaller than max |o| carries its absolute error of o (which the prefill's own bar
    measures against max |o|) into y magnified; scaling the rows back compares y at the weight
    the prefill's bar gives o.
Both paths are covered: the output stage
inside the one-workgroup-per-head prefill kernel (bf16, 128 x 128 heads, at least 256 (sequence,
head) pairs) and the prefill followed by the output-stage kernel (everything else).  Beside the
oracle:
  * o (when asked for) and hT are bit-identical to kda_chunk_fwd's;
  * y agrees with kda_output_gate applied to kda_chunk_fwd's o: bit for bit on the unfused path,
    and to within the one extra bf16 rounding of w * sigmoid(gate) on the fused path;
  * y may alias the gate (overwritten in place) and o may be omitted.
"""
import time

import numpy as np
import pytest
import torch

from conftest import to64

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-4}
FUSED_VS_UNFUSED = 1e-2    # one bf16 rounding of w * sigmoid(gate), relative to max |y|


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _say(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)


def err(x, ref):
    return float(np.abs(x - ref).max() / max(np.abs(ref).max(), 1e-30))


def _cu(x):
    return x.cu_seqlens.tolist() if x.cu_seqlens is not None else \
        [b * x.T for b in range(x.B + 1)]


def _gate_inputs(x, seed):
    from linear_attention_recurrence_08_amd import inputs
    _, z, w = inputs.make_output_gate_inputs(x.total_tokens, x.H, x.dv, x.dtype, seed)
    return z, w     # z packed [Ttot, H, dv]


def _on_device(xd, z, dev):
    """The gate on the device, shaped like the call's v view ([B, T, H, dv] or [Ttot, H, dv])."""
    return z.to(dev).reshape(xd.call_views()[2].shape)


def _reference(oracle_mod, x, z, w, eps, heads=None):
    """The oracle's y and final state, and the RMS of every row of its o ([Ttot, H', 1])."""
    hs = slice(None) if heads is None else list(heads)
    h0 = None if x.h0 is None else to64(x.h0[:, hs])
    q, k, v, g = (to64(t.reshape(x.total_tokens, x.H, t.shape[-1])[:, hs])
                  for t in (x.q, x.k, x.v, x.g))
    beta = to64(x.beta.reshape(x.total_tokens, x.H)[:, hs])
    o_ref, h_ref = oracle_mod.recurrence(q, k, v, g, beta, h0, _cu(x))
    zr = to64(z.reshape(x.total_tokens, x.H, x.dv)[:, hs])
    y_ref = oracle_mod.output_gate(o_ref, zr, to64(w), eps)
    rms = np.sqrt(np.mean(o_ref * o_ref, axis=-1, keepdims=True) + eps)
    return y_ref, h_ref, rms


def _stage_reference(oracle_mod, o_gpu, z, w, eps, shape, heads=None):
    """The oracle's output stage on the GPU's o (as stored, in dtype)."""
    hs = slice(None) if heads is None else list(heads)
    return oracle_mod.output_gate(to64(o_gpu.reshape(shape)[:, hs]),
                                  to64(z.reshape(shape)[:, hs]), to64(w), eps)


# (name, seq_lens, H, dtype, packed, want_o, fused, gate recipe)
CASES = [
    ("fused_varlen_ragged_empty", [100, 37, 16, 0, 50], 64, "bf16", True, True, True, "sigmoid"),
    ("fused_equal_lengths_no_o", [48, 48, 48, 48], 64, "bf16", False, False, True, "sigmoid"),
    ("fused_floor_gates", [80, 33, 21, 47], 64, "bf16", True, True, True, "floor"),
    ("unfused_small_batch", [70, 33], 2, "bf16", True, True, False, "sigmoid"),
    ("unfused_no_o_in_place", [70, 33], 2, "bf16", True, False, False, "sigmoid"),
    ("unfused_float32", [70, 33], 2, "f32", True, True, False, "sigmoid"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_gated_prefill_against_oracle(oracle_mod, case):
    from linear_attention_recurrence_08_amd import (inputs, kda_chunk_fwd, kda_chunk_fwd_gated,
                                                    kda_chunk_fwd_gated_fuses, kda_output_gate)
    dev = _dev()
    name, lens, H, dt, packed, want_o, fused, gate_recipe = case
    x = inputs.make_inputs(lens, H, 128, 128, dt, seed=sum(lens) + H, gate=gate_recipe,
                           h0_sigma=0.1, packed=packed)
    z, w = _gate_inputs(x, seed=len(lens))
    eps = 1e-6
    _say(f"gated {name}: lens={lens} H={H} {dt} want_o={want_o}")
    xd = x.to(dev)
    zd, wd = _on_device(xd, z, dev), w.to(dev)
    assert kda_chunk_fwd_gated_fuses(xd.q, x.num_seqs, x.B, H, 128, 128,
                                     xd.cu_seqlens is not None) == fused
    y, o, hT = kda_chunk_fwd_gated(*xd.call_views(), zd, weight=wd, eps=eps, h0=xd.h0,
                                   cu_seqlens=xd.cu_seqlens, want_o=want_o)
    o_plain, h_plain = kda_chunk_fwd(*xd.call_views(), h0=xd.h0, cu_seqlens=xd.cu_seqlens)
    y_unfused = kda_output_gate(o_plain, zd, wd, eps)
    torch.cuda.synchronize()
    assert (o is not None) == want_o
    if want_o:
        assert torch.equal(o, o_plain), "o differs from kda_chunk_fwd's"
    assert torch.equal(hT, h_plain), "hT differs from kda_chunk_fwd's"
    yv = to64(y.reshape(x.total_tokens, H, 128))
    yu = to64(y_unfused.reshape(x.total_tokens, H, 128))
    if fused:
        d = err(yv, yu)
        _say(f"  fused vs kda_output_gate(kda_chunk_fwd): {d:.3e}")
        assert d <= FUSED_VS_UNFUSED, d
    else:
        assert np.array_equal(yv, yu), "unfused y differs from kda_output_gate(kda_chunk_fwd)"
    shape = (x.total_tokens, H, 128)
    es = err(yv, _stage_reference(oracle_mod, o_plain, z, w, eps, shape))
    y_ref, h_ref, rms = _reference(oracle_mod, x, z, w, eps)
    ey, eh = err(yv * rms, y_ref * rms), err(to64(hT), h_ref)
    _say(f"  error: stage {es:.3e}, end to end (rows at their RMS) {ey:.3e}, hT {eh:.3e} "
         f"(bar {TOL[dt]})")
    assert np.isfinite(yv).all()
    assert es <= TOL[dt] and ey <= TOL[dt] and eh <= TOL[dt], (es, ey, eh)


def test_gated_prefill_y_aliases_gate(oracle_mod):
    """y may be the gate tensor itself (each element is read before it is overwritten), on the
    fused path."""
    from linear_attention_recurrence_08_amd import inputs, kda_chunk_fwd_gated
    dev = _dev()
    x = inputs.make_inputs([64, 40, 23, 80], 64, 128, 128, "bf16", seed=5, h0_sigma=0.1)
    z, w = _gate_inputs(x, seed=9)
    xd = x.to(dev)
    zd, wd = _on_device(xd, z, dev), w.to(dev)
    y_sep, _, _ = kda_chunk_fwd_gated(*xd.call_views(), zd, weight=wd, h0=xd.h0,
                                      cu_seqlens=xd.cu_seqlens)
    zin = zd.clone()
    y_al, _, _ = kda_chunk_fwd_gated(*xd.call_views(), zin, weight=wd, h0=xd.h0,
                                     cu_seqlens=xd.cu_seqlens, y=zin)
    torch.cuda.synchronize()
    assert y_al.data_ptr() == zin.data_ptr()
    assert torch.equal(y_al, y_sep)


@pytest.mark.timeout(900)
def test_gated_prefill_varlen_16seq_H96(oracle_mod):
    """The 16-sequence variable-length batch (1,536 pairs: the fused path) against the oracle on a
    sample of heads, and against kda_output_gate(kda_chunk_fwd) on every head."""
    from linear_attention_recurrence_08_amd import (inputs, kda_chunk_fwd, kda_chunk_fwd_gated,
                                                    kda_output_gate)
    dev = _dev()
    x = inputs.make_workload("varlen_16seq_H96_d128_bf16")
    z, w = _gate_inputs(x, seed=61)
    xd = x.to(dev)
    zd, wd = _on_device(xd, z, dev), w.to(dev)
    _say(f"gated varlen: Ttot={x.total_tokens} N={x.num_seqs} H={x.H}")
    y, _, hT = kda_chunk_fwd_gated(*xd.call_views(), zd, weight=wd, h0=xd.h0,
                                   cu_seqlens=xd.cu_seqlens)
    o_plain, h_plain = kda_chunk_fwd(*xd.call_views(), h0=xd.h0, cu_seqlens=xd.cu_seqlens)
    y_unfused = kda_output_gate(o_plain, zd, wd)
    torch.cuda.synchronize()
    assert torch.equal(hT, h_plain)
    d = err(to64(y), to64(y_unfused))
    _say(f"  all heads, fused vs unfused: {d:.3e}")
    assert d <= FUSED_VS_UNFUSED, d
    heads = [0, 47, 95]
    shape = (x.total_tokens, x.H, x.dv)
    es = err(to64(y[:, heads]), _stage_reference(oracle_mod, o_plain, z, w, 1e-6, shape, heads))
    del o_plain, y_unfused
    y_ref, h_ref, rms = _reference(oracle_mod, x, z, w, 1e-6, heads=heads)
    ey = err(to64(y[:, heads]) * rms, y_ref * rms)
    eh = err(to64(hT[:, heads]), h_ref)
    _say(f"  heads {heads}: error stage {es:.3e}, end to end {ey:.3e}, hT {eh:.3e}")
    assert es <= TOL["bf16"] and ey <= TOL["bf16"] and eh <= TOL["bf16"], (es, ey, eh)
