"""GPU parity of the whole token mixer on the HIP path: kda_frontend, then kda_chunk_fwd_gated for a
prompt and kda_decode_step_gated for each further token, against the oracle's input stage,
recurrence and output stage ("Kimi K3's hybrid block, from first principles", section "From linear
attention to the delta rule": a short convolution, Swish and unit-length normalisation of q and k,
the bounded log-decay and the sigmoid beta; the recurrence; each head's output row normalised by its
root mean square and scaled by a sigmoid gate of the token).

The GPU path stores q, k, v, g and beta in the call's dtype between the input stage and the
recurrence.  The reference chain therefore takes the oracle's float64 input stage, rounds its five
outputs to that dtype (round to nearest even, as every store of the path rounds), and runs the
oracle's recurrence and output stage in float64.  Bars: the prefill's, 2e-2 max-normalised for
bf16 and 1e-4 for float32; y is compared with every row scaled back by the reference row's RMS, the
measure of the gated-prefill tests (the output stage divides each row by its own RMS, so a small
row would otherwise carry o's absolute error magnified).

The serving case hands everything over the way a server would: the prompt's convolution state
(conv_out) and recurrent state (hT) go into the decode steps, which update both in place, one
token per sequence per step; every y of prompt and continuation is checked against one oracle run
over the whole sequences.
"""
import time

import numpy as np
import pytest
import torch

from conftest import to64

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-4}
EPS_NORM, EPS_RMS, G_MIN = 1e-6, 1e-6, -5.0


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _say(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)


def err(x, ref):
    return float(np.abs(x - ref).max() / max(np.abs(ref).max(), 1e-30))


def _as_stored(a, dt):
    """float64 values rounded to the dtype the path stores them in (bf16: nearest even)."""
    t = torch.from_numpy(np.ascontiguousarray(a))
    t = t.to(torch.bfloat16) if dt == "bf16" else t.to(torch.float32)
    return t.double().numpy()


def _oracle_layer(oracle_mod, f, z, w, h0, dt, heads):
    """The oracle's chain on the heads listed: input stage (all heads: it is cheap), the stored
    rounding, the recurrence and the output stage.  Returns (y, hT, rms of every o row)."""
    cin = None if f.conv_in is None else to64(f.conv_in)
    q, k, v, g, beta, conv = oracle_mod.frontend(
        to64(f.x_q), to64(f.x_k), to64(f.x_v), to64(f.x_z), to64(f.x_b), to64(f.w_q),
        to64(f.w_k), to64(f.w_v), to64(f.z_bias), to64(f.A), G_MIN, f.cu_seqlens.tolist(), cin,
        EPS_NORM)
    q, k, v, g, beta = (_as_stored(t[:, heads], dt) for t in (q, k, v, g, beta))
    o, hT = oracle_mod.recurrence(q, k, v, g, beta, to64(h0[:, heads]), f.cu_seqlens.tolist())
    y = oracle_mod.output_gate(o, to64(z[:, heads]), to64(w), EPS_RMS)
    rms = np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + EPS_RMS)
    return y, hT, rms, conv


def _inputs(lens, H, dt, seed):
    from linear_attention_recurrence_08_amd import inputs
    f = inputs.make_frontend_inputs(lens, H, 128, 128, dt, seed=seed, with_state=True)
    _, z, w = inputs.make_output_gate_inputs(sum(lens), H, 128, dt, seed + 1)
    g = torch.Generator().manual_seed(seed + 2)
    h0 = (0.1 * torch.randn((len(lens), H, 128, 128), generator=g)).float()
    return f, z, w, h0


# (name, prompt lengths, H, dtype): 64 heads x 4 sequences fill 256 (sequence, head) pairs, so the
# output stage runs inside the prefill kernel; the others take the prefill and the output-stage
# kernel
PROMPTS = [
    ("fused_ragged_with_empty", [70, 33, 0, 18], 64, "bf16"),
    ("unfused_bf16", [41, 16, 3], 3, "bf16"),
    ("unfused_float32", [50, 17], 2, "f32"),
]


@pytest.mark.parametrize("case", PROMPTS, ids=lambda c: c[0])
def test_layer_prefill_against_oracle(oracle_mod, case):
    from linear_attention_recurrence_08_amd import (kda_chunk_fwd_gated,
                                                    kda_chunk_fwd_gated_fuses, kda_frontend)
    dev = _dev()
    name, lens, H, dt = case
    f, z, w, h0 = _inputs(lens, H, dt, seed=sum(lens) + H)
    _say(f"layer prefill {name}: lens={lens} H={H} {dt}")
    fd = f.to(dev)
    q, k, v, g, beta, conv = kda_frontend(fd.x_q, fd.x_k, fd.x_v, fd.x_z, fd.x_b, fd.w_q, fd.w_k,
                                          fd.w_v, fd.z_bias, fd.A, G_MIN, EPS_NORM,
                                          cu_seqlens=fd.cu_seqlens, conv_in=fd.conv_in,
                                          output_conv_state=True)
    fused = kda_chunk_fwd_gated_fuses(q, len(lens), 1, H, 128, 128, True)
    assert fused == (len(lens) * H >= 256 and dt == "bf16")
    y, _, hT = kda_chunk_fwd_gated(q, k, v, g, beta, z.to(dev), weight=w.to(dev), eps=EPS_RMS,
                                   h0=h0.to(dev), cu_seqlens=fd.cu_seqlens)
    torch.cuda.synchronize()
    heads = list(range(H)) if H <= 8 else [0, 17, 40, H - 1]
    y_ref, h_ref, rms, conv_ref = _oracle_layer(oracle_mod, f, z, w, h0, dt, heads)
    yv = to64(y[:, heads])
    ey, eh = err(yv * rms, y_ref * rms), err(to64(hT[:, heads]), h_ref)
    _say(f"  fused={fused} error: y (rows at their RMS) {ey:.3e}, hT {eh:.3e} (bar {TOL[dt]})")
    assert np.isfinite(yv).all()
    assert ey <= TOL[dt] and eh <= TOL[dt], (ey, eh)
    # the saved convolution state is a copy of inputs: exact
    assert np.array_equal(to64(conv), conv_ref)


@pytest.mark.parametrize("decode", ["three_kernels", "one_kernel"])
def test_layer_prefill_then_decode_against_oracle(oracle_mod, decode):
    """A server's flow: the prompts through the input stage and the gated prefill, then five decode
    steps that take over the convolution state and the recurrent state and update both in place,
    either as kda_frontend then kda_decode_step_gated or as kda_decode_step_layer (one launch;
    its q, k, v, g and beta stay in float32, where the reference rounds them to bf16 as the other
    paths store them).  Every y of prompt and continuation against one oracle run over the whole
    sequences."""
    from linear_attention_recurrence_08_amd import (kda_chunk_fwd_gated, kda_decode_step_gated,
                                                    kda_decode_step_layer, kda_frontend)
    dev = _dev()
    prompts, steps, H, dt = [70, 33, 0, 18], 5, 64, "bf16"
    full = [p + steps for p in prompts]
    f, z, w, h0 = _inputs(full, H, dt, seed=401)
    cu = f.cu_seqlens.tolist()
    # packed row of every prompt token, and of decode step j of every sequence
    prompt_rows = np.array([cu[n] + i for n, p in enumerate(prompts) for i in range(p)])
    step_rows = [np.array([cu[n] + prompts[n] + j for n in range(len(prompts))])
                 for j in range(steps)]
    cu_p = torch.tensor(np.concatenate([[0], np.cumsum(prompts)]), dtype=torch.int32).to(dev)
    ones = torch.arange(len(prompts) + 1, dtype=torch.int32, device=dev)
    fd = f.to(dev)
    zd, wd = z.to(dev), w.to(dev)
    xs = (fd.x_q, fd.x_k, fd.x_v, fd.x_z, fd.x_b)
    taps = (fd.w_q, fd.w_k, fd.w_v, fd.z_bias, fd.A)
    _say(f"layer serve: prompts={prompts} then {steps} decode steps ({decode}), H={H} {dt}")
    pr = torch.from_numpy(prompt_rows).to(dev)
    q, k, v, g, beta, conv = kda_frontend(*(x[pr] for x in xs), *taps, G_MIN, EPS_NORM,
                                          cu_seqlens=cu_p, conv_in=fd.conv_in,
                                          output_conv_state=True)
    y_p, _, S = kda_chunk_fwd_gated(q, k, v, g, beta, zd[pr], weight=wd, eps=EPS_RMS,
                                    h0=h0.to(dev), cu_seqlens=cu_p)
    y_steps = []
    for r in step_rows:
        rd = torch.from_numpy(r).to(dev)
        if decode == "one_kernel":
            y, _ = kda_decode_step_layer(*(x[rd] for x in xs), *taps, conv, S, zd[rd], wd,
                                         g_min=G_MIN, norm_eps=EPS_NORM, eps=EPS_RMS)
        else:
            q, k, v, g, beta, _ = kda_frontend(*(x[rd] for x in xs), *taps, G_MIN, EPS_NORM,
                                               cu_seqlens=ones, conv_in=conv, conv_out=conv)
            _, y = kda_decode_step_gated(q, k, v, g, beta, S, zd[rd], wd, eps=EPS_RMS)
        y_steps.append(y)
    torch.cuda.synchronize()
    heads = [0, 21, 63]
    y_ref, h_ref, rms, conv_ref = _oracle_layer(oracle_mod, f, z, w, h0, dt, heads)
    ey_p = err(to64(y_p[:, heads]) * rms[prompt_rows], y_ref[prompt_rows] * rms[prompt_rows])
    ey_d = max(err(to64(y[:, heads]) * rms[r], y_ref[r] * rms[r])
               for r, y in zip(step_rows, y_steps))
    eh = err(to64(S[:, heads]), h_ref)
    _say(f"  error: prompt y {ey_p:.3e}, decode y {ey_d:.3e}, final state {eh:.3e}")
    assert ey_p <= TOL[dt] and ey_d <= TOL[dt] and eh <= TOL[dt], (ey_p, ey_d, eh)
    # the convolution state after the last step holds the last three inputs: exact
    assert np.array_equal(to64(conv), conv_ref)


@pytest.mark.timeout(600)
def test_layer_T4096_H96(oracle_mod):
    """The benchmark prompt (T = 4096, 96 heads, batch 1: the prefill and the output-stage kernel)
    through the whole mixer, on a sample of heads."""
    from linear_attention_recurrence_08_amd import kda_chunk_fwd_gated, kda_frontend
    dev = _dev()
    f, z, w, h0 = _inputs([4096], 96, "bf16", seed=402)
    fd = f.to(dev)
    _say("layer T=4096 H=96: GPU")
    q, k, v, g, beta, _ = kda_frontend(fd.x_q, fd.x_k, fd.x_v, fd.x_z, fd.x_b, fd.w_q, fd.w_k,
                                       fd.w_v, fd.z_bias, fd.A, G_MIN, EPS_NORM,
                                       cu_seqlens=fd.cu_seqlens, conv_in=fd.conv_in)
    y, _, hT = kda_chunk_fwd_gated(q, k, v, g, beta, z.to(dev), weight=w.to(dev), eps=EPS_RMS,
                                   h0=h0.to(dev), cu_seqlens=fd.cu_seqlens)
    torch.cuda.synchronize()
    heads = [0, 47, 95]
    y_ref, h_ref, rms, _ = _oracle_layer(oracle_mod, f, z, w, h0, "bf16", heads)
    ey, eh = err(to64(y[:, heads]) * rms, y_ref * rms), err(to64(hT[:, heads]), h_ref)
    _say(f"  heads {heads}: error y {ey:.3e}, hT {eh:.3e}")
    assert ey <= TOL["bf16"] and eh <= TOL["bf16"], (ey, eh)


# (N, H, dtype): 256 x 96 (two heads per workgroup); 3 x 3 (an odd unit count: one head per
# workgroup); float32
DECODES = [(256, 96, "bf16"), (3, 3, "bf16"), (5, 2, "f32")]


@pytest.mark.parametrize("N,H,dt", DECODES, ids=lambda c: str(c))
def test_layer_decode_step_against_oracle(oracle_mod, N, H, dt):
    """kda_decode_step_layer (the input stage, the decode step and the output stage in one launch)
    and kda_frontend followed by kda_decode_step_gated, both against the oracle's chain on the
    same token.  The two GPU paths differ by the rounding of q, k, v, g and beta to dtype between
    the two launches of the second (about 1e-2 of max |y| in bf16; the one-launch path keeps them
    in float32 and lands closer to the oracle); in float32 they agree to 1e-4."""
    from linear_attention_recurrence_08_amd import (inputs, kda_decode_step_gated,
                                                    kda_decode_step_layer, kda_frontend)
    dev = _dev()
    f = inputs.make_frontend_inputs([1] * N, H, 128, 128, dt, seed=700 + N, with_state=True)
    _, z, w = inputs.make_output_gate_inputs(N, H, 128, dt, 701 + N)
    S0 = inputs.make_decode_inputs(N, H, 128, 128, dt, seed=702 + N).h0
    fd = f.to(dev)
    zd, wd = z.to(dev), w.to(dev)
    xs = (fd.x_q, fd.x_k, fd.x_v, fd.x_z, fd.x_b)
    taps = (fd.w_q, fd.w_k, fd.w_v, fd.z_bias, fd.A)
    _say(f"layer decode N={N} H={H} {dt}")
    S1, conv1 = S0.to(dev), fd.conv_in.clone()
    y1, o1 = kda_decode_step_layer(*xs, *taps, conv1, S1, zd, wd, g_min=G_MIN,
                                   norm_eps=EPS_NORM, eps=EPS_RMS, want_o=True)
    S2, conv2 = S0.to(dev), fd.conv_in.clone()
    ones = torch.arange(N + 1, dtype=torch.int32, device=dev)
    q, k, v, g, beta, _ = kda_frontend(*xs, *taps, G_MIN, EPS_NORM, cu_seqlens=ones,
                                       conv_in=conv2, conv_out=conv2)
    o2, y2 = kda_decode_step_gated(q, k, v, g, beta, S2, zd, wd, eps=EPS_RMS)
    torch.cuda.synchronize()
    assert torch.equal(conv1, conv2), "the convolution state moves on the same way"
    # the oracle's chain in float64 on a sample of (sequence, head) units
    rng = np.random.default_rng(N)
    units = sorted(set(map(tuple, rng.integers(0, [N, H], size=(min(96, N * H), 2)).tolist())) |
                   {(N - 1, H - 1)})
    ns, hs = [u[0] for u in units], [u[1] for u in units]
    fq, fk, fv, fg, fb, conv_ref = oracle_mod.frontend(
        to64(f.x_q), to64(f.x_k), to64(f.x_v), to64(f.x_z), to64(f.x_b), to64(f.w_q),
        to64(f.w_k), to64(f.w_v), to64(f.z_bias), to64(f.A), G_MIN, f.cu_seqlens.tolist(),
        to64(f.conv_in), EPS_NORM)
    assert np.array_equal(to64(conv1), conv_ref)
    sel = lambda a: a[ns, hs][:, None]
    o_ref, S_ref = oracle_mod.decode_step(sel(fq), sel(fk), sel(fv), sel(fg), fb[ns, hs][:, None],
                                          to64(S0[ns, hs])[:, None])
    y_ref = oracle_mod.output_gate(o_ref[:, 0], to64(z[ns, hs]), to64(w), EPS_RMS)
    eo = err(to64(o1[ns, hs]), o_ref[:, 0])
    ey = err(to64(y1[ns, hs]), y_ref)
    es = err(to64(S1[ns, hs]), S_ref[:, 0])
    eo2, ey2 = err(to64(o2[ns, hs]), o_ref[:, 0]), err(to64(y2[ns, hs]), y_ref)
    es2 = err(to64(S2[ns, hs]), S_ref[:, 0])
    d = err(to64(y1), to64(y2))
    _say(f"  one launch: error o={eo:.3e} y={ey:.3e} S={es:.3e}; three launches: o={eo2:.3e} "
         f"y={ey2:.3e} S={es2:.3e}; between them {d:.3e}")
    assert eo <= TOL[dt] and ey <= TOL[dt] and es <= TOL[dt], (eo, ey, es)
    assert eo2 <= TOL[dt] and ey2 <= TOL[dt] and es2 <= TOL[dt], (eo2, ey2, es2)
    if dt == "f32":
        assert d <= 1e-4, d


def test_layer_decode_step_y_aliases_gate():
    """kda_decode_step_layer may write y over the gate (each element is read before it is
    overwritten) and over o; the results are those of separate buffers."""
    from linear_attention_recurrence_08_amd import inputs, kda_decode_step_layer
    dev = _dev()
    N, H = 6, 32
    f = inputs.make_frontend_inputs([1] * N, H, 128, 128, "bf16", seed=710,
                                    with_state=True).to(dev)
    _, z, w = (t.to(dev) for t in inputs.make_output_gate_inputs(N, H, 128, "bf16", 711))
    S0 = inputs.make_decode_inputs(N, H, 128, 128, "bf16", seed=712).h0.to(dev)
    args = (f.x_q, f.x_k, f.x_v, f.x_z, f.x_b, f.w_q, f.w_k, f.w_v, f.z_bias, f.A)
    S1, c1 = S0.clone(), f.conv_in.clone()
    y_sep, o_sep = kda_decode_step_layer(*args, c1, S1, z, w, want_o=True)
    S2, c2, z2 = S0.clone(), f.conv_in.clone(), z.clone()
    y_al, _ = kda_decode_step_layer(*args, c2, S2, z2, w, y=z2)
    S3, c3, z3 = S0.clone(), f.conv_in.clone(), z.clone()
    o3 = torch.empty_like(z)
    y_o, o_o = kda_decode_step_layer(*args, c3, S3, z3, w, o=o3, y=o3)
    torch.cuda.synchronize()
    assert y_al.data_ptr() == z2.data_ptr() and torch.equal(y_al, y_sep)
    assert y_o.data_ptr() == o3.data_ptr() and torch.equal(y_o, y_sep)
    assert torch.equal(S1, S2) and torch.equal(S1, S3) and torch.equal(c1, c2)
