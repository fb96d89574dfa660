"""GPU parity at the largest sizes the library takes, on every entry point.

* The widest token rows: H * max(dk, dv) = 2^20 (8,192 heads of 128 values), the limit the C ABI
  states.  Prefill (two packed sequences: one full tile and a ragged one), decode, the output
  stage and the input stage; the first, middle and last heads against the oracle.
* Tensors past 4 GiB: 180,007 tokens x 96 heads x 128 values in bf16 is 4.4 GB per tensor, so
  byte offsets into q, k, v, g and o pass 2^32 after token 174,762.
  * Prefill on both kernels: one sequence (96 pairs: two workgroups per head), and three packed
    sequences (288 pairs: one workgroup per head, with the output stage fused into it).
  * The output stage and the input stage over the same token count.
  * A decode step over 4.4 GB of states (700 sequences).
  Every token of the checked heads goes to the oracle, so the rows past the 4 GiB mark are
  among them.

The inputs are drawn on the device from a seeded generator, with the recipes of the benchmark
configurations: q and k L2-normalised rows, v ~ N(0, 1), g = -5 sigmoid(N(0, 1)),
beta = sigmoid(N(0, 1)), states ~ N(0, 0.05).  Host copies of these sizes would take minutes to
draw.  The oracle receives the same values, copied back for the heads it checks.  Bars as in the
other parity tests: 2e-2 max-normalised for bf16 prefill and decode outputs and final states,
1e-2 for the output and input stages (one bf16 rounding), and 1e-2 between the fused and
unfused output stage.
"""
import time

import numpy as np
import pytest
import torch

from conftest import to64

pytestmark = pytest.mark.gpu

TOL = 2e-2           # prefill and decode, bf16 inputs
STAGE_TOL = 1e-2     # the output and input stages: one bf16 rounding of each result
WIDE_H = 8192        # H * 128 = 2^20
BIG_T = 180_007      # 180,007 x 96 x 128 x 2 B = 4.42e9 B > 2^32
BIG_H = 96


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _say(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)


def err(x, ref):
    return float(np.abs(x - ref).max() / max(np.abs(ref).max(), 1e-30))


def _draw(shape, gen, kind, dev, dtype=torch.bfloat16):
    """A tensor of the given recipe, drawn in slices of the leading axis (bounded temporaries)."""
    out = torch.empty(shape, dtype=dtype, device=dev)
    inner = int(np.prod(shape[1:])) if len(shape) > 1 else 1
    step = max(1, (1 << 26) // inner)
    for a in range(0, shape[0], step):
        b = min(shape[0], a + step)
        x = torch.randn((b - a, *shape[1:]), generator=gen, device=dev, dtype=torch.float32)
        if kind == "unit":
            x = x / x.norm(dim=-1, keepdim=True)
        elif kind == "gate":
            x = -5.0 * torch.sigmoid(x)
        elif kind == "sigmoid":
            x = torch.sigmoid(x)
        elif kind == "state":
            x = 0.05 * x
        out[a:b] = x.to(dtype)
    return out


def _prefill_inputs(Ttot, H, N, seed, dev):
    gen = torch.Generator(device=dev).manual_seed(seed)
    q = _draw((Ttot, H, 128), gen, "unit", dev)
    k = _draw((Ttot, H, 128), gen, "unit", dev)
    v = _draw((Ttot, H, 128), gen, "normal", dev)
    g = _draw((Ttot, H, 128), gen, "gate", dev)
    beta = _draw((Ttot, H), gen, "sigmoid", dev)
    h0 = _draw((N, H, 128, 128), gen, "state", dev, torch.float32)
    return q, k, v, g, beta, h0


def _oracle_heads(oracle_mod, q, k, v, g, beta, h0, cu, heads):
    sel = lambda t: to64(t[:, heads])
    return oracle_mod.recurrence(sel(q), sel(k), sel(v), sel(g), sel(beta), sel(h0), cu)


def _check_prefill(oracle_mod, o, hT, ins, cu, heads, label):
    t0 = time.time()
    o_ref, h_ref = _oracle_heads(oracle_mod, *ins, cu, heads)
    og, hg = to64(o[:, heads]), to64(hT[:, heads])
    eo, eh = err(og, o_ref), err(hg, h_ref)
    _say(f"{label}: heads {heads}, error o={eo:.3e} hT={eh:.3e} "
         f"(oracle {time.time() - t0:.1f} s)")
    assert np.isfinite(og).all() and np.isfinite(hg).all()
    assert eo <= TOL and eh <= TOL, (eo, eh)


# ------------------------------------------------------------------------------------------------
# the widest rows the ABI takes: 8,192 heads of 128
# ------------------------------------------------------------------------------------------------
@pytest.mark.timeout(600)
def test_widest_rows_prefill_decode_output_stage(oracle_mod):
    from linear_attention_recurrence_08_amd import (kda_chunk_fwd, kda_decode_step,
                                                    kda_output_gate)
    dev = _dev()
    lens = [20, 7]
    cu = np.concatenate([[0], np.cumsum(lens)]).tolist()
    ins = _prefill_inputs(sum(lens), WIDE_H, len(lens), 501, dev)
    _say(f"widest rows: prefill lens={lens} H={WIDE_H}")
    cud = torch.tensor(cu, dtype=torch.int32, device=dev)
    o, hT = kda_chunk_fwd(*ins[:5], h0=ins[5], cu_seqlens=cud)
    torch.cuda.synchronize()
    heads = [0, 1, WIDE_H // 2, WIDE_H - 2, WIDE_H - 1]
    _check_prefill(oracle_mod, o, hT, ins, cu, heads, "widest rows prefill")

    # decode: three sequences, one token each, states updated in place
    gen = torch.Generator(device=dev).manual_seed(502)
    qd = _draw((3, WIDE_H, 128), gen, "unit", dev)
    kd = _draw((3, WIDE_H, 128), gen, "unit", dev)
    vd = _draw((3, WIDE_H, 128), gen, "normal", dev)
    gd = _draw((3, WIDE_H, 128), gen, "gate", dev)
    bd = _draw((3, WIDE_H), gen, "sigmoid", dev)
    S = _draw((3, WIDE_H, 128, 128), gen, "state", dev, torch.float32)
    sel = lambda t: to64(t[:, heads])
    S_in = sel(S)
    od = kda_decode_step(qd, kd, vd, gd, bd, S)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_mod.decode_step(sel(qd), sel(kd), sel(vd), sel(gd), sel(bd), S_in)
    eo, es = err(sel(od), o_ref), err(sel(S), S_ref)
    _say(f"widest rows decode: error o={eo:.3e} S={es:.3e}")
    assert eo <= TOL and es <= TOL, (eo, es)
    del S

    # the output stage on the prefill's o
    z = _draw(tuple(o.shape), gen, "normal", dev)
    w = (1.0 + 0.1 * torch.randn(128, generator=gen, device=dev)).float()
    y = kda_output_gate(o, z, w, 1e-6)
    torch.cuda.synchronize()
    y_ref = oracle_mod.output_gate(sel(o), sel(z), to64(w), 1e-6)
    ey = err(sel(y), y_ref)
    _say(f"widest rows output stage: error {ey:.3e}")
    assert ey <= STAGE_TOL, ey


def _front_weights(H, gen, dev):
    u = lambda *shape: (torch.rand(shape, generator=gen, device=dev) - 0.5).float()
    return (u(H * 128, 4), u(H * 128, 4), u(H * 128, 4),
            (0.5 * torch.randn(H * 128, generator=gen, device=dev)).float(),
            (0.5 + 1.5 * torch.rand(H, generator=gen, device=dev)).float())


def _check_frontend(oracle_mod, xs, taps, conv_in, cu, out, heads, label):
    """The oracle's input stage on the listed heads (each head's channels are independent of the
    others' except through its own L2 norm, so a subset of heads is exact)."""
    H = xs[0].shape[1]
    ch = torch.tensor([h * 128 + c for h in heads for c in range(128)], device=xs[0].device)
    x_q, x_k, x_v, x_z, x_b = (to64(x[:, heads]) for x in xs)
    w_q, w_k, w_v, zb = (to64(t[ch]) for t in taps[:4])
    A = to64(taps[4][heads])
    cin = None
    if conv_in is not None:
        cols = torch.cat([ch, H * 128 + ch, 2 * H * 128 + ch])
        cin = to64(conv_in[:, :, cols])
    t0 = time.time()
    ref = oracle_mod.frontend(x_q, x_k, x_v, x_z, x_b, w_q, w_k, w_v, zb, A, -5.0, cu, cin, 1e-6)
    errs = [err(to64(t[:, heads]), r) for t, r in zip(out[:5], ref[:5])]
    _say(f"{label}: heads {heads}, error q/k/v/g/beta " + " ".join(f"{e:.2e}" for e in errs) +
         f" (oracle {time.time() - t0:.1f} s)")
    assert all(e <= STAGE_TOL for e in errs), errs
    if out[5] is not None:
        cols = torch.cat([ch, H * 128 + ch, 2 * H * 128 + ch])
        assert np.array_equal(to64(out[5][:, :, cols]), ref[5])


@pytest.mark.timeout(600)
def test_widest_rows_input_stage(oracle_mod):
    from linear_attention_recurrence_08_amd import kda_frontend
    dev = _dev()
    lens = [20, 7]
    cu = np.concatenate([[0], np.cumsum(lens)]).tolist()
    gen = torch.Generator(device=dev).manual_seed(503)
    xs = [_draw((sum(lens), WIDE_H, 128), gen, "normal", dev) for _ in range(4)]
    xs.append(_draw((sum(lens), WIDE_H), gen, "normal", dev))
    taps = _front_weights(WIDE_H, gen, dev)
    conv_in = _draw((len(lens), 3, WIDE_H * 384), gen, "normal", dev)
    cud = torch.tensor(cu, dtype=torch.int32, device=dev)
    _say(f"widest rows: input stage lens={lens} H={WIDE_H}")
    out = kda_frontend(*xs, *taps, -5.0, 1e-6, cu_seqlens=cud, conv_in=conv_in,
                       output_conv_state=True)
    torch.cuda.synchronize()
    _check_frontend(oracle_mod, xs, taps, conv_in, cu, out, [0, WIDE_H // 2, WIDE_H - 1],
                    "widest rows input stage")


# ------------------------------------------------------------------------------------------------
# tensors past 4 GiB
# ------------------------------------------------------------------------------------------------
@pytest.mark.timeout(900)
def test_past_4gib_prefill_one_sequence(oracle_mod):
    """One sequence of 180,007 tokens at 96 heads: two 64-column workgroups per head."""
    from linear_attention_recurrence_08_amd import kda_chunk_fwd
    dev = _dev()
    ins = _prefill_inputs(BIG_T, BIG_H, 1, 511, dev)
    assert ins[0].numel() * 2 > 2 ** 32
    _say(f"past 4 GiB: one sequence of {BIG_T} tokens, H={BIG_H}")
    q, k, v, g, beta, h0 = ins
    o, hT = kda_chunk_fwd(q[None], k[None], v[None], g[None], beta[None], h0=h0)
    torch.cuda.synchronize()
    _check_prefill(oracle_mod, o[0], hT, ins, [0, BIG_T], [0, BIG_H - 1], "past 4 GiB, B=1")


@pytest.mark.timeout(900)
def test_past_4gib_packed_prefill_fused_output_stage(oracle_mod):
    """Three packed sequences (288 pairs: one workgroup per head, longest first) with the output
    stage inside the prefill kernel, then the output-stage kernel over the same 4.4 GB rows."""
    from linear_attention_recurrence_08_amd import (kda_chunk_fwd, kda_chunk_fwd_gated,
                                                    kda_chunk_fwd_gated_fuses, kda_output_gate)
    dev = _dev()
    lens = [60_000, 100_003, 20_004]
    cu = np.concatenate([[0], np.cumsum(lens)]).tolist()
    assert cu[-1] == BIG_T
    ins = _prefill_inputs(BIG_T, BIG_H, len(lens), 512, dev)
    cud = torch.tensor(cu, dtype=torch.int32, device=dev)
    _say(f"past 4 GiB: packed lens={lens}, H={BIG_H}")
    o, hT = kda_chunk_fwd(*ins[:5], h0=ins[5], cu_seqlens=cud)
    torch.cuda.synchronize()
    heads = [3, BIG_H - 1]
    _check_prefill(oracle_mod, o, hT, ins, cu, heads, "past 4 GiB, packed")

    gen = torch.Generator(device=dev).manual_seed(513)
    z = _draw(tuple(o.shape), gen, "normal", dev)
    w = (1.0 + 0.1 * torch.randn(128, generator=gen, device=dev)).float()
    assert kda_chunk_fwd_gated_fuses(ins[0], len(lens), 1, BIG_H, 128, 128, True)
    y, _, hT2 = kda_chunk_fwd_gated(*ins[:5], z, weight=w, h0=ins[5], cu_seqlens=cud)
    torch.cuda.synchronize()
    assert torch.equal(hT2, hT)
    del hT2
    yu = kda_output_gate(o, z, w, 1e-6)
    torch.cuda.synchronize()
    d = float((y.float() - yu.float()).abs().max() / yu.float().abs().max())
    _say(f"  fused vs unfused output stage, every head: {d:.3e}")
    assert d <= STAGE_TOL, d
    # the output stage against the oracle on the last 4,096 rows of the checked heads (past the
    # 4 GiB mark) and the first 4,096
    rows = torch.cat([torch.arange(4096), torch.arange(BIG_T - 4096, BIG_T)]).to(dev)
    pick = lambda t: to64(t[rows][:, heads])
    y_ref = oracle_mod.output_gate(pick(o), pick(z), to64(w), 1e-6)
    ey = err(pick(yu), y_ref)
    _say(f"  output stage on rows past 4 GiB: error {ey:.3e}")
    assert ey <= STAGE_TOL, ey


@pytest.mark.timeout(900)
def test_past_4gib_input_stage(oracle_mod):
    from linear_attention_recurrence_08_amd import kda_frontend
    dev = _dev()
    lens = [60_000, 100_003, 20_004]
    cu = np.concatenate([[0], np.cumsum(lens)]).tolist()
    gen = torch.Generator(device=dev).manual_seed(514)
    xs = [_draw((BIG_T, BIG_H, 128), gen, "normal", dev) for _ in range(4)]
    xs.append(_draw((BIG_T, BIG_H), gen, "normal", dev))
    taps = _front_weights(BIG_H, gen, dev)
    cud = torch.tensor(cu, dtype=torch.int32, device=dev)
    _say(f"past 4 GiB: input stage lens={lens}, H={BIG_H}")
    out = kda_frontend(*xs, *taps, -5.0, 1e-6, cu_seqlens=cud, output_conv_state=True)
    torch.cuda.synchronize()
    _check_frontend(oracle_mod, xs, taps, None, cu, out, [0, BIG_H - 1], "past 4 GiB input stage")


@pytest.mark.timeout(600)
def test_past_4gib_decode_states(oracle_mod):
    """A decode step over 700 x 96 states of 64 KiB (4.4 GB), in place; the units with the largest
    offsets and a spread of others against the oracle."""
    from linear_attention_recurrence_08_amd import kda_decode_step
    dev = _dev()
    N = 700
    gen = torch.Generator(device=dev).manual_seed(515)
    q = _draw((N, BIG_H, 128), gen, "unit", dev)
    k = _draw((N, BIG_H, 128), gen, "unit", dev)
    v = _draw((N, BIG_H, 128), gen, "normal", dev)
    g = _draw((N, BIG_H, 128), gen, "gate", dev)
    beta = _draw((N, BIG_H), gen, "sigmoid", dev)
    S = _draw((N, BIG_H, 128, 128), gen, "state", dev, torch.float32)
    assert S.numel() * 4 > 2 ** 32
    rng = np.random.default_rng(7)
    units = sorted(set(map(tuple, rng.integers(0, [N, BIG_H], size=(48, 2)).tolist())) |
                   {(N - 1, h) for h in range(BIG_H - 16, BIG_H)} | {(0, 0)})
    ns = torch.tensor([u[0] for u in units], device=dev)
    hs = torch.tensor([u[1] for u in units], device=dev)
    sel = lambda t: to64(t[ns, hs])[:, None]
    S_in = sel(S)
    _say(f"past 4 GiB: decode N={N} H={BIG_H}, {len(units)} units checked")
    o = kda_decode_step(q, k, v, g, beta, S)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_mod.decode_step(sel(q), sel(k), sel(v), sel(g),
                                          to64(beta[ns, hs])[:, None], S_in)
    eo, es = err(sel(o), o_ref), err(sel(S), S_ref)
    _say(f"  error o={eo:.3e} S={es:.3e}")
    assert eo <= TOL and es <= TOL, (eo, es)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("N,H", [(2, WIDE_H), (700, BIG_H)], ids=["widest_rows", "past_4gib"])
def test_layer_decode_at_the_limits(oracle_mod, N, H):
    """kda_decode_step_layer (input stage, decode step and output stage in one launch) on rows of
    2^20 values, and over 4.4 GB of states; sampled heads against the oracle's chain."""
    from linear_attention_recurrence_08_amd import kda_decode_step_layer
    dev = _dev()
    gen = torch.Generator(device=dev).manual_seed(520 + N)
    xs = [_draw((N, H, 128), gen, "normal", dev) for _ in range(4)]
    xs.append(_draw((N, H), gen, "normal", dev))
    taps = _front_weights(H, gen, dev)
    conv = _draw((N, 3, H * 384), gen, "normal", dev)
    S = _draw((N, H, 128, 128), gen, "state", dev, torch.float32)
    z = _draw((N, H, 128), gen, "normal", dev)
    w = (1.0 + 0.1 * torch.randn(128, generator=gen, device=dev)).float()
    heads = [0, H // 2, H - 1]
    ch = torch.tensor([h * 128 + c for h in heads for c in range(128)], device=dev)
    cols = torch.cat([ch, H * 128 + ch, 2 * H * 128 + ch])
    conv_in, S_in = to64(conv[:, :, cols]), to64(S[:, heads])
    _say(f"layer decode at the limits: N={N} H={H} (states {S.numel() * 4 / 1e9:.2f} GB)")
    y, o = kda_decode_step_layer(*xs, *taps, conv, S, z, w, want_o=True)
    torch.cuda.synchronize()
    fq, fk, fv, fg, fb, conv_ref = oracle_mod.frontend(
        *(to64(x[:, heads]) for x in xs), *(to64(t[ch]) for t in taps[:4]),
        to64(taps[4][heads]), -5.0, list(range(N + 1)), conv_in, 1e-6)
    o_ref, S_ref = oracle_mod.decode_step(fq, fk, fv, fg, fb, S_in)
    y_ref = oracle_mod.output_gate(o_ref, to64(z[:, heads]), to64(w), 1e-6)
    eo, ey = err(to64(o[:, heads]), o_ref), err(to64(y[:, heads]), y_ref)
    es = err(to64(S[:, heads]), S_ref)
    _say(f"  error o={eo:.3e} y={ey:.3e} S={es:.3e}")
    assert eo <= TOL and ey <= TOL and es <= TOL, (eo, ey, es)
    assert np.array_equal(to64(conv[:, :, cols]), conv_ref)
