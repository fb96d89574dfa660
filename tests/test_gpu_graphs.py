"""Calls captured into HIP graphs (torch.cuda.CUDAGraph) and replayed.

The compute entry points enqueue kernels on the caller's stream and nothing else: no allocation,
no host synchronisation and no memset inside the library (the validation mode, KDA_VALIDATE, is
the exception: it copies to the host).  A caller can therefore capture the per-token step of a
decode loop, or whole prefills, once and replay them; for small decode batches the launches
otherwise cost more than the kernels.

Each graph is replayed several times with new input contents, with the program's own eager work
and synchronisations between the replays, and every replay is compared bit for bit with the same
calls run eagerly on the same inputs (the kernels are deterministic).
"""
import dataclasses
import time

import pytest
import torch

pytestmark = pytest.mark.gpu


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _say(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)


@pytest.mark.parametrize("decode", ["three_kernels", "one_kernel"])
def test_decode_token_loop_in_a_graph(decode):
    """The serving step of the token mixer for a batch of 4 sequences (the input stage with its
    convolution state updated in place, then the gated decode with the recurrent state updated in
    place; as kda_frontend and kda_decode_step_gated, or as kda_decode_step_layer), captured once
    and replayed for six tokens, against the eager loop."""
    from linear_attention_recurrence_08_amd import (inputs, kda_decode_step_gated,
                                                    kda_decode_step_layer, kda_frontend)
    dev = _dev()
    N, H, steps = 4, 96, 6
    f = inputs.make_frontend_inputs([steps] * N, H, 128, 128, "bf16", seed=601,
                                    with_state=True).to(dev)
    _, z, w = inputs.make_output_gate_inputs(N * steps, H, 128, "bf16", 602)
    z, w = z.to(dev), w.to(dev)
    S0 = inputs.make_decode_inputs(N, H, 128, 128, "bf16", seed=603).h0.to(dev)
    xs = (f.x_q, f.x_k, f.x_v, f.x_z, f.x_b)
    taps = (f.w_q, f.w_k, f.w_v, f.z_bias, f.A)
    ones = torch.arange(N + 1, dtype=torch.int32, device=dev)
    rows = [torch.tensor([n * steps + j for n in range(N)], device=dev) for j in range(steps)]

    def mixer_step(x5, zz, S, conv):
        if decode == "one_kernel":
            return kda_decode_step_layer(*x5, *taps, conv, S, zz, w)[0]
        q, k, v, g, b, _ = kda_frontend(*x5, *taps, -5.0, 1e-6, cu_seqlens=ones, conv_in=conv,
                                        conv_out=conv)
        return kda_decode_step_gated(q, k, v, g, b, S, zz, w)[1]

    # warm-up on copies of the states (loads the library outside the capture)
    mixer_step([x[rows[0]] for x in xs], z[rows[0]], S0.clone(), f.conv_in.clone())
    torch.cuda.synchronize()

    x_static = [x[rows[0]].clone() for x in xs]
    z_static = z[rows[0]].clone()
    S_g, conv_g = S0.clone(), f.conv_in.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        y_static = mixer_step(x_static, z_static, S_g, conv_g)
    # capturing runs nothing: the states are untouched
    torch.cuda.synchronize()
    assert torch.equal(S_g, S0) and torch.equal(conv_g, f.conv_in)

    S_e, conv_e = S0.clone(), f.conv_in.clone()
    for j in range(steps):
        y_e = mixer_step([x[rows[j]] for x in xs], z[rows[j]], S_e, conv_e).clone()
        torch.cuda.synchronize()
        for dst, x in zip(x_static, xs):
            dst.copy_(x[rows[j]])
        z_static.copy_(z[rows[j]])
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_static, y_e), f"token {j}: the replay differs from the eager step"
        # unrelated eager work between replays
        (torch.randn(256, 256, device=dev) @ torch.randn(256, 256, device=dev)).sum().item()
    assert torch.equal(S_g, S_e) and torch.equal(conv_g, conv_e)
    _say(f"decode loop ({decode}): {steps} replays bit-identical to the eager steps, states too")


def test_prefill_entry_points_in_a_graph():
    """One graph holding five prefills (two 64-column workgroups per head; one per head with the
    output stage fused; one per head without it, whose kernel spills registers to scratch
    memory; the token-range split in the library's static workspace) and the output-stage
    kernel, replayed three times on new inputs."""
    from linear_attention_recurrence_08_amd import (inputs, kda_chunk_fwd, kda_chunk_fwd_gated,
                                                    kda_chunk_fwd_gated_fuses,
                                                    kda_chunk_fwd_split_noalloc,
                                                    kda_output_gate)
    dev = _dev()
    sets = []
    for r in range(3):
        a = inputs.make_inputs([300], 96, 128, 128, "bf16", seed=610 + r, h0_sigma=0.1,
                               packed=False).to(dev)
        b = inputs.make_inputs([100, 37, 16, 50], 64, 128, 128, "bf16", seed=620 + r,
                               h0_sigma=0.1).to(dev)
        c = inputs.make_inputs([1024], 12, 128, 128, "bf16", seed=630 + r, h0_sigma=0.1,
                               packed=False).to(dev)
        d = inputs.make_inputs([200, 64, 131, 16], 64, 128, 128, "bf16", seed=650 + r,
                               h0_sigma=0.1).to(dev)
        _, zb, wb = inputs.make_output_gate_inputs(b.total_tokens, 64, 128, "bf16", 640 + r)
        sets.append((a, b, c, d, zb.to(dev).reshape(b.call_views()[2].shape), wb.to(dev)))
    assert kda_chunk_fwd_gated_fuses(sets[0][1].q, 4, 1, 64, 128, 128, True)

    def run(a, b, c, d, zb, wb):
        oa, ha = kda_chunk_fwd(*a.call_views(), h0=a.h0)
        yb, _, hb = kda_chunk_fwd_gated(*b.call_views(), zb, weight=wb, h0=b.h0,
                                        cu_seqlens=b.cu_seqlens)
        oc, hc = kda_chunk_fwd_split_noalloc(*c.call_views(), h0=c.h0)
        od, hd = kda_chunk_fwd(*d.call_views(), h0=d.h0, cu_seqlens=d.cu_seqlens)
        ya = kda_output_gate(oa, a.call_views()[2], None)   # v serves as a gate of o's shape
        return oa, ha, yb, hb, oc, hc, od, hd, ya

    run(*sets[0])       # warm-up (the split's first call sets up its static workspace)
    torch.cuda.synchronize()

    # the graph reads static copies of one input set, refilled before each replay
    fields = ("q", "k", "v", "g", "beta", "h0", "cu_seqlens")
    clone = lambda x: dataclasses.replace(x, **{n: getattr(x, n).clone() for n in fields
                                                if getattr(x, n) is not None})
    A, B, Cc, Dd = (clone(x) for x in sets[0][:4])
    zs, ws = sets[0][4].clone(), sets[0][5].clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = run(A, B, Cc, Dd, zs, ws)
    names = ("o (64-column)", "hT (64-column)", "y (fused gated)", "hT (fused gated)",
             "o (split)", "hT (split)", "o (128-column)", "hT (128-column)", "y (output stage)")
    for r in (2, 0, 1):
        a, b, c, d, zb, wb = sets[r]
        ref = [t.clone() for t in run(a, b, c, d, zb, wb)]
        torch.cuda.synchronize()
        for src, dst in ((a, A), (b, B), (c, Cc), (d, Dd)):
            for n in fields:
                if getattr(src, n) is not None:
                    getattr(dst, n).copy_(getattr(src, n))
        zs.copy_(zb)
        ws.copy_(wb)
        graph.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(names, outs, ref):
            assert torch.equal(got, want), f"input set {r}: {name} differs from the eager call"
        (torch.randn(256, 256, device=dev) @ torch.randn(256, 256, device=dev)).sum().item()
    _say("prefill graph: 3 replays bit-identical to the eager calls")
