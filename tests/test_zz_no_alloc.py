"""kda_chunk_fwd_split_noalloc (the split prefill with its workspace in the library's static device
array) against kda_chunk_fwd_split with a caller workspace, through the C ABI, bit for bit: two
calls in a row on the shared array, the second with a smaller input, then a call whose workspace
would exceed the array, which is refused before anything runs."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 32 << 20


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _pair(x, dev, segments, **kw):
    """(noalloc result, caller-workspace result) for one input; o and hT preallocated so that the
    noalloc call allocates nothing."""
    from linear_attention_recurrence_08_amd import kda_chunk_fwd_split, kda_chunk_fwd_split_noalloc
    xd = x.to(dev)
    views = xd.call_views()
    o_n = torch.empty_like(views[2])
    h_n = torch.empty((x.num_seqs, x.H, x.dk, x.dv), dtype=torch.float32, device=dev)
    kda_chunk_fwd_split_noalloc(*views, h0=xd.h0, cu_seqlens=xd.cu_seqlens, segments=segments,
                                o=o_n, hT=h_n, **kw)
    o_w, h_w = kda_chunk_fwd_split(*views, h0=xd.h0, cu_seqlens=xd.cu_seqlens, segments=segments,
                                   **kw)
    torch.cuda.synchronize()
    return (o_n, h_n), (o_w, h_w)


def test_noalloc_matches_workspace_entry_point():
    dev = _dev()
    from linear_attention_recurrence_08_amd import inputs, kda_chunk_fwd_split_workspace_bytes
    # first call: 12 heads x 4,096 tokens (the automatic 5-segment plan, 20.4 MB of workspace)
    big = inputs.make_inputs([4096], H=12, dk=128, dv=128, dtype="bf16", seed=401,
                             h0_sigma=0.05, packed=False)
    need = kda_chunk_fwd_split_workspace_bytes(big.q, 1, 4096, 12, 128, 128, 0)
    assert 0 < need <= SCRATCH_BYTES
    (o_n, h_n), (o_w, h_w) = _pair(big, dev, 0)
    print(f"noalloc big: workspace {need} bytes, o equal {torch.equal(o_n, o_w)}, "
          f"hT equal {torch.equal(h_n, h_w)}", flush=True)
    assert torch.equal(o_n, o_w) and torch.equal(h_n, h_w)
    # second call, smaller, on the array the first call left behind: a packed batch
    small = inputs.make_inputs([700, 0, 333], H=2, dk=128, dv=128, dtype="bf16", seed=402,
                               h0_sigma=0.1, packed=True)
    (o_n, h_n), (o_w, h_w) = _pair(small, dev, 3)
    print(f"noalloc small: o equal {torch.equal(o_n, o_w)}, hT equal {torch.equal(h_n, h_w)}",
          flush=True)
    assert torch.equal(o_n, o_w) and torch.equal(h_n, h_w)
    assert np.isfinite(o_n.float().cpu().numpy()).all()


def test_noalloc_refuses_more_than_the_array():
    dev = _dev()
    from linear_attention_recurrence_08_amd import (KDAError, inputs, kda_chunk_fwd_split_noalloc,
                                                    kda_chunk_fwd_split_workspace_bytes)
    from linear_attention_recurrence_08_amd.kda import KDA_ERR_SCRATCH
    x = inputs.make_inputs([16384], H=12, dk=128, dv=128, dtype="bf16", seed=403, packed=False)
    need = kda_chunk_fwd_split_workspace_bytes(x.q, 1, 16384, 12, 128, 128, 0)
    assert need > SCRATCH_BYTES
    xd = x.to(dev)
    o = torch.full_like(xd.call_views()[2], 7.0)
    with pytest.raises(KDAError) as ei:
        kda_chunk_fwd_split_noalloc(*xd.call_views(), segments=0, o=o)
    torch.cuda.synchronize()
    assert ei.value.code == KDA_ERR_SCRATCH
    assert bool((o == 7.0).all())          # refused before anything ran
