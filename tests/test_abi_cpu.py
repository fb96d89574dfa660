"""CPU-side checks of the C ABI: the library loads, exports every symbol the header declares, and
rejects bad arguments with the documented status codes before touching the GPU."""
import ctypes
import os
import re
import shutil
import subprocess

import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "kda.h")
LIB = os.path.join(ROOT, "linear_attention_recurrence_08_amd", "libkda.so")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(kda_\w+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from linear_attention_recurrence_08_amd import build
        build.build()
    from linear_attention_recurrence_08_amd import kda
    return kda.load_library()


def test_header_declares_the_boundary():
    assert _declared_functions() == ["kda_chunk_fwd", "kda_chunk_fwd_chunk64",
                                     "kda_chunk_fwd_chunk64_workspace_bytes",
                                     "kda_chunk_fwd_gated", "kda_chunk_fwd_gated_fuses",
                                     "kda_chunk_fwd_snapshots", "kda_chunk_fwd_split",
                                     "kda_chunk_fwd_split_noalloc",
                                     "kda_chunk_fwd_split_segments",
                                     "kda_chunk_fwd_split_workspace_bytes",
                                     "kda_decode_step", "kda_decode_step_gated",
                                     "kda_decode_step_layer", "kda_frontend",
                                     "kda_output_gate", "kda_status_string", "kda_version"]


def test_every_declared_symbol_is_exported(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    from linear_attention_recurrence_08_amd.kda import kda_status_string
    assert kda_status_string(0) == "ok"
    for code in range(-11, 0):
        s = kda_status_string(code)
        assert s and s != "unknown status"
    assert kda_status_string(-99) == "unknown status"
    assert lib.kda_version() >= 100


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first


def _prefill(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, h0=None, cu=None, num_seqs=0, o=FAKE,
             hT=FAKE, B=1, T=16, H=2, dk=128, dv=128, dtype=0)
    a.update(kw)
    return lib.kda_chunk_fwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["h0"], a["cu"],
                             a["num_seqs"], a["o"], a["hT"], a["B"], a["T"], a["H"], a["dk"],
                             a["dv"], a["dtype"], None)


def _prefill_snap(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, h0=None, cu=None, num_seqs=0, o=FAKE,
             hT=FAKE, snaps=FAKE, offs=None, stride=64, B=1, T=128, H=2, dk=128, dv=128, dtype=0)
    a.update(kw)
    return lib.kda_chunk_fwd_snapshots(a["q"], a["k"], a["v"], a["g"], a["beta"], a["h0"],
                                       a["cu"], a["num_seqs"], a["o"], a["hT"], a["snaps"],
                                       a["offs"], a["stride"], a["B"], a["T"], a["H"], a["dk"],
                                       a["dv"], a["dtype"], None)


def _decode(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, S=FAKE, o=FAKE, N=4, H=2, dk=128,
             dv=128, dtype=0)
    a.update(kw)
    return lib.kda_decode_step(a["q"], a["k"], a["v"], a["g"], a["beta"], a["S"], a["o"],
                               a["N"], a["H"], a["dk"], a["dv"], a["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=2), -3), (dict(dtype=-1), -3),
    (dict(B=-1), -2), (dict(T=-5), -2), (dict(H=0), -2), (dict(num_seqs=-1), -2),
    (dict(dk=130), -4), (dict(dk=8), -4), (dict(dv=120), -4), (dict(dk=144), -4), (dict(dv=0), -4),
    (dict(q=None), -1), (dict(k=None), -1), (dict(v=None), -1), (dict(g=None), -1),
    (dict(beta=None), -1), (dict(o=None), -1),
    (dict(cu=FAKE, B=2, num_seqs=3), -5),
    # one token's row may hold at most 2^20 elements (H * max(dk, dv))
    (dict(H=8193), -2), (dict(H=65537, dk=16, dv=16), -2),
])
def test_prefill_argument_errors(lib, kw, code):
    assert _prefill(lib, **kw) == code


def _chunk64(lib, ws=None, ws_bytes=0, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, h0=None, cu=None, num_seqs=0, o=FAKE,
             hT=FAKE, B=1, T=16, H=2, dk=128, dv=128, dtype=0)
    a.update(kw)
    return lib.kda_chunk_fwd_chunk64(a["q"], a["k"], a["v"], a["g"], a["beta"], a["h0"], a["cu"],
                                     a["num_seqs"], a["o"], a["hT"], a["B"], a["T"], a["H"],
                                     a["dk"], a["dv"], a["dtype"], ws, ws_bytes, None)


def _ws_bytes(lib, cu=None, num_seqs=0, B=1, T=16, H=2, dk=128, dv=128, dtype=0):
    return lib.kda_chunk_fwd_chunk64_workspace_bytes(cu, num_seqs, B, T, H, dk, dv, dtype)


RECORD = 82432      # workspace bytes per (64-token chunk, head) of the matrix-core path


def test_chunk64_workspace_size(lib):
    # bf16 with dk = dv = 128: chunk offsets (rounded to 256 bytes), then one record per
    # (chunk, head); equal lengths provision B * ceil(T / 64) chunks
    assert _ws_bytes(lib, B=3, T=130, H=5) == 256 + 3 * 3 * 5 * RECORD
    assert _ws_bytes(lib, B=2, T=64, H=1) == 256 + 2 * 1 * RECORD
    # a variable-length batch provisions Ttot // 64 + N chunks (sum of ceil(len / 64) <= that)
    assert _ws_bytes(lib, cu=FAKE, num_seqs=3, B=1, T=200, H=4) == 256 + (3 + 3) * 4 * RECORD
    assert _ws_bytes(lib, cu=FAKE, num_seqs=100, B=1, T=64, H=1) == \
        (101 * 4 + 255) // 256 * 256 + 101 * RECORD
    # the float32 path (other dtype or head size) needs none; nor do rejected arguments
    assert _ws_bytes(lib, dtype=1) == 0
    assert _ws_bytes(lib, dk=64) == 0
    assert _ws_bytes(lib, dtype=5) == 0 and _ws_bytes(lib, H=0) == 0
    assert _ws_bytes(lib, cu=FAKE, B=2, num_seqs=2) == 0
    assert _ws_bytes(lib, B=0) == 0


def test_chunk64_workspace_errors(lib):
    need = _ws_bytes(lib)
    aligned = ctypes.c_void_p(0x10000)   # never dereferenced: the calls fail validation first
    assert _chunk64(lib) == -10                                   # missing
    assert _chunk64(lib, ws=aligned, ws_bytes=need - 1) == -10    # too small
    assert _chunk64(lib, ws=ctypes.c_void_p(0x10010), ws_bytes=need) == -10   # misaligned
    # argument errors come first, as in kda_chunk_fwd
    assert _chunk64(lib, dtype=2) == -3 and _chunk64(lib, q=None) == -1
    # the float32 path takes no workspace: its argument errors come through without one
    assert _chunk64(lib, dtype=1, dk=96, q=None) == -1
    assert _chunk64(lib, B=0) == 0


def _split(lib, ws=None, ws_bytes=0, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, h0=None, cu=None, num_seqs=0, max_seqlen=0,
             o=FAKE, hT=FAKE, B=1, T=4096, H=12, dk=128, dv=128, dtype=0, segments=0)
    a.update(kw)
    return lib.kda_chunk_fwd_split(a["q"], a["k"], a["v"], a["g"], a["beta"], a["h0"], a["cu"],
                                   a["num_seqs"], a["max_seqlen"], a["o"], a["hT"], a["B"],
                                   a["T"], a["H"], a["dk"], a["dv"], a["dtype"], a["segments"],
                                   ws, ws_bytes, None)


def _seg(lib, B, T, H, dk=128, dv=128, dtype=0, segments=0, cu=None, num_seqs=0, max_seqlen=0):
    return lib.kda_chunk_fwd_split_segments(cu, num_seqs, max_seqlen, B, T, H, dk, dv, dtype,
                                            segments)


def _split_ws(lib, B, T, H, dk=128, dv=128, dtype=0, segments=0, cu=None, num_seqs=0,
              max_seqlen=0):
    return lib.kda_chunk_fwd_split_workspace_bytes(cu, num_seqs, max_seqlen, B, T, H, dk, dv,
                                                   dtype, segments)


def test_split_plan(lib):
    # automatic: the largest P with 2 (2 P - 1) N H <= 256 workgroups and >= 256 tokens each
    assert _seg(lib, 1, 4096, 12) == 5        # 2 * 12 * 9 = 216 workgroups
    assert _seg(lib, 1, 4096, 24) == 3        # 2 * 24 * 5 = 240
    assert _seg(lib, 1, 4096, 96) == 1        # 192 workgroups already
    assert _seg(lib, 1, 512, 12) == 2         # 256 tokens per segment at least
    assert _seg(lib, 1, 300, 12) == 1
    # requested: capped at 16; segments are whole multiples of 64 tokens, so fewer may result
    assert _seg(lib, 1, 4096, 96, segments=3) == 3
    assert _seg(lib, 1, 4096, 1, segments=40) == 16
    assert _seg(lib, 1, 100, 1, segments=4) == 2          # 64-token segments: 64 + 36
    assert _seg(lib, 1, 64, 1, segments=4) == 1
    # other dtypes and head sizes, and batches beyond the grid's y extent, do not split
    assert _seg(lib, 1, 4096, 12, dtype=1) == 1
    assert _seg(lib, 1, 4096, 12, dk=64) == 1
    assert _seg(lib, 65536, 4096, 1, segments=4) == 1
    assert _seg(lib, 1, 4096, 12, segments=-1) == 1
    # variable-length batches plan for max_seqlen tokens and N sequences (contents not read)
    assert _seg(lib, 1, 9000, 6, cu=FAKE, num_seqs=2, max_seqlen=8000) == 5   # 2*12*9 = 216
    assert _seg(lib, 1, 9000, 6, cu=FAKE, num_seqs=2, max_seqlen=0) == 1
    assert _seg(lib, 2, 9000, 6, cu=FAKE, num_seqs=2, max_seqlen=8000) == 1   # B must be 1


def test_split_workspace(lib):
    # M_t^T q_t in bf16 for every token, then 2 final states per segment and (sequence, head)
    assert _split_ws(lib, 1, 4096, 12) == 4096 * 12 * 256 + 5 * 2 * 12 * 65536
    assert _split_ws(lib, 2, 1000, 3, segments=2) == \
        (2 * 1000 * 3 * 256 + 255) // 256 * 256 + 2 * 2 * 6 * 65536
    assert _split_ws(lib, 1, 9000, 6, cu=FAKE, num_seqs=2, max_seqlen=8000) == \
        9000 * 6 * 256 + 5 * 2 * 12 * 65536
    assert _split_ws(lib, 1, 4096, 96) == 0 and _split_ws(lib, 1, 4096, 12, dtype=1) == 0
    need = _split_ws(lib, 1, 4096, 12)
    aligned = ctypes.c_void_p(0x10000)   # never dereferenced: the calls fail validation first
    assert _split(lib) == -10                                        # missing
    assert _split(lib, ws=aligned, ws_bytes=need - 1) == -10         # too small
    assert _split(lib, ws=ctypes.c_void_p(0x10010), ws_bytes=need) == -10   # misaligned
    assert _split(lib, segments=-1) == -2
    assert _split(lib, cu=FAKE, num_seqs=2, max_seqlen=-1) == -2
    assert _split(lib, q=None) == -1 and _split(lib, dtype=3) == -3
    # varlen: cu_seqlens needs B == 1, as in kda_chunk_fwd
    assert _split(lib, cu=FAKE, num_seqs=2, max_seqlen=4000, B=2) == -5
    assert _split(lib, cu=FAKE, num_seqs=2, max_seqlen=4000) == -10  # a split: workspace needed
    # no split (one segment, or the float32 path): kda_chunk_fwd's errors, no workspace needed
    assert _split(lib, H=96, q=None) == -1 and _split(lib, dtype=1, dk=96, q=None) == -1
    assert _split(lib, B=0) == 0


def test_prefill_empty_is_noop(lib):
    # no sequences, or no tokens and no final state requested: nothing to launch
    assert _prefill(lib, B=0) == 0
    assert _prefill(lib, T=0, hT=None) == 0
    assert _prefill(lib, cu=FAKE, B=1, T=0, num_seqs=0) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(stride=0), -8), (dict(stride=-16), -8), (dict(stride=24), -8), (dict(stride=8), -8),
    (dict(cu=FAKE, num_seqs=2, offs=None), -1),     # varlen snapshots need their offsets
    (dict(snaps=None), -1),                         # T >= stride: snapshots are due
    (dict(dk=96, dtype=2), -3), (dict(H=0), -2), (dict(dv=8), -4), (dict(q=None), -1),
])
def test_snapshot_argument_errors(lib, kw, code):
    assert _prefill_snap(lib, **kw) == code


def test_snapshot_empty_is_noop(lib):
    assert _prefill_snap(lib, B=0) == 0
    # no sequence reaches the stride: an empty snapshot buffer may be NULL (nothing launched here
    # because there are no tokens and no final state)
    assert _prefill_snap(lib, T=0, hT=None, snaps=None) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=3), -3), (dict(N=-1), -2), (dict(H=0), -2), (dict(dk=100), -4),
    (dict(dv=256), -4), (dict(q=None), -1), (dict(S=None), -1), (dict(o=None), -1),
    (dict(beta=None), -1), (dict(H=8193), -2),
])
def test_decode_argument_errors(lib, kw, code):
    assert _decode(lib, **kw) == code


def test_decode_empty_is_noop(lib):
    assert _decode(lib, N=0, q=None) == 0


def test_binding_rejects_cpu_tensors():
    import torch
    from linear_attention_recurrence_08_amd import kda_chunk_fwd
    x = torch.zeros(16, 2, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        kda_chunk_fwd(x, x, x, x, torch.zeros(16, 2, dtype=torch.bfloat16))


UNALIGNED = ctypes.c_void_p(0x1008)


def _gate(lib, **kw):
    a = dict(o=FAKE, gate=FAKE, w=None, eps=1e-6, y=FAKE, T=16, H=2, dv=128, dtype=0)
    a.update(kw)
    return lib.kda_output_gate(a["o"], a["gate"], a["w"], a["eps"], a["y"], a["T"], a["H"],
                               a["dv"], a["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=2), -3), (dict(T=-1), -2), (dict(H=0), -2), (dict(dv=8), -4), (dict(dv=144), -4),
    (dict(eps=-1.0), -6), (dict(eps=float("nan")), -6), (dict(eps=float("inf")), -6),
    (dict(o=None), -1), (dict(gate=None), -1), (dict(y=None), -1),
    (dict(o=UNALIGNED), -9), (dict(gate=UNALIGNED), -9), (dict(y=UNALIGNED), -9),
    (dict(H=8193), -2),
])
def test_output_gate_argument_errors(lib, kw, code):
    assert _gate(lib, **kw) == code


def test_output_gate_empty_is_noop(lib):
    assert _gate(lib, T=0, o=None, gate=None, y=None) == 0


def _decode_gated(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, S=FAKE, gate=FAKE, w=None, eps=1e-6,
             o=FAKE, y=FAKE, N=4, H=2, dk=64, dv=64, dtype=0)
    a.update(kw)
    return lib.kda_decode_step_gated(a["q"], a["k"], a["v"], a["g"], a["beta"], a["S"], a["gate"],
                                     a["w"], a["eps"], a["o"], a["y"], a["N"], a["H"], a["dk"],
                                     a["dv"], a["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=5), -3), (dict(N=-1), -2), (dict(dk=100), -4), (dict(eps=-0.5), -6),
    (dict(gate=None), -1), (dict(y=None), -1), (dict(o=None), -1), (dict(S=None), -1),
    # the unfused fallback (64 x 64 heads) needs 16-byte aligned output-stage rows
    (dict(y=UNALIGNED), -9), (dict(gate=UNALIGNED), -9),
    (dict(H=16385), -2),
])
def test_decode_gated_argument_errors(lib, kw, code):
    assert _decode_gated(lib, **kw) == code


def _front(lib, **kw):
    a = dict(xq=FAKE, xk=FAKE, xv=FAKE, xz=FAKE, xb=FAKE, wq=FAKE, wk=FAKE, wv=FAKE, zb=FAKE,
             A=FAKE, gmin=-5.0, eps=1e-6, cu=None, num_seqs=0, cin=None, cout=None, q=FAKE,
             k=FAKE, v=FAKE, g=FAKE, beta=FAKE, B=2, T=16, H=2, dk=128, dv=128, dtype=0)
    a.update(kw)
    return lib.kda_frontend(*(a[n] for n in ("xq", "xk", "xv", "xz", "xb", "wq", "wk", "wv", "zb",
                                             "A", "gmin", "eps", "cu", "num_seqs", "cin", "cout",
                                             "q", "k", "v", "g", "beta", "B", "T", "H", "dk",
                                             "dv", "dtype")), None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=2), -3), (dict(B=-1), -2), (dict(H=0), -2), (dict(dk=8), -4), (dict(dv=136), -4),
    (dict(gmin=0.0), -6), (dict(gmin=1.0), -6), (dict(eps=-1.0), -6),
    (dict(cu=FAKE, B=2, num_seqs=1), -5),
    (dict(xq=None), -1), (dict(wv=None), -1), (dict(A=None), -1), (dict(beta=None), -1),
    (dict(q=UNALIGNED), -9), (dict(xv=UNALIGNED), -9), (dict(cin=UNALIGNED), -9),
    (dict(H=8193), -2),
])
def test_frontend_argument_errors(lib, kw, code):
    assert _front(lib, **kw) == code


def test_frontend_empty_is_noop(lib):
    assert _front(lib, B=0) == 0
    assert _front(lib, T=0) == 0


def _layer(lib, **kw):
    a = dict(xq=FAKE, xk=FAKE, xv=FAKE, xz=FAKE, xb=FAKE, wq=FAKE, wk=FAKE, wv=FAKE, zb=FAKE,
             A=FAKE, gmin=-5.0, neps=1e-6, conv=FAKE, S=FAKE, gate=FAKE, w=None, eps=1e-6,
             o=None, y=FAKE, N=4, H=2, dk=128, dv=128, dtype=0)
    a.update(kw)
    return lib.kda_decode_step_layer(*(a[n] for n in (
        "xq", "xk", "xv", "xz", "xb", "wq", "wk", "wv", "zb", "A", "gmin", "neps", "conv", "S",
        "gate", "w", "eps", "o", "y", "N", "H", "dk", "dv", "dtype")), None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=2), -3), (dict(N=-1), -2), (dict(H=0), -2),
    # the fused kernel's head size only
    (dict(dk=64), -4), (dict(dv=64), -4), (dict(dk=96, dv=96), -4),
    (dict(gmin=0.0), -6), (dict(neps=-1.0), -6), (dict(eps=-1.0), -6),
    (dict(eps=float("nan")), -6), (dict(gmin=float("-inf")), -6),
    (dict(xq=None), -1), (dict(xb=None), -1), (dict(wv=None), -1), (dict(zb=None), -1),
    (dict(A=None), -1), (dict(conv=None), -1), (dict(S=None), -1), (dict(gate=None), -1),
    (dict(y=None), -1),
    (dict(S=UNALIGNED), -9), (dict(o=ctypes.c_void_p(0x1004)), -9),
    (dict(y=ctypes.c_void_p(0x1004)), -9), (dict(gate=UNALIGNED, dtype=1), -9),
    (dict(H=8193), -2),
])
def test_layer_decode_argument_errors(lib, kw, code):
    assert _layer(lib, **kw) == code


def test_layer_decode_empty_is_noop(lib):
    assert _layer(lib, N=0, xq=None, conv=None, S=None, y=None) == 0


class _NoCalls:
    """Stands in for the library: any call into it fails the test (the binding must reject the
    arguments before reaching the C ABI)."""
    def __getattr__(self, name):
        raise AssertionError(f"the binding called {name} with arguments it should have rejected")


@pytest.fixture
def host_binding(monkeypatch):
    """The binding with its device checks relaxed so that host tensors reach the shape checks."""
    import torch
    from linear_attention_recurrence_08_amd import kda

    def check(t, name, device, dtype=None):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if dtype is not None and t.dtype != dtype:
            raise TypeError(f"{name} must be {dtype}")
    monkeypatch.setattr(kda, "_check", check)
    monkeypatch.setattr(kda, "_stream", lambda dev: None)
    monkeypatch.setattr(kda, "load_library", lambda: _NoCalls())
    return kda, torch


def _bf(torch, *shape):
    return torch.zeros(*shape, dtype=torch.bfloat16)


@pytest.mark.parametrize("which,shape", [
    ("o", (16, 2, 64)), ("o", (15, 2, 128)), ("o", (16, 3, 128)),
    ("hT", (1, 2, 128, 64)), ("hT", (2, 2, 128, 128)),
])
def test_binding_rejects_small_prefill_outputs(host_binding, which, shape):
    """A caller's o or hT whose shape differs from (lead, H, dv) / (N, H, dk, dv) is rejected:
    the kernels write every row, so a smaller buffer would be written past its end."""
    kda, torch = host_binding
    x = _bf(torch, 16, 2, 128)
    kw = {which: _bf(torch, *shape) if which == "o" else torch.zeros(*shape)}
    with pytest.raises(ValueError):
        kda.kda_chunk_fwd(x, x, x, x, _bf(torch, 16, 2), **kw)


def test_binding_rejects_small_decode_outputs(host_binding):
    kda, torch = host_binding
    q = _bf(torch, 4, 2, 128)
    S = torch.zeros(4, 2, 128, 128)
    with pytest.raises(ValueError):
        kda.kda_decode_step(q, q, q, q, _bf(torch, 4, 2), S, o=_bf(torch, 3, 2, 128))
    with pytest.raises(ValueError):
        kda.kda_decode_step_gated(q, q, q, q, _bf(torch, 4, 2), S, q, y=_bf(torch, 4, 2, 64))


@pytest.mark.parametrize("bad", ["conv_state", "S", "y", "gate", "w_v"])
def test_binding_rejects_wrong_layer_decode_buffers(host_binding, bad):
    """kda_decode_step_layer writes the whole convolution state, S and y in place: a buffer of
    another shape is rejected before the C ABI is reached."""
    kda, torch = host_binding
    N, H = 4, 2
    x = _bf(torch, N, H, 128)
    a = dict(conv_state=_bf(torch, N, 3, H * 384), S=torch.zeros(N, H, 128, 128),
             gate=_bf(torch, N, H, 128), y=None, w_v=torch.zeros(H * 128, 4))
    a[bad] = {"conv_state": _bf(torch, N, 3, H * 384 - 8), "S": torch.zeros(N - 1, H, 128, 128),
              "y": _bf(torch, N, H, 64), "gate": _bf(torch, N, H + 1, 128),
              "w_v": torch.zeros(H * 128, 3)}[bad]
    taps = torch.zeros(H * 128, 4)
    with pytest.raises(ValueError):
        kda.kda_decode_step_layer(x, x, x, x, _bf(torch, N, H), taps, taps, a["w_v"],
                                  torch.zeros(H * 128), torch.ones(H), a["conv_state"], a["S"],
                                  a["gate"], y=a["y"])


def test_binding_rejects_small_snapshot_buffers(host_binding):
    kda, torch = host_binding
    x = _bf(torch, 64, 2, 128)
    # equal-length batch: 64 / 16 = 4 snapshots needed
    with pytest.raises(ValueError):
        kda.kda_chunk_fwd_snapshots(x, x, x, x, _bf(torch, 64, 2), 16,
                                    snaps=torch.zeros(3, 2, 128, 128))
    # packed batch: the offsets say 5 snapshots (lengths 48 and 32 at stride 16)
    cu = torch.tensor([0, 48, 80], dtype=torch.int32)
    offs = torch.tensor([0, 3, 5], dtype=torch.int32)
    xp = _bf(torch, 80, 2, 128)
    with pytest.raises(ValueError):
        kda.kda_chunk_fwd_snapshots(xp, xp, xp, xp, _bf(torch, 80, 2), 16, cu_seqlens=cu,
                                    snap_offsets=offs, snaps=torch.zeros(4, 2, 128, 128))


def _gated(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, h0=None, cu=None, num_seqs=0, gate=FAKE,
             weight=None, eps=1e-6, o=None, y=FAKE, hT=FAKE, B=1, T=16, H=2, dk=128, dv=128,
             dtype=0)
    a.update(kw)
    return lib.kda_chunk_fwd_gated(a["q"], a["k"], a["v"], a["g"], a["beta"], a["h0"], a["cu"],
                                   a["num_seqs"], a["gate"], a["weight"], ctypes.c_float(a["eps"]),
                                   a["o"], a["y"], a["hT"], a["B"], a["T"], a["H"], a["dk"],
                                   a["dv"], a["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=2), -3), (dict(H=0), -2), (dict(dk=120), -4),
    (dict(eps=-1.0), -6), (dict(eps=float("nan")), -6), (dict(eps=float("inf")), -6),
    (dict(q=None), -1), (dict(gate=None), -1), (dict(y=None), -1),
    (dict(gate=ctypes.c_void_p(0x1008)), -9), (dict(y=ctypes.c_void_p(0x1004)), -9),
    (dict(o=ctypes.c_void_p(0x1002)), -9),
    (dict(cu=FAKE, B=2, num_seqs=3), -5),
])
def test_gated_prefill_argument_errors(lib, kw, code):
    assert _gated(lib, **kw) == code


def test_gated_prefill_fuses_query(lib):
    # the output stage runs inside the prefill kernel for bf16 128 x 128 heads and >= 256 pairs
    assert lib.kda_chunk_fwd_gated_fuses(0, 2, 128, 128, 128, 0, 0) == 1
    assert lib.kda_chunk_fwd_gated_fuses(0, 1, 255, 128, 128, 0, 0) == 0
    assert lib.kda_chunk_fwd_gated_fuses(16, 1, 96, 128, 128, 0, 1) == 1
    assert lib.kda_chunk_fwd_gated_fuses(0, 2, 128, 128, 128, 1, 0) == 0    # float32
    assert lib.kda_chunk_fwd_gated_fuses(0, 2, 128, 64, 128, 0, 0) == 0     # dk = 64
    assert lib.kda_chunk_fwd_gated_fuses(0, -1, 128, 128, 128, 0, 0) == 0


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_header_is_plain_c(tmp_path, lib):
    """include/kda.h is a C ABI: a C99 program that includes it compiles with -pedantic -Werror,
    links against libkda.so and calls it (argument validation only, no GPU)."""
    src = tmp_path / "use_kda.c"
    src.write_text(
        '#include "kda.h"\n#include <stdio.h>\n#include <string.h>\n'
        "int main(void) {\n"
        "    if (kda_version() < 100) return 1;\n"
        "    if (strcmp(kda_status_string(KDA_OK), \"ok\") != 0) return 2;\n"
        "    /* a NULL q with tokens present is rejected before anything runs */\n"
        "    if (kda_chunk_fwd(NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL, NULL, 1, 16, 2,\n"
        "                      128, 128, KDA_BF16, NULL) != KDA_ERR_NULL) return 3;\n"
        "    puts(\"c ok\");\n"
        "    return 0;\n"
        "}\n")
    libdir = os.path.join(ROOT, "linear_attention_recurrence_08_amd")
    exe = str(tmp_path / "use_kda")
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                        "-I", os.path.join(ROOT, "include"), str(src), "-L", libdir, "-lkda",
                        f"-Wl,-rpath,{libdir}", "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and "c ok" in r.stdout, (r.returncode, r.stdout, r.stderr)
