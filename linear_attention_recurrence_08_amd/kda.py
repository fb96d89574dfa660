"""Python binding of libkda.so (ctypes).  Argument marshalling only: every step of the KDA path runs
in the library's HIP kernels.  PyTorch supplies device memory and the current stream.

    kda_chunk_fwd(q, k, v, g, beta, h0=None, cu_seqlens=None, output_final_state=True)
        -> (o, hT)
    kda_chunk_fwd_chunk64(...)   the same with 64-token chunks of four 16-token sub-tiles
    kda_chunk_fwd_split(q, k, v, g, beta, h0=None, cu_seqlens=None, max_seqlen=None,
                        segments=0, ...) -> (o, hT)
                                 the same with each sequence also cut into token ranges that run
                                 concurrently (small batches)
    kda_chunk_fwd_snapshots(q, k, v, g, beta, snap_stride, ...) -> (o, hT, snaps, snap_offsets)
    kda_decode_step(q, k, v, g, beta, S) -> o         (S is updated in place)
    kda_decode_step_gated(q, k, v, g, beta, S, gate, weight=None, eps=...) -> (o, y)
    kda_output_gate(o, gate, weight=None, eps=...) -> y
    kda_frontend(x_q, x_k, x_v, x_z, x_b, w_q, w_k, w_v, z_bias, A, ...)
        -> (q, k, v, g, beta, conv_state)
    kda_decode_step_layer(x_q, x_k, x_v, x_z, x_b, w_q, w_k, w_v, z_bias, A, conv_state, S,
                          gate, ...) -> (y, o)
                                 the input stage, the decode step and the output stage in one
                                 launch (conv_state and S updated in place)
    kda_status_string(code) -> str

Layouts (see include/kda.h): q, k, g [B, T, H, dk] or packed [Ttot, H, dk]; v [.., H, dv];
beta [B, T, H] or [Ttot, H]; h0 / hT / S float32 [N, H, dk, dv]; cu_seqlens int32 [N+1] on the
device (packed inputs only).  q, k, v, g, beta and o share one dtype: bfloat16 or float32.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkda.so")

KDA_BF16, KDA_F32 = 0, 1
KDA_OK = 0
KDA_ERR_STRIDE = -8
KDA_ERR_SCRATCH = -11
_lib = None


class KDAError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {kda_status_string(code)} (status {code})")
        self.code = code


def load_library():
    """Open libkda.so; raises if the HIP library has not been built (there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build the HIP library first "
                               "(python -c 'import __graft_entry__ as g; g.build()')")
        lib = ctypes.CDLL(LIB_PATH)
        vp, i32 = ctypes.c_void_p, ctypes.c_int
        lib.kda_chunk_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, vp, vp,
                                      i32, i32, i32, i32, i32, i32, vp]
        lib.kda_chunk_fwd.restype = i32
        lib.kda_chunk_fwd_chunk64.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, vp, vp,
                                              i32, i32, i32, i32, i32, i32, vp, ctypes.c_size_t,
                                              vp]
        lib.kda_chunk_fwd_chunk64.restype = i32
        lib.kda_chunk_fwd_chunk64_workspace_bytes.argtypes = [vp, i32, i32, i32, i32, i32, i32,
                                                              i32]
        lib.kda_chunk_fwd_chunk64_workspace_bytes.restype = ctypes.c_size_t
        lib.kda_chunk_fwd_split.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, vp, vp, i32,
                                            i32, i32, i32, i32, i32, i32, vp, ctypes.c_size_t,
                                            vp]
        lib.kda_chunk_fwd_split.restype = i32
        lib.kda_chunk_fwd_split_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, vp, vp,
                                                    i32, i32, i32, i32, i32, i32, i32, vp]
        lib.kda_chunk_fwd_split_noalloc.restype = i32
        lib.kda_chunk_fwd_split_segments.argtypes = [vp, i32, i32, i32, i32, i32, i32, i32, i32,
                                                     i32]
        lib.kda_chunk_fwd_split_segments.restype = i32
        lib.kda_chunk_fwd_split_workspace_bytes.argtypes = [vp, i32, i32, i32, i32, i32, i32, i32,
                                                            i32, i32]
        lib.kda_chunk_fwd_split_workspace_bytes.restype = ctypes.c_size_t
        lib.kda_chunk_fwd_snapshots.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp,
                                                i32, i32, i32, i32, i32, i32, i32, vp]
        lib.kda_chunk_fwd_snapshots.restype = i32
        lib.kda_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp]
        lib.kda_decode_step.restype = i32
        f32 = ctypes.c_float
        lib.kda_output_gate.argtypes = [vp, vp, vp, f32, vp, i32, i32, i32, i32, vp]
        lib.kda_chunk_fwd_gated.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, f32, vp, vp,
                                            vp, i32, i32, i32, i32, i32, i32, vp]
        lib.kda_chunk_fwd_gated.restype = i32
        lib.kda_chunk_fwd_gated_fuses.argtypes = [i32, i32, i32, i32, i32, i32, i32]
        lib.kda_chunk_fwd_gated_fuses.restype = i32
        lib.kda_output_gate.restype = i32
        lib.kda_decode_step_gated.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, f32, vp, vp, i32,
                                              i32, i32, i32, i32, vp]
        lib.kda_decode_step_gated.restype = i32
        lib.kda_frontend.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, f32, f32, vp, i32,
                                     vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp]
        lib.kda_frontend.restype = i32
        lib.kda_decode_step_layer.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, f32, f32,
                                              vp, vp, vp, vp, f32, vp, vp, i32, i32, i32, i32,
                                              i32, vp]
        lib.kda_decode_step_layer.restype = i32
        lib.kda_status_string.argtypes = [i32]
        lib.kda_status_string.restype = ctypes.c_char_p
        lib.kda_version.argtypes = []
        lib.kda_version.restype = i32
        _lib = lib
    return _lib


def kda_status_string(code: int) -> str:
    return load_library().kda_status_string(int(code)).decode()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float32:
        return KDA_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t: torch.Tensor, name: str, device, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _prefill_args(q, k, v, g, beta, h0, cu_seqlens, output_final_state, o, hT, want_o=True):
    """Shape/device checks shared by the prefill entry points; allocates o (when wanted) and hT
    if needed."""
    dev = q.device
    dt = q.dtype
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta)):
        _check(t, name, dev, dt)
    if q.dim() == 4:
        if cu_seqlens is not None:
            raise ValueError("cu_seqlens needs packed [Ttot, H, d] inputs")
        B, T, H, dk = q.shape
        dv = v.shape[-1]
        lead = (B, T)
    elif q.dim() == 3:
        T, H, dk = q.shape
        dv = v.shape[-1]
        B = 1
        lead = (T,)
    else:
        raise ValueError("q must be [B, T, H, dk] or [Ttot, H, dk]")
    if k.shape != q.shape or g.shape != q.shape or v.shape != (*lead, H, dv) \
            or beta.shape != (*lead, H):
        raise ValueError("inconsistent q/k/v/g/beta shapes")
    if cu_seqlens is not None:
        _check(cu_seqlens, "cu_seqlens", dev, torch.int32)
        N = cu_seqlens.numel() - 1
    else:
        N = B
    if h0 is not None:
        _check(h0, "h0", dev, torch.float32)
        if h0.shape != (N, H, dk, dv):
            raise ValueError(f"h0 must be [{N}, {H}, {dk}, {dv}]")
    if o is None:
        if want_o:
            o = torch.empty((*lead, H, dv), dtype=dt, device=dev)
    else:
        # the kernels write every (token, head) row of o: a smaller buffer would be overrun
        _check(o, "o", dev, dt)
        if tuple(o.shape) != (*lead, H, dv):
            raise ValueError(f"o must be {[*lead, H, dv]}, got {list(o.shape)}")
    if output_final_state:
        if hT is None:
            hT = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
        else:
            _check(hT, "hT", dev, torch.float32)
            if tuple(hT.shape) != (N, H, dk, dv):
                raise ValueError(f"hT must be [{N}, {H}, {dk}, {dv}], got {list(hT.shape)}")
    else:
        hT = None
    return dev, B, T, H, dk, dv, N, o, hT


def kda_chunk_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                  beta: torch.Tensor, h0: Optional[torch.Tensor] = None,
                  cu_seqlens: Optional[torch.Tensor] = None, output_final_state: bool = True,
                  o: Optional[torch.Tensor] = None, hT: Optional[torch.Tensor] = None
                  ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunkwise KDA prefill.  Returns (o, hT); hT is None when output_final_state is False.
    o / hT may be passed preallocated (hT may be h0 itself for an in-place state update)."""
    dev, B, T, H, dk, dv, N, o, hT = _prefill_args(q, k, v, g, beta, h0, cu_seqlens,
                                                   output_final_state, o, hT)
    st = load_library().kda_chunk_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(cu_seqlens), N,
        _ptr(o), _ptr(hT), B, T, H, dk, dv, _dtype_code(q), _stream(dev))
    if st != KDA_OK:
        raise KDAError(st, "kda_chunk_fwd")
    return o, hT


def kda_chunk_fwd_gated(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                        beta: torch.Tensor, gate: torch.Tensor,
                        weight: Optional[torch.Tensor] = None, eps: float = 1e-6,
                        h0: Optional[torch.Tensor] = None,
                        cu_seqlens: Optional[torch.Tensor] = None,
                        output_final_state: bool = True, want_o: bool = False,
                        o: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None,
                        hT: Optional[torch.Tensor] = None
                        ) -> Tuple[torch.Tensor, Optional[torch.Tensor], Optional[torch.Tensor]]:
    """Chunkwise KDA prefill followed by the output stage y = RMSNorm(o) * weight * sigmoid(gate)
    (inside the prefill kernel for bf16 128 x 128 heads with at least 256 (sequence, head) pairs).
    gate has o's shape; weight [dv] float32 or None.  Returns (y, o, hT): o is None unless want_o
    is set or o is passed; hT is None when output_final_state is False."""
    dev, B, T, H, dk, dv, N, o, hT = _prefill_args(q, k, v, g, beta, h0, cu_seqlens,
                                                   output_final_state, o, hT,
                                                   want_o=want_o)
    lead = tuple(v.shape[:-2])
    _check(gate, "gate", dev, q.dtype)
    if tuple(gate.shape) != (*lead, H, dv):
        raise ValueError(f"gate must be {[*lead, H, dv]}, got {list(gate.shape)}")
    weight = _gate_weight(weight, dv, dev)
    if y is None:
        y = torch.empty((*lead, H, dv), dtype=q.dtype, device=dev)
    else:
        _check(y, "y", dev, q.dtype)
        if tuple(y.shape) != (*lead, H, dv):
            raise ValueError(f"y must be {[*lead, H, dv]}, got {list(y.shape)}")
    st = load_library().kda_chunk_fwd_gated(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(cu_seqlens), N,
        _ptr(gate), _ptr(weight), float(eps), _ptr(o), _ptr(y), _ptr(hT), B, T, H, dk, dv,
        _dtype_code(q), _stream(dev))
    if st != KDA_OK:
        raise KDAError(st, "kda_chunk_fwd_gated")
    return y, o, hT


def kda_chunk_fwd_gated_fuses(q: torch.Tensor, num_seqs: int, B: int, H: int, dk: int, dv: int,
                              varlen: bool) -> bool:
    """Whether kda_chunk_fwd_gated runs the output stage inside the prefill kernel."""
    return bool(load_library().kda_chunk_fwd_gated_fuses(num_seqs, B, H, dk, dv, _dtype_code(q),
                                                         1 if varlen else 0))


def kda_chunk_fwd_chunk64_workspace_bytes(q: torch.Tensor, cu_seqlens: Optional[torch.Tensor],
                                          num_seqs: int, B: int, T: int, H: int, dk: int,
                                          dv: int) -> int:
    """Workspace bytes kda_chunk_fwd_chunk64 needs for these arguments (0: none)."""
    return int(load_library().kda_chunk_fwd_chunk64_workspace_bytes(
        _ptr(cu_seqlens), num_seqs, B, T, H, dk, dv, _dtype_code(q)))


def kda_chunk_fwd_chunk64(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                          beta: torch.Tensor, h0: Optional[torch.Tensor] = None,
                          cu_seqlens: Optional[torch.Tensor] = None,
                          output_final_state: bool = True, o: Optional[torch.Tensor] = None,
                          hT: Optional[torch.Tensor] = None,
                          workspace: Optional[torch.Tensor] = None
                          ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """kda_chunk_fwd computed with 64-token chunks of four 16-token sub-tiles (one state carry per
    chunk).  Same arguments and results as kda_chunk_fwd; `workspace` (a contiguous device tensor
    of at least kda_chunk_fwd_chunk64_workspace_bytes bytes) is allocated here when not given."""
    dev, B, T, H, dk, dv, N, o, hT = _prefill_args(q, k, v, g, beta, h0, cu_seqlens,
                                                   output_final_state, o, hT)
    need = kda_chunk_fwd_chunk64_workspace_bytes(q, cu_seqlens, N, B, T, H, dk, dv)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load_library().kda_chunk_fwd_chunk64(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(cu_seqlens), N,
        _ptr(o), _ptr(hT), B, T, H, dk, dv, _dtype_code(q), _ptr(workspace), nbytes, _stream(dev))
    if st != KDA_OK:
        raise KDAError(st, "kda_chunk_fwd_chunk64")
    return o, hT


def kda_chunk_fwd_split_segments(q: torch.Tensor, B: int, T: int, H: int, dk: int, dv: int,
                                 segments: int = 0, cu_seqlens: Optional[torch.Tensor] = None,
                                 num_seqs: int = 0, max_seqlen: int = 0) -> int:
    """Segments kda_chunk_fwd_split plans for these sizes and request (1: no split)."""
    return int(load_library().kda_chunk_fwd_split_segments(
        _ptr(cu_seqlens), num_seqs, max_seqlen, B, T, H, dk, dv, _dtype_code(q), segments))


def kda_chunk_fwd_split_workspace_bytes(q: torch.Tensor, B: int, T: int, H: int, dk: int,
                                        dv: int, segments: int = 0,
                                        cu_seqlens: Optional[torch.Tensor] = None,
                                        num_seqs: int = 0, max_seqlen: int = 0) -> int:
    """Workspace bytes kda_chunk_fwd_split needs for these sizes and request (0: none)."""
    return int(load_library().kda_chunk_fwd_split_workspace_bytes(
        _ptr(cu_seqlens), num_seqs, max_seqlen, B, T, H, dk, dv, _dtype_code(q), segments))


def kda_chunk_fwd_split(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                        beta: torch.Tensor, h0: Optional[torch.Tensor] = None,
                        cu_seqlens: Optional[torch.Tensor] = None,
                        max_seqlen: Optional[int] = None,
                        output_final_state: bool = True, segments: int = 0,
                        o: Optional[torch.Tensor] = None, hT: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None
                        ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """kda_chunk_fwd with each sequence also cut into token ranges that run concurrently
    (segments = 0: the library's choice).  Same results as kda_chunk_fwd.  With cu_seqlens the
    plan assumes sequences of max_seqlen tokens; when it is None it is read from cu_seqlens (one
    device-to-host copy).  `workspace` (a contiguous device tensor of at least
    kda_chunk_fwd_split_workspace_bytes bytes) is allocated here when not given."""
    dev, B, T, H, dk, dv, N, o, hT = _prefill_args(q, k, v, g, beta, h0, cu_seqlens,
                                                   output_final_state, o, hT)
    if cu_seqlens is not None and max_seqlen is None:
        max_seqlen = int((cu_seqlens[1:] - cu_seqlens[:-1]).max().item()) if N > 0 else 0
    msl = int(max_seqlen or 0)
    need = kda_chunk_fwd_split_workspace_bytes(q, B, T, H, dk, dv, segments, cu_seqlens, N, msl)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load_library().kda_chunk_fwd_split(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(cu_seqlens), N, msl,
        _ptr(o), _ptr(hT), B, T, H, dk, dv, _dtype_code(q), int(segments), _ptr(workspace),
        nbytes, _stream(dev))
    if st != KDA_OK:
        raise KDAError(st, "kda_chunk_fwd_split")
    return o, hT


def kda_chunk_fwd_split_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                                g: torch.Tensor, beta: torch.Tensor,
                                h0: Optional[torch.Tensor] = None,
                                cu_seqlens: Optional[torch.Tensor] = None,
                                max_seqlen: Optional[int] = None,
                                output_final_state: bool = True, segments: int = 0,
                                o: Optional[torch.Tensor] = None,
                                hT: Optional[torch.Tensor] = None
                                ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """kda_chunk_fwd_split with its workspace in the library's static device array (32 MiB per
    device) instead of a caller buffer: the C call allocates nothing.  Pass o (and hT) to keep
    this function from allocating them.  Calls that overlap on one GPU share the array and race.
    With cu_seqlens and no max_seqlen, max_seqlen is read from cu_seqlens (one synchronisation)."""
    dev, B, T, H, dk, dv, N, o, hT = _prefill_args(q, k, v, g, beta, h0, cu_seqlens,
                                                   output_final_state, o, hT)
    if cu_seqlens is not None and max_seqlen is None:
        max_seqlen = int((cu_seqlens[1:] - cu_seqlens[:-1]).max().item()) if N > 0 else 0
    st = load_library().kda_chunk_fwd_split_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(cu_seqlens), N,
        int(max_seqlen or 0), _ptr(o), _ptr(hT), B, T, H, dk, dv, _dtype_code(q), int(segments),
        _stream(dev))
    if st != KDA_OK:
        raise KDAError(st, "kda_chunk_fwd_split_noalloc")
    return o, hT


def kda_chunk_fwd_snapshots(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                            beta: torch.Tensor, snap_stride: int,
                            h0: Optional[torch.Tensor] = None,
                            cu_seqlens: Optional[torch.Tensor] = None,
                            snap_offsets: Optional[torch.Tensor] = None,
                            output_final_state: bool = True, o: Optional[torch.Tensor] = None,
                            hT: Optional[torch.Tensor] = None,
                            snaps: Optional[torch.Tensor] = None):
    """Prefill that also saves the state every snap_stride tokens of each sequence (prefix
    caching).  Returns (o, hT, snaps, snap_offsets): snapshot j (1-based) of sequence n, the state
    after its first j * snap_stride tokens, is snaps[snap_offsets[n] + j - 1] (snap_offsets is
    None for equal-length batches, where the index is n * (T // snap_stride) + j - 1).

    With cu_seqlens and no snap_offsets, the offsets are derived from the sequence lengths on the
    device; sizing snaps then reads their total back to the host (one synchronisation), which a
    caller avoids by passing both snap_offsets and snaps."""
    dev, B, T, H, dk, dv, N, o, hT = _prefill_args(q, k, v, g, beta, h0, cu_seqlens,
                                                   output_final_state, o, hT)
    stride = int(snap_stride)
    if stride <= 0 or stride % 16:
        raise KDAError(KDA_ERR_STRIDE, "kda_chunk_fwd_snapshots")
    if cu_seqlens is not None:
        if snap_offsets is None:
            counts = torch.div(cu_seqlens[1:] - cu_seqlens[:-1], stride, rounding_mode="floor")
            snap_offsets = torch.zeros(N + 1, dtype=torch.int32, device=dev)
            snap_offsets[1:] = torch.cumsum(counts, 0)
        _check(snap_offsets, "snap_offsets", dev, torch.int32)
        if snap_offsets.numel() != N + 1:
            raise ValueError(f"snap_offsets must have {N + 1} entries")
        # the kernels write snapshot rows up to snap_offsets[-1]: the buffer must hold them all
        # (reading that count back is one device-to-host synchronisation)
        n_snaps = int(snap_offsets[-1].item()) if N > 0 else 0
        if snaps is None:
            snaps = torch.empty((n_snaps, H, dk, dv), dtype=torch.float32, device=dev)
        elif snaps.dim() != 4 or snaps.shape[0] < n_snaps:
            raise ValueError(f"snaps needs {n_snaps} entries, got {list(snaps.shape)}")
    else:
        if snap_offsets is not None:
            raise ValueError("snap_offsets is only used with cu_seqlens")
        if snaps is None:
            snaps = torch.empty((N * (T // stride), H, dk, dv), dtype=torch.float32, device=dev)
        elif snaps.dim() != 4 or snaps.shape[0] < N * (T // stride):
            raise ValueError(f"snaps needs {N * (T // stride)} entries, got {list(snaps.shape)}")
    _check(snaps, "snaps", dev, torch.float32)
    if snaps.shape[1:] != (H, dk, dv):
        raise ValueError(f"snaps must be [*, {H}, {dk}, {dv}]")
    st = load_library().kda_chunk_fwd_snapshots(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(cu_seqlens), N,
        _ptr(o), _ptr(hT), _ptr(snaps) if snaps.numel() else None, _ptr(snap_offsets), stride,
        B, T, H, dk, dv, _dtype_code(q), _stream(dev))
    if st != KDA_OK:
        raise KDAError(st, "kda_chunk_fwd_snapshots")
    return o, hT, snaps, snap_offsets


def _decode_args(q, k, v, g, beta, S, o):
    dev = q.device
    dt = q.dtype
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta)):
        _check(t, name, dev, dt)
    _check(S, "S", dev, torch.float32)
    if q.dim() != 3:
        raise ValueError("q must be [N, H, dk]")
    N, H, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or g.shape != q.shape or v.shape != (N, H, dv) or beta.shape != (N, H) \
            or S.shape != (N, H, dk, dv):
        raise ValueError("inconsistent decode shapes")
    if o is None:
        o = torch.empty((N, H, dv), dtype=dt, device=dev)
    else:
        _check(o, "o", dev, dt)
        if tuple(o.shape) != (N, H, dv):
            raise ValueError(f"o must be [{N}, {H}, {dv}], got {list(o.shape)}")
    return dev, N, H, dk, dv, o


def kda_decode_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                    beta: torch.Tensor, S: torch.Tensor,
                    o: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One token per sequence: q, k, g [N, H, dk], v [N, H, dv], beta [N, H]; S float32
    [N, H, dk, dv] is updated in place.  Returns o [N, H, dv]."""
    dev, N, H, dk, dv, o = _decode_args(q, k, v, g, beta, S, o)
    st = load_library().kda_decode_step(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S), _ptr(o), N, H, dk, dv,
        _dtype_code(q), _stream(dev))
    if st != KDA_OK:
        raise KDAError(st, "kda_decode_step")
    return o


def _gate_weight(weight, dv, dev):
    if weight is None:
        return None
    _check(weight, "weight", dev, torch.float32)
    if weight.shape != (dv,):
        raise ValueError(f"weight must be [{dv}]")
    return weight


def kda_decode_step_gated(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                          beta: torch.Tensor, S: torch.Tensor, gate: torch.Tensor,
                          weight: Optional[torch.Tensor] = None, eps: float = 1e-6,
                          o: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None
                          ) -> Tuple[torch.Tensor, torch.Tensor]:
    """kda_decode_step followed by the output stage y = RMSNorm(o) * weight * sigmoid(gate) (fused
    into the decode kernel for 128 x 128 heads).  gate [N, H, dv]; weight [dv] float32 or None.
    Returns (o, y)."""
    dev, N, H, dk, dv, o = _decode_args(q, k, v, g, beta, S, o)
    _check(gate, "gate", dev, q.dtype)
    if gate.shape != (N, H, dv):
        raise ValueError("gate must be [N, H, dv]")
    weight = _gate_weight(weight, dv, dev)
    if y is None:
        y = torch.empty_like(o)
    else:
        _check(y, "y", dev, q.dtype)
        if tuple(y.shape) != (N, H, dv):
            raise ValueError(f"y must be [{N}, {H}, {dv}], got {list(y.shape)}")
    st = load_library().kda_decode_step_gated(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S), _ptr(gate), _ptr(weight),
        float(eps), _ptr(o), _ptr(y), N, H, dk, dv, _dtype_code(q), _stream(dev))
    if st != KDA_OK:
        raise KDAError(st, "kda_decode_step_gated")
    return o, y


def kda_output_gate(o: torch.Tensor, gate: torch.Tensor, weight: Optional[torch.Tensor] = None,
                    eps: float = 1e-6, y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The output stage on [..., H, dv] rows: y = o / sqrt(mean(o^2) + eps) * weight *
    sigmoid(gate).  Returns y (may be passed preallocated; may be o itself)."""
    dev = o.device
    _check(o, "o", dev)
    _check(gate, "gate", dev, o.dtype)
    if gate.shape != o.shape or o.dim() < 2:
        raise ValueError("o and gate must have the same [..., H, dv] shape")
    H, dv = o.shape[-2], o.shape[-1]
    rows = o.numel() // (H * dv) if o.numel() else 0
    weight = _gate_weight(weight, dv, dev)
    if y is None:
        y = torch.empty_like(o)
    else:
        _check(y, "y", dev, o.dtype)
        if y.shape != o.shape:
            raise ValueError("y must have o's shape")
    st = load_library().kda_output_gate(_ptr(o), _ptr(gate), _ptr(weight), float(eps), _ptr(y),
                                        rows, H, dv, _dtype_code(o), _stream(dev))
    if st != KDA_OK:
        raise KDAError(st, "kda_output_gate")
    return y


def kda_frontend(x_q: torch.Tensor, x_k: torch.Tensor, x_v: torch.Tensor, x_z: torch.Tensor,
                 x_b: torch.Tensor, w_q: torch.Tensor, w_k: torch.Tensor, w_v: torch.Tensor,
                 z_bias: torch.Tensor, A: torch.Tensor, g_min: float = -5.0, eps: float = 1e-6,
                 cu_seqlens: Optional[torch.Tensor] = None, conv_in: Optional[torch.Tensor] = None,
                 output_conv_state: bool = False, conv_out: Optional[torch.Tensor] = None):
    """The input stage: pre-activations x_q, x_k, x_z [.., H, dk], x_v [.., H, dv], x_b [.., H]
    ([B, T, ...] or packed [Ttot, ...] with cu_seqlens) -> (q, k, v, g, beta, conv_state) in the
    layouts kda_chunk_fwd takes.  Taps w_q, w_k [H*dk, 4], w_v [H*dv, 4], z_bias [H*dk] and A [H]
    are float32.  conv_in / the returned state [N, 3, H*(2dk+dv)] hold the last three inputs of
    every sequence (pass conv_out=conv_in to update it in place); conv_state is None unless
    output_conv_state or conv_out is given."""
    dev = x_q.device
    dt = x_q.dtype
    for name, t in (("x_q", x_q), ("x_k", x_k), ("x_v", x_v), ("x_z", x_z), ("x_b", x_b)):
        _check(t, name, dev, dt)
    if x_q.dim() == 4:
        if cu_seqlens is not None:
            raise ValueError("cu_seqlens needs packed [Ttot, H, d] inputs")
        B, T, H, dk = x_q.shape
        lead = (B, T)
    elif x_q.dim() == 3:
        T, H, dk = x_q.shape
        B = 1
        lead = (T,)
    else:
        raise ValueError("x_q must be [B, T, H, dk] or [Ttot, H, dk]")
    dv = x_v.shape[-1]
    if x_k.shape != x_q.shape or x_z.shape != x_q.shape or x_v.shape != (*lead, H, dv) \
            or x_b.shape != (*lead, H):
        raise ValueError("inconsistent pre-activation shapes")
    for name, t, shape in (("w_q", w_q, (H * dk, 4)), ("w_k", w_k, (H * dk, 4)),
                           ("w_v", w_v, (H * dv, 4)), ("z_bias", z_bias, (H * dk,)),
                           ("A", A, (H,))):
        _check(t, name, dev, torch.float32)
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} must be {list(shape)}")
    if cu_seqlens is not None:
        _check(cu_seqlens, "cu_seqlens", dev, torch.int32)
        N = cu_seqlens.numel() - 1
    else:
        N = B
    C = H * (2 * dk + dv)
    if conv_in is not None:
        _check(conv_in, "conv_in", dev, dt)
        if tuple(conv_in.shape) != (N, 3, C):
            raise ValueError(f"conv_in must be [{N}, 3, {C}]")
    if conv_out is None and output_conv_state:
        conv_out = torch.empty((N, 3, C), dtype=dt, device=dev)
    if conv_out is not None:
        _check(conv_out, "conv_out", dev, dt)
        if tuple(conv_out.shape) != (N, 3, C):
            raise ValueError(f"conv_out must be [{N}, 3, {C}]")
    q = torch.empty_like(x_q)
    k = torch.empty_like(x_k)
    v = torch.empty_like(x_v)
    g = torch.empty_like(x_z)
    beta = torch.empty_like(x_b)
    st = load_library().kda_frontend(
        _ptr(x_q), _ptr(x_k), _ptr(x_v), _ptr(x_z), _ptr(x_b), _ptr(w_q), _ptr(w_k), _ptr(w_v),
        _ptr(z_bias), _ptr(A), float(g_min), float(eps), _ptr(cu_seqlens), N, _ptr(conv_in),
        _ptr(conv_out), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), B, T, H, dk, dv,
        _dtype_code(x_q), _stream(dev))
    if st != KDA_OK:
        raise KDAError(st, "kda_frontend")
    return q, k, v, g, beta, conv_out


def kda_decode_step_layer(x_q: torch.Tensor, x_k: torch.Tensor, x_v: torch.Tensor,
                          x_z: torch.Tensor, x_b: torch.Tensor, w_q: torch.Tensor,
                          w_k: torch.Tensor, w_v: torch.Tensor, z_bias: torch.Tensor,
                          A: torch.Tensor, conv_state: torch.Tensor, S: torch.Tensor,
                          gate: torch.Tensor, weight: Optional[torch.Tensor] = None,
                          g_min: float = -5.0, norm_eps: float = 1e-6, eps: float = 1e-6,
                          want_o: bool = False, o: Optional[torch.Tensor] = None,
                          y: Optional[torch.Tensor] = None
                          ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """The whole token mixer for one token per sequence in one launch: the input stage (the
    convolution state [N, 3, H*(2dk+dv)] updated in place), the decode step (S [N, H, dk, dv]
    float32 updated in place) and the output stage.  x_q, x_k, x_z [N, H, dk], x_v [N, H, dv],
    x_b [N, H] and gate [N, H, dv] in one dtype; taps, z_bias, A and weight float32 as in
    kda_frontend and kda_decode_step_gated.  dk = dv = 128.  Returns (y, o); o is None unless
    want_o is set or o is passed."""
    dev = x_q.device
    dt = x_q.dtype
    for name, t in (("x_q", x_q), ("x_k", x_k), ("x_v", x_v), ("x_z", x_z), ("x_b", x_b),
                    ("gate", gate), ("conv_state", conv_state)):
        _check(t, name, dev, dt)
    if x_q.dim() != 3:
        raise ValueError("x_q must be [N, H, dk]")
    N, H, dk = x_q.shape
    dv = x_v.shape[-1]
    if x_k.shape != x_q.shape or x_z.shape != x_q.shape or x_v.shape != (N, H, dv) \
            or x_b.shape != (N, H) or gate.shape != (N, H, dv):
        raise ValueError("inconsistent pre-activation or gate shapes")
    if tuple(conv_state.shape) != (N, 3, H * (2 * dk + dv)):
        raise ValueError(f"conv_state must be [{N}, 3, {H * (2 * dk + dv)}]")
    _check(S, "S", dev, torch.float32)
    if tuple(S.shape) != (N, H, dk, dv):
        raise ValueError(f"S must be [{N}, {H}, {dk}, {dv}]")
    for name, t, shape in (("w_q", w_q, (H * dk, 4)), ("w_k", w_k, (H * dk, 4)),
                           ("w_v", w_v, (H * dv, 4)), ("z_bias", z_bias, (H * dk,)),
                           ("A", A, (H,))):
        _check(t, name, dev, torch.float32)
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} must be {list(shape)}")
    weight = _gate_weight(weight, dv, dev)
    for name in ("o", "y"):
        t = o if name == "o" else y
        if t is not None:
            _check(t, name, dev, dt)
            if tuple(t.shape) != (N, H, dv):
                raise ValueError(f"{name} must be [{N}, {H}, {dv}], got {list(t.shape)}")
    if o is None and want_o:
        o = torch.empty((N, H, dv), dtype=dt, device=dev)
    if y is None:
        y = torch.empty((N, H, dv), dtype=dt, device=dev)
    st = load_library().kda_decode_step_layer(
        _ptr(x_q), _ptr(x_k), _ptr(x_v), _ptr(x_z), _ptr(x_b), _ptr(w_q), _ptr(w_k), _ptr(w_v),
        _ptr(z_bias), _ptr(A), float(g_min), float(norm_eps), _ptr(conv_state), _ptr(S),
        _ptr(gate), _ptr(weight), float(eps), _ptr(o), _ptr(y), N, H, dk, dv, _dtype_code(x_q),
        _stream(dev))
    if st != KDA_OK:
        raise KDAError(st, "kda_decode_step_layer")
    return y, o
