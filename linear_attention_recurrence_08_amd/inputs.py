"""Seeded synthetic KDA workloads.

This module only draws random inputs; it holds none of the recurrence's arithmetic.  It is the one
piece shared by the CPU oracle's tests and the GPU path's tests and benchmark, so both sides see the
exact same numbers: every tensor is drawn in float32 with numpy's PCG64, prepared (L2 norm of q and
k, sigmoid for beta, the gate recipe for g = log alpha), then rounded once to the dtype the GPU
receives.  The oracle upcasts those rounded values to float64.

Shapes follow the K3 KDA layer described in "Kimi K3's hybrid block, from first principles"
(section "From linear attention to the delta rule", paragraph "What the state costs"): 96 heads,
a 128 x 128 state per head.  Layouts are token-major and packed:

    q, k, g : [Ttot, H, dk]      v, o : [Ttot, H, dv]      beta : [Ttot, H]
    h0, hT  : [N, H, dk, dv] float32 (N sequences)

with Ttot = B * T for equal-length batches, or the sum of the sequence lengths for a packed
variable-length batch described by cu_seqlens (int32 [N + 1]).

Draw order, fixed for reproducibility: every block of BLOCK_TOKENS packed tokens has its own PCG64
stream, seeded by SeedSequence([seed, block]), from which q, k, v, the beta logits and the gate
noise are drawn in that order; sequence i's initial state comes from SeedSequence([seed, 10**6 + i])
and variable-length batches draw their lengths from SeedSequence([seed, 2 * 10**6]).  Independent
streams let the blocks be drawn in parallel threads with a result that does not depend on the
thread count.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional, Sequence

import numpy as np
import torch

BLOCK_TOKENS = 2048  # token block of the draw order (one random stream per block)
H0_STREAM = 10 ** 6
LEN_STREAM = 2 * 10 ** 6

GATE_RECIPES = ("sigmoid", "sigmoid_shift1", "sigmoid_shiftm1", "bimodal", "zero", "floor",
                "floor_half")
BETA_RECIPES = ("sigmoid", "zero", "one")


@dataclasses.dataclass
class KDAInputs:
    """One synthetic batch, as host tensors in the dtype the GPU receives."""

    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    g: torch.Tensor
    beta: torch.Tensor
    h0: Optional[torch.Tensor]
    cu_seqlens: Optional[torch.Tensor]  # int32 [N+1] or None (equal lengths)
    B: int
    T: int  # per-sequence length when cu_seqlens is None, else the packed total
    H: int
    dk: int
    dv: int
    dtype: str  # "bf16" | "f32"
    name: str = ""

    @property
    def num_seqs(self) -> int:
        return self.B if self.cu_seqlens is None else int(self.cu_seqlens.numel() - 1)

    @property
    def total_tokens(self) -> int:
        return int(self.q.shape[0])

    def seq_bounds(self):
        """(start, end) token indices of every sequence in the packed layout."""
        if self.cu_seqlens is None:
            return [(b * self.T, (b + 1) * self.T) for b in range(self.B)]
        cu = self.cu_seqlens.tolist()
        return [(cu[i], cu[i + 1]) for i in range(len(cu) - 1)]

    def call_views(self):
        """(q, k, v, g, beta) shaped for the binding: [B, T, H, d] for equal-length batches,
        packed [Ttot, H, d] when cu_seqlens describes the sequences."""
        if self.cu_seqlens is not None:
            return self.q, self.k, self.v, self.g, self.beta
        B, T = self.B, self.T
        return (self.q.view(B, T, *self.q.shape[1:]), self.k.view(B, T, *self.k.shape[1:]),
                self.v.view(B, T, *self.v.shape[1:]), self.g.view(B, T, *self.g.shape[1:]),
                self.beta.view(B, T, *self.beta.shape[1:]))

    def to(self, device) -> "KDAInputs":
        f = lambda t: None if t is None else t.to(device)
        return dataclasses.replace(
            self, q=f(self.q), k=f(self.k), v=f(self.v), g=f(self.g), beta=f(self.beta),
            h0=f(self.h0), cu_seqlens=f(self.cu_seqlens))


def _torch_dtype(dtype: str):
    if dtype == "bf16":
        return torch.bfloat16
    if dtype == "f32":
        return torch.float32
    raise ValueError(f"unknown dtype {dtype!r}")


def _stream(seed: int, index: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), int(index)])))


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(8, n))


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return (1.0 / (1.0 + np.exp(-x))).astype(np.float32)


def _l2_normalise(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32))
    return (x / np.maximum(n, np.float32(1e-30))).astype(np.float32)


def _gate(z: np.ndarray, recipe: str) -> np.ndarray:
    """g = log(alpha) from standard-normal noise z, per the workload recipe; values in [-5, 0]."""
    if recipe == "sigmoid":          # -5 * sigmoid(N(0,1))
        return (-5.0 * _sigmoid(z)).astype(np.float32)
    if recipe == "sigmoid_shift1":   # -5 * sigmoid(N(1,1)), as the varlen workload states it
        return (-5.0 * _sigmoid(z + 1.0)).astype(np.float32)
    if recipe == "sigmoid_shiftm1":  # -5 * sigmoid(N(-1,1)): slower decay, long carries
        return (-5.0 * _sigmoid(z - 1.0)).astype(np.float32)
    if recipe == "bimodal":          # half the key channels slow (-0.005), half fast (-4.5)
        dk = z.shape[-1]
        centre = np.where(np.arange(dk) < dk // 2, np.float32(-0.005), np.float32(-4.5))
        return np.clip(centre + np.float32(0.01) * z, -5.0, 0.0).astype(np.float32)
    if recipe == "zero":             # alpha = 1 everywhere
        return np.zeros_like(z, dtype=np.float32)
    if recipe == "floor":            # every channel at the log-decay floor -5 (exact in bf16)
        return np.full_like(z, -5.0, dtype=np.float32)
    if recipe == "floor_half":       # key channels [0, dk/2) at the floor, the rest at 0
        dk = z.shape[-1]
        row = np.where(np.arange(dk) < dk // 2, np.float32(-5.0), np.float32(0.0))
        return np.broadcast_to(row, z.shape).astype(np.float32)
    raise ValueError(f"unknown gate recipe {recipe!r}")


def _beta(b: np.ndarray, recipe: str) -> np.ndarray:
    """beta from standard-normal noise b: sigmoid(N(0,1)), or the constants 0 and 1."""
    if recipe == "sigmoid":
        return _sigmoid(b)
    if recipe == "zero":
        return np.zeros_like(b, dtype=np.float32)
    if recipe == "one":
        return np.ones_like(b, dtype=np.float32)
    raise ValueError(f"unknown beta recipe {recipe!r}")


def make_inputs(seq_lens: Sequence[int], H: int, dk: int, dv: int, dtype: str, seed: int,
                gate: str = "sigmoid", h0_sigma: Optional[float] = None,
                packed: Optional[bool] = None, name: str = "",
                beta: str = "sigmoid") -> KDAInputs:
    """Draw one batch.

    seq_lens: the sequence lengths.  With packed=False (default when all lengths are equal) the
    batch is B equal-length sequences without cu_seqlens; otherwise it is one packed batch with
    cu_seqlens.  h0_sigma None means h0 = zeros (passed as None).  gate and beta name the
    recipes for g (GATE_RECIPES) and beta (BETA_RECIPES); the draw order does not depend on
    them, so two recipes give the same q, k and v.
    """
    beta_recipe = beta
    seq_lens = [int(s) for s in seq_lens]
    if packed is None:
        packed = len(set(seq_lens)) > 1
    if not packed and len(set(seq_lens)) > 1:
        raise ValueError("unequal lengths need packed=True")
    tdt = _torch_dtype(dtype)
    ttot = int(sum(seq_lens))
    q = torch.empty((ttot, H, dk), dtype=tdt)
    k = torch.empty((ttot, H, dk), dtype=tdt)
    v = torch.empty((ttot, H, dv), dtype=tdt)
    g = torch.empty((ttot, H, dk), dtype=tdt)
    beta_t = torch.empty((ttot, H), dtype=tdt)

    def draw_block(b):
        t0 = b * BLOCK_TOKENS
        n = min(BLOCK_TOKENS, ttot - t0)
        rng = _stream(seed, b)
        qb = rng.standard_normal((n, H, dk), dtype=np.float32)
        kb = rng.standard_normal((n, H, dk), dtype=np.float32)
        vb = rng.standard_normal((n, H, dv), dtype=np.float32)
        bb = rng.standard_normal((n, H), dtype=np.float32)
        zb = rng.standard_normal((n, H, dk), dtype=np.float32)
        q[t0:t0 + n] = torch.from_numpy(_l2_normalise(qb)).to(tdt)
        k[t0:t0 + n] = torch.from_numpy(_l2_normalise(kb)).to(tdt)
        v[t0:t0 + n] = torch.from_numpy(vb).to(tdt)
        beta_t[t0:t0 + n] = torch.from_numpy(_beta(bb, beta_recipe)).to(tdt)
        g[t0:t0 + n] = torch.from_numpy(_gate(zb, gate)).to(tdt)

    N = len(seq_lens)
    h0 = None
    if h0_sigma is not None:
        h0 = torch.empty((N, H, dk, dv), dtype=torch.float32)

    def draw_h0(i):
        rng = _stream(seed, H0_STREAM + i)
        h0[i] = torch.from_numpy(
            rng.standard_normal((H, dk, dv), dtype=np.float32) * np.float32(h0_sigma))

    nblocks = (ttot + BLOCK_TOKENS - 1) // BLOCK_TOKENS
    with ThreadPoolExecutor(max_workers=_workers()) as ex:
        list(ex.map(draw_block, range(nblocks)))
        if h0 is not None:
            list(ex.map(draw_h0, range(N)))
    if packed:
        cu = torch.tensor(np.concatenate([[0], np.cumsum(seq_lens)]), dtype=torch.int32)
        return KDAInputs(q, k, v, g, beta_t, h0, cu, 1, ttot, H, dk, dv, dtype, name)
    B = N
    T = seq_lens[0] if N else 0
    return KDAInputs(q, k, v, g, beta_t, h0, None, B, T, H, dk, dv, dtype, name)


def varlen_lengths(seed: int, n: int = 16, lo: int = 1024, hi: int = 16384):
    """Sequence lengths uniform on [lo, hi] (inclusive) from the workload's length stream."""
    rng = _stream(seed, LEN_STREAM)
    return rng.integers(lo, hi, size=n, endpoint=True).tolist()


# Named workloads.  Index = seed.
WORKLOADS = {
    # tiny fp32 forward: B=1, H=2, T=64, dk=dv=32, h0 = 0
    "tiny_T64_H2_d32_f32": dict(kind="prefill", seq_lens=[64], H=2, dk=32, dv=32, dtype="f32",
                                seed=0, gate="sigmoid", h0_sigma=None),
    # one K3 KDA layer, prefill: B=1, T=4096, H=96, d=128, bf16, h0 = 0
    "prefill_T4096_H96_d128_bf16": dict(kind="prefill", seq_lens=[4096], H=96, dk=128, dv=128,
                                        dtype="bf16", seed=1, gate="sigmoid", h0_sigma=None),
    # packed variable-length prefill: 16 sequences of U[1024, 16384] tokens, h0 ~ N(0, 0.02)
    "varlen_16seq_H96_d128_bf16": dict(kind="varlen", n_seqs=16, H=96, dk=128, dv=128,
                                       dtype="bf16", seed=2, gate="sigmoid_shift1",
                                       h0_sigma=0.02),
    # long-context prefill: B=1, T=131072, bimodal per-channel decay
    "long_T131072_H96_d128_bf16": dict(kind="prefill", seq_lens=[131072], H=96, dk=128, dv=128,
                                       dtype="bf16", seed=3, gate="bimodal", h0_sigma=None),
    # batched decode: 256 sequences x 1 token, S ~ N(0, 0.05) read and written in place
    "decode_N256_H96_d128_bf16": dict(kind="decode", N=256, H=96, dk=128, dv=128, dtype="bf16",
                                      seed=4, gate="sigmoid", s_sigma=0.05),
}


def make_workload(name: str, gate: Optional[str] = None) -> KDAInputs:
    """Build a named workload on the host.  gate overrides the gate recipe (parity variants)."""
    w = dict(WORKLOADS[name])
    gate = gate or w["gate"]
    kind = w["kind"]
    if kind == "prefill":
        return make_inputs(w["seq_lens"], w["H"], w["dk"], w["dv"], w["dtype"], w["seed"],
                           gate=gate, h0_sigma=w["h0_sigma"], packed=False, name=name)
    if kind == "varlen":
        lens = varlen_lengths(w["seed"], w["n_seqs"])
        return make_inputs(lens, w["H"], w["dk"], w["dv"], w["dtype"], w["seed"],
                           gate=gate, h0_sigma=w["h0_sigma"], packed=True, name=name)
    if kind == "decode":
        return make_decode_inputs(w["N"], w["H"], w["dk"], w["dv"], w["dtype"], w["seed"],
                                  gate=gate, s_sigma=w["s_sigma"], name=name)
    raise ValueError(kind)


def make_decode_inputs(N: int, H: int, dk: int, dv: int, dtype: str, seed: int,
                       gate: str = "sigmoid", s_sigma: float = 0.05, name: str = "") -> KDAInputs:
    """One token for each of N sequences plus their float32 states S [N, H, dk, dv] (in h0)."""
    inp = make_inputs([1] * N, H, dk, dv, dtype, seed, gate=gate, h0_sigma=s_sigma,
                      packed=False, name=name)
    return inp


def make_output_gate_inputs(Ttot: int, H: int, dv: int, dtype: str, seed: int):
    """Inputs of the output stage: rows o [Ttot, H, dv] ~ N(0, 0.3^2) (the scale of a mixer output;
    the stage is scale-free), gate logits [Ttot, H, dv] ~ N(0, 1) (a full-rank projection of the
    token) and the norm's gain [dv] = 1 + 0.1 N(0, 1) in float32.  Streams SeedSequence([seed,
    3 * 10**6 + i]) for i = 0 (o), 1 (gate), 2 (gain).  Returns CPU tensors (o, gate, weight)."""
    shape = (int(Ttot), int(H), int(dv))
    o = (_stream(seed, 3 * 10**6).standard_normal(shape, dtype=np.float32) * np.float32(0.3))
    z = _stream(seed, 3 * 10**6 + 1).standard_normal(shape, dtype=np.float32)
    w = (1.0 + 0.1 * _stream(seed, 3 * 10**6 + 2).standard_normal(dv)).astype(np.float32)
    td = _torch_dtype(dtype)
    return (torch.from_numpy(o).to(td), torch.from_numpy(z).to(td), torch.from_numpy(w))


@dataclasses.dataclass
class FrontInputs:
    """Inputs of the input stage (pre-activations, taps, bias, per-head scale) on the CPU."""
    x_q: torch.Tensor
    x_k: torch.Tensor
    x_v: torch.Tensor
    x_z: torch.Tensor
    x_b: torch.Tensor
    w_q: torch.Tensor
    w_k: torch.Tensor
    w_v: torch.Tensor
    z_bias: torch.Tensor
    A: torch.Tensor
    cu_seqlens: Optional[torch.Tensor]
    conv_in: Optional[torch.Tensor]

    def to(self, dev) -> "FrontInputs":
        f = lambda t: None if t is None else t.to(dev)
        return FrontInputs(*(f(getattr(self, fl.name)) for fl in dataclasses.fields(self)))


def make_frontend_inputs(seq_lens: Sequence[int], H: int, dk: int, dv: int, dtype: str,
                         seed: int, with_state: bool = False) -> FrontInputs:
    """Pre-activations x_q, x_k, x_v, x_z ~ N(0, 1) and x_b ~ N(0, 1) (projection outputs), packed
    [Ttot, H, d] with cu_seqlens; taps ~ U(-1/2, 1/2) (the usual width-4 convolution scale); the
    decay bias ~ N(0, 1/4); A_h ~ U(1/2, 2); with_state adds a saved convolution state ~ N(0, 1)
    [N, 3, H (2 dk + dv)].  Streams SeedSequence([seed, 4 * 10**6 + i])."""
    lens = [int(x) for x in seq_lens]
    Ttot, N = sum(lens), len(lens)
    td = _torch_dtype(dtype)
    r = lambda i, *shape: _stream(seed, 4 * 10**6 + i).standard_normal(shape, dtype=np.float32)
    u = lambda i, lo, hi, *shape: _stream(seed, 4 * 10**6 + i).uniform(lo, hi, shape).astype(
        np.float32)
    t = lambda a, dt=td: torch.from_numpy(np.ascontiguousarray(a)).to(dt)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
    C = H * (2 * dk + dv)
    return FrontInputs(
        x_q=t(r(0, Ttot, H, dk)), x_k=t(r(1, Ttot, H, dk)), x_v=t(r(2, Ttot, H, dv)),
        x_z=t(r(3, Ttot, H, dk)), x_b=t(r(4, Ttot, H)),
        w_q=t(u(5, -0.5, 0.5, H * dk, 4), torch.float32),
        w_k=t(u(6, -0.5, 0.5, H * dk, 4), torch.float32),
        w_v=t(u(7, -0.5, 0.5, H * dv, 4), torch.float32),
        z_bias=t(0.5 * r(8, H * dk), torch.float32), A=t(u(9, 0.5, 2.0, H), torch.float32),
        cu_seqlens=cu, conv_in=t(r(10, N, 3, C)) if with_state else None)
