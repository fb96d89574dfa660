"""KDA oracle, Python side: the C float64 recurrence plus three independent forms used to pin it.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this module.  It shares no code with the HIP path (no kernels, headers, helpers or
constants) and never imports the product package.

Functions
---------
recurrence(...)   the plain token-by-token recurrence in float64 (C, threads over
                  (sequence, head)); the oracle every GPU result is compared with.
decode_step(...)  one token for each of N sequences: the recurrence with length-1 sequences.
chunked(...)      an independent chunkwise form (numpy float64): parallel inside C-token tiles,
                  recurrent across tiles.
brute_force(...)  the unrolled sum of explicit dk x dk transition products (tiny inputs only).
exact(...)        the recurrence in exact rational arithmetic (fractions.Fraction; tiny inputs).
output_gate(...)  the output stage after the mixer: per-head RMSNorm times a sigmoid gate.
frontend(...)     the input stage before the mixer: short convolution, Swish, L2 norm, the sigmoid
                  write strength and the bounded log-decay.

The recurrence these compute (decay first, then erase-and-write, then read the updated state):
    S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,   o_t = S_t^T q_t,
with alpha_t = exp(g_t) one retention factor per key channel.  Sources: "Kimi K3's hybrid block,
from first principles", section "From linear attention to the delta rule"; "Kimi K3, explained",
section "Kimi Delta Attention: making the radical option work"; "What's new in Kimi K3", section
"KDA in one page".  The C file states the recurrence step by step.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from fractions import Fraction
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_kda.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with the host compiler (plain IEEE float64: no fast-math, no FMA
    contraction, so every operation rounds exactly once in program order)."""
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fPIC",
               "-shared", "-pthread", _SRC, "-o", _LIB + ".tmp", "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def load_library(path: str):
    """Open a compiled oracle library (the default one, or a test-built variant)."""
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    lib.kda_oracle_recurrence.argtypes = [dp, dp, dp, dp, dp, dp,
                                          ctypes.POINTER(ctypes.c_int64), ctypes.c_int64,
                                          ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                          ctypes.c_int, dp, dp, ctypes.c_int]
    lib.kda_oracle_recurrence.restype = ctypes.c_int
    lib.kda_oracle_recurrence_snap.argtypes = [dp, dp, dp, dp, dp, dp,
                                               ctypes.POINTER(ctypes.c_int64), ctypes.c_int64,
                                               ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                               ctypes.c_int, dp, dp, ctypes.c_int64,
                                               ctypes.POINTER(ctypes.c_int64), dp, ctypes.c_int]
    lib.kda_oracle_recurrence_snap.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        variant = os.environ.get("KDA_ORACLE_LIB")   # a test-built variant (sanitizer runs)
        if variant:
            _lib = load_library(variant)
        else:
            if not os.path.exists(_LIB):
                build(force=True)
            _lib = load_library(_LIB)
    return _lib


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def recurrence(q, k, v, g, beta, h0=None, cu_seqlens: Optional[Sequence[int]] = None,
               gate_is_alpha: bool = False, nthreads: Optional[int] = None, lib=None,
               snapshot_stride: Optional[int] = None):
    """The token-by-token recurrence in float64.

    q, k, g: [Ttot, H, dk]; v: [Ttot, H, dv]; beta: [Ttot, H]; h0: [N, H, dk, dv] or None
    (zeros).  cu_seqlens: [N+1] sequence boundaries in the packed token axis; None means one
    sequence over all Ttot tokens.  lib: a library from load_library (default: the built one).
    Returns (o [Ttot, H, dv], hT [N, H, dk, dv]), and with snapshot_stride = s also
    (snaps [sum_n len_n // s, H, dk, dv], snap_cu [N+1]): the state after token j*s of sequence n
    (j = 1 .. len_n // s) is snaps[snap_cu[n] + j - 1], the state that resumes that prefix
    ("Kimi K3's hybrid block, from first principles", paragraph "The cache, in bytes").
    """
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    g = np.ascontiguousarray(g, dtype=np.float64)
    beta = np.ascontiguousarray(beta, dtype=np.float64)
    Ttot, H, dk = q.shape
    dv = v.shape[2]
    if k.shape != q.shape or g.shape != q.shape or v.shape[:2] != (Ttot, H) \
            or beta.shape != (Ttot, H):
        raise ValueError("shape mismatch")
    cu = np.asarray([0, Ttot] if cu_seqlens is None else cu_seqlens, dtype=np.int64)
    N = cu.size - 1
    if cu[0] != 0 or cu[-1] != Ttot or np.any(np.diff(cu) < 0):
        raise ValueError("bad cu_seqlens")
    if h0 is not None:
        h0 = np.ascontiguousarray(h0, dtype=np.float64)
        if h0.shape != (N, H, dk, dv):
            raise ValueError("h0 shape")
    o = np.zeros((Ttot, H, dv), dtype=np.float64)
    hT = np.zeros((N, H, dk, dv), dtype=np.float64)
    stride = int(snapshot_stride or 0)
    if stride < 0:
        raise ValueError("snapshot_stride must be positive")
    snap_cu = np.zeros(N + 1, dtype=np.int64)
    if stride:
        snap_cu[1:] = np.cumsum(np.diff(cu) // stride)
    snaps = np.zeros((int(snap_cu[-1]), H, dk, dv), dtype=np.float64)
    st = (lib or _load()).kda_oracle_recurrence_snap(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0),
        cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), N, H, dk, dv,
        1 if gate_is_alpha else 0, _ptr(o), _ptr(hT), stride,
        snap_cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), _ptr(snaps),
        nthreads or default_threads())
    if st != 0:
        raise RuntimeError(f"oracle failed with status {st}")
    if stride:
        return o, hT, snaps, snap_cu
    return o, hT


def decode_step(q, k, v, g, beta, S, nthreads: Optional[int] = None):
    """One token per sequence: q,k,g [N,H,dk], v [N,H,dv], beta [N,H], S [N,H,dk,dv].
    Returns (o [N,H,dv], S_new [N,H,dk,dv]); the input S is not modified."""
    N = q.shape[0]
    return recurrence(q, k, v, g, beta, h0=S, cu_seqlens=np.arange(N + 1), nthreads=nthreads)


# ---------------------------------------------------------------------------------------------
# Independent chunkwise form.  Follows "Kimi K3's hybrid block, from first principles", section
# "From linear attention to the delta rule" (the tokens of a chunk are handled together and a state
# is passed from chunk to chunk; the cumulative log-decay is taken over a 16-token tile) and "Kimi K3", section
# "Forgetting different features at different rates" (the chunked algorithm gives the same
# result as the token loop).
#
# Inside a tile with entering state S and inclusive per-channel cumulative log-decay
# Gam_i = sum_{j<=i} g_j, unrolling the recurrence gives
#     S_i = Diag(e^{Gam_i}) S + sum_{j<=i} Diag(e^{Gam_i - Gam_j}) k_j u_j^T
# where u_j = beta_j (v_j - S'_j^T k_j) are the written errors.  Collecting the u's:
#     (I + Diag(beta) A) U = Diag(beta) (V - (K.e^Gam) S),  A_ij = sum_c k_ic k_jc e^{Gam_ic-Gam_jc}
# for j < i (strictly lower), then
#     O = (Q.e^Gam) S + P U,   P_ij = sum_c q_ic k_jc e^{Gam_ic-Gam_jc} for j <= i,
#     S <- Diag(e^{Gam_C}) S + (K.e^{Gam_C - Gam})^T U.
# ---------------------------------------------------------------------------------------------
def _chunk_one(Q, K, V, G, b, S, C, gate_is_alpha):
    Tn, dk = K.shape
    O = np.zeros((Tn, V.shape[1]))
    for t0 in range(0, Tn, C):
        t1 = min(Tn, t0 + C)
        Qc, Kc, Vc, bc = Q[t0:t1], K[t0:t1], V[t0:t1], b[t0:t1]
        if gate_is_alpha:
            eG = np.cumprod(G[t0:t1], axis=0)          # e^{Gam}
            eGinv = 1.0 / eG                            # e^{-Gam}
            eC = eG[-1]                                 # e^{Gam_C}
            eCm = eC[None, :] / eG                      # e^{Gam_C - Gam}
        else:
            Gam = np.cumsum(G[t0:t1], axis=0)
            eG, eGinv = np.exp(Gam), np.exp(-Gam)
            eC = np.exp(Gam[-1])
            eCm = np.exp(Gam[-1][None, :] - Gam)
        Kp, Kn, Qp = Kc * eG, Kc * eGinv, Qc * eG
        L = t1 - t0
        A = np.tril(Kp @ Kn.T, -1)
        P = np.tril(Qp @ Kn.T, 0)
        rhs = bc[:, None] * (Vc - Kp @ S)
        M = np.eye(L) + bc[:, None] * A
        U = np.zeros_like(rhs)
        for i in range(L):                              # forward substitution (unit lower)
            U[i] = rhs[i] - M[i, :i] @ U[:i]
        O[t0:t1] = Qp @ S + P @ U
        S = eC[:, None] * S + (Kc * eCm).T @ U
    return O, S


def chunked(q, k, v, g, beta, h0=None, cu_seqlens=None, chunk: int = 16,
            gate_is_alpha: bool = False):
    """Chunkwise evaluation (float64 numpy), tiles restarting at every sequence start."""
    q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
    Ttot, H, dk = q.shape
    dv = v.shape[2]
    cu = [0, Ttot] if cu_seqlens is None else [int(c) for c in cu_seqlens]
    N = len(cu) - 1
    o = np.zeros((Ttot, H, dv))
    hT = np.zeros((N, H, dk, dv))
    for n in range(N):
        a, e = cu[n], cu[n + 1]
        for h in range(H):
            S = np.zeros((dk, dv)) if h0 is None else np.array(h0[n, h], dtype=np.float64)
            O, S = _chunk_one(q[a:e, h], k[a:e, h], v[a:e, h], g[a:e, h], beta[a:e, h], S,
                              chunk, gate_is_alpha)
            o[a:e, h] = O
            hT[n, h] = S
    return o, hT


# ---------------------------------------------------------------------------------------------
# Brute force: the unrolled sum of explicit transition products, for tiny inputs.
#     M_i = (I - beta_i k_i k_i^T) Diag(alpha_i)
#     S_t = (M_t ... M_1) h0 + sum_{j<=t} (M_t ... M_{j+1}) beta_j k_j v_j^T,   o_t = S_t^T q_t
# Written with plain Python lists so that it runs on floats and on Fractions alike.
# ---------------------------------------------------------------------------------------------
def _mat_mul(X, Y):
    n, m, p = len(X), len(Y), len(Y[0])
    return [[sum((X[i][l] * Y[l][j] for l in range(m)), X[i][0] * 0) for j in range(p)]
            for i in range(n)]


def _eye(n, one):
    return [[one if i == j else one * 0 for j in range(n)] for i in range(n)]


def _brute_one(qs, ks, vs, alphas, bs, h0, one):
    T = len(ks)
    dk, dv = len(ks[0]) if T else len(h0), len(h0[0])
    M = []
    for i in range(T):
        Mi = [[((one if r == c else one * 0) - bs[i] * ks[i][r] * ks[i][c]) * alphas[i][c]
               for c in range(dk)] for r in range(dk)]
        M.append(Mi)
    outs = []
    S = None
    for t in range(T):
        # prefix products Phi_{t,j} = M_t ... M_{j+1}, built from j = t downwards
        Phi = _eye(dk, one)
        acc = [[one * 0 for _ in range(dv)] for _ in range(dk)]
        for j in range(t, -1, -1):
            wj = [[bs[j] * ks[j][r] * vs[j][c] for c in range(dv)] for r in range(dk)]
            contrib = _mat_mul(Phi, wj)
            acc = [[acc[r][c] + contrib[r][c] for c in range(dv)] for r in range(dk)]
            Phi = _mat_mul(Phi, M[j])
        base = _mat_mul(Phi, h0)  # Phi = M_t ... M_1
        S = [[acc[r][c] + base[r][c] for c in range(dv)] for r in range(dk)]
        outs.append([sum((S[r][c] * qs[t][r] for r in range(dk)), one * 0) for c in range(dv)])
    if S is None:
        S = [row[:] for row in h0]
    return outs, S


def brute_force(q, k, v, g, beta, h0=None, cu_seqlens=None, gate_is_alpha: bool = False,
                exact_rational: bool = False):
    """Unrolled transition-product form.  Inputs are nested sequences or arrays of shape
    [Ttot, H, d]; with exact_rational the values must be Fractions (or ints) and alpha must be
    passed directly (gate_is_alpha=True).  Returns (o, hT) as nested lists [Ttot][H][dv] and
    [N][H][dk][dv]."""
    one = Fraction(1) if exact_rational else 1.0
    conv = (lambda x: Fraction(x)) if exact_rational else float
    q, k, v, g, beta = (np.asarray(x, dtype=object) for x in (q, k, v, g, beta))
    Ttot, H, dk = q.shape
    dv = v.shape[2]
    cu = [0, Ttot] if cu_seqlens is None else [int(c) for c in cu_seqlens]
    N = len(cu) - 1
    o = [[None] * H for _ in range(Ttot)]
    hT = [[None] * H for _ in range(N)]
    for n in range(N):
        a, e = cu[n], cu[n + 1]
        for h in range(H):
            qs = [[conv(q[t, h, r]) for r in range(dk)] for t in range(a, e)]
            ks = [[conv(k[t, h, r]) for r in range(dk)] for t in range(a, e)]
            vs = [[conv(v[t, h, c]) for c in range(dv)] for t in range(a, e)]
            if gate_is_alpha:
                al = [[conv(g[t, h, r]) for r in range(dk)] for t in range(a, e)]
            else:
                al = [[float(np.exp(float(g[t, h, r]))) for r in range(dk)] for t in range(a, e)]
            bs = [conv(beta[t, h]) for t in range(a, e)]
            S0 = [[(conv(h0[n][h][r][c]) if h0 is not None else one * 0) for c in range(dv)]
                  for r in range(dk)]
            outs, S = _brute_one(qs, ks, vs, al, bs, S0, one)
            for i, t in enumerate(range(a, e)):
                o[t][h] = outs[i]
            hT[n][h] = S
    return o, hT


def exact(q, k, v, alpha, beta, h0=None, cu_seqlens=None):
    """The recurrence in exact rational arithmetic (alpha given directly, as Fractions or
    dyadic floats).  Token-by-token: fade, error, write, read.  Returns nested lists."""
    F = Fraction
    q, k, v, alpha, beta = (np.asarray(x, dtype=object) for x in (q, k, v, alpha, beta))
    Ttot, H, dk = q.shape
    dv = v.shape[2]
    cu = [0, Ttot] if cu_seqlens is None else [int(c) for c in cu_seqlens]
    N = len(cu) - 1
    o = [[None] * H for _ in range(Ttot)]
    hT = [[None] * H for _ in range(N)]
    for n in range(N):
        for h in range(H):
            S = [[F(h0[n][h][r][c]) if h0 is not None else F(0) for c in range(dv)]
                 for r in range(dk)]
            for t in range(cu[n], cu[n + 1]):
                a = [F(alpha[t, h, r]) for r in range(dk)]
                kt = [F(k[t, h, r]) for r in range(dk)]
                qt = [F(q[t, h, r]) for r in range(dk)]
                vt = [F(v[t, h, c]) for c in range(dv)]
                bt = F(beta[t, h])
                S = [[a[r] * S[r][c] for c in range(dv)] for r in range(dk)]
                pred = [sum((S[r][c] * kt[r] for r in range(dk)), F(0)) for c in range(dv)]
                u = [bt * (vt[c] - pred[c]) for c in range(dv)]
                S = [[S[r][c] + kt[r] * u[c] for c in range(dv)] for r in range(dk)]
                o[t][h] = [sum((S[r][c] * qt[r] for r in range(dk)), F(0)) for c in range(dv)]
            hT[n][h] = S
    return o, hT


# ---------------------------------------------------------------------------------------------
# Output stage.  "Kimi K3's hybrid block, from first principles", section "From linear attention
# to the delta rule": each head's output row is divided by its root mean square, then scaled
# element by element by a sigmoid gate computed at full rank from the token; the output
# projection comes after.  Per (token, head) row of dv outputs:
#     y = o / sqrt(mean_c o_c^2 + eps) * w * sigmoid(gate)
# with w the norm's gain per value channel (ones when not given).
# ---------------------------------------------------------------------------------------------
def output_gate(o, gate, weight=None, eps: float = 1e-6):
    """o, gate: [..., dv]; weight: [dv] or None; returns y [..., dv] in float64."""
    o = np.asarray(o, dtype=np.float64)
    gate = np.asarray(gate, dtype=np.float64)
    if gate.shape != o.shape:
        raise ValueError("o and gate shapes differ")
    mean_sq = np.mean(o * o, axis=-1, keepdims=True)
    normed = o / np.sqrt(mean_sq + eps)
    if weight is not None:
        normed = normed * np.asarray(weight, dtype=np.float64)
    return normed / (1.0 + np.exp(-gate))


# ---------------------------------------------------------------------------------------------
# Input stage.  "Kimi K3's hybrid block, from first principles", section "From linear attention to
# the delta rule": q and k get a four-tap causal convolution, the Swish activation and unit-length
# normalisation, v the convolution and Swish only; beta_t comes from a sigmoid over a projection
# of the token; the decay logit z_t is a low-rank projection with a bias per channel, and the
# log-decay has the floor g_min = -5 and one learned scale A_h per head (so every retention
# factor lies between e^-5 and 1).  Readings where the pages are silent or garbled:
#   * the convolution is causal and depthwise along tokens, y[t,c] = sum_{i<4} w[c,i] x[t-3+i,c]
#     (w[c,3] weighs the current token), without bias, restarting at every sequence start from a
#     saved state of the last three inputs (zeros when none is given);
#   * L2 normalisation divides by sqrt(sum_c x_c^2 + eps) per (token, head), eps = 1e-6;
#   * the bounded log-decay is g = g_min * sigmoid(A_h (z + bias_c)), which lies in (g_min, 0).
# Layouts: x_q, x_k, x_z [Ttot, H, dk]; x_v [Ttot, H, dv]; x_b [Ttot, H]; conv weights w_q, w_k
# [H*dk, 4] and w_v [H*dv, 4]; z_bias [H*dk]; A [H].  The convolution state holds, per sequence,
# the last three inputs of q, k and v: [N, 3, H*dk + H*dk + H*dv], oldest first.
# ---------------------------------------------------------------------------------------------
def _swish(x):
    return x / (1.0 + np.exp(-x))


def frontend(x_q, x_k, x_v, x_z, x_b, w_q, w_k, w_v, z_bias, A, g_min: float = -5.0,
             cu_seqlens=None, conv_in=None, eps: float = 1e-6):
    """Returns (q, k, v, g, beta, conv_out) in float64; conv_out [N, 3, H*(2dk+dv)]."""
    f = lambda a: np.asarray(a, dtype=np.float64)
    x_q, x_k, x_v, x_z, x_b = f(x_q), f(x_k), f(x_v), f(x_z), f(x_b)
    w_q, w_k, w_v, z_bias, A = f(w_q), f(w_k), f(w_v), f(z_bias), f(A)
    Ttot, H, dk = x_q.shape
    dv = x_v.shape[2]
    cu = np.asarray([0, Ttot] if cu_seqlens is None else cu_seqlens, dtype=np.int64)
    N = cu.size - 1
    C = H * (2 * dk + dv)
    state = np.zeros((N, 3, C)) if conv_in is None else f(conv_in).reshape(N, 3, C)
    rows = np.concatenate([x_q.reshape(Ttot, H * dk), x_k.reshape(Ttot, H * dk),
                           x_v.reshape(Ttot, H * dv)], axis=1)          # [Ttot, C]
    w = np.concatenate([w_q, w_k, w_v], axis=0)                          # [C, 4]
    conv = np.zeros((Ttot, C))
    conv_out = np.zeros((N, 3, C))
    for n in range(N):
        a, e = int(cu[n]), int(cu[n + 1])
        seq = np.concatenate([state[n], rows[a:e]], axis=0)             # [3 + len, C]
        for t in range(e - a):
            conv[a + t] = np.sum(w.T * seq[t:t + 4], axis=0)            # taps t-3 .. t
        conv_out[n] = seq[-3:]
    act = _swish(conv)
    q = act[:, :H * dk].reshape(Ttot, H, dk)
    k = act[:, H * dk:2 * H * dk].reshape(Ttot, H, dk)
    v = act[:, 2 * H * dk:].reshape(Ttot, H, dv)
    q = q / np.sqrt(np.sum(q * q, axis=-1, keepdims=True) + eps)
    k = k / np.sqrt(np.sum(k * k, axis=-1, keepdims=True) + eps)
    zz = A[None, :, None] * (x_z + z_bias.reshape(H, dk)[None])
    g = g_min / (1.0 + np.exp(-zz))
    beta = 1.0 / (1.0 + np.exp(-x_b))
    return q, k, v, g, beta, conv_out
