"""FP64 CPU oracle for the KDA token mixer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module. It shares no code with the HIP library
and never imports it.

Sources (the pages this follows):

* [flozi-KDA] "Ling-3.1-flash: Grouped Routing and Two Different MLA Caches"
  (flozi.net), section "KDA replaces a token list with a recurrent matrix":
  q/k/v projections of width 64x128, one causal short convolution of width four
  with SiLU per projection, reshape to [B,T,64,128], q/k normalisation,
  channel-dependent retention, a delta-rule write, a read of the per-head
  matrix, then an output normalisation and a sigmoid gate before the projection
  back to width 4096; safe forget gate with log-retention lower bound -5.
* [satyajit-Eq] "Ling-3.1-flash: a 560B hybrid-attention MoE, counted from its
  safetensors headers", section "How KDA and MLA split the work": the decay
  comes from f_proj and A_log, the write strength from b_proj (one scalar per
  head), full-rank 4096->8192 decay and gate projections (no_kda_lora).
* [asivanadi-Memory] "Ling-3.1-flash: What 63 Linear-Attention Layers Do to the
  KV Budget", section "The memory math": FP32 state of 64x128x128 per layer,
  kernel size 4 short convolution.

Readings where the pages are silent (each is a choice, listed with its reason in
the design notes): delta-rule write (not the additive form printed in
[satyajit-Eq]); retention before the write, read after it; state rows are key
channels; readout scale is an argument (1.0 by default); g is a natural-log
retention clamped at ``lower_bound`` on use; conv taps run oldest -> newest with
the last tap on the current token, no bias; q/k L2-normalised per head with
eps 1e-6 inside the square root; per-head RMSNorm over dv with eps 1e-6;
g = max(-exp(A_log[h]) * softplus(f), -5); beta = sigmoid(b); W stored
[out, in] with y = x W^T.

The token-serial recurrence is in C (``kda_oracle.c``) for speed; everything
else is numpy float64. The chunked form here is the oracle's own cross-check of
the chunk reorganisation (an exact rewrite of the recurrence) and is checked
against the serial form in the tests.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        path = _build.build(force=False)
        lib = ctypes.CDLL(path)
        f = lib.oracle_kda_serial
        f.restype = ctypes.c_int
        f.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                              ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
                                              ctypes.c_double, ctypes.c_double,
                                              ctypes.c_void_p, ctypes.c_void_p,
                                              ctypes.c_void_p, ctypes.c_int]
        _LIB = lib
    return _LIB


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


# --------------------------------------------------------------------------
# KDA core: token-serial recurrence (the definition) -- [flozi-KDA]
# --------------------------------------------------------------------------
def kda_serial(q, k, v, g, beta, cu_seqlens=None, initial_state=None, scale=1.0,
               lower_bound=-5.0, nthreads=None):
    """Token-serial FP64 KDA recurrence.

    q, k, g: [T, H, dk]; v: [T, H, dv]; beta: [T, H] (any float dtype; values are
    taken as given, i.e. already bf16-rounded where the inputs are bf16).
    cu_seqlens: int [N+1] packed sequence boundaries, or None for one sequence.
    initial_state: [N, H, dk, dv] or None (zeros).
    Returns (o [T, H, dv] float64, final_state [N, H, dk, dv] float64).
    """
    q, k, v, g, beta = (_f32(x) for x in (q, k, v, g, beta))
    T, H, dk = q.shape
    dv = v.shape[2]
    assert k.shape == (T, H, dk) and g.shape == (T, H, dk)
    assert v.shape == (T, H, dv) and beta.shape == (T, H)
    if cu_seqlens is None:
        cu = np.array([0, T], dtype=np.int64)
    else:
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
    N = cu.shape[0] - 1
    s0 = None
    if initial_state is not None:
        s0 = np.ascontiguousarray(initial_state, dtype=np.float64)
        assert s0.shape == (N, H, dk, dv)
    o = np.empty((T, H, dv), dtype=np.float64)
    sT = np.empty((N, H, dk, dv), dtype=np.float64)
    rc = _lib().oracle_kda_serial(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), T, H, dk, dv,
                                  _ptr(cu), N, float(scale), float(lower_bound), _ptr(s0),
                                  _ptr(o), _ptr(sT), int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError("oracle_kda_serial failed with code %d" % rc)
    return o, sT


# --------------------------------------------------------------------------
# States at fixed positions -- [asivanadi-Memory], sections "Where the hybrid
# makes serving harder" (a recurrent state can be resumed only where it was
# saved: snapshots at cache-block boundaries) and "Fitting it on a node"
# (multi-token-prediction drafts, verified a few tokens at a time: the state
# after every draft token is kept so rejected ones can be dropped)
# --------------------------------------------------------------------------
def kda_serial_snapshots(q, k, v, g, beta, interval, cu_seqlens=None, initial_state=None, scale=1.0,
                         lower_bound=-5.0, nthreads=None):
    """The token-serial recurrence, also returning each sequence's state after
    every `interval` tokens.

    Each sequence is cut at the multiples of `interval` and the pieces are run
    in order through ``kda_serial``, the FP64 state of one piece being the
    initial state of the next (exactly the serial run: the state is carried in
    FP64 between the pieces).
    Returns (o [T, H, dv], final_state [N, H, dk, dv],
    snaps [N, max_j, H, dk, dv]) in float64, where snaps[n, j] is the state of
    sequence n after its first (j + 1) * interval tokens and entries past a
    sequence's last whole interval are NaN.
    """
    q, k, v, g, beta = (_f32(x) for x in (q, k, v, g, beta))
    T, H, dk = q.shape
    dv = v.shape[2]
    cu = np.array([0, T], dtype=np.int64) if cu_seqlens is None else np.asarray(cu_seqlens, dtype=np.int64)
    N = cu.shape[0] - 1
    lengths = cu[1:] - cu[:-1]
    max_j = int(lengths.max() // interval) if N else 0
    o = np.empty((T, H, dv), dtype=np.float64)
    sT = np.empty((N, H, dk, dv), dtype=np.float64)
    snaps = np.full((N, max_j, H, dk, dv), np.nan)
    for n in range(N):
        S = np.zeros((1, H, dk, dv)) if initial_state is None else \
            np.asarray(initial_state[n:n + 1], dtype=np.float64)
        a, e = int(cu[n]), int(cu[n + 1])
        cuts = list(range(a, e, interval)) + [e]
        for j, (s0, s1) in enumerate(zip(cuts[:-1], cuts[1:])):
            sl = slice(s0, s1)
            o[sl], S = kda_serial(q[sl], k[sl], v[sl], g[sl], beta[sl], initial_state=S, scale=scale,
                                  lower_bound=lower_bound, nthreads=nthreads)
            if s1 - s0 == interval:
                snaps[n, j] = S[0]
        if a == e:
            o[a:e] = 0.0
        sT[n] = S[0]
    return o, sT, snaps


# --------------------------------------------------------------------------
# KDA core: chunked reorganisation, FP64 numpy (cross-check of the serial form)
# --------------------------------------------------------------------------
def kda_chunked_one(q, k, v, g, beta, S0=None, chunk=64, scale=1.0, lower_bound=-5.0):
    """One (sequence, head): the recurrence reorganised over chunks of ``chunk``.

    Inside a chunk with start state S0 and tokens r = 1..n (b_r = cumulative
    log-retention, per key channel):
      A[r,i] = beta_r sum_c k_rc k_ic exp(b_rc - b_ic)      (i < r)
      T      = (I + A)^-1
      U      = T diag(beta) (V - (K o e^B) S0)              corrected writes
      P[r,i] = sum_c q_rc k_ic exp(b_rc - b_ic)             (i <= r)
      O      = scale ((Q o e^B) S0 + P U)
      S_n    = Diag(e^{b_n}) S0 + (K o e^{b_n - B})^T U
    Arrays are [T, dk] / [T, dv] / [T]; returns (o [T, dv], S [dk, dv]).
    """
    q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
    T, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.zeros((T, dv))
    g = np.maximum(g, lower_bound)
    for s in range(0, T, chunk):
        e = min(s + chunk, T)
        n = e - s
        Q, K, V, B = q[s:e], k[s:e], v[s:e], beta[s:e]
        b = np.cumsum(g[s:e], axis=0)                       # [n, dk]
        diff = b[:, None, :] - b[None, :, :]                # [r, i, c] = b_r - b_i
        lower_incl = np.tril(np.ones((n, n), dtype=bool))
        dec = np.exp(np.where(lower_incl[:, :, None], diff, -np.inf))
        KK = np.einsum("rc,ic,ric->ri", K, K, dec)
        A = B[:, None] * np.tril(KK, -1)
        Tm = np.linalg.inv(np.eye(n) + A)
        eB = np.exp(b)
        U = Tm @ (B[:, None] * (V - (K * eB) @ S))
        P = np.einsum("rc,ic,ric->ri", Q, K, dec)
        o[s:e] = scale * ((Q * eB) @ S + P @ U)
        Kbar = K * np.exp(b[-1][None, :] - b)
        S = np.exp(b[-1])[:, None] * S + Kbar.T @ U
    return o, S


def kda_chunked_segment_map(k, g, beta, lower_bound=-5.0):
    """Affine map of one chunk on the state: S_out = M S_in + N_v (for v given).

    Returns M [dk, dk] and the matrix K_bar^T T diag(beta) [dk, n] so that
    N = K_bar^T T diag(beta) V. Used to pin linearity of the chunk in S_in.
    """
    k, g, beta = (np.asarray(x, dtype=np.float64) for x in (k, g, beta))
    n, dk = k.shape
    g = np.maximum(g, lower_bound)
    b = np.cumsum(g, axis=0)
    diff = b[:, None, :] - b[None, :, :]
    lower = np.tril(np.ones((n, n), dtype=bool), -1)
    dec = np.exp(np.where(lower[:, :, None], diff, -np.inf))
    A = beta[:, None] * np.einsum("rc,ic,ric->ri", k, k, dec)
    Tm = np.linalg.inv(np.eye(n) + A)
    W = Tm @ (beta[:, None] * (k * np.exp(b)))
    Kbar = k * np.exp(b[-1][None, :] - b)
    M = np.diag(np.exp(b[-1])) - Kbar.T @ W
    Nmat = Kbar.T @ Tm @ np.diag(beta)
    return M, Nmat


# --------------------------------------------------------------------------
# Affine segment maps -- the state after a stretch of tokens is an affine
# function of the state before it ([flozi-KDA]: the per-token update is
# linear in the state, S_t = A_t S_{t-1} + beta_t k_t v_t^T with
# A_t = (I - beta_t k_t k_t^T) Diag(alpha_t)), which is what lets a long
# sequence be cut into segments processed apart and stitched together
# --------------------------------------------------------------------------
def kda_segment_maps(k, v, g, beta, cu_seqlens=None, lower_bound=-5.0, nthreads=None):
    """Affine map of each segment (a sequence of ``cu_seqlens``) on the state:
    S_out = M S_in + N, with M = A_T ... A_1 (dk x dk) and N the state after the
    segment from a zero state (dk x dv).

    Written out from the definition with the serial recurrence: N is its final
    state from S_in = 0; with v = 0 the update is S_t = A_t S_{t-1}, so its final
    state from S_in = I (dk x dk) is the product M. Needs dk == dv for the
    identity start. Returns (M [N, H, dk, dk], N [N, H, dk, dv]) in float64.
    """
    q = np.zeros_like(np.asarray(k, dtype=np.float64))
    T, H, dk = q.shape
    dv = np.asarray(v).shape[2]
    assert dk == dv, "identity start state needs dk == dv"
    cu = np.array([0, T], dtype=np.int64) if cu_seqlens is None else np.asarray(cu_seqlens, dtype=np.int64)
    nseq = cu.shape[0] - 1
    _, Nmap = kda_serial(q, k, v, g, beta, cu_seqlens=cu, lower_bound=lower_bound, nthreads=nthreads)
    eye = np.broadcast_to(np.eye(dk), (nseq, H, dk, dk)).copy()
    _, Mmap = kda_serial(q, k, np.zeros_like(np.asarray(v, dtype=np.float64)), g, beta, cu_seqlens=cu,
                         initial_state=eye, lower_bound=lower_bound, nthreads=nthreads)
    return Mmap, Nmap


def affine_apply(M, X, N=None):
    """Y = M X (+ N) over leading batch dimensions: the map (M, N) applied to a
    state X, or, with X the M of an earlier map, the first half of composing
    two maps: (M2, N2) after (M1, N1) is (M2 M1, M2 N1 + N2)."""
    Y = np.matmul(np.asarray(M, dtype=np.float64), np.asarray(X, dtype=np.float64))
    return Y if N is None else Y + np.asarray(N, dtype=np.float64)


# --------------------------------------------------------------------------
# Prologue / epilogue pieces (numpy float64)
# --------------------------------------------------------------------------
def round_bf16(x):
    """Round float64 values to the nearest bfloat16 (ties to even), return float64.

    bfloat16 keeps 8 significant bits and the float32 exponent range. Values are
    split as m * 2^e with m in [0.5, 1); m is rounded to 8 bits with numpy's
    round-half-even. Below 2^-126 the spacing is fixed at 2^-133 (subnormals);
    beyond the largest finite bfloat16 the result is +-inf.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    flat_in, flat_out = x.reshape(-1), out.reshape(-1)
    step = 1 << 20  # element-wise, so taken in pieces (small temporaries)
    for i in range(0, flat_in.size, step):
        flat_out[i:i + step] = _round_bf16_piece(flat_in[i:i + step])
    return out


def _round_bf16_piece(x):
    out = np.empty_like(x)
    m, e = np.frexp(x)
    normal = np.abs(x) >= 2.0 ** -126
    out[normal] = np.ldexp(np.rint(m[normal] * 256.0) / 256.0, e[normal])
    sub = ~normal
    out[sub] = np.rint(x[sub] * 2.0 ** 133) * 2.0 ** -133
    big = np.abs(out) > 3.3895313892515355e38
    out[big] = np.sign(out[big]) * np.inf
    return out


def silu(x):
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def sigmoid(x):
    x = np.asarray(x, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-x))


def softplus(x):
    return np.logaddexp(0.0, np.asarray(x, dtype=np.float64))


def conv_causal(x, w, cu_seqlens=None, state_in=None, apply_silu=True, bias=None):
    """Depthwise causal convolution of width W per sequence, then SiLU.

    [flozi-KDA]: one causal short convolution of width four with SiLU per stream.
    x: [T, C]; w: [C, W] with w[:, W-1] applied to the current token and
    w[:, 0] to the token W-1 steps back; state_in: [N, W-1, C] (oldest first) or
    None for zero history; bias: [C] added before the activation (the model
    uses none; the library accepts one). Returns (y [T, C] float64,
    state_out [N, W-1, C]): the last W-1 inputs of each sequence, including
    history when it is shorter.
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    T, C = x.shape
    W = w.shape[1]
    cu = np.array([0, T]) if cu_seqlens is None else np.asarray(cu_seqlens, dtype=np.int64)
    N = len(cu) - 1
    y = np.empty((T, C))
    state_out = np.empty((N, W - 1, C))
    for n in range(N):
        s, e = int(cu[n]), int(cu[n + 1])
        hist = np.zeros((W - 1, C)) if state_in is None else np.asarray(state_in[n], np.float64)
        ext = np.concatenate([hist, x[s:e]], axis=0)      # [W-1 + L, C]
        L = e - s
        acc = np.zeros((L, C))
        if bias is not None:
            acc += np.asarray(bias, dtype=np.float64)[None, :]
        for j in range(W):                                 # tap j sees token t - (W-1-j)
            acc += w[None, :, j] * ext[j:j + L]
        y[s:e] = silu(acc) if apply_silu else acc
        state_out[n] = ext[L:L + W - 1]
    return y, state_out


def l2norm_groups(y, group=128, eps=1e-6):
    """Per-group (per-head) L2 normalisation: y / sqrt(sum(y^2) + eps)."""
    y = np.asarray(y, dtype=np.float64)
    shp = y.shape
    z = y.reshape(shp[:-1] + (shp[-1] // group, group))
    z = z / np.sqrt(np.sum(z * z, axis=-1, keepdims=True) + eps)
    return z.reshape(shp)


def gate_prologue(f, b, A_log, lower_bound=-5.0):
    """Log-retention and write strength from the raw projections.

    f: [T, H, dk] (f_proj output); b: [T, H] (b_proj output); A_log: [H].
    g = max(-exp(A_log[h]) * softplus(f), lower_bound); beta = sigmoid(b).
    """
    f = np.asarray(f, dtype=np.float64)
    A = np.exp(np.asarray(A_log, dtype=np.float64))
    g = np.maximum(-A[None, :, None] * softplus(f), lower_bound)
    return g, sigmoid(b)


def output_norm_gate(o, gate, w, eps=1e-6):
    """Per-head RMSNorm over dv, times weight, times sigmoid(gate).

    o: [T, H, dv]; gate: [T, H*dv] or [T, H, dv]; w: [dv]. Returns [T, H, dv].
    """
    o = np.asarray(o, dtype=np.float64)
    gate = np.asarray(gate, dtype=np.float64).reshape(o.shape)
    r = o / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    return r * np.asarray(w, dtype=np.float64)[None, None, :] * sigmoid(gate)


def layer_forward(x, Wq, Wk, Wv, Wf, Wg, Wb, Wo, conv_q, conv_k, conv_v, A_log, norm_w,
                  H, d=128, scale=1.0, lower_bound=-5.0, l2_eps=1e-6, rms_eps=1e-6,
                  nthreads=None, return_parts=False, initial_state=None):
    """Whole KDA token mixer on one sequence, FP64, rounding to bfloat16 exactly
    where the library stores bfloat16 (projection outputs, conv outputs, gate
    outputs, epilogue output).

    x: [T, hidden]; W*: [out, in] (y = x W^T); conv_*: [H*d, 4];
    initial_state: the KDA state [1, H, d, d] before the first token, or None
    (zeros). Returns out [T, hidden] float64 (and a dict of intermediates,
    the final state among them as "S", if asked).
    """
    x = np.asarray(x, dtype=np.float64)
    T = x.shape[0]
    mm = lambda a, W: a @ np.asarray(W, dtype=np.float64).T
    q_pre = round_bf16(mm(x, Wq))
    k_pre = round_bf16(mm(x, Wk))
    v_pre = round_bf16(mm(x, Wv))
    f_pre = round_bf16(mm(x, Wf))
    g_pre = round_bf16(mm(x, Wg))
    b_pre = round_bf16(mm(x, Wb))
    q = round_bf16(l2norm_groups(conv_causal(q_pre, conv_q)[0], d, l2_eps))
    k = round_bf16(l2norm_groups(conv_causal(k_pre, conv_k)[0], d, l2_eps))
    v = round_bf16(conv_causal(v_pre, conv_v)[0])
    g, beta = gate_prologue(f_pre.reshape(T, H, d), b_pre, A_log, lower_bound)
    g, beta = round_bf16(g), round_bf16(beta)
    o, S = kda_serial(q.reshape(T, H, d), k.reshape(T, H, d), v.reshape(T, H, d), g, beta,
                      initial_state=initial_state, scale=scale, lower_bound=lower_bound, nthreads=nthreads)
    y = round_bf16(output_norm_gate(o, g_pre, norm_w, rms_eps)).reshape(T, H * d)
    out = mm(y, Wo)
    if return_parts:
        return out, dict(q=q, k=k, v=v, g=g, beta=beta, o=o, S=S, y=y, gate=g_pre)
    return out


# --------------------------------------------------------------------------
# Block FP8 -- [flozi-KDA] section "Production boundaries" (block FP8 E4M3
# weights with 128 x 128 scaling blocks and dynamic activation quantization)
# and [satyajit-Eq] section "What is in the files" (E4M3 weights, one fp32
# scale per 128 x 128 block). E4M3 here is the OCP FP8 E4M3 ("FN") format:
# 1 sign, 4 exponent (bias 7) and 3 mantissa bits, subnormals when the
# exponent field is 0, no infinities, 0x7F / 0xFF are NaN, largest finite 448.
# --------------------------------------------------------------------------
E4M3_MAX = 448.0


def e4m3_decode(codes):
    """uint8 codes -> float64 values (the format's definition, written out)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    val = sign * val
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


def e4m3_encode_brute(x):
    """float64 -> uint8 codes, round to nearest, ties to even, saturating at
    +-448 (values are scaled into range before encoding); the format is
    sign-magnitude, so a negative value (or -0) that rounds to zero keeps its
    sign bit (code 0x80, -0), as IEEE rounding does. Brute force over the
    127 non-negative finite codes: the nearest one, and on a tie the even one.
    (Memory grows as 127 x the input: small inputs only.)"""
    x = np.asarray(x, dtype=np.float64)
    grid = e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))   # codes 0 .. 126, increasing
    a = np.minimum(np.abs(x), E4M3_MAX)
    d = np.abs(a[..., None] - grid)                          # distance to every code
    best = d.min(axis=-1, keepdims=True)
    ties = d == best
    # among the nearest codes, prefer the even code (mantissa LSB 0)
    even = (np.arange(0, 0x7F) % 2 == 0)
    pick = np.where(ties & even, 1, 0) + np.where(ties, 2, 0)
    code = np.argmax(pick, axis=-1).astype(np.uint8)
    return np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)


def e4m3_encode(x):
    """The same rounding as e4m3_encode_brute for inputs of any size: the
    non-negative codes 0 .. 126 increase with their values, so the nearest
    code is one of the two grid neighbours that a binary search finds; the
    nearer one is taken, and on a tie the even one."""
    x = np.asarray(x, dtype=np.float64)
    grid = e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.minimum(np.searchsorted(grid, a, side="left"), 0x7E)  # first code with value >= a
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = a - grid[lo], grid[hi] - a
    code = np.where(d_hi < d_lo, hi, np.where(d_lo < d_hi, lo, np.where(lo % 2 == 0, lo, hi))).astype(np.uint8)
    return np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)


def gemv_fp8_blocks(x, codes, scales, block=128):
    """y = x W^T with W[n, k] = decode(codes[n, k]) * scales[n // 128, k // 128],
    in float64. x: [M, K]; codes: [N, K] uint8; scales: [ceil(N/128), K/128]."""
    W = e4m3_decode(codes)
    s = np.asarray(scales, dtype=np.float64)
    W = W * np.repeat(np.repeat(s, block, axis=0), block, axis=1)[:W.shape[0], :W.shape[1]]
    return np.asarray(x, dtype=np.float64) @ W.T


def quantize_fp8_groups(y, group=128):
    """Dynamic activation quantization of [T, C] values in groups of 128
    consecutive channels: scale = amax / 448 (1 when the group is all zero),
    codes = e4m3(y / scale). Returns (codes [T, C] uint8, scales [T, C/128])."""
    y = np.asarray(y, dtype=np.float64)
    T, C = y.shape
    g = y.reshape(T, C // group, group)
    amax = np.max(np.abs(g), axis=-1)
    scale = np.where(amax > 0, amax / E4M3_MAX, 1.0)
    codes = e4m3_encode(g / scale[..., None]).reshape(T, C)
    return codes, scale


def layer_forward_fp8(x, Win_codes, Win_scales, Wo_codes, Wo_scales, conv_q, conv_k, conv_v, A_log, norm_w,
                      H, d=128, scale=1.0, lower_bound=-5.0, l2_eps=1e-6, rms_eps=1e-6,
                      nthreads=None, return_parts=False, initial_state=None):
    """The token mixer with block-FP8 (W8A8) projections -- [flozi-KDA]
    section "Production boundaries" (E4M3 weights in 128 x 128 blocks with
    dynamic activation quantization): the input x is quantized per (token,
    128 channels) with float32 decisions (as a float32 implementation takes
    them), the packed input projection P = X W_in^T is the exact product of the
    decoded codes, stored as bfloat16; convolution, gate, core and epilogue are
    those of ``layer_forward``; the epilogue output y (float64, not rounded) is
    quantized per (token, head) and the output projection is the exact
    product with W_o's codes.

    Win_codes: [5*H*d + H, hidden] uint8 (rows q | k | v | f | gate | b),
    Win_scales: [ceil(rows/128), hidden/128]; Wo_codes: [hidden, H*d] uint8,
    Wo_scales: [hidden/128, H*d/128]. Returns out [T, hidden] float64 (and the
    intermediates if asked)."""
    x = np.asarray(x, dtype=np.float64)
    T = x.shape[0]
    W = H * d
    xq, xs = quantize_fp8_groups_f32(x)
    P = round_bf16(gemm_fp8_w8a8(xq, xs, Win_codes, Win_scales))
    q_pre, k_pre, v_pre, f_pre, g_pre = (P[:, i * W:(i + 1) * W] for i in range(5))
    b_pre = P[:, 5 * W:5 * W + H]
    q = round_bf16(l2norm_groups(conv_causal(q_pre, conv_q)[0], d, l2_eps))
    k = round_bf16(l2norm_groups(conv_causal(k_pre, conv_k)[0], d, l2_eps))
    v = round_bf16(conv_causal(v_pre, conv_v)[0])
    g, beta = gate_prologue(f_pre.reshape(T, H, d), b_pre, A_log, lower_bound)
    g, beta = round_bf16(g), round_bf16(beta)
    o, S = kda_serial(q.reshape(T, H, d), k.reshape(T, H, d), v.reshape(T, H, d), g, beta,
                      initial_state=initial_state, scale=scale, lower_bound=lower_bound, nthreads=nthreads)
    y = output_norm_gate(o, g_pre, norm_w, rms_eps).reshape(T, W)
    yq, ys = quantize_fp8_groups(y)
    out = gemm_fp8_w8a8(yq, ys, Wo_codes, Wo_scales)
    if return_parts:
        return out, dict(P=P, q=q, k=k, v=v, g=g, beta=beta, o=o, S=S, y=y, yq=yq, ys=ys)
    return out


def quantize_fp8_groups_f32(x, group=128):
    """The dynamic activation quantization of ``quantize_fp8_groups`` with
    every rounding decision taken in float32, as a float32 implementation
    takes it: the values are float32, amax is exact, scale = fl32(amax / 448)
    (1 for an all-zero group), r = fl32(x / scale) by IEEE division, and the
    code is the E4M3 value nearest to r (ties to even, saturating at 448),
    decided exactly from the float32 r. Returns (codes [T, C] uint8,
    scales [T, C/128] float32)."""
    x = np.asarray(x, dtype=np.float32)
    T, C = x.shape
    g = x.reshape(T, C // group, group)
    amax = np.max(np.abs(g), axis=-1)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    r = (g / scale[..., None]).astype(np.float32)
    codes = e4m3_encode(r.astype(np.float64)).reshape(T, C)
    return codes, scale


def gemm_fp8_w8a8(x_codes, x_scales, w_codes, w_scales, block=128):
    """y = X W^T with both operands block FP8, in float64 (W8A8):
    X[m, k] = decode(x_codes[m, k]) * x_scales[m, k // 128] (activations,
    quantized per token and group of 128 channels) and
    W[n, k] = decode(w_codes[n, k]) * w_scales[n // 128, k // 128] (weights,
    128 x 128 blocks). x_codes: [M, K]; x_scales: [M, K/128]; w_codes: [N, K];
    w_scales: [ceil(N/128), K/128]. Returns [M, N] float64."""
    xc = np.asarray(x_codes)
    X = e4m3_decode(xc) * np.repeat(np.asarray(x_scales, dtype=np.float64), block, axis=1)[:, :xc.shape[1]]
    W = e4m3_decode(w_codes)
    s = np.asarray(w_scales, dtype=np.float64)
    W = W * np.repeat(np.repeat(s, block, axis=0), block, axis=1)[:W.shape[0], :W.shape[1]]
    return X @ W.T
