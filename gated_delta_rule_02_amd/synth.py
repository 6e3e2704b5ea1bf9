"""Seeded synthetic inputs for the KDA token mixer.

This module only draws random numbers and shapes them into the input
distributions of the workloads; it holds none of the mixer's arithmetic and is
the one piece of code that both the HIP path (via the tests and the bench) and
the CPU oracle consume. Every array is produced on the host with
``numpy.random.default_rng(seed)`` in a fixed draw order, so both sides see
bit-identical inputs.

Recipes (the pages give the model's shapes -- 64 heads of 128 channels, width-4
short convolutions, hidden width 4096 -- but no data, so the distributions are
choices of this project):

* q, k ~ N(0, 1), then scaled to unit L2 norm per (token, head) in float32;
* v ~ N(0, 1);
* log-retention g = max(-softplus(z), -5) with z ~ N(0, 1) (natural log);
* write strength beta = 1 / (1 + exp(-z)) with z ~ N(0, 1);
* bfloat16 inputs are the float32 draws rounded to nearest-even bfloat16 after
  the steps above.
"""
from __future__ import annotations

import numpy as np

CORE_D = 128


def bf16_round(x):
    """float32 -> nearest-even bfloat16, returned as (float32 values, uint16 bits)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # finite inputs cannot overflow 32 bits here: 0xff7fffff + 0x8000 < 2^32
    r = (u >> np.uint32(16)) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r &= np.uint32(0xFFFF0000)
    bits = (r >> np.uint32(16)).astype(np.uint16)
    return r.view(np.float32), bits


class Tensor:
    """A host array in its library dtype: ``vals`` (float32 values, exact for
    bf16) and ``bits`` (uint16 bfloat16 bit patterns, or None for float32)."""

    __slots__ = ("vals", "bits", "dtype")

    def __init__(self, vals, bits=None):
        self.vals = vals
        self.bits = bits
        self.dtype = "bf16" if bits is not None else "f32"

    @property
    def shape(self):
        return self.vals.shape

    def host(self):
        """The array as stored in device memory (uint16 bits or float32)."""
        return self.bits if self.bits is not None else self.vals


def _as(x, bf16):
    if bf16:
        v, b = bf16_round(x)
        return Tensor(v, b)
    return Tensor(np.ascontiguousarray(x, dtype=np.float32))


def _unit_rows(x):
    n = np.sqrt(np.sum(x.astype(np.float32) ** 2, axis=-1, keepdims=True, dtype=np.float32))
    return (x / n).astype(np.float32)


def _softplus32(z):
    return np.logaddexp(np.float32(0), z).astype(np.float32)


def core_inputs(rng, T, H, dk=CORE_D, dv=CORE_D, bf16=True, lower_bound=-5.0, g_scale=1.0):
    """q, k, v, g, beta for T packed tokens and H heads (draw order q, k, v, g, beta).
    g_scale < 1 gives slower retention (longer memory): g = max(-g_scale softplus(z), lower_bound)."""
    q = _unit_rows(rng.standard_normal((T, H, dk), dtype=np.float32))
    k = _unit_rows(rng.standard_normal((T, H, dk), dtype=np.float32))
    v = rng.standard_normal((T, H, dv), dtype=np.float32)
    zg = rng.standard_normal((T, H, dk), dtype=np.float32)
    g = np.maximum(-np.float32(g_scale) * _softplus32(zg), np.float32(lower_bound)).astype(np.float32)
    zb = rng.standard_normal((T, H), dtype=np.float32)
    beta = (1.0 / (1.0 + np.exp(-zb))).astype(np.float32)
    return dict(q=_as(q, bf16), k=_as(k, bf16), v=_as(v, bf16), g=_as(g, bf16),
                beta=_as(beta, bf16))


def states(rng, N, H, dk=CORE_D, dv=CORE_D, std=0.02):
    """float32 [N, H, dk, dv] ~ N(0, std^2)."""
    return (rng.standard_normal((N, H, dk, dv), dtype=np.float32) * np.float32(std)).astype(np.float32)


def varlen_lengths(rng, n, lo, hi):
    """n sequence lengths drawn uniformly from [lo, hi] (inclusive)."""
    return rng.integers(lo, hi, size=n, endpoint=True).astype(np.int64)


def cu_from_lengths(lengths):
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    return cu


def normal(rng, shape, std=1.0, bf16=True):
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x = (x * np.float32(std)).astype(np.float32)
    return _as(x, bf16)


# --------------------------------------------------------------------------
# The five workloads. Seed = 1000 + workload index.
# --------------------------------------------------------------------------
def workload_core_fp32(T=256, H=4, seed=1000):
    """Core only, CPU-tractable: B=1, T=256, H=4, d=128, float32, zero state."""
    rng = np.random.default_rng(seed)
    d = core_inputs(rng, T, H, bf16=False)
    d["cu_seqlens"] = np.array([0, T], dtype=np.int32)
    d["initial_state"] = None
    return d


def workload_prefill(T=4096, H=64, seed=1001):
    """Single-layer prefill: B=1, T=4096, H=64, bf16 inputs, zero fp32 state."""
    rng = np.random.default_rng(seed)
    d = core_inputs(rng, T, H, bf16=True)
    d["cu_seqlens"] = np.array([0, T], dtype=np.int32)
    d["initial_state"] = None
    return d


def workload_decode(B=256, H=64, C=8192, seed=1002):
    """Batched decode step: B sequences, one token each, bf16 inputs, fp32 state
    [B, H, 128, 128] ~ N(0, 0.02^2); conv input [B, C], conv state [B, 3, C] and
    conv weight [C, 4] (x, state ~ N(0,1); weight ~ N(0, 0.5^2))."""
    rng = np.random.default_rng(seed)
    d = core_inputs(rng, B, H, bf16=True)
    d["state"] = states(rng, B, H)
    d["conv_x"] = normal(rng, (B, C))
    d["conv_state"] = normal(rng, (B, 3, C))
    d["conv_w"] = normal(rng, (C, 4), std=0.5)
    return d


def workload_decode_multi(B=256, Tq=4, H=64, seed=1005):
    """Draft verification: B sequences with Tq tokens each (packed [B*Tq, H,
    d], sequence-major), bf16 inputs, fp32 state [B, H, 128, 128] ~ N(0, 0.02^2)."""
    rng = np.random.default_rng(seed)
    d = core_inputs(rng, B * Tq, H, bf16=True)
    d["state"] = states(rng, B, H)
    d["Tq"] = Tq
    return d


def workload_varlen(n=8, lo=1024, hi=32768, H=64, seed=1003):
    """Packed variable-length prefill: n lengths ~ U[lo, hi], bf16 inputs,
    fp32 initial states [n, H, 128, 128] ~ N(0, 0.02^2)."""
    rng = np.random.default_rng(seed)
    lengths = varlen_lengths(rng, n, lo, hi)
    T = int(lengths.sum())
    d = core_inputs(rng, T, H, bf16=True)
    d["cu_seqlens"] = cu_from_lengths(lengths)
    d["initial_state"] = states(rng, n, H)
    return d


def workload_layer(T=8192, hidden=4096, H=64, seed=1004):
    """Full token-mixer layer: hidden [T, hidden] ~ N(0,1) bf16; projection
    weights [out, in] ~ N(0, 0.02^2) bf16; depthwise conv weights [H*128, 4]
    ~ N(0, 0.5^2) bf16; A_log = 0; norm weight = 1."""
    rng = np.random.default_rng(seed)
    W = H * CORE_D
    d = dict(x=normal(rng, (T, hidden)))
    for name in ("Wq", "Wk", "Wv", "Wg", "Wf"):
        d[name] = normal(rng, (W, hidden), std=0.02)
    d["Wb"] = normal(rng, (H, hidden), std=0.02)
    d["Wo"] = normal(rng, (hidden, W), std=0.02)
    for name in ("conv_q", "conv_k", "conv_v"):
        d[name] = normal(rng, (W, 4), std=0.5)
    d["A_log"] = np.zeros(H, dtype=np.float32)
    d["norm_w"] = np.ones(CORE_D, dtype=np.float32)
    d["H"] = H
    return d


def fp8_codes(rng, shape, exp_lo=3, exp_hi=9):
    """Random E4M3 bit patterns: uniform sign, exponent field uniform in
    [exp_lo, exp_hi] (never the NaN pattern), uniform 3-bit mantissa."""
    e = rng.integers(exp_lo, exp_hi + 1, shape)
    m = rng.integers(0, 8, shape)
    s = rng.integers(0, 2, shape)
    return ((s << 7) | (e << 3) | m).astype(np.uint8)


def workload_layer_fp8(T=8192, hidden=4096, H=64, seed=1006):
    """The token-mixer layer with its weights in the release's block-FP8
    storage: E4M3 codes (``fp8_codes``: magnitudes 2^-4 .. 7.5) with one
    float32 scale per 128 x 128 block drawn U(0.006, 0.010), so that the
    weights' RMS is about 0.02 as in the bf16 layer. The packed input
    projection has rows q | k | v | f | gate (H*128 each) | b (H). Input x, conv
    weights, A_log and the norm weight as ``workload_layer``."""
    rng = np.random.default_rng(seed)
    W = H * CORE_D
    rows = 5 * W + H
    d = dict(x=normal(rng, (T, hidden)))
    d["Win_codes"] = fp8_codes(rng, (rows, hidden))
    d["Win_scales"] = rng.uniform(0.006, 0.010, ((rows + 127) // 128, hidden // 128)).astype(np.float32)
    d["Wo_codes"] = fp8_codes(rng, (hidden, W))
    d["Wo_scales"] = rng.uniform(0.006, 0.010, (hidden // 128, W // 128)).astype(np.float32)
    for name in ("conv_q", "conv_k", "conv_v"):
        d[name] = normal(rng, (W, 4), std=0.5)
    d["A_log"] = np.zeros(H, dtype=np.float32)
    d["norm_w"] = np.ones(CORE_D, dtype=np.float32)
    d["H"] = H
    return d
