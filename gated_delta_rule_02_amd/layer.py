"""The whole KDA token mixer of one layer, composed from the C-ABI calls.

Data flow of "Ling-3.1-flash: Grouped Routing and Two Different MLA Caches"
(flozi.net), section "KDA replaces a token list with a recurrent matrix":
hidden [T, 4096] -> q, k, v projections of width 64 x 128, each through its own
causal width-4 convolution with SiLU, q and k normalised per head -> retention +
delta-rule write + read per head -> output normalisation x sigmoid gate ->
projection back to 4096. Decay and gate projections are full rank 4096 -> 8192
and beta comes from a per-head projection ("Ling-3.1-flash: a 560B
hybrid-attention MoE, counted from its safetensors headers", section "How KDA
and MLA split the work").

Every arithmetic step runs in libkda.so; this module only holds device
buffers and sequences the calls. The six input projections are packed into one
[5*H*128 + H (+ zero rows to a multiple of 8), hidden] weight so a single GEMM
produces q|k|v|f|gate|b.
"""
from __future__ import annotations

import numpy as np
import torch

from . import kda as K

D = 128


def _dev_bf16(t):
    return torch.from_numpy(np.ascontiguousarray(t.bits).view(np.int16)).view(torch.bfloat16).cuda()


class KDAMixer:
    def __init__(self, W_in, conv_q, conv_k, conv_v, A_log, norm_w, Wo, H, scale=1.0,
                 lower_bound=-5.0, l2_eps=1e-6, rms_eps=1e-6):
        self.W_in, self.Wo = W_in, Wo
        self.conv = (conv_q, conv_k, conv_v)
        self.A_log, self.norm_w = A_log, norm_w
        self.H = H
        self.W = H * D
        self.hidden = Wo.shape[0]
        self.scale, self.lower_bound, self.l2_eps, self.rms_eps = scale, lower_bound, l2_eps, rms_eps
        self._bufs = {}

    @classmethod
    def from_host(cls, d):
        """Build from the seeded host weights of ``synth.workload_layer``."""
        rows = [_dev_bf16(d[n]) for n in ("Wq", "Wk", "Wv", "Wf", "Wg", "Wb")]
        pad = (-sum(r.shape[0] for r in rows)) % 8  # keep packed rows 16-byte aligned
        if pad:
            rows.append(torch.zeros((pad, rows[0].shape[1]), dtype=torch.bfloat16, device="cuda"))
        W_in = torch.cat(rows, dim=0).contiguous()
        return cls(W_in, _dev_bf16(d["conv_q"]), _dev_bf16(d["conv_k"]), _dev_bf16(d["conv_v"]),
                   torch.from_numpy(d["A_log"]).cuda(), torch.from_numpy(d["norm_w"]).cuda(),
                   _dev_bf16(d["Wo"]), d["H"])

    def flops_per_token(self):
        core = 2 * 4468736  # per chunk-head of 64 tokens -> per token-head x 64 heads / 64 tokens
        rows = 5 * self.W + self.H
        return 2 * (rows * self.W_in.shape[1] + self.Wo.shape[0] * self.Wo.shape[1]) + core * self.H // 64

    def _buf(self, name, shape, dtype):
        b = self._bufs.get(name)
        if b is None or tuple(b.shape) != tuple(shape) or b.dtype != dtype:
            b = torch.empty(shape, dtype=dtype, device="cuda")
            self._bufs[name] = b
        return b

    def projections(self, x):
        """P = x W_in^T (bf16): columns q | k | v | f | gate | b."""
        T = x.shape[0]
        P = self._buf("P", (T, self.W_in.shape[0]), torch.bfloat16)
        K.kda_gemm(x, self.W_in, P)
        W = self.W
        return P, [P[:, i * W:(i + 1) * W] for i in range(5)] + [P[:, 5 * W:5 * W + self.H]]

    def output(self, o, gp, tag=""):
        """y = RMSNorm(o) x w x sigmoid(gate) (bf16), out = y W_o^T (float32)."""
        T = o.shape[0]
        y = self._buf(tag + "y", (T, self.W), torch.bfloat16)
        K.kda_output_norm_gate(o, gp, self.norm_w, y, eps=self.rms_eps)
        out = self._buf(tag + "out", (T, self.hidden), torch.float32)
        K.kda_gemm(y, self.Wo, out)
        return out, y

    def forward(self, x, cu_seqlens=None, cu_seqlens_host=None, initial_state=None, final_state=None,
                conv_state_in=None, conv_state_out=None, return_parts=False):
        """x [T, hidden] bf16 (packed sequences if cu_seqlens is given) ->
        out [T, hidden] float32. Optional conv states are [3, N, 3, H*128]."""
        T = x.shape[0]
        H, W = self.H, self.W
        P, (qp, kp, vp, fp, gp, bp) = self.projections(x)
        qkv = []
        for i, (src, l2) in enumerate(((qp, D), (kp, D), (vp, 0))):
            y = self._buf("c%d" % i, (T, W), torch.bfloat16)
            K.kda_conv_prefill(src, self.conv[i], y, cu_seqlens=cu_seqlens, cu_seqlens_host=cu_seqlens_host,
                               conv_state_in=None if conv_state_in is None else conv_state_in[i],
                               conv_state_out=None if conv_state_out is None else conv_state_out[i],
                               apply_silu=True, l2norm_group=l2, l2norm_eps=self.l2_eps)
            qkv.append(y.view(T, H, D))
        # the gate prologue runs inside the prefill: g and beta are formed from
        # the f and b columns of P in registers and never stored
        o = self._buf("o", (T, H, D), torch.float32)
        K.kda_prefill_gated(qkv[0], qkv[1], qkv[2], fp, bp, self.A_log, o, cu_seqlens=cu_seqlens,
                            cu_seqlens_host=cu_seqlens_host, initial_state=initial_state,
                            final_state=final_state, scale=self.scale, lower_bound=self.lower_bound)
        out, y = self.output(o, gp)
        if return_parts:
            return out, dict(q=qkv[0], k=qkv[1], v=qkv[2], o=o, y=y, P=P)
        return out

    def decode(self, x, state, conv_states):
        """One token per sequence: x [B, hidden] bf16; state float32 [B, H, 128, 128]
        and conv_states bf16 [3, B, 3, H*128] are updated in place. Returns
        out [B, hidden] float32."""
        B = x.shape[0]
        H, W = self.H, self.W
        P, (qp, kp, vp, fp, gp, bp) = self.projections(x)
        qkv = []
        for i, (src, l2) in enumerate(((qp, D), (kp, D), (vp, 0))):
            y = self._buf("dc%d" % i, (B, W), torch.bfloat16)
            K.kda_conv_state_update(src, conv_states[i], self.conv[i], y, apply_silu=True,
                                    l2norm_group=l2, l2norm_eps=self.l2_eps)
            qkv.append(y.view(B, H, D))
        g = self._buf("dg", (B, H, D), torch.bfloat16)
        beta = self._buf("dbeta", (B, H), torch.bfloat16)
        K.kda_gate_prologue(fp, bp, self.A_log, g, beta, H, D, lower_bound=self.lower_bound)
        o = self._buf("do", (B, H, D), torch.float32)
        K.kda_decode_step(qkv[0], qkv[1], qkv[2], g, beta, state, o, scale=self.scale,
                          lower_bound=self.lower_bound)
        out, _ = self.output(o, gp, tag="d")
        return out


class DecodeGraph:
    """One decode step of a mixer captured as a HIP graph: the step's kernels
    (projections, the three conv updates, gate, decode step, epilogue, output
    projection) are replayed without a host launch each, which at a few
    sequences is a large part of the step. The graph reads x from, and writes
    out to, its own buffers and updates the given state and conv states in
    place, so each replay advances those sequences by one token. Every call
    it makes allocates nothing and enqueues no memset (the library never
    does), and the mixer's buffers are allocated by an eager step before the
    capture."""

    def __init__(self, mixer, B, state, conv_states):
        self.x = torch.zeros((B, mixer.hidden), dtype=torch.bfloat16, device="cuda")
        self.state, self.conv_states = state, conv_states
        # an eager step on copies allocates every buffer the step uses
        mixer.decode(self.x, state.clone(), conv_states.clone())
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(self.graph, stream=s):
                self.out = mixer.decode(self.x, state, conv_states)
        torch.cuda.current_stream().wait_stream(s)

    def step(self, x):
        """Copy x [B, hidden] in, replay, return the output buffer."""
        self.x.copy_(x)
        self.graph.replay()
        return self.out


class KDAMixerFP8(KDAMixer):
    """The same mixer with its projections in block FP8 (W8A8): E4M3 weights
    in 128 x 128 blocks with float32 block scales, as the release stores them,
    and activations quantized dynamically ("Ling-3.1-flash: Grouped Routing
    and Two Different MLA Caches", section "Production boundaries"). The input
    x is quantized per (token, 128 channels) by kda_quantize_fp8 and the
    epilogue writes its output quantized per (token, head)
    (kda_output_norm_gate_fp8); both projections run kda_gemm_fp8 (weight
    streaming up to 8 tokens, the FP8 matrix cores beyond)."""

    def __init__(self, Win_codes, Win_scales, Wo_codes, Wo_scales, conv_q, conv_k, conv_v, A_log, norm_w, H,
                 **kw):
        super().__init__(Win_codes, conv_q, conv_k, conv_v, A_log, norm_w, Wo_codes, H, **kw)
        self.W_in_s, self.Wo_s = Win_scales, Wo_scales

    @classmethod
    def from_host(cls, d):
        """Build from the seeded host weights of ``synth.workload_layer_fp8``."""
        u8 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
        # packed rows padded with zero codes to a multiple of 8 (16-byte aligned
        # column slices of the projection output), with block scales to match
        codes, scales = d["Win_codes"], d["Win_scales"]
        pad = (-codes.shape[0]) % 8
        if pad:
            codes = np.concatenate([codes, np.zeros((pad, codes.shape[1]), np.uint8)])
        need = (codes.shape[0] + 127) // 128
        if scales.shape[0] < need:
            scales = np.concatenate([scales, np.ones((need - scales.shape[0], scales.shape[1]), np.float32)])
        return cls(u8(codes), u8(scales), u8(d["Wo_codes"]), u8(d["Wo_scales"]),
                   _dev_bf16(d["conv_q"]), _dev_bf16(d["conv_k"]), _dev_bf16(d["conv_v"]),
                   torch.from_numpy(d["A_log"]).cuda(), torch.from_numpy(d["norm_w"]).cuda(), d["H"])

    def projections(self, x):
        """x quantized per (token, 128 channels), then P = X W_in^T (bf16)."""
        T, hidden = x.shape
        xq = self._buf("xq", (T, hidden), torch.uint8)
        xs = self._buf("xs", (T, hidden // 128), torch.float32)
        K.kda_quantize_fp8(x, xq, xs)
        P = self._buf("P", (T, self.W_in.shape[0]), torch.bfloat16)
        K.kda_gemm_fp8(xq, xs, self.W_in, self.W_in_s, P)
        W = self.W
        return P, [P[:, i * W:(i + 1) * W] for i in range(5)] + [P[:, 5 * W:5 * W + self.H]]

    def output(self, o, gp, tag=""):
        """The epilogue quantized per (token, head), then out = Y W_o^T (float32)."""
        T = o.shape[0]
        yq = self._buf(tag + "yq", (T, self.W), torch.uint8)
        ys = self._buf(tag + "ys", (T, self.H), torch.float32)
        K.kda_output_norm_gate_fp8(o, gp, self.norm_w, yq, ys, eps=self.rms_eps)
        out = self._buf(tag + "out", (T, self.hidden), torch.float32)
        K.kda_gemm_fp8(yq, ys, self.Wo, self.Wo_s, out)
        return out, (yq, ys)
