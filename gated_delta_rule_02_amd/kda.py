"""Thin Python binding of the C ABI in ``include/kda.h`` (ctypes).

Each function has the name of the C entry point it calls and only marshals
arguments: torch tensors become device pointers and sizes, the current HIP
stream is passed through, and a non-OK status raises ``KDAError`` with the
library's message. All computation happens in ``libkda.so``; if the library is
not built, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkda.so")

KDA_F32, KDA_BF16 = 0, 1
KDA_OK, KDA_ERR_INVALID_ARG, KDA_ERR_UNSUPPORTED, KDA_ERR_WORKSPACE, KDA_ERR_HIP = 0, -1, -2, -3, -4

_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_F = ctypes.c_float
_SZ = ctypes.c_size_t

_SIGS = {
    "kda_prefill": (_I, [_P] * 5 + [_I, _I64, _I, _I, _I, _P, _P, _I, _F, _F, _P, _P, _P, _I, _P, _SZ, _P]),
    "kda_prefill_workspace_bytes": (_SZ, [_I64, _I, _I, _I, _I, _I]),
    "kda_prefill_noalloc": (_I, [_P] * 5 + [_I, _I64, _I, _I, _I, _P, _P, _I, _F, _F, _P, _P, _P, _I, _P]),
    "kda_prefill_gated": (_I, [_P] * 4 + [_I64, _P, _I64, _P, _I, _I64, _I, _I, _I, _P, _P, _I, _F, _F, _P, _P,
                                          _P, _I, _P, _SZ, _P]),
    "kda_prefill_noalloc_scratch_bytes": (_SZ, []),
    "kda_prefill_snapshots": (_I, [_P] * 5 + [_I, _I64, _I, _I, _I, _P, _P, _I, _F, _F, _P, _P, _P, _I, _P, _SZ,
                                              _I64, _I64, _P, _P]),
    "kda_prefill_segment_maps": (_I, [_P] * 4 + [_I, _I64, _I, _I, _I, _P, _P, _I, _F, _P, _P, _P, _SZ, _P]),
    "kda_affine_apply": (_I, [_P, _P, _P, _P, _I64, _I, _I, _P]),
    "kda_decode_step": (_I, [_P] * 5 + [_I, _I, _I, _I, _I, _F, _F, _P, _P, _I, _P]),
    "kda_decode_multi": (_I, [_P] * 5 + [_I, _I, _I, _I, _I, _I, _F, _F, _P, _P, _I, _P, _I, _P]),
    "kda_decode_commit": (_I, [_P, _P, _I, _I, _I, _I, _I, _P, _I, _P]),
    "kda_state_convert": (_I, [_P, _I, _P, _I, _I64, _P]),
    "kda_gemv_fp8": (_I, [_P, _I64, _P, _I64, _P, _I64, _P, _I64, _I, _I64, _I64, _I, _I, _P]),
    "kda_output_norm_gate_fp8": (_I, [_P, _I, _P, _I64, _I, _P, _I64, _I, _I, _F, _P, _P, _P]),
    "kda_quantize_fp8": (_I, [_P, _I64, _I, _I64, _I64, _P, _I64, _P, _I64, _P]),
    "kda_gemm_fp8": (_I, [_P, _I64, _P, _I64, _P, _I64, _P, _I64, _P, _I64, _I64, _I64, _I64, _I, _P]),
    "kda_conv_state_update": (_I, [_P, _I64, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P, _P]),
    "kda_conv_prefill": (_I, [_P, _I64, _I64, _I, _I, _P, _P, _I, _P, _P, _P, _P, _I, _I, _F, _P, _I64, _I, _P]),
    "kda_gate_prologue": (_I, [_P, _I64, _P, _I64, _P, _I64, _I, _I, _F, _I, _P, _P, _I, _P]),
    "kda_output_norm_gate": (_I, [_P, _I, _P, _I64, _P, _I64, _I, _I, _F, _P, _I, _P]),
    "kda_gemm": (_I, [_P, _I64, _P, _I64, _P, _I64, _I64, _I64, _I64, _I, _I, _P]),
    "kda_state_bytes": (_SZ, [_I, _I, _I, _I]),
    "kda_conv_state_bytes": (_SZ, [_I, _I, _I, _I]),
    "kda_last_error": (ctypes.c_char_p, []),
    "kda_version": (_I, []),
}
EXPORTED = tuple(_SIGS)

_lib = None


class KDAError(RuntimeError):
    def __init__(self, name, status, message):
        super().__init__("%s failed with status %d: %s" % (name, status, message))
        self.status = status


def lib():
    """Load libkda.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libkda.so is not built (expected at %s); run __graft_entry__.build()" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _call(name, *args):
    rc = getattr(lib(), name)(*args)
    if rc != KDA_OK:
        raise KDAError(name, rc, lib().kda_last_error().decode())
    return rc


def _dt(t):
    if t.dtype == torch.float32:
        return KDA_F32
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    raise TypeError("unsupported dtype %s (float32 or bfloat16 expected)" % t.dtype)


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on a GPU device")
    return t.data_ptr()


def _dense(t, name):
    if t is not None and not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _cu(cu_seqlens, cu_seqlens_host):
    if cu_seqlens is None:
        return None, None, None
    if cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    host = cu_seqlens_host
    if host is None:
        host = cu_seqlens.cpu()  # one device->host copy when no mirror is given
    host = host.to(torch.int32).contiguous()
    return _ptr(_dense(cu_seqlens, "cu_seqlens")), host.data_ptr(), host


# --------------------------------------------------------------------------
_workspaces = {}


def _workspace(device, nbytes):
    """A cached device buffer of at least nbytes (one per device; grows on demand)."""
    key = torch.device(device).index
    buf = _workspaces.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
        _workspaces[key] = buf
    return buf


def kda_prefill(q, k, v, g, beta, o, cu_seqlens=None, cu_seqlens_host=None, num_seqs=None,
                initial_state=None, final_state=None, scale=1.0, lower_bound=-5.0,
                workspace="auto", stream=None, snapshots=None, snapshot_interval=None):
    """KDA core over packed sequences. q,k,g [T,H,128], v [T,H,128], beta [T,H]
    (one dtype), o [T,H,128] (float32 or bfloat16), states float32 [N,H,128,128].

    workspace: "auto" (a cached buffer of kda_prefill_workspace_bytes bytes, so
    bfloat16 inputs take the two-pass form), None (no workspace: single-pass
    form), or a caller-owned uint8 device tensor. Calls sharing the cached
    buffer must be ordered on one stream.

    snapshots: float32 [N, slots, H, 128, 128] with snapshot_interval (a
    multiple of 64): calls kda_prefill_snapshots, which also stores the state
    after every snapshot_interval tokens of each sequence."""
    for n_, t_ in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("o", o),
                   ("initial_state", initial_state), ("final_state", final_state), ("snapshots", snapshots)):
        _dense(t_, n_)
    T, H, dk = q.shape
    dv = v.shape[2]
    cu_dev, cu_host, keep = _cu(cu_seqlens, cu_seqlens_host)
    if num_seqs is None:
        num_seqs = (keep.numel() - 1) if keep is not None else 1
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError("workspace must be 'auto', None or a tensor")
        need = lib().kda_prefill_workspace_bytes(T, num_seqs, H, dk, dv, _dt(q))
        workspace = _workspace(q.device, need) if need else None
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if snapshots is None:
        _call("kda_prefill", _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _dt(q), T, H, dk, dv,
              cu_dev, cu_host, num_seqs, scale, lower_bound, _ptr(initial_state), _ptr(final_state),
              _ptr(o), _dt(o), _ptr(workspace), ws_bytes, _stream(stream))
    else:
        if snapshot_interval is None or snapshots.dim() != 5:
            raise ValueError("snapshots [N, slots, H, 128, 128] needs a snapshot_interval")
        _call("kda_prefill_snapshots", _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _dt(q), T, H, dk, dv,
              cu_dev, cu_host, num_seqs, scale, lower_bound, _ptr(initial_state), _ptr(final_state),
              _ptr(o), _dt(o), _ptr(workspace), ws_bytes, int(snapshot_interval), snapshots.shape[1],
              _ptr(snapshots), _stream(stream))
    return o


def kda_prefill_gated(q, k, v, f, b, A_log, o, cu_seqlens=None, cu_seqlens_host=None, num_seqs=None,
                      initial_state=None, final_state=None, scale=1.0, lower_bound=-5.0, workspace="auto",
                      stream=None):
    """kda_prefill with the gate prologue inside it: f rows [T, >=H*128] and
    b rows [T, >=H] (bfloat16, contiguous rows, any row stride), A_log float32
    [H] in place of g and beta. Results equal kda_gate_prologue followed by
    kda_prefill. bfloat16 q, k, v and a workspace ("auto" or a tensor)."""
    for n_, t_ in (("q", q), ("k", k), ("v", v), ("A_log", A_log), ("o", o),
                   ("initial_state", initial_state), ("final_state", final_state)):
        _dense(t_, n_)
    if f.stride(-1) != 1 or b.stride(-1) != 1:
        raise ValueError("f and b rows must be contiguous")
    T, H, dk = q.shape
    dv = v.shape[2]
    cu_dev, cu_host, keep = _cu(cu_seqlens, cu_seqlens_host)
    if num_seqs is None:
        num_seqs = (keep.numel() - 1) if keep is not None else 1
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError("workspace must be 'auto' or a tensor")
        need = lib().kda_prefill_workspace_bytes(T, num_seqs, H, dk, dv, _dt(q))
        workspace = _workspace(q.device, need) if need else None
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _call("kda_prefill_gated", _ptr(q), _ptr(k), _ptr(v), _ptr(f), f.stride(0), _ptr(b), b.stride(0),
          _ptr(A_log), _dt(q), T, H, dk, dv, cu_dev, cu_host, num_seqs, scale, lower_bound,
          _ptr(initial_state), _ptr(final_state), _ptr(o), _dt(o), _ptr(workspace), ws_bytes, _stream(stream))
    return o


def kda_prefill_noalloc(q, k, v, g, beta, o, cu_seqlens=None, cu_seqlens_host=None, num_seqs=None,
                        initial_state=None, final_state=None, scale=1.0, lower_bound=-5.0, stream=None):
    """kda_prefill with the library's device-resident scratch in place of a
    workspace (allocates nothing). Arguments as kda_prefill."""
    for n_, t_ in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("o", o),
                   ("initial_state", initial_state), ("final_state", final_state)):
        _dense(t_, n_)
    T, H, dk = q.shape
    dv = v.shape[2]
    cu_dev, cu_host, keep = _cu(cu_seqlens, cu_seqlens_host)
    if num_seqs is None:
        num_seqs = (keep.numel() - 1) if keep is not None else 1
    _call("kda_prefill_noalloc", _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _dt(q), T, H, dk, dv,
          cu_dev, cu_host, num_seqs, scale, lower_bound, _ptr(initial_state), _ptr(final_state),
          _ptr(o), _dt(o), _stream(stream))
    return o


def kda_prefill_noalloc_scratch_bytes():
    return lib().kda_prefill_noalloc_scratch_bytes()


def kda_prefill_workspace_bytes(num_tokens, num_seqs, H, dk=128, dv=128, in_dtype=KDA_BF16):
    return lib().kda_prefill_workspace_bytes(num_tokens, num_seqs, H, dk, dv, in_dtype)


def kda_prefill_segment_maps(k, v, g, beta, M_out, N_out, cu_seqlens=None, cu_seqlens_host=None, num_seqs=None,
                             lower_bound=-5.0, workspace="auto", stream=None):
    """Affine map S_out = M S_in + N of every segment (sequence of cu_seqlens).
    k, g [T,H,128], v [T,H,128], beta [T,H] bfloat16; M_out, N_out float32
    [N,H,128,128]. workspace as for kda_prefill (required: "auto" or a tensor)."""
    for n_, t_ in (("k", k), ("v", v), ("g", g), ("beta", beta), ("M_out", M_out), ("N_out", N_out)):
        _dense(t_, n_)
    T, H, dk = k.shape
    dv = v.shape[2]
    cu_dev, cu_host, keep = _cu(cu_seqlens, cu_seqlens_host)
    if num_seqs is None:
        num_seqs = (keep.numel() - 1) if keep is not None else 1
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError("workspace must be 'auto' or a tensor")
        workspace = _workspace(k.device, max(lib().kda_prefill_workspace_bytes(max(T, 1), num_seqs, H, dk, dv, _dt(k)), 16))
    ws_bytes = workspace.numel() * workspace.element_size()
    _call("kda_prefill_segment_maps", _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _dt(k), T, H, dk, dv,
          cu_dev, cu_host, num_seqs, lower_bound, _ptr(M_out), _ptr(N_out), _ptr(workspace), ws_bytes,
          _stream(stream))
    return M_out, N_out


def kda_affine_apply(M, X, Y, N=None, stream=None):
    """Y = M X (+ N) for float32 [..., 128, 128] batches (segment maps applied
    to states, or composed)."""
    for n_, t_ in (("M", M), ("X", X), ("Y", Y), ("N", N)):
        _dense(t_, n_)
    count = M.numel() // (128 * 128)
    if X.numel() != M.numel() or Y.numel() != M.numel() or (N is not None and N.numel() != M.numel()):
        raise ValueError("M, X, N and Y must hold the same number of 128 x 128 matrices")
    _call("kda_affine_apply", _ptr(M), _ptr(X), _ptr(N), _ptr(Y), count, 128, 128, _stream(stream))
    return Y


def kda_decode_step(q, k, v, g, beta, state, o, scale=1.0, lower_bound=-5.0, stream=None):
    """One token per sequence. q,k,g,v [B,H,128], beta [B,H]; state float32
    [B,H,128,128] updated in place; o [B,H,128]."""
    for n_, t_ in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("state", state), ("o", o)):
        _dense(t_, n_)
    B, H, dk = q.shape
    dv = v.shape[2]
    _call("kda_decode_step", _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _dt(q), B, H, dk, dv,
          scale, lower_bound, _ptr(state), _ptr(o), _dt(o), _stream(stream))
    return o


def kda_decode_multi(q, k, v, g, beta, state, o, token_states=None, scale=1.0, lower_bound=-5.0, stream=None):
    """Several tokens per sequence. q,k,g,v [B,Tq,H,128], beta [B,Tq,H]; state
    [B,H,128,128] in float32 or bfloat16 (its dtype is the state dtype); o
    [B,Tq,H,128]. token_states None: state becomes the state after the last
    token; else token_states [B,Tq,H,128,128] (the state's dtype) receives the
    state after every token and state is only read."""
    for n_, t_ in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("state", state), ("o", o),
                   ("token_states", token_states)):
        _dense(t_, n_)
    if token_states is not None and token_states.dtype != state.dtype:
        raise TypeError("token_states must have the state's dtype")
    B, Tq, H, dk = q.shape
    dv = v.shape[3]
    _call("kda_decode_multi", _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _dt(q), B, Tq, H, dk, dv,
          scale, lower_bound, _ptr(state), _ptr(token_states), _dt(state), _ptr(o), _dt(o), _stream(stream))
    return o


def kda_decode_commit(token_states, accepted, state, stream=None):
    """state[b] <- token_states[b, accepted[b] - 1] where 1 <= accepted[b] <= Tq
    (accepted: int32 [B] on the device; states float32 or bfloat16)."""
    for n_, t_ in (("token_states", token_states), ("accepted", accepted), ("state", state)):
        _dense(t_, n_)
    if accepted.dtype != torch.int32:
        raise TypeError("accepted must be int32")
    if token_states.dtype != state.dtype:
        raise TypeError("token_states and state must have one dtype")
    B, Tq, H, dk, dv = token_states.shape
    _call("kda_decode_commit", _ptr(token_states), _ptr(accepted), B, Tq, H, dk, dv, _ptr(state), _dt(state),
          _stream(stream))
    return state


def kda_state_convert(src, dst, stream=None):
    """dst <- src converted between float32 and bfloat16 (same number of elements)."""
    _dense(src, "src")
    _dense(dst, "dst")
    if src.numel() != dst.numel():
        raise ValueError("src and dst must have the same number of elements")
    _call("kda_state_convert", _ptr(src), _dt(src), _ptr(dst), _dt(dst), src.numel(), _stream(stream))
    return dst


def kda_conv_state_update(x, conv_state, weight, y, bias=None, apply_silu=True, l2norm_group=0,
                          l2norm_eps=1e-6, stream=None):
    """x rows [B, >=C] (row stride x.stride(0)), conv_state [B,W-1,C] (in place),
    weight [C,W], y [B,C]."""
    for n_, t_ in (("conv_state", conv_state), ("weight", weight), ("y", y), ("bias", bias)):
        _dense(t_, n_)
    if x.stride(1) != 1:
        raise ValueError("x rows must be contiguous")
    B = x.shape[0]
    C, W = weight.shape
    _call("kda_conv_state_update", _ptr(x), x.stride(0), _ptr(conv_state), _ptr(weight), _ptr(bias), _dt(x), B, C, W,
          int(bool(apply_silu)), l2norm_group, l2norm_eps, _ptr(y), _stream(stream))
    return y


def kda_conv_prefill(x, weight, y, cu_seqlens=None, cu_seqlens_host=None, num_seqs=None, bias=None,
                     conv_state_in=None, conv_state_out=None, apply_silu=True, l2norm_group=0,
                     l2norm_eps=1e-6, stream=None):
    """x rows [T, >=C] (row stride x.stride(0)), weight [C,W], y rows [T, >=C]."""
    for n_, t_ in (("weight", weight), ("bias", bias), ("conv_state_in", conv_state_in),
                   ("conv_state_out", conv_state_out)):
        _dense(t_, n_)
    if x.stride(1) != 1 or y.stride(1) != 1:
        raise ValueError("x and y rows must be contiguous")
    T = x.shape[0]
    C, W = weight.shape
    cu_dev, cu_host, keep = _cu(cu_seqlens, cu_seqlens_host)
    if num_seqs is None:
        num_seqs = (keep.numel() - 1) if keep is not None else 1
    _call("kda_conv_prefill", _ptr(x), x.stride(0), T, C, W, cu_dev, cu_host, num_seqs, _ptr(weight),
          _ptr(bias), _ptr(conv_state_in), _ptr(conv_state_out), int(bool(apply_silu)), l2norm_group,
          l2norm_eps, _ptr(y), y.stride(0), _dt(x), _stream(stream))
    return y


def kda_gate_prologue(f, b, A_log, g_out, beta_out, H, dk=128, lower_bound=-5.0, stream=None):
    """f rows [T, >=H*dk], b rows [T, >=H], A_log float32 [H]; g_out [T,H,dk], beta_out [T,H]."""
    _dense(A_log, "A_log"); _dense(g_out, "g_out"); _dense(beta_out, "beta_out")
    if f.stride(-1) != 1 or b.stride(-1) != 1:
        raise ValueError("f and b rows must be contiguous")
    T = f.shape[0]
    _call("kda_gate_prologue", _ptr(f), f.stride(0), _ptr(b), b.stride(0), _ptr(A_log), T, H, dk,
          lower_bound, _dt(f), _ptr(g_out), _ptr(beta_out), _dt(g_out), _stream(stream))
    return g_out, beta_out


def kda_output_norm_gate(o, gate, norm_weight, y, eps=1e-6, stream=None):
    """o [T,H,dv], gate rows [T, >=H*dv] (dtype of y), norm_weight float32 [dv], y [T,H*dv]."""
    _dense(o, "o"); _dense(norm_weight, "norm_weight"); _dense(y, "y")
    if gate.stride(-1) != 1:
        raise ValueError("gate rows must be contiguous")
    T, H, dv = o.shape
    _call("kda_output_norm_gate", _ptr(o), _dt(o), _ptr(gate), gate.stride(0), _ptr(norm_weight), T, H,
          dv, eps, _ptr(y), _dt(y), _stream(stream))
    return y


def kda_gemm(A, B, C, stream=None):
    """C[M,N] = A[M,K] B[N,K]^T (rows may be strided; last dims contiguous)."""
    for n_, t_ in (("A", A), ("B", B), ("C", C)):
        if t_.stride(-1) != 1:
            raise ValueError("%s rows must be contiguous" % n_)
    M, K = A.shape
    N = B.shape[0]
    _call("kda_gemm", _ptr(A), A.stride(0), _ptr(B), B.stride(0), _ptr(C), C.stride(0), M, N, K,
          _dt(A), _dt(C), _stream(stream))
    return C


def kda_gemv_fp8(x, w, w_scale, y, stream=None):
    """y[M,N] = x[M,K] W^T, W = e4m3(w) (uint8 [N,K]) x w_scale[N/128, K/128]
    blocks; x bf16, 1 <= M <= 8 (row strides allowed, last dims contiguous)."""
    for n_, t_ in (("x", x), ("w", w), ("w_scale", w_scale), ("y", y)):
        if t_.stride(-1) != 1:
            raise ValueError("%s rows must be contiguous" % n_)
    if w.dtype != torch.uint8 or w_scale.dtype != torch.float32:
        raise TypeError("w must be uint8 E4M3 codes and w_scale float32")
    M, Kd = x.shape
    N = w.shape[0]
    _call("kda_gemv_fp8", _ptr(x), x.stride(0), _ptr(w), w.stride(0), _ptr(w_scale), w_scale.stride(0),
          _ptr(y), y.stride(0), M, N, Kd, _dt(x), _dt(y), _stream(stream))
    return y


def kda_quantize_fp8(x, codes, scales, stream=None):
    """x [M,K] float32/bfloat16 -> codes uint8 [M,K] (E4M3), scales float32 [M,K/128]
    (row strides allowed, last dims contiguous)."""
    for n_, t_ in (("x", x), ("codes", codes), ("scales", scales)):
        if t_.stride(-1) != 1:
            raise ValueError("%s rows must be contiguous" % n_)
    if codes.dtype != torch.uint8 or scales.dtype != torch.float32:
        raise TypeError("codes must be uint8 and scales float32")
    M, Kd = x.shape
    _call("kda_quantize_fp8", _ptr(x), x.stride(0), _dt(x), M, Kd, _ptr(codes), codes.stride(0), _ptr(scales),
          scales.stride(0), _stream(stream))
    return codes, scales


def kda_gemm_fp8(x, x_scale, w, w_scale, y, stream=None):
    """y[M,N] = X W^T with X = e4m3(x) x x_scale[M, K/128] and W = e4m3(w) x
    w_scale[N/128, K/128] (x, w uint8 codes; row strides allowed)."""
    for n_, t_ in (("x", x), ("x_scale", x_scale), ("w", w), ("w_scale", w_scale), ("y", y)):
        if t_.stride(-1) != 1:
            raise ValueError("%s rows must be contiguous" % n_)
    if x.dtype != torch.uint8 or w.dtype != torch.uint8:
        raise TypeError("x and w must be uint8 E4M3 codes")
    if x_scale.dtype != torch.float32 or w_scale.dtype != torch.float32:
        raise TypeError("scales must be float32")
    M, Kd = x.shape
    N = w.shape[0]
    _call("kda_gemm_fp8", _ptr(x), x.stride(0), _ptr(x_scale), x_scale.stride(0), _ptr(w), w.stride(0),
          _ptr(w_scale), w_scale.stride(0), _ptr(y), y.stride(0), M, N, Kd, _dt(y), _stream(stream))
    return y


def kda_output_norm_gate_fp8(o, gate, norm_weight, y_codes, y_scales, eps=1e-6, stream=None):
    """o [T,H,128]; gate rows [T, >=H*128]; y_codes uint8 [T, H*128]; y_scales float32 [T, H]."""
    for n_, t_ in (("o", o), ("norm_weight", norm_weight), ("y_codes", y_codes), ("y_scales", y_scales)):
        _dense(t_, n_)
    if gate.stride(1) != 1:
        raise ValueError("gate rows must be contiguous")
    T, H, dv = o.shape
    _call("kda_output_norm_gate_fp8", _ptr(o), _dt(o), _ptr(gate), gate.stride(0), _dt(gate), _ptr(norm_weight),
          T, H, dv, eps, _ptr(y_codes), _ptr(y_scales), _stream(stream))
    return y_codes, y_scales


def kda_state_bytes(H, dk=128, dv=128, dtype=KDA_F32):
    return lib().kda_state_bytes(H, dk, dv, dtype)


def kda_conv_state_bytes(streams, W, C, dtype=KDA_BF16):
    return lib().kda_conv_state_bytes(streams, W, C, dtype)


def kda_last_error():
    return lib().kda_last_error().decode()


def kda_version():
    return lib().kda_version()
