"""kda_prefill_gated (the gate prologue inside the prefill) against
kda_gate_prologue followed by kda_prefill: the two must agree bit for bit,
outputs and final states, since the fused form rounds g and beta to bfloat16
exactly as the prologue stores them. Both halves of the unfused chain are
checked against the FP64 oracle by their own tests (test_gate_prologue, the
prefill tests); the token-mixer layer, whose forward pass uses the fused form,
is checked against the oracle's layer in test_gpu_layer.py.

The gate rows are column slices of a wider projection matrix (row stride
larger than H * 128, as in the layer), and their values are drawn so that
many decays fall below the floor (the clamp is exercised)."""
import numpy as np
import pytest
import torch

from gated_delta_rule_02_amd import kda as K
from tests.gpu_util import announce

pytestmark = pytest.mark.gpu


def _inputs(T, H, width, seed):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    rn = lambda *s: torch.randn(*s, device="cuda", generator=gen)
    unit = lambda x: x / x.norm(dim=-1, keepdim=True)
    q = unit(rn(T, H, 128)).to(torch.bfloat16)
    k = unit(rn(T, H, 128)).to(torch.bfloat16)
    v = rn(T, H, 128).to(torch.bfloat16)
    # projection rows: f at column 3 * H * 128, b after the five H * 128 blocks;
    # f ~ N(0, 2^2) with exp(A_log) up to 4.5 sends many decays below -5
    P = (2.0 * rn(T, width)).to(torch.bfloat16)
    W = H * 128
    f, b = P[:, 3 * W:4 * W], P[:, 5 * W:5 * W + H]
    A_log = (torch.rand(H, device="cuda", generator=gen) * 2.5 - 1.0).float()
    return q, k, v, f, b, A_log


def _both(q, k, v, f, b, A_log, cu, s0, out_dtype, lb):
    T, H, _ = q.shape
    N = 1 if cu is None else len(cu) - 1
    cu_d = None if cu is None else torch.tensor(cu, dtype=torch.int32, device="cuda")
    cu_h = None if cu is None else torch.tensor(cu, dtype=torch.int32)
    g = torch.empty(T, H, 128, dtype=torch.bfloat16, device="cuda")
    beta = torch.empty(T, H, dtype=torch.bfloat16, device="cuda")
    K.kda_gate_prologue(f, b, A_log, g, beta, H, lower_bound=lb)
    o1 = torch.full((T, H, 128), float("nan"), dtype=out_dtype, device="cuda")
    o2 = torch.full_like(o1, float("nan"))
    s1 = torch.empty(N, H, 128, 128, device="cuda")
    s2 = torch.empty_like(s1)
    K.kda_prefill(q, k, v, g, beta, o1, cu_seqlens=cu_d, cu_seqlens_host=cu_h, num_seqs=N, initial_state=s0,
                  final_state=s1, lower_bound=lb)
    K.kda_prefill_gated(q, k, v, f, b, A_log, o2, cu_seqlens=cu_d, cu_seqlens_host=cu_h, num_seqs=N,
                        initial_state=s0, final_state=s2, lower_bound=lb)
    torch.cuda.synchronize()
    clamped = float((g.float() <= lb).float().mean())
    return o1, o2, s1, s2, clamped


def _same(a, b):
    return torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a.view(torch.int16),
                       b.view(torch.int32) if b.dtype == torch.float32 else b.view(torch.int16))


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("lb", [-5.0, -2.0])
def test_gated_prefill_equals_prologue_then_prefill(out_dtype, lb):
    # ragged lengths: one token, a chunk minus and plus one, an empty sequence,
    # several windows' worth of chunks for the longest
    lens = [1, 63, 64, 65, 0, 130, 200, 70]
    cu = [0] + list(np.cumsum(lens))
    H = 4
    T = cu[-1]
    announce("gated prefill varlen T=%d H=%d lb=%g out=%s" % (T, H, lb, out_dtype))
    q, k, v, f, b, A_log = _inputs(T, H, 5 * H * 128 + H + 12, seed=41)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(42)
    s0 = 0.05 * torch.randn(len(lens), H, 128, 128, device="cuda", generator=gen)
    o1, o2, s1, s2, clamped = _both(q, k, v, f, b, A_log, cu, s0, out_dtype, lb)
    assert clamped > 0.05, clamped  # the floor is reached
    assert not torch.isnan(o1.float()).any() and not torch.isnan(s1).any()
    assert _same(o1, o2) and _same(s1, s2)


def test_gated_prefill_layer_shape():
    """The layer workload's shape: T = 8192, H = 64, gate rows inside the
    41,024-column projection output."""
    T, H = 8192, 64
    announce("gated prefill T=%d H=%d" % (T, H))
    q, k, v, f, b, A_log = _inputs(T, H, 5 * H * 128 + H, seed=43)
    o1, o2, s1, s2, _ = _both(q, k, v, f, b, A_log, None, None, torch.float32, -5.0)
    assert not torch.isnan(o1).any() and not torch.isnan(s1).any()
    assert _same(o1, o2) and _same(s1, s2)
