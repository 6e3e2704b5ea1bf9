"""kda_prefill_noalloc (the prefill with the library's device-resident
scratch in place of a caller workspace) against kda_prefill with a workspace,
through the C ABI: two calls in a row, the second with a smaller input. The
scratch keeps the first call's contents; the second must not depend on them.
Outputs and final states equal kda_prefill's bit for bit (same kernels, same
windows) and the FP64 oracle within 2e-3."""
import ctypes

import numpy as np
import pytest
import torch

from gated_delta_rule_02_amd import kda as K
from gated_delta_rule_02_amd import synth
from oracle import reference as R
from tests.gpu_util import TOL_BF16, announce, dev, host64, relerr

pytestmark = pytest.mark.gpu


def run_both(d, cu=None, s0=None):
    q, k, v, g, b = (dev(d[x]) for x in ("q", "k", "v", "g", "beta"))
    T, H, _ = q.shape
    N = 1 if cu is None else len(cu) - 1
    cu_d = None if cu is None else torch.from_numpy(np.asarray(cu, np.int32)).cuda()
    cu_h = None if cu is None else torch.from_numpy(np.asarray(cu, np.int32))
    s0_d = None if s0 is None else dev(s0)
    outs = []
    for noalloc in (True, False):
        o = torch.full((T, H, 128), float("nan"), dtype=torch.float32, device="cuda")
        sT = torch.full((N, H, 128, 128), float("nan"), dtype=torch.float32, device="cuda")
        st = torch.cuda.current_stream().cuda_stream
        if noalloc:
            rc = K.lib().kda_prefill_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(), b.data_ptr(),
                                             K.KDA_BF16, T, H, 128, 128,
                                             None if cu_d is None else cu_d.data_ptr(),
                                             None if cu_h is None else cu_h.data_ptr(), N, 1.0, -5.0,
                                             None if s0_d is None else s0_d.data_ptr(), sT.data_ptr(), o.data_ptr(),
                                             K.KDA_F32, st)
            assert rc == K.KDA_OK, K.kda_last_error()
        else:
            K.kda_prefill(q, k, v, g, b, o, cu_seqlens=cu_d, cu_seqlens_host=cu_h, num_seqs=N,
                          initial_state=s0_d, final_state=sT, workspace="auto")
        torch.cuda.synchronize()
        outs.append((o, sT))
    return outs


def test_noalloc_matches_workspace_entry_two_calls():
    assert K.kda_prefill_noalloc_scratch_bytes() == 160 << 20
    announce("noalloc: call 1, prefill workload T=4096 H=64")
    d = synth.workload_prefill()
    (o1, s1), (o2, s2) = run_both(d)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    ro, rS = R.kda_serial(d["q"].vals, d["k"].vals, d["v"].vals, d["g"].vals, d["beta"].vals)
    eo, es = relerr(host64(o1), ro), relerr(host64(s1[0]), rS[0])
    print("  o err %.3e  state err %.3e" % (eo, es), flush=True)
    assert eo < TOL_BF16 and es < TOL_BF16

    announce("noalloc: call 2, smaller packed input with initial states")
    lens = [300, 64, 0, 129]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    rng = np.random.default_rng(900)
    H = 3
    d = synth.core_inputs(rng, int(cu[-1]), H, bf16=True)
    s0 = synth.states(rng, len(lens), H, std=0.3)
    (o1, s1), (o2, s2) = run_both(d, cu=cu, s0=s0)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    ro, rS = R.kda_serial(d["q"].vals, d["k"].vals, d["v"].vals, d["g"].vals, d["beta"].vals, cu_seqlens=cu,
                          initial_state=s0.astype(np.float64))
    eo = relerr(host64(o1), ro)
    es = max(relerr(host64(s1[n]), rS[n]) for n in range(len(lens)))
    print("  o err %.3e  state err %.3e" % (eo, es), flush=True)
    assert eo < TOL_BF16 and es < TOL_BF16
    assert np.array_equal(host64(s1[2]), s0[2].astype(np.float64))  # the empty sequence keeps its state
