"""GPU parity of the sequence-parallel pieces: the affine map S_out = M S_in + N
of every segment (kda_prefill_segment_maps), map application and composition
(kda_affine_apply), and a long prefill cut into segments, their maps chained
and the segments run from their true incoming states, against the FP64
oracle's plain serial run."""
import numpy as np
import pytest
import torch

from gated_delta_rule_02_amd import kda as K
from gated_delta_rule_02_amd import synth
from oracle import reference as R
from tests.gpu_util import TOL_BF16, announce, dev, host64, relerr

pytestmark = pytest.mark.gpu

SLOT = K.kda_prefill_workspace_bytes(64, 1, 1)


def inputs(d):
    return [dev(d[x]) for x in ("q", "k", "v", "g", "beta")]


def gpu_maps(d, cu, workspace="auto"):
    q, k, v, g, b = inputs(d)
    H = k.shape[1]
    N = len(cu) - 1
    M = torch.full((N, H, 128, 128), float("nan"), device="cuda")
    Nm = torch.full((N, H, 128, 128), float("nan"), device="cuda")
    cu_d = torch.from_numpy(np.asarray(cu, np.int32)).cuda()
    cu_h = torch.from_numpy(np.asarray(cu, np.int32))
    K.kda_prefill_segment_maps(k, v, g, b, M, Nm, cu_seqlens=cu_d, cu_seqlens_host=cu_h, num_seqs=N,
                               workspace=workspace)
    torch.cuda.synchronize()
    return M, Nm


def check_maps(M, Nm, rM, rN, tol=TOL_BF16):
    # M acts on states: its natural scale is that of the identity, and over
    # long segments of strong retention it decays to nothing, so its error is
    # taken against max(max|M|, 1); N's against max|N| (per segment)
    eM = max(float(np.max(np.abs(host64(M[n]) - rM[n]))) / max(float(np.max(np.abs(rM[n]))), 1.0)
             for n in range(rM.shape[0]))
    eN = max(relerr(host64(Nm[n]), rN[n]) for n in range(rN.shape[0]) if np.any(rN[n]))
    print("  M err %.3e  N err %.3e  (tol %.0e)" % (eM, eN, tol), flush=True)
    assert eM < tol and eN < tol


@pytest.mark.parametrize("lens,H,g_scale", [([200, 64, 0, 130], 2, 0.02), ([1, 63, 65, 300], 1, 1.0),
                                            ([4096], 3, 1.0), ([700, 1200], 2, 0.01)])
def test_segment_maps_match_oracle(lens, H, g_scale):
    """M and N of every segment (an empty one included) within 2e-3 of the
    FP64 oracle, with the workload's retention and with slow retention (M then
    stays of order one over hundreds of tokens); the empty segment's map is
    exactly (I, 0)."""
    announce("segment maps lens=%s H=%d g_scale=%g" % (lens, H, g_scale))
    rng = np.random.default_rng(500 + sum(lens))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    d = synth.core_inputs(rng, int(cu[-1]), H, bf16=True, g_scale=g_scale)
    M, Nm = gpu_maps(d, cu)
    rM, rN = R.kda_segment_maps(d["k"].vals, d["v"].vals, d["g"].vals, d["beta"].vals, cu_seqlens=cu)
    check_maps(M, Nm, rM, rN)
    for n, L in enumerate(lens):
        if L == 0:
            assert torch.equal(M[n], torch.eye(128, device="cuda").expand(H, 128, 128))
            assert torch.count_nonzero(Nm[n]) == 0


def test_segment_maps_windows_bit_identical():
    """A workspace of one chunk slot per unit (plus the carry) forces one-chunk
    windows, the maps carried between them in the outputs: bit-identical to
    one window."""
    announce("segment maps windows")
    rng = np.random.default_rng(510)
    lens = [300, 90, 511]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    H = 2
    d = synth.core_inputs(rng, int(cu[-1]), H, bf16=True)
    U = len(lens) * H
    small = torch.empty(U * SLOT + U * 128 * 128 * 4, dtype=torch.uint8, device="cuda")
    big = torch.empty(U * SLOT * ((max(lens) + 63) // 64), dtype=torch.uint8, device="cuda")
    M1, N1 = gpu_maps(d, cu, workspace=small)
    M2, N2 = gpu_maps(d, cu, workspace=big)
    assert torch.equal(M1, M2) and torch.equal(N1, N2)


def test_affine_apply_matches_float64():
    """Y = M X + N and Y = M X on random float32 batches, within 1e-6 of
    float64 (float32 accumulation of 128 products), and Y = N in place."""
    announce("affine apply")
    rng = np.random.default_rng(520)
    M, X, N = (rng.standard_normal((5, 128, 128)).astype(np.float32) for _ in range(3))
    Md, Xd, Nd = dev(M), dev(X), dev(N)
    Y = torch.empty_like(Xd)
    K.kda_affine_apply(Md, Xd, Y, N=Nd)
    Y2 = torch.empty_like(Xd)
    K.kda_affine_apply(Md, Xd, Y2)
    K.kda_affine_apply(Md, Xd, Nd, N=Nd)  # in place on N
    torch.cuda.synchronize()
    ref = M.astype(np.float64) @ X.astype(np.float64)
    e1, e2, e3 = relerr(host64(Y), ref + N), relerr(host64(Y2), ref), relerr(host64(Nd), ref + N)
    print("  errs %.2e %.2e %.2e" % (e1, e2, e3), flush=True)
    assert max(e1, e2, e3) < 1e-6
    assert torch.equal(Y, Nd)


def seqpar_prefill(d, cuts, s0):
    """One sequence cut at `cuts` (segment boundaries, [0, ..., T]): every
    segment's map at once, the incoming states chained on the device
    (S_{s+1} = M_s S_s + N_s), then every segment's outputs at once from its
    incoming state. Returns (o, final state)."""
    q, k, v, g, b = inputs(d)
    T, H, _ = q.shape
    P = len(cuts) - 1
    cu_d = torch.from_numpy(np.asarray(cuts, np.int32)).cuda()
    cu_h = torch.from_numpy(np.asarray(cuts, np.int32))
    M = torch.empty((P, H, 128, 128), device="cuda")
    Nm = torch.empty_like(M)
    K.kda_prefill_segment_maps(k, v, g, b, M, Nm, cu_seqlens=cu_d, cu_seqlens_host=cu_h, num_seqs=P)
    S = torch.empty((P, H, 128, 128), device="cuda")
    S[0] = dev(s0)[0]
    for s in range(1, P):
        K.kda_affine_apply(M[s - 1], S[s - 1], S[s], N=Nm[s - 1])
    o = torch.empty((T, H, 128), dtype=torch.float32, device="cuda")
    sT = torch.empty_like(S)
    K.kda_prefill(q, k, v, g, b, o, cu_seqlens=cu_d, cu_seqlens_host=cu_h, num_seqs=P,
                  initial_state=S, final_state=sT)
    torch.cuda.synchronize()
    return o, sT[P - 1:P]


@pytest.mark.parametrize("T,cuts,H,g_scale", [(1000, [0, 300, 520, 777, 1000], 2, 0.01),
                                              (4096, [0, 1024, 2048, 3072, 4096], 64, 1.0)])
def test_sequence_parallel_prefill_matches_serial(T, cuts, H, g_scale):
    """A sequence cut into segments (ragged cuts with slow retention, so that
    the state crossing each cut matters; and the 4096 x 64-head prefill workload
    in four segments), stitched by the segment maps, gives the outputs and final
    state of the oracle's plain serial run within 2e-3."""
    announce("sequence-parallel prefill T=%d cuts=%s H=%d g_scale=%g" % (T, cuts, H, g_scale))
    rng = np.random.default_rng(530 + T)
    d = synth.core_inputs(rng, T, H, bf16=True, g_scale=g_scale)
    s0 = synth.states(rng, 1, H, std=0.05)
    o, sT = seqpar_prefill(d, cuts, s0)
    ro, rS = R.kda_serial(d["q"].vals, d["k"].vals, d["v"].vals, d["g"].vals, d["beta"].vals,
                          initial_state=s0.astype(np.float64))
    eo, es = relerr(host64(o), ro), relerr(host64(sT[0]), rS[0])
    print("  o err %.3e  state err %.3e" % (eo, es), flush=True)
    assert eo < TOL_BF16 and es < TOL_BF16
