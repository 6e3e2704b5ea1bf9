"""Chunked prefill on the GPU vs the FP64 token-serial oracle.

bfloat16 cases run both forms of the library: the two-pass form (a workspace
is given: per-chunk products for all chunks, then the state pass) and the
single-pass form (no workspace)."""
import numpy as np
import pytest
import torch

from gated_delta_rule_02_amd import kda as K
from gated_delta_rule_02_amd import synth
from oracle import reference as R
from tests.gpu_util import TOL_BF16, TOL_F32, announce, dev, host64, relerr

# workspace bytes of one chunk slot (one 64-token chunk of one (sequence, head));
# a workspace of one slot per unit plus the float32 state carry forces one-chunk windows
SLOT = K.kda_prefill_workspace_bytes(64, 1, 1)

pytestmark = pytest.mark.gpu


PATHS = ["split", "single"]


def gpu_prefill(d, cu=None, s0=None, out_dtype=torch.float32, final=True, in_place=False, path="split",
                workspace=None, snapshots=None, interval=None):
    q, k, v, g, b = (dev(d[x]) for x in ("q", "k", "v", "g", "beta"))
    T, H, _ = q.shape
    o = torch.empty((T, H, 128), dtype=out_dtype, device="cuda")
    cu_d = None if cu is None else torch.from_numpy(np.asarray(cu, np.int32)).cuda()
    cu_h = None if cu is None else torch.from_numpy(np.asarray(cu, np.int32))
    N = 1 if cu is None else len(cu) - 1
    s0_d = None if s0 is None else dev(s0)
    sT = None
    if final:
        sT = s0_d if in_place else torch.empty((N, H, 128, 128), dtype=torch.float32, device="cuda")
    ws = workspace if workspace is not None else ("auto" if path == "split" else None)
    K.kda_prefill(q, k, v, g, b, o, cu_seqlens=cu_d, cu_seqlens_host=cu_h, num_seqs=N,
                  initial_state=s0_d, final_state=sT, workspace=ws, snapshots=snapshots, snapshot_interval=interval)
    torch.cuda.synchronize()
    return o, sT


def oracle(d, cu=None, s0=None):
    return R.kda_serial(d["q"].vals, d["k"].vals, d["v"].vals, d["g"].vals, d["beta"].vals,
                        cu_seqlens=cu, initial_state=None if s0 is None else s0.astype(np.float64))


def check(o, sT, ro, rS, tol):
    eo = relerr(host64(o), ro)
    es = max(relerr(host64(sT[n]), rS[n]) for n in range(rS.shape[0]))
    print("  o err %.3e  state err %.3e  (tol %.0e)" % (eo, es, tol), flush=True)
    assert eo < tol and es < tol


def test_core_fp32_workload():
    """B=1, T=256, H=4, float32 inputs, zero state: 1e-5."""
    announce("prefill fp32 T=256 H=4")
    d = synth.workload_core_fp32()
    o, sT = gpu_prefill(d)
    ro, rS = oracle(d)
    check(o, sT, ro, rS, TOL_F32)


@pytest.mark.parametrize("T,H,bf16,path", [(1, 2, True, "split"), (15, 1, True, "split"), (64, 2, True, "split"),
                                           (200, 3, True, "split"), (1, 2, True, "single"), (15, 1, True, "single"),
                                           (64, 2, True, "single"), (200, 3, True, "single"),
                                           (77, 2, False, "single"), (333, 1, False, "single")])
def test_ragged_lengths_with_state(T, H, bf16, path):
    announce("prefill ragged T=%d H=%d bf16=%s %s" % (T, H, bf16, path))
    rng = np.random.default_rng(1000 + T)
    d = synth.core_inputs(rng, T, H, bf16=bf16)
    s0 = synth.states(rng, 1, H, std=0.3)
    o, sT = gpu_prefill(d, s0=s0, path=path)
    ro, rS = oracle(d, s0=s0)
    check(o, sT, ro, rS, TOL_BF16 if bf16 else TOL_F32)


@pytest.mark.parametrize("path", PATHS)
def test_varlen_small_with_empty_sequences(path):
    announce("prefill varlen small %s" % path)
    lens = [1, 63, 64, 65, 0, 130, 7, 0]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    rng = np.random.default_rng(42)
    H = 2
    d = synth.core_inputs(rng, int(cu[-1]), H, bf16=True)
    s0 = synth.states(rng, len(lens), H, std=0.1)
    o, sT = gpu_prefill(d, cu=cu, s0=s0, path=path)
    ro, rS = oracle(d, cu=cu, s0=s0)
    check(o, sT, ro, rS, TOL_BF16)
    # empty sequences return their initial state unchanged
    for n in (4, 7):
        np.testing.assert_array_equal(sT[n].cpu().numpy(), s0[n])


@pytest.mark.parametrize("path", PATHS)
def test_prefill_workload_full_size(path):
    """B=1, T=4096, H=64, bf16 inputs, chunk 64, zero state."""
    announce("prefill full T=4096 H=64 %s" % path)
    d = synth.workload_prefill()
    o, sT = gpu_prefill(d, path=path)
    ro, rS = oracle(d)
    check(o, sT, ro, rS, TOL_BF16)


def test_read_after_write_identity():
    """beta = 1, q = k: every output equals its value (per-token identity)."""
    announce("prefill identity")
    rng = np.random.default_rng(3)
    d = synth.core_inputs(rng, 150, 2, bf16=False)
    d["q"] = d["k"]
    d["beta"] = synth.Tensor(np.ones((150, 2), np.float32))
    o, _ = gpu_prefill(d, s0=synth.states(rng, 1, 2, std=1.0))
    v = d["v"].vals
    assert np.max(np.abs(host64(o) - v)) < 1e-4 * np.max(np.abs(v))


@pytest.mark.parametrize("path", PATHS)
def test_split_invariance_and_decode_continuation(path):
    """prefill(T) then prefill(rest) from its state == prefill(all), and
    prefill(T) + one decode step == prefill(T+1)."""
    announce("prefill split + decode continuation %s" % path)
    rng = np.random.default_rng(4)
    T, H = 300, 2
    d = synth.core_inputs(rng, T + 1, H, bf16=True)
    head = {k_: synth.Tensor(v_.vals[:100], None if v_.bits is None else v_.bits[:100]) for k_, v_ in d.items()}
    tail = {k_: synth.Tensor(v_.vals[100:T], None if v_.bits is None else v_.bits[100:T]) for k_, v_ in d.items()}
    first = {k_: synth.Tensor(v_.vals[:T], None if v_.bits is None else v_.bits[:T]) for k_, v_ in d.items()}
    o_all, s_all = gpu_prefill(first, path=path)
    o1, s1 = gpu_prefill(head, path=path)
    o2, s2 = gpu_prefill(tail, s0=s1.cpu().numpy(), path=path)
    ref = host64(o_all)
    assert relerr(host64(torch.cat([o1, o2])), ref) < 1e-3
    assert relerr(host64(s2), host64(s_all)) < 1e-3
    # one more token by decode, compared to the oracle on T+1 tokens
    last = {k_: dev(synth.Tensor(v_.vals[T:], None if v_.bits is None else v_.bits[T:])) for k_, v_ in d.items()}
    st = s_all[0].clone().unsqueeze(0).contiguous()
    od = torch.empty((1, H, 128), dtype=torch.float32, device="cuda")
    K.kda_decode_step(last["q"], last["k"], last["v"], last["g"], last["beta"], st, od)
    torch.cuda.synchronize()
    ro, rS = oracle(d)
    assert relerr(host64(od[0]), ro[T]) < TOL_BF16 * 2
    assert relerr(host64(st[0]), rS[0]) < TOL_BF16


@pytest.mark.parametrize("path", PATHS)
def test_in_place_state_and_determinism(path):
    announce("prefill in-place + determinism %s" % path)
    rng = np.random.default_rng(5)
    T, H = 257, 3
    d = synth.core_inputs(rng, T, H, bf16=True)
    s0 = synth.states(rng, 1, H, std=0.2)
    o1, s1 = gpu_prefill(d, s0=s0, path=path)
    o2, s2 = gpu_prefill(d, s0=s0, in_place=True, path=path)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


@pytest.mark.parametrize("path", PATHS)
def test_outputs_stay_in_bounds(path):
    """Guard bands around o and the final state are left untouched."""
    announce("prefill guard bands %s" % path)
    rng = np.random.default_rng(6)
    T, H = 70, 2
    d = synth.core_inputs(rng, T, H, bf16=True)
    q, k, v, g, b = (dev(d[x]) for x in ("q", "k", "v", "g", "beta"))
    pad = 4096
    obuf = torch.full((T * H * 128 + 2 * pad,), 7.0, device="cuda")
    sbuf = torch.full((H * 128 * 128 + 2 * pad,), 7.0, device="cuda")
    o = obuf[pad:pad + T * H * 128].view(T, H, 128)
    sT = sbuf[pad:pad + H * 128 * 128].view(1, H, 128, 128)
    K.kda_prefill(q, k, v, g, b, o, final_state=sT, workspace="auto" if path == "split" else None)
    torch.cuda.synchronize()
    for buf in (obuf, sbuf):
        assert torch.all(buf[:pad] == 7.0) and torch.all(buf[-pad:] == 7.0)


@pytest.mark.parametrize("path", PATHS)
def test_bf16_output(path):
    """bfloat16 output equals the float32 output of the same kernel rounded to
    bfloat16 (same arithmetic, only the store differs)."""
    announce("prefill bf16 out %s" % path)
    rng = np.random.default_rng(7)
    d = synth.core_inputs(rng, 128, 2, bf16=True)
    o16, s16 = gpu_prefill(d, out_dtype=torch.bfloat16, path=path)
    o32, s32 = gpu_prefill(d, out_dtype=torch.float32, path=path)
    diff = (o16.float() - o32.to(torch.bfloat16).float()).abs()
    if diff.max() > 0:
        idx = np.unravel_index(int(torch.argmax(diff).item()), tuple(diff.shape))
        print("  max diff at", idx, "bf16", o16[idx].item(), "fp32", o32[idx].item(),
              "mismatches", int((diff > 0).sum().item()), flush=True)
    assert torch.equal(o16.float(), o32.to(torch.bfloat16).float())
    assert torch.equal(s16, s32)
    ro, _ = oracle(d)
    assert relerr(host64(o16), ro) < 6e-3


@pytest.mark.parametrize("lens", [[333], [1, 63, 64, 65, 0, 130, 7, 0, 200]])
def test_split_windows_match_one_window(lens):
    """A workspace of one chunk slot per (sequence, head) plus the state carry
    forces one-chunk windows; outputs and states equal the one-window run bit
    for bit (the windows change only where the state waits between chunks)
    and match the oracle. Sequences end in different windows."""
    announce("prefill split windows lens=%s" % lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    rng = np.random.default_rng(11)
    H = 2
    N = len(lens)
    d = synth.core_inputs(rng, int(cu[-1]), H, bf16=True)
    s0 = synth.states(rng, N, H, std=0.2)
    U = N * H
    small = torch.empty(U * SLOT + U * 128 * 128 * 4, dtype=torch.uint8, device="cuda")
    big = torch.empty(U * SLOT * ((max(lens) + 63) // 64), dtype=torch.uint8, device="cuda")
    o1, s1 = gpu_prefill(d, cu=cu, s0=s0, workspace=small)
    o2, s2 = gpu_prefill(d, cu=cu, s0=s0, workspace=big)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    ro, rS = oracle(d, cu=cu, s0=s0)
    check(o1, s1, ro, rS, TOL_BF16)


def test_packed_sequences_equal_separate_calls():
    """Packed sequences that end in different windows (32-chunk windows: the
    later ones have fewer (sequence, head) units running, so the intra pass
    spreads each unit's chunks over more workgroups and the state pass moves
    from 64- to 32-column workgroups) give, bit for bit, the outputs and final
    states of one call per sequence; an empty sequence keeps its state."""
    lens = [5000, 2500, 200, 64, 0, 1000]
    announce("prefill packed vs separate lens=%s" % lens)
    H = 16
    N = len(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    rng = np.random.default_rng(31)
    d = synth.core_inputs(rng, int(cu[-1]), H, bf16=True)
    s0 = synth.states(rng, N, H, std=0.05)
    o, sT = gpu_prefill(d, cu=cu, s0=s0)
    q, k, v, g, b = (dev(d[x]) for x in ("q", "k", "v", "g", "beta"))
    s0_d = dev(s0)
    for n, L in enumerate(lens):
        if L == 0:
            continue
        a, e = int(cu[n]), int(cu[n + 1])
        on = torch.empty((L, H, 128), dtype=torch.float32, device="cuda")
        sn = torch.empty((1, H, 128, 128), dtype=torch.float32, device="cuda")
        K.kda_prefill(q[a:e], k[a:e], v[a:e], g[a:e], b[a:e], on, initial_state=s0_d[n:n + 1].contiguous(),
                      final_state=sn, workspace="auto")
        torch.cuda.synchronize()
        assert torch.equal(on, o[a:e]), "sequence %d: o differs" % n
        assert torch.equal(sn[0], sT[n]), "sequence %d: final state differs" % n
    assert torch.equal(sT[4], s0_d[4])


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_random_varlen_two_chunk_windows(seed):
    """Random packings (1-40 sequences of 0-700 tokens, 1-5 heads, random
    initial states) run in two-chunk windows, so that the count of units still
    running changes from window to window (and with it the intra-pass grouping
    and the state-pass width): bit-identical to the run in one window, and
    within 2e-3 of the oracle."""
    rng = np.random.default_rng(900 + seed)
    N = int(rng.integers(1, 41))
    H = int(rng.integers(1, 6))
    lens = [int(x) for x in rng.integers(0, 701, N)]
    if sum(lens) == 0:
        lens[0] = 1
    announce("prefill random varlen seed=%d N=%d H=%d T=%d" % (seed, N, H, sum(lens)))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    d = synth.core_inputs(rng, int(cu[-1]), H, bf16=True)
    s0 = synth.states(rng, N, H, std=0.1)
    U = N * H
    small = torch.empty(2 * U * SLOT + U * 128 * 128 * 4, dtype=torch.uint8, device="cuda")
    big = torch.empty(U * SLOT * ((max(lens) + 63) // 64), dtype=torch.uint8, device="cuda")
    o1, s1 = gpu_prefill(d, cu=cu, s0=s0, workspace=small)
    o2, s2 = gpu_prefill(d, cu=cu, s0=s0, workspace=big)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    ro, rS = oracle(d, cu=cu, s0=s0)
    check(o1, s1, ro, rS, TOL_BF16)


def test_varlen_workload_full_size():
    """Packed varlen workload at full size: 8 sequences (123,444 tokens, up to
    447 chunks each), H = 64, bf16 inputs, random fp32 initial states, final
    states returned; default two-pass form with windows of up to 32 chunks.
    Every head of every sequence is compared with the oracle (o and final
    state). The oracle runs in slices of 8 heads to bound host memory; the
    error of each sequence's o and final state is max|gpu - ref| / max|ref|
    over all of its heads, accumulated across the slices."""
    announce("prefill varlen full size (all heads)")
    d = synth.workload_varlen()
    cu = d["cu_seqlens"]
    q, k, v, g, b = (dev(d[x]) for x in ("q", "k", "v", "g", "beta"))
    T, H, _ = q.shape
    N = len(cu) - 1
    s0 = torch.from_numpy(d["initial_state"]).cuda()
    sT = torch.empty_like(s0)
    o = torch.empty((T, H, 128), dtype=torch.float32, device="cuda")
    cu_d = torch.from_numpy(cu).cuda()
    K.kda_prefill(q, k, v, g, b, o, cu_seqlens=cu_d, cu_seqlens_host=torch.from_numpy(cu), num_seqs=N,
                  initial_state=s0, final_state=sT)
    torch.cuda.synchronize()
    del q, k, v, g, b
    sTh = host64(sT)
    o_diff, o_ref = np.zeros(N), np.zeros(N)
    s_diff, s_ref = np.zeros(N), np.zeros(N)
    HS = 8
    for h0 in range(0, H, HS):
        sl = slice(h0, h0 + HS)
        ro, rS = R.kda_serial(d["q"].vals[:, sl], d["k"].vals[:, sl], d["v"].vals[:, sl], d["g"].vals[:, sl],
                              d["beta"].vals[:, sl], cu_seqlens=cu,
                              initial_state=d["initial_state"][:, sl].astype(np.float64))
        oh = o[:, sl].cpu().numpy().astype(np.float64)
        for n in range(N):
            a_, e_ = int(cu[n]), int(cu[n + 1])
            o_diff[n] = max(o_diff[n], float(np.max(np.abs(oh[a_:e_] - ro[a_:e_]))))
            o_ref[n] = max(o_ref[n], float(np.max(np.abs(ro[a_:e_]))))
            s_diff[n] = max(s_diff[n], float(np.max(np.abs(sTh[n, sl] - rS[n]))))
            s_ref[n] = max(s_ref[n], float(np.max(np.abs(rS[n]))))
        print("  heads %d-%d done" % (h0, h0 + HS - 1), flush=True)
        del ro, rS, oh
    for n in range(N):
        eo, es = o_diff[n] / o_ref[n], s_diff[n] / s_ref[n]
        print("  seq %d (T=%d): o err %.3e  state err %.3e" % (n, int(cu[n + 1] - cu[n]), eo, es), flush=True)
        assert eo < TOL_BF16 and es < TOL_BF16


# ------------------------------------------------------------ state snapshots
def snap_buffer(N, slots, H):
    return torch.full((N, slots, H, 128, 128), float("nan"), dtype=torch.float32, device="cuda")


def check_snapshots(snaps, rsnaps, lens, interval, tol):
    sh = host64(snaps)
    worst = 0.0
    for n, ln in enumerate(lens):
        for j in range(snaps.shape[1]):
            if j < ln // interval:
                e = relerr(sh[n, j], rsnaps[n, j])
                worst = max(worst, e)
                assert e < tol, (n, j, e)
            else:
                assert np.isnan(sh[n, j]).all(), (n, j)  # slots past the last whole interval stay untouched
    print("  snapshot err %.3e" % worst, flush=True)


@pytest.mark.parametrize("path,interval,bf16", [("split", 64, True), ("split", 128, True), ("single", 64, True),
                                                ("single", 192, True), ("single", 64, False)])
def test_snapshots_varlen_small(path, interval, bf16):
    """States after every `interval` tokens of each sequence (ragged and empty
    sequences, lengths on and off the interval) vs the oracle; o and final
    states as without snapshots."""
    announce("prefill snapshots %s interval=%d bf16=%s" % (path, interval, bf16))
    lens = [200, 64, 0, 130, 384, 63]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    rng = np.random.default_rng(50 + interval)
    H, N = 3, len(lens)
    d = synth.core_inputs(rng, int(cu[-1]), H, bf16=bf16)
    s0 = synth.states(rng, N, H, std=0.3)
    slots = max(lens) // interval + 1  # one spare slot that must stay untouched
    snaps = snap_buffer(N, slots, H)
    o, sT = gpu_prefill(d, cu=cu, s0=s0, path=path, snapshots=snaps, interval=interval)
    ro, rS, rsn = R.kda_serial_snapshots(d["q"].vals, d["k"].vals, d["v"].vals, d["g"].vals, d["beta"].vals,
                                         interval, cu_seqlens=cu, initial_state=s0.astype(np.float64))
    tol = TOL_BF16 if bf16 else TOL_F32
    check(o, sT, ro, rS, tol)
    check_snapshots(snaps, rsn, lens, interval, tol)
    o2, s2 = gpu_prefill(d, cu=cu, s0=s0, path=path)
    assert torch.equal(o, o2) and torch.equal(sT, s2)


def test_snapshots_across_windows_bit_equal():
    """One-chunk windows (the smallest workspace) give the same snapshots, bit
    for bit, as one window holding every chunk."""
    announce("prefill snapshots across windows")
    lens = [333, 64, 0, 257]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    rng = np.random.default_rng(61)
    H, N = 2, len(lens)
    d = synth.core_inputs(rng, int(cu[-1]), H, bf16=True)
    s0 = synth.states(rng, N, H, std=0.2)
    U = N * H
    small = torch.empty(U * SLOT + U * 128 * 128 * 4, dtype=torch.uint8, device="cuda")
    big = torch.empty(U * SLOT * ((max(lens) + 63) // 64), dtype=torch.uint8, device="cuda")
    s1, s2 = snap_buffer(N, 5, H), snap_buffer(N, 5, H)
    gpu_prefill(d, cu=cu, s0=s0, workspace=small, snapshots=s1, interval=64)
    gpu_prefill(d, cu=cu, s0=s0, workspace=big, snapshots=s2, interval=64)
    assert torch.equal(torch.nan_to_num(s1, nan=7.0), torch.nan_to_num(s2, nan=7.0))
    _, _, rsn = R.kda_serial_snapshots(d["q"].vals, d["k"].vals, d["v"].vals, d["g"].vals, d["beta"].vals, 64,
                                       cu_seqlens=cu, initial_state=s0.astype(np.float64))
    check_snapshots(s1, rsn, lens, 64, TOL_BF16)


def test_snapshots_prefill_workload_full_size():
    """The prefill workload (T = 4096, H = 64) with a snapshot every 1024
    tokens, as bench.py launches it (two-pass form, two 32-chunk windows):
    every head of every snapshot against the oracle."""
    announce("prefill snapshots full size")
    d = synth.workload_prefill()
    snaps = snap_buffer(1, 4, 64)
    o, sT = gpu_prefill(d, snapshots=snaps, interval=1024)
    sh = host64(snaps)
    ro, rS, rsn = R.kda_serial_snapshots(d["q"].vals, d["k"].vals, d["v"].vals, d["g"].vals, d["beta"].vals, 1024)
    for j in range(4):
        e = relerr(sh[0, j], rsn[0, j])
        print("  snapshot %d err %.3e" % (j, e), flush=True)
        assert e < TOL_BF16
    assert np.array_equal(sh[0, 3], host64(sT[0]))  # the last snapshot is the final state
    check(o, sT, ro, rS, TOL_BF16)


def test_wide_state_pass_matches_narrow_bit_for_bit():
    """More than 64 (sequence, head) units switch the state pass to workgroups
    of 64 columns (two tiles per wavefront). Adding an empty sequence to a
    33-head problem crosses that line; the real sequence's outputs and final
    state must not change by a bit, and both match the oracle."""
    announce("prefill wide vs narrow state pass")
    rng = np.random.default_rng(71)
    H, T = 33, 300
    d = synth.core_inputs(rng, T, H, bf16=True)
    s0 = synth.states(rng, 2, H, std=0.3)
    o1, s1 = gpu_prefill(d, cu=np.array([0, T], np.int32), s0=s0[:1])          # 33 units: narrow
    o2, s2 = gpu_prefill(d, cu=np.array([0, T, T], np.int32), s0=s0)           # 66 units: wide
    assert torch.equal(o1, o2) and torch.equal(s1[0], s2[0])
    assert np.array_equal(host64(s2[1]), s0[1].astype(np.float64))             # the empty sequence keeps its state
    ro, rS = oracle(d, cu=np.array([0, T]), s0=s0[:1])
    check(o2, s2[:1], ro, rS, TOL_BF16)


def test_wide_state_pass_windows_and_snapshots():
    """80 units (wide state pass), ragged and empty sequences, one-chunk
    windows vs one window, with snapshots: bit-equal, and equal to the oracle."""
    announce("prefill wide state pass, windows + snapshots")
    lens = [200, 64, 130, 0, 257]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    rng = np.random.default_rng(72)
    H, N = 16, len(lens)
    d = synth.core_inputs(rng, int(cu[-1]), H, bf16=True)
    s0 = synth.states(rng, N, H, std=0.2)
    U = N * H
    small = torch.empty(U * SLOT + U * 128 * 128 * 4, dtype=torch.uint8, device="cuda")
    big = torch.empty(U * SLOT * ((max(lens) + 63) // 64), dtype=torch.uint8, device="cuda")
    n1, n2 = snap_buffer(N, 4, H), snap_buffer(N, 4, H)
    o1, s1 = gpu_prefill(d, cu=cu, s0=s0, workspace=small, snapshots=n1, interval=64)
    o2, s2 = gpu_prefill(d, cu=cu, s0=s0, workspace=big, snapshots=n2, interval=64)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    assert torch.equal(torch.nan_to_num(n1, nan=7.0), torch.nan_to_num(n2, nan=7.0))
    ro, rS, rsn = R.kda_serial_snapshots(d["q"].vals, d["k"].vals, d["v"].vals, d["g"].vals, d["beta"].vals, 64,
                                         cu_seqlens=cu, initial_state=s0.astype(np.float64))
    check(o1, s1, ro, rS, TOL_BF16)
    check_snapshots(n1, rsn, lens, 64, TOL_BF16)
