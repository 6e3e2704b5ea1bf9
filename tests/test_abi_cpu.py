"""C-ABI checks that need no GPU: the library loads, exports every entry point
declared in include/kda.h, its size helpers reproduce the pages' figures, and
host-side validation rejects bad arguments before anything reaches the device
(every call below fails validation, so no kernel is launched)."""
import ctypes
import json
import os
import re

import numpy as np
import pytest

from gated_delta_rule_02_amd import kda as K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_\w+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = K.lib()
    declared = header_functions()
    assert declared, "no declarations parsed"
    for name in declared:
        assert hasattr(L, name), name
    assert sorted(K.EXPORTED) == declared


def test_version_and_sizes_match_page_figures():
    fig = json.load(open(os.path.join(ROOT, "tests", "golden", "page_figures.json")))
    assert K.kda_version() == 100
    per_layer = K.kda_state_bytes(64, 128, 128, K.KDA_F32)
    assert per_layer == 4 * 2 ** 20
    assert 63 * per_layer == fig["state_per_sequence_63_layers_mib"]["value"] * 2 ** 20
    assert 63 * K.kda_state_bytes(64, 128, 128, K.KDA_BF16) == fig["state_per_sequence_bf16_mib"]["value"] * 2 ** 20
    conv = K.kda_conv_state_bytes(3, 4, 8192, K.KDA_BF16)
    assert conv == 147456
    total = 63 * conv
    assert total < fig["conv_tails_per_sequence"]["under_mib"] * 2 ** 20
    assert round(total / 1e6) == fig["conv_tails_per_sequence"]["about_mb"]
    # crossover vs an all-MLA cache: 252 MiB / (63 layers x 1152 B per token)
    mla = fig["mla_bytes_per_token_all_9_layers"]["per_layer"]
    assert abs(63 * per_layer / (63 * mla) - fig["kda_vs_all_mla_crossover_tokens"]["fp32_about"]) < 50
    assert K.kda_state_bytes(0, 128, 128, K.KDA_F32) == 0


# ---- validation: fake, aligned, never-dereferenced device addresses -----------
BASE = 1 << 40


def fake(i, size=1 << 30):
    return BASE + i * size


def call(name, *args):
    fn = getattr(K.lib(), name)
    return fn(*args), K.kda_last_error()


def cu_host(values):
    arr = (ctypes.c_int32 * len(values))(*values)
    return arr


def prefill(**over):
    a = dict(q=fake(1), k=fake(2), v=fake(3), g=fake(4), beta=fake(5), in_dtype=K.KDA_BF16,
             T=256, H=4, dk=128, dv=128, cu_dev=None, cu_host=None, N=1, scale=1.0, lb=-5.0,
             s0=None, sT=None, o=fake(6), out_dtype=K.KDA_F32, ws=None, ws_bytes=0, stream=None)
    a.update(over)
    return call("kda_prefill", a["q"], a["k"], a["v"], a["g"], a["beta"], a["in_dtype"], a["T"], a["H"],
                a["dk"], a["dv"], a["cu_dev"], a["cu_host"], a["N"], a["scale"], a["lb"], a["s0"], a["sT"],
                a["o"], a["out_dtype"], a["ws"], a["ws_bytes"], a["stream"])


def test_prefill_validation():
    assert prefill(q=None)[0] == K.KDA_ERR_INVALID_ARG
    rc, msg = prefill(dk=64)
    assert rc == K.KDA_ERR_UNSUPPORTED and "dk = dv = 128" in msg
    assert prefill(in_dtype=7)[0] == K.KDA_ERR_INVALID_ARG
    assert prefill(q=fake(1) + 8)[0] == K.KDA_ERR_INVALID_ARG          # misaligned
    assert prefill(N=3)[0] == K.KDA_ERR_INVALID_ARG                    # 256 % 3 != 0
    h = cu_host([0, 100, 50, 256])
    rc, msg = prefill(cu_dev=fake(7), cu_host=h, N=3)
    assert rc == K.KDA_ERR_INVALID_ARG and "non-decreasing" in msg
    h = cu_host([0, 100, 200])
    rc, msg = prefill(cu_dev=fake(7), cu_host=h, N=2)
    assert rc == K.KDA_ERR_INVALID_ARG and "must equal num_tokens" in msg
    h = cu_host([1, 100, 256])
    assert prefill(cu_dev=fake(7), cu_host=h, N=2)[0] == K.KDA_ERR_INVALID_ARG
    assert prefill(cu_dev=fake(7), cu_host=None)[0] == K.KDA_ERR_INVALID_ARG
    # o overlapping an input
    assert prefill(o=fake(1) + 4096)[0] == K.KDA_ERR_INVALID_ARG
    # partial overlap of the two state buffers
    rc, msg = prefill(s0=fake(8), sT=fake(8) + 1024)
    assert rc == K.KDA_ERR_INVALID_ARG and "overlap" in msg
    # final_state overlapping q
    assert prefill(sT=fake(1) + 64)[0] == K.KDA_ERR_INVALID_ARG


def test_decode_validation():
    args = [fake(1), fake(2), fake(3), fake(4), fake(5), K.KDA_BF16, 256, 64, 128, 128, 1.0, -5.0,
            fake(6, 1 << 34), fake(9), K.KDA_F32, None]
    a = list(args); a[0] = None
    assert call("kda_decode_step", *a)[0] == K.KDA_ERR_INVALID_ARG
    a = list(args); a[8] = 96
    assert call("kda_decode_step", *a)[0] == K.KDA_ERR_UNSUPPORTED
    a = list(args); a[13] = fake(6, 1 << 34) + 256          # o inside the state
    rc, msg = call("kda_decode_step", *a)
    assert rc == K.KDA_ERR_INVALID_ARG and "overlap" in msg
    a = list(args); a[6] = 0
    assert call("kda_decode_step", *a)[0] == K.KDA_ERR_INVALID_ARG


def test_conv_and_misc_validation():
    # conv update: W out of range, C not a multiple of 128, y aliasing the state
    base = [fake(1), 8192, fake(2), fake(3), None, K.KDA_BF16, 256, 8192, 4, 1, 0, 1e-6, fake(4), None]
    a = list(base); a[8] = 9
    assert call("kda_conv_state_update", *a)[0] == K.KDA_ERR_UNSUPPORTED
    a = list(base); a[7] = 100
    assert call("kda_conv_state_update", *a)[0] == K.KDA_ERR_UNSUPPORTED
    a = list(base); a[12] = fake(2)
    assert call("kda_conv_state_update", *a)[0] == K.KDA_ERR_INVALID_ARG
    a = list(base); a[10] = 64
    assert call("kda_conv_state_update", *a)[0] == K.KDA_ERR_UNSUPPORTED
    a = list(base); a[1] = 100
    assert call("kda_conv_state_update", *a)[0] == K.KDA_ERR_INVALID_ARG
    # conv prefill: y aliasing x; bad cu_seqlens
    h = cu_host([0, 10, 5])
    rc, _ = call("kda_conv_prefill", fake(1), 8192, 10, 8192, 4, fake(2), h, 2, fake(3), None, None, None,
                 1, 0, 1e-6, fake(4), 8192, K.KDA_BF16, None)
    assert rc == K.KDA_ERR_INVALID_ARG
    rc, _ = call("kda_conv_prefill", fake(1), 8192, 10, 8192, 4, None, None, 1, fake(3), None, None, None,
                 1, 0, 1e-6, fake(1), 8192, K.KDA_BF16, None)
    assert rc == K.KDA_ERR_INVALID_ARG
    # gemm: unsupported fp32 operands, misaligned ld
    rc, _ = call("kda_gemm", fake(1), 4096, fake(2), 4096, fake(3), 8192, 64, 8192, 4096, K.KDA_F32, K.KDA_F32, None)
    assert rc == K.KDA_ERR_UNSUPPORTED
    rc, _ = call("kda_gemm", fake(1), 4095, fake(2), 4096, fake(3), 8192, 64, 8192, 4095, K.KDA_BF16, K.KDA_F32, None)
    assert rc != K.KDA_OK
    # gate and epilogue: dk != 128
    rc, _ = call("kda_gate_prologue", fake(1), 8192, fake(2), 64, fake(3), 8, 64, 64, -5.0, K.KDA_BF16,
                 fake(4), fake(5), K.KDA_BF16, None)
    assert rc == K.KDA_ERR_UNSUPPORTED
    rc, _ = call("kda_output_norm_gate", fake(1), K.KDA_F32, fake(2), 8192, fake(3), 8, 64, 128, 1e-6,
                 fake(1), K.KDA_BF16, None)
    assert rc == K.KDA_ERR_INVALID_ARG


def test_error_message_cleared_on_success_path_helpers():
    prefill(q=None)
    assert K.kda_last_error() != ""


def snapshots_call(interval=128, slots=2, snap=None, **over):
    a = dict(q=fake(1), k=fake(2), v=fake(3), g=fake(4), beta=fake(5), in_dtype=K.KDA_BF16,
             T=256, H=4, dk=128, dv=128, cu_dev=None, cu_host=None, N=1, scale=1.0, lb=-5.0,
             s0=None, sT=None, o=fake(6), out_dtype=K.KDA_F32, ws=None, ws_bytes=0, stream=None)
    a.update(over)
    return call("kda_prefill_snapshots", a["q"], a["k"], a["v"], a["g"], a["beta"], a["in_dtype"], a["T"], a["H"],
                a["dk"], a["dv"], a["cu_dev"], a["cu_host"], a["N"], a["scale"], a["lb"], a["s0"], a["sT"],
                a["o"], a["out_dtype"], a["ws"], a["ws_bytes"], interval, slots,
                fake(10) if snap is None else snap, a["stream"])


def test_prefill_snapshots_validation():
    rc, msg = snapshots_call(interval=100)
    assert rc == K.KDA_ERR_INVALID_ARG and "multiple of 64" in msg
    assert snapshots_call(interval=0)[0] == K.KDA_ERR_INVALID_ARG
    rc, msg = snapshots_call(interval=64, slots=3)          # 256 tokens need 4 slots
    assert rc == K.KDA_ERR_INVALID_ARG and "4 snapshot slots" in msg
    h = cu_host([0, 64, 256])                               # longest sequence 192 -> 3 slots of 64
    assert snapshots_call(interval=64, slots=2, cu_dev=fake(7), cu_host=h, N=2)[0] == K.KDA_ERR_INVALID_ARG
    rc, msg = snapshots_call(snap=fake(6) + 4096)           # snapshots inside o
    assert rc == K.KDA_ERR_INVALID_ARG and "overlap" in msg
    assert snapshots_call(snap=fake(10) + 8)[0] == K.KDA_ERR_INVALID_ARG   # misaligned
    fn = getattr(K.lib(), "kda_prefill_snapshots")
    rc = fn(fake(1), fake(2), fake(3), fake(4), fake(5), K.KDA_BF16, 256, 4, 128, 128, None, None, 1, 1.0, -5.0,
            None, None, fake(6), K.KDA_F32, None, 0, 128, 2, None, None)
    assert rc == K.KDA_ERR_INVALID_ARG and "null snapshots" in K.kda_last_error()


def test_decode_multi_and_commit_validation():
    # q k v g beta dtype B Tq H dk dv scale lb state token_states state_dtype o out_dtype stream
    args = [fake(1), fake(2), fake(3), fake(4), fake(5), K.KDA_BF16, 64, 4, 16, 128, 128, 1.0, -5.0,
            fake(6, 1 << 34), fake(7, 1 << 34), K.KDA_F32, fake(9), K.KDA_F32, None]
    a = list(args); a[7] = 0
    assert call("kda_decode_multi", *a)[0] == K.KDA_ERR_INVALID_ARG
    a = list(args); a[9] = 64
    assert call("kda_decode_multi", *a)[0] == K.KDA_ERR_UNSUPPORTED
    a = list(args); a[14] = fake(6, 1 << 34) + 4096         # token_states inside the state
    rc, msg = call("kda_decode_multi", *a)
    assert rc == K.KDA_ERR_INVALID_ARG and "token_states overlaps" in msg
    a = list(args); a[16] = fake(7, 1 << 34) + 1024         # o inside token_states
    assert call("kda_decode_multi", *a)[0] == K.KDA_ERR_INVALID_ARG
    a = list(args); a[14] = fake(7, 1 << 34) + 4            # misaligned
    assert call("kda_decode_multi", *a)[0] == K.KDA_ERR_INVALID_ARG
    a = list(args); a[15] = 5                               # bad state dtype
    assert call("kda_decode_multi", *a)[0] == K.KDA_ERR_INVALID_ARG
    # a bf16 state is half the bytes: o right after a bf16 state of 64*16*32 KiB does not overlap it
    a = list(args); a[15] = K.KDA_BF16; a[16] = fake(6, 1 << 34) + 64 * 16 * 32768
    a[14] = None
    fn = getattr(K.lib(), "kda_decode_multi")
    a2 = list(a); a2[16] = fake(6, 1 << 34) + 64 * 16 * 32768 - 16   # but 16 bytes earlier it does
    assert call("kda_decode_multi", *a2)[0] == K.KDA_ERR_INVALID_ARG
    # commit: state overlapping token_states, bad sizes, unsupported dk, bad dtype
    rc, msg = call("kda_decode_commit", fake(1, 1 << 34), fake(2), 64, 4, 16, 128, 128, fake(1, 1 << 34) + 65536,
                   K.KDA_F32, None)
    assert rc == K.KDA_ERR_INVALID_ARG and "overlaps" in msg
    assert call("kda_decode_commit", fake(1, 1 << 34), fake(2), 64, 0, 16, 128, 128, fake(3, 1 << 34),
                K.KDA_F32, None)[0] == K.KDA_ERR_INVALID_ARG
    assert call("kda_decode_commit", fake(1, 1 << 34), fake(2), 64, 4, 16, 128, 64, fake(3, 1 << 34),
                K.KDA_F32, None)[0] == K.KDA_ERR_UNSUPPORTED
    assert call("kda_decode_commit", None, fake(2), 64, 4, 16, 128, 128, fake(3, 1 << 34),
                K.KDA_F32, None)[0] == K.KDA_ERR_INVALID_ARG
    assert call("kda_decode_commit", fake(1, 1 << 34), fake(2), 64, 4, 16, 128, 128, fake(3, 1 << 34),
                9, None)[0] == K.KDA_ERR_INVALID_ARG


def test_state_convert_validation():
    assert call("kda_state_convert", fake(1), K.KDA_F32, fake(1) + 1024, K.KDA_BF16, 4096, None)[0] == \
        K.KDA_ERR_INVALID_ARG                                  # overlap
    assert call("kda_state_convert", fake(1), K.KDA_F32, fake(2) + 8, K.KDA_BF16, 4096, None)[0] == \
        K.KDA_ERR_INVALID_ARG                                  # misaligned
    assert call("kda_state_convert", fake(1), 3, fake(2), K.KDA_BF16, 4096, None)[0] == K.KDA_ERR_INVALID_ARG
    assert call("kda_state_convert", fake(1), K.KDA_F32, fake(2), K.KDA_BF16, -1, None)[0] == K.KDA_ERR_INVALID_ARG
    assert call("kda_state_convert", None, K.KDA_F32, None, K.KDA_BF16, 0, None)[0] == K.KDA_OK  # nothing to do


def test_fp8_validation():
    # x ldx w ldw ws ws_ld y ldy M N K x_dtype y_dtype stream
    base = [fake(1), 4096, fake(2), 4096, fake(3), 32, fake(4), 8192, 1, 8192, 4096, K.KDA_BF16, K.KDA_F32, None]
    a = list(base); a[8] = 9
    assert call("kda_gemv_fp8", *a)[0] == K.KDA_ERR_UNSUPPORTED          # M > 8
    a = list(base); a[10] = 4000; a[1] = 4000; a[3] = 4000
    assert call("kda_gemv_fp8", *a)[0] == K.KDA_ERR_UNSUPPORTED          # K not a multiple of 128
    a = list(base); a[3] = 4104
    assert call("kda_gemv_fp8", *a)[0] == K.KDA_ERR_INVALID_ARG          # ldw not a multiple of 16
    a = list(base); a[11] = K.KDA_F32
    assert call("kda_gemv_fp8", *a)[0] == K.KDA_ERR_UNSUPPORTED          # x must be bf16
    a = list(base); a[6] = fake(2) + 1024
    rc, msg = call("kda_gemv_fp8", *a)
    assert rc == K.KDA_ERR_INVALID_ARG and "overlaps" in msg
    a = list(base); a[5] = 16
    assert call("kda_gemv_fp8", *a)[0] == K.KDA_ERR_INVALID_ARG          # ws_ld < K/128
    # epilogue: dv != 128, outputs overlapping
    e = [fake(1), K.KDA_F32, fake(2), 8192, K.KDA_BF16, fake(3), 16, 64, 128, 1e-6, fake(4), fake(5), None]
    a = list(e); a[8] = 64
    assert call("kda_output_norm_gate_fp8", *a)[0] == K.KDA_ERR_UNSUPPORTED
    a = list(e); a[11] = fake(4) + 64
    assert call("kda_output_norm_gate_fp8", *a)[0] == K.KDA_ERR_INVALID_ARG
    a = list(e); a[10] = fake(1) + 256
    assert call("kda_output_norm_gate_fp8", *a)[0] == K.KDA_ERR_INVALID_ARG


def test_w8a8_validation():
    """kda_quantize_fp8 and kda_gemm_fp8 refuse bad groups, strides and overlaps
    before any launch."""
    # quantize: x ldx x_dtype M K codes ldc scales ld_scale stream
    q = [fake(1), 4096, K.KDA_BF16, 64, 4096, fake(2), 4096, fake(3), 32, None]
    a = list(q); a[4] = 4000; a[1] = 4000; a[6] = 4000
    assert call("kda_quantize_fp8", *a)[0] == K.KDA_ERR_UNSUPPORTED       # K not a multiple of 128
    a = list(q); a[8] = 31
    assert call("kda_quantize_fp8", *a)[0] == K.KDA_ERR_INVALID_ARG       # ld_scale < K/128
    a = list(q); a[5] = fake(1) + 4096
    rc, msg = call("kda_quantize_fp8", *a)
    assert rc == K.KDA_ERR_INVALID_ARG and "overlap" in msg               # codes over x
    a = list(q); a[7] = fake(2) + 1024
    assert call("kda_quantize_fp8", *a)[0] == K.KDA_ERR_INVALID_ARG       # scales over codes
    a = list(q); a[0] = None
    assert call("kda_quantize_fp8", *a)[0] == K.KDA_ERR_INVALID_ARG
    a = list(q); a[3] = 0
    assert call("kda_quantize_fp8", *a)[0] == K.KDA_OK                    # no rows: nothing to do
    # gemm: x ldx xs xs_ld w ldw ws ws_ld y ldy M N K y_dtype stream
    g = [fake(1), 4096, fake(2), 32, fake(3), 4096, fake(4), 32, fake(5), 8192, 512, 8192, 4096, K.KDA_BF16, None]
    a = list(g); a[12] = 4000; a[1] = 4000; a[5] = 4000
    assert call("kda_gemm_fp8", *a)[0] == K.KDA_ERR_UNSUPPORTED           # K not a multiple of 128
    a = list(g); a[1] = 4104
    assert call("kda_gemm_fp8", *a)[0] == K.KDA_ERR_INVALID_ARG           # ldx not a multiple of 16
    a = list(g); a[3] = 16
    assert call("kda_gemm_fp8", *a)[0] == K.KDA_ERR_INVALID_ARG           # xs_ld < K/128
    a = list(g); a[8] = fake(3) + 4096
    rc, msg = call("kda_gemm_fp8", *a)
    assert rc == K.KDA_ERR_INVALID_ARG and "overlaps" in msg
    a = list(g); a[2] = None
    assert call("kda_gemm_fp8", *a)[0] == K.KDA_ERR_INVALID_ARG
    a = list(g); a[10] = 0
    assert call("kda_gemm_fp8", *a)[0] == K.KDA_OK


def segmaps(**over):
    a = dict(k=fake(2), v=fake(3), g=fake(4), beta=fake(5), in_dtype=K.KDA_BF16, T=256, H=4, dk=128, dv=128,
             cu_dev=None, cu_host=None, N=1, lb=-5.0, M=fake(7), Nout=fake(8), ws=fake(9), ws_bytes=1 << 28,
             stream=None)
    a.update(over)
    return call("kda_prefill_segment_maps", a["k"], a["v"], a["g"], a["beta"], a["in_dtype"], a["T"], a["H"],
                a["dk"], a["dv"], a["cu_dev"], a["cu_host"], a["N"], a["lb"], a["M"], a["Nout"], a["ws"],
                a["ws_bytes"], a["stream"])


def test_segment_maps_validation():
    """Rejected before any launch: float32 inputs (no two-pass form), other
    head sizes, missing outputs or workspace, a workspace below one slot per
    unit plus the carry, overlapping outputs, misalignment, bad boundaries."""
    assert segmaps(in_dtype=K.KDA_F32)[0] == K.KDA_ERR_UNSUPPORTED
    assert segmaps(dk=64)[0] == K.KDA_ERR_UNSUPPORTED
    assert segmaps(M=None)[0] == K.KDA_ERR_INVALID_ARG
    assert segmaps(Nout=None)[0] == K.KDA_ERR_INVALID_ARG
    rc, msg = segmaps(ws=None)
    assert rc == K.KDA_ERR_WORKSPACE and "workspace" in msg
    assert segmaps(ws_bytes=1000)[0] == K.KDA_ERR_WORKSPACE
    rc, msg = segmaps(Nout=fake(7) + 2 * 128 * 128 * 4)  # inside M_out (4 units x 64 KiB)
    assert rc == K.KDA_ERR_INVALID_ARG and "overlaps" in msg
    assert segmaps(M=fake(7) + 8)[0] == K.KDA_ERR_INVALID_ARG
    assert segmaps(k=None)[0] == K.KDA_ERR_INVALID_ARG
    cu = cu_host([0, 200, 100, 256])
    assert segmaps(cu_dev=fake(10), cu_host=cu, N=3)[0] == K.KDA_ERR_INVALID_ARG
    assert segmaps(ws=fake(2) + 4096)[0] == K.KDA_ERR_INVALID_ARG  # workspace inside k


def test_affine_apply_validation():
    """Rejected before any launch: other sizes, negative counts, missing
    operands, Y overlapping M or X, Y partly overlapping N, misalignment;
    count = 0 does nothing and succeeds."""
    f = lambda M=fake(1), X=fake(2), N=fake(3), Y=fake(4), count=4, dk=128, dv=128: \
        call("kda_affine_apply", M, X, N, Y, count, dk, dv, None)
    assert f(dk=64)[0] == K.KDA_ERR_UNSUPPORTED
    assert f(count=-1)[0] == K.KDA_ERR_INVALID_ARG
    assert f(count=0)[0] == K.KDA_OK
    assert f(M=None)[0] == K.KDA_ERR_INVALID_ARG
    assert f(Y=fake(2) + 65536)[0] == K.KDA_ERR_INVALID_ARG       # inside X
    assert f(Y=fake(1))[0] == K.KDA_ERR_INVALID_ARG               # is M
    assert f(Y=fake(3) + 65536)[0] == K.KDA_ERR_INVALID_ARG       # partly N
    assert f(X=fake(2) + 4)[0] == K.KDA_ERR_INVALID_ARG


def test_lower_bound_validation():
    """The log-retention floor is checked before any launch. The chunked forms
    (prefill, snapshots, segment maps) take floors in [-5.4, 0]: below that a
    block of 16 clamped log-retentions would push a decay factor 2^x out of the
    normal float32 range. NaN and positive floors are invalid everywhere; the
    token-serial decode and the gate take any floor <= 0 (-inf: no clamp)."""
    nan, inf = float("nan"), float("inf")
    for lb in (nan, 0.5, inf):
        rc, msg = prefill(lb=lb)
        assert rc == K.KDA_ERR_INVALID_ARG and "lower_bound" in msg, (lb, rc, msg)
        rc, msg = segmaps(lb=lb)
        assert rc == K.KDA_ERR_INVALID_ARG and "lower_bound" in msg, (lb, rc, msg)
    for lb in (-5.41, -6.0, -20.0, -inf):
        rc, msg = prefill(lb=lb)
        assert rc == K.KDA_ERR_UNSUPPORTED and "lower_bound" in msg, (lb, rc, msg)
        rc, msg = segmaps(lb=lb)
        assert rc == K.KDA_ERR_UNSUPPORTED and "lower_bound" in msg, (lb, rc, msg)
    # in range: validation moves on to the next check (a misaligned q here)
    for lb in (-5.4, -5.0, -1.0, 0.0):
        rc, msg = prefill(lb=lb, q=fake(1) + 8)
        assert rc == K.KDA_ERR_INVALID_ARG and "aligned" in msg, (lb, rc, msg)
    dec = [fake(1), fake(2), fake(3), fake(4), fake(5), K.KDA_BF16, 256, 64, 128, 128, 1.0, -5.0,
           fake(6, 1 << 34), fake(9), K.KDA_F32, None]
    for lb in (nan, 0.5):
        a = list(dec); a[11] = lb
        rc, msg = call("kda_decode_step", *a)
        assert rc == K.KDA_ERR_INVALID_ARG and "lower_bound" in msg
    for lb in (-6.0, -inf):
        a = list(dec); a[11] = lb; a[0] = fake(1) + 8
        rc, msg = call("kda_decode_step", *a)
        assert rc == K.KDA_ERR_INVALID_ARG and "aligned" in msg
    gate = [fake(1), 8192, fake(2), 64, fake(3), 16, 64, 128, -5.0, K.KDA_BF16, fake(4), fake(5), K.KDA_BF16, None]
    a = list(gate); a[8] = nan
    rc, msg = call("kda_gate_prologue", *a)
    assert rc == K.KDA_ERR_INVALID_ARG and "lower_bound" in msg


def test_prefill_noalloc_validation():
    """kda_prefill_noalloc validates like kda_prefill and rejects a problem
    whose minimum workspace exceeds the static scratch before touching the
    device (1,300 units x (72,192-byte slot + 64 KiB carry) > 160 MiB)."""
    assert K.kda_prefill_noalloc_scratch_bytes() == 160 << 20
    f = lambda T=256, H=4, N=1, lb=-5.0, q=fake(1), in_dtype=K.KDA_BF16: call(
        "kda_prefill_noalloc", q, fake(2), fake(3), fake(4), fake(5), in_dtype, T, H, 128, 128, None, None, N,
        1.0, lb, None, None, fake(6), K.KDA_F32, None)
    rc, msg = f(T=2 * 1300 * 64, H=1300, N=1)
    assert rc == K.KDA_ERR_WORKSPACE and "static scratch" in msg, msg
    rc, msg = f(lb=-6.0)
    assert rc == K.KDA_ERR_UNSUPPORTED and "lower_bound" in msg
    assert f(q=None)[0] == K.KDA_ERR_INVALID_ARG
    assert f(q=fake(1) + 8)[0] == K.KDA_ERR_INVALID_ARG


def prefill_gated(**over):
    a = dict(q=fake(1), k=fake(2), v=fake(3), f=fake(4), f_ld=4 * 128, b=fake(5), b_ld=4, A_log=fake(7),
             in_dtype=K.KDA_BF16, T=256, H=4, dk=128, dv=128, cu_dev=None, cu_host=None, N=1, scale=1.0,
             lb=-5.0, s0=None, sT=None, o=fake(6), out_dtype=K.KDA_F32, ws=fake(8), ws_bytes=1 << 29,
             stream=None)
    a.update(over)
    return call("kda_prefill_gated", a["q"], a["k"], a["v"], a["f"], a["f_ld"], a["b"], a["b_ld"], a["A_log"],
                a["in_dtype"], a["T"], a["H"], a["dk"], a["dv"], a["cu_dev"], a["cu_host"], a["N"], a["scale"],
                a["lb"], a["s0"], a["sT"], a["o"], a["out_dtype"], a["ws"], a["ws_bytes"], a["stream"])


def test_prefill_gated_validation():
    """kda_prefill_gated: the two-pass form only, strided gate rows checked
    for shape, alignment and overlap (every call below fails validation)."""
    rc, msg = prefill_gated(in_dtype=K.KDA_F32)
    assert rc == K.KDA_ERR_UNSUPPORTED and "bfloat16" in msg
    rc, msg = prefill_gated(ws=None, ws_bytes=0)
    assert rc == K.KDA_ERR_WORKSPACE
    rc, msg = prefill_gated(f_ld=4 * 128 - 8)           # shorter than H * 128
    assert rc == K.KDA_ERR_INVALID_ARG and "f_ld" in msg
    assert prefill_gated(f_ld=4 * 128 + 4)[0] == K.KDA_ERR_INVALID_ARG   # not a multiple of 8
    assert prefill_gated(f_ld=1 << 24)[0] == K.KDA_ERR_INVALID_ARG
    rc, msg = prefill_gated(b_ld=3)
    assert rc == K.KDA_ERR_INVALID_ARG and "b_ld" in msg
    rc, msg = prefill_gated(A_log=None)
    assert rc == K.KDA_ERR_INVALID_ARG and "A_log" in msg
    assert prefill_gated(f=fake(4) + 2)[0] == K.KDA_ERR_INVALID_ARG    # f misaligned
    assert prefill_gated(b=fake(5) + 1)[0] == K.KDA_ERR_INVALID_ARG    # b misaligned
    # the strided f rows reach into o; b rows into the workspace
    rc, msg = prefill_gated(f=fake(6) - 255 * 4 * 128 * 2, f_ld=4 * 128 + 8)
    assert rc == K.KDA_ERR_INVALID_ARG and "o overlaps" in msg
    rc, msg = prefill_gated(b=fake(8) - 1024, b_ld=64)
    assert rc == K.KDA_ERR_INVALID_ARG and "workspace overlaps" in msg
    assert prefill_gated(lb=-6.0)[0] == K.KDA_ERR_UNSUPPORTED
    assert prefill_gated(dk=64)[0] == K.KDA_ERR_UNSUPPORTED
