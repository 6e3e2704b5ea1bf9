"""Block FP8 on the GPU against the oracle: the FP8-weight GEMV (decode) and
the epilogue with its output quantized to E4M3 per (token, head)."""
import numpy as np
import pytest
import torch

from gated_delta_rule_02_amd import kda as K
from gated_delta_rule_02_amd import synth
from oracle import reference as R
from tests.gpu_util import TOL_BF16, announce, dev, host64, relerr

pytestmark = pytest.mark.gpu


def fp8_weights(rng, N, Kd):
    """Random finite E4M3 codes (NaN codes replaced) and per-block scales."""
    codes = rng.integers(0, 256, (N, Kd), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3C
    scales = rng.uniform(1e-3, 1e-2, ((N + 127) // 128, Kd // 128)).astype(np.float32)
    return codes, scales


def run_gemv(M, N, Kd, out_dtype=torch.float32, seed=0):
    rng = np.random.default_rng(seed)
    codes, scales = fp8_weights(rng, N, Kd)
    x = synth.normal(rng, (M, Kd))
    y = torch.full((M, N), float("nan"), dtype=out_dtype, device="cuda")
    K.kda_gemv_fp8(dev(x), torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(), y)
    torch.cuda.synchronize()
    ref = R.gemv_fp8_blocks(x.vals, codes, scales)
    return y, ref


@pytest.mark.parametrize("M,N,Kd", [(1, 300, 128), (3, 257, 1152), (8, 1000, 4096), (2, 16, 2048), (5, 4099, 256),
                                    (6, 130, 384), (7, 64, 8192), (1, 1, 3072)])
def test_gemv_fp8_small(M, N, Kd):
    announce("gemv fp8 M=%d N=%d K=%d" % (M, N, Kd))
    y, ref = run_gemv(M, N, Kd, seed=M * 7 + N)
    e = relerr(host64(y), ref)
    print("  err %.2e" % e, flush=True)
    assert e < 2e-5


def test_gemv_fp8_strided_rows():
    """x, y and the weight codes as row-strided views of wider buffers (ldx > K,
    ldy > N, ldw > K), for one token, for four (row form) and for six (the
    matrix-core form)."""
    for M, N, Kd in ((1, 777, 2048), (4, 300, 1024), (6, 333, 1536)):
        announce("gemv fp8 strided M=%d N=%d K=%d" % (M, N, Kd))
        rng = np.random.default_rng(40 + M)
        codes, scales = fp8_weights(rng, N, Kd)
        x = synth.normal(rng, (M, Kd))
        xb = torch.zeros((M, Kd + 64), dtype=torch.bfloat16, device="cuda")
        xb[:, :Kd] = dev(x)
        wb = torch.full((N, Kd + 48), 0x7F, dtype=torch.uint8)  # NaN codes in the padding: never read
        wb[:, :Kd] = torch.from_numpy(codes)
        wb = wb.cuda()
        yb = torch.full((M, N + 5), float("nan"), dtype=torch.float32, device="cuda")
        K.kda_gemv_fp8(xb[:, :Kd], wb[:, :Kd], torch.from_numpy(scales).cuda(), yb[:, :N])
        torch.cuda.synchronize()
        assert relerr(host64(yb[:, :N]), R.gemv_fp8_blocks(x.vals, codes, scales)) < 2e-5
        assert torch.isnan(yb[:, N:]).all()


def test_gemv_fp8_bf16_output():
    announce("gemv fp8 bf16 out")
    y, ref = run_gemv(4, 513, 1024, out_dtype=torch.bfloat16, seed=3)
    assert relerr(host64(y), ref) < 5e-3


@pytest.mark.parametrize("M,N,Kd", [(1, 5 * 8192 + 64, 4096), (1, 4096, 8192), (8, 5 * 8192 + 64, 4096),
                                    (6, 4096, 8192)])
def test_gemv_fp8_layer_shapes_full(M, N, Kd):
    """The layer's projections at full size: the input projection (41,024 x
    4,096) and the output projection (4,096 x 8,192), for one decode token and
    for several (the matrix-core form); every output checked."""
    announce("gemv fp8 full M=%d N=%d K=%d" % (M, N, Kd))
    y, ref = run_gemv(M, N, Kd, seed=N + M)
    e = relerr(host64(y), ref)
    print("  err %.2e" % e, flush=True)
    assert e < 2e-5


def test_output_norm_gate_fp8():
    """Codes and scales per (token, head): scales equal the oracle's to 1e-6;
    every dequantized value within half an E4M3 step (plus float32 slack) of
    the oracle's exact value; the group maximum sits on +-448; at least 99% of
    the codes equal the oracle's (the rest are float32 rounding at a tie)."""
    announce("output norm gate fp8")
    rng = np.random.default_rng(50)
    T, H = 37, 5
    o = (rng.standard_normal((T, H, 128)) * rng.uniform(0.01, 3.0, (T, H, 1))).astype(np.float32)
    o[3, 2] = 0.0  # an all-zero head: scale 1, codes 0
    gate = synth.normal(rng, (T, H * 128 + 8))
    w = rng.uniform(0.5, 1.5, 128).astype(np.float32)
    codes = torch.empty((T, H * 128), dtype=torch.uint8, device="cuda")
    scales = torch.empty((T, H), dtype=torch.float32, device="cuda")
    K.kda_output_norm_gate_fp8(torch.from_numpy(o).cuda(), dev(gate), torch.from_numpy(w).cuda(), codes, scales)
    torch.cuda.synchronize()
    y = R.output_norm_gate(o, gate.vals[:, :H * 128], w).reshape(T, H * 128)
    rc, rs = R.quantize_fp8_groups(y)
    gc, gs = codes.cpu().numpy(), scales.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(gs - rs) / rs) < 1e-6
    assert np.all(gc[3, 256:384] == 0) and gs[3, 2] == 1.0
    deq = R.e4m3_decode(gc) * np.repeat(gs, 128, axis=1)
    bound = np.maximum(2.0 ** -4 * np.abs(y), 2.0 ** -10 * np.repeat(rs, 128, axis=1)) * (1 + 2e-3) + 1e-7 * np.abs(y)
    assert np.all(np.abs(deq - y) <= bound)
    mx = np.max(gc.reshape(T, H, 128) & 0x7F, axis=-1)
    assert np.all(mx[rs != 1.0] == 0x7E)
    same = np.mean(gc == rc)
    print("  codes equal to the oracle's: %.4f" % same, flush=True)
    assert same >= 0.99


# ------------------------------------------------------------ block FP8 W8A8
def fp8_codes(rng, shape):
    """Random finite E4M3 codes (NaN codes replaced)."""
    c = rng.integers(0, 256, shape, dtype=np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x3C
    return c


@pytest.mark.parametrize("M,Kd,xdt,ld_pad", [(1, 128, "bf16", 0), (7, 384, "bf16", 16), (64, 4096, "bf16", 0),
                                            (33, 640, "f32", 8), (8192, 4096, "bf16", 0)])
def test_quantize_fp8_bit_exact(M, Kd, xdt, ld_pad):
    """Dynamic activation quantization: codes and scales equal the oracle's
    float32-decision quantizer bit for bit (magnitudes over 2^-20 .. 2^20 per
    row, all-zero groups, groups with one large outlier; ragged 512-column
    strips; row-strided input and output); the prefill shape 8192 x 4096 in full."""
    announce("quantize fp8 M=%d Kd=%d %s" % (M, Kd, xdt))
    rng = np.random.default_rng(70 + M + Kd)
    xv = (rng.standard_normal((M, Kd)) * np.exp2(rng.integers(-20, 20, (M, 1)))).astype(np.float32)
    xv[0, :128] = 0.0
    if M > 2:
        xv[2, 5] = 3e4 * np.abs(xv[2]).max()
    if xdt == "bf16":
        xt = torch.from_numpy(xv).to(torch.bfloat16)
        xv = xt.float().numpy()            # the values the kernel sees
        buf = torch.zeros((M, Kd + ld_pad), dtype=torch.bfloat16)
        buf[:, :Kd] = xt
    else:
        buf = torch.zeros((M, Kd + ld_pad), dtype=torch.float32)
        buf[:, :Kd] = torch.from_numpy(xv)
    x = buf.cuda()[:, :Kd]
    codes_b = torch.full((M, Kd + ld_pad), 0xEE, dtype=torch.uint8, device="cuda")
    scales_b = torch.full((M, Kd // 128 + 1), -1.0, dtype=torch.float32, device="cuda")
    K.kda_quantize_fp8(x, codes_b[:, :Kd], scales_b[:, :Kd // 128])
    torch.cuda.synchronize()
    rc, rs = R.quantize_fp8_groups_f32(xv)
    gc, gs = codes_b[:, :Kd].cpu().numpy(), scales_b[:, :Kd // 128].cpu().numpy()
    nbad = int(np.sum(gc != rc))
    print("  codes differing: %d of %d; scales equal: %s" % (nbad, gc.size, np.array_equal(gs, rs)), flush=True)
    assert nbad == 0
    np.testing.assert_array_equal(gs, rs)
    assert np.all(codes_b[:, Kd:].cpu().numpy() == 0xEE) and np.all(scales_b[:, Kd // 128:].cpu().numpy() == -1.0)


def run_w8a8(M, N, Kd, out_dtype=torch.float32, seed=0, pad=0):
    rng = np.random.default_rng(seed)
    xc = fp8_codes(rng, (M, Kd))
    xs = rng.uniform(1e-2, 1.0, (M, Kd // 128)).astype(np.float32)
    wc = fp8_codes(rng, (N, Kd))
    ws = rng.uniform(1e-3, 1e-2, ((N + 127) // 128, Kd // 128)).astype(np.float32)
    xb = torch.zeros((M, Kd + pad), dtype=torch.uint8)
    xb[:, :Kd] = torch.from_numpy(xc)
    y = torch.full((M, N + pad), float("nan"), dtype=out_dtype, device="cuda")
    K.kda_gemm_fp8(xb.cuda()[:, :Kd], torch.from_numpy(xs).cuda(), torch.from_numpy(wc).cuda(),
                   torch.from_numpy(ws).cuda(), y[:, :N])
    torch.cuda.synchronize()
    if pad:
        assert torch.isnan(y[:, N:]).all()
    return y[:, :N], R.gemm_fp8_w8a8(xc, xs, wc, ws)


# Bounds of the W8A8 paths against the exact product. The GEMV forms (M <= 8)
# convert the codes exactly to bfloat16 or float32 and accumulate in float32:
# 2e-5. The FP8 matrix instruction sums the 128 E4M3 products of a block with
# about 14 bits of relative precision (measured 6-7e-5 of the largest output
# for normal and subnormal codes alike; sums of subnormal products alone come
# out to 1e-7), and the blocks are then summed in float32 after scaling:
# 2.5e-4 leaves a 3.5x margin. Either is far below the quantization error of
# W8A8 itself (about 2^-4 per value).
TOL_W8A8_GEMV, TOL_W8A8_MFMA = 2e-5, 2.5e-4


@pytest.mark.parametrize("M,N,Kd", [(1, 300, 128), (4, 257, 1152), (6, 130, 384), (8, 1000, 4096),
                                    (9, 300, 256), (100, 513, 512), (300, 356, 1024), (257, 1000, 2048),
                                    (1000, 64, 128), (512, 512, 8192)])
def test_gemm_fp8_w8a8(M, N, Kd):
    """W8A8 against the oracle's float64 product of the decoded, scaled codes:
    the GEMV forms (M <= 8) and the matrix-core GEMM (ragged M and N, one to
    64 scale blocks along K)."""
    announce("gemm fp8 w8a8 M=%d N=%d K=%d" % (M, N, Kd))
    y, ref = run_w8a8(M, N, Kd, seed=M * 13 + N)
    e = relerr(host64(y), ref)
    print("  err %.2e" % e, flush=True)
    assert e < (TOL_W8A8_GEMV if M <= 8 else TOL_W8A8_MFMA)


def test_gemm_fp8_w8a8_strided_and_bf16():
    for M in (5, 200):
        announce("gemm fp8 w8a8 strided/bf16 M=%d" % M)
        y, ref = run_w8a8(M, 300, 1024, seed=90 + M, pad=48)
        assert relerr(host64(y), ref) < (TOL_W8A8_GEMV if M <= 8 else TOL_W8A8_MFMA)
        y, ref = run_w8a8(M, 300, 1024, out_dtype=torch.bfloat16, seed=91 + M, pad=16)
        assert relerr(host64(y), ref) < 5e-3


@pytest.mark.parametrize("M,N,Kd", [(8192, 5 * 8192 + 64, 4096), (8192, 4096, 8192), (1, 5 * 8192 + 64, 4096),
                                    (6, 4096, 8192)])
def test_gemm_fp8_w8a8_layer_shapes_full(M, N, Kd):
    """The layer's projections in W8A8 at full size, every output: the input
    projection (41,024 x 4,096) and the output projection (4,096 x 8,192) for
    the 8,192-token prefill and for decode tokens."""
    announce("gemm fp8 w8a8 full M=%d N=%d K=%d" % (M, N, Kd))
    y, ref = run_w8a8(M, N, Kd, out_dtype=torch.bfloat16 if M > 8 else torch.float32, seed=N + M)
    e = relerr(host64(y), ref)
    print("  err %.2e" % e, flush=True)
    assert e < (5e-3 if M > 8 else TOL_W8A8_GEMV)


def test_epilogue_fp8_feeds_w8a8_projection():
    """The output projection takes the quantized epilogue directly (codes
    [T, H*128], one scale per (token, head) = per 128-column group): the GPU
    chain against the oracle's own chain (float64 epilogue, its quantizer,
    the W8A8 product). The two quantizers may round a value lying within
    float32 rounding of a tie differently (about 1% of the codes; one code
    step each), so the bound is 1% of the largest output."""
    for T in (6, 300):
        announce("epilogue fp8 -> w8a8 projection T=%d" % T)
        rng = np.random.default_rng(95 + T)
        H, N = 16, 1000
        o = (rng.standard_normal((T, H, 128)) * rng.uniform(0.1, 3.0, (T, H, 1))).astype(np.float32)
        gate = synth.normal(rng, (T, H * 128))
        w = rng.uniform(0.5, 1.5, 128).astype(np.float32)
        wc = fp8_codes(rng, (N, H * 128))
        ws = rng.uniform(1e-3, 1e-2, ((N + 127) // 128, H)).astype(np.float32)
        codes = torch.empty((T, H * 128), dtype=torch.uint8, device="cuda")
        scales = torch.empty((T, H), dtype=torch.float32, device="cuda")
        K.kda_output_norm_gate_fp8(torch.from_numpy(o).cuda(), dev(gate), torch.from_numpy(w).cuda(), codes, scales)
        y = torch.empty((T, N), dtype=torch.float32, device="cuda")
        K.kda_gemm_fp8(codes, scales, torch.from_numpy(wc).cuda(), torch.from_numpy(ws).cuda(), y)
        torch.cuda.synchronize()
        yo = R.output_norm_gate(o, gate.vals, w).reshape(T, H * 128)
        rc, rs = R.quantize_fp8_groups(yo)
        ref = R.gemm_fp8_w8a8(rc, rs, wc, ws)
        e = relerr(host64(y), ref)
        print("  err %.2e" % e, flush=True)
        assert e < 1e-2
