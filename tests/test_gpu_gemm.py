"""The projection GEMM (C = A B^T, bfloat16 inputs, float32 accumulate) on the
GPU against float64 numpy matmul of the same bfloat16 values (the oracle's
definition of the layer's projections)."""
import numpy as np
import pytest
import torch

from gated_delta_rule_02_amd import kda as K
from gated_delta_rule_02_amd import synth
from tests.gpu_util import announce, dev, host64, relerr

pytestmark = pytest.mark.gpu


def run(M, N, Kd, out_dtype=torch.float32, lda=None, ldb=None, ldc=None, seed=0):
    rng = np.random.default_rng(seed)
    lda, ldb, ldc = lda or Kd, ldb or Kd, ldc or N
    A = synth.normal(rng, (M, lda))
    B = synth.normal(rng, (N, ldb), std=0.05)
    Ad, Bd = dev(A), dev(B)
    C = torch.full((M, ldc), float("nan"), dtype=out_dtype, device="cuda")
    K.kda_gemm(Ad[:, :Kd], Bd[:, :Kd], C[:, :N])
    torch.cuda.synchronize()
    ref = A.vals[:, :Kd].astype(np.float64) @ B.vals[:, :Kd].astype(np.float64).T
    return C, ref


@pytest.mark.parametrize("M,N,Kd", [(300, 520, 512), (64, 64, 4096), (256, 256, 64), (1, 700, 128), (513, 255, 192),
                                     (300, 356, 512), (129, 384, 256)])
def test_gemm_main_path_ragged(M, N, Kd):
    """K a multiple of 64 (256 x 256 tiles): ragged M and N, single rows, a single K step; N mod 256 of
    100 and 128 take the tail tiles of 128 columns (4 column tiles per wavefront)."""
    announce("gemm M=%d N=%d K=%d" % (M, N, Kd))
    C, ref = run(M, N, Kd, ldc=(N + 3) // 4 * 4, seed=M + N)
    e = relerr(host64(C[:, :N]), ref)
    print("  err %.2e" % e, flush=True)
    assert e < 2e-5


@pytest.mark.parametrize("M,N,Kd", [(257, 129, 96), (33, 70, 8)])
def test_gemm_fallback_path(M, N, Kd):
    """K not a multiple of 64: the 128 x 128 fallback kernel."""
    announce("gemm fallback M=%d N=%d K=%d" % (M, N, Kd))
    C, ref = run(M, N, Kd, ldc=(N + 3) // 4 * 4, seed=7)
    assert relerr(host64(C[:, :N]), ref) < 2e-5


@pytest.mark.parametrize("M,N,Kd,out", [(77, 256 + 37, 1024, torch.float32), (1000, 64, 256, torch.bfloat16),
                                         (33, 512 + 64, 768, torch.float32), (300, 520, 512, torch.bfloat16)])
def test_gemm_narrow_tail(M, N, Kd, out):
    """Up to 64 columns past the 256-column tiles with K a multiple of 256: the
    narrow kernel (32-row workgroups, K split over four wavefronts, partial tiles
    summed in LDS); ragged M, N mod 256 from 8 to 64, a padded row stride of C."""
    announce("gemm narrow tail M=%d N=%d K=%d %s" % (M, N, Kd, out))
    ldc = (N + 7) // 8 * 8 + 8
    C, ref = run(M, N, Kd, out_dtype=out, ldc=ldc, seed=M + Kd)
    e = relerr(host64(C[:, :N]), ref)
    print("  err %.2e" % e, flush=True)
    assert e < (2e-5 if out == torch.float32 else 5e-3)
    assert torch.isnan(C[:, N:].float()).all()


def test_gemm_tail_tiles_bf16_output():
    """The 128-column tail tiles (N mod 256 = 100) with a bfloat16 output."""
    announce("gemm tail tiles bf16 out")
    C, ref = run(300, 356, 512, out_dtype=torch.bfloat16, ldc=360, seed=5)
    assert relerr(host64(C[:, :356]), ref) < 5e-3
    assert torch.isnan(C[:, 356:].float()).all()


def test_gemm_strides_and_bf16_output():
    """Row strides larger than the logical sizes; bfloat16 output (one rounding,
    2^-9 relative); the padding columns of C stay untouched."""
    announce("gemm strides + bf16 out")
    C, ref = run(300, 260, 320, out_dtype=torch.bfloat16, lda=384, ldb=448, ldc=272, seed=3)
    assert relerr(host64(C[:, :260]), ref) < 5e-3
    assert torch.isnan(C[:, 260:].float()).all()


def test_gemm_layer_projection_full_size():
    """The layer's input projection at full size, M = 8192 tokens, K = 4096,
    N = 5 x 8192 + 64 outputs, bfloat16 out as the layer stores it; every
    output against numpy in float64 (bfloat16 output: one rounding, 2^-9)."""
    announce("gemm full size 8192 x 41024 x 4096")
    rng = np.random.default_rng(11)
    M, N, Kd = 8192, 5 * 8192 + 64, 4096
    A = synth.normal(rng, (M, Kd))
    B = synth.normal(rng, (N, Kd), std=0.02)
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    K.kda_gemm(dev(A), dev(B), C)
    torch.cuda.synchronize()
    Bt = B.vals.astype(np.float64).T
    den = 0.0
    diff = 0.0
    for r0 in range(0, M, 2048):
        ref = A.vals[r0:r0 + 2048].astype(np.float64) @ Bt
        diff = max(diff, float(np.max(np.abs(host64(C[r0:r0 + 2048]) - ref))))
        den = max(den, float(np.max(np.abs(ref))))
    e = diff / den
    print("  err %.2e" % e, flush=True)
    assert e < 5e-3
