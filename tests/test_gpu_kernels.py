"""GEMM kernel parity through the C-ABI test entry point (fp16 MFMA and fp32 VALU paths)."""
import numpy as np
import pytest

from tests.gpu_harness import log, require_gpu

pytestmark = pytest.mark.gpu

# (M, N, K): ragged M, every tile configuration the launcher picks (128x128, 64x64, 64x32, 32x32)
SHAPES_F16 = [(1, 64, 64), (7, 96, 128), (65, 192, 768), (300, 5376, 768), (64, 50304, 768),
              (256, 768, 3840), (2050, 768, 3840), (4096, 2304, 768)]
SHAPES_F32 = [(1, 1, 1), (5, 70, 33), (64, 448, 64), (130, 64, 320)]


@pytest.mark.parametrize("M,N,K", SHAPES_F16)
def test_gemm_f16_mfma(M, N, K):
    torch = require_gpu()
    import hierarchical_global_local_amd as hg
    log(f"gemm f16 M={M} N={N} K={K}")
    rng = np.random.default_rng([M, N, K])
    a = rng.standard_normal((M, K)).astype(np.float16)
    w = rng.standard_normal((N, K)).astype(np.float16)
    c = hg.gemm(torch.from_numpy(a).cuda(), torch.from_numpy(w).cuda(), scale=0.5).cpu().numpy()
    ref = 0.5 * (a.astype(np.float64) @ w.astype(np.float64).T)
    err = np.abs(c - ref).max()
    assert err <= 2e-6 * K * np.sqrt(K) + 1e-5, err


@pytest.mark.parametrize("M,N,K", SHAPES_F32)
def test_gemm_f32_valu(M, N, K):
    torch = require_gpu()
    import hierarchical_global_local_amd as hg
    log(f"gemm f32 M={M} N={N} K={K}")
    rng = np.random.default_rng([M, N, K, 1])
    a = rng.standard_normal((M, K)).astype(np.float32)
    w = rng.standard_normal((N, K)).astype(np.float32)
    c = hg.gemm(torch.from_numpy(a).cuda(), torch.from_numpy(w).cuda()).cpu().numpy()
    ref = a.astype(np.float64) @ w.astype(np.float64).T
    assert np.abs(c - ref).max() <= 1e-6 * K * np.sqrt(K) + 1e-6
