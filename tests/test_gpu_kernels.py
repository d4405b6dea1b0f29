"""GEMM kernel parity through the C-ABI test entry point (fp16 MFMA and fp32 VALU paths)."""
import numpy as np
import pytest

from tests.gpu_harness import log, require_gpu


# (M, N, K): ragged M; every skinny configuration (M <= 256: 16/32/64/128/256-row workgroups, 2 or 4
# column groups per wave) and every tile configuration of the LDS-tiled kernel (128x128, 64x64,
# 64x32, 32x32)
SHAPES_F16 = [(1, 64, 64), (7, 96, 128), (20, 160, 192), (65, 192, 768), (128, 14336, 256), (200, 512, 320),
              (256, 768, 3840), (64, 50304, 768), (300, 5376, 768), (700, 256, 128), (2050, 768, 3840),
              (4096, 2304, 768)]
# the 256 x 256 large-tile kernel serves [q|k|v|up] and [out|down] only (fused epilogues): its shapes
# are covered by the full-size parity tests of the 1.2B config and the prefill-heavy [out|down]


def to_operand_order(x):
    """[R, K] -> the library's fp16 operand order: rows padded to 16, then 16 x 32 tiles (g, s)
    g-major, and inside a tile the 8-element runs (r, q) at position 16 q + r."""
    R, K = x.shape
    Rp = (R + 15) // 16 * 16
    xp = np.zeros((Rp, K), dtype=x.dtype)
    xp[:R] = x
    t = xp.reshape(Rp // 16, 16, K // 32, 4, 8)         # [g, r, s, q, e]
    return np.ascontiguousarray(t.transpose(0, 2, 3, 1, 4)).reshape(-1)   # [g, s, q, r, e]


def test_operand_order_matches_mfma_lane_layout():
    """Element (row, k) of tile (g, s) lands where lane 16 q + r, element e of a 16x32 MFMA operand
    lives: row = 16 g + r, k = 32 s + 8 q + e."""
    x = np.arange(32 * 64, dtype=np.int64).reshape(32, 64)
    f = to_operand_order(x)
    for g in range(2):
        for s in range(2):
            tile = f[(g * 2 + s) * 512:(g * 2 + s + 1) * 512].reshape(64, 8)
            for lane in range(64):
                r, q = lane % 16, lane // 16
                assert list(tile[lane]) == [x[16 * g + r, 32 * s + 8 * q + e] for e in range(8)]
SHAPES_F32 = [(1, 1, 1), (5, 70, 33), (64, 448, 64), (130, 64, 320)]


@pytest.mark.gpu
@pytest.mark.parametrize("M,N,K", SHAPES_F16)
def test_gemm_f16_mfma(M, N, K):
    torch = require_gpu()
    import hierarchical_global_local_amd as hg
    log(f"gemm f16 M={M} N={N} K={K}")
    rng = np.random.default_rng([M, N, K])
    a = rng.standard_normal((M, K)).astype(np.float16)
    w = rng.standard_normal((N, K)).astype(np.float16)
    c = hg.gemm(torch.from_numpy(to_operand_order(a)).cuda(), torch.from_numpy(to_operand_order(w)).cuda(),
                M, N, K, scale=0.5).cpu().numpy()
    ref = 0.5 * (a.astype(np.float64) @ w.astype(np.float64).T)
    err = np.abs(c - ref).max()
    assert err <= 2e-6 * K * np.sqrt(K) + 1e-5, err


@pytest.mark.gpu
@pytest.mark.parametrize("M,N,K", SHAPES_F32)
def test_gemm_f32_valu(M, N, K):
    torch = require_gpu()
    import hierarchical_global_local_amd as hg
    log(f"gemm f32 M={M} N={N} K={K}")
    rng = np.random.default_rng([M, N, K, 1])
    a = rng.standard_normal((M, K)).astype(np.float32)
    w = rng.standard_normal((N, K)).astype(np.float32)
    c = hg.gemm(torch.from_numpy(a).cuda(), torch.from_numpy(w).cuda(), M, N, K).cpu().numpy()
    ref = a.astype(np.float64) @ w.astype(np.float64).T
    assert np.abs(c - ref).max() <= 1e-6 * K * np.sqrt(K) + 1e-6
