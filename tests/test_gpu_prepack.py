"""The prepared weight forms written by moe_prepack_weights, checked element
by element against the layouts the header documents, from either storage
order of the logical matrix (layout KN = [K][N], NK = [N][K])."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

KN, NK = 0, 1


def packed_reference(w: np.ndarray) -> np.ndarray:
    """w: logical [K][N].  Block (n/16, k/32) at block index
    (n/16)*(K/32) + k/32; inside a block lane L = n%16 + 16*((k%32)//8)
    holds elements k%8 = 0..7."""
    K, N = w.shape
    out = np.empty(K * N, dtype=w.dtype)
    for n in range(N):
        for k in range(K):
            blk = (n // 16) * (K // 32) + k // 32
            lane = n % 16 + 16 * ((k % 32) // 8)
            out[blk * 512 + lane * 8 + k % 8] = w[k, n]
    return out


@pytest.mark.parametrize("layout", [KN, NK])
@pytest.mark.parametrize("K,N", [(32, 16), (96, 48), (256, 128)])
def test_prepack_bf16_layout(K, N, layout):
    import torch
    import expert_moe_fp32_amd as m
    from expert_moe_fp32_amd import _lib as L
    rng = np.random.default_rng(K + N)
    w = rng.integers(0, 2**16, size=(K, N), dtype=np.uint16)
    src_np = w if layout == KN else np.ascontiguousarray(w.T)
    src = torch.from_numpy(src_np.view(np.int16)).cuda()
    dst = torch.zeros_like(src)
    m.moe_prepack_weights(src, K, N, L.MOE_BF16, layout, dst)
    torch.cuda.synchronize()
    got = dst.cpu().numpy().view(np.uint16).ravel()
    assert np.array_equal(got, packed_reference(w))


@pytest.mark.parametrize("layout", [KN, NK])
def test_prepack_f32_is_the_logical_layout(layout):
    import torch
    import expert_moe_fp32_amd as m
    from expert_moe_fp32_amd import _lib as L
    rng = np.random.default_rng(5)
    K, N = 40, 24
    w = rng.standard_normal((K, N)).astype(np.float32)
    src = torch.from_numpy(w if layout == KN else np.ascontiguousarray(w.T)).cuda()
    dst = torch.zeros_like(src)
    m.moe_prepack_weights(src, K, N, L.MOE_F32, layout, dst)
    torch.cuda.synchronize()
    assert np.array_equal(dst.cpu().numpy().reshape(K, N), w)
