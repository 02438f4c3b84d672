"""The packed bf16 weight layout written by moe_prepack_weights, checked
element by element against the layout the header documents."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def packed_reference(w: np.ndarray) -> np.ndarray:
    """Block (r/16, c/32) at block index (r/16)*(C/32) + c/32; inside a block
    lane L = r%16 + 16*((c%32)//8) holds elements c%8 = 0..7."""
    R, C = w.shape
    out = np.empty(R * C, dtype=w.dtype)
    for r in range(R):
        for c in range(C):
            blk = (r // 16) * (C // 32) + c // 32
            lane = r % 16 + 16 * ((c % 32) // 8)
            out[blk * 512 + lane * 8 + c % 8] = w[r, c]
    return out


@pytest.mark.parametrize("R,C", [(16, 32), (48, 96), (128, 256)])
def test_prepack_layout(R, C):
    import torch
    import expert_moe_fp32_amd as m
    from expert_moe_fp32_amd import _lib as L
    rng = np.random.default_rng(R + C)
    w = rng.integers(0, 2**16, size=(R, C), dtype=np.uint16)
    src = torch.from_numpy(w.view(np.int16)).cuda()
    dst = torch.zeros_like(src)
    m.moe_prepack_weights(src, R, C, L.MOE_BF16, dst)
    torch.cuda.synchronize()
    got = dst.cpu().numpy().view(np.uint16).ravel()
    assert np.array_equal(got, packed_reference(w))
