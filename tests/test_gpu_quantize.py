"""mxfp8_quantize on the GPU against the oracle: bit-exact codes and scales."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as S

pytestmark = pytest.mark.gpu


def _mx():
    import mxfp8_grouped_gemm_amd as mx
    return mx


def _all_bf16_groups(seed):
    """Every finite bf16 pattern, shuffled into groups of 32 (rows of 32)."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = (bits & 0x7F80) != 0x7F80
    bits = bits[finite]
    rng = np.random.default_rng(seed)
    bits = bits[rng.permutation(bits.size)]
    bits = bits[: bits.size // 32 * 32]
    return bits.reshape(-1, 32)


@pytest.mark.parametrize("fmt", [0, 1])
def test_quantize_every_bf16_pattern(fmt):
    mx = _mx()
    for seed in range(3):
        g = _all_bf16_groups(seed)
        # also a copy where each group's values are scaled into one binade region
        g2 = (g & np.uint16(0x807F)) | np.uint16(0x3F00)      # magnitudes in [0.5, 1)
        g3 = g & np.uint16(0x80FF)                            # tiny: subnormal / small normals
        for arr in (g, g2, g3):
            x = S.from_bits(arr, "cuda")
            codes, scales = mx.mxfp8_quantize(x, 1, fmt)
            rc, rs = oracle.quantize(arr, 1, fmt)
            assert np.array_equal(codes.cpu().numpy(), rc)
            assert np.array_equal(scales.cpu().numpy(), rs)
            # axis 0 on the transpose
            xt = S.from_bits(np.ascontiguousarray(arr.T), "cuda")
            c0, s0 = mx.mxfp8_quantize(xt, 0, fmt)
            assert np.array_equal(c0.cpu().numpy(), rc.T) and np.array_equal(s0.cpu().numpy(), rs.T)


@pytest.mark.parametrize("shape", [(32, 32), (64, 96), (4096, 4096), (96, 100), (160, 8200), (32, 7)])
@pytest.mark.parametrize("fmt", [0, 1])
def test_quantize_shapes(shape, fmt):
    mx = _mx()
    R, Cc = shape
    x = S.normal_bf16((R, Cc), 1.0, 5, 77, "cuda")
    bits = S.bf16_bits(x)
    if Cc % 32 == 0:
        c, s = mx.mxfp8_quantize(x, 1, fmt)
        rc, rs = oracle.quantize(bits, 1, fmt)
        assert np.array_equal(c.cpu().numpy(), rc) and np.array_equal(s.cpu().numpy(), rs)
    if R % 32 == 0:
        c, s = mx.mxfp8_quantize(x, 0, fmt)
        rc, rs = oracle.quantize(bits, 0, fmt)
        assert np.array_equal(c.cpu().numpy(), rc) and np.array_equal(s.cpu().numpy(), rs)


def test_quantize_rejects_bad_arguments():
    mx = _mx()
    x = torch.zeros((32, 48), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mx.MxError):
        mx.mxfp8_quantize(x, 1, 0)          # 48 % 32 != 0
    with pytest.raises(mx.MxError):
        mx.mxfp8_quantize(x, 1, 7)
