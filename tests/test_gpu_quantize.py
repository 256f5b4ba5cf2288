"""GPU parity of mok_mxfp8_quantize against the oracle quantizer: codes
and scales bit-exact, for bf16 and fp32 sources, along rows (axis 1) and
down columns (axis 0), including every finite bf16 bit pattern, all-zero
blocks, blocks that saturate, subnormal magnitudes, and strided sources."""
import numpy as np
import pytest

from mokutil import ROOT  # noqa: F401

from oracle import mxfp8
from workloads import CONFIGS, bf16_bits_to_f32, make_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import mixture_experts_layer_build_amd as mok  # noqa: E402


def bf16_dev(bits: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def check(src_vals: np.ndarray, dev_src, axis: int):
    codes, scales = mok.mxfp8_quantize(dev_src, axis=axis)
    rc, rs = mxfp8.quantize(src_vals, axis=1 if axis == 1 else 0)
    np.testing.assert_array_equal(codes.cpu().numpy(), rc)
    np.testing.assert_array_equal(scales.cpu().numpy(), rs)


def all_finite_bf16_patterns():
    """The 65280 finite bf16 bit patterns, shuffled (seeded)."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    bits = bits[np.isfinite(bf16_bits_to_f32(bits))]
    assert bits.size == 65280
    np.random.default_rng(0).shuffle(bits)
    return bits


@pytest.mark.parametrize("axis", [1, 0])
def test_quantize_every_bf16_pattern(axis):
    # 65280 = 255 x 256 (blocks along rows) = 32 x 2040 (one block down each column)
    bits = all_finite_bf16_patterns().reshape((255, 256) if axis == 1 else (32, 2040))
    check(bf16_bits_to_f32(bits).astype(np.float64), bf16_dev(bits), axis)


@pytest.mark.parametrize("axis", [1, 0])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("shape", [(64, 256), (96, 2048), (32, 32), (1024, 96)])
def test_quantize_random(axis, dtype, shape):
    rng = np.random.default_rng([axis, len(dtype), *shape])
    v = (rng.standard_normal(shape) * np.exp2(rng.integers(-30, 30, size=shape))).astype(np.float32)
    # special blocks: zeros, exact 448*2^s, saturating, subnormal-scale
    v[0, :32] = 0.0
    v[-1, -32:] = np.float32(448.0 * 2.0 ** -3)
    v[-1, -1] = np.float32(470.0 * 2.0 ** -3)
    if shape[0] > 2:
        v[1, :32] = np.float32(1e-40) * np.arange(32, dtype=np.float32)
    if dtype == "bf16":
        from workloads import f32_to_bf16_bits
        bits = f32_to_bf16_bits(v)
        check(bf16_bits_to_f32(bits).astype(np.float64), bf16_dev(bits), axis)
    else:
        check(v.astype(np.float64), torch.from_numpy(v).cuda(), axis)


def test_quantize_weights_of_8192_token_workload():
    c = CONFIGS["t8192_mxfp8_fwd"].with_(E=4)
    inp = make_inputs(c, T=64)
    for name, axis in (("w_gate", 1), ("w_down", 1), ("w_down", 0)):
        bits = inp[name]
        E, R, K = bits.shape
        flat = bits.reshape(E * R, K)
        check(bf16_bits_to_f32(flat).astype(np.float64), bf16_dev(flat), axis)


def test_quantize_strided_source_and_destination():
    rng = np.random.default_rng(9)
    v = rng.standard_normal((64, 160)).astype(np.float32)
    from workloads import f32_to_bf16_bits
    bits = f32_to_bf16_bits(v)
    dev = bf16_dev(bits)
    sub = dev[:, :128]  # row stride 160 elements
    out = torch.full((64, 136), 0xAB, dtype=torch.uint8, device="cuda")
    sc = torch.empty((64, 4), dtype=torch.uint8, device="cuda")
    lib = mok.lib()
    import ctypes as C
    st = lib.mok_mxfp8_quantize(C.c_void_p(sub.data_ptr()), 0, 64, 128, 160, 1, C.c_void_p(out.data_ptr()), 136,
                                C.c_void_p(sc.data_ptr()), C.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    rc, rs = mxfp8.quantize(bf16_bits_to_f32(bits[:, :128]).astype(np.float64), axis=1)
    o = out.cpu().numpy()
    np.testing.assert_array_equal(o[:, :128], rc)
    assert np.all(o[:, 128:] == 0xAB)  # padding columns untouched
    np.testing.assert_array_equal(sc.cpu().numpy(), rs)


def test_quantize_every_block_exponent():
    # one 32-element fp32 block per block exponent X = -127 .. 127 (several
    # blocks each): magnitudes up to 2^(X+8) .. 448 * 2^X with E4M3 rounding
    # ties and values in the saturation band, down to fp32 subnormals
    rng = np.random.default_rng(11)
    blocks = []
    grid = np.array([(m / 8.0) * 2.0 ** (-6) if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
                     for e in range(16) for m in range(8)][:127])  # E4M3 magnitudes up to 448
    for X in range(-127, 128):
        for rep in range(4):
            b = np.empty(32)
            kind = rep % 4
            if kind == 0:      # random magnitudes below the block maximum
                b[:] = rng.uniform(0, 1, 32) * 2.0 ** (X + 8) * rng.choice([-1, 1], 32)
            elif kind == 1:    # rounding ties between neighbouring E4M3 values
                i = rng.integers(0, 126, 32)
                b[:] = 0.5 * (grid[i] + grid[i + 1]) * 2.0 ** X * rng.choice([-1, 1], 32)
            elif kind == 2:    # saturation band 448 .. 480 (times 2^X)
                b[:] = rng.uniform(440, 480, 32) * 2.0 ** X * rng.choice([-1, 1], 32)
            else:              # exact grid values
                b[:] = grid[rng.integers(0, 127, 32)] * 2.0 ** X * rng.choice([-1, 1], 32)
            b[0] = 2.0 ** (X + 8) * 1.5  # pins the block maximum's binade at X + 8
            blocks.append(b)
    v = np.stack(blocks).astype(np.float32)  # fp32 rounding of each value
    v[~np.isfinite(v)] = 0.0
    v = v.reshape(-1, 64)  # two blocks per row
    check(v.astype(np.float64), torch.from_numpy(np.ascontiguousarray(v)).cuda(), 1)
