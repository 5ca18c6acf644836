"""GPU parity of the standalone elementwise GELU (include/spgelu.h) against the oracle.

Bound (the accepted reading): |y - g| <= ulp_out(g)/2 + 2^-16 |g| + 2^-120 with g the
exact gelu of the stored input (oracle.metrics.compare_elementwise): rounding of the
output, the fp32 evaluation, and the fp32 exp overflow far on the negative side.  NaN
inputs give NaN, +inf gives +inf.
"""

import numpy as np
import pytest

import oracle
import software_pipelined_tiled_gemm_amd as spg
import workloads as W
from oracle import metrics
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def _run(x_bits, dtype, offset_x=0, offset_y=0, inplace=False):
    """Copy x to the device at an element offset, run gelu_run, return y's bits and the
    guard elements around y (which must stay untouched)."""
    import torch
    tdt = torch.int32 if dtype == "f32" else torch.int16
    n = x_bits.size
    guard = 16 // (4 if dtype == "f32" else 2)   # 16 bytes: offset 0 stays 16-byte aligned
    X = torch.full((n + 2 * guard + offset_x,), 0x1234, dtype=tdt, device=G.torch_dev())
    xs = torch.from_numpy(x_bits.view(np.int32 if dtype == "f32" else np.int16).copy())
    X[guard + offset_x: guard + offset_x + n] = xs.to(G.torch_dev())
    xv = X[guard + offset_x: guard + offset_x + n]
    if inplace:
        Y, yv = X, xv
    else:
        Y = torch.full((n + 2 * guard + offset_y,), 0x4321, dtype=tdt, device=G.torch_dev())
        yv = Y[guard + offset_y: guard + offset_y + n]
    spg.gelu_run(xv.data_ptr(), yv.data_ptr(), n, dtype, torch.cuda.current_stream())
    torch.cuda.synchronize()
    y = yv.cpu().numpy().view(np.uint32 if dtype == "f32" else np.uint16)
    outside = torch.cat([Y[:guard + (offset_x if inplace else offset_y)],
                         Y[guard + (offset_x if inplace else offset_y) + n:]]).cpu().numpy()
    return y, outside


def _values(bits, dtype):
    if dtype == "f32":
        return bits.view(np.float32).astype(np.float64)
    return oracle.decode(bits, dtype)


def _check(x_bits, y_bits, dtype):
    g = oracle.gelu_elementwise(x_bits, dtype)
    res = metrics.compare_elementwise(_values(y_bits, dtype), g, dtype)
    assert res["ok"], res
    return res


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_every_bit_pattern(dtype):
    x = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    y, outside = _run(x, dtype)
    res = _check(x, y, dtype)
    print(f"{dtype}: all 65536 patterns, excess over the bound {res['excess']:.3e}, "
          f"correctly rounded {100 * res['exact_frac']:.3f}%", flush=True)
    assert res["exact_frac"] > 0.99
    assert np.all(outside == 0x4321)


def test_fp32_across_magnitudes():
    r = np.random.Generator(np.random.PCG64(5))
    x = np.concatenate([r.normal(0, 1, 200000), r.normal(0, 30, 200000),
                        r.uniform(-12, 12, 200000), np.exp2(r.uniform(-140, 127, 100000)),
                        -np.exp2(r.uniform(-140, 127, 100000)),
                        [0.0, -0.0, np.inf, -np.inf, np.nan, 3.4e38, -3.4e38]]).astype(np.float32)
    y, _ = _run(x.view(np.uint32), "f32")
    res = _check(x.view(np.uint32), y, "f32")
    print(f"f32: excess {res['excess']:.3e}, correctly rounded {100 * res['exact_frac']:.2f}%",
          flush=True)


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
def test_sizes_alignment_in_place(dtype):
    r = np.random.Generator(np.random.PCG64(6))
    for n in (1, 5, 7, 8, 9, 63, 1023, 1024, 1025, 4 * 1024 + 3, 3 * 8192 + 7):
        xv = r.normal(0, 2, n).astype(np.float32)
        x = xv.view(np.uint32) if dtype == "f32" else W.float32_to_bits(xv, dtype)
        for ox, oy, inplace in ((0, 0, False), (1, 0, False), (0, 3, False), (0, 0, True),
                                (1, 1, True)):
            y, outside = _run(x, dtype, ox, oy, inplace)
            _check(x, y, dtype)
            fill = 0x1234 if inplace else 0x4321
            assert np.all(outside == fill), (n, ox, oy, inplace)


def test_xla_loop_fusion_tensor():
    # the XLA:GPU emitters page's example: bf16 [6,512,4096] through the tanh GELU
    x = W.make_matrix((6 * 512, 4096), "bf16", ("normal", 1.0), W.SEED_A).reshape(-1)
    y, outside = _run(x, "bf16")
    res = _check(x, y, "bf16")
    print(f"bf16 [6,512,4096]: excess {res['excess']:.3e}, correctly rounded "
          f"{100 * res['exact_frac']:.3f}%", flush=True)
    assert np.all(outside == 0x4321)


def test_empty_is_a_no_op():
    spg.gelu_run(None, None, 0, "bf16")
