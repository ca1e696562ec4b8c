"""The column conversions' bounded waits on the GPU.

Every wait of a column kernel for another wave's progress counter is bounded.  With
the wait limit forced to one poll from the host, waves give up (a give-up only ends a
wave early: every wave still leaves the kernel normally), part of the output stays
unwritten, and the device's wait status reports it: mxfp4_validate_offsets fails with
MXFP4_ERR_HIP while the status is set, mxfp4_wait_status raises once and clears it.
With the default limit back, the same calls match the oracle byte for byte again and
leave the status clear.
"""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import block_scaled_precision_bf16tofp4row_amd as mx  # noqa: E402
import workloads  # noqa: E402
from gpu_path import (canary, check_chain, check_fp8q_both, check_fp8q_cols, dev,  # noqa: E402
                      gpu_cols, gpu_fp8q_cols, gpu_quantize, host)

# several strips per workgroup in every column tile, an empty-ish expert, ragged tails
COUNTS = [1500, 3, 2200, 700]
K = 2048


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _default_limit_and_clear_status():
    lib = mx.load_library()
    lib.mxfp4_set_wait_limit(0)
    torch.cuda.synchronize()
    lib.mxfp4_wait_status(None)
    yield
    lib.mxfp4_set_wait_limit(0)
    torch.cuda.synchronize()
    lib.mxfp4_wait_status(None)


def _segment(seed):
    return workloads.ragged_case(COUNTS, K, seed=seed, values="t3", M_cap=sum(COUNTS) + 7)


def _expect_give_up_reported(offs_d, M_cap):
    with pytest.raises(mx.Mxfp4Error) as e:
        mx.mxfp4_validate_offsets(offs_d, M_cap=M_cap)      # reports without clearing
    assert e.value.status == mx.MXFP4_ERR_HIP
    with pytest.raises(mx.Mxfp4Error) as e:
        mx.mxfp4_wait_status()                              # reports and clears
    assert e.value.status == mx.MXFP4_ERR_HIP
    mx.mxfp4_wait_status()
    assert mx.mxfp4_validate_offsets(offs_d, M_cap=M_cap)


def test_status_clear_after_normal_calls():
    seg = _segment(1)
    check_chain(seg.x_bits, seg.offs, kernels=("quantize", "cols"))
    mx.mxfp4_wait_status()
    assert mx.mxfp4_validate_offsets(dev(seg.offs), M_cap=seg.M_cap)


def test_mxfp4_cols_give_up_is_reported_then_exact_again():
    seg = _segment(2)
    offs_d = dev(seg.offs)
    codes, scales = gpu_quantize(seg.x_bits, seg.offs, offs_d=offs_d)
    exact_T, _ = gpu_cols(codes, scales, offs_d, seg.M_cap, K, seg.G)
    mx.mxfp4_wait_status()
    say(f"MXFP4 -> FP8 columns with a one-poll wait limit: counts={COUNTS} K={K}")
    mx.mxfp4_set_wait_limit(1)
    cut_T, _ = gpu_cols(codes, scales, offs_d, seg.M_cap, K, seg.G)
    mx.mxfp4_set_wait_limit(0)
    torch.cuda.synchronize()
    assert not np.array_equal(host(cut_T), host(exact_T)), "no wave gave up"
    _expect_give_up_reported(offs_d, seg.M_cap)
    say("default limit again")
    check_chain(seg.x_bits, seg.offs, kernels=("quantize", "cols"))
    mx.mxfp4_wait_status()


def test_fp8_cols_give_up_is_reported_then_exact_again():
    seg = _segment(3)
    offs_d = dev(seg.offs)
    x_d = dev(seg.x_bits)
    exact_T, _ = gpu_fp8q_cols(x_d, offs_d, seg.M_cap, K, seg.G)
    mx.mxfp4_wait_status()
    say(f"BF16 -> FP8 columns with a one-poll wait limit: counts={COUNTS} K={K}")
    mx.mxfp4_set_wait_limit(1)
    cut_T, _ = gpu_fp8q_cols(x_d, offs_d, seg.M_cap, K, seg.G)
    mx.mxfp4_set_wait_limit(0)
    torch.cuda.synchronize()
    assert not np.array_equal(host(cut_T), host(exact_T)), "no wave gave up"
    _expect_give_up_reported(offs_d, seg.M_cap)
    say("default limit again")
    check_fp8q_cols(seg.x_bits, seg.offs)
    mx.mxfp4_wait_status()


def test_fp8_both_layouts_give_up_is_reported_then_exact_again():
    seg = _segment(4)
    offs_d = dev(seg.offs)
    x_d = dev(seg.x_bits)
    G, M_cap = seg.G, seg.M_cap
    say(f"BF16 -> FP8 both layouts with a one-poll wait limit: counts={COUNTS} K={K}")
    y, ys = canary((M_cap, K)), canary((M_cap, K // 128))
    yT = canary((M_cap * K,))
    ysT = canary((mx.mxfp4_cols_scale_capacity(M_cap, K, G),))
    mx.mxfp4_set_wait_limit(1)
    mx.mxfp4_bf16_to_fp8_rows_cols_ragged(x_d, y, ys, yT, ysT, offs_d, G=G, M_cap=M_cap, K=K)
    mx.mxfp4_set_wait_limit(0)
    torch.cuda.synchronize()
    _expect_give_up_reported(offs_d, M_cap)
    say("default limit again")
    check_fp8q_both(seg.x_bits, seg.offs)
    mx.mxfp4_wait_status()
