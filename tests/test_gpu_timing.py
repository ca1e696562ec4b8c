"""The measurement hook mxfp4_time_next_launch on the GPU: HIP events armed for the next
call are bound to its kernels (the first and the last of the call), so they time the
kernels' own execution; the call's output is byte-identical to an unarmed call; the
events are used once (a second call leaves them as the first one recorded them).  Also
the benchmark's memory-only column traffic kernel stays inside the buffers it is given."""
from __future__ import annotations

import ctypes
import os
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import block_scaled_precision_bf16tofp4row_amd as mx  # noqa: E402
import workloads  # noqa: E402
from gpu_path import dev  # noqa: E402


class Hip:
    """hipEventCreate / hipEventElapsedTime / hipEventDestroy of the HIP runtime."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        P = ctypes.c_void_p
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(P)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), P, P]
        self.lib.hipEventSynchronize.argtypes = [P]
        self.lib.hipEventDestroy.argtypes = [P]

    def event(self):
        e = ctypes.c_void_p()
        assert self.lib.hipEventCreate(ctypes.byref(e)) == 0
        return e.value

    def elapsed_us(self, a, b):
        assert self.lib.hipEventSynchronize(b) == 0
        ms = ctypes.c_float()
        assert self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return 1000.0 * ms.value

    def destroy(self, *evs):
        for e in evs:
            self.lib.hipEventDestroy(e)


@pytest.fixture(scope="module")
def hip():
    mx.load_library()
    return Hip()


def _segment():
    return workloads.ragged_case([700, 0, 1300, 45], 2048, seed=5, values="t3", M_cap=2100)


def test_armed_call_times_its_kernel_and_keeps_its_output(hip):
    seg = _segment()
    x, offs = dev(seg.x_bits), dev(seg.offs)
    # rows past offs[G] are never written: both outputs start from the same canary
    c0, s0 = [t.fill_(0xA5) for t in mx.alloc_quantize_outputs(seg.M_cap, seg.K)]
    c1, s1 = [t.fill_(0xA5) for t in mx.alloc_quantize_outputs(seg.M_cap, seg.K)]
    a, b = hip.event(), hip.event()
    mx.mxfp4_quantize_rows(x, c0, s0, offs)
    mx.mxfp4_time_next_launch(a, b)
    mx.mxfp4_quantize_rows(x, c1, s1, offs)
    us = hip.elapsed_us(a, b)
    torch.cuda.synchronize()
    assert 0.0 < us < 1e6
    assert torch.equal(c0, c1) and torch.equal(s0, s1)
    # used once: an unarmed call afterwards records nothing into them
    mx.mxfp4_quantize_rows(x, c1, s1, offs)
    torch.cuda.synchronize()
    assert hip.elapsed_us(a, b) == us
    hip.destroy(a, b)


def test_column_conversion_timed_like_the_chain(hip):
    seg = _segment()
    x, offs = dev(seg.x_bits), dev(seg.offs)
    c, s = mx.alloc_quantize_outputs(seg.M_cap, seg.K)
    mx.mxfp4_quantize_rows(x, c, s, offs)
    yT0, ysT0 = [t.fill_(0xA5) for t in mx.alloc_cols_outputs(seg.M_cap, seg.K, seg.G)]
    yT1, ysT1 = [t.fill_(0xA5) for t in mx.alloc_cols_outputs(seg.M_cap, seg.K, seg.G)]
    mx.mxfp4_to_fp8_cols_ragged(c, s, yT0, ysT0, offs)
    a, b = hip.event(), hip.event()
    mx.mxfp4_time_next_launch(a, b)
    mx.mxfp4_to_fp8_cols_ragged(c, s, yT1, ysT1, offs)
    assert 0.0 < hip.elapsed_us(a, b) < 1e6
    torch.cuda.synchronize()
    assert torch.equal(yT0, yT1) and torch.equal(ysT0, ysT1)
    mx.mxfp4_wait_status()
    hip.destroy(a, b)


def test_three_kernel_call_is_timed_first_to_last(hip):
    """The NVFP4 quantizer launches three kernels (amax reset, tensor amax, quantize):
    the start event goes with the first, the stop event with the last."""
    seg = _segment()
    x, offs = dev(seg.x_bits), dev(seg.offs)
    nc, ns, na = mx.alloc_nvfp4_outputs(seg.M_cap, seg.K)
    a, b, c_, d_ = hip.event(), hip.event(), hip.event(), hip.event()
    mx.mxfp4_nvfp4_quantize_rows(x, nc, ns, na, offs)
    mx.mxfp4_time_next_launch(a, b)
    mx.mxfp4_nvfp4_quantize_rows(x, nc, ns, na, offs)
    whole = hip.elapsed_us(a, b)
    # the quantizer alone (start and stop both on a one-kernel call of similar size)
    c0, s0 = mx.alloc_quantize_outputs(seg.M_cap, seg.K)
    mx.mxfp4_time_next_launch(c_, d_)
    mx.mxfp4_quantize_rows(x, c0, s0, offs)
    one = hip.elapsed_us(c_, d_)
    assert 0.0 < one < 1e6 and 0.0 < whole < 1e6
    assert whole > one
    hip.destroy(a, b, c_, d_)


@pytest.mark.parametrize("sequential", [False, True])
@pytest.mark.parametrize("kind", ["codes", "bf16"])
def test_cols_traffic_ceiling_stays_in_its_buffers(kind, sequential):
    """The benchmark's memory-only column traffic (libmxfp4bench bench_cols_traffic)
    writes nothing outside the output and block-scale ranges it is given, and leaves its
    inputs unchanged: canaries on both sides of every buffer, on a ragged case with a
    narrow last tile and a partial last strip."""
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import bench
    traffic = bench.ColsTraffic()
    K = 640
    counts = [0, 300, 129, 5]
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    M = int(offs[-1])
    strips = torch.from_numpy(bench.strip_table(offs, K)).cuda()
    n = strips.shape[0]
    pad = 4096
    if kind == "codes":
        inp = torch.randint(0, 255, (M, K // 2), dtype=torch.uint8, device="cuda")
        sc = torch.randint(0, 255, (M, K // 32), dtype=torch.uint8, device="cuda")
        tib = 128
    else:
        inp = torch.randint(-2000, 2000, (M, K), dtype=torch.int16, device="cuda")
        sc = None
        tib = 512
    inp0 = inp.clone()
    sc0 = sc.clone() if sc is not None else None
    out_bytes = (((K + 255) // 256) * n * 256 * 128) if sequential else M * K
    big = torch.full((out_bytes + 2 * pad,), 0xA5, dtype=torch.uint8, device="cuda")
    out = big[pad:pad + out_bytes]
    sbig = torch.full((n * K + 2 * pad,), 0x5A, dtype=torch.uint8, device="cuda")
    out_scales = sbig[pad:pad + n * K]
    traffic(torch, inp, tib, sc, out, out_scales, strips, K, sequential)
    torch.cuda.synchronize()
    assert bool((big[:pad] == 0xA5).all()) and bool((big[pad + out_bytes:] == 0xA5).all())
    assert bool((sbig[:pad] == 0x5A).all()) and bool((sbig[pad + n * K:] == 0x5A).all())
    assert torch.equal(inp, inp0) and (sc is None or torch.equal(sc, sc0))
