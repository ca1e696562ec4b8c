"""The newer entry points on a side stream and twice in a row: the expert GEMM, the
weight-gradient GEMM, the NVFP4 quantizer and the both-layouts backward quantizer give
the same bytes on torch's default stream and on a second stream.  The GEMMs use no
atomics and the NVFP4 amax is an atomic max, whose result does not depend on order, so
runs are bit-identical."""
from __future__ import annotations

import os
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

import torch  # noqa: E402

import block_scaled_precision_bf16tofp4row_amd as mx  # noqa: E402
import workloads  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _lib():
    mx.load_library()


def _on(stream, fn):
    """fn() on `stream` (None: the default stream), the result copied to the host."""
    if stream is None:
        out = fn()
        torch.cuda.synchronize()
        return [t.cpu() for t in out]
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        out = fn()
    stream.synchronize()
    return [t.cpu() for t in out]


def _same_everywhere(fn):
    side = torch.cuda.Stream()
    ref = _on(None, fn)
    for got in (_on(None, fn), _on(side, fn), _on(side, fn)):
        for a, b in zip(ref, got):
            assert torch.equal(a, b)


def _case(counts, K, seed):
    seg = workloads.ragged_case(counts, K, seed=seed, M_cap=sum(counts) + 7)
    x = torch.from_numpy(seg.x_bits.view(np.int16)).cuda()
    offs = torch.from_numpy(seg.offs).cuda()
    return seg, x, offs


def test_forward_gemm_streams():
    seg, x, offs = _case([0, 300, 45, 129], 512, 31)
    G, N = seg.G, 256
    c, s = mx.alloc_quantize_outputs(seg.M_cap, seg.K)
    y, ys = mx.alloc_rows_outputs(seg.M_cap, seg.K)
    mx.mxfp4_quantize_rows(x, c, s, offs)
    mx.mxfp4_to_fp8_rows(c, s, y, ys, offs)
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    w = torch.randint(0, 126, (G, N, seg.K), device="cuda", dtype=torch.int32, generator=g).to(torch.uint8)
    ws = torch.randint(120, 134, (G, N, seg.K // 128), device="cuda", dtype=torch.int32, generator=g).to(torch.uint8)

    def run():
        out = torch.zeros((seg.M_cap, N), dtype=torch.int16, device="cuda")
        mx.mxfp4_fp8_grouped_gemm(y, ys, w, ws, out, offs)
        return [out]

    _same_everywhere(run)


def test_wgrad_gemm_streams():
    seg, x, offs = _case([0, 300, 45, 129], 256, 32)
    G, N, K = seg.G, 256, seg.K
    c, s = mx.alloc_quantize_outputs(seg.M_cap, K)
    xT, xsT = mx.alloc_cols_outputs(seg.M_cap, K, G)
    mx.mxfp4_quantize_rows(x, c, s, offs)
    mx.mxfp4_to_fp8_cols_ragged(c, s, xT, xsT, offs)
    grad = workloads.ragged_case([0, 300, 45, 129], N, seed=33, M_cap=seg.M_cap)
    gx = torch.from_numpy(grad.x_bits.view(np.int16)).cuda()
    dT, dsT = mx.alloc_cols_outputs(seg.M_cap, N, G)
    mx.mxfp4_bf16_to_fp8_cols_ragged(gx, dT, dsT, offs)

    def run():
        dw = torch.zeros((G * N * K,), dtype=torch.int16, device="cuda")
        mx.mxfp4_fp8_grouped_gemm_wgrad(dT, dsT, xT, xsT, dw, offs, N=N, K=K, G=G, M_cap=seg.M_cap)
        return [dw]

    _same_everywhere(run)


def test_nvfp4_streams():
    seg, x, offs = _case([0, 300, 45, 129], 7168, 34)

    def run():
        nc, ns, na = mx.alloc_nvfp4_outputs(seg.M_cap, seg.K)
        nc.zero_()
        ns.zero_()
        mx.mxfp4_nvfp4_quantize_rows(x, nc, ns, na, offs)
        return [nc, ns, na]

    _same_everywhere(run)


def test_both_layouts_streams():
    seg, x, offs = _case([0, 300, 45, 129], 7168, 35)

    def run():
        y, ys = mx.alloc_fp8q_rows_outputs(seg.M_cap, seg.K)
        yT, ysT = mx.alloc_cols_outputs(seg.M_cap, seg.K, seg.G)
        for t in (y, ys, yT, ysT):
            t.zero_()
        mx.mxfp4_bf16_to_fp8_rows_cols_ragged(x, y, ys, yT, ysT, offs)
        return [y, ys, yT, ysT]

    _same_everywhere(run)
