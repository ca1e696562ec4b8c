"""The hot path under HIP graph capture: the forward chain (quantize, row conversion,
column conversion), the backward quantizer in both layouts and the NVFP4 quantizer,
captured once into a graph (torch.cuda.CUDAGraph) and replayed several times, with the
program's own eager work in between (the outputs are overwritten with a canary before
each replay).  Every replay must give the bytes the same calls give eagerly.  No call of
the path records a memset: the NVFP4 amax reset is a kernel of its own."""
from __future__ import annotations

import os
import sys

import pytest

pytestmark = pytest.mark.gpu

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import block_scaled_precision_bf16tofp4row_amd as mx  # noqa: E402
import workloads  # noqa: E402
from gpu_path import CANARY, dev  # noqa: E402


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _lib():
    mx.load_library()


def test_captured_path_replays_bit_exact():
    counts = [700, 0, 1300, 45, 257]
    K = 2048
    say(f"graph capture counts={counts} K={K}")
    seg = workloads.ragged_case(counts, K, seed=31, values="t3", M_cap=sum(counts) + 9)
    M_cap, G = seg.M_cap, seg.G
    x = dev(seg.x_bits)
    offs = dev(seg.offs)
    codes, scales = mx.alloc_quantize_outputs(M_cap, K)
    y, ys = mx.alloc_rows_outputs(M_cap, K)
    yT, ysT = mx.alloc_cols_outputs(M_cap, K, G)
    qy, qys = mx.alloc_fp8q_rows_outputs(M_cap, K)
    qyT, qysT = mx.alloc_cols_outputs(M_cap, K, G)
    nc, ns, na = mx.alloc_nvfp4_outputs(M_cap, K)
    outs = [codes, scales, y, ys, yT, ysT, qy, qys, qyT, qysT, nc, ns, na]

    def path():
        mx.mxfp4_quantize_rows(x, codes, scales, offs)
        mx.mxfp4_to_fp8_rows(codes, scales, y, ys, offs)
        mx.mxfp4_to_fp8_cols_ragged(codes, scales, yT, ysT, offs)
        mx.mxfp4_bf16_to_fp8_rows_cols_ragged(x, qy, qys, qyT, qysT, offs)
        mx.mxfp4_nvfp4_quantize_rows(x, nc, ns, na, offs)

    def fill():
        for t in outs:
            t.view(torch.uint8).fill_(CANARY)

    fill()
    path()
    torch.cuda.synchronize()
    eager = [t.clone() for t in outs]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm-up on a side stream, as capture requires
        path()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    fill()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        path()
    torch.cuda.synchronize()
    for rep in range(3):
        fill()                             # eager work between the replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(eager, outs)):
            assert torch.equal(a, b), f"replay {rep}: output {i} differs from the eager call"
    mx.mxfp4_wait_status()
