"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects bad arguments synchronously (before any HIP call)
with the documented status codes."""
import ctypes
import functools
import os
import re

import pytest

import block_scaled_precision_bf16tofp4row_amd as mx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxfp4cvt.h")

# fake, never-dereferenced device addresses (validation fails before any launch)
A = 0x7F0000000000
A2 = A + 0x100000
A3 = A + 0x200000
A4 = A + 0x300000
OFFS = A + 0x400000


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mxfp4_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return mx.load_library()


def test_header_and_binding_agree():
    assert declared_functions() == sorted(mx.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    nm = ctypes.CDLL(mx.LIB_PATH)
    for name in declared_functions():
        getattr(nm, name)


def test_status_strings(lib):
    for code in range(5):
        s = mx.mxfp4_status_string(code)
        assert s.startswith("MXFP4_")
    assert mx.mxfp4_status_string(99) == "unknown status"


def test_cols_scale_capacity():
    assert mx.mxfp4_cols_scale_capacity(32768, 2048, 32) == 2048 * (256 + 32)
    assert mx.mxfp4_cols_scale_capacity(1, 128, 1) == 128 * 2
    assert mx.mxfp4_cols_scale_capacity(0, 128, 3) == 128 * 3
    assert mx.mxfp4_cols_scale_capacity(10, 100, 1) == -1
    assert mx.mxfp4_cols_scale_capacity(10, 128, 0) == -1


def _q(lib, x=A, c=A2, s=A3, o=OFFS, G=1, M=4, K=64):
    return lib.mxfp4_quantize_rows(x, c, s, o, G, M, K, None)


def _r(lib, fn, c=A, s=A2, y=A3, ys=A4, o=OFFS, G=1, M=4, K=128):
    return getattr(lib, fn)(c, s, y, ys, o, G, M, K, None)


def test_quantize_argument_errors(lib):
    assert _q(lib, x=None) == mx.MXFP4_ERR_NULL
    assert _q(lib, c=None) == mx.MXFP4_ERR_NULL
    assert _q(lib, s=None) == mx.MXFP4_ERR_NULL
    assert _q(lib, o=None) == mx.MXFP4_ERR_NULL
    assert _q(lib, K=48) == mx.MXFP4_ERR_SHAPE
    assert _q(lib, K=0) == mx.MXFP4_ERR_SHAPE
    assert _q(lib, K=-32) == mx.MXFP4_ERR_SHAPE
    assert _q(lib, M=-1) == mx.MXFP4_ERR_SHAPE
    assert _q(lib, G=0) == mx.MXFP4_ERR_SHAPE
    assert _q(lib, M=1 << 40, K=1 << 20) == mx.MXFP4_ERR_SHAPE
    assert _q(lib, x=A + 2) == mx.MXFP4_ERR_ALIGN
    assert _q(lib, c=A2 + 8) == mx.MXFP4_ERR_ALIGN
    assert _q(lib, s=A3 + 1) == mx.MXFP4_ERR_ALIGN
    assert _q(lib, o=OFFS + 2) == mx.MXFP4_ERR_ALIGN
    # K = 32 is legal for the quantizer; M_cap = 0 enqueues nothing and succeeds
    assert _q(lib, M=0, K=32) == mx.MXFP4_OK


@pytest.mark.parametrize("fn", ["mxfp4_to_fp8_rows", "mxfp4_to_fp8_cols_ragged"])
def test_conversion_argument_errors(lib, fn):
    for kw in ("c", "s", "y", "ys", "o"):
        assert _r(lib, fn, **{kw: None}) == mx.MXFP4_ERR_NULL
    assert _r(lib, fn, K=64) == mx.MXFP4_ERR_SHAPE      # conversions need K % 128 == 0
    assert _r(lib, fn, K=0) == mx.MXFP4_ERR_SHAPE
    assert _r(lib, fn, M=-5) == mx.MXFP4_ERR_SHAPE
    assert _r(lib, fn, G=-1) == mx.MXFP4_ERR_SHAPE
    assert _r(lib, fn, M=(1 << 31), K=128) == mx.MXFP4_ERR_SHAPE
    assert _r(lib, fn, c=A + 4) == mx.MXFP4_ERR_ALIGN
    assert _r(lib, fn, y=A3 + 1) == mx.MXFP4_ERR_ALIGN
    assert _r(lib, fn, ys=A4 + 3) == mx.MXFP4_ERR_ALIGN
    assert _r(lib, fn, o=OFFS + 1) == mx.MXFP4_ERR_ALIGN
    assert _r(lib, fn, M=0) == mx.MXFP4_OK
    if fn == "mxfp4_to_fp8_cols_ragged":      # documented K limit of the column call
        assert _r(lib, fn, M=1, K=(1 << 24) + 128) == mx.MXFP4_ERR_SHAPE
        assert _r(lib, fn, M=0, K=1 << 24) == mx.MXFP4_OK


def _f(lib, x=A, y=A2, ys=A3, o=OFFS, G=1, M=4, K=128):
    return lib.mxfp4_bf16_to_fp8_rows(x, y, ys, o, G, M, K, None)


def test_fp8_quantizer_argument_errors(lib):
    for kw in ("x", "y", "ys", "o"):
        assert _f(lib, **{kw: None}) == mx.MXFP4_ERR_NULL
    assert _f(lib, K=64) == mx.MXFP4_ERR_SHAPE           # 1x128 blocks need K % 128 == 0
    assert _f(lib, K=0) == mx.MXFP4_ERR_SHAPE
    assert _f(lib, M=-1) == mx.MXFP4_ERR_SHAPE
    assert _f(lib, G=0) == mx.MXFP4_ERR_SHAPE
    assert _f(lib, M=1 << 40, K=1 << 20) == mx.MXFP4_ERR_SHAPE
    assert _f(lib, x=A + 2) == mx.MXFP4_ERR_ALIGN
    assert _f(lib, y=A2 + 8) == mx.MXFP4_ERR_ALIGN
    assert _f(lib, ys=A3 + 1) == mx.MXFP4_ERR_ALIGN
    assert _f(lib, o=OFFS + 2) == mx.MXFP4_ERR_ALIGN
    assert _f(lib, M=0) == mx.MXFP4_OK


def _fc(lib, x=A, y=A2, ys=A3, o=OFFS, G=1, M=4, K=128):
    return lib.mxfp4_bf16_to_fp8_cols_ragged(x, y, ys, o, G, M, K, None)


def test_fp8_column_quantizer_argument_errors(lib):
    for kw in ("x", "y", "ys", "o"):
        assert _fc(lib, **{kw: None}) == mx.MXFP4_ERR_NULL
    assert _fc(lib, K=64) == mx.MXFP4_ERR_SHAPE
    assert _fc(lib, K=0) == mx.MXFP4_ERR_SHAPE
    assert _fc(lib, M=-1) == mx.MXFP4_ERR_SHAPE
    assert _fc(lib, G=0) == mx.MXFP4_ERR_SHAPE
    assert _fc(lib, M=(1 << 31), K=128) == mx.MXFP4_ERR_SHAPE
    assert _fc(lib, M=1, K=(1 << 24) + 128) == mx.MXFP4_ERR_SHAPE      # documented K limit
    assert _fc(lib, x=A + 2) == mx.MXFP4_ERR_ALIGN
    assert _fc(lib, y=A2 + 1) == mx.MXFP4_ERR_ALIGN
    assert _fc(lib, ys=A3 + 3) == mx.MXFP4_ERR_ALIGN
    assert _fc(lib, o=OFFS + 1) == mx.MXFP4_ERR_ALIGN
    assert _fc(lib, M=0) == mx.MXFP4_OK
    assert _fc(lib, M=0, K=1 << 24) == mx.MXFP4_OK


def _fb(lib, x=A, y=A2, ys=A3, yT=A4, ysT=A, o=OFFS, G=1, M=4, K=128):
    return lib.mxfp4_bf16_to_fp8_rows_cols_ragged(x, y, ys, yT, ysT, o, G, M, K, None)


def test_fp8_both_layouts_quantizer_argument_errors(lib):
    for kw in ("x", "y", "ys", "yT", "ysT", "o"):
        assert _fb(lib, **{kw: None}) == mx.MXFP4_ERR_NULL
    assert _fb(lib, K=64) == mx.MXFP4_ERR_SHAPE
    assert _fb(lib, G=0) == mx.MXFP4_ERR_SHAPE
    assert _fb(lib, M=-1) == mx.MXFP4_ERR_SHAPE
    assert _fb(lib, M=1, K=(1 << 24) + 128) == mx.MXFP4_ERR_SHAPE
    assert _fb(lib, x=A + 2) == mx.MXFP4_ERR_ALIGN
    assert _fb(lib, y=A2 + 1) == mx.MXFP4_ERR_ALIGN
    assert _fb(lib, ys=A3 + 8) == mx.MXFP4_ERR_ALIGN
    assert _fb(lib, yT=A4 + 4) == mx.MXFP4_ERR_ALIGN
    assert _fb(lib, ysT=A + 3) == mx.MXFP4_ERR_ALIGN
    assert _fb(lib, o=OFFS + 1) == mx.MXFP4_ERR_ALIGN
    assert _fb(lib, M=0) == mx.MXFP4_OK


def _gm(lib, a=A, sa=A2, w=A3, sw=A4, y=A, o=OFFS, G=1, M=4, N=256, K=128):
    return lib.mxfp4_fp8_grouped_gemm(a, sa, w, sw, y, o, G, M, N, K, None)


def test_grouped_gemm_argument_errors(lib):
    for kw in ("a", "sa", "w", "sw", "y", "o"):
        assert _gm(lib, **{kw: None}) == mx.MXFP4_ERR_NULL
    assert _gm(lib, K=64) == mx.MXFP4_ERR_SHAPE           # K % 128
    assert _gm(lib, N=128) == mx.MXFP4_ERR_SHAPE          # N % 256
    assert _gm(lib, N=0) == mx.MXFP4_ERR_SHAPE
    assert _gm(lib, K=(1 << 20) + 128) == mx.MXFP4_ERR_SHAPE
    assert _gm(lib, N=(1 << 20) + 256) == mx.MXFP4_ERR_SHAPE
    assert _gm(lib, G=0) == mx.MXFP4_ERR_SHAPE
    assert _gm(lib, M=-1) == mx.MXFP4_ERR_SHAPE
    assert _gm(lib, a=A + 4) == mx.MXFP4_ERR_ALIGN
    assert _gm(lib, y=A + 2) == mx.MXFP4_ERR_ALIGN
    assert _gm(lib, sw=A4 + 1) == mx.MXFP4_ERR_ALIGN
    assert _gm(lib, o=OFFS + 2) == mx.MXFP4_ERR_ALIGN
    assert _gm(lib, M=0) == mx.MXFP4_OK


def _nv(lib, x=A, c=A2, s=A3, am=A4, o=OFFS, G=1, M=4, K=32, sr=False):
    if sr:
        return lib.mxfp4_nvfp4_quantize_rows_sr(x, c, s, am, o, G, M, K, 0x1234, None)
    return lib.mxfp4_nvfp4_quantize_rows(x, c, s, am, o, G, M, K, None)


@pytest.mark.parametrize("sr", [False, True])
def test_nvfp4_quantizer_argument_errors(lib, sr):
    # rejected before anything is enqueued (a valid call writes the amax even for
    # M_cap == 0, so it needs a GPU); the stochastic-rounding entry checks the same
    _nv = functools.partial(globals()["_nv"], sr=sr)
    for kw in ("x", "c", "s", "am", "o"):
        assert _nv(lib, **{kw: None}) == mx.MXFP4_ERR_NULL
    assert _nv(lib, K=8) == mx.MXFP4_ERR_SHAPE            # K % 16
    assert _nv(lib, K=0) == mx.MXFP4_ERR_SHAPE
    assert _nv(lib, G=0) == mx.MXFP4_ERR_SHAPE
    assert _nv(lib, M=-1) == mx.MXFP4_ERR_SHAPE
    assert _nv(lib, x=A + 8) == mx.MXFP4_ERR_ALIGN
    assert _nv(lib, c=A2 + 4) == mx.MXFP4_ERR_ALIGN
    assert _nv(lib, s=A3 + 1) == mx.MXFP4_ERR_ALIGN
    assert _nv(lib, am=A4 + 2) == mx.MXFP4_ERR_ALIGN
    assert _nv(lib, o=OFFS + 2) == mx.MXFP4_ERR_ALIGN


def _wg(lib, dy=A, sdy=A2, x=A3, sx=A4, dw=A, o=OFFS, G=1, M=4, N=256, K=256):
    return lib.mxfp4_fp8_grouped_gemm_wgrad(dy, sdy, x, sx, dw, o, G, M, N, K, None)


def test_wgrad_gemm_argument_errors(lib):
    # every case is rejected before anything is enqueued (the valid call, which writes
    # the zero gradient even for M_cap == 0, needs a GPU)
    for kw in ("dy", "sdy", "x", "sx", "dw", "o"):
        assert _wg(lib, **{kw: None}) == mx.MXFP4_ERR_NULL
    assert _wg(lib, K=128) == mx.MXFP4_ERR_SHAPE          # K % 256
    assert _wg(lib, N=128) == mx.MXFP4_ERR_SHAPE          # N % 256
    assert _wg(lib, N=0) == mx.MXFP4_ERR_SHAPE
    assert _wg(lib, K=(1 << 20) + 256) == mx.MXFP4_ERR_SHAPE
    assert _wg(lib, N=(1 << 20) + 256) == mx.MXFP4_ERR_SHAPE
    assert _wg(lib, M=(1 << 22) + 1, N=256) == mx.MXFP4_ERR_SHAPE      # N * M_cap > 2^30
    assert _wg(lib, M=(1 << 21) + 1, K=512) == mx.MXFP4_ERR_SHAPE      # K * M_cap > 2^30
    assert _wg(lib, G=0) == mx.MXFP4_ERR_SHAPE
    assert _wg(lib, M=-1) == mx.MXFP4_ERR_SHAPE
    assert _wg(lib, dy=A + 4) == mx.MXFP4_ERR_ALIGN
    assert _wg(lib, x=A3 + 8) == mx.MXFP4_ERR_ALIGN
    assert _wg(lib, sx=A4 + 1) == mx.MXFP4_ERR_ALIGN
    assert _wg(lib, dw=A + 2) == mx.MXFP4_ERR_ALIGN
    assert _wg(lib, o=OFFS + 2) == mx.MXFP4_ERR_ALIGN


def test_validate_offsets_argument_errors(lib):
    assert lib.mxfp4_validate_offsets(None, 1, 4, None) == mx.MXFP4_ERR_NULL
    assert lib.mxfp4_validate_offsets(OFFS, 0, 4, None) == mx.MXFP4_ERR_SHAPE
    assert lib.mxfp4_validate_offsets(OFFS, 1, -1, None) == mx.MXFP4_ERR_SHAPE


def test_python_binding_raises_on_error_status():
    # raw device addresses pass through the binding unchecked and reach the library's
    # own validation (a misaligned BF16 pointer)
    with pytest.raises(mx.Mxfp4Error) as ei:
        mx.mxfp4_quantize_rows(A + 2, A2, A3, OFFS, G=1, M_cap=4, K=64, stream=0)
    assert ei.value.status == mx.MXFP4_ERR_ALIGN


def test_python_binding_checks_tensor_arguments():
    """Tensor arguments are checked before any pointer reaches the library: size for
    the launch, dtype, contiguity, device (CPU tensors here, so no launch happens)."""
    import torch
    M, K = 4, 256
    x = torch.zeros((M, K), dtype=torch.bfloat16)
    codes = torch.zeros((M, K // 2), dtype=torch.uint8)
    scales = torch.zeros((M, K // 32), dtype=torch.uint8)
    offs = torch.tensor([0, M], dtype=torch.int32)
    y = torch.zeros((M, K), dtype=torch.uint8)
    ys = torch.zeros((M, K // 128), dtype=torch.uint8)
    with pytest.raises(ValueError, match="codes holds 448 bytes, the launch needs 512"):
        mx.mxfp4_quantize_rows(x, codes[:, :112], scales, offs, stream=0)
    with pytest.raises(ValueError, match="y_scales holds"):
        mx.mxfp4_to_fp8_rows(codes, scales, y, ys[:3], offs, stream=0)
    with pytest.raises(ValueError, match="dtype"):
        mx.mxfp4_quantize_rows(x.float(), codes, scales, offs, stream=0)
    with pytest.raises(ValueError, match="group_offsets has dtype"):
        mx.mxfp4_to_fp8_rows(codes, scales, y, ys, offs.long(), stream=0)
    with pytest.raises(ValueError, match="contiguous"):
        mx.mxfp4_to_fp8_rows(codes, scales, torch.zeros((K, M), dtype=torch.uint8).t(), ys, offs, M_cap=M,
                             K=K, stream=0)
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        mx.mxfp4_quantize_rows(x, codes, scales, offs, stream=0)


def test_python_binding_checks_cols_scale_capacity(lib):
    import torch
    M, K, G = 300, 256, 3
    codes = torch.zeros((M, K // 2), dtype=torch.uint8)
    scales = torch.zeros((M, K // 32), dtype=torch.uint8)
    offs = torch.tensor([0, 100, 200, 300], dtype=torch.int32)
    yT = torch.zeros(M * K, dtype=torch.uint8)
    cap = mx.mxfp4_cols_scale_capacity(M, K, G)
    assert cap == K * ((M + 127) // 128 + G)
    with pytest.raises(ValueError, match="yT_scales holds"):
        mx.mxfp4_to_fp8_cols_ragged(codes, scales, yT, torch.zeros(cap - 1, dtype=torch.uint8), offs, stream=0)
    with pytest.raises(ValueError, match="yT holds"):
        mx.mxfp4_to_fp8_cols_ragged(codes, scales, yT[:-1], torch.zeros(cap, dtype=torch.uint8), offs, stream=0)


def test_product_package_does_not_import_oracle():
    pkg = os.path.join(ROOT, "block_scaled_precision_bf16tofp4row_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "oracle.c" not in text, f


# Valid calls with a launch to make: without a GPU the launch itself fails and the call
# reports MXFP4_ERR_HIP (never a crash, never OK).  Only run where no GPU exists: on a
# GPU these fake addresses would reach a kernel.
needs_no_gpu = pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="a GPU is present")


@needs_no_gpu
def test_valid_calls_without_a_device_report_hip_error(lib):
    E = mx.MXFP4_ERR_HIP
    assert _q(lib, M=4, K=64) == E
    assert _r(lib, "mxfp4_to_fp8_rows") == E
    assert _r(lib, "mxfp4_to_fp8_cols_ragged") == E
    assert _f(lib) == E
    assert _fc(lib) == E
    assert _fb(lib) == E
    assert _gm(lib) == E
    assert lib.mxfp4_fp8_grouped_gemm_wgrad(A, A2, A3, A4, A, OFFS, 1, 4, 256, 256, None) == E
    assert _nv(lib) == E
    assert _nv(lib, sr=True) == E
    assert lib.mxfp4_validate_offsets(OFFS, 1, 4, None) == E
    assert lib.mxfp4_wait_status(None) == E


def test_wait_limit_hook_is_host_only(lib):
    # sets a process-wide number; no HIP call, so it works without a device
    lib.mxfp4_set_wait_limit(3)
    lib.mxfp4_set_wait_limit(0)
    with pytest.raises(ValueError):
        mx.mxfp4_set_wait_limit(-1)


def test_timing_hook_is_host_only(lib):
    # arming and disarming only set this thread's two handles: no HIP call, works
    # without a device (the events themselves are used by the next launch)
    assert lib.mxfp4_time_next_launch(None, None) == mx.MXFP4_OK
    mx.mxfp4_time_next_launch(None, None)


def test_library_binds_the_hip_runtime_torch_loads():
    """Loading the library before anything imports torch must still leave one HIP
    runtime in the process, torch's own copy: both ask for it by the same soname, and
    the first copy loaded serves every later request."""
    import subprocess
    import sys
    code = (
        "import sys\n"
        "import block_scaled_precision_bf16tofp4row_amd as mx\n"
        "assert 'torch' not in sys.modules\n"
        "mx.load_library()\n"
        "import torch, os\n"
        "maps = open('/proc/self/maps').read().split()\n"
        "hip = sorted({os.path.realpath(p) for p in maps if '/libamdhip64.so' in p})\n"
        "want = os.path.realpath(os.path.join(os.path.dirname(torch.__file__), 'lib'))\n"
        "assert len(hip) == 1 and hip[0].startswith(want + os.sep), hip\n"
    )
    subprocess.run([sys.executable, "-c", code], cwd=ROOT, check=True, timeout=300)
