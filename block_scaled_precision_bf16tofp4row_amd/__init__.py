"""MI355X-native BF16 -> MXFP4 -> block-scaled FP8 conversion path.

Thin ctypes binding over ``libmxfp4cvt.so`` (C ABI in ``include/mxfp4cvt.h``).
The Python layer only marshals arguments: every step of the path runs in the
gfx950 HIP kernels of the library.  PyTorch provides device memory and streams.

Method: "Practical FP4 Training for Large-Scale MoE Models on Hopper GPUs",
technical summary section 2 (Methodology), items 1-3.

The binding has the same names as the C ABI:

* ``mxfp4_quantize_rows(x, codes, scales, offs, ...)``
* ``mxfp4_nvfp4_quantize_rows(x, codes, scales, tensor_amax, offs, ...)`` (NVFP4 variant)
* ``mxfp4_nvfp4_quantize_rows_sr(x, codes, scales, tensor_amax, offs, seed, ...)`` (the same,
  element codes rounded stochastically)
* ``mxfp4_to_fp8_rows(codes, scales, y, y_scales, offs, ...)``
* ``mxfp4_to_fp8_cols_ragged(codes, scales, yT, yT_scales, offs, ...)``
* ``mxfp4_bf16_to_fp8_rows(x, y, y_scales, offs, ...)`` and
  ``mxfp4_bf16_to_fp8_cols_ragged(x, yT, yT_scales, offs, ...)`` (backward FP8 quantizer), and
  ``mxfp4_bf16_to_fp8_rows_cols_ragged(x, y, y_scales, yT, yT_scales, offs, ...)`` (both
  layouts from one read)
* ``mxfp4_fp8_grouped_gemm(a, a_scales, w, w_scales, y, offs, ...)`` (FP8 expert GEMM)
* ``mxfp4_fp8_grouped_gemm_wgrad(dyT, dyT_scales, xT, xT_scales, dw, offs, ...)``
  (FP8 weight-gradient GEMM over the column layouts)
* ``mxfp4_cols_scale_capacity(M_cap, K, G)``, ``mxfp4_validate_offsets(offs, ...)``,
  ``mxfp4_status_string(status)``
* ``mxfp4_wait_status(stream)`` (raises if a column conversion's bounded wait gave up
  since the last check) and ``mxfp4_set_wait_limit(polls)`` (its test hook)
* ``mxfp4_time_next_launch(start, stop)`` (binds two HIP event handles to the kernels
  of this thread's next call, for kernel-only timing)

Array arguments are torch tensors on the GPU (BF16 input as ``torch.bfloat16``
or ``torch.int16``/``torch.uint16`` bits; uint8 outputs; int32 offsets), or raw
device addresses as ints (passed through unchecked).  Tensor arguments are
checked before the call (size for the launch, dtype, contiguity, device) and a
violation raises ``ValueError``.  The stream defaults to torch's current stream.
A non-OK status raises ``Mxfp4Error``.  If the library is not built the import
still works but every call raises; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmxfp4cvt.so")

MXFP4_OK = 0
MXFP4_ERR_NULL = 1
MXFP4_ERR_SHAPE = 2
MXFP4_ERR_ALIGN = 3
MXFP4_ERR_HIP = 4

EXPORTED = (
    "mxfp4_quantize_rows",
    "mxfp4_nvfp4_quantize_rows",
    "mxfp4_nvfp4_quantize_rows_sr",
    "mxfp4_to_fp8_rows",
    "mxfp4_to_fp8_cols_ragged",
    "mxfp4_bf16_to_fp8_rows",
    "mxfp4_bf16_to_fp8_cols_ragged",
    "mxfp4_bf16_to_fp8_rows_cols_ragged",
    "mxfp4_fp8_grouped_gemm",
    "mxfp4_fp8_grouped_gemm_wgrad",
    "mxfp4_cols_scale_capacity",
    "mxfp4_validate_offsets",
    "mxfp4_wait_status",
    "mxfp4_set_wait_limit",
    "mxfp4_time_next_launch",
    "mxfp4_status_string",
)


class Mxfp4Error(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {mxfp4_status_string(status)}")


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libmxfp4cvt.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m block_scaled_precision_bf16tofp4row_amd.build`")
    # The library and PyTorch both ask for the HIP runtime by the same soname
    # (libamdhip64.so.7), and the first one loaded serves the whole process.  PyTorch
    # ships its own build of it, and the device memory and streams handed to the
    # library come from PyTorch, so PyTorch is loaded first: loaded the other way
    # round, ROCm's system runtime would serve both and the library's calls fail.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    st = ctypes.c_int
    lib.mxfp4_quantize_rows.argtypes = [P, P, P, P, I32, I64, I64, P]
    lib.mxfp4_quantize_rows.restype = st
    lib.mxfp4_to_fp8_rows.argtypes = [P, P, P, P, P, I32, I64, I64, P]
    lib.mxfp4_to_fp8_rows.restype = st
    lib.mxfp4_to_fp8_cols_ragged.argtypes = [P, P, P, P, P, I32, I64, I64, P]
    lib.mxfp4_to_fp8_cols_ragged.restype = st
    lib.mxfp4_bf16_to_fp8_rows.argtypes = [P, P, P, P, I32, I64, I64, P]
    lib.mxfp4_bf16_to_fp8_rows.restype = st
    lib.mxfp4_bf16_to_fp8_cols_ragged.argtypes = [P, P, P, P, I32, I64, I64, P]
    lib.mxfp4_bf16_to_fp8_cols_ragged.restype = st
    lib.mxfp4_fp8_grouped_gemm.argtypes = [P, P, P, P, P, P, I32, I64, I64, I64, P]
    lib.mxfp4_fp8_grouped_gemm.restype = st
    lib.mxfp4_fp8_grouped_gemm_wgrad.argtypes = [P, P, P, P, P, P, I32, I64, I64, I64, P]
    lib.mxfp4_nvfp4_quantize_rows.argtypes = [P, P, P, P, P, I32, I64, I64, P]
    lib.mxfp4_nvfp4_quantize_rows_sr.argtypes = [P, P, P, P, P, I32, I64, I64, ctypes.c_uint64, P]
    lib.mxfp4_bf16_to_fp8_rows_cols_ragged.argtypes = [P, P, P, P, P, P, I32, I64, I64, P]
    lib.mxfp4_bf16_to_fp8_rows_cols_ragged.restype = st
    lib.mxfp4_nvfp4_quantize_rows.restype = st
    lib.mxfp4_nvfp4_quantize_rows_sr.restype = st
    lib.mxfp4_fp8_grouped_gemm_wgrad.restype = st
    lib.mxfp4_cols_scale_capacity.argtypes = [I64, I64, I32]
    lib.mxfp4_cols_scale_capacity.restype = I64
    lib.mxfp4_validate_offsets.argtypes = [P, I32, I64, P]
    lib.mxfp4_validate_offsets.restype = st
    lib.mxfp4_wait_status.argtypes = [P]
    lib.mxfp4_wait_status.restype = st
    lib.mxfp4_set_wait_limit.argtypes = [ctypes.c_uint32]
    lib.mxfp4_set_wait_limit.restype = None
    lib.mxfp4_time_next_launch.argtypes = [P, P]
    lib.mxfp4_time_next_launch.restype = st
    lib.mxfp4_status_string.argtypes = [st]
    lib.mxfp4_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def mxfp4_status_string(status: int) -> str:
    return load_library().mxfp4_status_string(int(status)).decode()


def mxfp4_cols_scale_capacity(M_cap: int, K: int, G: int) -> int:
    return int(load_library().mxfp4_cols_scale_capacity(int(M_cap), int(K), int(G)))


# ---- marshalling -------------------------------------------------------------------

def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, what: str):
    if status != MXFP4_OK:
        raise Mxfp4Error(status, what)


def _need(what: str, args):
    """Check the tensor arguments before any pointer reaches the library: each large
    enough for the launch, of an accepted dtype and contiguous, then all on the GPU.
    `args` holds (tensor, bytes needed, name, accepted dtypes); raw int device
    addresses and None are passed through unchecked."""
    tensors = [a for a in args if a[0] is not None and not isinstance(a[0], int)]
    for t, nbytes, name, dtypes in tensors:
        have = t.numel() * t.element_size()
        if have < nbytes:
            raise ValueError(f"{what}: {name} holds {have} bytes, the launch needs {nbytes}")
        if str(t.dtype).replace("torch.", "") not in dtypes:
            raise ValueError(f"{what}: {name} has dtype {t.dtype}, expected one of {', '.join(dtypes)}")
        if not t.is_contiguous():
            raise ValueError(f"{what}: {name} must be contiguous")
    for t, _, name, _ in tensors:
        if not t.is_cuda:
            raise ValueError(f"{what}: {name} must be a GPU tensor")


_U8 = ("uint8",)
_FP8 = ("uint8", "float8_e4m3fn")


def _dims(x, offs, G, M_cap, K):
    if G is None:
        G = offs.numel() - 1
    if M_cap is None:
        M_cap = x.shape[0]
    if K is None:
        K = x.shape[1]
    return int(G), int(M_cap), int(K)


def mxfp4_quantize_rows(x, codes, scales, offs, G=None, M_cap=None, K=None, stream=None):
    """BF16 [M_cap, K] -> codes [M_cap, K/2] uint8 + scales [M_cap, K/32] uint8."""
    G, M_cap, K = _dims(x, offs, G, M_cap, K)
    n = max(M_cap, 0) * max(K, 0)
    _need("mxfp4_quantize_rows", [(x, 2 * n, "x", ("bfloat16", "int16", "uint16")),
                                  (codes, n // 2, "codes", _U8), (scales, n // 32, "scales", _U8),
                                  (offs, 4 * (G + 1), "group_offsets", ("int32",))])
    lib = load_library()
    _check(lib.mxfp4_quantize_rows(_ptr(x), _ptr(codes), _ptr(scales), _ptr(offs), G, M_cap, K,
                                   _stream(stream)), "mxfp4_quantize_rows")


def mxfp4_to_fp8_rows(codes, scales, y, y_scales, offs, G=None, M_cap=None, K=None, stream=None):
    """codes/scales -> E4M3 y [M_cap, K] + UE8M0 y_scales [M_cap, K/128]."""
    if K is None:
        K = codes.shape[1] * 2
    G, M_cap, K = _dims(codes, offs, G, M_cap, K)
    n = max(M_cap, 0) * max(K, 0)
    _need("mxfp4_to_fp8_rows", [(codes, n // 2, "codes", _U8), (scales, n // 32, "scales", _U8),
                                (y, n, "y", _FP8), (y_scales, n // 128, "y_scales", _U8),
                                (offs, 4 * (G + 1), "group_offsets", ("int32",))])
    lib = load_library()
    _check(lib.mxfp4_to_fp8_rows(_ptr(codes), _ptr(scales), _ptr(y), _ptr(y_scales), _ptr(offs),
                                 G, M_cap, K, _stream(stream)), "mxfp4_to_fp8_rows")


def mxfp4_to_fp8_cols_ragged(codes, scales, yT, yT_scales, offs, G=None, M_cap=None, K=None,
                             stream=None):
    """codes/scales -> per-expert transposed E4M3 yT + UE8M0 yT_scales (see the header)."""
    if K is None:
        K = codes.shape[1] * 2
    G, M_cap, K = _dims(codes, offs, G, M_cap, K)
    n = max(M_cap, 0) * max(K, 0)
    cap = mxfp4_cols_scale_capacity(M_cap, K, G) if n > 0 and G >= 1 else 0
    _need("mxfp4_to_fp8_cols_ragged", [(codes, n // 2, "codes", _U8), (scales, n // 32, "scales", _U8),
                                       (yT, n, "yT", _FP8), (yT_scales, max(cap, 0), "yT_scales", _U8),
                                       (offs, 4 * (G + 1), "group_offsets", ("int32",))])
    lib = load_library()
    _check(lib.mxfp4_to_fp8_cols_ragged(_ptr(codes), _ptr(scales), _ptr(yT), _ptr(yT_scales),
                                        _ptr(offs), G, M_cap, K, _stream(stream)),
           "mxfp4_to_fp8_cols_ragged")


def mxfp4_bf16_to_fp8_rows(x, y, y_scales, offs, G=None, M_cap=None, K=None, stream=None):
    """BF16 [M_cap, K] -> E4M3 y [M_cap, K] + UE8M0 y_scales [M_cap, K/128] (1x128 blocks)."""
    G, M_cap, K = _dims(x, offs, G, M_cap, K)
    n = max(M_cap, 0) * max(K, 0)
    _need("mxfp4_bf16_to_fp8_rows", [(x, 2 * n, "x", ("bfloat16", "int16", "uint16")),
                                     (y, n, "y", _FP8), (y_scales, n // 128, "y_scales", _U8),
                                     (offs, 4 * (G + 1), "group_offsets", ("int32",))])
    lib = load_library()
    _check(lib.mxfp4_bf16_to_fp8_rows(_ptr(x), _ptr(y), _ptr(y_scales), _ptr(offs), G, M_cap, K,
                                      _stream(stream)), "mxfp4_bf16_to_fp8_rows")


def mxfp4_bf16_to_fp8_cols_ragged(x, yT, yT_scales, offs, G=None, M_cap=None, K=None, stream=None):
    """BF16 [M_cap, K] -> per-expert transposed E4M3 yT + UE8M0 yT_scales (1x128 blocks
    along the tokens; layout as mxfp4_to_fp8_cols_ragged, see the header)."""
    G, M_cap, K = _dims(x, offs, G, M_cap, K)
    n = max(M_cap, 0) * max(K, 0)
    cap = mxfp4_cols_scale_capacity(M_cap, K, G) if n > 0 and G >= 1 else 0
    _need("mxfp4_bf16_to_fp8_cols_ragged", [(x, 2 * n, "x", ("bfloat16", "int16", "uint16")),
                                            (yT, n, "yT", _FP8), (yT_scales, max(cap, 0), "yT_scales", _U8),
                                            (offs, 4 * (G + 1), "group_offsets", ("int32",))])
    lib = load_library()
    _check(lib.mxfp4_bf16_to_fp8_cols_ragged(_ptr(x), _ptr(yT), _ptr(yT_scales), _ptr(offs), G, M_cap, K,
                                             _stream(stream)), "mxfp4_bf16_to_fp8_cols_ragged")


def mxfp4_bf16_to_fp8_rows_cols_ragged(x, y, y_scales, yT, yT_scales, offs, G=None, M_cap=None, K=None,
                                       stream=None):
    """Both layouts of the backward FP8 quantizer from one read of x: what
    mxfp4_bf16_to_fp8_rows and mxfp4_bf16_to_fp8_cols_ragged write (see the header)."""
    G, M_cap, K = _dims(x, offs, G, M_cap, K)
    n = max(M_cap, 0) * max(K, 0)
    cap = mxfp4_cols_scale_capacity(M_cap, K, G) if n > 0 and G >= 1 else 0
    _need("mxfp4_bf16_to_fp8_rows_cols_ragged",
          [(x, 2 * n, "x", ("bfloat16", "int16", "uint16")), (y, n, "y", _FP8), (y_scales, n // 128, "y_scales", _U8),
           (yT, n, "yT", _FP8), (yT_scales, max(cap, 0), "yT_scales", _U8),
           (offs, 4 * (G + 1), "group_offsets", ("int32",))])
    lib = load_library()
    _check(lib.mxfp4_bf16_to_fp8_rows_cols_ragged(_ptr(x), _ptr(y), _ptr(y_scales), _ptr(yT), _ptr(yT_scales),
                                                  _ptr(offs), G, M_cap, K, _stream(stream)),
           "mxfp4_bf16_to_fp8_rows_cols_ragged")


def mxfp4_fp8_grouped_gemm(a, a_scales, w, w_scales, y, offs, G=None, M_cap=None, N=None, K=None,
                           stream=None):
    """E4M3 a [M_cap, K] (+ UE8M0 [M_cap, K/128]) x per-expert E4M3 w [G, N, K]
    (+ [G, N, K/128]) -> BF16 y [M_cap, N] (see the header)."""
    if G is None:
        G = offs.numel() - 1
    if M_cap is None:
        M_cap = a.shape[0]
    if K is None:
        K = a.shape[1]
    if N is None:
        N = w.shape[1]
    G, M_cap, N, K = int(G), int(M_cap), int(N), int(K)
    m, k = max(M_cap, 0), max(K, 0)
    _need("mxfp4_fp8_grouped_gemm", [(a, m * k, "a", _FP8), (a_scales, m * k // 128, "a_scales", _U8),
                                     (w, max(G, 0) * max(N, 0) * k, "w", _FP8),
                                     (w_scales, max(G, 0) * max(N, 0) * k // 128, "w_scales", _U8),
                                     (y, 2 * m * max(N, 0), "y", ("bfloat16", "int16", "uint16")),
                                     (offs, 4 * (G + 1), "group_offsets", ("int32",))])
    lib = load_library()
    _check(lib.mxfp4_fp8_grouped_gemm(_ptr(a), _ptr(a_scales), _ptr(w), _ptr(w_scales), _ptr(y), _ptr(offs),
                                      G, M_cap, N, K, _stream(stream)), "mxfp4_fp8_grouped_gemm")


def mxfp4_fp8_grouped_gemm_wgrad(dyT, dyT_scales, xT, xT_scales, dw, offs, N, K, G=None, M_cap=None,
                                 stream=None):
    """Column-layout E4M3 dY^T (width N) and X^T (width K) with their block scales ->
    BF16 dW [G, N, K] (see the header).  M_cap defaults to the capacity of xT (its
    bytes / K)."""
    if G is None:
        G = offs.numel() - 1
    if M_cap is None:
        M_cap = xT.numel() // int(K)
    G, M_cap, N, K = int(G), int(M_cap), int(N), int(K)
    m, g = max(M_cap, 0), max(G, 0)
    cap_n = mxfp4_cols_scale_capacity(M_cap, N, G) if N > 0 and G > 0 else 0
    cap_k = mxfp4_cols_scale_capacity(M_cap, K, G) if K > 0 and G > 0 else 0
    _need("mxfp4_fp8_grouped_gemm_wgrad",
          [(dyT, m * max(N, 0), "dyT", _FP8), (dyT_scales, max(cap_n, 0), "dyT_scales", _U8),
           (xT, m * max(K, 0), "xT", _FP8), (xT_scales, max(cap_k, 0), "xT_scales", _U8),
           (dw, 2 * g * max(N, 0) * max(K, 0), "dw", ("bfloat16", "int16", "uint16")),
           (offs, 4 * (G + 1), "group_offsets", ("int32",))])
    lib = load_library()
    _check(lib.mxfp4_fp8_grouped_gemm_wgrad(_ptr(dyT), _ptr(dyT_scales), _ptr(xT), _ptr(xT_scales), _ptr(dw),
                                            _ptr(offs), G, M_cap, N, K, _stream(stream)),
           "mxfp4_fp8_grouped_gemm_wgrad")


def mxfp4_nvfp4_quantize_rows(x, codes, scales, tensor_amax, offs, G=None, M_cap=None, K=None, stream=None,
                              seed=None):
    """BF16 [M_cap, K] -> NVFP4 codes [M_cap, K/2], E4M3 block scales [M_cap, K/16] and
    the tensor amax (one float32 on the GPU); see the header.  With a seed the element
    codes are rounded stochastically (mxfp4_nvfp4_quantize_rows_sr)."""
    if G is None:
        G = offs.numel() - 1
    if M_cap is None:
        M_cap = x.shape[0]
    if K is None:
        K = x.shape[1]
    G, M_cap, K = int(G), int(M_cap), int(K)
    m, k = max(M_cap, 0), max(K, 0)
    _need("mxfp4_nvfp4_quantize_rows", [(x, 2 * m * k, "x", ("bfloat16", "int16", "uint16")), (codes, m * k // 2, "codes", _U8),
                                        (scales, m * k // 16, "scales", _U8),
                                        (tensor_amax, 4, "tensor_amax", ("float32",)),
                                        (offs, 4 * (G + 1), "group_offsets", ("int32",))])
    lib = load_library()
    if seed is None:
        _check(lib.mxfp4_nvfp4_quantize_rows(_ptr(x), _ptr(codes), _ptr(scales), _ptr(tensor_amax), _ptr(offs),
                                             G, M_cap, K, _stream(stream)), "mxfp4_nvfp4_quantize_rows")
    else:
        _check(lib.mxfp4_nvfp4_quantize_rows_sr(_ptr(x), _ptr(codes), _ptr(scales), _ptr(tensor_amax), _ptr(offs),
                                                G, M_cap, K, int(seed) & 0xFFFFFFFFFFFFFFFF, _stream(stream)),
               "mxfp4_nvfp4_quantize_rows_sr")


def mxfp4_nvfp4_quantize_rows_sr(x, codes, scales, tensor_amax, offs, seed, G=None, M_cap=None, K=None,
                                 stream=None):
    """NVFP4 with the element codes rounded stochastically (Philox4x32-10 bits under the
    64-bit seed); see the header."""
    mxfp4_nvfp4_quantize_rows(x, codes, scales, tensor_amax, offs, G=G, M_cap=M_cap, K=K, stream=stream, seed=seed)


def alloc_nvfp4_outputs(M_cap: int, K: int, device="cuda"):
    import torch
    return (torch.empty((max(1, M_cap), K // 2), dtype=torch.uint8, device=device),
            torch.empty((max(1, M_cap), K // 16), dtype=torch.uint8, device=device),
            torch.empty(1, dtype=torch.float32, device=device))


def mxfp4_validate_offsets(offs, G=None, M_cap=None, stream=None) -> bool:
    """True if the device offsets satisfy the preconditions (synchronizes the stream)."""
    if G is None:
        G = offs.numel() - 1
    if M_cap is None:
        raise ValueError("M_cap is required")
    _need("mxfp4_validate_offsets", [(offs, 4 * (int(G) + 1), "group_offsets", ("int32",))])
    st = load_library().mxfp4_validate_offsets(_ptr(offs), int(G), int(M_cap), _stream(stream))
    if st == MXFP4_ERR_SHAPE:
        return False
    _check(st, "mxfp4_validate_offsets")
    return True


def mxfp4_wait_status(stream=None) -> None:
    """Synchronize the stream; raise Mxfp4Error (MXFP4_ERR_HIP) if a bounded wait of a
    column conversion on this device gave up since the last check (the status is
    cleared by the check)."""
    _check(load_library().mxfp4_wait_status(_stream(stream)),
           "mxfp4_wait_status (a column conversion left part of its output unwritten)")


def mxfp4_set_wait_limit(polls: int) -> None:
    """Polls per bounded wait of the column conversions launched after this call
    (0: the default, 2^24).  A test hook for the give-up path."""
    if not 0 <= int(polls) < 2 ** 32:
        raise ValueError("polls must fit in 32 bits")
    load_library().mxfp4_set_wait_limit(int(polls))


def mxfp4_time_next_launch(start, stop) -> None:
    """Bind two HIP event handles (ints, created by the caller with hipEventCreate) to
    the first and last kernel of this thread's next entry-point call, so that their
    elapsed time is the kernels' own execution; (None, None) disarms."""
    _check(load_library().mxfp4_time_next_launch(start or None, stop or None), "mxfp4_time_next_launch")


# ---- output allocation (plumbing: torch device memory) ----------------------------

def alloc_quantize_outputs(M_cap: int, K: int, device="cuda"):
    import torch
    return (torch.empty((M_cap, K // 2), dtype=torch.uint8, device=device),
            torch.empty((M_cap, K // 32), dtype=torch.uint8, device=device))


def alloc_rows_outputs(M_cap: int, K: int, device="cuda"):
    import torch
    return (torch.empty((M_cap, K), dtype=torch.uint8, device=device),
            torch.empty((M_cap, K // 128), dtype=torch.uint8, device=device))


def alloc_fp8q_rows_outputs(M_cap: int, K: int, device="cuda"):
    return alloc_rows_outputs(M_cap, K, device)


def alloc_cols_outputs(M_cap: int, K: int, G: int, device="cuda"):
    import torch
    cap = mxfp4_cols_scale_capacity(M_cap, K, G)
    return (torch.empty(max(1, M_cap * K), dtype=torch.uint8, device=device),
            torch.empty(max(1, cap), dtype=torch.uint8, device=device))
