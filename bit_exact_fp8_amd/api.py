"""Thin ctypes binding of ``libemu_fp8gemm.so`` (C ABI in ``include/emu_fp8gemm.h``).

Argument marshalling only: every step of the computation runs in the HIP
library's kernels.  PyTorch supplies device memory and the current stream.
There is no CPU fallback: without the built library every call raises.

``scaled_mm`` keeps the argument order of ``torch._scaled_mm`` as the mmaemu
user guide (section 3) describes it: ``mat1`` is ``[M, K]`` row-major, ``mat2``
is ``[K, N]`` column-major, i.e. ``w.t()`` for a row-major weight ``w [N, K]``.

Every call takes optional plan options for testing and tuning (``tile``: a
tile configuration index into ``TILE_CONFIGS``; ``defer``: a key of
``DEFER_MODES``); results never depend on them, and nothing is kept between
calls.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIBNAME = "libemu_fp8gemm.so"

# Enumerations of include/emu_fp8gemm.h
EMU_OK, EMU_ERR_INVALID_ARG, EMU_ERR_REJECTED, EMU_ERR_UNSUPPORTED, EMU_ERR_WORKSPACE, EMU_ERR_DEVICE = range(6)
FP8_FORMAT = {torch.float8_e4m3fn: 0, torch.float8_e5m2: 1}
FP8_FORMAT_NAME = {"e4m3fn": 0, "e5m2": 1}
OUT_DTYPE = {torch.bfloat16: 0, torch.float16: 1, torch.float32: 2, torch.float8_e4m3fn: 3,
             torch.float8_e5m2: 4}
PROFILE = {"hopper": 0, "ada-serial": 1, "ada-pairwise": 2}


class PlanOptions(ctypes.Structure):
    """emu_plan_options of include/emu_fp8gemm.h."""
    _fields_ = [("tile", ctypes.c_int), ("defer", ctypes.c_int)]


class EmuError(RuntimeError):
    """A non-OK status from the C ABI."""

    def __init__(self, status: int, message: str):
        super().__init__(f"emu status {status}: {message}")
        self.status = status


def library_path() -> str:
    return os.path.join(_PKG, _LIBNAME)


_LIB = None


def _lib():
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is not built: run __graft_entry__.build() (there is no CPU fallback)")
    lib = ctypes.CDLL(path, mode=ctypes.RTLD_GLOBAL)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    opt = ctypes.POINTER(PlanOptions)
    common = [vp, i32, i64, vp, i32, i64, i64, i64, i64]
    lib.emu_scaled_mm.argtypes = common + [vp, vp, vp, vp, i32, i64, i32, i32, i32, vp, ctypes.c_size_t, vp, opt]
    lib.emu_scaled_mm.restype = i32
    lib.emu_accumulate.argtypes = common + [vp, i64, i32, i32, i32, vp, ctypes.c_size_t, vp, opt]
    lib.emu_accumulate.restype = i32
    lib.emu_accumulate_c.argtypes = common + [vp, i64, vp, i64, i32, vp, opt]
    lib.emu_accumulate_c.restype = i32
    lib.emu_scaled_mm_noalloc.argtypes = common + [vp, vp, vp, vp, i32, i64, i32, i32, i32, vp, opt]
    lib.emu_scaled_mm_noalloc.restype = i32
    lib.emu_workspace_bytes.argtypes = [i64, i64, i64, i32, i32, i32, opt]
    lib.emu_workspace_bytes.restype = ctypes.c_size_t
    lib.emu_status_string.argtypes = [i32]
    lib.emu_status_string.restype = ctypes.c_char_p
    lib.emu_last_error_message.restype = ctypes.c_char_p
    lib.emu_abi_version.restype = i32
    _LIB = lib
    return lib


def abi_version() -> int:
    return _lib().emu_abi_version()


TILE_CONFIGS = ("64x128", "64x64", "32x64", "32x32", "16x16_g2", "16x16_g4", "64x64_mx", "64x128_mx",
                "16x8_g4", "16x64_mx", "32x32_s4", "32x32_mx_s4", "32x16_mx_s5")
DEFER_MODES = {"auto": -1, "off": 0, "on": 1}


def plan_options(tile: int | None = None, defer: str | None = None):
    """A pointer to emu_plan_options for one call, or None (all automatic).
    tile: an index into TILE_CONFIGS (None or -1: automatic); defer: a key of
    DEFER_MODES (the deferred-infinity plan)."""
    if tile is None and defer is None:
        return None
    t = -1 if tile is None else int(tile)
    if not -1 <= t < len(TILE_CONFIGS):
        raise ValueError(f"invalid tile configuration {tile}")
    if defer is not None and defer not in DEFER_MODES:
        raise ValueError(f"invalid deferred-infinity mode {defer}")
    return ctypes.pointer(PlanOptions(t, DEFER_MODES[defer or "auto"]))


def _check(status: int):
    if status != EMU_OK:
        lib = _lib()
        raise EmuError(status, (lib.emu_last_error_message() or b"").decode())


def workspace_bytes(M: int, N: int, K: int, split_S: int = 1, use_fast_accum: bool = True,
                    profile: str = "hopper", tile: int | None = None, defer: str | None = None) -> int:
    return int(_lib().emu_workspace_bytes(M, N, K, split_S, int(use_fast_accum), PROFILE[profile],
                                          plan_options(tile, defer)))


def _fmt(t: torch.Tensor) -> int:
    if t.dtype in FP8_FORMAT:
        return FP8_FORMAT[t.dtype]
    raise TypeError(f"expected a float8_e4m3fn or float8_e5m2 tensor, got {t.dtype}")


def _on_device(name: str, t: torch.Tensor, device):
    if t.device.type != "cuda" or t.device != device:
        raise ValueError(f"{name} must be a CUDA tensor on the operands' device ({device}), not {t.device}")


def _scale_ptr(s: torch.Tensor, device) -> int:
    if not isinstance(s, torch.Tensor) or s.numel() != 1 or s.dtype != torch.float32:
        raise ValueError("tensor-wise scales must be one-element float32 tensors")
    if s.device != device:
        raise ValueError("scales must live on the operands' device")
    return s.data_ptr()


def _stream_handle(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _operands(mat1, mat2):
    if mat1.dim() != 2 or mat2.dim() != 2:
        raise ValueError("mat1 and mat2 must be 2-D")
    M, K = mat1.shape
    K2, N = mat2.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    # the codes of a row must be contiguous whenever a row holds more than
    # one (the row stride of a single row is never used)
    if mat1.stride(1) != 1 and K > 1:
        raise ValueError("mat1 must be row-major [M, K] (unit stride along K)")
    w = mat2.t()  # [N, K]
    if w.stride(1) != 1 and K > 1:
        raise ValueError("mat2 must be column-major [K, N] (pass w.t() for a row-major w)")
    if mat1.device.type != "cuda":
        raise ValueError(f"the operands must be CUDA tensors, not {mat1.device}")
    _on_device("mat2", w, mat1.device)
    ldx = mat1.stride(0) if (M > 1 and K > 0) else K
    ldw = w.stride(0) if (N > 1 and K > 0) else K
    return mat1, w, M, N, K, ldx, ldw


def scaled_mm(mat1: torch.Tensor, mat2: torch.Tensor, scale_a: torch.Tensor, scale_b: torch.Tensor,
              out_dtype=None, use_fast_accum: bool = False, split_S: int = 1,
              profile: str = "hopper", out: torch.Tensor | None = None,
              scale_result: torch.Tensor | None = None, tile: int | None = None,
              defer: str | None = None) -> torch.Tensor:
    """y = (mat1 @ mat2) * scale_a * scale_b with the emulated FP8 arithmetic.

    Defaults follow torch (user guide, section 3): use_fast_accum=False and
    out_dtype = the input dtype.  scale_result (FP8 outputs only) is a
    one-element float32 tensor multiplied in before the saturating FP8
    conversion.  tile, defer: plan options (testing and tuning)."""
    x, w, M, N, K, ldx, ldw = _operands(mat1, mat2)
    if out_dtype is None:
        out_dtype = mat1.dtype
    if out_dtype not in OUT_DTYPE:
        raise EmuError(EMU_ERR_UNSUPPORTED, f"output dtype {out_dtype} is not supported")
    dev = x.device
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=dev)
    else:
        _on_device("out", out, dev)
        if out.shape != (M, N) or out.dtype != out_dtype or (N > 1 and out.stride(1) != 1):
            raise ValueError("out must be a row-major [M, N] tensor of out_dtype")
    ldo = out.stride(0) if M > 1 else N
    plan = plan_options(tile, defer)
    ws = workspace_bytes(M, N, K, split_S, use_fast_accum, profile, tile, defer)
    wsbuf = torch.empty(max(ws, 1), dtype=torch.uint8, device=dev)
    lib = _lib()
    sr = _scale_ptr(scale_result, dev) if scale_result is not None else None
    _check(lib.emu_scaled_mm(x.data_ptr(), _fmt(x), ldx, w.data_ptr(), _fmt(w), ldw, M, N, K,
                             _scale_ptr(scale_a, dev), _scale_ptr(scale_b, dev), sr, out.data_ptr(),
                             OUT_DTYPE[out_dtype], ldo, int(use_fast_accum), int(split_S),
                             PROFILE[profile], wsbuf.data_ptr(), ws, _stream_handle(dev), plan))
    return out


NOALLOC_SCRATCH_BYTES = 64 << 20   # EMU_NOALLOC_SCRATCH_BYTES


def scaled_mm_noalloc(mat1: torch.Tensor, mat2: torch.Tensor, scale_a: torch.Tensor, scale_b: torch.Tensor,
                      out: torch.Tensor, use_fast_accum: bool = False, split_S: int = 1,
                      profile: str = "hopper", scale_result: torch.Tensor | None = None,
                      tile: int | None = None, defer: str | None = None) -> torch.Tensor:
    """scaled_mm through emu_scaled_mm_noalloc, for callers that cannot
    allocate device memory: the caller gives the output tensor (its dtype is
    the output type), and the library's fixed per-GPU scratch takes the place
    of the workspace.  Calls on one GPU that may overlap share that scratch
    and must be ordered by the caller."""
    x, w, M, N, K, ldx, ldw = _operands(mat1, mat2)
    dev = x.device
    _on_device("out", out, dev)
    if out.shape != (M, N) or out.dtype not in OUT_DTYPE or (N > 1 and out.stride(1) != 1):
        raise ValueError("out must be a row-major [M, N] tensor of a supported output dtype")
    ldo = out.stride(0) if M > 1 else N
    sr = _scale_ptr(scale_result, dev) if scale_result is not None else None
    _check(_lib().emu_scaled_mm_noalloc(x.data_ptr(), _fmt(x), ldx, w.data_ptr(), _fmt(w), ldw, M, N, K,
                                        _scale_ptr(scale_a, dev), _scale_ptr(scale_b, dev), sr, out.data_ptr(),
                                        OUT_DTYPE[out.dtype], ldo, int(use_fast_accum), int(split_S),
                                        PROFILE[profile], _stream_handle(dev), plan_options(tile, defer)))
    return out


def accumulate(x: torch.Tensor, w: torch.Tensor, use_fast_accum: bool, split_S: int = 1,
               profile: str = "hopper", c: torch.Tensor | None = None, tile: int | None = None,
               defer: str | None = None) -> torch.Tensor:
    """The binary32 accumulator, without the epilogue.  Both operands are
    [rows, K] (user guide, section 3: this call takes w itself rather than
    w.t(), and use_fast_accum must be given).  c: optional incoming accumulators ([M, N] float32,
    row-major): the fast chains start from them instead of +0 (fast
    accumulation and split_S = 1 only).  tile, defer: plan options."""
    xx, ww, M, N, K, ldx, ldw = _operands(x, w.t())
    dev = xx.device
    acc = torch.empty((M, N), dtype=torch.float32, device=dev)
    ldacc = acc.stride(0) if M > 1 else N
    plan = plan_options(tile, defer)
    if c is not None:
        if not use_fast_accum or split_S != 1:
            raise EmuError(EMU_ERR_UNSUPPORTED, "incoming accumulators need fast accumulation and split_S = 1")
        if c.shape != (M, N) or c.dtype != torch.float32 or c.device != dev or (N > 1 and c.stride(1) != 1):
            raise ValueError("c must be a row-major [M, N] float32 tensor on the operands' device")
        ldc = c.stride(0) if M > 1 else N
        _check(_lib().emu_accumulate_c(xx.data_ptr(), _fmt(xx), ldx, ww.data_ptr(), _fmt(ww), ldw, M, N, K,
                                       c.data_ptr(), ldc, acc.data_ptr(), ldacc, PROFILE[profile],
                                       _stream_handle(dev), plan))
        return acc
    ws = workspace_bytes(M, N, K, split_S, use_fast_accum, profile, tile, defer)
    wsbuf = torch.empty(max(ws, 1), dtype=torch.uint8, device=dev)
    lib = _lib()
    _check(lib.emu_accumulate(xx.data_ptr(), _fmt(xx), ldx, ww.data_ptr(), _fmt(ww), ldw, M, N, K,
                              acc.data_ptr(), ldacc, int(use_fast_accum), int(split_S),
                              PROFILE[profile], wsbuf.data_ptr(), ws, _stream_handle(dev), plan))
    return acc
