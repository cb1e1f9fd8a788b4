"""Python binding of libw4a4 (the MI355X packed W4A4 block-scaled linear).

Argument marshalling only: every step of the path runs in the gfx950
kernels behind the C ABI declared in include/w4a4.h.  torch supplies device
memory and the current HIP stream.  The raw C functions are available on
``lib()`` under their C names; the wrappers below keep the same names
without the ``w4a4_`` prefix:

    codes, scales, t = quantize_act(x_bf16, c_fp32, "mxfp4")
    blob             = pack_weight(w_codes, w_scales, t_w, r, "mxfp4")
    y_bf16           = linear(codes, scales, t, blob, "mxfp4", N, K)

There is no fallback: if the library is missing or fails to load, the
functions raise.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

__all__ = ["FORMATS", "lib", "library_path", "block_size", "scale_dtype", "quantize_act", "pack_weight",
           "unpack_weight", "linear", "linear_noalloc", "linear_workspace", "packed_weight_bytes", "W4A4Error"]

FORMATS = {"mxfp4": 0, "nvfp4": 1, "mxint4": 2, "int4g64": 3, "mxfp8": 4, "mxint8": 5, "int8g128": 6}
_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


class W4A4Error(RuntimeError):
    """A non-OK status from the C ABI (message from w4a4_last_error)."""

    def __init__(self, status: int, message: str):
        super().__init__(f"w4a4 status {status}: {message}")
        self.status = status


def library_path() -> str:
    """The in-tree libw4a4.so, or the file W4A4_LIBRARY names (a variant build
    of the same sources, e.g. the AddressSanitizer one)."""
    return os.environ.get("W4A4_LIBRARY") or os.path.join(_HERE, "libw4a4.so")


def lib() -> ctypes.CDLL:
    """Load libw4a4.so (built in-tree by build.py); raise if it is missing."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           f"`python -m w4a4_block_scaled_amd.build` (no fallback exists)")
    L = ctypes.CDLL(path)
    i64, sz, vp, i32 = ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int
    L.w4a4_block_size.argtypes = [i32]
    L.w4a4_block_size.restype = i32
    for name in ("w4a4_act_codes_bytes", "w4a4_act_scales_bytes",
                 "w4a4_quantize_workspace_bytes", "w4a4_packed_weight_bytes"):
        getattr(L, name).argtypes = [i32, i64, i64]
        getattr(L, name).restype = sz
    L.w4a4_linear_workspace_bytes.argtypes = [i32, i64, i64, i64]
    L.w4a4_linear_workspace_bytes.restype = sz
    L.w4a4_quantize_act.argtypes = [i32, i64, i64, vp, vp, vp, vp, vp, vp, sz, vp]
    L.w4a4_quantize_act.restype = i32
    L.w4a4_quantize_act_multi.argtypes = [i32, i64, i64, vp, i32, vp, vp, vp, vp, vp, sz, vp]
    L.w4a4_quantize_act_multi.restype = i32
    L.w4a4_linear_grouped.argtypes = [i32, i32, i64, i64, vp, vp, vp, vp, vp, vp, vp]
    L.w4a4_linear_grouped.restype = i32
    L.w4a4_pack_weight.argtypes = [i32, i64, i64, vp, vp, vp, vp, vp, vp]
    L.w4a4_pack_weight.restype = i32
    L.w4a4_unpack_weight.argtypes = [i32, i64, i64, vp, vp, vp, vp, vp, vp]
    L.w4a4_unpack_weight.restype = i32
    L.w4a4_linear.argtypes = [i32, i64, i64, i64, vp, vp, vp, vp, vp, vp, sz, vp]
    L.w4a4_linear.restype = i32
    L.w4a4_linear_noalloc.argtypes = [i32, i64, i64, i64, vp, vp, vp, vp, vp, vp]
    L.w4a4_linear_noalloc.restype = i32
    L.w4a4_dualquant_workspace_bytes.argtypes = [i32, i64, i64]
    L.w4a4_dualquant_workspace_bytes.restype = sz
    L.w4a4_dualquant_solve.argtypes = [i32, i64, i64, vp, i32, vp, vp, vp, vp, vp, vp, sz, vp]
    L.w4a4_dualquant_solve.restype = i32
    L.w4a4_probe_stream_read.argtypes = [vp, sz, vp, vp]
    L.w4a4_probe_stream_read.restype = i32
    L.w4a4_probe_empty.argtypes = [vp]
    L.w4a4_probe_empty.restype = i32
    L.w4a4_probe_mfma_fp4.argtypes = [vp, ctypes.c_int, ctypes.c_int, vp, vp]
    L.w4a4_probe_mfma_fp4.restype = i32
    L.w4a4_last_error.argtypes = []
    L.w4a4_last_error.restype = ctypes.c_char_p
    L.w4a4_version.argtypes = []
    L.w4a4_version.restype = ctypes.c_char_p
    _LIB = L
    return L


def _fmt(fmt) -> int:
    if isinstance(fmt, str):
        return FORMATS[fmt]
    return int(fmt)


def _check(status: int) -> None:
    if status != 0:
        raise W4A4Error(status, lib().w4a4_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def scale_dtype(fmt) -> torch.dtype:
    """Element type of block scales: bytes (E8M0 / UE4M3), BF16 for INT4 G=64 and INT8 G=128."""
    return torch.bfloat16 if _fmt(fmt) in (FORMATS["int4g64"], FORMATS["int8g128"]) else torch.uint8


def code_cols(fmt, K: int) -> int:
    """Bytes of canonical codes per row of K elements (K/2; K for the 8-bit formats)."""
    return K if _fmt(fmt) in (FORMATS["mxfp8"], FORMATS["mxint8"], FORMATS["int8g128"]) else K // 2


def block_size(fmt) -> int:
    return lib().w4a4_block_size(_fmt(fmt))


def packed_weight_bytes(fmt, N: int, K: int) -> int:
    return lib().w4a4_packed_weight_bytes(_fmt(fmt), N, K)


def quantize_act(x: torch.Tensor, c: Optional[torch.Tensor], fmt,
                 out: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None,
                 workspace: Optional[torch.Tensor] = None):
    """w4a4_quantize_act: x bf16 [M, K], c fp32 [K] or None -> (codes, scales, t).

    codes uint8 [M, K/2] ([M, K] for MXFP8 / MXINT8), scales [M, K/G] (uint8;
    bfloat16 for INT4 G=64),
    t fp32 [1] (NVFP4 tensor scale; unused for the other formats).
    """
    f = _fmt(fmt)
    L = lib()
    M, K = x.shape
    G = L.w4a4_block_size(f)
    if out is None:
        codes = torch.empty((M, code_cols(fmt, K)), dtype=torch.uint8, device=x.device)
        scales = torch.empty((M, K // G), dtype=scale_dtype(fmt), device=x.device)
        t = torch.ones(1, dtype=torch.float32, device=x.device)
    else:
        codes, scales, t = out
    ws_bytes = L.w4a4_quantize_workspace_bytes(f, M, K)
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=x.device)
    _check(L.w4a4_quantize_act(f, M, K, _ptr(x), _ptr(c), _ptr(codes), _ptr(scales), _ptr(t),
                               _ptr(workspace), workspace.numel() if workspace is not None else 0,
                               _stream(x.device)))
    return codes, scales, t


def quantize_act_multi(x: torch.Tensor, cs, fmt, workspace: Optional[torch.Tensor] = None):
    """w4a4_quantize_act_multi: bf16 [M, K] and P column-scale vectors -> a list of
    (codes [M, K/2], scales [M, K/G], t [1] for NVFP4 else None), X read once."""
    f = _fmt(fmt)
    L = lib()
    M, K = x.shape
    P = len(cs)
    G = block_size(fmt)
    outs = [(torch.empty((M, K // 2), dtype=torch.uint8, device=x.device),
             torch.empty((M, K // G), dtype=torch.uint8, device=x.device),
             torch.ones(1, dtype=torch.float32, device=x.device) if f == FORMATS["nvfp4"] else None)
            for _ in range(P)]
    ws_bytes = P * L.w4a4_quantize_workspace_bytes(f, M, K)
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=x.device)
    arr = ctypes.c_void_p * max(P, 1)
    c_arr = arr(*[_ptr(c) for c in cs])
    codes_arr = arr(*[_ptr(o[0]) for o in outs])
    scales_arr = arr(*[_ptr(o[1]) for o in outs])
    t_arr = arr(*[_ptr(o[2]) for o in outs])
    _check(L.w4a4_quantize_act_multi(f, M, K, _ptr(x), P, c_arr, codes_arr, scales_arr,
                                     t_arr if f == FORMATS["nvfp4"] else None, _ptr(workspace),
                                     workspace.numel() if workspace is not None else 0,
                                     _stream(x.device)))
    return outs


def pack_weight(codes: torch.Tensor, scales: torch.Tensor, t_w: Optional[torch.Tensor],
                r: torch.Tensor, fmt) -> torch.Tensor:
    """w4a4_pack_weight: canonical codes [N, K/2] ([N, K] for the 8-bit formats),
    scales, t_w [1] or None, r [N] -> blob."""
    f = _fmt(fmt)
    L = lib()
    N = codes.shape[0]
    K = codes.shape[1] * (1 if code_cols(fmt, 2) == 2 else 2)     # one byte or one nibble per code
    nbytes = L.w4a4_packed_weight_bytes(f, N, K)
    if nbytes == 0:
        raise W4A4Error(2, f"invalid packed weight shape N={N} K={K}")
    G = L.w4a4_block_size(f)
    if codes.dim() != 2 or tuple(scales.shape) != (N, K // G) or r.numel() != N:
        raise W4A4Error(2, f"pack_weight: codes {tuple(codes.shape)}, scales {tuple(scales.shape)} and "
                           f"r {tuple(r.shape)} do not describe one N={N} x K={K} weight")
    blob = torch.empty(nbytes, dtype=torch.uint8, device=codes.device)
    _check(L.w4a4_pack_weight(f, N, K, _ptr(codes), _ptr(scales), _ptr(t_w), _ptr(r), _ptr(blob),
                              _stream(codes.device)))
    return blob


def unpack_weight(blob: torch.Tensor, fmt, N: int, K: int):
    """w4a4_unpack_weight -> (codes [N, K/2], scales [N, K/G], r [N], t_w [1])."""
    f = _fmt(fmt)
    L = lib()
    G = L.w4a4_block_size(f)
    dev = blob.device
    codes = torch.empty((N, code_cols(fmt, K)), dtype=torch.uint8, device=dev)
    scales = torch.empty((N, K // G), dtype=scale_dtype(fmt), device=dev)
    r = torch.empty(N, dtype=torch.float32, device=dev)
    t_w = torch.empty(1, dtype=torch.float32, device=dev)
    _check(L.w4a4_unpack_weight(f, N, K, _ptr(blob), _ptr(codes), _ptr(scales), _ptr(r), _ptr(t_w),
                                _stream(dev)))
    return codes, scales, r, t_w


_LINEAR_WS = {}


def linear_workspace(device, nbytes: int) -> torch.Tensor:
    """A cached, zero-filled linear workspace of `device`, at least `nbytes`
    long (needed by the MXFP4 split-K GEMM; its synchronization words start
    at zero and every call leaves them at zero, so the one buffer serves all
    calls issued in order on one stream)."""
    device = torch.device(device)
    ws = _LINEAR_WS.get(device)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device=device)
        _LINEAR_WS[device] = ws
    return ws


def linear(a_codes: torch.Tensor, a_scales: torch.Tensor, t_act: Optional[torch.Tensor],
           blob: torch.Tensor, fmt, N: int, K: int, out: Optional[torch.Tensor] = None,
           workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """w4a4_linear: quantized activations [M, K/2] x packed weight -> bf16 [M, N].

    Without `workspace`, shapes that need one use linear_workspace().
    """
    f = _fmt(fmt)
    L = lib()
    M = a_codes.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a_codes.device)
    ws_bytes = L.w4a4_linear_workspace_bytes(f, M, N, K)
    if ws_bytes and workspace is None:
        workspace = linear_workspace(a_codes.device, ws_bytes)
    _check(L.w4a4_linear(f, M, N, K, _ptr(a_codes), _ptr(a_scales), _ptr(t_act), _ptr(blob),
                         _ptr(out), _ptr(workspace),
                         workspace.numel() if workspace is not None else 0,
                         _stream(a_codes.device)))
    return out


def linear_noalloc(a_codes: torch.Tensor, a_scales: torch.Tensor, t_act: Optional[torch.Tensor],
                   blob: torch.Tensor, fmt, N: int, K: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """w4a4_linear_noalloc: as linear(), with the split-K workspace taken from
    the library's own per-device scratch array (nothing is allocated by the
    library; `out` is allocated here only when not given)."""
    f = _fmt(fmt)
    L = lib()
    M = a_codes.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a_codes.device)
    _check(L.w4a4_linear_noalloc(f, M, N, K, _ptr(a_codes), _ptr(a_scales), _ptr(t_act), _ptr(blob),
                                 _ptr(out), _stream(a_codes.device)))
    return out


def dualquant_solve(w: torch.Tensor, fmt, iters: int = 15, workspace: Optional[torch.Tensor] = None):
    """w4a4_dualquant_solve: fp32 weights [N, K] -> (r [N], c [K], codes [N, K/2],
    scales [N, K/G], t_w [1] for NVFP4 else None).

    The offline dual-scale solver; W ~ diag(r) Q diag(c) (x t_w for NVFP4).
    Without `workspace`, one of w4a4_dualquant_workspace_bytes() bytes is
    allocated here.
    """
    f = _fmt(fmt)
    L = lib()
    N, K = w.shape
    ws_bytes = L.w4a4_dualquant_workspace_bytes(f, N, K)
    if ws_bytes == 0:
        raise W4A4Error(2, f"dualquant_solve: unsupported format or shape N={N} K={K}")
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=w.device)
    r = torch.empty(N, dtype=torch.float32, device=w.device)
    c = torch.empty(K, dtype=torch.float32, device=w.device)
    codes = torch.empty((N, K // 2), dtype=torch.uint8, device=w.device)
    scales = torch.empty((N, K // block_size(fmt)), dtype=torch.uint8, device=w.device)
    t_w = torch.ones(1, dtype=torch.float32, device=w.device) if f == FORMATS["nvfp4"] else None
    _check(L.w4a4_dualquant_solve(f, N, K, _ptr(w), int(iters), _ptr(r), _ptr(c), _ptr(codes),
                                  _ptr(scales), _ptr(t_w), _ptr(workspace), workspace.numel(),
                                  _stream(w.device)))
    return r, c, codes, scales, t_w


def linear_grouped(problems, fmt, K: int, outs=None):
    """w4a4_linear_grouped: problems = [(a_codes, a_scales, t_act, blob, N), ...]
    sharing M and K -> list of bf16 [M, N_p] outputs."""
    f = _fmt(fmt)
    L = lib()
    P = len(problems)
    M = problems[0][0].shape[0]
    dev = problems[0][0].device
    if outs is None:
        outs = [torch.empty((M, pr[4]), dtype=torch.bfloat16, device=dev) for pr in problems]
    arr = ctypes.c_void_p * P
    Ns = (ctypes.c_int64 * P)(*[int(pr[4]) for pr in problems])
    _check(L.w4a4_linear_grouped(f, P, M, K, Ns, arr(*[_ptr(pr[0]) for pr in problems]),
                                 arr(*[_ptr(pr[1]) for pr in problems]),
                                 arr(*[_ptr(pr[2]) for pr in problems]) if f == FORMATS["nvfp4"] else None,
                                 arr(*[_ptr(pr[3]) for pr in problems]), arr(*[_ptr(o) for o in outs]),
                                 _stream(dev)))
    return outs


def probe_stream_read(buf: torch.Tensor, sink: torch.Tensor) -> None:
    """w4a4_probe_stream_read: read all of `buf` (contiguous, its byte size a
    multiple of 16) once; `sink` a device buffer of at least 1 KiB."""
    _check(lib().w4a4_probe_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                        _stream(buf.device)))


def probe_mfma_fp4(ops: torch.Tensor, iters: int, workgroups: int, sink: torch.Tensor) -> None:
    """w4a4_probe_mfma_fp4: `iters` rounds of 16 scaled FP4 MFMAs per wave on
    the 16 KiB of operand fragments in `ops`, over `workgroups` workgroups of
    4 waves; `sink` a device buffer of at least 1 KiB."""
    if ops.numel() * ops.element_size() < 16384:
        raise ValueError("probe_mfma_fp4: ops must hold 16 KiB")
    _check(lib().w4a4_probe_mfma_fp4(_ptr(ops), int(iters), int(workgroups), _ptr(sink), _stream(ops.device)))


def probe_empty(device) -> None:
    """w4a4_probe_empty: one empty kernel on the current stream of `device`."""
    _check(lib().w4a4_probe_empty(_stream(torch.device(device))))

