"""ctypes binding of libattn.so (the C ABI in ``include/attn.h``).

Argument marshalling only: torch supplies device memory and the current HIP
stream; every step of the attention forward runs in the HIP library.  There
is no fallback -- if the library is missing or a tensor is not on the GPU the
call raises.
"""
from __future__ import annotations

import ctypes
import math
import os
import threading
from typing import Optional, Tuple

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn.so")
_lib = None
_lock = threading.Lock()

# attn_dtype
F32, BF16, BF16_OUT_F32, F16, F16_OUT_F32 = 0, 1, 2, 3, 4
# causal argument: no mask, mask aligned to the end of the keys, to their start
NON_CAUSAL, CAUSAL_END, CAUSAL_START = 0, 1, 2
# attn_status
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_MISALIGNED, ERR_HIP = 0, 1, 2, 3, 4
STATUS_NAMES = {OK: "ATTN_OK", ERR_INVALID_ARG: "ATTN_ERR_INVALID_ARG",
                ERR_UNSUPPORTED: "ATTN_ERR_UNSUPPORTED", ERR_MISALIGNED: "ATTN_ERR_MISALIGNED",
                ERR_HIP: "ATTN_ERR_HIP"}

EXPORTED = ("attn_fwd", "attn_fwd_tiles", "attn_select_tiles", "attn_fwd_split",
            "attn_select_splits", "attn_split_workspace_bytes", "attn_fwd_split_noalloc",
            "attn_last_error", "attn_version")
# bytes of the library's static per-device scratch (attn_fwd_split_noalloc)
NOALLOC_SCRATCH_BYTES = 64 << 20


class AttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def lib_path() -> str:
    return _LIB_PATH


def load() -> ctypes.CDLL:
    """Load libattn.so (built in-tree by ``tiled_online_softmax_05_amd.build``)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                               "`python -m tiled_online_softmax_05_amd.build`")
        lib = ctypes.CDLL(_LIB_PATH)
        vp, ip, fp = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        fwd_args = [vp, vp, vp, vp, vp, ip, ip, ip, ip, ip, fp, ip, ip, vp]
        lib.attn_fwd.argtypes = fwd_args
        lib.attn_fwd.restype = ip
        lib.attn_fwd_tiles.argtypes = fwd_args + [ip, ip]
        lib.attn_fwd_tiles.restype = ip
        pi = ctypes.POINTER(ctypes.c_int)
        lib.attn_select_tiles.argtypes = [ip, ip, ip, ip, ip, ip, pi, pi, pi, pi]
        lib.attn_select_tiles.restype = ip
        ll = ctypes.c_longlong
        lib.attn_fwd_split.argtypes = fwd_args + [ip, vp, ll]
        lib.attn_fwd_split.restype = ip
        lib.attn_fwd_split_noalloc.argtypes = fwd_args + [ip]
        lib.attn_fwd_split_noalloc.restype = ip
        lib.attn_select_splits.argtypes = [ip, ip, ip, ip, ip, ip, pi, pi]
        lib.attn_select_splits.restype = ip
        lib.attn_split_workspace_bytes.argtypes = [ip, ip, ip, ip, ip]
        lib.attn_split_workspace_bytes.restype = ll
        lib.attn_last_error.argtypes = []
        lib.attn_last_error.restype = ctypes.c_char_p
        lib.attn_version.argtypes = []
        lib.attn_version.restype = ip
        _lib = lib
        return lib


def last_error() -> str:
    return load().attn_last_error().decode()


def check(status: int) -> None:
    if status != OK:
        raise AttnError(status, last_error())


def select_tiles(d: int, Sq: int, Skv: int, BH: int, dtype: int, causal: bool
                 ) -> Tuple[int, int, int, int]:
    """The library's tile selector: (block_m, block_n, waves, lds_bytes)."""
    lib = load()
    out = [ctypes.c_int(0) for _ in range(4)]
    check(lib.attn_select_tiles(d, Sq, Skv, BH, dtype, int(causal), *[ctypes.byref(x) for x in out]))
    return tuple(x.value for x in out)


def select_splits(d: int, Sq: int, Skv: int, BH: int, dtype: int, causal: bool
                  ) -> Tuple[int, int]:
    """The library's key-chunk choice for attn_fwd_split: (n_splits, kv_chunk)."""
    lib = load()
    n, chunk = ctypes.c_int(0), ctypes.c_int(0)
    check(lib.attn_select_splits(d, Sq, Skv, BH, dtype, int(causal), ctypes.byref(n),
                                 ctypes.byref(chunk)))
    return n.value, chunk.value


def split_workspace_bytes(B: int, H: int, Sq: int, d: int, n_splits: int) -> int:
    """Workspace bytes attn_fwd_split needs for n_splits key chunks."""
    r = load().attn_split_workspace_bytes(B, H, Sq, d, n_splits)
    if r < 0:
        raise AttnError(ERR_INVALID_ARG, last_error())
    return int(r)


def _dtype_code(t: torch.dtype, out_dtype: Optional[torch.dtype]) -> int:
    if t == torch.float32:
        if out_dtype not in (None, torch.float32):
            raise ValueError("fp32 inputs produce an fp32 output")
        return F32
    if t == torch.bfloat16:
        if out_dtype in (None, torch.bfloat16):
            return BF16
        if out_dtype == torch.float32:
            return BF16_OUT_F32
        raise ValueError("bf16 inputs produce a bf16 or fp32 output")
    if t == torch.float16:
        if out_dtype in (None, torch.float16):
            return F16
        if out_dtype == torch.float32:
            return F16_OUT_F32
        raise ValueError("fp16 inputs produce an fp16 or fp32 output")
    raise TypeError(f"unsupported input dtype {t}")


def fwd_raw(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, lse_ptr: Optional[int], B: int,
            H: int, Sq: int, Skv: int, d: int, scale: float, causal: bool, dtype: int,
            stream: int, tiles: Optional[Tuple[int, int]] = None) -> None:
    """Direct call of ``attn_fwd`` / ``attn_fwd_tiles`` on raw device
    pointers (no checks beyond the library's own)."""
    lib = load()
    args = (q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, H, Sq, Skv, d, float(scale), int(causal),
            dtype, stream)
    if tiles is None:
        check(lib.attn_fwd(*args))
    else:
        check(lib.attn_fwd_tiles(*args, int(tiles[0]), int(tiles[1])))


def fwd_split_raw(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, lse_ptr: Optional[int],
                  B: int, H: int, Sq: int, Skv: int, d: int, scale: float, causal: bool,
                  dtype: int, stream: int, n_splits: int, ws_ptr: Optional[int],
                  ws_bytes: int) -> None:
    """Direct call of ``attn_fwd_split`` on raw device pointers."""
    check(load().attn_fwd_split(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, H, Sq, Skv, d,
                                float(scale), int(causal), dtype, stream, int(n_splits),
                                ws_ptr, int(ws_bytes)))


def fwd_split_noalloc_raw(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int,
                          lse_ptr: Optional[int], B: int, H: int, Sq: int, Skv: int, d: int,
                          scale: float, causal: bool, dtype: int, stream: int,
                          n_splits: int) -> None:
    """Direct call of ``attn_fwd_split_noalloc`` on raw device pointers (the
    library's static scratch holds the chunks' partial states)."""
    check(load().attn_fwd_split_noalloc(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, H, Sq, Skv, d,
                                        float(scale), int(causal), dtype, stream,
                                        int(n_splits)))


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
        scale: Optional[float] = None, out_dtype: Optional[torch.dtype] = None,
        tiles: Optional[Tuple[int, int]] = None, with_lse: bool = True,
        out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
        splits: Optional[int] = None, noalloc: bool = False
        ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """O, LSE = attention(q, k, v) on the GPU through ``attn_fwd``.

    ``q`` is ``[B, H, Sq, d]``, ``k`` and ``v`` ``[B, H, Skv, d]``, contiguous
    CUDA(HIP) tensors of one dtype (float32, bfloat16 or float16).  ``scale`` defaults to
    ``1/sqrt(d)``.  ``tiles=(block_m, block_n)`` forces a tile shape.
    ``causal`` is False/True (end-aligned) or ``CAUSAL_START``.
    ``splits`` (an int, 0 = the library's choice) calls ``attn_fwd_split``
    instead, with a workspace allocated here, or -- with ``noalloc=True`` --
    ``attn_fwd_split_noalloc``, which uses the library's static scratch (pass
    ``out`` and ``lse`` as well for a call that allocates nothing).  The call
    is enqueued on torch's current stream of q's device."""
    lib = load()
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k, v must be GPU tensors (there is no CPU path)")
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("expected 4-D [B, H, S, d] tensors")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    B, H, Sq, d = q.shape
    if k.shape[:2] != (B, H) or v.shape != k.shape or k.shape[3] != d:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)}")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    Skv = k.shape[2]
    code = _dtype_code(q.dtype, out_dtype)
    odt = {F32: torch.float32, BF16_OUT_F32: torch.float32, F16_OUT_F32: torch.float32,
           BF16: torch.bfloat16, F16: torch.float16}[code]
    if out is None:
        out = torch.empty((B, H, Sq, d), dtype=odt, device=q.device)
    elif out.shape != (B, H, Sq, d) or out.dtype != odt or not out.is_contiguous():
        raise ValueError("out has the wrong shape, dtype or layout")
    if with_lse and lse is None:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    lse_ptr = lse.data_ptr() if lse is not None else None
    if noalloc and splits is None:
        raise ValueError("noalloc applies to the split path: give splits as well")
    with torch.cuda.device(q.device):
        if splits is None:
            fwd_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse_ptr, B, H, Sq,
                    Skv, d, scale, causal, code, stream, tiles)
        else:
            if tiles is not None:
                raise ValueError("tiles and splits cannot be combined")
            if noalloc:
                fwd_split_noalloc_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                      lse_ptr, B, H, Sq, Skv, d, scale, causal, code, stream,
                                      int(splits))
                return out, lse
            n = int(splits) if splits > 0 else select_splits(d, Sq, Skv, B * H, code, causal)[0]
            nbytes = split_workspace_bytes(B, H, Sq, d, max(n, 1))
            ws = torch.empty(nbytes + 256, dtype=torch.uint8, device=q.device)
            base = (ws.data_ptr() + 255) // 256 * 256
            fwd_split_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse_ptr, B,
                          H, Sq, Skv, d, scale, causal, code, stream, n, base, nbytes)
    return out, lse
