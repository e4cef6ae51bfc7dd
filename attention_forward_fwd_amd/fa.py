"""Thin Python binding of libfa.so (include/fa.h): argument marshalling only.

Every step of the attention forward runs in the HIP kernels of libfa.so; PyTorch supplies
device memory and the current HIP stream.  There is no CPU fallback: if the library is not
built, or the tensors are not on a GPU, the call raises.
"""

from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

FA_MASK_NONE, FA_MASK_CAUSAL, FA_MASK_BITMASK = 0, 1, 2
FA_DTYPE_F16, FA_DTYPE_BF16 = 0, 1
MODES = {"none": FA_MASK_NONE, "causal": FA_MASK_CAUSAL, "bitmask": FA_MASK_BITMASK}
DTYPES = {torch.float16: FA_DTYPE_F16, torch.bfloat16: FA_DTYPE_BF16}
STATUS = {0: "FA_OK", 1: "FA_ERR_NULL_PTR", 2: "FA_ERR_BAD_SHAPE", 3: "FA_ERR_UNSUPPORTED",
          4: "FA_ERR_BAD_MASK_MODE", 5: "FA_ERR_HIP", 6: "FA_ERR_BAD_SCALE", 7: "FA_ERR_WORKSPACE",
          8: "FA_ERR_SCRATCH_LIMIT"}
EXPORTS = ("fa_fwd", "fa_fwd_lse", "fa_fwd_ex", "fa_fwd_noalloc", "fa_fwd_plan", "fa_pack_mask",
           "fa_mask_tiles", "fa_status_string", "fa_abi_version", "fa_set_kernel_events")

_lib = None


class FaPlan(ctypes.Structure):
    """fa_plan of include/fa.h."""
    _fields_ = [("rows_per_workgroup", ctypes.c_int), ("packed_v", ctypes.c_int),
                ("kv_splits", ctypes.c_int), ("kernels", ctypes.c_int),
                ("workgroups", ctypes.c_int64), ("workspace_bytes", ctypes.c_uint64)]


class FaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class _OnDevice:
    """Makes `index` the current HIP device for the call when it is not already (the library
    launches on the current device); yields torch's current stream handle on that device."""
    __slots__ = ("index", "prev")

    def __init__(self, device):
        self.index = device.index if device.index is not None else torch.cuda.current_device()
        self.prev = None

    def __enter__(self):
        cur = torch.cuda.current_device()
        if cur != self.index:
            self.prev = cur
            torch.cuda.set_device(self.index)
        return torch.cuda.current_stream(self.index).cuda_stream

    def __exit__(self, *exc):
        if self.prev is not None:
            torch.cuda.set_device(self.prev)
        return False


def lib_path() -> str:
    return _LIB_PATH


def load() -> ctypes.CDLL:
    """Load libfa.so (built in-tree by attention_forward_fwd_amd.build); raises if missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"{_LIB_PATH} is not built; run `python -m attention_forward_fwd_amd.build`")
        lib = ctypes.CDLL(_LIB_PATH)
        lib.fa_fwd.restype = ctypes.c_int
        lib.fa_fwd.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                               ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_void_p,
                               ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                               ctypes.c_void_p]
        lib.fa_fwd_lse.restype = ctypes.c_int
        lib.fa_fwd_lse.argtypes = lib.fa_fwd.argtypes[:13] + [ctypes.c_void_p, ctypes.c_void_p]
        lib.fa_fwd_ex.restype = ctypes.c_int
        lib.fa_fwd_ex.argtypes = (lib.fa_fwd.argtypes[:12] + [ctypes.c_void_p, ctypes.c_int]
                                  + [ctypes.c_void_p] * 3 + [ctypes.c_uint64, ctypes.c_void_p])
        lib.fa_fwd_noalloc.restype = ctypes.c_int
        lib.fa_fwd_noalloc.argtypes = (lib.fa_fwd.argtypes[:12] + [ctypes.c_void_p, ctypes.c_int]
                                       + [ctypes.c_void_p] * 3)
        for name in ("fa_pack_mask", "fa_mask_tiles"):
            f = getattr(lib, name)
            f.restype = ctypes.c_int
            f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                          ctypes.c_void_p, ctypes.c_void_p]
        lib.fa_fwd_plan.restype = ctypes.c_int
        lib.fa_fwd_plan.argtypes = [ctypes.c_int] * 9 + [ctypes.POINTER(FaPlan)]
        lib.fa_status_string.restype = ctypes.c_char_p
        lib.fa_status_string.argtypes = [ctypes.c_int]
        lib.fa_abi_version.restype = ctypes.c_int
        lib.fa_abi_version.argtypes = []
        lib.fa_set_kernel_events.restype = ctypes.c_int
        lib.fa_set_kernel_events.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        _lib = lib
    return _lib


def fa_status_string(status: int) -> str:
    return load().fa_status_string(int(status)).decode()


def set_kernel_events(start=None, stop=None) -> None:
    """Measurement hook (fa_set_kernel_events): the next call made on this thread records the
    torch.cuda.Events `start` and `stop` (already recorded once, so that they exist) on its
    stream around its attention kernel; start.elapsed_time(stop) is then that kernel's duration.
    (None, None) clears the hook."""
    if (start is None) != (stop is None):
        raise ValueError("give both events or neither")
    handles = []
    for ev in (start, stop):
        h = 0 if ev is None else int(ev.cuda_event)
        if ev is not None and h == 0:
            raise ValueError("record each event once before passing it (torch creates it then)")
        handles.append(h)
    st = load().fa_set_kernel_events(handles[0] or None, handles[1] or None)
    if st != 0:
        raise FaError(st, fa_status_string(st))


def fa_fwd_raw(dtype: int, mask_mode: int, batch: int, n_q_heads: int, n_kv_heads: int,
               seq_len: int, head_dim: int, scale: float, q: int, k: int, v: int, mask: int,
               o: int, stream: int) -> int:
    """Direct call of the C entry point with integer pointers; returns the fa_status code."""
    return load().fa_fwd(dtype, mask_mode, batch, n_q_heads, n_kv_heads, seq_len, head_dim,
                         ctypes.c_float(scale), q, k, v, mask, o, stream)


def fa_fwd_lse_raw(dtype: int, mask_mode: int, batch: int, n_q_heads: int, n_kv_heads: int,
                   seq_len: int, head_dim: int, scale: float, q: int, k: int, v: int, mask: int,
                   o: int, lse: int, stream: int) -> int:
    """Direct call of fa_fwd_lse with integer pointers; returns the fa_status code."""
    return load().fa_fwd_lse(dtype, mask_mode, batch, n_q_heads, n_kv_heads, seq_len, head_dim,
                             ctypes.c_float(scale), q, k, v, mask, o, lse, stream)


def fa_fwd_ex_raw(dtype: int, mask_mode: int, batch: int, n_q_heads: int, n_kv_heads: int,
                  seq_len: int, head_dim: int, scale: float, q: int, k: int, v: int, mask: int,
                  tiles: int, kv_splits: int, o: int, lse: int, workspace: int,
                  workspace_bytes: int, stream: int) -> int:
    """Direct call of fa_fwd_ex with integer pointers (0 = NULL); returns the fa_status code."""
    return load().fa_fwd_ex(dtype, mask_mode, batch, n_q_heads, n_kv_heads, seq_len, head_dim,
                            ctypes.c_float(scale), q, k, v, mask, tiles, kv_splits, o, lse,
                            workspace, workspace_bytes, stream)


def fa_fwd_noalloc_raw(dtype: int, mask_mode: int, batch: int, n_q_heads: int, n_kv_heads: int,
                       seq_len: int, head_dim: int, scale: float, q: int, k: int, v: int,
                       mask: int, tiles: int, kv_splits: int, o: int, lse: int,
                       stream: int) -> int:
    """Direct call of fa_fwd_noalloc with integer pointers (0 = NULL); returns the fa_status."""
    return load().fa_fwd_noalloc(dtype, mask_mode, batch, n_q_heads, n_kv_heads, seq_len,
                                 head_dim, ctypes.c_float(scale), q, k, v, mask, tiles, kv_splits,
                                 o, lse, stream)


def _ws_args(workspace, device):
    """(pointer, bytes) of a caller workspace tensor (any dtype, contiguous, on `device`), or
    (0, 0) for None (the library's pool)."""
    if workspace is None:
        return 0, 0
    if not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    _same_gpu("workspace", workspace, device)
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def _same_gpu(name, t, device):
    """Raises unless tensor t is on GPU `device` (the library writes or reads it there)."""
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be a GPU tensor on {device} (got {t.device})")


def _tiles_ptr(tiles, mode, B, Hq, S, device):
    if tiles is None:
        return 0
    if mode != "bitmask":
        raise ValueError("a tile summary applies to mode 'bitmask' only")
    R = (S + 63) // 64
    shape = (B, Hq, R, (R + 31) // 32)
    if (tuple(tiles.shape) != shape or tiles.dtype not in (torch.int32, getattr(torch, "uint32", torch.int32))
            or not tiles.is_contiguous()):
        raise ValueError(f"tiles must be a contiguous 32-bit GPU tensor of shape {shape}")
    _same_gpu("tiles", tiles, device)
    return tiles.data_ptr()


def _args(q, k, v, mode, scale, mask, out):
    """Checks the tensors and returns (B, S, Hq, Hkv, D, scale, mask pointer, out)."""
    if mode not in MODES:
        raise ValueError(f"mode must be one of {sorted(MODES)}")
    if not q.is_cuda:
        raise ValueError("q must be a GPU tensor (there is no CPU path)")
    for name, t in (("q", q), ("k", k), ("v", v)):
        _same_gpu(name, t, q.device)
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D [B, S, H, D]")
    if q.dtype not in DTYPES or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share dtype bfloat16 or float16")
    B, S, Hq, D = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[1] != S or k.shape[3] != D:
        raise ValueError("k and v must be [B, S, Hkv, D] matching q")
    Hkv = k.shape[2]
    if scale is None:
        scale = D ** -0.5
    mptr = 0
    if mode == "bitmask":
        W = (S + 31) // 32
        if mask is None or tuple(mask.shape) != (B, Hq, S, W):
            raise ValueError(f"bitmask mode needs mask of shape {(B, Hq, S, W)}")
        if mask.dtype not in (torch.int32, getattr(torch, "uint32", torch.int32)):
            raise ValueError("mask must hold 32-bit words")
        if not mask.is_contiguous():
            raise ValueError("mask must be a contiguous GPU tensor")
        _same_gpu("mask", mask, q.device)
        mptr = mask.data_ptr()
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like q")
    else:
        _same_gpu("out", out, q.device)
    return B, S, Hq, Hkv, D, float(scale), mptr, out


def fa_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, mode: str = "none",
           scale: float | None = None, mask: torch.Tensor | None = None,
           out: torch.Tensor | None = None, tiles: torch.Tensor | None = None,
           kv_splits: int = 1, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """O = softmax(scale Q K^T + mask) V on the GPU (see include/fa.h for the definition).

    q [B,S,Hq,D], k/v [B,S,Hkv,D] (bf16 or fp16, contiguous, on one GPU); mask [B,Hq,S,ceil(S/32)]
    int32/uint32 words for mode "bitmask"; tiles (optional, bitmask mode) the mask's per-block
    summary from mask_tiles, so dead 64-key tiles are not loaded; kv_splits: 1 = no split-KV,
    0 = automatic, 2..16 = that many key ranges per row tile; workspace (optional) a GPU buffer
    of at least workspace_bytes(...) bytes used instead of the library's pool.  Enqueued on
    torch's current stream; returns o."""
    B, S, Hq, Hkv, D, scale, mptr, out = _args(q, k, v, mode, scale, mask, out)
    tptr = _tiles_ptr(tiles, mode, B, Hq, S, q.device)
    wptr, wbytes = _ws_args(workspace, q.device)
    with _OnDevice(q.device) as stream:
        if tptr or kv_splits != 1 or wptr:
            st = fa_fwd_ex_raw(DTYPES[q.dtype], MODES[mode], B, Hq, Hkv, S, D, scale, q.data_ptr(),
                               k.data_ptr(), v.data_ptr(), mptr, tptr, int(kv_splits),
                               out.data_ptr(), 0, wptr, wbytes, stream)
        else:
            st = fa_fwd_raw(DTYPES[q.dtype], MODES[mode], B, Hq, Hkv, S, D, scale, q.data_ptr(),
                            k.data_ptr(), v.data_ptr(), mptr, out.data_ptr(), stream)
    if st != 0:
        raise FaError(st, fa_status_string(st))
    return out


def fa_fwd_lse(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, mode: str = "none",
               scale: float | None = None, mask: torch.Tensor | None = None,
               out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
               tiles: torch.Tensor | None = None, kv_splits: int = 1,
               workspace: torch.Tensor | None = None):
    """As fa_fwd, also returning the log-sum-exp of each row's kept scores.

    Returns (o, lse) with lse [B, Hq, S] float32 (-inf for a row with no kept key)."""
    B, S, Hq, Hkv, D, scale, mptr, out = _args(q, k, v, mode, scale, mask, out)
    tptr = _tiles_ptr(tiles, mode, B, Hq, S, q.device)
    if lse is None:
        lse = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
    elif (tuple(lse.shape) != (B, Hq, S) or lse.dtype != torch.float32 or not lse.is_contiguous()
          or lse.device != q.device):
        raise ValueError(f"lse must be a contiguous float32 tensor of shape {(B, Hq, S)} on q's device")
    wptr, wbytes = _ws_args(workspace, q.device)
    with _OnDevice(q.device) as stream:
        st = fa_fwd_ex_raw(DTYPES[q.dtype], MODES[mode], B, Hq, Hkv, S, D, scale, q.data_ptr(),
                           k.data_ptr(), v.data_ptr(), mptr, tptr, int(kv_splits),
                           out.data_ptr(), lse.data_ptr(), wptr, wbytes, stream)
    if st != 0:
        raise FaError(st, fa_status_string(st))
    return out, lse


def fa_pack_mask_raw(batch: int, n_heads: int, seq_len: int, mask_bytes: int, mask_words: int,
                     stream: int) -> int:
    return load().fa_pack_mask(batch, n_heads, seq_len, mask_bytes, mask_words, stream)


def fa_mask_tiles_raw(batch: int, n_heads: int, seq_len: int, mask_words: int, tiles: int,
                      stream: int) -> int:
    return load().fa_mask_tiles(batch, n_heads, seq_len, mask_words, tiles, stream)


def pack_mask(mask: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Byte or bool mask [B, H, S, S] on the GPU (nonzero keeps) -> int32 words [B, H, S, ceil(S/32)]
    in the layout fa_fwd reads (see include/fa.h)."""
    if not mask.is_cuda or not mask.is_contiguous():
        raise ValueError("mask must be a contiguous GPU tensor (there is no CPU path)")
    if mask.dtype not in (torch.uint8, torch.bool, torch.int8) or mask.dim() != 4:
        raise ValueError("mask must be a 4-D uint8/int8/bool tensor [B, H, S, S]")
    B, H, S, S2 = mask.shape
    if S != S2:
        raise ValueError("mask must be square in its last two dimensions")
    W = (S + 31) // 32
    if out is None:
        out = torch.empty((B, H, S, W), dtype=torch.int32, device=mask.device)
    elif tuple(out.shape) != (B, H, S, W) or out.dtype != torch.int32 or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous int32 tensor of shape {(B, H, S, W)}")
    else:
        _same_gpu("out", out, mask.device)
    with _OnDevice(mask.device) as stream:
        st = fa_pack_mask_raw(B, H, S, mask.data_ptr(), out.data_ptr(), stream)
    if st != 0:
        raise FaError(st, fa_status_string(st))
    return out


def mask_tiles(words: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Packed mask words [B, H, S, ceil(S/32)] on the GPU -> int32 summary [B, H, R, ceil(R/32)],
    R = ceil(S/64): bit t of block r set iff rows [64r, 64r+64) x keys [64t, 64t+64) keep a key."""
    if not words.is_cuda or not words.is_contiguous() or words.dim() != 4:
        raise ValueError("words must be a contiguous 4-D GPU tensor")
    if words.dtype not in (torch.int32, getattr(torch, "uint32", torch.int32)):
        raise ValueError("words must hold 32-bit words")
    B, H, S, W = words.shape
    if W != (S + 31) // 32:
        raise ValueError("words must be [B, H, S, ceil(S/32)]")
    R = (S + 63) // 64
    TW = (R + 31) // 32
    if out is None:
        out = torch.empty((B, H, R, TW), dtype=torch.int32, device=words.device)
    elif tuple(out.shape) != (B, H, R, TW) or out.dtype != torch.int32 or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous int32 tensor of shape {(B, H, R, TW)}")
    else:
        _same_gpu("out", out, words.device)
    with _OnDevice(words.device) as stream:
        st = fa_mask_tiles_raw(B, H, S, words.data_ptr(), out.data_ptr(), stream)
    if st != 0:
        raise FaError(st, fa_status_string(st))
    return out


def fa_fwd_plan(dtype: int, mask_mode: int, batch: int, n_q_heads: int, n_kv_heads: int,
                seq_len: int, head_dim: int, with_tiles: bool = False, kv_splits: int = 1) -> dict:
    """The launch plan of a call with these sizes (see include/fa.h); raises FaError on bad sizes."""
    plan = FaPlan()
    st = load().fa_fwd_plan(dtype, mask_mode, batch, n_q_heads, n_kv_heads, seq_len, head_dim,
                            int(bool(with_tiles)), kv_splits, ctypes.byref(plan))
    if st != 0:
        raise FaError(st, fa_status_string(st))
    return {name: getattr(plan, name) for name, _ in FaPlan._fields_}


def workspace_bytes(q: torch.Tensor, k: torch.Tensor, mode: str = "none", tiles: bool = False,
                    kv_splits: int = 1) -> int:
    """Bytes of device workspace a call with these tensors needs (0 if none): the size of the
    `workspace` buffer a caller passes to avoid the library's pool."""
    B, S, Hq, D = q.shape
    return fa_fwd_plan(DTYPES[q.dtype], MODES[mode], B, Hq, k.shape[2], S, D, tiles,
                       kv_splits)["workspace_bytes"]


def fa_fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
                   mode: str = "none", scale: float | None = None,
                   mask: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                   tiles: torch.Tensor | None = None, kv_splits: int = 1) -> torch.Tensor:
    """fa_fwd through fa_fwd_noalloc: nothing is allocated, neither by the library (its device
    scratch is a static array, FA_NOALLOC_SCRATCH_BYTES per GPU) nor here (out, and lse when
    wanted, are the caller's).  Calls that may overlap on one GPU share that array and race.
    Returns out."""
    if out is None:
        raise ValueError("fa_fwd_noalloc writes into the caller's out (it allocates nothing)")
    B, S, Hq, Hkv, D, scale, mptr, out = _args(q, k, v, mode, scale, mask, out)
    tptr = _tiles_ptr(tiles, mode, B, Hq, S, q.device)
    lptr = 0
    if lse is not None:
        if (tuple(lse.shape) != (B, Hq, S) or lse.dtype != torch.float32
                or not lse.is_contiguous()):
            raise ValueError(f"lse must be a contiguous float32 tensor of shape {(B, Hq, S)}")
        _same_gpu("lse", lse, q.device)
        lptr = lse.data_ptr()
    with _OnDevice(q.device) as stream:
        st = fa_fwd_noalloc_raw(DTYPES[q.dtype], MODES[mode], B, Hq, Hkv, S, D, scale,
                                q.data_ptr(), k.data_ptr(), v.data_ptr(), mptr, tptr,
                                int(kv_splits), out.data_ptr(), lptr, stream)
    if st != 0:
        raise FaError(st, fa_status_string(st))
    return out
