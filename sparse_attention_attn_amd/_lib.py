"""ctypes marshalling for libattn.so (see include/attn.h for the contract of each call)."""

from __future__ import annotations

import ctypes
import functools
import os

import numpy as np

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))

ATTN_OK = 0
ATTN_ERR_INVALID_ARG = -1
ATTN_ERR_UNSUPPORTED = -2
ATTN_ERR_WORKSPACE = -3
ATTN_ERR_LAUNCH = -4

# Every function include/attn.h declares.
EXPORTED_SYMBOLS = (
    "attn_fwd",
    "attn_splitkv_num_splits",
    "attn_splitkv_workspace_bytes",
    "attn_fwd_splitkv",
    "attn_combine_lse",
    "attn_fwd_decode",
    "attn_decode_workspace_bytes",
    "attn_fwd_decode_noalloc",
    "attn_fwd_blocksparse",
    "attn_blocksparse_check",
    "attn_fwd_vertical_slash",
    "attn_vertical_slash_workspace_bytes",
    "attn_vertical_slash_check",
    "attn_build_sparse_index",
    "attn_sparse_index_sizes",
    "attn_sparse_index_workspace_bytes",
    "attn_build_vslash_index",
    "attn_status_string",
    "attn_last_error",
)


class AttnError(RuntimeError):
    """A library call returned a negative attn_status."""

    def __init__(self, fn: str, status: int, message: str):
        self.status = status
        super().__init__(f"{fn} failed with {_status_name(status)} ({status}): {message}")


class AttnTensorC(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("stride_b", ctypes.c_int64),
        ("stride_l", ctypes.c_int64),
        ("stride_h", ctypes.c_int64),
    ]


def lib_path() -> str:
    return os.environ.get("ATTN_LIB", os.path.join(_PKG_DIR, "libattn.so"))


_LIB = None


def load_library():
    """Load libattn.so once. Raises RuntimeError if it is missing (no fallback exists)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} not found: build the HIP library first "
            "(python -m sparse_attention_attn_amd.build)")
    lib = ctypes.CDLL(path)
    T = AttnTensorC
    i32, i64, f32, vp = ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p
    fp = ctypes.POINTER(ctypes.c_float)
    ip = ctypes.c_void_p
    lib.attn_fwd.argtypes = [T, T, T, T, vp, i32, i32, i32, i32, i32, i32, i32, i32, f32, vp]
    lib.attn_fwd.restype = i32
    lib.attn_splitkv_num_splits.argtypes = [i32] * 7
    lib.attn_splitkv_num_splits.restype = i32
    lib.attn_splitkv_workspace_bytes.argtypes = [i32] * 5
    lib.attn_splitkv_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_fwd_splitkv.argtypes = [T, T, T, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, i32,
                                     f32, vp]
    lib.attn_fwd_splitkv.restype = i32
    lib.attn_combine_lse.argtypes = [vp, vp, i32, T, vp, i32, i32, i32, i32, vp]
    lib.attn_combine_lse.restype = i32
    lib.attn_fwd_decode.argtypes = [T, T, T, T, vp, i32, i32, i32, i32, i32, i32, i32, i32, f32,
                                    vp, ctypes.c_size_t, vp]
    lib.attn_fwd_decode.restype = i32
    lib.attn_fwd_decode_noalloc.argtypes = [T, T, T, T, vp, i32, i32, i32, i32, i32, i32, i32, i32,
                                            f32, vp]
    lib.attn_fwd_decode_noalloc.restype = i32
    lib.attn_decode_workspace_bytes.argtypes = [i32] * 7
    lib.attn_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_fwd_blocksparse.argtypes = [T, T, T, T, vp, i32, i32, i32, i32, i32, i32, i32, i32,
                                         f32, i32, i32, ip, ip, ip, ip, vp]
    lib.attn_fwd_blocksparse.restype = i32
    lib.attn_blocksparse_check.argtypes = [ip, ip, ip, ip, i32, i32, i32, i32, i32, i32]
    lib.attn_blocksparse_check.restype = i32
    lib.attn_fwd_vertical_slash.argtypes = [T, T, T, T, vp, i32, i32, i32, i32, i32, i32, i32,
                                            i32, f32, ip, ip, ip, ip, ip, ip, vp,
                                            ctypes.c_size_t, vp]
    lib.attn_fwd_vertical_slash.restype = i32
    lib.attn_vertical_slash_workspace_bytes.argtypes = [i32, i32, i32]
    lib.attn_vertical_slash_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_vertical_slash_check.argtypes = [ip, ip, i32, i32, i32]
    lib.attn_vertical_slash_check.restype = i32
    lib.attn_build_sparse_index.argtypes = [T, T, i32, i32, i32, i32, i32, f32, i32, i32, vp, vp,
                                            vp, vp, vp, ctypes.c_size_t, vp]
    lib.attn_build_sparse_index.restype = i32
    lib.attn_sparse_index_sizes.argtypes = [i32, i32, i32, i32, i32, ctypes.POINTER(i64),
                                            ctypes.POINTER(i64)]
    lib.attn_sparse_index_sizes.restype = i32
    lib.attn_sparse_index_workspace_bytes.argtypes = [i32] * 5
    lib.attn_sparse_index_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_build_vslash_index.argtypes = [T, T, i32, i32, i32, i32, i32, f32, i32, i32, vp, vp,
                                            vp, vp, vp, ctypes.c_size_t, vp]
    lib.attn_build_vslash_index.restype = i32
    lib.attn_status_string.argtypes = [i32]
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_last_error.argtypes = []
    lib.attn_last_error.restype = ctypes.c_char_p
    del fp, i64
    _LIB = lib
    return lib


def _status_name(status: int) -> str:
    return load_library().attn_status_string(int(status)).decode()


def attn_status_string(status: int) -> str:
    return _status_name(status)


def attn_last_error() -> str:
    return load_library().attn_last_error().decode()


def _check(fn: str, status: int):
    if status != ATTN_OK:
        raise AttnError(fn, status, attn_last_error())


# ------------------------------------------------------------------------------------ helpers
# The helpers below run on every call, so they keep Python work small: torch is looked up once,
# each tensor's strides are read in one call, and the stream comes from torch's raw-stream query
# (the one its own generated kernels use) instead of building a Stream object.
_TORCH = None
_RAW_STREAM = None


def _torch():
    global _TORCH, _RAW_STREAM
    if _TORCH is None:
        import torch
        _RAW_STREAM = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        _TORCH = torch
    return _TORCH


def _tensor_desc(t, name):
    if t.dtype != _torch().bfloat16:
        raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
    st = t.stride()
    if len(st) != 4:
        raise ValueError(f"{name} must be [B, L, H, D], got shape {tuple(t.shape)}")
    if st[3] != 1:
        raise ValueError(f"{name} must have a contiguous head dimension")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    return AttnTensorC(t.data_ptr(), st[0], st[1], st[2])


def _opt_ptr(t, name, dtype_name="float32"):
    if t is None:
        return None
    if t.dtype != getattr(_torch(), dtype_name):
        raise TypeError(f"{name} must be {dtype_name}")
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous GPU tensor")
    return t.data_ptr()


def _stream(stream, device):
    """The HIP stream to launch on: the caller's, else torch's current stream on `device`."""
    if stream is not None:
        return int(stream)
    torch = _torch()
    if _RAW_STREAM is not None and device.index is not None:
        return _RAW_STREAM(device.index)
    return torch.cuda.current_stream(device).cuda_stream


# Shape checks. The C ABI receives raw pointers and cannot see buffer sizes, so every wrapper
# checks here, before any pointer is taken, that the tensors agree with the sizes it passes: a
# mismatch would otherwise become an out-of-bounds device access. They run before the GPU
# placement checks, so they hold for CPU tensors too.
def _shape(t, name, want):
    if tuple(t.shape) != tuple(want):
        raise ValueError(f"{name} must have shape {tuple(want)}, got {tuple(t.shape)}")


def _rank(t, name, n, what):
    if t.dim() != n:
        raise ValueError(f"{name} must be {what}, got shape {tuple(t.shape)}")


def _numel_at_least(t, name, n):
    if t.numel() < n:
        raise ValueError(f"{name} must hold at least {n} elements, got {t.numel()}")


def _bytes_at_least(t, name, n):
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() * t.element_size() < n:
        raise ValueError(f"{name} must hold at least {n} bytes, got "
                         f"{t.numel() * t.element_size()}")


def _numel(t, name, n):
    if t.numel() != n:
        raise ValueError(f"{name} must hold {n} elements, got {t.numel()}")


def _one_device(named):
    d0 = named[0][1].device
    for _, t in named:
        if t is not None and t.device != d0:
            names = ", ".join(f"{n}: {t.device}" for n, t in named if t is not None)
            raise ValueError(f"all tensors must be on one device ({names})")


def _qkv_sizes(q, k, v):
    """(B, Lq, Hq, Dqk, Lk, Hkv, Dv) after checking that q, k, v agree."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _rank(t, n, 4, "[B, L, H, D]")
    B, Lq, Hq, Dqk = q.shape
    Bk, Lk, Hkv, Dk = k.shape
    Bv, Lv, Hv, Dv = v.shape
    if Bk != B or Bv != B:
        raise ValueError(f"batch sizes differ: q {B}, k {Bk}, v {Bv}")
    if Lv != Lk or Hv != Hkv:
        raise ValueError(f"k [{Bk}, {Lk}, {Hkv}, {Dk}] and v [{Bv}, {Lv}, {Hv}, {Dv}] must agree "
                         "on length and heads")
    if Dk != Dqk:
        raise ValueError(f"k head dim {Dk} differs from q head dim {Dqk}")
    return B, Lq, Hq, Dqk, Lk, Hkv, Dv


def _index_qk_sizes(q, k):
    """(B, L, Hq, D) of the index builders' square inputs, after checking q and k agree."""
    _rank(q, "q", 4, "[B, L, Hq, D]")
    _rank(k, "k", 4, "[B, L, Hkv, D]")
    B, L, Hq, D = q.shape
    if k.shape[0] != B or k.shape[1] != L or k.shape[3] != D:
        raise ValueError(f"k {tuple(k.shape)} must be [B, L, Hkv, D] with q's B, L and D "
                         f"(q {tuple(q.shape)})")
    return B, L, Hq, D


def _check_out(o, lse, B, Lq, Hq, Dv):
    _shape(o, "o", (B, Lq, Hq, Dv))
    if lse is not None:
        _numel(lse, "lse", B * Hq * Lq)


# ------------------------------------------------------------------------------- entry points
def attn_fwd(q, k, v, o, lse=None, causal=True, scale=None, stream=None):
    """Dense attention forward: O (and LSE [B, Hq, Lq] fp32 if given) from Q, K, V."""
    B, Lq, Hq, Dqk, Lk, Hkv, Dv = _qkv_sizes(q, k, v)
    _check_out(o, lse, B, Lq, Hq, Dv)
    _one_device([("q", q), ("k", k), ("v", v), ("o", o), ("lse", lse)])
    if scale is None:
        scale = Dqk ** -0.5
    st = load_library().attn_fwd(
        _tensor_desc(q, "q"), _tensor_desc(k, "k"), _tensor_desc(v, "v"), _tensor_desc(o, "o"),
        _opt_ptr(lse, "lse"), B, Hq, Hkv, Lq, Lk, Dqk, Dv, int(bool(causal)), float(scale),
        _stream(stream, q.device))
    _check("attn_fwd", st)
    return o


def attn_splitkv_num_splits(B, Hq, Hkv, Lq, Lk, Dqk, Dv) -> int:
    return int(load_library().attn_splitkv_num_splits(B, Hq, Hkv, Lq, Lk, Dqk, Dv))


def attn_splitkv_workspace_bytes(B, Hq, Lq, Dv, num_splits) -> int:
    return int(load_library().attn_splitkv_workspace_bytes(B, Hq, Lq, Dv, num_splits))


def attn_fwd_splitkv(q, k, v, o_part, lse_part, causal=False, scale=None, stream=None):
    """Per-split partials: o_part fp32 [S, B, Hq, Lq, Dv], lse_part fp32 [S, B, Hq, Lq]."""
    B, Lq, Hq, Dqk, Lk, Hkv, Dv = _qkv_sizes(q, k, v)
    _rank(o_part, "o_part", 5, "[S, B, Hq, Lq, Dv]")
    S = o_part.shape[0]
    _shape(o_part, "o_part", (S, B, Hq, Lq, Dv))
    _shape(lse_part, "lse_part", (S, B, Hq, Lq))
    _one_device([("q", q), ("k", k), ("v", v), ("o_part", o_part), ("lse_part", lse_part)])
    if scale is None:
        scale = Dqk ** -0.5
    st = load_library().attn_fwd_splitkv(
        _tensor_desc(q, "q"), _tensor_desc(k, "k"), _tensor_desc(v, "v"),
        _opt_ptr(o_part, "o_part"), _opt_ptr(lse_part, "lse_part"), S, B, Hq, Hkv, Lq, Lk, Dqk,
        Dv, int(bool(causal)), float(scale), _stream(stream, q.device))
    _check("attn_fwd_splitkv", st)
    return o_part, lse_part


def attn_combine_lse(o_part, lse_part, o, lse=None, stream=None):
    """Merge split partials into O (bf16 [B, Lq, Hq, Dv], strided) and LSE."""
    _rank(o_part, "o_part", 5, "[S, B, Hq, Lq, Dv]")
    S, B, Hq, Lq, Dv = o_part.shape
    _shape(lse_part, "lse_part", (S, B, Hq, Lq))
    _check_out(o, lse, B, Lq, Hq, Dv)
    _one_device([("o_part", o_part), ("lse_part", lse_part), ("o", o), ("lse", lse)])
    st = load_library().attn_combine_lse(
        _opt_ptr(o_part, "o_part"), _opt_ptr(lse_part, "lse_part"), S, _tensor_desc(o, "o"),
        _opt_ptr(lse, "lse"), B, Hq, Lq, Dv, _stream(stream, o.device))
    _check("attn_combine_lse", st)
    return o


def splitkv_decode(q, k, v, o, lse=None, causal=False, scale=None, num_splits=None, stream=None,
                   workspace=None):
    """Convenience: allocate partials (unless given) and run attn_fwd_splitkv + attn_combine_lse.

    The MLA latent shape passes v = k[..., :512] (a view of k: same pointer and strides)."""
    torch = _torch()
    B, Lq, Hq, Dqk, Lk, Hkv, Dv = _qkv_sizes(q, k, v)
    S = num_splits or attn_splitkv_num_splits(B, Hq, Hkv, Lq, Lk, Dqk, Dv)
    if workspace is None:
        o_part = torch.empty((S, B, Hq, Lq, Dv), dtype=torch.float32, device=q.device)
        lse_part = torch.empty((S, B, Hq, Lq), dtype=torch.float32, device=q.device)
    else:
        o_part, lse_part = workspace
    attn_fwd_splitkv(q, k, v, o_part, lse_part, causal=causal, scale=scale, stream=stream)
    attn_combine_lse(o_part, lse_part, o, lse, stream=stream)
    return o


@functools.lru_cache(maxsize=256)
def attn_decode_workspace_bytes(B, Hq, Hkv, Lq, Lk, Dqk, Dv) -> int:
    return int(load_library().attn_decode_workspace_bytes(B, Hq, Hkv, Lq, Lk, Dqk, Dv))


def attn_fwd_decode(q, k, v, o, lse=None, causal=False, scale=None, workspace=None, stream=None):
    """Split-KV decode plus combine in one call; the partials go to `workspace` (allocated
    here unless given)."""
    torch = _torch()
    B, Lq, Hq, Dqk, Lk, Hkv, Dv = _qkv_sizes(q, k, v)
    _check_out(o, lse, B, Lq, Hq, Dv)
    if scale is None:
        scale = Dqk ** -0.5
    need = attn_decode_workspace_bytes(B, Hq, Hkv, Lq, Lk, Dqk, Dv)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _bytes_at_least(workspace, "workspace", need)
    _one_device([("q", q), ("k", k), ("v", v), ("o", o), ("lse", lse), ("workspace", workspace)])
    st = load_library().attn_fwd_decode(
        _tensor_desc(q, "q"), _tensor_desc(k, "k"), _tensor_desc(v, "v"), _tensor_desc(o, "o"),
        _opt_ptr(lse, "lse"), B, Hq, Hkv, Lq, Lk, Dqk, Dv, int(bool(causal)), float(scale),
        ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size(),
        _stream(stream, q.device))
    _check("attn_fwd_decode", st)
    return o


# Size of the library's per-device scratch array (ATTN_DECODE_SCRATCH_BYTES in include/attn.h).
ATTN_DECODE_SCRATCH_BYTES = 16 << 20


def attn_fwd_decode_noalloc(q, k, v, o, lse=None, causal=False, scale=None, stream=None):
    """attn_fwd_decode with the partials in the library's per-device scratch array: allocates
    nothing (for callers that cannot allocate). Calls that overlap on one GPU race."""
    B, Lq, Hq, Dqk, Lk, Hkv, Dv = _qkv_sizes(q, k, v)
    _check_out(o, lse, B, Lq, Hq, Dv)
    _one_device([("q", q), ("k", k), ("v", v), ("o", o), ("lse", lse)])
    if scale is None:
        scale = Dqk ** -0.5
    st = load_library().attn_fwd_decode_noalloc(
        _tensor_desc(q, "q"), _tensor_desc(k, "k"), _tensor_desc(v, "v"), _tensor_desc(o, "o"),
        _opt_ptr(lse, "lse"), B, Hq, Hkv, Lq, Lk, Dqk, Dv, int(bool(causal)), float(scale),
        _stream(stream, q.device))
    _check("attn_fwd_decode_noalloc", st)
    return o


def _int_ptr(a, name):
    """Device int32 tensor -> pointer (the kernel reads the lists on the GPU)."""
    torch = _torch()
    if a.dtype != torch.int32 or not a.is_cuda or not a.is_contiguous():
        raise ValueError(f"{name} must be a contiguous int32 GPU tensor")
    return ctypes.c_void_p(a.data_ptr())


def attn_fwd_blocksparse(q, k, v, o, blk_ptr, blk_idx, col_ptr, col_idx, lse=None, causal=True,
                         scale=None, block_m=64, block_n=64, stream=None):
    """Block-sparse forward over CSR lists (int32 GPU tensors, layout in include/attn.h).

    The list contents are read on the GPU and not checked here (attn_blocksparse_check checks
    host copies); their pointer arrays must have the sizes the layout fixes."""
    B, Lq, Hq, Dqk, Lk, Hkv, Dv = _qkv_sizes(q, k, v)
    _check_out(o, lse, B, Lq, Hq, Dv)
    _numel(blk_ptr, "blk_ptr", B * Hq * (-(-Lq // 64)) + 1)
    _numel(col_ptr, "col_ptr", B * Hq + 1)
    _one_device([("q", q), ("k", k), ("v", v), ("o", o), ("lse", lse), ("blk_ptr", blk_ptr),
                 ("blk_idx", blk_idx), ("col_ptr", col_ptr), ("col_idx", col_idx)])
    if scale is None:
        scale = Dqk ** -0.5
    st = load_library().attn_fwd_blocksparse(
        _tensor_desc(q, "q"), _tensor_desc(k, "k"), _tensor_desc(v, "v"), _tensor_desc(o, "o"),
        _opt_ptr(lse, "lse"), B, Hq, Hkv, Lq, Lk, Dqk, Dv, int(bool(causal)), float(scale),
        block_m, block_n, _int_ptr(blk_ptr, "blk_ptr"), _int_ptr(blk_idx, "blk_idx"),
        _int_ptr(col_ptr, "col_ptr"), _int_ptr(col_idx, "col_idx"), _stream(stream, q.device))
    _check("attn_fwd_blocksparse", st)
    return o


def attn_blocksparse_check(blk_ptr, blk_idx, col_ptr, col_idx, B, Hq, Lq, Lk, block_m=64,
                           block_n=64) -> int:
    """Validate HOST index lists (numpy int32 arrays). Returns ATTN_OK or raises AttnError."""
    arrs = [np.ascontiguousarray(np.asarray(x, dtype=np.int32))
            for x in (blk_ptr, blk_idx, col_ptr, col_idx)]
    ptrs = [ctypes.c_void_p(a.ctypes.data) if a.size else ctypes.c_void_p(None) for a in arrs]
    st = load_library().attn_blocksparse_check(*ptrs, B, Hq, Lq, Lk, block_m, block_n)
    _check("attn_blocksparse_check", st)
    return st


def attn_vertical_slash_workspace_bytes(B, Hq, Lk) -> int:
    return int(load_library().attn_vertical_slash_workspace_bytes(B, Hq, Lk))


def attn_fwd_vertical_slash(q, k, v, o, blk_ptr, blk_idx, col_ptr, col_idx, slash_ptr,
                            slash_idx, lse=None, causal=True, scale=None, workspace=None,
                            stream=None):
    """Block-sparse forward with per-head slash lines added to the union (int32 GPU tensors,
    layout in include/attn.h). Allocates the bitmap workspace with torch unless given."""
    torch = _torch()
    B, Lq, Hq, Dqk, Lk, Hkv, Dv = _qkv_sizes(q, k, v)
    _check_out(o, lse, B, Lq, Hq, Dv)
    _numel(blk_ptr, "blk_ptr", B * Hq * (-(-Lq // 64)) + 1)
    _numel(col_ptr, "col_ptr", B * Hq + 1)
    _numel(slash_ptr, "slash_ptr", B * Hq + 1)
    if scale is None:
        scale = Dqk ** -0.5
    wsb = attn_vertical_slash_workspace_bytes(B, Hq, Lk)
    if workspace is None:
        workspace = torch.empty(max(wsb, 1), dtype=torch.uint8, device=q.device)
    _bytes_at_least(workspace, "workspace", wsb)
    _one_device([("q", q), ("k", k), ("v", v), ("o", o), ("lse", lse), ("blk_ptr", blk_ptr),
                 ("blk_idx", blk_idx), ("col_ptr", col_ptr), ("col_idx", col_idx),
                 ("slash_ptr", slash_ptr), ("slash_idx", slash_idx), ("workspace", workspace)])
    st = load_library().attn_fwd_vertical_slash(
        _tensor_desc(q, "q"), _tensor_desc(k, "k"), _tensor_desc(v, "v"), _tensor_desc(o, "o"),
        _opt_ptr(lse, "lse"), B, Hq, Hkv, Lq, Lk, Dqk, Dv, int(bool(causal)), float(scale),
        _int_ptr(blk_ptr, "blk_ptr"), _int_ptr(blk_idx, "blk_idx"), _int_ptr(col_ptr, "col_ptr"),
        _int_ptr(col_idx, "col_idx"), _int_ptr(slash_ptr, "slash_ptr"),
        _int_ptr(slash_idx, "slash_idx"), ctypes.c_void_p(workspace.data_ptr()),
        workspace.numel() * workspace.element_size(), _stream(stream, q.device))
    _check("attn_fwd_vertical_slash", st)
    return o


def attn_vertical_slash_check(slash_ptr, slash_idx, B, Hq, Lk) -> int:
    """Validate HOST slash lists (numpy int32 arrays). Returns ATTN_OK or raises AttnError."""
    arrs = [np.ascontiguousarray(np.asarray(x, dtype=np.int32)) for x in (slash_ptr, slash_idx)]
    ptrs = [ctypes.c_void_p(a.ctypes.data) if a.size else ctypes.c_void_p(None) for a in arrs]
    st = load_library().attn_vertical_slash_check(*ptrs, B, Hq, Lk)
    _check("attn_vertical_slash_check", st)
    return st


def attn_sparse_index_sizes(B, Hq, L, topk_blocks, n_cols):
    """(entries of blk_idx, entries of col_idx) that attn_build_sparse_index writes."""
    nb, nc = ctypes.c_int64(0), ctypes.c_int64(0)
    st = load_library().attn_sparse_index_sizes(B, Hq, L, topk_blocks, n_cols, ctypes.byref(nb),
                                                ctypes.byref(nc))
    _check("attn_sparse_index_sizes", st)
    return nb.value, nc.value


def attn_sparse_index_workspace_bytes(B, Hq, Hkv, L, D) -> int:
    return int(load_library().attn_sparse_index_workspace_bytes(B, Hq, Hkv, L, D))


def attn_build_sparse_index(q, k, topk_blocks, n_cols, scale=None, outputs=None, workspace=None,
                            stream=None):
    """Block and column lists (CSR, int32 GPU tensors: blk_ptr, blk_idx, col_ptr, col_idx) for
    the block-sparse forward, built from Q [B, L, Hq, D] and K [B, L, Hkv, D] by the library's
    estimator (see include/attn.h). Allocates the outputs and the workspace with torch unless
    given."""
    torch = _torch()
    B, L, Hq, D = _index_qk_sizes(q, k)
    Hkv = k.shape[2]
    if scale is None:
        scale = D ** -0.5
    nb, nc = attn_sparse_index_sizes(B, Hq, L, topk_blocks, n_cols)
    nqb = -(-L // 64)
    if outputs is None:
        mk = lambda n: torch.empty(max(int(n), 1), dtype=torch.int32, device=q.device)
        outputs = (mk(B * Hq * nqb + 1), mk(nb), mk(B * Hq + 1), mk(nc))
    blk_ptr, blk_idx, col_ptr, col_idx = outputs
    _numel(blk_ptr, "blk_ptr", B * Hq * nqb + 1)
    _numel_at_least(blk_idx, "blk_idx", nb)
    _numel(col_ptr, "col_ptr", B * Hq + 1)
    _numel_at_least(col_idx, "col_idx", nc)
    wsb = attn_sparse_index_workspace_bytes(B, Hq, Hkv, L, D)
    if workspace is None:
        workspace = torch.empty(max(wsb, 1), dtype=torch.uint8, device=q.device)
    _bytes_at_least(workspace, "workspace", wsb)
    _one_device([("q", q), ("k", k), ("blk_ptr", blk_ptr), ("blk_idx", blk_idx),
                 ("col_ptr", col_ptr), ("col_idx", col_idx), ("workspace", workspace)])
    st = load_library().attn_build_sparse_index(
        _tensor_desc(q, "q"), _tensor_desc(k, "k"), B, Hq, Hkv, L, D, float(scale),
        int(topk_blocks), int(n_cols), _int_ptr(blk_ptr, "blk_ptr"), _int_ptr(blk_idx, "blk_idx"),
        _int_ptr(col_ptr, "col_ptr"), _int_ptr(col_idx, "col_idx"),
        ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size(),
        _stream(stream, q.device))
    _check("attn_build_sparse_index", st)
    return blk_ptr, blk_idx[:nb], col_ptr, col_idx[:nc]


def attn_build_vslash_index(q, k, n_cols, n_slash, scale=None, outputs=None, workspace=None,
                            stream=None):
    """Column and slash-line lists (CSR, int32 GPU tensors: col_ptr, col_idx, slash_ptr,
    slash_idx) for attn_fwd_vertical_slash, built from Q [B, L, Hq, D] and K [B, L, Hkv, D]
    with the library's probe (see include/attn.h). Allocates the outputs and the workspace
    with torch unless given."""
    torch = _torch()
    B, L, Hq, D = _index_qk_sizes(q, k)
    Hkv = k.shape[2]
    if scale is None:
        scale = D ** -0.5
    nc = B * Hq * min(max(int(n_cols), 0), L)
    ns = B * Hq * min(max(int(n_slash), 0), L)
    if outputs is None:
        mk = lambda n: torch.empty(max(int(n), 1), dtype=torch.int32, device=q.device)
        outputs = (mk(B * Hq + 1), mk(nc), mk(B * Hq + 1), mk(ns))
    col_ptr, col_idx, slash_ptr, slash_idx = outputs
    _numel(col_ptr, "col_ptr", B * Hq + 1)
    _numel_at_least(col_idx, "col_idx", nc)
    _numel(slash_ptr, "slash_ptr", B * Hq + 1)
    _numel_at_least(slash_idx, "slash_idx", ns)
    wsb = attn_sparse_index_workspace_bytes(B, Hq, Hkv, L, D)
    if workspace is None:
        workspace = torch.empty(max(wsb, 1), dtype=torch.uint8, device=q.device)
    _bytes_at_least(workspace, "workspace", wsb)
    _one_device([("q", q), ("k", k), ("col_ptr", col_ptr), ("col_idx", col_idx),
                 ("slash_ptr", slash_ptr), ("slash_idx", slash_idx), ("workspace", workspace)])
    st = load_library().attn_build_vslash_index(
        _tensor_desc(q, "q"), _tensor_desc(k, "k"), B, Hq, Hkv, L, D, float(scale), int(n_cols),
        int(n_slash), _int_ptr(col_ptr, "col_ptr"), _int_ptr(col_idx, "col_idx"),
        _int_ptr(slash_ptr, "slash_ptr"), _int_ptr(slash_idx, "slash_idx"),
        ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size(),
        _stream(stream, q.device))
    _check("attn_build_vslash_index", st)
    return col_ptr, col_idx[:nc], slash_ptr, slash_idx[:ns]
