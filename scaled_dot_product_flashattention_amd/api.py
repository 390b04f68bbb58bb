"""Python binding of libattn: the C-ABI entry points under the same names.

Argument marshalling only. torch supplies device memory (outputs, workspaces)
and the current stream; every step of the computation runs in libattn's HIP
kernels. There is no fallback: a missing library raises ImportError and any
nonzero status from the library raises AttnError.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

from .build import library_path

_DTYPE = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
_LAYOUT = {"bhsd": 0, "bshd": 1}


def layout_code(layout: str) -> int:
    """"bhsd" = [B,H,S,d], "bshd" = [B,S,H,d], "split:g" = [B,H/g,S,g,d]
    (ATTN_LAYOUT_SPLIT(g): heads in groups of g)."""
    if layout in _LAYOUT:
        return _LAYOUT[layout]
    if isinstance(layout, str) and layout.startswith("split:"):
        return 0x10000 | int(layout[6:])
    raise ValueError(f"layout must be 'bhsd', 'bshd' or 'split:g', not {layout!r}")


def layout_shape(layout: str, B: int, H: int, S: int, d: int) -> tuple:
    if layout == "bhsd":
        return (B, H, S, d)
    if layout == "bshd":
        return (B, S, H, d)
    g = layout_code(layout) & 0xffff
    return (B, H // g, S, g, d)


class TileInfo(ctypes.Structure):
    """attn_tile_info of attn.h: one tile variant of the fused kernel."""
    _fields_ = [("rows", ctypes.c_int), ("keys", ctypes.c_int), ("waves", ctypes.c_int),
                ("stages", ctypes.c_int), ("lds_bytes", ctypes.c_int)]


class AttnError(RuntimeError):
    """A libattn call returned a nonzero status."""

    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {attn_status_string(status)} (status {status})")
        self.status = status


_lib = None


def load_library() -> ctypes.CDLL:
    """Load libattn.so from the package directory (built in-tree)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(f"libattn.so is not built at {path}; build it with "
                          "`python -m scaled_dot_product_flashattention_amd.build`")
    L = ctypes.CDLL(path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    tensors = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, i, vp]
    L.attn_fwd.argtypes = tensors + [vp, sz, vp]
    L.attn_fwd.restype = i
    L.attn_fwd_splitk.argtypes = tensors + [i, vp, sz, vp]
    L.attn_fwd_splitk.restype = i
    L.attn_fwd_naive.argtypes = tensors + [vp, sz, vp]
    L.attn_fwd_naive.restype = i
    L.attn_fwd_workspace_size.argtypes = [i, i, i, i, i, i, i]
    L.attn_fwd_workspace_size.restype = sz
    L.attn_fwd_plan.argtypes = [i, i, i, i, i, i, i, ctypes.POINTER(i)]
    L.attn_fwd_plan.restype = i
    L.attn_splitk_workspace_size.argtypes = [i, i, i, i, i]
    L.attn_splitk_workspace_size.restype = sz
    L.attn_naive_scratch_size.argtypes = [i, i, i, i, i]
    L.attn_naive_scratch_size.restype = sz
    L.attn_qkv_proj.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, vp]
    L.attn_qkv_proj.restype = i
    L.attn_softmax_rows.argtypes = [vp, vp, vp, ctypes.c_int64, i, f, i, i, vp]
    L.attn_softmax_rows.restype = i
    L.attn_fwd_tile_count.argtypes = [i, i]
    L.attn_fwd_tile_count.restype = i
    L.attn_fwd_tile_info.argtypes = [i, i, i, ctypes.POINTER(TileInfo)]
    L.attn_fwd_tile_info.restype = i
    L.attn_fwd_tile_choice.argtypes = [i, i, i, i, i, i, i, ctypes.POINTER(i)]
    L.attn_fwd_tile_choice.restype = i
    L.attn_qkv_proj_tiling.argtypes = [i, i, i, i, i, ctypes.POINTER(i)]
    L.attn_qkv_proj_tiling.restype = i
    L.attn_fwd_tiled.argtypes = tensors + [i, i, vp, sz, vp]
    L.attn_fwd_tiled.restype = i
    L.attn_fwd_noalloc.argtypes = tensors + [vp]
    L.attn_fwd_noalloc.restype = i
    L.attn_status_string.argtypes = [i]
    L.attn_status_string.restype = ctypes.c_char_p
    L.attn_version.argtypes = []
    L.attn_version.restype = i
    _lib = L
    return L


# ---- host-only queries ---------------------------------------------------------
def attn_status_string(status: int) -> str:
    return load_library().attn_status_string(int(status)).decode()


def attn_version() -> int:
    return load_library().attn_version()


def dtype_code(dtype: torch.dtype) -> int:
    if dtype not in _DTYPE:
        raise TypeError(f"unsupported dtype {dtype}")
    return _DTYPE[dtype]


def attn_fwd_plan(B: int, H: int, Sq: int, Sk: int, d: int, dtype: torch.dtype,
                  causal: bool = False) -> int:
    n = ctypes.c_int(0)
    rc = load_library().attn_fwd_plan(B, H, Sq, Sk, d, dtype_code(dtype), int(bool(causal)),
                                      ctypes.byref(n))
    if rc:
        raise AttnError("attn_fwd_plan", rc)
    return n.value


def attn_fwd_tile_count(d: int, dtype: torch.dtype) -> int:
    return load_library().attn_fwd_tile_count(d, dtype_code(dtype))


def attn_fwd_tile_info(d: int, dtype: torch.dtype, tile: int) -> dict:
    info = TileInfo()
    rc = load_library().attn_fwd_tile_info(d, dtype_code(dtype), tile, ctypes.byref(info))
    if rc:
        raise AttnError("attn_fwd_tile_info", rc)
    return {name: getattr(info, name) for name, _ in TileInfo._fields_}


def attn_fwd_tile_choice(B: int, H: int, Sq: int, Sk: int, d: int, dtype: torch.dtype,
                         causal: bool = False) -> int:
    t = ctypes.c_int(-1)
    rc = load_library().attn_fwd_tile_choice(B, H, Sq, Sk, d, dtype_code(dtype), int(bool(causal)),
                                             ctypes.byref(t))
    if rc:
        raise AttnError("attn_fwd_tile_choice", rc)
    return t.value


def attn_qkv_proj_tiling(B: int, S: int, H: int, d: int, n_cu: int) -> int:
    """Tiling attn_qkv_proj runs for these tokens and columns on n_cu CUs
    (0: 128 x 192 tiles, 1: 256 x 256)."""
    t = ctypes.c_int(-1)
    rc = load_library().attn_qkv_proj_tiling(B, S, H, d, n_cu, ctypes.byref(t))
    if rc:
        raise AttnError("attn_qkv_proj_tiling", rc)
    return t.value


def attn_fwd_workspace_size(B: int, H: int, Sq: int, Sk: int, d: int, dtype: torch.dtype,
                            causal: bool = False) -> int:
    return load_library().attn_fwd_workspace_size(B, H, Sq, Sk, d, dtype_code(dtype),
                                                  int(bool(causal)))


def attn_splitk_workspace_size(B: int, H: int, Sq: int, d: int, n_split: int) -> int:
    return load_library().attn_splitk_workspace_size(B, H, Sq, d, n_split)


def attn_naive_scratch_size(B: int, H: int, Sq: int, Sk: int, dtype: torch.dtype) -> int:
    return load_library().attn_naive_scratch_size(B, H, Sq, Sk, dtype_code(dtype))


# ---- marshalling -----------------------------------------------------------------
def dims(q: torch.Tensor, k: torch.Tensor, layout: str):
    if layout == "bhsd":
        B, H, Sq, d = q.shape
        Sk = k.shape[2]
    elif layout == "bshd":
        B, Sq, H, d = q.shape
        Sk = k.shape[1]
    elif isinstance(layout, str) and layout.startswith("split:"):
        B, G, Sq, g, d = q.shape
        H, Sk = G * g, k.shape[2]
        if g != (layout_code(layout) & 0xffff):
            raise ValueError(f"q has groups of {g} heads, layout says {layout!r}")
    else:
        raise ValueError(f"layout must be 'bhsd', 'bshd' or 'split:g', not {layout!r}")
    return int(B), int(H), int(Sq), int(Sk), int(d)


def _check_buffer(name, t, device, shape=None, dtype=None):
    """A caller-supplied buffer: on `device`, dense, and of the stated shape
    and dtype; anything else would hand the kernels a wrong address or size."""
    if not isinstance(t, torch.Tensor) or t.device != device:
        raise ValueError(f"{name} must be a tensor on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, not {t.dtype}")


def _prepare(q, k, v, layout, kv_len, scale, lse, return_lse, out):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
            raise ValueError(f"{name} must be a CUDA (HIP) tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous in the {layout} layout")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k and v must be on one device")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v must share one dtype")
    if q.dim() != k.dim() or tuple(k.shape) != tuple(v.shape):
        raise ValueError("q, k, v must have the same rank and k, v the same shape")
    B, H, Sq, Sk, d = dims(q, k, layout)
    kshape = layout_shape(layout, B, H, Sk, d)
    if tuple(k.shape) != kshape:
        raise ValueError(f"k has shape {tuple(k.shape)}, expected {kshape}")
    if kv_len is not None:
        if kv_len.device != q.device or kv_len.dtype != torch.int32 or tuple(kv_len.shape) != (B,):
            raise ValueError("kv_len must be an int32 tensor of shape [B] on q's device")
        kv_len = kv_len.contiguous()
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty_like(q) if out is None else out
    _check_buffer("out", o, q.device, q.shape, q.dtype)
    if lse is None and return_lse:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    elif lse is not None:
        _check_buffer("lse", lse, q.device, (B, H, Sq), torch.float32)
    return (B, H, Sq, Sk, d), kv_len, float(scale), o, lse


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(q, stream):
    if stream is None:
        return torch.cuda.current_stream(q.device).cuda_stream
    return stream.cuda_stream if isinstance(stream, torch.cuda.Stream) else int(stream)


def _scratch(nbytes, device, given):
    if given is not None:
        _check_buffer("workspace", given, device)
        return given
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def attn_fwd(q, k, v, *, scale=None, causal=False, layout="bhsd", kv_len=None, return_lse=True,
             out=None, lse=None, workspace=None, stream=None):
    """Fused forward. Returns (o, lse); lse is None when return_lse is False."""
    (B, H, Sq, Sk, d), kv_len, scale, o, lse = _prepare(q, k, v, layout, kv_len, scale, lse,
                                                        return_lse, out)
    dt = dtype_code(q.dtype)
    # a caller's workspace is checked against the plan by the library itself
    nbytes = 0 if workspace is not None else attn_fwd_workspace_size(B, H, Sq, Sk, d, q.dtype, causal)
    ws = _scratch(nbytes, q.device, workspace)
    rc = load_library().attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Sq, Sk, d,
                                 scale, int(bool(causal)), layout_code(layout), dt, _ptr(kv_len),
                                 _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                                 _stream(q, stream))
    if rc:
        raise AttnError("attn_fwd", rc)
    return o, lse


def attn_fwd_noalloc(q, k, v, *, scale=None, causal=False, layout="bhsd", kv_len=None,
                     return_lse=True, out=None, lse=None, stream=None):
    """attn_fwd with the library's static workspace in place of a caller's:
    with ``out`` (and ``lse`` or return_lse=False) given, the call allocates
    no device memory. Plans needing more than ATTN_NOALLOC_SCRATCH_BYTES of
    workspace raise AttnError (ATTN_E_SCRATCH_LIMIT). Calls that may overlap
    on one GPU share that workspace and race."""
    (B, H, Sq, Sk, d), kv_len, scale, o, lse = _prepare(q, k, v, layout, kv_len, scale, lse,
                                                        return_lse, out)
    rc = load_library().attn_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Sq,
                                         Sk, d, scale, int(bool(causal)), layout_code(layout),
                                         dtype_code(q.dtype), _ptr(kv_len), _stream(q, stream))
    if rc:
        raise AttnError("attn_fwd_noalloc", rc)
    return o, lse


def attn_fwd_tiled(q, k, v, *, tile=-1, n_split=1, scale=None, causal=False, layout="bhsd",
                   kv_len=None, return_lse=True, out=None, lse=None, workspace=None, stream=None):
    """The fused kernel with tile variant ``tile`` (-1: the tuned table's
    choice) over ``n_split`` key ranges (more than 1: per-range records in
    the workspace, then the merge), never the split-over-keys pair.
    Returns (o, lse)."""
    (B, H, Sq, Sk, d), kv_len, scale, o, lse = _prepare(q, k, v, layout, kv_len, scale, lse,
                                                        return_lse, out)
    n_split = int(n_split)
    nbytes = attn_splitk_workspace_size(B, H, Sq, d, n_split) if n_split > 1 else 0
    ws = _scratch(nbytes, q.device, workspace)
    rc = load_library().attn_fwd_tiled(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Sq, Sk,
                                       d, scale, int(bool(causal)), layout_code(layout),
                                       dtype_code(q.dtype), _ptr(kv_len), int(tile), n_split,
                                       _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                                       _stream(q, stream))
    if rc:
        raise AttnError("attn_fwd_tiled", rc)
    return o, lse


def attn_fwd_splitk(q, k, v, *, n_split, scale=None, causal=False, layout="bhsd", kv_len=None,
                    return_lse=True, out=None, lse=None, workspace=None, stream=None):
    """Split-over-keys forward with an explicit split count. Returns (o, lse)."""
    (B, H, Sq, Sk, d), kv_len, scale, o, lse = _prepare(q, k, v, layout, kv_len, scale, lse,
                                                        return_lse, out)
    nbytes = attn_splitk_workspace_size(B, H, Sq, d, int(n_split))
    ws = _scratch(nbytes, q.device, workspace)
    rc = load_library().attn_fwd_splitk(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Sq,
                                        Sk, d, scale, int(bool(causal)), layout_code(layout),
                                        dtype_code(q.dtype), _ptr(kv_len), int(n_split), _ptr(ws),
                                        0 if ws is None else ws.numel() * ws.element_size(),
                                        _stream(q, stream))
    if rc:
        raise AttnError("attn_fwd_splitk", rc)
    return o, lse


def attn_fwd_naive(q, k, v, *, scale=None, causal=False, layout="bhsd", kv_len=None,
                   return_lse=True, out=None, lse=None, scratch=None, stream=None):
    """Unfused three-kernel baseline (materialised S and P). Returns (o, lse)."""
    (B, H, Sq, Sk, d), kv_len, scale, o, lse = _prepare(q, k, v, layout, kv_len, scale, lse,
                                                        return_lse, out)
    nbytes = attn_naive_scratch_size(B, H, Sq, Sk, q.dtype)
    sc = _scratch(nbytes, q.device, scratch)
    rc = load_library().attn_fwd_naive(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Sq,
                                       Sk, d, scale, int(bool(causal)), layout_code(layout),
                                       dtype_code(q.dtype), _ptr(kv_len), _ptr(sc),
                                       0 if sc is None else sc.numel() * sc.element_size(),
                                       _stream(q, stream))
    if rc:
        raise AttnError("attn_fwd_naive", rc)
    return o, lse


def attn_qkv_proj(x, w, *, H, d, layout="bhsd", out=None, stream=None):
    """QKV projection: x [B, S, D] and the out-major weight w [3*H*d, D] into
    (q, k, v) in `layout`, the inputs of attn_fwd. `out` may supply the three
    output tensors."""
    for name, t in (("x", x), ("w", w)):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
            raise ValueError(f"{name} must be a CUDA (HIP) tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if x.dim() != 3 or w.dim() != 2 or x.dtype != w.dtype:
        raise ValueError("x must be [B, S, D] and w [3*H*d, D] of one dtype")
    B, S, D = (int(n) for n in x.shape)
    if tuple(w.shape) != (3 * H * d, D):
        raise ValueError(f"w has shape {tuple(w.shape)}, expected {(3 * H * d, D)}")
    shape = layout_shape(layout, B, int(H), S, int(d))
    if x.device != w.device:
        raise ValueError("x and w must be on one device")
    if out is None:
        out = tuple(torch.empty(shape, dtype=x.dtype, device=x.device) for _ in range(3))
    if len(out) != 3:
        raise ValueError("out must hold three tensors (q, k, v)")
    for name, t in zip(("out q", "out k", "out v"), out):
        _check_buffer(name, t, x.device, shape, x.dtype)
    rc = load_library().attn_qkv_proj(_ptr(x), _ptr(w), *(_ptr(t) for t in out), B, S, D, int(H),
                                      int(d), layout_code(layout), dtype_code(x.dtype),
                                      _stream(x, stream))
    if rc:
        raise AttnError("attn_qkv_proj", rc)
    return tuple(out)


_SOFTMAX_MODES = {"online": 0, "three_pass": 1}


def attn_softmax_rows(x, *, scale=1.0, mode="online", return_lse=True, out=None, lse=None,
                      stream=None):
    """Row softmax of x [rows, n] (2-D, contiguous, on the GPU). mode is
    "online" or "three_pass". Returns (y, lse); lse is None when return_lse
    is False."""
    if not isinstance(x, torch.Tensor) or x.device.type != "cuda" or x.dim() != 2:
        raise ValueError("x must be a 2-D CUDA (HIP) tensor")
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    if mode not in _SOFTMAX_MODES:
        raise ValueError(f"mode must be 'online' or 'three_pass', not {mode!r}")
    rows, n = (int(a) for a in x.shape)
    y = torch.empty_like(x) if out is None else out
    _check_buffer("out", y, x.device, x.shape, x.dtype)
    if lse is None and return_lse:
        lse = torch.empty((rows,), dtype=torch.float32, device=x.device)
    elif lse is not None:
        _check_buffer("lse", lse, x.device, (rows,), torch.float32)
    rc = load_library().attn_softmax_rows(_ptr(x), _ptr(y), _ptr(lse), rows, n, float(scale),
                                          dtype_code(x.dtype), _SOFTMAX_MODES[mode],
                                          _stream(x, stream))
    if rc:
        raise AttnError("attn_softmax_rows", rc)
    return y, lse
