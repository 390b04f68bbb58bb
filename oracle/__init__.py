"""Scaled-dot-product attention oracle (fp64, CPU).

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the
benchmark's CPU-baseline leg are the only callers. The GPU library never loads
this module and shares no code with it.

This wrapper only marshals arguments to ``liboracle_attn.so`` (built from
``attn_oracle.c`` next to this file, plain C in fp64). The arithmetic, with
its citations of the pages, is in that C file:

* scores, scale, three-step softmax, weighted sum: chapter
  "2. 自注意力机制算子：QKV投影、注意力分数计算、Softmax、加权求和，以及FlashAttention优化",
  §2.2-§2.4;
* the per-element online recurrence: page "[Performance] [WebGPU] Proposal:
  Add an option to use online softmax instead of naive softmax", §四;
* the (m, l) block merge: page "WebGPU 算子优化：QKV 内存合并与 FlashAttention
  分块计算", section "FlashAttention 分块计算原理与浏览器适配";
* the QKV projection against the concatenated weight: the chapter's §2.1;
* the softmax of rows on their own: the chapter's §2.3 steps, as the online
  softmax page's §三-§四 treat it.

Inputs are torch CPU tensors (float32, float16, bfloat16) or numpy arrays
(float32, float16) in layout "bhsd" = [B, H, S, d], "bshd" = [B, S, H, d] or
"split:g" = [B, H/g, S, g, d].
Outputs are float64 numpy arrays: O in the layout of q, LSE as [B, H, Sq].
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np

from .build import build as _build, library_path

_DTYPE_CODES = {"f32": 0, "f16": 1, "bf16": 2}
_LAYOUT_CODES = {"bhsd": 0, "bshd": 1}


def layout_code(layout: str) -> int:
    """"bhsd" = [B,H,S,d], "bshd" = [B,S,H,d], "split:g" = [B,H/g,S,g,d]."""
    if layout in _LAYOUT_CODES:
        return _LAYOUT_CODES[layout]
    if layout.startswith("split:"):
        return 0x10000 | int(layout[6:])
    raise ValueError(f"unknown layout {layout!r}")


def layout_shape(layout: str, B: int, H: int, S: int, d: int) -> tuple:
    if layout == "bhsd":
        return (B, H, S, d)
    if layout == "bshd":
        return (B, S, H, d)
    g = layout_code(layout) & 0xffff
    return (B, H // g, S, g, d)

def host_threads() -> int:
    """Threads the oracle uses by default: OMP_NUM_THREADS when set (a shared
    machine sets it to the CPUs it allots to the job), else every CPU this
    process may run on."""
    env = os.environ.get("OMP_NUM_THREADS", "").strip()
    if env.isdigit() and int(env) > 0:
        return int(env)
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


_c_i64 = ctypes.c_int64
_c_int = ctypes.c_int
_c_dbl = ctypes.c_double
_c_vp = ctypes.c_void_p


class Oracle:
    """Handle on one build of the oracle library (the default one, or a
    variant built from edited source by the mutation tests)."""

    def __init__(self, path: str | None = None):
        if path is None:
            path = library_path()
            if not os.path.exists(path):
                _build()
        self.path = path
        lib = ctypes.CDLL(path)
        common = [_c_vp, _c_vp, _c_vp, _c_int, _c_int, _c_i64, _c_i64, _c_i64, _c_i64,
                  _c_i64, _c_dbl, _c_int, _c_vp]
        lib.oracle_attn.argtypes = common + [_c_vp, _c_vp, _c_int]
        lib.oracle_attn.restype = _c_int
        lib.oracle_attn_rows.argtypes = common + [_c_vp, _c_i64, _c_vp, _c_vp, _c_int]
        lib.oracle_attn_rows.restype = _c_int
        lib.oracle_partial.argtypes = common + [_c_i64, _c_i64, _c_i64, _c_vp, _c_vp, _c_vp]
        lib.oracle_partial.restype = _c_int
        lib.oracle_online_softmax.argtypes = [_c_vp, _c_i64, _c_vp, _c_vp, _c_vp]
        lib.oracle_online_softmax.restype = None
        lib.oracle_merge.argtypes = [_c_i64, _c_vp, _c_vp, _c_vp, _c_i64, _c_vp, _c_vp]
        lib.oracle_merge.restype = None
        lib.oracle_qkv_proj.argtypes = [_c_vp, _c_vp, _c_int, _c_int, _c_i64, _c_i64, _c_i64,
                                        _c_i64, _c_i64, _c_vp, _c_vp, _c_vp, _c_int]
        lib.oracle_qkv_proj.restype = _c_int
        lib.oracle_softmax_rows.argtypes = [_c_vp, _c_int, _c_i64, _c_i64, _c_dbl, _c_vp, _c_vp,
                                            _c_int]
        lib.oracle_softmax_rows.restype = _c_int
        lib.oracle_decode.argtypes = [_c_vp, _c_i64, _c_int]
        lib.oracle_decode.restype = _c_dbl
        self.lib = lib

    # -- argument marshalling ------------------------------------------------
    @staticmethod
    def _buffer(x):
        """Return (keep-alive object, pointer, dtype code) for a tensor/array."""
        try:
            import torch
        except ImportError:  # pragma: no cover
            torch = None
        if torch is not None and isinstance(x, torch.Tensor):
            if x.device.type != "cpu":
                raise ValueError("the oracle reads host memory: pass CPU tensors")
            x = x.contiguous()
            code = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}.get(x.dtype)
            if code is None:
                raise TypeError(f"unsupported dtype {x.dtype}")
            return x, x.data_ptr(), _DTYPE_CODES[code]
        a = np.ascontiguousarray(x)
        code = {np.dtype(np.float32): "f32", np.dtype(np.float16): "f16"}.get(a.dtype)
        if code is None:
            raise TypeError(f"unsupported dtype {a.dtype}")
        return a, a.ctypes.data, _DTYPE_CODES[code]

    @staticmethod
    def _dims(q, k, layout):
        if layout == "bhsd":
            B, H, Sq, d = q.shape
            Sk = k.shape[2]
        elif layout == "bshd":
            B, Sq, H, d = q.shape
            Sk = k.shape[1]
        elif layout.startswith("split:"):
            B, G, Sq, g, d = q.shape
            H, Sk = G * g, k.shape[2]
        else:
            raise ValueError(f"unknown layout {layout!r}")
        return int(B), int(H), int(Sq), int(Sk), int(d)

    def _common(self, q, k, v, scale, causal, layout, kv_len):
        B, H, Sq, Sk, d = self._dims(q, k, layout)
        if tuple(k.shape) != tuple(v.shape):
            raise ValueError("k and v must have the same shape")
        if scale is None:
            scale = 1.0 / math.sqrt(d)
        qa, qp, qc = self._buffer(q)
        ka, kp, kc = self._buffer(k)
        va, vp, vc = self._buffer(v)
        if not (qc == kc == vc):
            raise TypeError("q, k and v must share one dtype")
        keep = [qa, ka, va]
        lp = None
        if kv_len is not None:
            try:
                import torch
                if isinstance(kv_len, torch.Tensor):
                    kv_len = kv_len.cpu().numpy()
            except ImportError:  # pragma: no cover
                pass
            la = np.ascontiguousarray(np.asarray(kv_len, dtype=np.int32))
            if la.shape != (B,):
                raise ValueError("kv_len must have shape [B]")
            keep.append(la)
            lp = la.ctypes.data
        args = [qp, kp, vp, qc, layout_code(layout), B, H, Sq, Sk, d, float(scale),
                int(bool(causal)), lp]
        return keep, args, (B, H, Sq, Sk, d)

    @staticmethod
    def _threads(nthreads):
        return int(nthreads) if nthreads else host_threads()

    # -- entry points --------------------------------------------------------
    def attention(self, q, k, v, *, scale=None, causal=False, layout="bhsd", kv_len=None,
                  nthreads=None):
        """Full attention by definition. Returns (O float64 in q's layout, LSE [B,H,Sq])."""
        keep, args, (B, H, Sq, Sk, d) = self._common(q, k, v, scale, causal, layout, kv_len)
        o = np.empty(tuple(q.shape), dtype=np.float64)
        lse = np.empty((B, H, Sq), dtype=np.float64)
        rc = self.lib.oracle_attn(*args, o.ctypes.data, lse.ctypes.data, self._threads(nthreads))
        if rc:
            raise RuntimeError(f"oracle_attn failed with code {rc}")
        del keep
        return o, lse

    def attention_rows(self, q, k, v, rows, *, scale=None, causal=False, layout="bhsd",
                       kv_len=None, nthreads=None):
        """Selected rows, row = (b*H + h)*Sq + i. Returns (O [n, d], LSE [n])."""
        keep, args, (B, H, Sq, Sk, d) = self._common(q, k, v, scale, causal, layout, kv_len)
        r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        o = np.empty((r.size, d), dtype=np.float64)
        lse = np.empty((r.size,), dtype=np.float64)
        rc = self.lib.oracle_attn_rows(*args, r.ctypes.data, r.size, o.ctypes.data,
                                       lse.ctypes.data, self._threads(nthreads))
        if rc:
            raise RuntimeError(f"oracle_attn_rows failed with code {rc}")
        del keep
        return o, lse

    def partial(self, q, k, v, row, j0, j1, *, scale=None, causal=False, layout="bhsd",
                kv_len=None):
        """Unnormalised partial (m, l, o[d]) of one row over keys [j0, j1)."""
        keep, args, (B, H, Sq, Sk, d) = self._common(q, k, v, scale, causal, layout, kv_len)
        m = ctypes.c_double()
        l = ctypes.c_double()
        o = np.empty((d,), dtype=np.float64)
        rc = self.lib.oracle_partial(*args, int(row), int(j0), int(j1), ctypes.addressof(m),
                                     ctypes.addressof(l), o.ctypes.data)
        if rc:
            raise RuntimeError(f"oracle_partial failed with code {rc}")
        del keep
        return m.value, l.value, o

    def merge(self, m, l, o):
        """Merge partials: m[n], l[n], o[n, d] -> (O[d], LSE)."""
        m = np.ascontiguousarray(np.asarray(m, dtype=np.float64))
        l = np.ascontiguousarray(np.asarray(l, dtype=np.float64))
        o = np.ascontiguousarray(np.asarray(o, dtype=np.float64))
        n, d = o.shape
        out = np.empty((d,), dtype=np.float64)
        lse = ctypes.c_double()
        self.lib.oracle_merge(n, m.ctypes.data, l.ctypes.data, o.ctypes.data, d, out.ctypes.data,
                              ctypes.addressof(lse))
        return out, lse.value

    def online_softmax(self, s):
        """Per-element online recurrence. Returns (m_trace, l_trace, p)."""
        s = np.ascontiguousarray(np.asarray(s, dtype=np.float64))
        n = s.size
        mt = np.empty(n)
        lt = np.empty(n)
        p = np.empty(n)
        self.lib.oracle_online_softmax(s.ctypes.data, n, mt.ctypes.data, lt.ctypes.data,
                                       p.ctypes.data)
        return mt, lt, p

    def qkv_proj(self, x, w, *, H, d, layout="bhsd", nthreads=None):
        """QKV projection by definition: x [B, S, D], w [3*H*d, D] (out-major).
        Returns (q, k, v) float64 in `layout` ([B,H,S,d] or [B,S,H,d])."""
        B, S, D = (int(n) for n in x.shape)
        if tuple(w.shape) != (3 * H * d, D):
            raise ValueError(f"w must have shape [3*H*d, D] = {(3 * H * d, D)}")
        xa, xp, xc = self._buffer(x)
        wa, wp, wc = self._buffer(w)
        if xc != wc:
            raise TypeError("x and w must share one dtype")
        shape = layout_shape(layout, B, H, S, d)
        outs = [np.empty(shape, dtype=np.float64) for _ in range(3)]
        rc = self.lib.oracle_qkv_proj(xp, wp, xc, layout_code(layout), B, S, D, H, d,
                                      *(o.ctypes.data for o in outs), self._threads(nthreads))
        if rc:
            raise RuntimeError(f"oracle_qkv_proj failed with code {rc}")
        del xa, wa
        return tuple(outs)

    def softmax_rows(self, x, *, scale=1.0, nthreads=None):
        """Row softmax of x [rows, n] by definition. Returns (y [rows, n],
        lse [rows]) as float64."""
        rows, n = (int(a) for a in x.shape)
        xa, xp, xc = self._buffer(x)
        y = np.empty((rows, n), dtype=np.float64)
        lse = np.empty((rows,), dtype=np.float64)
        rc = self.lib.oracle_softmax_rows(xp, xc, rows, n, float(scale), y.ctypes.data,
                                          lse.ctypes.data, self._threads(nthreads))
        if rc:
            raise RuntimeError(f"oracle_softmax_rows failed with code {rc}")
        del xa
        return y, lse

    def decode(self, x):
        """Every element of x decoded to float64 by the oracle's own reader."""
        keep, ptr, code = self._buffer(x)
        n = int(np.prod(tuple(x.shape)))
        out = np.empty(n, dtype=np.float64)
        for i in range(n):
            out[i] = self.lib.oracle_decode(ptr, i, code)
        del keep
        return out.reshape(tuple(x.shape))


_default: Oracle | None = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def attention(*a, **kw):
    return default().attention(*a, **kw)


def attention_rows(*a, **kw):
    return default().attention_rows(*a, **kw)


def partial(*a, **kw):
    return default().partial(*a, **kw)


def merge(*a, **kw):
    return default().merge(*a, **kw)


def online_softmax(*a, **kw):
    return default().online_softmax(*a, **kw)


def decode(*a, **kw):
    return default().decode(*a, **kw)


def qkv_proj(*a, **kw):
    return default().qkv_proj(*a, **kw)


def softmax_rows(*a, **kw):
    return default().softmax_rows(*a, **kw)
