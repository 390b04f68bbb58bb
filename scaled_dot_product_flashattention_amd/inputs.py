"""Seeded synthetic inputs shared by the GPU path's tests, the oracle's tests
and the benchmark.

This module draws random numbers and casts them to the storage dtype; it holds
none of the attention arithmetic. Recipe (the pages fix no seeds or
distributions beyond the shapes):

* ``numpy.random.default_rng(seed)`` (PCG64, stable across numpy versions);
* ``standard_normal(shape, dtype=float32)`` in the storage order of the
  layout, drawn in the order q, k, v, then the per-sequence key lengths;
* an optional float32 multiplier on q and k (the long causal workload uses
  2.0 to widen the score spread);
* per-sequence key lengths ``rng.integers(lo, hi + 1, size=B)`` when the
  workload pads keys;
* optionally a score offset: column 0 of q is set to 8 and column 0 of key j
  to o_j / (8 * scale), so that every row's scaled scores gain o_j, which
  runs linearly from ``score_shift[0]`` at the first key to
  ``score_shift[1]`` at the last (natural-log units; softmax ignores a
  common offset, so this probes the kernels' handling of very low or rising
  scores);
* a round-to-nearest-even cast to the storage dtype with torch ``.to``.

The oracle and the GPU path read exactly these quantised tensors.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    Sq: int
    Sk: int
    d: int
    dtype: str            # "f32" | "f16" | "bf16"
    layout: str           # "bhsd" | "bshd" | "split:g"
    causal: bool = False
    qk_mult: float = 1.0  # multiplier applied to q and k before the cast
    kv_len_range: tuple[int, int] | None = None  # inclusive range of valid key counts
    # offset of the scaled scores at the first and the last key (see above)
    score_shift: tuple[float, float] | None = None
    seed: int = 0
    description: str = ""

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def shape(self, S: int) -> tuple:
        if self.layout == "bhsd":
            return (self.B, self.H, S, self.d)
        if self.layout == "bshd":
            return (self.B, S, self.H, self.d)
        g = int(self.layout.split(":")[1])  # "split:g": heads in groups of g
        return (self.B, self.H // g, S, g, self.d)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads of the fused-forward study. The medium prefill shape is
# the B=1, h=16, S=4096, D=1024 example of the memory table in §2.5 of the
# self-attention chapter (d = 1024 / 16 = 64).
WORKLOADS: dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("tiny_fp32", B=1, H=2, Sq=256, Sk=256, d=64, dtype="f32", layout="bhsd", seed=0,
                 description="tiny non-causal fp32, B1 H2 S256 d64, [B,H,S,d]"),
        Workload("medium_bf16", B=1, H=16, Sq=4096, Sk=4096, d=64, dtype="bf16", layout="bhsd",
                 seed=1, description="medium prefill bf16, B1 H16 S4096 d64, [B,H,S,d], LSE out"),
        Workload("long_causal_bf16", B=2, H=16, Sq=8192, Sk=8192, d=128, dtype="bf16",
                 layout="bshd", causal=True, qk_mult=2.0, seed=2,
                 description="long causal prefill bf16, B2 H16 S8192 d128, [B,S,H,d], q,k x2.0"),
        Workload("bert_pad_fp16", B=32, H=12, Sq=512, Sk=512, d=64, dtype="f16", layout="bhsd",
                 kv_len_range=(256, 512), seed=3,
                 description="batched short fp16, B32 H12 S512 d64, key padding 256..512"),
        Workload("decode_bf16", B=8, H=32, Sq=1, Sk=32768, d=128, dtype="bf16", layout="bhsd",
                 seed=4, description="single-query decode bf16, B8 H32 Sq1 Sk32768 d128, split-K"),
    ]
}


def generate(w: Workload, seed: int | None = None) -> dict:
    """Draw q, k, v (torch CPU tensors in w.dtype and w.layout) and kv_len
    (torch int32 [B] or None) for workload ``w``."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    tdt = DTYPES[w.dtype]
    out = {}
    for name, S in (("q", w.Sq), ("k", w.Sk), ("v", w.Sk)):
        a = rng.standard_normal(w.shape(S), dtype=np.float32)
        if name in ("q", "k") and w.qk_mult != 1.0:
            a *= np.float32(w.qk_mult)
        out[name] = torch.from_numpy(a).to(tdt)
        del a
    if w.kv_len_range is not None:
        lo, hi = w.kv_len_range
        out["kv_len"] = torch.from_numpy(rng.integers(lo, hi + 1, size=w.B).astype(np.int32))
    else:
        out["kv_len"] = None
    if w.score_shift is not None:
        _shift_scores(out["q"], out["k"], w)
    return out


def _key_axis(layout: str) -> int:
    return 1 if layout == "bshd" else 2


def _shift_scores(q: torch.Tensor, k: torch.Tensor, w: Workload) -> None:
    """Column 0 of q := 8 and column 0 of key j := o_j / (8 * scale), in place
    (o_j linear from score_shift[0] to score_shift[1] over the keys)."""
    lo, hi = w.score_shift
    ramp = np.linspace(lo, hi, w.Sk, dtype=np.float64) / (8.0 * w.scale)
    shape = [1] * k.dim()
    shape[_key_axis(w.layout)] = w.Sk
    q[..., 0] = 8.0
    k[..., 0] = torch.from_numpy(ramp.astype(np.float32)).reshape(shape[:-1]).to(k.dtype)


def generate_periodic_keys(w: Workload, period: int, seed: int | None = None) -> dict:
    """Like ``generate`` but K and V repeat a random block of ``period`` key
    rows along the sequence (key j is block row j mod period), so very long
    key ranges cost one block of random draws. q is drawn in full. A prime
    period keeps any offset error of a power-of-two size from landing on an
    identical key. [B,S,H,d] layout only."""
    if w.layout != "bshd":
        raise ValueError("periodic keys are drawn for the [B,S,H,d] layout")
    rng = np.random.default_rng(w.seed if seed is None else seed)
    tdt = DTYPES[w.dtype]
    out = {"q": torch.from_numpy(rng.standard_normal(w.shape(w.Sq), dtype=np.float32)).to(tdt)}
    reps = -(-w.Sk // period)
    for name in ("k", "v"):
        block = torch.from_numpy(rng.standard_normal((w.B, period, w.H, w.d), dtype=np.float32)).to(tdt)
        out[name] = block.repeat(1, reps, 1, 1)[:, :w.Sk].contiguous()
        del block
    if w.kv_len_range is not None:
        lo, hi = w.kv_len_range
        out["kv_len"] = torch.from_numpy(rng.integers(lo, hi + 1, size=w.B).astype(np.int32))
    else:
        out["kv_len"] = None
    return out


def generate_qkv_proj(B: int, S: int, D: int, H: int, d: int, dtype: str, seed: int) -> dict:
    """Tokens x [B, S, D] ~ N(0, 1) and an out-major weight w [3*H*d, D] ~
    N(0, 1/D) (a standard linear-layer initialisation: outputs of unit scale),
    drawn in that order in float32 and cast to ``dtype`` (torch CPU tensors)."""
    rng = np.random.default_rng(seed)
    tdt = DTYPES[dtype]
    x = rng.standard_normal((B, S, D), dtype=np.float32)
    w = rng.standard_normal((3 * H * d, D), dtype=np.float32) * np.float32(1.0 / np.sqrt(D))
    return {"x": torch.from_numpy(x).to(tdt), "w": torch.from_numpy(w).to(tdt)}


def generate_softmax_rows(rows: int, n: int, dtype: str, seed: int, std: float = 2.0) -> torch.Tensor:
    """Score-like rows x [rows, n] ~ N(0, std^2) in float32, cast to ``dtype``
    (torch CPU tensor)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, n), dtype=np.float32) * np.float32(std)
    return torch.from_numpy(x).to(DTYPES[dtype])


def poison_padding(k: torch.Tensor, v: torch.Tensor, kv_len, layout: str) -> None:
    """Fill the key/value rows at or beyond each sequence's valid length with
    NaN, in place, so that any read of them shows up in the output."""
    if kv_len is None:
        return
    for b, n in enumerate(torch.as_tensor(kv_len).tolist()):
        if layout == "bshd":
            k[b, n:] = float("nan")
            v[b, n:] = float("nan")
        else:  # [B, H, S, d] or [B, H/g, S, g, d]: rows are the third index
            k[b, :, n:] = float("nan")
            v[b, :, n:] = float("nan")
