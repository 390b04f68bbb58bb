"""Seeded random shapes on every path, element by element against the fp64
oracle: batch, heads, query and key lengths (1..700), head size, type,
layout (including head groups), causal mask, key padding with NaN-poisoned
rows past the length, and, for the fused kernel, a random tile variant.
The cases come from one fixed seed, so a failure names a reproducible case.
Runs on an MI355X only."""
import numpy as np
import pytest

from parity_util import full_case
from scaled_dot_product_flashattention_amd.inputs import WORKLOADS

pytestmark = pytest.mark.gpu

N_TILES = {64: 6, 128: 4}


def cases(n=128, seed=20261202):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        B = int(rng.integers(1, 4))
        H = int(rng.choice([1, 2, 3, 4, 6]))
        Sq = int(rng.integers(1, 701))
        Sk = int(rng.integers(1, 701))
        d = int(rng.choice([64, 128]))
        dtype = str(rng.choice(["bf16", "f16", "f32"]))
        groups = [g for g in (1, 2, 3, 6) if H % g == 0]
        layout = str(rng.choice(["bhsd", "bshd"] + [f"split:{g}" for g in groups]))
        causal = bool(rng.integers(0, 2))
        pad = None
        if rng.integers(0, 2):
            lo = int(rng.integers(0, Sk + 1))
            pad = (lo, Sk)
        path = str(rng.choice(["fused", "tile", "naive", "splitk"]))
        if path == "tile" and dtype == "f32":
            path = "fused"
        tile = int(rng.integers(0, N_TILES[d])) if path == "tile" else None
        n_split = int(rng.integers(1, 9)) if path == "splitk" else None
        out.append((i, B, H, Sq, Sk, d, dtype, layout, causal, pad, path, tile, n_split))
    return out


@pytest.mark.parametrize("case", cases(), ids=lambda c: f"case{c[0]}")
def test_random_shape(case):
    i, B, H, Sq, Sk, d, dtype, layout, causal, pad, path, tile, n_split = case
    w = WORKLOADS["medium_bf16"].replace(name=f"random{i}", B=B, H=H, Sq=Sq, Sk=Sk, d=d, dtype=dtype,
                                         layout=layout, causal=causal, kv_len_range=pad, seed=900 + i)
    p = f"tile:{tile}" if path == "tile" else path
    full_case(w, path=p, n_split=n_split, poison=pad is not None)
