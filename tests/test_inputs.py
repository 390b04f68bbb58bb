"""The seeded input generator: determinism, shapes, storage types, and the
score statistics that §2.2 of the self-attention chapter predicts for i.i.d.
N(0,1) queries and keys (dot-product variance D_k, variance 1 after the
1/sqrt(D_k) scale)."""
import math

import numpy as np
import pytest
import torch

from scaled_dot_product_flashattention_amd.inputs import WORKLOADS, generate, poison_padding


def small(name, **kw):
    w = WORKLOADS[name]
    return w.replace(**{"B": 1, "H": 2, "Sq": min(w.Sq, 128), "Sk": min(w.Sk, 256), **kw})


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_shapes_types_and_determinism(name):
    w = small(name)
    a = generate(w)
    b = generate(w)
    for t in ("q", "k", "v"):
        assert a[t].dtype == {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[w.dtype]
        assert torch.equal(a[t].view(torch.uint8) if a[t].dtype != torch.float32 else a[t],
                           b[t].view(torch.uint8) if b[t].dtype != torch.float32 else b[t])
    assert tuple(a["q"].shape) == w.shape(w.Sq)
    assert tuple(a["k"].shape) == w.shape(w.Sk)
    if w.kv_len_range:
        lo, hi = w.kv_len_range
        assert a["kv_len"].dtype == torch.int32
        assert int(a["kv_len"].min()) >= lo and int(a["kv_len"].max()) <= hi
    else:
        assert a["kv_len"] is None
    c = generate(w, seed=w.seed + 100)
    assert not torch.equal(a["q"].float(), c["q"].float())


@pytest.mark.parametrize("name,expect", [("medium_bf16", 1.0), ("long_causal_bf16", 16.0),
                                         ("tiny_fp32", 1.0), ("bert_pad_fp16", 1.0)])
def test_score_variance(name, expect):
    """var(q.k) = d * mult^4 and var(scale * q.k) = mult^4 (mult = 2 gives 16),
    within 4 standard errors of the sample variance."""
    w = WORKLOADS[name].replace(B=1, H=1, Sq=256, Sk=256)
    t = generate(w)
    q = t["q"].double().reshape(-1, w.d)
    k = t["k"].double().reshape(-1, w.d)
    s = (q @ k.T).flatten()
    n = s.numel()
    var = float(s.var())
    # q rows are independent, so use the effective sample count of one row group
    se = expect * w.d * math.sqrt(2.0 / 256)
    assert abs(var - expect * w.d) < 4 * se, (var, expect * w.d)
    var_scaled = float((s * w.scale).var())
    assert abs(var_scaled - expect) < 4 * se / w.d
    assert n == 256 * 256


def test_poison_padding():
    w = small("bert_pad_fp16", B=3, kv_len_range=(100, 200))
    t = generate(w)
    k, v = t["k"].clone(), t["v"].clone()
    poison_padding(k, v, t["kv_len"], w.layout)
    for b, n in enumerate(t["kv_len"].tolist()):
        assert torch.isnan(k[b, :, n:, :]).all() and torch.isfinite(k[b, :, :n, :]).all()
        assert torch.isnan(v[b, :, n:, :]).all()
