"""GPU parity of the fused path (attn_fwd) with the fp64 oracle on seeded
inputs: the five workloads at oracle-friendly sizes (whole outputs), an edge
grid of shapes, masks, layouts and types, and the workloads at full size
(every row). Runs on an MI355X only."""
import numpy as np
import pytest
import torch

from parity_util import full_case, full_size_case, say
from scaled_dot_product_flashattention_amd.inputs import WORKLOADS

pytestmark = pytest.mark.gpu

W = WORKLOADS


# the five workloads, shrunk where the oracle would take long, keeping several
# tiles and a ragged tail
REDUCED = {
    "tiny_fp32": W["tiny_fp32"],
    "medium_bf16": W["medium_bf16"].replace(H=2, Sq=1000, Sk=1000),
    "long_causal_bf16": W["long_causal_bf16"].replace(B=2, H=2, Sq=700, Sk=700),
    "bert_pad_fp16": W["bert_pad_fp16"].replace(B=4, H=3),
    "decode_bf16": W["decode_bf16"].replace(B=2, H=3, Sk=5000),
}


@pytest.mark.parametrize("name", sorted(REDUCED))
def test_workload_reduced(name):
    full_case(REDUCED[name], poison=REDUCED[name].kv_len_range is not None)


EDGE = []
for (Sq, Sk) in [(1, 1), (1, 7), (7, 1), (63, 64), (64, 63), (65, 65), (129, 1000), (1000, 129),
                 (127, 129), (200, 64), (300, 513)]:
    for d in (64, 128):
        EDGE.append((Sq, Sk, d))


@pytest.mark.parametrize("Sq,Sk,d", EDGE)
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_edge_shapes(Sq, Sk, d, dtype):
    rng = np.random.default_rng(Sq * 1000 + Sk + d)
    causal = bool(rng.integers(0, 2))
    layout = ["bhsd", "bshd"][int(rng.integers(0, 2))]
    w = W["medium_bf16"].replace(name=f"edge_{Sq}_{Sk}_{d}", B=2, H=3, Sq=Sq, Sk=Sk, d=d,
                                 dtype=dtype, layout=layout, causal=causal,
                                 seed=int(rng.integers(0, 1 << 30)))
    full_case(w)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("layout", ["bhsd", "bshd"])
@pytest.mark.parametrize("d", [64, 128])
def test_padding_with_nan_poison(causal, layout, d):
    """Keys/values past each sequence's length are NaN; none may be read.
    Lengths include 0 (empty rows: O = 0, LSE = -inf) and non-multiples of
    the tile."""
    w = W["bert_pad_fp16"].replace(name="pad", B=6, H=2, Sq=200, Sk=300, d=d, layout=layout,
                                   causal=causal, kv_len_range=(0, 300), seed=77 + d)
    full_case(w, poison=True)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_scale_zero_is_uniform(dtype):
    w = W["medium_bf16"].replace(name="scale0", B=1, H=2, Sq=130, Sk=257, dtype=dtype)
    full_case(w, scale=0.0)


def test_qk_stress_scale():
    """Large scores (q, k x 4): the running max moves a lot across tiles."""
    w = W["long_causal_bf16"].replace(name="stress", B=1, H=2, Sq=400, Sk=400, qk_mult=4.0)
    full_case(w)


def test_determinism():
    import scaled_dot_product_flashattention_amd as sdpa
    from scaled_dot_product_flashattention_amd.inputs import generate
    w = W["medium_bf16"].replace(H=4, Sq=1024, Sk=1024)
    t = generate(w)
    q, k, v = (t[n].cuda() for n in ("q", "k", "v"))
    o1, l1 = sdpa.attn_fwd(q, k, v, layout=w.layout)
    o2, l2 = sdpa.attn_fwd(q, k, v, layout=w.layout)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["medium_bf16", "long_causal_bf16", "bert_pad_fp16", "decode_bf16"])
def test_workload_full_size(name):
    """Each workload at its full size, every output row against the oracle
    (the long causal one takes the oracle about a minute on 16 threads)."""
    full_size_case(W[name], poison=W[name].kv_len_range is not None)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("layout,causal,pad", [("bhsd", False, False), ("bshd", True, False),
                                               ("bhsd", True, True), ("bshd", False, True)])
def test_long_keys_head64(dtype, layout, causal, pad):
    """Head size 64 over >= 2048 keys (the 8-wave kernel), ragged lengths."""
    w = W["medium_bf16"].replace(name="long64", B=2 if pad else 1, H=2, Sq=2100, Sk=2300,
                                 dtype=dtype, layout=layout, causal=causal,
                                 kv_len_range=(1500, 2300) if pad else None, seed=31)
    full_case(w, poison=pad)


@pytest.mark.parametrize("g", [1, 2, 4])
@pytest.mark.parametrize("dtype,d,Sk", [("bf16", 64, 300), ("bf16", 64, 2200), ("f16", 128, 300),
                                         ("f32", 64, 200)])
def test_split_layout(g, dtype, d, Sk):
    """The page's head-group layout [B, H/g, S, g, d] (ATTN_LAYOUT_SPLIT(g)),
    with padding and causal rows, on every kernel shape (4-wave and 8-wave
    16-bit, fp32)."""
    w = W["medium_bf16"].replace(name=f"split{g}", B=2, H=4, Sq=Sk if Sk < 1000 else 260, Sk=Sk,
                                 d=d, dtype=dtype, layout=f"split:{g}", causal=(g == 2),
                                 kv_len_range=(Sk // 2, Sk), seed=50 + g)
    full_case(w, poison=True)


@pytest.mark.parametrize("path", ["splitk", "naive"])
def test_split_layout_other_paths(path):
    w = W["decode_bf16"].replace(name="split_dec", B=2, H=4, Sq=1 if path == "splitk" else 100,
                                 Sk=3000, layout="split:2", seed=61)
    full_case(w, path=path, n_split=6 if path == "splitk" else None)


def test_split_layout_full_size():
    """Medium prefill shape (B1 H16 S4096 d64 bf16) in groups of 4 heads, at
    full size, every row."""
    full_size_case(W["medium_bf16"].replace(name="medium_split4", layout="split:4"))


def test_binding_rejects_bad_buffers():
    """Host-side rejection of buffers that would send a kernel a wrong address
    or size: nothing is launched for any of these calls."""
    import scaled_dot_product_flashattention_amd as sdpa
    from scaled_dot_product_flashattention_amd.inputs import generate
    w = W["medium_bf16"].replace(H=2, Sq=64, Sk=64)
    t = generate(w)
    q, k, v = (t[n].cuda() for n in ("q", "k", "v"))
    bad = [dict(lse=torch.empty(1, 2, 64)),                                  # host LSE
           dict(lse=torch.empty(1, 2, 63, device="cuda")),                   # short LSE
           dict(lse=torch.empty(1, 2, 64, device="cuda", dtype=torch.float16)),
           dict(out=torch.empty_like(q).cpu()),                              # host output
           dict(workspace=torch.empty(1 << 20, dtype=torch.uint8))]          # host workspace
    for kw in bad:
        with pytest.raises(ValueError):
            sdpa.attn_fwd(q, k, v, **kw)
    with pytest.raises(ValueError):
        sdpa.attn_softmax_rows(q.view(-1, 64), lse=torch.empty(5, device="cuda"))
    with pytest.raises(ValueError):
        sdpa.attn_softmax_rows(q.view(-1, 64), mode="two_pass")


# Causal grids with B*H a multiple of 8 and small K/V: the fused kernel runs
# the query tiles of each XCD's heads interleaved, longest first, in place of
# head by head. Every tile variant, ragged query tiles, Sq != Sk.
CAUSAL_MIX = [(d, t, shape) for d, n in ((64, 5), (128, 4)) for t in range(n)
              for shape in ((2, 4, 700, 700, "bhsd", "bf16"), (1, 8, 300, 900, "bshd", "f16"))]


@pytest.mark.parametrize("d,tile,shape", CAUSAL_MIX)
def test_causal_interleaved_heads(d, tile, shape):
    B, H, Sq, Sk, layout, dtype = shape
    w = W["long_causal_bf16"].replace(name=f"causal_mix_{B}x{H}_{Sq}_{Sk}_d{d}_t{tile}", B=B, H=H,
                                      Sq=Sq, Sk=Sk, d=d, layout=layout, dtype=dtype,
                                      seed=4000 + 10 * d + tile)
    full_case(w, path=f"tile:{tile}:1")
