"""GPU parity of the QKV projection (attn_qkv_proj) with the fp64 oracle on
seeded inputs, element by element.

Bar (derived from the arithmetic; the projection has no stated tolerance):
each output is an fp32-accumulated product rounded once to the storage type
(nearest even), so |out - exact| <= u * |exact| + a, with u the storage
type's unit roundoff (2^-8 bf16, 2^-11 fp16) and a = 1e-4 covering the fp32
accumulation over D <= 1024 terms of unit-scale products (about
D * 2^-24 * max|x_i w_i|). Runs on an MI355X only."""
import numpy as np
import pytest
import torch

import oracle
import scaled_dot_product_flashattention_amd as sdpa
from parity_util import say
from scaled_dot_product_flashattention_amd.inputs import generate_qkv_proj

pytestmark = pytest.mark.gpu

UNIT = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}
ABS = 1e-4


def check(got, want, dtype, what):
    g = got.float().cpu().numpy().astype(np.float64)
    err = np.abs(g - want)
    bound = UNIT[dtype] * np.abs(want) + ABS
    worst = float((err - bound).max())
    say(f"  {what}: max|d| = {err.max():.3e}, max(|d| - bound) = {worst:.3e}")
    assert not np.isnan(g).any(), f"{what}: NaN"
    assert (err <= bound).all(), f"{what}: {int((err > bound).sum())} elements beyond one rounding"


SHAPES = [  # (B, S, D, H, d): column tails, row tails, one and several K steps
    (1, 128, 64, 1, 64),
    (2, 200, 128, 2, 64),
    (1, 300, 256, 3, 64),
    (2, 77, 192, 2, 128),
    (3, 50, 64, 5, 8),
    # sequences shorter than the rows between one thread's stores: several
    # batches per step of the store loop
    (9, 7, 64, 2, 64),
    (40, 1, 128, 3, 32),
    (1, 512, 1024, 16, 64),
    # enough 128 x 192 tiles for two rounds over 256 CUs but one of 256 x 256:
    # the second tiling (exact fit, then row and column tails)
    (1, 4096, 64, 20, 64),
    (1, 4000, 128, 21, 64),
    (2, 2000, 64, 21, 64),  # a 256-row tile spans the two batches
]


@pytest.mark.parametrize("layout", ["bhsd", "bshd", "split:2"])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("shape", [s for s in SHAPES], ids=lambda s: "x".join(map(str, s)))
def test_qkv_proj_matches_oracle(shape, dtype, layout):
    B, S, D, H, d = shape
    if layout.startswith("split") and H % 2:
        layout = f"split:{H}"
    say(f"qkv_proj B{B} S{S} D{D} H{H} d{d} {dtype} {layout}")
    t = generate_qkv_proj(B, S, D, H, d, dtype, seed=B * 1000 + S + D + d)
    want = oracle.qkv_proj(t["x"], t["w"], H=H, d=d, layout=layout)
    got = sdpa.attn_qkv_proj(t["x"].cuda(), t["w"].cuda(), H=H, d=d, layout=layout)
    torch.cuda.synchronize()
    for name, g, wnt in zip("qkv", got, want):
        check(g, wnt, dtype, f"{name}")


def test_qkv_proj_shapes_cover_both_tilings():
    """The shapes above run both tilings of the projection on this GPU."""
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    used = {sdpa.attn_qkv_proj_tiling(B, S, H, d, n_cu) for B, S, D, H, d in SHAPES}
    say(f"tilings used on {n_cu} CUs: {sorted(used)}")
    assert used == {0, 1}


@pytest.mark.parametrize("layout", ["bhsd", "bshd"])
def test_qkv_proj_full_size(layout):
    """Medium width at full length (B1 S4096 D1024 H16 d64), every output
    element against the oracle."""
    B, S, D, H, d = 1, 4096, 1024, 16, 64
    t = generate_qkv_proj(B, S, D, H, d, "bf16", seed=7)
    got = sdpa.attn_qkv_proj(t["x"].cuda(), t["w"].cuda(), H=H, d=d, layout=layout)
    torch.cuda.synchronize()
    want = oracle.qkv_proj(t["x"], t["w"], H=H, d=d, layout=layout)
    for name, g, wnt in zip("qkv", got, want):
        check(g, wnt, "bf16", f"{name} full")


def test_qkv_proj_feeds_attention():
    """Projection output goes straight into attn_fwd: the attention of the
    projected tensors matches the oracle's attention of the oracle's
    projections rounded to the storage type."""
    B, S, D, H, d = 2, 256, 256, 4, 64
    t = generate_qkv_proj(B, S, D, H, d, "bf16", seed=9)
    q, k, v = sdpa.attn_qkv_proj(t["x"].cuda(), t["w"].cuda(), H=H, d=d, layout="bshd")
    o, lse = sdpa.attn_fwd(q, k, v, layout="bshd", causal=True)
    torch.cuda.synchronize()
    qr, kr, vr = (torch.from_numpy(a).to(torch.bfloat16)
                  for a in oracle.qkv_proj(t["x"], t["w"], H=H, d=d, layout="bshd"))
    # the projections themselves are within one rounding, so compare attention
    # on the GPU's own projections (exact inputs for both sides)
    o_ref, lse_ref = oracle.attention(q.cpu(), k.cpu(), v.cpu(), layout="bshd", causal=True)
    err = np.abs(o.float().cpu().numpy() - o_ref).max()
    say(f"  attention of the projections: max|dO| = {err:.3e}")
    assert err <= 2e-2
    # and the projections agree with the oracle's rounded ones to one bf16 step
    for g, r in zip((q, k, v), (qr, kr, vr)):
        assert (g.cpu().float() - r.float()).abs().max().item() <= 2.0 ** -7 * max(1.0, r.float().abs().max().item())
