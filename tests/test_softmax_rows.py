"""GPU parity of the row softmax (attn_softmax_rows, online and three-pass)
with the fp64 oracle, and the online page's equality guard between the two
forms (page "[Performance] [WebGPU] Proposal: Add an option to use online
softmax instead of naive softmax", §七: the two agree to 1e-3).

Bar (derived from the arithmetic): y is computed in fp32 with base-2
exponentials and rounded once, so |y - exact| <= u*|y| + 1e-6 with u the
storage type's unit roundoff (2^-8 bf16, 2^-11 fp16) or 2^-16 for fp32
(covering the fp32 exponent and the fp32 row sum over <= 2^17 terms);
lse within 1e-5 * max(1, |lse|). Runs on an MI355X only."""
import numpy as np
import pytest
import torch

import oracle
import scaled_dot_product_flashattention_amd as sdpa
from parity_util import say
from scaled_dot_product_flashattention_amd.inputs import generate_softmax_rows

pytestmark = pytest.mark.gpu

UNIT = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11, "f32": 2.0 ** -16}


def check(y, lse, y_ref, lse_ref, dtype, what):
    g = y.float().cpu().numpy().astype(np.float64)
    err = np.abs(g - y_ref)
    bound = UNIT[dtype] * np.abs(y_ref) + 1e-6
    say(f"  {what}: max|dy| = {err.max():.3e}")
    assert not np.isnan(g).any(), f"{what}: NaN"
    assert (err <= bound).all(), f"{what}: {int((err > bound).sum())} elements beyond the bar"
    lg = lse.cpu().numpy().astype(np.float64)
    both = np.isneginf(lg) & np.isneginf(lse_ref)
    with np.errstate(invalid="ignore"):
        dl = np.where(both, 0.0, np.abs(lg - lse_ref))
    assert (dl <= 1e-5 * np.maximum(1.0, np.abs(np.where(both, 0.0, lse_ref)))).all(), \
        f"{what}: lse off by {np.nanmax(dl):.3e}"


CASES = [  # rows, n: a chunk, a few, one full register load, the most, streamed
    (3, 8), (5, 64), (7, 1000 - 1000 % 8), (4, 4096), (3, 32768), (2, 40000), (2, 65536),
    # the edges of 4 rows per wave (<= 512), 2 rows per wave (<= 1024) and one
    (37, 512), (37, 520), (19, 1024), (19, 1032),
]


@pytest.mark.parametrize("mode", ["online", "three_pass"])
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("rows,n", CASES)
def test_softmax_rows_matches_oracle(rows, n, dtype, mode):
    if dtype == "f32" and n % 4:
        pytest.skip("fp32 rows are multiples of 4")
    say(f"softmax_rows rows{rows} n{n} {dtype} {mode}")
    x = generate_softmax_rows(rows, n, dtype, seed=rows * 100000 + n)
    y_ref, lse_ref = oracle.softmax_rows(x, scale=0.7)
    y, lse = sdpa.attn_softmax_rows(x.cuda(), scale=0.7, mode=mode)
    torch.cuda.synchronize()
    check(y, lse, y_ref, lse_ref, dtype, f"{mode} {dtype}")


@pytest.mark.parametrize("mode", ["online", "three_pass"])
def test_softmax_rows_masked_and_scale_zero(mode):
    """-inf entries get probability 0, an all -inf row gives 0 and -inf, and
    scale 0 gives uniform rows over the finite entries."""
    x = generate_softmax_rows(4, 4096, "bf16", seed=11)
    x[0, 100:] = float("-inf")
    x[1, :] = float("-inf")
    x[2, ::2] = float("-inf")
    for scale in (1.0, 0.0):
        y_ref, lse_ref = oracle.softmax_rows(x, scale=scale)
        y, lse = sdpa.attn_softmax_rows(x.cuda(), scale=scale, mode=mode)
        torch.cuda.synchronize()
        check(y, lse, y_ref, lse_ref, "bf16", f"{mode} masked scale {scale}")


@pytest.mark.parametrize("mode", ["online", "three_pass"])
@pytest.mark.parametrize("n", [512, 1024])
def test_short_rows_masked(mode, n):
    """Rows held several to a wave: masked entries, an all -inf row between
    live ones, and a row count that leaves the last wave partly empty."""
    x = generate_softmax_rows(23, n, "bf16", seed=n + 3)
    x[0, 100:] = float("-inf")
    x[5, :] = float("-inf")
    x[6, ::3] = float("-inf")
    y_ref, lse_ref = oracle.softmax_rows(x, scale=0.9)
    y, lse = sdpa.attn_softmax_rows(x.cuda(), scale=0.9, mode=mode)
    torch.cuda.synchronize()
    check(y, lse, y_ref, lse_ref, "bf16", f"{mode} short masked n{n}")


@pytest.mark.parametrize("n", [512, 1024, 4096, 32768, 65536])
def test_online_equals_three_pass(n):
    """The page's guard: both forms agree within 1e-3 (here much closer)."""
    x = generate_softmax_rows(16, n, "f32", seed=n, std=4.0).cuda()
    y1, l1 = sdpa.attn_softmax_rows(x, mode="online")
    y3, l3 = sdpa.attn_softmax_rows(x, mode="three_pass")
    torch.cuda.synchronize()
    d = (y1 - y3).abs().max().item()
    say(f"  n{n}: max|online - three_pass| = {d:.3e}")
    assert d <= 1e-3
    assert (l1 - l3).abs().max().item() <= 1e-4
