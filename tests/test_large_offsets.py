"""Element offsets past 2^31 on every attention path.

K and V in [B,S,H,d] with H = 16, Sk = 2^20 and d = 128 hold 2^31 elements
each, so the last keys of every head sit past any 32-bit element offset.
Keys repeat a random block of 4099 rows (a prime period), so a wrapped
offset would read a different key. Every output row is checked against the
fp64 oracle (2e-2 max-abs, the 16-bit bar). Runs on an MI355X only; needs
about 8 GiB of device memory and 8 GiB of host memory."""
import numpy as np
import pytest
import torch

import oracle
import scaled_dot_product_flashattention_amd as sdpa
from parity_util import TOL_16, errors, say
from scaled_dot_product_flashattention_amd.inputs import WORKLOADS, generate_periodic_keys

pytestmark = pytest.mark.gpu

SK = 1 << 20


@pytest.fixture(scope="module")
def long_keys():
    w = WORKLOADS["decode_bf16"].replace(name="offsets_2_31", B=1, H=16, Sq=4, Sk=SK,
                                         layout="bshd", seed=91)
    t = generate_periodic_keys(w, period=4099)
    assert t["k"].numel() == 1 << 31
    dev = {n: t[n].cuda() for n in ("q", "k", "v")}
    torch.cuda.synchronize()
    return w, t, dev


def check(w, t, o, lse, kv_len=None, what=""):
    rows = np.arange(w.B * w.H * w.Sq, dtype=np.int64)
    o_ref, lse_ref = oracle.attention_rows(t["q"], t["k"], t["v"], rows, scale=w.scale,
                                           causal=False, layout="bshd", kv_len=kv_len)
    oc = o.float().cpu()
    got = np.stack([oc[0, r % w.Sq, (r // w.Sq) % w.H].numpy() for r in rows]).astype(np.float64)
    got_l = lse.cpu().numpy().reshape(-1).astype(np.float64)
    eo, el = np.abs(got - o_ref).max(), np.abs(got_l - lse_ref).max()
    say(f"  {what}: max|dO| = {eo:.3e}, max|dLSE| = {el:.3e}")
    assert eo <= TOL_16 and el <= TOL_16, what


@pytest.mark.parametrize("path", ["plan", "fused", "naive"])
def test_offsets_past_2_31(long_keys, path):
    w, t, d = long_keys
    say(f"case offsets past 2^31: B1 H16 Sq{w.Sq} Sk{SK} d128 bf16 [B,S,H,d] {path}")
    kw = dict(layout="bshd")
    if path == "plan":
        o, lse = sdpa.attn_fwd(d["q"], d["k"], d["v"], **kw)
    elif path == "fused":
        o, lse = sdpa.attn_fwd_tiled(d["q"], d["k"], d["v"], **kw)
    else:
        o, lse = sdpa.attn_fwd_naive(d["q"], d["k"], d["v"], **kw)
    torch.cuda.synchronize()
    check(w, t, o, lse, what=path)


def test_offsets_past_2_31_with_key_length(long_keys):
    """A key length that ends inside the last period, on the split plan."""
    w, t, d = long_keys
    kv = torch.tensor([SK - 12345], dtype=torch.int32)
    say(f"case offsets past 2^31 with kv_len {SK - 12345}")
    o, lse = sdpa.attn_fwd(d["q"], d["k"], d["v"], layout="bshd", kv_len=kv.cuda())
    torch.cuda.synchronize()
    check(w, t, o, lse, kv_len=kv, what="plan, kv_len")
