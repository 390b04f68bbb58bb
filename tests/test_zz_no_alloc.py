"""attn_fwd_noalloc, the entry point that allocates nothing, against attn_fwd
on the same inputs, through the C ABI.

Its workspace is the library's static per-GPU buffer, so two calls in a row
share it: the second call here has a smaller input than the first and must
not see the first one's records. Shapes cover both plans that need a
workspace: the split-over-keys decode pair and the fused kernel over key
ranges. Bar: 2e-2 max-abs on O and LSE against attn_fwd (the oracle's bar
for 16-bit inputs); the two share their kernels, so equal bits are
expected too. Runs on an MI355X only."""
import ctypes

import pytest
import torch

import scaled_dot_product_flashattention_amd as sdpa
from parity_util import say
from scaled_dot_product_flashattention_amd.api import dtype_code, layout_code
from scaled_dot_product_flashattention_amd.inputs import WORKLOADS, generate

pytestmark = pytest.mark.gpu

W = WORKLOADS
NOALLOC_BYTES = 64 << 20
E_SCRATCH_LIMIT = 8

# (first call, second call): each pair's second input is smaller
PAIRS = {
    "decode": (W["decode_bf16"].replace(name="na_dec1", B=4, H=32, Sk=32768),
               W["decode_bf16"].replace(name="na_dec2", B=2, H=8, Sk=8192, kv_len_range=(1, 8192))),
    "key_ranges": (W["medium_bf16"].replace(name="na_kr1", B=1, H=4, Sq=1024, Sk=32768, d=128),
                   W["medium_bf16"].replace(name="na_kr2", B=2, H=2, Sq=300, Sk=9000, dtype="f16",
                                            kv_len_range=(2000, 9000), layout="bshd")),
}


def raw_noalloc(q, k, v, w, kv_len, o, lse):
    """One call of the C symbol attn_fwd_noalloc on torch's current stream."""
    lib = sdpa.load_library()
    rc = lib.attn_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                              w.B, w.H, w.Sq, w.Sk, w.d, ctypes.c_float(w.scale), int(w.causal),
                              layout_code(w.layout), dtype_code(q.dtype),
                              None if kv_len is None else kv_len.data_ptr(),
                              torch.cuda.current_stream().cuda_stream)
    return rc


@pytest.mark.parametrize("pair", list(PAIRS))
def test_noalloc_matches_attn_fwd_twice(pair):
    for w in PAIRS[pair]:
        t = generate(w)
        q, k, v = (t[n].cuda() for n in ("q", "k", "v"))
        kv_len = None if t["kv_len"] is None else t["kv_len"].cuda()
        dt = q.dtype
        need = sdpa.attn_fwd_workspace_size(w.B, w.H, w.Sq, w.Sk, w.d, dt, w.causal)
        say(f"noalloc {w.name}: B{w.B} H{w.H} Sq{w.Sq} Sk{w.Sk} d{w.d} {w.dtype} {w.layout} "
            f"causal={w.causal} pad={w.kv_len_range}: workspace {need} bytes")
        assert 0 < need <= NOALLOC_BYTES  # the plan uses the static buffer
        o_ref, l_ref = sdpa.attn_fwd(q, k, v, scale=w.scale, causal=w.causal, layout=w.layout,
                                     kv_len=kv_len)
        o = torch.full_like(q, float("nan"))
        lse = torch.full((w.B, w.H, w.Sq), float("nan"), dtype=torch.float32, device="cuda")
        assert raw_noalloc(q, k, v, w, kv_len, o, lse) == 0
        torch.cuda.synchronize()
        eo = float((o.float() - o_ref.float()).abs().max())
        fin = torch.isfinite(l_ref)
        assert torch.equal(fin, torch.isfinite(lse))
        el = float((lse[fin] - l_ref[fin]).abs().max()) if fin.any() else 0.0
        say(f"  max|dO| = {eo:.3e}, max|dLSE| = {el:.3e} against attn_fwd")
        assert eo <= 2e-2 and el <= 2e-2
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
        assert torch.equal(lse, l_ref)


def test_noalloc_without_workspace_plan():
    """A plan with no key split needs no buffer: same bits as attn_fwd."""
    w = W["medium_bf16"].replace(name="na_plain", H=2, Sq=300, Sk=300)
    t = generate(w)
    q, k, v = (t[n].cuda() for n in ("q", "k", "v"))
    assert sdpa.attn_fwd_workspace_size(w.B, w.H, w.Sq, w.Sk, w.d, q.dtype, w.causal) == 0
    o_ref, l_ref = sdpa.attn_fwd(q, k, v)
    o, lse = sdpa.attn_fwd_noalloc(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)) and torch.equal(lse, l_ref)
