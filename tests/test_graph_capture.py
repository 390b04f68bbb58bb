"""The fused forward and the split-K decode pair captured in a HIP graph
(through torch.cuda.graph) and replayed: every replay must give the same
bits as the eager call on the same inputs. The library allocates nothing
and clears no memory inside a call (workspaces are passed in), so the
captured launches are its kernels only. Replays are interleaved with eager
work and synchronisations, and the inputs change between replays. Runs on an
MI355X only."""
import pytest
import torch

import scaled_dot_product_flashattention_amd as sdpa
from parity_util import say
from scaled_dot_product_flashattention_amd.inputs import WORKLOADS, generate

pytestmark = pytest.mark.gpu


SHAPES = {"medium_bf16": dict(H=4, Sq=512, Sk=512),
          "decode_bf16": dict(B=2, H=8, Sk=8192),
          "key_ranges": dict(H=2, Sq=256, Sk=8192)}  # the fused kernel over key ranges


@pytest.mark.parametrize("name", list(SHAPES))
def test_graph_replay_matches_eager(name):
    base = WORKLOADS["medium_bf16" if name == "key_ranges" else name]
    w = base.replace(**SHAPES[name])
    inputs = [generate(w, seed=s) for s in (31, 32, 33)]
    dev = torch.device("cuda:0")
    q, k, v = (inputs[0][n].to(dev) for n in ("q", "k", "v"))
    B, H, Sq, Sk, d = w.B, w.H, w.Sq, w.Sk, w.d
    n_split = sdpa.attn_fwd_plan(B, H, Sq, Sk, d, q.dtype, w.causal)
    say(f"graph capture {name}: B{B} H{H} Sq{Sq} Sk{Sk} d{d} n_split={n_split}")
    ws = torch.empty(max(sdpa.attn_fwd_workspace_size(B, H, Sq, Sk, d, q.dtype, w.causal), 16), dtype=torch.uint8,
                     device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device=dev)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm the path up off the capture stream
        sdpa.attn_fwd(q, k, v, workspace=ws, out=o, lse=lse)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sdpa.attn_fwd(q, k, v, workspace=ws, out=o, lse=lse)
    torch.cuda.synchronize()

    for rep in range(6):
        t = inputs[rep % 3]
        for n, dst in (("q", q), ("k", k), ("v", v)):
            dst.copy_(t[n].to(dev))
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got_o, got_l = o.clone(), lse.clone()
        # eager work between replays, then the eager reference
        scratch = torch.randn(1 << 20, device=dev).sum()
        ref_o, ref_l = sdpa.attn_fwd(q, k, v)
        torch.cuda.synchronize()
        assert torch.isfinite(scratch)
        assert torch.equal(got_o, ref_o), f"replay {rep}: O differs from eager"
        assert torch.equal(got_l, ref_l), f"replay {rep}: LSE differs from eager"
    say(f"  {name}: 6 replays bit-identical to eager")
