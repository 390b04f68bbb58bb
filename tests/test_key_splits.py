"""The fused 16-bit kernel over key ranges against the fp64 oracle.

With n_split > 1 each (batch, head, query tile, key range) workgroup writes
per query row the unnormalised record of its range (reference max, sum,
weighted sum of V), and the merge kernel combines the ranges by the block
rule. Every tile variant runs on shapes that exercise the edges of the
ranges: ranges past the valid keys (empty records), more ranges than key
tiles, causal rows that see no key of a range, key padding with
NaN-poisoned rows past kv_len (kv_len 0 included), large scores that move
the reference max, scale 0, the fp16 probability window, rows shifted far
below zero, and the head-group layout. attn_fwd must take the same path, bit for bit, where its
plan splits, and the full-size few-head shapes are checked on every row.
Bar: 2e-2 max-abs on O and LSE. Runs on an MI355X only."""
import pytest
import torch

import scaled_dot_product_flashattention_amd as sdpa
from parity_util import full_case, full_size_case, say
from scaled_dot_product_flashattention_amd.inputs import WORKLOADS, generate

pytestmark = pytest.mark.gpu

W = WORKLOADS
N_TILES = {64: 6, 128: 4}
CASES = [(dt, d, t) for dt, d in (("bf16", 64), ("f16", 64), ("bf16", 128), ("f16", 128))
         for t in range(N_TILES[d])]
# name: (B, H, Sq, Sk, causal, kv_len range, layout, n_split, extra workload fields)
SHAPES = {
    # ranges of 640 keys; rows with kv_len 0 have every record empty
    "ragged_pad": (2, 3, 300, 2500, False, (0, 2500), "bhsd", 4, {}),
    # causal rows 0..519 over 2000 keys in 5 ranges: most ranges are past
    # the diagonal of most rows
    "causal": (1, 2, 520, 2000, True, None, "bshd", 5, {}),
    # 40 ranges of 128 keys over 3000 keys: ranges 24.. are empty
    "more_ranges_than_tiles": (1, 2, 7, 3000, False, None, "bhsd", 40, {}),
    "groups_causal_pad": (2, 4, 130, 2100, True, (1000, 2100), "split:2", 3, {}),
    # q, k x 4: the ranges' reference maxima differ widely
    "large_scores": (1, 2, 64, 4000, False, (2000, 4000), "bhsd", 6, {"qk_mult": 4.0}),
    "scale_zero": (2, 2, 65, 1500, True, (1, 1500), "bshd", 3, {"scale": 0.0}),
    "wide_spread": (1, 2, 100, 3000, False, None, "bhsd", 4, {"scale": 0.69}),
    # every score shifted by -8 .. -20 (natural log): each range's reference
    # starts at its own first tile's maximum
    "shift_m8": (1, 2, 100, 3000, False, None, "bhsd", 4, {"score_shift": (-8.0, -8.0)}),
    "shift_m14": (1, 2, 130, 2500, True, None, "bshd", 4, {"score_shift": (-14.0, -14.0)}),
    "shift_m20": (2, 2, 100, 3000, False, (1, 3000), "bhsd", 5, {"score_shift": (-20.0, -20.0)}),
    # scores rising by 12 (fp16 probabilities overflow inside a range) and
    # falling by 20 over the keys (the ranges' maxima differ by 20)
    "fp16_overflow_window": (1, 2, 100, 3000, False, None, "bhsd", 4, {"score_shift": (0.0, 12.0)}),
    "falling_scores": (1, 2, 100, 3000, False, None, "bhsd", 4, {"score_shift": (0.0, -20.0)}),
    "two_queries": (1, 3, 2, 5000, False, (1, 5000), "bhsd", 8, {}),
}


@pytest.mark.parametrize("shape", list(SHAPES))
@pytest.mark.parametrize("dtype,d,tile", CASES)
def test_key_ranges_match_oracle(dtype, d, tile, shape):
    B, H, Sq, Sk, causal, pad, layout, n_split, extra = SHAPES[shape]
    extra = dict(extra)
    scale = extra.pop("scale", None)
    w = W["medium_bf16"].replace(name=f"{shape}_t{tile}_n{n_split}", B=B, H=H, Sq=Sq, Sk=Sk, d=d,
                                 dtype=dtype, causal=causal, kv_len_range=pad, layout=layout,
                                 seed=170 + tile + d, **extra)
    full_case(w, path=f"tile:{tile}:{n_split}", poison=pad is not None, scale=scale)


def test_plan_path_is_the_forced_split():
    """Where the plan splits a prefill shape, attn_fwd gives the same bits as
    attn_fwd_tiled with the plan's split count and the key-range variant."""
    w = W["medium_bf16"].replace(name="plan_split", B=1, H=4, Sq=200, Sk=8192)
    t = generate(w)
    q, k, v = (t[n].cuda() for n in ("q", "k", "v"))
    n = sdpa.attn_fwd_plan(w.B, w.H, w.Sq, w.Sk, w.d, q.dtype, w.causal)
    assert n > 1
    say(f"plan for B{w.B} H{w.H} Sq{w.Sq} Sk{w.Sk} d{w.d}: {n} key ranges")
    tile = sdpa.attn_fwd_tile_choice(w.B, w.H, w.Sq, w.Sk, w.d, q.dtype, w.causal)
    o1, l1 = sdpa.attn_fwd(q, k, v)
    o2, l2 = sdpa.attn_fwd_tiled(q, k, v, n_split=n)
    o3, l3 = sdpa.attn_fwd_tiled(q, k, v, n_split=n, tile=tile)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o1, o3) and torch.equal(l1, l3)


FULL = {  # few heads and query tiles over long keys, where the plan splits
    "h32_q64_k32768_d128": dict(B=1, H=32, Sq=64, Sk=32768, d=128),
    "b2_h32_q128_k16384_d64": dict(B=2, H=32, Sq=128, Sk=16384, d=64),
    "h2_causal_s8192_d64": dict(B=1, H=2, Sq=8192, Sk=8192, d=64, causal=True),
    "h8_q300_k20000_pad_f16": dict(B=2, H=4, Sq=300, Sk=20000, d=128, dtype="f16",
                                   kv_len_range=(1, 20000), layout="bshd"),
}


@pytest.mark.parametrize("name", list(FULL))
def test_planned_split_full_size(name):
    w = W["medium_bf16"].replace(name=name, seed=181, **FULL[name])
    dt = torch.float16 if w.dtype == "f16" else torch.bfloat16
    n = sdpa.attn_fwd_plan(w.B, w.H, w.Sq, w.Sk, w.d, dt, w.causal)
    say(f"{name}: plan {n} key ranges")
    assert n > 1
    full_size_case(w, path="fused", poison=w.kv_len_range is not None)
