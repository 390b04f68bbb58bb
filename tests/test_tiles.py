"""Every tile variant of the fused kernel against the fp64 oracle.

The tuned table may send any shape to any variant, so each variant is held
to the same bar as the default path (2e-2 max-abs for 16-bit inputs) on
shapes that exercise its edges: a single partial tile, ragged query and key
tails, causal masks with Sq != Sk, key padding with NaN-poisoned rows past
kv_len, the head-group layout, rows whose scores all sit far below zero or
rise or fall steeply over the keys, and the full workload sizes. Runs on an
MI355X only."""
import pytest
import torch

import scaled_dot_product_flashattention_amd as sdpa
from parity_util import full_case, full_size_case, say
from scaled_dot_product_flashattention_amd.inputs import WORKLOADS, generate

pytestmark = pytest.mark.gpu

W = WORKLOADS
N_TILES = {64: 6, 128: 4}  # variants per head size (the ABI tests check the library agrees)
CASES = [(dt, d, t) for dt, d in (("bf16", 64), ("f16", 64), ("bf16", 128), ("f16", 128))
         for t in range(N_TILES[d])]
SHAPES = {  # name: (B, H, Sq, Sk, causal, kv_len range, layout, extra workload fields)
    "single_tile": (1, 1, 40, 70, False, None, "bhsd", {}),
    "ragged": (2, 3, 300, 700, False, (200, 700), "bhsd", {}),
    "causal_square": (1, 2, 520, 520, True, None, "bshd", {}),
    "causal_more_queries": (2, 2, 300, 100, True, (0, 100), "bhsd", {}),
    "split_groups": (2, 4, 260, 2100, True, (1000, 2100), "split:2", {}),
    # q, k x 4: the sums leave range, the reference max moves between tiles
    "large_scores": (1, 2, 400, 900, True, (500, 900), "bhsd", {"qk_mult": 4.0}),
    # scale * log2(e) > 1: queries are not pre-scaled
    "scale_above_one": (1, 2, 300, 700, False, None, "bhsd", {"scale": 2.0}),
    # scale * log2(e) ~ 1 on large scores
    "scale_at_one": (1, 2, 300, 700, False, None, "bhsd", {"scale": 0.69, "qk_mult": 2.0}),
    # wide score spread (about 8 in log2 units): later tiles' maxima sit
    # above the first tile's, which sets the reference
    "wide_spread": (1, 2, 300, 700, False, None, "bhsd", {"scale": 0.69}),
    # every score of a row shifted by -8 .. -20 (natural log): softmax is
    # unchanged; fp16 probabilities against a reference far above the row's
    # maximum would fall into the subnormal range
    "shift_m8": (1, 2, 300, 700, False, None, "bhsd", {"score_shift": (-8.0, -8.0)}),
    "shift_m14": (1, 2, 300, 700, True, None, "bshd", {"score_shift": (-14.0, -14.0)}),
    "shift_m17": (2, 2, 300, 700, False, (300, 700), "bhsd", {"score_shift": (-17.0, -17.0)}),
    "shift_m20": (1, 2, 300, 700, False, None, "bhsd", {"score_shift": (-20.0, -20.0)}),
    # scores falling by 20 over the keys: the first tile holds the maxima
    "falling_scores": (1, 2, 300, 700, False, None, "bhsd", {"score_shift": (0.0, -20.0)}),
    # scores rising by 12 over the keys: later fp16 probabilities pass 65504
    # against the first tile's reference while the sums stay below 2^32; the
    # infinite sum sends the tile to the exact-maximum path
    "fp16_overflow_window": (1, 2, 300, 700, False, None, "bhsd", {"score_shift": (0.0, 12.0)}),
    # scores rising by 30: the sums pass 2^32 for both types
    "rising_scores": (1, 2, 300, 700, True, (400, 700), "bshd", {"score_shift": (0.0, 30.0)}),
    # scale 0 (uniform weights over the valid keys), with causal rows and padding
    "scale_zero": (2, 2, 200, 333, True, (1, 333), "bshd", {"scale": 0.0}),
}


@pytest.mark.parametrize("shape", list(SHAPES))
@pytest.mark.parametrize("dtype,d,tile", CASES)
def test_tile_variant_matches_oracle(dtype, d, tile, shape):
    B, H, Sq, Sk, causal, pad, layout, extra = SHAPES[shape]
    extra = dict(extra)
    scale = extra.pop("scale", None)
    w = W["medium_bf16"].replace(name=f"{shape}_t{tile}", B=B, H=H, Sq=Sq, Sk=Sk, d=d, dtype=dtype,
                                 causal=causal, kv_len_range=pad, layout=layout,
                                 seed=70 + tile + d, **extra)
    full_case(w, path=f"tile:{tile}", poison=pad is not None, scale=scale)


@pytest.mark.parametrize("name,tile", [(n, t) for n in ("medium_bf16", "long_causal_bf16", "bert_pad_fp16")
                                       for t in range(N_TILES[WORKLOADS[n].d])])
@pytest.mark.timeout(900)
def test_tile_variant_full_size(name, tile):
    """Each variant at a full workload size, every row (the oracle's result
    is computed once per workload and shared by its variants)."""
    full_size_case(W[name], path=f"tile:{tile}", poison=W[name].kv_len_range is not None)


def test_table_choice_is_the_default_path():
    """attn_fwd and attn_fwd_tiled(tile=-1) run the table's variant: the same
    bits as forcing that variant."""
    w = W["medium_bf16"].replace(name="choice", Sq=1024, Sk=1024, H=4)
    t = generate(w)
    q, k, v = (t[n].cuda() for n in ("q", "k", "v"))
    tile = sdpa.attn_fwd_tile_choice(w.B, w.H, w.Sq, w.Sk, w.d, q.dtype, w.causal)
    say(f"table choice for B{w.B} H{w.H} S{w.Sq} d{w.d}: variant {tile}")
    o1, l1 = sdpa.attn_fwd(q, k, v)
    o2, l2 = sdpa.attn_fwd_tiled(q, k, v)
    o3, l3 = sdpa.attn_fwd_tiled(q, k, v, tile=tile)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(o1, o3)
    assert torch.equal(l1, l2) and torch.equal(l1, l3)


# Key walks of exactly 1 .. 6 tiles (and a ragged last tile): the pipeline's
# ends, and with rings of six stages the barrier taken at even tiles only.
WALKS = [(d, t, sk) for d in (64, 128) for t in range(N_TILES[d]) for sk in (64, 128, 191, 256, 320, 383)]


@pytest.mark.parametrize("d,tile,Sk", WALKS)
def test_short_key_walks(d, tile, Sk):
    w = W["medium_bf16"].replace(name=f"walk_{Sk}_d{d}_t{tile}", B=1, H=2, Sq=300, Sk=Sk, d=d,
                                 seed=900 + Sk + tile)
    full_case(w, path=f"tile:{tile}")
