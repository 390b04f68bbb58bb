"""Pins of the fp64 attention oracle against facts fixed by the pages and by
mathematics, not by the oracle itself.

Each ``pin_*`` takes an ``oracle.Oracle`` handle and raises AssertionError
when the oracle disagrees. ``tests/test_oracle.py`` runs them against the
oracle as built; ``tests/test_oracle_mutants.py`` runs them against copies of
the oracle with planted mistakes and requires every copy to fail one of them.

Sources of the facts (pages cited by title and section):
  chapter "2. 自注意力机制算子：QKV投影、注意力分数计算、Softmax、加权求和，以及FlashAttention优化"
    §2.2 scores and 1/sqrt(D_k) scale, §2.3 three-step softmax and the max
    shift against exp(1000) overflow, §2.4 weighted sum, §2.6 online update;
  page "[Performance] [WebGPU] Proposal: Add an option to use online softmax
    instead of naive softmax", §四 repro row, §七 numeric test;
  page "WebGPU 算子优化：QKV 内存合并与 FlashAttention 分块计算", section
    "FlashAttention 分块计算原理与浏览器适配": block merge of (m, l);
  the chapter's §2.1: Q, K, V as one product with the concatenated weight.
"""
from __future__ import annotations

import decimal
import json
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

_CTX = decimal.Context(prec=50)
D = decimal.Decimal


# ---------------------------------------------------------------------------
# independent references
# ---------------------------------------------------------------------------
def to_bhsd(x: np.ndarray, layout: str) -> np.ndarray:
    return x if layout == "bhsd" else np.transpose(x, (0, 2, 1, 3))


def from_bhsd(x: np.ndarray, layout: str) -> np.ndarray:
    return x if layout == "bhsd" else np.transpose(x, (0, 2, 1, 3))


def f64(t) -> np.ndarray:
    """Decode a tensor to float64 with the library's own conversion."""
    if isinstance(t, torch.Tensor):
        return t.to(torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def brute_force(q, k, v, layout, scale, causal=False, kv_len=None):
    """Direct formula at 50 significant digits, with no max shift:
    O_i = sum_j exp(s_ij) v_j / sum_j exp(s_ij), LSE_i = ln sum_j exp(s_ij),
    over keys j < n_b and (causal) j <= i. Inputs are float64 arrays."""
    q, k, v = (to_bhsd(np.asarray(x), layout) for x in (q, k, v))
    B, H, Sq, d = q.shape
    Sk = k.shape[2]
    o = np.zeros((B, H, Sq, d))
    lse = np.zeros((B, H, Sq))
    sc = D(float(scale))
    for b in range(B):
        nb = Sk if kv_len is None else min(max(int(kv_len[b]), 0), Sk)
        for h in range(H):
            for i in range(Sq):
                ws = []
                for j in range(Sk):
                    if j >= nb or (causal and j > i):
                        continue
                    s = _CTX.multiply(sc, sum((_CTX.multiply(D(float(q[b, h, i, c])), D(float(k[b, h, j, c])))
                                               for c in range(d)), D(0)))
                    ws.append((_CTX.exp(s), j))
                if not ws:
                    lse[b, h, i] = -math.inf
                    continue
                z = sum((w for w, _ in ws), D(0))
                for c in range(d):
                    num = sum((_CTX.multiply(w, D(float(v[b, h, j, c]))) for w, j in ws), D(0))
                    o[b, h, i, c] = float(_CTX.divide(num, z))
                lse[b, h, i] = float(_CTX.ln(z))
    return from_bhsd(o, layout), lse


def torch_layout(x: torch.Tensor, layout: str) -> torch.Tensor:
    return x if layout == "bhsd" else x.transpose(1, 2)


def rand(rng, shape, dtype=np.float32):
    return rng.standard_normal(shape).astype(dtype)


def shape_of(layout, B, H, S, d):
    return (B, H, S, d) if layout == "bhsd" else (B, S, H, d)


def close(a, b, atol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    with np.errstate(invalid="ignore"):
        err = np.where(both_inf, 0.0, np.abs(a - b))
    worst = float(np.nanmax(err)) if err.size else 0.0
    assert not np.isnan(err).any(), f"{what}: NaN mismatch"
    assert worst <= atol, f"{what}: max |diff| {worst:.3e} > {atol:.1e}"


# ---------------------------------------------------------------------------
# pins
# ---------------------------------------------------------------------------
def pin_decode_exact(orc):
    """Every fp16 and bf16 bit pattern decodes to the value numpy / torch give."""
    bits = np.arange(65536, dtype=np.uint16)
    f16 = bits.view(np.float16)
    mine = orc.decode(f16)
    ref = f16.astype(np.float64)
    assert np.array_equal(np.isnan(mine), np.isnan(ref)), "fp16 NaN patterns"
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok]), "fp16 decode"
    bf = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16)
    mine = orc.decode(bf)
    ref = bf.to(torch.float64).numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(ref)), "bf16 NaN patterns"
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok]), "bf16 decode"


def pin_rows_sum_to_one(orc):
    """With V = I (d = Sk) the output row is the probability row: entries are
    >= 0, exactly 0 at masked keys, and each row sums to 1."""
    rng = np.random.default_rng(11)
    B, H, Sq, Sk = 2, 2, 9, 12
    kv_len = np.array([12, 5], dtype=np.int32)
    for layout in ("bhsd", "bshd"):
        for causal in (False, True):
            for lens in (None, kv_len):
                q = rand(rng, shape_of(layout, B, H, Sq, Sk)) * 2
                k = rand(rng, shape_of(layout, B, H, Sk, Sk)) * 2
                eye = np.zeros((B, H, Sk, Sk), dtype=np.float32)
                eye[:, :, np.arange(Sk), np.arange(Sk)] = 1.0
                v = np.ascontiguousarray(from_bhsd(eye, layout))
                o, _ = orc.attention(q, k, v, scale=0.3, causal=causal, layout=layout, kv_len=lens)
                p = to_bhsd(o, layout)
                assert (p >= 0).all(), "negative probability"
                for b in range(B):
                    nb = Sk if lens is None else int(lens[b])
                    for i in range(Sq):
                        lim = min(nb, i + 1) if causal else nb
                        assert np.all(p[b, :, i, lim:] == 0.0), "mass on a masked key"
                close(p.sum(-1), np.ones((B, H, Sq)), 1e-12, "row sums")


def pin_zero_query_mean(orc):
    """q = 0 gives uniform weights: O_i is the mean of V over the valid keys
    and LSE_i = ln(number of valid keys)."""
    rng = np.random.default_rng(12)
    B, H, Sq, Sk, d = 2, 3, 10, 13, 8
    kv_len = np.array([13, 4], dtype=np.int32)
    for layout in ("bhsd", "bshd"):
        for causal in (False, True):
            for lens in (None, kv_len):
                q = np.zeros(shape_of(layout, B, H, Sq, d), dtype=np.float32)
                k = rand(rng, shape_of(layout, B, H, Sk, d))
                v = rand(rng, shape_of(layout, B, H, Sk, d))
                o, lse = orc.attention(q, k, v, scale=0.5, causal=causal, layout=layout, kv_len=lens)
                vb = to_bhsd(v, layout).astype(np.float64)
                ref = np.zeros((B, H, Sq, d))
                rl = np.zeros((B, H, Sq))
                for b in range(B):
                    nb = Sk if lens is None else int(lens[b])
                    for i in range(Sq):
                        lim = min(nb, i + 1) if causal else nb
                        ref[b, :, i, :] = vb[b, :, :lim, :].mean(axis=1)
                        rl[b, :, i] = math.log(lim)
                close(to_bhsd(o, layout), ref, 1e-14, "q=0 output")
                close(lse, rl, 1e-14, "q=0 lse")


def pin_dominant_key(orc):
    """A key whose score beats every other by >= 50 takes all the weight:
    O_i = V_{j*} up to (Sk-1) e^-50 max|V|."""
    rng = np.random.default_rng(13)
    B, H, Sq, Sk, d = 1, 2, 6, 20, 16
    for layout in ("bhsd", "bshd"):
        q = rand(rng, shape_of(layout, B, H, Sq, d))
        k = rand(rng, shape_of(layout, B, H, Sk, d)) * 0.1
        v = rand(rng, shape_of(layout, B, H, Sk, d))
        qb = to_bhsd(q, layout)
        kb = to_bhsd(k, layout).copy()
        star = {}
        for h in range(H):
            i = 2 + h
            j = int(rng.integers(0, Sk))
            kb[0, h, j, :] = qb[0, h, i, :] * np.float32(200.0 / float(qb[0, h, i] @ qb[0, h, i]))
            star[h] = (i, j)
        k = np.ascontiguousarray(from_bhsd(kb, layout))
        o, _ = orc.attention(q, k, v, scale=1.0, layout=layout)
        ob = to_bhsd(o, layout)
        vb = to_bhsd(v, layout).astype(np.float64)
        for h, (i, j) in star.items():
            others = [float(qb[0, h, i].astype(np.float64) @ kb[0, h, jj].astype(np.float64))
                      for jj in range(Sk) if jj != j]
            top = float(qb[0, h, i].astype(np.float64) @ kb[0, h, j].astype(np.float64))
            assert top - max(others) >= 50.0, "test construction: margin"
            tol = (Sk - 1) * math.exp(-50.0) * np.abs(vb).max() + 1e-13
            close(ob[0, h, i], vb[0, h, j], tol, "dominant key")


def pin_online_worked_example(orc):
    """The page's row [1.0, 2.0, 0.5, 3.0]: the online recurrence and the
    three-step softmax agree with the 50-digit closed form."""
    with open(os.path.join(GOLDEN, "online_softmax_row.json")) as f:
        fx = json.load(f)
    s = fx["scores"]
    n = len(s)
    # closed forms: running max; l_t = sum_{j<=t} e^{s_j - m_t}; p_j = e^{s_j} / sum e^{s}
    m_ref, l_ref = [], []
    for t in range(n):
        m_t = max(s[: t + 1])
        m_ref.append(m_t)
        l_ref.append(float(sum((_CTX.exp(D(x) - D(m_t)) for x in s[: t + 1]), D(0))))
    z = sum((_CTX.exp(D(x)) for x in s), D(0))
    p_ref = [float(_CTX.exp(D(x)) / z) for x in s]
    lse_ref = float(_CTX.ln(z))
    mt, lt, p = orc.online_softmax(s)
    close(mt, m_ref, 0.0, "online m trace")
    close(lt, l_ref, 1e-15, "online l trace")
    close(p, p_ref, 1e-15, "online probabilities")
    # the same row through the attention definition: q = e0, k_j = s_j e0, V = I
    q = np.zeros((1, 1, 1, n), dtype=np.float32)
    q[0, 0, 0, 0] = 1.0
    k = np.zeros((1, 1, n, n), dtype=np.float32)
    k[0, 0, :, 0] = s
    v = np.eye(n, dtype=np.float32).reshape(1, 1, n, n)
    o, lse = orc.attention(q, k, v, scale=1.0)
    close(o[0, 0, 0], p_ref, 1e-15, "three-step softmax of the page's row")
    close(lse[0, 0, 0], lse_ref, 1e-15, "lse of the page's row")
    # the page's own test tolerance between the online and the naive result
    close(o[0, 0, 0], p, fx["page_atol"], "online vs naive (page tolerance)")


def _tiny_cases():
    rng = np.random.default_rng(14)
    cases = []
    for layout in ("bhsd", "bshd"):
        for (B, H, Sq, Sk, d) in ((1, 1, 1, 1, 1), (2, 2, 5, 8, 4), (1, 2, 8, 3, 8), (2, 1, 7, 7, 8)):
            for causal in (False, True):
                for pad in (False, True):
                    lens = None
                    if pad:
                        lens = rng.integers(0 if B > 1 else 1, Sk + 1, size=B).astype(np.int32)
                    cases.append((layout, B, H, Sq, Sk, d, causal, lens, rng))
    return cases


def pin_brute_force(orc):
    """Tiny shapes (S <= 8, d <= 8), every mask, both layouts, all storage
    types: the oracle equals the 50-digit direct formula."""
    for (layout, B, H, Sq, Sk, d, causal, lens, rng) in _tiny_cases():
        for dt in (torch.float32, torch.float16, torch.bfloat16):
            q = torch.from_numpy(rand(rng, shape_of(layout, B, H, Sq, d)) * 1.5).to(dt)
            k = torch.from_numpy(rand(rng, shape_of(layout, B, H, Sk, d)) * 1.5).to(dt)
            v = torch.from_numpy(rand(rng, shape_of(layout, B, H, Sk, d))).to(dt)
            scale = 0.7
            o, lse = orc.attention(q, k, v, scale=scale, causal=causal, layout=layout, kv_len=lens)
            ro, rl = brute_force(f64(q), f64(k), f64(v), layout, scale, causal, lens)
            close(o, ro, 1e-13, f"brute force O {layout} {dt} causal={causal} lens={lens}")
            close(lse, rl, 1e-13, f"brute force LSE {layout} {dt}")


def pin_shift_invariance(orc):
    """Adding a constant to every score of a row leaves O unchanged and adds
    that constant to LSE. With +1000 (the exp(1000) example of §2.3) a softmax
    without the max shift overflows."""
    rng = np.random.default_rng(15)
    B, H, Sq, Sk, d = 1, 2, 5, 9, 64
    scale = 1.0 / 8.0
    for layout in ("bhsd", "bshd"):
        q = rand(rng, shape_of(layout, B, H, Sq, d))
        k = rand(rng, shape_of(layout, B, H, Sk, d))
        v = rand(rng, shape_of(layout, B, H, Sk, d))
        qb = to_bhsd(q, layout).copy()
        kb = to_bhsd(k, layout).copy()
        qb[..., 0] = 1.0
        kb[..., 0] = np.round(kb[..., 0] * 4) / 4  # exact after adding 8000 in fp32
        k2 = kb.copy()
        k2[..., 0] += np.float32(8000.0)  # shift = scale * 1 * 8000 = 1000
        q = np.ascontiguousarray(from_bhsd(qb, layout))
        k = np.ascontiguousarray(from_bhsd(kb, layout))
        k2 = np.ascontiguousarray(from_bhsd(k2, layout))
        o1, l1 = orc.attention(q, k, v, scale=scale, layout=layout)
        o2, l2 = orc.attention(q, k2, v, scale=scale, layout=layout)
        assert np.isfinite(o2).all() and np.isfinite(l2).all(), "overflow under a +1000 shift"
        close(o2, o1, 1e-12, "shift-invariant O")
        close(l2 - l1, np.full_like(l1, 1000.0), 1e-11, "LSE shifts by 1000")


def pin_permutation(orc):
    """Permuting the key/value rows together (no mask) changes nothing."""
    rng = np.random.default_rng(16)
    B, H, Sq, Sk, d = 2, 2, 6, 11, 8
    for layout in ("bhsd", "bshd"):
        q = rand(rng, shape_of(layout, B, H, Sq, d))
        k = rand(rng, shape_of(layout, B, H, Sk, d))
        v = rand(rng, shape_of(layout, B, H, Sk, d))
        perm = rng.permutation(Sk)
        ax = 2 if layout == "bhsd" else 1
        kp = np.ascontiguousarray(np.take(k, perm, axis=ax))
        vp = np.ascontiguousarray(np.take(v, perm, axis=ax))
        o1, l1 = orc.attention(q, k, v, scale=0.4, layout=layout)
        o2, l2 = orc.attention(q, kp, vp, scale=0.4, layout=layout)
        close(o2, o1, 1e-14, "permuted keys O")
        close(l2, l1, 1e-14, "permuted keys LSE")


def pin_value_linearity(orc):
    """Equal V rows c give O = c; O is linear in V."""
    rng = np.random.default_rng(17)
    B, H, Sq, Sk, d = 1, 2, 7, 10, 8
    for layout in ("bhsd", "bshd"):
        for causal in (False, True):
            q = rand(rng, shape_of(layout, B, H, Sq, d))
            k = rand(rng, shape_of(layout, B, H, Sk, d))
            c = np.round(rand(rng, (d,)) * 8) / 8
            v = np.ascontiguousarray(np.broadcast_to(c, shape_of(layout, B, H, Sk, d)).astype(np.float32))
            o, _ = orc.attention(q, k, v, scale=0.6, causal=causal, layout=layout)
            close(o, np.broadcast_to(c, o.shape), 1e-14, "constant V")
            v1 = (np.round(rand(rng, shape_of(layout, B, H, Sk, d)) * 8) / 8).astype(np.float32)
            v2 = (np.round(rand(rng, shape_of(layout, B, H, Sk, d)) * 8) / 8).astype(np.float32)
            o1, _ = orc.attention(q, k, v1, scale=0.6, causal=causal, layout=layout)
            o2, _ = orc.attention(q, k, v2, scale=0.6, causal=causal, layout=layout)
            o3, _ = orc.attention(q, k, (3 * v1 - 2 * v2).astype(np.float32), scale=0.6,
                                  causal=causal, layout=layout)
            close(o3, 3 * o1 - 2 * o2, 1e-13, "linearity in V")


def pin_causal_edges(orc):
    """Causal row 0 sees only key 0: O_0 = V_0, LSE_0 = s_00. With one key
    every row gives V_0."""
    rng = np.random.default_rng(18)
    B, H, S, d = 2, 2, 6, 8
    for layout in ("bhsd", "bshd"):
        q = rand(rng, shape_of(layout, B, H, S, d))
        k = rand(rng, shape_of(layout, B, H, S, d))
        v = rand(rng, shape_of(layout, B, H, S, d))
        o, lse = orc.attention(q, k, v, scale=0.3, causal=True, layout=layout)
        qb, kb, vb, ob = (to_bhsd(x, layout).astype(np.float64) for x in (q, k, v, o))
        close(ob[:, :, 0, :], vb[:, :, 0, :], 0.0, "causal row 0 output")
        s00 = 0.3 * np.einsum("bhc,bhc->bh", qb[:, :, 0, :], kb[:, :, 0, :])
        close(lse[:, :, 0], s00, 1e-14, "causal row 0 LSE")
        k1 = np.ascontiguousarray(np.take(k, [0], axis=2 if layout == "bhsd" else 1))
        v1 = np.ascontiguousarray(np.take(v, [0], axis=2 if layout == "bhsd" else 1))
        o1, _ = orc.attention(q, k1, v1, scale=0.3, layout=layout)
        ob1 = to_bhsd(o1, layout)
        close(ob1, np.broadcast_to(to_bhsd(v1, layout).astype(np.float64), ob1.shape), 0.0,
              "single key")


def pin_split_merge(orc):
    """Partials over any partition of the keys (empty parts included) merge
    to the unsplit result."""
    rng = np.random.default_rng(19)
    B, H, Sq, Sk, d = 2, 2, 5, 37, 8
    kv_len = np.array([37, 20], dtype=np.int32)
    for layout in ("bhsd", "bshd"):
        for causal in (False, True):
            q = rand(rng, shape_of(layout, B, H, Sq, d)) * 2
            k = rand(rng, shape_of(layout, B, H, Sk, d)) * 2
            v = rand(rng, shape_of(layout, B, H, Sk, d))
            o, lse = orc.attention(q, k, v, scale=0.5, causal=causal, layout=layout, kv_len=kv_len)
            ob = to_bhsd(o, layout)
            for row in range(B * H * Sq):
                i, h, b = row % Sq, (row // Sq) % H, row // (Sq * H)
                n_parts = int(rng.integers(1, 8))
                cuts = np.sort(rng.integers(0, Sk + 1, size=n_parts - 1))
                edges = [0, *cuts.tolist(), Sk]
                ms, ls, os_ = [], [], []
                for j0, j1 in zip(edges[:-1], edges[1:]):
                    m, l, op = orc.partial(q, k, v, row, j0, j1, scale=0.5, causal=causal,
                                           layout=layout, kv_len=kv_len)
                    ms.append(m)
                    ls.append(l)
                    os_.append(op)
                om, lm = orc.merge(ms, ls, np.array(os_))
                close(om, ob[b, h, i], 1e-13, "merged partials O")
                close(lm, lse[b, h, i], 1e-13, "merged partials LSE")


def pin_torch_sdpa(orc):
    """Library cross-check: torch's scaled_dot_product_attention in float64 on
    the CPU (math path), with a boolean mask built from the same rule."""
    rng = np.random.default_rng(20)
    B, H, Sq, Sk, d = 2, 3, 40, 56, 32
    kv_len = np.array([56, 23], dtype=np.int32)
    for layout in ("bhsd", "bshd"):
        for causal in (False, True):
            for lens in (None, kv_len):
                q = rand(rng, shape_of(layout, B, H, Sq, d))
                k = rand(rng, shape_of(layout, B, H, Sk, d))
                v = rand(rng, shape_of(layout, B, H, Sk, d))
                o, _ = orc.attention(q, k, v, scale=0.2, causal=causal, layout=layout, kv_len=lens)
                tq, tk, tv = (torch_layout(torch.from_numpy(x).double(), layout) for x in (q, k, v))
                jj = torch.arange(Sk).view(1, 1, 1, Sk)
                ii = torch.arange(Sq).view(1, 1, Sq, 1)
                nb = torch.full((B,), Sk) if lens is None else torch.from_numpy(lens).long()
                mask = jj < nb.view(B, 1, 1, 1)
                if causal:
                    mask = mask & (jj <= ii)
                mask = mask.expand(B, H, Sq, Sk)
                ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask,
                                                                       scale=0.2)
                ref = torch_layout(ref, layout).contiguous().numpy()
                close(o, ref, 1e-12, f"torch sdpa {layout} causal={causal}")


def pin_empty_rows(orc):
    """A sequence with no valid key gives O = 0 and LSE = -inf."""
    rng = np.random.default_rng(21)
    B, H, Sq, Sk, d = 2, 2, 3, 5, 4
    q = rand(rng, (B, H, Sq, d))
    k = rand(rng, (B, H, Sk, d))
    v = rand(rng, (B, H, Sk, d))
    o, lse = orc.attention(q, k, v, scale=1.0, kv_len=np.array([0, 5], dtype=np.int32))
    assert np.all(o[0] == 0.0), "empty row output"
    assert np.all(np.isneginf(lse[0])), "empty row LSE"
    assert np.isfinite(lse[1]).all()


def pin_rows_api(orc):
    """Selected rows equal the same rows of the full result."""
    rng = np.random.default_rng(22)
    B, H, Sq, Sk, d = 2, 3, 9, 14, 8
    for layout in ("bhsd", "bshd"):
        q = rand(rng, shape_of(layout, B, H, Sq, d))
        k = rand(rng, shape_of(layout, B, H, Sk, d))
        v = rand(rng, shape_of(layout, B, H, Sk, d))
        lens = np.array([14, 6], dtype=np.int32)
        o, lse = orc.attention(q, k, v, scale=0.3, causal=True, layout=layout, kv_len=lens)
        rows = rng.choice(B * H * Sq, size=12, replace=False)
        orow, lrow = orc.attention_rows(q, k, v, rows, scale=0.3, causal=True, layout=layout,
                                        kv_len=lens)
        ob = to_bhsd(o, layout)
        for n, r in enumerate(rows):
            i, h, b = r % Sq, (r // Sq) % H, r // (Sq * H)
            close(orow[n], ob[b, h, i], 0.0, "rows API output")
            close(lrow[n], lse[b, h, i], 0.0, "rows API LSE")



def _qkv_split(x64, w64, H, d, layout):
    """numpy reference of the projection: y = x w^T, columns split into
    (t, h, c) = (Q/K/V, head, dim), arranged in `layout`."""
    B, S, _ = x64.shape
    y = np.einsum("bsi,ni->bsn", x64, w64).reshape(B, S, 3, H, d)
    outs = []
    for t in range(3):
        yt = y[:, :, t]                      # [B, S, H, d]
        outs.append(yt if layout == "bshd" else np.transpose(yt, (0, 2, 1, 3)))
    return outs


def pin_qkv_identity(orc):
    """With D = H*d and the concatenated weight [I | 2I | 3I] the projections
    are x, 2x and 3x, each cut into heads of d consecutive columns: this fixes
    the order Q, K, V, the head split and both output layouts exactly."""
    rng = np.random.default_rng(21)
    for layout in ("bhsd", "bshd"):
        for (B, S, H, d) in [(2, 3, 2, 4), (1, 5, 3, 2)]:
            D_ = H * d
            x = rng.integers(-8, 9, size=(B, S, D_)).astype(np.float32)
            w = np.concatenate([np.eye(D_) * (t + 1) for t in range(3)]).astype(np.float32)
            q, k, v = orc.qkv_proj(x, w, H=H, d=d, layout=layout)
            heads = x.reshape(B, S, H, d)
            want = heads if layout == "bshd" else np.transpose(heads, (0, 2, 1, 3))
            for t, got in enumerate((q, k, v)):
                assert np.array_equal(got, (t + 1) * want), f"qkv identity {layout} output {t}"


def pin_qkv_library(orc):
    """Library cross-check: numpy's einsum of x with the weight, in float64,
    for random inputs in every storage type and both layouts."""
    rng = np.random.default_rng(22)
    for layout in ("bhsd", "bshd"):
        for dt in (torch.float32, torch.float16, torch.bfloat16):
            B, S, D_, H, d = 2, 7, 24, 3, 4
            x = torch.from_numpy(rand(rng, (B, S, D_))).to(dt)
            w = torch.from_numpy(rand(rng, (3 * H * d, D_))).to(dt)
            got = orc.qkv_proj(x, w, H=H, d=d, layout=layout)
            want = _qkv_split(f64(x), f64(w), H, d, layout)
            for t in range(3):
                close(got[t], want[t], 1e-12, f"qkv vs einsum {layout} {dt} output {t}")



def pin_softmax_rows_closed_forms(orc):
    """Row softmax: the page's row [1.0, 2.0, 0.5, 3.0] against the 50-digit
    closed form, rows summing to 1, the +1000 shift (a max-free softmax
    overflows, this one may not), scale 0 giving uniform rows, -inf entries
    taking no weight and an all -inf row giving 0 and lse = -inf."""
    with open(os.path.join(GOLDEN, "online_softmax_row.json")) as f:
        s = json.load(f)["scores"]
    z = sum((_CTX.exp(D(x)) for x in s), D(0))
    y, lse = orc.softmax_rows(np.array([s], dtype=np.float32))
    close(y[0], [float(_CTX.exp(D(x)) / z) for x in s], 1e-15, "page row softmax")
    close(lse[0], float(_CTX.ln(z)), 1e-15, "page row lse")
    rng = np.random.default_rng(31)
    # multiples of 2^-8, so that x + 1000 is exact in float32
    x = (np.round(rand(rng, (6, 37)) * 3 * 256) / 256).astype(np.float32)
    for sc in (1.0, 0.37):
        y, lse = orc.softmax_rows(x, scale=sc)
        close(y.sum(axis=1), np.ones(6), 1e-13, "row sums")
        y2, lse2 = orc.softmax_rows(x + np.float32(1000.0), scale=sc)
        close(y2, y, 1e-9, "shift by +1000")
        close(lse2, lse + sc * 1000.0, 1e-9, "lse shift by +1000")
    y, lse = orc.softmax_rows(x, scale=0.0)
    close(y, np.full(x.shape, 1.0 / 37), 1e-15, "scale 0 is uniform")
    close(lse, np.full(6, math.log(37)), 1e-13, "scale 0 lse")
    xm = x.copy()
    xm[0, 5:] = -np.inf
    xm[1, :] = -np.inf
    y, lse = orc.softmax_rows(xm)
    close(y[0, 5:], np.zeros(32), 0.0, "-inf entries take no weight")
    y0, _ = orc.softmax_rows(x[:1, :5].copy())
    close(y[0, :5], y0[0], 1e-15, "-inf entries leave the rest unchanged")
    close(y[1], np.zeros(37), 0.0, "all -inf row")
    assert lse[1] == -np.inf, "all -inf row lse"


def pin_softmax_rows_torch(orc):
    """Library cross-check: torch.softmax / logsumexp in float64 on the
    decoded inputs, all storage types."""
    rng = np.random.default_rng(32)
    for dt in (torch.float32, torch.float16, torch.bfloat16):
        x = torch.from_numpy(rand(rng, (5, 129)) * 4).to(dt)
        y, lse = orc.softmax_rows(x, scale=0.6)
        xs = x.to(torch.float64) * 0.6
        close(y, torch.softmax(xs, dim=1).numpy(), 1e-14, f"softmax vs torch {dt}")
        close(lse, torch.logsumexp(xs, dim=1).numpy(), 1e-12, f"lse vs torch {dt}")



def _split_from_bhsd(x: np.ndarray, g: int) -> np.ndarray:
    """[B, H, S, d] -> [B, H/g, S, g, d] (groups of g heads)."""
    B, H, S, d = x.shape
    return np.ascontiguousarray(x.reshape(B, H // g, g, S, d).transpose(0, 1, 3, 2, 4))


def pin_split_layout(orc):
    """The page's head-group ("Split") layout [B, H/g, S, g, d] holds the same
    heads: attention and the QKV projection in it equal their [B,H,S,d]
    results moved to that order, exactly, for g = 1, 2 and H."""
    rng = np.random.default_rng(41)
    B, H, S, d = 2, 4, 9, 8
    q, k, v = (rand(rng, (B, H, S, d)) for _ in range(3))
    o_ref, lse_ref = orc.attention(q, k, v, scale=0.3, causal=True, layout="bhsd", kv_len=[9, 5])
    for g in (1, 2, H):
        qs, ks, vs = (_split_from_bhsd(x, g) for x in (q, k, v))
        o, lse = orc.attention(qs, ks, vs, scale=0.3, causal=True, layout=f"split:{g}", kv_len=[9, 5])
        assert np.array_equal(o, _split_from_bhsd(o_ref, g)), f"split:{g} attention"
        assert np.array_equal(lse, lse_ref), f"split:{g} lse"
    x = rand(rng, (B, S, 16))
    w = rand(rng, (3 * H * d, 16))
    ref = orc.qkv_proj(x, w, H=H, d=d, layout="bhsd")
    for g in (1, 2, H):
        got = orc.qkv_proj(x, w, H=H, d=d, layout=f"split:{g}")
        for t in range(3):
            assert np.array_equal(got[t], _split_from_bhsd(ref[t], g)), f"split:{g} projection {t}"


ALL_PINS = [
    pin_decode_exact,
    pin_rows_sum_to_one,
    pin_zero_query_mean,
    pin_dominant_key,
    pin_online_worked_example,
    pin_brute_force,
    pin_shift_invariance,
    pin_permutation,
    pin_value_linearity,
    pin_causal_edges,
    pin_split_merge,
    pin_torch_sdpa,
    pin_empty_rows,
    pin_rows_api,
    pin_qkv_identity,
    pin_qkv_library,
    pin_softmax_rows_closed_forms,
    pin_softmax_rows_torch,
    pin_split_layout,
]
