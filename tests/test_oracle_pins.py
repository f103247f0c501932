"""Pins of the CPU oracle against things other than itself.

Each pin checks one oracle function against brute force on tiny inputs, a
library routine (torch's scaled_dot_product_attention and softmax in float64),
a closed form, or hand-worked values stored under tests/golden/. The pins
are written as functions of an oracle namespace so that the planted-mistake
tests at the bottom can hand them deliberately broken copies (on the CPU) and
show that each plausible slip fails at least one pin.
"""
import math
import os
import types

import numpy as np
import pytest
import torch

import oracle as real_oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _ns(**over):
    names = ["Q_BLOCK", "K_BLOCK", "num_blocks", "default_scale", "topk_count", "pool_blocks",
             "block_logits", "row_softmax", "select_topk", "predict_mask", "selected_keys",
             "attend_rows", "masked_attention", "masked_attention_rows", "compact_mask", "mask_parity",
             "causal_key_blocks", "cube_permutation", "morton_code", "morton_permutation",
             "permute_tokens", "select_cdf", "predict_mask_cdf", "mask_parity_cdf",
             "masked_attention_sampled"]
    d = {n: getattr(real_oracle, n) for n in names}
    d.update(over)
    return types.SimpleNamespace(**d)


def _golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def _sdpa(q, k, v, scale, bool_mask=None, is_causal=False):
    """torch's scaled_dot_product_attention in float64 on the CPU."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    m = None if bool_mask is None else torch.from_numpy(bool_mask)
    return torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=m, scale=scale, is_causal=is_causal).numpy()


def _expand(mask, n):
    """Token-level boolean mask (..., N, N) from a (..., Qb, Kb) block mask."""
    rq = np.minimum(np.arange(n) // 128, mask.shape[-2] - 1)
    ck = np.minimum(np.arange(n) // 64, mask.shape[-1] - 1)
    return mask[..., rq[:, None], ck[None, :]].astype(bool)


# --------------------------------------------------------------------------- pins

def pin_block_counts(o):
    for seq, qb, kb in _golden("mask_shapes.txt"):
        assert o.num_blocks(int(seq), o.Q_BLOCK) == int(qb), seq
        assert o.num_blocks(int(seq), o.K_BLOCK) == int(kb), seq


def pin_topk_count(o):
    for kb, topk, k in _golden("topk_counts.txt"):
        assert o.topk_count(int(kb), float(topk)) == int(k), (kb, topk)
    for bad in (0.0, -0.1, 1.5, float("nan")):
        with pytest.raises(ValueError):
            o.topk_count(10, bad)


def pin_pool(o):
    rng = np.random.default_rng(1)
    for n in (1, 63, 64, 65, 200, 300):
        x = rng.standard_normal((2, n, 5))
        for rows in (o.Q_BLOCK, o.K_BLOCK):
            got = o.pool_blocks(x, rows)
            nb = -(-n // rows)
            assert got.shape == (2, nb, 5)
            for b in range(2):
                for i in range(nb):
                    members = [r for r in range(n) if r // rows == i]
                    for d in range(5):
                        ref = sum(x[b, r, d] for r in members) / len(members)
                        assert abs(got[b, i, d] - ref) <= 1e-12 * (1 + abs(ref))
    # a block of identical rows pools to that row; aligned N equals reshape-mean
    x = np.repeat(rng.standard_normal((1, 1, 7)), 300, axis=1)
    assert np.allclose(o.pool_blocks(x, 128), x[:, :3], rtol=0, atol=1e-14)
    x = rng.standard_normal((3, 256, 4))
    assert np.allclose(o.pool_blocks(x, 64), x.reshape(3, 4, 64, 4).mean(axis=2), rtol=0, atol=1e-14)


def pin_scores(o):
    rng = np.random.default_rng(2)
    qb = rng.standard_normal((2, 3, 6))
    kb = rng.standard_normal((2, 5, 6))
    s = o.block_logits(qb, kb, 0.37)
    for b in range(2):
        for i in range(3):
            for j in range(5):
                ref = 0.37 * sum(qb[b, i, d] * kb[b, j, d] for d in range(6))
                assert abs(s[b, i, j] - ref) <= 1e-13
    p = o.row_softmax(s)
    assert np.allclose(p.sum(-1), 1.0, rtol=0, atol=1e-12)
    ref = torch.softmax(torch.from_numpy(s), dim=-1).numpy()
    assert np.allclose(p, ref, rtol=0, atol=1e-14)


def pin_select(o):
    rng = np.random.default_rng(3)
    for kb in (1, 2, 7, 33):
        p = rng.standard_normal((4, kb))
        p[0, : kb // 2] = p[0, kb // 2: 2 * (kb // 2)]   # exact duplicates in one row
        p[1, :] = 0.25                                   # a row that is all ties
        for k in sorted({1, max(1, kb // 3), kb}):
            m = o.select_topk(p, k)
            assert m.dtype == np.uint8 and set(np.unique(m)) <= {0, 1}
            for r in range(4):
                brute = sorted(range(kb), key=lambda j: (-p[r, j], j))[:k]
                ref = np.zeros(kb, dtype=np.uint8)
                ref[brute] = 1
                assert (m[r] == ref).all(), (kb, k, r)
                assert m[r].sum() == k


def pin_predict(o):
    rng = np.random.default_rng(4)
    n, d = 300, 16
    q = rng.standard_normal((1, 2, n, d))
    k = rng.standard_normal((1, 2, n, d))
    full = o.predict_mask(q, k, 1.0)
    assert full["mask"].shape == (1, 2, 3, 5) and full["mask"].all()
    r = o.predict_mask(q, k, 0.4)
    assert r["k"] == 2 and (r["mask"].sum(-1) == 2).all()
    # pooled means by brute force, then the kept set by brute force
    for h in range(2):
        for i in range(3):
            rows = range(128 * i, min(n, 128 * i + 128))
            qbar = np.mean([q[0, h, t] for t in rows], axis=0)
            sc = []
            for j in range(5):
                cols = range(64 * j, min(n, 64 * j + 64))
                kbar = np.mean([k[0, h, t] for t in cols], axis=0)
                sc.append(float(np.dot(qbar, kbar)) / math.sqrt(d))
            keep = sorted(range(5), key=lambda j: (-sc[j], j))[:2]
            assert sorted(np.flatnonzero(r["mask"][0, h, i]).tolist()) == sorted(keep)
    # selecting on the logits gives the same set as on the probabilities
    s = r["logits"].reshape(-1, 5)
    for row, mrow in zip(s, r["mask"].reshape(-1, 5)):
        keep = sorted(range(5), key=lambda j: (-row[j], j))[:2]
        assert sorted(np.flatnonzero(mrow).tolist()) == sorted(keep)


def pin_predict_ties(o):
    """Bit-identical key blocks: the lower block index must win the last slot."""
    rng = np.random.default_rng(5)
    n, d = 256, 8
    q = np.repeat(rng.standard_normal((1, 1, 1, d)), n, axis=2)
    k = rng.standard_normal((1, 1, n, d))
    k[0, 0, 192:256] = k[0, 0, 64:128]          # block 3 == block 1
    s = (q[0, 0, 0] @ k[0, 0].reshape(4, 64, d).mean(1).T)
    order = sorted(range(4), key=lambda j: (-s[j], j))
    # choose topk so the cut falls between the two equal blocks
    pos = order.index(1)
    kk = pos + 1
    r = o.predict_mask(q, k, kk / 4.0)
    assert r["mask"][0, 0, 0, 1] == 1 and r["mask"][0, 0, 0, 3] == 0
    assert r["mask"][0, 0].sum(-1).tolist() == [kk, kk]


def pin_attention(o):
    rng = np.random.default_rng(6)
    for n, d in ((200, 8), (256, 16), (131, 4)):
        q = rng.standard_normal((1, 2, n, d))
        k = rng.standard_normal((1, 2, n, d))
        v = rng.standard_normal((1, 2, n, d))
        qb, kb = -(-n // 128), -(-n // 64)
        sc = 1.0 / math.sqrt(d)
        # all-ones mask equals dense SDPA
        ones = np.ones((1, 2, qb, kb), dtype=np.uint8)
        assert np.abs(o.masked_attention(q, k, v, ones) - _sdpa(q, k, v, sc)).max() <= 1e-12
        # a random block mask (no empty row) equals SDPA with the token-level mask
        m = (rng.random((1, 2, qb, kb)) < 0.5).astype(np.uint8)
        m[..., 0, kb - 1] = 1
        m[..., :, 0] |= (m.sum(-1) == 0)
        ref = _sdpa(q, k, v, sc, _expand(m, n))
        got = o.masked_attention(q, k, v, m)
        assert np.abs(got - ref).max() <= 1e-12
        # an explicit scale is honoured
        got2 = o.masked_attention(q, k, v, m, scale=0.05)
        assert np.abs(got2 - _sdpa(q, k, v, 0.05, _expand(m, n))).max() <= 1e-12
        # brute-force triple loop on a few rows, including the ragged tail
        for row in (0, n - 1, min(n - 1, 130)):
            i = row // 128
            cols = [c for c in range(n) if m[0, 1, i, c // 64]]
            lg = [sc * sum(q[0, 1, row, t] * k[0, 1, c, t] for t in range(d)) for c in cols]
            mx = max(lg)
            w = [math.exp(x - mx) for x in lg]
            z = sum(w)
            for t in range(d):
                ref_t = sum(wi * v[0, 1, c, t] for wi, c in zip(w, cols)) / z
                assert abs(got[0, 1, row, t] - ref_t) <= 1e-12
        # one selected tile per row equals SDPA over that 64-key slice
        one = np.zeros_like(m)
        one[..., :, kb - 1] = 1
        lo = 64 * (kb - 1)
        ref = _sdpa(q, k[..., lo:, :], v[..., lo:, :], sc)
        assert np.abs(o.masked_attention(q, k, v, one) - ref).max() <= 1e-12


def pin_attention_closed_forms(o):
    rng = np.random.default_rng(7)
    n, d = 300, 6
    q = rng.standard_normal((1, 1, n, d))
    k = rng.standard_normal((1, 1, n, d))
    v = np.broadcast_to(rng.standard_normal((1, 1, 1, d)), (1, 1, n, d)).copy()
    m = (rng.random((1, 1, 3, 5)) < 0.6).astype(np.uint8)
    m[..., :, 4] = 1
    # constant V: the output is that constant
    assert np.abs(o.masked_attention(q, k, v, m) - v).max() <= 1e-12
    # zero queries: uniform weights, the output is the mean of the selected V rows
    v = rng.standard_normal((1, 1, n, d))
    z = np.zeros_like(q)
    out = o.masked_attention(z, k, v, m)
    for i in range(3):
        cols = [c for c in range(n) if m[0, 0, i, c // 64]]
        ref = np.mean(v[0, 0, cols], axis=0)
        assert np.abs(out[0, 0, 128 * i: min(n, 128 * i + 128)] - ref).max() <= 1e-12
    # an empty mask row outputs zeros
    m2 = m.copy()
    m2[..., 1, :] = 0
    out = o.masked_attention(q, k, v, m2)
    assert (out[0, 0, 128:256] == 0).all()
    # the order in which the selected keys are visited does not matter
    cols = [c for c in range(n) if m[0, 0, 0, c // 64]]
    perm = rng.permutation(cols)
    ref = _sdpa(q[..., :128, :], k[..., perm, :], v[..., perm, :], 1 / math.sqrt(d))
    assert np.abs(o.masked_attention(q, k, v, m)[..., :128, :] - ref).max() <= 1e-12


def pin_attention_rows(o):
    rng = np.random.default_rng(8)
    n, d = 333, 8
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    m = (rng.random((3, 6)) < 0.5).astype(np.uint8)
    m[:, 5] = 1
    rows = np.array([0, 5, 127, 128, 255, 256, 332])
    got = o.masked_attention_rows(q, k, v, m, rows)
    ref = _sdpa(q[None, None], k[None, None], v[None, None], 1 / math.sqrt(d), _expand(m, n))[0, 0][rows]
    assert np.abs(got - ref).max() <= 1e-12


def pin_attention_sampled(o):
    """Scattered rows, each against torch SDPA in float64 with the token-level mask."""
    rng = np.random.default_rng(18)
    for n, d in ((333, 8), (200, 16)):
        q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
        qb, kb = -(-n // 128), -(-n // 64)
        m = (rng.random((qb, kb)) < 0.5).astype(np.uint8)
        m[:, kb - 1] = 1
        rows = np.array(sorted({0, 5, 127, 128, min(n - 1, 255), n - 1, n // 2}))
        sc = 1 / math.sqrt(d)
        ref = _sdpa(q[None, None], k[None, None], v[None, None], sc, _expand(m, n))[0, 0][rows]
        got = o.masked_attention_sampled(q, k, v, m, rows, chunk=3)
        assert np.abs(got - ref).max() <= 1e-12
        assert np.abs(got - o.masked_attention_rows(q, k, v, m, rows)).max() <= 1e-12
        # an explicit scale, and rows given in any order
        perm = rows[::-1]
        got = o.masked_attention_sampled(q, k, v, m, perm, scale=0.3)
        ref = _sdpa(q[None, None], k[None, None], v[None, None], 0.3, _expand(m, n))[0, 0][perm]
        assert np.abs(got - ref).max() <= 1e-12
        # causal: the token mask AND the lower triangle; a row whose kept keys all
        # lie after it outputs zeros
        mc = m.copy()
        mc[0] = 0
        mc[0, 1] = 1                                    # block 0 sees only keys 64..127
        tok = _expand(mc, n) & np.tril(np.ones((n, n), dtype=bool))
        got = o.masked_attention_sampled(q, k, v, mc, rows, causal=True)
        for i, r in enumerate(rows):
            if tok[r].any():
                ref = _sdpa(q[None, None, r:r + 1], k[None, None], v[None, None], sc,
                            tok[None, None, r:r + 1])[0, 0, 0]
                assert np.abs(got[i] - ref).max() <= 1e-12
            else:
                assert (got[i] == 0).all()
        assert (got[0] == 0).all() and (got[1] == 0).all()   # rows 0 and 5 see no kept key
        # an empty mask row outputs zeros
        me = m.copy()
        me[1] = 0
        got = o.masked_attention_sampled(q, k, v, me, np.array([128, min(n - 1, 200)]))
        assert (got == 0).all()


def pin_compact(o):
    rng = np.random.default_rng(9)
    m = (rng.random((2, 3, 9)) < 0.4).astype(np.uint8)
    m[0, 0] = 0
    idx, cnt = o.compact_mask(m)
    for a in range(2):
        for b in range(3):
            ref = [j for j in range(9) if m[a, b, j]]
            assert cnt[a, b] == len(ref)
            assert idx[a, b, : len(ref)].tolist() == ref
            assert (idx[a, b, len(ref):] == -1).all()


def pin_mask_parity(o):
    s = np.array([[0.5, 0.4, 0.3, 0.1],              # well separated
                  [0.5, 0.400001, 0.400000, 0.1],    # near tie at the cut (k=2)
                  [0.9, 0.2, 0.1, 0.0]])
    om = np.array([[1, 1, 0, 0], [1, 1, 0, 0], [1, 1, 0, 0]], dtype=np.uint8)
    rep = o.mask_parity(s, om, om, 2)
    assert rep["failures"] == 0 and rep["candidates"] == 1 and rep["differing"] == 0
    dm = om.copy()
    dm[1] = [1, 0, 1, 0]                              # swap inside the near-tie band: allowed
    rep = o.mask_parity(s, om, dm, 2)
    assert rep["failures"] == 0 and rep["differing"] == 1
    dm = om.copy()
    dm[0] = [1, 0, 1, 0]                              # swap in a separated row: caught
    assert o.mask_parity(s, om, dm, 2)["failures"] == 1
    dm = om.copy()
    dm[1] = [1, 1, 1, 0]                              # wrong count in a near-tie row: caught
    assert o.mask_parity(s, om, dm, 2)["failures"] == 1
    dm = om.copy()
    dm[1] = [0, 1, 1, 0]                              # drops a clear winner: caught
    assert o.mask_parity(s, om, dm, 2)["failures"] == 1


def pin_causal_attention(o):
    rng = np.random.default_rng(10)
    for n, d in ((200, 8), (131, 4), (256, 16)):
        q, k, v = (rng.standard_normal((1, 2, n, d)) for _ in range(3))
        qb, kb = -(-n // 128), -(-n // 64)
        sc = 1.0 / math.sqrt(d)
        tril = np.tril(np.ones((n, n), dtype=bool))
        # all blocks kept: torch's causal SDPA
        ones = np.ones((1, 2, qb, kb), dtype=np.uint8)
        ref = _sdpa(q, k, v, sc, is_causal=True)
        assert np.abs(o.masked_attention(q, k, v, ones, causal=True) - ref).max() <= 1e-12
        # a random block mask that keeps block 0 (key 0 is visible to every row)
        m = (rng.random((1, 2, qb, kb)) < 0.5).astype(np.uint8)
        m[..., :, 0] = 1
        got = o.masked_attention(q, k, v, m, causal=True)
        assert np.abs(got - _sdpa(q, k, v, sc, _expand(m, n) & tril)).max() <= 1e-12
        # brute force on a few rows
        for row in (0, 63, 64, n - 1):
            i = row // 128
            cols = [c for c in range(n) if m[0, 1, i, c // 64] and c <= row]
            lg = [sc * sum(q[0, 1, row, t] * k[0, 1, c, t] for t in range(d)) for c in cols]
            mx = max(lg)
            w = [math.exp(x - mx) for x in lg]
            z = sum(w)
            for t in range(d):
                assert abs(got[0, 1, row, t] - sum(wi * v[0, 1, c, t] for wi, c in zip(w, cols)) / z) <= 1e-12
        # rows that see no kept key output zeros; the rest follow the masked SDPA
        late = np.zeros_like(m)
        late[..., :, kb - 1] = 1
        out = o.masked_attention(q, k, v, late, causal=True)
        first = 64 * (kb - 1)
        assert (out[..., :first, :] == 0).all()
        ref = _sdpa(q[..., first:, :], k[..., first:, :], v[..., first:, :], sc, is_causal=True)
        assert np.abs(out[..., first:, :] - ref).max() <= 1e-12
        # the row-sampled form agrees
        rows = np.array([0, 1, 64, n - 1])
        assert np.abs(o.masked_attention_rows(q[0, 0], k[0, 0], v[0, 0], m[0, 0], rows, causal=True)
                      - got[0, 0][rows]).max() <= 1e-12


def pin_causal_predict(o):
    # candidate blocks: brute force over (row, key) pairs
    for n in (1, 63, 64, 65, 128, 129, 200, 256, 300, 1000):
        qb, kb = -(-n // 128), -(-n // 64)
        for i in range(qb):
            seen = set()
            for r in range(128 * i, min(n, 128 * i + 128)):
                for c in range(0, r + 1):
                    seen.add(c // 64)
            assert o.causal_key_blocks(n, i) == len(seen) == max(seen) + 1
    rng = np.random.default_rng(11)
    n, d = 700, 8
    q, k = rng.standard_normal((1, 2, n, d)), rng.standard_normal((1, 2, n, d))
    qb, kb = -(-n // 128), -(-n // 64)
    full = o.predict_mask(q, k, 1.0, causal=True)
    for i in range(qb):
        c = 2 * i + 2 if 128 * i + 127 < n else kb
        assert full["mask"][..., i, :c].all() and not full["mask"][..., i, c:].any()
    for topk in (0.3, 0.55):
        r = o.predict_mask(q, k, topk, causal=True)
        s = np.einsum("bhid,bhjd->bhij", o.pool_blocks(q, 128), o.pool_blocks(k, 64)) / math.sqrt(d)
        for i in range(qb):
            c = o.causal_key_blocks(n, i)
            kk = max(1, min(c, math.ceil(topk * c - 1e-9)))
            assert int(r["k"][i]) == kk
            for h in range(2):
                order = sorted(range(c), key=lambda j: (-s[0, h, i, j], j))[:kk]
                assert sorted(np.flatnonzero(r["mask"][0, h, i]).tolist()) == sorted(order)
    # parity: a device row keeping a block outside its candidates fails
    r = o.predict_mask(q, k, 0.3, causal=True)
    dm = r["mask"].copy()
    dm[0, 0, 0, :] = 0
    dm[0, 0, 0, kb - 1] = 1
    dm[0, 0, 0, 0] = 1
    rep = o.mask_parity(r["logits"], r["mask"], dm, r["k"], cand=r["cand"])
    assert rep["failures"] >= 1
    assert o.mask_parity(r["logits"], r["mask"], r["mask"], r["k"], cand=r["cand"])["failures"] == 0


def pin_token_layouts(o):
    for row in _golden("token_layouts.txt"):
        colon = row.index(":")
        head, want = row[:colon], [int(x) for x in row[colon + 1:]]
        if head[0] == "cube":
            n_text, T, H, W, ct, ch, cw = (int(x) for x in head[1:])
            got = o.cube_permutation(n_text, T, H, W, (ct, ch, cw))
        else:
            n_text, T, H, W = (int(x) for x in head[1:])
            got = o.morton_permutation(n_text, T, H, W)
        assert got.tolist() == want, head
    # bijections on ragged grids
    for n_text, T, H, W in ((0, 5, 6, 7), (3, 4, 9, 13), (226, 3, 6, 9)):
        n = n_text + T * H * W
        for perm in (o.cube_permutation(n_text, T, H, W), o.morton_permutation(n_text, T, H, W)):
            assert sorted(perm.tolist()) == list(range(n))
            assert perm[:n_text].tolist() == list(range(n_text))
    # full 4x4x4 cubes are 64 consecutive positions covering one box
    T, H, W = 8, 8, 12
    perm = o.cube_permutation(0, T, H, W)
    for c in range(T * H * W // 64):
        tok = perm[64 * c: 64 * c + 64]
        t, h, w = tok // (H * W), (tok // W) % H, tok % W
        assert np.ptp(t) == 3 and np.ptp(h) == 3 and np.ptp(w) == 3
        assert t.min() % 4 == 0 and h.min() % 4 == 0 and w.min() % 4 == 0
    # Morton on a 4x4x4 grid: every aligned group of 8 is a 2x2x2 box, the first one at the corner
    perm = o.morton_permutation(0, 4, 4, 4)
    for g in range(8):
        tok = perm[8 * g: 8 * g + 8]
        t, h, w = tok // 16, (tok // 4) % 4, tok % 4
        assert np.ptp(t) == 1 and np.ptp(h) == 1 and np.ptp(w) == 1
    assert sorted(perm[:8].tolist()) == [0, 1, 4, 5, 16, 17, 20, 21]
    assert o.morton_code(1, 0, 0) == 4 and o.morton_code(0, 1, 0) == 2 and o.morton_code(0, 0, 2) == 8
    # gather / scatter round trip, and scatter equals the gather by the inverse permutation
    rng = np.random.default_rng(12)
    x = rng.standard_normal((2, 3, 226 + 3 * 6 * 9, 4))
    perm = o.cube_permutation(226, 3, 6, 9)
    y = o.permute_tokens(x, perm)
    assert np.array_equal(y[..., 5, :], x[..., perm[5], :])
    assert np.array_equal(o.permute_tokens(y, perm, inverse=True), x)
    assert np.array_equal(o.permute_tokens(y, perm, inverse=True), y[..., np.argsort(perm), :])
    # dense non-causal attention commutes with a token permutation applied to q, k and v
    q, k, v = (rng.standard_normal((1, 1, 300, 8)) for _ in range(3))
    perm = o.morton_permutation(12, 2, 8, 18)
    ones = np.ones((1, 1, 3, 5), dtype=np.uint8)
    a = o.masked_attention(o.permute_tokens(q, perm), o.permute_tokens(k, perm), o.permute_tokens(v, perm), ones)
    assert np.abs(o.permute_tokens(a, perm, inverse=True) - o.masked_attention(q, k, v, ones)).max() <= 1e-12


def pin_cdf_select(o):
    for row in _golden("cdf_select.txt"):
        text = " ".join(row)
        tau_s, p_s, keep_s = (x.strip() for x in text.split(":"))
        p = np.array([float(x) for x in p_s.split()])
        m = o.select_cdf(p[None], float(tau_s))[0]
        assert np.flatnonzero(m).tolist() == [int(x) for x in keep_s.split()], text
    rng = np.random.default_rng(13)
    p = rng.dirichlet(np.full(40, 0.3), size=50)
    prev = None
    for tau in (0.05, 0.3, 0.6, 0.9, 0.999, 1.0):
        m = o.select_cdf(p, tau)
        for r in range(p.shape[0]):
            kept = np.flatnonzero(m[r])
            k = kept.size
            # the kept set is the k largest (lower index on ties) ...
            assert sorted(kept.tolist()) == sorted(np.argsort(-p[r], kind="stable")[:k].tolist())
            # ... reaches tau, and one block fewer would not
            srt = np.sort(p[r])[::-1]
            if tau < 1.0:
                assert srt[:k].sum() >= tau and (k == 1 or srt[:k - 1].sum() < tau)
            else:
                assert k == p.shape[1]
        if prev is not None:
            assert (m >= prev).all()          # nested as tau grows
        prev = m
    # the CDF mask equals the top-k mask of its own count
    q, k = rng.standard_normal((1, 2, 500, 8)), rng.standard_normal((1, 2, 500, 8))
    r = o.predict_mask_cdf(q, k, 0.6)
    for h in range(2):
        for i in range(r["mask"].shape[2]):
            kk = int(r["mask"][0, h, i].sum())
            assert (o.select_topk(r["probs"][0, h, i][None], kk)[0] == r["mask"][0, h, i]).all()
    rc = o.predict_mask_cdf(q, k, 0.6, causal=True)
    for i in range(rc["mask"].shape[2]):
        assert not rc["mask"][..., i, rc["cand"][i]:].any()
    # parity: exact rows, a cut shifted inside the mass band, and real mistakes
    pr = np.array([[0.5, 0.3, 0.2]])
    lg = np.log(pr)
    tau = 0.8 + 1e-7
    om = o.select_cdf(pr, tau)
    assert om[0].tolist() == [1, 1, 1]
    assert o.mask_parity_cdf(lg, pr, om, om, tau)["failures"] == 0
    assert o.mask_parity_cdf(lg, pr, om, np.array([[1, 1, 0]]), tau)["failures"] == 0
    assert o.mask_parity_cdf(lg, pr, om, np.array([[1, 0, 1]]), tau)["failures"] == 1
    assert o.mask_parity_cdf(lg, pr, om, np.array([[1, 0, 0]]), tau)["failures"] == 1


PINS = [pin_block_counts, pin_topk_count, pin_pool, pin_scores, pin_select, pin_predict,
        pin_predict_ties, pin_attention, pin_attention_closed_forms, pin_attention_rows,
        pin_compact, pin_mask_parity, pin_causal_attention, pin_causal_predict, pin_token_layouts, pin_cdf_select,
        pin_attention_sampled]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(_ns())


# --------------------------------------------------------------- planted mistakes

def _broken_variants():
    o = real_oracle
    import oracle.sparge_oracle as src

    def pool_full_divisor(x, rows):
        x = np.asarray(x, dtype=np.float64)
        n, d = x.shape[-2], x.shape[-1]
        nb = -(-n // rows)
        out = np.empty(x.shape[:-2] + (nb, d))
        for i in range(nb):
            out[..., i, :] = x[..., i * rows:(i + 1) * rows, :].sum(-2) / rows
        return out

    def pool_drops_tail(x, rows):
        n = x.shape[-2]
        return o.pool_blocks(x[..., : max(rows, (n // rows) * rows), :], rows)

    def logits_no_scale(qb, kb, scale):
        return np.matmul(qb, np.swapaxes(kb, -1, -2))

    def softmax_wrong_axis(s):
        e = np.exp(s - s.max(axis=-2, keepdims=True))
        return e / e.sum(axis=-2, keepdims=True)

    def select_high_index_ties(p, k):
        flat = np.asarray(p).reshape(-1, p.shape[-1])
        m = np.zeros(flat.shape, dtype=np.uint8)
        for r in range(flat.shape[0]):
            order = np.argsort(-flat[r][::-1], kind="stable")
            m[r, (flat.shape[1] - 1 - order)[:k]] = 1
        return m.reshape(p.shape)

    def select_off_by_one(p, k):
        return o.select_topk(p, max(1, k - 1)) if k > 1 else o.select_topk(p, k)

    def topk_plain_ceil(kb, topk):
        if not (0 < topk <= 1):
            raise ValueError
        return max(1, min(kb, math.ceil(topk * kb)))

    def sampled_wrong_block(q_h, k_h, v_h, mask_h, rows, scale=None, causal=False, chunk=256):
        rows = np.asarray(rows)
        out = np.empty((rows.size, np.asarray(q_h).shape[1]))
        for i, r in enumerate(rows):
            m = np.zeros_like(np.asarray(mask_h))
            m[r // 128] = np.asarray(mask_h)[min(r // 64, m.shape[0] - 1)]
            out[i] = o.masked_attention_rows(q_h, k_h, v_h, m, [r], scale, causal)[0]
        return out

    def sampled_strict_causal(q_h, k_h, v_h, mask_h, rows, scale=None, causal=False, chunk=256):
        # the causal test written as c < r instead of c <= r
        q_h, k_h, v_h = (np.asarray(a, dtype=np.float64) for a in (q_h, k_h, v_h))
        n, d = q_h.shape
        sc = 1 / math.sqrt(d) if scale is None else scale
        rows = np.asarray(rows)
        kept = np.asarray(mask_h)[rows // 128][:, np.arange(n) // 64] != 0
        if causal:
            kept &= np.arange(n)[None, :] < rows[:, None]
        lg = np.where(kept, sc * (q_h[rows] @ k_h.T), -np.inf)
        anyk = kept.any(1)
        w = np.exp(lg - np.where(anyk, lg.max(1), 0.0)[:, None])
        return (w @ v_h) / np.where(anyk, w.sum(1), 1.0)[:, None]

    def attend_no_scale(qr, ks, vs, scale, rows=None, cols=None):
        return o.attend_rows(qr, ks, vs, 1.0, rows, cols)

    def attend_unnormalised(qr, ks, vs, scale, rows=None, cols=None):
        if ks.shape[0] == 0:
            return np.zeros((qr.shape[0], vs.shape[-1]))
        lg = scale * (qr @ ks.T)
        if rows is not None:
            lg = np.where(np.asarray(cols)[None, :] <= np.asarray(rows)[:, None], lg, -np.inf)
        return np.exp(lg - lg.max(-1, keepdims=True)) @ vs

    def selected_keys_wrong_block(mask_row, n):
        idx = []
        for j in np.flatnonzero(np.asarray(mask_row) != 0):
            idx.extend(range(j * 128, min(n, (j + 1) * 128)))
        return np.asarray(idx, dtype=np.int64)

    def selected_keys_drop_tail(mask_row, n):
        idx = []
        for j in np.flatnonzero(np.asarray(mask_row) != 0):
            if (j + 1) * 64 <= n:
                idx.extend(range(j * 64, (j + 1) * 64))
        return np.asarray(idx, dtype=np.int64)

    def attend_transposed_v(qr, ks, vs, scale, rows=None, cols=None):
        return o.attend_rows(qr, ks, ks, scale, rows, cols)   # uses K where V belongs

    def attend_causal_strict(qr, ks, vs, scale, rows=None, cols=None):
        if rows is None:
            return o.attend_rows(qr, ks, vs, scale)
        out = np.zeros((qr.shape[0], vs.shape[-1]))
        lg = scale * (qr @ ks.T)
        for r in range(qr.shape[0]):
            c = np.flatnonzero(np.asarray(cols) < rows[r])      # a row does not see its own key
            if c.size:
                out[r] = o.row_softmax(lg[r, c]) @ vs[c]
        return out

    def cube_w_major(n_text, T, H, W, cube=(4, 4, 4)):
        ct, ch, cw = cube
        perm = list(range(n_text))
        for t0 in range(0, T, ct):
            for h0 in range(0, H, ch):
                for w0 in range(0, W, cw):
                    for w in range(w0, min(W, w0 + cw)):
                        for h in range(h0, min(H, h0 + ch)):
                            for t in range(t0, min(T, t0 + ct)):
                                perm.append(n_text + (t * H + h) * W + w)
        return np.asarray(perm)

    def cube_drops_partial(n_text, T, H, W, cube=(4, 4, 4)):
        ct, ch, cw = cube
        perm = list(range(n_text))
        for t0 in range(0, T - ct + 1, ct):
            for h0 in range(0, H - ch + 1, ch):
                for w0 in range(0, W - cw + 1, cw):
                    for t in range(t0, t0 + ct):
                        for h in range(h0, h0 + ch):
                            for w in range(w0, w0 + cw):
                                perm.append(n_text + (t * H + h) * W + w)
        return np.asarray(perm)

    def morton_t_lowest(t, h, w):
        return o.morton_code(w, h, t)

    def inverse_as_gather(x, perm, inverse=False):
        return np.asarray(x)[..., np.asarray(perm), :]

    def cdf_strict(p, tau):
        p = np.asarray(p, dtype=np.float64)
        flat = p.reshape(-1, p.shape[-1])
        m = np.zeros(flat.shape, dtype=np.uint8)
        for r in range(flat.shape[0]):
            total = 0.0
            for j in np.argsort(-flat[r], kind="stable"):
                m[r, j] = 1
                total += flat[r, j]
                if total > tau or tau >= 1.0 and m[r].all():
                    break
        return m.reshape(p.shape)

    def _cdf_order(p, tau, ascending):
        p = np.asarray(p, dtype=np.float64)
        flat = p.reshape(-1, p.shape[-1])
        m = np.zeros(flat.shape, dtype=np.uint8)
        for r in range(flat.shape[0]):
            total = 0.0
            order = np.argsort(flat[r], kind="stable") if ascending else np.argsort(-flat[r], kind="stable")
            for j in order:
                m[r, j] = 1
                total += flat[r, j]
                if total >= tau:
                    break
        return m.reshape(p.shape)

    def cdf_ascending(p, tau):
        return _cdf_order(p, tau, ascending=True)

    def parity_cdf_no_mass_band(lg, pr, om, dm, tau, band=1e-5, mass_band=1e-5, cand=None):
        return o.mask_parity_cdf(lg, pr, om, dm, tau, band=band, mass_band=0.0, cand=cand)

    def causal_first_row(n, i):
        return (128 * i) // 64 + 1

    def causal_all_blocks(n, i):
        return -(-n // 64)

    def parity_no_band(logits, om, dm, k, band=1e-5, probs=None, cand=None):
        return o.mask_parity(logits, om, dm, k, band=0.0, probs=probs, cand=cand)

    return {
        "pool divides by the full block size": dict(pool_blocks=pool_full_divisor),
        "pool drops the ragged tail block": dict(pool_blocks=pool_drops_tail),
        "logits lose the scale": dict(block_logits=logits_no_scale),
        "softmax over the wrong axis": dict(row_softmax=softmax_wrong_axis),
        "ties go to the higher index": dict(select_topk=select_high_index_ties),
        "keeps k-1 blocks": dict(select_topk=select_off_by_one),
        "k without the integer guard": dict(topk_count=topk_plain_ceil),
        "attention without the scale": dict(attend_rows=attend_no_scale),
        "attention without normalisation": dict(attend_rows=attend_unnormalised),
        "key blocks of 128 rows": dict(selected_keys=selected_keys_wrong_block),
        "ragged last key block dropped": dict(selected_keys=selected_keys_drop_tail),
        "sampled rows take the mask row of the 64-row block": dict(masked_attention_sampled=sampled_wrong_block),
        "sampled causal rows exclude their own key": dict(masked_attention_sampled=sampled_strict_causal),
        "K used in place of V": dict(attend_rows=attend_transposed_v),
        "parity without the near-tie band": dict(mask_parity=parity_no_band),
        "causal row does not see its own key": dict(attend_rows=attend_causal_strict),
        "CDF stops only past tau": dict(select_cdf=cdf_strict),
        "CDF takes the smallest blocks first": dict(select_cdf=cdf_ascending),
        "CDF parity without the mass band": dict(mask_parity_cdf=parity_cdf_no_mass_band),
        "cube order w-major inside a cube": dict(cube_permutation=cube_w_major),
        "cube order drops the partial edge cubes": dict(cube_permutation=cube_drops_partial),
        "Morton code with t as the lowest bit": dict(morton_code=morton_t_lowest),
        "inverse permutation applied as a gather": dict(permute_tokens=inverse_as_gather),
        "causal candidates from the block's first row": dict(causal_key_blocks=causal_first_row),
        "causal candidates include future blocks": dict(causal_key_blocks=causal_all_blocks),
    }, src


def _run_with(over, src):
    """Run every pin with some oracle functions replaced, also inside the module."""
    saved = {name: getattr(src, name) for name in over}
    try:
        for name, fn in over.items():
            setattr(src, name, fn)
        failed = []
        for pin in PINS:
            try:
                pin(_ns(**{n: getattr(src, n) for n in over}))
            except Exception:
                failed.append(pin.__name__)
        return failed
    finally:
        for name, fn in saved.items():
            setattr(src, name, fn)


@pytest.mark.parametrize("mistake", list(_broken_variants()[0]))
def test_planted_mistake_is_caught(mistake):
    variants, src = _broken_variants()
    failed = _run_with(variants[mistake], src)
    assert failed, f"no pin caught: {mistake}"
