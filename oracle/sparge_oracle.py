"""Plain fp64 CPU oracle for SpargeAttn-style block-sparse self-attention.

TEST INFRASTRUCTURE. Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import or run this module. It shares no code
with the GPU path and the GPU path never calls it.

What it computes, in the order of the method:

1. Block mean pooling. Q is cut into 128-row blocks and K into 64-row blocks
   (the fixed 128x64 block size of SpargeAttention Documentation, "Mask
   Requirements"); each block is replaced by the mean of its rows. A ragged
   last block is averaged over the rows it really has.
2. Pooled block scoring. s[i, j] = scale * qbar_i . kbar_j and
   p[i, :] = softmax_j(s[i, :]) over all key blocks of the row.
3. Top-k selection. Each query block keeps the k = ceil(topk * n_kblocks) key
   blocks of largest p, ties going to the lowest key-block index. "topk" is the
   accuracy/sparsity knob of the recommended top-k API (SpargeAttention
   Documentation, the paragraph on spas_sage2_attn_meansim_topk_cuda). The
   result is mask_id of shape (B, H, ceil(N/128), ceil(N/64)) with 0/1 entries
   ("Mask Requirements").
4. Masked attention. For a query row in block i, the softmax runs over the
   keys of the selected key blocks only; the output is the softmax-weighted
   sum of their values. Non-causal, default scale 1/sqrt(D), since the API is
   a drop-in for torch's scaled_dot_product_attention (same page, top-k API
   paragraph and its is_causal=False call; block_sparse_sage2_attn_cuda for a
   given mask). Skipped blocks are never read: the "skip attention between
   tokens that don't meaningfully interact" idea of the Apply SpargeAttn page,
   opening section.

Causal variant (the API's is_causal flag, same paragraph; the pages give no
more): key c is visible to query row r when c <= r. Query block i may only
select the key blocks holding a key visible to one of its rows, j <= J(i) =
floor((last row of block i) / 64); it keeps ceil(topk * (J(i) + 1)) of them
(same rounding rule), ranked as above over those candidates only, and inside
the kept blocks each row attends to its visible keys only. A row left with no
visible kept key outputs zeros.

CDF-threshold selection (the inference scripts' "cdfthreshd" mode, SpargeAttention
Documentation, output-directory list; only the name and a value are given):
per query block, the key blocks are taken in decreasing softmax probability
(ties to the lower index) until their cumulative probability reaches the
threshold tau in (0, 1]; tau = 1 keeps every candidate. The number kept varies
from row to row.

Token layouts (optional, around the whole method; Official repository for
AB-Attention, "Optional cube layout"; Attention Mechanisms (LightX2V), Sol-Attn
on Wan2.1, "Tuning and implementation"): video tokens of a T x H x W grid,
stored raster order (w fastest) after a prefix of text tokens, may be reordered
before attention and restored after it, so that 128-query and 64-key blocks
cover compact spatiotemporal regions. Two orders are defined here: 4 x 4 x 4
cubes (cubes in raster order of the cube grid, tokens in raster order inside a
cube, partial cubes at the grid edges) and a Morton (Z-order) curve over
(t, h, w); text tokens keep their places.

Steps 1-3 are this build's plain reading of the API name meansim_topk: block
means, a similarity between them, top-k. The pages name the method but do not
spell it out. Step 4 is an exact mathematical result; any correct
implementation computes the same real numbers up to rounding.

Everything is float64 numpy; loops are plain Python over blocks.
"""
from __future__ import annotations

import math

import numpy as np

Q_BLOCK = 128   # query rows per block (SpargeAttention Documentation, "Mask Requirements")
K_BLOCK = 64    # key rows per block (same section)
TOPK_INT_GUARD = 1e-9


def num_blocks(n: int, rows: int) -> int:
    """ceil(n / rows): the mask dimensions ceil(seq_len/128) and ceil(seq_len/64)."""
    if n <= 0 or rows <= 0:
        raise ValueError("n and rows must be positive")
    return -(-n // rows)


def default_scale(d: int) -> float:
    """1/sqrt(D), the default of torch's scaled_dot_product_attention."""
    return 1.0 / math.sqrt(d)


def topk_count(n_kblocks: int, topk: float) -> int:
    """Number of key blocks each query block keeps: ceil(topk * n_kblocks).

    The product is taken in IEEE double; a product within 1e-9 of an integer
    counts as that integer (so 0.3 * 10 keeps 3 blocks, not 4). The result is
    clamped to [1, n_kblocks]. topk must lie in (0, 1].
    """
    if not (topk > 0.0 and topk <= 1.0):
        raise ValueError("topk must be in (0, 1]")
    x = float(topk) * float(n_kblocks)
    r = round(x)
    k = int(r) if abs(x - r) <= TOPK_INT_GUARD else int(math.ceil(x))
    return max(1, min(int(n_kblocks), k))


def pool_blocks(x: np.ndarray, rows: int) -> np.ndarray:
    """Mean of each run of `rows` consecutive tokens; x is (..., N, D) float64.

    Returns (..., ceil(N/rows), D). The last block divides by its real row count.
    """
    x = np.asarray(x, dtype=np.float64)
    n, d = x.shape[-2], x.shape[-1]
    nb = num_blocks(n, rows)
    out = np.empty(x.shape[:-2] + (nb, d), dtype=np.float64)
    for i in range(nb):
        lo, hi = i * rows, min(n, (i + 1) * rows)
        out[..., i, :] = x[..., lo:hi, :].sum(axis=-2) / float(hi - lo)
    return out


def block_logits(qbar: np.ndarray, kbar: np.ndarray, scale: float) -> np.ndarray:
    """s[..., i, j] = scale * sum_d qbar[..., i, d] * kbar[..., j, d]."""
    return float(scale) * np.matmul(qbar, np.swapaxes(kbar, -1, -2))


def row_softmax(s: np.ndarray) -> np.ndarray:
    """Softmax over the last axis: exp(s - max) / sum exp(s - max)."""
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=-1, keepdims=True)


def select_topk(p: np.ndarray, k: int) -> np.ndarray:
    """0/1 mask keeping, per row, the k largest entries; equal values go to the lower index."""
    p = np.asarray(p, dtype=np.float64)
    kb = p.shape[-1]
    if not 1 <= k <= kb:
        raise ValueError("k out of range")
    flat = p.reshape(-1, kb)
    mask = np.zeros(flat.shape, dtype=np.uint8)
    for r in range(flat.shape[0]):
        order = np.argsort(-flat[r], kind="stable")   # stable: ties keep ascending index
        mask[r, order[:k]] = 1
    return mask.reshape(p.shape)


def causal_key_blocks(n: int, i: int) -> int:
    """Key blocks 0 .. J(i) hold a key that some row of query block i may see
    under causal masking (key c visible to row r when c <= r); returns J(i) + 1,
    with J(i) = floor(last row of block i / 64)."""
    last_row = min(n, (i + 1) * Q_BLOCK) - 1
    return last_row // K_BLOCK + 1


def predict_mask(q: np.ndarray, k: np.ndarray, topk: float, scale: float | None = None,
                 causal: bool = False) -> dict:
    """Pool -> score -> select. q, k are (B, H, N, D) float64.

    Returns a dict with mask (uint8), logits s, probabilities p, the pooled
    qbar / kbar, the count k (an int, or with causal=True a per-query-block
    array) and the number of candidate key blocks per query block ("cand").
    With causal=True the softmax and the selection of query block i run over
    key blocks 0 .. J(i) only (see causal_key_blocks) and keep
    topk_count(J(i) + 1, topk) of them; the other entries of the row are 0.
    """
    n, d = q.shape[-2], q.shape[-1]
    scale = default_scale(d) if scale is None else float(scale)
    qbar = pool_blocks(q, Q_BLOCK)
    kbar = pool_blocks(k, K_BLOCK)
    s = block_logits(qbar, kbar, scale)
    n_qb, n_kb = qbar.shape[-2], kbar.shape[-2]
    if not causal:
        p = row_softmax(s)
        kk = topk_count(n_kb, topk)
        mask = select_topk(p, kk)
        return {"mask": mask, "logits": s, "probs": p, "qbar": qbar, "kbar": kbar, "k": kk,
                "cand": np.full(n_qb, n_kb, dtype=np.int64)}
    cand = np.array([causal_key_blocks(n, i) for i in range(n_qb)], dtype=np.int64)
    kk = np.array([topk_count(int(c), topk) for c in cand], dtype=np.int64)
    p = np.zeros_like(s)
    mask = np.zeros(s.shape, dtype=np.uint8)
    for i in range(n_qb):
        c = int(cand[i])
        p[..., i, :c] = row_softmax(s[..., i, :c])
        mask[..., i, :c] = select_topk(p[..., i, :c], int(kk[i]))
    return {"mask": mask, "logits": s, "probs": p, "qbar": qbar, "kbar": kbar, "k": kk, "cand": cand}


def select_cdf(p: np.ndarray, tau: float) -> np.ndarray:
    """0/1 mask keeping, per row, the fewest largest entries whose sum reaches tau
    (entries in decreasing order, equal values by lower index); tau >= 1 keeps all."""
    if not (tau > 0.0 and tau <= 1.0):
        raise ValueError("tau must be in (0, 1]")
    p = np.asarray(p, dtype=np.float64)
    kb = p.shape[-1]
    flat = p.reshape(-1, kb)
    mask = np.zeros(flat.shape, dtype=np.uint8)
    for r in range(flat.shape[0]):
        order = np.argsort(-flat[r], kind="stable")
        if tau >= 1.0:
            mask[r, :] = 1
            continue
        total = 0.0
        for j in order:
            mask[r, j] = 1
            total += flat[r, j]
            if total >= tau:
                break
    return mask.reshape(p.shape)


def predict_mask_cdf(q: np.ndarray, k: np.ndarray, tau: float, scale: float | None = None,
                     causal: bool = False) -> dict:
    """Pool -> score -> CDF-threshold selection (see select_cdf); with causal=True the
    softmax and the selection of query block i run over key blocks 0 .. J(i) only."""
    n, d = q.shape[-2], q.shape[-1]
    scale = default_scale(d) if scale is None else float(scale)
    qbar = pool_blocks(q, Q_BLOCK)
    kbar = pool_blocks(k, K_BLOCK)
    s = block_logits(qbar, kbar, scale)
    n_qb, n_kb = qbar.shape[-2], kbar.shape[-2]
    cand = np.array([causal_key_blocks(n, i) if causal else n_kb for i in range(n_qb)], dtype=np.int64)
    p = np.zeros_like(s)
    mask = np.zeros(s.shape, dtype=np.uint8)
    for i in range(n_qb):
        c = int(cand[i])
        p[..., i, :c] = row_softmax(s[..., i, :c])
        mask[..., i, :c] = select_cdf(p[..., i, :c], tau)
    return {"mask": mask, "logits": s, "probs": p, "qbar": qbar, "kbar": kbar, "cand": cand,
            "k": mask.sum(-1)}


def selected_keys(mask_row: np.ndarray, n: int) -> np.ndarray:
    """Token indices of the key blocks a 0/1 mask row selects (ascending)."""
    idx = []
    for j in np.flatnonzero(np.asarray(mask_row) != 0):
        idx.extend(range(j * K_BLOCK, min(n, (j + 1) * K_BLOCK)))
    return np.asarray(idx, dtype=np.int64)


def attend_rows(q_rows: np.ndarray, k_sel: np.ndarray, v_sel: np.ndarray, scale: float,
                row_ids: np.ndarray | None = None, col_ids: np.ndarray | None = None) -> np.ndarray:
    """Softmax attention of some query rows over one key/value set (float64).

    With row_ids / col_ids (token indices of the rows and of the keys) the
    attention is causal: row r only weighs keys c <= r; a row that sees no key
    outputs zeros.
    """
    out = np.zeros((q_rows.shape[0], v_sel.shape[-1]), dtype=np.float64)
    if k_sel.shape[0] == 0:
        return out
    logits = float(scale) * (q_rows @ k_sel.T)
    if row_ids is None:
        return row_softmax(logits) @ v_sel
    visible = np.asarray(col_ids)[None, :] <= np.asarray(row_ids)[:, None]
    for r in range(q_rows.shape[0]):
        cols = np.flatnonzero(visible[r])
        if cols.size:
            out[r] = row_softmax(logits[r, cols]) @ v_sel[cols]
    return out


def masked_attention(q, k, v, mask, scale: float | None = None, causal: bool = False) -> np.ndarray:
    """Block-masked attention; q, k, v (B, H, N, D) float64, mask (B, H, Qb, Kb).

    A query block with no selected key block outputs zeros. With causal=True a
    row r only sees the keys c <= r of its selected blocks (zeros if none).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, N, D = q.shape
    scale = default_scale(D) if scale is None else float(scale)
    qb, kb = num_blocks(N, Q_BLOCK), num_blocks(N, K_BLOCK)
    if mask.shape != (B, H, qb, kb):
        raise ValueError(f"mask shape {mask.shape} != {(B, H, qb, kb)}")
    out = np.empty((B, H, N, D), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            for i in range(qb):
                lo, hi = i * Q_BLOCK, min(N, (i + 1) * Q_BLOCK)
                cols = selected_keys(mask[b, h, i], N)
                rows = np.arange(lo, hi) if causal else None
                out[b, h, lo:hi] = attend_rows(q[b, h, lo:hi], k[b, h, cols], v[b, h, cols], scale,
                                               rows, cols if causal else None)
    return out


def masked_attention_rows(q_h, k_h, v_h, mask_h, rows, scale: float | None = None,
                          causal: bool = False) -> np.ndarray:
    """Outputs of chosen query rows of one head; q_h, k_h, v_h (N, D), mask_h (Qb, Kb)."""
    q_h = np.asarray(q_h, dtype=np.float64)
    N, D = q_h.shape
    scale = default_scale(D) if scale is None else float(scale)
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((rows.shape[0], D), dtype=np.float64)
    blocks = rows // Q_BLOCK
    for i in np.unique(blocks):
        sel = np.flatnonzero(blocks == i)
        cols = selected_keys(mask_h[i], N)
        out[sel] = attend_rows(q_h[rows[sel]], np.asarray(k_h, dtype=np.float64)[cols],
                               np.asarray(v_h, dtype=np.float64)[cols], scale,
                               rows[sel] if causal else None, cols if causal else None)
    return out


def masked_attention_sampled(q_h, k_h, v_h, mask_h, rows, scale: float | None = None,
                             causal: bool = False, chunk: int = 256) -> np.ndarray:
    """Outputs of scattered query rows of one head, each row on its own.

    The same quantity as masked_attention_rows, written as a masked softmax
    over the whole key axis: row r scores every key, keys outside the blocks
    its query block selects (and, with causal=True, keys after r) get weight
    zero, and the rest are normalised as usual. A row with no such key outputs
    zeros. Rows are handled in groups of `chunk` only to bound memory.
    q_h, k_h, v_h (N, D); mask_h (Qb, Kb); rows: token indices.
    """
    q_h = np.asarray(q_h, dtype=np.float64)
    k_h = np.asarray(k_h, dtype=np.float64)
    v_h = np.asarray(v_h, dtype=np.float64)
    mask_h = np.asarray(mask_h)
    N, D = q_h.shape
    scale = default_scale(D) if scale is None else float(scale)
    rows = np.asarray(rows, dtype=np.int64)
    key_block = np.arange(N) // K_BLOCK
    out = np.zeros((rows.shape[0], D), dtype=np.float64)
    for lo in range(0, rows.shape[0], chunk):
        r = rows[lo:lo + chunk]
        kept = mask_h[r // Q_BLOCK][:, key_block] != 0
        if causal:
            kept &= np.arange(N)[None, :] <= r[:, None]
        logits = np.where(kept, scale * (q_h[r] @ k_h.T), -np.inf)
        any_key = kept.any(axis=1)
        top = np.where(any_key, logits.max(axis=1), 0.0)
        w = np.exp(logits - top[:, None])
        den = np.where(any_key, w.sum(axis=1), 1.0)
        out[lo:lo + r.shape[0]] = (w @ v_h) / den[:, None]
    return out


def compact_mask(mask: np.ndarray):
    """Per row, the ascending list of selected key-block ids and its length.

    Returns (idx, cnt): idx (..., Kb) int32 padded with -1, cnt (...,) int32.
    """
    mask = np.asarray(mask)
    kb = mask.shape[-1]
    flat = mask.reshape(-1, kb)
    idx = np.full(flat.shape, -1, dtype=np.int32)
    cnt = np.zeros(flat.shape[0], dtype=np.int32)
    for r in range(flat.shape[0]):
        nz = np.flatnonzero(flat[r] != 0)
        idx[r, : nz.size] = nz
        cnt[r] = nz.size
    return idx.reshape(mask.shape), cnt.reshape(mask.shape[:-1])


def mask_parity(logits: np.ndarray, oracle_mask: np.ndarray, device_mask: np.ndarray, k,
                band: float = 1e-5, probs: np.ndarray | None = None, cand=None) -> dict:
    """Compare a device mask with the oracle's, allowing near-ties at the top-k boundary.

    Per row, with the row's candidate logits sorted in decreasing order, t is
    the k-th largest and the gap is t minus the (k+1)-th largest (infinite
    when k is the number of candidates). A row whose gap is at least `band`
    must equal the oracle row exactly. A row whose gap is below `band` is an
    exception candidate: it passes when it keeps exactly k blocks, keeps every
    block whose logit is at least t + band and drops every block whose logit
    is at most t - band. k and cand (candidates per row, default all key
    blocks) may be ints or per-query-block arrays; blocks past a row's
    candidates must never be kept.
    """
    s = np.asarray(logits, dtype=np.float64).reshape(-1, logits.shape[-1])
    om = np.asarray(oracle_mask).reshape(s.shape) != 0
    dm = np.asarray(device_mask).reshape(s.shape) != 0
    R, kb = s.shape
    n_qb = logits.shape[-2]
    kr = np.broadcast_to(np.asarray(k, dtype=np.int64), (n_qb,))
    cr = np.broadcast_to(np.asarray(kb if cand is None else cand, dtype=np.int64), (n_qb,))
    kr = np.tile(kr, R // n_qb)
    cr = np.tile(cr, R // n_qb)
    in_cand = np.arange(kb)[None, :] < cr[:, None]
    sc = np.where(in_cand, s, -np.inf)
    srt = -np.sort(-sc, axis=1)
    rows = np.arange(R)
    t = srt[rows, kr - 1]
    nxt = srt[rows, np.minimum(kr, kb - 1)]
    gap = np.where(kr < cr, t - nxt, np.inf)
    near = gap < band
    differ = (om != dm).any(axis=1)
    ok_exact = ~differ
    count_ok = dm.sum(axis=1) == kr
    outside_ok = ~(dm & ~in_cand).any(axis=1)
    must_keep = in_cand & (s >= (t + band)[:, None])
    must_drop = in_cand & (s <= (t - band)[:, None])
    ok_near = count_ok & outside_ok & ~(must_keep & ~dm).any(axis=1) & ~(must_drop & dm).any(axis=1)
    ok = np.where(near, ok_near, ok_exact)
    rep = {
        "rows": int(R),
        "candidates": int(near.sum()),
        "differing": int(differ.sum()),
        "failures": int((~ok).sum()),
        "failing_rows": np.flatnonzero(~ok)[:16].tolist(),
    }
    if probs is not None:
        ps = -np.sort(-np.where(in_cand, np.asarray(probs, dtype=np.float64).reshape(s.shape), -np.inf), axis=1)
        pgap = np.where(kr < cr, ps[rows, kr - 1] - ps[rows, np.minimum(kr, kb - 1)], np.inf)
        rep["prob_domain_candidates"] = int((pgap < band).sum())
    return rep


def cube_permutation(n_text: int, T: int, H: int, W: int, cube=(4, 4, 4)) -> np.ndarray:
    """New position p holds old token perm[p]: text tokens first, unchanged, then the
    video tokens cube by cube (cubes of cube = (ct, ch, cw) in raster order of the
    cube grid; a cube cut by the grid edge keeps the tokens it has), raster order
    (t, h, w; w fastest) inside each cube."""
    ct, ch, cw = (int(c) for c in cube)
    perm = list(range(n_text))
    for t0 in range(0, T, ct):
        for h0 in range(0, H, ch):
            for w0 in range(0, W, cw):
                for t in range(t0, min(T, t0 + ct)):
                    for h in range(h0, min(H, h0 + ch)):
                        for w in range(w0, min(W, w0 + cw)):
                            perm.append(n_text + (t * H + h) * W + w)
    return np.asarray(perm, dtype=np.int64)


def morton_code(t: int, h: int, w: int) -> int:
    """Bit interleave of (t, h, w): bit b of w goes to bit 3b, of h to 3b+1, of t to 3b+2."""
    code = 0
    for b in range(21):
        code |= ((w >> b) & 1) << (3 * b)
        code |= ((h >> b) & 1) << (3 * b + 1)
        code |= ((t >> b) & 1) << (3 * b + 2)
    return code


def morton_permutation(n_text: int, T: int, H: int, W: int) -> np.ndarray:
    """Text tokens first, unchanged, then the video tokens in increasing Morton code."""
    keyed = []
    for t in range(T):
        for h in range(H):
            for w in range(W):
                keyed.append((morton_code(t, h, w), n_text + (t * H + h) * W + w))
    keyed.sort()
    return np.asarray(list(range(n_text)) + [i for _, i in keyed], dtype=np.int64)


def permute_tokens(x: np.ndarray, perm: np.ndarray, inverse: bool = False) -> np.ndarray:
    """Reorder the token axis (-2): out[p] = x[perm[p]]; inverse: out[perm[p]] = x[p]."""
    x = np.asarray(x)
    perm = np.asarray(perm, dtype=np.int64)
    if not inverse:
        return x[..., perm, :]
    out = np.empty_like(x)
    out[..., perm, :] = x
    return out


def mask_parity_cdf(logits: np.ndarray, probs: np.ndarray, oracle_mask: np.ndarray,
                    device_mask: np.ndarray, tau: float, band: float = 1e-5, mass_band: float = 1e-5,
                    cand=None) -> dict:
    """Compare a device CDF-threshold mask with the oracle's.

    A row must equal the oracle's unless it sits at a float boundary. A differing
    row is excused when, with k its own count: it keeps k candidates and no
    other block; it keeps every candidate whose logit is at least t + band and
    none at most t - band, t being the k-th largest candidate logit (a valid
    top-k set up to near-ties); and the oracle's probabilities put the cut
    there up to mass_band: the k best reach at least tau - mass_band and the
    k - 1 best stay below tau + mass_band (tau = 1: k is every candidate).
    """
    s = np.asarray(logits, dtype=np.float64).reshape(-1, logits.shape[-1])
    pr = np.asarray(probs, dtype=np.float64).reshape(s.shape)
    om = np.asarray(oracle_mask).reshape(s.shape) != 0
    dm = np.asarray(device_mask).reshape(s.shape) != 0
    R, kb = s.shape
    n_qb = logits.shape[-2]
    cr = np.tile(np.broadcast_to(np.asarray(kb if cand is None else cand, dtype=np.int64), (n_qb,)), R // n_qb)
    excused, differing, failing = 0, 0, []
    for r in range(R):
        if (om[r] == dm[r]).all():
            continue
        differing += 1
        c = int(cr[r])
        in_cand = np.arange(kb) < c
        kd = int(dm[r].sum())
        ok = 1 <= kd <= c and not (dm[r] & ~in_cand).any()
        if ok:
            cum = np.cumsum(-np.sort(-pr[r, :c]))
            if tau >= 1.0:
                ok = kd == c
            else:
                ok = cum[kd - 1] >= tau - mass_band and (kd == 1 or cum[kd - 2] < tau + mass_band)
        if ok:
            t = -np.sort(-np.where(in_cand, s[r], -np.inf))[kd - 1]
            ok = (not (in_cand & (s[r] >= t + band) & ~dm[r]).any()
                  and not (in_cand & (s[r] <= t - band) & dm[r]).any())
        if ok:
            excused += 1
        elif len(failing) < 16:
            failing.append(r)
    return {"rows": int(R), "differing": differing, "excused": excused,
            "failures": differing - excused, "failing_rows": failing}
