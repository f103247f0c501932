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


def predict_mask(q: np.ndarray, k: np.ndarray, topk: float, scale: float | None = None) -> dict:
    """Pool -> score -> select. q, k are (B, H, N, D) float64.

    Returns a dict with mask (uint8), logits s, probabilities p, the pooled
    qbar / kbar and the per-row count kk.
    """
    d = q.shape[-1]
    scale = default_scale(d) if scale is None else float(scale)
    qbar = pool_blocks(q, Q_BLOCK)
    kbar = pool_blocks(k, K_BLOCK)
    s = block_logits(qbar, kbar, scale)
    p = row_softmax(s)
    kk = topk_count(kbar.shape[-2], topk)
    mask = select_topk(p, kk)
    return {"mask": mask, "logits": s, "probs": p, "qbar": qbar, "kbar": kbar, "k": kk}


def selected_keys(mask_row: np.ndarray, n: int) -> np.ndarray:
    """Token indices of the key blocks a 0/1 mask row selects (ascending)."""
    idx = []
    for j in np.flatnonzero(np.asarray(mask_row) != 0):
        idx.extend(range(j * K_BLOCK, min(n, (j + 1) * K_BLOCK)))
    return np.asarray(idx, dtype=np.int64)


def attend_rows(q_rows: np.ndarray, k_sel: np.ndarray, v_sel: np.ndarray, scale: float) -> np.ndarray:
    """Softmax attention of some query rows over one key/value set (float64)."""
    if k_sel.shape[0] == 0:
        return np.zeros((q_rows.shape[0], v_sel.shape[-1]), dtype=np.float64)
    logits = float(scale) * (q_rows @ k_sel.T)
    w = row_softmax(logits)
    return w @ v_sel


def masked_attention(q, k, v, mask, scale: float | None = None) -> np.ndarray:
    """Block-masked non-causal attention; q, k, v (B, H, N, D) float64, mask (B, H, Qb, Kb).

    A query block with no selected key block outputs zeros.
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
                out[b, h, lo:hi] = attend_rows(q[b, h, lo:hi], k[b, h, cols], v[b, h, cols], scale)
    return out


def masked_attention_rows(q_h, k_h, v_h, mask_h, rows, scale: float | None = None) -> np.ndarray:
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
                               np.asarray(v_h, dtype=np.float64)[cols], scale)
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


def mask_parity(logits: np.ndarray, oracle_mask: np.ndarray, device_mask: np.ndarray, k: int,
                band: float = 1e-5, probs: np.ndarray | None = None) -> dict:
    """Compare a device mask with the oracle's, allowing near-ties at the top-k boundary.

    Per row, with the row's logits sorted in decreasing order, t is the k-th
    largest and the gap is t minus the (k+1)-th largest (infinite when k is
    the row length). A row whose gap is at least `band` must equal the oracle
    row exactly. A row whose gap is below `band` is an exception candidate: it
    passes when it keeps exactly k blocks, keeps every block whose logit is
    at least t + band and drops every block whose logit is at most t - band.
    """
    s = np.asarray(logits, dtype=np.float64).reshape(-1, logits.shape[-1])
    om = np.asarray(oracle_mask).reshape(s.shape) != 0
    dm = np.asarray(device_mask).reshape(s.shape) != 0
    R, kb = s.shape
    srt = -np.sort(-s, axis=1)
    t = srt[:, k - 1]
    gap = t - srt[:, k] if k < kb else np.full(R, np.inf)
    near = gap < band
    differ = (om != dm).any(axis=1)
    ok_exact = ~differ
    count_ok = dm.sum(axis=1) == k
    must_keep = s >= (t + band)[:, None]
    must_drop = s <= (t - band)[:, None]
    ok_near = count_ok & ~(must_keep & ~dm).any(axis=1) & ~(must_drop & dm).any(axis=1)
    ok = np.where(near, ok_near, ok_exact)
    rep = {
        "rows": int(R),
        "candidates": int(near.sum()),
        "differing": int(differ.sum()),
        "failures": int((~ok).sum()),
        "failing_rows": np.flatnonzero(~ok)[:16].tolist(),
    }
    if probs is not None:
        ps = -np.sort(-np.asarray(probs, dtype=np.float64).reshape(s.shape), axis=1)
        pgap = ps[:, k - 1] - ps[:, k] if k < kb else np.full(R, np.inf)
        rep["prob_domain_candidates"] = int((pgap < band).sum())
    return rep
