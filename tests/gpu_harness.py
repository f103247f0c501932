"""Helpers shared by the GPU tests: move seeded bf16 inputs to the device and
compare device results with the CPU oracle. Nothing here computes any step of
the method."""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle
import synth

ATOL_MAX = 2e-2      # max |out_gpu - out_oracle| over compared elements
ATOL_MEAN = 2e-3     # mean |out_gpu - out_oracle| over compared elements
MASK_BAND = 1e-5     # near-tie band on pooled logits at the top-k boundary


def to_dev(bits: np.ndarray, device="cuda") -> torch.Tensor:
    """uint16 bf16 bit patterns -> bf16 tensor on the GPU (same bytes)."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def to_host_f64(t: torch.Tensor) -> np.ndarray:
    return synth.bf16_bits_to_f64(t.detach().view(torch.int16).cpu().numpy().view(np.uint16))


def rand_qkv(B, H, N, D, seed, grid=None, q_scale=1.0):
    wl = synth.custom(B, H, N, D, config_id=200 + (seed % 50), grid=grid, q_scale=q_scale)
    return synth.make_qkv(wl, seed=seed)


def compare_out(got: np.ndarray, ref: np.ndarray) -> dict:
    err = np.abs(got - ref)
    return {"max_abs": float(err.max()) if err.size else 0.0,
            "mean_abs": float(err.mean()) if err.size else 0.0,
            "n": int(err.size)}


def assert_close(got, ref, what=""):
    r = compare_out(got, ref)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    assert r["max_abs"] <= ATOL_MAX and r["mean_abs"] <= ATOL_MEAN, f"{what}: {r}"
    return r


def oracle_mask_parity(q64_heads, k64_heads, topk, mask_dev, scale=None, causal=False):
    """Run the oracle prediction per head and compare with a device mask.

    q64_heads / k64_heads: callables (b, h) -> (N, D) float64. mask_dev: (B, H, Qb, Kb) numpy.
    Returns the summed parity report.
    """
    B, H = mask_dev.shape[:2]
    tot = {"rows": 0, "candidates": 0, "differing": 0, "failures": 0, "prob_domain_candidates": 0}
    for b in range(B):
        for h in range(H):
            qh, kh = q64_heads(b, h), k64_heads(b, h)
            pr = oracle.predict_mask(qh[None, None], kh[None, None], topk, scale, causal=causal)
            rep = oracle.mask_parity(pr["logits"], pr["mask"], mask_dev[b, h][None, None], pr["k"],
                                     band=MASK_BAND, probs=pr["probs"], cand=pr["cand"])
            for key in tot:
                tot[key] += rep.get(key, 0)
    return tot


def host_threads() -> int:
    """Worker threads for oracle work: the host CPUs this process may use, at most 16."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def parallel_heads(fn, heads):
    """fn(b, h) for every (b, h), on host threads with single-threaded BLAS in each.

    The oracle's per-head work is independent, so the heads are spread over the
    host cores; returns the results in the order of `heads`."""
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1):
        with ThreadPoolExecutor(max_workers=host_threads()) as ex:
            return list(ex.map(lambda bh: fn(*bh), heads))
