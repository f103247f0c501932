"""Benchmark: top-k block-sparse attention on the 720p Wan2.1-14B-shaped workload.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--config 3] [--topk 0.3]

One step is the whole path on one batch of resident inputs: block pooling of
Q and K, pooled scoring with per-row top-k selection, and block-sparse
attention (sparge_attn_topk). Prints ONE JSON line on stdout; progress goes to
stderr. Alongside the step it reports:
  - the attention kernel alone (sparge_attn_from_list over the predicted
    lists), timed launch by launch with HIP events on the stream it runs on,
    as effective and dense-equivalent TFLOP/s against the bf16 MFMA peak;
  - pooling (GB/s) and prediction (GFLOP/s, GB/s) kernels;
  - block_sparse_attn with the predicted mask as a user mask (compaction + attention);
  - the fp64 CPU oracle timed on the host cores on a bounded sample, and (in the
    same CPU leg) every head's mask checked against the oracle's, with the count
    of rows whose pooled-logit gap at the top-k cut is under 1e-5.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # 256 CU x 4096 flop/clk x 2.4 GHz (MI355X dense bf16 MFMA)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
PEAK_FP32_TFLOPS = 157.3      # MI355X fp32 vector
COPY_BYTES = 1 << 30         # calibration copy for the traffic counters
METRIC = "block-sparse attn TFLOPS (effective + dense-equiv) & ms/call, N=75600 topk=0.3"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_wan14b-720p_topk0.3_traffic.json")
# the attention kernel's sources: the traffic figure is used only while they are unchanged
ATTN_SOURCES = [os.path.join(ROOT, "block_sparse_attention_sparge_amd", "csrc", f)
                for f in ("attn_fwd.hip", "attn_geometry.h", "common.h")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--config", type=int, default=3)
    p.add_argument("--topk", type=float, default=None)
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--causal", action="store_true", help="causal variant (is_causal=True)")
    p.add_argument("--tau", type=float, default=None,
                   help="CDF-threshold selection with this tau instead of top-k")
    p.add_argument("--layout", choices=["raster", "cube", "morton"], default="raster",
                   help="token order for the video grid: the step reorders Q, K, V, attends, restores O")
    p.add_argument("--recall-rows", type=int, default=0,
                   help="also report, for this many sampled rows of head 0, the share of the exact "
                        "attention weight that falls in the kept blocks")
    p.add_argument("--kernels-only", action="store_true",
                   help="launch each kernel once plus a plain copy of known size, for counter runs")
    return p.parse_args()


def block_rows_cols(N: int):
    """Valid query rows per query block and valid keys per key block."""
    qb, kb = -(-N // 128), -(-N // 64)
    rows = np.full(qb, 128.0)
    rows[-1] = N - 128 * (qb - 1)
    cols = np.full(kb, 64.0)
    cols[-1] = N - 64 * (kb - 1)
    return rows, cols


def tile_pairs(N: int, causal: bool) -> np.ndarray:
    """(Qb, Kb) number of (query row, key) pairs a tile computes: valid rows x valid keys,
    and with causal masking only the pairs with key <= row."""
    rows, cols = block_rows_cols(N)
    if not causal:
        return np.outer(rows, cols)
    qb, kb = rows.size, cols.size
    k0 = 64.0 * np.arange(kb)
    out = np.empty((qb, kb))
    for i in range(qb):
        r = np.arange(128 * i, 128 * i + int(rows[i]), dtype=np.float64)
        out[i] = np.clip(r[:, None] + 1.0 - k0[None, :], 0.0, cols[None, :]).sum(0)
    return out


def effective_flops(mask: np.ndarray, N: int, D: int, causal: bool = False) -> float:
    """4*D * sum over kept tiles of the (query row, key) pairs they compute; mask (..., Qb, Kb)."""
    qb, kb = mask.shape[-2:]
    pairs = tile_pairs(N, causal)
    return 4.0 * D * float((mask.reshape(-1, qb, kb).astype(np.float64) * pairs[None]).sum())


def recall_share(qh, kh, mask_h, rows, scale, causal):
    """Mean, over sampled query rows, of the exact softmax weight (over every visible key)
    that falls on the keys of the kept blocks: how much of the attention the selection keeps."""
    n = qh.shape[0]
    shares = []
    for r in rows:
        lg = scale * (kh @ qh[r])
        if causal:
            lg[r + 1:] = -np.inf
        w = np.exp(lg - lg.max())
        w /= w.sum()
        kept = np.repeat(mask_h[r // 128].astype(bool), 64)[:n]
        shares.append(float(w[kept].sum()))
    return {"rows": int(len(rows)), "mean": float(np.mean(shares)), "min": float(np.min(shares))}


def kernel_durations_ms(fn, iters):
    """Per-launch durations from HIP events recorded on the current stream around each launch."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    torch.cuda.synchronize()
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def source_hash(paths):
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str):
    """HBM bytes per attention launch from the committed rocprofv3 counter runs, if they
    were taken on this workload and the attention source has not changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("attn_fwd_source_sha256_16") != source_hash(ATTN_SOURCES) or t.get("workload") != workload:
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(wl, q, k, v, topk, budget_s, causal=False, tau=None):
    """The fp64 oracle on the host cores: head 0's full prediction plus attention for as
    many of its query blocks as fit in the time budget (in block order)."""
    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
    except ImportError:                                          # pragma: no cover
        threadpool_limits, threadpool_info = None, None
    cores = len(os.sched_getaffinity(0))
    ctx = threadpool_limits(cores) if threadpool_limits else None
    try:
        if ctx:
            ctx.__enter__()
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1]) if threadpool_info else 1
        f64 = synth.bf16_bits_to_f64
        qh, kh, vh = f64(q[0, 0]), f64(k[0, 0]), f64(v[0, 0])
        t0 = time.perf_counter()
        if tau is None:
            pr = oracle.predict_mask(qh[None, None], kh[None, None], topk, causal=causal)
        else:
            pr = oracle.predict_mask_cdf(qh[None, None], kh[None, None], tau, causal=causal)
        t_pred = time.perf_counter() - t0
        m = pr["mask"][0, 0]
        qb = m.shape[0]
        done, t_attn, flops = 0, 0.0, 0.0
        N, D = qh.shape
        pairs = tile_pairs(N, causal)
        while done < qb and (done < 4 or t_pred + t_attn < budget_s):
            rows = np.arange(128 * done, min(N, 128 * done + 128))
            t1 = time.perf_counter()
            oracle.masked_attention_rows(qh, kh, vh, m, rows, causal=causal)
            t_attn += time.perf_counter() - t1
            flops += 4.0 * D * float(m[done].astype(np.float64) @ pairs[done])
            done += 1
        bh = wl.B * wl.H
        full_attn_s = t_attn * (qb / done) * bh
        full_pred_s = t_pred * bh
        return {
            "value": flops / t_attn / 1e12,
            "unit": "TFLOPS",
            "cores": int(threads),
            "kind": "oracle",
            "sample": (f"head 0 of {bh}: full prediction ({t_pred:.2f} s) and masked attention of "
                       f"query blocks 0..{done - 1} of {qb} ({t_attn:.2f} s, {flops / 1e9:.1f} GFLOP); "
                       f"value = sampled attention flops / time"),
            "extrapolated_full_step_s": full_attn_s + full_pred_s,
            "host_cpus": cores,
        }
    finally:
        if ctx:
            ctx.__exit__(None, None, None)


def mask_parity_all_heads(q, k, m, topk, causal=False, tau=None):
    """Every head's device mask against the oracle's prediction: rows compared, rows
    whose pooled-logit gap at the cut is under 1e-5 (near ties), how many of those
    differ, and failures (rows that differ outside that band). Part of the CPU leg."""
    import oracle
    import synth
    f64 = synth.bf16_bits_to_f64
    B, H = m.shape[:2]
    tot = {"heads": B * H, "rows": 0, "near_tie_rows": 0, "differing": 0, "failures": 0}
    t0 = time.perf_counter()
    for b in range(B):
        for h in range(H):
            qh, kh = f64(q[b, h])[None, None], f64(k[b, h])[None, None]
            if tau is None:
                pr = oracle.predict_mask(qh, kh, topk, causal=causal)
                rep = oracle.mask_parity(pr["logits"], pr["mask"], m[b, h][None, None], pr["k"],
                                         probs=pr["probs"], cand=pr["cand"])
                tot["near_tie_rows"] += rep["candidates"]
            else:
                pr = oracle.predict_mask_cdf(qh, kh, tau, causal=causal)
                rep = oracle.mask_parity_cdf(pr["logits"], pr["probs"], pr["mask"], m[b, h][None, None],
                                             tau, cand=pr["cand"])
                tot["near_tie_rows"] += rep["excused"]
            tot["rows"] += rep["rows"]
            tot["differing"] += rep["differing"]
            tot["failures"] += rep["failures"]
    tot["seconds"] = time.perf_counter() - t0
    return tot


def device_info(torch) -> dict:
    """CU count and clocks the runtime reports for device 0 (rocminfo when present)."""
    props = torch.cuda.get_device_properties(0)
    info = {"name": props.name, "arch": getattr(props, "gcnArchName", None),
            "compute_units": props.multi_processor_count, "max_clock_mhz": None}
    try:
        import subprocess
        txt = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=30).stdout
        for agent in txt.split("Agent ")[1:]:
            if "gfx9" in agent and "Compute Unit:" in agent:
                for line in agent.splitlines():
                    if "Max Clock Freq. (MHz):" in line:
                        info["max_clock_mhz"] = int(line.split(":")[1].split()[0])
                    if "Compute Unit:" in line:
                        info["rocminfo_compute_units"] = int(line.split(":")[1].split()[0])
                break
    except (OSError, ValueError, subprocess.SubprocessError):
        pass
    return info


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the path shards by (batch, head) with no "
              "exchange, and multi-GPU runs are not part of this build.", file=sys.stderr)
        sys.exit(2)
    import torch

    import block_sparse_attention_sparge_amd as sp
    import synth

    wl = synth.WORKLOADS[args.config]
    topk = args.topk if args.topk is not None else (0.3 if args.config == 3 else wl.topks[0])
    B, H, N, D = wl.B, wl.H, wl.N, wl.D
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sp.load_library()

    log(f"generating {wl.describe()} seed={args.seed}")
    q, k, v = synth.make_qkv(wl, seed=args.seed)
    tod = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    dq, dk, dv = tod(q), tod(k), tod(v)
    out = torch.empty_like(dq)
    mask = torch.empty(sp.mask_shape(B, H, N), dtype=torch.uint8, device=dev)
    cdf = args.tau is not None
    ws = torch.empty(sp.workspace_bytes(B, H, N, D, 1.0 if cdf else topk), dtype=torch.uint8, device=dev)
    kk = sp.topk_count(mask.shape[-1], topk)

    causal = bool(args.causal)
    layout = args.layout
    if layout != "raster":
        if causal or wl.grid is None:
            raise SystemExit("--layout needs a video workload and non-causal attention")
        perm = sp.token_permutation(wl.n_text, wl.grid, layout)
        dperm = perm.to(dev)
        # the timed step starts from raster-order inputs and ends with a raster-order output
        rq, rk, rv = dq, dk, dv
        dq, dk, dv = (torch.empty_like(t) for t in (rq, rk, rv))
        out_l = torch.empty_like(out)

    def step():
        if cdf:
            sp.attn_cdf(dq, dk, dv, tau=args.tau, out=out, workspace=ws, is_causal=causal)
            return
        if layout == "raster":
            sp.attn_topk(dq, dk, dv, topk=topk, out=out, workspace=ws, is_causal=causal)
            return
        for src, dst in ((rq, dq), (rk, dk), (rv, dv)):
            sp.permute_tokens(src, dperm, out=dst)
        sp.attn_topk(dq, dk, dv, topk=topk, out=out_l, workspace=ws)
        sp.permute_tokens(out_l, dperm, inverse=True, out=out)

    # mask and lists once, for the per-kernel timings and the flop count
    step()
    torch.cuda.synchronize()
    qbar, kbar = sp.pool_blocks(dq, 128), sp.pool_blocks(dk, 64)
    if cdf:
        mask_t, idx, cnt = sp.predict_mask_cdf(qbar, kbar, N, args.tau, is_causal=causal)
    else:
        mask_t, idx, cnt = sp.predict_mask(qbar, kbar, N, topk, is_causal=causal)
    torch.cuda.synchronize()
    m = mask_t.cpu().numpy()
    eff = effective_flops(m, N, D, causal)
    dense = 4.0 * B * H * D * (N * (N + 1) / 2.0 if causal else float(N) * N)
    log(f"k={kk} of {m.shape[-1]} key blocks; effective {eff / 1e12:.2f} TFLOP, dense {dense / 1e12:.2f} TFLOP")

    if args.kernels_only:
        # one launch of each kernel and a device copy of COPY_BYTES (read + write),
        # whose FETCH_SIZE / WRITE_SIZE readings calibrate the counters
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        sp.attn_from_list(dq, dk, dv, idx, cnt, out=out, is_causal=causal)
        sp.pool_blocks(dq, 128)
        sp.pool_blocks(dk, 64)
        sp.predict_mask(qbar, kbar, N, topk, is_causal=causal)
        sp.compact_mask(mask_t, N)
        if wl.grid is not None:
            perm_k = sp.token_permutation(wl.n_text, wl.grid, "cube").to(dev)
            sp.permute_tokens(dq, perm_k, out=out)
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"kernels_only": True, "copy_bytes": COPY_BYTES, "workload": wl.name,
                          "topk": topk, "effective_flops": eff}), flush=True)
        return

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} done; timing {args.steps} steps")
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(args.steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    log(f"step {ms:.3f} ms")

    # attention kernel alone, launch by launch
    attn_iters = max(5, min(args.steps, 20))
    attn = kernel_durations_ms(lambda: sp.attn_from_list(dq, dk, dv, idx, cnt, out=out, is_causal=causal),
                               attn_iters)
    attn_ms = float(np.mean(attn))
    log(f"attention kernel {attn_ms:.3f} ms (min {min(attn):.3f})")
    pool_q = kernel_durations_ms(lambda: sp.pool_blocks(dq, 128), 10)
    pool_k = kernel_durations_ms(lambda: sp.pool_blocks(dk, 64), 10)
    if cdf:
        pred = kernel_durations_ms(lambda: sp.predict_mask_cdf(qbar, kbar, N, args.tau, is_causal=causal), 10)
    else:
        pred = kernel_durations_ms(lambda: sp.predict_mask(qbar, kbar, N, topk, return_mask=True,
                                                           is_causal=causal), 10)
    layout_info = {"name": layout}
    if layout != "raster":
        perm_ms = float(np.mean(kernel_durations_ms(lambda: sp.permute_tokens(rq, dperm, out=dq), 10)))
        layout_info.update({"permute_ms": perm_ms,
                            "permute_gbs": 2 * B * H * N * D * 2 / (perm_ms * 1e-3) / 1e9})
    if args.recall_rows > 0:
        qh = synth.bf16_bits_to_f64(q[0, 0])
        kh = synth.bf16_bits_to_f64(k[0, 0])
        if layout != "raster":
            p_np = perm.numpy().astype(np.int64)
            qh, kh = qh[p_np], kh[p_np]
        rows = np.random.default_rng(7).choice(N, size=min(N, args.recall_rows), replace=False)
        layout_info["recall"] = recall_share(qh, kh, m[0, 0], rows, 1.0 / np.sqrt(D), causal)
    bsa = kernel_durations_ms(lambda: sp.block_sparse_attn(dq, dk, dv, mask_id=mask_t, out=out,
                                                           is_causal=causal), 5)
    # plan reuse: the kept-block lists parked in pinned host memory between calls and brought back
    h_idx = torch.empty(idx.shape, dtype=idx.dtype, pin_memory=True)
    h_cnt = torch.empty(cnt.shape, dtype=cnt.dtype, pin_memory=True)

    def roundtrip():
        h_idx.copy_(idx, non_blocking=True)
        h_cnt.copy_(cnt, non_blocking=True)
        idx.copy_(h_idx, non_blocking=True)
        cnt.copy_(h_cnt, non_blocking=True)
    plan_rt = kernel_durations_ms(roundtrip, 5)
    plan_bytes = idx.numel() * 4 + cnt.numel() * 4

    qb_, kb_ = m.shape[-2:]
    pool_bytes_q = B * H * N * D * 2 + B * H * qb_ * D * 4
    pool_bytes_k = B * H * N * D * 2 + B * H * kb_ * D * 4
    pred_flops = 2.0 * B * H * qb_ * kb_ * D
    pred_bytes = B * H * (qb_ + kb_) * D * 4 + B * H * qb_ * (kb_ + 4 * kk + 4)
    achieved = eff / (attn_ms * 1e-3) / 1e12
    result = {
        "metric": METRIC,
        "value": eff / (ms * 1e-3) / 1e12,
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": B, "H": H, "N": N, "D": D, "topk": topk, "k": kk,
                   "causal": causal, "layout": layout, "tau": args.tau,
                   "kept_fraction": float(m.mean()),
                   "n_qblocks": int(qb_), "n_kblocks": int(kb_), "seed": args.seed,
                   "step": ("sparge_attn_cdf" if cdf else "sparge_attn_topk") + " (pool Q, pool K, predict, attention)"},
        "dense_equiv_tflops": dense / (ms * 1e-3) / 1e12,
        "frac_peak_effective": eff / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "frac_peak_dense_equiv": dense / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "effective_tflop_per_step": eff / 1e12,
        "attention_kernel": {"ms": attn_ms, "ms_min": float(min(attn)),
                             "effective_tflops": achieved,
                             "dense_equiv_tflops": dense / (attn_ms * 1e-3) / 1e12},
        "block_sparse_attn_ms": float(np.mean(bsa)),
        "plan_reuse": {"apply_ms": attn_ms, "predict_and_apply_ms": ms,
                       "lists_bytes": int(plan_bytes),
                       "pinned_roundtrip_ms": float(np.mean(plan_rt))},
        "pool_q": {"ms": float(np.mean(pool_q)), "gbs": pool_bytes_q / (np.mean(pool_q) * 1e-3) / 1e9},
        "pool_k": {"ms": float(np.mean(pool_k)), "gbs": pool_bytes_k / (np.mean(pool_k) * 1e-3) / 1e9},
        "predict": {"ms": float(np.mean(pred)),
                    "gflops_fp32": pred_flops / (np.mean(pred) * 1e-3) / 1e9,
                    "gbs": pred_bytes / (np.mean(pred) * 1e-3) / 1e9},
        "layout": layout_info,
        "device": device_info(torch),
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": None if (causal or cdf or layout != "raster") else load_traffic(f"{wl.name}_topk{topk}"),
                     "kernel": f"attn_fwd_kernel<{D}, {str(causal).lower()}, true> (sparge_attn_from_list; "
                               "K and V with equal token strides)"},
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle sample")
        result["cpu_baseline"] = cpu_baseline(wl, q, k, v, topk, args.cpu_seconds, causal, args.tau)
        if layout == "raster":
            log("checking every head's mask against the oracle")
            result["mask_parity"] = mask_parity_all_heads(q, k, m, topk, causal, args.tau)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
