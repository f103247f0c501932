"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Bars: pooled means within 1e-6 relative; masks bit-exact except rows whose
pooled-logit gap at the top-k boundary is below 1e-5 (those only need a valid
selection; the count is printed); attention outputs, with the oracle run on
the GPU's own mask, within max-abs 2e-2 and mean-abs 2e-3; block lists and
counts bit-exact.
"""
import math

import numpy as np
import pytest
import torch

import block_sparse_attention_sparge_amd as sp
import oracle
import synth
from gpu_harness import (assert_close, compare_out, oracle_mask_parity, parallel_heads, rand_qkv,
                         to_dev, to_host_f64)

pytestmark = pytest.mark.gpu

F64 = synth.bf16_bits_to_f64

# (B, H, N, D): several tiles with ragged query and key tails, plus aligned sizes.
SMALL = [(1, 2, 1000, 128), (2, 3, 777, 64), (1, 2, 1024, 64), (1, 1, 384, 128), (1, 3, 200, 128)]
EDGE_N = [1, 2, 63, 64, 65, 127, 128, 129, 191]


def _dev(q, k, v):
    return to_dev(q), to_dev(k), to_dev(v)


@pytest.mark.parametrize("B,H,N,D", SMALL + [(1, 1, n, 64) for n in (1, 65, 129)])
def test_pool_blocks(gpu_lib, B, H, N, D):
    q, k, _ = rand_qkv(B, H, N, D, seed=N + D)
    for x, rows in ((q, 128), (k, 64)):
        got = sp.pool_blocks(to_dev(x), rows).cpu().numpy().astype(np.float64)
        ref = oracle.pool_blocks(F64(x), rows)
        assert got.shape == ref.shape
        assert np.abs(got - ref).max() <= 1e-6 * max(1.0, np.abs(ref).max())


@pytest.mark.parametrize("B,H,N,D", SMALL)
@pytest.mark.parametrize("topk", [0.05, 0.3, 0.5, 1.0])
def test_predict_mask_and_lists(gpu_lib, B, H, N, D, topk):
    q, k, _ = rand_qkv(B, H, N, D, seed=7 * N + D, grid=None)
    dq, dk = to_dev(q), to_dev(k)
    qbar, kbar = sp.pool_blocks(dq, 128), sp.pool_blocks(dk, 64)
    mask, idx, cnt = sp.predict_mask(qbar, kbar, N, topk)
    torch.cuda.synchronize()
    mask, idx, cnt = mask.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy()
    kk = oracle.topk_count(mask.shape[-1], topk)
    assert idx.shape[-1] == kk and (cnt == kk).all()
    assert (mask.sum(-1) == kk).all()
    ref_idx, ref_cnt = oracle.compact_mask(mask)
    assert (ref_cnt == kk).all() and (idx == ref_idx[..., :kk]).all()
    rep = oracle_mask_parity(lambda b, h: F64(q[b, h]), lambda b, h: F64(k[b, h]), topk, mask)
    print("mask parity", rep)
    assert rep["failures"] == 0


def test_predict_ties_go_to_lower_index(gpu_lib):
    """Bit-identical key blocks: the lower index must win the last kept slot."""
    N, D = 1024, 64
    q, k, _ = rand_qkv(1, 1, N, D, seed=11)
    k[0, 0, 512:1024] = k[0, 0, 0:512]          # blocks 8..15 duplicate blocks 0..7
    q[0, 0] = q[0, 0, :1].repeat(N, axis=0)     # every query block pools to the same row
    for topk in (1 / 16, 3 / 16, 5 / 16, 0.5, 9 / 16):
        qbar, kbar = sp.pool_blocks(to_dev(q), 128), sp.pool_blocks(to_dev(k), 64)
        mask, _, _ = sp.predict_mask(qbar, kbar, N, topk)
        ref = oracle.predict_mask(F64(q), F64(k), topk)["mask"]
        assert (mask.cpu().numpy() == ref).all(), topk


def _random_mask(B, H, N, density, seed, empty_rows=True):
    rng = np.random.default_rng(seed)
    shape = sp.mask_shape(B, H, N)
    m = (rng.random(shape) < density).astype(np.uint8)
    if empty_rows and shape[2] > 1:
        m[:, :, 1, :] = 0                       # a query block with nothing selected
    return m


@pytest.mark.parametrize("B,H,N,D", SMALL)
@pytest.mark.parametrize("density", [0.1, 0.5, 1.0])
def test_block_sparse_attn_user_mask(gpu_lib, B, H, N, D, density):
    q, k, v = rand_qkv(B, H, N, D, seed=3 * N + D)
    m = _random_mask(B, H, N, density, seed=N)
    out = sp.block_sparse_attn(*_dev(q, k, v), mask_id=torch.from_numpy(m).cuda())
    got = to_host_f64(out)
    ref = oracle.masked_attention(F64(q), F64(k), F64(v), m)
    r = assert_close(got, ref, f"user mask {B, H, N, D, density}")
    if m.shape[2] > 1:
        assert (got[:, :, 128:256] == 0).all()   # empty row -> zeros
    print(r)


@pytest.mark.parametrize("N,D", [(1000, 128), (129, 64)])
def test_mask_value_check(gpu_lib, N, D):
    """The checking calls reject a mask byte other than 0/1 ("Mask Requirements")
    before computing anything, and otherwise equal the fast call bit for bit."""
    B, H = 1, 2
    q, k, v = _dev(*rand_qkv(B, H, N, D, seed=N + 3))
    m = torch.from_numpy(_random_mask(B, H, N, 0.5, seed=4)).cuda()
    ref = sp.block_sparse_attn(q, k, v, mask_id=m)
    got = sp.block_sparse_attn(q, k, v, mask_id=m, validate=True)
    torch.cuda.synchronize()
    assert torch.equal(ref.view(torch.int16), got.view(torch.int16))
    sp.check_mask(m, N)
    shape = m.shape
    for bad in (2, 255):
        mb = m.clone()
        mb[B - 1, H - 1, shape[2] - 1, shape[3] - 1] = bad      # the very last byte
        out = torch.full_like(ref, 3.0)
        with pytest.raises(sp.SpargeArgumentError) as e:
            sp.block_sparse_attn(q, k, v, mask_id=mb, validate=True, out=out)
        assert e.value.status == -9
        assert bool((out == 3.0).all())                          # nothing was computed
        with pytest.raises(sp.SpargeArgumentError):
            sp.check_mask(mb, N)
        mb = m.clone()
        mb[0, 0, 0, 0] = bad                                     # the first byte
        with pytest.raises(sp.SpargeArgumentError):
            sp.check_mask(mb, N)
    # the fast call counts any nonzero byte as kept
    m2 = m.clone()
    m2[m2 == 1] = 7
    fast = sp.block_sparse_attn(q, k, v, mask_id=m2)
    torch.cuda.synchronize()
    assert torch.equal(fast.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("B,H,N,D", SMALL)
def test_dense_and_topk_one(gpu_lib, B, H, N, D):
    q, k, v = rand_qkv(B, H, N, D, seed=5 * N + D)
    dq, dk, dv = _dev(q, k, v)
    dense = sp.block_sparse_attn(dq, dk, dv, mask_id=None)
    ones = sp.block_sparse_attn(dq, dk, dv, mask_id=torch.ones(sp.mask_shape(B, H, N), dtype=torch.uint8, device="cuda"))
    top1, mask = sp.attn_topk(dq, dk, dv, topk=1.0, return_mask=True)
    torch.cuda.synchronize()
    assert mask.cpu().numpy().all()
    # the same tiles in the same order: bit-identical
    assert torch.equal(dense.view(torch.int16), ones.view(torch.int16))
    assert torch.equal(dense.view(torch.int16), top1.view(torch.int16))
    t = lambda a: torch.from_numpy(F64(a))
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v)).numpy()
    assert_close(to_host_f64(dense), ref, "dense vs SDPA")


@pytest.mark.parametrize("N", EDGE_N)
@pytest.mark.parametrize("D", [64, 128])
def test_edge_lengths(gpu_lib, N, D):
    q, k, v = rand_qkv(1, 2, N, D, seed=N * 3 + D)
    dq, dk, dv = _dev(q, k, v)
    out, mask = sp.attn_topk(dq, dk, dv, topk=0.5, return_mask=True)
    m = mask.cpu().numpy()
    ref = oracle.masked_attention(F64(q), F64(k), F64(v), m)
    assert_close(to_host_f64(out), ref, f"edge N={N}")
    rep = oracle_mask_parity(lambda b, h: F64(q[b, h]), lambda b, h: F64(k[b, h]), 0.5, m)
    assert rep["failures"] == 0


@pytest.mark.parametrize("B,H,N,D", SMALL)
@pytest.mark.parametrize("topk", [0.2, 0.5])
def test_attn_topk_end_to_end(gpu_lib, B, H, N, D, topk):
    q, k, v = rand_qkv(B, H, N, D, seed=9 * N + D, q_scale=1 / math.sqrt(D))
    out, mask = sp.attn_topk(*_dev(q, k, v), topk=topk, return_mask=True)
    m = mask.cpu().numpy()
    rep = oracle_mask_parity(lambda b, h: F64(q[b, h]), lambda b, h: F64(k[b, h]), topk, m)
    assert rep["failures"] == 0, rep
    ref = oracle.masked_attention(F64(q), F64(k), F64(v), m)
    print(assert_close(to_host_f64(out), ref, "attn_topk"), rep)


def test_strided_layouts_and_scale(gpu_lib):
    B, H, N, D = 2, 3, 700, 128
    q, k, v = rand_qkv(B, H, N, D, seed=21)
    dq, dk, dv = _dev(q, k, v)
    # (B, N, H, D) storage viewed as (B, H, N, D), like a fused projection's output
    tq, tk, tv = (x.transpose(1, 2).contiguous().transpose(1, 2) for x in (dq, dk, dv))
    assert tq.stride() != dq.stride()
    out_t = torch.empty(B, N, H, D, dtype=torch.bfloat16, device="cuda").transpose(1, 2)
    m = torch.from_numpy(_random_mask(B, H, N, 0.4, seed=3)).cuda()
    a = sp.block_sparse_attn(dq, dk, dv, mask_id=m, scale=0.05)
    b = sp.block_sparse_attn(tq, tk, tv, mask_id=m, scale=0.05, out=out_t)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.contiguous().view(torch.int16))
    ref = oracle.masked_attention(F64(q), F64(k), F64(v), m.cpu().numpy(), scale=0.05)
    assert_close(to_host_f64(a), ref, "scale=0.05")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_kv_strides_differ(gpu_lib, D, causal):
    """K and V with different token strides (K contiguous, V stored (B, N, H, D))
    take the kernel's separate K and V tile bounds; ragged N, so the tail tile
    is bounded differently for each."""
    B, H, N = 2, 3, 700
    q, k, v = rand_qkv(B, H, N, D, seed=23)
    dq, dk, dv = _dev(q, k, v)
    tv = dv.transpose(1, 2).contiguous().transpose(1, 2)
    assert tv.stride(2) != dk.stride(2)
    m = torch.from_numpy(_random_mask(B, H, N, 0.4, seed=5)).cuda()
    a = sp.block_sparse_attn(dq, dk, dv, mask_id=m, is_causal=causal)
    b = sp.block_sparse_attn(dq, dk, tv, mask_id=m, is_causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    ref = oracle.masked_attention(F64(q), F64(k), F64(v), m.cpu().numpy(), causal=causal)
    assert_close(to_host_f64(b), ref, f"K/V strides differ, D={D}, causal={causal}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("pattern", ["growing", "shrinking", "wide"])
def test_softmax_reference_raised(gpu_lib, D, pattern):
    """Scores that climb far above the running max along the key walk (and the
    reverse, and a very wide spread) exercise the rescaling of O and l."""
    B, H, N = 1, 2, 1000
    q, k, v = rand_qkv(B, H, N, D, seed=41 + D)
    kf = F64(k)
    blk = np.arange(N) // 64
    if pattern == "growing":
        kf = kf * (1.0 + 1.5 * blk)[None, None, :, None]
    elif pattern == "shrinking":
        kf = kf * (1.0 + 1.5 * (blk.max() - blk))[None, None, :, None]
    else:
        kf = kf * 6.0
    kb = synth.f32_to_bf16_bits(kf.astype(np.float32))
    scale = 1.0 if pattern == "wide" else None
    out = sp.block_sparse_attn(*_dev(q, kb, v), mask_id=None, scale=scale)
    mask = np.ones(sp.mask_shape(B, H, N), dtype=np.uint8)
    ref = oracle.masked_attention(F64(q), F64(kb), F64(v), mask, scale=scale)
    print(assert_close(to_host_f64(out), ref, f"{pattern} D={D}"))


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_softmax_far_below_zero(gpu_lib, D, causal):
    """Every logit of every row pushed far below zero by one common offset
    (q = x - 40 e0, k = y + 40 e0): the softmax must not depend on that shift,
    although exp2 of the raw scores underflows to zero."""
    B, H, N = 1, 2, 700
    q, k, v = rand_qkv(B, H, N, D, seed=43 + D)
    qf, kf = F64(q), F64(k)
    qf[..., 0] -= 40.0
    kf[..., 0] += 40.0
    qb = synth.f32_to_bf16_bits(qf.astype(np.float32))
    kb = synth.f32_to_bf16_bits(kf.astype(np.float32))
    m = _random_mask(B, H, N, 0.5, seed=9, empty_rows=False)
    m[..., 0] = 1
    out = sp.block_sparse_attn(*_dev(qb, kb, v), mask_id=torch.from_numpy(m).cuda(), is_causal=causal)
    ref = oracle.masked_attention(F64(qb), F64(kb), F64(v), m, causal=causal)
    lg = (F64(qb)[0, 0, :8] @ F64(kb)[0, 0].T) / math.sqrt(D) * math.log2(math.e)
    assert lg.max() < -150      # exp2 of any raw logit is below the smallest fp32 normal
    print(assert_close(to_host_f64(out), ref, f"far below zero D={D} causal={causal}"))


def test_deterministic(gpu_lib):
    wl = synth.WORKLOADS[0]
    q, k, v = synth.make_qkv(wl)
    dq, dk, dv = _dev(q, k, v)
    o1, m1 = sp.attn_topk(dq, dk, dv, topk=0.5, return_mask=True)
    o2, m2 = sp.attn_topk(dq, dk, dv, topk=0.5, return_mask=True)
    torch.cuda.synchronize()
    assert torch.equal(m1, m2) and torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_from_list_reuse(gpu_lib):
    """A predicted list applied with attn_from_list equals the one-call top-k path."""
    B, H, N, D = 1, 4, 2000, 128
    q, k, v = rand_qkv(B, H, N, D, seed=33, q_scale=1 / math.sqrt(D))
    dq, dk, dv = _dev(q, k, v)
    mask, idx, cnt = sp.predict_mask(sp.pool_blocks(dq, 128), sp.pool_blocks(dk, 64), N, 0.3)
    a = sp.attn_from_list(dq, dk, dv, idx, cnt)
    b = sp.attn_topk(dq, dk, dv, topk=0.3)
    c = sp.block_sparse_attn(dq, dk, dv, mask_id=mask)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(a.view(torch.int16), c.view(torch.int16))


def test_plan_reuse_on_new_inputs(gpu_lib, parity_log):
    """A plan predicted on one step's inputs, parked in pinned host memory between
    calls, brought back and applied to the next step's inputs (AB-Attention README,
    "Paper settings, timing, and pipeline integration": plans refreshed every few
    steps and kept in pinned CPU memory; SpargeAttention Documentation,
    block_sparse_sage2_attn_cuda: attention under a given mask). Wan2.1-1.3B video
    grid (21x30x52 tokens, D=128), two heads; inputs A from seed 0, B from seed 1."""
    wl = synth.custom(1, 2, 32760, 128, config_id=1, grid=(21, 30, 52), q_scale=1 / math.sqrt(128))
    qa, ka, _ = synth.make_qkv(wl, seed=0)
    qb, kb, vb = synth.make_qkv(wl, seed=1)
    mask_a, idx, cnt = sp.predict_mask(sp.pool_blocks(to_dev(qa), 128), sp.pool_blocks(to_dev(ka), 64),
                                       wl.N, 0.5)
    torch.cuda.synchronize()
    want_idx, want_cnt, m_a = idx.cpu().numpy(), cnt.cpu().numpy(), mask_a.cpu().numpy()
    # park the plan in pinned host memory, clobber the device copy, bring it back
    h_idx = torch.empty(idx.shape, dtype=idx.dtype, pin_memory=True)
    h_cnt = torch.empty(cnt.shape, dtype=cnt.dtype, pin_memory=True)
    h_idx.copy_(idx, non_blocking=True)
    h_cnt.copy_(cnt, non_blocking=True)
    torch.cuda.synchronize()
    idx.fill_(-5)
    cnt.fill_(0)
    idx2, cnt2 = torch.empty_like(idx), torch.empty_like(cnt)
    idx2.copy_(h_idx, non_blocking=True)
    cnt2.copy_(h_cnt, non_blocking=True)
    torch.cuda.synchronize()
    assert np.array_equal(idx2.cpu().numpy(), want_idx) and np.array_equal(cnt2.cpu().numpy(), want_cnt)
    dqb, dkb, dvb = _dev(qb, kb, vb)
    out = sp.attn_from_list(dqb, dkb, dvb, idx2, cnt2)
    via_mask = sp.block_sparse_attn(dqb, dkb, dvb, mask_id=mask_a)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), via_mask.view(torch.int16))
    got = to_host_f64(out)
    res = parallel_heads(lambda b, h: compare_out(got[b, h], oracle.masked_attention(
        F64(qb[b, h])[None, None], F64(kb[b, h])[None, None], F64(vb[b, h])[None, None],
        m_a[b, h][None, None])[0, 0]), [(0, 0), (0, 1)])
    worst = {"max_abs": max(r["max_abs"] for r in res), "mean_abs": max(r["mean_abs"] for r in res)}
    parity_log.append(("plan reuse (wan1.3b grid, 2 heads, plan of seed 0 on seed 1)", worst))
    print(worst)
    assert worst["max_abs"] <= 2e-2 and worst["mean_abs"] <= 2e-3


@pytest.mark.parametrize("causal", [False, True])
def test_deterministic_full_size(gpu_lib, causal):
    """Bit-identical reruns at full occupancy (the Wan2.1-1.3B-shaped workload):
    masks, lists and outputs, through the one-call path and the list path."""
    wl = synth.WORKLOADS[1]
    dq, dk, dv = _dev(*synth.make_qkv(wl, seed=0))
    o1, m1 = sp.attn_topk(dq, dk, dv, topk=0.5, return_mask=True, is_causal=causal)
    o2, m2 = sp.attn_topk(dq, dk, dv, topk=0.5, return_mask=True, is_causal=causal)
    _, i1, c1 = sp.predict_mask(sp.pool_blocks(dq, 128), sp.pool_blocks(dk, 64), wl.N, 0.5, is_causal=causal)
    _, i2, c2 = sp.predict_mask(sp.pool_blocks(dq, 128), sp.pool_blocks(dk, 64), wl.N, 0.5, is_causal=causal)
    a1 = sp.attn_from_list(dq, dk, dv, i1, c1, is_causal=causal)
    a2 = sp.attn_from_list(dq, dk, dv, i2, c2, is_causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(m1, m2) and torch.equal(c1, c2)
    # list entries past a row's count are not written (causal rows keep fewer)
    valid = torch.arange(i1.shape[-1], device=i1.device) < c1.unsqueeze(-1).long()
    assert torch.equal(torch.where(valid, i1, 0), torch.where(valid, i2, 0))
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(a1.view(torch.int16), a2.view(torch.int16))
    assert torch.equal(a1.view(torch.int16), o1.view(torch.int16))


def test_predict_at_length_limit(gpu_lib):
    """The longest sequence the prediction accepts (one 48 KB score row per workgroup)."""
    N, D = 786432, 64
    wl = synth.custom(1, 1, N, D, config_id=300)
    q, k = synth.make_tensor(wl, "q"), synth.make_tensor(wl, "k")
    qbar, kbar = sp.pool_blocks(to_dev(q), 128), sp.pool_blocks(to_dev(k), 64)
    mask, idx, cnt = sp.predict_mask(qbar, kbar, N, 0.05)
    m = mask.cpu().numpy()
    kk = oracle.topk_count(N // 64, 0.05)
    assert (m.sum(-1) == kk).all() and (cnt.cpu().numpy() == kk).all()
    rep = oracle_mask_parity(lambda b, h: F64(q[b, h]), lambda b, h: F64(k[b, h]), 0.05, m)
    print(rep)
    assert rep["failures"] == 0
    with pytest.raises(sp.SpargeArgumentError):
        sp.predict_mask(torch.zeros(1, 1, 6145, D, device="cuda"),
                        torch.zeros(1, 1, 12289, D, device="cuda"), N + 64, 0.05)


# ------------------------------------------------------------ full-size workloads

def _sample_rows(N, rng, n=48):
    tail = np.arange(max(0, N - 16), N)
    head = np.arange(0, min(N, 8))
    mid = rng.choice(N, size=min(N, n), replace=False)
    return np.unique(np.concatenate([head, mid, tail]))


WORKLOAD_CASES = [(0, 0.5), (1, 0.5), (2, 0.4), (3, 0.3), (4, 0.1)]


def _block_rows(N):
    """The first row of every query block plus the last row of the sequence."""
    return np.unique(np.concatenate([np.arange(0, N, 128), [N - 1]]))


@pytest.mark.parametrize("cfg,topk", WORKLOAD_CASES, ids=[f"cfg{c}-topk{t}" for c, t in WORKLOAD_CASES])
def test_workload_parity(gpu_lib, parity_log, cfg, topk):
    """Every mask row at the workload's full size. Outputs: every row of every head
    on the three smaller workloads; on the two 720p workloads the first row of every
    query block (and the last row of the sequence) of every head."""
    wl = synth.WORKLOADS[cfg]
    print(f"workload {wl.describe()} topk={topk}", flush=True)
    q, k, v = synth.make_qkv(wl, seed=0)
    dq, dk, dv = _dev(q, k, v)
    out, mask = sp.attn_topk(dq, dk, dv, topk=topk, return_mask=True)
    torch.cuda.synchronize()
    m = mask.cpu().numpy()
    rep = oracle_mask_parity(lambda b, h: F64(q[b, h]), lambda b, h: F64(k[b, h]), topk, m)
    print("mask parity", rep, flush=True)
    assert rep["failures"] == 0
    outs = out.view(torch.int16).cpu().numpy().view(np.uint16)
    del dq, dk, dv, out
    heads = [(b, h) for b in range(wl.B) for h in range(wl.H)]
    full = cfg <= 2
    rows = np.arange(wl.N) if full else _block_rows(wl.N)

    def one(b, h):
        if full:
            ref = oracle.masked_attention(F64(q[b, h])[None, None], F64(k[b, h])[None, None],
                                          F64(v[b, h])[None, None], m[b, h][None, None])[0, 0]
        else:
            ref = oracle.masked_attention_sampled(F64(q[b, h]), F64(k[b, h]), F64(v[b, h]), m[b, h], rows)
        got = F64(outs[b, h][rows])
        assert np.isfinite(got).all(), (b, h)
        return compare_out(got, ref)

    res = parallel_heads(one, heads)
    worst_max = max(r["max_abs"] for r in res)
    mean = float(np.mean([r["mean_abs"] for r in res]))
    worst_mean = max(r["mean_abs"] for r in res)
    parity_log.append((f"{wl.name} topk={topk}", {
        "mask_rows": rep["rows"], "near_tie_rows": rep["candidates"], "differing": rep["differing"],
        "out_rows": int(len(rows) * len(heads)), "max_abs": worst_max, "mean_abs": mean}))
    print("output parity", {"rows": len(rows), "heads": len(heads), "max_abs": worst_max,
                            "mean_abs": mean, "worst_head_mean_abs": worst_mean}, flush=True)
    assert worst_max <= 2e-2 and worst_mean <= 2e-3


@pytest.mark.parametrize("topk", [0.1, 0.2, 0.5, 1.0])
def test_wan14b_topk_sweep(gpu_lib, topk):
    """The other points of the 720p Wan2.1-14B sweep: counts, one head's mask, sampled outputs."""
    wl = synth.WORKLOADS[3]
    heads = [(0, 0), (0, 39)]
    q, k, v = synth.make_qkv(wl, seed=0)
    out, mask = sp.attn_topk(*_dev(q, k, v), topk=topk, return_mask=True)
    m = mask.cpu().numpy()
    kk = oracle.topk_count(m.shape[-1], topk)
    assert (m.sum(-1) == kk).all()
    rng = np.random.default_rng(int(topk * 10))
    for b, h in heads:
        pr = oracle.predict_mask(F64(q[b, h])[None, None], F64(k[b, h])[None, None], topk)
        rep = oracle.mask_parity(pr["logits"], pr["mask"], m[b, h][None, None], kk)
        assert rep["failures"] == 0, rep
        rows = _sample_rows(wl.N, rng, 24)
        got = synth.bf16_bits_to_f64(out.view(torch.int16)[b, h, torch.from_numpy(rows).cuda()].cpu().numpy().view(np.uint16))
        ref = oracle.masked_attention_rows(F64(q[b, h]), F64(k[b, h]), F64(v[b, h]), m[b, h], rows)
        assert_close(got, ref, f"topk {topk} head {(b, h)}")

# ------------------------------------------------------------------ causal


@pytest.mark.parametrize("B,H,N,D", SMALL + [(1, 2, 2000, 128)])
@pytest.mark.parametrize("topk", [0.2, 0.5, 1.0])
def test_causal_predict(gpu_lib, B, H, N, D, topk):
    q, k, v = rand_qkv(B, H, N, D, seed=7 * N + D, q_scale=1 / math.sqrt(D))
    dq, dk = to_dev(q), to_dev(k)
    mask, idx, cnt = sp.predict_mask(sp.pool_blocks(dq, 128), sp.pool_blocks(dk, 64), N, topk,
                                     is_causal=True)
    m, idx, cnt = mask.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy()
    rep = oracle_mask_parity(lambda b, h: F64(q[b, h]), lambda b, h: F64(k[b, h]), topk, m, causal=True)
    assert rep["failures"] == 0, rep
    cand = np.array([oracle.causal_key_blocks(N, i) for i in range(m.shape[2])])
    kk = np.array([oracle.topk_count(int(c), topk) for c in cand])
    assert (cnt == kk[None, None]).all()
    assert (m.sum(-1) == kk[None, None]).all()
    for b in range(B):
        for h in range(H):
            for i in range(m.shape[2]):
                assert idx[b, h, i, : kk[i]].tolist() == np.flatnonzero(m[b, h, i]).tolist()


@pytest.mark.parametrize("B,H,N,D", SMALL)
def test_causal_user_mask(gpu_lib, B, H, N, D):
    q, k, v = rand_qkv(B, H, N, D, seed=11 * N + D)
    m = _random_mask(B, H, N, 0.5, seed=N + 1)
    out = sp.block_sparse_attn(*_dev(q, k, v), mask_id=torch.from_numpy(m).cuda(), is_causal=True)
    ref = oracle.masked_attention(F64(q), F64(k), F64(v), m, causal=True)
    print(assert_close(to_host_f64(out), ref, f"causal user mask {B, H, N, D}"))


@pytest.mark.parametrize("B,H,N,D", SMALL)
def test_causal_dense_and_topk_one(gpu_lib, B, H, N, D):
    q, k, v = rand_qkv(B, H, N, D, seed=13 * N + D)
    dq, dk, dv = _dev(q, k, v)
    dense = sp.block_sparse_attn(dq, dk, dv, mask_id=None, is_causal=True)
    top1, mask = sp.attn_topk(dq, dk, dv, topk=1.0, is_causal=True, return_mask=True)
    torch.cuda.synchronize()
    m = mask.cpu().numpy()
    cand = np.array([oracle.causal_key_blocks(N, i) for i in range(m.shape[2])])
    assert (m.sum(-1) == cand[None, None]).all()
    t = lambda a: torch.from_numpy(F64(a))
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=True).numpy()
    assert_close(to_host_f64(dense), ref, "dense causal vs SDPA")
    assert_close(to_host_f64(top1), ref, "topk 1.0 causal vs SDPA")
    # same kept tiles, but the dense walk also visits the future blocks (all masked): equal values
    assert np.abs(to_host_f64(dense) - to_host_f64(top1)).max() == 0.0


@pytest.mark.parametrize("N", EDGE_N + [255, 256, 257])
@pytest.mark.parametrize("D", [64, 128])
def test_causal_edge_lengths(gpu_lib, N, D):
    q, k, v = rand_qkv(1, 2, N, D, seed=N * 5 + D)
    dq, dk, dv = _dev(q, k, v)
    out, mask = sp.attn_topk(dq, dk, dv, topk=0.5, is_causal=True, return_mask=True)
    m = mask.cpu().numpy()
    ref = oracle.masked_attention(F64(q), F64(k), F64(v), m, causal=True)
    assert_close(to_host_f64(out), ref, f"causal edge N={N}")
    rep = oracle_mask_parity(lambda b, h: F64(q[b, h]), lambda b, h: F64(k[b, h]), 0.5, m, causal=True)
    assert rep["failures"] == 0


@pytest.mark.parametrize("cfg,topk", [(1, 0.5), (2, 0.4)], ids=["cfg1-topk0.5", "cfg2-topk0.4"])
def test_causal_workload_parity(gpu_lib, cfg, topk):
    """Causal top-k at a workload's full size: every mask row, sampled output rows."""
    wl = synth.WORKLOADS[cfg]
    print(f"causal workload {wl.describe()} topk={topk}", flush=True)
    q, k, v = synth.make_qkv(wl, seed=0)
    out, mask = sp.attn_topk(*_dev(q, k, v), topk=topk, is_causal=True, return_mask=True)
    torch.cuda.synchronize()
    m = mask.cpu().numpy()
    rep = oracle_mask_parity(lambda b, h: F64(q[b, h]), lambda b, h: F64(k[b, h]), topk, m, causal=True)
    print("mask parity", rep, flush=True)
    assert rep["failures"] == 0
    rng = np.random.default_rng(100 + cfg)
    outs = out.view(torch.int16)
    for b, h in sorted({(0, 0), (wl.B - 1, wl.H - 1)}):
        rows = _sample_rows(wl.N, rng)
        got = synth.bf16_bits_to_f64(outs[b, h, torch.from_numpy(rows).cuda()].cpu().numpy().view(np.uint16))
        ref = oracle.masked_attention_rows(F64(q[b, h]), F64(k[b, h]), F64(v[b, h]), m[b, h], rows, causal=True)
        print(assert_close(got, ref, f"causal cfg{cfg} head {(b, h)}"), flush=True)


# ------------------------------------------------------------ token layouts


@pytest.mark.parametrize("layout", ["cube", "morton"])
@pytest.mark.parametrize("D", [64, 128])
def test_permute_tokens(gpu_lib, layout, D):
    n_text, grid = 37, (5, 9, 14)
    N = n_text + grid[0] * grid[1] * grid[2]
    q, _, _ = rand_qkv(2, 3, N, D, seed=61 + D)
    perm = sp.token_permutation(n_text, grid, layout)
    dperm = perm.cuda()
    x = to_dev(q)
    y = sp.permute_tokens(x, dperm)
    back = sp.permute_tokens(y, dperm, inverse=True)
    # strided in and out: (B, N, H, D) storage
    xt = x.transpose(1, 2).contiguous().transpose(1, 2)
    yt = torch.empty(2, N, 3, D, dtype=torch.bfloat16, device="cuda").transpose(1, 2)
    sp.permute_tokens(xt, dperm, out=yt)
    torch.cuda.synchronize()
    want = oracle.permute_tokens(q, perm.numpy())
    assert np.array_equal(y.view(torch.int16).cpu().numpy().view(np.uint16), want)
    assert np.array_equal(back.view(torch.int16).cpu().numpy().view(np.uint16), q)
    assert torch.equal(yt.contiguous().view(torch.int16), y.view(torch.int16))


def test_permute_tokens_full_size(gpu_lib):
    """The Wan2.1-14B 720p grid (40 heads, 75600 tokens): bit-exact cube reorder and restore."""
    wl = synth.WORKLOADS[3]
    q = synth.make_tensor(wl, "q", heads=[(0, h) for h in range(wl.H)])
    perm = sp.token_permutation(0, wl.grid, "cube")
    x = to_dev(q)
    y = sp.permute_tokens(x, perm.cuda())
    back = sp.permute_tokens(y, perm.cuda(), inverse=True)
    torch.cuda.synchronize()
    p = perm.numpy().astype(np.int64)
    yh = y.view(torch.int16).cpu().numpy().view(np.uint16)
    for h in (0, 17, 39):
        assert np.array_equal(yh[0, h], q[0, h][p])
    assert torch.equal(back.view(torch.int16), x.view(torch.int16))


@pytest.mark.parametrize("layout", ["cube", "morton"])
def test_attention_in_cube_layout(gpu_lib, layout):
    """Reorder, top-k attention, restore: equals the oracle run in the reordered space."""
    small = synth.custom(1, 2, 226 + 4 * 10 * 12, 64, config_id=62, grid=(4, 10, 12), n_text=226, q_scale=0.125)
    q, k, v = synth.make_qkv(small, seed=0)
    perm = sp.token_permutation(226, (4, 10, 12), layout)
    dperm = perm.cuda()
    dq, dk, dv = (sp.permute_tokens(t, dperm) for t in _dev(q, k, v))
    out_p, mask = sp.attn_topk(dq, dk, dv, topk=0.4, return_mask=True)
    out = sp.permute_tokens(out_p, dperm, inverse=True)
    m = mask.cpu().numpy()
    p = perm.numpy()
    qp, kp, vp = (oracle.permute_tokens(F64(t), p) for t in (q, k, v))
    rep = oracle_mask_parity(lambda b, h: qp[b, h], lambda b, h: kp[b, h], 0.4, m)
    assert rep["failures"] == 0, rep
    ref = oracle.permute_tokens(oracle.masked_attention(qp, kp, vp, m), p, inverse=True)
    print(assert_close(to_host_f64(out), ref, f"{layout} layout"), rep)


# ------------------------------------------------------------ CDF-threshold selection


def _cdf_parity(q, k, tau, m, scale=None, causal=False):
    B, H = m.shape[:2]
    tot = {"rows": 0, "differing": 0, "excused": 0, "failures": 0}
    for b in range(B):
        for h in range(H):
            pr = oracle.predict_mask_cdf(F64(q[b, h])[None, None], F64(k[b, h])[None, None], tau, scale,
                                         causal=causal)
            rep = oracle.mask_parity_cdf(pr["logits"], pr["probs"], pr["mask"], m[b, h][None, None], tau,
                                         cand=pr["cand"])
            for key in tot:
                tot[key] += rep[key]
    return tot


@pytest.mark.parametrize("B,H,N,D", SMALL)
@pytest.mark.parametrize("tau", [0.3, 0.7, 0.95, 1.0])
@pytest.mark.parametrize("causal", [False, True])
def test_cdf_predict(gpu_lib, B, H, N, D, tau, causal):
    # a large logit scale makes the block probabilities uneven, so tau matters
    q, k, v = rand_qkv(B, H, N, D, seed=17 * N + D)
    scale = 40.0
    mask, idx, cnt = sp.predict_mask_cdf(sp.pool_blocks(to_dev(q), 128), sp.pool_blocks(to_dev(k), 64), N, tau,
                                         scale=scale, is_causal=causal)
    m, idx, cnt = mask.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy()
    rep = _cdf_parity(q, k, tau, m, scale, causal)
    print(rep, "kept fraction", m.mean())
    assert rep["failures"] == 0, rep
    assert (cnt == m.sum(-1)).all()
    for b in range(B):
        for h in range(H):
            for i in range(m.shape[2]):
                assert idx[b, h, i, : cnt[b, h, i]].tolist() == np.flatnonzero(m[b, h, i]).tolist()
    if tau == 1.0:
        cand = np.array([oracle.causal_key_blocks(N, i) if causal else m.shape[3] for i in range(m.shape[2])])
        assert (cnt == cand[None, None]).all()


@pytest.mark.parametrize("B,H,N,D", SMALL[:3])
@pytest.mark.parametrize("causal", [False, True])
def test_attn_cdf(gpu_lib, B, H, N, D, causal):
    q, k, v = rand_qkv(B, H, N, D, seed=19 * N + D)
    out, mask = sp.attn_cdf(*_dev(q, k, v), tau=0.6, scale=0.5, is_causal=causal, return_mask=True)
    m = mask.cpu().numpy()
    ref = oracle.masked_attention(F64(q), F64(k), F64(v), m, scale=0.5, causal=causal)
    print(assert_close(to_host_f64(out), ref, f"cdf {B, H, N, D} causal={causal}"), "kept", m.mean())
    rep = _cdf_parity(q, k, 0.6, m, 0.5, causal)
    assert rep["failures"] == 0, rep


# Rows of 2304 key blocks are the longest that eight share a workgroup's LDS;
# one more key block halves the rows per workgroup.
@pytest.mark.parametrize("N", [2304 * 64, 2304 * 64 + 1])
@pytest.mark.parametrize("mode", ["topk", "cdf"])
def test_predict_workgroup_sizes(gpu_lib, N, mode):
    D = 64
    wl = synth.custom(1, 1, N, D, config_id=301)
    q, k = synth.make_tensor(wl, "q"), synth.make_tensor(wl, "k")
    print(f"N={N} mode={mode}", flush=True)
    qbar, kbar = sp.pool_blocks(to_dev(q), 128), sp.pool_blocks(to_dev(k), 64)
    if mode == "topk":
        mask, idx, cnt = sp.predict_mask(qbar, kbar, N, 0.2)
        m = mask.cpu().numpy()
        rep = oracle_mask_parity(lambda b, h: F64(q[b, h]), lambda b, h: F64(k[b, h]), 0.2, m)
    else:
        mask, idx, cnt = sp.predict_mask_cdf(qbar, kbar, N, 0.5, scale=8.0)
        m = mask.cpu().numpy()
        rep = _cdf_parity(q, k, 0.5, m, 8.0)
    print(rep, flush=True)
    assert rep["failures"] == 0, rep
    idx, cnt = idx.cpu().numpy(), cnt.cpu().numpy()
    assert (cnt == m.sum(-1)).all()
    for i in range(m.shape[2]):
        assert idx[0, 0, i, : cnt[0, 0, i]].tolist() == np.flatnonzero(m[0, 0, i]).tolist()


@pytest.mark.parametrize("cfg,tau", [(1, 0.9), (2, 0.8)], ids=["cfg1-tau0.9", "cfg2-tau0.8"])
def test_cdf_workload_parity(gpu_lib, cfg, tau):
    """CDF selection at a workload's full size: every mask row, sampled output rows."""
    wl = synth.WORKLOADS[cfg]
    print(f"cdf workload {wl.describe()} tau={tau}", flush=True)
    q, k, v = synth.make_qkv(wl, seed=0)
    out, mask = sp.attn_cdf(*_dev(q, k, v), tau=tau, return_mask=True)
    torch.cuda.synchronize()
    m = mask.cpu().numpy()
    rep = _cdf_parity(q, k, tau, m)
    print("mask parity", rep, "kept fraction", float(m.mean()), flush=True)
    assert rep["failures"] == 0
    rng = np.random.default_rng(200 + cfg)
    outs = out.view(torch.int16)
    for b, h in sorted({(0, 0), (wl.B - 1, wl.H - 1)}):
        rows = _sample_rows(wl.N, rng)
        got = synth.bf16_bits_to_f64(outs[b, h, torch.from_numpy(rows).cuda()].cpu().numpy().view(np.uint16))
        ref = oracle.masked_attention_rows(F64(q[b, h]), F64(k[b, h]), F64(v[b, h]), m[b, h], rows)
        print(assert_close(got, ref, f"cdf cfg{cfg} head {(b, h)}"), flush=True)


# ------------------------------------------------------------ binding argument checks

def test_binding_rejects_misplaced_buffers(gpu_lib):
    """Outputs, lists, masks and workspaces that do not match q are refused before any launch."""
    B, H, N, D = 1, 2, 300, 64
    q, k, v = _dev(*rand_qkv(B, H, N, D, seed=5))
    qbar, kbar = sp.pool_blocks(q, 128), sp.pool_blocks(k, 64)
    mask, idx, cnt = sp.predict_mask(qbar, kbar, N, 0.5)
    bad_outs = [torch.empty(B, H, N - 1, D, dtype=torch.bfloat16, device="cuda"),   # wrong shape
                torch.empty(B, H, N, D, dtype=torch.float32, device="cuda"),        # wrong dtype
                torch.empty(B, H, N, D, dtype=torch.bfloat16),                      # host memory
                torch.empty(B, H, D, N, dtype=torch.bfloat16, device="cuda").transpose(2, 3)]  # D strided
    for bad in bad_outs:
        for call in (lambda o: sp.attn_topk(q, k, v, topk=0.5, out=o),
                     lambda o: sp.block_sparse_attn(q, k, v, mask_id=mask, out=o),
                     lambda o: sp.attn_from_list(q, k, v, idx, cnt, out=o),
                     lambda o: sp.attn_cdf(q, k, v, tau=0.5, out=o)):
            with pytest.raises(ValueError):
                call(bad)
    with pytest.raises(ValueError):
        sp.attn_from_list(q, k, v, idx.cpu(), cnt)
    with pytest.raises(ValueError):
        sp.attn_from_list(q, k, v, idx, cnt.cpu())
    with pytest.raises(ValueError):
        sp.block_sparse_attn(q, k, v, mask_id=mask.cpu())
    with pytest.raises(ValueError):
        sp.compact_mask(mask.cpu(), N)
    with pytest.raises(ValueError):
        sp.predict_mask(qbar.cpu(), kbar, N, 0.5)
    with pytest.raises(ValueError):
        sp.predict_mask_cdf(qbar, kbar.cpu(), N, 0.5)
    ws = torch.empty(sp.workspace_bytes(B, H, N, D, 0.5), dtype=torch.uint8)
    with pytest.raises(ValueError):
        sp.attn_topk(q, k, v, topk=0.5, workspace=ws)
    with pytest.raises(ValueError):
        sp.permute_tokens(q, torch.arange(N, dtype=torch.int32), out=None)   # host permutation
    torch.cuda.synchronize()


def test_strided_output(gpu_lib):
    """A caller's output view with padded rows receives the same bytes as a fresh tensor."""
    B, H, N, D = 2, 2, 700, 64
    q, k, v = _dev(*rand_qkv(B, H, N, D, seed=6))
    ref = sp.attn_topk(q, k, v, topk=0.4)
    big = torch.full((B, N, H, 2 * D), -7.0, dtype=torch.bfloat16, device="cuda")
    view = big[..., :D].transpose(1, 2)          # (B, H, N, D), token stride H * 2D
    got = sp.attn_topk(q, k, v, topk=0.4, out=view)
    torch.cuda.synchronize()
    assert got.data_ptr() == view.data_ptr()
    assert torch.equal(view.contiguous().view(torch.int16), ref.view(torch.int16))
    assert bool((big[..., D:] == -7.0).all())   # padding untouched
