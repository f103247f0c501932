"""The C-ABI library: it loads, exports what include/sparge.h declares, and its
host-side validation rejects bad arguments with the documented status before
any HIP call (so these tests run without a GPU; no call here is valid)."""
import ctypes
import os
import re

import pytest

import block_sparse_attention_sparge_amd as sp
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparge.h")

OK, NULL, SHAPE, TOPK, STRIDE, ALIAS, WORKSPACE, ARG, MASK_VALUE = 0, -1, -2, -3, -4, -5, -6, -7, -9


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) -
                  {"defined", "sizeof"})


@pytest.fixture(scope="module")
def lib():
    return sp.load_library()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"sparge_pool_blocks", "sparge_predict_mask", "block_sparse_attn", "sparge_attn_topk",
            "sparge_workspace_bytes", "sparge_status_string", "sparge_topk_count",
            "sparge_compact_mask", "sparge_attn_from_list"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code in (OK, NULL, SHAPE, TOPK, STRIDE, ALIAS, WORKSPACE, ARG, -8, MASK_VALUE, 12345):
        assert lib.sparge_status_string(code)
    assert b"0 or 1" in lib.sparge_status_string(MASK_VALUE)


def test_topk_count_matches_oracle_and_golden(lib):
    rows = [l.split() for l in open(os.path.join(ROOT, "tests", "golden", "topk_counts.txt"))
            if l.strip() and not l.startswith("#")]
    for kb, topk, k in rows:
        assert sp.topk_count(int(kb), float(topk)) == int(k)
    for kb in (1, 2, 3, 10, 16, 100, 278, 512, 1182, 1861, 4097):
        for t in range(1, 101):
            assert sp.topk_count(kb, t / 100) == oracle.topk_count(kb, t / 100), (kb, t)
    out = ctypes.c_int64(0)
    assert lib.sparge_topk_count(10, 0.0, ctypes.byref(out)) == TOPK
    assert lib.sparge_topk_count(10, 1.0000001, ctypes.byref(out)) == TOPK
    assert lib.sparge_topk_count(10, float("nan"), ctypes.byref(out)) == TOPK
    assert lib.sparge_topk_count(0, 0.5, ctypes.byref(out)) == ARG
    assert lib.sparge_topk_count(10, 0.5, None) == NULL


def test_workspace_bytes(lib):
    # topk path: qbar + kbar (fp32) + kept lists + counts, each 256-byte aligned
    B, H, N, D = 1, 40, 75600, 128
    qb, kb, k = 591, 1182, 355
    up = lambda x: (x + 255) // 256 * 256
    want = up(B * H * qb * D * 4) + up(B * H * kb * D * 4) + up(B * H * qb * k * 4) + up(B * H * qb * 4)
    assert sp.workspace_bytes(B, H, N, D, 0.3) == want
    assert sp.workspace_bytes(B, H, N, D) == up(B * H * qb * kb * 4) + up(B * H * qb * 4)
    assert sp.workspace_bytes(1, 1, 100, 96) == 0            # bad D
    assert sp.workspace_bytes(1, 1, 0, 64) == 0              # bad N
    assert sp.workspace_bytes(1, 1, 100, 64, 1.5) == 0       # bad topk


# Fake, 16-byte aligned, well separated "device" addresses: every call below is
# rejected by the host checks, so they are never dereferenced.
A, Bp, C, O, W, M = (0x10000000 * i for i in range(1, 7))
S = lambda *x: (ctypes.c_int64 * 3)(*x)


def contiguous(H, N, D):
    return S(H * N * D, N * D, D)


def attn_call(lib, fn, q=A, k=Bp, v=C, out=O, B=1, H=2, N=256, D=64, qs=None, ks=None, vs=None,
              os_=None, mask=None, ws=0, wsb=0, topk=0.5, causal=0):
    st = contiguous(H, N, D)
    qs, ks, vs, os_ = (x or st for x in (qs, ks, vs, os_))
    if fn == "topk":
        return lib.sparge_attn_topk(q, k, v, topk, out, B, H, N, D, qs, ks, vs, os_, 0.0, causal, mask,
                                    ws, wsb, None)
    if fn == "checked":
        return lib.block_sparse_attn_checked(q, k, v, mask, out, B, H, N, D, qs, ks, vs, os_, 0.0, causal,
                                             ws, wsb, None)
    return lib.block_sparse_attn(q, k, v, mask, out, B, H, N, D, qs, ks, vs, os_, 0.0, causal, ws, wsb,
                                 None)


@pytest.mark.parametrize("fn", ["topk", "mask", "checked"])
def test_attention_argument_errors(lib, fn):
    mask = None if fn == "topk" else M
    assert attn_call(lib, fn, q=None, mask=mask) == NULL
    assert attn_call(lib, fn, out=None, mask=mask) == NULL
    assert attn_call(lib, fn, D=96, mask=mask) == SHAPE
    assert attn_call(lib, fn, N=0, mask=mask) == SHAPE
    assert attn_call(lib, fn, B=0, mask=mask) == SHAPE
    assert attn_call(lib, fn, N=(1 << 31) - 127, mask=mask) == SHAPE                 # 32-bit key arithmetic
    assert attn_call(lib, fn, qs=S(2 * 256 * 64, 256 * 64, 60), mask=mask) == STRIDE   # not a multiple of 8
    assert attn_call(lib, fn, ks=S(-8, 256 * 64, 64), mask=mask) == STRIDE
    assert attn_call(lib, fn, q=A + 8, mask=mask) == STRIDE                          # misaligned
    assert attn_call(lib, fn, ks=S(256 * 64, 0, 0), mask=mask) == STRIDE              # K expanded along N
    assert attn_call(lib, fn, vs=S(2 * 256 * 32, 256 * 32, 32), mask=mask) == STRIDE  # V rows overlap
    assert attn_call(lib, fn, os_=S(2 * 256 * 64, 256 * 64, 32), mask=mask) == STRIDE  # rows overlap
    assert attn_call(lib, fn, out=A + 1024, mask=mask) == ALIAS                      # out inside q
    assert attn_call(lib, fn, out=C - 1024, mask=mask) == ALIAS                      # out runs into v
    for bad in (2, -1):
        assert attn_call(lib, fn, mask=mask, causal=bad, ws=W, wsb=1 << 30) == ARG
    assert attn_call(lib, fn, mask=mask, ws=0, wsb=0) == WORKSPACE
    assert attn_call(lib, fn, mask=mask, ws=W, wsb=16) == WORKSPACE
    need = sp.workspace_bytes(1, 2, 256, 64, 0.5 if fn == "topk" else None)
    assert attn_call(lib, fn, mask=mask, ws=O + 4096, wsb=need) == ALIAS              # workspace inside out
    if fn == "topk":
        for bad in (0.0, -0.5, 1.01, float("nan")):
            assert attn_call(lib, fn, topk=bad, ws=W, wsb=1 << 30) == TOPK
        assert attn_call(lib, fn, N=786433, ws=W, wsb=1 << 40) == SHAPE              # beyond the predict limit
        assert lib.sparge_attn_topk(A, Bp, C, 0.5, O, 1, 2, 256, 64, contiguous(2, 256, 64),
                                    contiguous(2, 256, 64), contiguous(2, 256, 64),
                                    contiguous(2, 256, 64), 0.0, 0, A + 64, W, need, None) == ALIAS
    else:
        assert attn_call(lib, fn, mask=O + 64, ws=W, wsb=need) == ALIAS                 # mask inside out
        assert attn_call(lib, fn, mask=W + 64, ws=W, wsb=need) == ALIAS                 # mask inside workspace


def test_check_mask_errors(lib):
    # every rejection happens on the host, before the device scan
    assert lib.sparge_check_mask(None, 1, 2, 256, W, 4096, None) == NULL
    assert lib.sparge_check_mask(M, 1, 0, 256, W, 4096, None) == SHAPE
    assert lib.sparge_check_mask(M, 1, 2, 256, None, 4096, None) == WORKSPACE
    assert lib.sparge_check_mask(M, 1, 2, 256, W, 0, None) == WORKSPACE       # needs 4 bytes (16 mask bytes)
    assert lib.sparge_check_mask(M, 1, 2, 256, W + 4, 4096, None) == WORKSPACE   # misaligned
    assert lib.sparge_check_mask(M, 1, 2, 256, M, 4096, None) == ALIAS
    # the workspace the checking attention call needs also holds the flags
    for n in (1, 63, 256, 75600):
        rows, kb = -(-n // 128), -(-n // 64)
        flags = 4 * min(1024, -(-(rows * kb) // 256))
        assert sp.workspace_bytes(1, 1, n, 64) >= flags


def test_pool_predict_compact_errors(lib):
    st = contiguous(2, 256, 64)
    assert lib.sparge_pool_blocks(None, 1, 2, 256, 64, st, 128, O, None) == NULL
    assert lib.sparge_pool_blocks(A, 1, 2, 256, 64, st, 96, O, None) == ARG
    assert lib.sparge_pool_blocks(A, 1, 2, 256, 80, st, 128, O, None) == SHAPE
    assert lib.sparge_pool_blocks(A, 1, 2, 256, 64, S(1, 2, 3), 128, O, None) == STRIDE
    assert lib.sparge_pool_blocks(A, 1, 2, 256, 64, st, 128, A + 512, None) == ALIAS
    assert lib.sparge_predict_mask(None, Bp, 1, 2, 256, 64, 0.5, 0.0, 0, None, C, O, None) == NULL
    assert lib.sparge_predict_mask(A, Bp, 1, 2, 256, 64, 0.5, 0.0, 0, None, None, O, None) == NULL
    assert lib.sparge_predict_mask(A, Bp, 1, 2, 256, 64, 2.0, 0.0, 0, None, C, O, None) == TOPK
    assert lib.sparge_predict_mask(A, Bp, 1, 2, 786433, 64, 0.5, 0.0, 0, None, C, O, None) == SHAPE
    assert lib.sparge_predict_mask(A, Bp, 1, 2, 256, 64, 0.5, 0.0, 0, None, A + 4, O, None) == ALIAS
    assert lib.sparge_predict_mask(A, Bp, 1, 2, 256, 64, 0.5, 0.0, 0, C, C + 4, O, None) == ALIAS
    assert lib.sparge_predict_mask(A, Bp, 1, 2, 256, 64, 0.5, 0.0, 3, None, C, O, None) == ARG
    assert lib.sparge_compact_mask(None, 1, 2, 256, Bp, C, None) == NULL
    assert lib.sparge_compact_mask(A, 1, 2, 0, Bp, C, None) == SHAPE
    assert lib.sparge_compact_mask(A, 1, 2, 256, A + 1, C, None) == ALIAS
    assert lib.sparge_attn_from_list(A, Bp, C, W, None, 4, O, 1, 2, 256, 64, st, st, st, st, 0.0,
                                     0, None) == NULL
    assert lib.sparge_attn_from_list(A, Bp, C, W, M, 0, O, 1, 2, 256, 64, st, st, st, st, 0.0,
                                     0, None) == ARG
    assert lib.sparge_attn_from_list(A, Bp, C, O + 64, M, 4, O, 1, 2, 256, 64, st, st, st, st, 0.0,
                                     0, None) == ALIAS
    assert lib.sparge_attn_from_list(A, Bp, C, W, M, 4, O, 1, 2, 256, 64, st, st, st, st, 0.0,
                                     5, None) == ARG


def test_cdf_errors(lib):
    st = contiguous(2, 256, 64)
    assert lib.sparge_predict_mask_cdf(None, Bp, 1, 2, 256, 64, 0.5, 0.0, 0, None, C, O, None) == NULL
    assert lib.sparge_predict_mask_cdf(A, Bp, 1, 2, 256, 64, 0.0, 0.0, 0, None, C, O, None) == TOPK
    assert lib.sparge_predict_mask_cdf(A, Bp, 1, 2, 256, 64, 1.5, 0.0, 0, None, C, O, None) == TOPK
    assert lib.sparge_predict_mask_cdf(A, Bp, 1, 2, 256, 64, 0.5, 0.0, 2, None, C, O, None) == ARG
    assert lib.sparge_predict_mask_cdf(A, Bp, 1, 2, 786433, 64, 0.5, 0.0, 0, None, C, O, None) == SHAPE
    assert lib.sparge_predict_mask_cdf(A, Bp, 1, 2, 256, 64, 0.5, 0.0, 0, None, A + 4, O, None) == ALIAS
    need = sp.workspace_bytes(1, 2, 256, 64, 1.0)
    call = lambda tau=0.5, causal=0, ws=W, wsb=need, out=O: lib.sparge_attn_cdf(
        A, Bp, C, tau, out, 1, 2, 256, 64, st, st, st, st, 0.0, causal, None, ws, wsb, None)
    assert call(out=None) == NULL
    assert call(tau=float("nan")) == TOPK
    assert call(causal=7) == ARG
    assert call(ws=0) == WORKSPACE
    assert call(wsb=need - 16) == WORKSPACE
    assert call(ws=O + 64) == ALIAS


def test_permute_tokens_errors(lib):
    st = contiguous(2, 256, 64)
    assert lib.sparge_permute_tokens(None, Bp, O, 1, 2, 256, 64, st, st, 0, None) == NULL
    assert lib.sparge_permute_tokens(A, None, O, 1, 2, 256, 64, st, st, 0, None) == NULL
    assert lib.sparge_permute_tokens(A, Bp, O, 1, 2, 256, 96, st, st, 0, None) == SHAPE
    assert lib.sparge_permute_tokens(A, Bp, O, 1, 2, 256, 64, S(1, 2, 3), st, 0, None) == STRIDE
    assert lib.sparge_permute_tokens(A + 8, Bp, O, 1, 2, 256, 64, st, st, 0, None) == STRIDE
    assert lib.sparge_permute_tokens(A, Bp, O, 1, 2, 256, 64, st, S(256 * 64, 256 * 64, 32), 0, None) == STRIDE
    assert lib.sparge_permute_tokens(A, Bp, O, 1, 2, 256, 64, st, st, 2, None) == ARG
    assert lib.sparge_permute_tokens(A, Bp, A + 4096, 1, 2, 256, 64, st, st, 0, None) == ALIAS
    assert lib.sparge_permute_tokens(A, O + 64, O, 1, 2, 256, 64, st, st, 0, None) == ALIAS


def test_python_wrapper_rejects_without_gpu():
    import torch
    x = torch.zeros(1, 1, 128, 64, dtype=torch.bfloat16)
    with pytest.raises(NotImplementedError):
        sp.attn_topk(x.float(), x, x)
    with pytest.raises(ValueError):
        sp.attn_topk(x, x, x)          # CPU tensor
    assert sp.mask_shape(1, 2, 75600) == (1, 2, 591, 1182)


def test_noalloc_scratch_limit(lib):
    """The no-allocation call refuses a shape whose workspace exceeds its fixed
    array on the host, before any HIP call (fake addresses, never dereferenced)."""
    assert sp.workspace_bytes(1, 40, 75600, 128, 0.9) > 128 << 20
    st = S(40 * 75600 * 128, 75600 * 128, 128)
    g = [0x40000000 * i for i in range(1, 5)]       # 1 GiB apart: the 774 MB operands do not overlap
    assert lib.sparge_attn_topk_noalloc(g[0], g[1], g[2], 0.9, g[3], 1, 40, 75600, 128, st, st, st, st, 0.0, 0,
                                        None, None) == -10
    # invalid arguments are reported by the regular call's checks
    assert lib.sparge_attn_topk_noalloc(A, Bp, C, 1.5, O, 1, 2, 256, 64, contiguous(2, 256, 64),
                                        contiguous(2, 256, 64), contiguous(2, 256, 64),
                                        contiguous(2, 256, 64), 0.0, 0, None, None) == TOPK
    assert lib.sparge_attn_topk_noalloc(None, Bp, C, 0.5, O, 1, 2, 256, 64, contiguous(2, 256, 64),
                                        contiguous(2, 256, 64), contiguous(2, 256, 64),
                                        contiguous(2, 256, 64), 0.0, 0, None, None) == NULL
    assert lib.sparge_attn_topk_noalloc(A, Bp, C, 0.5, A + 64, 1, 2, 256, 64, contiguous(2, 256, 64),
                                        contiguous(2, 256, 64), contiguous(2, 256, 64),
                                        contiguous(2, 256, 64), 0.0, 0, None, None) == ALIAS
    assert lib.sparge_attn_topk_noalloc(A, Bp, C, 0.5, O, 1, 2, 256, 64, contiguous(2, 256, 64),
                                        contiguous(2, 256, 64), contiguous(2, 256, 64),
                                        contiguous(2, 256, 64), 0.0, 0, A + 64, None) == ALIAS  # mask in q
