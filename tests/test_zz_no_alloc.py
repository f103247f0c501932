"""The no-allocation top-k call (sparge_attn_topk_noalloc, workspace in a fixed
device array) against the regular call with a caller workspace: bit-identical
outputs and masks on two calls in a row, the second on a smaller input, through
the C ABI."""
import ctypes
import math

import numpy as np
import pytest
import torch

import block_sparse_attention_sparge_amd as sp
from gpu_harness import rand_qkv, to_dev

pytestmark = pytest.mark.gpu


def _noalloc(lib, q, k, v, topk, out, mask, causal=0):
    B, H, N, D = q.shape
    st = lambda t: (ctypes.c_int64 * 3)(t.stride(0), t.stride(1), t.stride(2))
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return lib.sparge_attn_topk_noalloc(p(q), p(k), p(v), float(topk), p(out), B, H, N, D, st(q), st(k),
                                        st(v), st(out), 0.0, causal, p(mask), stream)


def test_noalloc_matches_workspace_call(gpu_lib):
    lib = sp.load_library()
    cases = [(1, 4, 9000, 128, 0.3, 0), (2, 3, 1500, 64, 0.5, 1)]      # the second call is smaller
    for B, H, N, D, topk, causal in cases:
        print(f"noalloc case B={B} H={H} N={N} D={D} topk={topk} causal={causal}", flush=True)
        q, k, v = (to_dev(x) for x in rand_qkv(B, H, N, D, seed=N + D, q_scale=1 / math.sqrt(D)))
        ref, ref_mask = sp.attn_topk(q, k, v, topk=topk, is_causal=bool(causal), return_mask=True)
        out = torch.full_like(q, 7.0)
        mask = torch.full(sp.mask_shape(B, H, N), 9, dtype=torch.uint8, device="cuda")
        assert _noalloc(lib, q, k, v, topk, out, mask, causal) == 0
        torch.cuda.synchronize()
        assert torch.equal(mask, ref_mask)
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


def test_noalloc_refuses_beyond_its_array(gpu_lib):
    lib = sp.load_library()
    # 720p Wan shape at topk 0.9 needs about 135 MiB of workspace: refused before any launch
    assert sp.workspace_bytes(1, 40, 75600, 128, 0.9) > 128 << 20
    S = lambda *x: (ctypes.c_int64 * 3)(*x)
    st = S(40 * 75600 * 128, 75600 * 128, 128)
    a, b, c, o = (0x40000000 * i for i in range(1, 5))    # 1 GiB apart: no overlap
    rc = lib.sparge_attn_topk_noalloc(a, b, c, 0.9, o, 1, 40, 75600, 128, st, st, st, st, 0.0, 0, None, None)
    assert rc == -10
    assert b"128 MiB" in lib.sparge_status_string(-10)
