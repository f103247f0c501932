"""Block-sparse (SpargeAttn-style) self-attention on AMD MI355X (gfx950).

Python binding of libsparge's C ABI (include/sparge.h). It only marshals
arguments: torch supplies device memory and the current HIP stream, and every
step of the computation runs in the library's HIP kernels. There is no CPU or
PyTorch fallback: a missing library or GPU raises.

    import block_sparse_attention_sparge_amd as sparge
    out = sparge.attn_topk(q, k, v, topk=0.5)               # drop-in for SDPA (non-causal)
    out = sparge.block_sparse_attn(q, k, v, mask_id=mask)   # given (B, H, ceil(N/128), ceil(N/64)) mask

The two calls mirror SpargeAttention Documentation's spas_sage2_attn_meansim_topk_cuda
and block_sparse_sage2_attn_cuda; the 128x64 block size and the mask_id shape
follow its "Mask Requirements".
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

__all__ = [
    "Q_BLOCK", "K_BLOCK", "LAYOUTS", "SpargeError", "SpargeArgumentError", "load_library", "library_path",
    "topk_count", "workspace_bytes", "pool_blocks", "predict_mask", "predict_mask_cdf", "compact_mask",
    "attn_from_list", "block_sparse_attn", "attn_topk", "attn_cdf", "mask_shape", "token_permutation",
    "permute_tokens", "check_mask",
]

Q_BLOCK = 128
K_BLOCK = 64

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libsparge.so")
_lib = None

_STATUS = {
    0: "SPARGE_OK", -1: "SPARGE_ERR_NULL", -2: "SPARGE_ERR_SHAPE", -3: "SPARGE_ERR_TOPK",
    -4: "SPARGE_ERR_STRIDE", -5: "SPARGE_ERR_ALIAS", -6: "SPARGE_ERR_WORKSPACE",
    -7: "SPARGE_ERR_ARG", -8: "SPARGE_ERR_LAUNCH", -9: "SPARGE_ERR_MASK_VALUE",
}


class SpargeError(RuntimeError):
    """A libsparge call returned a nonzero status."""

    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn}: {_STATUS.get(status, status)} ({message})")
        self.status = status


class SpargeArgumentError(SpargeError, ValueError):
    """libsparge rejected an argument (status -1 .. -7, or -9 for a mask value other
    than 0/1 found by a checking call); nothing was computed."""


def library_path() -> str:
    return _LIB_PATH


def load_library() -> ctypes.CDLL:
    """Load libsparge.so (built in-tree); raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing; build it with "
                           "`python -m block_sparse_attention_sparge_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i64, f32, f64, sz, ci = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_double,
                                 ctypes.c_size_t, ctypes.c_int)
    s3 = ctypes.POINTER(ctypes.c_int64)
    sig = {
        "sparge_status_string": (ctypes.c_char_p, [ci]),
        "sparge_topk_count": (ci, [i64, f64, ctypes.POINTER(ctypes.c_int64)]),
        "sparge_workspace_bytes": (sz, [i64, i64, i64, i64, f64]),
        "sparge_pool_blocks": (ci, [vp, i64, i64, i64, i64, s3, ci, vp, vp]),
        "sparge_predict_mask": (ci, [vp, vp, i64, i64, i64, i64, f64, f32, ci, vp, vp, vp, vp]),
        "sparge_compact_mask": (ci, [vp, i64, i64, i64, vp, vp, vp]),
        "sparge_attn_from_list": (ci, [vp, vp, vp, vp, vp, i64, vp, i64, i64, i64, i64,
                                       s3, s3, s3, s3, f32, ci, vp]),
        "block_sparse_attn": (ci, [vp, vp, vp, vp, vp, i64, i64, i64, i64, s3, s3, s3, s3, f32,
                                   ci, vp, sz, vp]),
        "sparge_attn_topk": (ci, [vp, vp, vp, f64, vp, i64, i64, i64, i64, s3, s3, s3, s3, f32,
                                  ci, vp, vp, sz, vp]),
        "sparge_token_permutation": (ci, [i64, i64, i64, i64, ci, s3, vp]),
        "sparge_predict_mask_cdf": (ci, [vp, vp, i64, i64, i64, i64, f64, f32, ci, vp, vp, vp, vp]),
        "sparge_attn_cdf": (ci, [vp, vp, vp, f64, vp, i64, i64, i64, i64, s3, s3, s3, s3, f32,
                                 ci, vp, vp, sz, vp]),
        "sparge_permute_tokens": (ci, [vp, vp, vp, i64, i64, i64, i64, s3, s3, ci, vp]),
        "sparge_check_mask": (ci, [vp, i64, i64, i64, vp, sz, vp]),
        "sparge_attn_topk_noalloc": (ci, [vp, vp, vp, f64, vp, i64, i64, i64, i64, s3, s3, s3, s3, f32,
                                          ci, vp, vp]),
        "block_sparse_attn_checked": (ci, [vp, vp, vp, vp, vp, i64, i64, i64, i64, s3, s3, s3, s3, f32,
                                           ci, vp, sz, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(fn: str, status: int) -> None:
    if status != 0:
        msg = load_library().sparge_status_string(status).decode()
        cls = SpargeError if status == -8 else SpargeArgumentError
        raise cls(fn, status, msg)


def _strides(t: torch.Tensor):
    return (ctypes.c_int64 * 3)(t.stride(0), t.stride(1), t.stride(2))


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _fits(t: torch.Tensor) -> bool:
    return (t.stride(-1) == 1 and all(s % 8 == 0 and s >= 0 for s in t.stride()[:3])
            and t.data_ptr() % 16 == 0)


def _operand(t: torch.Tensor, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != torch.bfloat16:
        raise NotImplementedError(f"{name}: only bfloat16 is supported (got {t.dtype})")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU device")
    if t.dim() != 4:
        raise ValueError(f"{name} must be (B, H, N, D)")
    if t.shape[-1] not in (64, 128):
        raise ValueError(f"{name}: head dimension must be 64 or 128 (got {t.shape[-1]})")
    # the kernels read 16-byte rows, and K/V tiles as whole non-overlapping rows;
    # other layouts (e.g. a token axis expanded with stride 0) are copied once
    return t if (_fits(t) and t.stride(2) >= t.shape[-1]) else t.contiguous()


def _output(out, like: torch.Tensor, name: str = "out") -> torch.Tensor:
    """A new output shaped like `like`, or a checked caller-supplied one (written in place)."""
    if out is None:
        return torch.empty_like(like)
    if (not isinstance(out, torch.Tensor) or out.dtype != torch.bfloat16 or out.device != like.device
            or tuple(out.shape) != tuple(like.shape)):
        raise ValueError(f"{name} must be a bfloat16 tensor of shape {tuple(like.shape)} on {like.device}")
    if not _fits(out):
        raise ValueError(f"{name} must be unit-stride in its last dimension, with the other strides "
                         "multiples of 8 elements and a 16-byte aligned start")
    return out


def _on_device(t: torch.Tensor, dev: torch.device, name: str) -> None:
    if not isinstance(t, torch.Tensor) or t.device != dev:
        raise ValueError(f"{name} must be a tensor on {dev}")


def _pooled(qbar, kbar):
    for t, name in ((qbar, "qbar"), (kbar, "kbar")):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or not t.is_cuda or t.dim() != 4:
            raise ValueError(f"{name} must be a (B, H, blocks, D) float32 tensor on a GPU device")
    if qbar.device != kbar.device:
        raise ValueError("qbar and kbar must be on the same device")
    return qbar.contiguous(), kbar.contiguous()


def _qkv(q, k, v):
    q, k, v = _operand(q, "q"), _operand(k, "k"), _operand(v, "v")
    if not (q.shape == k.shape == v.shape):
        raise ValueError(f"q, k, v must have the same shape (self-attention); got "
                         f"{tuple(q.shape)}, {tuple(k.shape)}, {tuple(v.shape)}")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on the same device")
    return q, k, v


def _scale(scale, D):
    if scale is None:
        return 0.0
    scale = float(scale)
    if not (scale > 0 and math.isfinite(scale)):
        raise ValueError("scale must be a positive finite number")
    return scale


def mask_shape(B: int, H: int, N: int):
    """(B, H, ceil(N/128), ceil(N/64)), the mask_id shape."""
    return (B, H, -(-N // Q_BLOCK), -(-N // K_BLOCK))


def topk_count(n_kblocks: int, topk: float) -> int:
    """Key blocks kept per query block for `topk` (host-side, no GPU needed)."""
    out = ctypes.c_int64(0)
    _check("sparge_topk_count", load_library().sparge_topk_count(int(n_kblocks), float(topk),
                                                                  ctypes.byref(out)))
    return out.value


def workspace_bytes(B, H, N, D, topk=None) -> int:
    """Workspace bytes for attn_topk (topk given) or block_sparse_attn (topk None)."""
    return int(load_library().sparge_workspace_bytes(int(B), int(H), int(N), int(D),
                                                     -1.0 if topk is None else float(topk)))


def _workspace(t, B, H, N, D, topk, workspace):
    need = workspace_bytes(B, H, N, D, topk)
    if workspace is None:
        return torch.empty(max(need, 16), dtype=torch.uint8, device=t.device)
    _on_device(workspace, t.device, "workspace")
    if workspace.numel() * workspace.element_size() < need or not workspace.is_contiguous():
        raise ValueError(f"workspace must be a contiguous buffer of at least {need} bytes")
    return workspace


def pool_blocks(x: torch.Tensor, block_rows: int) -> torch.Tensor:
    """Block means of x (B, H, N, D) bf16 over `block_rows` (128 or 64) rows -> fp32."""
    x = _operand(x, "x")
    B, H, N, D = x.shape
    out = torch.empty((B, H, -(-N // block_rows), D), dtype=torch.float32, device=x.device)
    _check("sparge_pool_blocks", load_library().sparge_pool_blocks(
        _ptr(x), B, H, N, D, _strides(x), int(block_rows), _ptr(out), _stream(x)))
    return out


def predict_mask(qbar: torch.Tensor, kbar: torch.Tensor, N: int, topk: float, scale=None,
                 return_mask: bool = True, is_causal: bool = False):
    """Top-k block selection from pooled means. Returns (mask_id or None, kv_idx, kv_cnt).

    With is_causal=True, query block i ranks only the key blocks holding a key
    one of its rows may see and keeps the top-k share of those (kv_cnt per row).
    """
    qbar, kbar = _pooled(qbar, kbar)
    B, H, n_qb, D = qbar.shape
    n_kb = kbar.shape[2]
    if (n_qb, n_kb) != mask_shape(B, H, N)[2:] or kbar.shape[:2] != (B, H) or kbar.shape[3] != D:
        raise ValueError("qbar / kbar shapes do not match N")
    kk = topk_count(n_kb, topk)
    dev = qbar.device
    mask = torch.empty((B, H, n_qb, n_kb), dtype=torch.uint8, device=dev) if return_mask else None
    idx = torch.empty((B, H, n_qb, kk), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, H, n_qb), dtype=torch.int32, device=dev)
    _check("sparge_predict_mask", load_library().sparge_predict_mask(
        _ptr(qbar), _ptr(kbar), B, H, N, D, float(topk), _scale(scale, D), int(bool(is_causal)),
        _ptr(mask), _ptr(idx), _ptr(cnt), _stream(qbar)))
    return mask, idx, cnt


def _mask_u8(mask_id, B, H, N, dev):
    if not isinstance(mask_id, torch.Tensor) or not mask_id.is_cuda:
        raise ValueError("mask_id must be a tensor on a GPU device")
    if mask_id.shape != mask_shape(B, H, N):
        raise ValueError(f"mask_id must have shape {mask_shape(B, H, N)}, got {tuple(mask_id.shape)}")
    if mask_id.device != dev:
        raise ValueError("mask_id must be on the same device as q")
    if mask_id.dtype != torch.uint8:
        mask_id = (mask_id != 0).to(torch.uint8)
    return mask_id.contiguous()


def compact_mask(mask_id: torch.Tensor, N: int):
    """Ascending kept-block lists of a mask: (kv_idx (B,H,Qb,Kb) int32, kv_cnt (B,H,Qb) int32)."""
    B, H = mask_id.shape[:2]
    mask_id = _mask_u8(mask_id, B, H, N, mask_id.device)
    idx = torch.empty(mask_id.shape, dtype=torch.int32, device=mask_id.device)
    cnt = torch.empty(mask_id.shape[:3], dtype=torch.int32, device=mask_id.device)
    _check("sparge_compact_mask", load_library().sparge_compact_mask(
        _ptr(mask_id), B, H, N, _ptr(idx), _ptr(cnt), _stream(mask_id)))
    return idx, cnt


def attn_from_list(q, k, v, kv_idx=None, kv_cnt=None, scale=None, out=None, is_causal=False):
    """Attention over precomputed kept-block lists (kv_idx None: dense)."""
    q, k, v = _qkv(q, k, v)
    B, H, N, D = q.shape
    out = _output(out, q)
    ld = 0
    if kv_idx is not None:
        if kv_idx.dtype != torch.int32 or kv_cnt is None or kv_cnt.dtype != torch.int32:
            raise ValueError("kv_idx and kv_cnt must be int32")
        _on_device(kv_idx, q.device, "kv_idx")
        _on_device(kv_cnt, q.device, "kv_cnt")
        kv_idx, kv_cnt = kv_idx.contiguous(), kv_cnt.contiguous()
        if kv_idx.shape[:3] != mask_shape(B, H, N)[:3] or kv_cnt.shape != kv_idx.shape[:3]:
            raise ValueError("kv_idx / kv_cnt shapes do not match q")
        ld = kv_idx.shape[3]
    _check("sparge_attn_from_list", load_library().sparge_attn_from_list(
        _ptr(q), _ptr(k), _ptr(v), _ptr(kv_idx), _ptr(kv_cnt), ld, _ptr(out), B, H, N, D,
        _strides(q), _strides(k), _strides(v), _strides(out), _scale(scale, D), int(bool(is_causal)),
        _stream(q)))
    return out


def block_sparse_attn(q, k, v, mask_id=None, scale=None, out=None, workspace=None, is_causal=False,
                      validate=False):
    """Attention restricted to the 128x64 tiles a 0/1 mask_id selects (None: dense).

    With is_causal=True each query row also ignores the keys after it. With
    validate=True the mask (uint8 or bool) is first checked on the device and a
    value other than 0/1 raises SpargeArgumentError (SPARGE_ERR_MASK_VALUE); that
    check synchronises the stream. Without it any nonzero entry counts as 1.
    """
    q, k, v = _qkv(q, k, v)
    B, H, N, D = q.shape
    out = _output(out, q)
    ws = None
    nbytes = 0
    if mask_id is not None:
        if validate and isinstance(mask_id, torch.Tensor) and mask_id.dtype not in (torch.uint8, torch.bool):
            raise ValueError("validate=True takes a uint8 or bool mask_id")
        mask_id = _mask_u8(mask_id, B, H, N, q.device)
        ws = _workspace(q, B, H, N, D, None, workspace)
        nbytes = ws.numel() * ws.element_size()
    name = "block_sparse_attn_checked" if validate else "block_sparse_attn"
    _check(name, getattr(load_library(), name)(
        _ptr(q), _ptr(k), _ptr(v), _ptr(mask_id), _ptr(out), B, H, N, D, _strides(q), _strides(k),
        _strides(v), _strides(out), _scale(scale, D), int(bool(is_causal)), _ptr(ws), nbytes,
        _stream(q)))
    return out


def check_mask(mask_id: torch.Tensor, N: int, workspace=None) -> None:
    """Raise SpargeArgumentError (SPARGE_ERR_MASK_VALUE) if a uint8 mask_id holds a value
    other than 0 or 1; checked on the device, synchronising the stream."""
    if not isinstance(mask_id, torch.Tensor) or mask_id.dtype != torch.uint8 or not mask_id.is_cuda:
        raise ValueError("mask_id must be a uint8 tensor on a GPU device")
    B, H = mask_id.shape[:2]
    if mask_id.shape != mask_shape(B, H, N):
        raise ValueError(f"mask_id must have shape {mask_shape(B, H, N)}, got {tuple(mask_id.shape)}")
    mask_id = mask_id.contiguous()
    ws = _workspace(mask_id, B, H, N, 64, None, workspace)
    _check("sparge_check_mask", load_library().sparge_check_mask(
        _ptr(mask_id), B, H, N, _ptr(ws), ws.numel() * ws.element_size(), _stream(mask_id)))


def attn_topk(q, k, v, topk=0.5, is_causal=False, scale=None, return_mask=False, out=None,
              workspace=None):
    """Top-k block-sparse attention; a drop-in for scaled dot-product attention.

    is_causal=True restricts each query block's candidates to the key blocks
    its rows may see (keeping the top-k share of those) and masks later keys
    per row. Returns out, or (out, mask_id) with return_mask=True.
    """
    q, k, v = _qkv(q, k, v)
    B, H, N, D = q.shape
    out = _output(out, q)
    mask = torch.empty(mask_shape(B, H, N), dtype=torch.uint8, device=q.device) if return_mask else None
    ws = _workspace(q, B, H, N, D, topk, workspace)
    _check("sparge_attn_topk", load_library().sparge_attn_topk(
        _ptr(q), _ptr(k), _ptr(v), float(topk), _ptr(out), B, H, N, D, _strides(q), _strides(k),
        _strides(v), _strides(out), _scale(scale, D), int(bool(is_causal)), _ptr(mask), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(q)))
    return (out, mask) if return_mask else out


LAYOUTS = {"raster": 0, "cube": 1, "morton": 2}


def token_permutation(n_text: int, grid, layout: str = "cube", cube=(4, 4, 4)) -> torch.Tensor:
    """Host-computed token order for a text prefix plus a (T, H, W) video grid:
    new position p holds old token perm[p]. Returns an int32 CPU tensor."""
    T, Hh, Ww = (int(g) for g in grid)
    if layout not in LAYOUTS:
        raise ValueError(f"layout must be one of {sorted(LAYOUTS)}")
    n = int(n_text) + T * Hh * Ww
    perm = torch.empty(n, dtype=torch.int32)
    c3 = (ctypes.c_int64 * 3)(*[int(c) for c in cube])
    _check("sparge_token_permutation", load_library().sparge_token_permutation(
        int(n_text), T, Hh, Ww, LAYOUTS[layout], c3, perm.data_ptr()))
    return perm


def permute_tokens(x: torch.Tensor, perm: torch.Tensor, inverse: bool = False, out=None) -> torch.Tensor:
    """Reorder the token axis of a (B, H, N, D) bf16 tensor: out[..., p, :] = x[..., perm[p], :]
    (inverse=True: out[..., perm[p], :] = x[..., p, :]). perm: int32 on x's device."""
    x = _operand(x, "x")
    B, H, N, D = x.shape
    if perm.dtype != torch.int32 or perm.device != x.device or perm.numel() != N:
        raise ValueError("perm must be an int32 tensor of N entries on x's device")
    perm = perm.contiguous()
    out = _output(out, x)
    _check("sparge_permute_tokens", load_library().sparge_permute_tokens(
        _ptr(x), _ptr(perm), _ptr(out), B, H, N, D, _strides(x), _strides(out), int(bool(inverse)),
        _stream(x)))
    return out


def predict_mask_cdf(qbar: torch.Tensor, kbar: torch.Tensor, N: int, tau: float, scale=None,
                     return_mask: bool = True, is_causal: bool = False):
    """CDF-threshold block selection from pooled means: per query block, key blocks in
    decreasing probability until their sum reaches tau. Returns (mask_id or None,
    kv_idx (B, H, Qb, Kb), kv_cnt)."""
    qbar, kbar = _pooled(qbar, kbar)
    B, H, n_qb, D = qbar.shape
    n_kb = kbar.shape[2]
    if (n_qb, n_kb) != mask_shape(B, H, N)[2:] or kbar.shape[:2] != (B, H) or kbar.shape[3] != D:
        raise ValueError("qbar / kbar shapes do not match N")
    dev = qbar.device
    mask = torch.empty((B, H, n_qb, n_kb), dtype=torch.uint8, device=dev) if return_mask else None
    idx = torch.empty((B, H, n_qb, n_kb), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, H, n_qb), dtype=torch.int32, device=dev)
    _check("sparge_predict_mask_cdf", load_library().sparge_predict_mask_cdf(
        _ptr(qbar), _ptr(kbar), B, H, N, D, float(tau), _scale(scale, D), int(bool(is_causal)),
        _ptr(mask), _ptr(idx), _ptr(cnt), _stream(qbar)))
    return mask, idx, cnt


def attn_cdf(q, k, v, tau=0.9, is_causal=False, scale=None, return_mask=False, out=None, workspace=None):
    """Block-sparse attention with CDF-threshold selection (see predict_mask_cdf).

    Returns out, or (out, mask_id) with return_mask=True.
    """
    q, k, v = _qkv(q, k, v)
    B, H, N, D = q.shape
    out = _output(out, q)
    mask = torch.empty(mask_shape(B, H, N), dtype=torch.uint8, device=q.device) if return_mask else None
    ws = _workspace(q, B, H, N, D, 1.0, workspace)
    _check("sparge_attn_cdf", load_library().sparge_attn_cdf(
        _ptr(q), _ptr(k), _ptr(v), float(tau), _ptr(out), B, H, N, D, _strides(q), _strides(k),
        _strides(v), _strides(out), _scale(scale, D), int(bool(is_causal)), _ptr(mask), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(q)))
    return (out, mask) if return_mask else out

