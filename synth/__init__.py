"""Seeded synthetic Q/K/V generators for the block-sparse attention workloads.

This module only makes input data. It holds none of the method's arithmetic
(no pooling, scoring, selection or attention), so both the CPU oracle harness
and the GPU path's tests and benchmark can draw the exact same bf16 bytes from
it without sharing any computation.

Workloads are synthetic stand-ins for the video-diffusion self-attention that
the SpargeAttention documentation targets (Wan2.1, CogVideoX, HunyuanVideo;
SpargeAttention Documentation page, model list). Token grids follow the
latent sizes of those models at the resolutions the AB-Attention README's
settings table gives (1280x720, 81 / 129 frames): text tokens first, then video
tokens in raster order (t, h, w) with w fastest.

Recipe per (config, tensor, batch, head): a numpy PCG64 stream seeded with
SeedSequence([seed, config_id, tensor_id, b, h]) (tensor ids Q=0, K=1, V=2).
Draw order on that stream: text tokens (n_text x D, i.i.d. N(0,1)), then one
mean vector per 8(h) x 8(w) x 4(t) spatiotemporal patch (N(0,1) per
component), then per-video-token noise (N(0,1), multiplied by 0.5). A video
token is its patch mean plus its noise. Values are drawn in float32, Q is then
multiplied by ``q_scale`` (text and video alike), and everything is rounded to
bf16 with round-to-nearest-even. i.i.d. configs draw N x D standard normals.
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np

TENSOR_IDS = {"q": 0, "k": 1, "v": 2}


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic attention workload (shape plus value recipe)."""

    config_id: int
    name: str
    B: int
    H: int
    D: int
    n_text: int = 0
    grid: tuple | None = None       # (T, Hh, W) latent video grid, or None for i.i.d. tokens
    n_iid: int = 0                  # token count for i.i.d. workloads
    q_scale: float = 1.0
    topks: tuple = (0.5,)
    patch: tuple = (4, 8, 8)        # (t, h, w) extent of one correlated patch
    noise_std: float = 0.5

    @property
    def N(self) -> int:
        if self.grid is None:
            return self.n_iid
        T, Hh, W = self.grid
        return self.n_text + T * Hh * W

    def describe(self) -> str:
        if self.grid is None:
            return f"{self.name}: B={self.B} H={self.H} N={self.N} D={self.D} iid N(0,1)"
        T, Hh, W = self.grid
        return (f"{self.name}: B={self.B} H={self.H} N={self.N} D={self.D} "
                f"({self.n_text} text + {T}x{Hh}x{W} video) q_scale={self.q_scale:.6g}")


# The five workloads: tiny i.i.d., then Wan2.1-1.3B, CogVideoX-2B, Wan2.1-14B 720p
# and HunyuanVideo 720p shaped self-attention.
WORKLOADS = (
    Workload(0, "tiny-iid", B=1, H=2, D=64, n_iid=1024, q_scale=1.0, topks=(0.5,)),
    Workload(1, "wan1.3b-480p", B=1, H=12, D=128, grid=(21, 30, 52),
             q_scale=1.0 / math.sqrt(128), topks=(0.5,)),
    Workload(2, "cogvideox-2b", B=2, H=30, D=64, n_text=226, grid=(13, 30, 45),
             q_scale=1.0 / math.sqrt(64), topks=(0.4,)),
    Workload(3, "wan14b-720p", B=1, H=40, D=128, grid=(21, 45, 80),
             q_scale=1.0 / math.sqrt(128), topks=(0.1, 0.2, 0.3, 0.5, 1.0)),
    Workload(4, "hunyuan-720p", B=1, H=24, D=128, n_text=256, grid=(33, 45, 80),
             q_scale=1.0 / math.sqrt(128), topks=(0.1,)),
)


def custom(B, H, N, D, *, config_id=100, grid=None, n_text=0, q_scale=1.0, name="custom"):
    """A workload of arbitrary shape (i.i.d. when ``grid`` is None)."""
    if grid is None:
        return Workload(config_id, name, B=B, H=H, D=D, n_iid=N, q_scale=q_scale)
    wl = Workload(config_id, name, B=B, H=H, D=D, n_text=n_text, grid=tuple(grid), q_scale=q_scale)
    if wl.N != N:
        raise ValueError(f"grid {grid} with {n_text} text tokens gives N={wl.N}, not {N}")
    return wl


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round to nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    nan = np.isnan(x)
    if nan.any():
        r = np.where(nan, np.uint32(0x7FC0), r)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float64 (exact)."""
    return bf16_bits_to_f32(bits).astype(np.float64)


def _rng(seed, wl, tensor, b, h):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(
        [int(seed), int(wl.config_id), TENSOR_IDS[tensor], int(b), int(h)])))


def head_f32(wl: Workload, tensor: str, b: int, h: int, seed: int = 0) -> np.ndarray:
    """The float32 values (before bf16 rounding) of one (N, D) head."""
    g = _rng(seed, wl, tensor, b, h)
    D = wl.D
    if wl.grid is None:
        x = g.standard_normal((wl.N, D), dtype=np.float32)
    else:
        T, Hh, W = wl.grid
        pt, ph, pw = wl.patch
        x = np.empty((wl.N, D), dtype=np.float32)
        if wl.n_text:
            x[: wl.n_text] = g.standard_normal((wl.n_text, D), dtype=np.float32)
        nT, nH, nW = -(-T // pt), -(-Hh // ph), -(-W // pw)
        means = g.standard_normal((nT, nH, nW, D), dtype=np.float32)
        noise = g.standard_normal((T * Hh * W, D), dtype=np.float32)
        noise *= np.float32(wl.noise_std)
        ti = np.arange(T) // pt
        hi = np.arange(Hh) // ph
        wi = np.arange(W) // pw
        pidx = ((ti[:, None, None] * nH + hi[None, :, None]) * nW + wi[None, None, :]).reshape(-1)
        noise += means.reshape(-1, D)[pidx]
        x[wl.n_text:] = noise
    if tensor == "q" and wl.q_scale != 1.0:
        x *= np.float32(wl.q_scale)
    return x


def head_bf16(wl: Workload, tensor: str, b: int, h: int, seed: int = 0) -> np.ndarray:
    """One (N, D) head as bf16 bit patterns (uint16)."""
    return f32_to_bf16_bits(head_f32(wl, tensor, b, h, seed))


def make_tensor(wl: Workload, tensor: str, seed: int = 0, heads=None, threads: int = 8) -> np.ndarray:
    """A (B, H, N, D) uint16 bf16 tensor; ``heads`` restricts to a list of (b, h) (others stay 0)."""
    out = np.zeros((wl.B, wl.H, wl.N, wl.D), dtype=np.uint16)
    todo = [(b, h) for b in range(wl.B) for h in range(wl.H)] if heads is None else list(heads)

    def work(bh):
        b, h = bh
        out[b, h] = head_bf16(wl, tensor, b, h, seed)

    if threads > 1 and len(todo) > 1:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(work, todo))
    else:
        for bh in todo:
            work(bh)
    return out


def make_qkv(wl: Workload, seed: int = 0, heads=None, threads: int = 8):
    """(q, k, v) as (B, H, N, D) uint16 bf16 tensors."""
    return tuple(make_tensor(wl, t, seed, heads, threads) for t in ("q", "k", "v"))
