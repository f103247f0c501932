"""The seeded input generator: bf16 rounding and reproducibility."""
import numpy as np
import torch

import synth


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-6, 6, 100000),
                        np.array([1.0, 1.00390625, 1.01171875, -2.5, 0.0, -0.0, 3.0e38], dtype=np.float32)])
    ours = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (ours == ref).all()
    assert synth.f32_to_bf16_bits(np.array([1.00390625], np.float32))[0] == 0x3F80   # tie -> even
    assert synth.f32_to_bf16_bits(np.array([1.01171875], np.float32))[0] == 0x3F82   # tie -> even


def test_widening_is_exact():
    bits = np.arange(0, 65536, 7, dtype=np.uint16)
    f = synth.bf16_bits_to_f32(bits)
    fin = np.isfinite(f)
    assert (synth.f32_to_bf16_bits(f[fin]) == bits[fin]).all()


def test_reproducible_and_head_independent():
    wl = synth.custom(1, 3, 4 * 8 * 8 * 2, 16, grid=(4, 8, 16))
    a = synth.make_tensor(wl, "k", seed=3)
    b = synth.make_tensor(wl, "k", seed=3, heads=[(0, 1)])
    assert (a[0, 1] == b[0, 1]).all() and not b[0, 0].any()
    assert not (a == synth.make_tensor(wl, "k", seed=4)).all()


def test_video_tokens_share_patch_means():
    wl = synth.custom(1, 1, 8 * 16 * 16, 64, grid=(8, 16, 16))
    x = synth.head_f32(wl, "v", 0, 0)
    tok = x.reshape(8, 16, 16, 64)
    same = np.corrcoef(tok[0, 0, 0], tok[3, 7, 7])[0, 1]      # same 4x8x8 patch
    other = np.corrcoef(tok[0, 0, 0], tok[4, 8, 8])[0, 1]     # different patch
    assert same > 0.5 and abs(other) < 0.5


def test_workload_sizes():
    assert [w.N for w in synth.WORKLOADS] == [1024, 32760, 17776, 75600, 119056]
