"""The oracle's exact element decoders against numpy / torch upcasts, over
every 16-bit pattern (bfloat16 and IEEE binary16) and a sweep of fp32 values."""
import numpy as np
import torch

import oracle


def _all_patterns():
    return np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


def _same(a, b):
    both_nan = np.isnan(a) & np.isnan(b)
    return np.all(both_nan | (a == b)) and np.array_equal(np.signbit(a) & ~both_nan,
                                                          np.signbit(b) & ~both_nan)


def test_bf16_all_patterns():
    bits = _all_patterns()
    ours = oracle.decode("bf16", bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert _same(ours, ref)


def test_f16_all_patterns():
    bits = _all_patterns()
    ours = oracle.decode("f16", bits)
    ref = bits.view(np.float16).astype(np.float64)
    assert _same(ours, ref)


def test_f32_values():
    rng = np.random.default_rng(0)
    vals = np.concatenate([rng.standard_normal(1000) * 10.0 ** rng.integers(-40, 38, 1000),
                           [0.0, -0.0, np.inf, -np.inf, 1e-45, -1e-45, 3.4e38]]).astype(np.float32)
    assert _same(oracle.decode("f32", vals), vals.astype(np.float64))
