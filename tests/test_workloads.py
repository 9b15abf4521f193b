"""Seeded input generation: determinism, shapes and the special constructions."""
import dataclasses
import hashlib
import math

import torch

from decode_attention_03_amd import workloads


def _digest(inp):
    h = hashlib.sha256()
    for key in ("q", "k", "v"):
        h.update(workloads.raw(inp[key]).tobytes())
    if inp["kv_lens"] is not None:
        h.update(inp["kv_lens"].numpy().tobytes())
    return h.hexdigest()


def test_same_seed_same_inputs():
    w = dataclasses.replace(workloads.WORKLOADS[2], batch=2, max_kv_len=64)
    assert _digest(workloads.generate(w)) == _digest(workloads.generate(w))
    w2 = dataclasses.replace(w, seed=w.seed + 1)
    assert _digest(workloads.generate(w)) != _digest(workloads.generate(w2))


def test_named_workload_shapes():
    c = workloads.WORKLOADS
    assert (c[1].batch, c[1].heads_q, c[1].head_dim, c[1].max_kv_len, c[1].num_splits) == (1, 1, 64, 1024, 4)
    assert (c[2].batch, c[2].heads_q, c[2].heads_kv, c[2].head_dim, c[2].max_kv_len) == (8, 32, 32, 128, 4096)
    assert (c[3].max_kv_len, c[3].dominant) == (65536, 16)
    assert (c[4].heads_q, c[4].heads_kv, c[4].group, c[4].ragged) == (64, 8, 8, (512, 32768))
    assert (c[5].head_dim, c[5].max_kv_len, c[5].dtype, c[5].std) == (256, 131072, "f16", 0.5)


def test_ragged_lengths_in_range_and_tail_poison():
    w = dataclasses.replace(workloads.WORKLOADS[4], batch=5, ragged=(3, 40))
    inp = workloads.generate(w, poison_tail=True)
    lens = inp["kv_lens"]
    assert lens.dtype == torch.int32 and lens.shape == (5,)
    assert int(lens.min()) >= 3 and int(lens.max()) <= 40
    assert inp["k"].shape[1] == int(lens.max())
    for b in range(5):
        n = int(lens[b])
        assert torch.isfinite(inp["k"][b, :n].float()).all()
        assert torch.isnan(inp["v"][b, n:].float()).all()


def test_dominant_keys_construction():
    w = dataclasses.replace(workloads.WORKLOADS[3], heads_q=2, heads_kv=2, max_kv_len=300)
    inp = workloads.generate(w)
    q = inp["q"].double()
    k = inp["k"].double()
    for h in range(2):
        s = (k[0, :, h] @ q[0, h]) * w.scale
        top = torch.topk(s, w.dominant + 1).values
        expect = w.dominant_factor * q[0, h].norm()
        # the 16 planted keys score ~6|q| (bf16 rounding of the key), the rest do not
        assert torch.allclose(top[: w.dominant], expect.expand(w.dominant), rtol=2e-2)
        assert top[w.dominant] < 0.5 * expect
    assert math.isclose(w.scale, 1 / math.sqrt(128))
