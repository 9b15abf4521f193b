"""GPU parity of the cascade (shared-prefix) decode through the C ABI.

Each sequence attends over one shared prefix cache followed by its own
suffix cache; the expected result is the oracle's attention over that
concatenation (workloads.cascade_concat lays it out; data movement only).
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from decode_attention_03_amd import fd, workloads

pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-5, 1e-5), "f16": (1.5e-2, 1e-3), "bf16": (1.5e-2, 1e-3)}


def _run(gpu, c, w, **kw):
    dev = lambda t: None if t is None else t.to(gpu)  # noqa: E731
    return fd.decode_cascade(dev(c["q"]), dev(c["k_prefix"]), dev(c["v_prefix"]),
                             dev(c["k_suffix"]), dev(c["v_suffix"]), dev(c["suffix_lens"]),
                             scale=w.scale, **kw)


def _reference(c, w):
    cc = workloads.cascade_concat(c)
    return oracle.attention(w.dtype, workloads.raw(cc["q"]), workloads.raw(cc["k"]),
                            workloads.raw(cc["v"]), cc["kv_lens"].numpy(), scale=w.scale)


def _check(name, o, lse, ro, rl, dtype):
    tol_o, tol_l = TOL[dtype]
    go = o.float().cpu().double().numpy().reshape(ro.shape)
    gl = lse.cpu().double().numpy().reshape(rl.shape)
    assert np.isfinite(go).all(), f"{name}: non-finite output"
    assert np.array_equal(np.isneginf(gl), np.isneginf(rl))
    fin = np.isfinite(rl)
    err_o = np.abs(go - ro).max()
    err_l = np.abs(gl[fin] - rl[fin]).max() if fin.any() else 0.0
    print(f"{name}: max|o-ref|={err_o:.3e} max|lse-ref|={err_l:.3e}", flush=True)
    assert err_o <= tol_o and err_l <= tol_l


@pytest.mark.parametrize("dtype,group,d", [("bf16", 8, 128), ("bf16", 1, 128), ("f32", 1, 64),
                                           ("f32", 4, 128), ("f16", 1, 256),
                                           ("f16", 4, 256), ("f16", 2, 64), ("bf16", 32, 128),
                                           ("bf16", 64, 128), ("f16", 40, 256)])
@pytest.mark.parametrize("prefix_len", [0, 1, 777, 5000])
def test_cascade_matches_concatenated_attention(gpu, dtype, group, d, prefix_len):
    w = workloads.Workload("cascade_test", batch=5, heads_q=2 * group, heads_kv=2, head_dim=d,
                           max_kv_len=3000, dtype=dtype, out_dtype=dtype,
                           seed=prefix_len + 10 * group + d, ragged=(0, 3000))
    c = workloads.cascade(w, prefix_len, poison_tail=True)
    o, lse = _run(gpu, c, w)
    torch.cuda.synchronize()
    ro, rl = _reference(c, w)
    _check(f"cascade_{dtype}_G{group}_d{d}_P{prefix_len}", o, lse, ro, rl, dtype)


@pytest.mark.parametrize("dtype,group,d,batch", [("f16", 4, 64, 40), ("bf16", 8, 128, 33),
                                                 ("bf16", 1, 256, 19), ("bf16", 8, 128, 16),
                                                 ("bf16", 8, 128, 12), ("f16", 4, 64, 20)])
def test_cascade_many_requests(gpu, dtype, group, d, batch):
    """Many requests per shared prefix: the prefix kernel's queries span many
    16-query tiles (partial last tile), several tiles per work-group; with
    five to eight tiles (128, 96 and 80 queries) the prefix runs on two
    four-wave work-groups per KV head and split, the second one partly empty
    for 96 and 80."""
    w = workloads.Workload("cascade_many", batch=batch, heads_q=2 * group, heads_kv=2,
                           head_dim=d, max_kv_len=700, dtype=dtype, out_dtype=dtype,
                           seed=batch + d, ragged=(0, 700))
    c = workloads.cascade(w, 3000, poison_tail=True)
    o, lse = _run(gpu, c, w)
    torch.cuda.synchronize()
    ro, rl = _reference(c, w)
    _check(f"cascade_many_{dtype}_G{group}_d{d}_b{batch}", o, lse, ro, rl, dtype)


def test_cascade_edge_cases(gpu):
    """Empty suffixes, no suffix lengths given, and an empty prefix with empty
    suffixes (o = 0, lse = -inf)."""
    w = workloads.Workload("cascade_edges", batch=4, heads_q=8, heads_kv=1, head_dim=128,
                           max_kv_len=300, dtype="bf16", out_dtype="bf16", seed=5)
    c = workloads.cascade(w, 400)
    c["suffix_lens"] = torch.tensor([0, 300, 0, 17], dtype=torch.int32)
    o, lse = _run(gpu, c, w)
    ro, rl = _reference(c, w)
    _check("cascade_empty_suffixes", o, lse, ro, rl, "bf16")
    c["suffix_lens"] = None  # every suffix full
    o, lse = _run(gpu, c, w)
    ro, rl = _reference(c, w)
    _check("cascade_full_suffixes", o, lse, ro, rl, "bf16")
    c0 = workloads.cascade(w, 0)
    c0["suffix_lens"] = torch.zeros(4, dtype=torch.int32)
    o, lse = _run(gpu, c0, w)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


def test_cascade_equals_plain_decode_on_concatenation(gpu):
    """The cascade and fd_decode over the materialised prefix + suffix caches
    agree to the bf16 bounds (named ragged grouped workload, 2048-token prefix)."""
    w = dataclasses.replace(workloads.WORKLOADS[4], batch=6, ragged=(16, 8192))
    c = workloads.cascade(w, 2048)
    o1, l1 = _run(gpu, c, w)
    cc = workloads.cascade_concat(c)
    o2, l2 = fd.decode(cc["q"].to(gpu), cc["k"].to(gpu), cc["v"].to(gpu),
                       cc["kv_lens"].to(gpu), scale=w.scale)
    torch.cuda.synchronize()
    assert (o1.float() - o2.float()).abs().max().item() <= 1.6e-2
    assert (l1 - l2).abs().max().item() <= 1e-3


def test_cascade_workspace_too_small(gpu):
    w = workloads.Workload("cascade_ws", batch=2, heads_q=4, heads_kv=2, head_dim=64,
                           max_kv_len=100, dtype="f32", out_dtype="f32", seed=1)
    c = workloads.cascade(w, 100)
    need = fd.cascade_workspace_bytes(2, 4, 2, 100, c["max_suffix_len"], 64, torch.float32, False)
    ws = torch.empty(need - 256, dtype=torch.uint8, device=gpu)
    with pytest.raises(fd.FDError) as e:
        _run(gpu, c, w, workspace=ws)
    assert e.value.code == fd.ERR_WORKSPACE
