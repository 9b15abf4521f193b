"""The library's launches can be captured in a HIP graph (torch.cuda.CUDAGraph)
and replayed: no entry point allocates, synchronises or issues memsets, and
every launch goes on the caller's stream.

Each case captures one decode step with preallocated outputs and workspace,
then replays it several times with eager work and synchronisation between
the replays; every replay must reproduce the eager result bit for bit (the
kernels are deterministic), and the eager result matches the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from decode_attention_03_amd import fd, workloads

pytestmark = pytest.mark.gpu


def _capture_and_replay(gpu, step, outs, replays=4):
    """Run `step` eagerly, capture it, replay it `replays` times; return the
    eager outputs and check every replay against them."""
    s = torch.cuda.Stream(device=gpu)
    s.wait_stream(torch.cuda.current_stream(gpu))
    with torch.cuda.stream(s):
        step()  # warm-up outside the capture (first-use setup happens here)
    s.synchronize()
    eager = [t.clone() for t in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    for r in range(replays):
        for t in outs:
            t.fill_(float("nan"))  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, e in zip(outs, eager):
            assert torch.equal(t, e), f"replay {r} differs from the eager run"
    return eager


def _decode_case(gpu, w, inp, num_splits=0):
    q, k, v = inp["q"].to(gpu), inp["k"].to(gpu), inp["v"].to(gpu)
    kl = None if inp["kv_lens"] is None else inp["kv_lens"].to(gpu)
    batch, hq, d = q.shape
    o = torch.empty((batch, hq, d), dtype=q.dtype, device=gpu)
    lse = torch.empty((batch, hq), dtype=torch.float32, device=gpu)
    need = fd.decode_workspace_bytes(batch, hq, w.heads_kv, k.shape[1], d, q.dtype,
                                     kl is not None, num_splits)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=gpu)

    def step():
        fd.decode(q, k, v, kl, scale=w.scale, num_splits=num_splits, workspace=ws, o=o, lse=lse)

    return step, [o, lse]


@pytest.mark.parametrize("case", ["fused_small_f32", "mha_one_split", "mha_splits_combine",
                                  "gqa_ragged_balanced", "mqa_ragged_four_waves",
                                  "mqa_two_wave_tiles", "mha_ragged_balanced_vector"])
def test_decode_graph_replay(gpu, case):
    if case == "fused_small_f32":
        w = workloads.WORKLOADS[1]
        inp = workloads.generate(w)
        B = w.num_splits
    elif case == "mha_one_split":
        w, inp = workloads.custom(8, 32, 32, 128, 2048, dtype="bf16", seed=41)
        B = 0
    elif case == "mha_splits_combine":
        w, inp = workloads.custom(1, 32, 32, 128, 20000, dtype="bf16", seed=42)
        B = 0
    elif case == "gqa_ragged_balanced":
        w, inp = workloads.custom(6, 32, 4, 128, 9000, dtype="bf16", seed=43,
                                  lens=[9000, 17, 0, 4096, 8191, 300])
        B = 0
    elif case == "mqa_ragged_four_waves":  # balanced plan, four waves per work-group
        w, inp = workloads.custom(4, 64, 1, 128, 5000, dtype="bf16", seed=45,
                                  lens=[5000, 0, 1234, 4097])
        B = 0
    elif case == "mha_ragged_balanced_vector":  # balanced plan on the vector kernel
        w, inp = workloads.custom(5, 16, 16, 128, 7000, dtype="bf16", seed=47,
                                  lens=[7000, 0, 33, 4096, 6999])
        B = 0
    else:  # tiled kernel, two waves of one tile each, fixed splits
        w, inp = workloads.custom(3, 32, 1, 128, 3000, dtype="f16", seed=46)
        B = 0
    step, outs = _decode_case(gpu, w, inp, B)
    o, lse = _capture_and_replay(gpu, step, outs)
    lens = inp["kv_lens"]
    ro, rl = oracle.attention(w.dtype, workloads.raw(inp["q"]), workloads.raw(inp["k"]),
                              workloads.raw(inp["v"]), None if lens is None else lens.numpy(),
                              scale=w.scale)
    tol_o, tol_l = (1e-5, 1e-5) if w.dtype == "f32" else (1.5e-2, 1e-3)
    go = o.float().cpu().double().numpy().reshape(ro.shape)
    gl = lse.cpu().double().numpy().reshape(rl.shape)
    fin = np.isfinite(rl)
    assert np.array_equal(np.isneginf(gl), np.isneginf(rl))
    assert np.abs(go - ro).max() <= tol_o
    assert np.abs(gl[fin] - rl[fin]).max() <= tol_l


def test_cascade_graph_replay(gpu):
    w = workloads.Workload("cascade_graph", batch=5, heads_q=16, heads_kv=2, head_dim=128,
                           max_kv_len=2000, dtype="bf16", out_dtype="bf16", seed=44,
                           ragged=(0, 2000))
    c = workloads.cascade(w, 3000)
    dev = {k: (t.to(gpu) if torch.is_tensor(t) else t) for k, t in c.items()}
    o = torch.empty((5, 16, 128), dtype=torch.bfloat16, device=gpu)
    lse = torch.empty((5, 16), dtype=torch.float32, device=gpu)
    need = fd.cascade_workspace_bytes(5, 16, 2, 3000, c["max_suffix_len"], 128, torch.bfloat16,
                                      True)
    ws = torch.empty(need, dtype=torch.uint8, device=gpu)

    def step():
        fd.decode_cascade(dev["q"], dev["k_prefix"], dev["v_prefix"], dev["k_suffix"],
                          dev["v_suffix"], dev["suffix_lens"], scale=w.scale, workspace=ws, o=o,
                          lse=lse)

    eo, el = _capture_and_replay(gpu, step, [o, lse])
    cc = workloads.cascade_concat(c)
    ro, rl = oracle.attention("bf16", workloads.raw(cc["q"]), workloads.raw(cc["k"]),
                              workloads.raw(cc["v"]), cc["kv_lens"].numpy(), scale=w.scale)
    assert np.abs(eo.float().cpu().double().numpy().reshape(ro.shape) - ro).max() <= 1.5e-2
    fin = np.isfinite(rl)
    assert np.abs(el.cpu().double().numpy().reshape(rl.shape)[fin] - rl[fin]).max() <= 1e-3
