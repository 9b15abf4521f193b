"""fd_decode_stages: the split launch and the combine launch of fd_decode as two
calls ("FlashDecoding 数学推导" §2.5: stage 1 writes the partial results, stage
2 reduces them).  Split then combine on one stream must give exactly what
fd_decode gives (the same kernels on the same plan), on every route; and the
result stays within the oracle's tolerances.  Also checks that the binding
refuses caller buffers of the wrong shape, dtype or device."""
import numpy as np
import pytest
import torch

import oracle
from decode_attention_03_amd import fd, workloads

pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-5, 1e-5), "f16": (1.5e-2, 1e-3), "bf16": (1.5e-2, 1e-3)}

CASES = [
    # (name, workload, num_splits): one case per route of the plan
    ("direct", workloads.Workload("st_direct", 8, 32, 32, 128, 2048, "bf16", "bf16", 21), 0),
    ("fused", workloads.Workload("st_fused", 1, 2, 2, 64, 1000, "f32", "f32", 22), 4),
    ("splits_vector", workloads.Workload("st_splits", 1, 16, 16, 128, 20000, "f16", "f16", 23),
     0),
    ("splits_grouped", workloads.Workload("st_grouped", 2, 16, 2, 128, 9000, "bf16", "bf16", 24),
     0),
    ("splits_tiled", workloads.Workload("st_tiled", 2, 64, 1, 64, 5000, "f16", "f16", 25), 0),
    ("balanced", workloads.Workload("st_bal", 6, 32, 4, 128, 7000, "bf16", "bf16", 26,
                                    ragged=(0, 7000)), 0),
    ("balanced_d256", workloads.Workload("st_bal256", 5, 16, 2, 256, 3000, "f16", "f16", 27,
                                         ragged=(1, 3000)), 0),
]


@pytest.mark.parametrize("route,w,B", CASES, ids=[c[0] for c in CASES])
def test_split_then_combine_equals_decode(gpu, route, w, B):
    inp = workloads.generate(w)
    lens = inp["kv_lens"]
    q, k, v = (inp[n].to(gpu) for n in ("q", "k", "v"))
    kl = None if lens is None else lens.to(gpu)
    plan = fd.decode_plan(w.batch, w.heads_q, w.heads_kv, inp["max_kv_len"], w.head_dim,
                          q.dtype, kl is not None, B)
    assert plan["route"] == route.split("_")[0], plan
    o_ref, lse_ref = fd.decode(q, k, v, kl, num_splits=B, scale=w.scale)
    ws_bytes = plan["workspace_bytes"]
    ws = torch.full((max(ws_bytes, 16) // 4,), float("nan"), device=gpu)
    o = torch.full_like(o_ref, float("nan"))
    lse = torch.full_like(lse_ref, float("nan"))
    fd.decode(q, k, v, kl, num_splits=B, scale=w.scale, o=o, lse=lse, workspace=ws,
              stages=fd.STAGE_SPLIT)
    if plan["launches"] == 2:  # the split stage alone leaves o untouched
        torch.cuda.synchronize()
        assert torch.isnan(o.float()).all()
    fd.decode(q, k, v, kl, num_splits=B, scale=w.scale, o=o, lse=lse, workspace=ws,
              stages=fd.STAGE_COMBINE)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16) if o.dtype != torch.float32 else o.view(torch.int32),
                       o_ref.view(torch.int16) if o.dtype != torch.float32
                       else o_ref.view(torch.int32)), route
    assert torch.equal(lse.view(torch.int32), lse_ref.view(torch.int32)), route
    ro, rl = oracle.attention(w.dtype, workloads.raw(inp["q"]), workloads.raw(inp["k"]),
                              workloads.raw(inp["v"]), None if lens is None else lens.numpy(),
                              scale=w.scale)
    go = o.float().cpu().double().numpy().reshape(ro.shape)
    gl = lse.cpu().double().numpy().reshape(rl.shape)
    tol_o, tol_l = TOL[w.dtype]
    fin = np.isfinite(rl)
    assert np.array_equal(np.isneginf(gl), np.isneginf(rl))
    assert np.abs(go - ro).max() <= tol_o
    assert (np.abs(gl[fin] - rl[fin]).max() if fin.any() else 0.0) <= tol_l


def test_caller_buffers_checked(gpu):
    """Outputs of the wrong shape, dtype or device are refused by the binding
    before any pointer reaches the library."""
    w = workloads.Workload("st_chk", 2, 8, 2, 64, 300, "bf16", "bf16", 28)
    inp = workloads.generate(w)
    q, k, v = (inp[n].to(gpu) for n in ("q", "k", "v"))
    for o in (torch.empty(2, 8, 32, dtype=torch.bfloat16, device=gpu),
              torch.empty(2, 8, 64, dtype=torch.float16, device=gpu),
              torch.empty(2, 8, 64, dtype=torch.bfloat16)):
        with pytest.raises(ValueError):
            fd.decode(q, k, v, o=o, out_dtype=torch.bfloat16)
    # an output type the library does not produce for bf16 inputs
    with pytest.raises(fd.FDError, match="out_dtype"):
        fd.decode(q, k, v, o=torch.empty(2, 8, 64, dtype=torch.float16, device=gpu))
    for lse in (torch.empty(2, 4, device=gpu), torch.empty(2, 8, dtype=torch.float64, device=gpu),
                torch.empty(2, 8)):
        with pytest.raises(ValueError):
            fd.decode(q, k, v, lse=lse)
    with pytest.raises(ValueError):
        fd.decode(q, k, v, num_splits=3, workspace=torch.empty(1 << 16, dtype=torch.uint8))
    with pytest.raises(ValueError):
        fd.decode_split(q, k, v, num_splits=3,
                        lse_part=torch.empty(2, 8, 2, device=gpu))
    o_part, lse_part = fd.decode_split(q, k, v, num_splits=3)
    with pytest.raises(ValueError):
        fd.combine(o_part, lse_part, o=torch.empty(2, 8, 64, dtype=torch.float32))
    torch.cuda.synchronize()
