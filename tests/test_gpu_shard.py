"""Sequence sharding emulated on one GPU.

Each shard of the KV sequence axis is decoded on its own, as the GPU holding
that shard would do it: fd_decode over the shard's tokens, with fp32 o and the
LSE as output.  The per-shard (o, LSE) pairs are then laid side by side as
partials and merged with fd_combine, as the owner of the rows would do after
the exchange.  The LSE merge is associative and the result is
partition-independent ("FlashDecoding 数学推导：传统 m/l/o 方法与 LSE 方法",
§2.3.5), so the merged result must match the oracle over the whole sequence
to the usual bounds.  Ragged lengths leave the later shards of short
sequences empty ((0, -inf) pairs the merge must ignore).
"""
import numpy as np
import pytest
import torch

import oracle
from decode_attention_03_amd import fd, workloads

pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-5, 1e-5), "f16": (1.5e-2, 1e-3), "bf16": (1.5e-2, 1e-3)}


@pytest.mark.parametrize("dtype,group,d,shards", [("bf16", 1, 128, 8), ("bf16", 8, 128, 4),
                                                  ("f32", 1, 64, 3), ("f16", 4, 256, 2)])
def test_sequence_shards_merge_to_whole(gpu, dtype, group, d, shards):
    lens = [4096, 1, 0, 2500, 4095]
    n_max = 4096
    w, inp = workloads.custom(len(lens), 2 * group, 2, d, n_max, dtype=dtype,
                              seed=50 + shards + group, lens=lens)
    q, k, v = inp["q"].to(gpu), inp["k"].to(gpu), inp["v"].to(gpu)
    batch, hq = q.shape[0], q.shape[1]
    per = -(-n_max // shards)
    o_part = torch.empty((batch, hq, shards, d), dtype=torch.float32, device=gpu)
    lse_part = torch.empty((batch, hq, shards), dtype=torch.float32, device=gpu)
    lens_t = inp["kv_lens"]
    for s in range(shards):
        lo, hi = s * per, min((s + 1) * per, n_max)
        ks, vs = k[:, lo:hi].contiguous(), v[:, lo:hi].contiguous()
        sl = (lens_t - lo).clamp(0, hi - lo).to(torch.int32).to(gpu)
        o_s, lse_s = fd.decode(q, ks, vs, sl, scale=w.scale, out_dtype=torch.float32)
        o_part[:, :, s] = o_s
        lse_part[:, :, s] = lse_s
    o, lse = fd.combine(o_part, lse_part, out_dtype=q.dtype)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(dtype, workloads.raw(inp["q"]), workloads.raw(inp["k"]),
                              workloads.raw(inp["v"]), np.array(lens, dtype=np.int32),
                              scale=w.scale)
    tol_o, tol_l = TOL[dtype]
    go = o.float().cpu().double().numpy().reshape(ro.shape)
    gl = lse.cpu().double().numpy().reshape(rl.shape)
    assert np.isfinite(go).all()
    assert np.array_equal(np.isneginf(gl), np.isneginf(rl))
    fin = np.isfinite(rl)
    err_o = np.abs(go - ro).max()
    err_l = np.abs(gl[fin] - rl[fin]).max()
    print(f"shards {shards} {dtype} G{group} d{d}: max|o-ref|={err_o:.3e} "
          f"max|lse-ref|={err_l:.3e}", flush=True)
    assert err_o <= tol_o and err_l <= tol_l
