"""GPU parity over seeded random shapes, through the C ABI, against the oracle.

Each case draws (from one fixed seed) a batch size, head counts and group
size (1 to 128 query heads per KV head, so every work-group shape from one
to eight waves appears), head size, input type, ragged
lengths (some empty), a split plan (automatic, one split, or an explicit
count and length) and the entry point: contiguous decode, paged decode, or
the split stage in either partial format followed by its combine.  The
combinations the targeted tests do not pair up (a paged large group with
explicit splits in fp16 at d = 256, say) are covered here at the usual
bounds.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from decode_attention_03_amd import fd, workloads

pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-5, 1e-5), "f16": (1.5e-2, 1e-3), "bf16": (1.5e-2, 1e-3)}
N_CASES = 120


def _draw(i):
    g = np.random.default_rng(1000 + i)
    group = int(g.choice([1, 1, 2, 4, 8, 16, 17, 32, 40, 80, 128]))
    hkv = int(g.integers(1, 4))
    d = int(g.choice([64, 128, 256]))
    dtype = str(g.choice(["f32", "bf16", "f16"]))
    batch = int(g.integers(1, 7))
    n_max = int(g.integers(1, 2500))
    lens = g.integers(0, n_max + 1, size=batch)
    lens[g.integers(0, batch)] = n_max
    route = str(g.choice(["decode", "paged", "split_lse", "split_mlo"]))
    plan = str(g.choice(["auto", "one", "explicit"]))
    splits = int(g.integers(2, 10))
    return dict(group=group, hkv=hkv, d=d, dtype=dtype, batch=batch, n_max=n_max,
                lens=[int(x) for x in lens], route=route, plan=plan, splits=splits,
                seed=2000 + i)


def _case_id(i):
    c = _draw(i)
    return (f"{i}-{c['route']}-{c['plan']}-{c['dtype']}-G{c['group']}x{c['hkv']}-d{c['d']}"
            f"-b{c['batch']}-n{c['n_max']}")


@pytest.mark.parametrize("i", range(N_CASES), ids=[_case_id(i) for i in range(N_CASES)])
def test_random_shape(gpu, i):
    c = _draw(i)
    w, inp = workloads.custom(c["batch"], c["group"] * c["hkv"], c["hkv"], c["d"], c["n_max"],
                              dtype=c["dtype"], seed=c["seed"], lens=c["lens"])
    q, k, v = inp["q"].to(gpu), inp["k"].to(gpu), inp["v"].to(gpu)
    kl = inp["kv_lens"].to(gpu)
    route, plan = c["route"], c["plan"]
    n_cache = c["n_max"]
    if route == "paged":
        ps = 16 << (i % 4)
        pg = workloads.paginate(inp, ps, seed=i)
        n_cache = pg["max_pages"] * ps  # the paged call's max_kv_len
    if route in ("split_lse", "split_mlo") or plan == "explicit":
        B = c["splits"]
        L = -(-n_cache // B)
        if route == "paged":
            L = -(-L // 16) * 16
    elif plan == "one":
        B, L = 1, 0
    else:
        B, L = 0, 0
    if route == "decode":
        o, lse = fd.decode(q, k, v, kl, scale=w.scale, num_splits=B, split_len=L)
    elif route == "paged":
        o, lse = fd.decode_paged(q, pg["k_pages"].to(gpu), pg["v_pages"].to(gpu),
                                 pg["block_table"].to(gpu), kl, scale=w.scale, num_splits=B,
                                 split_len=L if B else 0)
    elif route == "split_lse":
        o_part, lse_part = fd.decode_split(q, k, v, kl, num_splits=B, split_len=L, scale=w.scale)
        o, lse = fd.combine(o_part, lse_part, out_dtype=q.dtype)
    else:
        o_part, m_part, l_part = fd.decode_split_mlo(q, k, v, kl, num_splits=B, split_len=L,
                                                     scale=w.scale)
        o, lse = fd.combine_mlo(o_part, m_part, l_part, out_dtype=q.dtype)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(c["dtype"], workloads.raw(inp["q"]), workloads.raw(inp["k"]),
                              workloads.raw(inp["v"]), np.array(c["lens"], dtype=np.int32),
                              scale=w.scale)
    tol_o, tol_l = TOL[c["dtype"]]
    go = o.float().cpu().double().numpy().reshape(ro.shape)
    gl = lse.cpu().double().numpy().reshape(rl.shape)
    assert np.isfinite(go).all()
    assert np.array_equal(np.isneginf(gl), np.isneginf(rl))
    fin = np.isfinite(rl)
    err_o = float(np.abs(go - ro).max())
    err_l = float(np.abs(gl[fin] - rl[fin]).max()) if fin.any() else 0.0
    print(f"{_case_id(i)}: B={B} L={L} max|o-ref|={err_o:.3e} max|lse-ref|={err_l:.3e}",
          flush=True)
    assert err_o <= tol_o and err_l <= tol_l
    assert math.isfinite(err_o)
