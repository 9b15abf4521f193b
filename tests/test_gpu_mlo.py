"""GPU parity of the m/l/o partial format ("FlashDecoding 数学推导" §2.4.1
direct form and §2.4.2 merge) against the fp64 oracle, through the C ABI.

The split stage's (o, m, l) per split is compared with the oracle's triple
(o to the output tolerance, m to the LSE tolerance, l relatively to the LSE
tolerance, since log l is what enters the LSE), the m/l/o combine with the
oracle's m/l/o merge, and the whole m/l/o route with the oracle's attention.
"""
import numpy as np
import pytest
import torch

import oracle
from decode_attention_03_amd import fd, workloads
from tests.test_gpu_parity import combine_bounds

pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-5, 1e-5), "f16": (1.5e-2, 1e-3), "bf16": (1.5e-2, 1e-3)}


def _np(t):
    return t.float().cpu().double().numpy()


@pytest.mark.parametrize("dtype,group,d", [("f32", 1, 64), ("bf16", 1, 128), ("bf16", 8, 128),
                                           ("f16", 2, 256), ("f16", 4, 64), ("f32", 4, 128)])
def test_split_mlo_partials(gpu, dtype, group, d):
    lens = [1000, 0, 257, 64, 999]
    w, inp = workloads.custom(5, 2 * group, 2, d, 1000, dtype=dtype, seed=11 + group, lens=lens)
    q, k, v = inp["q"].to(gpu), inp["k"].to(gpu), inp["v"].to(gpu)
    kl = inp["kv_lens"].to(gpu)
    B, L = 5, 200
    shape = (5, 2 * group, B)
    o_part = torch.full((*shape, d), float("nan"), device=gpu)
    m_part = torch.full(shape, float("nan"), device=gpu)
    l_part = torch.full(shape, float("nan"), device=gpu)
    fd.decode_split_mlo(q, k, v, kl, num_splits=B, split_len=L, scale=w.scale, o_part=o_part,
                        m_part=m_part, l_part=l_part)
    _, lse_part = fd.decode_split(q, k, v, kl, num_splits=B, split_len=L, scale=w.scale)
    rop, rlp, rmp, rll = oracle.split_partials(dtype, workloads.raw(inp["q"]),
                                               workloads.raw(inp["k"]), workloads.raw(inp["v"]),
                                               np.array(lens, dtype=np.int32), B, L,
                                               scale=w.scale, with_mlo=True)
    tol_o, tol_l = TOL[dtype]
    go, gm, gl = _np(o_part), _np(m_part), _np(l_part)
    assert np.isfinite(go).all() and not np.isnan(gm).any() and np.isfinite(gl).all()
    empty = np.isneginf(rmp)
    assert np.array_equal(np.isneginf(gm), empty)
    assert np.all(gl[empty] == 0) and np.all(go[empty] == 0)
    err_o = np.abs(go - rop).max()
    err_m = np.abs(gm[~empty] - rmp[~empty]).max()
    err_l = (np.abs(gl[~empty] - rll[~empty]) / rll[~empty]).max()
    print(f"mlo {dtype} G{group} d{d}: o {err_o:.2e} m {err_m:.2e} l(rel) {err_l:.2e}", flush=True)
    assert err_o <= tol_o and err_m <= tol_l and err_l <= tol_l
    assert np.all(gl[~empty] >= 1.0 - 1e-6)  # the max token contributes exp(0) = 1
    # m + log l is the LSE the LSE format writes for the same split
    s = gm[~empty] + np.log(gl[~empty])
    assert np.abs(s - _np(lse_part)[~empty]).max() <= 1e-5 * max(1.0, np.abs(s).max())


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_combine_mlo_synthetic(gpu, out, d):
    """m/l/o merge alone on triples with empty splits, an all-empty row, a single
    finite split and spreads over 200 in m; o values ~ N(0, 0.5^2), held to
    the absolute bounds of the LSE combine's test (combine_bounds there)."""
    rng = np.random.default_rng(100 + d)
    batch, hq, B = 3, 5, 29
    op = 0.5 * rng.standard_normal((batch, hq, B, d))
    mp = rng.uniform(-40, 40, (batch, hq, B))
    lp = rng.uniform(1.0, 500.0, (batch, hq, B))
    mp[0, 0, :] = -np.inf
    mp[0, 1, :] = -np.inf
    mp[0, 1, 7] = 2.0
    mp[1, 2, 1::2] = -np.inf
    mp[2, 3, 0], mp[2, 3, 1] = 120.0, -100.0
    empty = np.isneginf(mp)
    lp[empty] = 0.0
    op[empty] = 0.0
    f32 = lambda a: torch.tensor(a, dtype=torch.float32)  # noqa: E731
    o_part, m_part, l_part = f32(op), f32(mp), f32(lp)
    ro, rm, rl = oracle.combine_mlo(o_part.double().numpy(), m_part.double().numpy(),
                                    l_part.double().numpy())
    rlse = np.where(np.isneginf(rm), -np.inf, rm + np.log(np.where(rl > 0, rl, 1.0)))
    o, lse = fd.combine_mlo(o_part.to(gpu), m_part.to(gpu), l_part.to(gpu),
                            out_dtype=workloads.TORCH_DTYPES[out])
    go, gl = _np(o), _np(lse)
    assert np.abs(op).max() < 4.0
    assert np.array_equal(np.isneginf(gl), np.isneginf(rlse))
    fin = np.isfinite(rlse)
    tol_o, tol_l = combine_bounds(out, rlse[fin])
    assert np.abs(go - ro).max() <= tol_o
    assert np.all(np.abs(gl[fin] - rlse[fin]) <= tol_l)
    assert np.all(go[0, 0] == 0)


@pytest.mark.parametrize("cfg,B", [(2, 4), (3, 16), (4, 8), (1, 4)])
def test_mlo_route_named_workloads(gpu, cfg, B):
    """split (m/l/o) -> combine (m/l/o) on the named workloads at full size
    against the oracle's attention."""
    w = workloads.WORKLOADS[cfg]
    inp = workloads.generate(w)
    q, k, v = inp["q"].to(gpu), inp["k"].to(gpu), inp["v"].to(gpu)
    kl = None if inp["kv_lens"] is None else inp["kv_lens"].to(gpu)
    op, mp, lp = fd.decode_split_mlo(q, k, v, kl, num_splits=B, scale=w.scale)
    o, lse = fd.combine_mlo(op, mp, lp, out_dtype=workloads.TORCH_DTYPES[w.out_dtype])
    torch.cuda.synchronize()
    del q, k, v, op
    lens = inp["kv_lens"]
    ro, rl = oracle.attention(w.dtype, workloads.raw(inp["q"]), workloads.raw(inp["k"]),
                              workloads.raw(inp["v"]), None if lens is None else lens.numpy(),
                              scale=w.scale)
    tol_o, tol_l = TOL[w.dtype]
    go = _np(o).reshape(ro.shape)
    gl = _np(lse).reshape(rl.shape)
    err_o, err_l = np.abs(go - ro).max(), np.abs(gl - rl).max()
    print(f"mlo route {w.name} B{B}: o {err_o:.2e} lse {err_l:.2e}", flush=True)
    assert err_o <= tol_o and err_l <= tol_l
