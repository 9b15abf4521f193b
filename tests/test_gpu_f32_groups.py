"""GPU parity of fp32 grouped-query heads on the vector kernel against the fp64
oracle, through the C ABI.

fp32 grouped heads run on the vector kernel with up to eight query heads of
one KV head per work-group (eight at d <= 128 when the group divides by eight,
else four, two when the group is only even, one when odd), every row of lanes
holding all of their q rows and running states.  These cases cover
each head count per work-group on every route the vector kernel serves: fixed
splits (the split stage alone, the m/l/o format, the whole decode), one split
per row, the automatic plan without lengths, the token-balanced partition for
ragged lengths (units of several query heads, their rows in one slot), and a
paged cache.  K/V rows past each length are NaN, so a read past a length shows
up as a non-finite result.
"""
import numpy as np
import pytest
import torch

import oracle
from decode_attention_03_amd import fd, workloads

pytestmark = pytest.mark.gpu

TOL_O, TOL_L = 1e-5, 1e-5

# name, batch, heads_kv, group, d, n_max, lens
CASES = [
    ("g4_d128", 5, 2, 4, 128, 3000, [3000, 0, 17, 2049, 1500]),
    ("g2_d64", 6, 3, 2, 64, 2500, [1, 2500, 999, 0, 64, 2047]),
    ("g8_d256", 3, 1, 8, 256, 1800, [1800, 700, 33]),
    ("g6_d64", 4, 2, 6, 64, 2000, [2000, 15, 1024, 0]),
    ("g3_d128", 4, 2, 3, 128, 1500, [1500, 3, 0, 777]),
    ("g8_d128", 4, 2, 8, 128, 2200, [2200, 1, 1100, 0]),
    ("g16_d64", 3, 2, 16, 64, 1700, [17, 1700, 900]),
    ("g32_d64_mqa", 2, 1, 32, 64, 3000, [3000, 640]),
]


def _inputs(name, batch, hkv, group, d, n_max, lens):
    seed = sum(map(ord, name)) + 7
    w, inp = workloads.custom(batch, hkv * group, hkv, d, n_max, dtype="f32", seed=seed,
                              lens=lens)
    for b, n in enumerate(lens):  # NaN past every length
        inp["k"][b, n:] = float("nan")
        inp["v"][b, n:] = float("nan")
    return w, inp


def _check(tag, o, lse, ro, rl):
    go = o.cpu().double().numpy().reshape(ro.shape)
    gl = lse.cpu().double().numpy().reshape(rl.shape)
    assert np.isfinite(go).all(), f"{tag}: non-finite output"
    assert np.array_equal(np.isneginf(gl), np.isneginf(rl)), f"{tag}: -inf pattern differs"
    fin = np.isfinite(rl)
    err_o = np.abs(go - ro).max()
    err_l = np.abs(gl[fin] - rl[fin]).max() if fin.any() else 0.0
    print(f"{tag}: max|o-ref|={err_o:.3e} max|lse-ref|={err_l:.3e}", flush=True)
    assert err_o <= TOL_O and err_l <= TOL_L, tag


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_f32_groups_every_route(gpu, case):
    name, batch, hkv, group, d, n_max, lens = case
    w, inp = _inputs(*case)
    q, k, v = inp["q"].to(gpu), inp["k"].to(gpu), inp["v"].to(gpu)
    kl = inp["kv_lens"].to(gpu)
    lens_np = np.array(lens, dtype=np.int32)
    raw = (workloads.raw(inp["q"]), workloads.raw(inp["k"]), workloads.raw(inp["v"]))
    ro, rl = oracle.attention("f32", *raw, lens_np, scale=w.scale)
    # ragged lengths given: the token-balanced partition on the vector kernel
    plan = fd.decode_plan(batch, hkv * group, hkv, n_max, d, q.dtype, True)
    assert plan["route"] == "balanced" and plan["kernel"] == "vector", plan
    o, lse = fd.decode(q, k, v, kl, scale=w.scale)
    torch.cuda.synchronize()
    _check(f"{name} balanced", o, lse, ro, rl)
    # fixed splits (5 of them: the plain combine), and one split per row
    for B in (5, 1):
        o, lse = fd.decode(q, k, v, kl, scale=w.scale, num_splits=B)
        torch.cuda.synchronize()
        _check(f"{name} B{B}", o, lse, ro, rl)
    # the split stage alone, against the oracle's partials, in both formats
    B, L = 3, 1008
    rop, rlp, rmp, rll = oracle.split_partials("f32", *raw, lens_np, B, L, scale=w.scale,
                                               with_mlo=True)
    op, lp = fd.decode_split(q, k, v, kl, num_splits=B, split_len=L, scale=w.scale)
    om, mp, lm = fd.decode_split_mlo(q, k, v, kl, num_splits=B, split_len=L, scale=w.scale)
    torch.cuda.synchronize()
    assert np.abs(op.cpu().double().numpy() - rop).max() <= TOL_O
    fin = np.isfinite(rlp)
    assert np.array_equal(np.isfinite(lp.cpu().numpy()), fin)
    assert np.abs(lp.cpu().double().numpy()[fin] - rlp[fin]).max() <= TOL_L
    assert np.abs(om.cpu().double().numpy() - rop).max() <= TOL_O
    empty = np.isneginf(rmp)
    gm = mp.cpu().double().numpy()
    assert np.array_equal(np.isneginf(gm), empty)
    assert np.abs(gm[~empty] - rmp[~empty]).max() <= TOL_L
    gl = lm.cpu().double().numpy()
    assert (np.abs(gl[~empty] - rll[~empty]) / rll[~empty]).max() <= TOL_L


@pytest.mark.parametrize("group,d", [(4, 128), (2, 64), (8, 128)])
def test_f32_groups_full_length_and_paged(gpu, group, d):
    """Every sequence full and no lengths: the automatic fixed-split plan; then
    the same cache in 16-token pages with ragged lengths (balanced) and fixed
    splits."""
    w, inp = workloads.custom(8, 2 * group, 2, d, 4096, dtype="f32", seed=60 + group)
    q, k, v = inp["q"].to(gpu), inp["k"].to(gpu), inp["v"].to(gpu)
    raw = (workloads.raw(inp["q"]), workloads.raw(inp["k"]), workloads.raw(inp["v"]))
    o, lse = fd.decode(q, k, v, scale=w.scale)
    torch.cuda.synchronize()
    ro, rl = oracle.attention("f32", *raw, None, scale=w.scale)
    _check(f"full G{group} d{d}", o, lse, ro, rl)
    lens = [4096, 1, 0, 2000, 4095, 17, 3000, 64]
    pin = dict(inp, kv_lens=torch.tensor(lens, dtype=torch.int32))
    pg = workloads.paginate(pin, 16, seed=5)
    kp, vp, bt = pg["k_pages"].to(gpu), pg["v_pages"].to(gpu), pg["block_table"].to(gpu)
    kl = pin["kv_lens"].to(gpu)
    ro, rl = oracle.attention("f32", *raw, np.array(lens, dtype=np.int32), scale=w.scale)
    for B in (0, 4):
        o, lse = fd.decode_paged(q, kp, vp, bt, kl, scale=w.scale, num_splits=B)
        torch.cuda.synchronize()
        _check(f"paged G{group} d{d} B{B}", o, lse, ro, rl)
