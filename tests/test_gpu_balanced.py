"""GPU parity of the token-balanced partition (fd_decode's automatic plan for
ragged batches: grouped heads on the matrix-core kernel, one query head per
KV head or fp32 on the vector kernel) against the fp64 oracle, through the C ABI.

The partition cuts the flattened (KV head, sequence, token) space into equal
shares; these cases aim at its corners: empty sequences between full ones,
every sequence empty, fewer positions than work-groups, more than 64
sequences (the in-kernel prefix scan runs over several 64-lane chunks), one
sequence spread over hundreds of pieces, clamped lengths, KV heads in
multiples of eight (the permuted share order) and not, groups of 17 to
32 query heads per KV head (two query tiles per piece), and larger groups on
work-groups of two or four waves.  K/V rows past each
length are NaN and the workspace starts NaN-filled, so a read past a length or
of an unwritten slot shows up as a wrong or non-finite result.
"""
import numpy as np
import pytest
import torch

import oracle
from decode_attention_03_amd import fd, workloads

pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-5, 1e-5), "f16": (1.5e-2, 1e-3), "bf16": (1.5e-2, 1e-3)}

# name, batch, heads_kv, group, d, dtype, max_kv_len, lens (None: drawn from seed)
CASES = [
    ("zeros_between", 7, 2, 8, 128, "bf16", 5000, [0, 5000, 0, 0, 17, 3000, 0]),
    ("all_empty", 5, 2, 4, 128, "bf16", 64, [0, 0, 0, 0, 0]),
    ("all_one_token", 40, 2, 2, 64, "f16", 8, [1] * 40),
    ("batch130", 130, 2, 4, 64, "f16", 700, None),
    ("one_long_row", 3, 1, 16, 256, "f16", 40000, [1, 40000, 2]),
    ("clamped", 4, 4, 8, 128, "bf16", 300, [0, 300, 5000, -3]),
    ("group2_d256", 6, 3, 2, 256, "bf16", 3000, [2999, 1, 1500, 0, 3000, 64]),
    # KV heads in multiples of 8: neighbouring work-groups take consecutive
    # heads of one share (the share index is permuted); 24 heads do not
    # divide the work-group count and keep the plain order
    ("hkv8_group8", 6, 8, 8, 128, "bf16", 3000, [3000, 0, 17, 2500, 1, 1999]),
    ("hkv16_group4_d64", 9, 16, 4, 64, "f16", 1200, [0, 1200, 5, 0, 777, 1199, 0, 64, 300]),
    ("hkv8_group32", 3, 8, 32, 128, "bf16", 2000, [2000, 1, 1500]),
    ("hkv24_group2", 2, 24, 2, 64, "bf16", 500, [500, 250]),
    # groups past one 16-query tile: every tile of a unit in the one work-group
    ("group32_d128_2waves", 6, 2, 32, 128, "bf16", 6000, [6000, 0, 17, 4099, 1, 2500]),
    ("group32_d64_mqa", 9, 1, 32, 64, "f16", 3000, [3000, 2, 0, 1777, 3000, 64, 500, 0, 2999]),
    ("group24_d64", 5, 2, 24, 64, "bf16", 2000, [1999, 0, 300, 2000, 33]),
    ("group17_d128", 4, 3, 17, 128, "f16", 2500, [2500, 1, 1024, 0]),
    # more tiles than one wave holds: two or four waves per work-group share
    # each staged K/V step (the last wave's last tile partial or empty)
    ("group48_d64_4waves", 5, 2, 48, 64, "f16", 2200, [2200, 0, 15, 1999, 640]),
    ("group96_d64_8waves", 3, 1, 96, 64, "bf16", 2100, [2100, 5, 1600]),
    ("group64_d128_4waves", 4, 2, 64, 128, "bf16", 3000, [3000, 1, 0, 2047]),
    ("group128_d128_8waves", 6, 1, 128, 128, "bf16", 2500, [2500, 17, 0, 1300, 2499, 64]),
    ("group40_d256_4waves", 3, 2, 40, 256, "f16", 1800, [1800, 900, 0]),
    ("group24_d256_2waves", 5, 1, 24, 256, "bf16", 1500, [0, 1500, 3, 777, 1499]),
    # the vector kernel's pieces: one unit per (sequence, query head); query
    # heads in multiples of 8 that divide the work-group count take the
    # permuted share order (8, 32), 40 and 3 the plain one
    ("vec_mha_zeros_between", 7, 4, 1, 128, "bf16", 5000, [0, 5000, 0, 0, 17, 3000, 0]),
    ("vec_mha_all_empty", 5, 2, 1, 64, "f16", 64, [0, 0, 0, 0, 0]),
    ("vec_mha_all_one_token", 40, 3, 1, 64, "bf16", 8, [1] * 40),
    ("vec_mha_batch130", 130, 2, 1, 128, "f16", 700, None),
    ("vec_mha_one_long_row", 3, 1, 1, 256, "f16", 40000, [1, 40000, 2]),
    ("vec_mha_clamped_h8", 4, 8, 1, 128, "bf16", 300, [0, 300, 5000, -3]),
    ("vec_mha_h32_d256", 5, 32, 1, 256, "bf16", 3000, [3000, 1, 0, 2047, 1500]),
    ("vec_mha_h40_d64", 3, 40, 1, 64, "f16", 1000, [999, 0, 1000]),
    ("vec_f32_mha_d64", 6, 4, 1, 64, "f32", 2000, [2000, 0, 17, 1999, 1, 640]),
    ("vec_f32_gqa4_d128", 5, 2, 4, 128, "f32", 1500, [1500, 3, 0, 777, 1499]),
    ("vec_f32_d256", 3, 2, 1, 256, "f32", 1000, [1000, 0, 999]),
]


def _case_inputs(name, batch, hkv, group, d, dtype, n_max, lens):
    seed = sum(map(ord, name))
    w, inp = workloads.custom(batch, hkv * group, hkv, d, n_max, dtype=dtype, seed=seed)
    if lens is None:
        g = np.random.default_rng(seed)
        lens = g.integers(0, n_max + 1, size=batch).tolist()
        lens[3] = 0
        lens[64] = n_max
    eff = [min(max(x, 0), n_max) for x in lens]
    for b, n in enumerate(eff):  # NaN past every length
        inp["k"][b, n:] = float("nan")
        inp["v"][b, n:] = float("nan")
    inp["kv_lens"] = torch.tensor(lens, dtype=torch.int32)
    return w, inp, eff


def _check(name, o, lse, ro, rl, dtype):
    tol_o, tol_l = TOL[dtype]
    go = o.float().cpu().double().numpy().reshape(ro.shape)
    gl = lse.cpu().double().numpy().reshape(rl.shape)
    assert np.isfinite(go).all(), f"{name}: non-finite output"
    assert np.array_equal(np.isneginf(gl), np.isneginf(rl)), f"{name}: -inf pattern differs"
    fin = np.isfinite(rl)
    err_o = np.abs(go - ro).max()
    err_l = np.abs(gl[fin] - rl[fin]).max() if fin.any() else 0.0
    print(f"{name}: max|o-ref|={err_o:.3e} max|lse-ref|={err_l:.3e}", flush=True)
    assert err_o <= tol_o and err_l <= tol_l
    assert np.all(go[~fin] == 0)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_balanced_partition_cases(gpu, case):
    name, batch, hkv, group, d, dtype, n_max, lens = case
    w, inp, eff = _case_inputs(*case)
    q, k, v = inp["q"].to(gpu), inp["k"].to(gpu), inp["v"].to(gpu)
    kl = inp["kv_lens"].to(gpu)
    need = fd.decode_workspace_bytes(batch, hkv * group, hkv, n_max, d, q.dtype, True)
    assert need > 0
    plan = fd.decode_plan(batch, hkv * group, hkv, n_max, d, q.dtype, True)
    assert plan["route"] == "balanced" and plan["workspace_bytes"] == need
    vector = name.startswith("vec_")
    assert (plan["kernel"] == "vector") == vector, plan
    if vector:  # one unit per (sequence, query head), one-wave work-groups
        assert plan["waves_per_group"] == 1 and plan["query_tiles"] == 0, plan
    if name.endswith("waves"):
        assert plan["waves_per_group"] == int(name[-6]), plan
    ws = torch.full((need // 4 + 1,), float("nan"), device=gpu)
    o, lse = fd.decode(q, k, v, kl, scale=w.scale, workspace=ws)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(dtype, workloads.raw(inp["q"]), workloads.raw(inp["k"]),
                              workloads.raw(inp["v"]), np.array(eff, dtype=np.int32),
                              scale=w.scale)
    _check(name, o, lse, ro, rl, dtype)


@pytest.mark.parametrize("group", [8, 1])
def test_balanced_matches_fixed_splits_and_repeats(gpu, group):
    """The balanced plan and a fixed-split plan of the same inputs agree to the
    bf16 bounds; two balanced runs are bitwise equal (matrix-core and vector
    kernels)."""
    w, inp, eff = _case_inputs("zeros_between", 7, 2, group, 128, "bf16", 5000,
                               [0, 5000, 0, 0, 17, 3000, 0])
    q, k, v = inp["q"].to(gpu), inp["k"].to(gpu), inp["v"].to(gpu)
    kl = inp["kv_lens"].to(gpu)
    o1, l1 = fd.decode(q, k, v, kl, scale=w.scale)
    o2, l2 = fd.decode(q, k, v, kl, scale=w.scale)
    of, lf = fd.decode(q, k, v, kl, scale=w.scale, num_splits=3)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert (o1.float() - of.float()).abs().max().item() <= 1.6e-2
    fin = torch.isfinite(lf)
    assert torch.equal(torch.isfinite(l1), fin)
    assert (l1[fin] - lf[fin]).abs().max().item() <= 1e-3


def test_balanced_workspace_too_small(gpu):
    w, inp, eff = _case_inputs("clamped", 4, 4, 8, 128, "bf16", 300, [0, 300, 5000, -3])
    q, k, v = inp["q"].to(gpu), inp["k"].to(gpu), inp["v"].to(gpu)
    kl = inp["kv_lens"].to(gpu)
    need = fd.decode_workspace_bytes(4, 32, 4, 300, 128, q.dtype, True)
    ws = torch.empty(need - 256, dtype=torch.uint8, device=gpu)
    with pytest.raises(fd.FDError) as e:
        fd.decode(q, k, v, kl, scale=w.scale, workspace=ws)
    assert e.value.code == fd.ERR_WORKSPACE
