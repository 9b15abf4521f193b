"""GPU parity at the library's limits, through the C ABI, against the oracle.

- K and V tensors past 4 GiB each: every address offset within a sequence's
  split is 32 bits wide, and sequence and split bases are 64 bits wide.  Both
  split kernels are covered: grouped bf16 on the token-balanced plan, and
  fp32 on the vector kernel.
- The largest query group a matrix-core wave holds (16 query heads per KV
  head), at each head size.
- The split-count cap of the automatic plan (512 splits of one long row), and
  an explicit count at that cap.
- Many sequences (more units than work-groups in the balanced partition, and
  most work-groups spanning several units), and many heads.
- Query groups larger than one matrix-core tile (32 query heads per KV head).
"""
import numpy as np
import pytest
import torch

import oracle
from decode_attention_03_amd import fd, workloads

pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-5, 1e-5), "f16": (1.5e-2, 1e-3), "bf16": (1.5e-2, 1e-3)}


def _check(name, o, lse, inp, w):
    lens = inp["kv_lens"]
    ro, rl = oracle.attention(w.dtype, workloads.raw(inp["q"]), workloads.raw(inp["k"]),
                              workloads.raw(inp["v"]), None if lens is None else lens.numpy(),
                              scale=w.scale)
    tol_o, tol_l = TOL[w.dtype]
    go = o.float().cpu().double().numpy().reshape(ro.shape)
    gl = lse.cpu().double().numpy().reshape(rl.shape)
    assert np.isfinite(go).all(), f"{name}: non-finite output"
    assert np.array_equal(np.isneginf(gl), np.isneginf(rl))
    fin = np.isfinite(rl)
    err_o = np.abs(go - ro).max()
    err_l = np.abs(gl[fin] - rl[fin]).max() if fin.any() else 0.0
    print(f"{name}: max|o-ref|={err_o:.3e} max|lse-ref|={err_l:.3e}", flush=True)
    assert err_o <= tol_o and err_l <= tol_l


def _run(gpu, inp, w, **kw):
    lens = inp["kv_lens"]
    q, k, v = inp["q"].to(gpu), inp["k"].to(gpu), inp["v"].to(gpu)
    o, lse = fd.decode(q, k, v, None if lens is None else lens.to(gpu), scale=w.scale, **kw)
    torch.cuda.synchronize()
    del q, k, v
    torch.cuda.empty_cache()
    return o, lse


@pytest.mark.parametrize("case", ["gqa_bf16_balanced", "mha_f32"])
def test_kv_tensors_past_4gib(gpu, case):
    if case == "gqa_bf16_balanced":
        # 2 x 2,228,224 tokens x 4 KV heads x 128 x 2 B = 4.56 GB per tensor
        n = (1 << 21) + (1 << 17)
        w, inp = workloads.custom(2, 32, 4, 128, n, dtype="bf16", seed=61, lens=[n, n - 12345])
        assert fd.decode_plan(2, 32, 4, n, 128, torch.bfloat16, True)["route"] == "balanced"
    else:
        # 1 x 4,456,448 tokens x 4 heads x 64 x 4 B = 4.56 GB per tensor
        n = (1 << 22) + (1 << 18)
        w, inp = workloads.custom(1, 4, 4, 64, n, dtype="f32", seed=62)
    nbytes = inp["k"].numel() * inp["k"].element_size()
    assert nbytes > (1 << 32)
    print(f"{case}: K and V {nbytes / 2**30:.2f} GiB each", flush=True)
    o, lse = _run(gpu, inp, w)
    _check(case, o, lse, inp, w)


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_largest_group_every_head_size(gpu, d, dtype):
    lens = [3001, 0, 16, 1777]
    w, inp = workloads.custom(4, 32, 2, d, max(lens), dtype=dtype, seed=63 + d, lens=lens)
    for splits in (0, 1, 6):
        o, lse = _run(gpu, inp, w, num_splits=splits)
        _check(f"G16_{dtype}_d{d}_B{splits}", o, lse, inp, w)


def test_split_count_cap(gpu):
    """One long row: the automatic plan reaches its cap of 512 splits, and an
    explicit 512 with the shortest split length that covers the row."""
    n = (1 << 20) + 5
    w, inp = workloads.custom(1, 1, 1, 64, n, dtype="f16", seed=64)
    b, length = fd.choose_splits(1, 1, 1, n, 64, torch.float16)
    assert b >= 500 and b * length >= n
    o, lse = _run(gpu, inp, w)
    _check(f"auto_B{b}", o, lse, inp, w)
    o, lse = _run(gpu, inp, w, num_splits=512, split_len=-(-n // 512))
    _check("B512", o, lse, inp, w)


@pytest.mark.parametrize("dtype,hq,hkv", [("bf16", 8, 2), ("f32", 4, 4)])
def test_many_sequences(gpu, dtype, hq, hkv):
    """600 ragged sequences, lengths 0..400: for the grouped case, 1200 units
    over fewer work-groups, so most work-groups finish one unit and start
    the next."""
    rng = np.random.default_rng(65)
    lens = rng.integers(0, 401, 600).tolist()
    w, inp = workloads.custom(600, hq, hkv, 128, max(lens), dtype=dtype, seed=65, lens=lens)
    for splits in (0, 2):
        o, lse = _run(gpu, inp, w, num_splits=splits)
        _check(f"b600_{dtype}_B{splits}", o, lse, inp, w)


def test_many_heads(gpu):
    lens = [2000, 1500]
    w, inp = workloads.custom(2, 128, 64, 64, 2000, dtype="bf16", seed=66, lens=lens)
    for splits in (0, 1, 4):
        o, lse = _run(gpu, inp, w, num_splits=splits)
        _check(f"hq128_hkv64_B{splits}", o, lse, inp, w)


@pytest.mark.parametrize("dtype,group,hkv,d", [("bf16", 32, 2, 128), ("f16", 64, 1, 64),
                                               ("bf16", 128, 1, 128), ("f16", 24, 2, 256),
                                               ("bf16", 17, 3, 128)])
def test_groups_larger_than_a_matrix_tile(gpu, dtype, group, hkv, d):
    """More than 16 query heads per KV head (up to multi-query attention): the
    group is cut into tiles of 16 (the last one partial for 17 and 24) and
    every tile reads the same K/V rows; ragged lengths, automatic plan,
    explicit splits, one split (direct output), and the split stage's
    partials in both formats against the oracle's."""
    lens = [2500, 1, 0, 777]
    w, inp = workloads.custom(4, group * hkv, hkv, d, max(lens), dtype=dtype,
                              seed=67 + group + d, lens=lens)
    for splits in (0, 1, 5):
        o, lse = _run(gpu, inp, w, num_splits=splits)
        _check(f"G{group}_{dtype}_d{d}_B{splits}", o, lse, inp, w)
    q, k, v = inp["q"].to(gpu), inp["k"].to(gpu), inp["v"].to(gpu)
    kl = inp["kv_lens"].to(gpu)
    B, L = 6, 432
    o_part, lse_part = fd.decode_split(q, k, v, kl, num_splits=B, split_len=L, scale=w.scale)
    o_m, m_part, l_part = fd.decode_split_mlo(q, k, v, kl, num_splits=B, split_len=L,
                                              scale=w.scale)
    torch.cuda.synchronize()
    rop, rlp, rmp, rll = oracle.split_partials(dtype, workloads.raw(inp["q"]),
                                               workloads.raw(inp["k"]), workloads.raw(inp["v"]),
                                               np.array(lens, dtype=np.int32), B, L,
                                               scale=w.scale, with_mlo=True)
    tol_o, tol_l = TOL[dtype]
    fin = np.isfinite(rlp)
    assert np.abs(o_part.cpu().double().numpy() - rop).max() <= tol_o
    assert np.array_equal(np.isneginf(lse_part.cpu().numpy()), ~fin)
    assert np.abs(lse_part.cpu().double().numpy()[fin] - rlp[fin]).max() <= tol_l
    assert np.abs(o_m.cpu().double().numpy() - rop).max() <= tol_o
    gm, gl = m_part.cpu().double().numpy(), l_part.cpu().double().numpy()
    # the triple's own S = m + log l against the oracle's LSE
    assert np.abs((gm + np.log(np.where(fin, gl, 1.0)))[fin] - rlp[fin]).max() <= tol_l
