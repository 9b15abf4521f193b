"""GPU parity of the paged K/V cache path (block-table indirection) through the
C ABI.

Pages are laid out from the same seeded inputs the contiguous tests use
(workloads.paginate: a seeded permutation of physical pages; pages nobody
owns hold NaN).  The expected result is the oracle's attention over the
original contiguous K/V, and with the same split count and length the paged
kernels must reproduce the contiguous kernels bit for bit: the page lookup
changes addresses, not arithmetic.
"""

import numpy as np
import pytest
import torch

import oracle
from decode_attention_03_amd import fd, workloads

pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-5, 1e-5), "f16": (1.5e-2, 1e-3), "bf16": (1.5e-2, 1e-3)}


def _lens_full(w, inp):
    if inp["kv_lens"] is not None:
        return inp["kv_lens"]
    return torch.full((w.batch,), inp["max_kv_len"], dtype=torch.int32)


def _paged_on(gpu, inp, page_size, seed):
    pg = workloads.paginate(inp, page_size, seed=seed)
    return (pg["k_pages"].to(gpu), pg["v_pages"].to(gpu), pg["block_table"].to(gpu), pg)


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


@pytest.mark.parametrize("cfg,page_size", [(1, 16), (2, 16), (3, 256), (4, 16), (4, 64),
                                           (5, 128)])
def test_paged_named_workloads(gpu, cfg, page_size):
    """The named workloads at full size through fd_decode_paged, library plan."""
    w = workloads.WORKLOADS[cfg]
    inp = workloads.generate(w)
    lens = _lens_full(w, inp)
    inp = dict(inp, kv_lens=lens)
    kp, vp, bt, pg = _paged_on(gpu, inp, page_size, seed=cfg)
    q = inp["q"].to(gpu)
    o, lse = fd.decode_paged(q, kp, vp, bt, lens.to(gpu), scale=w.scale,
                             num_splits=w.num_splits)
    torch.cuda.synchronize()
    del kp, vp
    ro, rl = oracle.attention(w.dtype, workloads.raw(inp["q"]), workloads.raw(inp["k"]),
                              workloads.raw(inp["v"]), lens.numpy(), scale=w.scale)
    _check(f"paged{page_size}_{w.name}", o, lse, ro, rl, w.dtype)


@pytest.mark.parametrize("dtype,group,d", [("f32", 1, 64), ("bf16", 1, 128), ("bf16", 8, 128),
                                           ("f16", 4, 256), ("f16", 2, 64), ("bf16", 32, 128),
                                           ("bf16", 128, 128), ("f16", 40, 256)])
@pytest.mark.parametrize("page_size", [16, 32, 1024])
def test_paged_split_bitwise_equal_contiguous(gpu, dtype, group, d, page_size):
    """Same split count and length: paged partials equal contiguous partials
    bit for bit; ragged lengths end mid-page, one sequence is empty."""
    lens = [1000, 0, 257, 64, 999, 17]
    w, inp = workloads.custom(6, 2 * group, 2, d, 1000, dtype=dtype, seed=31 + group,
                              lens=lens)
    kp, vp, bt, pg = _paged_on(gpu, inp, page_size, seed=page_size)
    q, k, v = inp["q"].to(gpu), inp["k"].to(gpu), inp["v"].to(gpu)
    kl = inp["kv_lens"].to(gpu)
    B, L = 5, 208  # L a multiple of 16
    op_c, lp_c = fd.decode_split(q, k, v, kl, num_splits=B, split_len=L, scale=w.scale)
    op_p, lp_p = fd.decode_split_paged(q, kp, vp, bt, kl, num_splits=B, split_len=L,
                                       scale=w.scale)
    torch.cuda.synchronize()
    # contiguous max_kv_len is 1000; paged is max_pages * page_size >= 1000: same splits
    assert torch.equal(op_c, op_p) and torch.equal(lp_c, lp_p)
    rop, rlp = oracle.split_partials(dtype, workloads.raw(inp["q"]), workloads.raw(inp["k"]),
                                     workloads.raw(inp["v"]), np.array(lens, dtype=np.int32),
                                     B, L, scale=w.scale)
    tol_o, tol_l = TOL[dtype]
    assert np.abs(op_p.cpu().double().numpy() - rop).max() <= tol_o
    fin = np.isfinite(rlp)
    assert np.abs(lp_p.cpu().double().numpy()[fin] - rlp[fin]).max() <= tol_l


@pytest.mark.parametrize("group", [1, 8, 40])
def test_paged_decode_plans(gpu, group):
    """Whole decode over pages: automatic plan (balanced for grouped ragged),
    one split, and explicit split counts, against the oracle; page size larger
    than a split and a table wider than any sequence needs."""
    lens = [3000, 1, 0, 2049, 16, 4095]
    w, inp = workloads.custom(6, 2 * group, 2, 128, 4096, dtype="bf16", seed=77 + group,
                              lens=lens)
    ro, rl = oracle.attention("bf16", workloads.raw(inp["q"]), workloads.raw(inp["k"]),
                              workloads.raw(inp["v"]), np.array(lens, dtype=np.int32),
                              scale=w.scale)
    q = inp["q"].to(gpu)
    kl = inp["kv_lens"].to(gpu)
    for page_size in (16, 512):
        kp, vp, bt, pg = _paged_on(gpu, inp, page_size, seed=page_size + group)
        for B in (0, 1, 3, 7):
            o, lse = fd.decode_paged(q, kp, vp, bt, kl, scale=w.scale, num_splits=B)
            _check(f"paged{page_size}_G{group}_B{B}", o, lse, ro, rl, "bf16")


def test_paged_rejects_bad_arguments(gpu):
    w, inp = workloads.custom(2, 4, 2, 64, 64, dtype="bf16", seed=3)
    kp, vp, bt, pg = _paged_on(gpu, dict(inp, kv_lens=None), 16, seed=1)
    q = inp["q"].to(gpu)
    with pytest.raises(fd.FDError) as e:
        fd.decode_paged(q, kp, vp, bt, num_splits=2, split_len=40)
    assert e.value.code == fd.ERR_INVALID
    kp20 = kp[:, :8]
    with pytest.raises(fd.FDError) as e:
        fd.decode_paged(q, kp20.contiguous(), vp[:, :8].contiguous(), bt, num_splits=1)
    assert e.value.code == fd.ERR_UNSUPPORTED
