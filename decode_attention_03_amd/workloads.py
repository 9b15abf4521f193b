"""Seeded synthetic decode-attention inputs.

This module only draws inputs; it holds none of the attention arithmetic and
is shared by the tests, the benchmark and the smoke check (the HIP library
and the oracle are each fed from it, and neither imports the other).

Every tensor piece is drawn by its own ``torch.Generator`` whose seed is the
first 8 bytes of SHA-256 over (workload seed, tag), so pieces can be drawn in
parallel threads and the result does not depend on the thread count:
  ("lens",)              per-sequence lengths, when they are ragged
  ("q",)                 q [batch, heads_q, d]
  ("k", b, c), ("v", b, c)
                         K/V rows [c*CHUNK, (c+1)*CHUNK) of sequence b
  ("dominant", b, h)     the dominant-key positions, when the workload has them
Values are fp32 ``randn`` times ``std``, rounded to nearest-even into the
storage dtype.  Shapes and distributions follow the pages' decode setting
(one query row per (sequence, head) against a long KV cache), at the sizes of
the five named workloads below.
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import hashlib
import math
import os

import numpy as np
import torch

TORCH_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads_q: int
    heads_kv: int
    head_dim: int
    max_kv_len: int
    dtype: str                 # storage dtype of q, K, V: "f32" | "f16" | "bf16"
    out_dtype: str             # dtype of o (LSE is always fp32)
    seed: int
    std: float = 1.0           # q, K, V ~ N(0, std^2)
    num_splits: int = 0        # 0: chosen by the library's heuristic
    ragged: tuple | None = None  # (lo, hi): lengths ~ U{lo..hi} inclusive
    dominant: int = 0          # keys per head set to factor * q / |q| * sqrt(d)
    dominant_factor: float = 6.0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def group(self) -> int:
        return self.heads_q // self.heads_kv

    def describe(self) -> dict:
        d = dataclasses.asdict(self)
        d["scale"] = self.scale
        return d


# The five named decode workloads.
WORKLOADS = {
    1: Workload("single_seq_f32_d64_n1024", batch=1, heads_q=1, heads_kv=1, head_dim=64,
                max_kv_len=1024, dtype="f32", out_dtype="f32", seed=1, num_splits=4),
    2: Workload("mha_bf16_b8_h32_d128_n4096", batch=8, heads_q=32, heads_kv=32, head_dim=128,
                max_kv_len=4096, dtype="bf16", out_dtype="bf16", seed=2),
    3: Workload("mha_bf16_b1_h32_d128_n65536_dominant16", batch=1, heads_q=32, heads_kv=32,
                head_dim=128, max_kv_len=65536, dtype="bf16", out_dtype="bf16", seed=3,
                dominant=16),
    4: Workload("gqa_bf16_b16_hq64_hkv8_d128_ragged512_32768", batch=16, heads_q=64, heads_kv=8,
                head_dim=128, max_kv_len=32768, dtype="bf16", out_dtype="bf16", seed=4,
                ragged=(512, 32768)),
    5: Workload("mha_f16_b4_h16_d256_n131072", batch=4, heads_q=16, heads_kv=16, head_dim=256,
                max_kv_len=131072, dtype="f16", out_dtype="f16", seed=5, std=0.5),
}


CHUNK = 4096  # K/V rows per independently seeded piece


def _gen(seed: int, *tag) -> torch.Generator:
    digest = hashlib.sha256(repr((int(seed),) + tuple(tag)).encode()).digest()
    g = torch.Generator(device="cpu")
    g.manual_seed(int.from_bytes(digest[:8], "little") & ((1 << 63) - 1))
    return g


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _randn(gen: torch.Generator, shape, std: float, dtype: str) -> torch.Tensor:
    x = torch.randn(shape, generator=gen, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(TORCH_DTYPES[dtype])


def generate(w: Workload, poison_tail: bool = False) -> dict:
    """Draw the workload's inputs on the CPU.

    Returns a dict with q, k, v (torch CPU tensors in w.dtype), kv_lens (int32
    tensor [batch], or None when every sequence is max_kv_len long) and
    max_kv_len (the K/V row count actually allocated).  With poison_tail,
    K/V rows at or beyond a sequence's length are set to NaN after the draw,
    so any read of them shows up in the result.
    """
    lens = None
    n_max = w.max_kv_len
    if w.ragged is not None:
        lo, hi = w.ragged
        lens = torch.randint(lo, hi + 1, (w.batch,), generator=_gen(w.seed, "lens"),
                             dtype=torch.int64)
        lens = lens.to(torch.int32)
        n_max = int(lens.max())
    q = _randn(_gen(w.seed, "q"), (w.batch, w.heads_q, w.head_dim), w.std, w.dtype)
    dt = TORCH_DTYPES[w.dtype]
    k = torch.empty((w.batch, n_max, w.heads_kv, w.head_dim), dtype=dt)
    v = torch.empty_like(k)

    def fill(job):
        name, b, c = job
        rows = min(CHUNK, n_max - c * CHUNK)
        dst = k if name == "k" else v
        dst[b, c * CHUNK: c * CHUNK + rows] = _randn(_gen(w.seed, name, b, c),
                                                     (rows, w.heads_kv, w.head_dim), w.std,
                                                     w.dtype)

    jobs = [(name, b, c) for b in range(w.batch) for name in ("k", "v")
            for c in range(-(-n_max // CHUNK))]
    # one torch thread per worker: the pieces already run in parallel, and
    # nested intra-op pools would start threads per worker
    intra = torch.get_num_threads()
    torch.set_num_threads(1)
    try:
        with concurrent.futures.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, jobs))
    finally:
        torch.set_num_threads(intra)
    if w.dominant:
        if w.group != 1:
            raise ValueError("dominant keys are defined for one query head per KV head")
        d = w.head_dim
        for b in range(w.batch):
            for h in range(w.heads_kv):
                nb = n_max if lens is None else int(lens[b])
                pos = torch.randperm(nb, generator=_gen(w.seed, "dominant", b, h))[: w.dominant]
                qv = q[b, h].to(torch.float64)
                key = (w.dominant_factor * math.sqrt(d) / qv.norm()) * qv
                k[b, pos, h, :] = key.to(dt)
    if poison_tail and lens is not None:
        for b in range(w.batch):
            k[b, int(lens[b]):] = float("nan")
            v[b, int(lens[b]):] = float("nan")
    return {"q": q, "k": k, "v": v, "kv_lens": lens, "max_kv_len": n_max}


def custom(batch, heads_q, heads_kv, head_dim, max_kv_len, dtype="f32", seed=0, std=1.0,
           lens=None, out_dtype=None, num_splits=0) -> tuple[Workload, dict]:
    """A workload of any shape (test matrices); lens is an optional list of lengths."""
    w = Workload(f"custom_b{batch}_hq{heads_q}_hkv{heads_kv}_d{head_dim}_n{max_kv_len}_{dtype}",
                 batch, heads_q, heads_kv, head_dim, max_kv_len, dtype, out_dtype or dtype, seed,
                 std=std, num_splits=num_splits)
    inp = generate(w)
    if lens is not None:
        inp["kv_lens"] = torch.tensor(lens, dtype=torch.int32)
    return w, inp


def cascade(w: Workload, prefix_len: int, poison_tail: bool = False) -> dict:
    """Shared-prefix inputs: the workload w supplies q and each sequence's
    suffix cache (its K/V and lengths); one prefix cache of prefix_len tokens
    [prefix_len, heads_kv, d], drawn from the same recipe with its own seed,
    is shared by every sequence."""
    inp = generate(w, poison_tail=poison_tail)
    pw = Workload(w.name + f"_prefix{prefix_len}", 1, w.heads_kv, w.heads_kv, w.head_dim,
                  prefix_len, w.dtype, w.out_dtype, seed=w.seed + 100003, std=w.std)
    pre = generate(pw) if prefix_len > 0 else None
    shape = (prefix_len, w.heads_kv, w.head_dim)
    empty = torch.empty(shape, dtype=TORCH_DTYPES[w.dtype])
    return {"q": inp["q"], "k_prefix": pre["k"][0] if pre else empty,
            "v_prefix": pre["v"][0] if pre else empty.clone(), "k_suffix": inp["k"],
            "v_suffix": inp["v"], "suffix_lens": inp["kv_lens"],
            "max_suffix_len": inp["max_kv_len"], "prefix_len": prefix_len}


def cascade_concat(c: dict) -> dict:
    """The cascade's inputs as one cache per sequence: prefix then suffix
    (data movement only), in generate()'s layout, for references."""
    k_pre, v_pre = c["k_prefix"], c["v_prefix"]
    batch, s_max = c["k_suffix"].shape[:2]
    p = c["prefix_len"]
    lens = c["suffix_lens"]
    n = [s_max] * batch if lens is None else [min(max(int(x), 0), s_max) for x in lens]
    k = torch.cat([k_pre.unsqueeze(0).expand(batch, *k_pre.shape), c["k_suffix"]], dim=1)
    v = torch.cat([v_pre.unsqueeze(0).expand(batch, *v_pre.shape), c["v_suffix"]], dim=1)
    return {"q": c["q"], "k": k.contiguous(), "v": v.contiguous(),
            "kv_lens": torch.tensor([p + x for x in n], dtype=torch.int32),
            "max_kv_len": p + s_max}


def paginate(inp: dict, page_size: int, seed: int = 0, spare_pages: int = 3) -> dict:
    """Lay a generated workload's K/V out as a paged cache (data movement only).

    Logical page j of sequence b (tokens [j*page_size, (j+1)*page_size)) goes to
    a physical page drawn from a seeded permutation; only the pages a sequence's
    length needs get one.  Returns k_pages / v_pages [num_pages, page_size,
    heads_kv, d], block_table int32 [batch, max_pages] (entries past a
    sequence's pages are -1, never read), num_pages.  Physical pages nobody
    owns (spare_pages of them, scattered) hold NaN, so a stray read shows.
    """
    k, v, lens = inp["k"], inp["v"], inp["kv_lens"]
    batch, n_max, heads_kv, d = k.shape
    max_pages = max(1, -(-n_max // page_size))
    eff = [n_max] * batch if lens is None else [min(max(int(x), 0), n_max) for x in lens]
    need = [-(-n // page_size) for n in eff]
    num_pages = sum(need) + spare_pages
    perm = torch.randperm(num_pages, generator=_gen(seed, "pages", page_size)).tolist()
    table = torch.full((batch, max_pages), -1, dtype=torch.int32)
    k_pages = torch.full((num_pages, page_size, heads_kv, d), float("nan"), dtype=k.dtype)
    v_pages = torch.full_like(k_pages, float("nan"))
    nxt = 0
    for b in range(batch):
        for j in range(need[b]):
            p = perm[nxt]
            nxt += 1
            table[b, j] = p
            t0, t1 = j * page_size, min((j + 1) * page_size, n_max)
            k_pages[p, : t1 - t0] = k[b, t0:t1]
            v_pages[p, : t1 - t0] = v[b, t0:t1]
    return {"k_pages": k_pages, "v_pages": v_pages, "block_table": table,
            "num_pages": num_pages, "page_size": page_size, "max_pages": max_pages}


def kv_bytes(w: Workload, kv_lens) -> int:
    """Bytes of K and V a decode step must read: sum_b N_b * heads_kv * d * 2 * elem."""
    elem = torch.tensor([], dtype=TORCH_DTYPES[w.dtype]).element_size()
    total_tokens = w.batch * w.max_kv_len if kv_lens is None else int(kv_lens.sum())
    return total_tokens * w.heads_kv * w.head_dim * 2 * elem


def digest(inp: dict) -> dict:
    """SHA-256 (first 16 hex digits) of each generated tensor's bytes, so that
    a run can name exactly which inputs it used."""
    out = {}
    for name in ("q", "k", "v", "kv_lens"):
        t = inp.get(name)
        if t is None:
            continue
        h = hashlib.sha256()
        arr = raw(t) if t.is_floating_point() else t.contiguous().numpy()
        h.update(memoryview(np.ascontiguousarray(arr)).cast("B"))
        out[name] = h.hexdigest()[:16]
    return out


def raw(t: torch.Tensor) -> np.ndarray:
    """Storage bits of a CPU tensor as numpy (uint16 for 16-bit types, float32 for f32)."""
    t = t.contiguous()
    if t.dtype == torch.float32:
        return t.numpy()
    return t.view(torch.int16).numpy().view(np.uint16)


def dtype_name(t: torch.Tensor) -> str:
    return {v: k for k, v in TORCH_DTYPES.items()}[t.dtype]
