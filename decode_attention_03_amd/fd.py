"""Thin Python binding of libfd (include/fd.h) over ctypes.

Argument marshalling only: shapes, dtypes and devices are checked here, device
pointers and torch's current HIP stream are handed to the C ABI, and every step
of the computation runs in the library's HIP kernels.  PyTorch provides device
memory and streams.  A missing or unloadable libfd.so raises; there is no
fallback implementation.

Layouts (see include/fd.h): q [batch, heads_q, d]; K/V [batch, max_kv_len,
heads_kv, d]; kv_lens int32 [batch] on the device (None: all max_kv_len);
o [batch, heads_q, d]; lse float32 [batch, heads_q].
"""
from __future__ import annotations

import contextlib
import ctypes
import json
import math
import os
import threading

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfd.so")
#: written beside libfd.so by the build: the hash of the sources it came from
BUILD_RECORD = os.path.join(_PKG, "libfd.build.json")

F32, F16, BF16 = 0, 1, 2
OK, ERR_INVALID, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, -1, -2, -3, -4
_CODES = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}
_ERR_NAMES = {ERR_INVALID: "FD_ERR_INVALID", ERR_UNSUPPORTED: "FD_ERR_UNSUPPORTED",
              ERR_WORKSPACE: "FD_ERR_WORKSPACE", ERR_HIP: "FD_ERR_HIP"}

#: every symbol include/fd.h declares
EXPORTS = ("fd_version", "fd_last_error", "fd_choose_splits", "fd_workspace_bytes",
           "fd_decode_workspace_bytes", "fd_decode_plan", "fd_decode_split",
           "fd_decode_split_mlo", "fd_combine", "fd_combine_mlo", "fd_decode", "fd_decode_stages",
           "fd_decode_noalloc", "fd_decode_split_paged", "fd_decode_paged",
           "fd_cascade_workspace_bytes", "fd_decode_cascade")

#: fd_decode_stages' stage bits
STAGE_SPLIT, STAGE_COMBINE = 1, 2

#: fd_plan.route and fd_plan.kernel codes, by name
ROUTES = ("direct", "fused", "splits", "balanced")
KERNELS = ("vector", "grouped", "tiled", "balanced")

_lock = threading.Lock()
_lib = None


class _Plan(ctypes.Structure):
    """struct fd_plan of include/fd.h."""
    _fields_ = [("route", ctypes.c_int), ("kernel", ctypes.c_int), ("num_splits", ctypes.c_int),
                ("split_len", ctypes.c_int), ("waves_per_group", ctypes.c_int),
                ("query_tiles", ctypes.c_int), ("launches", ctypes.c_int),
                ("work_groups", ctypes.c_int64), ("workspace_bytes", ctypes.c_size_t)]


class FDError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{_ERR_NAMES.get(code, code)}: {message}")
        self.code = code


def check_fresh(path: str | None = None, record: str | None = None,
                allow_flags: bool = False) -> dict:
    """Raise unless the library at path (default LIB_PATH) was built from the
    sources now in csrc/ and include/ (the build records their hash and its
    extra compiler flags beside it, at BUILD_RECORD), and, unless
    allow_flags, without extra flags.  Returns the record."""
    from decode_attention_03_amd import build

    path = LIB_PATH if path is None else path
    record = BUILD_RECORD if record is None else record
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -c 'import __graft_entry__ as g; g.build()'`")
    try:
        with open(record, encoding="utf-8") as f:
            rec = json.load(f)
    except (OSError, ValueError):
        rec = {}
    built = rec.get("sources_sha256")
    now = build.library_source_hash()
    if built != now or (rec.get("flags") and not allow_flags):
        raise RuntimeError(f"{path} was not built from the current sources (built from "
                           f"{built} with flags {rec.get('flags')}, sources now {now}): "
                           "rebuild it with "
                           "`python -c 'import __graft_entry__ as g; g.build()'`")
    return rec


_variant = None


def use_variant(path: str) -> dict:
    """Load a tuning variant (decode_attention_03_amd/build.py build_variant:
    the library built with extra -D knobs) instead of libfd.so; must come
    before the first library() call.  Returns its build record."""
    global _variant
    if _lib is not None:
        raise RuntimeError("the library is already loaded")
    from decode_attention_03_amd import build

    rec = check_fresh(path, build.record_path(path), allow_flags=True)
    _variant = path
    return rec


def library() -> ctypes.CDLL:
    """Open libfd.so (once).  Raises if it has not been built, or was built
    from other sources than the ones in the tree."""
    global _lib
    if _lib is not None:  # loaded: no lock on the per-call path
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        if _variant is None:
            check_fresh()
        lib = ctypes.CDLL(LIB_PATH if _variant is None else _variant)
        P, I, F, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        IP = ctypes.POINTER(ctypes.c_int)
        lib.fd_version.argtypes, lib.fd_version.restype = [], I
        lib.fd_last_error.argtypes, lib.fd_last_error.restype = [], ctypes.c_char_p
        lib.fd_choose_splits.argtypes = [I, I, I, I, I, I, I, I, IP, IP]
        lib.fd_choose_splits.restype = I
        lib.fd_workspace_bytes.argtypes, lib.fd_workspace_bytes.restype = [I, I, I, I], S
        lib.fd_decode_workspace_bytes.argtypes = [I, I, I, I, I, I, I, I, I, ctypes.POINTER(S)]
        lib.fd_decode_workspace_bytes.restype = I
        lib.fd_decode_plan.argtypes = [I, I, I, I, I, I, I, I, I, I, I, ctypes.POINTER(_Plan)]
        lib.fd_decode_plan.restype = I
        lib.fd_decode_split.argtypes = [P, P, P, P, I, I, I, I, I, I, F, I, I, P, P, P]
        lib.fd_decode_split.restype = I
        lib.fd_decode_split_mlo.argtypes = [P, P, P, P, I, I, I, I, I, I, F, I, I, P, P, P, P]
        lib.fd_decode_split_mlo.restype = I
        lib.fd_combine.argtypes = [P, P, I, I, I, I, P, I, P, P]
        lib.fd_combine.restype = I
        lib.fd_combine_mlo.argtypes = [P, P, P, I, I, I, I, P, I, P, P]
        lib.fd_combine_mlo.restype = I
        lib.fd_decode.argtypes = [P, P, P, P, I, I, I, I, I, I, I, F, I, I, P, P, P, S, P]
        lib.fd_decode.restype = I
        lib.fd_decode_stages.argtypes = [P, P, P, P, I, I, I, I, I, I, I, F, I, I, P, P, P, S, I,
                                         P]
        lib.fd_decode_stages.restype = I
        lib.fd_decode_noalloc.argtypes = [P, P, P, P, I, I, I, I, I, I, I, F, I, I, P, P, P]
        lib.fd_decode_noalloc.restype = I
        lib.fd_decode_split_paged.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, I, F, I, I, P,
                                              P, P]
        lib.fd_decode_split_paged.restype = I
        lib.fd_decode_paged.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, I, I, F, I, I, P, P,
                                        P, S, P]
        lib.fd_decode_paged.restype = I
        lib.fd_cascade_workspace_bytes.argtypes = [I, I, I, I, I, I, I, I, ctypes.POINTER(S)]
        lib.fd_cascade_workspace_bytes.restype = I
        lib.fd_decode_cascade.argtypes = [P, P, P, I, P, P, P, I, I, I, I, I, I, I, F, P, P, P, S,
                                          P]
        lib.fd_decode_cascade.restype = I
        _lib = lib
        return lib


def version() -> int:
    return library().fd_version()


def last_error() -> str:
    return library().fd_last_error().decode()


def _check(rc: int) -> None:
    if rc != OK:
        raise FDError(rc, last_error())


def _code(dtype: torch.dtype) -> int:
    if dtype not in _CODES:
        raise TypeError(f"unsupported dtype {dtype}")
    return _CODES[dtype]


def _ptr(t: torch.Tensor | None):
    # an int (or None) for a c_void_p parameter: ctypes converts it by argtypes
    return None if t is None else t.data_ptr()


# torch's current raw HIP stream of a device, without building a Stream object
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(device: torch.device):
    if _raw_stream is not None and device.index is not None:
        return _raw_stream(device.index)
    return torch.cuda.current_stream(device).cuda_stream


def _on(device: torch.device):
    """Make device current for the launches (and the plan, which depends on its
    compute units); no switch when it already is."""
    if device.index is None or device.index == torch.cuda.current_device():
        return contextlib.nullcontext()
    return torch.cuda.device(device)


#: fd_decode_workspace_bytes results by (device, arguments): the plan depends
#: only on them and on the device's compute-unit count
_ws_cache: dict = {}


def _on_device(name: str, t: torch.Tensor, device: torch.device) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _buffer(name: str, t: torch.Tensor, device: torch.device, shape: tuple,
            dtype: torch.dtype) -> None:
    """A caller-supplied output buffer: on the device, contiguous, exactly
    this shape and dtype (the kernels write all of it by raw pointer)."""
    _on_device(name, t, device)
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} {tuple(shape)}, got {t.dtype} "
                         f"{tuple(t.shape)}")


def _outputs(o, lse, return_lse: bool, shape: tuple, out_dtype, dev):
    """o [batch, heads_q, d] in out_dtype and lse [batch, heads_q] float32:
    allocated when not given, else checked."""
    if out_dtype not in _CODES:
        raise TypeError(f"unsupported output dtype {out_dtype}")
    if o is None:
        o = torch.empty(shape, dtype=out_dtype, device=dev)
    else:
        _buffer("o", o, dev, shape, out_dtype)
    if lse is None and return_lse:
        lse = torch.empty(shape[:2], dtype=torch.float32, device=dev)
    elif lse is not None:
        _buffer("lse", lse, dev, shape[:2], torch.float32)
    return o, lse


def _workspace(workspace, need: int, dev):
    """The caller's workspace (any dtype; on the device and contiguous), or a
    new one of `need` bytes; returns (tensor or None, its size in bytes)."""
    if workspace is None:
        if not need:
            return None, 0
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _on_device("workspace", workspace, dev)
    return workspace, workspace.numel() * workspace.element_size()


def _shapes(q, k, v, kv_lens):
    if q.dim() != 3 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("expected q [batch, heads_q, d] and K/V [batch, N, heads_kv, d]")
    batch, heads_q, d = q.shape
    kb, n_max, heads_kv, kd = k.shape
    if kb != batch or kd != d:
        raise ValueError(f"q {tuple(q.shape)} and K {tuple(k.shape)} disagree")
    if q.dtype != k.dtype or v.dtype != k.dtype:
        raise TypeError("q, K and V must share one dtype")
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a HIP device")
    for name, t in (("q", q), ("k", k), ("v", v)):
        _on_device(name, t, dev)
    if kv_lens is not None:
        _on_device("kv_lens", kv_lens, dev)
        if kv_lens.dtype != torch.int32 or kv_lens.shape != (batch,):
            raise ValueError("kv_lens must be int32 [batch]")
    return batch, heads_q, heads_kv, n_max, d


def choose_splits(batch: int, heads_q: int, heads_kv: int, max_kv_len: int, head_dim: int,
                  dtype: torch.dtype, ragged: bool = False, num_cus: int = 0) -> tuple[int, int]:
    """(num_splits, split_len) from the library heuristic (num_cus 0: the device's)."""
    b, length = ctypes.c_int(), ctypes.c_int()
    _check(library().fd_choose_splits(batch, heads_q, heads_kv, max_kv_len, head_dim,
                                      _code(dtype), int(bool(ragged)), num_cus, ctypes.byref(b),
                                      ctypes.byref(length)))
    return b.value, length.value


def workspace_bytes(batch: int, heads_q: int, num_splits: int, head_dim: int) -> int:
    return int(library().fd_workspace_bytes(batch, heads_q, num_splits, head_dim))


def decode_workspace_bytes(batch: int, heads_q: int, heads_kv: int, max_kv_len: int,
                           head_dim: int, dtype: torch.dtype, has_kv_lens: bool,
                           num_splits: int = 0, split_len: int = 0) -> int:
    """Workspace fd_decode needs for exactly these arguments (num_splits 0: the
    library's automatic plan)."""
    out = ctypes.c_size_t()
    _check(library().fd_decode_workspace_bytes(batch, heads_q, heads_kv, max_kv_len, head_dim,
                                               _code(dtype), int(bool(has_kv_lens)), num_splits,
                                               split_len, ctypes.byref(out)))
    return out.value


def decode_plan(batch: int, heads_q: int, heads_kv: int, max_kv_len: int, head_dim: int,
                dtype: torch.dtype, has_kv_lens: bool, num_splits: int = 0, split_len: int = 0,
                paged: bool = False, num_cus: int = 0) -> dict:
    """What fd_decode (paged: fd_decode_paged) launches for these arguments:
    route and kernel by name, B and L, waves and query tiles per work-group,
    launches, split-kernel work-groups and workspace bytes.  num_cus 0: the
    current device's compute units; > 0: plan for that many without a GPU."""
    p = _Plan()
    _check(library().fd_decode_plan(batch, heads_q, heads_kv, max_kv_len, head_dim, _code(dtype),
                                     int(bool(has_kv_lens)), int(bool(paged)), num_splits,
                                     split_len, num_cus, ctypes.byref(p)))
    return {"route": ROUTES[p.route], "kernel": KERNELS[p.kernel], "num_splits": p.num_splits,
            "split_len": p.split_len, "waves_per_group": p.waves_per_group,
            "query_tiles": p.query_tiles, "launches": p.launches, "work_groups": p.work_groups,
            "workspace_bytes": p.workspace_bytes}


def _parts(names_shapes, given: dict, dev) -> list:
    """Partial buffers (float32): allocated when not given, else checked."""
    out = []
    for name, shape in names_shapes:
        t = given.get(name)
        if t is None:
            t = torch.empty(shape, dtype=torch.float32, device=dev)
        else:
            _buffer(name, t, dev, shape, torch.float32)
        out.append(t)
    return out


def _splits(num_splits: int) -> int:
    num_splits = int(num_splits)
    if num_splits < 1:
        raise ValueError(f"num_splits must be >= 1, got {num_splits}")
    return num_splits


def decode_split(q, k, v, kv_lens=None, *, num_splits: int, split_len: int = 0, scale=None,
                 o_part=None, lse_part=None):
    """Split stage: returns (o_part [batch, Hq, B, d] f32, lse_part [batch, Hq, B] f32).
    split_len 0: the library's ceil(N / num_splits)."""
    batch, heads_q, heads_kv, n_max, d = _shapes(q, k, v, kv_lens)
    B = _splits(num_splits)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o_part, lse_part = _parts((("o_part", (batch, heads_q, B, d)),
                               ("lse_part", (batch, heads_q, B))),
                              {"o_part": o_part, "lse_part": lse_part}, q.device)
    with _on(q.device):  # launches go to the current device
        _check(library().fd_decode_split(_ptr(q), _ptr(k), _ptr(v), _ptr(kv_lens), batch,
                                         heads_q, heads_kv, n_max, d, _code(q.dtype), scale,
                                         B, int(split_len), _ptr(o_part), _ptr(lse_part),
                                         _stream(q.device)))
    return o_part, lse_part


def decode_split_mlo(q, k, v, kv_lens=None, *, num_splits: int, split_len: int = 0, scale=None,
                     o_part=None, m_part=None, l_part=None):
    """Split stage, m/l/o format: returns (o_part [batch, Hq, B, d], m_part
    [batch, Hq, B], l_part [batch, Hq, B]), all float32."""
    batch, heads_q, heads_kv, n_max, d = _shapes(q, k, v, kv_lens)
    B = _splits(num_splits)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    shape = (batch, heads_q, B)
    o_part, m_part, l_part = _parts((("o_part", (*shape, d)), ("m_part", shape),
                                     ("l_part", shape)),
                                    {"o_part": o_part, "m_part": m_part, "l_part": l_part},
                                    q.device)
    with _on(q.device):  # launches go to the current device
        _check(library().fd_decode_split_mlo(_ptr(q), _ptr(k), _ptr(v), _ptr(kv_lens), batch,
                                             heads_q, heads_kv, n_max, d, _code(q.dtype), scale,
                                             B, int(split_len), _ptr(o_part), _ptr(m_part),
                                             _ptr(l_part), _stream(q.device)))
    return o_part, m_part, l_part


def _partials_in(o_part, scalars: dict):
    """Checks the inputs of a combine: o_part float32 [batch, Hq, B, d] and
    each per-split scalar float32 [batch, Hq, B], all on one HIP device."""
    if not isinstance(o_part, torch.Tensor) or o_part.dim() != 4 or o_part.dtype != torch.float32:
        raise ValueError("o_part must be float32 [batch, Hq, B, d]")
    batch, heads_q, nb, d = o_part.shape
    dev = o_part.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a HIP device")
    _on_device("o_part", o_part, dev)
    for name, t in scalars.items():
        _buffer(name, t, dev, (batch, heads_q, nb), torch.float32)
    return batch, heads_q, nb, d, dev


def combine_mlo(o_part, m_part, l_part, out_dtype=None, o=None, lse=None, return_lse=True):
    """Combine stage, m/l/o format -> (o, lse)."""
    batch, heads_q, nb, d, dev = _partials_in(o_part, {"m_part": m_part, "l_part": l_part})
    o, lse = _outputs(o, lse, return_lse, (batch, heads_q, d),
                      out_dtype or (o.dtype if o is not None else torch.float32), dev)
    with _on(dev):  # launches go to the current device
        _check(library().fd_combine_mlo(_ptr(o_part), _ptr(m_part), _ptr(l_part), batch,
                                        heads_q, nb, d, _ptr(o), _code(o.dtype), _ptr(lse),
                                        _stream(dev)))
    return o, lse


def combine(o_part, lse_part, out_dtype=None, o=None, lse=None, return_lse=True):
    """Combine stage: LSE merge over the split axis -> (o, lse)."""
    batch, heads_q, nb, d, dev = _partials_in(o_part, {"lse_part": lse_part})
    o, lse = _outputs(o, lse, return_lse, (batch, heads_q, d),
                      out_dtype or (o.dtype if o is not None else torch.float32), dev)
    with _on(dev):  # launches go to the current device
        _check(library().fd_combine(_ptr(o_part), _ptr(lse_part), batch, heads_q, nb, d, _ptr(o),
                                    _code(o.dtype), _ptr(lse), _stream(dev)))
    return o, lse


def decode(q, k, v, kv_lens=None, *, scale=None, num_splits: int = 0, split_len: int = 0,
           out_dtype=None, return_lse: bool = True, workspace=None, o=None, lse=None,
           stages: int = STAGE_SPLIT | STAGE_COMBINE):
    """Whole decode step (split + combine) -> (o, lse or None).

    num_splits 0 lets the library plan the partition (fixed splits from
    fd_choose_splits, or the token-balanced partition for ragged grouped-head
    batches).  workspace (any dtype, on the device) is allocated here when not
    given and the plan needs one.  stages other than both bits calls
    fd_decode_stages: the split launch alone (STAGE_SPLIT) or the combine
    launch alone (STAGE_COMBINE, after a split call with the same arguments
    and workspace).
    """
    batch, heads_q, heads_kv, n_max, d = _shapes(q, k, v, kv_lens)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dev = q.device
    o, lse = _outputs(o, lse, return_lse, (batch, heads_q, d),
                      out_dtype or (o.dtype if o is not None else q.dtype), dev)
    key = (dev.index, batch, heads_q, heads_kv, n_max, d, q.dtype, kv_lens is not None,
           num_splits, split_len)
    need = _ws_cache.get(key)
    if need is None:
        with _on(dev):  # the plan depends on this device's compute units
            need = decode_workspace_bytes(batch, heads_q, heads_kv, n_max, d, q.dtype,
                                          kv_lens is not None, num_splits, split_len)
        if len(_ws_cache) > 4096:
            _ws_cache.clear()
        _ws_cache[key] = need
    workspace, ws_bytes = _workspace(workspace, need, dev)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(kv_lens), batch, heads_q, heads_kv, n_max, d,
            _code(q.dtype), _code(o.dtype), scale, num_splits, split_len, _ptr(o), _ptr(lse),
            _ptr(workspace), ws_bytes)
    with _on(dev):  # launches go to the current device
        if stages == STAGE_SPLIT | STAGE_COMBINE:
            _check(library().fd_decode(*args, _stream(dev)))
        else:
            _check(library().fd_decode_stages(*args, int(stages), _stream(dev)))
    return o, lse


def decode_noalloc(q, k, v, kv_lens=None, *, scale=None, num_splits: int = 0,
                   split_len: int = 0, out_dtype=None, return_lse: bool = True, o=None,
                   lse=None):
    """decode() through fd_decode_noalloc: the partials go to the library's own
    32 MiB scratch per GPU instead of a workspace (nothing is allocated by the
    library; o and lse are allocated here unless given).  Calls that overlap
    on one GPU race on that scratch."""
    batch, heads_q, heads_kv, n_max, d = _shapes(q, k, v, kv_lens)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dev = q.device
    o, lse = _outputs(o, lse, return_lse, (batch, heads_q, d),
                      out_dtype or (o.dtype if o is not None else q.dtype), dev)
    with _on(dev):  # launches go to the current device
        _check(library().fd_decode_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(kv_lens), batch,
                                           heads_q, heads_kv, n_max, d, _code(q.dtype),
                                           _code(o.dtype), scale, num_splits, split_len, _ptr(o),
                                           _ptr(lse), _stream(dev)))
    return o, lse


def _paged_shapes(q, k_pages, v_pages, block_table, kv_lens):
    if q.dim() != 3 or k_pages.dim() != 4 or v_pages.shape != k_pages.shape:
        raise ValueError("expected q [batch, heads_q, d] and K/V pages "
                         "[num_pages, page_size, heads_kv, d]")
    batch, heads_q, d = q.shape
    num_pages, page_size, heads_kv, kd = k_pages.shape
    if kd != d:
        raise ValueError(f"q {tuple(q.shape)} and K pages {tuple(k_pages.shape)} disagree")
    if q.dtype != k_pages.dtype or v_pages.dtype != k_pages.dtype:
        raise TypeError("q, K and V must share one dtype")
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a HIP device")
    for name, t in (("q", q), ("k_pages", k_pages), ("v_pages", v_pages),
                    ("block_table", block_table)):
        _on_device(name, t, dev)
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != batch:
        raise ValueError("block_table must be int32 [batch, max_pages_per_seq]")
    if kv_lens is not None:
        _on_device("kv_lens", kv_lens, dev)
        if kv_lens.dtype != torch.int32 or kv_lens.shape != (batch,):
            raise ValueError("kv_lens must be int32 [batch]")
    return batch, heads_q, heads_kv, page_size, block_table.shape[1], num_pages, d


def decode_split_paged(q, k_pages, v_pages, block_table, kv_lens=None, *, num_splits: int,
                       split_len: int = 0, scale=None, o_part=None, lse_part=None):
    """Split stage over a paged K/V cache -> (o_part, lse_part), as decode_split
    (split_len 0: the library's ceil(N / num_splits) in whole 16-token tiles)."""
    batch, heads_q, heads_kv, ps, max_pages, num_pages, d = _paged_shapes(
        q, k_pages, v_pages, block_table, kv_lens)
    B = _splits(num_splits)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o_part, lse_part = _parts((("o_part", (batch, heads_q, B, d)),
                               ("lse_part", (batch, heads_q, B))),
                              {"o_part": o_part, "lse_part": lse_part}, q.device)
    with _on(q.device):  # launches go to the current device
        _check(library().fd_decode_split_paged(
            _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table), _ptr(kv_lens), batch, heads_q,
            heads_kv, ps, max_pages, num_pages, d, _code(q.dtype), scale, B, int(split_len),
            _ptr(o_part), _ptr(lse_part), _stream(q.device)))
    return o_part, lse_part


def decode_paged(q, k_pages, v_pages, block_table, kv_lens=None, *, scale=None,
                 num_splits: int = 0, split_len: int = 0, out_dtype=None,
                 return_lse: bool = True, workspace=None, o=None, lse=None):
    """Whole decode step over a paged K/V cache -> (o, lse or None), as decode."""
    batch, heads_q, heads_kv, ps, max_pages, num_pages, d = _paged_shapes(
        q, k_pages, v_pages, block_table, kv_lens)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dev = q.device
    o, lse = _outputs(o, lse, return_lse, (batch, heads_q, d),
                      out_dtype or (o.dtype if o is not None else q.dtype), dev)
    with _on(dev):  # the plan depends on this device's compute units
        need = decode_workspace_bytes(batch, heads_q, heads_kv, max_pages * ps, d, q.dtype,
                                      kv_lens is not None, num_splits, split_len)
    workspace, ws_bytes = _workspace(workspace, need, dev)
    with _on(dev):  # launches go to the current device
        _check(library().fd_decode_paged(
            _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table), _ptr(kv_lens), batch,
            heads_q, heads_kv, ps, max_pages, num_pages, d, _code(q.dtype), _code(o.dtype), scale,
            num_splits, split_len, _ptr(o), _ptr(lse), _ptr(workspace), ws_bytes, _stream(dev)))
    return o, lse


def cascade_workspace_bytes(batch: int, heads_q: int, heads_kv: int, prefix_len: int,
                            max_suffix_len: int, head_dim: int, dtype: torch.dtype,
                            has_suffix_lens: bool) -> int:
    out = ctypes.c_size_t()
    _check(library().fd_cascade_workspace_bytes(batch, heads_q, heads_kv, prefix_len,
                                                max_suffix_len, head_dim, _code(dtype),
                                                int(bool(has_suffix_lens)), ctypes.byref(out)))
    return out.value


def decode_cascade(q, k_prefix, v_prefix, k_suffix, v_suffix, suffix_lens=None, *, scale=None,
                   out_dtype=None, return_lse: bool = True, workspace=None, o=None, lse=None):
    """Shared-prefix decode -> (o, lse or None).

    k_prefix / v_prefix [prefix_len, heads_kv, d] (one copy for the batch),
    k_suffix / v_suffix [batch, max_suffix_len, heads_kv, d], suffix_lens int32
    [batch] or None.  Equals decode() over each sequence's prefix + suffix.
    """
    if q.dim() != 3 or k_prefix.dim() != 3 or k_suffix.dim() != 4:
        raise ValueError("expected q [batch, Hq, d], prefix [P, Hkv, d], suffix [batch, S, Hkv, d]")
    if v_prefix.shape != k_prefix.shape or v_suffix.shape != k_suffix.shape:
        raise ValueError("K and V shapes differ")
    batch, heads_q, d = q.shape
    prefix_len, heads_kv, pd = k_prefix.shape
    sb, max_suffix_len, sh, sd = k_suffix.shape
    if sb != batch or sh != heads_kv or pd != d or sd != d:
        raise ValueError("q, prefix and suffix shapes disagree")
    if any(t.dtype != q.dtype for t in (k_prefix, v_prefix, k_suffix, v_suffix)):
        raise TypeError("q, K and V must share one dtype")
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a HIP device")
    for name, t in (("q", q), ("k_prefix", k_prefix), ("v_prefix", v_prefix),
                    ("k_suffix", k_suffix), ("v_suffix", v_suffix)):
        _on_device(name, t, dev)
    if suffix_lens is not None:
        _on_device("suffix_lens", suffix_lens, dev)
        if suffix_lens.dtype != torch.int32 or suffix_lens.shape != (batch,):
            raise ValueError("suffix_lens must be int32 [batch]")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o, lse = _outputs(o, lse, return_lse, (batch, heads_q, d),
                      out_dtype or (o.dtype if o is not None else q.dtype), dev)
    with _on(dev):  # the plan depends on this device's compute units
        need = cascade_workspace_bytes(batch, heads_q, heads_kv, prefix_len, max_suffix_len, d,
                                       q.dtype, suffix_lens is not None)
    workspace, ws_bytes = _workspace(workspace, max(need, 16), dev)
    with _on(dev):  # launches go to the current device
        _check(library().fd_decode_cascade(
            _ptr(q), _ptr(k_prefix), _ptr(v_prefix), prefix_len, _ptr(k_suffix), _ptr(v_suffix),
            _ptr(suffix_lens), batch, heads_q, heads_kv, max_suffix_len, d, _code(q.dtype),
            _code(o.dtype), scale, _ptr(o), _ptr(lse), _ptr(workspace), ws_bytes, _stream(dev)))
    return o, lse
