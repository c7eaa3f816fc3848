"""Python binding of libmkv: mixed FP8/TQ3 paged decode attention on MI355X.

Argument marshalling only.  Every operation runs in the HIP library
(libmkv.so, built in-tree by ``python -m decode_attention_mixed_amd.build``);
there is no Python or CPU fallback, and loading fails loudly when the library
is missing.  Tensors are torch tensors on the pool's device; streams default
to torch's current stream.

Function names match the C-ABI in include/mkv.h without the ``mkv_`` prefix:
pool_bytes, record_bytes, pool_create, pool_destroy, seq_reset, append,
demote, decode, seq_info, page_table, pool_stats, debug_gather,
debug_schedule, profile_enable, profile_read, status_string, last_error.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmkv.so")

FMT_FP8 = 0
FMT_TQ3 = 1
FMT_BF16 = 2
KIND_MIXED = 0
KIND_BF16 = 1

OK, EINVAL, ENOMEM, ESTATE, ERANGE, EHIP = 0, -1, -2, -3, -4, -5


class MkvError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


class PoolDesc(ctypes.Structure):
    _fields_ = [
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_seqs", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
        ("max_batch", ctypes.c_int32),
        ("max_q_heads", ctypes.c_int32),
        ("max_chunks", ctypes.c_int32),
        ("fp8_pages", ctypes.c_int64),
        ("tq3_pages", ctypes.c_int64),
        ("placement_seed", ctypes.c_uint64),
        ("kv_kind", ctypes.c_int32),
    ]


class Stats(ctypes.Structure):
    _fields_ = [
        ("live_tokens", ctypes.c_int64),
        ("fp8_pages_live", ctypes.c_int64),
        ("tq3_pages_live", ctypes.c_int64),
        ("fp8_pages_free", ctypes.c_int64),
        ("tq3_pages_free", ctypes.c_int64),
        ("kv_bytes", ctypes.c_int64),
        ("bytes_per_token", ctypes.c_double),
        ("ratio_vs_bf16", ctypes.c_double),
        ("ratio_vs_fp8", ctypes.c_double),
        ("dense_shadow_bytes", ctypes.c_int64),
        ("dense_fallbacks", ctypes.c_int64),
    ]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


class Profile(ctypes.Structure):
    _fields_ = [
        ("ms_partial", ctypes.c_double),
        ("ms_merge", ctypes.c_double),
        ("n_partial", ctypes.c_int64),
        ("n_merge", ctypes.c_int64),
        ("ms_append", ctypes.c_double),
        ("ms_demote", ctypes.c_double),
        ("n_append", ctypes.c_int64),
        ("n_demote", ctypes.c_int64),
    ]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


class ScheduleInfo(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("n_items", ctypes.c_int32),
        ("n_list", ctypes.c_int32),
        ("n_chunks", ctypes.c_int32),
        ("max_seq_chunks", ctypes.c_int32),
        ("heads_per_wave", ctypes.c_int32),
        ("resident_waves", ctypes.c_int32),
        ("pad0", ctypes.c_int32),
    ]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_ if f != "pad0"}


EXPORTED = [
    "mkv_pool_bytes", "mkv_record_bytes", "mkv_pool_create", "mkv_pool_destroy",
    "mkv_seq_reset", "mkv_append", "mkv_append_step", "mkv_demote", "mkv_materialize",
    "mkv_decode", "mkv_decode_static", "mkv_decode_step", "mkv_set_anchor_window", "mkv_protect_pages",
    "mkv_seq_info",
    "mkv_page_table", "mkv_pool_stats", "mkv_debug_gather", "mkv_debug_schedule", "mkv_debug_read_bandwidth", "mkv_profile_enable",
    "mkv_profile_read", "mkv_status_string", "mkv_last_error",
]

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m decode_attention_mixed_amd.build` (no CPU fallback exists)")
    import torch  # noqa: F401  -- load torch's HIP runtime first so libmkv shares it
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ, F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    sig = {
        "mkv_pool_bytes": (SZ, [ctypes.POINTER(PoolDesc)]),
        "mkv_record_bytes": (SZ, [ctypes.POINTER(PoolDesc), I32]),
        "mkv_pool_create": (I32, [ctypes.POINTER(PoolDesc), P, SZ, ctypes.POINTER(P)]),
        "mkv_pool_destroy": (I32, [P]),
        "mkv_seq_reset": (I32, [P, I32, P]),
        "mkv_append": (I32, [P, I32, I32, P, P, P]),
        "mkv_demote": (I32, [P, I32, P, I32, P]),
        "mkv_materialize": (I32, [P, I32, P, I32, P]),
        "mkv_append_step": (I32, [P, P, I32, P, P, P]),
        "mkv_decode": (I32, [P, P, I32, P, I32, F32, P, P, P]),
        "mkv_decode_static": (I32, [P, P, I32, P, I32, F32, P, P, P]),
        "mkv_decode_step": (I32, [P, P, I32, P, P, P, I32, F32, P, P, P]),
        "mkv_set_anchor_window": (I32, [P, I32]),
        "mkv_protect_pages": (I32, [P, I32, P, I32, I32]),
        "mkv_seq_info": (I32, [P, I32, ctypes.POINTER(I32), ctypes.POINTER(I32)]),
        "mkv_page_table": (I32, [P, I32, P, I32]),
        "mkv_pool_stats": (I32, [P, ctypes.POINTER(Stats)]),
        "mkv_debug_gather": (I32, [P, I32, I32, I32, P, P]),
        "mkv_debug_schedule": (I32, [P, ctypes.POINTER(ScheduleInfo), P, I32, P, I32, P, I32]),
        "mkv_debug_read_bandwidth": (I32, [P, SZ, P, P]),
        "mkv_profile_enable": (I32, [P, I32]),
        "mkv_profile_read": (I32, [P, ctypes.POINTER(Profile)]),
        "mkv_status_string": (ctypes.c_char_p, [I32]),
        "mkv_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _check(status: int):
    if status != OK:
        lib = _load()
        raise MkvError(status, f"{lib.mkv_status_string(status).decode()}: "
                               f"{lib.mkv_last_error().decode()}")


def _stream(stream):
    import torch
    if stream is None:
        # the raw handle of the current stream, without building a Stream
        # object (that costs a few microseconds per call)
        raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        if raw is not None:
            return ctypes.c_void_p(raw(torch.cuda.current_device()))
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dev_ptr(t, dtype=None, shape=None, name="tensor"):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _i32_array(values):
    vals = [int(x) for x in values]
    return (ctypes.c_int32 * max(1, len(vals)))(*vals), len(vals)


# ----------------------------------------------------------------- functions
def make_desc(*, num_kv_heads, head_dim, page_size, max_seqs, max_pages_per_seq, max_batch,
              max_q_heads, fp8_pages, tq3_pages, placement_seed=0, max_chunks=0,
              kv_kind=KIND_MIXED) -> PoolDesc:
    return PoolDesc(num_kv_heads, head_dim, page_size, max_seqs, max_pages_per_seq, max_batch,
                    max_q_heads, max_chunks, fp8_pages, tq3_pages, placement_seed, kv_kind)


def pool_bytes(desc: PoolDesc) -> int:
    return int(_load().mkv_pool_bytes(ctypes.byref(desc)))


def record_bytes(desc: PoolDesc, fmt: int) -> int:
    return int(_load().mkv_record_bytes(ctypes.byref(desc), fmt))


# (Hkv, d) of each live pool, keyed by handle value: the shape checks below
_POOL_GEOM: dict = {}


def _geom(pool):
    key = pool.value if isinstance(pool, ctypes.c_void_p) else int(pool)
    g = _POOL_GEOM.get(key)
    if g is None:
        raise ValueError("unknown pool handle (not created by pool_create, or destroyed)")
    return g


def _check_rows(name, t, lead, pool):
    """t must be [lead][Hkv][d] for the pool's geometry (lead=None: any)."""
    Hkv, d = _geom(pool)
    if t.dim() != 3 or tuple(t.shape[1:]) != (Hkv, d) or (lead is not None and t.shape[0] != lead):
        want = f"[{'n' if lead is None else lead}][{Hkv}][{d}]"
        raise ValueError(f"{name} must be {want}, got {tuple(t.shape)}")


def pool_create(desc: PoolDesc, device_mem=None):
    """Create a pool.  device_mem: None (library allocates) or a torch uint8
    device tensor of at least pool_bytes(desc) bytes that outlives the pool."""
    lib = _load()
    out = ctypes.c_void_p()
    if device_mem is None:
        _check(lib.mkv_pool_create(ctypes.byref(desc), None, 0, ctypes.byref(out)))
    else:
        ptr = _dev_ptr(device_mem, name="device_mem")
        nbytes = device_mem.numel() * device_mem.element_size()
        _check(lib.mkv_pool_create(ctypes.byref(desc), ptr, nbytes, ctypes.byref(out)))
    _POOL_GEOM[out.value] = (int(desc.num_kv_heads), int(desc.head_dim))
    return out


def pool_destroy(pool) -> None:
    _check(_load().mkv_pool_destroy(pool))
    _POOL_GEOM.pop(pool.value if isinstance(pool, ctypes.c_void_p) else int(pool), None)


def seq_reset(pool, seq: int, stream=None) -> None:
    _check(_load().mkv_seq_reset(pool, seq, _stream(stream)))


def append(pool, seq: int, k, v, stream=None) -> None:
    """Append fp32 rows k, v [n][Hkv][d] (device) to sequence seq as FP8."""
    import torch
    _check_rows("k", k, None, pool)
    n = k.shape[0]
    _check(_load().mkv_append(pool, seq, n, _dev_ptr(k, torch.float32, name="k"),
                              _dev_ptr(v, torch.float32, tuple(k.shape), name="v"),
                              _stream(stream)))


def demote(pool, seq: int, logical_pages, stream=None) -> None:
    arr, n = _i32_array(logical_pages)
    _check(_load().mkv_demote(pool, seq, arr, n, _stream(stream)))


def append_step(pool, seq_ids, k, v, stream=None) -> None:
    """One token per sequence: k, v fp32 device [B][Hkv][d], row b to seq_ids[b]."""
    import torch
    ids, B = _i32_array(seq_ids)
    _check_rows("k", k, B, pool)
    _check(_load().mkv_append_step(pool, ids, B, _dev_ptr(k, torch.float32, name="k"),
                                   _dev_ptr(v, torch.float32, tuple(k.shape), name="v"),
                                   _stream(stream)))


def materialize(src_pool, src_seq: int, dst_pool, dst_seq: int, stream=None) -> None:
    """Materialising profile: expand sequence src_seq of a mixed pool into the
    empty sequence dst_seq of a BF16 control pool (a diagnostic)."""
    _check(_load().mkv_materialize(src_pool, src_seq, dst_pool, dst_seq, _stream(stream)))


def _decode(fn, pool, seq_ids, q, softmax_scale, out, lse, stream):
    import torch
    ids, B = _i32_array(seq_ids)
    d = _geom(pool)[1]
    if q.dim() != 3 or q.shape[0] != B or q.shape[2] != d:
        raise ValueError(f"q must be [B][Hq][{d}] with B = len(seq_ids) = {B}, got {tuple(q.shape)}")
    Hq = q.shape[1]
    _check(fn(pool, ids, B, _dev_ptr(q, torch.bfloat16, name="q"), Hq,
              ctypes.c_float(softmax_scale),
              _dev_ptr(out, torch.float32, tuple(q.shape), name="out"),
              _dev_ptr(lse, torch.float32, tuple(q.shape[:2]), name="lse"),
              _stream(stream)))


def decode(pool, seq_ids, q, softmax_scale: float, out, lse, stream=None) -> None:
    """q: bf16 [B][Hq][d]; out: fp32 [B][Hq][d]; lse: fp32 [B][Hq] (all device)."""
    _decode(_load().mkv_decode, pool, seq_ids, q, softmax_scale, out, lse, stream)


def decode_step(pool, seq_ids, k, v, q, softmax_scale: float, out, lse, stream=None) -> None:
    """One decode-loop step: append k, v (fp32 device [B][Hkv][d], row b to
    seq_ids[b]), apply the anchor policy (set_anchor_window), decode q into
    out, lse (as decode)."""
    import torch
    ids, B = _i32_array(seq_ids)
    _check_rows("k", k, B, pool)
    d = _geom(pool)[1]
    if q.dim() != 3 or q.shape[0] != B or q.shape[2] != d:
        raise ValueError(f"q must be [B][Hq][{d}] with B = len(seq_ids) = {B}, got {tuple(q.shape)}")
    _check(_load().mkv_decode_step(pool, ids, B, _dev_ptr(k, torch.float32, name="k"),
                                   _dev_ptr(v, torch.float32, tuple(k.shape), name="v"),
                                   _dev_ptr(q, torch.bfloat16, name="q"), q.shape[1],
                                   ctypes.c_float(softmax_scale),
                                   _dev_ptr(out, torch.float32, tuple(q.shape), name="out"),
                                   _dev_ptr(lse, torch.float32, tuple(q.shape[:2]), name="lse"),
                                   _stream(stream)))


def set_anchor_window(pool, window_tokens: int) -> None:
    """Anchor policy of decode_step: pages wholly older than the last
    window_tokens tokens and not protected are converted to TQ3 (< 0: off)."""
    _check(_load().mkv_set_anchor_window(pool, int(window_tokens)))


def protect_pages(pool, seq: int, lps, on: bool = True) -> None:
    """Mark (on) or clear logical pages of seq as protected from the anchor policy."""
    arr, n = _i32_array(lps)
    _check(_load().mkv_protect_pages(pool, seq, arr, n, 1 if on else 0))


def decode_static(pool, seq_ids, q, softmax_scale: float, out, lse, stream=None) -> None:
    """decode() with the partial states in the library's fixed per-GPU
    workspace: allocates no device memory (calls on one GPU must not overlap)."""
    _decode(_load().mkv_decode_static, pool, seq_ids, q, softmax_scale, out, lse, stream)


def seq_info(pool, seq: int):
    n = ctypes.c_int32()
    p = ctypes.c_int32()
    _check(_load().mkv_seq_info(pool, seq, ctypes.byref(n), ctypes.byref(p)))
    return n.value, p.value


def page_table(pool, seq: int):
    import numpy as np
    _, n_pages = seq_info(pool, seq)
    buf = np.zeros(max(1, n_pages), dtype=np.int32)
    _check(_load().mkv_page_table(pool, seq, buf.ctypes.data_as(ctypes.c_void_p), buf.size))
    return buf[:n_pages]


def pool_stats(pool) -> dict:
    st = Stats()
    _check(_load().mkv_pool_stats(pool, ctypes.byref(st)))
    return st.as_dict()


def debug_gather(pool, seq: int, first: int, n: int, dst, stream=None) -> None:
    """dst: uint8 device tensor of n * max(record bytes) bytes."""
    _check(_load().mkv_debug_gather(pool, seq, first, n, _dev_ptr(dst, name="dst"),
                                    _stream(stream)))


def debug_schedule(pool, arrays: bool = True):
    """The device's copy of the cached decode schedule (synchronous): a dict of
    counts, plus (arrays=True) items int32 [n][8], entries int32 [n_list] and
    chunk_base int32 [B + 1] as numpy arrays."""
    import numpy as np
    lib = _load()
    info = ScheduleInfo()
    _check(lib.mkv_debug_schedule(pool, ctypes.byref(info), None, 0, None, 0, None, 0))
    out = info.as_dict()
    if arrays:
        items = np.zeros((max(1, info.n_items), 8), np.int32)
        ent = np.zeros(max(1, info.n_list), np.int32)
        base = np.zeros(info.batch + 1, np.int32)
        _check(lib.mkv_debug_schedule(pool, ctypes.byref(info), items.ctypes.data_as(ctypes.c_void_p),
                                      items.shape[0], ent.ctypes.data_as(ctypes.c_void_p), ent.size,
                                      base.ctypes.data_as(ctypes.c_void_p), base.size))
        out.update(items=items[:info.n_items], entries=ent[:info.n_list], chunk_base=base)
    return out


def debug_read_bandwidth(src, sink, stream=None) -> None:
    """Read every byte of the device tensor src once (read-ceiling calibration);
    sink: int32/uint32 device tensor of 256 elements."""
    nbytes = src.numel() * src.element_size()
    _check(_load().mkv_debug_read_bandwidth(_dev_ptr(src, name="src"), nbytes,
                                            _dev_ptr(sink, name="sink"), _stream(stream)))


def profile_enable(pool, on: bool) -> None:
    _check(_load().mkv_profile_enable(pool, 1 if on else 0))


def profile_read(pool) -> dict:
    pr = Profile()
    _check(_load().mkv_profile_read(pool, ctypes.byref(pr)))
    return pr.as_dict()


def status_string(status: int) -> str:
    return _load().mkv_status_string(status).decode()


def last_error() -> str:
    return _load().mkv_last_error().decode()
