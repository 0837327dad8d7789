"""Python binding of libpkv — paged KV-cache decode attention on MI355X (gfx950).

Argument marshalling only: every function below has the name of the C entry
point it calls (``include/pkv.h``), converts torch tensors to device pointers
and streams to ``hipStream_t`` handles, and raises :class:`PkvError` when the
call returns a non-zero status.  All computation happens in the HIP library;
if ``libpkv.so`` is missing, importing this package raises.

torch is imported first so that the library binds to the HIP runtime torch
already loaded (one runtime per process).
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (loads the HIP runtime the library must share)

_HERE = os.path.dirname(os.path.abspath(__file__))
# PKV_LIBRARY names another build of the same library to load instead (the
# CPU tests use it for the build whose host runtime carries sanitizers).
LIB_PATH = os.environ.get("PKV_LIBRARY") or os.path.join(_HERE, "libpkv.so")

PKV_OK = 0
PKV_ERR_INVALID_ARGUMENT = 1
PKV_ERR_BAD_STATE = 2
PKV_ERR_OUT_OF_PAGES = 3
PKV_ERR_CAPACITY_EXHAUSTED = 4
PKV_ERR_ALLOC = 5
PKV_ERR_DEVICE = 6

STATUS_NAMES = {0: "OK", 1: "INVALID_ARGUMENT", 2: "BAD_STATE", 3: "OUT_OF_PAGES",
                4: "CAPACITY_EXHAUSTED", 5: "ALLOC", 6: "DEVICE"}

PKV_DTYPE_F32 = 0
PKV_DTYPE_BF16 = 1
PKV_POOL_HOST_ONLY = 1
PKV_POOL_ADDRESS_ORDER = 2


class PkvError(RuntimeError):
    def __init__(self, status: int, func: str, message: str):
        self.status = status
        self.func = func
        super().__init__(f"{func}: {STATUS_NAMES.get(status, status)}: {message}")


class pkv_pool_desc(ctypes.Structure):
    _fields_ = [
        ("num_layers", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("head_width", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("max_context", ctypes.c_int32),
        ("max_caches", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("split_blocks", ctypes.c_int32),
        ("flags", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("k_storage", ctypes.c_void_p),
        ("v_storage", ctypes.c_void_p),
        ("free_list_seed", ctypes.c_uint64),
    ]


class pkv_counters(ctypes.Structure):
    _fields_ = [
        ("committed_tokens", ctypes.c_uint64),
        ("aborted_tokens", ctypes.c_uint64),
        ("cache_appends", ctypes.c_uint64),
        ("score_cells", ctypes.c_uint64),
        ("kv_bytes_read", ctypes.c_uint64),
        ("pages_free", ctypes.c_int32),
        ("pages_leased", ctypes.c_int32),
        ("cow_copies", ctypes.c_uint64),
        ("pages_shared", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class pkv_profile(ctypes.Structure):
    _fields_ = [
        ("attention_launches", ctypes.c_uint64),
        ("attention_ms", ctypes.c_double),
        ("merge_launches", ctypes.c_uint64),
        ("merge_ms", ctypes.c_double),
        ("algorithmic_bytes", ctypes.c_uint64),
        ("prefill_launches", ctypes.c_uint64),
        ("prefill_ms", ctypes.c_double),
        ("prefill_flops", ctypes.c_uint64),
    ]


PKV_OPT_SPLIT_BLOCKS = 1
PKV_OPT_MERGE_MODE = 2
PKV_OPT_PROFILING = 3
PKV_OPT_WAVES = 4
PKV_OPT_VALIDATE = 5
PKV_MERGE_SEPARATE = 0
PKV_MERGE_AUTO = 1
PKV_MERGE_LAST_ARRIVER = 2

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_PI32 = ctypes.POINTER(ctypes.c_int32)

# name -> (restype, argtypes)
SIGNATURES = {
    "pkv_version": (ctypes.c_char_p, []),
    "pkv_last_error": (ctypes.c_char_p, []),
    "pkv_pool_desc_init": (None, [ctypes.POINTER(pkv_pool_desc)]),
    "pkv_pool_create": (_I32, [ctypes.POINTER(pkv_pool_desc), ctypes.POINTER(_P)]),
    "pkv_pool_destroy": (_I32, [_P]),
    "pkv_pool_get_desc": (_I32, [_P, ctypes.POINTER(pkv_pool_desc)]),
    "pkv_pool_get_counters": (_I32, [_P, ctypes.POINTER(pkv_counters)]),
    "pkv_pool_set_option": (_I32, [_P, _I32, ctypes.c_int64]),
    "pkv_pool_get_profile": (_I32, [_P, ctypes.POINTER(pkv_profile), _I32]),
    "pkv_page_lease": (_I32, [_P, _PI32]),
    "pkv_page_release": (_I32, [_P, _I32]),
    "pkv_cache_create": (_I32, [_P, _I32, ctypes.POINTER(_P)]),
    "pkv_cache_destroy": (_I32, [_P]),
    "pkv_cache_reset": (_I32, [_P]),
    "pkv_cache_size": (_I32, [_P]),
    "pkv_cache_capacity": (_I32, [_P]),
    "pkv_cache_block_size": (_I32, [_P]),
    "pkv_cache_page_table": (_I32, [_P, _PI32, _I32, _PI32]),
    "pkv_cache_fork": (_I32, [_P, _I32, _I32, ctypes.POINTER(_P)]),
    "pkv_cache_grow": (_I32, [_P, _I32, _P]),
    "pkv_begin_token": (_I32, [_P, _PI32]),
    "pkv_append_and_attend": (_I32, [_P, _I32, _P, _P, _P, _P, _P]),
    "pkv_commit_token": (_I32, [_P]),
    "pkv_abort_token": (_I32, [_P]),
    "pkv_append_and_attend_batched": (_I32, [ctypes.POINTER(_P), _I32, _I32, _P, _P, _P, _P, _P]),
    "pkv_begin_token_batched": (_I32, [ctypes.POINTER(_P), _I32, _PI32]),
    "pkv_begin_tokens": (_I32, [_P, _I32, _PI32]),
    "pkv_begin_tokens_batched": (_I32, [ctypes.POINTER(_P), _I32, _PI32, _PI32]),
    "pkv_prefill_attention": (_I32, [_P, _I32, _I32, _P, _I32, _PI32, _PI32, _P, _P, _P, _P, _P]),
    "pkv_commit_token_batched": (_I32, [ctypes.POINTER(_P), _I32]),
    "pkv_plan_create": (_I32, [_P, ctypes.POINTER(_P)]),
    "pkv_plan_destroy": (_I32, [_P]),
    "pkv_plan_build": (_I32, [_P, _I32, _PI32, _I32, _P]),
    "pkv_plan_num_chunks": (_I32, [_P]),
    "pkv_plan_decode_attention": (_I32, [_P, _I32, _P, _P, _P, _P]),
    "pkv_plan_kv_append": (_I32, [_P, _I32, _P, _P, _P, _P]),
    "pkv_plan_append_and_attend": (_I32, [_P, _I32, _P, _P, _P, _P, _P, _P]),
    "pkv_decode_attention": (_I32, [_P, _I32, _I32, _P, _P, _I32, _PI32, _P, _P]),
    "pkv_kv_append": (_I32, [_P, _I32, _I32, _P, _I32, _PI32, _P, _P, _P]),
    "pkv_decode_attention_noalloc": (_I32, [_P, _I32, _I32, _P, _P, _I32, _PI32, _P, _P]),
}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python paged_kv_cache_attention_amd/build.py` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH, mode=ctypes.RTLD_GLOBAL)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _check_single_hip_runtime()
    return lib


def _check_single_hip_runtime():
    try:
        with open("/proc/self/maps") as f:
            paths = {line.split()[-1] for line in f if "libamdhip64" in line}
    except OSError:
        return
    if len(paths) > 1:
        raise ImportError(f"two HIP runtimes are loaded in this process: {sorted(paths)}")


_lib = _load()


def _check(status: int, func: str):
    if status != PKV_OK:
        raise PkvError(status, func, _lib.pkv_last_error().decode(errors="replace"))


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if isinstance(x, torch.Tensor):
        return x.data_ptr()
    raise TypeError(f"expected a tensor, an int address or None, got {type(x)}")


def _stream(stream):
    if stream is None:
        if torch.cuda.is_available():
            return torch.cuda.current_stream().cuda_stream
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _i32_array(values):
    values = [int(v) for v in values]
    return (ctypes.c_int32 * max(1, len(values)))(*values)


# --------------------------------------------------------------------- misc --
def pkv_version() -> str:
    return _lib.pkv_version().decode()


def pkv_last_error() -> str:
    return _lib.pkv_last_error().decode(errors="replace")


def pkv_pool_desc_init() -> pkv_pool_desc:
    d = pkv_pool_desc()
    _lib.pkv_pool_desc_init(ctypes.byref(d))
    return d


# --------------------------------------------------------------------- pool --
def pkv_pool_create(desc: pkv_pool_desc) -> int:
    h = ctypes.c_void_p()
    _check(_lib.pkv_pool_create(ctypes.byref(desc), ctypes.byref(h)), "pkv_pool_create")
    return h.value


def pkv_pool_destroy(pool: int) -> None:
    _check(_lib.pkv_pool_destroy(pool), "pkv_pool_destroy")


def pkv_pool_get_desc(pool: int) -> pkv_pool_desc:
    d = pkv_pool_desc()
    _check(_lib.pkv_pool_get_desc(pool, ctypes.byref(d)), "pkv_pool_get_desc")
    return d


def pkv_pool_get_counters(pool: int) -> pkv_counters:
    c = pkv_counters()
    _check(_lib.pkv_pool_get_counters(pool, ctypes.byref(c)), "pkv_pool_get_counters")
    return c


def pkv_pool_set_option(pool: int, option: int, value: int) -> None:
    _check(_lib.pkv_pool_set_option(pool, option, value), "pkv_pool_set_option")


def pkv_pool_get_profile(pool: int, reset: bool = True) -> pkv_profile:
    prof = pkv_profile()
    _check(_lib.pkv_pool_get_profile(pool, ctypes.byref(prof), 1 if reset else 0),
           "pkv_pool_get_profile")
    return prof


def pkv_page_lease(pool: int) -> int:
    p = ctypes.c_int32()
    _check(_lib.pkv_page_lease(pool, ctypes.byref(p)), "pkv_page_lease")
    return p.value


def pkv_page_release(pool: int, page: int) -> None:
    _check(_lib.pkv_page_release(pool, page), "pkv_page_release")


# ------------------------------------------------------------------- caches --
def pkv_cache_create(pool: int, max_context: int) -> int:
    h = ctypes.c_void_p()
    _check(_lib.pkv_cache_create(pool, max_context, ctypes.byref(h)), "pkv_cache_create")
    return h.value


def pkv_cache_destroy(cache: int) -> None:
    _check(_lib.pkv_cache_destroy(cache), "pkv_cache_destroy")


def pkv_cache_reset(cache: int) -> None:
    _check(_lib.pkv_cache_reset(cache), "pkv_cache_reset")


def pkv_cache_size(cache: int) -> int:
    return _lib.pkv_cache_size(cache)


def pkv_cache_capacity(cache: int) -> int:
    return _lib.pkv_cache_capacity(cache)


def pkv_cache_block_size(cache: int) -> int:
    return _lib.pkv_cache_block_size(cache)


def pkv_cache_page_table(cache: int) -> list:
    cap = max(1, pkv_cache_capacity(cache) + 1)
    buf = (ctypes.c_int32 * cap)()
    n = ctypes.c_int32()
    _check(_lib.pkv_cache_page_table(cache, buf, cap, ctypes.byref(n)), "pkv_cache_page_table")
    return list(buf[:n.value])


def pkv_cache_fork(src: int, n_tokens: int, max_context: int) -> int:
    h = ctypes.c_void_p()
    _check(_lib.pkv_cache_fork(src, n_tokens, max_context, ctypes.byref(h)), "pkv_cache_fork")
    return h.value


def pkv_cache_grow(cache: int, n_tokens: int, stream=None) -> None:
    _check(_lib.pkv_cache_grow(cache, n_tokens, _stream(stream)), "pkv_cache_grow")


# -------------------------------------------------------------- transaction --
def pkv_begin_token(cache: int) -> int:
    pos = ctypes.c_int32()
    _check(_lib.pkv_begin_token(cache, ctypes.byref(pos)), "pkv_begin_token")
    return pos.value


def pkv_begin_tokens(cache: int, count: int) -> int:
    pos = ctypes.c_int32()
    _check(_lib.pkv_begin_tokens(cache, count, ctypes.byref(pos)), "pkv_begin_tokens")
    return pos.value


def pkv_append_and_attend(cache: int, layer: int, q, k, v, out, stream=None) -> None:
    _check(_lib.pkv_append_and_attend(cache, layer, _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                      _stream(stream)), "pkv_append_and_attend")


def pkv_commit_token(cache: int) -> None:
    _check(_lib.pkv_commit_token(cache), "pkv_commit_token")


def pkv_abort_token(cache: int) -> None:
    _check(_lib.pkv_abort_token(cache), "pkv_abort_token")


def _cache_array(caches):
    if isinstance(caches, ctypes.Array):
        return caches, len(caches)
    return (ctypes.c_void_p * max(1, len(caches)))(*caches), len(caches)


def pkv_cache_array(caches):
    """A reusable C array of cache handles for the batched calls."""
    return _cache_array(caches)[0]


def pkv_begin_token_batched(caches) -> list:
    arr, n = _cache_array(caches)
    pos = (ctypes.c_int32 * max(1, n))()
    _check(_lib.pkv_begin_token_batched(arr, n, pos), "pkv_begin_token_batched")
    return list(pos[:n])


def pkv_begin_tokens_batched(caches, counts=None) -> list:
    arr, n = _cache_array(caches)
    pos = (ctypes.c_int32 * max(1, n))()
    cnt = None if counts is None else (ctypes.c_int32 * max(1, n))(*counts)
    _check(_lib.pkv_begin_tokens_batched(arr, n, cnt, pos), "pkv_begin_tokens_batched")
    return list(pos[:n])


def pkv_commit_token_batched(caches) -> None:
    arr, n = _cache_array(caches)
    _check(_lib.pkv_commit_token_batched(arr, n), "pkv_commit_token_batched")


def pkv_append_and_attend_batched(caches, layer: int, q, k, v, out, stream=None) -> None:
    arr, n = _cache_array(caches)
    _check(_lib.pkv_append_and_attend_batched(arr, n, layer, _ptr(q), _ptr(k), _ptr(v),
                                              _ptr(out), _stream(stream)),
           "pkv_append_and_attend_batched")


# -------------------------------------------------------------------- plans --
def pkv_plan_create(pool: int) -> int:
    h = ctypes.c_void_p()
    _check(_lib.pkv_plan_create(pool, ctypes.byref(h)), "pkv_plan_create")
    return h.value


def pkv_plan_destroy(plan: int) -> None:
    _check(_lib.pkv_plan_destroy(plan), "pkv_plan_destroy")


def pkv_plan_build(plan: int, seq_lens, pt_stride: int, stream=None) -> None:
    arr = _i32_array(seq_lens)
    _check(_lib.pkv_plan_build(plan, len(seq_lens), arr, pt_stride, _stream(stream)),
           "pkv_plan_build")


def pkv_plan_num_chunks(plan: int) -> int:
    return _lib.pkv_plan_num_chunks(plan)


def pkv_plan_decode_attention(plan: int, layer: int, q, page_table, out, stream=None) -> None:
    _check(_lib.pkv_plan_decode_attention(plan, layer, _ptr(q), _ptr(page_table), _ptr(out),
                                          _stream(stream)), "pkv_plan_decode_attention")


def pkv_plan_kv_append(plan: int, layer: int, page_table, k, v, stream=None) -> None:
    _check(_lib.pkv_plan_kv_append(plan, layer, _ptr(page_table), _ptr(k), _ptr(v),
                                   _stream(stream)), "pkv_plan_kv_append")


def pkv_plan_append_and_attend(plan: int, layer: int, page_table, q, k, v, out,
                               stream=None) -> None:
    _check(_lib.pkv_plan_append_and_attend(plan, layer, _ptr(page_table), _ptr(q), _ptr(k),
                                           _ptr(v), _ptr(out), _stream(stream)),
           "pkv_plan_append_and_attend")


def pkv_decode_attention(pool: int, layer: int, q, page_table, pt_stride: int, seq_lens, out,
                         stream=None) -> None:
    arr = _i32_array(seq_lens)
    _check(_lib.pkv_decode_attention(pool, layer, len(seq_lens), _ptr(q), _ptr(page_table),
                                     pt_stride, arr, _ptr(out), _stream(stream)),
           "pkv_decode_attention")


PKV_NOALLOC_SCRATCH_BYTES = 33554432
PKV_NOALLOC_MAX_REQUESTS = 4096
PKV_NOALLOC_MAX_CHUNKS = 32768
PKV_NOALLOC_MAX_COUNTERS = 262144
PKV_NOALLOC_MAX_PARTIAL_FLOATS = 7602176


def pkv_decode_attention_noalloc(pool: int, layer: int, q, page_table, pt_stride: int, seq_lens,
                                 out, stream=None) -> None:
    arr = _i32_array(seq_lens)
    _check(_lib.pkv_decode_attention_noalloc(pool, layer, len(seq_lens), _ptr(q),
                                             _ptr(page_table), pt_stride, arr, _ptr(out),
                                             _stream(stream)), "pkv_decode_attention_noalloc")


def pkv_kv_append(pool: int, layer: int, page_table, pt_stride: int, positions, k, v,
                  stream=None) -> None:
    arr = _i32_array(positions)
    _check(_lib.pkv_kv_append(pool, layer, len(positions), _ptr(page_table), pt_stride, arr,
                              _ptr(k), _ptr(v), _stream(stream)), "pkv_kv_append")


def pkv_prefill_attention(pool: int, layer: int, page_table, pt_stride: int, starts, counts, q,
                          k, v, out, stream=None) -> None:
    n = len(starts)
    if len(counts) != n:
        raise ValueError("starts and counts differ in length")
    st = (ctypes.c_int32 * max(1, n))(*starts)
    ct = (ctypes.c_int32 * max(1, n))(*counts)
    _check(_lib.pkv_prefill_attention(pool, layer, n, _ptr(page_table), pt_stride, st, ct, _ptr(q),
                                      _ptr(k), _ptr(v), _ptr(out), _stream(stream)),
           "pkv_prefill_attention")


__all__ = [n for n in list(globals()) if n.startswith("pkv_")] + [
    "PkvError", "STATUS_NAMES", "PKV_DTYPE_F32", "PKV_DTYPE_BF16",
    "PKV_POOL_HOST_ONLY", "PKV_POOL_ADDRESS_ORDER",
    "PKV_OPT_SPLIT_BLOCKS", "PKV_OPT_MERGE_MODE", "PKV_OPT_PROFILING", "PKV_OPT_WAVES",
    "PKV_OPT_VALIDATE", "PKV_MERGE_SEPARATE", "PKV_MERGE_AUTO", "PKV_MERGE_LAST_ARRIVER",
    "LIB_PATH", "SIGNATURES", "PKV_NOALLOC_SCRATCH_BYTES",
    "PKV_NOALLOC_MAX_REQUESTS", "PKV_NOALLOC_MAX_CHUNKS", "PKV_NOALLOC_MAX_COUNTERS",
    "PKV_NOALLOC_MAX_PARTIAL_FLOATS"]
