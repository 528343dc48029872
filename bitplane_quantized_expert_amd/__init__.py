"""Python binding of libpm (include/pm.h): argument marshalling only.

Every function here has the name of the C entry point it calls and passes
plain pointers through: device arrays are torch tensors (their data_ptr()),
host arrays are NumPy arrays, streams are torch streams (their HIP handle).
All computation happens in libpm's HIP kernels and host C++; if libpm.so has
not been built, loading fails loudly (there is no fallback).
"""
from __future__ import annotations

import atexit
import ctypes
import os
import sys
import weakref

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# PM_LIB selects another build of the same library (e.g. a tuning variant).
LIB_PATH = os.environ.get("PM_LIB") or os.path.join(_HERE, "libpm.so")

PM_OK = 0
PM_ERR_ARG = -1
PM_ERR_SHAPE = -2
PM_ERR_PREFIX = -3
PM_ERR_NOT_RESIDENT = -4
PM_ERR_OOM = -5
PM_ERR_HIP = -6
PM_ERR_STATE = -7
PM_STORE_HOST_FAKE = 1
PM_AUTO_TOPUP = 1
PM_BATCH_MFMA = 2
PM_READ_ONCE = 4
PM_DETERMINISTIC = 8
PM_GEMV_NOALLOC_MAX_PARTIALS = 524288

_STATUS = {0: "PM_OK", -1: "PM_ERR_ARG", -2: "PM_ERR_SHAPE", -3: "PM_ERR_PREFIX",
           -4: "PM_ERR_NOT_RESIDENT", -5: "PM_ERR_OOM", -6: "PM_ERR_HIP", -7: "PM_ERR_STATE"}


class PMError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


class pm_matrix_shape(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int32), ("cols", ctypes.c_int32), ("group", ctypes.c_int32)]


class pm_expert_shape(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32), ("group", ctypes.c_int32)]


_c = ctypes
_P = ctypes.c_void_p
_I = ctypes.c_int
_Z = ctypes.c_size_t
_U32 = ctypes.c_uint32
_MS = pm_matrix_shape
_ES = pm_expert_shape

# name -> (restype, argtypes)
SIGNATURES = {
    "pm_last_error": (_c.c_char_p, []),
    "pm_version": (_c.c_char_p, []),
    "pm_plane_words": (_Z, [_MS]),
    "pm_levels_floats": (_Z, [_MS]),
    "pm_level_offset": (_Z, [_MS, _I]),
    "pm_expert_plane_words": (_Z, [_ES]),
    "pm_expert_levels_floats": (_Z, [_ES]),
    "pm_expert_matrix_offsets": (_I, [_ES, _I, _P, _P, _P]),
    "pm_encode_matrix": (_I, [_MS, _P, _P, _P, _P, _Z, _P]),
    "pm_encode_expert": (_I, [_ES, _P, _P, _P, _P, _P]),
    "pm_encode_matrix_device": (_I, [_MS, _P, _P, _P, _P, _Z, _P, _P]),
    "pm_kmeans_codebook_device": (_I, [_MS, _P, _I, _P, _P, _P, _P, _P]),
    "pm_expert_gemv": (_I, [_MS, _I, _P, _Z, _P, _P, _P, _P]),
    "pm_expert_gemv_noalloc": (_I, [_MS, _I, _P, _Z, _P, _P, _P, _P]),
    "pm_route_topk": (_I, [_I, _I, _I, _P, _P, _P]),
    "pm_allocate_bits": (_I, [_I, _I, _P, _P, _I, _P, _I, _P]),
    "pm_store_create": (_I, [_ES, _I, _I, _Z, _U32, _P]),
    "pm_store_destroy": (_I, [_P]),
    "pm_store_slot": (_I, [_P, _I, _I, _P, _P]),
    "pm_store_usage": (_I, [_P, _P, _P, _P]),
    "pm_store_slot_info": (_I, [_P, _I, _I, _P, _P, _P]),
    "pm_store_set_resident": (_I, [_P, _I, _I, _I]),
    "pm_store_attach_host": (_I, [_P, _I, _I, _P, _P]),
    "pm_store_topup": (_I, [_P, _I, _I, _I, _P]),
    "pm_store_truncate": (_I, [_P, _I, _I, _I]),
    "pm_store_resident": (_I, [_P, _I, _I, _P]),
    "pm_store_copy_stats": (_I, [_P, _P, _P, _P, _P]),
    "pm_store_set_profile_events": (_I, [_P, _P, _I]),
    "pm_cache_create": (_I, [_I, _c.c_int64, _I, _P]),
    "pm_cache_destroy": (_I, [_P]),
    "pm_cache_access": (_I, [_P, _I, _I, _P, _P]),
    "pm_cache_replay": (_I, [_P, _P, _P, _Z]),
    "pm_cache_resident": (_I, [_P, _I, _P]),
    "pm_cache_stats": (_I, [_P, _P, _P, _P, _P, _P]),
    "pm_moe_token_forward": (_I, [_P, _I, _I, _I, _P, _P, _P, _P, _P, _P, _U32]),
    "pm_debug_unpack_prefix": (_I, [_MS, _I, _P, _Z, _P, _P]),
    "pm_debug_dequant": (_I, [_MS, _I, _P, _Z, _P, _P, _P]),
    "pm_materialize_fp16": (_I, [_MS, _I, _P, _Z, _P, _P, _P]),
    "pm_gemv_fp16": (_I, [_MS, _P, _P, _P, _P]),
    "pm_materialize_fp16_batch": (_I, [_I, _P, _P, _P, _P, _P, _P, _P]),
    "pm_gemv_fp16_batch": (_I, [_I, _P, _P, _P, _P, _P]),
}

_lib = None


def lib():
    """The loaded libpm.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python bitplane_quantized_expert_amd/build.py` (there is no fallback)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(st):
    if st != PM_OK:
        raise PMError(st, lib().pm_last_error().decode())
    return st


# ---------------------------------------------------------------- marshalling helpers
def _dptr(t):
    """Device pointer of a torch tensor (or None / an int)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _hptr(a):
    if a is None:
        return None
    if not (isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"]):
        raise ValueError("host arrays must be C-contiguous numpy arrays")
    return a.ctypes.data


def _stream(s):
    if s is None:
        return None
    if isinstance(s, int):
        return s
    return s.cuda_stream


def mshape(rows, cols, group):
    return pm_matrix_shape(rows, cols, group)


def eshape(hidden, inter, group):
    return pm_expert_shape(hidden, inter, group)


# ---------------------------------------------------------------- sizes
def pm_plane_words(s):
    return lib().pm_plane_words(s)


def pm_levels_floats(s):
    return lib().pm_levels_floats(s)


def pm_level_offset(s, d):
    return lib().pm_level_offset(s, d)


def pm_expert_plane_words(e):
    return lib().pm_expert_plane_words(e)


def pm_expert_levels_floats(e):
    return lib().pm_expert_levels_floats(e)


def pm_expert_matrix_offsets(e, m):
    pw = ctypes.c_size_t()
    lf = ctypes.c_size_t()
    sh = pm_matrix_shape()
    _check(lib().pm_expert_matrix_offsets(e, m, ctypes.byref(pw), ctypes.byref(lf),
                                          ctypes.byref(sh)))
    return pw.value, lf.value, sh


# ---------------------------------------------------------------- encoding
def pm_encode_matrix(s, codes, leaves, counts, planes_out, plane_stride_words, levels_out):
    return _check(lib().pm_encode_matrix(s, _hptr(codes), _hptr(leaves), _hptr(counts),
                                         _hptr(planes_out), plane_stride_words,
                                         _hptr(levels_out)))


def pm_encode_expert(e, codes3, leaves3, counts3, planes_out, levels_out):
    arr = lambda xs, T: (ctypes.c_void_p * 3)(*[_hptr(x) for x in xs]) if xs is not None else None
    return _check(lib().pm_encode_expert(e, arr(codes3, None), arr(leaves3, None),
                                         arr(counts3, None), _hptr(planes_out),
                                         _hptr(levels_out)))


def pm_encode_matrix_device(s, d_codes, d_leaves, d_counts, d_planes, plane_stride_words,
                            d_levels, stream=None):
    return _check(lib().pm_encode_matrix_device(s, _dptr(d_codes), _dptr(d_leaves),
                                                _dptr(d_counts), _dptr(d_planes),
                                                plane_stride_words, _dptr(d_levels),
                                                _stream(stream)))


# ---------------------------------------------------------------- GEMV and checks
def pm_kmeans_codebook_device(s, d_w, max_iters, d_codes, d_leaves, d_counts, d_iters=None,
                              stream=None):
    return _check(lib().pm_kmeans_codebook_device(s, _dptr(d_w), max_iters, _dptr(d_codes),
                                                  _dptr(d_leaves), _dptr(d_counts),
                                                  _dptr(d_iters), _stream(stream)))


def pm_expert_gemv(s, k, d_planes, plane_stride_words, d_levels, d_x, d_y, stream=None):
    return _check(lib().pm_expert_gemv(s, k, _dptr(d_planes), plane_stride_words,
                                       _dptr(d_levels), _dptr(d_x), _dptr(d_y),
                                       _stream(stream)))


def pm_expert_gemv_noalloc(s, k, d_planes, plane_stride_words, d_levels, d_x, d_y,
                           stream=None):
    return _check(lib().pm_expert_gemv_noalloc(s, k, _dptr(d_planes), plane_stride_words,
                                               _dptr(d_levels), _dptr(d_x), _dptr(d_y),
                                               _stream(stream)))


def pm_debug_unpack_prefix(s, k, d_planes, plane_stride_words, d_out, stream=None):
    return _check(lib().pm_debug_unpack_prefix(s, k, _dptr(d_planes), plane_stride_words,
                                               _dptr(d_out), _stream(stream)))


def pm_debug_dequant(s, k, d_planes, plane_stride_words, d_levels, d_out, stream=None):
    return _check(lib().pm_debug_dequant(s, k, _dptr(d_planes), plane_stride_words,
                                         _dptr(d_levels), _dptr(d_out), _stream(stream)))


def pm_materialize_fp16(s, k, d_planes, plane_stride_words, d_levels, d_out, stream=None):
    return _check(lib().pm_materialize_fp16(s, k, _dptr(d_planes), plane_stride_words,
                                            _dptr(d_levels), _dptr(d_out), _stream(stream)))


def pm_gemv_fp16(s, d_w, d_x, d_y, stream=None):
    return _check(lib().pm_gemv_fp16(s, _dptr(d_w), _dptr(d_x), _dptr(d_y), _stream(stream)))


def _ptr_array(ptrs):
    arr = (ctypes.c_void_p * max(1, len(ptrs)))(*[_dptr(p) for p in ptrs])
    return ctypes.cast(arr, ctypes.c_void_p)


def pm_materialize_fp16_batch(shapes, ks, d_planes, plane_stride_words, d_levels, d_w_fp16,
                              stream=None):
    """Lists of one length: matrix shapes, prefixes, device plane/level
    pointers (tensors or ints), plane strides (words) and fp16 outputs."""
    n = len(shapes)
    sh = (pm_matrix_shape * max(1, n))(*shapes)
    kk = np.ascontiguousarray(ks, dtype=np.int32)
    ps = np.ascontiguousarray(plane_stride_words, dtype=np.uint64)
    return _check(lib().pm_materialize_fp16_batch(
        n, ctypes.cast(sh, ctypes.c_void_p), _hptr(kk), _ptr_array(d_planes), _hptr(ps),
        _ptr_array(d_levels), _ptr_array(d_w_fp16), _stream(stream)))


def pm_gemv_fp16_batch(shapes, d_w, d_x, d_y, stream=None):
    n = len(shapes)
    sh = (pm_matrix_shape * max(1, n))(*shapes)
    return _check(lib().pm_gemv_fp16_batch(n, ctypes.cast(sh, ctypes.c_void_p), _ptr_array(d_w),
                                           _ptr_array(d_x), _ptr_array(d_y), _stream(stream)))


# ---------------------------------------------------------------- routing / allocation
def pm_route_topk(logits, top_k):
    """logits float32 [n_tokens][n_experts] -> (ids int32, w float32) [n_tokens][top_k]."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    if logits.ndim == 1:
        logits = logits[None]
    n, e = logits.shape
    ids = np.zeros((n, top_k), dtype=np.int32)
    w = np.zeros((n, top_k), dtype=np.float32)
    _check(lib().pm_route_topk(n, e, top_k, _hptr(logits), _hptr(ids), _hptr(w)))
    return ids, w


def pm_allocate_bits(ids, w, err_profiles, budget):
    """ids int32 [n][top_k], w float32 [n][top_k], err float64 [n_experts][8] ->
    k uint8 [n][top_k]."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    err = np.ascontiguousarray(err_profiles, dtype=np.float64)
    if ids.ndim == 1:
        ids, w = ids[None], w[None]
    n, top_k = ids.shape
    k = np.zeros((n, top_k), dtype=np.uint8)
    _check(lib().pm_allocate_bits(n, top_k, _hptr(ids), _hptr(w), err.shape[0], _hptr(err),
                                  int(budget), _hptr(k)))
    return k


# ---------------------------------------------------------------- handles
# Stores and caches still open when the interpreter exits are closed by an
# exit handler, in reverse order of creation, while the HIP runtime and torch
# are still whole.  A handle collected during interpreter shutdown is left to
# the process exit instead: nothing calls into the library (or HIP) from a
# finalizer then.
_live = weakref.WeakValueDictionary()
_live_next = [0]


def _track(obj):
    _live_next[0] += 1
    _live[_live_next[0]] = obj


@atexit.register
def _close_live_handles():
    for key in sorted(_live.keys(), reverse=True):
        obj = _live.get(key)
        if obj is not None:
            try:
                obj.close()
            except Exception:
                pass


class _Handle:
    _destroy = None

    def close(self):
        if self.handle:
            getattr(lib(), self._destroy)(self.handle)
            self.handle = None

    def __del__(self, _finalizing=sys.is_finalizing):
        # (bound at definition: module globals may already be gone here)
        if _finalizing():
            return
        try:
            self.close()
        except Exception:
            pass


# ---------------------------------------------------------------- store
class Store(_Handle):
    """Owner of a pm_store handle (pm_store_destroy on close).  Host sources
    attached to it must stay alive until it is closed."""
    _destroy = "pm_store_destroy"

    def __init__(self, e, n_layers, n_experts, capacity_bytes=0, flags=0):
        self.handle = None
        h = ctypes.c_void_p()
        _check(lib().pm_store_create(e, n_layers, n_experts, capacity_bytes, flags,
                                     ctypes.byref(h)))
        self.handle = h.value
        self.shape = e
        _track(self)


def pm_store_create(e, n_layers, n_experts, capacity_bytes=0, flags=0):
    return Store(e, n_layers, n_experts, capacity_bytes, flags)


def pm_store_destroy(store):
    store.close()


def pm_store_slot(store, layer, expert):
    """(planes pointer, levels pointer) of a slot, as ints."""
    p = ctypes.c_void_p()
    lv = ctypes.c_void_p()
    _check(lib().pm_store_slot(store.handle, layer, expert, ctypes.byref(p), ctypes.byref(lv)))
    return p.value, lv.value


def pm_store_usage(store):
    """(bytes held, plane chunks, slots holding levels)."""
    u, c, l = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().pm_store_usage(store.handle, ctypes.byref(u), ctypes.byref(c), ctypes.byref(l)))
    return u.value, c.value, l.value


def pm_store_set_resident(store, layer, expert, r):
    return _check(lib().pm_store_set_resident(store.handle, layer, expert, r))


def pm_store_attach_host(store, layer, expert, h_planes, h_levels):
    hp = h_planes if isinstance(h_planes, int) else (
        h_planes.data_ptr() if hasattr(h_planes, "data_ptr") else _hptr(h_planes))
    hl = h_levels if isinstance(h_levels, int) else (
        h_levels.data_ptr() if hasattr(h_levels, "data_ptr") else _hptr(h_levels))
    return _check(lib().pm_store_attach_host(store.handle, layer, expert, hp, hl))


def pm_store_topup(store, layer, expert, k, side=None):
    return _check(lib().pm_store_topup(store.handle, layer, expert, k, _stream(side)))


def pm_store_truncate(store, layer, expert, keep):
    return _check(lib().pm_store_truncate(store.handle, layer, expert, keep))


def pm_store_slot_info(store, layer, expert):
    """(planes address, levels address, plane chunks held) of a slot, as is."""
    p, lv, n = ctypes.c_void_p(), ctypes.c_void_p(), ctypes.c_int()
    _check(lib().pm_store_slot_info(store.handle, layer, expert, ctypes.byref(p),
                                    ctypes.byref(lv), ctypes.byref(n)))
    return p.value or 0, lv.value or 0, n.value


def pm_store_resident(store, layer, expert):
    r = ctypes.c_int()
    _check(lib().pm_store_resident(store.handle, layer, expert, ctypes.byref(r)))
    return r.value


def pm_store_copy_stats(store):
    a, b = ctypes.c_int(), ctypes.c_int()
    c, d = ctypes.c_uint64(), ctypes.c_uint64()
    _check(lib().pm_store_copy_stats(store.handle, ctypes.byref(a), ctypes.byref(b),
                                     ctypes.byref(c), ctypes.byref(d)))
    return a.value, b.value, c.value, d.value


def pm_store_set_profile_events(store, events):
    """events: list of 2 (gate/up launch only) or 4 (every stage)
    torch.cuda.Event, or [] to switch off."""
    if not events:
        return _check(lib().pm_store_set_profile_events(store.handle, None, 0))
    arr = (ctypes.c_void_p * len(events))(*[ev.cuda_event for ev in events])
    store._profile_events = (events, arr)
    return _check(lib().pm_store_set_profile_events(store.handle, arr, len(events)))


# ---------------------------------------------------------------- expert caches
PM_CACHE_PREFIX = 0
PM_CACHE_OBJECTS = 1
PM_CACHE_DOWNWARD = 2


class Cache(_Handle):
    """Owner of a pm_cache handle (pm_cache_destroy on close)."""
    _destroy = "pm_cache_destroy"

    def __init__(self, n_experts, capacity_planes, policy=PM_CACHE_PREFIX):
        self.handle = None
        h = ctypes.c_void_p()
        _check(lib().pm_cache_create(n_experts, capacity_planes, policy, ctypes.byref(h)))
        self.handle = h.value
        _track(self)


def pm_cache_create(n_experts, capacity_planes, policy=PM_CACHE_PREFIX):
    return Cache(n_experts, capacity_planes, policy)


def pm_cache_destroy(cache):
    cache.close()


def pm_cache_access(cache, expert, k):
    """(first, count): the 1-based planes this access reads."""
    a, b = ctypes.c_int(), ctypes.c_int()
    _check(lib().pm_cache_access(cache.handle, expert, k, ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


def pm_cache_replay(cache, experts, ks):
    """experts, ks: int32 numpy arrays of one length (host)."""
    experts = np.ascontiguousarray(experts, dtype=np.int32)
    ks = np.ascontiguousarray(ks, dtype=np.int32)
    if experts.shape != ks.shape or experts.ndim != 1:
        raise ValueError("experts and ks must be 1-D arrays of one length")
    return _check(lib().pm_cache_replay(cache.handle, _hptr(experts), _hptr(ks), experts.size))


def pm_cache_resident(cache, expert):
    r = ctypes.c_int()
    _check(lib().pm_cache_resident(cache.handle, expert, ctypes.byref(r)))
    return r.value


def pm_cache_stats(cache):
    """dict of accesses, hits, partial, planes_read, planes_held."""
    v = [ctypes.c_uint64() for _ in range(4)] + [ctypes.c_int64()]
    _check(lib().pm_cache_stats(cache.handle, *[ctypes.byref(x) for x in v]))
    return dict(zip(("accesses", "hits", "partial", "planes_read", "planes_held"),
                    (x.value for x in v)))


def pm_moe_token_forward_ptr(store, layer, n_tokens, top_k, ids_addr, w_addr, k_addr, x_addr,
                             y_addr, stream=None, flags=0):
    """pm_moe_token_forward on buffers given by address (ints), passed through
    unchanged: host int32 ids[n][top_k], float32 w[n][top_k],
    uint8 k[n][top_k][3]; device float32 x, y [n][hidden].  For callers that
    keep their own buffers (no numpy marshalling per call)."""
    return _check(lib().pm_moe_token_forward(store.handle, layer, n_tokens, top_k, ids_addr,
                                             w_addr, k_addr, x_addr, y_addr, _stream(stream),
                                             flags))


def pm_moe_token_forward(store, layer, ids, w, k, d_x, d_y, stream=None, flags=0):
    """ids int32 [n][top_k], w float32 [n][top_k], k uint8 [n][top_k][3] (host);
    d_x, d_y float32 [n][hidden] device tensors."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    k = np.ascontiguousarray(k, dtype=np.uint8)
    n, top_k = ids.shape
    if k.shape != (n, top_k, 3):
        raise ValueError("k must be [n_tokens][top_k][3]")
    return _check(lib().pm_moe_token_forward(store.handle, layer, n, top_k, _hptr(ids), _hptr(w),
                                             _hptr(k), _dptr(d_x), _dptr(d_y), _stream(stream),
                                             flags))
