"""Python binding of libhisparse: the C ABI of include/hisparse.h, same names.

Argument marshalling only: every step of the hot path runs in the library's
HIP kernels. Device arrays are torch tensors on the current HIP device (their
data_ptr() is passed through); `stream` defaults to torch's current stream.
A non-OK status raises HsError carrying hs_last_error()'s message. Loading
fails loudly if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# HS_LIB names another build to load (the sanitizer test's host-sanitized one)
LIB_PATH = os.environ.get("HS_LIB") or os.path.join(_HERE, "libhisparse.so")

HS_OK = 0
HS_E_INVAL = -1
HS_E_RANGE = -2
HS_E_NOMEM = -3
HS_E_HIP = -4
HS_E_DEVICE = -5
HS_E_STATE = -6

HS_ERR_RANGE = 1
HS_ERR_DUP = 2
HS_ERR_CLOCK = 4
HS_ERR_SLOT = 8
HS_ERR_INTERNAL = 16
HS_ERR_APPEND = 32

HS_KV_MHA = 0
HS_KV_LATENT = 1
HS_F32 = 0
HS_BF16 = 1
HS_MAX_K = 4096
HS_MAX_B = 16384
HS_NOALLOC_SCRATCH_BYTES = 64 << 20

# every symbol include/hisparse.h declares
EXPORTS = (
    "hs_status_str", "hs_last_error", "hs_set_tuning", "hs_get_tuning",
    "hs_pool_create", "hs_pool_destroy", "hs_pool_record_bytes", "hs_pool_capacity",
    "hs_pool_reserve", "hs_pool_release", "hs_pool_record_ptr", "hs_pool_page_ptr",
    "hs_pool_length", "hs_pool_set_length", "hs_pool_append", "hs_pool_append_batch",
    "hs_buffer_bytes", "hs_buffer_create", "hs_buffer_destroy", "hs_buffer_grow",
    "hs_buffer_reset",
    "hs_buffer_rows", "hs_buffer_state_get", "hs_buffer_state_set",
    "hs_buffer_shared_bytes", "hs_buffer_create_shared", "hs_buffer_grow_group",
    "hs_batch_create", "hs_batch_destroy", "hs_batch_status", "hs_resolve",
    "hs_sparse_attn_workspace", "hs_sparse_attn", "hs_sparse_attn_noalloc", "hs_resolve_attn",
    "hs_prefetch",
    "hs_stage_create", "hs_stage_destroy", "hs_stage_run", "hs_stage_set_step",
    "hs_stage_get_step",
    "hs_trace_enable", "hs_trace_read",
)


class HsError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"[{status}] {msg}")
        self.status = status


class PoolDesc(ctypes.Structure):
    _fields_ = [
        ("n_requests", ctypes.c_int32), ("n_layers", ctypes.c_int32),
        ("kind", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("latent_dim", ctypes.c_int32), ("rope_dim", ctypes.c_int32),
        ("capacity_tokens", ctypes.POINTER(ctypes.c_int64)),
        ("max_tokens", ctypes.POINTER(ctypes.c_int64)),
        ("page_tokens", ctypes.c_int32),
    ]


TRACE_CLASSES = ("resolve", "gather", "attn", "combine", "stage", "append")


class Trace(ctypes.Structure):
    _fields_ = [("total_us", ctypes.c_double * 6), ("launches", ctypes.c_int64 * 6),
                ("dropped", ctypes.c_int64)]


class Tuning(ctypes.Structure):
    _fields_ = [("attn_splits", ctypes.c_int32), ("latent_heads_per_wg", ctypes.c_int32),
                ("prefetch_workgroups", ctypes.c_int32), ("prefetch_batch", ctypes.c_int32),
                ("gather_bytes_per_lane", ctypes.c_int32), ("resolve_fetch", ctypes.c_int32),
                ("reserved", ctypes.c_int32 * 2)]


class StageRegion(ctypes.Structure):
    _fields_ = [("d_src", ctypes.c_void_p), ("d_dst", ctypes.c_void_p),
                ("bytes", ctypes.c_size_t), ("src_stride", ctypes.c_size_t)]


_lib = None


def lib():
    """The loaded library; raises if it is missing (no fallback exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run `python -m tiered_kv_cache_hs_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    i32, i64, u32, vp, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_size_t
    P = ctypes.POINTER
    sig = {
        "hs_status_str": ([i32], ctypes.c_char_p),
        "hs_last_error": ([], ctypes.c_char_p),
        "hs_set_tuning": ([P(Tuning)], i32),
        "hs_get_tuning": ([P(Tuning)], i32),
        "hs_pool_create": ([P(PoolDesc), P(vp)], i32),
        "hs_pool_destroy": ([vp], i32),
        "hs_pool_record_bytes": ([vp, P(sz)], i32),
        "hs_pool_capacity": ([vp, i32, P(i64), P(i64), P(i64)], i32),
        "hs_pool_reserve": ([vp, i32, i64], i32),
        "hs_pool_release": ([vp, i32], i32),
        "hs_pool_record_ptr": ([vp, i32, i32, i64, P(vp), P(sz)], i32),
        "hs_pool_page_ptr": ([vp, i32, i32, i64, P(vp)], i32),
        "hs_pool_length": ([vp, i32, i32, P(i64)], i32),
        "hs_pool_set_length": ([vp, i32, i32, i64], i32),
        "hs_pool_append": ([vp, i32, i32, i64, i64, vp, i32, vp], i32),
        "hs_pool_append_batch": ([vp, vp, vp], i32),
        "hs_buffer_bytes": ([vp, i32], sz),
        "hs_buffer_create": ([vp, i32, i32, i32, vp, sz, vp, P(vp)], i32),
        "hs_buffer_destroy": ([vp], i32),
        "hs_buffer_grow": ([vp, i32, vp, sz, vp], i32),
        "hs_buffer_reset": ([vp, vp], i32),
        "hs_buffer_rows": ([vp, P(vp), P(sz)], i32),
        "hs_buffer_state_get": ([vp, vp, vp, P(u32), P(i32), vp], i32),
        "hs_buffer_state_set": ([vp, vp, vp, u32, i32, vp], i32),
        "hs_buffer_shared_bytes": ([vp, i32], sz),
        "hs_buffer_create_shared": ([vp, i32, vp, sz, P(vp)], i32),
        "hs_buffer_grow_group": ([vp, P(vp), i32, i32, vp, sz, P(vp), P(sz), vp], i32),
        "hs_batch_create": ([P(vp), i32, P(vp)], i32),
        "hs_batch_destroy": ([vp], i32),
        "hs_batch_status": ([vp, vp, vp], i32),
        "hs_resolve": ([vp, vp, i32, vp, vp, vp], i32),
        "hs_sparse_attn_workspace": ([vp, i32, i32], sz),
        "hs_sparse_attn": ([vp, vp, i32, vp, i32, ctypes.c_float, vp, vp, sz, vp], i32),
        "hs_sparse_attn_noalloc": ([vp, vp, i32, vp, i32, ctypes.c_float, vp, vp], i32),
        "hs_resolve_attn": ([vp, vp, i32, vp, vp, vp, i32, ctypes.c_float, vp, vp, sz, vp], i32),
        "hs_prefetch": ([vp, vp], i32),
        "hs_stage_create": ([P(StageRegion), i32, i32, P(vp)], i32),
        "hs_stage_destroy": ([vp], i32),
        "hs_stage_run": ([vp, vp], i32),
        "hs_stage_set_step": ([vp, u32, vp], i32),
        "hs_stage_get_step": ([vp, P(u32)], i32),
        "hs_trace_enable": ([i32], i32),
        "hs_trace_read": ([P(Trace)], i32),
    }
    for name, (args, res) in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = res
    _lib = L
    return L


def _check(status: int) -> None:
    if status != HS_OK:
        raise HsError(status, lib().hs_last_error().decode())


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return int(stream) if not hasattr(stream, "cuda_stream") else int(stream.cuda_stream)
    import torch

    return int(torch.cuda.current_stream().cuda_stream)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return int(t.data_ptr())


# ------------------------------------------------------------------ misc

def hs_status_str(status: int) -> str:
    return lib().hs_status_str(status).decode()


def hs_last_error() -> str:
    return lib().hs_last_error().decode()


def hs_set_tuning(attn_splits: int = 0, prefetch_workgroups: int = 0, prefetch_batch: int = 0,
                  gather_bytes_per_lane: int = 0, latent_heads_per_wg: int = 0,
                  resolve_fetch: int = 0) -> None:
    """Library-wide knobs (0 = the library's choice); see include/hisparse.h."""
    t = Tuning(attn_splits, latent_heads_per_wg, prefetch_workgroups, prefetch_batch,
               gather_bytes_per_lane, resolve_fetch)
    _check(lib().hs_set_tuning(ctypes.byref(t)))


def hs_get_tuning() -> dict:
    t = Tuning()
    _check(lib().hs_get_tuning(ctypes.byref(t)))
    return {"attn_splits": t.attn_splits, "latent_heads_per_wg": t.latent_heads_per_wg,
            "prefetch_workgroups": t.prefetch_workgroups,
            "prefetch_batch": t.prefetch_batch,
            "gather_bytes_per_lane": t.gather_bytes_per_lane, "resolve_fetch": t.resolve_fetch}


# ------------------------------------------------------------------ pool

def hs_pool_create(n_requests: int, n_layers: int, kind: int, dtype: int,
                   capacity_tokens: Sequence[int], n_kv_heads: int = 0, head_dim: int = 0,
                   latent_dim: int = 0, rope_dim: int = 0,
                   max_tokens: Optional[Sequence[int]] = None, page_tokens: int = 0) -> int:
    cap = (ctypes.c_int64 * len(capacity_tokens))(*[int(c) for c in capacity_tokens])
    mx = None if max_tokens is None else (ctypes.c_int64 * len(max_tokens))(*[int(c) for c in max_tokens])
    d = PoolDesc(n_requests, n_layers, kind, dtype, n_kv_heads, head_dim, latent_dim, rope_dim,
                 cap, mx, int(page_tokens))
    out = ctypes.c_void_p()
    _check(lib().hs_pool_create(ctypes.byref(d), ctypes.byref(out)))
    return out.value


def hs_pool_destroy(pool: int) -> None:
    _check(lib().hs_pool_destroy(pool))


def hs_pool_record_bytes(pool: int) -> int:
    v = ctypes.c_size_t()
    _check(lib().hs_pool_record_bytes(pool, ctypes.byref(v)))
    return v.value


def hs_pool_capacity(pool: int, req: int):
    """(records allocated, maximum, records per page) of request req."""
    c, m, pg = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check(lib().hs_pool_capacity(pool, req, ctypes.byref(c), ctypes.byref(m), ctypes.byref(pg)))
    return c.value, m.value, pg.value


def hs_pool_reserve(pool: int, req: int, records: int) -> None:
    _check(lib().hs_pool_reserve(pool, req, int(records)))


def hs_pool_release(pool: int, req: int) -> None:
    """Return all of a finished request's pages (lengths and capacity 0)."""
    _check(lib().hs_pool_release(pool, req))


def hs_pool_record_ptr(pool: int, req: int, layer: int, pos: int) -> int:
    """Host address of record pos of unit (req, layer)."""
    p, rec = ctypes.c_void_p(), ctypes.c_size_t()
    _check(lib().hs_pool_record_ptr(pool, req, layer, int(pos), ctypes.byref(p), ctypes.byref(rec)))
    return p.value


def hs_pool_page_ptr(pool: int, req: int, layer: int, page: int) -> int:
    """Host address of page `page` of unit (req, layer)."""
    p = ctypes.c_void_p()
    _check(lib().hs_pool_page_ptr(pool, req, layer, int(page), ctypes.byref(p)))
    return p.value


def pool_pages(pool: int, req: int, layer: int):
    """[(first position, numpy uint8 view [page_tokens][rec_bytes])] of the
    unit's allocated pages (host memory, writable)."""
    cap, _, pg = hs_pool_capacity(pool, req)
    rec = hs_pool_record_bytes(pool)
    out = []
    for i in range(cap // pg):
        addr = hs_pool_page_ptr(pool, req, layer, i)
        buf = (ctypes.c_uint8 * (pg * rec)).from_address(addr)
        out.append((i * pg, np.frombuffer(buf, dtype=np.uint8).reshape(pg, rec)))
    return out


def pool_read(pool: int, req: int, layer: int, positions: Sequence[int]) -> np.ndarray:
    """Copies of the unit's host records at `positions`: uint8 [n][rec_bytes]."""
    _, _, pg = hs_pool_capacity(pool, req)
    pages = dict(pool_pages(pool, req, layer))
    pos = np.asarray(positions, dtype=np.int64)
    out = np.empty((pos.size, hs_pool_record_bytes(pool)), dtype=np.uint8)
    for j, p in enumerate(pos):
        first = int(p) // pg * pg
        out[j] = pages[first][int(p) - first]
    return out


def hs_pool_length(pool: int, req: int, layer: int) -> int:
    v = ctypes.c_int64()
    _check(lib().hs_pool_length(pool, req, layer, ctypes.byref(v)))
    return v.value


def hs_pool_set_length(pool: int, req: int, layer: int, length: int) -> None:
    _check(lib().hs_pool_set_length(pool, req, layer, int(length)))


def hs_pool_append(pool: int, req: int, layer: int, pos: int, src, n: Optional[int] = None,
                   stream=None) -> None:
    """src: a device tensor (enqueued on stream) or a host numpy uint8 array
    [n][rec_bytes] (copied synchronously)."""
    if isinstance(src, np.ndarray):
        src = np.ascontiguousarray(src, dtype=np.uint8)
        rec = hs_pool_record_bytes(pool)
        nn = src.size // rec if n is None else n
        _check(lib().hs_pool_append(pool, req, layer, int(pos), int(nn), src.ctypes.data, 0,
                                    _stream(stream)))
    else:
        rec = hs_pool_record_bytes(pool)
        nn = (src.numel() * src.element_size()) // rec if n is None else n
        _check(lib().hs_pool_append(pool, req, layer, int(pos), int(nn), _ptr(src), 1,
                                    _stream(stream)))


def hs_pool_append_batch(batch: int, src, stream=None) -> None:
    """Write-through append of src[u] (device tensor [n][rec_bytes]) at the
    end of every unit's pool; positions are read on the device."""
    _check(lib().hs_pool_append_batch(batch, _ptr(src), _stream(stream)))


# ------------------------------------------------------------------ buffers

def hs_buffer_bytes(pool: int, B: int) -> int:
    return int(lib().hs_buffer_bytes(pool, B))


def hs_buffer_create(pool: int, req: int, layer: int, B: int, mem, stream=None) -> int:
    """mem: a device tensor of at least hs_buffer_bytes(pool, B) bytes."""
    out = ctypes.c_void_p()
    nbytes = mem.numel() * mem.element_size()
    _check(lib().hs_buffer_create(pool, req, layer, B, _ptr(mem), nbytes, _stream(stream),
                                  ctypes.byref(out)))
    return out.value


def hs_buffer_shared_bytes(pool: int, B: int) -> int:
    return int(lib().hs_buffer_shared_bytes(pool, B))


def hs_buffer_create_shared(base: int, layer: int, mem) -> int:
    """Rows of `layer` attached to the state of buffer `base` (same request):
    layers that reuse one selection. mem: a device tensor of at least
    hs_buffer_shared_bytes(pool, B) bytes."""
    out = ctypes.c_void_p()
    nbytes = mem.numel() * mem.element_size()
    _check(lib().hs_buffer_create_shared(base, layer, _ptr(mem), nbytes, ctypes.byref(out)))
    return out.value


def hs_buffer_destroy(buf: int) -> None:
    _check(lib().hs_buffer_destroy(buf))


def hs_buffer_grow(buf: int, new_B: int, mem, stream=None) -> None:
    """Move the buffer into `mem` (a device tensor of at least
    hs_buffer_bytes(pool, new_B) bytes) with new_B - B empty slots added."""
    nbytes = mem.numel() * mem.element_size()
    _check(lib().hs_buffer_grow(buf, int(new_B), _ptr(mem), nbytes, _stream(stream)))


def hs_buffer_grow_group(base: int, members, new_B: int, mem, member_mems, stream=None) -> None:
    """Grow a layer group: base's state and rows move into `mem` (at least
    hs_buffer_bytes(pool, new_B) bytes), the rows of members[i] into
    member_mems[i] (at least hs_buffer_shared_bytes(pool, new_B) bytes).
    members must be every buffer sharing base's state."""
    n = len(members)
    if len(member_mems) != n:
        raise ValueError("one memory block per member")
    arr = (ctypes.c_void_p * max(n, 1))(*members)
    ptrs = (ctypes.c_void_p * max(n, 1))(*[_ptr(m) for m in member_mems])
    sizes = (ctypes.c_size_t * max(n, 1))(*[m.numel() * m.element_size() for m in member_mems])
    nbytes = mem.numel() * mem.element_size()
    _check(lib().hs_buffer_grow_group(base, arr, n, int(new_B), _ptr(mem), nbytes, ptrs, sizes,
                                      _stream(stream)))


def hs_buffer_reset(buf: int, stream=None) -> None:
    _check(lib().hs_buffer_reset(buf, _stream(stream)))


def hs_buffer_rows(buf: int):
    """(device address of row 0, record bytes)."""
    p, rec = ctypes.c_void_p(), ctypes.c_size_t()
    _check(lib().hs_buffer_rows(buf, ctypes.byref(p), ctypes.byref(rec)))
    return p.value, rec.value


def hs_buffer_state_get(buf: int, B: int, stream=None):
    """(pos int32[B], stamp uint32[B], clock, err) as numpy / ints."""
    pos = np.empty(B, dtype=np.int32)
    stamp = np.empty(B, dtype=np.uint32)
    clock, err = ctypes.c_uint32(), ctypes.c_int32()
    _check(lib().hs_buffer_state_get(buf, pos.ctypes.data, stamp.ctypes.data, ctypes.byref(clock),
                                     ctypes.byref(err), _stream(stream)))
    return pos, stamp, clock.value, err.value


def hs_buffer_state_set(buf: int, pos: np.ndarray, stamp: np.ndarray, clock: int, err: int = 0,
                        stream=None) -> None:
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    stamp = np.ascontiguousarray(stamp, dtype=np.uint32)
    _check(lib().hs_buffer_state_set(buf, pos.ctypes.data, stamp.ctypes.data, int(clock), int(err),
                                     _stream(stream)))


# ------------------------------------------------------------------ batches

def hs_batch_create(bufs: Sequence[int]) -> int:
    arr = (ctypes.c_void_p * len(bufs))(*bufs)
    out = ctypes.c_void_p()
    _check(lib().hs_batch_create(arr, len(bufs), ctypes.byref(out)))
    return out.value


def hs_batch_destroy(batch: int) -> None:
    _check(lib().hs_batch_destroy(batch))


def hs_batch_status(batch: int, n: int, stream=None):
    """(status, error words int32[n]): HS_E_DEVICE when any unit has error
    bits set (not raised), else HS_OK."""
    errs = np.zeros(n, dtype=np.int32)
    st = lib().hs_batch_status(batch, errs.ctypes.data, _stream(stream))
    if st not in (HS_OK, HS_E_DEVICE):
        _check(st)
    return st, errs


def hs_resolve(batch: int, topk, k: int, slots, miss=None, stream=None) -> None:
    """topk/slots: int32 device tensors [n][k]; miss: int32 [n] or None."""
    _check(lib().hs_resolve(batch, _ptr(topk), int(k), _ptr(slots), _ptr(miss), _stream(stream)))


def hs_sparse_attn_workspace(batch: int, n_q_heads: int, k: int) -> int:
    return int(lib().hs_sparse_attn_workspace(batch, n_q_heads, k))


def hs_sparse_attn(batch: int, q, n_q_heads: int, slots, k: int, sm_scale: float, out, ws=None,
                   stream=None) -> None:
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().hs_sparse_attn(batch, _ptr(q), int(n_q_heads), _ptr(slots), int(k),
                                float(sm_scale), _ptr(out), _ptr(ws), ws_bytes, _stream(stream)))


def hs_sparse_attn_noalloc(batch: int, q, n_q_heads: int, slots, k: int, sm_scale: float, out,
                           stream=None) -> None:
    """hs_sparse_attn with its split-k partials in the library's own device
    scratch (no workspace, no allocation; calls on one GPU must not overlap)."""
    _check(lib().hs_sparse_attn_noalloc(batch, _ptr(q), int(n_q_heads), _ptr(slots), int(k),
                                        float(sm_scale), _ptr(out), _stream(stream)))


def hs_resolve_attn(batch: int, topk, k: int, slots, miss, q, n_q_heads: int, sm_scale: float,
                    out, ws=None, stream=None) -> None:
    """hs_resolve + hs_sparse_attn with the miss fetch done by the attention
    kernels (identical results)."""
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().hs_resolve_attn(batch, _ptr(topk), int(k), _ptr(slots), _ptr(miss), _ptr(q),
                                 int(n_q_heads), float(sm_scale), _ptr(out), _ptr(ws), ws_bytes,
                                 _stream(stream)))


def hs_prefetch(batch: int, stream=None) -> None:
    """Fetch every unit's records of its state's last fetch list (the other
    layers of a group sharing one selection)."""
    _check(lib().hs_prefetch(batch, _stream(stream)))


# ------------------------------------------------------------------ stage

def hs_stage_create(regions, ring: int) -> int:
    """regions: [(src tensor, dst tensor, bytes per entry, src stride bytes)]."""
    arr = (StageRegion * len(regions))(*[StageRegion(_ptr(s), _ptr(d), int(b), int(st))
                                         for s, d, b, st in regions])
    out = ctypes.c_void_p()
    _check(lib().hs_stage_create(arr, len(regions), int(ring), ctypes.byref(out)))
    return out.value


def hs_stage_destroy(stage: int) -> None:
    _check(lib().hs_stage_destroy(stage))


def hs_stage_run(stage: int, stream=None) -> None:
    _check(lib().hs_stage_run(stage, _stream(stream)))


def hs_stage_set_step(stage: int, step: int, stream=None) -> None:
    _check(lib().hs_stage_set_step(stage, int(step), _stream(stream)))


def hs_stage_get_step(stage: int) -> int:
    v = ctypes.c_uint32()
    _check(lib().hs_stage_get_step(stage, ctypes.byref(v)))
    return v.value


# ------------------------------------------------------------------ tracing

def hs_trace_enable(on: bool) -> None:
    _check(lib().hs_trace_enable(1 if on else 0))


def hs_trace_read() -> dict:
    """{class: (total_us, launches)} plus 'dropped'; clears the record."""
    t = Trace()
    _check(lib().hs_trace_read(ctypes.byref(t)))
    out = {c: (t.total_us[i], int(t.launches[i])) for i, c in enumerate(TRACE_CLASSES)}
    out["dropped"] = int(t.dropped)
    return out
